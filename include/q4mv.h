/*
 * q4mv.h -- C ABI of libq4mv.so, the affine-Q4 row-batched matrix-vector engine for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (Constant BATCH_MSL page, quantized_rows section, fn_q4_rows_h and the
 * prefill helper fn_qmv_small_b): for each matrix m, activation row r < nb and output o,
 *
 *   y[m][r][o] = sum_g ( S[m][o][g] * sum_{j<64} q[m][o][64g+j] * x[m][r][64g+j]
 *                      + B[m][o][g] * sum_{j<64} x[m][r][64g+j] )
 *
 * i.e. the dequantised weight W = S*q + B (4-bit code q in 0..15, bf16 scale S and bias B per
 * 64-wide group) times nb activation rows.
 *
 * Conventions for every entry point:
 *  - All pointers are HIP device pointers owned by the caller. The library allocates,
 *    frees and synchronises nothing, and keeps no state between calls (reentrant).
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    asynchronously on it; errors raised by the device later surface on that stream.
 *  - Layouts are contiguous and row-major. Sizes are element counts.
 *  - Every argument is validated on the host before anything is launched. On failure the
 *    function returns a negative status and enqueues nothing.
 *  - Inputs are read-only. Outputs are written only inside their stated extent.
 */
#ifndef Q4MV_H
#define Q4MV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    Q4MV_OK = 0,
    Q4MV_ERR_NULL = -1,     /* a required pointer is NULL */
    Q4MV_ERR_SHAPE = -2,    /* a size is out of range (see each function) */
    Q4MV_ERR_ODD_ROWS = -3, /* q4mv_2row with an odd out_dim */
    Q4MV_ERR_ALIGN = -4,    /* a pointer is not aligned as required */
    Q4MV_ERR_LAUNCH = -5,   /* the HIP launch reported an error */
    Q4MV_ERR_PATH = -6,     /* q4mv_path: unknown kernel path */
    Q4MV_ERR_VALUE = -7     /* q4mv_silu: div is zero or not finite */
};

/* Largest activation batch accepted (rows per matrix). */
#define Q4MV_MAX_NB 16

/*
 * q4mv_pack_codes -- pack 4-bit codes eight per u32 word, low nibble first.
 *
 * Layout (Constant BATCH_MSL page, fn_qmv_small_b, which reads code i of a word at bits
 * 4i..4i+3; the same order as the 4-bit pack of TQ_QUANT on the inferencelayer forward.rs
 * page): word k holds codes 8k..8k+7, code 8k+i in bits [4i, 4i+4).
 *   codes : u8  [n_codes]   one code per byte; only bits 0..3 of each byte are used.
 *   w     : u32 [n_codes/8] output.
 * A matrix of codes u8 [n_mat][out_dim][in_dim] packs into the w layout that q4mv reads.
 * Errors: NULL pointer; n_codes < 8 or n_codes % 8 != 0 (SHAPE); codes not 8-byte or w not
 * 4-byte aligned (ALIGN).
 */
int q4mv_pack_codes(const uint8_t *codes, uint32_t *w, int64_t n_codes, void *stream);

/*
 * q4mv_quantize -- affine-Q4 quantisation of dense f32 weights into the layout q4mv reads.
 *
 * For each row and each 64-wide group, the steps of the affine 5-bit host codec
 * (host_quant_q5_row on the memra-engine qwen4exp_gpu.rs page) with 16 levels:
 *   mn = min, mx = max of the group;  d = (mx - mn) / 15;  id = 1 / d (0 when d == 0 or
 *   1/d is not finite);  q = clamp(round_half_even((w - mn) * id), 0, 15)
 * computed in f32 (correctly rounded division), scale = bf16(d) and bias = bf16(mn) (round to
 * nearest even). The dequantised weight scale*q + bias is then within d/2 of w plus the bf16
 * rounding of scale and bias.
 *   wf     : f32 [n_rows][in_dim]        (n_rows = n_mat * out_dim; rows are independent)
 *   w      : u32 [n_rows][in_dim/8]      packed codes (q4mv_pack_codes layout)
 *   scales, biases : u16 [n_rows][in_dim/64] bf16 bit patterns
 * Inputs must be finite (other values give unspecified codes, never a fault).
 * Errors: NULL pointer; n_rows < 1, in_dim < 64 or in_dim % 64 != 0 (SHAPE); wf not
 * 16-byte, w not 4-byte, scales/biases not 2-byte aligned (ALIGN).
 */
int q4mv_quantize(const float *wf, uint32_t *w, uint16_t *scales, uint16_t *biases,
                  int64_t n_rows, int in_dim, void *stream);

/*
 * q4mv_prepare_x -- activation prep for the GEMV.
 *
 * Constant BATCH_MSL page, fn_norm_prep_b (its prep half) and fn_moe_act_b: x is split into
 * f16 even/odd streams, and each 32-element chunk gets one sum, taken over the same
 * f16-rounded values the dot products use.
 *   x    : f32 [n_rows][in_dim]
 *   xe   : f16 [n_rows][in_dim/2]   xe[n][k] = f16(x[n][2k])     (round to nearest even)
 *   xo   : f16 [n_rows][in_dim/2]   xo[n][k] = f16(x[n][2k+1])
 *   xsum : f32 [n_rows][in_dim/32]  xsum[n][c] = sum_{i<32} f16(x[n][32c+i]) (f32 sum)
 * For q4mv, n_rows = n_mat * nb and matrix m uses rows m*nb .. m*nb+nb-1.
 * Errors: NULL pointer; n_rows < 1, in_dim < 64 or in_dim % 64 != 0 (SHAPE); x, xe or xo
 * not 16-byte aligned, xsum not 4-byte aligned (ALIGN).
 */
int q4mv_prepare_x(const float *x, int n_rows, int in_dim, void *xe, void *xo, float *xsum,
                   void *stream);

/*
 * q4mv -- the affine-Q4 GEMV over n_mat independent matrices and nb activation rows each.
 *
 *   w       : u32 [n_mat][out_dim][in_dim/8]   packed codes (q4mv_pack_codes layout)
 *   scales  : u16 [n_mat][out_dim][in_dim/64]  bf16 bit patterns
 *   biases  : u16 [n_mat][out_dim][in_dim/64]  bf16 bit patterns
 *   xe, xo, xsum : from q4mv_prepare_x with n_rows = n_mat*nb
 *   y       : f32 [n_mat][nb][out_dim]          fully overwritten, nothing written beyond
 * Matrix m reads activation rows m*nb .. m*nb+nb-1 (the expert layout of fn_moe_down_b on
 * the Constant BATCH_MSL page: expert u's rows start at u*NB).
 * Accumulation is f32 throughout. The kernel, its launch shape and its summation order are
 * chosen from (in_dim, nb, out_dim) alone (q4mv_auto_path), never from n_mat: a matrix
 * gives bitwise the same result alone, in a batch of n_mat, or as a slot of q4mv_experts,
 * and q4mv and q4mv_2row give bitwise the same result. On the VALU kernels (paths 1 and 2)
 * the result does not depend on out_dim either.
 * Rows of any length (the page's row kernels read the activations from device memory at
 * any row length): each workgroup stages its activation rows in LDS as f16, and where
 * those of a whole row do not fit in the 160 KB of a gfx950 compute unit the product runs
 * as K slices of the columns, one launch per slice in column order, each later slice adding
 * its partial product to what y holds (y is then read as well as written). The slices
 * depend on (in_dim, nb, out_dim) only.
 * Errors: NULL pointer; n_mat outside 1..65535, out_dim < 1, in_dim < 64, in_dim % 64 != 0,
 * nb outside 1..Q4MV_MAX_NB (SHAPE); w, xe or xo not 16-byte aligned, scales/biases not
 * 2-byte, xsum/y not 4-byte aligned (ALIGN); launch failure.
 */
int q4mv(const uint32_t *w, const uint16_t *scales, const uint16_t *biases, const void *xe,
         const void *xo, const float *xsum, float *y, int n_mat, int out_dim, int in_dim,
         int nb, void *stream);

/*
 * q4mv_2row -- same contract and bitwise-identical result; each lane group of a wavefront
 * owns two consecutive output rows and shares every activation read between them (the
 * two-row helper fn_q4_2rows_h and fn_moe_down_b on the Constant BATCH_MSL page). It takes
 * the MFMA kernel wherever q4mv does. (On MI355X the one-row kernel keeps its activations
 * in registers, so there is no activation read left to share, and it measured faster than
 * the two-row kernel on every shape, the 640-wide expert down projection included.)
 * Extra error: out_dim odd (ODD_ROWS).
 */
int q4mv_2row(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
              const void *xe, const void *xo, const float *xsum, float *y, int n_mat,
              int out_dim, int in_dim, int nb, void *stream);

/*
 * q4mv_path -- q4mv with an explicit kernel choice instead of the automatic dispatch.
 *   path 0: automatic (what q4mv does), 1: VALU dot-product kernel, one row per lane group,
 *   2: VALU kernel, two rows per lane group (q4mv_2row; out_dim must be even),
 *   3: MFMA kernel (16x16x32 or 32x32x16 f16 matrix cores).
 * Every path takes every nb and row length, with K slices as q4mv describes: the VALU
 * kernels stage min(nb, 8) rows per launch (larger batches run as launches over row ranges
 * of 8) at 2.125 bytes per value and slice where that exceeds the LDS; the MFMA kernel
 * stages nb * (in_dim/8 + 1) * 16 + in_dim bytes next to its per-wave scratch.
 * Same arguments, layouts and errors as q4mv, plus PATH for an unknown path. For testing and
 * measurement of every kernel at every nb.
 */
int q4mv_path(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
              const void *xe, const void *xo, const float *xsum, float *y, int n_mat,
              int out_dim, int in_dim, int nb, int path, void *stream);

/*
 * q4mv_fused -- q4mv_prepare_x and q4mv in one launch: the GEMV takes the f32 activations
 * and each workgroup does the prep of its rows while it stages them (f16 rounding of every
 * value, and per 32-column chunk the f32 sum of the rounded values with the same additions
 * in the same order as q4mv_prepare_x). The activation prep of fn_norm_prep_b /
 * fn_moe_act_b (Constant BATCH_MSL page) is thus folded into the product instead of being a
 * launch of its own, and no xe/xo/xsum buffers are needed.
 *   x     : f32 [n_mat*nb][in_dim], 16-byte aligned; matrix m reads rows m*nb .. m*nb+nb-1
 *   path  : as q4mv_path (0 = the automatic dispatch of q4mv)
 * Other arguments, layouts and errors as q4mv_path. The result is bitwise what
 * q4mv_prepare_x followed by q4mv_path gives on the same path.
 */
int q4mv_fused(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
               const float *x, float *y, int n_mat, int out_dim, int in_dim, int nb, int path,
               void *stream);

/*
 * q4mv_silu -- q4mv with the output passed through silu(y / div):
 *   y[m][r][o] = t / (1 + exp(-t)),  t = (the q4mv result) / div
 * the gated-residual bottleneck of fn_qmv_silu_b on the Constant BATCH_MSL page, fused into
 * the GEMV's store (one launch, no extra pass over y). t is formed in f32 by a division and
 * exp is the device library's single-precision exp. Same arguments, layouts, kernels and
 * errors as q4mv, plus VALUE when div is 0 or not finite.
 */
int q4mv_silu(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
              const void *xe, const void *xo, const float *xsum, float *y, int n_mat,
              int out_dim, int in_dim, int nb, float div, void *stream);

/* q4mv_silu with an explicit kernel path (as q4mv_path). */
int q4mv_path_silu(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                   const void *xe, const void *xo, const float *xsum, float *y, int n_mat,
                   int out_dim, int in_dim, int nb, float div, int path, void *stream);

/*
 * q4mv_swiglu_prep -- the SwiGLU activation of an expert MLP fused with the activation prep
 * of its down projection (fn_moe_act_b on the Constant BATCH_MSL page, whose input is the
 * stacked gate/up output of fn_moe_gate_up_b):
 *   gu   : f32 [n_rows][2*inter]   row n = gate[0..inter) then up[0..inter), e.g. the y of a
 *          q4mv over the stacked gate+up weights (out_dim = 2*inter; n_rows = n_mat*nb)
 *   h[n][j] = silu(gate[n][j]) * up[n][j], computed in f32 (silu(g) = g / (1 + exp(-g)))
 *   xe, xo, xsum : as q4mv_prepare_x would produce for x = h (in_dim = inter): the f16
 *          even/odd streams of h and the f32 sums of each 32 f16-rounded values.
 * Errors: NULL pointer; n_rows < 1, inter < 64 or inter % 64 != 0 (SHAPE); gu not 8-byte,
 * xe or xo not 16-byte, xsum not 4-byte aligned (ALIGN).
 */
int q4mv_swiglu_prep(const float *gu, int n_rows, int inter, void *xe, void *xo, float *xsum,
                     void *stream);

/*
 * q4mv_pack_lowbit -- pack 4-bit codes into the Q2 (bits = 2) or Q3 (bits = 3) layout.
 *
 * The low-bit code is the 4-bit code's top bits, q = q4 >> (4 - bits), as fn_q2_rows_h and
 * fn_q3_rows_h on the Constant BATCH_MSL page define them (codes q4 >> 2 and q4 >> 1). Each
 * 32-code chunk c of a row holds column t = 16i + 8u + p (i, u < 2, p < 8):
 *   Q2: q at bit 4p + 2u of word 2c + i (2 words per chunk);
 *   Q3: q >> 1 at that bit of word 3c + i, and q & 1 at bit 4p + 2i + u of word 3c + 2 (3
 *       words per chunk: its two upper-bit words, then its lowest-bit word; the two planes
 *       of fn_q3_rows_h, interleaved by chunk).
 * A row is C*bits words, C = in_dim/32, and a chunk bits consecutive words. (Every code sits
 * in the nibble of its column within its 8-column word, so one shift and one mask per word
 * give the Q4 nibble layout.)
 *   codes : u8  [n_rows][in_dim]          one 4-bit code per byte (bits 4..7 ignored)
 *   w     : u32 [n_rows][in_dim/32*bits]  output (n_rows = n_mat * out_dim)
 * Errors: NULL pointer; bits not 2 or 3 (VALUE); n_rows < 1, in_dim < 64, in_dim % 64 != 0,
 * n_rows*in_dim/32 >= 2^31 - 256 (SHAPE); codes not 16-byte or w not 4-byte aligned (ALIGN).
 */
int q4mv_pack_lowbit(int bits, const uint8_t *codes, uint32_t *w, int64_t n_rows, int in_dim,
                     void *stream);

/*
 * q4mv_lowbit -- the Q2 / Q3 GEMV (fn_q2_rows_h, fn_q3_rows_h on the Constant BATCH_MSL
 * page): each weight is reconstructed at the middle of the 4-bit codes its code stands for,
 *   Q2: w = (4q + 1.5) s + b,   Q3: w = (2q + 0.5) s + b,
 * with the scale s and bias b of the 64-wide group (the same bf16 arrays as q4mv), so per
 * 32-code chunk acc += K s sum(q x) + (M s + b) sum(x). Same arguments, layouts and
 * accumulation as q4mv except:
 *   bits : 2 or 3;  w : u32 [n_mat][out_dim][in_dim/32*bits] (q4mv_pack_lowbit layout)
 *   path : 0 automatic (3 for nb >= 4 where path 3 is accepted; else 1 for nb = 1 or odd
 *          out_dim, and 2 otherwise), 1 VALU kernel, one row per lane group, 2 VALU kernel,
 *          two rows per lane group (out_dim even; bitwise the same result as 1), 3 the MFMA
 *          kernel (the codes moved into the Q4 nibble layout as each tile is staged, the
 *          tiled product of the page's expert GEMM fn_expert_qmm; needs in_dim/64 a
 *          multiple of 4 and scales and biases 8-byte aligned). Long rows run as K slices
 *          as in q4mv.
 * Errors: as q4mv (w 8-byte aligned), plus VALUE for bits, PATH for a path outside 0..3,
 * ODD_ROWS for path 2 with odd out_dim, SHAPE for path 3 where it is not accepted.
 */
int q4mv_lowbit(int bits, const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                const void *xe, const void *xo, const float *xsum, float *y, int n_mat,
                int out_dim, int in_dim, int nb, int path, void *stream);

/*
 * q4mv_experts -- the GEMV over selected matrices of a bank (the selected-expert launch
 * launch_qmatvec_bf16w_sel on the qwen4exp_gpu.rs page: a bank, a device array of expert
 * ids and an activation stride that may be 0; and the unique-expert dispatch of
 * fn_moe_gate_up_b / fn_moe_down_b on the Constant BATCH_MSL page):
 *   w, scales, biases : the bank, n_bank matrices in the q4mv layout
 *   sel     : i32 [n_sel] device array; slot u computes with bank matrix sel[u]
 *   xe, xo, xsum : q4mv_prepare_x output with n_rows = nb (x_shared != 0: every slot reads
 *             activation rows 0..nb-1, e.g. the gate/up projection of one token batch) or
 *             n_rows = n_sel*nb (x_shared == 0: slot u reads rows u*nb .. u*nb+nb-1, e.g.
 *             the down projection of each expert's own SwiGLU output)
 *   y       : f32 [n_sel][nb][out_dim]   fully overwritten
 *   path    : as q4mv_path (0 = automatic dispatch on (in_dim, nb, out_dim))
 * Slot u's result is bitwise what q4mv gives for bank matrix sel[u] and the same
 * activation rows. The ids live on the device and are not read by the host: a slot whose
 * id is outside 0..n_bank-1 reads no memory outside the bank and its y rows are NaN.
 * Errors: NULL pointer; n_bank < 1, n_sel outside 1..65535, and the shape errors of q4mv
 * (SHAPE); sel not 4-byte aligned or the alignment errors of q4mv (ALIGN); PATH, ODD_ROWS,
 * and SHAPE for path 3 as q4mv_path; launch failure.
 */
int q4mv_experts(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                 int n_bank, const int32_t *sel, int n_sel, const void *xe, const void *xo,
                 const float *xsum, float *y, int out_dim, int in_dim, int nb, int x_shared,
                 int path, void *stream);

/*
 * q4mv_experts_fused -- q4mv_experts with the activation prep done inside the launch, from
 * f32 rows (as q4mv_fused does for q4mv):
 *   x      : f32, 16-byte aligned. swiglu = 0: rows of in_dim values, [nb][in_dim] when
 *            x_shared, else [n_sel*nb][in_dim] (slot u reads rows u*nb .. u*nb+nb-1);
 *            swiglu = 1: [gate | up] rows of 2*in_dim values in the same arrangement (the
 *            stacked output of the gate|up projection), and the activations are
 *            silu(gate) * up formed in f32 as q4mv_swiglu_prep forms them (fn_moe_act_b,
 *            Constant BATCH_MSL page: the SwiGLU of the expert MLP folded into the down
 *            projection's launch).
 * Other arguments and errors as q4mv_experts, plus VALUE for swiglu outside {0, 1}. The
 * result is bitwise what q4mv_prepare_x (or q4mv_swiglu_prep) followed by q4mv_experts
 * gives on the same path.
 */
int q4mv_experts_fused(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                       int n_bank, const int32_t *sel, int n_sel, const float *x, float *y,
                       int out_dim, int in_dim, int nb, int x_shared, int swiglu, int path,
                       void *stream);

/*
 * q4mv_combine -- routing-weighted sum of expert outputs (the expert sum of
 * fn_moe_combine_b on the Constant BATCH_MSL page, without its shared-expert gate):
 *   y    : f32 [n_u][nb][out_dim]   e.g. q4mv_experts output
 *   wmap : f32 [nb][n_u]            token r's weight for slot u (0 where r did not route to u)
 *   out  : f32 [nb][out_dim]        out[r][o] = sum over u = 0..n_u-1 of wmap[r][u]*y[u][r][o]
 * The sum runs in f32 in slot order, one fused multiply-add per slot, so the result is
 * deterministic. Errors: NULL pointer; n_u, nb or out_dim < 1, nb*out_dim > 2^31 (SHAPE);
 * a pointer not 4-byte aligned (ALIGN); launch failure.
 */
int q4mv_combine(const float *y, const float *wmap, float *out, int n_u, int nb, int out_dim,
                 void *stream);

/* Which path (1, 2 or 3) the automatic dispatch of q4mv (two_row = 0) or q4mv_2row
   (two_row = 1) takes for this shape; a negative status if the shape is invalid. The MFMA
   kernel for nb >= 4, for nb = 3 on matrices of at least 256 32-row tiles
   (out_dim > 8160) and for nb = 2 on matrices of at least 1024 tiles (out_dim > 32736);
   otherwise q4mv takes the one-row VALU kernel and q4mv_2row the two-row one (the two VALU
   kernels give bitwise the same result). in_dim does not enter the choice: every path takes
   every row length. */
int q4mv_auto_path(int in_dim, int nb, int two_row, int out_dim);

/* Static English text for a status code. */
const char *q4mv_status_str(int status);

/* Library version, major*10000 + minor*100 + patch. */
int q4mv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4MV_H */
