// Internal (host-side) interface between the C ABI and the kernel launchers of libq4mv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4mv_impl {

struct GemvArgs {
    const uint32_t *w;
    const uint16_t *scales;
    const uint16_t *biases;
    const void *xe;
    const void *xo;
    const float *xsum;
    float *y;
    int n_mat, out_dim, in_dim, nb;
    float epi_div;  // 0: y = the product; else y = silu(product / epi_div)
    hipStream_t stream;
    // Selected experts (sel null: matrix m is the m-th of the n_mat contiguous at w, scales,
    // biases): slot m uses bank matrix sel[m] of n_bank. x_shared: every slot reads
    // activation rows 0..nb-1 (else slot m reads rows m*nb .. m*nb+nb-1).
    const int *sel = nullptr;
    int n_bank = 0;
    int x_shared = 0;
    // Code width: 4 (affine-Q4), or the low-bit layouts 2 and 3 (VALU kernels only).
    int bits = 4;
    // f32 activations [rows][in_dim] (rows as for xe): the kernels stage them with the prep
    // done in the block (xe, xo and xsum are then not read).
    const float *xf = nullptr;
    // xf rows are [gate | up] (2*in_dim values) and the activations silu(gate) * up.
    int xf_glu = 0;
};

// Kernel paths (same numbering as q4mv_path in q4mv.h).
enum Path { kAuto = 0, kValu1 = 1, kValu2 = 2, kMfma = 3 };

// Lanes per output row for the VALU kernels: the largest power of two <= 64 dividing the
// number of 32-code chunks per row, so that every lane owns the same number of chunks.
inline int valu_log2g(int in_dim)
{
    const int chunks = in_dim / 32;
    int l = 0;
    while (l < 6 && (chunks % (2 << l)) == 0) l++;
    return l;
}

int auto_path(int in_dim, int nb, bool two_row, int out_dim);

hipError_t launch_pack(const uint8_t *codes, uint32_t *w, int64_t n_codes, hipStream_t s);
hipError_t launch_pack_lowbit(int bits, const uint8_t *codes, uint32_t *w, int64_t n_rows,
                              int in_dim, hipStream_t s);
hipError_t launch_combine(const float *y, const float *wmap, float *out, int n_u, int nb,
                          int out_dim, hipStream_t s);
hipError_t launch_quantize(const float *wf, uint32_t *w, uint16_t *scales, uint16_t *biases,
                           int64_t n_rows, int in_dim, hipStream_t s);
hipError_t launch_swiglu_prep(const float *gu, int n_rows, int inter, void *xe, void *xo,
                              float *xsum, hipStream_t s);
hipError_t launch_prep(const float *x, int n_rows, int in_dim, void *xe, void *xo, float *xsum,
                       hipStream_t s);
hipError_t launch_valu(const GemvArgs &a, int rows);
hipError_t launch_mfma(const GemvArgs &a);

// Compute units of the current device (cached per device).
int device_cus();

// Largest dynamic LDS a block may use on gfx950.
constexpr size_t kMaxLds = 160 * 1024;
// LDS bytes of the MFMA kernel for a shape: staged f16 activations + per-group sums + the
// per-wave staging votes and a zero operand (the partial-sum buffers of mfma_part_bytes come on top).
inline size_t mfma_lds_bytes(int in_dim, int nb)
{
    // nb rows of 4C + 1 pair units, then groups x 16 sums, then 16 ints and 32 zero bytes
    return (size_t)nb * (4 * (in_dim / 32) + 1) * 16 + (size_t)(in_dim / 64) * 16 * 4 + 96;
}
// Partial-sum buffers of the MFMA kernel: 2 steps x tile groups per block x (ks - 1) parts
// x lanes holding live rows x nacc accumulators.
inline size_t mfma_part_bytes(int wpb, int ks, int nacc, int lanes)
{
    return (size_t)2 * (wpb / ks) * (ks - 1) * lanes * nacc * 4;
}
// Launch shape of the MFMA kernel: waves per block and waves per tile (K-split); {0, 0} if
// the shape's LDS does not fit in one compute unit. need8: low-bit codes, which run on
// 8-wave blocks with a K-split of 1, 2, 4 or 8.
struct MfmaShape { int wpb, ks; };
MfmaShape mfma_shape(int in_dim, int nb, long tiles, bool need8);
// Columns per K slice of the MFMA kernel for a row of in_dim: in_dim when the staged
// activations of the whole row fit in LDS, else the length of the fewest equal slices that
// fit (8-wave blocks when need8); 0 if none does.
int mfma_slice(int in_dim, int nb, long tiles, bool need8);
// Columns per K slice of a VALU launch over nbp activation rows (same rule: in_dim when the
// whole row's staged activations fit in LDS).
int valu_slice(int in_dim, int nbp);
// Raise a kernel's dynamic LDS limit above the 64 KB default (once per kernel and size).
hipError_t ensure_lds(const void *fn, size_t bytes);
// Blocks of `fn` that can be resident on one CU at this block size and LDS (cached).
int resident_blocks(const void *fn, int threads, size_t lds);

}  // namespace q4mv_impl
