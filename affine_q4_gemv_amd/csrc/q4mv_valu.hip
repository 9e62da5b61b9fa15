// VALU kernels of libq4mv: affine-Q4 GEMV with packed f16 dot products (v_dot2c_f32_f16).
//
// Work mapping (wave64). A row of in_dim codes is C = in_dim/32 chunks of 32 codes (16
// bytes). G = 2^log2g lanes share a row, G the largest power of two <= 64 dividing C, so each
// lane owns CPL = C/G chunks: c = j, j+G, j+2G, ... for lane j of the group. A wave holds
// 64/G lane groups; each group owns ROWS consecutive output rows per step (ROWS = 2 is the
// two-row variant of fn_q4_2rows_h on the Constant BATCH_MSL page, which shares every
// activation read between two rows). Loads of codes are 16 bytes per lane and consecutive
// lanes read consecutive chunks of one row: 16*G contiguous bytes per row per instruction.
//
// Per chunk and activation row (quantized_rows section of the same page, fn_q4_rows_h):
//   acc += s * sum(q*x) + b * xsum[chunk]
// with sum(q*x) from f16 dot products: a code nibble masked into an f16 lane is the subnormal
// q*2^-24 (exact), odd nibbles come out as 16q*2^-24 and go to a second accumulator that is
// scaled by 1/16 (exact). All of acc is kept in units of 2^-24 (xsum is pre-scaled when it is
// staged) and multiplied by 2^24 once at the end. Every scaling is by a power of two, so the
// result is bitwise what the same f32 operations would give in natural units.
//
// Activations of the block's matrix are staged once per block in LDS (pair layout, see
// x_unit), and when NB*CPL is small they are held in registers for the whole kernel. Blocks
// are persistent: each wave strides over the row steps of its matrix.
#include "q4mv_device.h"
#include "q4mv_internal.h"

#include <algorithm>

namespace q4mv_impl {

constexpr int kValuThreads = 256;
constexpr int kValuMaxNB = 8;  // nb > 8 runs as two launches over activation-row ranges
// Launch shape (compile-time tunables, measured on MI355X): persistent blocks per CU, and
// whether a wave loads its next row step while computing the current one.
#ifndef Q4MV_VALU_BLOCKS_PER_CU
#define Q4MV_VALU_BLOCKS_PER_CU 4
#endif
#ifndef Q4MV_VALU1_BLOCKS_PER_CU
#define Q4MV_VALU1_BLOCKS_PER_CU 2  // one-row kernel
#endif
// ... and on long launches (every wave of a two-blocks-per-CU grid running at least
// SBLDS_MIN_STEPS row steps): LM head NB=1 35.57 -> 34.90 us with 3 (35.00 with 4); short
// launches are slower with more blocks (9728 x 2560 NB=1 5.90 -> 6.55 us with 3)
#ifndef Q4MV_VALU1_BLOCKS_PER_CU_LONG
#define Q4MV_VALU1_BLOCKS_PER_CU_LONG 3
#endif
#ifndef Q4MV_VALU_PREFETCH
#define Q4MV_VALU_PREFETCH 0
#endif
constexpr bool kValuPrefetch = Q4MV_VALU_PREFETCH != 0;
// Activations stay in registers for the whole kernel when NB * CPL is at most this.
#ifndef Q4MV_VALU_XREG_MAX
#define Q4MV_VALU_XREG_MAX 5
#endif
// Weights are read with non-temporal loads (each byte is used once; measured faster).
// (Activations loaded straight from device memory into registers, with no LDS staging,
// measured slower on MI355X: LM head NB=1 43 us against 36.5 us.)
#ifndef Q4MV_VALU_NT
#define Q4MV_VALU_NT 1
#endif
constexpr bool kValuNT = Q4MV_VALU_NT != 0;
#ifndef Q4MV_VALU_XFIRST
#define Q4MV_VALU_XFIRST 1
#endif
#ifndef Q4MV_VALU_BALANCE
#define Q4MV_VALU_BALANCE 0
#endif
// Low-bit widths: persistent blocks per CU of the one-row kernel, a floor on waves per SIMD
// (caps registers), and the next step's loads issued before the current step's compute.
#ifndef Q4MV_LOWBIT1_BLOCKS_PER_CU
#define Q4MV_LOWBIT1_BLOCKS_PER_CU 4
#endif
#ifndef Q4MV_LOWBIT_MIN_WAVES
#define Q4MV_LOWBIT_MIN_WAVES 1
#endif
#ifndef Q4MV_LOWBIT_PREFETCH
#define Q4MV_LOWBIT_PREFETCH 0
#endif
// Output rows per lane group in the paired kernel (2; 4 also gives the same bits).
#ifndef Q4MV_VALU_PAIR_ROWS
#define Q4MV_VALU_PAIR_ROWS 2
#endif
// Code widths whose one-row nb = 1 kernel uses the block-loaded scales (bit b: width b).
#ifndef Q4MV_VALU_SBLDS_BITS
#define Q4MV_VALU_SBLDS_BITS ((1 << 4) | (1 << 3) | (1 << 2))
#endif
// Scales and biases of a wave step: the step's rows are consecutive, so their scales (and
// their biases) form one contiguous block; it is read with 16-byte loads (one instruction
// for both arrays) into a per-wave LDS slot and each lane picks its values from there,
// instead of one 2-byte load per lane, chunk and array.
#ifndef Q4MV_VALU_SBLDS
#define Q4MV_VALU_SBLDS 1
#endif
// ... used when every wave runs at least this many steps: the LDS round trip lengthens a
// step's critical path, so short launches (a step or two per wave) are faster without it.
#ifndef Q4MV_VALU_SBLDS_MIN_STEPS
#define Q4MV_VALU_SBLDS_MIN_STEPS 4
#endif

// Per-wave LDS slot of the block-loaded scales and biases: 16-byte segments per array
// (0 where the shape does not use it). A wave step's rows hold 32 * ROWS * CPL groups.
constexpr int valu_sb_segs(int rows, int cpl, bool specialised)
{
    return Q4MV_VALU_SBLDS && specialised && rows * cpl <= 8 ? 4 * rows * cpl : 0;
}

// ---------------------------------------------------------------------------------------
// Code widths. BITS = 4 is the affine-Q4 layout (one 16-byte chunk of 32 codes). BITS = 2 and
// 3 are the low-bit variants of fn_q2_rows_h / fn_q3_rows_h (quantized_rows section of the
// Constant BATCH_MSL page): the 4-bit code's top 2 or 3 bits, reconstructed at the middle of
// the dropped range, w = (4q + 1.5) s + b and w = (2q + 0.5) s + b. A chunk of 32 codes is 2
// words (Q2) or 2 + 1 words (Q3: upper-two-bit plane and lowest-bit plane); the layouts put
// each code in the nibble of its column within its 8-column word, so that one shift and one
// mask per word (lowbit_chunk_to_q4) give the Q4 nibble layout (Q2 is split in place):
//   Q2 word i of chunk c covers columns 32c+16i .. +15; column 32c+16i+8u+p (u < 2, p < 8)
//      is the 2-bit field at bit 4p + 2u.
//   Q3 upper words: the code's upper two bits at those positions; lowest-bit word of chunk c:
//      the low bit of column 32c+16i+8u+p at bit 4p + 2i + u.
// Row layout: C chunks of BITS words (Q4 4 words; Q2 2 words; Q3 its 2 upper-bit words, then
// its lowest-bit word), so a row is C * BITS words and a chunk one contiguous load.

// One chunk's code words of row base wr (u32 units), streamed with non-temporal loads
// (each byte is used once). Q4: 4 words; Q2: 2 words (.x, .y); Q3: 2 upper words and the
// lowest-bit word (.z), one 12-byte load.
template <int BITS, bool NT>
__device__ __forceinline__ uint4 load_chunk(const uint32_t *wr, int c)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    if constexpr (BITS == 4) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(wr) + c;
        const u32x4 v = NT ? __builtin_nontemporal_load(p) : *p;
        return uint4{v[0], v[1], v[2], v[3]};
    } else {
        if constexpr (BITS == 2) {
            const u32x2 *p = reinterpret_cast<const u32x2 *>(wr) + c;
            const u32x2 v = NT ? __builtin_nontemporal_load(p) : *p;
            return uint4{v[0], v[1], 0u, 0u};
        } else {
            const uint32_t *q = wr + 3 * c;
            if constexpr (NT)
                return uint4{__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1),
                             __builtin_nontemporal_load(q + 2), 0u};
            else
                return uint4{q[0], q[1], q[2], 0u};
        }
    }
}

// Split one chunk into 16 f16 pairs: h[J][m] meets pair P_m of activation word J (pair
// layout, x_unit), masked fields read as f16 subnormals. Q4 (and Q3, first moved into the Q4
// nibble layout): P0 and P2 come out as q*2^-24, P1 and P3 as 16q*2^-24. Q2 is split in
// place, one shift per word: word i holds activation words 2i (fields at 4p) and 2i+1
// (fields at 4p+2), so P0/P2 of J = 2i come out as q*2^-24, of J = 2i+1 as 4q*2^-24, and
// P1/P3 as 16q and 64q (times 2^-24).
template <int BITS>
__device__ __forceinline__ void split_chunk(const uint4 cw, uint32_t (&h)[4][4])
{
    if constexpr (BITS == 2) {
        const uint32_t wd[2] = {cw.x, cw.y};
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const uint32_t w8 = wd[i] >> 8;
#pragma unroll
            for (int u = 0; u < 2; u++) {
                h[2 * i + u][0] = wd[i] & (0x00030003u << (2 * u));
                h[2 * i + u][1] = wd[i] & (0x00300030u << (2 * u));
                h[2 * i + u][2] = w8 & (0x00030003u << (2 * u));
                h[2 * i + u][3] = w8 & (0x00300030u << (2 * u));
            }
        }
    } else {
        const uint4 q = BITS == 4 ? cw : lowbit_chunk_to_q4<BITS>(cw.x, cw.y, cw.z);
        const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int J = 0; J < 4; J++) {
            const uint32_t w8 = wd[J] >> 8;
            h[J][0] = wd[J] & 0x000F000Fu;
            h[J][1] = wd[J] & 0x00F000F0u;
            h[J][2] = w8 & 0x000F000Fu;
            h[J][3] = w8 & 0x00F000F0u;
        }
    }
}

// sum(q * x) * 2^-24 of one chunk and one activation row from its split codes and the
// row's four pair-layout units: one accumulator per unit of the split.
template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint32_t (&h)[4][4], const uint4 (&xp)[4])
{
    if constexpr (BITS == 2) {
        // a[(J & 1) + 2 * (m & 1)]: units 1, 4, 16, 64
        float a[4];
#pragma unroll
        for (int u = 0; u < 2; u++) {
            a[u] = dot2_first(h[u][0], xp[u].x);
            a[u + 2] = dot2_first(h[u][1], xp[u].y);
            a[u] = dot2(h[u][2], xp[u].z, a[u]);
            a[u + 2] = dot2(h[u][3], xp[u].w, a[u + 2]);
            a[u] = dot2(h[u + 2][0], xp[u + 2].x, a[u]);
            a[u + 2] = dot2(h[u + 2][1], xp[u + 2].y, a[u + 2]);
            a[u] = dot2(h[u + 2][2], xp[u + 2].z, a[u]);
            a[u + 2] = dot2(h[u + 2][3], xp[u + 2].w, a[u + 2]);
        }
        return __builtin_fmaf(a[3], 0.015625f,
                              __builtin_fmaf(a[2], 0.0625f, __builtin_fmaf(a[1], 0.25f, a[0])));
    } else {
        float ae = dot2_first(h[0][0], xp[0].x);
        float ao = dot2_first(h[0][1], xp[0].y);
        ae = dot2(h[0][2], xp[0].z, ae);
        ao = dot2(h[0][3], xp[0].w, ao);
#pragma unroll
        for (int J = 1; J < 4; J++) {
            ae = dot2(h[J][0], xp[J].x, ae);
            ao = dot2(h[J][1], xp[J].y, ao);
            ae = dot2(h[J][2], xp[J].z, ae);
            ao = dot2(h[J][3], xp[J].w, ao);
        }
        return __builtin_fmaf(ao, 0.0625f, ae);
    }
}

// acc += s' * qd + b' * xsum with (s', b') = (s, b) for Q4, (4s, 1.5s + b) for Q2 and
// (2s, 0.5s + b) for Q3 (the chunk folds of fn_q4/q2/q3_rows_h).
template <int BITS>
__device__ __forceinline__ float chunk_fold(uint32_t sbits, uint32_t bbits, float qd, float xsv,
                                            float acc)
{
    const float s = bf16_to_f32(sbits), b = bf16_to_f32(bbits);
    if constexpr (BITS == 4) {
        return __builtin_fmaf(s, qd, __builtin_fmaf(b, xsv, acc));
    } else {
        constexpr float kq = BITS == 2 ? 4.0f : 2.0f, km = BITS == 2 ? 1.5f : 0.5f;
        return __builtin_fmaf(kq * s, qd, __builtin_fmaf(__builtin_fmaf(km, s, b), xsv, acc));
    }
}

// LOG2G, CPL > 0: lane-group size and chunks per lane fixed at compile time (the common row
// lengths); LOG2G = -1, CPL = 0: both taken at run time (any in_dim).
template <int NB, int ROWS, int LOG2G, int CPL, int BITS, bool SBL = false>
__global__ __launch_bounds__(kValuThreads, BITS == 4 ? 1 : Q4MV_LOWBIT_MIN_WAVES) void valu_kernel(
    const uint4 *__restrict__ w, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint2 *__restrict__ xe,
    const uint2 *__restrict__ xo, const float *__restrict__ xsum, float *__restrict__ y,
    int out_dim, int in_dim, int nb_total, int r0, int log2g_rt, int cpl_rt, float epi_div,
    const int *__restrict__ sel, int n_bank, int x_shared, const float *__restrict__ xf,
    int xf_glu, int in_full, int k0, int accum)
{
    const int log2g = LOG2G >= 0 ? LOG2G : log2g_rt;
    extern __shared__ uint4 lds[];
    constexpr bool XREG = CPL > 0 && NB * CPL <= Q4MV_VALU_XREG_MAX;
    const int m = blockIdx.y;
    // K slice: columns k0 .. k0+in_dim-1 of rows of in_full columns (in_dim == in_full and
    // k0 == 0 unless the activations of the whole row do not fit in LDS); C, groups and the
    // staged layout are the slice's, row strides the full row's
    const int C = in_dim >> 5;
    const int groups = in_dim >> 6;
    const int Cf = in_full >> 5, gf = in_full >> 6, kc0 = k0 >> 5, g0 = k0 >> 6;
    const int words8 = in_full >> 3;  // uint2 units (4 halves) per activation row

    // Stage activation rows r0 .. r0+NB-1 of matrix m (pair layout + scaled sums) in LDS.
    // stage_load issues one round of loads into registers and stage_store writes them, so a
    // wave can put its first weight loads between the two and the latencies overlap.
    const size_t xrow0 = (x_shared ? 0 : (size_t)m * nb_total) + r0;
    const uint2 *xe_m = xe + xrow0 * words8 + (k0 >> 3);
    const uint2 *xo_m = xo + xrow0 * words8 + (k0 >> 3);
    const float *xsum_m = xsum + xrow0 * Cf + kc0;
    float *xsw = reinterpret_cast<float *>(lds + NB * C * 4);
    const int units = NB * C * 4;  // 16-byte pair units; NB*C chunk sums
    struct XStage { uint2 e[4], o[4]; float sv; };
    auto stage_load = [&](int base, XStage &st) {
        // indices clamped: rounds past the end read valid data that stage_store drops
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int u = min(base + i * kValuThreads, units - 1);
            const int r = u / (C * 4), cj = u - r * (C * 4);
            st.e[i] = xe_m[(size_t)r * words8 + cj];
            st.o[i] = xo_m[(size_t)r * words8 + cj];
        }
        const int us = min((base - threadIdx.x) / 4 + (int)threadIdx.x, NB * C - 1);  // chunk sum
        const int rs = us / C;
        st.sv = xsum_m[(size_t)rs * Cf + (us - rs * C)];
    };
    auto stage_store = [&](int base, const XStage &st) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int u = base + i * kValuThreads;
            if (u < units) {
                const int r = u / (C * 4), cj = u - r * (C * 4);
                lds[x_unit(r, cj >> 2, cj & 3, C)] = make_pairs(st.e[i], st.o[i]);
            }
        }
        const int us = (base - threadIdx.x) / 4 + threadIdx.x;
        if (us < NB * C) xsw[us] = st.sv * kTwoM24;
    };
    // the remaining rounds and the barrier; the first round's loads are in st0
    auto stage_finish = [&](const XStage &st0) {
        stage_store(threadIdx.x, st0);
        for (int base = threadIdx.x + 4 * kValuThreads; base < units; base += 4 * kValuThreads) {
            XStage st;
            stage_load(base, st);
            stage_store(base, st);
        }
        __syncthreads();
    };
    // Fused prep (xf non-null: f32 activations): the block rounds its rows to f16 itself
    // and forms each 32-column chunk's sum of the rounded values with the additions of
    // q4mv_prepare_x (pair sums, then a balanced tree over the chunk's 16 pairs: each thread
    // adds its word's four pairs, two quad DPP steps add the chunk's four words), so the
    // staged LDS contents are bitwise those staged from q4mv_prepare_x's outputs. One thread
    // per 8-column word; a quad of lanes is one chunk (words per row are a multiple of 8).
    // With xf_glu the rows are [gate | up] and the values silu(gate) * up (as
    // q4mv_swiglu_prep forms them).
    const int wrow = in_dim >> 3, words = NB * wrow;
    const int rs4 = xf_glu ? in_full >> 1 : in_full >> 2;  // float4 per row
    const float4 *xf_m = xf ? reinterpret_cast<const float4 *>(xf) + xrow0 * (size_t)rs4 : nullptr;
    struct FStage { float4 v[2][4]; };
    auto fstage_load = [&](int base, FStage &st) {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int wi = min(base + i * kValuThreads, words - 1);
            const int r = wi / wrow;
            xword_load(xf_m + (size_t)r * rs4, (k0 >> 3) + wi - r * wrow, in_full, xf_glu, st.v[i]);
        }
    };
    auto fstage_store = [&](int base, const FStage &st) {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int wi = base + i * kValuThreads;
            if (wi < words) {  // uniform per quad
                const int r = wi / wrow, kw = wi - r * wrow;
                float f[8];
                xword_values(st.v[i], xf_glu, f);
                _Float16 h[8];
#pragma unroll
                for (int t = 0; t < 8; t++) h[t] = (_Float16)f[t];
                float ps[4];
#pragma unroll
                for (int q = 0; q < 4; q++) ps[q] = (float)h[2 * q] + (float)h[2 * q + 1];
                float sum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
                sum += dpp<0xB1>(sum);
                sum += dpp<0x4E>(sum);
                if ((kw & 3) == 0) xsw[r * C + (kw >> 2)] = sum * kTwoM24;
                // pair layout: (x0, x4) (x1, x5) (x2, x6) (x3, x7)
                uint4 u;
                u.x = __builtin_bit_cast(uint32_t, half2_t{h[0], h[4]});
                u.y = __builtin_bit_cast(uint32_t, half2_t{h[1], h[5]});
                u.z = __builtin_bit_cast(uint32_t, half2_t{h[2], h[6]});
                u.w = __builtin_bit_cast(uint32_t, half2_t{h[3], h[7]});
                lds[x_unit(r, kw >> 2, kw & 3, C)] = u;
            }
        }
    };
    auto fstage_finish = [&](const FStage &st0) {
        fstage_store(threadIdx.x, st0);
        for (int base = threadIdx.x + 2 * kValuThreads; base < words; base += 2 * kValuThreads) {
            FStage st;
            fstage_load(base, st);
            fstage_store(base, st);
        }
        __syncthreads();
    };
    auto stage = [&]() {
        if (xf) {
            FStage st0;
            fstage_load(threadIdx.x, st0);
            fstage_finish(st0);
            return;
        }
        XStage st0;
        stage_load(threadIdx.x, st0);
        stage_finish(st0);
    };
    const float *xs = reinterpret_cast<const float *>(lds + NB * C * 4);

    const int lane = threadIdx.x & 63;
    const int G = 1 << log2g;
    const int j = lane & (G - 1);
    const int grp = lane >> log2g;
    const int rows_per_wave = (64 >> log2g) * ROWS;
    const int wave_steps = (out_dim + rows_per_wave - 1) / rows_per_wave;
    const int wstride = gridDim.x * (kValuThreads / 64);
    const int cpl = CPL > 0 ? CPL : cpl_rt;

    // Weights: matrix m, or bank matrix sel[m]. An id outside the bank reads matrix 0 and
    // stores NaN (a NaN divisor makes the epilogue return NaN).
    int e = m;
    if (sel) {
        const int id = sel[m];
        const bool bad = (unsigned)id >= (unsigned)n_bank;
        e = bad ? 0 : id;
        if (bad) epi_div = __builtin_nanf("");
    }
    const uint32_t *w_m = reinterpret_cast<const uint32_t *>(w) + (size_t)e * out_dim * Cf * BITS;
    const uint16_t *s_m = scales + (size_t)e * out_dim * gf;
    const uint16_t *b_m = biases + (size_t)e * out_dim * gf;
    float *y_m = y + ((size_t)m * nb_total + r0) * out_dim;
    // stored value: the product (plus what y holds from the previous K slices), then the
    // epilogue; only the last slice of a sliced product has a nonzero epi_div
    auto out_value = [&](float v, size_t at) {
        if (accum) v += y_m[at];
        return gemv_epilogue(v, epi_div);
    };

    // activations in registers for the whole kernel when they fit
    uint4 xr[XREG ? CPL : 1][XREG ? NB : 1][4];
    float xsr[XREG ? CPL : 1][XREG ? NB : 1];
    auto load_xreg = [&]() {
        if constexpr (XREG) {
#pragma unroll
            for (int k = 0; k < CPL; k++) {
                const int c = j + (k << log2g);
#pragma unroll
                for (int r = 0; r < NB; r++) {
#pragma unroll
                    for (int J = 0; J < 4; J++) xr[k][r][J] = lds[x_unit(r, c, J, C)];
                    xsr[k][r] = xs[r * C + c];
                }
            }
        }
    };

    if constexpr (CPL > 0 && LOG2G >= 0) {
        // ---- fully unrolled chunk loop
        uint4 cc[ROWS][CPL];
        uint32_t scb[ROWS][CPL], bcb[ROWS][CPL];
        // block-loaded scales and biases (NSEG 16-byte segments per array): lanes 0..NSEG-1
        // load the step's scale block, NSEG..2*NSEG-1 its bias block; both arrays must be
        // 16-byte aligned (a step's block starts at a multiple of 64*ROWS*CPL bytes)
        constexpr bool kPrefetch = BITS == 4 ? kValuPrefetch : Q4MV_LOWBIT_PREFETCH != 0;
        constexpr int NSEG = (kPrefetch || !SBL) ? 0 : valu_sb_segs(ROWS, CPL, true);
        const bool sbl = NSEG > 0 && in_full == in_dim &&
            ((reinterpret_cast<uintptr_t>(s_m) | reinterpret_cast<uintptr_t>(b_m)) & 15) == 0;
        uint4 *const sbslot =
            reinterpret_cast<uint4 *>(reinterpret_cast<char *>(lds) +
                                      (((size_t)NB * C * 68 + 15) & ~(size_t)15)) +
            (threadIdx.x >> 6) * 2 * NSEG;
        uint4 sbv = {0u, 0u, 0u, 0u};
        // Loads are issued in the order compute() consumes them (chunk-major, then row), and
        // scales are converted where they are used, so the compiler's waits on the load
        // counter are progressive: a wave starts on its first chunk while the rest is still
        // in flight.
        auto load = [&](int ws, uint4 (&cw)[ROWS][CPL], uint32_t (&sv)[ROWS][CPL],
                        uint32_t (&bv)[ROWS][CPL]) {
            const uint32_t *wr[ROWS];
            const uint16_t *sr[ROWS], *br[ROWS];
#pragma unroll
            for (int t = 0; t < ROWS; t++) {
                const int row = min(ws * rows_per_wave + grp * ROWS + t, out_dim - 1);
                wr[t] = w_m + (size_t)row * Cf * BITS;
                sr[t] = s_m + (size_t)row * gf + g0;
                br[t] = b_m + (size_t)row * gf + g0;
            }
            if (sbl) {
                // segment L of the step's scale (L < NSEG) or bias block; the last step's
                // block may end past out_dim: a segment that crosses the end of the array
                // is read element by element up to it
                if (lane < 2 * NSEG) {
                    const bool isb = lane >= NSEG;
                    const uint16_t *arr = isb ? b_m : s_m;
                    const size_t e0 = (size_t)ws * rows_per_wave * groups + 8 * (lane - (isb ? NSEG : 0));
                    const size_t lim = (size_t)out_dim * groups;
                    if (e0 + 8 <= lim) {
                        typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
                        const u32x4v v = __builtin_nontemporal_load(
                            reinterpret_cast<const u32x4v *>(arr + e0));
                        sbv = uint4{v[0], v[1], v[2], v[3]};
                    } else {
                        uint32_t h[8];
#pragma unroll
                        for (int i = 0; i < 8; i++) h[i] = e0 + i < lim ? arr[e0 + i] : 0u;
                        sbv = uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                    h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < CPL; k++) {
                const int c = j + (k << log2g);
#pragma unroll
                for (int t = 0; t < ROWS; t++) {
                    cw[t][k] = load_chunk<BITS, kValuNT>(wr[t], kc0 + c);
                    if (sbl) continue;
#if Q4MV_VALU_NT
                    // streamed once: non-temporal loads (no reuse to keep in the caches)
                    sv[t][k] = __builtin_nontemporal_load(sr[t] + (c >> 1));
                    bv[t][k] = __builtin_nontemporal_load(br[t] + (c >> 1));
#else
                    sv[t][k] = sr[t][c >> 1];
                    bv[t][k] = br[t][c >> 1];
#endif
                }
            }
        };
        auto compute = [&](int ws) {
            if (sbl) {
                // this step's blocks into the wave's slot, then each lane's values (LDS
                // operations of one wave complete in order; the fences keep the compiler
                // from moving them across each other)
                asm volatile("" ::: "memory");
                if (lane < 2 * NSEG) sbslot[lane] = sbv;
                asm volatile("" ::: "memory");
                const uint16_t *sl = reinterpret_cast<const uint16_t *>(sbslot);
#pragma unroll
                for (int t = 0; t < ROWS; t++)
#pragma unroll
                    for (int k = 0; k < CPL; k++) {
                        const int el = (grp * ROWS + t) * groups + ((j + (k << log2g)) >> 1);
                        scb[t][k] = sl[el];
                        bcb[t][k] = sl[NSEG * 8 + el];
                    }
                asm volatile("" ::: "memory");
            }
            float acc[ROWS][NB];
#pragma unroll
            for (int t = 0; t < ROWS; t++)
#pragma unroll
                for (int r = 0; r < NB; r++) acc[t][r] = 0.0f;
#pragma unroll
            for (int k = 0; k < CPL; k++) {
                const int c = j + (k << log2g);
                // per-chunk fence for larger batches: bounds the LDS reads in flight
                if constexpr (NB > 1 || ROWS > 1) asm volatile("" ::: "memory");
                uint32_t h[ROWS][4][4];
#pragma unroll
                for (int t = 0; t < ROWS; t++) split_chunk<BITS>(cc[t][k], h[t]);
#pragma unroll
                for (int r = 0; r < NB; r++) {
                    uint4 xp[4];
                    float xsv;
                    if constexpr (XREG) {
#pragma unroll
                        for (int J = 0; J < 4; J++) xp[J] = xr[k][r][J];
                        xsv = xsr[k][r];
                    } else {
#pragma unroll
                        for (int J = 0; J < 4; J++) xp[J] = lds[x_unit(r, c, J, C)];
                        xsv = xs[r * C + c];
                    }
#pragma unroll
                    for (int t = 0; t < ROWS; t++)
                        acc[t][r] = chunk_fold<BITS>(scb[t][k], bcb[t][k],
                                                     chunk_dot<BITS>(h[t], xp), xsv, acc[t][r]);
                }
            }
            // all reductions first, then the stores (one divergent block at the very end)
#pragma unroll
            for (int t = 0; t < ROWS; t++)
#pragma unroll
                for (int r = 0; r < NB; r++) acc[t][r] = group_sum_ct<LOG2G>(acc[t][r]);
            if (j == 0) {
#pragma unroll
                for (int t = 0; t < ROWS; t++) {
                    const int row = ws * rows_per_wave + grp * ROWS + t;
                    if (row < out_dim) {
#pragma unroll
                        for (int r = 0; r < NB; r++)
                            y_m[(size_t)r * out_dim + row] =
                                out_value(acc[t][r] * kTwo24, (size_t)r * out_dim + row);
                    }
                }
            }
        };
        int ws = blockIdx.x * (kValuThreads / 64) + (threadIdx.x >> 6);
        if constexpr (BITS == 4 ? kValuPrefetch : Q4MV_LOWBIT_PREFETCH != 0) {
            // next step's codes are in flight while this step computes
            uint4 cn[ROWS][CPL];
            uint32_t sn[ROWS][CPL], bn[ROWS][CPL];
            if (ws < wave_steps) load(ws, cn, sn, bn);
            stage();
            load_xreg();
            for (; ws < wave_steps; ws += wstride) {
                asm volatile("" ::: "memory");
#pragma unroll
                for (int t = 0; t < ROWS; t++)
#pragma unroll
                    for (int k = 0; k < CPL; k++) {
                        cc[t][k] = cn[t][k];
                        scb[t][k] = sn[t][k];
                        bcb[t][k] = bn[t][k];
                    }
                if (ws + wstride < wave_steps) load(ws + wstride, cn, sn, bn);
                compute(ws);
            }
        } else {
#if Q4MV_VALU_XFIRST
            // activations first (small, mostly cache hits), then the first step's weights:
            // the staging only waits for its own loads
            if (xf) {
                FStage st0;
                fstage_load(threadIdx.x, st0);
                if (ws < wave_steps) load(ws, cc, scb, bcb);
                fstage_finish(st0);
            } else {
                XStage st0;
                stage_load(threadIdx.x, st0);
                if (ws < wave_steps) load(ws, cc, scb, bcb);
                stage_finish(st0);
            }
#else
            if (ws < wave_steps) load(ws, cc, scb, bcb);  // first step's weights, before staging
            stage();
#endif
            load_xreg();
            for (bool first = true; ws < wave_steps; ws += wstride, first = false) {
                // Compiler fence: keeps the per-step LDS activation reads inside the loop
                // (hoisting them all out of it multiplies register use and spills).
                asm volatile("" ::: "memory");
                if (!first) load(ws, cc, scb, bcb);
                compute(ws);
            }
        }
    } else {
        // ---- generic chunk count: runtime loop in batches of 4 chunks
        stage();
        for (int ws = blockIdx.x * (kValuThreads / 64) + (threadIdx.x >> 6); ws < wave_steps;
             ws += wstride) {
            asm volatile("" ::: "memory");
            float acc[ROWS][NB];
#pragma unroll
            for (int t = 0; t < ROWS; t++)
#pragma unroll
                for (int r = 0; r < NB; r++) acc[t][r] = 0.0f;
            int rowc[ROWS];
#pragma unroll
            for (int t = 0; t < ROWS; t++)
                rowc[t] = min(ws * rows_per_wave + grp * ROWS + t, out_dim - 1);
            for (int k0 = 0; k0 < cpl; k0 += 4) {
                uint4 cc[ROWS][4];
                uint32_t sc[ROWS][4], bc[ROWS][4];
#pragma unroll
                for (int t = 0; t < ROWS; t++)
#pragma unroll
                    for (int kk = 0; kk < 4; kk++) {
                        // clamped, unconditional loads (chunks past cpl are never used)
                        const int c = j + (min(k0 + kk, cpl - 1) << log2g);
                        cc[t][kk] = load_chunk<BITS, false>(w_m + (size_t)rowc[t] * Cf * BITS, kc0 + c);
                        sc[t][kk] = s_m[(size_t)rowc[t] * gf + g0 + (c >> 1)];
                        bc[t][kk] = b_m[(size_t)rowc[t] * gf + g0 + (c >> 1)];
                    }
#pragma unroll
                for (int kk = 0; kk < 4; kk++) {
                    if (k0 + kk >= cpl) break;
                    const int c = j + ((k0 + kk) << log2g);
#pragma unroll
                    for (int r = 0; r < NB; r++) {
                        uint4 xp[4];
#pragma unroll
                        for (int J = 0; J < 4; J++) xp[J] = lds[x_unit(r, c, J, C)];
                        const float xsv = xs[r * C + c];
#pragma unroll
                        for (int t = 0; t < ROWS; t++) {
                            uint32_t h[4][4];
                            split_chunk<BITS>(cc[t][kk], h);
                            acc[t][r] = chunk_fold<BITS>(sc[t][kk], bc[t][kk],
                                                         chunk_dot<BITS>(h, xp), xsv, acc[t][r]);
                        }
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < ROWS; t++) {
                const int row = ws * rows_per_wave + grp * ROWS + t;
#pragma unroll
                for (int r = 0; r < NB; r++) {
                    const float v = group_sum(acc[t][r], log2g);
                    if (j == 0 && row < out_dim)
                        y_m[(size_t)r * out_dim + row] =
                            out_value(v * kTwo24, (size_t)r * out_dim + row);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// host side

typedef void (*ValuFn)(const uint4 *, const uint16_t *, const uint16_t *, const uint2 *,
                       const uint2 *, const float *, float *, int, int, int, int, int, int,
                       float, const int *, int, int, const float *, int, int, int, int);

// (log2 G, CPL) of the specialised row lengths: in_dim = 32 * CPL << log2G.
#define Q4MV_VALU_SHAPES(X)                                                                   \
    X(4, 1) /* 512 */ X(2, 5) /* 640 */ X(5, 1) /* 1024 */ X(4, 3) /* 1536 */                 \
    X(6, 1) /* 2048 */ X(4, 5) /* 2560 */ X(5, 3) /* 3072 */ X(4, 7) /* 3584 */               \
    X(6, 2) /* 4096 */ X(5, 5) /* 5120 */ X(6, 3) /* 6144 */ X(5, 7) /* 7168 */               \
    X(6, 4) /* 8192 */ X(6, 7) /* 14336 */

// Low-bit codes: the expert row lengths only (640 and 2560); other lengths take the
// generic kernel.
#define Q4MV_LOWBIT_SHAPES(X) X(2, 5) /* 640 */ X(4, 5) /* 2560 */

// Whether (log2 G, CPL) is one of the specialised row lengths of code width bits.
static bool valu_specialised(int log2g, int cpl, int bits)
{
#define Q4MV_IS(L, K) \
    if (log2g == L && cpl == K) return true;
    if (bits == 4) {
        Q4MV_VALU_SHAPES(Q4MV_IS)
    } else {
        Q4MV_LOWBIT_SHAPES(Q4MV_IS)
    }
#undef Q4MV_IS
    return false;
}

// sbl: the block-loaded scale variant (one-row, nb = 1, Q4 only).
template <int NB, int ROWS, int BITS>
static ValuFn pick_shape(int log2g, int cpl, bool sbl = false)
{
#define Q4MV_PICK(L, K)                                                                   \
    if (log2g == L && cpl == K) {                                                         \
        if constexpr (NB == 1 && ROWS == 1 && ((Q4MV_VALU_SBLDS_BITS >> BITS) & 1) &&       \
                      valu_sb_segs(1, K, true) > 0)                                       \
            if (sbl) return valu_kernel<NB, ROWS, L, K, BITS, true>;                      \
        return valu_kernel<NB, ROWS, L, K, BITS>;                                         \
    }
    if constexpr (BITS == 4) {
        Q4MV_VALU_SHAPES(Q4MV_PICK)
    } else {
        Q4MV_LOWBIT_SHAPES(Q4MV_PICK)
    }
#undef Q4MV_PICK
    return valu_kernel<NB, ROWS, -1, 0, BITS>;
}

template <int ROWS, int BITS>
static ValuFn pick_nb(int nb, int log2g, int cpl, bool sbl)
{
    switch (nb) {
    case 1: return pick_shape<1, ROWS, BITS>(log2g, cpl, sbl);
    case 2: return pick_shape<2, ROWS, BITS>(log2g, cpl);
    case 3: return pick_shape<3, ROWS, BITS>(log2g, cpl);
    case 4: return pick_shape<4, ROWS, BITS>(log2g, cpl);
    // larger batches: generic kernel (the MFMA kernel is the fast path there)
    case 5: return valu_kernel<5, ROWS, -1, 0, BITS>;
    case 6: return valu_kernel<6, ROWS, -1, 0, BITS>;
    case 7: return valu_kernel<7, ROWS, -1, 0, BITS>;
    default: return valu_kernel<8, ROWS, -1, 0, BITS>;
    }
}

template <int BITS>
static ValuFn pick(int rows, int nb, int log2g, int cpl, bool sbl)
{
    return rows == 1 ? pick_nb<1, BITS>(nb, log2g, cpl, sbl)
                     : pick_nb<Q4MV_VALU_PAIR_ROWS, BITS>(nb, log2g, cpl, false);
}

// LDS of a VALU launch: nbp staged rows of C chunks (64 bytes of pairs and a 4-byte sum per
// chunk), then the per-wave scale/bias slots (nseg 16-byte segments per array).
static size_t valu_lds(int nbp, int C, int nseg)
{
    return (((size_t)nbp * C * 68 + 15) & ~(size_t)15) + (size_t)(kValuThreads / 64) * 2 * nseg * 16;
}

// One launch over activation rows r0 .. r0+nbp-1 and columns k0 .. k0+klen-1 (the whole row
// when klen == a.in_dim); accum: add to y instead of overwriting it; epi_div: the epilogue.
static hipError_t launch_valu_part(const GemvArgs &a, int rows, int r0, int nbp, int k0, int klen,
                                   int accum, float epi_div)
{
    const int log2g = valu_log2g(klen);
    const int C = klen / 32;
    const int cpl = C >> log2g;
    if (rows == 2) rows = Q4MV_VALU_PAIR_ROWS;
    const int rows_per_wave = (64 >> log2g) * rows;
    const long wave_steps = (a.out_dim + rows_per_wave - 1) / rows_per_wave;
    const long blocks_needed = (wave_steps + 3) / 4;
    // block-loaded scales (one-row kernel, nb = 1, whole rows) when the waves of two blocks
    // per CU would each run several steps
    const bool prefetch = a.bits == 4 ? kValuPrefetch : Q4MV_LOWBIT_PREFETCH != 0;
    const bool long_launch =
        wave_steps * a.n_mat >= (long)Q4MV_VALU_SBLDS_MIN_STEPS * device_cus() * 2 * 4;
    const int nseg =
        prefetch || rows != 1 || nbp != 1 || klen != a.in_dim ||
                !((Q4MV_VALU_SBLDS_BITS >> a.bits) & 1) || !long_launch
            ? 0 : valu_sb_segs(rows, cpl, valu_specialised(log2g, cpl, a.bits));
    ValuFn fn = a.bits == 2   ? pick<2>(rows, nbp, log2g, cpl, nseg > 0)
                : a.bits == 3 ? pick<3>(rows, nbp, log2g, cpl, nseg > 0)
                              : pick<4>(rows, nbp, log2g, cpl, nseg > 0);
    const size_t lds = valu_lds(nbp, C, nseg);
    if (lds > kMaxLds) return hipErrorInvalidValue;  // the slice length keeps it inside
    hipError_t e = ensure_lds(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess) return e;
    // persistent blocks: enough to fill every CU a few times over, shared by the matrices
    // (one round of blocks sized to the row steps, so that no wave runs a second step, was
    // measured slower on the 9728 x 2560 projection: 6.65 against 5.97 us)
    const long per_cu = std::min<long>(rows != 1      ? Q4MV_VALU_BLOCKS_PER_CU
                                       : a.bits != 4 ? Q4MV_LOWBIT1_BLOCKS_PER_CU
                                       : long_launch ? Q4MV_VALU1_BLOCKS_PER_CU_LONG
                                                     : Q4MV_VALU1_BLOCKS_PER_CU,
                                       resident_blocks(reinterpret_cast<const void *>(fn),
                                                       kValuThreads, lds));
    const long cap = std::max(1L, (long)device_cus() * per_cu / a.n_mat);
    long gx = std::max(1L, std::min(blocks_needed, cap));
#if Q4MV_VALU_BALANCE
    // every wave takes the same number of row steps: the fewest blocks that keep the
    // number of rounds of the full grid (no partly filled last round)
    const long rounds = (wave_steps + 4 * gx - 1) / (4 * gx);
    gx = std::max(1L, (wave_steps + 4 * rounds - 1) / (4 * rounds));
#endif
    hipLaunchKernelGGL(fn, dim3((unsigned)gx, (unsigned)a.n_mat), dim3(kValuThreads), lds,
                       a.stream, reinterpret_cast<const uint4 *>(a.w), a.scales, a.biases,
                       static_cast<const uint2 *>(a.xe), static_cast<const uint2 *>(a.xo),
                       a.xsum, a.y, a.out_dim, klen, a.nb, r0, log2g, cpl, epi_div,
                       a.sel, a.n_bank, a.x_shared, a.xf, a.xf_glu, a.in_dim, k0, accum);
    return hipGetLastError();
}

int valu_slice(int in_dim, int nbp)
{
    // the largest per-wave scale/bias slot (one-row nb = 1 launches) comes on top
    const size_t slot = (size_t)(kValuThreads / 64) * 2 * valu_sb_segs(1, 8, true) * 16;
    auto ok = [&](int len) { return valu_lds(nbp, len / 32, 0) + slot <= kMaxLds; };
    if (ok(in_dim)) return in_dim;
    // the fewest equal slices (the last one shorter) whose staged activations fit
    for (int ns = 2;; ns++) {
        const int len = ((in_dim + ns - 1) / ns + 63) / 64 * 64;
        if (ok(len)) return len;
        if (len <= 64) return 0;
    }
}

hipError_t launch_valu(const GemvArgs &a, int rows)
{
    // batches above kValuMaxNB rows run as launches over row ranges; rows whose staged
    // activations do not fit in LDS run as K slices, one launch each, in column order: each
    // later slice adds its partial product to y, and the epilogue comes with the last
    for (int r0 = 0; r0 < a.nb; r0 += kValuMaxNB) {
        const int nbp = std::min(kValuMaxNB, a.nb - r0);
        const int klen = valu_slice(a.in_dim, nbp);
        if (klen == 0) return hipErrorInvalidValue;
        for (int k0 = 0; k0 < a.in_dim; k0 += klen) {
            const int len = std::min(klen, a.in_dim - k0);
            const bool last = k0 + len == a.in_dim;
            hipError_t e =
                launch_valu_part(a, rows, r0, nbp, k0, len, k0 > 0, last ? a.epi_div : 0.0f);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace q4mv_impl
