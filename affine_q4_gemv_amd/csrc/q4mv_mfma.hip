// MFMA kernel of libq4mv: the affine-Q4 GEMV as a real contraction for larger activation
// batches, on gfx950's v_mfma_f32_16x16x32_f16 (D[16][16] += A[16][32] * B[32][16]).
//
// Operands: A = activations (16 rows = activation rows, padded with zeros past nb), taken
// from LDS in the pair layout; B = codes (16 columns = 16 output rows), unpacked in
// registers to f16 subnormals q*2^-24 (exact) by masking nibbles. One MFMA covers one
// 32-code chunk, so its sum belongs to a single scale group, and the group's scale and bias
// are applied in f32 after the two MFMAs of the group (the per-group fold of fn_q4_rows_h,
// Constant BATCH_MSL page, quantized_rows section); the dequantised weight is never formed
// (the page's tiled expert GEMM dequantises to f16 tiles instead).
//
// Loads: a wave owns 16 output rows; for K step k (chunks 4k..4k+3) lane (n, q)
// (n = lane % 16, q = lane / 16) reads 16 bytes = the whole chunk 4k+q of row n, so each row
// is read 64 contiguous bytes at a time, and KB K steps are in flight per lane. The MFMA wants lane (n, q) to hold word q of one chunk instead, so the four
// lane groups exchange words with a 4x4 transpose built from v_permlane32_swap and
// v_permlane16_swap (gfx950).
#include "q4mv_device.h"
#include "q4mv_internal.h"

#include <algorithm>

// Launch shape (compile-time tunable, measured on MI355X): the cap on blocks per CU.
#ifndef Q4MV_MFMA_BLOCKS_PER_CU
#define Q4MV_MFMA_BLOCKS_PER_CU 4
#endif

namespace q4mv_impl {

// KB: K steps whose loads are in flight together (the whole row when it fits).
// SMODE: how a row's scales and biases are loaded -- 2: groups % 4 == 0, two K steps per
// aligned 8-byte load; 1: even group count, one aligned dword per K step; 0: 2-byte loads.
template <int WAVES, int KB, int SMODE>
__global__ __launch_bounds__(WAVES * 64) void mfma_kernel(
    const uint4 *__restrict__ w, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint2 *__restrict__ xe,
    const uint2 *__restrict__ xo, const float *__restrict__ xsum, float *__restrict__ y,
    int out_dim, int in_dim, int nb)
{
    extern __shared__ uint4 lds[];
    const int m = blockIdx.y;
    const int C = in_dim >> 5;
    const int groups = in_dim >> 6;
    const int words8 = in_dim >> 3;

    // Stage activations (pair layout) and per-group sums xsg[g][16] * 2^-24. Called after
    // each wave has issued its first weight loads, so the two latencies overlap.
    auto stage = [&]() {
        constexpr int TH = WAVES * 64;
        const size_t xrow0 = (size_t)m * nb;
        const uint2 *xe_m = xe + xrow0 * words8;
        const uint2 *xo_m = xo + xrow0 * words8;
        const float *xsum_m = xsum + xrow0 * C;
        const int units = nb * C * 4;
        // each round issues all of its loads before any LDS write: one memory round trip
        for (int base = threadIdx.x; base < units; base += 4 * TH) {
            uint2 e[4], o[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int u = min(base + i * TH, units - 1);
                const int r = u / (C * 4), cj = u - r * (C * 4);
                e[i] = xe_m[(size_t)r * words8 + cj];
                o[i] = xo_m[(size_t)r * words8 + cj];
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int u = base + i * TH;
                if (u < units) {
                    const int r = u / (C * 4), cj = u - r * (C * 4);
                    lds[x_unit(r, cj >> 2, cj & 3, C)] = make_pairs(e[i], o[i]);
                }
            }
        }
        float *xsw = reinterpret_cast<float *>(lds + nb * C * 4);
        for (int u = threadIdx.x; u < groups * 16; u += TH) {
            const int g = u >> 4, r = u & 15;
            const int rr = min(r, nb - 1);
            const float a = xsum_m[(size_t)rr * C + 2 * g], b = xsum_m[(size_t)rr * C + 2 * g + 1];
            xsw[u] = r < nb ? (a + b) * kTwoM24 : 0.0f;
        }
        __syncthreads();
    };
    const float4_t *xsg = reinterpret_cast<const float4_t *>(lds + nb * C * 4);

    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int q = lane >> 4;
    const int wave_steps = (out_dim + 15) >> 4;
    const int wstride = gridDim.x * WAVES;
    const int ksteps = (C + 3) >> 2;           // K steps of 4 chunks (2 groups)
    const int nbatch = (ksteps + KB - 1) / KB;  // loads are issued KB K steps at a time

    const uint4 *w_m = w + (size_t)m * out_dim * C;
    const uint16_t *s_m = scales + (size_t)m * out_dim * groups;
    const uint16_t *b_m = biases + (size_t)m * out_dim * groups;
    float *y_m = y + (size_t)m * nb * out_dim;
    const bool xrow_live = n < nb;

    // One batch = KB K steps: per lane one 16-byte chunk of codes and the scale and bias
    // pairs of the step's two groups. Loads are unconditional -- indices past the end are
    // clamped to the last chunk, group or K step, whose duplicates are never consumed (a
    // guarded load would make the compiler wait for it before issuing the next one).
    uint4 cw[KB];
    uint32_t sv[KB], bv[KB];
    auto load = [&](const uint4 *wr, const uint16_t *sr, const uint16_t *br, int bt) {
#pragma unroll
        for (int kk = 0; kk < KB; kk++) {
            const int ks = min(bt * KB + kk, ksteps - 1);
            cw[kk] = wr[min(4 * ks + q, C - 1)];
        }
        if constexpr (SMODE == 2) {  // group count % 4 == 0: two K steps per 8-byte load
#pragma unroll
            for (int kk = 0; kk < KB; kk += 2) {
                const int ks = min(bt * KB + kk, ksteps - 2);
                const uint2 s2 = *reinterpret_cast<const uint2 *>(sr + 2 * ks);
                const uint2 b2 = *reinterpret_cast<const uint2 *>(br + 2 * ks);
                sv[kk] = s2.x;
                sv[kk + 1] = s2.y;
                bv[kk] = b2.x;
                bv[kk + 1] = b2.y;
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < KB; kk++) {
                const int g0 = 2 * min(bt * KB + kk, ksteps - 1);  // < groups
                if constexpr (SMODE == 1) {  // even group count: one dword per group pair
                    sv[kk] = *reinterpret_cast<const uint32_t *>(sr + g0);
                    bv[kk] = *reinterpret_cast<const uint32_t *>(br + g0);
                } else {
                    const int g1 = min(g0 + 1, groups - 1);
                    sv[kk] = (uint32_t)sr[g0] | ((uint32_t)sr[g1] << 16);
                    bv[kk] = (uint32_t)br[g0] | ((uint32_t)br[g1] << 16);
                }
            }
        }
    };

    // Every wave of the block takes part in the staging barrier exactly once, after its
    // first weight loads are in flight; waves with no row step stage before leaving.
    bool staged = false;
    for (int ws = blockIdx.x * WAVES + (threadIdx.x >> 6); ws < wave_steps; ws += wstride) {
        asm volatile("" ::: "memory");
        const int row = min(ws * 16 + n, out_dim - 1);
        const uint4 *wr = w_m + (size_t)row * C;
        const uint16_t *sr = s_m + (size_t)row * groups;
        const uint16_t *br = b_m + (size_t)row * groups;
        float4_t acc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        for (int bt = 0; bt < nbatch; bt++) {
            load(wr, sr, br, bt);
            if (!staged) {
                stage();
                staged = true;
            }
#pragma unroll
            for (int kk = 0; kk < KB; kk++) {
                const int ks = bt * KB + kk;
                if (ks < ksteps) {  // uniform; a predicated body keeps the loop unrollable
                // 4x4 transpose across lane groups: afterwards R[i] = word q of chunk 4ks+i
                uint32_t R[4] = {cw[kk].x, cw[kk].y, cw[kk].z, cw[kk].w};
                auto p = __builtin_amdgcn_permlane32_swap(R[0], R[2], false, false);
                R[0] = p[0];
                R[2] = p[1];
                p = __builtin_amdgcn_permlane32_swap(R[1], R[3], false, false);
                R[1] = p[0];
                R[3] = p[1];
                p = __builtin_amdgcn_permlane16_swap(R[0], R[1], false, false);
                R[0] = p[0];
                R[1] = p[1];
                p = __builtin_amdgcn_permlane16_swap(R[2], R[3], false, false);
                R[2] = p[0];
                R[3] = p[1];
#pragma unroll
                for (int gi = 0; gi < 2; gi++) {
                    const int g = 2 * ks + gi;
                    if (g < groups) {  // uniform: only the last K step can be half
                    float4_t d = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int h = 0; h < 2; h++) {
                        const int c = 4 * ks + 2 * gi + h;
                        const uint4 xa =
                            xrow_live ? lds[x_unit(n, c, q, C)] : uint4{0u, 0u, 0u, 0u};
                        const uint32_t wd = R[2 * gi + h];
                        uint4 bu;
                        bu.x = wd & 0x000F000Fu;
                        bu.y = (wd >> 4) & 0x000F000Fu;
                        bu.z = (wd >> 8) & 0x000F000Fu;
                        bu.w = (wd >> 12) & 0x000F000Fu;
                        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(half8_t, xa), __builtin_bit_cast(half8_t, bu), d,
                            0, 0, 0);
                    }
                    const float4_t xs4 = xsg[g * 4 + q];
                    const float s = bf16_to_f32(gi ? sv[kk] >> 16 : sv[kk] & 0xFFFFu);
                    const float b = bf16_to_f32(gi ? bv[kk] >> 16 : bv[kk] & 0xFFFFu);
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        acc[i] = __builtin_fmaf(s, d[i], __builtin_fmaf(b, xs4[i], acc[i]));
                    }
                }
                }
            }
        }
        // D layout: lane (n, q) holds activation rows 4q..4q+3 of output row n
        const int orow = ws * 16 + n;
        if (orow < out_dim) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = 4 * q + i;
                if (r < nb) y_m[(size_t)r * out_dim + orow] = acc[i] * kTwo24;
            }
        }
    }
    if (!staged) stage();
}

typedef void (*MfmaFn)(const uint4 *, const uint16_t *, const uint16_t *, const uint2 *,
                       const uint2 *, const float *, float *, int, int, int);

template <int WAVES, int KB>
static MfmaFn pick_smode(int groups)
{
    if (groups % 4 == 0 && KB % 2 == 0) return mfma_kernel<WAVES, KB, 2>;
    if (groups % 2 == 0) return mfma_kernel<WAVES, KB, 1>;
    return mfma_kernel<WAVES, KB, 0>;
}

template <int WAVES>
static MfmaFn pick_kb(int ksteps, int groups, int *kb)
{
    // the smallest batch holding the whole row, else batches of 16 K steps
    if (ksteps <= 1) { *kb = 1; return pick_smode<WAVES, 1>(groups); }
    if (ksteps <= 2) { *kb = 2; return pick_smode<WAVES, 2>(groups); }
    if (ksteps <= 4) { *kb = 4; return pick_smode<WAVES, 4>(groups); }
    if (ksteps <= 5) { *kb = 5; return pick_smode<WAVES, 5>(groups); }
    if (ksteps <= 8) { *kb = 8; return pick_smode<WAVES, 8>(groups); }
    if (ksteps <= 10) { *kb = 10; return pick_smode<WAVES, 10>(groups); }
    if (ksteps <= 12) { *kb = 12; return pick_smode<WAVES, 12>(groups); }
    if (ksteps <= 16) { *kb = 16; return pick_smode<WAVES, 16>(groups); }
    if (ksteps <= 20) { *kb = 20; return pick_smode<WAVES, 20>(groups); }
    *kb = 16;
    return pick_smode<WAVES, 16>(groups);
}

hipError_t launch_mfma(const GemvArgs &a)
{
    const size_t lds = mfma_lds_bytes(a.in_dim, a.nb);
    const int groups = a.in_dim / 64;
    const int ksteps = (a.in_dim / 32 + 3) / 4;
    // one block per CU when two would not fit in the 160 KB of LDS: then 8 waves per block
    const bool big = 2 * lds > kMaxLds;
    int kb = 0;
    MfmaFn fn = big ? pick_kb<8>(ksteps, groups, &kb) : pick_kb<4>(ksteps, groups, &kb);
    const int waves = big ? 8 : 4;
    hipError_t e = ensure_lds(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess) return e;
    const long wave_steps = (a.out_dim + 15) / 16;
    const long blocks_needed = (wave_steps + waves - 1) / waves;
    const long per_cu = std::min<long>(
        Q4MV_MFMA_BLOCKS_PER_CU,
        resident_blocks(reinterpret_cast<const void *>(fn), waves * 64, lds));
    const long cap = std::max(1L, (long)device_cus() * per_cu / a.n_mat);
    const long gx = std::max(1L, std::min(blocks_needed, cap));
    hipLaunchKernelGGL(fn, dim3((unsigned)gx, (unsigned)a.n_mat), dim3(waves * 64), lds,
                       a.stream, reinterpret_cast<const uint4 *>(a.w), a.scales, a.biases,
                       static_cast<const uint2 *>(a.xe), static_cast<const uint2 *>(a.xo),
                       a.xsum, a.y, a.out_dim, a.in_dim, a.nb);
    return hipGetLastError();
}

}  // namespace q4mv_impl
