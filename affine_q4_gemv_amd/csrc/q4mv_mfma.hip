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
// Loads: lane (n, q) (n = lane % 16, q = lane / 16) reads 16 bytes = one whole chunk
// (4 + 4q of a 4-chunk K step) of output row n, so each row is read 64 contiguous bytes
// at a time. The MFMA wants lane (n, q) to hold word q of one chunk instead, so the four
// lane groups exchange words with a 4x4 transpose built from v_permlane32_swap and
// v_permlane16_swap (gfx950).
#include "q4mv_device.h"
#include "q4mv_internal.h"

#include <algorithm>

namespace q4mv_impl {

template <int WAVES, int T>
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

    // ---- stage: activations (pair layout) and per-group sums xsg[g][16] * 2^-24
    {
        const size_t xrow0 = (size_t)m * nb;
        const uint2 *xe_m = xe + xrow0 * words8;
        const uint2 *xo_m = xo + xrow0 * words8;
        const int units = nb * C * 4;
        for (int u = threadIdx.x; u < units; u += WAVES * 64) {
            const int r = u / (C * 4);
            const int cj = u - r * (C * 4);
            lds[x_unit(r, cj >> 2, cj & 3, C)] =
                make_pairs(xe_m[(size_t)r * words8 + cj], xo_m[(size_t)r * words8 + cj]);
        }
        float *xsg = reinterpret_cast<float *>(lds + nb * C * 4);
        const float *xsum_m = xsum + xrow0 * C;
        for (int u = threadIdx.x; u < groups * 16; u += WAVES * 64) {
            const int g = u >> 4, r = u & 15;
            xsg[u] = r < nb ? (xsum_m[(size_t)r * C + 2 * g] + xsum_m[(size_t)r * C + 2 * g + 1]) *
                                  kTwoM24
                            : 0.0f;
        }
    }
    __syncthreads();
    const float4_t *xsg = reinterpret_cast<const float4_t *>(lds + nb * C * 4);

    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int q = lane >> 4;
    const int rows_per_wave = 16 * T;
    const int wave_steps = (out_dim + rows_per_wave - 1) / rows_per_wave;
    const int wstride = gridDim.x * WAVES;
    const int ksteps = (C + 3) >> 2;

    const uint4 *w_m = w + (size_t)m * out_dim * C;
    const uint16_t *s_m = scales + (size_t)m * out_dim * groups;
    const uint16_t *b_m = biases + (size_t)m * out_dim * groups;
    float *y_m = y + (size_t)m * nb * out_dim;
    const bool xrow_live = n < nb;

    for (int ws = blockIdx.x * WAVES + (threadIdx.x >> 6); ws < wave_steps; ws += wstride) {
        int row[T];
        float4_t acc[T];
#pragma unroll
        for (int t = 0; t < T; t++) {
            row[t] = min(ws * rows_per_wave + t * 16 + n, out_dim - 1);
            acc[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
        // prefetch K step 0
        uint4 cw[T];
        uint32_t sv[T][2], bv[T][2];
        auto load = [&](int ks) {
            const int c = 4 * ks + q;
            const int g0 = 2 * ks;
            const bool g1 = g0 + 1 < groups;
#pragma unroll
            for (int t = 0; t < T; t++) {
                cw[t] = c < C ? w_m[(size_t)row[t] * C + c] : uint4{0u, 0u, 0u, 0u};
                const uint16_t *sr = s_m + (size_t)row[t] * groups;
                const uint16_t *br = b_m + (size_t)row[t] * groups;
                sv[t][0] = sr[g0];
                bv[t][0] = br[g0];
                sv[t][1] = g1 ? sr[g0 + 1] : 0u;
                bv[t][1] = g1 ? br[g0 + 1] : 0u;
            }
        };
        load(0);
        for (int ks = 0; ks < ksteps; ks++) {
            uint32_t R[T][4];
            uint32_t sc[T][2], bc[T][2];
#pragma unroll
            for (int t = 0; t < T; t++) {
                R[t][0] = cw[t].x;
                R[t][1] = cw[t].y;
                R[t][2] = cw[t].z;
                R[t][3] = cw[t].w;
                sc[t][0] = sv[t][0];
                sc[t][1] = sv[t][1];
                bc[t][0] = bv[t][0];
                bc[t][1] = bv[t][1];
            }
            if (ks + 1 < ksteps) load(ks + 1);
            // 4x4 transpose across lane groups: afterwards R[t][i] = word q of chunk 4ks+i
#pragma unroll
            for (int t = 0; t < T; t++) {
                auto p = __builtin_amdgcn_permlane32_swap(R[t][0], R[t][2], false, false);
                R[t][0] = p[0];
                R[t][2] = p[1];
                p = __builtin_amdgcn_permlane32_swap(R[t][1], R[t][3], false, false);
                R[t][1] = p[0];
                R[t][3] = p[1];
                p = __builtin_amdgcn_permlane16_swap(R[t][0], R[t][1], false, false);
                R[t][0] = p[0];
                R[t][1] = p[1];
                p = __builtin_amdgcn_permlane16_swap(R[t][2], R[t][3], false, false);
                R[t][2] = p[0];
                R[t][3] = p[1];
            }
#pragma unroll
            for (int gi = 0; gi < 2; gi++) {
                const int g = 2 * ks + gi;
                if (g >= groups) break;  // uniform: only the last K step can be half
                half8_t A[2];
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const int c = 4 * ks + 2 * gi + h;
                    const uint4 p = xrow_live ? lds[x_unit(n, c, q, C)] : uint4{0u, 0u, 0u, 0u};
                    A[h] = __builtin_bit_cast(half8_t, p);
                }
                const float4_t xs4 = xsg[g * 4 + q];
#pragma unroll
                for (int t = 0; t < T; t++) {
                    float4_t d = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int h = 0; h < 2; h++) {
                        const uint32_t wd = R[t][2 * gi + h];
                        uint4 bu;
                        bu.x = wd & 0x000F000Fu;
                        bu.y = (wd >> 4) & 0x000F000Fu;
                        bu.z = (wd >> 8) & 0x000F000Fu;
                        bu.w = (wd >> 12) & 0x000F000Fu;
                        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            A[h], __builtin_bit_cast(half8_t, bu), d, 0, 0, 0);
                    }
                    const float s = bf16_to_f32(sc[t][gi]);
                    const float b = bf16_to_f32(bc[t][gi]);
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        acc[t][i] = __builtin_fmaf(s, d[i], __builtin_fmaf(b, xs4[i], acc[t][i]));
                }
            }
        }
        // D layout: lane (n, q) holds activation rows 4q..4q+3 of output row n
#pragma unroll
        for (int t = 0; t < T; t++) {
            const int orow = ws * rows_per_wave + t * 16 + n;
            if (orow < out_dim) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int r = 4 * q + i;
                    if (r < nb) y_m[(size_t)r * out_dim + orow] = acc[t][i] * kTwo24;
                }
            }
        }
    }
}

typedef void (*MfmaFn)(const uint4 *, const uint16_t *, const uint16_t *, const uint2 *,
                       const uint2 *, const float *, float *, int, int, int);

hipError_t launch_mfma(const GemvArgs &a)
{
    const size_t lds = mfma_lds_bytes(a.in_dim, a.nb);
    constexpr int T = 2;
    // one block per CU when two would not fit in the 160 KB of LDS: then use 16 waves
    const bool big = 2 * lds > 160 * 1024;
    MfmaFn fn = big ? mfma_kernel<16, T> : mfma_kernel<4, T>;
    const int waves = big ? 16 : 4;
    hipError_t e = ensure_lds(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess) return e;
    const long wave_steps = (a.out_dim + 16 * T - 1) / (16 * T);
    const long blocks_needed = (wave_steps + waves - 1) / waves;
    const long per_cu = big ? 1 : std::max(1L, std::min(4L, (long)(160 * 1024 / lds)));
    const long cap = std::max(1L, (long)device_cus() * per_cu / a.n_mat);
    const long gx = std::max(1L, std::min(blocks_needed, cap));
    hipLaunchKernelGGL(fn, dim3((unsigned)gx, (unsigned)a.n_mat), dim3(waves * 64), lds,
                       a.stream, reinterpret_cast<const uint4 *>(a.w), a.scales, a.biases,
                       static_cast<const uint2 *>(a.xe), static_cast<const uint2 *>(a.xo),
                       a.xsum, a.y, a.out_dim, a.in_dim, a.nb);
    return hipGetLastError();
}

}  // namespace q4mv_impl
