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

template <int NB, int ROWS, int CPL>
__global__ __launch_bounds__(kValuThreads) void valu_kernel(
    const uint4 *__restrict__ w, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint2 *__restrict__ xe,
    const uint2 *__restrict__ xo, const float *__restrict__ xsum, float *__restrict__ y,
    int out_dim, int in_dim, int nb_total, int r0, int log2g, int cpl_rt)
{
    extern __shared__ uint4 lds[];
    constexpr bool XREG = CPL > 0 && NB * CPL <= 4;
    const int m = blockIdx.y;
    const int C = in_dim >> 5;
    const int groups = in_dim >> 6;
    const int words8 = in_dim >> 3;  // uint2 units (4 halves) per activation row

    // ---- stage activation rows r0 .. r0+NB-1 of matrix m (pair layout + scaled sums)
    {
        const size_t xrow0 = (size_t)m * nb_total + r0;
        const uint2 *xe_m = xe + xrow0 * words8;
        const uint2 *xo_m = xo + xrow0 * words8;
        const int units = NB * C * 4;
        for (int u = threadIdx.x; u < units; u += kValuThreads) {
            const int r = u / (C * 4);
            const int cj = u - r * (C * 4);
            lds[x_unit(r, cj >> 2, cj & 3, C)] =
                make_pairs(xe_m[(size_t)r * words8 + cj], xo_m[(size_t)r * words8 + cj]);
        }
        float *xs = reinterpret_cast<float *>(lds + NB * C * 4);
        const float *xsum_m = xsum + xrow0 * C;
        for (int u = threadIdx.x; u < NB * C; u += kValuThreads) xs[u] = xsum_m[u] * kTwoM24;
    }
    __syncthreads();
    const float *xs = reinterpret_cast<const float *>(lds + NB * C * 4);

    const int lane = threadIdx.x & 63;
    const int G = 1 << log2g;
    const int j = lane & (G - 1);
    const int grp = lane >> log2g;
    const int rows_per_wave = (64 >> log2g) * ROWS;
    const int wave_steps = (out_dim + rows_per_wave - 1) / rows_per_wave;
    const int wstride = gridDim.x * (kValuThreads / 64);
    const int cpl = CPL > 0 ? CPL : cpl_rt;

    const uint4 *w_m = w + (size_t)m * out_dim * C;
    const uint16_t *s_m = scales + (size_t)m * out_dim * groups;
    const uint16_t *b_m = biases + (size_t)m * out_dim * groups;
    float *y_m = y + ((size_t)m * nb_total + r0) * out_dim;

    // activations in registers for the whole kernel when they fit
    uint4 xr[XREG ? CPL : 1][XREG ? NB : 1][4];
    float xsr[XREG ? CPL : 1][XREG ? NB : 1];
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

    if constexpr (CPL > 0) {
        // ---- fully unrolled chunk loop: all loads of a step are issued before any use
        for (int ws = blockIdx.x * (kValuThreads / 64) + (threadIdx.x >> 6); ws < wave_steps;
             ws += wstride) {
            // Compiler fence: keeps the per-step LDS activation reads inside the loop (hoisting
            // them all out of it multiplies register use and spills).
            asm volatile("" ::: "memory");
            uint4 cc[ROWS][CPL];
            uint32_t sc[ROWS][CPL], bc[ROWS][CPL];
#pragma unroll
            for (int t = 0; t < ROWS; t++) {
                const int row = min(ws * rows_per_wave + grp * ROWS + t, out_dim - 1);
                const uint4 *wr = w_m + (size_t)row * C;
                const uint16_t *sr = s_m + (size_t)row * groups;
                const uint16_t *br = b_m + (size_t)row * groups;
#pragma unroll
                for (int k = 0; k < CPL; k++) {
                    const int c = j + (k << log2g);
                    cc[t][k] = wr[c];
                    sc[t][k] = sr[c >> 1];
                    bc[t][k] = br[c >> 1];
                }
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
                if constexpr (NB > 1) asm volatile("" ::: "memory");
                uint32_t h[ROWS][4][4];
#pragma unroll
                for (int t = 0; t < ROWS; t++) {
                    const uint32_t wd[4] = {cc[t][k].x, cc[t][k].y, cc[t][k].z, cc[t][k].w};
#pragma unroll
                    for (int J = 0; J < 4; J++) {
                        const uint32_t w8 = wd[J] >> 8;
                        h[t][J][0] = wd[J] & 0x000F000Fu;
                        h[t][J][1] = wd[J] & 0x00F000F0u;
                        h[t][J][2] = w8 & 0x000F000Fu;
                        h[t][J][3] = w8 & 0x00F000F0u;
                    }
                }
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
                    for (int t = 0; t < ROWS; t++) {
                        float ae = 0.0f, ao = 0.0f;
#pragma unroll
                        for (int J = 0; J < 4; J++) {
                            ae = dot2(h[t][J][0], xp[J].x, ae);
                            ao = dot2(h[t][J][1], xp[J].y, ao);
                            ae = dot2(h[t][J][2], xp[J].z, ae);
                            ao = dot2(h[t][J][3], xp[J].w, ao);
                        }
                        const float qd = __builtin_fmaf(ao, 0.0625f, ae);
                        acc[t][r] = __builtin_fmaf(bf16_to_f32(sc[t][k]), qd,
                                                   __builtin_fmaf(bf16_to_f32(bc[t][k]), xsv,
                                                                  acc[t][r]));
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < ROWS; t++) {
                const int row = ws * rows_per_wave + grp * ROWS + t;
#pragma unroll
                for (int r = 0; r < NB; r++) {
                    const float v = group_sum(acc[t][r], log2g);
                    if (j == 0 && row < out_dim) y_m[(size_t)r * out_dim + row] = v * kTwo24;
                }
            }
        }
    } else {
        // ---- generic chunk count: runtime loop in batches of 4 chunks
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
                        if (k0 + kk < cpl) {
                            const int c = j + ((k0 + kk) << log2g);
                            cc[t][kk] = w_m[(size_t)rowc[t] * C + c];
                            sc[t][kk] = s_m[(size_t)rowc[t] * groups + (c >> 1)];
                            bc[t][kk] = b_m[(size_t)rowc[t] * groups + (c >> 1)];
                        }
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
                            const uint32_t wd[4] = {cc[t][kk].x, cc[t][kk].y, cc[t][kk].z,
                                                    cc[t][kk].w};
                            float ae = 0.0f, ao = 0.0f;
#pragma unroll
                            for (int J = 0; J < 4; J++) {
                                const uint32_t w8 = wd[J] >> 8;
                                ae = dot2(wd[J] & 0x000F000Fu, xp[J].x, ae);
                                ao = dot2(wd[J] & 0x00F000F0u, xp[J].y, ao);
                                ae = dot2(w8 & 0x000F000Fu, xp[J].z, ae);
                                ao = dot2(w8 & 0x00F000F0u, xp[J].w, ao);
                            }
                            const float qd = __builtin_fmaf(ao, 0.0625f, ae);
                            acc[t][r] = __builtin_fmaf(bf16_to_f32(sc[t][kk]), qd,
                                                       __builtin_fmaf(bf16_to_f32(bc[t][kk]),
                                                                      xsv, acc[t][r]));
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
                    if (j == 0 && row < out_dim) y_m[(size_t)r * out_dim + row] = v * kTwo24;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// host side

typedef void (*ValuFn)(const uint4 *, const uint16_t *, const uint16_t *, const uint2 *,
                       const uint2 *, const float *, float *, int, int, int, int, int, int);

template <int NB, int ROWS>
static ValuFn pick_cpl(int cpl)
{
    switch (cpl) {
    case 1: return valu_kernel<NB, ROWS, 1>;
    case 2: return valu_kernel<NB, ROWS, 2>;
    case 3: return valu_kernel<NB, ROWS, 3>;
    case 4: return valu_kernel<NB, ROWS, 4>;
    case 5: return valu_kernel<NB, ROWS, 5>;
    case 6: return valu_kernel<NB, ROWS, 6>;
    case 7: return valu_kernel<NB, ROWS, 7>;
    default: return valu_kernel<NB, ROWS, 0>;
    }
}

template <int ROWS>
static ValuFn pick_nb(int nb, int cpl)
{
    switch (nb) {
    case 1: return pick_cpl<1, ROWS>(cpl);
    case 2: return pick_cpl<2, ROWS>(cpl);
    case 3: return pick_cpl<3, ROWS>(cpl);
    case 4: return pick_cpl<4, ROWS>(cpl);
    case 5: return pick_cpl<5, ROWS>(cpl);
    case 6: return pick_cpl<6, ROWS>(cpl);
    case 7: return pick_cpl<7, ROWS>(cpl);
    default: return pick_cpl<8, ROWS>(cpl);
    }
}

static hipError_t launch_valu_part(const GemvArgs &a, int rows, int r0, int nbp)
{
    const int log2g = valu_log2g(a.in_dim);
    const int C = a.in_dim / 32;
    const int cpl = C >> log2g;
    ValuFn fn = rows == 2 ? pick_nb<2>(nbp, cpl) : pick_nb<1>(nbp, cpl);
    const size_t lds = (size_t)nbp * C * 64 + (size_t)nbp * C * 4;
    hipError_t e = ensure_lds(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess) return e;
    const int rows_per_wave = (64 >> log2g) * rows;
    const long wave_steps = (a.out_dim + rows_per_wave - 1) / rows_per_wave;
    const long blocks_needed = (wave_steps + 3) / 4;
    // persistent blocks: enough to fill every CU a few times over, shared by the matrices
    const long cap = std::max(1L, (long)device_cus() * 4 / a.n_mat);
    const long gx = std::max(1L, std::min(blocks_needed, cap));
    hipLaunchKernelGGL(fn, dim3((unsigned)gx, (unsigned)a.n_mat), dim3(kValuThreads), lds,
                       a.stream, reinterpret_cast<const uint4 *>(a.w), a.scales, a.biases,
                       static_cast<const uint2 *>(a.xe), static_cast<const uint2 *>(a.xo),
                       a.xsum, a.y, a.out_dim, a.in_dim, a.nb, r0, log2g, cpl);
    return hipGetLastError();
}

hipError_t launch_valu(const GemvArgs &a, int rows)
{
    for (int r0 = 0; r0 < a.nb; r0 += kValuMaxNB) {
        const int nbp = std::min(kValuMaxNB, a.nb - r0);
        hipError_t e = launch_valu_part(a, rows, r0, nbp);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q4mv_impl
