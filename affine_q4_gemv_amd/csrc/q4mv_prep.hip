// Code packing and activation prep kernels of libq4mv.
#include "q4mv_device.h"
#include "q4mv_internal.h"

namespace q4mv_impl {

// One thread per output word: eight code bytes -> eight nibbles, code i of the word at bits
// [4i, 4i+4) (low nibble first).
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint2 *__restrict__ codes,
                                                         uint32_t *__restrict__ w,
                                                         int64_t n_words)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_words) return;
    const uint2 b = codes[i];
    // gather the low nibble of each byte: byte k of b.x -> nibble k, byte k of b.y -> k+4
    uint32_t lo = b.x & 0x0F0F0F0Fu, hi = b.y & 0x0F0F0F0Fu;
    lo = (lo | (lo >> 4)) & 0x00FF00FFu;  // nibbles 0,1 in byte 0; 2,3 in byte 2
    hi = (hi | (hi >> 4)) & 0x00FF00FFu;
    lo = (lo | (lo >> 8)) & 0x0000FFFFu;
    hi = (hi | (hi >> 8)) & 0x0000FFFFu;
    w[i] = lo | (hi << 16);
}

// Low-bit pack (the stores behind fn_q2_rows_h / fn_q3_rows_h on the Constant BATCH_MSL page):
// one thread per (row, 32-code chunk). The code kept is the 4-bit code's top BITS bits;
// column 16i + 8u + p of the chunk (u < 2, p < 8) goes to bit 4p + 2u of word i (Q2 word, or
// Q3 upper-two-bit word), and for Q3 its lowest bit to bit 4p + 2i + u of the chunk's
// lowest-bit word. Rows are C*BITS words: Q2 2 words per chunk; Q3 the 2C upper words, then
// the C lowest-bit words.
template <int BITS>
__global__ __launch_bounds__(256) void pack_lowbit_kernel(const uint4 *__restrict__ codes,
                                                          uint32_t *__restrict__ w,
                                                          int64_t n_chunks, int C)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_chunks) return;
    const int64_t row = i / C;
    const int c = (int)(i - row * C);
    uint32_t b[8];
    {
        const uint4 v0 = codes[2 * i], v1 = codes[2 * i + 1];
        b[0] = v0.x; b[1] = v0.y; b[2] = v0.z; b[3] = v0.w;
        b[4] = v1.x; b[5] = v1.y; b[6] = v1.z; b[7] = v1.w;
    }
    uint32_t word[2] = {0u, 0u}, low = 0u;
#pragma unroll
    for (int col = 0; col < 32; col++) {
        const uint32_t q4 = (b[col >> 2] >> (8 * (col & 3))) & 0xFu;
        const uint32_t q = q4 >> (4 - BITS);
        const int wi = col >> 4, u = (col >> 3) & 1, p = col & 7;
        if constexpr (BITS == 2) {
            word[wi] |= q << (4 * p + 2 * u);
        } else {
            word[wi] |= (q >> 1) << (4 * p + 2 * u);
            low |= (q & 1u) << (4 * p + 2 * wi + u);
        }
    }
    // a chunk is BITS consecutive words: Q2 its two words, Q3 its two upper-bit words, then
    // its lowest-bit word
    uint32_t *wr = w + row * C * BITS + (int64_t)c * BITS;
    wr[0] = word[0];
    wr[1] = word[1];
    if constexpr (BITS == 3) wr[2] = low;
}

hipError_t launch_pack_lowbit(int bits, const uint8_t *codes, uint32_t *w, int64_t n_rows,
                              int in_dim, hipStream_t s)
{
    const int C = in_dim / 32;
    const int64_t n_chunks = n_rows * C;
    const int64_t blocks = (n_chunks + 255) / 256;
    auto fn = bits == 2 ? pack_lowbit_kernel<2> : pack_lowbit_kernel<3>;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint4 *>(codes), w, n_chunks, C);
    return hipGetLastError();
}

// Activation prep. One thread per (row, even/odd pair k): x[2k], x[2k+1] -> f16 into
// xe[k], xo[k]; the 16 threads of a 32-column chunk then sum their f16-rounded values.
// in_dim % 64 == 0, so a chunk's 16 threads are one aligned 16-lane DPP row.
__global__ __launch_bounds__(256) void prep_kernel(const float2 *__restrict__ x,
                                                   _Float16 *__restrict__ xe,
                                                   _Float16 *__restrict__ xo,
                                                   float *__restrict__ xsum, int64_t n_pairs)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // n_pairs is a multiple of 32, and blocks hold 256 threads, so a 16-lane row is either
    // entirely inside the range or entirely outside it.
    if (i >= n_pairs) return;
    const float2 v = x[i];
    const _Float16 a = (_Float16)v.x, b = (_Float16)v.y;
    xe[i] = a;
    xo[i] = b;
    float s = (float)a + (float)b;
    s += dpp<0xB1>(s);
    s += dpp<0x4E>(s);
    s += dpp<0x141>(s);
    s += dpp<0x140>(s);
    if ((threadIdx.x & 15) == 0) xsum[i >> 4] = s;
}

// SwiGLU activation fused with the prep of the down projection's input (fn_moe_act_b on the
// Constant BATCH_MSL page): row n of gu holds gate[0..inter) then up[0..inter); h = silu(gate)
// * up in f32 becomes the f16 even/odd streams of an inter-wide activation row, and each
// 32-column chunk gets the sum of its f16-rounded values. One thread per (row, pair k).
__global__ __launch_bounds__(256) void swiglu_prep_kernel(const float2 *__restrict__ gu,
                                                          _Float16 *__restrict__ xe,
                                                          _Float16 *__restrict__ xo,
                                                          float *__restrict__ xsum,
                                                          int64_t n_pairs, int half_inter)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // n_pairs and half_inter are multiples of 32: a 16-lane row is entirely in range or out
    if (i >= n_pairs) return;
    const int64_t row = i / half_inter, k = i - row * half_inter;
    const float2 g = gu[row * (2 * half_inter) + k];               // gate[2k], gate[2k+1]
    const float2 u = gu[row * (2 * half_inter) + half_inter + k];  // up[2k], up[2k+1]
    const float he = swiglu_f32(g.x, u.x);
    const float ho = swiglu_f32(g.y, u.y);
    const _Float16 a = (_Float16)he, b = (_Float16)ho;
    xe[i] = a;
    xo[i] = b;
    float s = (float)a + (float)b;
    s += dpp<0xB1>(s);
    s += dpp<0x4E>(s);
    s += dpp<0x141>(s);
    s += dpp<0x140>(s);
    if ((threadIdx.x & 15) == 0) xsum[i >> 4] = s;
}

hipError_t launch_swiglu_prep(const float *gu, int n_rows, int inter, void *xe, void *xo,
                              float *xsum, hipStream_t s)
{
    const int64_t n_pairs = (int64_t)n_rows * (inter / 2);
    const int64_t blocks = (n_pairs + 255) / 256;
    hipLaunchKernelGGL(swiglu_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const float2 *>(gu), static_cast<_Float16 *>(xe),
                       static_cast<_Float16 *>(xo), xsum, n_pairs, inter / 2);
    return hipGetLastError();
}

// Affine-Q4 quantiser for dense rows, one 16-lane row per 64-wide group. The
// steps are those of the affine 5-bit host codec on the memra-engine qwen4exp_gpu.rs page
// (host_quant_q5_row), with 16 levels and a 64-wide group: min and max of the group,
// d = (max - min) / 15, id = 1 / d (0 when d is 0 or id is not finite),
// q = clamp(round_half_even((w - min) * id), 0, 15), all in f32 with correctly rounded
// division; scale = bf16(d), bias = bf16(min), round to nearest even. Codes go straight into
// the packed layout q4mv reads (code i of a word at bits [4i, 4i+4)).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x)
{
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float row_min(float v)
{
    v = fminf(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
    v = fminf(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fminf(v, dpp<0x141>(v));  // row_half_mirror
    return fminf(v, dpp<0x140>(v));  // row_mirror
}
__device__ __forceinline__ float row_max(float v)
{
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    return fmaxf(v, dpp<0x140>(v));
}

// One 16-lane DPP row per group: lane j of the row holds columns 4j .. 4j+3.
__global__ __launch_bounds__(256) void quantize_kernel(const float4 *__restrict__ wf,
                                                       uint32_t *__restrict__ w,
                                                       uint16_t *__restrict__ scales,
                                                       uint16_t *__restrict__ biases,
                                                       int64_t n_groups)
{
    const int64_t grp = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
    if (grp >= n_groups) return;  // whole 16-lane rows: the DPP below stays inside live rows
    const int j = threadIdx.x & 15;
    const float4 v = wf[grp * 16 + j];
    const float mn = row_min(fminf(fminf(v.x, v.y), fminf(v.z, v.w)));
    const float mx = row_max(fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
    const float d = __fdiv_rn(mx - mn, 15.0f);
    float id = d != 0.0f ? __frcp_rn(d) : 0.0f;
    if (!isfinite(id)) id = 0.0f;
    auto code = [&](float x) {
        return (uint32_t)fminf(fmaxf(rintf((x - mn) * id), 0.0f), 15.0f);
    };
    const uint32_t h = code(v.x) | (code(v.y) << 4) | (code(v.z) << 8) | (code(v.w) << 12);
    // lanes 2i and 2i+1 make word i of the group (codes 8i .. 8i+7)
    const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0xB1, 0xF, 0xF, true);
    if ((j & 1) == 0) w[grp * 8 + (j >> 1)] = h | (other << 16);
    if (j == 0) {
        scales[grp] = (uint16_t)f32_to_bf16_rne(d);
        biases[grp] = (uint16_t)f32_to_bf16_rne(mn);
    }
}

hipError_t launch_quantize(const float *wf, uint32_t *w, uint16_t *scales, uint16_t *biases,
                           int64_t n_rows, int in_dim, hipStream_t s)
{
    const int64_t n_groups = n_rows * (in_dim / 64);
    const int64_t blocks = (n_groups + 15) / 16;  // 16 groups of 16 lanes per block
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const float4 *>(wf), w, scales, biases, n_groups);
    return hipGetLastError();
}

// Routing-weighted combine of expert outputs (the combine of the grouped-expert dispatch on
// the Constant BATCH_MSL page): out[r][o] = sum over u of wmap[r][u] * y[u][r][o], u taken in
// order 0..n_u-1 with one fused multiply-add each. One thread per (r, o).
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y,
                                                      const float *__restrict__ wmap,
                                                      float *__restrict__ out, int n_u, int nb,
                                                      int out_dim)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)nb * out_dim) return;
    const int r = (int)(i / out_dim);
    const int64_t stride = (int64_t)nb * out_dim;
    float acc = 0.0f;
    for (int u = 0; u < n_u; u++) acc = __builtin_fmaf(wmap[(int64_t)r * n_u + u], y[u * stride + i], acc);
    out[i] = acc;
}

hipError_t launch_combine(const float *y, const float *wmap, float *out, int n_u, int nb,
                          int out_dim, hipStream_t s)
{
    const int64_t n = (int64_t)nb * out_dim;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, y,
                       wmap, out, n_u, nb, out_dim);
    return hipGetLastError();
}

hipError_t launch_pack(const uint8_t *codes, uint32_t *w, int64_t n_codes, hipStream_t s)
{
    const int64_t n_words = n_codes / 8;
    const int64_t blocks = (n_words + 255) / 256;
    hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint2 *>(codes), w, n_words);
    return hipGetLastError();
}

hipError_t launch_prep(const float *x, int n_rows, int in_dim, void *xe, void *xo, float *xsum,
                       hipStream_t s)
{
    const int64_t n_pairs = (int64_t)n_rows * (in_dim / 2);
    const int64_t blocks = (n_pairs + 255) / 256;
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const float2 *>(x), static_cast<_Float16 *>(xe),
                       static_cast<_Float16 *>(xo), xsum, n_pairs);
    return hipGetLastError();
}

}  // namespace q4mv_impl
