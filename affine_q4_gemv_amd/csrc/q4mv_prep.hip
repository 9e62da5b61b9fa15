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
    const float he = g.x / (1.0f + expf(-g.x)) * u.x;
    const float ho = g.y / (1.0f + expf(-g.y)) * u.y;
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
