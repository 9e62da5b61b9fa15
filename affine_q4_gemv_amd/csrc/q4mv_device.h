// Device-side helpers shared by the GEMV kernels of libq4mv (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef Q4MV_DOT2_FIRST_ASM
#define Q4MV_DOT2_FIRST_ASM 1
#endif

namespace q4mv_impl {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

// 2^24 and 2^-24. A code nibble masked into an f16 lane without an exponent is the f16
// subnormal q * 2^-24 (exact); the kernels accumulate in those units and rescale once.
constexpr float kTwo24 = 16777216.0f;
constexpr float kTwoM24 = 5.9604644775390625e-08f;
constexpr float kTwo20 = 1048576.0f;
constexpr float kTwoM20 = 9.5367431640625e-07f;

// Whether either f16 of a pair has magnitude 4096 or more (or is NaN): 16 times it would
// not be finite in f16.
__device__ __forceinline__ int f16x2_big(half2_t p)
{
    const uint32_t v = __builtin_bit_cast(uint32_t, p);
    return (int)((v & 0x7FFFu) >= 0x6C00u) | (int)(((v >> 16) & 0x7FFFu) >= 0x6C00u);
}

// bf16 bit pattern (in the low 16 bits) -> f32: the bits are the high half of the f32.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// Output epilogue of the GEMV: silu(v / div) = t / (1 + e^-t) with t = v / div (the gated
// bottleneck of fn_qmv_silu_b, Constant BATCH_MSL page); div == 0 stores v unchanged. div is a
// kernel argument, so the branch is uniform.
__device__ __forceinline__ float gemv_epilogue(float v, float div)
{
    if (div == 0.0f) return v;
    const float t = v / div;
    return t / (1.0f + expf(-t));
}

// a.lo*b.lo + a.hi*b.hi + c with f16 inputs and f32 accumulation (v_dot2c_f32_f16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b),
                                  c, false);
}

// a.lo*b.lo + a.hi*b.hi with a zero accumulator, as one VOP3P instruction (the builtin with
// c = 0 becomes a move of zero plus v_dot2c). Same operation and rounding as dot2(a, b, 0).
__device__ __forceinline__ float dot2_first(uint32_t a, uint32_t b)
{
#if Q4MV_DOT2_FIRST_ASM
    float r;
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
#else
    return dot2(a, b, 0.0f);
#endif
}

// LDS layout of staged activations ("pair layout").
// For activation row r, chunk c (32 columns) and word J (8 columns 32c+8J .. 32c+8J+7) one
// 16-byte unit holds four f16 pairs
//   P0 = (x0, x4), P1 = (x1, x5), P2 = (x2, x6), P3 = (x3, x7)
// matching how a u32 word of codes is split by masks: (w & 0x000F000F) gives codes 0 and 4,
// (w & 0x00F000F0) codes 1 and 5 (times 16), and the same on w >> 8 gives 2, 6 and 3, 7.
// Units are swizzled so that 8 consecutive chunks (same r, J) or 8 consecutive rows (same
// c, J) land on 8 distinct 16-byte bank quads: no ds_read_b128 bank conflicts in either
// kernel's access pattern.
__device__ __forceinline__ int x_unit(int r, int c, int J, int C)
{
    return (r * C + (c ^ (r & 1))) * 4 + ((J + (c >> 1) + (r >> 1)) & 3);
}

// Build the four pairs of one word from the even/odd f16 streams:
// e = (x0, x2 | x4, x6), o = (x1, x3 | x5, x7) as two u32 each.
__device__ __forceinline__ uint4 make_pairs(uint2 e, uint2 o)
{
    uint4 p;
    p.x = (e.x & 0xFFFFu) | (e.y << 16);
    p.y = (o.x & 0xFFFFu) | (o.y << 16);
    p.z = (e.x >> 16) | (e.y & 0xFFFF0000u);
    p.w = (o.x >> 16) | (o.y & 0xFFFF0000u);
    return p;
}

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// Packed maximum of two pairs of u16 (v_pk_max_u16).
__device__ __forceinline__ uint32_t pkmax_u16(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                   __builtin_bit_cast(u16x2_t, b)));
}

// One 8-column word x0..x7 of f32 activations, as the prep forms it: every value rounded to
// f16 (nearest even), the four consecutive pairs summed in f32 ((float)a + (float)b), and
// those sums added as (s01 + s23) + (s45 + s67). (A v_dot2_f32_f16 against (1, 1) is not a
// substitute for the pair sum: it measured different bits from the f32 addition on pairs
// whose sum must be rounded.) Returns the word in the pair layout
// (x0,x4) (x1,x5) (x2,x6) (x3,x7), the word's sum, and the packed maximum of the f16
// magnitudes' bit patterns (halves: the even and the odd columns).
struct XWord {
    uint4 p;
    float sum;
    uint32_t mag;
};
__device__ __forceinline__ XWord x_word(const float (&f)[8])
{
    uint32_t q[4];
#pragma unroll
    for (int t = 0; t < 4; t++)
        q[t] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)f[2 * t], (_Float16)f[2 * t + 1]});
    float ps[4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
        const half2_t h = __builtin_bit_cast(half2_t, q[t]);
        ps[t] = (float)h[0] + (float)h[1];
    }
    XWord w;
    w.sum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    // bytes of q[0] (x0,x1), q[1] (x2,x3), q[2] (x4,x5), q[3] (x6,x7)
    w.p.x = __builtin_amdgcn_perm(q[2], q[0], 0x05040100u);  // (x0, x4)
    w.p.y = __builtin_amdgcn_perm(q[2], q[0], 0x07060302u);  // (x1, x5)
    w.p.z = __builtin_amdgcn_perm(q[3], q[1], 0x05040100u);  // (x2, x6)
    w.p.w = __builtin_amdgcn_perm(q[3], q[1], 0x07060302u);  // (x3, x7)
    w.mag = pkmax_u16(pkmax_u16(q[0] & 0x7FFF7FFFu, q[1] & 0x7FFF7FFFu),
                      pkmax_u16(q[2] & 0x7FFF7FFFu, q[3] & 0x7FFF7FFFu));
    return w;
}

// Q2/Q3 codes in the Q4 nibble layout. One 32-code chunk (upper words u0, u1; Q3's low-bit
// word l) -> its four Q4 words: Q4 word 2i + j, nibble p is the code of column
// 32c + 16i + 8j + p, whose 2-bit field (Q2, or Q3's upper two bits) sits at bit 4p + 2j of
// upper word i and whose Q3 lowest bit at bit 4p + 2i + j of the low-bit word: a shift and a
// mask per word (Q3: the upper field one bit up, the lowest bit merged below it). The codes
// stay below 8, so every masked nibble field of the Q4 split is a subnormal f16 pattern.
template <int BITS>
__device__ __forceinline__ uint4 lowbit_chunk_to_q4(uint32_t u0, uint32_t u1, uint32_t l)
{
    if constexpr (BITS == 2)
        return uint4{u0 & 0x33333333u, (u0 >> 2) & 0x33333333u, u1 & 0x33333333u,
                     (u1 >> 2) & 0x33333333u};
    else
        return uint4{((u0 << 1) & 0x66666666u) | (l & 0x11111111u),
                     ((u0 >> 1) & 0x66666666u) | ((l >> 1) & 0x11111111u),
                     ((u1 << 1) & 0x66666666u) | ((l >> 2) & 0x11111111u),
                     ((u1 >> 1) & 0x66666666u) | ((l >> 3) & 0x11111111u)};
}

// Whether a packed maximum of f16 magnitude patterns reaches 4096 (or is NaN / inf).
__device__ __forceinline__ int mag_big(uint32_t m)
{
    return (int)((m & 0xFFFFu) >= 0x6C00u) | (int)((m >> 16) >= 0x6C00u);
}

// silu(g) * u in f32 (fn_moe_act_b, Constant BATCH_MSL page): g / (1 + e^-g) * u, with the
// product rounded to f32 before any later conversion. The empty asm keeps the compiler from
// merging the product with a following f32 -> f16 conversion into one mixed-precision FMA
// (v_fma_mixlo_f16), which rounds the exact product to f16 once and so differs from
// f16(f32(product)) when the f32 product falls on an f16 rounding midpoint.
__device__ __forceinline__ float swiglu_f32(float g, float u)
{
    float h = g / (1.0f + expf(-g)) * u;
    asm("" : "+v"(h));
    return h;
}

// One 8-column word of f32 activations for the prep done inside the GEMV: a plain row
// (glu = 0, rows of in_dim values) or a [gate | up] row of 2*in_dim values whose word is
// silu(gate) * up (glu = 1), formed as the SwiGLU prep forms it (swiglu_f32). row points at
// the row's first float4.
__device__ __forceinline__ void xword_load(const float4 *row, int kw, int in_dim, int glu,
                                           float4 (&v)[4])
{
    v[0] = row[2 * kw];
    v[1] = row[2 * kw + 1];
    if (glu) {
        v[2] = row[(in_dim >> 2) + 2 * kw];
        v[3] = row[(in_dim >> 2) + 2 * kw + 1];
    }
}

__device__ __forceinline__ void xword_values(const float4 (&v)[4], int glu, float (&f)[8])
{
    const float g[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
    if (glu) {
        const float u[8] = {v[2].x, v[2].y, v[2].z, v[2].w, v[3].x, v[3].y, v[3].z, v[3].w};
#pragma unroll
        for (int t = 0; t < 8; t++) f[t] = swiglu_f32(g[t], u[t]);
    } else {
#pragma unroll
        for (int t = 0; t < 8; t++) f[t] = g[t];
    }
}

// DPP helpers (row = 16 lanes). quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over an aligned group of G = 2^log2g lanes. Every lane of the group ends with the same
// bits (each step adds a value to its partner's value; IEEE addition commutes), and the
// order of additions depends only on G, so a given row always reduces identically. The
// steps past log2g add +0.0 instead of branching: straight-line code keeps the compiler from
// splitting (and reordering work around) the caller's loop body.
template <int LOG2G>
__device__ __forceinline__ float group_sum_ct(float v)
{
    if constexpr (LOG2G >= 1) v += dpp<0xB1>(v);
    if constexpr (LOG2G >= 2) v += dpp<0x4E>(v);
    if constexpr (LOG2G >= 3) v += dpp<0x141>(v);
    if constexpr (LOG2G >= 4) v += dpp<0x140>(v);
    if constexpr (LOG2G >= 5) v += __shfl_xor(v, 16, 64);
    if constexpr (LOG2G >= 6) v += __shfl_xor(v, 32, 64);
    return v;
}

// Runtime-G form of group_sum_ct (same additions in the same order).
__device__ __forceinline__ float group_sum(float v, int log2g)
{
    v += log2g >= 1 ? dpp<0xB1>(v) : 0.0f;
    v += log2g >= 2 ? dpp<0x4E>(v) : 0.0f;
    v += log2g >= 3 ? dpp<0x141>(v) : 0.0f;
    v += log2g >= 4 ? dpp<0x140>(v) : 0.0f;
    const float a = __shfl_xor(v, 16, 64);
    v += log2g >= 5 ? a : 0.0f;
    const float b = __shfl_xor(v, 32, 64);
    v += log2g >= 6 ? b : 0.0f;
    return v;
}

}  // namespace q4mv_impl
