// MFMA kernel of libq4mv: the affine-Q4 GEMV as a real contraction for larger activation
// batches, on gfx950's v_mfma_f32_32x32x16_f16 (D[32][32] += A[32][16] * B[16][32]) or
// v_mfma_f32_16x16x32_f16 (D[16][16] += A[16][32] * B[32][16]).
//
// Operands: A = activations (32 rows = activation rows; rows past nb are never stored), read
// from LDS; B = codes of 32 output rows, unpacked in registers to f16 subnormals q*2^-24
// (exact) by masking nibbles. A wave owns a tile of 32 output rows. For scale group g of row
// n, lane (n, h) (h = lane / 32) takes the 16-byte chunk 2g+h, so the lane pair (n, 0),
// (n, 1) holds the whole group: MFMA j (j = 0..3) takes word j of both chunks, its 16-long K
// slice lies inside one group, and the four MFMAs of a group sum to that group's sum(q*x)
// for every (activation row, output row). A word's eight codes become one B operand: the
// masks give (c0,c4), 16*(c1,c5), (c2,c6), 16*(c3,c7), and the matching activations are
// staged as 16*(x0,x4), (x1,x5), 16*(x2,x6), (x3,x7) (exact in f16 while the staged |x| stay
// below 4096; else (x0,x4), (x1,x5)/16, ..., see the staging), so a single accumulator holds
// 16*sum(q*x). The group's scale and bias are then applied in f32 (the
// per-group fold of fn_q4_rows_h, Constant BATCH_MSL page, quantized_rows section). The
// dequantised weight is never formed (the page's tiled expert GEMM dequantises to f16 tiles
// instead). With 16x16x32 the tile is two 16-row halves: lane (n16, kb) (kb = lane / 16)
// takes words 2kb and 2kb+1 of a group for row n16 of each half, one word per MFMA, and the
// same two words' activations of activation row n16 (rows 0..15 fill the A operand, half
// the A reads of the 32-row shape); two MFMAs per half and group.
//
// Loads: a wave's work unit is (tile, quad) = 32 rows x 4 scale groups (128 bytes of codes
// per row). It is read from HBM as whole 128-byte lines (8 lanes per row, 8 rows per load
// instruction), written to a per-wave LDS scratch, and read back in the MFMA operand layout;
// the next unit's loads are issued right after the scratch writes, so they are in flight
// while the current unit computes. Scales and biases (lanes 0..31 a row's scales, 32..63
// its biases) are the costly part of the load stream: each lane reads a different row, so
// one instruction touches dozens of cache lines. Where the layout allows, one 16-byte load
// covers two quads and is made only by the unit that starts the pair; else 8 bytes per unit.
//
// Work split: KS waves (a tile group) share one 32-row tile; with KS > 2 they take
// interleaved quads (wave q: q, q+KS, ...), so at each step they read adjacent pieces of
// every row, else contiguous ranges (which the paired scale loads need). Their partial sums
// meet in LDS and are added in a fixed order (part 0 + 1 + ...), so results do not depend
// on the grid. A block holds WPB / KS tile groups and strides over tiles.
#include "q4mv_device.h"
#include "q4mv_internal.h"

#include <algorithm>

// Launch shape (compile-time tunables, measured on MI355X): the cap on blocks per CU and the
// tile counts below which the K-split is 4 and 8 (2 above).
#ifndef Q4MV_MFMA_KS4_BELOW
#define Q4MV_MFMA_KS4_BELOW 1024
#endif
#ifndef Q4MV_MFMA_KS8_BELOW
#define Q4MV_MFMA_KS8_BELOW 256
#endif
#ifndef Q4MV_MFMA_KS_BIG
#define Q4MV_MFMA_KS_BIG 2
#endif
#ifndef Q4MV_MFMA_NT
#define Q4MV_MFMA_NT 1
#endif
#ifndef Q4MV_MFMA_BALANCE
#define Q4MV_MFMA_BALANCE 0
#endif
// The KS waves of a tile take interleaved quads (wave q: q, q+KS, ...) instead of
// contiguous ranges when the K-split is above 2 (measured faster for small tile counts).
#ifndef Q4MV_MFMA_INTERLEAVE
#define Q4MV_MFMA_INTERLEAVE 1
#endif
// 16-byte scale and bias loads (one per two quads) where the layout allows and the K-split
// is at most SB16_MAX_KS.
#ifndef Q4MV_MFMA_SB16
#define Q4MV_MFMA_SB16 1
#endif
#ifndef Q4MV_MFMA_SB16_MAX_KS
#define Q4MV_MFMA_SB16_MAX_KS 2
#endif
// Matrix-core shape: 16x16x32 (two 16-row output halves per 32-row tile; activation rows
// 0..15 in one operand) for many tiles (at least KS4_BELOW) with K-split at most 2 and
// nb outside 5..8, else 32x32x16 (activation rows padded to 32): each measured faster
// (LM head NB 4 and 16 by about 2%; NB 8 and the short expert rows slower).
#ifndef Q4MV_MFMA_MF16
#define Q4MV_MFMA_MF16 1
#endif
// The 16x16x32 shape for nb 5..8 as well (two 8-row group slots per accumulation).
#ifndef Q4MV_MFMA_MF16_R8
#define Q4MV_MFMA_MF16_R8 1
#endif
// Short launches (fewer than KS8_BELOW tiles, nb <= 8) whose rows hold 3, 5, 6, 10 or 12
// quads: one quad per wave (K-split = quads).
#ifndef Q4MV_MFMA_KSQ
#define Q4MV_MFMA_KSQ 1
#endif
// nb 5..8 on many tiles: two 4-wave blocks per CU instead of one 8-wave block (the staged
// rows of 8 activations leave room for one 8-wave block): LM head NB 6 44.2 -> 43.6 us,
// NB 8 45.0 -> 44.8 us.
#ifndef Q4MV_MFMA_NB8_WPB4
#define Q4MV_MFMA_NB8_WPB4 1
#endif
// Tile-block scale loads (SBW = 32) where they apply.
#ifndef Q4MV_MFMA_TBS
#define Q4MV_MFMA_TBS 1
#endif
#ifndef Q4MV_MFMA_BLOCKS_PER_CU
#define Q4MV_MFMA_BLOCKS_PER_CU 4
#endif
// Short launches (K-split above 2: one block per CU, registers to spare): each thread loads
// its first words of f32 activations before its weight loads, at most Q4MV_MFMA_XPRE in
// 8-wave blocks. A wave's loads complete in issue order, so staging loads issued after the
// weight loads wait for them.
#ifndef Q4MV_MFMA_XPRE
#define Q4MV_MFMA_XPRE 6
#endif

namespace q4mv_impl {

// Waves per block: 8 (two per SIMD), or 4 when the LDS of 8 does not fit; on short launches
// with one quad per wave, the row's quad count (times two tile groups up to 6 quads).
constexpr int kMfmaWaves = 8;
// Per-wave LDS scratch of one unit: codes 32 rows x 128 B, then scales and biases
// 2 x 32 rows x 8 B, or x 16 B with 16-byte scale loads (in 16-byte units).
constexpr int kScratchUnits = 32 * 8 + 32;
constexpr int scratch_units(int sbw) { return 32 * 8 + (sbw == 32 ? 0 : sbw == 16 ? 64 : 32); }
// Tile-block scales (SBW = 32): each tile group keeps its tile's scales and biases (32 rows x
// groups x 2 arrays of bf16) in an LDS buffer; a lane loads at most kTbPieces 16-byte pieces
// of the next tile's block.
constexpr int kTbPieces = 3;
constexpr int kTbMaxGroups = 48;  // 8 * groups pieces <= 128 lanes x kTbPieces
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// A unit's scales and biases in flight: two dwords (one 8-byte load per lane) or four
// 2-byte values (compact loads).
struct SbRegs { uint32_t v[4]; };

// Low-bit chunks enter through lowbit_to_q4 (q4mv_device.h): the same Q4 nibble words as a
// Q4 chunk, so the rest of the kernel is unchanged.
template <int BITS>
__device__ __forceinline__ u32x4 lowbit_to_q4(const u32x4 v)
{
    const uint4 o = lowbit_chunk_to_q4<BITS>(v[0], v[1], v[2]);
    return u32x4{o.x, o.y, o.z, o.w};
}

// WPB: waves per block. KS: waves per tile (K-split). NB16: activation rows 8..15 are live
// (nb > 8; with MF16 the code is the same, the instance separate). Tile-block MF16 kernels for
// nb <= 8 are held to 128 VGPRs (four waves per SIMD: two 8-wave blocks per CU). SBW: how the scales and biases are loaded: 32 = per tile, the tile's whole
// block (its 32 rows' scales, then their biases: two contiguous runs of 64 * groups bytes)
// read with coalesced 16-byte loads shared by the KS = 2 waves of the tile group, one tile
// ahead, into a per-tile-group LDS buffer (groups % 8 == 0, at most kTbMaxGroups, whole rows,
// 16-byte aligned arrays; in a read-only probe of the LM head's access pattern the scattered
// loads below cost 8 us beyond the codes and this one 4.3 us); else per unit, lanes 0..31 a
// row's scales and lanes 32..63 its biases:
// 16 = one aligned 16-byte load for two quads, made by the unit of the even quad (or the
// first unit of a part) and kept in the scratch for the next (groups % 8 == 0, 16-byte
// aligned arrays; halves the scattered scale loads); 8 = one aligned 8-byte load per quad
// (groups % 4 == 0, 8-byte aligned); 2 = four 2-byte loads with clamped indices.
template <int WPB, int KS, bool NB16, int SBW, bool MF16, int BITS = 4, bool R8 = false,
          int XPRE = 0>
__global__ __launch_bounds__(WPB * 64, (MF16 && SBW == 32 && !NB16 && !R8) ? 4 : 1) void mfma_kernel(
    const uint4 *__restrict__ w, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint2 *__restrict__ xe,
    const uint2 *__restrict__ xo, const float *__restrict__ xsum, float *__restrict__ y,
    int out_dim, int in_dim, int nb, float epi_div, const int *__restrict__ sel,
    int n_bank, int x_shared, const float *__restrict__ xf, int xf_glu, int in_full, int k0,
    int accum)
{
    constexpr int TH = WPB * 64;
    constexpr int TPB = WPB / KS;  // tile groups per block
    constexpr int NACC = (MF16 || NB16) ? 8 : 4;
    extern __shared__ uint4 lds[];
    const int m = blockIdx.y;
    // K slice: columns k0 .. k0+in_dim-1 of rows of in_full columns (in_dim == in_full and
    // k0 == 0 unless the staged activations of the whole row do not fit in LDS); C, groups,
    // quads and the staged layout are the slice's, row strides the full row's
    const int C = in_dim >> 5;
    const int groups = in_dim >> 6;
    const int Cf = in_full >> 5, gf = in_full >> 6, kc0 = k0 >> 5, g0 = k0 >> 6;
    const int words8 = in_full >> 3;
    const int quads = (groups + 3) >> 2;

    // LDS: activations | group sums xsg[g][16] * 2^-24 | partial sums | per-wave scratch.
    // Activation layout: row r, chunk c, word j (columns 32c+8j .. +7) is the 16-byte unit
    // r*RS + 4c + j = (x0,x4) (x1/16,x5/16) (x2,x6) (x3/16,x7/16), the A operand matching the
    // word's B operand. RS = 4C + 1 (odd) puts 8 consecutive rows on 8 distinct bank quads.
    // Lanes of activation rows past nb read row nb - 1 instead: row m of D depends on row m
    // of A only, and rows past nb are never stored, so every A read is unconditional.
    // Partial sums: part[2][TPB][KS-1][NACC][plan] (double-buffered by tile step; plan =
    // the lanes that hold activation rows below nb).
    const int RS = 4 * C + 1;
    float4_t *const xsg_w = reinterpret_cast<float4_t *>(lds + nb * RS);
    // one int per wave for the staging scale vote (16 slots, 64 bytes), two zero units (32
    // bytes: the A operand of rows outside their group slot), then the partial sums
    static_assert(WPB <= 16, "one vote slot per wave");
    int *const vote = reinterpret_cast<int *>(xsg_w + groups * 4);
    int *const zero_units = vote + 16;
    float *const part = reinterpret_cast<float *>(vote + 24);
    // lanes whose accumulators hold activation rows below nb (16x16x32: rows 4kb .. 4kb+3)
    const int plan = MF16 ? 16 * ((nb + 3) >> 2) : 64;
    uint4 *const scratch_all =
        reinterpret_cast<uint4 *>(part + (KS > 1 ? 2 * TPB * (KS - 1) * plan * NACC : 0));

    // Stage activations and group sums. Called after each wave has issued its first weight
    // loads, so the two latencies overlap.
    // Staging scale. A word's codes split into the pairs (c0,c4), 16 (c1,c5), (c2,c6),
    // 16 (c3,c7) (masked nibbles as f16 subnormals). The matching activation pairs are staged
    // as 16 x (even pairs) and x (odd pairs), both exact in f16 while every staged |x| is
    // below 4096, so each product is 16 c x, the group sums are staged times 16 as well, and
    // the store scales by 2^20 (up = true). If a staged |x| reaches 4096 (16 x would
    // overflow), the block stages again with x (even) and x/16 (odd; exact for |x| >= 2^-10,
    // else rounded to the f16 subnormal spacing) and the store scales by 2^24. The choice
    // depends only on the staged rows, so every block of a matrix makes the same one.
    // Thread t takes words (units) t, t + TH, t + 2 TH, ... of the nb * in_dim / 8 staged
    // words; their row and column are advanced incrementally (no division per word). The
    // staging runs after each wave has issued its first weight loads, in rounds (2 words per
    // thread with f32 activations, 4 units with the prepared ones); the next round's loads
    // are issued before the current round is converted and written. On short launches
    // staging f32 rows the first words are loaded ahead of the weight loads (xpre below); on
    // the LM head's launches that measured slower (the registers they hold across those
    // loads cost it its second block per CU).
    const int wrow = in_dim >> 3, words = nb * wrow;
    const int dr = TH / wrow, dk = TH - dr * wrow;  // advance by TH words
    auto adv = [&](int &r, int &kw) __attribute__((always_inline)) {
        r += dr;
        kw += dk;
        if (kw >= wrow) {
            kw -= wrow;
            r++;
        }
    };
    const size_t xrow0 = x_shared ? 0 : (size_t)m * nb;
    const int rs4 = xf_glu ? in_full >> 1 : in_full >> 2;  // float4 per row
    const float4 *const xf_m =
        xf ? reinterpret_cast<const float4 *>(xf) + xrow0 * (size_t)rs4 : nullptr;
    // word (r, kw) of the plain f32 rows (rows past nb read row nb - 1)
    auto fword_ptr = [&](int r, int kw) __attribute__((always_inline)) {
        return xf_m + (size_t)min(r, nb - 1) * rs4 + 2 * ((k0 >> 3) + kw);
    };
    // The words loaded ahead of the weight loads on short launches staging f32 rows: XPRE
    // 1 (plain rows) and 2 ([gate | up] rows) instances; XPRE 0 keeps the staging after the
    // weight loads, which measured faster from the prepared streams (2560 x 2560 NB 4 6.22
    // against 6.43 us). Plain rows: up to 6 words per thread in 8-wave blocks, 4 in 10- and
    // 12-wave blocks (all they need at nb <= 8), 1 in 6-wave blocks (640- and 768-column
    // expert rows), where more registers would keep two blocks off one compute unit
    // (8 x 2560 x 640 NB 4 6.90 -> 6.70 us). [gate | up] rows: a word takes two entries
    // (gate, up): 3, 2 and 1 words.
    constexpr int kXPreWords = XPRE != 1 || KS <= 2 ? 0 : WPB == 6 ? 1
                               : WPB >= 10 && Q4MV_MFMA_XPRE > 4 ? 4 : Q4MV_MFMA_XPRE;
    constexpr int kXPreGlu = XPRE != 2 || KS <= 2 ? 0 : WPB == 6 ? 1
                             : WPB >= 10 && Q4MV_MFMA_XPRE > 4 ? 2 : Q4MV_MFMA_XPRE / 2;
    constexpr int kXPre = XPRE == 2 ? 2 * kXPreGlu : kXPreWords;  // register entries
    const bool xpre_on = kXPreWords > 0 && xf && !xf_glu;
    const bool xpre_glu = kXPreGlu > 0 && xf && xf_glu;
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    // (entries a thread does not load are zeroed: they still pass through the asm
    // statements below, and are never read after them)
    f32x4 xpre[kXPre > 0 ? kXPre : 1][2];
    // Fused prep (xf non-null: f32 activations): the f16 rounding and the chunk sums of
    // q4mv_prepare_x done here with the same additions (pair sums, a balanced tree over a
    // chunk's 16 pairs: each thread adds its word's four pairs, two quad DPP steps add the
    // chunk's four words; then a group's two chunks in order), so the LDS contents are
    // bitwise those staged from q4mv_prepare_x's outputs. A quad of lanes is one chunk, 8
    // lanes one group (words per row are a multiple of 8). With xf_glu the rows are
    // [gate | up] and the values silu(gate) * up (as q4mv_swiglu_prep forms them). Returns
    // whether this thread saw an |x| of 4096 or more.
    auto fstage = [&](bool up) __attribute__((always_inline)) {
        float *xsw = reinterpret_cast<float *>(xsg_w);
        const half2_t sixteen = {(_Float16)16.0f, (_Float16)16.0f};
        const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
        const float sum_scale = up ? kTwoM20 : kTwoM24;
        uint32_t mag = 0;
        // one word: f16 values, chunk sum (a quad of lanes is a chunk) and group sum (8
        // lanes), and its LDS unit r*RS + 4c + j = the pairs (x0,x4) (x1,x5) (x2,x6) (x3,x7)
        // scaled for the staging
        auto fword = [&](int r, int kw, const float (&f)[8]) __attribute__((always_inline)) {
            const XWord xw = x_word(f);
            mag = pkmax_u16(mag, xw.mag);
            float sum = xw.sum;
            sum += dpp<0xB1>(sum);
            sum += dpp<0x4E>(sum);
            const float other = __shfl_xor(sum, 4, 64);  // the group's other chunk
            if ((kw & 7) == 0) xsw[(kw >> 3) * 16 + r] = (sum + other) * sum_scale;
            uint4 u = xw.p;
            if (up) {
                u.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, u.x) * sixteen);
                u.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, u.z) * sixteen);
            } else {
                u.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, u.y) * sixteenth);
                u.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, u.w) * sixteenth);
            }
            lds[r * RS + kw] = u;
        };
        if (xf_glu) {
            // [gate | up] rows: one word per thread at a time (the words loaded ahead first)
            int wi = threadIdx.x;
            if (up && xpre_glu) {
#pragma unroll
                for (int i = 0; i < kXPreGlu; i++) {
                    if (wi < words) {  // uniform per 8 lanes
                        const int r = wi / wrow, kw = wi - r * wrow;
                        const f32x4 g0 = xpre[2 * i][0], g1 = xpre[2 * i][1];
                        const f32x4 u0 = xpre[2 * i + 1][0], u1 = xpre[2 * i + 1][1];
                        const float4 v[4] = {{g0[0], g0[1], g0[2], g0[3]},
                                             {g1[0], g1[1], g1[2], g1[3]},
                                             {u0[0], u0[1], u0[2], u0[3]},
                                             {u1[0], u1[1], u1[2], u1[3]}};
                        float f[8];
                        xword_values(v, 1, f);
                        fword(r, kw, f);
                    }
                    wi += TH;
                }
            }
            for (; wi < words; wi += TH) {  // uniform per 8 lanes
                const int r = wi / wrow, kw = wi - r * wrow;
                float4 v[4];
                xword_load(xf_m + (size_t)r * rs4, (k0 >> 3) + kw, in_full, 1, v);
                float f[8];
                xword_values(v, 1, f);
                fword(r, kw, f);
            }
        } else {
            // plain rows: rounds of 2 words per thread, the next round's loads in flight
            // while the current one is written
            auto fload = [&](const int (&r)[2], const int (&kw)[2], float4 (&v)[2][2])
                __attribute__((always_inline)) {
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    const float4 *p = fword_ptr(r[i], kw[i]);
                    v[i][0] = p[0];
                    v[i][1] = p[1];
                }
            };
            auto fput = [&](const int (&r)[2], const int (&kw)[2], const float4 (&v)[2][2])
                __attribute__((always_inline)) {
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    if (r[i] < nb) {  // uniform per 8 lanes
                        const float f[8] = {v[i][0].x, v[i][0].y, v[i][0].z, v[i][0].w,
                                            v[i][1].x, v[i][1].y, v[i][1].z, v[i][1].w};
                        fword(r[i], kw[i], f);
                    }
                }
            };
            auto next = [&](const int (&r)[2], const int (&kw)[2], int (&rn)[2], int (&kn)[2])
                __attribute__((always_inline)) {
                rn[0] = r[1];
                kn[0] = kw[1];
                adv(rn[0], kn[0]);
                rn[1] = rn[0];
                kn[1] = kn[0];
                adv(rn[1], kn[1]);
            };
            float4 va[2][2], vb[2][2];
            int ra[2], ka[2], rb[2], kb2[2];
            ra[0] = threadIdx.x / wrow;
            ka[0] = threadIdx.x - ra[0] * wrow;
            if (up && xpre_on) {
                // the words loaded ahead first, then the rest in rounds
#pragma unroll
                for (int i = 0; i < kXPreWords; i++) {
                    if (ra[0] < nb) {  // uniform per 8 lanes
                        const float f[8] = {xpre[i][0].x, xpre[i][0].y, xpre[i][0].z,
                                            xpre[i][0].w, xpre[i][1].x, xpre[i][1].y,
                                            xpre[i][1].z, xpre[i][1].w};
                        fword(ra[0], ka[0], f);
                    }
                    adv(ra[0], ka[0]);
                }
            }
            ra[1] = ra[0];
            ka[1] = ka[0];
            adv(ra[1], ka[1]);
            if (ra[0] < nb) fload(ra, ka, va);
            while (ra[0] < nb) {
                next(ra, ka, rb, kb2);
                if (rb[0] < nb) fload(rb, kb2, vb);
                fput(ra, ka, va);
                if (rb[0] >= nb) break;
                next(rb, kb2, ra, ka);
                if (ra[0] < nb) fload(ra, ka, va);
                fput(rb, kb2, vb);
            }
        }
        for (int u = threadIdx.x; u < groups * 16; u += TH)
            if ((u & 15) >= nb) xsw[u] = 0.0f;
        return mag_big(mag);
    };
    // the same from q4mv_prepare_x's outputs (xf null): unit (r, 4c + j) from the even and odd
    // streams, rounds of 4 units per thread
    auto pstage = [&](bool up) __attribute__((always_inline)) {
        const size_t xrow0 = x_shared ? 0 : (size_t)m * nb;
        const uint2 *xe_m = xe + xrow0 * words8 + (k0 >> 3);
        const uint2 *xo_m = xo + xrow0 * words8 + (k0 >> 3);
        const float *xsum_m = xsum + xrow0 * Cf + kc0;
        const half2_t sixteen = {(_Float16)16.0f, (_Float16)16.0f};
        const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
        const float sum_scale = up ? kTwoM20 : kTwoM24;
        uint32_t mag = 0;
        struct PRound { uint2 e[4], o[4]; int r[4], kw[4]; };
        auto ppos = [&](PRound &p, int r, int kw) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                p.r[i] = r;
                p.kw[i] = kw;
                adv(r, kw);
            }
        };
        auto pload = [&](PRound &p) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const size_t at = (size_t)min(p.r[i], nb - 1) * words8 + p.kw[i];
                p.e[i] = xe_m[at];
                p.o[i] = xo_m[at];
            }
        };
        auto pput = [&](const PRound &p) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if (p.r[i] < nb) {
                    uint4 pr = make_pairs(p.e[i], p.o[i]);
                    mag = pkmax_u16(mag, pkmax_u16(pkmax_u16(p.e[i].x & 0x7FFF7FFFu,
                                                              p.e[i].y & 0x7FFF7FFFu),
                                                    pkmax_u16(p.o[i].x & 0x7FFF7FFFu,
                                                              p.o[i].y & 0x7FFF7FFFu)));
                    if (up) {
                        pr.x = __builtin_bit_cast(uint32_t,
                                                  __builtin_bit_cast(half2_t, pr.x) * sixteen);
                        pr.z = __builtin_bit_cast(uint32_t,
                                                  __builtin_bit_cast(half2_t, pr.z) * sixteen);
                    } else {
                        pr.y = __builtin_bit_cast(uint32_t,
                                                  __builtin_bit_cast(half2_t, pr.y) * sixteenth);
                        pr.w = __builtin_bit_cast(uint32_t,
                                                  __builtin_bit_cast(half2_t, pr.w) * sixteenth);
                    }
                    lds[p.r[i] * RS + p.kw[i]] = pr;
                }
            }
        };
        PRound pa, pb;
        {
            const int r0 = threadIdx.x / wrow;
            ppos(pa, r0, threadIdx.x - r0 * wrow);
        }
        if (pa.r[0] < nb) pload(pa);
        while (pa.r[0] < nb) {
            {
                int r = pa.r[3], kw = pa.kw[3];
                adv(r, kw);
                ppos(pb, r, kw);
            }
            if (pb.r[0] < nb) pload(pb);
            pput(pa);
            if (pb.r[0] >= nb) break;
            {
                int r = pb.r[3], kw = pb.kw[3];
                adv(r, kw);
                ppos(pa, r, kw);
            }
            if (pa.r[0] < nb) pload(pa);
            pput(pb);
        }
        float *xsw = reinterpret_cast<float *>(xsg_w);
        for (int u = threadIdx.x; u < groups * 16; u += TH) {
            const int g = u >> 4, r = u & 15;
            const int rr = min(r, nb - 1);
            const float a = xsum_m[(size_t)rr * Cf + 2 * g], b = xsum_m[(size_t)rr * Cf + 2 * g + 1];
            xsw[u] = r < nb ? (a + b) * sum_scale : 0.0f;
        }
        return mag_big(mag);
    };
    // stages with the x16 scale unless a staged |x| reaches 4096; returns the output scale.
    // Each wave writes its own vote (so nothing needs clearing first); after the barrier
    // every thread reads all of them.
    auto stage = [&]() __attribute__((always_inline)) {
        if constexpr (kXPre == 0) {
            if (threadIdx.x < 8) zero_units[threadIdx.x] = 0;
        }
        const int mine = __any(xf ? fstage(true) : pstage(true)) ? 1 : 0;
        if ((threadIdx.x & 63) == 0) vote[threadIdx.x >> 6] = mine;
        __syncthreads();
        int big = 0;
#pragma unroll
        for (int i = 0; i < WPB; i++) big |= vote[i];
        if (!big) return kTwo20;
        if (xf)
            fstage(false);
        else
            pstage(false);
        __syncthreads();
        return kTwo24;
    };
    const float4_t *xsg = xsg_w;

    const int lane = threadIdx.x & 63;
    const int n = lane & 31;  // output row of the tile (B, D); activation row (A)
    const int h = lane >> 5;  // which chunk of the group this lane holds
    // 16x16x32: lane (n16, kb) takes output row n16 of each 16-row half (B, D), activation
    // row n16 (A), K slot kb: words 2kb and 2kb+1 of a group, one per MFMA; D rows
    // 4kb .. 4kb+3
    const int n16 = lane & 15, kb = lane >> 4;
    // wave index, made visibly wave-uniform so everything derived from it lives in SGPRs
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slot = wv / KS;     // tile group of this wave within the block
    const int quarter = wv % KS;  // which part of the quads this wave sums
    // parts split the row on quad boundaries; the unit count per tile comes from the
    // largest part, so it is the same for every wave of the block and every wave meets the
    // per-tile barrier equally often (units past a wave's part are computed with zero
    // scales and biases)
    // (16-byte scale loads pair consecutive quads, so K-splits of 2 or less, where those
    // loads apply, keep contiguous parts whatever the scale load width: the summation order
    // then does not depend on the alignment of the scale arrays)
    constexpr bool kInterleave = Q4MV_MFMA_INTERLEAVE && KS > 2;
    const int q_begin = kInterleave ? quarter : quarter * quads / KS;
    const int q_step = kInterleave ? KS : 1;
    const int q_end = kInterleave ? quads : (quarter + 1) * quads / KS;
    const int nunit = (quads + KS - 1) / KS;
    const int tiles = (out_dim + 31) >> 5;
    const int tstride = gridDim.x * TPB;

    // Rows: a tile covers rows rb .. rb+31 where the last tile is shifted back to end at
    // out_dim (its overlap with the previous tile is recomputed but not stored: every output
    // is stored once, by the tile it belongs to). Only when out_dim < 32 are rows clamped.
    const bool narrow = out_dim < 32;
    // Weights: matrix m, or bank matrix sel[m]. An id outside the bank reads matrix 0 and
    // stores NaN (a NaN divisor makes the epilogue return NaN).
    int e = m;
    if (sel) {
        const int id = sel[m];
        const bool bad = (unsigned)id >= (unsigned)n_bank;
        e = bad ? 0 : id;
        if (bad) epi_div = __builtin_nanf("");
    }
    const uint4 *const w_m = w + (size_t)e * out_dim * Cf;
    // low-bit codes: rows of C * BITS words (Q2: 2 words per chunk; Q3: 2C upper words,
    // then C low-bit words)
    const uint32_t *const wl_m =
        reinterpret_cast<const uint32_t *>(w) + (size_t)e * out_dim * Cf * BITS;
    const uint16_t *const s_m = scales + (size_t)e * out_dim * gf + g0;
    const uint16_t *const b_m = biases + (size_t)e * out_dim * gf + g0;
    float *const y_m = y + (size_t)m * nb * out_dim;
    auto tile_row = [&](int tile) { return narrow ? 0 : min(tile * 32, out_dim - 32); };

    // Loads of one unit (tile, quad qd): load instruction r covers rows 8r .. 8r+7 of the
    // tile, lane l row 8r + l/8 and 16-byte chunk 8*qd + l%8 of it (whole 128-byte lines;
    // chunks past the row end are clamped and their groups masked). Lanes 0..31 load the
    // quad's four scales of row l, lanes 32..63 its four biases.
    const int lr8 = lane >> 3, lc = lane & 7;
    const int sbrow = narrow ? min(lane & 31, out_dim - 1) : (lane & 31);
    const uint16_t *const sb_m = lane < 32 ? s_m : b_m;
    auto load = [&](int tile, int qd, int u, u32x4 (&cw)[4], SbRegs &sb) {
        const int trow = tile_row(tile);
        const int chunk = min(8 * qd + lc, C - 1);
        if constexpr (BITS != 4) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int row = narrow ? min(8 * r + lr8, out_dim - 1) : 8 * r + lr8;
                // a chunk is BITS consecutive words (Q3: two upper-bit words, then the
                // lowest-bit word)
                const uint32_t *wr = wl_m + (size_t)(trow + row) * Cf * BITS + BITS * (kc0 + chunk);
                if constexpr (BITS == 2) {
                    const u32x2 up = *reinterpret_cast<const u32x2 *>(wr);
                    cw[r] = u32x4{up[0], up[1], 0u, 0u};
                } else {
                    cw[r] = u32x4{wr[0], wr[1], wr[2], 0u};
                }
            }
        }
#pragma unroll
        for (int r = 0; r < (BITS == 4 ? 4 : 0); r++) {
            const int row = narrow ? min(8 * r + lr8, out_dim - 1) : 8 * r + lr8;
#if Q4MV_MFMA_NT
            // each 128-byte line is read whole, once: non-temporal
            cw[r] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(w_m) + (size_t)(trow + row) * Cf + kc0 + chunk);
#else
            cw[r] = reinterpret_cast<const u32x4 *>(w_m)[(size_t)(trow + row) * Cf + kc0 + chunk];
#endif
        }
        const uint16_t *srow = sb_m + (size_t)(trow + sbrow) * gf;
        if constexpr (SBW == 32) {
            (void)srow;  // the tile's block is in LDS
        } else if constexpr (SBW == 16) {
            // only units that start a pair load (measured faster than a dummy load)
            if ((qd & 1) == 0 || u == 0) {
                const uint4 v = *reinterpret_cast<const uint4 *>(srow + 4 * (qd & ~1));
                sb.v[0] = v.x;
                sb.v[1] = v.y;
                sb.v[2] = v.z;
                sb.v[3] = v.w;
            }
        } else if constexpr (SBW == 8) {
            const uint2 v = *reinterpret_cast<const uint2 *>(srow + 4 * qd);
            sb.v[0] = v.x;
            sb.v[1] = v.y;
        } else {
            uint32_t v[4];
#pragma unroll
            for (int i = 0; i < 4; i++) v[i] = srow[min(4 * qd + i, groups - 1)];
            sb.v[0] = v[0] | (v[1] << 16);
            sb.v[1] = v[2] | (v[3] << 16);
        }
    };
    // This wave's scratch: codes of row r, chunk slot c at r*8 + (c ^ (r & 7)) (the XOR
    // keeps both the row-major writes and the MFMA-layout reads free of bank conflicts),
    // then scales of rows 0..31 and biases of rows 0..31 as 8-byte (16-byte) entries.
    uint4 *const scratch = scratch_all + wv * scratch_units(SBW);
    uint2 *const sbs = reinterpret_cast<uint2 *>(scratch + 32 * 8);
    // tile-block scales: this tile group's buffer, scales [32][groups] then biases, bf16
    uint4 *const tbuf = scratch_all + WPB * scratch_units(SBW) + slot * 8 * groups;
    const uint16_t *const tbs = reinterpret_cast<const uint16_t *>(tbuf);
    uint4 tb0 = {0u, 0u, 0u, 0u}, tb1 = tb0, tb2 = tb0;  // kTbPieces pieces in flight
    // the block of `tile` into registers: lane l of wave `quarter` takes pieces
    // 64 * quarter + l + 128 i of the 8 * groups (scales, then biases)
    auto tb_load = [&](int tile) __attribute__((always_inline)) {
        if constexpr (SBW == 32) {
            const size_t trow = (size_t)tile_row(min(tile, tiles - 1)) * groups;
            const uint4 *sp = reinterpret_cast<const uint4 *>(s_m + trow);
            const uint4 *bp = reinterpret_cast<const uint4 *>(b_m + trow);
            // every load is made (pieces past the block re-read its last piece), so the
            // registers stay registers and the loads stay in flight
            auto piece = [&](int i) __attribute__((always_inline)) {
                const int pc = min(64 * quarter + lane + 128 * i, 8 * groups - 1);
                return *(pc < 4 * groups ? sp + pc : bp + (pc - 4 * groups));
            };
            static_assert(kTbPieces == 3, "three pieces per lane");
            tb0 = piece(0);
            tb1 = piece(1);
            tb2 = piece(2);
        }
    };
    auto tb_store = [&]() __attribute__((always_inline)) {
        if constexpr (SBW == 32) {
            const int pc = 64 * quarter + lane;
            if (pc < 8 * groups) tbuf[pc] = tb0;
            if (pc + 128 < 8 * groups) tbuf[pc + 128] = tb1;
            if (pc + 256 < 8 * groups) tbuf[pc + 256] = tb2;
        }
    };
    auto put = [&](const u32x4 (&cw)[4], const SbRegs &sb, int qd, int u) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = 8 * r + lr8;
            reinterpret_cast<u32x4 *>(scratch)[row * 8 + (lc ^ (row & 7))] =
                BITS == 4 ? cw[r] : lowbit_to_q4<BITS>(cw[r]);
        }
        if constexpr (SBW == 16) {
            if ((qd & 1) == 0 || u == 0)
                reinterpret_cast<uint4 *>(sbs)[lane] = uint4{sb.v[0], sb.v[1], sb.v[2], sb.v[3]};
        } else if constexpr (SBW != 32) {
            sbs[lane] = uint2{sb.v[0], sb.v[1]};
        }
    };

    // this lane's activation row in LDS (row nb - 1 past nb), offset to its chunk parity
    // 16x16x32 group slots: RG activation rows per slot (4 for nb <= 4, 8 for nb 5..8, 16
    // above), NS slots, ND accumulations per unit and half; sa: the slot of this lane's A
    // rows, kbd: the slot of its D rows
    constexpr int RG = NB16 ? 16 : R8 ? 8 : 4;
    constexpr int NS = 16 / RG, ND = 4 / NS;
    const int sa = n16 / RG, kbd = kb / (RG / 4);
    const uint4 *const xrow = MF16 ? lds + min(n16 % RG, nb - 1) * RS + 2 * kb
                                   : lds + min(n, nb - 1) * RS + 4 * h;
    // 16x16x32: this lane's scratch word offset (8-byte words) of group g4 of a unit, for
    // row n16 (row 16 + n16 is 256 words further on: the XOR swizzle of rows n16 and
    // 16 + n16 is the same)
    int boff[4];
#pragma unroll
    for (int g4 = 0; g4 < 4; g4++)
        boff[g4] = (n16 * 8 + ((2 * g4 + (kb >> 1)) ^ (n16 & 7))) * 2 + (kb & 1);
    // zeros for A rows outside their group's slot
    const uint4 *const zrow = reinterpret_cast<const uint4 *>(zero_units);
    float acc[NACC];
    // Low-bit codes reconstruct at the middle of the 4-bit range each stands for:
    // w = (4q + 1.5) s + b (Q2), (2q + 0.5) s + b (Q3); the fold takes K s and M s + b (formed
    // in f32 with one rounding), as the VALU kernels' low-bit fold does.
    auto midpoint = [](float &s, float &b) {
        if constexpr (BITS != 4) {
            constexpr float kq = BITS == 2 ? 4.0f : 2.0f, km = BITS == 2 ? 1.5f : 0.5f;
            b = __builtin_fmaf(km, s, b);
            s = kq * s;
        }
    };

    // The block walks tile steps in lockstep when KS > 1 (one barrier per tile); with
    // KS = 1 each wave stops on its own.
    auto more = [&](int b) { return KS == 1 ? b + slot < tiles : b < tiles; };
    int base = blockIdx.x * TPB;
    int ui = 0;  // unit of the current tile
    int step = 0;
    auto unit_quad = [&](int u) { return min(q_begin + q_step * u, quads - 1); };

    // Loads run two units ahead: (abase, aui) is the unit the next load fetches, and the
    // two register sets alternate (the loop is unrolled by two so each set is static).
    int abase = base, aui = 0;
    auto advance = [&](int &b, int &u) {
        if (u + 1 == nunit) {
            u = 0;
            b += tstride;
        } else {
            u++;
        }
    };
    u32x4 c0[4], c1[4];
    SbRegs s0, s1;
    if constexpr (kXPre > 0) {
        if (threadIdx.x < 8) zero_units[threadIdx.x] = 0;  // read after the staging barrier
    }
    if (xpre_on) {
        // Issued ahead of the weight loads (a wave's loads complete in issue order, so they
        // wait for nothing else), only as many rounds as the block's words need (uniform).
        // Unconditional within a round (words past the rows re-read row nb - 1), so no
        // branch invites the compiler to convert, and wait for, a word before the next
        // load is issued.
        const int npre = min(kXPreWords, (words + TH - 1) / TH);
        int r = threadIdx.x / wrow, kw = threadIdx.x - r * wrow;
#pragma unroll
        for (int i = 0; i < kXPreWords; i++) {
            if (i < npre) {
                const f32x4 *p = reinterpret_cast<const f32x4 *>(fword_ptr(min(r, nb - 1), kw));
                xpre[i][0] = p[0];
                xpre[i][1] = p[1];
            } else {
                xpre[i][0] = xpre[i][1] = f32x4{};
            }
            adv(r, kw);
        }
    } else if (xpre_glu) {
        // [gate | up] words, as fstage's loop takes them (a clamped row past nb)
        const int npre = min(kXPreGlu, (words + TH - 1) / TH);
        int r = threadIdx.x / wrow, kw = threadIdx.x - r * wrow;
#pragma unroll
        for (int i = 0; i < kXPreGlu; i++) {
            if (i < npre) {
                float4 v[4];
                xword_load(xf_m + (size_t)min(r, nb - 1) * rs4, (k0 >> 3) + kw, in_full, 1, v);
                xpre[2 * i][0] = f32x4{v[0].x, v[0].y, v[0].z, v[0].w};
                xpre[2 * i][1] = f32x4{v[1].x, v[1].y, v[1].z, v[1].w};
                xpre[2 * i + 1][0] = f32x4{v[2].x, v[2].y, v[2].z, v[2].w};
                xpre[2 * i + 1][1] = f32x4{v[3].x, v[3].y, v[3].z, v[3].w};
            } else {
                xpre[2 * i][0] = xpre[2 * i][1] = f32x4{};
                xpre[2 * i + 1][0] = xpre[2 * i + 1][1] = f32x4{};
            }
            adv(r, kw);
        }
    } else {
#pragma unroll
        for (int i = 0; i < kXPre; i++) xpre[i][0] = xpre[i][1] = f32x4{};
    }
    // the first tile's scale block (visible to the tile group after the staging barrier)
    tb_load(base + slot);  // (a tile past the end re-reads the last one: unused)
    // With words loaded ahead the first unit's loads are unconditional (a tile past the end
    // re-reads the last tile's rows, unused), so the waits below know which loads follow
    // the words on every path.
    if (kXPre > 0 || more(abase)) load(abase + slot, unit_quad(aui), aui, c0, s0);
    advance(abase, aui);
    // The words loaded ahead are used from here on (the empty asm statements: the compiler
    // waits for them here, with only the first unit's loads issued after them, and not
    // later, where loads issued on only some paths would make it wait for weights too).
    // The next unit's loads follow. (Ahead of that wait, they measured slower: its waits
    // then also covered the first unit's loads on some paths.)
#pragma unroll
    for (int i = 0; i < kXPre; i++)
        asm volatile("; staged words" : "+v"(xpre[i][0]), "+v"(xpre[i][1]));
    if (more(abase)) load(abase + slot, unit_quad(aui), aui, c1, s1);
    advance(abase, aui);
    if (more(base)) tb_store();
    const float yscale = stage();  // every wave joins the staging barriers
    if (!more(base)) return;
    auto step_unit = [&](u32x4 (&cc)[4], SbRegs &sb) {
        const int tile = base + slot;
        const int qd = q_begin + q_step * ui;  // may be past this wave's part: then masked
        const bool last = ui + 1 == nunit;
        const int qx = min(qd, quads - 1);
        put(cc, sb, qx, ui);  // waits for this unit's loads
        if (more(abase)) load(abase + slot, unit_quad(aui), aui, cc, sb);
        advance(abase, aui);
        if (ui == 0) {
#pragma unroll
            for (int i = 0; i < NACC; i++) acc[i] = 0.0f;
            // the next tile's scale block, in flight during this tile
            tb_load(base + tstride + slot);
        }
        if constexpr (MF16) {
            // Group slots: the 16 A rows hold NS = 16 / RG slots of RG activation rows, and
            // an A row of slot sl carries its activations only while group sl (mod NS) of
            // the unit is multiplied (else it reads zeros), so D rows of slot sl accumulate
            // that group alone: D_j (j < ND) takes groups j*NS .. j*NS+NS-1 of the unit.
            // Lane (n16, kb) holds D rows 4kb .. 4kb+3 = slot kb / (RG/4), activation rows
            // 4 (kb % (RG/4)) .. +3: one fold per lane, D and half covers NS groups.
            // scales and biases of this lane's two output rows: the quad's four (one slot),
            // or this lane's group in each D (several slots)
            // (tile-block scales with several slots: read at the fold, one bf16 each)
            uint2 s4[2], b4[2];
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const int row = 16 * t + n16;
                if constexpr (SBW == 32 && NS > 1) {
                    (void)row;
                } else if constexpr (SBW == 32) {
                    s4[t] = *reinterpret_cast<const uint2 *>(tbs + row * groups + 4 * qx);
                    b4[t] = *reinterpret_cast<const uint2 *>(tbs + (32 + row) * groups + 4 * qx);
                } else {
                    s4[t] = SBW == 16 ? sbs[2 * row + (qx & 1)] : sbs[row];
                    b4[t] = SBW == 16 ? sbs[2 * (32 + row) + (qx & 1)] : sbs[32 + row];
                }
            }
            // scale and bias (f32) of this lane's group in D_j, output row 16t + n16
            auto sb_of = [&](int t, int j, float &sj, float &bj) __attribute__((always_inline)) {
                const int g4 = j * NS + kbd;
                const int g = 4 * qx + g4;
                // with tile-block scales every group of every unit is live (whole rows of 8k
                // groups split in two equal parts of whole quads), so no mask and no clamp
                const bool live = SBW == 32 || (qd < q_end && g < groups);
                uint32_t sbits, bbits;
                if constexpr (SBW == 32 && NS > 1) {
                    const int row = 16 * t + n16;
                    const int gx = SBW == 32 ? g : min(g, groups - 1);
                    sbits = (uint32_t)tbs[row * groups + gx] << 16;
                    bbits = (uint32_t)tbs[(32 + row) * groups + gx] << 16;
                } else {
                    const uint32_t sw = (g4 < 2) ? s4[t].x : s4[t].y;
                    const uint32_t bwd = (g4 < 2) ? b4[t].x : b4[t].y;
                    sbits = (g4 & 1) ? (sw & 0xFFFF0000u) : (sw << 16);
                    bbits = (g4 & 1) ? (bwd & 0xFFFF0000u) : (bwd << 16);
                }
                sj = __uint_as_float(live ? sbits : 0u);
                bj = __uint_as_float(live ? bbits : 0u);
                midpoint(sj, bj);
            };
#pragma unroll
            for (int j = 0; j < ND; j++) {
                float4_t d[2];
#pragma unroll
                for (int sl = 0; sl < NS; sl++) {
                    const int g4 = j * NS + sl;
                    const int gx = SBW == 32 ? 4 * qx + g4 : min(4 * qx + g4, groups - 1);
                    // this lane's A rows carry activations for group g4 only in slot sl
                    const uint4 *xg = (NS == 1 || sa == sl) ? xrow + 8 * gx : zrow;
                    const half8_t a0 = __builtin_bit_cast(half8_t, xg[0]);
                    const half8_t a1 = __builtin_bit_cast(half8_t, xg[1]);
#pragma unroll
                    for (int t = 0; t < 2; t++) {
                        // words 2kb, 2kb+1 of the group: chunk 2g4 + kb/2, bytes 8(kb%2) ..
                        // of row 16t + n16 (the half's 16 rows are 2 KB further on)
                        const uint2 bw = reinterpret_cast<const uint2 *>(scratch)[boff[g4] + 256 * t];
                        const uint32_t wd[2] = {bw.x, bw.y};
#pragma unroll
                        for (int i = 0; i < 2; i++) {
                            const uint32_t w8 = wd[i] >> 8;
                            const uint4 bq = {wd[i] & 0x000F000Fu, wd[i] & 0x00F000F0u,
                                              w8 & 0x000F000Fu, w8 & 0x00F000F0u};
                            d[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                i == 0 ? a0 : a1, __builtin_bit_cast(half8_t, bq),
                                (i == 0 && sl == 0) ? float4_t{} : d[t], 0, 0, 0);
                        }
                    }
                }
                // fold: this lane's group's scale on its sums, its bias on the group sums of
                // its activation rows
                const int gx = SBW == 32 ? 4 * qx + j * NS + kbd
                                         : min(4 * qx + j * NS + kbd, groups - 1);
                const float4_t xa4 = xsg[gx * 4 + (kb % (RG / 4))];
#pragma unroll
                for (int t = 0; t < 2; t++) {
                    float sj, bj;
                    sb_of(t, j, sj, bj);
#pragma unroll
                    for (int v = 0; v < 4; v++)
                        acc[4 * t + v] =
                            __builtin_fmaf(sj, d[t][v], __builtin_fmaf(bj, xa4[v], acc[4 * t + v]));
                }
            }
        } else {
            const uint2 s4 = SBW == 32   ? *reinterpret_cast<const uint2 *>(tbs + n * groups + 4 * qx)
                             : SBW == 16 ? sbs[2 * n + (qx & 1)] : sbs[n];
            const uint2 b4 = SBW == 32
                                 ? *reinterpret_cast<const uint2 *>(tbs + (32 + n) * groups + 4 * qx)
                             : SBW == 16 ? sbs[2 * (32 + n) + (qx & 1)] : sbs[32 + n];
    #pragma unroll
            for (int g4 = 0; g4 < 4; g4++) {
                const int g = 4 * qx + g4;
                // uniform: the group lies in this wave's part and inside the row
                const bool live = qd < q_end && g < groups;
                const uint32_t sw = (g4 < 2) ? s4.x : s4.y, bw = (g4 < 2) ? b4.x : b4.y;
                const uint32_t sbits = (g4 & 1) ? (sw & 0xFFFF0000u) : (sw << 16);
                const uint32_t bbits = (g4 & 1) ? (bw & 0xFFFF0000u) : (bw << 16);
                float s = __uint_as_float(live ? sbits : 0u);
                float b = __uint_as_float(live ? bbits : 0u);
                midpoint(s, b);
                const uint4 bc = scratch[n * 8 + ((2 * g4 + h) ^ (n & 7))];
                const int gx = min(g, groups - 1);
                const uint4 *xg = xrow + 8 * gx;
                const uint32_t wd[4] = {bc.x, bc.y, bc.z, bc.w};
                float16_t d;
    #pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint32_t w8 = wd[j] >> 8;
                    const uint4 bq = {wd[j] & 0x000F000Fu, wd[j] & 0x00F000F0u, w8 & 0x000F000Fu,
                                      w8 & 0x00F000F0u};
                    const half8_t aj = __builtin_bit_cast(half8_t, xg[j]);
                    d = __builtin_amdgcn_mfma_f32_32x32x16_f16(aj, __builtin_bit_cast(half8_t, bq),
                                                               j == 0 ? float16_t{} : d, 0, 0, 0);
                }
                // D layout: lane (n, h), register i holds activation row 8*(i/4) + 4h + i%4.
                const float4_t xa4 = xsg[gx * 4 + h];
    #pragma unroll
                for (int i = 0; i < 4; i++)
                    acc[i] = __builtin_fmaf(s, d[i], __builtin_fmaf(b, xa4[i], acc[i]));
                if constexpr (NB16) {
                    const float4_t xb4 = xsg[gx * 4 + 2 + h];
    #pragma unroll
                    for (int i = 0; i < 4; i++)
                        acc[4 + i] = __builtin_fmaf(s, d[4 + i], __builtin_fmaf(b, xb4[i], acc[4 + i]));
                }
            }
        }
        if (last) {
            // 16x16x32 with several group slots: add the slots' sums of each activation row
            // (lanes kb, kb ^ (RG/4), ...: xor 16 then 32 for 4 slots, xor 32 for 2), after
            // which lanes kb < RG/4 hold rows 4kb .. 4kb+3 as with one slot
            if constexpr (MF16 && NS > 1) {
#pragma unroll
                for (int i = 0; i < NACC; i++) {
                    if constexpr (NS == 4) acc[i] += __shfl_xor(acc[i], 16, 64);
                    acc[i] += __shfl_xor(acc[i], 32, 64);
                }
            }
            // combine the parts in LDS: parts 1..KS-1 publish, part 0 adds them in order
            if constexpr (KS > 1) {
                float *pbuf =
                    part + (size_t)(((step & 1) * TPB + slot) * (KS - 1)) * plan * NACC;
                if (quarter > 0 && lane < plan) {
#pragma unroll
                    for (int i = 0; i < NACC; i++)
                        pbuf[((quarter - 1) * NACC + i) * plan + lane] = acc[i];
                }
                __syncthreads();
                if (quarter == 0 && lane < plan) {
#pragma unroll
                    for (int qq = 0; qq < KS - 1; qq++)
#pragma unroll
                        for (int i = 0; i < NACC; i++)
                            acc[i] += pbuf[(qq * NACC + i) * plan + lane];
                }
            }
            if (quarter == 0) {
#pragma unroll
                for (int i = 0; i < NACC; i++) {
                    // 16x16x32: half i/4, activation row 4kb + i%4; 32x32x16: activation
                    // row 8(i/4) + 4h + i%4
                    const int orow = tile_row(tile) + (MF16 ? 16 * (i / 4) + n16 : n);
                    const int r = MF16 ? 4 * kb + (i % 4) : 8 * (i / 4) + 4 * h + (i % 4);
                    // the shifted last tile stores only rows that no earlier tile stores
                    if (tile < tiles && orow >= tile * 32 && orow < out_dim && r < nb) {
                        float v = acc[i] * yscale;
                        // K slices after the first add to what the earlier slices stored;
                        // only the last slice has a nonzero epi_div
                        if (accum) v += y_m[(size_t)r * out_dim + orow];
                        y_m[(size_t)r * out_dim + orow] = gemv_epilogue(v, epi_div);
                    }
                }
            }
            step++;
            // every wave of the block has read this tile's scale block (the combine barrier
            // above): the next one replaces it, and is visible after the second barrier
            if constexpr (SBW == 32) {
                if (more(base + tstride)) tb_store();
                __syncthreads();
            }
        }
        advance(base, ui);
        return more(base);
    };
    while (step_unit(c0, s0) && step_unit(c1, s1)) {
    }
}

typedef void (*MfmaFn)(const uint4 *, const uint16_t *, const uint16_t *, const uint2 *,
                       const uint2 *, const float *, float *, int, int, int, float,
                       const int *, int, int, const float *, int, int, int, int);

static bool use_mf16(int ks, int nb, long tiles)
{
    return Q4MV_MFMA_MF16 && ks <= 2 && tiles >= Q4MV_MFMA_KS4_BELOW &&
           (nb <= 4 || nb > 8 || Q4MV_MFMA_MF16_R8);
}

template <int WPB, int KS, bool NB16, bool MF16, bool R8 = false, int XPRE = 0>
static MfmaFn pick_sb(int sbw)
{
    if constexpr (KS == 2 && (WPB == kMfmaWaves || (Q4MV_MFMA_NB8_WPB4 && WPB == 4)))
        if (sbw == 32) return mfma_kernel<WPB, KS, NB16, 32, MF16, 4, R8>;
    return sbw == 16 ? mfma_kernel<WPB, KS, NB16, 16, MF16, 4, R8, XPRE>
           : sbw == 8 ? mfma_kernel<WPB, KS, NB16, 8, MF16, 4, R8, XPRE>
                      : mfma_kernel<WPB, KS, NB16, 2, MF16, 4, R8, XPRE>;
}

// Low-bit codes: 8-wave blocks and 8- or 16-byte scale loads only (q4mv_lowbit checks).
template <int BITS, int KS>
static MfmaFn pick_lowbit_ks(bool nb16, int sbw, bool mf16, bool r8)
{
    if constexpr (KS <= 2)
        if (mf16) {
            // 16x16x32: the group slots follow nb (4 rows, 8 rows, or one slot of 16)
            if constexpr (KS == 2)
                if (sbw == 32)
                    return nb16 ? mfma_kernel<kMfmaWaves, KS, true, 32, true, BITS>
                           : r8 ? mfma_kernel<kMfmaWaves, KS, false, 32, true, BITS, true>
                                : mfma_kernel<kMfmaWaves, KS, false, 32, true, BITS>;
            if (nb16)
                return sbw == 16 ? mfma_kernel<kMfmaWaves, KS, true, 16, true, BITS>
                                 : mfma_kernel<kMfmaWaves, KS, true, 8, true, BITS>;
            if (r8)
                return sbw == 16 ? mfma_kernel<kMfmaWaves, KS, false, 16, true, BITS, true>
                                 : mfma_kernel<kMfmaWaves, KS, false, 8, true, BITS, true>;
            return sbw == 16 ? mfma_kernel<kMfmaWaves, KS, false, 16, true, BITS>
                             : mfma_kernel<kMfmaWaves, KS, false, 8, true, BITS>;
        }
    if constexpr (KS == 2)
        if (sbw == 32)
            return nb16 ? mfma_kernel<kMfmaWaves, KS, true, 32, false, BITS>
                        : mfma_kernel<kMfmaWaves, KS, false, 32, false, BITS>;
    if (nb16)
        return sbw == 16 ? mfma_kernel<kMfmaWaves, KS, true, 16, false, BITS>
                         : mfma_kernel<kMfmaWaves, KS, true, 8, false, BITS>;
    return sbw == 16 ? mfma_kernel<kMfmaWaves, KS, false, 16, false, BITS>
                     : mfma_kernel<kMfmaWaves, KS, false, 8, false, BITS>;
}

template <int BITS>
static MfmaFn pick_lowbit(int ks, bool nb16, int sbw, bool mf16, bool r8)
{
    return ks == 1   ? pick_lowbit_ks<BITS, 1>(nb16, sbw, mf16, r8)
           : ks == 2 ? pick_lowbit_ks<BITS, 2>(nb16, sbw, mf16, r8)
           : ks == 4 ? pick_lowbit_ks<BITS, 4>(nb16, sbw, mf16, r8)
                     : pick_lowbit_ks<BITS, 8>(nb16, sbw, mf16, r8);
}

template <int WPB, int KS>
static MfmaFn pick(bool nb16, int sbw, bool mf16, bool r8, int xmode)
{
    // one quad per wave (K-split 3, 5, 6, 10 or 12): chosen for nb <= 8 only, on 32x32x16
    constexpr bool kOneQuad = KS > 2 && KS != 4 && KS != 8;
    if constexpr (kOneQuad) {
        if (nb16) return nullptr;
        // short launches staging f32 rows (xmode 1 plain, 2 [gate | up]): the instances
        // that load them ahead
        if (xmode == 1) return pick_sb<WPB, KS, false, false, false, 1>(sbw);
        if (xmode == 2) return pick_sb<WPB, KS, false, false, false, 2>(sbw);
        return pick_sb<WPB, KS, false, false>(sbw);
    } else {
        if constexpr (KS > 2) {
            if (xmode == 1)
                return nb16 ? pick_sb<WPB, KS, true, false, false, 1>(sbw)
                            : pick_sb<WPB, KS, false, false, false, 1>(sbw);
            if (xmode == 2)
                return nb16 ? pick_sb<WPB, KS, true, false, false, 2>(sbw)
                            : pick_sb<WPB, KS, false, false, false, 2>(sbw);
        }
        // the 16x16x32 path covers 16 activation rows either way; nb > 8 gets an instance
        // of its own so that the register cap for two blocks per CU (tile-block scales,
        // nb <= 8) does not apply where the LDS allows only one
        if constexpr (KS <= 2)
            if (mf16)
                return nb16 ? pick_sb<WPB, KS, true, true>(sbw)
                       : r8 ? pick_sb<WPB, KS, false, true, true>(sbw)
                            : pick_sb<WPB, KS, false, true>(sbw);
        return nb16 ? pick_sb<WPB, KS, true, false>(sbw) : pick_sb<WPB, KS, false, false>(sbw);
    }
}

// Partial-sum bytes of a launch shape: accumulators per lane, and the lanes that hold
// activation rows below nb (the ones that publish).
static size_t part_bytes(int wpb, int ks, int nb, long tiles)
{
    return use_mf16(ks, nb, tiles) ? mfma_part_bytes(wpb, ks, 8, 16 * ((nb + 3) / 4))
                                   : mfma_part_bytes(wpb, ks, nb > 8 ? 8 : 4, 64);
}

static int mfma_ks(long tiles, int quads)
{
    int ks = tiles < Q4MV_MFMA_KS8_BELOW ? 8 : tiles < Q4MV_MFMA_KS4_BELOW ? 4 : Q4MV_MFMA_KS_BIG;
    while (ks > 1 && ks > quads) ks >>= 1;  // at least one quad per part
    return ks;
}

// One quad per wave on short launches: the K-split equals the row's quads, for these quad
// counts (rows of 640/768, 1280, 1536, 2560 and 3072 columns), with two tile groups per
// block where the K-split is at most 6. Measured (fused launches, us, against K-split 8 or 2
// with up to two units per wave): 2560 x 2560 NB 4 7.56 -> 6.41, NB 8 8.48 -> 7.56;
// 8 x 2560 x 640 NB 4 7.56 -> 6.88, NB 8 7.70 -> 7.13. From 256 tiles on the grid outgrows
// one round (9728 x 2560 NB 4 9.31 -> 9.76 with a K-split of 10), and above nb 8 the staging
// of 16 rows per block outweighs it (8 x 2560 x 640 NB 16 8.58 -> 10.89).
static int ksq_waves(int quads)
{
    switch (quads) {
    case 3: return 6;
    case 5: return 10;
    case 6: return 12;
    case 10: return 10;
    case 12: return 12;
    default: return 0;
    }
}

MfmaShape mfma_shape(int in_dim, int nb, long tiles, bool need8)
{
    const int quads = (in_dim / 64 + 3) / 4;
    if (Q4MV_MFMA_KSQ && !need8 && nb <= 8 && tiles < Q4MV_MFMA_KS8_BELOW &&
        ksq_waves(quads) != 0) {
        const int wpb = ksq_waves(quads);
        if (mfma_lds_bytes(in_dim, nb) + (size_t)wpb * kScratchUnits * 16 +
                part_bytes(wpb, quads, nb, tiles) <= kMaxLds)
            return {wpb, quads};
    }
    // nb 5..8 on many tiles: 4-wave blocks where two of them (with tile-block scales) fit
    if (Q4MV_MFMA_NB8_WPB4 && !need8 && nb > 4 && nb <= 8 && tiles >= Q4MV_MFMA_KS4_BELOW) {
        const size_t base = mfma_lds_bytes(in_dim, nb) + (size_t)4 * kScratchUnits * 16;
        if (base + part_bytes(4, 2, nb, tiles) + 2 * 128 * (size_t)(in_dim / 64) <= kMaxLds / 2)
            return {4, 2};
    }
    // 8 waves per block when the activations, the per-wave scratch and the partial sums fit
    // in LDS (with a smaller K-split if need be), else 4 waves
    for (int wpb = kMfmaWaves; wpb >= 4; wpb >>= 1) {
        const size_t base = mfma_lds_bytes(in_dim, nb) + (size_t)wpb * kScratchUnits * 16;
        for (int ks = std::min(mfma_ks(tiles, quads), wpb); ks >= 1; ks >>= 1)
            if (base + part_bytes(wpb, ks, nb, tiles) <= kMaxLds) return {wpb, ks};
    }
    return {0, 0};
}

// Alignment of K-slice boundaries (columns): whole 8-group (16-byte scale load) or 4-group
// (8-byte) blocks where the row length allows.
static int mfma_slice_align(int in_dim)
{
    return in_dim % 512 == 0 ? 512 : in_dim % 256 == 0 ? 256 : 64;
}

int mfma_slice(int in_dim, int nb, long tiles, bool need8)
{
    auto ok = [&](int len) {
        const MfmaShape sh = mfma_shape(len, nb, tiles, need8);
        return sh.wpb != 0 && (!need8 || sh.wpb == kMfmaWaves);
    };
    if (ok(in_dim)) return in_dim;
    // the fewest equal slices (the last one shorter) whose staged activations fit
    const int al = mfma_slice_align(in_dim);
    for (int ns = 2;; ns++) {
        const int len = ((in_dim + ns - 1) / ns + al - 1) / al * al;
        if (ok(len)) return len;
        if (len <= al) return 0;
    }
}

// One launch over columns k0 .. k0+klen-1 (the whole row when klen == a.in_dim); accum: add
// to y instead of overwriting it; epi_div: the epilogue (0: none).
static hipError_t launch_mfma_slice(const GemvArgs &a, int k0, int klen, int accum, float epi_div)
{
    const int groups = klen / 64, gf = a.in_dim / 64, g0 = k0 / 64;
    const bool nb16 = a.nb > 8;
    const long tiles = (a.out_dim + 31) / 32;
    // every choice that changes the arithmetic (K-split, matrix-core shape) comes from one
    // matrix's tile count, so a matrix gives the same bits alone, batched or as an expert slot
    const MfmaShape sh = mfma_shape(klen, a.nb, tiles, a.bits != 4);
    if (sh.wpb == 0) return hipErrorInvalidValue;  // rejected on the host before this point
    const bool mf16 = use_mf16(sh.ks, a.nb, tiles);
    const bool r8 = mf16 && a.nb > 4 && a.nb <= 8;  // 16x16x32 with two 8-row group slots
    const int xmode = !a.xf ? 0 : a.xf_glu ? 2 : 1;  // f32 rows staged in the launch
    const size_t lds0 = mfma_lds_bytes(klen, a.nb) + part_bytes(sh.wpb, sh.ks, a.nb, tiles);
    // 16-byte scale loads when the layout allows and their larger scratch still fits (every
    // row's slice of scales must start on an 8- or 16-byte boundary)
    int sbw = groups % 4 == 0 && gf % 4 == 0 && g0 % 4 == 0 && (uintptr_t)a.scales % 8 == 0 &&
                      (uintptr_t)a.biases % 8 == 0
                  ? 8 : 2;
    if (Q4MV_MFMA_SB16 && sh.ks <= Q4MV_MFMA_SB16_MAX_KS && groups % 8 == 0 && gf % 8 == 0 &&
        g0 % 8 == 0 && (uintptr_t)a.scales % 16 == 0 && (uintptr_t)a.biases % 16 == 0 &&
        lds0 + (size_t)sh.wpb * scratch_units(16) * 16 <= kMaxLds)
        sbw = 16;
    // tile-block scales (K-split 2, whole rows of 8k groups, full tiles) where their LDS
    // buffers fit next to the rest
    const size_t tb_bytes = (size_t)(sh.wpb / std::max(1, sh.ks)) * 128 * groups;
    const bool tb_waves = sh.wpb == kMfmaWaves || (Q4MV_MFMA_NB8_WPB4 && sh.wpb == 4);
    if (Q4MV_MFMA_TBS && sh.ks == 2 && tb_waves && groups % 8 == 0 &&
        groups <= kTbMaxGroups && klen == a.in_dim && a.out_dim >= 32 &&
        (uintptr_t)a.scales % 16 == 0 && (uintptr_t)a.biases % 16 == 0 &&
        lds0 + (size_t)sh.wpb * scratch_units(32) * 16 + tb_bytes <= kMaxLds)
        sbw = 32;
    const size_t lds =
        lds0 + (size_t)sh.wpb * scratch_units(sbw) * 16 + (sbw == 32 ? tb_bytes : 0);
    // the instance of exactly this (waves, K-split); any other pair is an error, never a
    // kernel of another shape
    MfmaFn fn = nullptr;
    const int wk = sh.wpb * 100 + sh.ks;
    if (a.bits != 4) {
        if (sh.wpb != kMfmaWaves || sbw == 2) return hipErrorInvalidValue;  // checked on the host
        if (sh.ks == 1 || sh.ks == 2 || sh.ks == 4 || sh.ks == 8)
            fn = a.bits == 2 ? pick_lowbit<2>(sh.ks, nb16, sbw, mf16, r8)
                             : pick_lowbit<3>(sh.ks, nb16, sbw, mf16, r8);
    } else {
        switch (wk) {
        case 801: fn = pick<8, 1>(nb16, sbw, mf16, r8, xmode); break;
        case 802: fn = pick<8, 2>(nb16, sbw, mf16, r8, xmode); break;
        case 804: fn = pick<8, 4>(nb16, sbw, mf16, r8, xmode); break;
        case 808: fn = pick<8, 8>(nb16, sbw, mf16, r8, xmode); break;
        case 401: fn = pick<4, 1>(nb16, sbw, mf16, r8, xmode); break;
        case 402: fn = pick<4, 2>(nb16, sbw, mf16, r8, xmode); break;
        case 404: fn = pick<4, 4>(nb16, sbw, mf16, r8, xmode); break;
#if Q4MV_MFMA_KSQ
        case 603: fn = pick<6, 3>(nb16, sbw, mf16, r8, xmode); break;
        case 1005: fn = pick<10, 5>(nb16, sbw, mf16, r8, xmode); break;
        case 1206: fn = pick<12, 6>(nb16, sbw, mf16, r8, xmode); break;
        case 1010: fn = pick<10, 10>(nb16, sbw, mf16, r8, xmode); break;
        case 1212: fn = pick<12, 12>(nb16, sbw, mf16, r8, xmode); break;
#endif
        default: break;
        }
    }
    if (!fn) return hipErrorInvalidValue;
    hipError_t e = ensure_lds(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess) return e;
    const int tpb = sh.wpb / sh.ks;
    const long blocks_needed = (tiles + tpb - 1) / tpb;
    const long per_cu = std::min<long>(
        Q4MV_MFMA_BLOCKS_PER_CU,
        resident_blocks(reinterpret_cast<const void *>(fn), sh.wpb * 64, lds));
    const long cap = std::max(1L, (long)device_cus() * std::max(1L, per_cu) / a.n_mat);
    long gx = std::max(1L, std::min(blocks_needed, cap));
#if Q4MV_MFMA_BALANCE
    // the fewest blocks that keep the number of tile rounds: every tile group gets the same
    // number of tiles (no partly filled last round)
    const long rounds = (tiles + gx * tpb - 1) / (gx * tpb);
    gx = std::max(1L, ((tiles + rounds - 1) / rounds + tpb - 1) / tpb);
#endif
    hipLaunchKernelGGL(fn, dim3((unsigned)gx, (unsigned)a.n_mat), dim3(sh.wpb * 64), lds,
                       a.stream, reinterpret_cast<const uint4 *>(a.w), a.scales, a.biases,
                       static_cast<const uint2 *>(a.xe), static_cast<const uint2 *>(a.xo),
                       a.xsum, a.y, a.out_dim, klen, a.nb, epi_div, a.sel, a.n_bank,
                       a.x_shared, a.xf, a.xf_glu, a.in_dim, k0, accum);
    return hipGetLastError();
}

hipError_t launch_mfma(const GemvArgs &a)
{
    // rows whose staged activations do not fit in LDS run as K slices, one launch each, in
    // column order: each later slice adds its partial product to y, and the epilogue comes
    // with the last
    const int klen = mfma_slice(a.in_dim, a.nb, (a.out_dim + 31) / 32, a.bits != 4);
    if (klen == 0) return hipErrorInvalidValue;  // rejected on the host before this point
    for (int k0 = 0; k0 < a.in_dim; k0 += klen) {
        const int len = std::min(klen, a.in_dim - k0);
        const bool last = k0 + len == a.in_dim;
        const hipError_t e = launch_mfma_slice(a, k0, len, k0 > 0, last ? a.epi_div : 0.0f);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q4mv_impl
