// MFMA kernel of libq4mv: the affine-Q4 GEMV as a real contraction for larger activation
// batches, on gfx950's v_mfma_f32_32x32x16_f16 (D[32][32] += A[32][16] * B[16][32]).
//
// Operands: A = activations (32 rows = activation rows; rows past nb are zero), read from
// LDS in the pair layout; B = codes of 32 output rows, unpacked in registers to f16
// subnormals q*2^-24 (exact) by masking nibbles. A wave owns a tile of 32 output rows. For
// scale group g of row n, lane (n, h) (h = lane / 32) loads the 16-byte chunk 2g+h, so the
// lane pair (n, 0), (n, 1) holds the whole group: MFMA i (i = 0..3) takes word i of both
// chunks, its 16-long K slice lies inside one group, and the four MFMAs of a group sum to
// that group's sum(q*x) for every (activation row, output row). The group's scale and bias
// are then applied in f32 (the per-group fold of fn_q4_rows_h, Constant BATCH_MSL page,
// quantized_rows section). The dequantised weight is never formed (the page's tiled expert
// GEMM dequantises to f16 tiles instead), and no cross-lane shuffle of codes is needed.
//
// Work split: KS waves (a tile group) share one 32-row tile, each taking a contiguous part
// of the row's scale groups; with KS > 1 their partial sums meet in LDS and are added in a
// fixed order (part 0 + 1 + ...), so results do not depend on the grid. KS is 1 when there
// are enough tiles to fill the GPU (no partial sums, no barrier after staging) and 2 or 4
// for short output dimensions. A block holds WPB / KS tile groups and strides over tiles.
// Loads are unconditional (indices clamped) and issued in batches of KB groups.
#include "q4mv_device.h"
#include "q4mv_internal.h"

#include <algorithm>

// Launch shape and pipelining (compile-time tunables, measured on MI355X): the cap on blocks
// per CU; the tile counts below which the K-split is 2 and 4 (measured: 4 is best down to
// NB = 1 even for the LM head's 4748 tiles); double-buffered weight loads
// across units; A operands read one group ahead.
#ifndef Q4MV_MFMA_KS2_BELOW
#define Q4MV_MFMA_KS2_BELOW (1 << 30)
#endif
#ifndef Q4MV_MFMA_KS4_BELOW
#define Q4MV_MFMA_KS4_BELOW (1 << 30)
#endif
#ifndef Q4MV_MFMA_PINGPONG
#define Q4MV_MFMA_PINGPONG 0
#endif
#ifndef Q4MV_MFMA_APREFETCH
#define Q4MV_MFMA_APREFETCH 0
#endif
// Non-temporal weight loads (each byte is used once).
#ifndef Q4MV_MFMA_NT
#define Q4MV_MFMA_NT 0
#endif
#ifndef Q4MV_MFMA_BLOCKS_PER_CU
#define Q4MV_MFMA_BLOCKS_PER_CU 4
#endif

namespace q4mv_impl {

// Waves per block: 8 (two per SIMD); with the per-lane register budget of 8-wave blocks the
// kernels stay in VGPRs (no AGPR spill area), so the CU can hold several blocks when LDS
// allows.
constexpr int kMfmaWaves = 8;

// WPB: waves per block. KS: waves per tile (K-split). KB: groups per load batch (even). NB16: activation
// rows 8..15 are live (nb > 8). SMODE: 1 = even group count and 4-byte aligned scale and
// bias arrays, a group pair is one dword; 0 = 2-byte loads.
// CLAMP: the row has fewer groups than KB, so group indices are clamped to the row.
template <int WPB, int KS, int KB, bool NB16, int SMODE, bool CLAMP>
__global__ __launch_bounds__(WPB * 64) void mfma_kernel(
    const uint4 *__restrict__ w, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint2 *__restrict__ xe,
    const uint2 *__restrict__ xo, const float *__restrict__ xsum, float *__restrict__ y,
    int out_dim, int in_dim, int nb)
{
    constexpr int TH = WPB * 64;
    constexpr int TPB = WPB / KS;  // tile groups per block
    constexpr int NACC = NB16 ? 8 : 4;
    extern __shared__ uint4 lds[];
    const int m = blockIdx.y;
    const int C = in_dim >> 5;
    const int groups = in_dim >> 6;
    const int words8 = in_dim >> 3;

    // LDS: activations | group sums xsg[g][16] * 2^-24 | partial sums
    // part[2][TPB][KS-1][64][NACC] (double-buffered by tile step).
    // Activation layout: row r, chunk c has four 16-byte units at r*RS + 4c + u,
    //   u = 0: (x0,x4)(x2,x6) of word 0, then of word 1   -- even code positions
    //   u = 1: (x1,x5)(x3,x7) of word 0, then of word 1   -- odd code positions
    //   u = 2, 3: the same for words 2 and 3,
    // matching how a pair of code words splits into an even-nibble and an odd-nibble MFMA
    // operand. RS = 4C + 1 (odd) puts 8 consecutive rows on 8 distinct bank quads. Lanes of
    // activation rows past nb read row nb - 1 instead: row m of D depends on row m of A only,
    // and rows past nb are never stored, so every A read is unconditional.
    const int RS = 4 * C + 1;
    float4_t *const xsg_w = reinterpret_cast<float4_t *>(lds + nb * RS);
    float *const part = reinterpret_cast<float *>(xsg_w + groups * 4);

    // Stage activations and group sums. Called after each wave has issued its first weight
    // loads, so the two latencies overlap.
    auto stage = [&]() {
        const size_t xrow0 = (size_t)m * nb;
        const uint2 *xe_m = xe + xrow0 * words8;
        const uint2 *xo_m = xo + xrow0 * words8;
        const float *xsum_m = xsum + xrow0 * C;
        const int units = nb * C * 2;  // one per (row, chunk, word pair)
        // each round issues all of its loads before any LDS write: one memory round trip
        for (int base = threadIdx.x; base < units; base += 2 * TH) {
            uint2 e[4], o[4];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int u = min(base + i * TH, units - 1);
                const int r = u / (C * 2), cp = u - r * (C * 2);  // cp = 2c + word pair
                const size_t at = (size_t)r * words8 + 2 * cp;
                e[2 * i] = xe_m[at];
                o[2 * i] = xo_m[at];
                e[2 * i + 1] = xe_m[at + 1];
                o[2 * i + 1] = xo_m[at + 1];
            }
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int u = base + i * TH;
                if (u < units) {
                    const int r = u / (C * 2), cp = u - r * (C * 2);
                    const uint4 pa = make_pairs(e[2 * i], o[2 * i]);
                    const uint4 pb = make_pairs(e[2 * i + 1], o[2 * i + 1]);
                    uint4 *dst = lds + r * RS + 2 * cp;
                    dst[0] = uint4{pa.x, pa.z, pb.x, pb.z};
                    dst[1] = uint4{pa.y, pa.w, pb.y, pb.w};
                }
            }
        }
        float *xsw = reinterpret_cast<float *>(xsg_w);
        for (int u = threadIdx.x; u < groups * 16; u += TH) {
            const int g = u >> 4, r = u & 15;
            const int rr = min(r, nb - 1);
            const float a = xsum_m[(size_t)rr * C + 2 * g], b = xsum_m[(size_t)rr * C + 2 * g + 1];
            xsw[u] = r < nb ? (a + b) * kTwoM24 : 0.0f;
        }
        __syncthreads();
    };
    const float4_t *xsg = xsg_w;

    const int lane = threadIdx.x & 63;
    const int n = lane & 31;  // output row of the tile (B, D); activation row (A)
    const int h = lane >> 5;  // which chunk of the group this lane holds
    // wave index, made visibly wave-uniform so everything derived from it lives in SGPRs
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slot = wv / KS;     // tile group of this wave within the block
    const int quarter = wv % KS;  // which part of the groups this wave sums
    // parts split the row on group-pair boundaries (so every batch starts on an even
    // group); the batch count comes from the largest part, so it is the same for every
    // wave of the block and every wave meets the per-step barrier equally often
    const int pairs = (groups + 1) >> 1;
    const int p_begin = quarter * pairs / KS;
    const int p_end = (quarter + 1) * pairs / KS;
    const int g_begin = 2 * p_begin;
    const int g_end = min(2 * p_end, groups);
    const int nbatch = max(1, (2 * ((pairs + KS - 1) / KS) + KB - 1) / KB);
    const int tiles = (out_dim + 31) >> 5;
    const int tstride = gridDim.x * TPB;

    // Row addressing with wave-uniform bases: a tile covers rows rb .. rb+31 where the last
    // tile is shifted back to end at out_dim (its overlap with the previous tile is
    // recomputed with identical arithmetic and stored again with the same bits). Only when
    // out_dim < 32 are lanes' rows clamped.
    const bool narrow = out_dim < 32;
    const int lrow = narrow ? min(n, out_dim - 1) : n;
    const uint4 *const w_m = w + (size_t)m * out_dim * C;
    const uint16_t *const s_m = scales + (size_t)m * out_dim * groups;
    const uint16_t *const b_m = biases + (size_t)m * out_dim * groups;
    float *const y_m = y + (size_t)m * nb * out_dim;
    auto tile_row = [&](int tile) { return narrow ? 0 : min(tile * 32, out_dim - 32); };

    // One load unit = (tile, batch): KB chunks of codes (lane (n, h): chunk 2g + h of its row)
    // and the scale and bias pairs of its KB groups. A batch past the end of the row is
    // shifted back to end at the row's last group when the row has at least KB groups (so
    // the loads need no per-element clamp); its repeated groups are masked out below.
    auto batch_start = [&](int bt) {
        const int gb = g_begin + bt * KB;
        return CLAMP ? 0 : min(gb, groups - KB);
    };
    // Addresses: a wave-uniform base (tile row, batch start) plus a loop-invariant lane
    // offset plus an immediate per element, so address arithmetic stays off the VALU.
    const int lw = lrow * C + h;   // lane offset into the tile's codes, in 16-byte chunks
    const int ls = lrow * groups;  // lane offset into the tile's scales and biases
    auto load = [&](int tile, int bt, uint4 (&cw)[KB], uint32_t (&sv)[KB / 2],
                    uint32_t (&bv)[KB / 2]) {
        const size_t trow = (size_t)tile_row(tile);
        const int gl = batch_start(bt);
        const uint4 *wt = w_m + trow * C + 2 * gl;
        const uint16_t *st = s_m + trow * groups + gl;
        const uint16_t *bt_ = b_m + trow * groups + gl;
#pragma unroll
        for (int kk = 0; kk < KB; kk++) {
            // only rows with fewer groups than KB need the clamp (then gl = 0)
            const int k = CLAMP ? min(kk, groups - 1) : kk;
#if Q4MV_MFMA_NT
            {
                typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                const u32x4 v =
                    __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wt + lw + 2 * k));
                cw[kk] = uint4{v[0], v[1], v[2], v[3]};
            }
#else
            cw[kk] = wt[lw + 2 * k];
#endif
        }
#pragma unroll
        for (int kp = 0; kp < KB / 2; kp++) {
            const int k0 = CLAMP ? min(2 * kp, groups - 1) : 2 * kp;
            if constexpr (SMODE == 1) {  // gl and k0 are even: an aligned dword
#if Q4MV_MFMA_NT
                sv[kp] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(st + ls + k0));
                bv[kp] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(bt_ + ls + k0));
#else
                sv[kp] = *reinterpret_cast<const uint32_t *>(st + ls + k0);
                bv[kp] = *reinterpret_cast<const uint32_t *>(bt_ + ls + k0);
#endif
            } else {
                const int k1 = CLAMP ? min(k0 + 1, groups - 1) : k0 + 1;
                sv[kp] = (uint32_t)st[ls + k0] | ((uint32_t)st[ls + k1] << 16);
                bv[kp] = (uint32_t)bt_[ls + k0] | ((uint32_t)bt_[ls + k1] << 16);
            }
        }
    };

    // this lane's activation row in LDS (row nb - 1 past nb), offset to its chunk parity
    const uint4 *const xrow = lds + min(n, nb - 1) * RS + 4 * h;
    float acc[NACC];

    // Whether the tile step at block base b has work: with KS > 1 the whole block walks tile
    // steps in lockstep (one barrier per step); with KS = 1 each wave stops on its own.
    auto more = [&](int b) { return KS == 1 ? b + slot < tiles : b < tiles; };

    // One unit of work: issue the next unit's loads into (nc, ns, nbv), then compute the
    // current one from (cc, sc, bc). Returns false when the block has no more tiles.
    int base = blockIdx.x * TPB;
    int bt = 0;
    int step = 0;
    auto unit = [&](uint4 (&cc)[KB], uint32_t (&sc)[KB / 2], uint32_t (&bc)[KB / 2],
                    uint4 (&nc)[KB], uint32_t (&ns)[KB / 2], uint32_t (&nbv)[KB / 2]) {
        asm volatile("" ::: "memory");
        const int tile = base + slot;
        const bool last = bt + 1 == nbatch;
        const int nbase = last ? base + tstride : base;
        const int nbt = last ? 0 : bt + 1;
        if (Q4MV_MFMA_PINGPONG && more(nbase)) load(nbase + slot, nbt, nc, ns, nbv);
        if (bt == 0) {
#pragma unroll
            for (int i = 0; i < NACC; i++) acc[i] = 0.0f;
        }
        const int gl = batch_start(bt);
        const int lo = g_begin + bt * KB;  // this batch's own groups: [lo, hi)
        const int hi = min(lo + KB, g_end);
        uint4 a_cur[4], a_nxt[4];
        const uint4 *xb = xrow + 8 * gl;
        auto read_a = [&](int kk, uint4 (&a)[4]) {
            const uint4 *xg = xb + 8 * (CLAMP ? min(kk, groups - 1) : kk);
#pragma unroll
            for (int u = 0; u < 4; u++) a[u] = xg[u];
        };
        read_a(0, a_cur);
#pragma unroll
        for (int kk = 0; kk < KB; kk++) {
            if (Q4MV_MFMA_APREFETCH && kk + 1 < KB) read_a(kk + 1, a_nxt);  // one group ahead
            if (!Q4MV_MFMA_APREFETCH && kk > 0) read_a(kk, a_cur);
            const int g = gl + kk;
            // scale and bias: both halves of a pair, zeroed for groups outside [lo, hi)
            const uint32_t sp = sc[kk >> 1], bp = bc[kk >> 1];
            const bool live = g >= lo && g < hi;  // uniform
            const uint32_t sbits = (kk & 1) ? (sp & 0xFFFF0000u) : (sp << 16);
            const uint32_t bbits = (kk & 1) ? (bp & 0xFFFF0000u) : (bp << 16);
            const float s = __uint_as_float(live ? sbits : 0u);
            const float b = __uint_as_float(live ? bbits : 0u);
            const uint32_t wd[4] = {cc[kk].x, cc[kk].y, cc[kk].z, cc[kk].w};
            float16_t de, dq;
#pragma unroll
            for (int p = 0; p < 2; p++) {
                const uint32_t wa = wd[2 * p], wb = wd[2 * p + 1];
                const uint32_t wa8 = wa >> 8, wb8 = wb >> 8;
                const uint4 be = {wa & 0x000F000Fu, wa8 & 0x000F000Fu, wb & 0x000F000Fu,
                                  wb8 & 0x000F000Fu};
                const uint4 bo = {wa & 0x00F000F0u, wa8 & 0x00F000F0u, wb & 0x00F000F0u,
                                  wb8 & 0x00F000F0u};
                const half8_t ae = __builtin_bit_cast(half8_t, a_cur[2 * p]);
                const half8_t ao = __builtin_bit_cast(half8_t, a_cur[2 * p + 1]);
                if (p == 0) {
                    de = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        ae, __builtin_bit_cast(half8_t, be), float16_t{}, 0, 0, 0);
                    dq = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        ao, __builtin_bit_cast(half8_t, bo), float16_t{}, 0, 0, 0);
                } else {
                    de = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        ae, __builtin_bit_cast(half8_t, be), de, 0, 0, 0);
                    dq = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        ao, __builtin_bit_cast(half8_t, bo), dq, 0, 0, 0);
                }
            }
            // odd-position codes came out times 16: d = de + dq / 16 (exact scaling).
            // D layout: lane (n, h), register i holds activation row 8*(i/4) + 4h + i%4.
            const int gx = CLAMP ? min(g, groups - 1) : g;
            const float4_t xa4 = xsg[gx * 4 + h];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float d = __builtin_fmaf(dq[i], 0.0625f, de[i]);
                acc[i] = __builtin_fmaf(s, d, __builtin_fmaf(b, xa4[i], acc[i]));
            }
            if constexpr (NB16) {
                const float4_t xb4 = xsg[gx * 4 + 2 + h];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float d = __builtin_fmaf(dq[4 + i], 0.0625f, de[4 + i]);
                    acc[4 + i] = __builtin_fmaf(s, d, __builtin_fmaf(b, xb4[i], acc[4 + i]));
                }
            }
            if (Q4MV_MFMA_APREFETCH) {
#pragma unroll
                for (int u = 0; u < 4; u++) a_cur[u] = a_nxt[u];
            }
        }
        if (last) {
            // combine the parts in LDS: parts 1..KS-1 publish, part 0 adds them in order
            if constexpr (KS > 1) {
                float *pbuf = part + (size_t)(((step & 1) * TPB + slot) * (KS - 1)) * 64 * NACC;
                if (quarter > 0) {
#pragma unroll
                    for (int i = 0; i < NACC; i++)
                        pbuf[((quarter - 1) * NACC + i) * 64 + lane] = acc[i];
                }
                __syncthreads();
                if (quarter == 0) {
#pragma unroll
                    for (int qq = 0; qq < KS - 1; qq++)
#pragma unroll
                        for (int i = 0; i < NACC; i++) acc[i] += pbuf[(qq * NACC + i) * 64 + lane];
                }
            }
            if (quarter == 0) {
                const int orow = tile_row(tile) + n;
                if (tile < tiles && orow < out_dim) {
#pragma unroll
                    for (int i = 0; i < NACC; i++) {
                        const int r = 8 * (i / 4) + 4 * h + (i % 4);
                        if (r < nb) y_m[(size_t)r * out_dim + orow] = acc[i] * kTwo24;
                    }
                }
            }
            step++;
        }
        if (!Q4MV_MFMA_PINGPONG && more(nbase)) load(nbase + slot, nbt, nc, ns, nbv);
        base = nbase;
        bt = nbt;
        return more(base);
    };

    // With KS > 1 the block walks tile steps in lockstep, so its loop count is uniform:
    // slots whose tile is past the end compute on a valid tile and store nothing.
    uint4 c0[KB], c1[KB];
    uint32_t s0[KB / 2], s1[KB / 2], b0[KB / 2], b1[KB / 2];
    if (more(base)) load(base + slot, 0, c0, s0, b0);
    stage();  // every wave joins the staging barrier exactly once
    if (more(base)) {
        if constexpr (Q4MV_MFMA_PINGPONG) {
            // ping-pong between the two load buffers: no register copies per unit
            while (unit(c0, s0, b0, c1, s1, b1) && unit(c1, s1, b1, c0, s0, b0)) {
            }
        } else {
            // one buffer: the next unit's loads are issued after this unit's compute
            while (unit(c0, s0, b0, c0, s0, b0)) {
            }
        }
    }
}

typedef void (*MfmaFn)(const uint4 *, const uint16_t *, const uint16_t *, const uint2 *,
                       const uint2 *, const float *, float *, int, int, int);

template <int WPB, int KS, int KB>
static MfmaFn pick_mode(bool nb16, bool dword_pairs)
{
    if (nb16)
        return dword_pairs ? mfma_kernel<WPB, KS, KB, true, 1, false>
                           : mfma_kernel<WPB, KS, KB, true, 0, false>;
    return dword_pairs ? mfma_kernel<WPB, KS, KB, false, 1, false>
                       : mfma_kernel<WPB, KS, KB, false, 0, false>;
}

// Groups per load batch: every group of a batch is computed, so the batch should divide a
// wave's part of the row (at most kMaxKB groups in flight per wave).
constexpr int kMaxKB = 12;
static int mfma_kb(int in_dim, int ks)
{
    const int pairs = (in_dim / 64 + 1) / 2;
    const int qgroups = 2 * ((pairs + ks - 1) / ks);  // the largest part
    const int nbatch = (qgroups + kMaxKB - 1) / kMaxKB;
    const int kb = 2 * ((qgroups / 2 + nbatch - 1) / nbatch);
    // a batch never reaches past the row (batches are shifted back to end at its last
    // group); only a one-group row keeps kb = 2, with clamped indices
    const int groups = in_dim / 64;
    return kb > groups && groups >= 2 ? groups & ~1 : kb;
}

template <int WPB, int KS>
static MfmaFn pick_kb(int kb, bool nb16, bool dword_pairs, bool clamp)
{
    // fewer groups than the batch (a single-group row): 2-byte scale loads, clamped indices
    if (clamp)
        return nb16 ? mfma_kernel<WPB, KS, 2, true, 0, true>
                    : mfma_kernel<WPB, KS, 2, false, 0, true>;
    switch (kb) {
    case 2: return pick_mode<WPB, KS, 2>(nb16, dword_pairs);
    case 4: return pick_mode<WPB, KS, 4>(nb16, dword_pairs);
    case 6: return pick_mode<WPB, KS, 6>(nb16, dword_pairs);
    case 8: return pick_mode<WPB, KS, 8>(nb16, dword_pairs);
    case 10: return pick_mode<WPB, KS, 10>(nb16, dword_pairs);
    default: return pick_mode<WPB, KS, 12>(nb16, dword_pairs);
    }
}

MfmaShape mfma_shape(int in_dim, int nb, long tiles)
{
    const bool nb16 = nb > 8;
    const size_t base = mfma_lds_bytes(in_dim, nb);
    // K-split: 1 when the tiles alone fill the GPU, else 2 or 4 waves per tile; 1 also when
    // the partial sums would not fit beside the activations
    const int ks = tiles < Q4MV_MFMA_KS4_BELOW ? 4 : tiles < Q4MV_MFMA_KS2_BELOW ? 2 : 1;
    if (base + mfma_part_bytes(kMfmaWaves, ks, nb16) <= kMaxLds) return {kMfmaWaves, ks};
    if (base <= kMaxLds) return {kMfmaWaves, 1};
    return {0, 0};
}

hipError_t launch_mfma(const GemvArgs &a)
{
    const int groups = a.in_dim / 64;
    const bool nb16 = a.nb > 8;
    const long tiles = (a.out_dim + 31) / 32;
    const MfmaShape sh = mfma_shape(a.in_dim, a.nb, tiles * a.n_mat);
    if (sh.wpb == 0) return hipErrorInvalidValue;  // rejected on the host before this point
    const size_t lds = mfma_lds_bytes(a.in_dim, a.nb) + mfma_part_bytes(sh.wpb, sh.ks, nb16);
    const int kb = mfma_kb(a.in_dim, sh.ks);
    const bool dword_pairs = groups % 2 == 0 && (uintptr_t)a.scales % 4 == 0 &&
                             (uintptr_t)a.biases % 4 == 0;
    const bool clamp = groups < kb;  // only a one-group row (kb = 2)
    MfmaFn fn = sh.ks == 1 ? pick_kb<kMfmaWaves, 1>(kb, nb16, dword_pairs, clamp)
              : sh.ks == 2 ? pick_kb<kMfmaWaves, 2>(kb, nb16, dword_pairs, clamp)
                           : pick_kb<kMfmaWaves, 4>(kb, nb16, dword_pairs, clamp);
    hipError_t e = ensure_lds(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess) return e;
    const int tpb = sh.wpb / sh.ks;
    const long blocks_needed = (tiles + tpb - 1) / tpb;
    const long per_cu = std::min<long>(
        Q4MV_MFMA_BLOCKS_PER_CU,
        resident_blocks(reinterpret_cast<const void *>(fn), sh.wpb * 64, lds));
    const long cap = std::max(1L, (long)device_cus() * per_cu / a.n_mat);
    const long gx = std::max(1L, std::min(blocks_needed, cap));
    hipLaunchKernelGGL(fn, dim3((unsigned)gx, (unsigned)a.n_mat), dim3(sh.wpb * 64), lds,
                       a.stream, reinterpret_cast<const uint4 *>(a.w), a.scales, a.biases,
                       static_cast<const uint2 *>(a.xe), static_cast<const uint2 *>(a.xo),
                       a.xsum, a.y, a.out_dim, a.in_dim, a.nb);
    return hipGetLastError();
}

}  // namespace q4mv_impl
