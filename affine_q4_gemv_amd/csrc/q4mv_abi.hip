// C ABI of libq4mv: argument validation (all on the host, before any launch) and dispatch.
#include "../../include/q4mv.h"
#include "q4mv_internal.h"

#include <cmath>

#include <mutex>

namespace q4mv_impl {

// The automatic choice between the VALU dot-product kernels and the MFMA kernel, by the
// activation rows and the 32-row tiles of one matrix (never by the number of matrices, so a
// matrix gives the same bits alone, batched or as an expert slot). The MFMA kernel costs
// more per launch (it stages every activation row in LDS, and each of its units runs on a
// 32-row tile whatever nb is), the VALU kernels more per activation row and weight.
// Measured on MI355X (graph-timed fused launches, us, one-row VALU against MFMA):
//   2560 x 2560 (80 tiles)        nb 2: 5.2 / 7.0, nb 3: 6.0 / 7.2, nb 4: 6.9 / 7.6, nb 5: 9.9 / 7.9
//   8 x 2560 x 640 (80 tiles)     nb 2: 6.1 / 7.3, nb 3: 6.7 / 7.4, nb 4: 7.5 / 7.6, nb 5: 8.7 / 7.6
//   8 x 1280 x 2560 (40 tiles)    nb 4: the expert gate|up projection, about 3 us slower on
//                                 the VALU kernel (the MoE MLP chain 21.7 against 18.6)
//   9728 x 2560 (304 tiles)       nb 2: 7.7 / 8.7, nb 3: 9.1 / 8.9, nb 4: 10.6 / 9.3
//   151936 x 2560 (4748 tiles)    nb 2: 46.2 / 40.5, nb 3: 56.6 / 41.4
// A single small matrix favours the VALU kernel up to nb 4, a batch of experts the MFMA
// kernel from nb 4; a per-matrix rule cannot tell them apart, and the expert batches are the
// case the batched kernels exist for. So: the MFMA kernel from nb 4; at nb 3 from 256 tiles;
// at nb 2 from 1024 tiles.
constexpr int kValuAutoMaxNB = 3;
constexpr long kMfmaMinTilesNb3 = 256;
constexpr long kMfmaMinTilesNb2 = 1024;

// The automatic choice, from (nb, out_dim) only (the MFMA kernel runs K-sliced where the
// staged activations of a whole row do not fit in LDS). On the VALU side q4mv runs the
// one-row kernel (on MI355X as fast or faster than the two-row kernel at every measured
// shape, the 640-wide expert down projection included) and q4mv_2row the two-row kernel.
// The one-row and two-row kernels give bitwise the same result, so q4mv and q4mv_2row agree
// whichever they take.
int auto_path(int in_dim, int nb, bool two_row, int out_dim)
{
    (void)in_dim;
    const long tiles = (out_dim + 31) / 32;
    if (nb > kValuAutoMaxNB || (nb == 3 && tiles >= kMfmaMinTilesNb3) ||
        (nb == 2 && tiles >= kMfmaMinTilesNb2))
        return kMfma;
    return two_row ? kValu2 : kValu1;
}

int device_cus()
{
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess ||
            cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

hipError_t ensure_lds(const void *fn, size_t bytes)
{
    if (bytes <= 64 * 1024) return hipSuccess;
    static std::mutex mu;
    static const void *fns[256];
    static size_t sizes[256];
    static int n = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n; i++)
        if (fns[i] == fn && sizes[i] >= bytes) return hipSuccess;
    hipError_t e =
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    if (e == hipSuccess && n < 256) {
        fns[n] = fn;
        sizes[n] = kMaxLds;
        n++;
    }
    return e;
}

int resident_blocks(const void *fn, int threads, size_t lds)
{
    static std::mutex mu;
    struct Ent {
        const void *fn;
        int threads;
        size_t lds;
        int blocks;
    };
    static Ent ents[512];
    static int n = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n; i++)
        if (ents[i].fn == fn && ents[i].threads == threads && ents[i].lds == lds)
            return ents[i].blocks;
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, threads, lds) != hipSuccess ||
        blocks < 1)
        blocks = 1;
    if (n < 512) ents[n++] = Ent{fn, threads, lds, blocks};
    return blocks;
}

}  // namespace q4mv_impl

using namespace q4mv_impl;

static inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Checks shared by every GEMV entry point: weights, output and shape.
static int check_weights(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                         float *y, int n_mat, int out_dim, int in_dim, int nb)
{
    if (!w || !scales || !biases || !y) return Q4MV_ERR_NULL;
    // (matrices are the grid's second dimension, at most 65535 blocks)
    if (n_mat < 1 || n_mat > 65535 || out_dim < 1 || in_dim < 64 || in_dim % 64 != 0 ||
        nb < 1 || nb > Q4MV_MAX_NB)
        return Q4MV_ERR_SHAPE;
    if (!aligned(w, 16) || !aligned(scales, 2) || !aligned(biases, 2) || !aligned(y, 4))
        return Q4MV_ERR_ALIGN;
    return Q4MV_OK;
}

// ... plus the prepared activations.
static int check_gemv(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                      const void *xe, const void *xo, const float *xsum, float *y, int n_mat,
                      int out_dim, int in_dim, int nb)
{
    if (!xe || !xo || !xsum) return Q4MV_ERR_NULL;
    const int st = check_weights(w, scales, biases, y, n_mat, out_dim, in_dim, nb);
    if (st != Q4MV_OK) return st;
    if (!aligned(xe, 16) || !aligned(xo, 16) || !aligned(xsum, 4)) return Q4MV_ERR_ALIGN;
    return Q4MV_OK;
}

static int run_path(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                    const void *xe, const void *xo, const float *xsum, float *y, int n_mat,
                    int out_dim, int in_dim, int nb, int path, void *stream,
                    float epi_div = 0.0f)
{
    int st = check_gemv(w, scales, biases, xe, xo, xsum, y, n_mat, out_dim, in_dim, nb);
    if (st != Q4MV_OK) return st;
    if (path < kAuto || path > kMfma) return Q4MV_ERR_PATH;
    if (path == kAuto) path = auto_path(in_dim, nb, false, out_dim);
    if (path == kValu2 && (out_dim & 1)) return Q4MV_ERR_ODD_ROWS;
    if (path == kMfma && mfma_slice(in_dim, nb, (out_dim + 31) / 32, false) == 0)
        return Q4MV_ERR_SHAPE;
    GemvArgs a{w, scales, biases, xe, xo, xsum, y, n_mat, out_dim, in_dim, nb, epi_div,
               static_cast<hipStream_t>(stream)};
    hipError_t e = path == kMfma ? launch_mfma(a) : launch_valu(a, path == kValu2 ? 2 : 1);
    return e == hipSuccess ? Q4MV_OK : Q4MV_ERR_LAUNCH;
}

// Shared body of q4mv_experts and q4mv_experts_fused (activations as prepared streams, or
// as f32 rows xf when xf is non-null; those pointers are checked by the callers).
static int run_experts(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                       int n_bank, const int32_t *sel, int n_sel, const void *xe,
                       const void *xo, const float *xsum, const float *xf, int xf_glu,
                       float *y, int out_dim, int in_dim, int nb, int x_shared, int path,
                       void *stream)
{
    if (!w || !scales || !biases || !sel || !y) return Q4MV_ERR_NULL;
    if (n_bank < 1 || n_sel < 1 || n_sel > 65535 || out_dim < 1 || in_dim < 64 ||
        in_dim % 64 != 0 || nb < 1 || nb > Q4MV_MAX_NB)
        return Q4MV_ERR_SHAPE;
    if (!aligned(w, 16) || !aligned(scales, 2) || !aligned(biases, 2) || !aligned(sel, 4) ||
        !aligned(y, 4))
        return Q4MV_ERR_ALIGN;
    if (path < kAuto || path > kMfma) return Q4MV_ERR_PATH;
    if (path == kAuto) path = auto_path(in_dim, nb, false, out_dim);
    if (path < 0) return path;
    if (path == kValu2 && (out_dim & 1)) return Q4MV_ERR_ODD_ROWS;
    if (path == kMfma && mfma_slice(in_dim, nb, (out_dim + 31) / 32, false) == 0)
        return Q4MV_ERR_SHAPE;
    GemvArgs a{w, scales, biases, xe, xo, xsum, y, n_sel, out_dim, in_dim, nb, 0.0f,
               static_cast<hipStream_t>(stream), sel, n_bank, x_shared != 0};
    a.xf = xf;
    a.xf_glu = xf_glu;
    hipError_t e = path == kMfma ? launch_mfma(a) : launch_valu(a, path == kValu2 ? 2 : 1);
    return e == hipSuccess ? Q4MV_OK : Q4MV_ERR_LAUNCH;
}

extern "C" {

int q4mv_pack_codes(const uint8_t *codes, uint32_t *w, int64_t n_codes, void *stream)
{
    if (!codes || !w) return Q4MV_ERR_NULL;
    if (n_codes < 8 || n_codes % 8 != 0) return Q4MV_ERR_SHAPE;
    if (!aligned(codes, 8) || !aligned(w, 4)) return Q4MV_ERR_ALIGN;
    hipError_t e = launch_pack(codes, w, n_codes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q4MV_OK : Q4MV_ERR_LAUNCH;
}

int q4mv_prepare_x(const float *x, int n_rows, int in_dim, void *xe, void *xo, float *xsum,
                   void *stream)
{
    if (!x || !xe || !xo || !xsum) return Q4MV_ERR_NULL;
    if (n_rows < 1 || in_dim < 64 || in_dim % 64 != 0) return Q4MV_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(xe, 16) || !aligned(xo, 16) || !aligned(xsum, 4))
        return Q4MV_ERR_ALIGN;
    hipError_t e = launch_prep(x, n_rows, in_dim, xe, xo, xsum, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q4MV_OK : Q4MV_ERR_LAUNCH;
}

int q4mv(const uint32_t *w, const uint16_t *scales, const uint16_t *biases, const void *xe,
         const void *xo, const float *xsum, float *y, int n_mat, int out_dim, int in_dim,
         int nb, void *stream)
{
    return run_path(w, scales, biases, xe, xo, xsum, y, n_mat, out_dim, in_dim, nb,
                    auto_path(in_dim, nb, false, out_dim), stream);
}

int q4mv_fused(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
               const float *x, float *y, int n_mat, int out_dim, int in_dim, int nb, int path,
               void *stream)
{
    if (!x) return Q4MV_ERR_NULL;
    const int st = check_weights(w, scales, biases, y, n_mat, out_dim, in_dim, nb);
    if (st != Q4MV_OK) return st;
    if (!aligned(x, 16)) return Q4MV_ERR_ALIGN;
    if (path < kAuto || path > kMfma) return Q4MV_ERR_PATH;
    if (path == kAuto) path = auto_path(in_dim, nb, false, out_dim);
    if (path == kValu2 && (out_dim & 1)) return Q4MV_ERR_ODD_ROWS;
    if (path == kMfma && mfma_slice(in_dim, nb, (out_dim + 31) / 32, false) == 0)
        return Q4MV_ERR_SHAPE;
    GemvArgs a{w, scales, biases, nullptr, nullptr, nullptr, y, n_mat, out_dim, in_dim, nb,
               0.0f, static_cast<hipStream_t>(stream)};
    a.xf = x;
    hipError_t e = path == kMfma ? launch_mfma(a) : launch_valu(a, path == kValu2 ? 2 : 1);
    return e == hipSuccess ? Q4MV_OK : Q4MV_ERR_LAUNCH;
}

int q4mv_silu(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
              const void *xe, const void *xo, const float *xsum, float *y, int n_mat,
              int out_dim, int in_dim, int nb, float div, void *stream)
{
    int st = check_gemv(w, scales, biases, xe, xo, xsum, y, n_mat, out_dim, in_dim, nb);
    if (st != Q4MV_OK) return st;
    if (!(div != 0.0f) || !std::isfinite(div)) return Q4MV_ERR_VALUE;
    return run_path(w, scales, biases, xe, xo, xsum, y, n_mat, out_dim, in_dim, nb,
                    auto_path(in_dim, nb, false, out_dim), stream, div);
}

int q4mv_path_silu(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                   const void *xe, const void *xo, const float *xsum, float *y, int n_mat,
                   int out_dim, int in_dim, int nb, float div, int path, void *stream)
{
    int st = check_gemv(w, scales, biases, xe, xo, xsum, y, n_mat, out_dim, in_dim, nb);
    if (st != Q4MV_OK) return st;
    if (!(div != 0.0f) || !std::isfinite(div)) return Q4MV_ERR_VALUE;
    return run_path(w, scales, biases, xe, xo, xsum, y, n_mat, out_dim, in_dim, nb, path, stream,
                    div);
}

int q4mv_experts(const uint32_t *w, const uint16_t *scales, const uint16_t *biases, int n_bank,
                 const int32_t *sel, int n_sel, const void *xe, const void *xo,
                 const float *xsum, float *y, int out_dim, int in_dim, int nb, int x_shared,
                 int path, void *stream)
{
    if (!xe || !xo || !xsum) return Q4MV_ERR_NULL;
    if (!aligned(xe, 16) || !aligned(xo, 16) || !aligned(xsum, 4)) return Q4MV_ERR_ALIGN;
    return run_experts(w, scales, biases, n_bank, sel, n_sel, xe, xo, xsum, nullptr, 0, y,
                       out_dim, in_dim, nb, x_shared, path, stream);
}

int q4mv_experts_fused(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                       int n_bank, const int32_t *sel, int n_sel, const float *x, float *y,
                       int out_dim, int in_dim, int nb, int x_shared, int swiglu, int path,
                       void *stream)
{
    if (!x) return Q4MV_ERR_NULL;
    if (!aligned(x, 16)) return Q4MV_ERR_ALIGN;
    if (swiglu != 0 && swiglu != 1) return Q4MV_ERR_VALUE;
    return run_experts(w, scales, biases, n_bank, sel, n_sel, nullptr, nullptr, nullptr, x,
                       swiglu, y, out_dim, in_dim, nb, x_shared, path, stream);
}

int q4mv_pack_lowbit(int bits, const uint8_t *codes, uint32_t *w, int64_t n_rows, int in_dim,
                     void *stream)
{
    if (!codes || !w) return Q4MV_ERR_NULL;
    if (bits != 2 && bits != 3) return Q4MV_ERR_VALUE;
    if (n_rows < 1 || in_dim < 64 || in_dim % 64 != 0 ||
        n_rows * (in_dim / 32) > (1LL << 31) - 256)
        return Q4MV_ERR_SHAPE;
    if (!aligned(codes, 16) || !aligned(w, 4)) return Q4MV_ERR_ALIGN;
    hipError_t e = launch_pack_lowbit(bits, codes, w, n_rows, in_dim,
                                      static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q4MV_OK : Q4MV_ERR_LAUNCH;
}

int q4mv_lowbit(int bits, const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                const void *xe, const void *xo, const float *xsum, float *y, int n_mat,
                int out_dim, int in_dim, int nb, int path, void *stream)
{
    if (!w || !scales || !biases || !xe || !xo || !xsum || !y) return Q4MV_ERR_NULL;
    if (bits != 2 && bits != 3) return Q4MV_ERR_VALUE;
    if (n_mat < 1 || n_mat > 65535 || out_dim < 1 || in_dim < 64 || in_dim % 64 != 0 ||
        nb < 1 || nb > Q4MV_MAX_NB)
        return Q4MV_ERR_SHAPE;
    if (!aligned(w, 8) || !aligned(xe, 16) || !aligned(xo, 16) || !aligned(scales, 2) ||
        !aligned(biases, 2) || !aligned(xsum, 4) || !aligned(y, 4))
        return Q4MV_ERR_ALIGN;
    if (path < kAuto || path > kMfma) return Q4MV_ERR_PATH;
    // the MFMA kernel takes low-bit codes with 8-wave blocks and 8- or 16-byte scale loads
    const bool mfma_fits = (in_dim / 64) % 4 == 0 && aligned(scales, 8) && aligned(biases, 8) &&
                           mfma_slice(in_dim, nb, (out_dim + 31) / 32, true) != 0;
    // automatic: the MFMA kernel from nb = 4 where it fits (measured faster there, slower at
    // nb = 2), else the VALU kernels as q4mv chooses them
    if (path == kAuto)
        path = nb > 3 && mfma_fits ? kMfma : (nb > 1 && out_dim % 2 == 0) ? kValu2 : kValu1;
    if (path == kValu2 && (out_dim & 1)) return Q4MV_ERR_ODD_ROWS;
    if (path == kMfma && !mfma_fits) return Q4MV_ERR_SHAPE;
    GemvArgs a{w, scales, biases, xe, xo, xsum, y, n_mat, out_dim, in_dim, nb, 0.0f,
               static_cast<hipStream_t>(stream)};
    a.bits = bits;
    hipError_t e = path == kMfma ? launch_mfma(a) : launch_valu(a, path == kValu2 ? 2 : 1);
    return e == hipSuccess ? Q4MV_OK : Q4MV_ERR_LAUNCH;
}

int q4mv_combine(const float *y, const float *wmap, float *out, int n_u, int nb, int out_dim,
                 void *stream)
{
    if (!y || !wmap || !out) return Q4MV_ERR_NULL;
    if (n_u < 1 || nb < 1 || out_dim < 1 || (long long)nb * out_dim > (1LL << 31))
        return Q4MV_ERR_SHAPE;
    if (!aligned(y, 4) || !aligned(wmap, 4) || !aligned(out, 4)) return Q4MV_ERR_ALIGN;
    hipError_t e = launch_combine(y, wmap, out, n_u, nb, out_dim, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q4MV_OK : Q4MV_ERR_LAUNCH;
}

int q4mv_quantize(const float *wf, uint32_t *w, uint16_t *scales, uint16_t *biases,
                  int64_t n_rows, int in_dim, void *stream)
{
    if (!wf || !w || !scales || !biases) return Q4MV_ERR_NULL;
    if (n_rows < 1 || in_dim < 64 || in_dim % 64 != 0 || n_rows * (in_dim / 64) > (1LL << 40))
        return Q4MV_ERR_SHAPE;
    if (!aligned(wf, 16) || !aligned(w, 4) || !aligned(scales, 2) || !aligned(biases, 2))
        return Q4MV_ERR_ALIGN;
    hipError_t e =
        launch_quantize(wf, w, scales, biases, n_rows, in_dim, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q4MV_OK : Q4MV_ERR_LAUNCH;
}

int q4mv_swiglu_prep(const float *gu, int n_rows, int inter, void *xe, void *xo, float *xsum,
                     void *stream)
{
    if (!gu || !xe || !xo || !xsum) return Q4MV_ERR_NULL;
    if (n_rows < 1 || inter < 64 || inter % 64 != 0) return Q4MV_ERR_SHAPE;
    if (!aligned(gu, 8) || !aligned(xe, 16) || !aligned(xo, 16) || !aligned(xsum, 4))
        return Q4MV_ERR_ALIGN;
    hipError_t e =
        launch_swiglu_prep(gu, n_rows, inter, xe, xo, xsum, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q4MV_OK : Q4MV_ERR_LAUNCH;
}

int q4mv_2row(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
              const void *xe, const void *xo, const float *xsum, float *y, int n_mat,
              int out_dim, int in_dim, int nb, void *stream)
{
    int st = check_gemv(w, scales, biases, xe, xo, xsum, y, n_mat, out_dim, in_dim, nb);
    if (st != Q4MV_OK) return st;
    if (out_dim & 1) return Q4MV_ERR_ODD_ROWS;
    return run_path(w, scales, biases, xe, xo, xsum, y, n_mat, out_dim, in_dim, nb,
                    auto_path(in_dim, nb, true, out_dim), stream);
}

int q4mv_path(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
              const void *xe, const void *xo, const float *xsum, float *y, int n_mat,
              int out_dim, int in_dim, int nb, int path, void *stream)
{
    return run_path(w, scales, biases, xe, xo, xsum, y, n_mat, out_dim, in_dim, nb, path,
                    stream);
}

int q4mv_auto_path(int in_dim, int nb, int two_row, int out_dim)
{
    if (in_dim < 64 || in_dim % 64 != 0 || nb < 1 || nb > Q4MV_MAX_NB || out_dim < 1)
        return Q4MV_ERR_SHAPE;
    if (two_row && (out_dim & 1)) return Q4MV_ERR_ODD_ROWS;
    return auto_path(in_dim, nb, two_row != 0, out_dim);
}

const char *q4mv_status_str(int status)
{
    switch (status) {
    case Q4MV_OK: return "ok";
    case Q4MV_ERR_NULL: return "a required pointer is NULL";
    case Q4MV_ERR_SHAPE: return "a size is out of range";
    case Q4MV_ERR_ODD_ROWS: return "out_dim must be even for the two-row kernel";
    case Q4MV_ERR_ALIGN: return "a pointer is not aligned as required";
    case Q4MV_ERR_LAUNCH: return "the HIP kernel launch failed";
    case Q4MV_ERR_PATH: return "unknown kernel path";
    case Q4MV_ERR_VALUE: return "an argument value is invalid (div must be finite and nonzero)";
    default: return "unknown status";
    }
}

int q4mv_version(void) { return 500; }

}  // extern "C"
