// Reference kernels for measurement (libq4mv_probe.so): a streaming read of a buffer with the
// GEMV's weight-load instruction, and an empty kernel. Not on the GEMV path.
#include "../../../include/q4mv.h"
#include "../../../include/q4mv_probe.h"

#include <hip/hip_runtime.h>

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 4;  // 16-byte loads in flight per thread

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4 *__restrict__ p, int64_t n,
                                                         uint32_t *__restrict__ sink)
{
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t nth = (int64_t)gridDim.x * kThreads;
    uint32_t acc = 0;
    int64_t i = tid;
    for (; i + (kInFlight - 1) * nth < n; i += kInFlight * nth) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; u++) v[u] = __builtin_nontemporal_load(p + i + u * nth);
#pragma unroll
        for (int u = 0; u < kInFlight; u++) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n; i += nth) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    sink[tid] = acc;
}

__global__ __launch_bounds__(kThreads) void empty_kernel() {}

int cus()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        return 256;
    return n;
}

}  // namespace

extern "C" {

int64_t q4mv_probe_sink_words(int blocks_per_cu)
{
    if (blocks_per_cu < 1 || blocks_per_cu > 16) return Q4MV_ERR_SHAPE;
    return (int64_t)blocks_per_cu * cus() * kThreads;
}

int q4mv_probe_read(const void *src, int64_t bytes, uint32_t *sink, int blocks_per_cu,
                    void *stream)
{
    if (!src || !sink) return Q4MV_ERR_NULL;
    if (bytes <= 0 || bytes % 16 != 0 || blocks_per_cu < 1 || blocks_per_cu > 16)
        return Q4MV_ERR_SHAPE;
    if ((uintptr_t)src % 16 != 0 || (uintptr_t)sink % 4 != 0) return Q4MV_ERR_ALIGN;
    const int blocks = blocks_per_cu * cus();
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(src),
                       bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? Q4MV_OK : Q4MV_ERR_LAUNCH;
}

int q4mv_probe_empty(int blocks, void *stream)
{
    if (blocks < 1 || blocks > (1 << 20)) return Q4MV_ERR_SHAPE;
    hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? Q4MV_OK : Q4MV_ERR_LAUNCH;
}

}  // extern "C"
