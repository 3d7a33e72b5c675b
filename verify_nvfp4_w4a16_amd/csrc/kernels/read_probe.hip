// Plain-read probe: one pass of 16-byte loads over two device buffers (a
// product's packed weights and its scales), so a benchmark can time the bytes
// a product must stream with nothing else in the kernel.  "10 Kernels" 10.7
// times kernels over working sets larger than the caches (its cold-bandwidth
// tool); this is the ceiling a product kernel is compared with, launch ramp
// and tail included.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "nvfp4_w4a16.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kLoads = 4;   // 16-byte loads in flight per thread

__global__ void __launch_bounds__(kThreads)
nvfp4_read_probe_kernel(const u32x4* a, int64_t na, const u32x4* b, int64_t nb, uint32_t* sink) {
    const int64_t total = na + nb;
    const int64_t step = int64_t(gridDim.x) * kThreads * kLoads;
    uint32_t acc = 0;
    for (int64_t i0 = int64_t(blockIdx.x) * kThreads * kLoads + threadIdx.x; i0 < total; i0 += step) {
        u32x4 v[kLoads];
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int64_t i = i0 + int64_t(u) * kThreads;
            v[u] = u32x4{0, 0, 0, 0};
            if (i < total) v[u] = __builtin_nontemporal_load(i < na ? a + i : b + (i - na));
        }
#pragma unroll
        for (int u = 0; u < kLoads; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    // Practically never taken; it keeps the loads from being removed.
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

extern "C" int nvfp4_read_probe(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes, void* sink,
                                void* stream) {
    if ((!a && a_bytes) || (!b && b_bytes) || !sink) return NVFP4_ERR_NULL;
    if (a_bytes < 0 || b_bytes < 0 || a_bytes % 16 || b_bytes % 16) return NVFP4_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15 ||
        reinterpret_cast<uintptr_t>(sink) & 3)
        return NVFP4_ERR_ALIGN;
    const int64_t total = (a_bytes + b_bytes) / 16;
    if (total == 0) return NVFP4_OK;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return NVFP4_ERR_HIP;
    const int64_t per_block = int64_t(kThreads) * kLoads;
    int64_t blocks = (total + per_block - 1) / per_block;
    if (blocks > int64_t(cus) * 16) blocks = int64_t(cus) * 16;
    hipLaunchKernelGGL(nvfp4_read_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(a), a_bytes / 16,
                       static_cast<const u32x4*>(b), b_bytes / 16, static_cast<uint32_t*>(sink));
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}
