// The third regime of "10 Kernels" 10.2 as the pages run it: above about
// 1,024 rows the weight is expanded to bf16 once and the product is the
// platform's library GEMM (the expand path's "Module ops" entry
// dequant_nvfp4_to_bf16, then the vendor GEMM; hipBLASLt on MI355X):
//   y[m, n] = t * sum_k x[m, k] * w_bf16[n, k]
// with fp32 accumulation, t applied to the fp32 sum, one rounding to y's type.
// The library chooses its own kernel and K order per shape, so the bits are
// not nvfp4_gemm's, and a row may differ in its last bits between row counts;
// repeated calls of one shape give the same bits.
//
// Host code only: per device one library handle and a 32 MiB workspace
// (created on the first call on that device), per (device, shape, output
// type) a plan (descriptors and the library's first heuristic choice) made on
// the first call with that shape and kept until the process ends.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cstdint>
#include <map>
#include <mutex>
#include <tuple>

#include "nvfp4_w4a16.h"
#include "setup.h"

namespace {

constexpr size_t kWorkspaceBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

struct DeviceLib {
    hipblasLtHandle_t handle = nullptr;
    void* workspace = nullptr;
};

struct Plan {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    size_t workspace = 0;
};

std::mutex g_mu;
DeviceLib g_dev[kMaxDevices];
std::map<std::tuple<int, int64_t, int64_t, int64_t, int>, Plan> g_plans;

bool ok(hipblasStatus_t s) { return s == HIPBLAS_STATUS_SUCCESS; }

// Column-major view of the row-major product: y^T [N, M] = w [N, K] x^T.
// A is the weight stored as K x N (leading dimension K) taken transposed, B
// the activations stored as K x M taken as they are, D the output N x M.
int make_plan(hipblasLtHandle_t h, int64_t m, int64_t n, int64_t k, int y_dtype, Plan* p) {
    const hipDataType yt = y_dtype == NVFP4_OUT_F32 ? HIP_R_32F : HIP_R_16BF;
    if (!ok(hipblasLtMatmulDescCreate(&p->desc, HIPBLAS_COMPUTE_32F, HIP_R_32F))) return NVFP4_ERR_LIBRARY;
    const int32_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    if (!ok(hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof ta)) ||
        !ok(hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof tb)) ||
        !ok(hipblasLtMatrixLayoutCreate(&p->a, HIP_R_16BF, k, n, k)) ||
        !ok(hipblasLtMatrixLayoutCreate(&p->b, HIP_R_16BF, k, m, k)) ||
        !ok(hipblasLtMatrixLayoutCreate(&p->d, yt, n, m, n)))
        return NVFP4_ERR_LIBRARY;
    hipblasLtMatmulPreference_t pref = nullptr;
    if (!ok(hipblasLtMatmulPreferenceCreate(&pref))) return NVFP4_ERR_LIBRARY;
    const uint64_t ws = kWorkspaceBytes;
    hipblasLtMatmulHeuristicResult_t res[1];
    int found = 0;
    const bool got =
        ok(hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws, sizeof ws)) &&
        ok(hipblasLtMatmulAlgoGetHeuristic(h, p->desc, p->a, p->b, p->d, p->d, pref, 1, res, &found)) &&
        found > 0 && ok(res[0].state) && res[0].workspaceSize <= kWorkspaceBytes;
    hipblasLtMatmulPreferenceDestroy(pref);
    if (!got) return NVFP4_ERR_LIBRARY;
    p->algo = res[0].algo;
    p->workspace = res[0].workspaceSize;
    return NVFP4_OK;
}

// The current device's handle and workspace and the plan of this shape,
// created once each; descriptors are never changed after creation.
int lookup(int64_t m, int64_t n, int64_t k, int y_dtype, DeviceLib** lib, const Plan** plan) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceLib& d = g_dev[dev];
    if (!d.handle) {
        if (!ok(hipblasLtCreate(&d.handle))) {
            d.handle = nullptr;
            return NVFP4_ERR_LIBRARY;
        }
    }
    if (!d.workspace && hipMalloc(&d.workspace, kWorkspaceBytes) != hipSuccess) {
        d.workspace = nullptr;
        return NVFP4_ERR_HIP;
    }
    const auto key = std::make_tuple(dev, m, n, k, y_dtype);
    auto it = g_plans.find(key);
    if (it == g_plans.end()) {
        Plan p;
        const int st = make_plan(d.handle, m, n, k, y_dtype, &p);
        if (st != NVFP4_OK) return st;       // descriptors of a failed plan are left behind (few bytes)
        it = g_plans.emplace(key, p).first;
    }
    *lib = &d;
    *plan = &it->second;
    return NVFP4_OK;
}

}  // namespace

extern "C" int nvfp4_gemm_library(const void* x_bf16, const void* w_bf16, float tensor_scale, void* y, int64_t m,
                                  int64_t n, int64_t k, int y_dtype, void* stream) {
    int st = nvfp4_gemm_shape_ok(m, n, k);
    if (st != NVFP4_OK) return st;
    if (y_dtype != NVFP4_OUT_BF16 && y_dtype != NVFP4_OUT_F32) return NVFP4_ERR_DTYPE;
    if (m == 0) return NVFP4_OK;
    if (!x_bf16 || !w_bf16 || !y) return NVFP4_ERR_NULL;
    auto misaligned = [](const void* p, uintptr_t al) { return (reinterpret_cast<uintptr_t>(p) & (al - 1)) != 0; };
    if (misaligned(x_bf16, 16) || misaligned(w_bf16, 16) || misaligned(y, y_dtype == NVFP4_OUT_F32 ? 4 : 2))
        return NVFP4_ERR_ALIGN;
    st = nvfp4::device_setup();
    if (st != NVFP4_OK) return st;
    DeviceLib* lib = nullptr;
    const Plan* plan = nullptr;
    st = lookup(m, n, k, y_dtype, &lib, &plan);
    if (st != NVFP4_OK) return st;
    const float alpha = tensor_scale, beta = 0.0f;
    if (!ok(hipblasLtMatmul(lib->handle, plan->desc, &alpha, w_bf16, plan->a, x_bf16, plan->b, &beta, y, plan->d, y,
                            plan->d, &plan->algo, lib->workspace, plan->workspace,
                            static_cast<hipStream_t>(stream))))
        return NVFP4_ERR_LIBRARY;
    return NVFP4_OK;
}

extern "C" int nvfp4_matmul_expand(const void* x_bf16, const uint8_t* w_packed, const uint8_t* scales_e4m3,
                                   float tensor_scale, void* y, int64_t m, int64_t n, int64_t k, int y_dtype,
                                   void* w_bf16_scratch, int64_t expand_min_m, void* stream) {
    if (expand_min_m < 0) return NVFP4_ERR_SHAPE;
    // From 768 rows on, expanding once per call and running the library GEMM
    // is ahead of nvfp4_matmul on MI355X on all four decode-round shapes
    // (same-box, order-balanced: 66-186 us against 88-233 us at 768 rows,
    // 76-203 against 94-282 at 1,024, about half the time at 4,096; at 384
    // and 512 rows it depends on the shape, within 10 %).  The pages put the
    // boundary at about 1,024 rows.
    const int64_t from = expand_min_m == 0 ? 768 : expand_min_m;
    if (m < from) return nvfp4_matmul(x_bf16, w_packed, scales_e4m3, tensor_scale, y, m, n, k, y_dtype, stream);
    int st = nvfp4_gemm_shape_ok(m, n, k);
    if (st != NVFP4_OK) return st;
    if (!w_bf16_scratch) return NVFP4_ERR_NULL;
    st = nvfp4_dequant_bf16(w_packed, scales_e4m3, tensor_scale, 0, w_bf16_scratch, n, k, stream);
    if (st != NVFP4_OK) return st;
    return nvfp4_gemm_library(x_bf16, w_bf16_scratch, tensor_scale, y, m, n, k, y_dtype, stream);
}
