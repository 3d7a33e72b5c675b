// Fused forms of the NVFP4 skinny product (M <= 32), "Module ops":
//  * w4a16_gemv_silu_input: the activation is silu(gate) * up, per element;
//  * w4a16_gemv_dual (+ _batch2/_batch3): two projections over one x in one
//    launch, and moe_w4a16_grouped_gemm_ptrtable: one launch over a device
//    table of (x, weight, y) entries, e.g. the experts of a MoE layer;
//  * w4a16_gemv_qg / w4a16_gemv_qkvz: the weight's rows interleave parts per
//    head or group (Q|gate, Q|K|V|Z) and the output is stored de-interleaved.
// The dual, grouped and de-interleaved forms run nvfp4_linear's own kernels
// (blockIdx.y picking the product, the de-interleaving map applied to the
// store); the silu input is formed by this file's kernel into the device
// buffer, then multiplied by nvfp4_linear.  Every output has the bits
// nvfp4_linear gives the same row of the same activation and weight ("10
// Kernels" 10.1), and the weights stream as fast as in the plain product.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "nvfp4_w4a16.h"
#include "nvfp4_common.h"
#include "setup.h"
#include "../host/tiles.h"

namespace {

// The activation alone: h = bf16(silu(gate) * up), eight elements a thread.
__global__ void __launch_bounds__(256)
nvfp4_silu_mul_kernel(const uint16_t* gate, const uint16_t* up, uint16_t* h, int64_t vecs) {
    const int64_t v = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (v >= vecs) return;
    const u32x4 g = load16(gate + 8 * v);
    const u32x4 u = load16(up + 8 * v);
    uint16_t gv[8], uv[8], hv[8];
    __builtin_memcpy(gv, &g, 16);
    __builtin_memcpy(uv, &u, 16);
#pragma unroll
    for (int i = 0; i < 8; ++i) hv[i] = silu_mul(gv[i], uv[i]);
    u32x4 o;
    __builtin_memcpy(&o, hv, 16);
    *reinterpret_cast<u32x4*>(h + 8 * v) = o;
}

bool misaligned(const void* p, uintptr_t al) { return (reinterpret_cast<uintptr_t>(p) & (al - 1)) != 0; }

int check_entry(const void* x, const uint8_t* wp, const uint8_t* sc, const void* y, int y_dtype) {
    if (!x || !wp || !sc || !y) return NVFP4_ERR_NULL;
    if (misaligned(x, 16) || misaligned(wp, 16) || misaligned(sc, 16) || misaligned(y, y_dtype == NVFP4_OUT_F32 ? 4 : 2))
        return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

int check_common(int64_t m, int64_t n, int64_t k, int y_dtype) {
    int st = nvfp4_linear_shape_ok(m, n, k);
    if (st != NVFP4_OK) return st;
    if (n > 0x7fffffff / 2) return NVFP4_ERR_SHAPE;
    if (y_dtype != NVFP4_OUT_BF16 && y_dtype != NVFP4_OUT_F32) return NVFP4_ERR_DTYPE;
    return NVFP4_OK;
}

}  // namespace

extern "C" int nvfp4_linear_dual(const void* x_bf16, const uint8_t* w_packed0, const uint8_t* scales0,
                                 float tensor_scale0, void* y0, const uint8_t* w_packed1, const uint8_t* scales1,
                                 float tensor_scale1, void* y1, int64_t m, int64_t n, int64_t k, int y_dtype,
                                 void* stream) {
    int st = check_common(m, n, k, y_dtype);
    if (st != NVFP4_OK) return st;
    if (m == 0) return NVFP4_OK;
    if ((st = check_entry(x_bf16, w_packed0, scales0, y0, y_dtype)) != NVFP4_OK) return st;
    if ((st = check_entry(x_bf16, w_packed1, scales1, y1, y_dtype)) != NVFP4_OK) return st;
    // the skinny product's kernels, blockIdx.y picking the weight
    nvfp4::MultiLaunch ml;
    ml.count = 2;
    ml.wp1 = w_packed1;
    ml.sc1 = scales1;
    ml.y1 = y1;
    ml.t1 = tensor_scale1;
    return nvfp4::launch_multi(x_bf16, w_packed0, scales0, tensor_scale0, y0, m, n, k, y_dtype, stream, ml);
}

extern "C" int nvfp4_linear_silu_input(const void* gate_bf16, const void* up_bf16, const uint8_t* w_packed,
                                       const uint8_t* scales_e4m3, float tensor_scale, void* y, int64_t m, int64_t n,
                                       int64_t k, int y_dtype, void* stream) {
    int st = check_common(m, n, k, y_dtype);
    if (st != NVFP4_OK) return st;
    if (m == 0) return NVFP4_OK;
    if ((st = check_entry(gate_bf16, w_packed, scales_e4m3, y, y_dtype)) != NVFP4_OK) return st;
    if (!up_bf16) return NVFP4_ERR_NULL;
    if (misaligned(up_bf16, 16)) return NVFP4_ERR_ALIGN;
    if (nvfp4::load_tile_override() != NVFP4_OK) return NVFP4_ERR_TILEFILE;
    // One kernel at one row where the product runs on the per-tile kernel:
    // each wavefront stages its slices of gate and up and forms the
    // activation in LDS while its first weights are in flight (measured on
    // MI355X at 4096x12288: 10.8 us against 11.9 us for two launches; at two
    // rows the in-kernel activation, twice the work on every wavefront,
    // took 15.7 us against 12.6 us, so from two rows on it is formed first).
    if (m == 1) {
        nvfp4::MultiLaunch ml;
        ml.up = up_bf16;
        st = nvfp4::launch_multi(gate_bf16, w_packed, scales_e4m3, tensor_scale, y, m, n, k, y_dtype, stream, ml);
        if (st != nvfp4::kNotFused) return st;
    }
    // Else the activation first, into the device buffer nvfp4_init allocates
    // (M * K * 2 bytes, at most its 64 MiB), then nvfp4_linear on it: the
    // product's weights then stream through its direct-to-LDS kernels, which
    // cannot form the activation themselves (an LDS store drains their loads;
    // measured on MI355X: 12.0 us at 4096x12288 and one row, against 16.9 us
    // for one kernel forming it in LDS with its weights loaded to registers).
    float* buf = nullptr;
    size_t bytes = 0;
    int cus = 256;
    if ((st = nvfp4::gemm_partials(&buf, &bytes, &cus)) != NVFP4_OK) return st;
    if (!buf || size_t(m) * size_t(k) * sizeof(uint16_t) > bytes) return NVFP4_ERR_HIP;   // no device buffer
    uint16_t* h = reinterpret_cast<uint16_t*>(buf);
    const int64_t vecs = m * k / 8;
    hipLaunchKernelGGL(nvfp4_silu_mul_kernel, dim3(static_cast<unsigned>((vecs + 255) / 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(gate_bf16),
                       static_cast<const uint16_t*>(up_bf16), h, vecs);
    if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
    return nvfp4_linear(h, w_packed, scales_e4m3, tensor_scale, y, m, n, k, y_dtype, stream);
}

extern "C" int nvfp4_linear_deinterleave(const void* x_bf16, const uint8_t* w_packed, const uint8_t* scales_e4m3,
                                         float tensor_scale, void* y, int64_t m, int64_t n, int64_t k, int y_dtype,
                                         int parts, const int* widths, void* stream) {
    int st = check_common(m, n, k, y_dtype);
    if (st != NVFP4_OK) return st;
    if (!widths) return NVFP4_ERR_NULL;
    if (parts < 1 || parts > 4) return NVFP4_ERR_SHAPE;
    int64_t gw = 0;
    for (int p = 0; p < parts; ++p) {
        if (widths[p] < 1) return NVFP4_ERR_SHAPE;
        gw += widths[p];
    }
    if (n % gw != 0) return NVFP4_ERR_SHAPE;
    if (m == 0) return NVFP4_OK;
    if ((st = check_entry(x_bf16, w_packed, scales_e4m3, y, y_dtype)) != NVFP4_OK) return st;
    // the skinny product's kernels with the de-interleaving map on the store
    nvfp4::MultiLaunch ml;
    ml.omap_parts = parts;
    for (int p = 0; p < parts; ++p) ml.omap_width[p] = widths[p];
    ml.omap_gwidth = static_cast<int>(gw);
    ml.omap_ngroups = static_cast<int>(n / gw);
    return nvfp4::launch_multi(x_bf16, w_packed, scales_e4m3, tensor_scale, y, m, n, k, y_dtype, stream, ml);
}

extern "C" int nvfp4_linear_grouped(const nvfp4_group_t* table, int64_t count, int64_t max_m, int64_t n, int64_t k,
                                    int y_dtype, void* stream) {
    int st = check_common(max_m, n, k, y_dtype);
    if (st != NVFP4_OK) return st;
    if (count < 0 || count > 65535) return NVFP4_ERR_SHAPE;
    if (count == 0 || max_m == 0) return NVFP4_OK;
    if (!table) return NVFP4_ERR_NULL;
    if (misaligned(table, 8)) return NVFP4_ERR_ALIGN;
    // the skinny product's kernels, blockIdx.y picking the table row
    nvfp4::MultiLaunch ml;
    ml.table = table;
    ml.count = static_cast<int>(count);
    return nvfp4::launch_multi(nullptr, nullptr, nullptr, 0.0f, nullptr, max_m, n, k, y_dtype, stream, ml);
}
