// Fused forms of the NVFP4 skinny product (M <= 32), "Module ops":
//  * w4a16_gemv_silu_input: the activation is silu(gate) * up, computed per
//    element inside the kernel from the two bf16 vectors (this file's kernel);
//  * w4a16_gemv_dual (+ _batch2/_batch3): two projections over one x in one
//    launch, and moe_w4a16_grouped_gemm_ptrtable: one launch over a device
//    table of (x, weight, y) entries, e.g. the experts of a MoE layer;
//  * w4a16_gemv_qg / w4a16_gemv_qkvz: the weight's rows interleave parts per
//    head or group (Q|gate, Q|K|V|Z) and the output is stored de-interleaved.
// The last two run nvfp4_linear's own kernels (blockIdx.y picking the
// product, the de-interleaving map applied to the store), so they stream the
// weights as fast as the plain product does.
//
// The silu-input kernel: a workgroup per 16-column tile, its wavefronts one K
// segment each of the (N, K) tile, the activation silu(gate) * up formed in
// LDS (rounded once to bf16), the weights loaded straight into registers and
// decoded into the B operand of v_mfma_f32_16x16x32_bf16.  The segment sums
// are added in the tile's two-level order, so every output has the bits
// nvfp4_linear gives the same row of that activation and weight ("10
// Kernels" 10.1).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "nvfp4_w4a16.h"
#include "nvfp4_common.h"
#include "setup.h"
#include "../host/tiles.h"

namespace {

struct FusedArgs {
    const uint16_t* gate;   // bf16 [M, K]
    const uint16_t* up;     // bf16 [M, K]
    const uint8_t* wp;
    const uint8_t* sc;
    void* y;
    float t;
    int m, n, k, k_per_wave, group;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return bits_f32(uint32_t(b) << 16); }

// silu(g) * u in fp32 (one division and the library exponential), rounded
// once to bf16
__device__ __forceinline__ uint16_t silu_mul(uint16_t g, uint16_t u) {
    const float gf = bf16_to_f32(g);
    const float s = gf / (1.0f + expf(-gf));
    return f32_to_bf16_rne(s * bf16_to_f32(u));
}

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

template <int U>
struct FChunk {
    u32x4 w[U];
    uint64_t s[U];
};

template <int MT, int U, bool OUT_F32>
__global__ void __launch_bounds__(512)
nvfp4_silu_input_kernel(FusedArgs fa) {
    extern __shared__ __align__(16) uint16_t lds[];   // the activation [M][K + 8], then segment partials
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int waves = blockDim.x / kWave;
    const int col_lane = lane % 16;
    const int kq = lane / 16;
    const int col_base = blockIdx.x * 16;
    const int pitch = fa.k + 8;
    const int n_load = min(col_base + col_lane, fa.n - 1);
    const uint8_t* wrow = fa.wp + (int64_t)n_load * (fa.k / 2);
    const uint8_t* srow = fa.sc + (int64_t)n_load * (fa.k / 16);
    int xr[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) xr[t] = min(16 * t + col_lane, fa.m - 1);

    // the activation silu(gate) * up into LDS, rounded once to bf16 (rows
    // past M are never read)
    {
        const int vec_per_row = fa.k / 8;
        const int total = fa.m * vec_per_row;
        for (int v = threadIdx.x; v < total; v += blockDim.x) {
            const int r = v / vec_per_row, c = v % vec_per_row;
            u32x4 d = load16(fa.gate + (int64_t)r * fa.k + 8 * c);
            const u32x4 u = load16(fa.up + (int64_t)r * fa.k + 8 * c);
            uint16_t gv[8], uv[8], hv[8];
            __builtin_memcpy(gv, &d, 16);
            __builtin_memcpy(uv, &u, 16);
#pragma unroll
            for (int i = 0; i < 8; ++i) hv[i] = silu_mul(gv[i], uv[i]);
            __builtin_memcpy(&d, hv, 16);
            *reinterpret_cast<u32x4*>(lds + r * pitch + 8 * c) = d;
        }
        __syncthreads();
    }

    auto load = [&](FChunk<U>& ch, int kb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = kb + kBlockK * u;
            ch.w[u] = load16_stream(wrow + k / 2 + 16 * kq);
            ch.s[u] = load8_stream(srow + k / 16);
        }
    };

    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const FChunk<U>& ch, int kb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = kb + kBlockK * u;
            const uint32_t d = static_cast<uint32_t>(ch.s[u] >> (16 * kq));
            const float g0 = __builtin_amdgcn_cvt_f32_fp8(d, 0);
            const float g1 = __builtin_amdgcn_cvt_f32_fp8(d, 1);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 b = decode8(ch.w[u][s], s < 2 ? g0 : g1);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const u32x4 xa = *reinterpret_cast<const u32x4*>(lds + xr[t] * pitch + k + 32 * kq + 8 * s);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), b, acc[t], 0, 0, 0);
                }
            }
        }
    };

    // this wavefront's segment, one chunk ahead, strictly in increasing k
    const int k0 = wave * fa.k_per_wave;
    const int nchunks = fa.k_per_wave / (kBlockK * U);
    FChunk<U> A, B;
    load(A, k0);
    int i = 0;
    for (; i + 2 <= nchunks; i += 2) {
        load(B, k0 + (i + 1) * kBlockK * U);
        compute(A, k0 + i * kBlockK * U);
        if (i + 2 < nchunks) load(A, k0 + (i + 2) * kBlockK * U);
        compute(B, k0 + (i + 1) * kBlockK * U);
    }
    if (i < nchunks) compute(A, k0 + i * kBlockK * U);

    // segment sums in the two-level order: wavefront 0 folds in those of
    // wavefronts 1, 2, ... (chains in segment order within a group, then the
    // group sums in group order), through the LDS that held the activation
    f32x4 tot[MT];
    if (waves > 1) {
        float* partials = reinterpret_cast<float*>(lds);
        __syncthreads();
        if (wave != 0) {
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) partials[((wave * MT + t) * 4 + j) * kWave + lane] = acc[t][j];
        }
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int t = 0; t < MT; ++t) tot[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int w2 = 1; w2 < waves; ++w2) {
            const bool starts = w2 % fa.group == 0;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const float* p = partials + (w2 * MT + t) * 4 * kWave + lane;
                const f32x4 v = f32x4{p[0], p[kWave], p[2 * kWave], p[3 * kWave]};
                const f32x4 closed = w2 == fa.group ? acc[t] : tot[t] + acc[t];
                tot[t] = starts ? closed : tot[t];
                acc[t] = starts ? v : acc[t] + v;
            }
        }
        if (fa.group < waves) {
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[t] = tot[t] + acc[t];
        }
    }
    const int n = col_base + col_lane;
    if (n >= fa.n) return;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = 16 * t + 4 * kq + j;
            if (m < fa.m) {
                const float r = acc[t][j] * fa.t;
                if (OUT_F32)
                    static_cast<float*>(fa.y)[(int64_t)m * fa.n + n] = r;
                else
                    static_cast<uint16_t*>(fa.y)[(int64_t)m * fa.n + n] = f32_to_bf16_rne(r);
            }
        }
}

using FusedFn = void (*)(FusedArgs);

template <int MT>
FusedFn pick_silu_u(int u, int y_dtype) {
    const bool f = y_dtype == NVFP4_OUT_F32;
    if (u == 4) return f ? nvfp4_silu_input_kernel<MT, 4, true> : nvfp4_silu_input_kernel<MT, 4, false>;
    if (u == 2) return f ? nvfp4_silu_input_kernel<MT, 2, true> : nvfp4_silu_input_kernel<MT, 2, false>;
    return f ? nvfp4_silu_input_kernel<MT, 1, true> : nvfp4_silu_input_kernel<MT, 1, false>;
}

FusedFn pick_silu(int mt, int u, int y_dtype) {
    return mt == 1 ? pick_silu_u<1>(u, y_dtype) : pick_silu_u<2>(u, y_dtype);
}

constexpr size_t kXLdsMax = 64 * 1024;

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

namespace nvfp4 {

int fused_setup() {
    for (int mt = 1; mt <= 2; ++mt)
        for (int u = 1; u <= 4; u *= 2)
            for (int od = 0; od <= 1; ++od)
                if (hipFuncSetAttribute(reinterpret_cast<const void*>(pick_silu(mt, u, od)),
                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                        static_cast<int>(kXLdsMax)) != hipSuccess)
                    return NVFP4_ERR_HIP;
    return NVFP4_OK;
}

}  // namespace nvfp4

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
    // The activation first, into the device buffer nvfp4_init allocates
    // (M * K * 2 bytes, at most its 64 MiB), then nvfp4_linear on it: the
    // product's weights then stream through its direct-to-LDS kernels, which
    // cannot form the activation themselves (an LDS store drains their loads).
    float* buf = nullptr;
    size_t bytes = 0;
    int cus = 256;
    if ((st = nvfp4::gemm_partials(&buf, &bytes, &cus)) != NVFP4_OK) return st;
    if (buf && size_t(m) * size_t(k) * sizeof(uint16_t) <= bytes) {
        uint16_t* h = reinterpret_cast<uint16_t*>(buf);
        const int64_t vecs = m * k / 8;
        hipLaunchKernelGGL(nvfp4_silu_mul_kernel, dim3(static_cast<unsigned>((vecs + 255) / 256)), dim3(256), 0,
                           static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(gate_bf16),
                           static_cast<const uint16_t*>(up_bf16), h, vecs);
        if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
        return nvfp4_linear(h, w_packed, scales_e4m3, tensor_scale, y, m, n, k, y_dtype, stream);
    }
    // Without that buffer: one kernel forming the activation in its LDS.
    if (size_t(m) * (k + 8) * sizeof(uint16_t) > kXLdsMax) return NVFP4_ERR_SHAPE;
    if ((st = nvfp4::device_setup()) != NVFP4_OK) return st;
    const nvfp4::Tile tile = nvfp4::tile_for(n, k);
    FusedArgs fa;
    fa.gate = static_cast<const uint16_t*>(gate_bf16);
    fa.up = static_cast<const uint16_t*>(up_bf16);
    fa.wp = w_packed;
    fa.sc = scales_e4m3;
    fa.y = y;
    fa.t = tensor_scale;
    fa.m = static_cast<int>(m);
    fa.n = static_cast<int>(n);
    fa.k = static_cast<int>(k);
    fa.k_per_wave = static_cast<int>(k / tile.waves);
    fa.group = tile.waves / tile.split;
    const int mt = m <= 16 ? 1 : 2;
    // pipeline depth: whole 128-k blocks of the segment, at most four
    const int64_t blocks = k / tile.waves / kBlockK;
    const int u = blocks % 4 == 0 ? 4 : blocks % 2 == 0 ? 2 : 1;
    const size_t x_bytes = size_t(m) * (k + 8) * sizeof(uint16_t);
    const size_t part_bytes = tile.waves > 1 ? size_t(tile.waves) * mt * 4 * kWave * sizeof(float) : 0;
    const size_t lds = x_bytes > part_bytes ? x_bytes : part_bytes;
    hipLaunchKernelGGL(pick_silu(mt, u, y_dtype), dim3(static_cast<unsigned>((n + 15) / 16)),
                       dim3(static_cast<unsigned>(kWave * tile.waves)), lds, static_cast<hipStream_t>(stream), fa);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
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
