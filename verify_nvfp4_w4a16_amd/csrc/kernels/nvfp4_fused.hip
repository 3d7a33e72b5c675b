// Fused and grouped forms of the NVFP4 skinny product (M <= 32), "Module ops":
//  * w4a16_gemv_dual (+ _batch2/_batch3): two projections over one x in one
//    launch, blockIdx picking the weight;
//  * w4a16_gemv_silu_input: the activation is silu(gate) * up, computed per
//    element inside the kernel from the two bf16 vectors;
//  * w4a16_gemv_qg / w4a16_gemv_qkvz: the weight's rows interleave parts per
//    head or group (Q|gate, Q|K|V|Z) and the output is stored de-interleaved;
//  * moe_w4a16_grouped_gemm_ptrtable: one launch over a device table of
//    (x, weight, y) entries, e.g. the experts of a MoE layer.
//
// One kernel serves all of them: a workgroup per 16-column tile of one entry
// (blockIdx.y), its wavefronts one K segment each of the (N, K) tile, the
// weights loaded straight into registers and decoded into the B operand of
// v_mfma_f32_16x16x32_bf16, x staged in LDS when it fits (which the silu
// prologue needs: it forms silu(gate) * up there, rounded once to bf16) and
// otherwise read per chunk.  The segment sums are added in the tile's
// two-level order, so every output has the bits nvfp4_linear gives the same
// row of the same x and weight ("10 Kernels" 10.1).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "nvfp4_w4a16.h"
#include "nvfp4_common.h"
#include "setup.h"
#include "../host/tiles.h"

namespace {

struct FusedEntry {
    const uint16_t* x;      // bf16 [M, K]; with silu: the gate
    const uint16_t* up;     // with silu: bf16 [M, K]
    const uint8_t* wp;
    const uint8_t* sc;
    void* y;
    float t;
    int m;
};

constexpr int kMaxParts = 4;

struct FusedArgs {
    FusedEntry e[2];               // entries by blockIdx.y when table is NULL
    const nvfp4_group_t* table;    // device table of entries (grouped form)
    int n, k, k_per_wave, group;
    int silu;                      // x = bf16(silu(gate) * up)
    int parts;                     // de-interleaving parts per group, 0 = none
    int width[kMaxParts];          // output columns of each part per group
    int gwidth;                    // sum of the widths
    int ngroups;                   // N / gwidth
    int max_m;                     // rows of an entry past this are not computed
};

// Output column of weight row n under the de-interleaving map: row r of group
// g in part p (r counted from the part's first row) goes to column
// ngroups * (columns of parts before p) + g * width[p] + r.
__device__ __forceinline__ int out_column(const FusedArgs& fa, int n) {
    if (fa.parts == 0) return n;
    const int g = n / fa.gwidth;
    int r = n - g * fa.gwidth;
    int before = 0;
#pragma unroll
    for (int p = 0; p < kMaxParts; ++p) {
        if (p < fa.parts && r < fa.width[p]) return fa.ngroups * before + g * fa.width[p] + r;
        if (p < fa.parts) {
            r -= fa.width[p];
            before += fa.width[p];
        }
    }
    return n;   // unreachable for a valid map
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return bits_f32(uint32_t(b) << 16); }

// silu(g) * u in fp32 (one division and the library exponential), rounded
// once to bf16
__device__ __forceinline__ uint16_t silu_mul(uint16_t g, uint16_t u) {
    const float gf = bf16_to_f32(g);
    const float s = gf / (1.0f + expf(-gf));
    return f32_to_bf16_rne(s * bf16_to_f32(u));
}

template <int MT, int U, bool XLDS>
struct FChunk {
    u32x4 w[U];
    uint64_t s[U];
    u32x4 x[XLDS ? 1 : MT][XLDS ? 1 : U][4];
};

template <int MT, int U, bool XLDS, bool OUT_F32>
__global__ void __launch_bounds__(512)
nvfp4_fused_kernel(FusedArgs fa) {
    extern __shared__ __align__(16) uint16_t lds[];
    FusedEntry e;
    if (fa.table) {
        const nvfp4_group_t& g = fa.table[blockIdx.y];
        e.x = static_cast<const uint16_t*>(g.x);
        e.up = nullptr;
        e.wp = g.w_packed;
        e.sc = g.scales_e4m3;
        e.y = g.y;
        e.t = g.tensor_scale;
        e.m = g.m;
    } else {
        e = fa.e[blockIdx.y];
    }
    e.m = min(e.m, fa.max_m);                       // the LDS and row tiles are sized for max_m
    if (e.m <= 0) return;                           // uniform over the workgroup
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int waves = blockDim.x / kWave;
    const int col_lane = lane % 16;
    const int kq = lane / 16;
    const int col_base = blockIdx.x * 16;
    const int pitch = fa.k + 8;
    const int n_load = min(col_base + col_lane, fa.n - 1);
    const uint8_t* wrow = e.wp + (int64_t)n_load * (fa.k / 2);
    const uint8_t* srow = e.sc + (int64_t)n_load * (fa.k / 16);
    int xr[MT];
    const uint16_t* xrow[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        xr[t] = min(16 * t + col_lane, e.m - 1);
        xrow[t] = e.x + (int64_t)xr[t] * fa.k;
    }

    // x [M, K] into LDS (rows past M are never read): silu(gate) * up when
    // asked, rounded once to bf16, else x as given.
    if constexpr (XLDS) {
        const int vec_per_row = fa.k / 8;
        const int total = e.m * vec_per_row;
        for (int v = threadIdx.x; v < total; v += blockDim.x) {
            const int r = v / vec_per_row, c = v % vec_per_row;
            u32x4 d = load16(e.x + (int64_t)r * fa.k + 8 * c);
            if (fa.silu) {
                const u32x4 u = load16(e.up + (int64_t)r * fa.k + 8 * c);
                uint16_t gv[8], uv[8], hv[8];
                __builtin_memcpy(gv, &d, 16);
                __builtin_memcpy(uv, &u, 16);
#pragma unroll
                for (int i = 0; i < 8; ++i) hv[i] = silu_mul(gv[i], uv[i]);
                __builtin_memcpy(&d, hv, 16);
            }
            *reinterpret_cast<u32x4*>(lds + r * pitch + 8 * c) = d;
        }
        __syncthreads();
    }

    auto load = [&](FChunk<MT, U, XLDS>& ch, int kb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = kb + kBlockK * u;
            ch.w[u] = load16_stream(wrow + k / 2 + 16 * kq);
            ch.s[u] = load8_stream(srow + k / 16);
        }
        if constexpr (!XLDS) {
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int s = 0; s < 4; ++s) ch.x[t][u][s] = load16(xrow[t] + kb + kBlockK * u + 32 * kq + 8 * s);
        }
    };

    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const FChunk<MT, U, XLDS>& ch, int kb) {
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
                    u32x4 xa;
                    if constexpr (XLDS)
                        xa = *reinterpret_cast<const u32x4*>(lds + xr[t] * pitch + k + 32 * kq + 8 * s);
                    else
                        xa = ch.x[t][u][s];
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), b, acc[t], 0, 0, 0);
                }
            }
        }
    };

    // this wavefront's segment, one chunk ahead, strictly in increasing k
    const int k0 = wave * fa.k_per_wave;
    const int nchunks = fa.k_per_wave / (kBlockK * U);
    FChunk<MT, U, XLDS> A, B;
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
    // group sums in group order), through the LDS that held x
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
    const int on = out_column(fa, n);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = 16 * t + 4 * kq + j;
            if (m < e.m) {
                const float r = acc[t][j] * e.t;
                if (OUT_F32)
                    static_cast<float*>(e.y)[(int64_t)m * fa.n + on] = r;
                else
                    static_cast<uint16_t*>(e.y)[(int64_t)m * fa.n + on] = f32_to_bf16_rne(r);
            }
        }
}

using FusedFn = void (*)(FusedArgs);

template <int MT, bool XLDS>
FusedFn pick_fused_u(int u, int y_dtype) {
    const bool f = y_dtype == NVFP4_OUT_F32;
    if (!XLDS) return f ? nvfp4_fused_kernel<MT, 1, false, true> : nvfp4_fused_kernel<MT, 1, false, false>;
    if (u == 4) return f ? nvfp4_fused_kernel<MT, 4, true, true> : nvfp4_fused_kernel<MT, 4, true, false>;
    if (u == 2) return f ? nvfp4_fused_kernel<MT, 2, true, true> : nvfp4_fused_kernel<MT, 2, true, false>;
    return f ? nvfp4_fused_kernel<MT, 1, true, true> : nvfp4_fused_kernel<MT, 1, true, false>;
}

FusedFn pick_fused(int mt, int u, bool xlds, int y_dtype) {
    if (mt == 1) return xlds ? pick_fused_u<1, true>(u, y_dtype) : pick_fused_u<1, false>(u, y_dtype);
    return xlds ? pick_fused_u<2, true>(u, y_dtype) : pick_fused_u<2, false>(u, y_dtype);
}

constexpr size_t kXLdsMax = 64 * 1024;

// Validates the shared part of every fused form and launches `count` entries
// (blockIdx.y) with rows up to max_m.
int fused_launch(FusedArgs& fa, int64_t count, int64_t max_m, int64_t n, int64_t k, int y_dtype, void* stream,
                 bool need_xlds) {
    if (nvfp4::load_tile_override() != NVFP4_OK) return NVFP4_ERR_TILEFILE;
    int st = nvfp4::device_setup();
    if (st != NVFP4_OK) return st;
    const nvfp4::Tile tile = nvfp4::tile_for(n, k);
    fa.n = static_cast<int>(n);
    fa.k = static_cast<int>(k);
    fa.k_per_wave = static_cast<int>(k / tile.waves);
    fa.group = tile.waves / tile.split;
    fa.max_m = static_cast<int>(max_m);
    const int mt = max_m <= 16 ? 1 : 2;
    const size_t x_bytes = size_t(max_m) * (k + 8) * sizeof(uint16_t);
    const bool xlds = x_bytes <= kXLdsMax;
    if (need_xlds && !xlds) return NVFP4_ERR_SHAPE;
    // pipeline depth: whole 128-k blocks of the segment, at most four (one
    // with x read per chunk, which holds the A operands in registers)
    const int64_t blocks = k / tile.waves / kBlockK;
    const int u = !xlds ? 1 : blocks % 4 == 0 ? 4 : blocks % 2 == 0 ? 2 : 1;
    const size_t part_bytes = tile.waves > 1 ? size_t(tile.waves) * mt * 4 * kWave * sizeof(float) : 0;
    const size_t lds = xlds && x_bytes > part_bytes ? x_bytes : part_bytes;
    const dim3 grid(static_cast<unsigned>((n + 15) / 16), static_cast<unsigned>(count));
    hipLaunchKernelGGL(pick_fused(mt, u, xlds, y_dtype), grid, dim3(static_cast<unsigned>(kWave * tile.waves)), lds,
                       static_cast<hipStream_t>(stream), fa);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
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

FusedArgs plain_args() {
    FusedArgs fa;
    std::memset(&fa, 0, sizeof fa);
    return fa;
}

}  // namespace

namespace nvfp4 {

int fused_setup() {
    for (int mt = 1; mt <= 2; ++mt)
        for (int u = 1; u <= 4; u *= 2)
            for (int xl = 0; xl <= 1; ++xl)
                for (int od = 0; od <= 1; ++od)
                    if (hipFuncSetAttribute(reinterpret_cast<const void*>(pick_fused(mt, u, xl != 0, od)),
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
    FusedArgs fa = plain_args();
    fa.e[0] = FusedEntry{static_cast<const uint16_t*>(x_bf16), nullptr, w_packed0, scales0, y0, tensor_scale0,
                         static_cast<int>(m)};
    fa.e[1] = FusedEntry{static_cast<const uint16_t*>(x_bf16), nullptr, w_packed1, scales1, y1, tensor_scale1,
                         static_cast<int>(m)};
    return fused_launch(fa, 2, m, n, k, y_dtype, stream, false);
}

extern "C" int nvfp4_linear_silu_input(const void* gate_bf16, const void* up_bf16, const uint8_t* w_packed,
                                       const uint8_t* scales_e4m3, float tensor_scale, void* y, int64_t m, int64_t n,
                                       int64_t k, int y_dtype, void* stream) {
    int st = check_common(m, n, k, y_dtype);
    if (st != NVFP4_OK) return st;
    if (size_t(m) * (k + 8) * sizeof(uint16_t) > kXLdsMax) return NVFP4_ERR_SHAPE;
    if (m == 0) return NVFP4_OK;
    if ((st = check_entry(gate_bf16, w_packed, scales_e4m3, y, y_dtype)) != NVFP4_OK) return st;
    if (!up_bf16) return NVFP4_ERR_NULL;
    if (misaligned(up_bf16, 16)) return NVFP4_ERR_ALIGN;
    FusedArgs fa = plain_args();
    fa.e[0] = FusedEntry{static_cast<const uint16_t*>(gate_bf16), static_cast<const uint16_t*>(up_bf16), w_packed,
                         scales_e4m3, y, tensor_scale, static_cast<int>(m)};
    fa.silu = 1;
    return fused_launch(fa, 1, m, n, k, y_dtype, stream, true);
}

extern "C" int nvfp4_linear_deinterleave(const void* x_bf16, const uint8_t* w_packed, const uint8_t* scales_e4m3,
                                         float tensor_scale, void* y, int64_t m, int64_t n, int64_t k, int y_dtype,
                                         int parts, const int* widths, void* stream) {
    int st = check_common(m, n, k, y_dtype);
    if (st != NVFP4_OK) return st;
    if (!widths) return NVFP4_ERR_NULL;
    if (parts < 1 || parts > kMaxParts) return NVFP4_ERR_SHAPE;
    int64_t gw = 0;
    for (int p = 0; p < parts; ++p) {
        if (widths[p] < 1) return NVFP4_ERR_SHAPE;
        gw += widths[p];
    }
    if (n % gw != 0) return NVFP4_ERR_SHAPE;
    if (m == 0) return NVFP4_OK;
    if ((st = check_entry(x_bf16, w_packed, scales_e4m3, y, y_dtype)) != NVFP4_OK) return st;
    FusedArgs fa = plain_args();
    fa.e[0] = FusedEntry{static_cast<const uint16_t*>(x_bf16), nullptr, w_packed, scales_e4m3, y, tensor_scale,
                         static_cast<int>(m)};
    fa.parts = parts;
    for (int p = 0; p < parts; ++p) fa.width[p] = widths[p];
    fa.gwidth = static_cast<int>(gw);
    fa.ngroups = static_cast<int>(n / gw);
    return fused_launch(fa, 1, m, n, k, y_dtype, stream, false);
}

extern "C" int nvfp4_linear_grouped(const nvfp4_group_t* table, int64_t count, int64_t max_m, int64_t n, int64_t k,
                                    int y_dtype, void* stream) {
    int st = check_common(max_m, n, k, y_dtype);
    if (st != NVFP4_OK) return st;
    if (count < 0 || count > 65535) return NVFP4_ERR_SHAPE;
    if (count == 0 || max_m == 0) return NVFP4_OK;
    if (!table) return NVFP4_ERR_NULL;
    if (misaligned(table, 8)) return NVFP4_ERR_ALIGN;
    FusedArgs fa = plain_args();
    fa.table = table;
    return fused_launch(fa, count, max_m, n, k, y_dtype, stream, false);
}
