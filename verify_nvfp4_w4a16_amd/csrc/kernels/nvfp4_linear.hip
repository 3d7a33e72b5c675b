// NVFP4 weight-only skinny product for gfx950 (MI355X):
//   y[m, n] = t * sum_k x[m, k] * e4m3(s[n, k/16]) * e2m1(q[n, k]),  M <= 32.
//
// What is computed follows "Module ops" (metrale_model_layers::layers::ops):
// w4a16_gemm / w4a16_gemv / w4a16_tc_rows give C = A @ dequant(B) for bf16 A
// [M, K] and a row-major NVFP4 weight [N, K] (packed e2m1 [N, K/2] with the
// low nibble holding the even k, e4m3 scales [N, K/16], fp32 per-tensor scale).
//
// Design for CDNA4, not a translation of the pages' GB10 kernel ("10 Kernels",
// section 10.2, whose mma.m16n8k16 operands come straight from an e2m1->f16
// converter):
//  * Weights are the B operand of v_mfma_f32_16x16x32_bf16: lane l owns weight
//    row (output column) l % 16 and, per instruction, 8 consecutive k of it.
//    One 16-byte load per lane brings 32 k of one row (4 instructions' worth);
//    the 4 lanes that share a row read 64 contiguous bytes.  Weights never
//    pass through LDS.
//  * Decode is in registers: v_cvt_scalef32_pk_f32_fp4 turns one packed byte
//    into two fp32 e2m1 values (its scale operand contributes only an
//    exponent, so it is given 1.0), a multiply by the group's e4m3 scale
//    (decoded once per 16 k by v_cvt_f32_fp8, the OCP e4m3 decoder) makes the
//    exact product, and v_cvt_pk_bf16_f32 packs two of them into the bf16
//    operand.  e2m1 times e4m3 has at most 6 significant bits, so the bf16
//    weight is exact ("10 Kernels", 10.2, makes the same point for fp16).
//  * Activations are the A operand: 16 rows per instruction, one 16-row tile
//    for M <= 16 and two for 17..32; rows >= M are zero.
//  * Every M, including M = 1, runs the same instruction sequence on each
//    output element: the K order is fixed by the (N, K) tile, wavefront
//    partials are added in wavefront order through LDS, and nothing uses
//    atomics ("10 Kernels", 10.1).  The M = 1 entry is a GEMV-shaped
//    instantiation (one A tile, x fetched straight into registers).
//  * Epilogue: fp32 sum times t, one round-to-nearest-even to bf16, or fp32.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "nvfp4_w4a16.h"
#include "../host/tiles.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlockK = 128;    // k covered by one 16-byte weight load per lane (4 MFMAs)

struct Args {
    const uint16_t* x;     // bf16 [M, K]
    const uint8_t* wp;     // [N, K/2]
    const uint8_t* sc;     // [N, K/16]
    void* y;               // [M, N] bf16 or fp32
    float t;
    int m, n, k;
    int k_per_wave;
};

__device__ __forceinline__ u32x4 load16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Two e2m1 codes of byte `sel` of `w` times the group scale, as a bf16 pair.
template <int sel>
__device__ __forceinline__ bf16x2 decode_pair(uint32_t w, float scale) {
    f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, sel);
    f32x2 p = {v[0] * scale, v[1] * scale};
    return __builtin_convertvector(p, bf16x2);
}

// 8 consecutive k (one dword of packed nibbles) as the B operand.
__device__ __forceinline__ bf16x8 decode8(uint32_t w, float scale) {
    bf16x2 a = decode_pair<0>(w, scale);
    bf16x2 b = decode_pair<1>(w, scale);
    bf16x2 c = decode_pair<2>(w, scale);
    bf16x2 d = decode_pair<3>(w, scale);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, sizeof r);
    return r;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    bf16x2 p = __builtin_convertvector(f32x2{f, 0.0f}, bf16x2);
    uint16_t out;
    __builtin_memcpy(&out, &p, sizeof out);
    return out;
}

// C: 16-column tiles per wavefront.  MT: 16-row A tiles (1 for M <= 16).
// OUT_F32: y element type.
template <int C, int MT, bool OUT_F32>
__global__ void __launch_bounds__(1024)
nvfp4_skinny(Args a) {
    extern __shared__ float partials[];            // [waves][C][MT][4][64] fp32
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int waves = blockDim.x / kWave;
    const int col_lane = lane % 16;                // B column / A row within a tile
    const int kq = lane / 16;                      // which 8-k quarter of an instruction
    const int col_base = blockIdx.x * 16 * C;
    const int64_t row_bytes = a.k / 2;
    const int64_t scale_bytes = a.k / 16;

    const uint8_t* wrow[C];
    const uint8_t* srow[C];
    bool wvalid[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        int n = col_base + 16 * c + col_lane;
        wvalid[c] = n < a.n;
        int nn = wvalid[c] ? n : 0;
        wrow[c] = a.wp + nn * row_bytes;
        srow[c] = a.sc + nn * scale_bytes;
    }
    const uint16_t* xrow[MT];
    bool xvalid[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        int m = 16 * t + col_lane;
        xvalid[t] = m < a.m;
        xrow[t] = a.x + (int64_t)(xvalid[t] ? m : 0) * a.k;
    }

    f32x4 acc[C][MT];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int k0 = wave * a.k_per_wave;
    const int k1 = k0 + a.k_per_wave;
    for (int kb = k0; kb < k1; kb += kBlockK) {
        u32x4 w[C];
        uint32_t s2[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (wvalid[c]) {
                w[c] = load16(wrow[c] + kb / 2 + 16 * kq);
                s2[c] = *reinterpret_cast<const uint16_t*>(srow[c] + kb / 16 + 2 * kq);
            } else {
                w[c] = u32x4{0, 0, 0, 0};
                s2[c] = 0;
            }
        }
        u32x4 xa[MT][4];
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                xa[t][s] = xvalid[t] ? load16(xrow[t] + kb + 32 * kq + 8 * s) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < C; ++c) {
            float g0 = __builtin_amdgcn_cvt_f32_fp8(s2[c], 0);
            float g1 = __builtin_amdgcn_cvt_f32_fp8(s2[c], 1);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 b = decode8(w[c][s], s < 2 ? g0 : g1);
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[t][s]), b,
                                                                       acc[c][t], 0, 0, 0);
            }
        }
    }

    // Wavefront partials, added in wavefront order: wavefront 0 keeps its
    // own sum in registers and adds those of wavefronts 1, 2, ... in turn.
    if (waves > 1) {
        if (wave != 0) {
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        partials[((wave * C + c) * MT + t) * 4 * kWave + j * kWave + lane] = acc[c][t][j];
        }
        __syncthreads();
        if (wave != 0) return;
        for (int w2 = 1; w2 < waves; ++w2) {
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[c][t][j] += partials[((w2 * C + c) * MT + t) * 4 * kWave + j * kWave + lane];
        }
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int n = col_base + 16 * c + col_lane;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = 16 * t + 4 * kq + j;
                if (m < a.m && n < a.n) {
                    float r = acc[c][t][j] * a.t;
                    if (OUT_F32)
                        static_cast<float*>(a.y)[(int64_t)m * a.n + n] = r;
                    else
                        static_cast<uint16_t*>(a.y)[(int64_t)m * a.n + n] = f32_to_bf16_rne(r);
                }
            }
    }
}

using KernelFn = void (*)(Args);

template <int C, int MT>
KernelFn pick_out(int y_dtype) {
    return y_dtype == NVFP4_OUT_F32 ? nvfp4_skinny<C, MT, true> : nvfp4_skinny<C, MT, false>;
}

template <int MT>
KernelFn pick_c(int cols, int y_dtype) {
    switch (cols) {
        case 16: return pick_out<1, MT>(y_dtype);
        case 32: return pick_out<2, MT>(y_dtype);
        default: return pick_out<4, MT>(y_dtype);
    }
}

KernelFn pick_kernel(int mt, int cols, int y_dtype) {
    return mt == 1 ? pick_c<1>(cols, y_dtype) : pick_c<2>(cols, y_dtype);
}

std::once_flag g_init_once;
int g_init_status = NVFP4_OK;

void do_init() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) { g_init_status = NVFP4_ERR_HIP; return; }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) { g_init_status = NVFP4_ERR_HIP; return; }
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) { g_init_status = NVFP4_ERR_DEVICE; return; }
    int st = nvfp4::load_tile_override();
    if (st != NVFP4_OK) { g_init_status = st; return; }
    // Touch every kernel so its code object is loaded before any graph capture.
    const int cols[3] = {16, 32, 64};
    for (int mt = 1; mt <= 2; ++mt)
        for (int ci = 0; ci < 3; ++ci)
            for (int od = 0; od <= 1; ++od) {
                hipFuncAttributes attr;
                if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(pick_kernel(mt, cols[ci], od))) != hipSuccess) {
                    g_init_status = NVFP4_ERR_HIP;
                    return;
                }
            }
}

}  // namespace

extern "C" int nvfp4_init(void) {
    std::call_once(g_init_once, do_init);
    return g_init_status;
}

extern "C" int nvfp4_tile_info(int64_t n, int64_t k, char* buf, int64_t buflen) {
    if (!buf) return NVFP4_ERR_NULL;
    if (nvfp4_linear_shape_ok(1, n, k) != NVFP4_OK) return NVFP4_ERR_SHAPE;
    if (nvfp4::load_tile_override() != NVFP4_OK) return NVFP4_ERR_TILEFILE;
    std::string s = nvfp4::tile_text(n, k, nvfp4::tile_for(n, k));
    if ((int64_t)s.size() + 1 > buflen) return NVFP4_ERR_BUFFER;
    std::memcpy(buf, s.c_str(), s.size() + 1);
    return NVFP4_OK;
}

extern "C" int nvfp4_linear(const void* x_bf16, const uint8_t* w_packed, const uint8_t* scales_e4m3,
                            float tensor_scale, void* y, int64_t m, int64_t n, int64_t k, int y_dtype,
                            void* stream) {
    int st = nvfp4_linear_shape_ok(m, n, k);
    if (st != NVFP4_OK) return st;
    if (y_dtype != NVFP4_OUT_BF16 && y_dtype != NVFP4_OUT_F32) return NVFP4_ERR_DTYPE;
    if (m == 0) return NVFP4_OK;
    if (!x_bf16 || !w_packed || !scales_e4m3 || !y) return NVFP4_ERR_NULL;
    auto misaligned = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; };
    if (misaligned(x_bf16, 16) || misaligned(w_packed, 16) || misaligned(scales_e4m3, 16) ||
        misaligned(y, y_dtype == NVFP4_OUT_F32 ? 4 : 2))
        return NVFP4_ERR_ALIGN;
    st = nvfp4_init();
    if (st != NVFP4_OK) return st;

    const nvfp4::Tile tile = nvfp4::tile_for(n, k);
    const int mt = m <= 16 ? 1 : 2;
    Args a;
    a.x = static_cast<const uint16_t*>(x_bf16);
    a.wp = w_packed;
    a.sc = scales_e4m3;
    a.y = y;
    a.t = tensor_scale;
    a.m = static_cast<int>(m);
    a.n = static_cast<int>(n);
    a.k = static_cast<int>(k);
    a.k_per_wave = static_cast<int>(k / tile.waves);
    const int c = tile.cols / 16;
    const size_t lds = tile.waves > 1 ? size_t(tile.waves) * c * mt * 4 * kWave * sizeof(float) : 0;
    const dim3 grid(static_cast<unsigned>((n + tile.cols - 1) / tile.cols));
    const dim3 block(static_cast<unsigned>(kWave * tile.waves));
    hipLaunchKernelGGL(pick_kernel(mt, tile.cols, y_dtype), grid, block, lds,
                       static_cast<hipStream_t>(stream), a);
    if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
    return NVFP4_OK;
}
