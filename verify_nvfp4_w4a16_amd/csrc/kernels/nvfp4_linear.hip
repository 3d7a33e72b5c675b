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
constexpr int kMaxLdsBytes = 160 * 1024;

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

__device__ __forceinline__ u32x4 load16_stream(const void* p) {
    // Weights are read exactly once: a non-temporal load keeps them from
    // displacing the activations in the caches.
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ uint64_t load8_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(p));
}

// Registers holding the operands of one chunk of U 128-k blocks.  With x in
// LDS only the weights are held; otherwise the A operands ride along.
template <int C, int MT, int U, bool XLDS>
struct Chunk {
    u32x4 w[C][U];          // packed nibbles: 32 k of one weight row per lane per block
    uint64_t s[C][U];       // the block's 8 scale bytes of that row
    u32x4 x[XLDS ? 1 : MT][XLDS ? 1 : U][4];   // A operand: 8 k of one x row per lane per MFMA
};

// Activation row pitch in LDS, in bf16 elements: K plus 8 so that the 16 rows
// one A-operand read touches start in different banks.
__device__ __forceinline__ int lds_pitch(int k) { return k + 8; }

// C: 16-column tiles per wavefront.  MT: 16-row A tiles (1 for M <= 16).
// U: 128-k blocks per pipeline step.  OUT_F32: y element type.
//
// One workgroup owns 16*C output columns; its `waves` wavefronts cut K into
// `waves` equal segments.  Wavefront w sums segment w as one chain of MFMAs in
// increasing k, and the segment sums are added in segment order.  C and U
// change neither the chains nor the final sum: only the segment count enters
// the arithmetic, and it is fixed by the (N, K) tile.
//
// XLDS: x [M, K] is first copied into LDS (rows >= M are never read: their A
// operand is zero), so the weight pipeline holds only weights in registers.
// Otherwise (x too large for LDS) each chunk also fetches its A operands.
template <int C, int MT, int U, bool XLDS, bool OUT_F32>
__global__ void __launch_bounds__(512)
nvfp4_skinny(Args a) {
    extern __shared__ __align__(16) uint16_t lds[];   // x rows, then reused for segment partials
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int waves = blockDim.x / kWave;
    const int col_lane = lane % 16;                // B column / A row within a tile
    const int kq = lane / 16;                      // which 8-k quarter of an instruction
    const int col_base = blockIdx.x * 16 * C;
    const int64_t row_bytes = a.k / 2;
    const int64_t scale_bytes = a.k / 16;
    const int pitch = lds_pitch(a.k);

    // Columns past N and rows past M read a valid row instead (the last one):
    // MFMA output (m, n) depends only on A row m and B column n, and those
    // outputs are never stored, so every load can be unconditional and the
    // load/wait schedule stays free of branches.
    const uint8_t* wrow[C];
    const uint8_t* srow[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int n = min(col_base + 16 * c + col_lane, a.n - 1);
        wrow[c] = a.wp + n * row_bytes;
        srow[c] = a.sc + n * scale_bytes;
    }
    int xr[MT];                                    // x row feeding A row 16t + col_lane
    const uint16_t* xrow[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        xr[t] = min(16 * t + col_lane, a.m - 1);
        xrow[t] = a.x + (int64_t)xr[t] * a.k;
    }

    auto load = [&](Chunk<C, MT, U, XLDS>& ch, int kb) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = kb + kBlockK * u;
                ch.w[c][u] = load16_stream(wrow[c] + k / 2 + 16 * kq);
                ch.s[c][u] = load8_stream(srow[c] + k / 16);
            }
        }
        if constexpr (!XLDS) {
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        ch.x[t][u][s] = load16(xrow[t] + kb + kBlockK * u + 32 * kq + 8 * s);
        }
    };

    const int k0 = wave * a.k_per_wave;
    const int nchunks = a.k_per_wave / (kBlockK * U);
    Chunk<C, MT, U, XLDS> A, B;

    // Stage x[0:M, 0:K] in LDS.  The x loads go out first and the weight
    // loads of the first chunk right after, so storing x into LDS waits for
    // x alone.  Indices past the end are clamped (a repeated store of the
    // same value), which keeps the sequence free of branches.
    if constexpr (XLDS) {
        constexpr int kStage = 4;                  // 16-byte vectors per thread per round
        const int vec_per_row = a.k / 8;
        const int total = a.m * vec_per_row;
        const int per_round = kStage * (int)blockDim.x;
        auto stage_round = [&](int base, bool first) {
            u32x4 d[kStage];
            int v[kStage];
#pragma unroll
            for (int r = 0; r < kStage; ++r) {
                v[r] = min(base + r * (int)blockDim.x + (int)threadIdx.x, total - 1);
                d[r] = load16(a.x + (int64_t)(v[r] / vec_per_row) * a.k + (v[r] % vec_per_row) * 8);
            }
            if (first) load(A, k0);
#pragma unroll
            for (int r = 0; r < kStage; ++r)
                *reinterpret_cast<u32x4*>(lds + (v[r] / vec_per_row) * pitch + (v[r] % vec_per_row) * 8) = d[r];
        };
        stage_round(0, true);
        for (int base = per_round; base < total; base += per_round) stage_round(base, false);
        __syncthreads();
    } else {
        load(A, k0);
    }

    f32x4 acc[C][MT];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Chunk<C, MT, U, XLDS>& ch, int kb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = kb + kBlockK * u;
            u32x4 xa[MT][4];
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if constexpr (XLDS)
                        xa[t][s] = *reinterpret_cast<const u32x4*>(lds + xr[t] * pitch + k + 32 * kq + 8 * s);
                    else
                        xa[t][s] = ch.x[t][u][s];
                }
#pragma unroll
            for (int c = 0; c < C; ++c) {
                // lanes of quarter kq need scale bytes 2kq and 2kq+1 of the block
                const uint32_t d = static_cast<uint32_t>(ch.s[c][u] >> (16 * kq));
                const float g0 = __builtin_amdgcn_cvt_f32_fp8(d, 0);
                const float g1 = __builtin_amdgcn_cvt_f32_fp8(d, 1);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    bf16x8 b = decode8(ch.w[c][u][s], s < 2 ? g0 : g1);
#pragma unroll
                    for (int t = 0; t < MT; ++t)
                        acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[t][s]), b,
                                                                           acc[c][t], 0, 0, 0);
                }
            }
        }
    };

    // Software pipeline over the segment: chunk i+1 is loaded while chunk i is
    // multiplied.  Chunks are computed strictly in increasing k.
    int i = 0;
    for (; i + 2 <= nchunks; i += 2) {
        load(B, k0 + (i + 1) * kBlockK * U);
        compute(A, k0 + i * kBlockK * U);
        if (i + 2 < nchunks) load(A, k0 + (i + 2) * kBlockK * U);
        compute(B, k0 + (i + 1) * kBlockK * U);
    }
    if (i < nchunks) compute(A, k0 + i * kBlockK * U);

    // Segment partials, added in segment order: wavefront 0 keeps its own sum
    // in registers and adds those of wavefronts 1, 2, ... in turn.  The LDS
    // that held x is reused once every wavefront is done with it.
    if (waves > 1) {
        float* partials = reinterpret_cast<float*>(lds);
        __syncthreads();
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

// Persistent variant for x small enough to sit in LDS whole (the M = 1 GEMV
// regime and small M).  A few workgroups per CU walk the column tiles
// t = blockIdx.x, blockIdx.x + gridDim.x, ...; each tile is 16*C columns and
// its `waves` wavefronts take the same K segments as the non-persistent
// kernel, so every output has the same chain and the same segment order (the
// two variants give identical bits).  The weight stream of one wavefront is a
// single pipeline over (tile, chunk): the loads of the next chunk -- in the
// next tile at a tile boundary -- are in flight while the current chunk is
// decoded, and x is staged once per workgroup instead of once per tile.
template <int C, int MT, int U, bool OUT_F32>
__global__ void __launch_bounds__(512)
nvfp4_skinny_persistent(Args a) {
    extern __shared__ __align__(16) uint16_t lds[];   // x rows, then 2 x partial buffers
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int waves = blockDim.x / kWave;
    const int col_lane = lane % 16;
    const int kq = lane / 16;
    const uint32_t row_bytes = static_cast<uint32_t>(a.k) / 2;
    const uint32_t scale_bytes = static_cast<uint32_t>(a.k) / 16;
    const int pitch = lds_pitch(a.k);
    float* partials = reinterpret_cast<float*>(lds + a.m * pitch);   // [2][waves][C][MT][4][64]
    const int part_stride = waves * C * MT * 4 * kWave;

    const int tiles = (a.n + 16 * C - 1) / (16 * C);
    const int my_tiles = tiles > (int)blockIdx.x ? (tiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 0;
    const int k0 = wave * a.k_per_wave;
    const int nch = a.k_per_wave / (kBlockK * U);     // chunks per tile per wavefront
    const int total = my_tiles * nch;
    if (total == 0) return;                           // uniform over the workgroup

    int xr[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) xr[t] = min(16 * t + col_lane, a.m - 1);

    // chunk j -> tile blockIdx.x + (j / nch) * gridDim.x, k = k0 + (j % nch) * 128U
    auto load = [&](Chunk<C, MT, U, true>& ch, int j) {
        const int tile = (int)blockIdx.x + (j / nch) * (int)gridDim.x;
        const uint32_t kb = static_cast<uint32_t>(k0 + (j % nch) * kBlockK * U);
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const uint32_t n = static_cast<uint32_t>(min(tile * 16 * C + 16 * c + col_lane, a.n - 1));
            const uint8_t* wr = a.wp + static_cast<uint64_t>(n) * row_bytes + kb / 2 + 16 * kq;
            const uint8_t* sr = a.sc + static_cast<uint64_t>(n) * scale_bytes + kb / 16;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                ch.w[c][u] = load16_stream(wr + (kBlockK / 2) * u);
                ch.s[c][u] = load8_stream(sr + (kBlockK / 16) * u);
            }
        }
    };

    Chunk<C, MT, U, true> A, B;
    // Stage x first (all loads issued before the first weights), then the
    // first chunk's weights, then the LDS stores of x.
    {
        constexpr int kStage = 4;
        const int vec_per_row = a.k / 8;
        const int xtotal = a.m * vec_per_row;
        const int per_round = kStage * (int)blockDim.x;
        auto stage_round = [&](int base, bool first) {
            u32x4 d[kStage];
            int v[kStage];
#pragma unroll
            for (int r = 0; r < kStage; ++r) {
                v[r] = min(base + r * (int)blockDim.x + (int)threadIdx.x, xtotal - 1);
                d[r] = load16(a.x + (int64_t)(v[r] / vec_per_row) * a.k + (v[r] % vec_per_row) * 8);
            }
            if (first) load(A, 0);
#pragma unroll
            for (int r = 0; r < kStage; ++r)
                *reinterpret_cast<u32x4*>(lds + (v[r] / vec_per_row) * pitch + (v[r] % vec_per_row) * 8) = d[r];
        };
        stage_round(0, true);
        for (int base = per_round; base < xtotal; base += per_round) stage_round(base, false);
        __syncthreads();
    }

    f32x4 acc[C][MT];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Chunk<C, MT, U, true>& ch, int j) {
        const int kb = k0 + (j % nch) * kBlockK * U;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = kb + kBlockK * u;
            u32x4 xa[MT][4];
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    xa[t][s] = *reinterpret_cast<const u32x4*>(lds + xr[t] * pitch + k + 32 * kq + 8 * s);
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const uint32_t d = static_cast<uint32_t>(ch.s[c][u] >> (16 * kq));
                const float g0 = __builtin_amdgcn_cvt_f32_fp8(d, 0);
                const float g1 = __builtin_amdgcn_cvt_f32_fp8(d, 1);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    bf16x8 b = decode8(ch.w[c][u][s], s < 2 ? g0 : g1);
#pragma unroll
                    for (int t = 0; t < MT; ++t)
                        acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[t][s]), b,
                                                                           acc[c][t], 0, 0, 0);
                }
            }
        }
    };

    // After the last chunk of a tile: segment partials through LDS (two
    // buffers, so one barrier per tile), wavefront 0 adds them in segment
    // order, scales, rounds and stores.
    int parity = 0;
    auto finish_tile = [&](int j) {
        const int tile = (int)blockIdx.x + (j / nch) * (int)gridDim.x;
        float* buf = partials + parity * part_stride;
        parity ^= 1;
        if (waves > 1) {
            if (wave != 0) {
#pragma unroll
                for (int c = 0; c < C; ++c)
#pragma unroll
                    for (int t = 0; t < MT; ++t)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            buf[((wave * C + c) * MT + t) * 4 * kWave + jj * kWave + lane] = acc[c][t][jj];
            }
            __syncthreads();
        }
        if (wave == 0) {
            for (int w2 = 1; w2 < waves; ++w2) {
#pragma unroll
                for (int c = 0; c < C; ++c)
#pragma unroll
                    for (int t = 0; t < MT; ++t)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            acc[c][t][jj] += buf[((w2 * C + c) * MT + t) * 4 * kWave + jj * kWave + lane];
            }
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int n = tile * 16 * C + 16 * c + col_lane;
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int m = 16 * t + 4 * kq + jj;
                        if (m < a.m && n < a.n) {
                            float r = acc[c][t][jj] * a.t;
                            if (OUT_F32)
                                static_cast<float*>(a.y)[(int64_t)m * a.n + n] = r;
                            else
                                static_cast<uint16_t*>(a.y)[(int64_t)m * a.n + n] = f32_to_bf16_rne(r);
                        }
                    }
            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // One pipeline over all (tile, chunk) of this wavefront; the loads past
    // the end repeat the last chunk (never computed), keeping them unconditional.
    for (int j = 0; j < total; j += 2) {
        load(B, min(j + 1, total - 1));
        compute(A, j);
        if (j % nch == nch - 1) finish_tile(j);
        if (j + 1 >= total) break;
        load(A, min(j + 2, total - 1));
        compute(B, j + 1);
        if ((j + 1) % nch == nch - 1) finish_tile(j + 1);
    }
}

using KernelFn = void (*)(Args);

template <int C, int MT, int U>
KernelFn pick_out(bool xlds, int y_dtype) {
    if (xlds)
        return y_dtype == NVFP4_OUT_F32 ? nvfp4_skinny<C, MT, U, true, true> : nvfp4_skinny<C, MT, U, true, false>;
    return y_dtype == NVFP4_OUT_F32 ? nvfp4_skinny<C, MT, U, false, true> : nvfp4_skinny<C, MT, U, false, false>;
}

template <int C, int MT>
KernelFn pick_u(int unroll, bool xlds, int y_dtype) {
    switch (unroll) {
        case 1: return pick_out<C, MT, 1>(xlds, y_dtype);
        case 2: return pick_out<C, MT, 2>(xlds, y_dtype);
        default: return pick_out<C, MT, 4>(xlds, y_dtype);
    }
}

template <int MT>
KernelFn pick_c(int cols, int unroll, bool xlds, int y_dtype) {
    switch (cols) {
        case 16: return pick_u<1, MT>(unroll, xlds, y_dtype);
        case 32: return pick_u<2, MT>(unroll, xlds, y_dtype);
        default: return pick_u<4, MT>(unroll, xlds, y_dtype);
    }
}

KernelFn pick_kernel(int mt, int cols, int unroll, bool xlds, int y_dtype) {
    return mt == 1 ? pick_c<1>(cols, unroll, xlds, y_dtype) : pick_c<2>(cols, unroll, xlds, y_dtype);
}

template <int C, int MT, int U>
KernelFn pick_p_out(int y_dtype) {
    return y_dtype == NVFP4_OUT_F32 ? nvfp4_skinny_persistent<C, MT, U, true>
                                    : nvfp4_skinny_persistent<C, MT, U, false>;
}

template <int C, int MT>
KernelFn pick_p_u(int unroll, int y_dtype) {
    switch (unroll) {
        case 1: return pick_p_out<C, MT, 1>(y_dtype);
        case 2: return pick_p_out<C, MT, 2>(y_dtype);
        default: return pick_p_out<C, MT, 4>(y_dtype);
    }
}

KernelFn pick_persistent(int mt, int cols, int unroll, int y_dtype) {
    if (mt == 1) return cols == 16 ? pick_p_u<1, 1>(unroll, y_dtype) : pick_p_u<2, 1>(unroll, y_dtype);
    return cols == 16 ? pick_p_u<1, 2>(unroll, y_dtype) : pick_p_u<2, 2>(unroll, y_dtype);
}

// Multiprocessor count per device, filled by nvfp4_init.
constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices] = {};

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
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess) { g_init_status = NVFP4_ERR_HIP; return; }
    for (int d = 0; d < ndev && d < kMaxDevices; ++d) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, d) != hipSuccess) { g_init_status = NVFP4_ERR_HIP; return; }
        g_cu_count[d] = p.multiProcessorCount;
    }
    // Touch every kernel so its code object is loaded before any graph capture.
    const int cols[3] = {16, 32, 64};
    for (int mt = 1; mt <= 2; ++mt)
        for (int ci = 0; ci < 3; ++ci)
            for (int un = 1; un <= 4; un *= 2)
                for (int xl = 0; xl <= 1; ++xl)
                for (int od = 0; od <= 1; ++od) {
                    const void* fn = reinterpret_cast<const void*>(pick_kernel(mt, cols[ci], un, xl != 0, od));
                    hipFuncAttributes attr;
                    if (hipFuncGetAttributes(&attr, fn) != hipSuccess ||
                        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                            kMaxLdsBytes) != hipSuccess) {
                        g_init_status = NVFP4_ERR_HIP;
                        return;
                    }
                }
    for (int mt = 1; mt <= 2; ++mt)
        for (int cc = 16; cc <= 32; cc += 16)
            for (int un = 1; un <= 4; un *= 2)
                for (int od = 0; od <= 1; ++od) {
                    const void* fn = reinterpret_cast<const void*>(pick_persistent(mt, cc, un, od));
                    hipFuncAttributes attr;
                    if (hipFuncGetAttributes(&attr, fn) != hipSuccess ||
                        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                            kMaxLdsBytes) != hipSuccess) {
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

namespace {

int launch(const void* x_bf16, const uint8_t* w_packed, const uint8_t* scales_e4m3, float tensor_scale,
           void* y, int64_t m, int64_t n, int64_t k, int y_dtype, void* stream, const nvfp4::Tile& tile) {
    int st = nvfp4_linear_shape_ok(m, n, k);
    if (st != NVFP4_OK) return st;
    if (y_dtype != NVFP4_OUT_BF16 && y_dtype != NVFP4_OUT_F32) return NVFP4_ERR_DTYPE;
    if (m == 0) return NVFP4_OK;
    if (!x_bf16 || !w_packed || !scales_e4m3 || !y) return NVFP4_ERR_NULL;
    auto misaligned = [](const void* p, uintptr_t al) { return (reinterpret_cast<uintptr_t>(p) & (al - 1)) != 0; };
    if (misaligned(x_bf16, 16) || misaligned(w_packed, 16) || misaligned(scales_e4m3, 16) ||
        misaligned(y, y_dtype == NVFP4_OUT_F32 ? 4 : 2))
        return NVFP4_ERR_ALIGN;
    st = nvfp4_init();
    if (st != NVFP4_OK) return st;

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
    // x [M, K] small enough to share the LDS of one workgroup with two
    // buffers of segment partials, in at most 64 KB so a CU holds two such
    // workgroups: the persistent kernel.
    const size_t x_bytes = size_t(m) * (k + 8) * sizeof(uint16_t);
    const size_t pers_bytes = x_bytes + 2 * size_t(tile.waves) * c * mt * 4 * kWave * sizeof(float);
    if (tile.cols <= 32 && pers_bytes <= size_t(64 * 1024)) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return NVFP4_ERR_HIP;
        const int cus = dev < kMaxDevices && g_cu_count[dev] > 0 ? g_cu_count[dev] : 256;
        const int64_t tiles = (n + tile.cols - 1) / tile.cols;
        const int per_cu = tile.waves >= 8 ? 2 : 4;
        const int64_t grid_p = tiles < int64_t(per_cu) * cus ? tiles : int64_t(per_cu) * cus;
        hipLaunchKernelGGL(pick_persistent(mt, tile.cols, tile.unroll, y_dtype),
                           dim3(static_cast<unsigned>(grid_p)), dim3(static_cast<unsigned>(kWave * tile.waves)),
                           pers_bytes, static_cast<hipStream_t>(stream), a);
        if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
        return NVFP4_OK;
    }
    // Otherwise the per-tile kernel; x goes through LDS when it fits in 64 KB.
    // With x fetched per chunk, one 128-k block per step keeps the A operands
    // of two row tiles in registers (the pipeline depth never changes bits).
    const bool xlds = x_bytes <= size_t(64 * 1024);
    const size_t part_bytes = tile.waves > 1 ? size_t(tile.waves) * c * mt * 4 * kWave * sizeof(float) : 0;
    const size_t lds = xlds && x_bytes > part_bytes ? x_bytes : part_bytes;
    const dim3 grid(static_cast<unsigned>((n + tile.cols - 1) / tile.cols));
    const dim3 block(static_cast<unsigned>(kWave * tile.waves));
    const int unroll = xlds ? tile.unroll : 1;
    hipLaunchKernelGGL(pick_kernel(mt, tile.cols, unroll, xlds, y_dtype), grid, block, lds,
                       static_cast<hipStream_t>(stream), a);
    if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
    return NVFP4_OK;
}

}  // namespace

extern "C" int nvfp4_linear(const void* x_bf16, const uint8_t* w_packed, const uint8_t* scales_e4m3,
                            float tensor_scale, void* y, int64_t m, int64_t n, int64_t k, int y_dtype,
                            void* stream) {
    int st = nvfp4_linear_shape_ok(m, n, k);
    if (st != NVFP4_OK) return st;
    if (nvfp4::load_tile_override() != NVFP4_OK) return NVFP4_ERR_TILEFILE;
    return launch(x_bf16, w_packed, scales_e4m3, tensor_scale, y, m, n, k, y_dtype, stream,
                  nvfp4::tile_for(n, k));
}

extern "C" int nvfp4_linear_tiled(const void* x_bf16, const uint8_t* w_packed, const uint8_t* scales_e4m3,
                                  float tensor_scale, void* y, int64_t m, int64_t n, int64_t k, int y_dtype,
                                  int cols, int waves, int unroll, void* stream) {
    int st = nvfp4_linear_shape_ok(m, n, k);
    if (st != NVFP4_OK) return st;
    nvfp4::Tile tile;
    tile.cols = cols;
    tile.waves = waves;
    tile.unroll = unroll;
    if (!nvfp4::tile_valid(tile, n, k)) return NVFP4_ERR_TILE;
    return launch(x_bf16, w_packed, scales_e4m3, tensor_scale, y, m, n, k, y_dtype, stream, tile);
}
