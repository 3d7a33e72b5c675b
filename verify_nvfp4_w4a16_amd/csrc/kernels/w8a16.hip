// FP8 block-scaled weight-only product (W8A16) for 1..32 rows:
//   y[m, n] = sum over 128-k blocks b of S[n / 128, b] * (sum_{k in b} x[m, k] * e4m3(B[n, k]))
// "10 Kernels" 10.3: the checkpoint's block-scaled FP8 read as stored, a tile
// 128 wide along K so that each step covers one scale block, the scale one
// number applied to the fp32 sum; "Module ops" w8a16_gemm / w8a16_tc_rows
// (weight [N, K] e4m3, block scale [N/128, K/128] fp32, N and K multiples of
// 128).
//
// Same machine layout as the NVFP4 kernels' register path: a workgroup per
// 16 output columns, its wavefronts one K segment each, weights loaded into
// registers (two 16-byte loads per lane per 128-k block, 64 contiguous bytes
// of a row per load instruction) and converted exactly to the bf16 B operand
// of v_mfma_f32_16x16x32_bf16 by v_cvt_scalef32_pk_bf16_fp8 at scale 1 (e4m3
// has 4 significant bits).  Each block's four MFMAs start from zero; the block
// sum joins the segment's chain as fma(S, block, chain), blocks in increasing
// k; the segment chains are added in the two-level order of the (N, K) tile,
// so a row's bits do not depend on M or on the other rows ("10 Kernels" 10.1).
//
// Where x does not fit the LDS, fp8_w8a16_linear runs the NVFP4 many-row
// kernel's FP8 form instead (fp8_w8a16_split, nvfp4_linear.hip): x in 512-k
// windows shared by the workgroup's 16-column wavefronts, the codes and scales
// by direct-to-LDS loads, the same MFMA inputs, block chains and two-level
// order, the segment groups meeting through the tagged exchange.
//
// fp8_w8a16_gemm_kernel is the same product for any row count (the pages'
// w8a16_gemm_n128_m128 and pipelined forms for prefill chunks), laid out like
// nvfp4_gemm_kernel: one workgroup of eight wavefronts per CU owns 128 rows x
// 128 columns (wavefronts 2 x 4, each 64 rows x 32 columns), x and the e4m3
// codes come into LDS by direct-to-LDS loads two 128-k blocks ahead, and each
// wavefront walks every segment of K in order, so the MFMA inputs, the block
// chains and the two-level fold are those of fp8_w8a16_kernel: every row has
// the bits fp8_w8a16_linear gives it.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "nvfp4_w4a16.h"
#include "nvfp4_common.h"
#include "setup.h"
#include "../host/tiles.h"

namespace {

constexpr int kFp8Block = 128;

struct W8Args {
    const uint16_t* x;     // bf16 [M, K]
    const uint8_t* w;      // e4m3 [N, K]
    const float* s;        // fp32 [N/128, K/128]
    void* y;               // [M, N]
    int m, n, k;
    int k_per_wave;        // segment length, a multiple of 128
    int group;             // segments per segment group
    float* part;           // parts > 1: group sums [parts][M][N]; workgroup (x, y) runs group y
    int parts;
};

template <int MT, int C, bool XLDS>
struct W8Chunk {
    u32x4 w[C][2];         // per column tile: bytes 16 kq .. +15 and 64 + 16 kq .. +15 of the lane's row
    float s;               // the block's scale (the wavefront's 16 C columns lie in one 128-row block)
    u32x4 x[XLDS ? 1 : MT][XLDS ? 1 : 4];
};

// MFMA s of a block takes, in lane quarter kq, k = 64 (s / 2) + 16 kq + 8 (s % 2) .. + 7
// of the block, for the weight and the activation alike.
__device__ __forceinline__ int slot_k(int s, int kq) { return 64 * (s / 2) + 16 * kq + 8 * (s % 2); }

// C column tiles per wavefront share every x operand (x read once per 16 C
// columns where it does not fit the LDS).
template <int MT, int C, bool XLDS, bool OUT_F32>
__global__ void __launch_bounds__(512)
fp8_w8a16_kernel(W8Args a) {
    extern __shared__ __align__(16) uint16_t lds[];
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int waves = blockDim.x / kWave;
    const int col_lane = lane % 16;
    const int kq = lane / 16;
    const int col_base = blockIdx.x * 16 * C;   // N is a multiple of 128 and of 16 C: no column past N
    const int pitch = a.k + 8;
    const int kblocks = a.k / kFp8Block;
    const uint8_t* wrow[C];
#pragma unroll
    for (int c = 0; c < C; ++c) wrow[c] = a.w + (int64_t)(col_base + 16 * c + col_lane) * a.k;
    const float* srow = a.s + (int64_t)(col_base / kFp8Block) * kblocks;
    int xr[MT];
    const uint16_t* xrow[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        xr[t] = min(16 * t + col_lane, a.m - 1);
        xrow[t] = a.x + (int64_t)xr[t] * a.k;
    }
    if constexpr (XLDS) {
        const int vec_per_row = a.k / 8;
        const int total = a.m * vec_per_row;
        for (int v = threadIdx.x; v < total; v += blockDim.x) {
            const int r = v / vec_per_row, c = v % vec_per_row;
            *reinterpret_cast<u32x4*>(lds + r * pitch + 8 * c) = load16(a.x + (int64_t)r * a.k + 8 * c);
        }
        __syncthreads();
    }

    auto load = [&](W8Chunk<MT, C, XLDS>& ch, int kb) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            ch.w[c][0] = load16_stream(wrow[c] + kb + 16 * kq);
            ch.w[c][1] = load16_stream(wrow[c] + kb + 64 + 16 * kq);
        }
        ch.s = srow[kb / kFp8Block];
        if constexpr (!XLDS) {
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int s = 0; s < 4; ++s) ch.x[t][s] = load16(xrow[t] + kb + slot_k(s, kq));
        }
    };

    f32x4 acc[C][MT];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const W8Chunk<MT, C, XLDS>& ch, int kb) {
        f32x4 blk[C][MT];
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int t = 0; t < MT; ++t) blk[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 b[C];
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const u32x4 p = ch.w[c][s / 2];
                b[c] = fp8x8_to_bf16(p[2 * (s % 2)], p[2 * (s % 2) + 1]);
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                u32x4 xa;
                if constexpr (XLDS)
                    xa = *reinterpret_cast<const u32x4*>(lds + xr[t] * pitch + kb + slot_k(s, kq));
                else
                    xa = ch.x[t][s];
#pragma unroll
                for (int c = 0; c < C; ++c)
                    blk[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), b[c], blk[c][t], 0, 0, 0);
            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[c][t][j] = __builtin_fmaf(ch.s, blk[c][t][j], acc[c][t][j]);
    };

    const int k0 = ((int)blockIdx.y * waves + wave) * a.k_per_wave;   // blockIdx.y > 0 only when K is split
    const int nchunks = a.k_per_wave / kFp8Block;
    W8Chunk<MT, C, XLDS> A, B;
    load(A, k0);
    int i = 0;
    for (; i + 2 <= nchunks; i += 2) {
        load(B, k0 + (i + 1) * kFp8Block);
        compute(A, k0 + i * kFp8Block);
        if (i + 2 < nchunks) load(A, k0 + (i + 2) * kFp8Block);
        compute(B, k0 + (i + 1) * kFp8Block);
    }
    if (i < nchunks) compute(A, k0 + i * kFp8Block);

    // segment chains in the two-level order, through the LDS that held x
    if (waves > 1) {
        f32x4 tot[C][MT];
        float* partials = reinterpret_cast<float*>(lds);
        __syncthreads();
        if (wave != 0) {
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        partials[(((wave * C + c) * MT + t) * 4 + j) * kWave + lane] = acc[c][t][j];
        }
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int t = 0; t < MT; ++t) tot[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int w2 = 1; w2 < waves; ++w2) {
            const bool starts = w2 % a.group == 0;
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const float* p = partials + ((w2 * C + c) * MT + t) * 4 * kWave + lane;
                    const f32x4 v = f32x4{p[0], p[kWave], p[2 * kWave], p[3 * kWave]};
                    const f32x4 closed = w2 == a.group ? acc[c][t] : tot[c][t] + acc[c][t];
                    tot[c][t] = starts ? closed : tot[c][t];
                    acc[c][t] = starts ? v : acc[c][t] + v;
                }
        }
        if (a.group < waves) {
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[c][t] = tot[c][t] + acc[c][t];
        }
    }
    // this workgroup's group sum, when the groups are added by a second kernel
    void* out = a.y;
    const bool part_out = a.parts > 1;
    if (part_out) out = a.part + (int64_t)blockIdx.y * a.m * a.n;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int n = col_base + 16 * c + col_lane;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = 16 * t + 4 * kq + j;
                if (m < a.m && part_out) {
                    static_cast<float*>(out)[(int64_t)m * a.n + n] = acc[c][t][j];
                } else if (m < a.m) {
                    if (OUT_F32)
                        static_cast<float*>(a.y)[(int64_t)m * a.n + n] = acc[c][t][j];
                    else
                        static_cast<uint16_t*>(a.y)[(int64_t)m * a.n + n] = f32_to_bf16_rne(acc[c][t][j]);
                }
            }
    }
}

// ---- many rows ----------------------------------------------------------

constexpr int kGRows = 128;                 // rows per workgroup
constexpr int kGCols = 128;                 // columns per workgroup: one scale block
constexpr int kGMT = 4;                     // 16-row tiles per wavefront
constexpr int kGC = 2;                      // 16-column tiles per wavefront
constexpr int kGWavesN = kGCols / (16 * kGC);
constexpr int kGWaves = (kGRows / (16 * kGMT)) * kGWavesN;
constexpr int kGThreads = kGWaves * kWave;
constexpr int kGXRowsPerWave = kGRows / kGWaves;
constexpr int kGXLoads = kGXRowsPerWave / 4;                 // 1 KB direct loads of x per wavefront per block
constexpr int kGRing = 3;                                    // blocks in the LDS rings
constexpr size_t kGXBytes = size_t(kGRing) * kGRows * kFp8Block * sizeof(uint16_t);
// per block: the codes of the 128 columns (per column tile two 1 KB halves:
// lane l of half h holds column 16 c + l % 16, bytes 64 h + 16 (l / 16) .. +15
// of the block), then each wavefront's copy of the block's scale (256 B: one
// float per lane, all equal)
constexpr int kGWCodes = kGCols * kFp8Block;
constexpr int kGWStage = kGWCodes + kGWaves * 256;
constexpr size_t kGLds = kGXBytes + size_t(kGRing) * kGWStage;
constexpr int kGWTilesPerWave = kGCols / 16 / kGWaves;
constexpr int kGWLoads = 3 * kGWTilesPerWave;                // per block: two code halves and the scale
static_assert(kGWTilesPerWave == 1, "one column tile staged per wavefront");
static_assert(kGXLoads * 4 * kGWaves == kGRows, "x staging");
static_assert(kGLds <= size_t(kMaxLdsBytes), "LDS");

struct W8GemmArgs {
    const uint16_t* x;     // bf16 [M, K]
    const uint8_t* w;      // e4m3 [N, K]
    const float* s;        // fp32 [N/128, K/128]
    void* y;               // [M, N]
    int m, n, k;
    int k_per_wave;        // segment length (fp8_tile)
    int group;             // segments per segment group
    float* part;           // parts > 1: group sums [parts][M][N] (blockIdx.z is the group)
    int parts;
};

template <bool OUT_F32>
__global__ void __launch_bounds__(kGThreads, 1)
fp8_w8a16_gemm_kernel(W8GemmArgs a) {
    extern __shared__ __align__(16) uint16_t xs[];     // [kGRing][kGRows][128], then the weight ring
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / kGWavesN, wn = wave % kGWavesN;
    const int col_lane = lane % 16;
    const int kq = lane / 16;
    const int row0 = blockIdx.y * kGRows;
    const int colwg = blockIdx.x * kGCols;
    const int col0 = colwg + wn * kGC * 16;
    const int nblocks = a.k / kFp8Block / a.parts;
    const int kbase = static_cast<int>(blockIdx.z) * nblocks * kFp8Block;
    const int seg_blocks = a.k_per_wave / kFp8Block;

    // x rows as in nvfp4_gemm_kernel: row r's 16-byte piece p sits at slot
    // p ^ (r % 16), so the 16 rows of one A read meet 16 bank groups
    const int xslot = lane % 16;
    const char* xwg = reinterpret_cast<const char*>(a.x + (int64_t)row0 * a.k + kbase);
    uint32_t xoff[kGXLoads];
#pragma unroll
    for (int i = 0; i < kGXLoads; ++i) {
        const int r = kGXRowsPerWave * wave + 4 * i + lane / 16;
        const int rr = min(row0 + r, a.m - 1) - row0;          // rows past M read row M - 1 (never stored)
        xoff[i] = static_cast<uint32_t>(rr * a.k + 8 * (xslot ^ (r % 16))) * 2u;
    }
    auto load_x = [&](int kl, int buf) {
        const char* base = xwg + 2 * kl;
#pragma unroll
        for (int i = 0; i < kGXLoads; ++i)
            __builtin_amdgcn_global_load_lds(base + xoff[i],
                                             xs + (buf * kGRows + kGXRowsPerWave * wave + 4 * i) * kFp8Block, 16, 0, 0);
    };
    // wavefront w stages column tile w of each block and a copy of its scale
    uint8_t* wls = reinterpret_cast<uint8_t*>(xs) + kGXBytes;
    const uint8_t* wsrc = a.w + (int64_t)(colwg + 16 * wave + lane % 16) * a.k + kbase + 16 * (lane / 16);
    const float* ssrc = a.s + (int64_t)(colwg / kFp8Block) * (a.k / kFp8Block) + kbase / kFp8Block;
    auto load_w = [&](int kl, int st) {
        uint8_t* d = wls + st * kGWStage;
        __builtin_amdgcn_global_load_lds(wsrc + kl, d + wave * 2048, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(wsrc + kl + 64, d + wave * 2048 + 1024, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(ssrc + kl / kFp8Block, d + kGWCodes + wave * 256, 4, 0, 0);
    };

    f32x4 blk[kGMT][kGC], acc[kGMT][kGC], grp[kGMT][kGC], tot[kGMT][kGC];
#pragma unroll
    for (int t = 0; t < kGMT; ++t)
#pragma unroll
        for (int c = 0; c < kGC; ++c) acc[t][c] = grp[t][c] = tot[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    load_x(0, 0);
    load_w(0, 0);
    if (nblocks > 1) {
        load_x(kFp8Block, 1);
        load_w(kFp8Block, 1);
        gemm_wait_vm<kGXLoads + kGWLoads>();              // block 0 has landed
    } else {
        gemm_wait_vm<0>();
    }
    gemm_lds_barrier();

    const int nseg = nblocks / seg_blocks;
    for (int sg = 0; sg < nseg; ++sg) {
      for (int bb = 0; bb < seg_blocks; ++bb) {
        const int b = sg * seg_blocks + bb;
        if (b + 2 < nblocks) {
            load_x((b + 2) * kFp8Block, (b + 2) % kGRing);
            load_w((b + 2) * kFp8Block, (b + 2) % kGRing);
        }
        const uint16_t* xb = xs + (b % kGRing) * kGRows * kFp8Block;
        const uint8_t* wst = wls + (b % kGRing) * kGWStage;
        u32x4 wv[kGC][2];
#pragma unroll
        for (int c = 0; c < kGC; ++c) {
            const int ct = wn * kGC + c;
            wv[c][0] = *reinterpret_cast<const u32x4*>(wst + ct * 2048 + 16 * lane);
            wv[c][1] = *reinterpret_cast<const u32x4*>(wst + ct * 2048 + 1024 + 16 * lane);
        }
        const float scale = *reinterpret_cast<const float*>(wst + kGWCodes + wave * 256 + 4 * lane);
        // A operands one MFMA step ahead; step s takes k = slot_k(s, kq) .. + 7
        u32x4 xa[2][kGMT];
        auto read_a = [&](u32x4 (&dst)[kGMT], int s) {
            const int piece = slot_k(s, kq) / 8;
#pragma unroll
            for (int t = 0; t < kGMT; ++t) {
                const int r = wm * 16 * kGMT + 16 * t + col_lane;
                dst[t] = *reinterpret_cast<const u32x4*>(xb + r * kFp8Block + 8 * (piece ^ col_lane));
            }
        };
#pragma unroll
        for (int t = 0; t < kGMT; ++t)
#pragma unroll
            for (int c = 0; c < kGC; ++c) blk[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        read_a(xa[0], 0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) read_a(xa[(s + 1) & 1], s + 1);
            bf16x8 bv[kGC];
#pragma unroll
            for (int c = 0; c < kGC; ++c) {
                const u32x4 q = wv[c][s / 2];
                bv[c] = fp8x8_to_bf16(q[2 * (s % 2)], q[2 * (s % 2) + 1]);
            }
#pragma unroll
            for (int t = 0; t < kGMT; ++t)
#pragma unroll
                for (int c = 0; c < kGC; ++c)
                    blk[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[s & 1][t]), bv[c], blk[t][c],
                                                                        0, 0, 0);
        }
        // the block sum joins the segment's chain with its scale
#pragma unroll
        for (int t = 0; t < kGMT; ++t)
#pragma unroll
            for (int c = 0; c < kGC; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[t][c][j] = __builtin_fmaf(scale, blk[t][c][j], acc[t][c][j]);
        if (b + 1 < nblocks) {
            if (b + 2 < nblocks)
                gemm_wait_vm<kGXLoads + kGWLoads>();      // block b + 1 has landed
            else
                gemm_wait_vm<0>();
            gemm_lds_barrier();
        }
      }
      // end of segment sg: the two-level order of the tile
      {
        const bool gfirst_seg = sg % a.group == 0;
        const bool gend = (sg + 1) % a.group == 0;
        const bool first_group = sg / a.group == 0;
#pragma unroll
        for (int t = 0; t < kGMT; ++t)
#pragma unroll
            for (int c = 0; c < kGC; ++c) {
                grp[t][c] = gfirst_seg ? acc[t][c] : grp[t][c] + acc[t][c];
                acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (gend) tot[t][c] = first_group ? grp[t][c] : tot[t][c] + grp[t][c];
            }
      }
    }

    const bool part_out = a.parts > 1;
    float* dst = part_out ? a.part + (int64_t)blockIdx.z * a.m * a.n : nullptr;
#pragma unroll
    for (int t = 0; t < kGMT; ++t)
#pragma unroll
        for (int c = 0; c < kGC; ++c) {
            const int n = col0 + 16 * c + col_lane;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = row0 + wm * 16 * kGMT + 16 * t + 4 * kq + j;
                if (m >= a.m) continue;
                if (part_out)
                    dst[(int64_t)m * a.n + n] = grp[t][c][j];
                else if (OUT_F32)
                    static_cast<float*>(a.y)[(int64_t)m * a.n + n] = tot[t][c][j];
                else
                    static_cast<uint16_t*>(a.y)[(int64_t)m * a.n + n] = f32_to_bf16_rne(tot[t][c][j]);
            }
        }
}

using W8Fn = void (*)(W8Args);

template <int MT>
W8Fn pick_w8_mt(int c, bool xlds, bool f) {
    if (xlds) return f ? fp8_w8a16_kernel<MT, 1, true, true> : fp8_w8a16_kernel<MT, 1, true, false>;
    if (c == 2) return f ? fp8_w8a16_kernel<MT, 2, false, true> : fp8_w8a16_kernel<MT, 2, false, false>;
    return f ? fp8_w8a16_kernel<MT, 1, false, true> : fp8_w8a16_kernel<MT, 1, false, false>;
}

// c: column tiles per wavefront, 1 or 2 (2 only with x read from memory)
W8Fn pick_w8(int mt, int c, bool xlds, int y_dtype) {
    const bool f = y_dtype == NVFP4_OUT_F32;
    return mt == 1 ? pick_w8_mt<1>(c, xlds, f) : pick_w8_mt<2>(c, xlds, f);
}

constexpr size_t kXLdsMax = 64 * 1024;

// Segments of the FP8 tile: K cut into the most of 8, 4, 2, 1 equal parts of
// whole 128-k blocks; groups of them by the NVFP4 table's default rule.  A
// function of (N, K) only.
void fp8_tile(int64_t n, int64_t k, int* waves, int* group) {
    const int64_t blocks = k / kFp8Block;
    int w = 8;
    while (w > 1 && blocks % w != 0) w /= 2;
    *waves = w;
    *group = w / nvfp4::default_split(n, w);
}

}  // namespace

namespace nvfp4 {

int w8a16_setup() {
    for (int od = 0; od <= 1; ++od)
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(od ? fp8_w8a16_gemm_kernel<true>
                                                                  : fp8_w8a16_gemm_kernel<false>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kGLds)) != hipSuccess)
            return NVFP4_ERR_HIP;
    for (int mt = 1; mt <= 2; ++mt)
        for (int c = 1; c <= 2; ++c)
            for (int xl = 0; xl <= 1; ++xl)
                for (int od = 0; od <= 1; ++od)
                    if (hipFuncSetAttribute(reinterpret_cast<const void*>(pick_w8(mt, c, xl != 0, od)),
                                            hipFuncAttributeMaxDynamicSharedMemorySize,
                                            static_cast<int>(kXLdsMax)) != hipSuccess)
                        return NVFP4_ERR_HIP;
    return NVFP4_OK;
}

}  // namespace nvfp4

extern "C" int fp8_w8a16_linear(const void* x_bf16, const uint8_t* w_e4m3, const float* block_scales, void* y,
                                int64_t m, int64_t n, int64_t k, int y_dtype, void* stream) {
    int st = fp8_w8a16_shape_ok(m, n, k);
    if (st != NVFP4_OK) return st;
    if (y_dtype != NVFP4_OUT_BF16 && y_dtype != NVFP4_OUT_F32) return NVFP4_ERR_DTYPE;
    if (m == 0) return NVFP4_OK;
    if (!x_bf16 || !w_e4m3 || !block_scales || !y) return NVFP4_ERR_NULL;
    auto misaligned = [](const void* p, uintptr_t al) { return (reinterpret_cast<uintptr_t>(p) & (al - 1)) != 0; };
    if (misaligned(x_bf16, 16) || misaligned(w_e4m3, 16) || misaligned(block_scales, 4) ||
        misaligned(y, y_dtype == NVFP4_OUT_F32 ? 4 : 2))
        return NVFP4_ERR_ALIGN;
    st = nvfp4::device_setup();
    if (st != NVFP4_OK) return st;
    W8Args a;
    a.x = static_cast<const uint16_t*>(x_bf16);
    a.w = w_e4m3;
    a.s = block_scales;
    a.y = y;
    a.m = static_cast<int>(m);
    a.n = static_cast<int>(n);
    a.k = static_cast<int>(k);
    int waves = 1, group = 1;
    fp8_tile(n, k, &waves, &group);
    a.k_per_wave = static_cast<int>(k / waves);
    a.group = group;
    a.part = nullptr;
    a.parts = 1;
    const int mt = m <= 16 ? 1 : 2;
    const size_t x_bytes = size_t(m) * (k + 8) * sizeof(uint16_t);
    const bool xlds = x_bytes <= kXLdsMax;
    if (!xlds) {
        // The many-row kernel where its segments are whole 512-k windows: x
        // comes in windows shared by a workgroup's columns and the codes by
        // direct-to-LDS loads.  Every segment group in one workgroup where
        // that still gives each CU a workgroup (the most wavefronts per
        // workgroup that do and whose LDS fits), else four wavefronts with the
        // groups meeting through the workspace.  Same bits as the kernel
        // below.  Measured on MI355X on the decode round's shapes against it:
        // 1.11-1.46x faster at 16 and 32 rows (24576x4096 at 16 rows: 22.3
        // against 32.6 us), 0.96-1.3x at 8 rows.
        const int cus = nvfp4::device_cus();
        bool launched = false;
        for (int w : {6, 4, 2}) {
            if (n / (16 * w) < cus) continue;
            st = nvfp4::launch_fp8_split(x_bf16, w_e4m3, block_scales, y, m, n, k, y_dtype, waves, group, w, true,
                                         stream, &launched);
            if (st != NVFP4_OK || launched) return st;
        }
        st = nvfp4::launch_fp8_split(x_bf16, w_e4m3, block_scales, y, m, n, k, y_dtype, waves, group, 4, false,
                                     stream, &launched);
        if (st != NVFP4_OK || launched) return st;
    }
    // Otherwise, where x is read from memory, each workgroup reads its x
    // slice once for its 16 c columns: two column tiles per wavefront halve
    // those reads where 32-column workgroups still cover the CUs.  Where they do not and
    // there are two row tiles (x reads largest), K is split into the tile's
    // segment groups instead, one per workgroup, their sums added in order
    // by a second kernel through the buffer nvfp4_init allocates (same bits).
    // Measured on MI355X at 16 and 32 rows on the decode round's shapes:
    // two tiles 1.1-1.3x faster on 8192 and 24576 columns; the split with two
    // tiles 1.04-1.14x faster on 4096 columns at 32 rows and no faster
    // elsewhere; four tiles never faster than two.
    int c = 1, parts = 1;
    float* buf = nullptr;
    if (!xlds) {
        const int cus = nvfp4::device_cus();
        const int split = waves / group;
        if (n / 32 >= cus) {
            c = 2;
        } else if (mt == 2 && split > 1 && (n / 32) * split >= cus) {
            size_t bytes = 0;
            int cus2 = cus;
            st = nvfp4::gemm_partials(&buf, &bytes, &cus2);
            if (st != NVFP4_OK) return st;
            if (buf && size_t(split) * size_t(m) * size_t(n) * 4 <= bytes) {
                c = 2;
                parts = split;
            }
        }
    }
    const int wg_waves = waves / parts;
    if (parts > 1) {
        a.part = buf;
        a.parts = parts;
    }
    const size_t part_bytes = wg_waves > 1 ? size_t(wg_waves) * c * mt * 4 * kWave * sizeof(float) : 0;
    const size_t lds = xlds && x_bytes > part_bytes ? x_bytes : part_bytes;
    hipLaunchKernelGGL(pick_w8(mt, c, xlds, y_dtype), dim3(static_cast<unsigned>(n / (16 * c)), parts),
                       dim3(static_cast<unsigned>(kWave * wg_waves)), lds, static_cast<hipStream_t>(stream), a);
    if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
    if (parts > 1) return nvfp4::launch_ordered_sum(buf, parts, m * n, 1.0f, y, y_dtype, stream);
    return NVFP4_OK;
}

extern "C" int fp8_w8a16_gemm(const void* x_bf16, const uint8_t* w_e4m3, const float* block_scales, void* y,
                              int64_t m, int64_t n, int64_t k, int y_dtype, void* stream) {
    int st = fp8_w8a16_gemm_shape_ok(m, n, k);
    if (st != NVFP4_OK) return st;
    if (y_dtype != NVFP4_OUT_BF16 && y_dtype != NVFP4_OUT_F32) return NVFP4_ERR_DTYPE;
    if (m == 0) return NVFP4_OK;
    if (!x_bf16 || !w_e4m3 || !block_scales || !y) return NVFP4_ERR_NULL;
    auto misaligned = [](const void* p, uintptr_t al) { return (reinterpret_cast<uintptr_t>(p) & (al - 1)) != 0; };
    if (misaligned(x_bf16, 16) || misaligned(w_e4m3, 16) || misaligned(block_scales, 4) ||
        misaligned(y, y_dtype == NVFP4_OUT_F32 ? 4 : 2))
        return NVFP4_ERR_ALIGN;
    st = nvfp4::device_setup();
    if (st != NVFP4_OK) return st;
    W8GemmArgs a;
    a.x = static_cast<const uint16_t*>(x_bf16);
    a.w = w_e4m3;
    a.s = block_scales;
    a.y = y;
    a.m = static_cast<int>(m);
    a.n = static_cast<int>(n);
    a.k = static_cast<int>(k);
    int waves = 1, group = 1;
    fp8_tile(n, k, &waves, &group);
    a.k_per_wave = static_cast<int>(k / waves);
    a.group = group;
    a.part = nullptr;
    a.parts = 1;
    const int64_t col_tiles = n / kGCols, row_tiles = (m + kGRows - 1) / kGRows;
    // Tiles for at most half the CUs: one workgroup per segment group, the
    // group sums added in order by a second kernel through the buffer
    // nvfp4_init allocates (same bits), as nvfp4_gemm does.
    const int split = waves / group;
    float* buf = nullptr;
    if (split > 1) {
        size_t bytes = 0;
        int cus = 256;
        st = nvfp4::gemm_partials(&buf, &bytes, &cus);
        if (st != NVFP4_OK) return st;
        if (buf && 2 * row_tiles * col_tiles <= int64_t(cus) && size_t(split) * size_t(m) * size_t(n) * 4 <= bytes) {
            a.part = buf;
            a.parts = split;
        }
    }
    auto fn = y_dtype == NVFP4_OUT_F32 ? fp8_w8a16_gemm_kernel<true> : fp8_w8a16_gemm_kernel<false>;
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(col_tiles), static_cast<unsigned>(row_tiles),
                                static_cast<unsigned>(a.parts)),
                       dim3(kGThreads), kGLds, static_cast<hipStream_t>(stream), a);
    if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
    if (a.parts > 1) return nvfp4::launch_ordered_sum(a.part, a.parts, m * n, 1.0f, y, y_dtype, stream);
    return NVFP4_OK;
}

extern "C" int fp8_w8a16_matmul(const void* x_bf16, const uint8_t* w_e4m3, const float* block_scales, void* y,
                                int64_t m, int64_t n, int64_t k, int y_dtype, void* stream) {
    if (m >= 0 && m <= NVFP4_MAX_M)
        return fp8_w8a16_linear(x_bf16, w_e4m3, block_scales, y, m, n, k, y_dtype, stream);
    return fp8_w8a16_gemm(x_bf16, w_e4m3, block_scales, y, m, n, k, y_dtype, stream);
}
