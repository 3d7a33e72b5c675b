// NVFP4 weight-only product for many rows (the prefill regime of "10 Kernels"
// 10.2, rows 33 to about 1024, and beyond through the expanded weight):
//   y[m, n] = t * sum_k x[m, k] * e4m3(s[n, k/16]) * e2m1(q[n, k]),  any M.
//
// "Module ops" w4a16_gemm (C = A @ dequant(B), A bf16 [M, K], B NVFP4) is the
// operation; w4a16_gemm_n128_m128 loads one weight tile for 128 rows.  Here a
// workgroup of eight wavefronts (one per CU, two per SIMD) owns 128 rows x 128
// columns.  x and the packed weights come into LDS one 128-k block at a time
// by direct-to-LDS loads, two blocks ahead of the multiply (rings of three
// blocks, waited for by count, one barrier per block); each wavefront decodes
// the weights of its 32 columns from LDS into registers and multiplies them
// with 64 rows of x (v_mfma_f32_16x16x32_bf16, 4 x 2 tiles), so one decoded
// operand serves four MFMAs.  nvfp4_gemm64_kernel is the same body on 64-row
// tiles (four wavefronts, two workgroups per CU) for row counts whose
// 128-row tiles would leave a partial second round of workgroups.  Column tiles are the fastest grid dimension, so
// the eight XCDs (workgroups dealt round-robin) each keep one eighth of the
// weight columns in their L2 across the row tiles.
//
// The K order is the one of every other kernel of this library, fixed by the
// (N, K) tile: K cut into `waves` segments, each one MFMA chain in increasing
// k, added in the two-level order (chains in segment order within a group,
// group sums in group order).  The MFMA inputs of an output element are the
// same bf16 values too (x as given, the exactly decoded weight), so every row
// here has the bits nvfp4_linear gives it at 1..32 rows ("10 Kernels" 10.1),
// at every M.
//
// With BF16W the weight is read as an already expanded bf16 matrix [N, K]
// holding e2m1 x e4m3 exactly (nvfp4_dequant_bf16 without the tensor scale),
// the pages' "expand to BF16 once" path for very large M; the tensor scale is
// still applied once to the fp32 sum, so the bits are the same again.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <algorithm>
#include <cstring>
#include <mutex>

#include "nvfp4_w4a16.h"
#include "nvfp4_common.h"
#include "setup.h"
#include "../host/tiles.h"

namespace {

constexpr int kCols = 128;              // columns per workgroup
constexpr int kMT = 4;                  // 16-row tiles per wavefront
constexpr int kC = 2;                   // 16-column tiles per wavefront
constexpr int kWavesN = kCols / (16 * kC);             // wavefronts across the columns
constexpr int kPitch = kBlockK;         // LDS row of an x block: 16 pieces of 8 k, swizzled
constexpr int kXBufs = 3;               // x blocks in the LDS ring
// NVFP4 weights come into LDS too, three 128-k blocks deep: per block the
// packed bytes of the 128 columns (eight 1 KB column tiles: lane l of tile c
// holds column 16 c + l % 16, 32-k quarter l / 16) and their scale bytes
// (256 B per column tile, the first 128 B used: 8 bytes per column).  With
// BF16W the weights are register loads one block ahead.
constexpr int kWStages = 3;
constexpr int kWPacked = kCols * kBlockK / 2;
constexpr int kWStage = kWPacked + (kCols / 16) * 256;

// A workgroup tile of ROWS rows x kCols columns: 128 (eight wavefronts, one
// workgroup per CU) or 64 (four wavefronts, two workgroups per CU); each
// wavefront keeps 64 rows x 32 columns.
template <int ROWS>
struct GemmTile {
    static constexpr int kRows = ROWS;
    static constexpr int kWaves = (ROWS / (16 * kMT)) * kWavesN;     // (rows) x 4 (columns)
    static constexpr int kThreads = kWaves * kWave;
    static constexpr int kXRowsPerWave = ROWS / kWaves;              // x rows each wavefront stages
    static constexpr int kXLoads = kXRowsPerWave / 4;                // 1 KB direct loads (4 rows) per block
    static constexpr size_t kXBytes = kXBufs * size_t(ROWS) * kPitch * sizeof(uint16_t);
    static constexpr size_t kLdsNv = kXBytes + size_t(kWStages) * kWStage;
    static constexpr size_t kLdsBf = kXBytes;
    static constexpr int kWTilesPerWave = kCols / 16 / kWaves;       // weight column tiles each wavefront stages
    static constexpr int kWLoads = 2 * kWTilesPerWave;                // its direct loads per block (packed, scales)
    static_assert(kWTilesPerWave >= 1 && kWTilesPerWave * kWaves * 16 == kCols, "weight staging");
    static_assert(kXLoads >= 1 && kXLoads * 4 * kWaves == ROWS, "x staging");
};

constexpr int64_t kChunkedMaxM = 64;    // nvfp4_matmul: 32-row slices of the skinny product up to here

struct GemmArgs {
    const uint16_t* x;      // bf16 [M, K]
    const uint8_t* wp;      // [N, K/2] packed e2m1 (or bf16 [N, K] with BF16W)
    const uint8_t* sc;      // [N, K/16] e4m3 (unused with BF16W)
    void* y;                // [M, N]
    float t;
    int m, n, k;
    int k_per_wave;         // segment length
    int group;              // segments per segment group
    float* part;            // parts > 1: group sums or segment chains [parts][M][N] (fp32, t not applied)
    int parts;              // workgroups along K (blockIdx.z): 1, one per segment group, or one per segment
};

// The B operands of one 128-k block for a lane's kC columns: with NVFP4
// weights 16 packed bytes (32 k) and the block's 8 scale bytes per column;
// with bf16 weights the 4 x 8 k of the column.
template <bool BF16W>
struct BRegs;

template <>
struct BRegs<false> {
    u32x4 w[kC];
    uint64_t s[kC];
};

template <>
struct BRegs<true> {
    u32x4 w[kC][4];
};

template <int ROWS, bool BF16W, bool OUT_F32>
__device__ __forceinline__ void gemm_body(const GemmArgs& a) {
    using T = GemmTile<ROWS>;
    constexpr int kRows = T::kRows, kWaves = T::kWaves, kXRowsPerWave = T::kXRowsPerWave, kXLoads = T::kXLoads,
                  kWTilesPerWave = T::kWTilesPerWave, kWLoads = T::kWLoads;
    constexpr size_t kXBytes = T::kXBytes;
    extern __shared__ __align__(16) uint16_t xs[];     // [kXBufs][kRows][kPitch], then the weight ring
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    const int col_lane = lane % 16;
    const int kq = lane / 16;
    const int row0 = blockIdx.y * kRows;
    const int col0 = blockIdx.x * kCols + wn * kC * 16;
    // K blocks of this workgroup: all of K, or one segment group's
    const int nblocks = a.k / kBlockK / a.parts;
    const int kbase = static_cast<int>(blockIdx.z) * nblocks * kBlockK;
    const int seg_blocks = a.k_per_wave / kBlockK;

    // Rows past M and columns past N read the last valid one (never stored).
    const uint8_t* wrow[kC];
    const uint8_t* srow[kC];
#pragma unroll
    for (int c = 0; c < kC; ++c) {
        const int n = min(col0 + 16 * c + col_lane, a.n - 1);
        if constexpr (BF16W) {
            wrow[c] = a.wp + (int64_t)n * a.k * 2;
            srow[c] = nullptr;
        } else {
            wrow[c] = a.wp + (int64_t)n * (a.k / 2);
            srow[c] = a.sc + (int64_t)n * (a.k / 16);
        }
    }
    // x block rows r = 32 wave + 4 i + lane / 16 come in by direct-to-LDS
    // loads: lane l writes slot l % 16 of its row, which holds the row's
    // 16-byte piece p = slot ^ (r % 16) (8 k), so the 16 rows of one A read
    // fall into 16 different bank groups.  Rows past M read row M - 1.
    const int xslot = lane % 16;

    // Plain (cached) loads: every row tile of the grid reads these weights
    // again, and the later readers find them in L2 (measured on MI355X: 15-20 %
    // faster than non-temporal loads at 256..4096 rows).
    auto load_b = [&](BRegs<BF16W>& b, int kl) {
        const int kb = kbase + kl;
#pragma unroll
        for (int c = 0; c < kC; ++c) {
            if constexpr (BF16W) {
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    b.w[c][s] = load16(wrow[c] + (int64_t)(kb + 32 * kq + 8 * s) * 2);
            } else {
                b.w[c] = load16(wrow[c] + kb / 2 + 16 * kq);
                b.s[c] = *reinterpret_cast<const uint64_t*>(srow[c] + kb / 16);
            }
        }
    };
    // NVFP4: wavefront w stages column tiles kWTilesPerWave w + j of each
    // block (per tile one 16-byte direct load of packed bytes and one 4-byte
    // load of scale bytes per lane; lanes 32..63 repeat the scale bytes of
    // lanes 0..31).
    uint8_t* wls = reinterpret_cast<uint8_t*>(xs) + kXBytes;
    const uint8_t* wsrc[kWTilesPerWave];
    const uint8_t* ssrc[kWTilesPerWave];
#pragma unroll
    for (int j = 0; j < kWTilesPerWave; ++j) {
        const int ct = kWTilesPerWave * wave + j;
        const int wcol = min(static_cast<int>(blockIdx.x) * kCols + 16 * ct + lane % 16, a.n - 1);
        const int scol = min(static_cast<int>(blockIdx.x) * kCols + 16 * ct + (lane % 32) / 2, a.n - 1);
        wsrc[j] = a.wp + (int64_t)wcol * (a.k / 2) + kbase / 2 + 16 * (lane / 16);
        ssrc[j] = a.sc + (int64_t)scol * (a.k / 16) + kbase / 16 + 4 * (lane % 2);
    }
    auto load_w = [&](int kl, int st) {
        uint8_t* d = wls + st * kWStage;
#pragma unroll
        for (int j = 0; j < kWTilesPerWave; ++j) {
            const int ct = kWTilesPerWave * wave + j;
            __builtin_amdgcn_global_load_lds(wsrc[j] + kl / 2, d + ct * 1024, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(ssrc[j] + kl / 16, d + kWPacked + ct * 256, 4, 0, 0);
        }
    };
    const char* xwg = reinterpret_cast<const char*>(a.x + (int64_t)row0 * a.k + kbase);
    uint32_t xoff[kXLoads];
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
        const int r = kXRowsPerWave * wave + 4 * i + lane / 16;
        const int rr = min(row0 + r, a.m - 1) - row0;
        xoff[i] = static_cast<uint32_t>(rr * a.k + 8 * (xslot ^ (r % 16))) * 2u;
    }
    auto load_x = [&](int kl, int buf) {
        const char* base = xwg + 2 * kl;
#pragma unroll
        for (int i = 0; i < kXLoads; ++i)
            __builtin_amdgcn_global_load_lds(base + xoff[i], xs + (buf * kRows + kXRowsPerWave * wave + 4 * i) * kPitch,
                                             16, 0, 0);
    };

    f32x4 acc[kMT][kC], grp[kMT][kC], tot[kMT][kC];
#pragma unroll
    for (int t = 0; t < kMT; ++t)
#pragma unroll
        for (int c = 0; c < kC; ++c) acc[t][c] = grp[t][c] = tot[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    BRegs<BF16W> bcur, bnext;
    // blocks 0 and 1 go out first; block 0 must have landed
    load_x(0, 0);
    if constexpr (BF16W) {
        load_b(bcur, 0);
        if (nblocks > 1) {
            load_x(kBlockK, 1);
            gemm_wait_vm<kXLoads>();
        } else {
            gemm_wait_vm<0>();
        }
    } else {
        load_w(0, 0);
        if (nblocks > 1) {
            load_x(kBlockK, 1);
            load_w(kBlockK, 1);
            gemm_wait_vm<kXLoads + kWLoads>();
        } else {
            gemm_wait_vm<0>();
        }
    }
    gemm_lds_barrier();

    // segments, then their 128-k blocks: the fold runs once per segment
    const int nseg = nblocks / seg_blocks;
    for (int sg = 0; sg < nseg; ++sg) {
      for (int bb = 0; bb < seg_blocks; ++bb) {
        const int b = sg * seg_blocks + bb;
        const bool more = b + 1 < nblocks;
        // block b + 2's x (and NVFP4 weights) go out two blocks ahead
        if (b + 2 < nblocks) load_x((b + 2) * kBlockK, (b + 2) % kXBufs);
        if constexpr (BF16W) {
            if (more) load_b(bnext, (b + 1) * kBlockK);
        } else {
            if (b + 2 < nblocks) load_w((b + 2) * kBlockK, (b + 2) % kWStages);
            // this block's B operands from its stage
            const uint8_t* wst = wls + (b % kWStages) * kWStage;
#pragma unroll
            for (int c = 0; c < kC; ++c) {
                const int ct = wn * kC + c;
                bcur.w[c] = *reinterpret_cast<const u32x4*>(wst + ct * 1024 + 16 * lane);
                bcur.s[c] = *reinterpret_cast<const uint16_t*>(wst + kWPacked + ct * 256 + 8 * col_lane + 2 * kq);
            }
        }
        // multiply block b: per 32-k slice, the wavefront's kC B operands,
        // then each of its kMT A operands against them
        const uint16_t* xb = xs + (b % kXBufs) * kRows * kPitch;
        float g0[kC], g1[kC];
        if constexpr (!BF16W) {
#pragma unroll
            for (int c = 0; c < kC; ++c) {
                const uint32_t d = static_cast<uint32_t>(bcur.s[c]);
                g0[c] = __builtin_amdgcn_cvt_f32_fp8(d, 0);
                g1[c] = __builtin_amdgcn_cvt_f32_fp8(d, 1);
            }
        }
        // A operands one 32-k slice ahead of the MFMAs that use them
        u32x4 xa[2][kMT];
        auto read_a = [&](u32x4 (&dst)[kMT], int s) {
#pragma unroll
            for (int t = 0; t < kMT; ++t) {
                const int r = wm * 16 * kMT + 16 * t + col_lane;
                dst[t] = *reinterpret_cast<const u32x4*>(xb + r * kPitch + 8 * ((4 * kq + s) ^ col_lane));
            }
        };
        read_a(xa[0], 0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) read_a(xa[(s + 1) & 1], s + 1);
            bf16x8 bv[kC];
#pragma unroll
            for (int c = 0; c < kC; ++c) {
                if constexpr (BF16W)
                    bv[c] = as_bf16x8(bcur.w[c][s]);
                else
                    bv[c] = decode8(bcur.w[c][s], s < 2 ? g0[c] : g1[c]);
            }
#pragma unroll
            for (int t = 0; t < kMT; ++t)
#pragma unroll
                for (int c = 0; c < kC; ++c)
                    acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[s & 1][t]), bv[c], acc[t][c],
                                                                          0, 0, 0);
        }
        if (more) {
            // block b + 1 has landed; block b + 2's loads may be in flight
            if constexpr (BF16W) {
                gemm_wait_vm<0>();
                bcur = bnext;
            } else {
                if (b + 2 < nblocks)
                    gemm_wait_vm<kXLoads + kWLoads>();
                else
                    gemm_wait_vm<0>();
            }
            gemm_lds_barrier();
        }
      }
      // end of segment sg: its chain joins its group's sum, and at the end
      // of a group the group sum joins the total (first ones as they are);
      // segments are numbered within this workgroup's K range, which is all
      // of K or exactly one group
      {
        const int seg = sg;
        const bool gfirst_seg = seg % a.group == 0;
        const bool gend = (seg + 1) % a.group == 0;
        const bool first_group = seg / a.group == 0;
#pragma unroll
        for (int t = 0; t < kMT; ++t)
#pragma unroll
            for (int c = 0; c < kC; ++c) {
                grp[t][c] = gfirst_seg ? acc[t][c] : grp[t][c] + acc[t][c];
                acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (gend) tot[t][c] = first_group ? grp[t][c] : tot[t][c] + grp[t][c];
            }
      }
    }

    if (a.parts > 1) {
        // one group's sum (or one segment's chain) per output; launch_ordered_sum
        // adds them in the two-level order
        float* dst = a.part + (int64_t)blockIdx.z * a.m * a.n;
#pragma unroll
        for (int t = 0; t < kMT; ++t)
#pragma unroll
            for (int c = 0; c < kC; ++c) {
                const int n = col0 + 16 * c + col_lane;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int m = row0 + wm * 16 * kMT + 16 * t + 4 * kq + j;
                    if (m < a.m && n < a.n) dst[(int64_t)m * a.n + n] = grp[t][c][j];
                }
            }
        return;
    }
#pragma unroll
    for (int t = 0; t < kMT; ++t)
#pragma unroll
        for (int c = 0; c < kC; ++c) {
            const int n = col0 + 16 * c + col_lane;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = row0 + wm * 16 * kMT + 16 * t + 4 * kq + j;
                if (m < a.m && n < a.n) {
                    const float r = tot[t][c][j] * a.t;
                    if (OUT_F32)
                        static_cast<float*>(a.y)[(int64_t)m * a.n + n] = r;
                    else
                        static_cast<uint16_t*>(a.y)[(int64_t)m * a.n + n] = f32_to_bf16_rne(r);
                }
            }
        }
}

template <bool BF16W, bool OUT_F32>
__global__ void __launch_bounds__(GemmTile<128>::kThreads, 1)
nvfp4_gemm_kernel(GemmArgs a) {
    gemm_body<128, BF16W, OUT_F32>(a);
}

// The same product on 64-row workgroup tiles, two workgroups per CU.
template <bool BF16W, bool OUT_F32>
__global__ void __launch_bounds__(GemmTile<64>::kThreads, 2)
nvfp4_gemm64_kernel(GemmArgs a) {
    gemm_body<64, BF16W, OUT_F32>(a);
}

// The partial sums of a K-split product [parts][M][N] added in the tile's
// two-level order, times t, one rounding: `group` consecutive parts form a
// group (1: each part is already a group sum), each group summed in part
// order, then the group sums in group order, the first of each as it is.
// Each thread four consecutive outputs of the flattened [M][N].
template <bool OUT_F32>
__global__ void __launch_bounds__(256)
nvfp4_gemm_reduce(const float* part, int parts, int group, int64_t mn, float t, void* y) {
    const int64_t i0 = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (i0 >= mn) return;
    const int cnt = mn - i0 < 4 ? static_cast<int>(mn - i0) : 4;
    float tot[4];
    for (int j = 0; j < cnt; ++j) tot[j] = part[i0 + j];
    if (group == 1) {
        for (int q = 1; q < parts; ++q)
            for (int j = 0; j < cnt; ++j) tot[j] = tot[j] + part[(int64_t)q * mn + i0 + j];
    } else {
        float grp[4];
        for (int q = 1; q < group; ++q)
            for (int j = 0; j < cnt; ++j) tot[j] = tot[j] + part[(int64_t)q * mn + i0 + j];
        for (int g = group; g < parts; g += group) {
            for (int j = 0; j < cnt; ++j) grp[j] = part[(int64_t)g * mn + i0 + j];
            for (int q = g + 1; q < g + group; ++q)
                for (int j = 0; j < cnt; ++j) grp[j] = grp[j] + part[(int64_t)q * mn + i0 + j];
            for (int j = 0; j < cnt; ++j) tot[j] = tot[j] + grp[j];
        }
    }
    for (int j = 0; j < cnt; ++j) {
        const float r = tot[j] * t;
        if (OUT_F32)
            static_cast<float*>(y)[i0 + j] = r;
        else
            static_cast<uint16_t*>(y)[i0 + j] = f32_to_bf16_rne(r);
    }
}

// Expands NVFP4 to bf16 [N, K]: each thread one packed dword (8 k) of one
// row.  e2m1 x e4m3 is exact in fp32 and in bf16; with APPLY_T it is then
// multiplied by t in fp32 (one rounding) and rounded to bf16 (a second), which
// equals one rounding of the exact t * e4m3 * e2m1 to bf16 since fp32 carries
// more than twice bf16's significand bits plus two.
template <bool APPLY_T>
__global__ void __launch_bounds__(256)
nvfp4_dequant_kernel(const uint8_t* wp, const uint8_t* sc, float t, uint16_t* dst, int64_t n, int64_t k) {
    const int64_t per_row = k / 8;
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n * per_row) return;
    const int64_t row = i / per_row, c8 = i % per_row;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(wp + row * (k / 2) + c8 * 4);
    const float scale = __builtin_amdgcn_cvt_f32_fp8(static_cast<uint32_t>(sc[row * (k / 16) + c8 / 2]), 0);
    f32x2 v[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0),
                  __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1),
                  __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2),
                  __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3)};
    uint16_t out[8];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        float p0 = v[b][0] * scale, p1 = v[b][1] * scale;
        if (APPLY_T) {
            p0 = p0 * t;
            p1 = p1 * t;
        }
        out[2 * b] = f32_to_bf16_rne(p0);
        out[2 * b + 1] = f32_to_bf16_rne(p1);
    }
    u32x4 o;
    __builtin_memcpy(&o, out, sizeof o);
    *reinterpret_cast<u32x4*>(dst + row * k + c8 * 8) = o;
}

using GemmFn = void (*)(GemmArgs);

// rows: the workgroup tile's rows, 128 or 64
GemmFn pick_gemm(bool bf16w, int y_dtype, int rows) {
    const bool f = y_dtype == NVFP4_OUT_F32;
    if (rows == 64) {
        if (bf16w) return f ? nvfp4_gemm64_kernel<true, true> : nvfp4_gemm64_kernel<true, false>;
        return f ? nvfp4_gemm64_kernel<false, true> : nvfp4_gemm64_kernel<false, false>;
    }
    if (bf16w) return f ? nvfp4_gemm_kernel<true, true> : nvfp4_gemm_kernel<true, false>;
    return f ? nvfp4_gemm_kernel<false, true> : nvfp4_gemm_kernel<false, false>;
}

int gemm_launch(const void* x, const void* w, const uint8_t* scales, float t, void* y, int64_t m, int64_t n,
                int64_t k, int y_dtype, void* stream, bool bf16w) {
    int st = nvfp4_gemm_shape_ok(m, n, k);
    if (st != NVFP4_OK) return st;
    if (y_dtype != NVFP4_OUT_BF16 && y_dtype != NVFP4_OUT_F32) return NVFP4_ERR_DTYPE;
    if (m == 0) return NVFP4_OK;
    if (!x || !w || (!bf16w && !scales) || !y) return NVFP4_ERR_NULL;
    auto misaligned = [](const void* p, uintptr_t al) { return (reinterpret_cast<uintptr_t>(p) & (al - 1)) != 0; };
    if (misaligned(x, 16) || misaligned(w, 16) || (!bf16w && misaligned(scales, 16)) ||
        misaligned(y, y_dtype == NVFP4_OUT_F32 ? 4 : 2))
        return NVFP4_ERR_ALIGN;
    if (nvfp4::load_tile_override() != NVFP4_OK) return NVFP4_ERR_TILEFILE;
    st = nvfp4::device_setup();
    if (st != NVFP4_OK) return st;
    const nvfp4::Tile tile = nvfp4::tile_for(n, k);
    GemmArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.wp = static_cast<const uint8_t*>(w);
    a.sc = scales;
    a.y = y;
    a.t = t;
    a.m = static_cast<int>(m);
    a.n = static_cast<int>(n);
    a.k = static_cast<int>(k);
    a.k_per_wave = static_cast<int>(k / tile.waves);
    a.group = tile.waves / tile.split;
    a.part = nullptr;
    a.parts = 1;
    float* part = nullptr;
    size_t bytes = 0;
    int cus = 256;
    if (tile.split > 1) {
        st = nvfp4::gemm_partials(&part, &bytes, &cus);
        if (st != NVFP4_OK) return st;
    } else {
        cus = nvfp4::device_cus();
    }
    const int64_t col_tiles = (n + kCols - 1) / kCols;
    // Tiles for at most half the CUs (one workgroup per CU): one workgroup
    // per segment group instead (the tile's split), the group sums added in
    // order by a second kernel, so the bits do not change.  Needs the
    // partial-sum buffer nvfp4_init allocates.  (Measured on MI355X: faster
    // at 256..512 rows on the decode round's products; with tiles for every
    // CU, e.g. 4096 columns at 1024 rows, the extra partial-sum traffic costs
    // more than the split gains.)  Where the segment groups still leave half
    // the CUs idle, one workgroup per segment instead; the reduce then forms
    // the group sums first (same order, same bits).
    auto parts_for = [&](int64_t row_tiles) {
        int parts = 1;
        if (tile.split > 1 && part && 2 * row_tiles * col_tiles <= int64_t(cus) &&
            size_t(tile.split) * size_t(m) * size_t(n) * sizeof(float) <= bytes) {
            parts = tile.split;
            if (2 * row_tiles * col_tiles * tile.split <= int64_t(cus) && tile.waves > tile.split &&
                size_t(tile.waves) * size_t(m) * size_t(n) * sizeof(float) <= bytes)
                parts = tile.waves;
        }
        return parts;
    };
    // 64-row tiles (two workgroups per CU) up to 256 rows where the 128-row
    // plan would need more than one round of workgroups: measured on MI355X
    // (same-box, order-balanced) 8192x4096 at 256 rows 37.7 against 45.5 us,
    // 24576x4096 81.0 against 90.8; elsewhere the 128-row tiles were level
    // or ahead (64-row tiles 3-9 % slower at 1,024 rows, 10-20 % at 128).
    int rows = 128;
    int64_t row_tiles = (m + 127) / 128;
    a.parts = parts_for(row_tiles);
    if (m <= 256 && row_tiles * col_tiles * a.parts > int64_t(cus)) {
        rows = 64;
        row_tiles = (m + 63) / 64;
        a.parts = parts_for(row_tiles);
    }
    if (a.parts > 1) a.part = part;
    const dim3 grid(static_cast<unsigned>(col_tiles), static_cast<unsigned>(row_tiles),
                    static_cast<unsigned>(a.parts));
    const size_t lds = rows == 64 ? (bf16w ? GemmTile<64>::kLdsBf : GemmTile<64>::kLdsNv)
                                  : (bf16w ? GemmTile<128>::kLdsBf : GemmTile<128>::kLdsNv);
    const int threads = rows == 64 ? GemmTile<64>::kThreads : GemmTile<128>::kThreads;
    hipLaunchKernelGGL(pick_gemm(bf16w, y_dtype, rows), grid, dim3(threads), lds, static_cast<hipStream_t>(stream),
                       a);
    if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
    if (a.parts > 1)
        return nvfp4::launch_ordered_sum(a.part, a.parts, m * n, t, y, y_dtype, stream, a.parts / tile.split);
    return NVFP4_OK;
}

}  // namespace

namespace nvfp4 {

int launch_ordered_sum(const float* part, int parts, int64_t mn, float t, void* y, int y_dtype, void* stream,
                       int group) {
    if (group < 1 || parts % group != 0) return NVFP4_ERR_SHAPE;
    const int64_t blocks = (mn + 1023) / 1024;
    auto red = y_dtype == NVFP4_OUT_F32 ? nvfp4_gemm_reduce<true> : nvfp4_gemm_reduce<false>;
    hipLaunchKernelGGL(red, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       part, parts, group, mn, t, y);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

int gemm_setup() {
    for (int bw = 0; bw <= 1; ++bw)
        for (int od = 0; od <= 1; ++od) {
            if (hipFuncSetAttribute(reinterpret_cast<const void*>(pick_gemm(bw != 0, od, 128)),
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    static_cast<int>(bw ? GemmTile<128>::kLdsBf : GemmTile<128>::kLdsNv)) !=
                hipSuccess)
                return NVFP4_ERR_HIP;
            if (hipFuncSetAttribute(reinterpret_cast<const void*>(pick_gemm(bw != 0, od, 64)),
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    static_cast<int>(bw ? GemmTile<64>::kLdsBf : GemmTile<64>::kLdsNv)) !=
                hipSuccess)
                return NVFP4_ERR_HIP;
        }
    return NVFP4_OK;
}

}  // namespace nvfp4

extern "C" int nvfp4_gemm(const void* x_bf16, const uint8_t* w_packed, const uint8_t* scales_e4m3,
                          float tensor_scale, void* y, int64_t m, int64_t n, int64_t k, int y_dtype, void* stream) {
    return gemm_launch(x_bf16, w_packed, scales_e4m3, tensor_scale, y, m, n, k, y_dtype, stream, false);
}

extern "C" int nvfp4_gemm_expanded(const void* x_bf16, const void* w_bf16, float tensor_scale, void* y,
                                   int64_t m, int64_t n, int64_t k, int y_dtype, void* stream) {
    return gemm_launch(x_bf16, w_bf16, nullptr, tensor_scale, y, m, n, k, y_dtype, stream, true);
}

extern "C" int nvfp4_dequant_bf16(const uint8_t* w_packed, const uint8_t* scales_e4m3, float tensor_scale,
                                  int apply_tensor_scale, void* w_bf16, int64_t n, int64_t k, void* stream) {
    if (!w_packed || !scales_e4m3 || !w_bf16) return NVFP4_ERR_NULL;
    if (n < 1 || n > (int64_t(1) << 28) || k < 16 || k > (int64_t(1) << 20) || k % 16) return NVFP4_ERR_SHAPE;
    if (apply_tensor_scale != 0 && apply_tensor_scale != 1) return NVFP4_ERR_DTYPE;
    if ((reinterpret_cast<uintptr_t>(w_packed) & 3) || (reinterpret_cast<uintptr_t>(w_bf16) & 15))
        return NVFP4_ERR_ALIGN;
    const int64_t threads = n * (k / 8);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffff) return NVFP4_ERR_SHAPE;
    auto fn = apply_tensor_scale ? nvfp4_dequant_kernel<true> : nvfp4_dequant_kernel<false>;
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       w_packed, scales_e4m3, tensor_scale, static_cast<uint16_t*>(w_bf16), n, k);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

extern "C" int nvfp4_matmul(const void* x_bf16, const uint8_t* w_packed, const uint8_t* scales_e4m3,
                            float tensor_scale, void* y, int64_t m, int64_t n, int64_t k, int y_dtype,
                            void* stream) {
    if (m >= 0 && m <= NVFP4_MAX_M)
        return nvfp4_linear(x_bf16, w_packed, scales_e4m3, tensor_scale, y, m, n, k, y_dtype, stream);
    int st = nvfp4_gemm_shape_ok(m, n, k);
    if (st != NVFP4_OK) return st;
    if (m > kChunkedMaxM)
        return nvfp4_gemm(x_bf16, w_packed, scales_e4m3, tensor_scale, y, m, n, k, y_dtype, stream);
    // 33..64 rows: the skinny product's kernels on 32-row slices, all slices
    // in one launch (blockIdx.y picks the slice; same bits), which stream the
    // weight at a few TB/s where the 128-row GEMM tile leaves most CUs idle
    // (measured on MI355X on the decode round's shapes: 21-40 us at 33..64
    // rows against 23-50 us for the GEMM; the GEMM ahead or level from 80
    // rows).
    nvfp4::MultiLaunch ml;
    ml.slice_rows = NVFP4_MAX_M;
    ml.rows_total = static_cast<int>(m);
    ml.count = static_cast<int>((m + NVFP4_MAX_M - 1) / NVFP4_MAX_M);
    return nvfp4::launch_multi(x_bf16, w_packed, scales_e4m3, tensor_scale, y, NVFP4_MAX_M, n, k, y_dtype, stream,
                               ml);
}
