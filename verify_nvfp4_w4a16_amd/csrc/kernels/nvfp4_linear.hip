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
//    A lane's 16-byte operand piece holds 32 k of one row (4 instructions'
//    worth).  The streaming kernels bring weights into LDS with direct-to-LDS
//    loads that read 8 rows x 128 contiguous bytes each (an XOR swizzle keeps
//    the 16 rows of one operand read in different bank groups); the generic
//    kernel loads the pieces straight into registers.
//  * Decode is in registers: v_cvt_scalef32_pk_f32_fp4 turns one packed byte
//    into two fp32 e2m1 values (its scale operand contributes only an
//    exponent, so it is given 1.0), a multiply by the group's e4m3 scale
//    (decoded once per 16 k by v_cvt_f32_fp8, the OCP e4m3 decoder) makes the
//    exact product, and v_cvt_pk_bf16_f32 packs two of them into the bf16
//    operand.  e2m1 times e4m3 has at most 6 significant bits, so the bf16
//    weight is exact ("10 Kernels", 10.2, makes the same point for fp16).
//  * Activations are the A operand: 16 rows per instruction, one 16-row tile
//    for M <= 16 and two for 17..32; rows >= M repeat row M - 1 and are never
//    stored.
//  * Every M, including M = 1, runs the same instruction sequence on each
//    output element: the K order is fixed by the (N, K) tile (segments, each
//    one MFMA chain in increasing k, added in a fixed two-level order), and
//    nothing uses atomics ("10 Kernels", 10.1).  The kernels differ only in
//    how work and data are laid over the machine: one workgroup per column
//    tile (few rows), persistent workgroups walking the tiles, many-row
//    workgroups sharing x windows (their segment groups meet through device
//    memory), and a generic register-load kernel for any shape.
//  * Epilogue: fp32 sum times t, one round-to-nearest-even to bf16, or fp32.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <type_traits>

#include "nvfp4_w4a16.h"
#include "nvfp4_common.h"
#include "setup.h"
#include "../host/tiles.h"

namespace {

struct Args {
    const uint16_t* x;     // bf16 [M, K]
    const uint8_t* wp;     // [N, K/2]
    const uint8_t* sc;     // [N, K/16]
    void* y;               // [M, N] bf16 or fp32
    float t;
    int m, n, k;
    int k_per_wave;        // segment length
    int group;             // segments per segment group
    // Several products of one (N, K) in one launch, blockIdx.y picking one:
    // rows of a device table (m above is then the largest m of an entry),
    // or, without a table, a second weight over the same x (product 1).
    const nvfp4_group_t* table;
    const uint8_t* wp1;
    const uint8_t* sc1;
    void* y1;
    float t1;
    // De-interleaved store (omap_parts > 0): weight row r of part p of group
    // g goes to output column ngroups * (widths of parts before p) + g *
    // width[p] + r.
    int omap_parts;
    int omap_width[4];
    int omap_gwidth;
    int omap_ngroups;
    // Row slices of one product (slice_rows > 0): product e is rows
    // [e * slice_rows, e * slice_rows + slice_rows) of x and y, of rows_total.
    int slice_rows;
    int rows_total;
    int y_bytes;           // bytes per output element (2 or 4)
    // The silu input (per-tile kernel only): x is the gate, xu the up
    // activation, and the kernel multiplies silu(x) * xu (rounded to bf16).
    const uint16_t* xu;
};

// The product of this workgroup (blockIdx.y) in a several-product launch;
// m <= 0 means there is nothing to do (uniform over the workgroup).
__device__ __forceinline__ Args entry_args(const Args& in) {
    Args a = in;
    if (in.table) {
        const nvfp4_group_t& g = in.table[blockIdx.y];
        a.x = static_cast<const uint16_t*>(g.x);
        a.wp = g.w_packed;
        a.sc = g.scales_e4m3;
        a.y = g.y;
        a.t = g.tensor_scale;
        a.m = min(g.m, in.m);
    } else if (in.slice_rows > 0) {
        const int r0 = static_cast<int>(blockIdx.y) * in.slice_rows;
        a.x = in.x + (int64_t)r0 * in.k;
        a.y = static_cast<uint8_t*>(in.y) + (int64_t)r0 * in.n * in.y_bytes;
        a.m = min(in.slice_rows, in.rows_total - r0);
    } else if (blockIdx.y == 1) {
        a.wp = in.wp1;
        a.sc = in.sc1;
        a.y = in.y1;
        a.t = in.t1;
    }
    return a;
}

// Output column of weight row n (the de-interleaving map, or n itself).
__device__ __forceinline__ int out_col(const Args& a, int n) {
    if (a.omap_parts == 0) return n;
    const int g = n / a.omap_gwidth;
    int r = n - g * a.omap_gwidth;
    int before = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        if (p < a.omap_parts) {
            if (r < a.omap_width[p]) return a.omap_ngroups * before + g * a.omap_width[p] + r;
            r -= a.omap_width[p];
            before += a.omap_width[p];
        }
    }
    return n;   // unreachable for a valid map
}

// Folds segment sum `v` of segment `w` (w >= 1) into the running sums of the
// two-level order: `grp` is the sum of the current group so far, `tot` the
// sum of the finished groups (valid once w >= group).
__device__ __forceinline__ void fold_segment(f32x4& grp, f32x4& tot, f32x4 v, int w, int group) {
    // branch-free (selects), so the caller's control flow stays simple
    const bool starts = w % group == 0;
    const f32x4 closed = w == group ? grp : tot + grp;
    tot = starts ? closed : tot;
    grp = starts ? v : grp + v;
}

// Keeps the machine scheduler from moving instructions across this point.
// Placed after the loads of the next pipeline chunk, it makes them go out
// before the waits for the current chunk, so two chunks are in flight while
// one waits (left alone, the scheduler sinks those loads below the waits).
__device__ __forceinline__ void issue_point() { __builtin_amdgcn_sched_barrier(0); }

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

// x rows staged by direct-to-LDS loads keep the four 32-k quarters of each
// 128-k block rotated by the row's group of four: quarter q of row r sits at
// slot (q + r / 4) % 4.  An A read (16 rows x 4 quarters) of unrotated rows
// took 8 LDS cycles per instruction, half of them bank conflicts; rotated, it
// takes 4, as a contiguous read does (ds_read_b128 pattern probe on MI355X).
__device__ __forceinline__ int xslot(int q, int r) { return (q + (r >> 2)) & 3; }
// Global 16-byte piece of x row r that load lane u (LDS piece u of a 1 KB
// run: block u / 16, slot (u / 4) % 4, eighth u % 4) fetches.
__device__ __forceinline__ int xpiece(int u, int r) {
    return (u & ~12) | ((((u >> 2) - (r >> 2)) & 3) << 2);
}

// C: 16-column tiles per wavefront.  MT: 16-row A tiles (1 for M <= 16).
// U: 128-k blocks per pipeline step.  OUT_F32: y element type.
//
// One workgroup owns 16*C output columns; its `waves` wavefronts cut K into
// `waves` equal segments.  Wavefront w sums segment w as one chain of MFMAs in
// increasing k, and the segment sums are added in the two-level order of the
// tile (consecutive segments form `waves / group` groups; each group's chains
// are added in segment order, then the group sums in group order).  C and U
// change neither the chains nor the final sum: only the segment count and
// grouping enter the arithmetic, and both are fixed by the (N, K) tile.
//
// XLDS: x [M, K] is first copied into LDS (A rows >= M repeat row M-1; their
// outputs are never stored), so the weight pipeline holds only weights in
// registers.
// Otherwise (x too large for LDS) each chunk also fetches its A operands.
template <int C, int MT, int U, bool XLDS, bool OUT_F32, bool MULTI>
__global__ void __launch_bounds__(512)
nvfp4_skinny(Args a_in) {
    const Args a = MULTI ? entry_args(a_in) : a_in;
    if (MULTI && a.m <= 0) return;                // an empty entry (uniform over the workgroup)
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
        issue_point();
        compute(A, k0 + i * kBlockK * U);
        if (i + 2 < nchunks) load(A, k0 + (i + 2) * kBlockK * U);
        issue_point();
        compute(B, k0 + (i + 1) * kBlockK * U);
    }
    if (i < nchunks) compute(A, k0 + i * kBlockK * U);

    // Segment sums, added in the two-level order: wavefront 0 keeps its own
    // sum in registers and folds in those of wavefronts 1, 2, ... in turn
    // (group sums in segment order, then the group sums in group order).  The
    // LDS that held x is reused once every wavefront is done with it.
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
        f32x4 tot[C][MT] = {};
        for (int w2 = 1; w2 < waves; ++w2) {
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int t = 0; t < MT; ++t)
                {
                    const float* p = partials + ((w2 * C + c) * MT + t) * 4 * kWave + lane;
                    fold_segment(acc[c][t], tot[c][t], f32x4{p[0], p[kWave], p[2 * kWave], p[3 * kWave]}, w2, a.group);
                }
        }
        if (a.group < waves) {
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[c][t] = tot[c][t] + acc[c][t];
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
                        static_cast<float*>(a.y)[(int64_t)m * a.n + (MULTI ? out_col(a, n) : n)] = r;
                    else
                        static_cast<uint16_t*>(a.y)[(int64_t)m * a.n + (MULTI ? out_col(a, n) : n)] = f32_to_bf16_rne(r);
                }
            }
    }
}

// ---- Weight chunks staged in LDS ---------------------------------------
// The streaming kernels bring weights through LDS.  A chunk is 512 k of the
// 16 weight rows of one column tile: 256 bytes of nibbles and 32 scale bytes
// per row.  Direct-to-LDS loads (global_load_lds) bring it in, each load
// instruction reading whole 128-byte lines (8 rows x 128 bytes); loading the MFMA operand
// layout straight into registers instead touches 16 rows x 64 bytes per
// instruction (half of each 128-byte line), which streams at roughly half the
// HBM bandwidth.  The operands are then read from LDS in the MFMA layout.
//
// Layout of one column tile's chunk: 16 rows x 32 scale bytes, loaded first
// (rows 8..15 16 bytes further on, so that rows n and n + 8 fall into
// different LDS banks: the two-byte scale read of a block took 8 LDS cycles,
// three quarters of them bank conflicts, with the rows 32 bytes apart
// throughout), then 4 groups (1024 bytes + 64 of padding each) of 8 rows x 128 bytes:
// group u holds half h = u / 2 of the chunk (k 256h .. 256h + 255) of rows
// 8 (u % 2) .. 8 (u % 2) + 7.  Row r of a group sits at 128 r, its 16-byte
// piece p (of 8 in the half) at 16 (p ^ (r / 2)); the load lane l = 8 r + j
// fetches piece j ^ (r / 2) of row r and lands at 16 l, so each instruction
// reads whole 128-byte lines, and the 16 rows of one operand read fall into
// 16 different 16-byte bank groups.  The first half of a chunk is complete
// once its scale loads and first two weight loads have landed, so the
// multiply of blocks 0 and 1 starts while the second half is in flight.
constexpr int kChunkK = 512;                      // k per chunk
constexpr int kGrpBytes = 8 * 128 + 64;
constexpr int kSHalfBytes = 8 * 32 + 16;          // 8 rows of scale bytes + padding
constexpr int kSBytes = 2 * kSHalfBytes;
constexpr int kWBytes = 4 * kGrpBytes;
constexpr int kTileBytes = kSBytes + kWBytes;     // one column tile's chunk in LDS
constexpr int kDmaPerTile = 6;                    // load instructions per column tile's chunk
constexpr int kDmaHalf1 = 2;                      // of those, the last ones: the chunk's second half

// Waits until at most N vector memory operations of this wavefront are
// outstanding (the direct-to-LDS loads count there), and keeps both the
// compiler and the scheduler from moving LDS reads above the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier for LDS traffic: waits for this wavefront's LDS
// operations only (__syncthreads would also drain every outstanding global
// load, emptying the weight pipeline at each barrier), then synchronises.
// Direct-to-LDS loads that others must see are waited for with wait_vm first.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Stores v to LDS at p (16-byte aligned) through an instruction the compiler
// does not track: a plain LDS store issued while direct-to-LDS loads are in
// flight makes the compiler wait for every outstanding load first (it may
// alias their destinations), which would empty the weight pipeline.  Callers
// order it with lds_barrier, which waits for all LDS operations of the
// wavefront.
__device__ __forceinline__ void lds_store_f32x4(float* p, f32x4 v) {
    const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
    asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// Folds the segment sums of wavefronts 1 .. waves-1 into wavefront 0's acc in
// the two-level order.  Wavefront w's vector (c, t) of lane l is at
// part(w) + 4 * ((c * MT + t) * 64 + l) (one 16-byte read); the reads of a
// batch of wavefronts are issued together, then folded in wavefront order.
template <int C, int MT, typename PartFn>
__device__ __forceinline__ void fold_waves(f32x4 (&acc)[C][MT], PartFn part, int waves, int group, int lane) {
    constexpr int kB = C * MT == 1 ? 7 : C * MT == 2 ? 4 : 2;
    f32x4 tot[C][MT] = {};
    int pos = group == 1 ? 0 : 1;        // position of segment w0 in its group
    for (int w0 = 1; w0 < waves; w0 += kB) {
        f32x4 v[kB][C][MT];
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            const float* p = part(min(w0 + i, waves - 1));   // past the last: re-read, unused
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    v[i][c][t] = *reinterpret_cast<const f32x4*>(p + 4 * ((c * MT + t) * kWave + lane));
        }
        // The fold decisions are wavefront-uniform: scalar branches and a
        // running position in the group keep this serial tail short.
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            if (w0 + i >= waves) break;
            if (pos == 0) {                                   // segment w0 + i starts a group
                if (w0 + i == group) {
#pragma unroll
                    for (int c = 0; c < C; ++c)
#pragma unroll
                        for (int t = 0; t < MT; ++t) tot[c][t] = acc[c][t];
                } else {
#pragma unroll
                    for (int c = 0; c < C; ++c)
#pragma unroll
                        for (int t = 0; t < MT; ++t) tot[c][t] = tot[c][t] + acc[c][t];
                }
#pragma unroll
                for (int c = 0; c < C; ++c)
#pragma unroll
                    for (int t = 0; t < MT; ++t) acc[c][t] = v[i][c][t];
            } else {
#pragma unroll
                for (int c = 0; c < C; ++c)
#pragma unroll
                    for (int t = 0; t < MT; ++t) acc[c][t] = acc[c][t] + v[i][c][t];
            }
            pos = pos + 1 == group ? 0 : pos + 1;
        }
    }
    if (group < waves) {
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[c][t] = tot[c][t] + acc[c][t];
    }
}

// Issues the loads of the chunk at byte `kb` of each row (k = 2 kb) of weight
// rows row0 .. row0 + 15 (rows past nmax read row nmax, never used) into dst.
__device__ __forceinline__ void issue_tile_chunk(uint8_t* dst, const uint8_t* wp, const uint8_t* sc, int row0,
                                                 int nmax, uint32_t row_bytes, uint32_t scale_bytes, uint32_t kb,
                                                 int lane) {
    const int r = lane / 8, j = lane % 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t row = static_cast<uint32_t>(min(row0 + 8 * h + r, nmax));
        __builtin_amdgcn_global_load_lds(sc + static_cast<uint64_t>(row) * scale_bytes + kb / 8 + 4 * j,
                                         dst + h * kSHalfBytes, 4, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint32_t row = static_cast<uint32_t>(min(row0 + 8 * (u % 2) + r, nmax));
        __builtin_amdgcn_global_load_lds(wp + static_cast<uint64_t>(row) * row_bytes + kb + 128 * (u / 2) +
                                             16 * (j ^ (r / 2)),
                                         dst + kSBytes + u * kGrpBytes, 16, 0, 0);
    }
}

// 16-byte piece p (32 k) of row n of a staged chunk: the B operand of lane
// (n, kq) for 128-k block b is piece 4 b + kq.
__device__ __forceinline__ u32x4 chunk_piece(const uint8_t* src, int n, int p) {
    const int r = n % 8;
    return *reinterpret_cast<const u32x4*>(src + kSBytes + (2 * (p / 8) + n / 8) * kGrpBytes + 128 * r +
                                           16 * ((p % 8) ^ (r / 2)));
}

// The two scale bytes of row n that lane quarter kq needs in 128-k block b
// of a staged chunk (groups 8b + 2kq and 8b + 2kq + 1), in the low 16 bits.
__device__ __forceinline__ uint32_t chunk_scale_pair(const uint8_t* src, int n, int b, int kq) {
    return *reinterpret_cast<const uint16_t*>(src + (n / 8) * kSHalfBytes + 32 * (n % 8) + 8 * b + 2 * kq);
}

// LDS operands of one 128-k block: A pieces of every row tile, and per
// column tile the packed nibbles and the two scale bytes.
template <int C, int MT>
struct BlockOps {
    u32x4 xa[MT][4];
    u32x4 w[C];
    uint32_t d[C];
};

// Multiplies one staged chunk into acc: C column tiles (chunks at
// wsrc + c * kTileBytes), MT row tiles of A read from LDS at xsrc (row pitch
// `pitch` elements, k of the chunk's first element at 0).  Per 128-k block and
// 32-k slice the MFMA sequence is the one of every kernel here.
//
// The LDS reads of block b + 1 are issued before block b is decoded and
// multiplied (a scheduling barrier keeps them there), so their latency is
// covered by block b's work instead of stalling each MFMA.
template <int C, int MT, int H>
__device__ __forceinline__ void mma_half(f32x4 (&acc)[C][MT], const uint8_t* wsrc, const uint16_t* xsrc,
                                         int pitch, const int (&xr)[MT], int col_lane, int kq) {
    BlockOps<C, MT> ops[2];
    auto fetch = [&](BlockOps<C, MT>& o, int b) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                o.xa[t][s] = *reinterpret_cast<const u32x4*>(xsrc + xr[t] * pitch + kBlockK * b +
                                                             32 * xslot(kq, xr[t]) + 8 * s);
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const uint8_t* src = wsrc + c * kTileBytes;
            o.d[c] = chunk_scale_pair(src, col_lane, b, kq);
            o.w[c] = chunk_piece(src, col_lane, 4 * b + kq);
        }
    };
    fetch(ops[0], 2 * H);
#pragma unroll
    for (int b = 2 * H; b < 2 * H + 2; ++b) {
        const BlockOps<C, MT>& o = ops[b & 1];
        // Block b's reads (issued one block earlier) are waited for before
        // block b + 1's go out, so this wait does not also cover those.
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0); vmcnt and expcnt not waited for
        __builtin_amdgcn_sched_barrier(0);
        if (b + 1 < 2 * H + 2) fetch(ops[(b + 1) & 1], b + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const float g0 = __builtin_amdgcn_cvt_f32_fp8(o.d[c], 0);
            const float g1 = __builtin_amdgcn_cvt_f32_fp8(o.d[c], 1);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 bv = decode8(o.w[c][s], s < 2 ? g0 : g1);
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(o.xa[t][s]), bv, acc[c][t], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Multiplies a staged chunk whose loads are the last ones issued except for
// `After` more: waits for its first half, multiplies blocks 0 and 1, waits
// for the second half, multiplies blocks 2 and 3.
template <int C, int MT, int After>
__device__ __forceinline__ void mma_chunk(f32x4 (&acc)[C][MT], const uint8_t* wsrc, const uint16_t* xsrc,
                                          int pitch, const int (&xr)[MT], int col_lane, int kq) {
    wait_vm<After + kDmaHalf1>();
    mma_half<C, MT, 0>(acc, wsrc, xsrc, pitch, xr, col_lane, kq);
    wait_vm<After>();
    mma_half<C, MT, 1>(acc, wsrc, xsrc, pitch, xr, col_lane, kq);
}

// Persistent kernel for x small enough to sit in LDS whole (the M = 1 GEMV
// regime and small M).  A few workgroups per CU walk the column tiles
// t = blockIdx.x, blockIdx.x + gridDim.x, ...; a tile is 16*C columns and its
// `waves` wavefronts take the K segments of the tile (same chains and the
// same two-level order as every other kernel).  Each wavefront streams its
// (tile, chunk) sequence through two LDS chunk buffers of its own: the next
// chunk's loads are in flight while the current one is multiplied, across
// tile boundaries too.  x is staged once per workgroup.  With NB = 3 chunk
// buffers per wavefront two chunks are in flight while one is multiplied
// (NB = 2: one), which is what keeps enough bytes in flight per CU when a
// single workgroup fits a CU's LDS.
//
// LDS: x [M][K + 8] bf16 | 2 x segment partials | per wavefront NB chunk buffers.
template <int C, int MT, int NB, bool OUT_F32, bool MULTI>
__global__ void __launch_bounds__(512)
nvfp4_skinny_persistent(Args a_in) {
    const Args a = MULTI ? entry_args(a_in) : a_in;
    if (MULTI && a.m <= 0) return;                         // an empty entry (uniform over the workgroup)
    extern __shared__ __align__(16) uint16_t lds[];
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
    uint8_t* wbuf = reinterpret_cast<uint8_t*>(partials + 2 * part_stride) + wave * NB * C * kTileBytes;

    const int tiles = (a.n + 16 * C - 1) / (16 * C);
    const int my_tiles = tiles > (int)blockIdx.x ? (tiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 0;
    const int k0 = wave * a.k_per_wave;
    const int nch = a.k_per_wave / kChunkK;           // chunks per tile per wavefront
    const int total = my_tiles * nch;
    if (total == 0) return;                           // uniform over the workgroup

    int xr[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) xr[t] = min(16 * t + col_lane, a.m - 1);

    // chunk j -> tile blockIdx.x + (j / nch) * gridDim.x, k = k0 + (j % nch) * 512
    auto issue = [&](int j) {
        const int tile = (int)blockIdx.x + (j / nch) * (int)gridDim.x;
        const uint32_t kb = static_cast<uint32_t>(k0 + (j % nch) * kChunkK) / 2;
        uint8_t* dst = wbuf + (j % NB) * C * kTileBytes;
#pragma unroll
        for (int c = 0; c < C; ++c)
            issue_tile_chunk(dst + c * kTileBytes, a.wp, a.sc, tile * 16 * C + 16 * c, a.n - 1, row_bytes,
                             scale_bytes, kb, lane);
    };

    // Stage x with direct-to-LDS loads, then the first chunks' loads.  (An
    // LDS store issued while direct-to-LDS loads are in flight makes the
    // compiler wait for all of them first, as it may alias their
    // destinations, so this kernel stores nothing to LDS on that path.)  Row r
    // of x is ceil(K / 512) loads of up to 1 KB; load i is issued by
    // wavefront i % waves.
    {
        const int per_row = (a.k + kChunkK - 1) / kChunkK;
        const int xloads = a.m * per_row;
        for (int i = wave; i < xloads; i += waves) {
            const int r = i / per_row, p = i % per_row;
            const int valid = min(kWave, (a.k - p * kChunkK) / 8);    // 16-byte pieces in this load
            if (lane < valid)
                __builtin_amdgcn_global_load_lds(a.x + (int64_t)r * a.k + p * kChunkK + 8 * xpiece(lane, r),
                                                 lds + r * pitch + p * kChunkK, 16, 0, 0);
        }
        issue(0);
        if (NB > 2 && total > 1) {
            issue(1);
            wait_vm<2 * kDmaPerTile * C>();           // this wavefront's x loads have landed
        } else {
            wait_vm<kDmaPerTile * C>();
        }
        lds_barrier();                                // ... and everyone's
    }

    f32x4 acc[C][MT];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // chunk j, once at most `after` loads issued after its own are outstanding
    auto compute = [&](int j, auto after) {
        mma_chunk<C, MT, decltype(after)::value>(acc, wbuf + (j % NB) * C * kTileBytes,
                                                 lds + k0 + (j % nch) * kChunkK, pitch, xr, col_lane, kq);
    };

    // After the last chunk of a tile: segment partials through LDS (two
    // buffers, so one barrier per tile), wavefront 0 adds them in the
    // two-level order, scales, rounds and stores.
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
                        lds_store_f32x4(buf + 4 * (((wave * C + c) * MT + t) * kWave + lane), acc[c][t]);
            }
            lds_barrier();
        }
        if (wave == 0) {
            fold_waves<C, MT>(acc, [&](int w2) { return buf + 4 * w2 * C * MT * kWave; }, waves, a.group, lane);
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
                                static_cast<float*>(a.y)[(int64_t)m * a.n + (MULTI ? out_col(a, n) : n)] = r;
                            else
                                static_cast<uint16_t*>(a.y)[(int64_t)m * a.n + (MULTI ? out_col(a, n) : n)] = f32_to_bf16_rne(r);
                        }
                    }
            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // One pipeline over all (tile, chunk) of this wavefront, NB - 1 chunks
    // ahead, with its single exit at the bottom; the last chunks are peeled,
    // so no load is repeated.
    constexpr int kAhead = NB - 1;
    int j = 0;
    for (; j + kAhead < total; ++j) {
        issue(j + kAhead);
        compute(j, std::integral_constant<int, kAhead * kDmaPerTile * C>{});
        if (j % nch == nch - 1) finish_tile(j);
    }
    if (NB > 2 && j + 1 < total) {
        compute(j, std::integral_constant<int, kDmaPerTile * C>{});
        if (j % nch == nch - 1) finish_tile(j);
        ++j;
    }
    compute(j, std::integral_constant<int, 0>{});
    finish_tile(j);                                   // the last chunk ends a tile
}

// LDS bytes of the persistent kernel with nb chunk buffers per wavefront.
size_t persistent_lds_bytes(int64_t m, int64_t k, int waves, int c, int mt, int nb) {
    return size_t(m) * (k + 8) * sizeof(uint16_t) + 2 * size_t(waves) * c * mt * 4 * kWave * sizeof(float) +
           size_t(waves) * nb * c * kTileBytes;
}

// Per-tile kernel: one workgroup per column tile of 16*C columns, its
// `waves` wavefronts one K segment each.  Every wavefront stages its own
// slice of x (M rows x k_per_wave) and streams its segment's chunks through
// NB LDS buffers of its own, all by direct-to-LDS loads, so no wavefront
// waits for another until the segment sums are added: each writes its sum
// into its first chunk buffer, and after one barrier wavefront 0 adds them in
// the two-level order, scales, rounds and stores.  With workgroups short and
// small, several share a CU and one's reduction overlaps the others' loads.
//
// LDS per wavefront: x slice [M][k_per_wave + 8] bf16 | NB chunk buffers.
template <int C, int MT, int NB, bool OUT_F32, bool MULTI>
__global__ void __launch_bounds__(512)
nvfp4_skinny_tile(Args a_in) {
    const Args a = MULTI ? entry_args(a_in) : a_in;
    if (MULTI && a.m <= 0) return;                         // an empty entry (uniform over the workgroup)
    extern __shared__ __align__(16) uint8_t ldsb[];
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int waves = blockDim.x / kWave;
    const int col_lane = lane % 16;
    const int kq = lane / 16;
    const int ks = a.k_per_wave;
    const int nch = ks / kChunkK;
    const int xpitch = ks + 8;
    const uint32_t row_bytes = static_cast<uint32_t>(a.k) / 2;
    const uint32_t scale_bytes = static_cast<uint32_t>(a.k) / 16;
    // the silu input: the up slice follows the gate slice
    const bool silu = MULTI && a.xu != nullptr;
    const int xbytes = a.m * xpitch * 2 * (silu ? 2 : 1);
    const int wave_bytes = xbytes + NB * C * kTileBytes;
    uint16_t* xs = reinterpret_cast<uint16_t*>(ldsb + wave * wave_bytes);
    uint8_t* wbuf = ldsb + wave * wave_bytes + xbytes;
    const int col0 = (int)blockIdx.x * 16 * C;
    const int k0 = wave * ks;

    int xr[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) xr[t] = min(16 * t + col_lane, a.m - 1);

    // this wavefront's x slice: M x nch loads of 1 KB
    for (int i = 0; i < a.m * nch; ++i) {
        const int r = i / nch, p = i % nch;
        __builtin_amdgcn_global_load_lds(a.x + (int64_t)r * a.k + k0 + p * kChunkK + 8 * xpiece(lane, r),
                                         xs + r * xpitch + p * kChunkK, 16, 0, 0);
    }
    if (silu)
        for (int i = 0; i < a.m * nch; ++i) {
            const int r = i / nch, p = i % nch;
            __builtin_amdgcn_global_load_lds(a.xu + (int64_t)r * a.k + k0 + p * kChunkK + 8 * xpiece(lane, r),
                                             xs + a.m * xpitch + r * xpitch + p * kChunkK, 16, 0, 0);
        }
    auto issue = [&](int j) {
        const uint32_t kb = static_cast<uint32_t>(k0 + j * kChunkK) / 2;
        uint8_t* dst = wbuf + (j % NB) * C * kTileBytes;
#pragma unroll
        for (int c = 0; c < C; ++c)
            issue_tile_chunk(dst + c * kTileBytes, a.wp, a.sc, col0 + 16 * c, a.n - 1, row_bytes, scale_bytes, kb,
                             lane);
    };

    f32x4 acc[C][MT];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // chunk j, once at most `after` loads issued after its own are outstanding
    auto compute = [&](int j, auto after) {
        mma_chunk<C, MT, decltype(after)::value>(acc, wbuf + (j % NB) * C * kTileBytes, xs + j * kChunkK, xpitch,
                                                 xr, col_lane, kq);
    };

    // NB - 1 chunks ahead; the last ones peeled so no load is repeated.
    constexpr int kAhead = NB - 1;
    for (int q = 0; q < kAhead && q < nch; ++q) issue(q);
    if (silu) {
        // The gate and up slices have landed (the chunk loads issued after
        // them may still be in flight); each lane turns the 16 bytes its own
        // loads brought in into the activation, in place over the gate.  The
        // store is one the compiler does not track, so it does not wait for
        // the chunk loads; LDS operations of one wavefront run in order.
        if (nch >= kAhead)
            wait_vm<kAhead * kDmaPerTile * C>();
        else
            wait_vm<0>();
        for (int i = 0; i < a.m * nch; ++i) {
            const int r = i / nch, p = i % nch;
            uint16_t* g = xs + r * xpitch + p * kChunkK + 8 * lane;
            uint16_t gv[8], uv[8], hv[8];
            const u32x4 gw = *reinterpret_cast<const u32x4*>(g);
            const u32x4 uw = *reinterpret_cast<const u32x4*>(g + a.m * xpitch);
            __builtin_memcpy(gv, &gw, 16);
            __builtin_memcpy(uv, &uw, 16);
#pragma unroll
            for (int e = 0; e < 8; ++e) hv[e] = silu_mul(gv[e], uv[e]);
            f32x4 hw;
            __builtin_memcpy(&hw, hv, 16);
            lds_store_f32x4(reinterpret_cast<float*>(g), hw);
        }
    }
    int j = 0;
    for (; j + kAhead < nch; ++j) {
        issue(j + kAhead);
        compute(j, std::integral_constant<int, kAhead * kDmaPerTile * C>{});   // x and chunk j have landed
    }
    if (NB > 2 && j + 1 < nch) {
        compute(j, std::integral_constant<int, kDmaPerTile * C>{});
        ++j;
    }
    if (j < nch) compute(j, std::integral_constant<int, 0>{});

    // segment sums: each wavefront's into its first chunk buffer, then
    // wavefront 0 adds them in the two-level order
    float* mine = reinterpret_cast<float*>(wbuf);
    if (wave != 0) {
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int t = 0; t < MT; ++t) lds_store_f32x4(mine + 4 * ((c * MT + t) * kWave + lane), acc[c][t]);
    }
    lds_barrier();
    if (wave != 0) return;
    fold_waves<C, MT>(
        acc, [&](int w2) { return reinterpret_cast<const float*>(ldsb + w2 * wave_bytes + xbytes); },
        waves, a.group, lane);
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int n = col0 + 16 * c + col_lane;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int m = 16 * t + 4 * kq + jj;
                if (m < a.m && n < a.n) {
                    float r = acc[c][t][jj] * a.t;
                    if (OUT_F32)
                        static_cast<float*>(a.y)[(int64_t)m * a.n + (MULTI ? out_col(a, n) : n)] = r;
                    else
                        static_cast<uint16_t*>(a.y)[(int64_t)m * a.n + (MULTI ? out_col(a, n) : n)] = f32_to_bf16_rne(r);
                }
            }
    }
}

// LDS bytes of the per-tile kernel.
size_t tile_lds_bytes(int64_t m, int64_t ks, int waves, int c, int nb) {
    return size_t(waves) * (size_t(m) * (ks + 8) * 2 + size_t(nb) * c * kTileBytes);
}

// Many-row kernel (x too large to sit whole in one workgroup's LDS).  A
// workgroup owns 16*C*W output columns (W wavefronts with C column tiles
// each) and a K range of whole segment groups: one group when the groups of
// a column group meet across workgroups (parts == split), all of them when
// one workgroup runs the whole K (parts == 1).  x comes into LDS in windows
// of 512 k (one chunk), double-buffered, each row of a window one
// direct-to-LDS load; every window is read by all W wavefronts, so x is
// fetched once per 16*C*W columns instead of once per 16*C.  Each wavefront
// streams its weight chunks through two LDS buffers of its own, runs the
// chains of its segments one after the other and adds them in the two-level
// order (chains in segment order within a group, group sums in group order).
//
// With parts == split > 1 the column group's `split` workgroups are
// blockIdx = part * groups + column_group and meet through device memory
// (the workspace nvfp4_init allocates, or the fixed scratch array of
// nvfp4_linear_noalloc).  Producers (parts 0..split-2) store each group sum
// as one 64-bit word, a tag in the high half and the fp32 bits in the low
// half, so no flag, fence or barrier has to order one location against
// another: a consumer (the workgroup of the last part) that reads a word with
// the tag it expects has read the value stored with it.  Tags come from
// generation words, one per 1024-word block of the workspace.  A column
// group's words sit in blocks of its own (its region is rounded up to whole
// blocks), every workgroup reads the generations g of the blocks it touches as
// it starts, producers tag with g + 1, and the consumer, once it has read
// every word (bounded wait), advances each block of its region to g + 1.  Every
// word's tag is therefore at most its block's generation, and a call waits for
// a tag above it: no word left by an earlier call (another shape's, a replayed
// graph's, a late producer's) is ever taken.  A consumer that gives up (about
// a second) writes NaN to its outputs, sets the time-out word the host reads
// with nvfp4_timeout_status and still advances its generations.  Workgroups
// are dispatched in index order, so each part's producers are resident or done
// before its consumer waits, and producers never wait.  No read-modify-write
// atomics are used.
struct SplitArgs {
    Args a;               // a.k_per_wave: segment length; a.group: segments per group
    uint64_t* work;       // column group g at work + g * region: [split-1][W][C][MT][4][64] tagged sums
    uint32_t* gens;       // generation of each 1024-word block of `work`
    int region;           // words per column group, a whole number of blocks
    uint32_t* status;     // time-out word (set to 1 by a consumer that gave up)
    int split;            // segment groups of the tile
    int parts;            // workgroups per column group: split, or 1 (every group in one workgroup)
    int groups;           // column groups of 16*C*W
    uint32_t spin_limit;  // polls of the tagged sums before giving up
    int test_mode;        // test hook: 1 producers store nothing; 2 producers store late
};

constexpr uint32_t kSpinLimit = 1u << 20;   // polls of the tagged sums before giving up (about a second)
constexpr uint32_t kTestSpinLimit = 64;     // with the NVFP4_TEST_SPLIT_TIMEOUT hook
constexpr int kXPitch = kChunkK + 8;        // LDS row pitch of an x window (bf16 elements)
constexpr int kGenBlock = 1024;             // workspace words per generation word
constexpr int kMaxParts = 8;                // largest split

// Weight formats of the many-row kernel.  For one 512-k window of one
// 16-column tile: the LDS bytes it takes (kBytes), the direct-to-LDS loads
// that bring it in (kDma, issued by `issue`; the last kDmaSecond of them hold
// the window's second half, blocks 2 and 3), and `mma`, which multiplies half
// H of a staged window into the chains acc[C][MT] with the A operands of x
// rows xr from an x window laid out as `issue_x` stages it.

// NVFP4: the chunk layout and MFMA sequence of every NVFP4 kernel.
struct Nvfp4Window {
    static constexpr int kBytes = kTileBytes;
    static constexpr int kDma = kDmaPerTile;
    static constexpr int kDmaSecond = kDmaHalf1;
    __device__ static __forceinline__ void issue(uint8_t* dst, const Args& a, int row0, int kwin, int lane) {
        issue_tile_chunk(dst, a.wp, a.sc, row0, a.n - 1, static_cast<uint32_t>(a.k) / 2,
                         static_cast<uint32_t>(a.k) / 16, static_cast<uint32_t>(kwin) / 2, lane);
    }
    template <int C, int MT, int H>
    __device__ static __forceinline__ void mma(f32x4 (&acc)[C][MT], const uint8_t* wsrc, const uint16_t* xsrc,
                                               int pitch, const int (&xr)[MT], int col_lane, int kq) {
        mma_half<C, MT, H>(acc, wsrc, xsrc, pitch, xr, col_lane, kq);
    }
};

// FP8 block-scaled weights ("10 Kernels" 10.3): e4m3 codes [N, K] (Args::wp)
// and fp32 scales [N/128, K/128] (Args::sc).  A window of a tile holds 256
// bytes of scales (lane i's word: the tile's scale of the window's block
// i % 4; a 16-column tile lies in one 128-row scale block), then blocks 0-1
// and blocks 2-3 as 16 rows x 256 bytes each, the 16-byte piece p of row n at
// slot p ^ n so that the 16 rows of one B read meet 16 bank groups.  Each
// 128-k block is four MFMAs from zero, then fma(scale, block, chain): the
// arithmetic of fp8_w8a16_kernel, with the same k in each MFMA slot.
struct Fp8Window {
    static constexpr int kBytes = 256 + 2 * 16 * 256;
    static constexpr int kDma = 9;
    static constexpr int kDmaSecond = 4;
    __device__ static __forceinline__ void issue(uint8_t* dst, const Args& a, int row0, int kwin, int lane) {
        const int nmax = a.n - 1;
        const float* sc = reinterpret_cast<const float*>(a.sc) + (int64_t)(min(row0, nmax) / 128) * (a.k / 128) +
                          kwin / 128;
        __builtin_amdgcn_global_load_lds(sc + lane % 4, dst, 4, 0, 0);
        const int r = lane / 16, j = lane % 16;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int n = 4 * (u % 4) + r;
            const int row = min(row0 + n, nmax);
            __builtin_amdgcn_global_load_lds(a.wp + (int64_t)row * a.k + kwin + 256 * (u / 4) + 16 * (j ^ n),
                                             dst + 256 + 4096 * (u / 4) + 1024 * (u % 4), 16, 0, 0);
        }
    }
    template <int MT>
    struct Ops {
        u32x4 xa[MT][4];
        u32x4 w[2];
        float s;
    };
    template <int C, int MT, int H>
    __device__ static __forceinline__ void mma(f32x4 (&acc)[C][MT], const uint8_t* wsrc, const uint16_t* xsrc,
                                               int pitch, const int (&xr)[MT], int col_lane, int kq) {
        static_assert(C == 1, "one column tile per wavefront");
        Ops<MT> ops[2];
        // MFMA slot s of lane quarter kq takes k = 64 (s / 2) + 16 kq + 8 (s % 2) .. + 7 of the block:
        // 32-k quarter 2 (s / 2) + kq / 2 of the staged x row, eighth 2 (kq % 2) + s % 2
        auto fetch = [&](Ops<MT>& o, int b) {
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    o.xa[t][s] = *reinterpret_cast<const u32x4*>(
                        xsrc + xr[t] * pitch + kBlockK * b + 32 * xslot(2 * (s / 2) + kq / 2, xr[t]) +
                        16 * (kq % 2) + 8 * (s % 2));
#pragma unroll
            for (int h = 0; h < 2; ++h)
                o.w[h] = *reinterpret_cast<const u32x4*>(wsrc + 256 + 4096 * (b / 2) + 256 * col_lane +
                                                         16 * ((8 * (b % 2) + 4 * h + kq) ^ col_lane));
            o.s = *reinterpret_cast<const float*>(wsrc + 4 * b);
        };
        fetch(ops[0], 2 * H);
#pragma unroll
        for (int b = 2 * H; b < 2 * H + 2; ++b) {
            const Ops<MT>& o = ops[b & 1];
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0); vmcnt and expcnt not waited for
            __builtin_amdgcn_sched_barrier(0);
            if (b + 1 < 2 * H + 2) fetch(ops[(b + 1) & 1], b + 1);
            __builtin_amdgcn_sched_barrier(0);
            f32x4 blk[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) blk[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32x4 q = o.w[s / 2];
                const bf16x8 bv = fp8x8_to_bf16(q[2 * (s % 2)], q[2 * (s % 2) + 1]);
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    blk[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(o.xa[t][s]), bv, blk[t], 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[0][t][j] = __builtin_fmaf(o.s, blk[t][j], acc[0][t][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
};

template <class F, int C, int MT, int W, bool OUT_F32, bool MULTI>
__device__ __forceinline__ void split_body(const SplitArgs& sa) {
    constexpr int kXLoads = (16 * MT + W - 1) / W;      // x rows one wavefront loads per window
    extern __shared__ __align__(16) uint16_t lds[];    // x windows [2][M][kXPitch] | chunk buffers
    Args a_entry;
    if constexpr (MULTI) a_entry = entry_args(sa.a);
    const Args& a = MULTI ? a_entry : sa.a;
    if (MULTI && a.m <= 0) return;                     // an empty entry: no part of it runs
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int col_lane = lane % 16;
    const int kq = lane / 16;
    const int cgroup = (int)blockIdx.x % sa.groups;
    const int part = (int)blockIdx.x / sa.groups;
    const int krange = a.k / sa.parts;
    const int kbase = part * krange;
    const int nwin = krange / kChunkK;
    const int seg_chunks = a.k_per_wave / kChunkK;
    const int group_chunks = seg_chunks * a.group;
    const bool exchange = sa.parts > 1;
    // Exchange words of this lane: part q's row i (of kVals) is word
    // region0 + q * kSlot + lrow + 64 i (+ lane).  The generations of their
    // blocks are read as the workgroup starts (waited for only where they are
    // used, after the last window): for each part whose words the lane
    // touches, those of the blocks of its first and last row (the rows of one
    // part span at most two blocks); the consumer's wavefront 0 also reads one
    // block of its region per lane, the ones it advances at the end.
    constexpr int kSlot = W * C * MT * 4 * kWave;
    constexpr int kVals = C * MT * 4;
    const int64_t region0 = ((MULTI ? (int64_t)blockIdx.y * sa.groups : 0) + cgroup) * sa.region;
    const int lrow = wave * kVals * kWave;
    auto blk = [&](int q, int i) { return (region0 + (int64_t)q * kSlot + lrow + i * kWave) / kGenBlock; };
    uint32_t glo[kMaxParts - 1] = {}, ghi[kMaxParts - 1] = {};
    uint32_t gown = 0;
    const int nblk = exchange ? ((sa.split - 1) * kSlot + kGenBlock - 1) / kGenBlock : 0;
    if (exchange) {
        const bool consumer = part == sa.split - 1;
#pragma unroll
        for (int q = 0; q < kMaxParts - 1; ++q)
            if ((consumer && q < sa.split - 1) || q == part) {
                glo[q] = __hip_atomic_load(sa.gens + blk(q, 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ghi[q] = __hip_atomic_load(sa.gens + blk(q, kVals - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        // (every lane of every part loads it, clamped, to keep the load out
        // of a divergent branch)
        gown = __hip_atomic_load(sa.gens + region0 / kGenBlock + min(lane, nblk - 1), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    }
    // tag of row i of part q: one above its block's generation
    auto tag_of = [&](int q, int i) { return (blk(q, i) == blk(q, 0) ? glo[q] : ghi[q]) + 1; };
    const int slice = a.m * kXPitch;
    const int col_base = (cgroup * W + wave) * 16 * C;
    uint8_t* wbuf = reinterpret_cast<uint8_t*>(lds + 2 * slice) + wave * 2 * C * F::kBytes;

    int xr[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) xr[t] = min(16 * t + col_lane, a.m - 1);

    // x window `win`: rows wave, wave + W, ... (clamped to M-1: a repeated
    // load of identical data), each 1 KB landing at its LDS row.
    auto issue_x = [&](int win) {
        uint16_t* dst = lds + (win & 1) * slice;
#pragma unroll
        for (int i = 0; i < kXLoads; ++i) {
            const int r = min(wave + i * W, a.m - 1);
            __builtin_amdgcn_global_load_lds(a.x + (int64_t)r * a.k + kbase + win * kChunkK + 8 * xpiece(lane, r),
                                             dst + r * kXPitch, 16, 0, 0);
        }
    };
    auto issue_w = [&](int win) {
        const int kwin = kbase + win * kChunkK;
        uint8_t* dst = wbuf + (win & 1) * C * F::kBytes;
#pragma unroll
        for (int c = 0; c < C; ++c) F::issue(dst + c * F::kBytes, a, col_base + 16 * c, kwin, lane);
    };

    f32x4 acc[C][MT], grp[C][MT], tot[C][MT];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[c][t] = grp[c][t] = tot[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute_half = [&](int win, auto h) {
        F::template mma<C, MT, decltype(h)::value>(acc, wbuf + (win & 1) * C * F::kBytes, lds + (win & 1) * slice,
                                                   kXPitch, xr, col_lane, kq);
    };
    // window win: its first half is in LDS (and, with `barrier`, every
    // wavefront's x rows of it); waits for the second half (at most `after`
    // later loads outstanding), multiplies it, folds at a segment end
    auto compute = [&](int win, auto after) {
        compute_half(win, std::integral_constant<int, 0>{});
        wait_vm<decltype(after)::value>();
        compute_half(win, std::integral_constant<int, 1>{});
        // end of a segment: its chain joins the group sum; at the end of a
        // group (several per workgroup only when parts == 1) the group sum
        // joins the total.  The first chain and the first group sum are
        // taken as they are, so a -0 sum keeps its sign.
        if ((win + 1) % seg_chunks == 0) {
            const bool first = (win + 1 - seg_chunks) % group_chunks == 0;
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    grp[c][t] = first ? acc[c][t] : grp[c][t] + acc[c][t];
                    acc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            if (!exchange && (win + 1) % group_chunks == 0) {
                const bool gfirst = win + 1 == group_chunks;
#pragma unroll
                for (int c = 0; c < C; ++c)
#pragma unroll
                    for (int t = 0; t < MT; ++t) tot[c][t] = gfirst ? grp[c][t] : tot[c][t] + grp[c][t];
            }
        }
    };

    if (MT == 1 && nwin == 2) {
        // Both windows requested at once: with one row tile the multiply of
        // window 0 is short, and issuing window 1 only after window 0 has
        // landed left the wavefronts waiting about one memory latency for it
        // (measured on MI355X; with two row tiles, or more windows, the
        // one-ahead schedule below is faster).
        issue_x(0);
        issue_w(0);
        issue_x(1);
        issue_w(1);
        wait_vm<kXLoads + F::kDma * C + F::kDmaSecond>();   // window 0's x rows and first half have landed
        lds_barrier();                                      // ... for every wavefront
        compute(0, std::integral_constant<int, kXLoads + F::kDma * C>{});
        wait_vm<F::kDmaSecond>();
        lds_barrier();
        compute(1, std::integral_constant<int, 0>{});
    } else {
        // Window w is multiplied while window w + 1 (x and weights) is in
        // flight.
        issue_x(0);
        issue_w(0);
        wait_vm<F::kDmaSecond>();                       // x rows and the first half of window 0
        lds_barrier();
        int win = 0;
        for (; win + 1 < nwin; ++win) {
            issue_x(win + 1);
            issue_w(win + 1);
            wait_vm<kXLoads + F::kDma * C + F::kDmaSecond>();   // window win's first half has landed
            compute(win, std::integral_constant<int, kXLoads + F::kDma * C>{});
            wait_vm<F::kDma * C>();             // this wavefront's x rows of win + 1 have landed
            lds_barrier();                          // ... and everyone's; buffer win & 1 is free
        }
        wait_vm<F::kDmaSecond>();
        compute(win, std::integral_constant<int, 0>{});
    }

    if (exchange) {
        const int P = sa.split;
        uint64_t* work = sa.work + region0;
        const int base = lrow + lane;
        if (part < P - 1) {
            if (sa.test_mode == 1) return;                   // test hook: nothing arrives
            if (sa.test_mode == 2)                           // test hook: a producer far behind its consumer
                for (int i = 0; i < 4096; ++i) __builtin_amdgcn_s_sleep(127);
            uint64_t* slot = work + (size_t)part * kSlot + base;
#pragma unroll
            for (int q = 0; q < kMaxParts - 1; ++q)
                if (q == part)
#pragma unroll
                    for (int c = 0; c < C; ++c)
#pragma unroll
                        for (int t = 0; t < MT; ++t)
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const int i = (c * MT + t) * 4 + j;
                                __hip_atomic_store(slot + i * kWave,
                                                   (uint64_t(tag_of(q, i)) << 32) |
                                                       f32_bits(grp[c][t][j]),
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            }
            return;
        }
        // The consumer reads the tagged sums of the parts in batches (all
        // loads of a batch in flight together) until every tag of the batch
        // is this call's, polling a bounded number of times; then adds them
        // in group order, its own last.  Each wavefront waits on its own
        // lanes' words only.
        constexpr int kBatch = 32 / kVals;
        bool bad = false;
#pragma unroll
        for (int q0 = 0; q0 < kMaxParts - 1; q0 += kBatch) {
            if (q0 >= P - 1 || bad) break;
            uint64_t v[kBatch][kVals];
            for (uint32_t spins = 0;; ++spins) {
#pragma unroll
                for (int b = 0; b < kBatch; ++b)
                    if (q0 + b < P - 1)
#pragma unroll
                        for (int i = 0; i < kVals; ++i)
                            v[b][i] = __hip_atomic_load(work + (size_t)(q0 + b) * kSlot + base + i * kWave,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                bool here = true;
#pragma unroll
                for (int b = 0; b < kBatch; ++b)
                    if (q0 + b < P - 1)
#pragma unroll
                        for (int i = 0; i < kVals; ++i) here &= uint32_t(v[b][i] >> 32) == tag_of(q0 + b, i);
                if (__all(here)) break;
                if (spins >= sa.spin_limit) {
                    bad = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                if (q0 + b < P - 1)
#pragma unroll
                    for (int c = 0; c < C; ++c)
#pragma unroll
                        for (int t = 0; t < MT; ++t)
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const float g = bits_f32(uint32_t(v[b][(c * MT + t) * 4 + j]));
                                tot[c][t][j] = q0 + b == 0 ? g : tot[c][t][j] + g;
                            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    grp[c][t][j] = bad ? __builtin_nanf("") : tot[c][t][j] + grp[c][t][j];
        if (bad && lane == 0) __hip_atomic_store(sa.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // The next call on these blocks waits for the next tag.  (The empty
        // asm keeps the compiler from adding 1 to the loaded generation right
        // after its load, which would wait for it before the first window.)
        asm volatile("" : "+v"(gown));
        if (wave == 0 && lane < nblk)
            __hip_atomic_store(sa.gens + region0 / kGenBlock + lane, gown + 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    } else if (a.group < a.k / a.k_per_wave) {
        // every group in this workgroup: the output is the total
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int t = 0; t < MT; ++t) grp[c][t] = tot[c][t];
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
                    float r = grp[c][t][j] * a.t;
                    if (OUT_F32)
                        static_cast<float*>(a.y)[(int64_t)m * a.n + (MULTI ? out_col(a, n) : n)] = r;
                    else
                        static_cast<uint16_t*>(a.y)[(int64_t)m * a.n + (MULTI ? out_col(a, n) : n)] = f32_to_bf16_rne(r);
                }
            }
    }
}

template <int C, int MT, int W, bool OUT_F32, bool MULTI>
__global__ void __launch_bounds__(64 * W)
nvfp4_skinny_split(SplitArgs sa) {
    split_body<Nvfp4Window, C, MT, W, OUT_F32, MULTI>(sa);
}

// The many-row kernel on FP8 block-scaled weights (a.t is 1).
template <int MT, int W, bool OUT_F32>
__global__ void __launch_bounds__(64 * W)
fp8_w8a16_split(SplitArgs sa) {
    split_body<Fp8Window, 1, MT, W, OUT_F32, false>(sa);
}

// LDS bytes of the many-row kernel (dynamic part); tile_bytes: a window of
// one column tile.
size_t split_lds_bytes(int64_t m, int w, int c, int tile_bytes = kTileBytes) {
    return 2 * size_t(m) * kXPitch * sizeof(uint16_t) + size_t(w) * 2 * c * tile_bytes;
}

using KernelFn = void (*)(Args);
using SplitFn = void (*)(SplitArgs);

// y_dtype may carry kMulti: the instantiation of a several-product launch.
constexpr int kMulti = 0x100;

template <int C, int MT, int U, bool XLDS>
KernelFn pick_out(int y_dtype) {
    const bool f = (y_dtype & 0xff) == NVFP4_OUT_F32;
    if (y_dtype & kMulti) return f ? nvfp4_skinny<C, MT, U, XLDS, true, true> : nvfp4_skinny<C, MT, U, XLDS, false, true>;
    return f ? nvfp4_skinny<C, MT, U, XLDS, true, false> : nvfp4_skinny<C, MT, U, XLDS, false, false>;
}

// Pipeline depth of the generic kernel, capped where deeper steps would spill
// registers to scratch (measured with the compiler's resource-usage report):
// with A operands fetched per chunk (no x in LDS) one 128-k block per step,
// and with four column tiles per wavefront at most two blocks per step.  The
// depth never changes bits.
constexpr int generic_unroll(int unroll, int c, bool xlds) {
    return !xlds ? 1 : (c == 4 && unroll > 2) ? 2 : unroll;
}

template <int C, int MT>
KernelFn pick_u(int unroll, bool xlds, int y_dtype) {
    if (!xlds) return pick_out<C, MT, 1, false>(y_dtype);
    switch (generic_unroll(unroll, C, true)) {
        case 1: return pick_out<C, MT, 1, true>(y_dtype);
        case 2: return pick_out<C, MT, 2, true>(y_dtype);
        default: return pick_out<C, MT, C == 4 ? 2 : 4, true>(y_dtype);
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

template <int C, int MT, int NB>
KernelFn pick_p_out(int y_dtype) {
    const bool f = (y_dtype & 0xff) == NVFP4_OUT_F32;
    if (y_dtype & kMulti)
        return f ? nvfp4_skinny_persistent<C, MT, NB, true, true> : nvfp4_skinny_persistent<C, MT, NB, false, true>;
    return f ? nvfp4_skinny_persistent<C, MT, NB, true, false> : nvfp4_skinny_persistent<C, MT, NB, false, false>;
}

template <int NB>
KernelFn pick_p_c(int mt, int c, int y_dtype) {
    if (mt == 1) return c == 1 ? pick_p_out<1, 1, NB>(y_dtype) : pick_p_out<2, 1, NB>(y_dtype);
    return c == 1 ? pick_p_out<1, 2, NB>(y_dtype) : pick_p_out<2, 2, NB>(y_dtype);
}

// c: column tiles per wavefront (1 or 2); nb: chunk buffers per wavefront (2 or 3)
KernelFn pick_persistent(int mt, int c, int nb, int y_dtype) {
    return nb == 3 ? pick_p_c<3>(mt, c, y_dtype) : pick_p_c<2>(mt, c, y_dtype);
}

template <int C, int MT, int NB>
KernelFn pick_t_out(int y_dtype) {
    const bool f = (y_dtype & 0xff) == NVFP4_OUT_F32;
    if (y_dtype & kMulti) return f ? nvfp4_skinny_tile<C, MT, NB, true, true> : nvfp4_skinny_tile<C, MT, NB, false, true>;
    return f ? nvfp4_skinny_tile<C, MT, NB, true, false> : nvfp4_skinny_tile<C, MT, NB, false, false>;
}

template <int NB>
KernelFn pick_t_c(int mt, int c, int y_dtype) {
    if (mt == 1) return c == 1 ? pick_t_out<1, 1, NB>(y_dtype) : pick_t_out<2, 1, NB>(y_dtype);
    return c == 1 ? pick_t_out<1, 2, NB>(y_dtype) : pick_t_out<2, 2, NB>(y_dtype);
}

// per-tile kernel; c: column tiles per wavefront (1 or 2); nb: chunk buffers (1..3)
KernelFn pick_tile(int mt, int c, int nb, int y_dtype) {
    return nb == 3 ? pick_t_c<3>(mt, c, y_dtype) : nb == 2 ? pick_t_c<2>(mt, c, y_dtype) : pick_t_c<1>(mt, c, y_dtype);
}

template <int C, int MT, int W>
SplitFn pick_s_out(int y_dtype) {
    const bool f = (y_dtype & 0xff) == NVFP4_OUT_F32;
    if (y_dtype & kMulti) return f ? nvfp4_skinny_split<C, MT, W, true, true> : nvfp4_skinny_split<C, MT, W, false, true>;
    return f ? nvfp4_skinny_split<C, MT, W, true, false> : nvfp4_skinny_split<C, MT, W, false, false>;
}

template <int MT>
SplitFn pick_s_w(int c, int w, int y_dtype) {
    if (c == 1)
        return w == 4 ? pick_s_out<1, MT, 4>(y_dtype) : w == 6 ? pick_s_out<1, MT, 6>(y_dtype) : pick_s_out<1, MT, 8>(y_dtype);
    return w == 4 ? pick_s_out<2, MT, 4>(y_dtype) : w == 6 ? pick_s_out<2, MT, 6>(y_dtype) : pick_s_out<2, MT, 8>(y_dtype);
}

// c: column tiles per wavefront (1 or 2), w: wavefronts per workgroup (4, 6 or 8)
SplitFn pick_split(int mt, int c, int w, int y_dtype) {
    return mt == 1 ? pick_s_w<1>(c, w, y_dtype) : pick_s_w<2>(c, w, y_dtype);
}

template <int MT>
SplitFn pick_f8s_w(int w, bool f) {
    if (w == 2) return f ? fp8_w8a16_split<MT, 2, true> : fp8_w8a16_split<MT, 2, false>;
    if (w == 4) return f ? fp8_w8a16_split<MT, 4, true> : fp8_w8a16_split<MT, 4, false>;
    return f ? fp8_w8a16_split<MT, 6, true> : fp8_w8a16_split<MT, 6, false>;
}

// The FP8 many-row kernel; w: wavefronts per workgroup (2, 4 or 6)
SplitFn pick_fp8_split(int mt, int w, int y_dtype) {
    const bool f = y_dtype == NVFP4_OUT_F32;
    return mt == 1 ? pick_f8s_w<1>(w, f) : pick_f8s_w<2>(w, f);
}

constexpr int kMaxDevices = 64;
constexpr size_t kWorkBytes = size_t(32) << 20;      // tagged group sums of the many-row kernel
constexpr size_t kGenWords = kWorkBytes / sizeof(uint64_t) / kGenBlock;   // one per block of them
constexpr size_t kStatusWords = 64;                  // the time-out word, on its own 256 bytes
constexpr size_t kGemmPartBytes = size_t(64) << 20;  // per-group partial sums of the many-row GEMM

// Fixed scratch of nvfp4_linear_noalloc, in 32-bit words: 8 MiB of tagged
// group sums, their generation words, then the time-out word.
constexpr size_t kScratchSumBytes = size_t(8) << 20;
constexpr size_t kScratchGenWords = kScratchSumBytes / sizeof(uint64_t) / kGenBlock;
constexpr size_t kScratchWords = kScratchSumBytes / 4 + kScratchGenWords + kStatusWords;

}  // namespace

// The many-row kernel's exchange memory for callers that cannot allocate
// (nvfp4_linear_noalloc): one copy per device, zero when the code object is
// loaded, held until the process ends.  Host code never passes this name to a
// kernel: it uses the device address hipGetSymbolAddress returns for it.
static __device__ __align__(256) uint32_t scratch[kScratchWords];

namespace {

// Where the many-row kernel's column groups meet: tagged group sums, the
// generation words of their blocks, the time-out word.  All start at zero;
// generations only ever advance, so the memory is never cleared again.
struct Workspace {
    float* sums = nullptr;
    uint32_t* gens = nullptr;
    uint32_t* status = nullptr;
    size_t sum_bytes = 0;
    size_t gen_words = 0;
};

// Per-device state: the set-up that allocates nothing (kernel attributes,
// the fixed scratch address), and the workspace nvfp4_init allocates.
struct DeviceState {
    std::once_flag setup_once, alloc_once;
    int setup_status = NVFP4_OK;
    int cus = 0;
    Workspace heap;                 // device memory, never freed
    float* gemm_part = nullptr;     // device memory, never freed: the GEMM's group partial sums
    Workspace fixed;                // this device's `scratch` array
};
DeviceState g_dev[kMaxDevices];

template <typename Fn>
bool allow_full_lds(Fn fn) {
    const void* f = reinterpret_cast<const void*>(fn);
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, f) != hipSuccess) return false;
    // the static LDS of the kernel counts against the same 160 KB
    const int dyn = kMaxLdsBytes - static_cast<int>(attr.sharedSizeBytes);
    return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, dyn) == hipSuccess;
}

// Set-up of the current device `dev`, once per device; allocates nothing.
int setup_device(int dev) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return NVFP4_ERR_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return NVFP4_ERR_DEVICE;
    DeviceState& d = g_dev[dev];
    d.cus = prop.multiProcessorCount;
    // Touch every kernel so its code object is loaded before any graph
    // capture, and let each use the whole LDS.
    const int cols[3] = {16, 32, 64};
    for (int mt = 1; mt <= 2; ++mt)
        for (int od : {int(NVFP4_OUT_BF16), int(NVFP4_OUT_F32), NVFP4_OUT_BF16 | kMulti, NVFP4_OUT_F32 | kMulti}) {
            for (int ci = 0; ci < 3; ++ci)
                for (int un = 1; un <= 4; un *= 2)
                    for (int xl = 0; xl <= 1; ++xl)
                        if (!allow_full_lds(pick_kernel(mt, cols[ci], un, xl != 0, od))) return NVFP4_ERR_HIP;
            for (int c = 1; c <= 2; ++c)
                for (int nb = 2; nb <= 3; ++nb)
                    if (!allow_full_lds(pick_persistent(mt, c, nb, od))) return NVFP4_ERR_HIP;
            for (int c = 1; c <= 2; ++c)
                for (int nb = 1; nb <= 3; ++nb)
                    if (!allow_full_lds(pick_tile(mt, c, nb, od))) return NVFP4_ERR_HIP;
            for (int c = 1; c <= 2; ++c)
                for (int w = 4; w <= 8; w += 2)
                    if (!allow_full_lds(pick_split(mt, c, w, od))) return NVFP4_ERR_HIP;
            if (!(od & kMulti))
                for (int w = 2; w <= 6; w += 2)
                    if (!allow_full_lds(pick_fp8_split(mt, w, od))) return NVFP4_ERR_HIP;
        }
    int st = nvfp4::gemm_setup();
    if (st == NVFP4_OK) st = nvfp4::w8a16_setup();
    if (st != NVFP4_OK) return st;
    // This device's copy of the fixed scratch array, by its device address.
    void* sp = nullptr;
    if (hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch)) != hipSuccess || sp == nullptr) return NVFP4_ERR_HIP;
    uint32_t* words = static_cast<uint32_t*>(sp);
    d.fixed.sums = reinterpret_cast<float*>(words);
    d.fixed.gens = words + kScratchSumBytes / 4;
    d.fixed.status = d.fixed.gens + kScratchGenWords;
    d.fixed.sum_bytes = kScratchSumBytes;
    d.fixed.gen_words = kScratchGenWords;
    return NVFP4_OK;
}

// The workspace of `dev`, once per device: ordinary device memory (every
// access to it is an agent-scope atomic, so the L2 of one XCD never hides a
// store from another; measured 1-2 % faster than uncached memory).  Without it the
// many-row kernel runs only where no exchange is needed (the other kernels
// give the same bits).
void alloc_workspace(int dev) {
    DeviceState& d = g_dev[dev];
    void* work = nullptr;
    void* gens = nullptr;
    const size_t gen_bytes = (kGenWords + kStatusWords) * sizeof(uint32_t);
    if (hipMalloc(&work, kWorkBytes) == hipSuccess && hipMalloc(&gens, gen_bytes) == hipSuccess &&
        hipMemset(gens, 0, gen_bytes) == hipSuccess && hipMemset(work, 0, kWorkBytes) == hipSuccess &&
        hipDeviceSynchronize() == hipSuccess) {
        d.heap.sums = static_cast<float*>(work);
        d.heap.gens = static_cast<uint32_t*>(gens);
        d.heap.status = d.heap.gens + kGenWords;
        d.heap.sum_bytes = kWorkBytes;
        d.heap.gen_words = kGenWords;
    } else {
        (void)hipGetLastError();   // clear the failure; the memory (if any) stays unused
    }
    // The many-row GEMM's per-group partial sums: written in full before they
    // are read by every call that uses them, so never cleared.
    void* part = nullptr;
    if (hipMalloc(&part, kGemmPartBytes) == hipSuccess)
        d.gemm_part = static_cast<float*>(part);
    else
        (void)hipGetLastError();   // the GEMM then runs every group in one workgroup
}

std::once_flag g_init_once;
int g_init_status = NVFP4_OK;
// Test hook, read once per process (NVFP4_TEST_SPLIT_TIMEOUT): 1 makes the
// many-row kernel's producers store no group sums, 2 makes them store them
// only after a long bounded delay; either way its consumers give up after a
// few polls, so a test can see the time-out path (every kernel still exits
// normally).
int g_test_split_timeout = 0;

int current_device(int* dev) {
    if (hipGetDevice(dev) != hipSuccess) return NVFP4_ERR_HIP;
    if (*dev < 0 || *dev >= kMaxDevices) return NVFP4_ERR_DEVICE;
    return NVFP4_OK;
}

// Process-wide set-up (test hook, tile override) and the current device's
// set-up; allocates nothing.  *dev is the current device.
int setup_current(int* dev) {
    std::call_once(g_init_once, [] {
        const char* hook = std::getenv("NVFP4_TEST_SPLIT_TIMEOUT");
        g_test_split_timeout = hook ? std::atoi(hook) : 0;
        if (g_test_split_timeout != 1 && g_test_split_timeout != 2) g_test_split_timeout = 0;
        g_init_status = nvfp4::load_tile_override();
    });
    if (g_init_status != NVFP4_OK) return g_init_status;
    int st = current_device(dev);
    if (st != NVFP4_OK) return st;
    DeviceState& d = g_dev[*dev];
    std::call_once(d.setup_once, [&] { d.setup_status = setup_device(*dev); });
    return d.setup_status;
}

}  // namespace

namespace nvfp4 {

int device_setup() {
    int dev = 0;
    return setup_current(&dev);
}

int device_cus() {
    int dev = 0;
    if (current_device(&dev) != NVFP4_OK || g_dev[dev].cus <= 0) return 256;
    return g_dev[dev].cus;
}

}  // namespace nvfp4

extern "C" int nvfp4_init(void) {
    int dev = 0;
    const int st = setup_current(&dev);
    if (st != NVFP4_OK) return st;
    DeviceState& d = g_dev[dev];
    std::call_once(d.alloc_once, [&] { alloc_workspace(dev); });
    return NVFP4_OK;
}

namespace nvfp4 {

int gemm_partials(float** part, size_t* bytes, int* cus) {
    *part = nullptr;
    *bytes = 0;
    const int st = nvfp4_init();
    if (st != NVFP4_OK) return st;
    int dev = 0;
    if (current_device(&dev) != NVFP4_OK) return NVFP4_ERR_HIP;
    *cus = g_dev[dev].cus > 0 ? g_dev[dev].cus : 256;
    if (g_dev[dev].gemm_part) {
        *part = g_dev[dev].gemm_part;
        *bytes = kGemmPartBytes;
    }
    return NVFP4_OK;
}

int launch_fp8_split(const void* x, const uint8_t* w, const float* s, void* y, int64_t m, int64_t n, int64_t k,
                     int y_dtype, int waves, int group, int wg_waves, bool whole, void* stream, bool* launched) {
    *launched = false;
    int st = nvfp4_init();
    if (st != NVFP4_OK) return st;
    int dev = 0;
    st = current_device(&dev);
    if (st != NVFP4_OK) return st;
    const Workspace& ws = g_dev[dev].heap;
    const int64_t seg = k / waves;
    if (m < 1 || m > 32 || seg % kChunkK != 0 || (wg_waves != 2 && wg_waves != 4 && wg_waves != 6))
        return NVFP4_OK;
    const int mt = m <= 16 ? 1 : 2;
    const size_t lds = split_lds_bytes(m, wg_waves, 1, Fp8Window::kBytes);
    if (lds + 256 > size_t(kMaxLdsBytes)) return NVFP4_OK;
    const int split = waves / group;
    const int64_t groups = (n + 16 * wg_waves - 1) / (16 * wg_waves);
    int parts = 1;
    int64_t region = 0;
    if (split > 1 && !whole) {
        const int64_t slot = int64_t(wg_waves) * mt * 4 * kWave;     // words of one workgroup
        region = ((split - 1) * slot + kGenBlock - 1) / kGenBlock * kGenBlock;
        const size_t words = size_t(groups) * size_t(region);
        if (!ws.sums || words * sizeof(uint64_t) > ws.sum_bytes || words / kGenBlock > ws.gen_words)
            return NVFP4_OK;
        parts = split;
    }
    Args a{};
    a.x = static_cast<const uint16_t*>(x);
    a.wp = w;
    a.sc = reinterpret_cast<const uint8_t*>(s);
    a.y = y;
    a.t = 1.0f;
    a.m = static_cast<int>(m);
    a.n = static_cast<int>(n);
    a.k = static_cast<int>(k);
    a.k_per_wave = static_cast<int>(seg);
    a.group = group;
    SplitArgs sa;
    sa.a = a;
    sa.work = reinterpret_cast<uint64_t*>(ws.sums);
    sa.gens = ws.gens;
    sa.region = static_cast<int>(region);
    sa.status = ws.status;
    sa.split = split;
    sa.parts = parts;
    sa.spin_limit = g_test_split_timeout ? kTestSpinLimit : kSpinLimit;
    sa.test_mode = g_test_split_timeout;
    sa.groups = static_cast<int>(groups);
    hipLaunchKernelGGL(pick_fp8_split(mt, wg_waves, y_dtype), dim3(static_cast<unsigned>(groups * parts)),
                       dim3(static_cast<unsigned>(kWave * wg_waves)), lds, static_cast<hipStream_t>(stream), sa);
    if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
    *launched = true;
    return NVFP4_OK;
}

}  // namespace nvfp4

extern "C" int nvfp4_timeout_status(int* timed_out) {
    if (!timed_out) return NVFP4_ERR_NULL;
    int dev = 0;
    const int st = setup_current(&dev);
    if (st != NVFP4_OK) return st;
    DeviceState& d = g_dev[dev];
    if (hipDeviceSynchronize() != hipSuccess) return NVFP4_ERR_HIP;
    uint32_t any = 0;
    for (const Workspace* w : {&d.heap, &d.fixed}) {
        if (!w->status) continue;
        uint32_t v = 0;
        if (hipMemcpy(&v, w->status, sizeof v, hipMemcpyDeviceToHost) != hipSuccess) return NVFP4_ERR_HIP;
        if (v != 0) {
            const uint32_t zero = 0;
            if (hipMemcpy(w->status, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess) return NVFP4_ERR_HIP;
        }
        any |= v;
    }
    *timed_out = any != 0;
    return NVFP4_OK;
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

// Launch plan of the many-row kernel; false if it cannot run this call.
// `ws` is the workspace the call may use (NULL: none), `parts` what runs:
// split when the groups meet through the workspace, else 1.
struct SplitPlan {
    int c = 1, w = 8;
    int parts = 1;
    int64_t region = 0;             // exchange words per column group
    bool scratch_short = false;     // an exchange was needed and did not fit `ws`
    int64_t groups = 0;
    size_t lds = 0;
};

bool plan_split(const nvfp4::Tile& tile, int64_t m, int64_t n, int64_t k, const Workspace* ws, bool whole,
                SplitPlan* p, int64_t count = 1) {
    const int64_t seg = k / tile.waves;
    if (seg % kChunkK != 0) return false;
    p->c = tile.cols == 16 ? 1 : 2;
    // mwaves 0: four wavefronts per workgroup up to 16 rows, eight above
    // (measured on MI355X; never changes bits; six suits N = 96 * 256)
    p->w = tile.mwaves != 0 ? tile.mwaves : m <= 16 ? 4 : 8;
    const int64_t cols = int64_t(16) * p->c * p->w;
    p->groups = (n + cols - 1) / cols;
    p->lds = split_lds_bytes(m, p->w, p->c);
    if (p->lds + 256 > size_t(kMaxLdsBytes)) return false;
    p->parts = 1;
    if (tile.split > 1 && !whole) {
        const int mt = m <= 16 ? 1 : 2;
        const int64_t slot = int64_t(p->w) * p->c * mt * 4 * kWave;     // words of one workgroup
        p->region = ((tile.split - 1) * slot + kGenBlock - 1) / kGenBlock * kGenBlock;
        if (!ws || !ws->sums) return false;
        // the words, and one generation word per block of them (regions of
        // their own for each product of a several-product launch)
        const size_t words = size_t(count) * size_t(p->groups) * size_t(p->region);
        if (words * sizeof(uint64_t) > ws->sum_bytes || words / kGenBlock > ws->gen_words) {
            p->scratch_short = true;
            return false;
        }
        p->parts = tile.split;
    }
    return p->groups * tile.split <= int64_t(0x7fffffff);
}

// The kernel a launch runs, as its template name reads in a kernel trace.
std::string kernel_text(const char* fn, std::initializer_list<int> params, int y_dtype, dim3 grid, dim3 block,
                        size_t lds) {
    std::string s = fn;
    s += "<";
    for (int v : params) s += std::to_string(v) + ", ";
    s += y_dtype == NVFP4_OUT_F32 ? "true, false>" : "false, false>";   // output type; not a several-product launch
    s += " grid=" + std::to_string(grid.x) + " block=" + std::to_string(block.x) + " lds=" + std::to_string(lds);
    return s;
}

// Validates and launches one product (or, with `ml`, the products of a
// several-product launch, m then bounding every product's rows); with
// `describe` set it launches nothing and writes there the kernel it would
// run (pointers unchecked).  The pointers a device table holds are the
// caller's to check.
int launch(const void* x_bf16, const uint8_t* w_packed, const uint8_t* scales_e4m3, float tensor_scale,
           void* y, int64_t m, int64_t n, int64_t k, int y_dtype, void* stream, const nvfp4::Tile& tile,
           int kernel, bool noalloc, std::string* describe = nullptr, const nvfp4::MultiLaunch* ml = nullptr) {
    int st = nvfp4_linear_shape_ok(m, n, k);
    if (st != NVFP4_OK) return st;
    if (y_dtype != NVFP4_OUT_BF16 && y_dtype != NVFP4_OUT_F32) return NVFP4_ERR_DTYPE;
    if (m == 0) {
        if (describe) *describe = "none";
        return NVFP4_OK;
    }
    const bool tabled = ml && ml->table;
    if (!describe && !tabled) {
        if (!x_bf16 || !w_packed || !scales_e4m3 || !y) return NVFP4_ERR_NULL;
        auto misaligned = [](const void* p, uintptr_t al) { return (reinterpret_cast<uintptr_t>(p) & (al - 1)) != 0; };
        if (misaligned(x_bf16, 16) || misaligned(w_packed, 16) || misaligned(scales_e4m3, 16) ||
            misaligned(y, y_dtype == NVFP4_OUT_F32 ? 4 : 2))
            return NVFP4_ERR_ALIGN;
    }
    int dev = 0;
    if (noalloc) {
        st = setup_current(&dev);               // no allocation: the fixed scratch
    } else {
        st = nvfp4_init();
        if (st == NVFP4_OK) st = current_device(&dev);
    }
    if (st != NVFP4_OK) return st;
    const DeviceState& d = g_dev[dev];
    const Workspace* ws = noalloc ? &d.fixed : &d.heap;

    const int mt = m <= 16 ? 1 : 2;
    Args a{};
    a.x = static_cast<const uint16_t*>(x_bf16);
    a.wp = w_packed;
    a.sc = scales_e4m3;
    a.y = y;
    a.t = tensor_scale;
    a.m = static_cast<int>(m);
    a.n = static_cast<int>(n);
    a.k = static_cast<int>(k);
    a.k_per_wave = static_cast<int>(k / tile.waves);
    a.group = tile.waves / tile.split;
    const unsigned count = ml ? static_cast<unsigned>(ml->count) : 1u;
    const int yd = y_dtype | (ml ? kMulti : 0);   // the kernels' instantiation
    if (ml) {
        a.table = ml->table;
        a.wp1 = ml->wp1;
        a.sc1 = ml->sc1;
        a.y1 = ml->y1;
        a.t1 = ml->t1;
        a.omap_parts = ml->omap_parts;
        for (int i = 0; i < 4; ++i) a.omap_width[i] = ml->omap_width[i];
        a.omap_gwidth = ml->omap_gwidth;
        a.omap_ngroups = ml->omap_ngroups;
        a.slice_rows = ml->slice_rows;
        a.rows_total = ml->rows_total;
        a.y_bytes = y_dtype == NVFP4_OUT_F32 ? 4 : 2;
        a.xu = static_cast<const uint16_t*>(ml->up);
    }
    const int c = tile.cols / 16;
    const hipStream_t hs = static_cast<hipStream_t>(stream);

    // The persistent kernel when x [M, K], two buffers of segment partials
    // and the wavefronts' chunk buffers fit one workgroup's LDS and the
    // segments are whole chunks; two workgroups per CU when two fit.
    const size_t x_bytes = size_t(m) * (k + 8) * sizeof(uint16_t);
    // Three chunk buffers per wavefront when they fit, else two.
    const int pc = tile.cols == 16 ? 1 : 2;
    const int pnb = persistent_lds_bytes(m, k, tile.waves, pc, mt, 3) + 256 <= size_t(kMaxLdsBytes) ? 3 : 2;
    const size_t pers_bytes = persistent_lds_bytes(m, k, tile.waves, pc, mt, pnb);
    const bool pers_ok = tile.cols <= 32 && (k / tile.waves) % kChunkK == 0 &&
                         pers_bytes + 256 <= size_t(kMaxLdsBytes) && x_bytes <= size_t(64 * 1024);
    SplitPlan plan;
    const bool whole = kernel == NVFP4_KERNEL_WHOLE;
    const bool split_ok = plan_split(tile, m, n, k, ws, whole, &plan, count);
    if (whole) kernel = NVFP4_KERNEL_SPLIT;
    // The per-tile kernel: each wavefront's x slice and chunk buffers (up to
    // three, at most one per chunk of its segment) within the LDS: the most
    // that fit, except that where a CU has to take several workgroups, fewer
    // buffers are used if that keeps at least three of them resident
    // (measured on MI355X: 24576x4096 at M = 2 and 4, two buffers leave two
    // workgroups per CU and take 17.4 and 19.0 us, one buffer four and three,
    // 14.9 and 17.6 us; at M = 1 three fit with two buffers, which is faster).
    const int64_t ks = k / tile.waves;
    int tnb = int(std::min<int64_t>(3, std::max<int64_t>(1, ks / kChunkK)));
    while (tnb > 1 && tile_lds_bytes(m, ks, tile.waves, pc, tnb) + 256 > size_t(kMaxLdsBytes)) --tnb;
    const int cus = d.cus > 0 ? d.cus : 256;
    const int64_t tile_per_cu = ((n + 16 * pc - 1) / (16 * pc) + cus - 1) / cus;   // workgroups each CU must run
    auto tile_resident = [&](int nb) {
        return int64_t(kMaxLdsBytes) / int64_t(tile_lds_bytes(m, ks, tile.waves, pc, nb) + 256);
    };
    {
        const int64_t want = std::min<int64_t>(3, tile_per_cu);
        while (tnb > 1 && tile_resident(tnb) < want && tile_resident(tnb - 1) > tile_resident(tnb)) --tnb;
    }
    size_t tile_bytes = tile_lds_bytes(m, ks, tile.waves, pc, tnb);
    const bool tile_ok = tile.cols <= 32 && ks % kChunkK == 0 && tile_bytes + 256 <= size_t(kMaxLdsBytes);
    // Measured on MI355X (decode-round and output-head shapes, M = 1..8): the
    // per-tile kernel leads at one row; up to four rows too (its workgroups
    // are short and several share a CU), unless each CU would run more than
    // three rounds of them and the many-row kernel needs no exchange between
    // workgroups (151552x4096 at M = 2..4: 89-96 us per-tile, 69-76 us
    // many-row); up to eight rows while all its workgroups are resident at
    // once (each workgroup stages all of x, so its x traffic grows with M).
    // Then the many-row kernel where its segment groups need no exchange
    // (split 1), the persistent one while x fits, and the many-row kernel.
    const bool many_rounds = tile_per_cu > 3 * tile_resident(tnb);
    const bool tile_first =
        tile_ok && (m == 1 || (m <= 4 && !(many_rounds && split_ok && tile.split == 1)) ||
                    (m <= 8 && tile_resident(tnb) >= tile_per_cu));
    if (ml && ml->up) {
        // The silu input runs in one kernel only where the product's own
        // choice is the per-tile kernel and its LDS also holds the up slices
        // (as many chunk buffers as fit); otherwise the caller forms the
        // activation first.
        if (kernel != NVFP4_KERNEL_AUTO || !tile_first) return nvfp4::kNotFused;
        int snb = tnb;
        while (snb > 1 && tile_lds_bytes(2 * m, ks, tile.waves, pc, snb) + 256 > size_t(kMaxLdsBytes)) --snb;
        if (tile_lds_bytes(2 * m, ks, tile.waves, pc, snb) + 256 > size_t(kMaxLdsBytes)) return nvfp4::kNotFused;
        tnb = snb;
        tile_bytes = tile_lds_bytes(2 * m, ks, tile.waves, pc, snb);
        kernel = NVFP4_KERNEL_TILE;
    }
    if (kernel == NVFP4_KERNEL_AUTO) {
        // The fixed scratch has a stated size: a call whose exchange would
        // need more of it is refused, not run another way.
        if (noalloc && plan.scratch_short && !tile_first && !pers_ok) return NVFP4_ERR_SCRATCH;
        kernel = tile_first                   ? NVFP4_KERNEL_TILE
                 : split_ok && tile.split == 1 ? NVFP4_KERNEL_SPLIT
                 : pers_ok                     ? NVFP4_KERNEL_PERSISTENT
                 : split_ok                    ? NVFP4_KERNEL_SPLIT
                                               : NVFP4_KERNEL_GENERIC;
    }
    if ((kernel == NVFP4_KERNEL_PERSISTENT && !pers_ok) || (kernel == NVFP4_KERNEL_SPLIT && !split_ok) ||
        (kernel == NVFP4_KERNEL_TILE && !tile_ok))
        return NVFP4_ERR_TILE;

    if (kernel == NVFP4_KERNEL_PERSISTENT) {
        const int64_t tiles = (n + tile.cols - 1) / tile.cols;
        const int per_cu = std::max(1, std::min(64 / tile.waves, int(kMaxLdsBytes / (pers_bytes + 256))));
        const int64_t grid_p = tiles < int64_t(per_cu) * cus ? tiles : int64_t(per_cu) * cus;
        const dim3 grid(static_cast<unsigned>(grid_p), count), block(static_cast<unsigned>(kWave * tile.waves));
        if (describe) {
            *describe = kernel_text("nvfp4_skinny_persistent", {pc, mt, pnb}, y_dtype, grid, block, pers_bytes);
            return NVFP4_OK;
        }
        hipLaunchKernelGGL(pick_persistent(mt, pc, pnb, yd), grid, block, pers_bytes, hs, a);
    } else if (kernel == NVFP4_KERNEL_SPLIT) {
        SplitArgs sa;
        sa.a = a;
        sa.work = reinterpret_cast<uint64_t*>(ws->sums);
        sa.gens = ws->gens;
        sa.region = static_cast<int>(plan.region);
        sa.status = ws->status;
        sa.split = tile.split;
        sa.parts = plan.parts;
        sa.spin_limit = g_test_split_timeout ? kTestSpinLimit : kSpinLimit;
        sa.test_mode = g_test_split_timeout;
        sa.groups = static_cast<int>(plan.groups);
        const dim3 grid(static_cast<unsigned>(plan.groups * plan.parts), count),
            block(static_cast<unsigned>(kWave * plan.w));
        if (describe) {
            *describe = kernel_text("nvfp4_skinny_split", {plan.c, mt, plan.w}, y_dtype, grid, block, plan.lds) +
                        " parts=" + std::to_string(plan.parts);
            return NVFP4_OK;
        }
        hipLaunchKernelGGL(pick_split(mt, plan.c, plan.w, yd), grid, block, plan.lds, hs, sa);
    } else if (kernel == NVFP4_KERNEL_TILE) {
        const dim3 grid(static_cast<unsigned>((n + 16 * pc - 1) / (16 * pc)), count),
            block(static_cast<unsigned>(kWave * tile.waves));
        if (describe) {
            *describe = kernel_text("nvfp4_skinny_tile", {pc, mt, tnb}, y_dtype, grid, block, tile_bytes);
            return NVFP4_OK;
        }
        hipLaunchKernelGGL(pick_tile(mt, pc, tnb, yd), grid, block, tile_bytes, hs, a);
    } else {
        // The generic per-tile kernel (register loads, any shape); x goes
        // through LDS when it fits in 64 KB.  pick_kernel caps the pipeline
        // depth where a deeper one would spill (generic_unroll).
        const bool xlds = x_bytes <= size_t(64 * 1024);
        const size_t part_bytes = tile.waves > 1 ? size_t(tile.waves) * c * mt * 4 * kWave * sizeof(float) : 0;
        const size_t lds = xlds && x_bytes > part_bytes ? x_bytes : part_bytes;
        const dim3 grid(static_cast<unsigned>((n + tile.cols - 1) / tile.cols), count);
        const dim3 block(static_cast<unsigned>(kWave * tile.waves));
        if (describe) {
            *describe = kernel_text("nvfp4_skinny", {c, mt, generic_unroll(tile.unroll, c, xlds), xlds ? 1 : 0},
                                    y_dtype, grid, block, lds);
            return NVFP4_OK;
        }
        hipLaunchKernelGGL(pick_kernel(mt, tile.cols, tile.unroll, xlds, yd), grid, block, lds, hs, a);
    }
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
                  nvfp4::tile_for(n, k), NVFP4_KERNEL_AUTO, false);
}

extern "C" int nvfp4_linear_noalloc(const void* x_bf16, const uint8_t* w_packed, const uint8_t* scales_e4m3,
                                    float tensor_scale, void* y, int64_t m, int64_t n, int64_t k, int y_dtype,
                                    void* stream) {
    int st = nvfp4_linear_shape_ok(m, n, k);
    if (st != NVFP4_OK) return st;
    if (nvfp4::load_tile_override() != NVFP4_OK) return NVFP4_ERR_TILEFILE;
    return launch(x_bf16, w_packed, scales_e4m3, tensor_scale, y, m, n, k, y_dtype, stream,
                  nvfp4::tile_for(n, k), NVFP4_KERNEL_AUTO, true);
}

namespace nvfp4 {

int launch_multi(const void* x, const uint8_t* wp, const uint8_t* sc, float t, void* y, int64_t m, int64_t n,
                 int64_t k, int y_dtype, void* stream, const MultiLaunch& ml) {
    if (load_tile_override() != NVFP4_OK) return NVFP4_ERR_TILEFILE;
    return launch(x, wp, sc, t, y, m, n, k, y_dtype, stream, tile_for(n, k), NVFP4_KERNEL_AUTO, false, nullptr,
                  &ml);
}

}  // namespace nvfp4

extern "C" int nvfp4_launch_info(int64_t m, int64_t n, int64_t k, int y_dtype, char* buf, int64_t buflen) {
    if (!buf) return NVFP4_ERR_NULL;
    int st = nvfp4_linear_shape_ok(m, n, k);
    if (st != NVFP4_OK) return st;
    if (nvfp4::load_tile_override() != NVFP4_OK) return NVFP4_ERR_TILEFILE;
    std::string s;
    st = launch(nullptr, nullptr, nullptr, 1.0f, nullptr, m, n, k, y_dtype, nullptr, nvfp4::tile_for(n, k),
                NVFP4_KERNEL_AUTO, false, &s);
    if (st != NVFP4_OK) return st;
    if ((int64_t)s.size() + 1 > buflen) return NVFP4_ERR_BUFFER;
    std::memcpy(buf, s.c_str(), s.size() + 1);
    return NVFP4_OK;
}

extern "C" int nvfp4_linear_tiled(const void* x_bf16, const uint8_t* w_packed, const uint8_t* scales_e4m3,
                                  float tensor_scale, void* y, int64_t m, int64_t n, int64_t k, int y_dtype,
                                  const nvfp4_tile_t* t, void* stream) {
    int st = nvfp4_linear_shape_ok(m, n, k);
    if (st != NVFP4_OK) return st;
    if (!t) return NVFP4_ERR_NULL;
    nvfp4::Tile tile;
    tile.cols = t->cols;
    tile.waves = t->waves;
    tile.unroll = t->unroll;
    tile.split = t->split;
    tile.mwaves = t->mwaves;
    if (!nvfp4::tile_valid(tile, n, k)) return NVFP4_ERR_TILE;
    if (t->kernel < NVFP4_KERNEL_AUTO || t->kernel > NVFP4_KERNEL_WHOLE) return NVFP4_ERR_TILE;
    return launch(x_bf16, w_packed, scales_e4m3, tensor_scale, y, m, n, k, y_dtype, stream, tile, t->kernel,
                  false);
}
