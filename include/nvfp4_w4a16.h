/*
 * nvfp4_w4a16.h - C ABI of the NVFP4 weight-only (W4A16) skinny product for
 * AMD Instinct MI355X (gfx950).
 *
 *   y[m, n] = sum_k x[m, k] * Wd[n, k],   0 <= m < M <= 32
 *   Wd[n, k] = tensor_scale * e4m3(scales[n, k / 16]) * e2m1(q[n, k])
 *
 * The operation is the one "Module ops" (metrale_model_layers::layers::ops)
 * lists as w4a16_gemm / w4a16_gemv / w4a16_tc_rows: C = A @ dequant(B) with A
 * bf16 [M, K] and B an NVFP4 weight stored row-major as packed e2m1 nibbles
 * [N, K/2] (low nibble = even k, per nvfp4_mmq_repack), one e4m3 scale per 16
 * consecutive k [N, K/16], and one fp32 per-tensor scale that multiplies the
 * dequantised weight (dequant_nvfp4_to_bf16).  Row counts 1..32 are the decode
 * and verify regime of "10 Kernels", section 10.2.
 *
 * Conventions ("CUDA Kernel Engineering", conventions and anti-patterns):
 *  - every function returns an int status: NVFP4_OK (0) or a negative
 *    NVFP4_ERR_* code; nvfp4_strerror() names it;
 *  - arguments are validated before any HIP call; on error nothing is launched
 *    and no output is written (as DENSE_GEMM_M16_BF16_MAX_M in "Module ops"
 *    prefers an error to a stale output);
 *  - the launch path allocates nothing and never synchronises the device, so
 *    nvfp4_linear can be captured into a HIP graph once nvfp4_init() has run;
 *  - no read-modify-write atomics: a row's output bits do not depend on M or
 *    on the other rows ("10 Kernels", section 10.1).
 */
#ifndef NVFP4_W4A16_H
#define NVFP4_W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Output element type of nvfp4_linear. */
enum {
    NVFP4_OUT_BF16 = 0, /* y is bf16, one round-to-nearest-even of the fp32 result */
    NVFP4_OUT_F32 = 1   /* y is fp32 (e.g. output-head logits, "10 Kernels" 10.5) */
};

/* Status codes. */
enum {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = -1,      /* a required pointer is NULL */
    NVFP4_ERR_SHAPE = -2,     /* M, N or K outside the contract */
    NVFP4_ERR_ALIGN = -3,     /* a pointer is not aligned as documented */
    NVFP4_ERR_DTYPE = -4,     /* y_dtype is not an NVFP4_OUT_* value */
    NVFP4_ERR_NONFINITE = -5, /* nvfp4_pack: a weight is NaN or infinite */
    NVFP4_ERR_BADSCALE = -6,  /* nvfp4_check_scales: a negative or NaN scale byte */
    NVFP4_ERR_HIP = -7,       /* a HIP runtime call failed */
    NVFP4_ERR_DEVICE = -8,    /* the current device is not gfx950 */
    NVFP4_ERR_TILEFILE = -9,  /* the NVFP4_TILES override file is unreadable or invalid */
    NVFP4_ERR_BUFFER = -10,   /* nvfp4_tile_info: the text buffer is too small */
    NVFP4_ERR_TILE = -11,     /* nvfp4_linear_tiled: the tile does not fit the shape */
    NVFP4_ERR_SCRATCH = -12,  /* nvfp4_linear_noalloc: the call needs more than the fixed scratch */
    NVFP4_ERR_LIBRARY = -13   /* nvfp4_gemm_library: the GEMM library reported an error */
};

/* Largest row count of one nvfp4_linear call. */
#define NVFP4_MAX_M 32
/* K must be a positive multiple of this (whole 16-byte scale loads per lane). */
#define NVFP4_K_MULTIPLE 256

/*
 * Host.  Quantise a row-major fp32 matrix w[N, K] into NVFP4, writing into
 * caller-owned host buffers:
 *   w_packed[N * K / 2]  byte j of row n holds k = 2j (low nibble) and 2j + 1;
 *   scales_e4m3[N * K / 16]  byte g of row n scales k in [16g, 16g + 16);
 *   *tensor_scale  fp32 per-tensor scale.
 * Rule (IEEE binary64, in this order): t = fp32(max|w| / (6 * 448)), or 1 when
 * that is 0; per group u = (max|w_group| / 6) / t rounded to the nearest e4m3
 * (ties to even, saturating at 448); e2m1 code of w / (e4m3(s) * t) rounded to
 * nearest (ties to even, saturating at 6), all-zero codes when the group scale
 * is 0.  The group scale is absmax / 6, as "Module ops" quantize_bf16_to_nvfp4
 * stores one e4m3 scale per 16 elements; 448 is E4M3_MAX of the same page.
 * Deterministic and independent of the number of threads used.
 * Errors: NULL; SHAPE (N < 1, K < 16 or K % 16 != 0); NONFINITE.
 */
int nvfp4_pack(const float* w, int64_t n, int64_t k, uint8_t* w_packed,
               uint8_t* scales_e4m3, float* tensor_scale);

/*
 * Host, pure.  NVFP4_ERR_BADSCALE if any of the N * K / 16 scale bytes is
 * negative (sign bit set) or NaN (0x7F, 0xFF); NVFP4_OK otherwise.  This is the
 * "bad" flag of "Module ops" nvfp4_tc_lean_repack; nvfp4_linear does not check
 * scales per call (it would cost bandwidth) and decodes them literally.
 * Errors: NULL; SHAPE (N < 1, K < 16 or K % 16 != 0).
 */
int nvfp4_check_scales(const uint8_t* scales_e4m3, int64_t n, int64_t k);

/*
 * Host, pure.  The shape contract of nvfp4_linear, testable without a GPU
 * (like "Module ops" w4a16_tc_rows_shape_ok): 0 <= M <= 32, 1 <= N <= 2^28,
 * 256 <= K <= 2^20 with K % 256 == 0.  Returns NVFP4_OK or NVFP4_ERR_SHAPE.
 */
int nvfp4_linear_shape_ok(int64_t m, int64_t n, int64_t k);

/*
 * Host.  Set-up before graph capture: "CUDA Kernel Engineering" (CUDA graphs)
 * captures every launch once at start-up and needs fixed buffer addresses and
 * no allocation in the replayed loop; "10 Kernels" 10.6 replays every verify
 * from graphs.  This call does every allocation and code-object load the
 * launches need, so nothing of the kind happens under capture.
 * Checks that the current HIP device is gfx950, loads the kernels'
 * code objects and the (N, K) tile table once per process (the table may be
 * overridden by the file named in the environment variable NVFP4_TILES, read
 * here only), and sets up the current device's workspace once per device: 32
 * MiB of tagged partial sums plus 16 KiB of generation words in device
 * memory, zeroed once and kept until the process ends (the many-row
 * kernel exchanges segment-group sums through it; generations only advance,
 * so it is never cleared again), and a 64 MiB buffer, written in full before
 * it is read by every call that uses it: the group sums of a K-split
 * nvfp4_gemm or fp8_w8a16_linear, the activation of nvfp4_linear_silu_input.
 * Call on every device before capturing any of this library's device calls
 * into a HIP graph; the first call on a device that needs the workspace runs
 * it otherwise.  Safe to call more than once.  If the workspace cannot be
 * allocated, nvfp4_linear, nvfp4_gemm and fp8_w8a16_linear still work (with
 * kernels that do not need it) and give the same bits; the silu input then
 * fails with HIP.
 * Test hook, read once per process: NVFP4_TEST_SPLIT_TIMEOUT=1 makes the
 * many-row kernel's producer workgroups store no partial sums, =2 makes them
 * store them only after a long bounded delay; with either, its consumers give
 * up after a few polls, so tests can check the time-out path.
 * Errors: HIP, DEVICE, TILEFILE.
 */
int nvfp4_init(void);

/*
 * Device, asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *   y[M, N] = x[M, K] . Wd[N, K]^T with Wd as at the top of this file: the
 * product of "Module ops" w4a16_gemm / w4a16_tc_rows (C = A @ dequant(B)) at
 * the 1..32-row decode and verify counts of "10 Kernels" 10.2, with the row
 * invariance of 10.1.
 * x:           device, bf16 [M, K] row-major (pitch K elements), 16-byte aligned.
 * w_packed:    device, [N, K/2] bytes, 16-byte aligned.
 * scales_e4m3: device, [N, K/16] bytes, 16-byte aligned.
 * tensor_scale: fp32 value; applied once to the fp32 sum, then one rounding.
 * y:           device, [M, N] row-major (pitch N), bf16 (2-byte aligned) or
 *              fp32 (4-byte aligned) by y_dtype.  Must not overlap the inputs.
 * All buffers belong to the caller and must stay alive until the stream has
 * passed this call.  M == 0 returns NVFP4_OK and launches nothing.  Rows
 * r < M of y are written in full; nothing else is written.  The reduction over
 * K runs in an order fixed by (N, K) alone (see nvfp4_tile_t), so a row's bits
 * are the same for every M and every position of the row in x.  No
 * allocation, no host sync.
 * Shapes whose tile has split > 1 run, for M >= 2, through the device
 * workspace set up by nvfp4_init: such calls on one device must not overlap in
 * time (calls on one stream, or on streams ordered by events, never do).  A
 * workgroup that waits for another's partial sums gives up after about a
 * second, writes NaN to its outputs instead of hanging and sets the device's
 * time-out word (nvfp4_timeout_status).
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP, DEVICE, TILEFILE.
 */
int nvfp4_linear(const void* x_bf16, const uint8_t* w_packed,
                 const uint8_t* scales_e4m3, float tensor_scale, void* y,
                 int64_t m, int64_t n, int64_t k, int y_dtype, void* stream);

/*
 * Host, synchronous (waits for the current device to finish its work).  For
 * callers that need to know whether an exchange of partial sums gave up (see
 * nvfp4_linear): *timed_out = 1 if a many-row workgroup on the current device
 * gave up waiting since the last call, else 0; the word is then cleared.
 * "10 Kernels" 10.7 checks results before timing them; this is the check the
 * bounded wait leaves to the host.  Errors: NULL, HIP, DEVICE, TILEFILE.
 */
int nvfp4_timeout_status(int* timed_out);

/*
 * Device, asynchronous: nvfp4_linear for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results (bits) and errors as
 * nvfp4_linear, plus SCRATCH.  It never allocates: neither this call nor its
 * set-up calls hipMalloc, hipFree or any allocating routine.  Where
 * nvfp4_linear exchanges partial sums through the workspace nvfp4_init
 * allocates, this call uses a fixed scratch array built into the library
 * instead: 8 MiB of tagged sums plus 4 KiB of generation words per device,
 * held by each device the library runs on until the process ends.  A call
 * whose exchange needs more returns NVFP4_ERR_SCRATCH and launches nothing:
 * a column group takes (split - 1) x 2 KiB per 16-row tile, 16-column tile and
 * wavefront of its workgroups, e.g. 224 KiB for 128 columns at 17..32 rows and
 * split 8, so N up to 4608 fits there; every product of the 48-layer decode
 * round fits.  Every call on a device shares that device's array, which keeps the last call's contents (no
 * clearing is needed: generations only advance); calls on one device that
 * overlap in time race on it, as calls of nvfp4_linear do on the workspace.
 * The first call on a device does the device's set-up (kernel attributes, the
 * array's device address) unless nvfp4_init has done it.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP, DEVICE, TILEFILE, SCRATCH.
 */
int nvfp4_linear_noalloc(const void* x_bf16, const uint8_t* w_packed,
                         const uint8_t* scales_e4m3, float tensor_scale, void* y,
                         int64_t m, int64_t n, int64_t k, int y_dtype, void* stream);

/* Kernel choice of nvfp4_linear_tiled (nvfp4_linear always chooses itself).
 * Every kernel computes the same bits for the same tile waves and split. */
enum {
    NVFP4_KERNEL_AUTO = 0,       /* as nvfp4_linear: by M, the shape, the LDS fit and the workspace */
    NVFP4_KERNEL_PERSISTENT = 1, /* workgroups walk the column tiles with x [M, K] whole in LDS; needs
                                    K / waves % 512 == 0, M * (K + 8) * 2 <= 64 KB, cols <= 32 */
    NVFP4_KERNEL_TILE = 2,       /* one workgroup per column tile, each wavefront streaming its K segment
                                    through LDS; needs K / waves % 512 == 0, cols <= 32 and M small enough
                                    for the wavefronts' x slices to fit the LDS */
    NVFP4_KERNEL_SPLIT = 3,      /* many-row kernel: one segment group per workgroup, x windows in LDS;
                                    needs K / waves % 512 == 0 and, for split > 1, the device workspace */
    NVFP4_KERNEL_GENERIC = 4,    /* one workgroup per column tile, register loads; any shape */
    NVFP4_KERNEL_WHOLE = 5       /* many-row kernel with every segment group of a column group in one
                                    workgroup (two-level sum inside it, no workspace); needs
                                    K / waves % 512 == 0 */
};

/*
 * Launch tile ("10 Kernels", section 10.2: the per-shape tables hold the
 * launch settings a sweep picked).  The K reduction of every output is: K cut
 * into `waves` equal segments, each summed as one chain of MFMAs in increasing
 * k; the segments cut into `split` groups of consecutive segments; a group's
 * sum adds its chains in segment order, and the output adds the group sums in
 * group order.  Only waves and split change result bits.
 */
typedef struct nvfp4_tile {
    int cols;   /* output columns per wavefront: 16, 32 or 64 */
    int waves;  /* K segments, 1..8 (wavefronts per workgroup of the one-group kernels) */
    int unroll; /* 128-k blocks per pipeline step: 1, 2 or 4; K % (128 * unroll * waves) == 0 */
    int split;  /* segment groups: 1, 2, 4 or 8, dividing waves */
    int mwaves; /* wavefronts per workgroup of the many-row kernel: 4, 6 or 8; 0 = by M (4 up to 16 rows) */
    int kernel; /* NVFP4_KERNEL_*; ignored by the (N, K) table */
} nvfp4_tile_t;

/*
 * Device, asynchronous: nvfp4_linear with an explicit launch tile and kernel
 * instead of the (N, K) table's, for tile sweeps and for tests that every
 * kernel gives the same bits for the same waves and split.  "10 Kernels" 10.1
 * keeps only tile choices bit-identical to the default at 1 to 32 rows and
 * 10.2 fills the per-shape tables from such sweeps.  `tile` is a host
 * pointer read during the call only.
 * Errors: those of nvfp4_linear, NULL for tile == NULL, and TILE for a tile
 * that does not fit the shape or a kernel that cannot run it.
 */
int nvfp4_linear_tiled(const void* x_bf16, const uint8_t* w_packed,
                       const uint8_t* scales_e4m3, float tensor_scale, void* y,
                       int64_t m, int64_t n, int64_t k, int y_dtype,
                       const nvfp4_tile_t* tile, void* stream);

/*
 * Host.  Writes a one-line text description of the tile nvfp4_linear uses for
 * an (N, K) weight into buf (NUL-terminated): the table entry, the K split and
 * the grid.  The tile is the per-shape table entry of "10 Kernels" 10.2 (launch
 * settings a sweep picked, one per weight shape), keyed by (N, K) and never by
 * the row count as 10.1 requires; tests read it to launch every kernel with
 * the same K order.  Errors: NULL, SHAPE, BUFFER, TILEFILE.
 */
int nvfp4_tile_info(int64_t n, int64_t k, char* buf, int64_t buflen);

/*
 * Device, asynchronous.  Two products over one x in one launch, like
 * "Module ops" w4a16_gemv_dual (and its 2- and 3-row forms): y0 = x . W0^T and
 * y1 = x . W1^T, both weights [N, K] (each with its scales and tensor scale),
 * both outputs [M, N].  Shape contract, layouts and alignment of
 * nvfp4_linear; every output has the bits nvfp4_linear gives it.  It runs
 * nvfp4_linear's kernels with the weight picked per workgroup, so like
 * nvfp4_linear it may use the device workspace (same rule on overlap).
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP, DEVICE, TILEFILE.
 */
int nvfp4_linear_dual(const void* x_bf16, const uint8_t* w_packed0, const uint8_t* scales0,
                      float tensor_scale0, void* y0, const uint8_t* w_packed1, const uint8_t* scales1,
                      float tensor_scale1, void* y1, int64_t m, int64_t n, int64_t k, int y_dtype,
                      void* stream);

/*
 * Device, asynchronous.  "Module ops" w4a16_gemv_silu_input: the product's
 * activation is silu(gate) * up, formed per element from the bf16 gate
 * [M, K] and up [M, K] (16-byte aligned): silu(g) = g / (1 + exp(-g)) and
 * the product with u in fp32, rounded once to bf16, then the product of
 * nvfp4_linear with that x (same bits as nvfp4_linear on it).  At M = 1,
 * where the product runs on the per-tile kernel, one launch: each wavefront
 * forms the activation of its K slice in LDS.  Otherwise two launches: a
 * small kernel writes the activation (M * K * 2 bytes) to the device buffer
 * nvfp4_init allocates, then nvfp4_linear runs on it; calls that use the
 * device workspace must not overlap in time on one device.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP (also: the device buffer could not
 * be allocated), DEVICE, TILEFILE.
 */
int nvfp4_linear_silu_input(const void* gate_bf16, const void* up_bf16, const uint8_t* w_packed,
                            const uint8_t* scales_e4m3, float tensor_scale, void* y, int64_t m,
                            int64_t n, int64_t k, int y_dtype, void* stream);

/*
 * Device, asynchronous.  "Module ops" w4a16_gemv_qg / w4a16_gemv_qkvz: the
 * weight's rows interleave `parts` parts per group (Q and gate per head; Q,
 * K, V and Z per group), widths[p] rows of part p in each group of
 * G = sum(widths) rows, N = groups * G; the output is stored de-interleaved,
 * all groups' part 0, then all groups' part 1, ...: row r of part p of group
 * g lands in column groups * (widths[0] + .. + widths[p-1]) + g * widths[p] + r.
 * widths: host array of `parts` (1..4) positive counts, read during the call.
 * Values and bits are nvfp4_linear's, only the columns move (nvfp4_linear's
 * kernels with the map on the store; same workspace rule).
 * Errors: NULL, SHAPE (also N not a multiple of G), ALIGN, DTYPE, HIP, DEVICE,
 * TILEFILE.
 */
int nvfp4_linear_deinterleave(const void* x_bf16, const uint8_t* w_packed,
                              const uint8_t* scales_e4m3, float tensor_scale, void* y, int64_t m,
                              int64_t n, int64_t k, int y_dtype, int parts, const int* widths,
                              void* stream);

/* One product of a grouped launch (nvfp4_linear_grouped): device pointers
 * with nvfp4_linear's layouts and alignment; m rows (0 skips the entry). */
typedef struct nvfp4_group {
    const void* x;                 /* bf16 [m, K] */
    const uint8_t* w_packed;       /* [N, K/2] */
    const uint8_t* scales_e4m3;    /* [N, K/16] */
    void* y;                       /* [m, N], bf16 or fp32 by the launch's y_dtype */
    float tensor_scale;
    int32_t m;                     /* 0 <= m <= max_m */
} nvfp4_group_t;

/*
 * Device, asynchronous.  "Module ops" moe_w4a16_grouped_gemm_ptrtable: one
 * launch over `count` products with the same N and K (e.g. the experts of a
 * MoE layer, each with the rows routed to it), read from `table`, a device
 * array of count nvfp4_group_t (8-byte aligned) that must stay valid until the
 * stream passes the call.  max_m (0..32) bounds every entry's m; rows of an
 * entry past max_m are not computed.  Each output has the bits nvfp4_linear
 * gives it: nvfp4_linear's kernels, sized for max_m, run with the entry
 * picked per workgroup (same workspace rule; where the many-row kernel's
 * exchange for every entry would not fit the workspace, another kernel of
 * the same tile runs).  Entry pointers are not checked
 * on the host (they are in device memory): they must satisfy nvfp4_linear's
 * contract.
 * Errors: NULL, SHAPE (also count > 65535), ALIGN, DTYPE, HIP, DEVICE, TILEFILE.
 */
int nvfp4_linear_grouped(const nvfp4_group_t* table, int64_t count, int64_t max_m, int64_t n,
                         int64_t k, int y_dtype, void* stream);

/*
 * FP8 block-scaled weights (W8A16), the pages' second weight format ("10
 * Kernels" 10.3; "Module ops" w8a16_gemm / w8a16_tc_rows): a weight [N, K] of
 * e4m3 codes (OCP "fn": bias 7, max 448, NaN = 0x7F/0xFF) and one fp32 scale
 * per 128 x 128 block, [N/128, K/128] row-major:
 *   y[m, n] = sum over 128-k blocks b of S[n/128, b] * sum_{k in b} x[m, k] * e4m3(W[n, k]).
 */

/*
 * Host.  Quantise a row-major fp32 w[N, K] (N, K multiples of 128) into e4m3
 * codes w_e4m3[N * K] and block scales block_scales[(N/128) * (K/128)], host
 * buffers owned by the caller.  Rule (IEEE binary64, in this order): per block
 * S = fp32(max|w| / 448), 1 when that is 0; code = e4m3 of w / S rounded to
 * nearest, ties to even, saturating at 448, sign kept except for a zero code.
 * The layout is the one "10 Kernels" 10.3 reads as stored (and 448 is
 * "Module ops" E4M3_MAX); the pages' checkpoints come quantised, so the rule
 * for choosing S is this library's reading.  Errors: NULL, SHAPE, NONFINITE.
 */
int fp8_w8a16_pack(const float* w, int64_t n, int64_t k, uint8_t* w_e4m3, float* block_scales);

/*
 * Host, pure.  The shape contract of fp8_w8a16_linear, like "Module ops"
 * w8a16_tc_rows_shape_ok: 0 <= M <= 32, N and K positive multiples of 128,
 * N <= 2^28, K <= 2^20.  Returns NVFP4_OK or NVFP4_ERR_SHAPE.
 */
int fp8_w8a16_shape_ok(int64_t m, int64_t n, int64_t k);

/*
 * Device, asynchronous on `stream`.  The W8A16 product above at 1..32 rows:
 * x bf16 [M, K] (16-byte aligned), w_e4m3 [N, K] (16-byte aligned),
 * block_scales fp32 [N/128, K/128] (4-byte aligned), y [M, N] bf16 or fp32,
 * all device memory owned by the caller.  Each 128-k block's partial sum
 * starts from zero and joins the row's chain as one fused multiply-add by its
 * scale, blocks in increasing k; K is cut into segments (a function of N and
 * K) added in a fixed order, so a row's bits do not depend on M ("10 Kernels"
 * 10.1).  M == 0 launches nothing; no host sync.  Where x [M, K] does not
 * fit 64 KB of LDS and K's segments are whole 512-k windows, the many-row
 * kernel runs it (the same bits): x in windows shared by a workgroup's
 * columns; where fewer than one workgroup per CU would hold every segment
 * group, the groups run in separate workgroups and meet through nvfp4_init's
 * workspace (tagged sums, as nvfp4_linear's many-row kernel; a consumer that
 * gives up writes NaN and sets the word nvfp4_timeout_status reads).
 * Otherwise, at 17..32 rows on weights with fewer than 32 columns per CU, the
 * segment groups run in separate workgroups and a second kernel adds their
 * sums in order, through the device buffer nvfp4_init allocates.  The first
 * call on a device that needs the workspace runs nvfp4_init's set-up: calls
 * that use it must not overlap in time on one device.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP, DEVICE, TILEFILE.
 */
int fp8_w8a16_linear(const void* x_bf16, const uint8_t* w_e4m3, const float* block_scales, void* y,
                     int64_t m, int64_t n, int64_t k, int y_dtype, void* stream);

/*
 * Host, pure.  The shape contract of fp8_w8a16_gemm and fp8_w8a16_matmul:
 * 0 <= M <= 65535 * 128, N and K positive multiples of 128, N <= 2^28,
 * K <= 2^20, M * N <= 2^40 ("Module ops" w8a16_tc_rows_shape_ok checks a
 * kernel's contract likewise).  Returns NVFP4_OK or NVFP4_ERR_SHAPE.
 */
int fp8_w8a16_gemm_shape_ok(int64_t m, int64_t n, int64_t k);

/*
 * Device, asynchronous on `stream`.  fp8_w8a16_linear's product for any row
 * count, the prefill forms of the FP8 family ("Module ops" w8a16_gemm,
 * w8a16_gemm_n128_m128 and the pipelined forms; "10 Kernels" 10.3 for the
 * format): same arguments, layouts and alignment, shape contract
 * fp8_w8a16_gemm_shape_ok; M == 0 launches nothing.  Same MFMA inputs, block
 * chains and two-level segment order as fp8_w8a16_linear, so each row's bits
 * are those it gives the row at 1..32 rows ("10 Kernels" 10.1).  Workgroups
 * own 128 rows x 128 columns; where that gives workgroups for at most half
 * the CUs and the tile has more than one segment group, the K split goes
 * through the device buffer nvfp4_init allocates (same bits): such calls on
 * one device must not overlap in time.  No allocation (the first call on a
 * device runs nvfp4_init's set-up unless it has run), no host sync.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP, DEVICE.
 */
int fp8_w8a16_gemm(const void* x_bf16, const uint8_t* w_e4m3, const float* block_scales, void* y,
                   int64_t m, int64_t n, int64_t k, int y_dtype, void* stream);

/*
 * Device, asynchronous.  Picks the FP8 kernel by row count ("10 Kernels"
 * 10.2's regimes over the format of 10.3): fp8_w8a16_linear for M <= 32,
 * fp8_w8a16_gemm above; both give every row the same bits.  Shape contract:
 * fp8_w8a16_gemm_shape_ok.  Errors: those of the call it makes.
 */
int fp8_w8a16_matmul(const void* x_bf16, const uint8_t* w_e4m3, const float* block_scales, void* y,
                     int64_t m, int64_t n, int64_t k, int y_dtype, void* stream);

/*
 * Host, pure.  The shape contract of nvfp4_gemm and nvfp4_gemm_expanded:
 * 0 <= M <= 65535 * 128, 1 <= N <= 2^28, 256 <= K <= 2^20 with K % 256 == 0,
 * M * N <= 2^40 ("Module ops" w4a16_tc_rows_shape_ok likewise checks a
 * kernel's contract without a GPU).  Returns NVFP4_OK or NVFP4_ERR_SHAPE.
 */
int nvfp4_gemm_shape_ok(int64_t m, int64_t n, int64_t k);

/*
 * Device, asynchronous on `stream`.  The product of nvfp4_linear for any row
 * count: the regime of "10 Kernels" 10.2 for 33 to about 1,024 rows
 * (prefill chunks), the "Module ops" w4a16_gemm / w4a16_gemm_n128_m128
 * operation C = A @ dequant(B).  Arguments, layouts, alignment and ownership
 * as nvfp4_linear; M == 0 launches nothing.  The K order is the (N, K) tile's
 * (as nvfp4_linear), so each row's bits are those nvfp4_linear gives it, for
 * every M ("10 Kernels" 10.1).  No allocation (the first call on a device
 * runs nvfp4_init's set-up unless it has run), no host sync.  Workgroups own
 * 128 rows x 128 columns; when that gives workgroups for at most half the
 * CUs and the tile has split > 1, each workgroup takes one segment group
 * (one segment where even the groups would leave half the CUs idle) and a
 * second kernel adds the partial sums in the tile's order through the device
 * buffer nvfp4_init allocates (same bits): such calls on one device must not
 * overlap in time (calls on one stream, or on streams ordered by events,
 * never do).
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP, DEVICE, TILEFILE.
 */
int nvfp4_gemm(const void* x_bf16, const uint8_t* w_packed, const uint8_t* scales_e4m3,
               float tensor_scale, void* y, int64_t m, int64_t n, int64_t k, int y_dtype,
               void* stream);

/*
 * Device, asynchronous.  Picks the kernel by row count over one stored
 * format, as "10 Kernels" 10.2's table does: nvfp4_linear for M <= 32,
 * nvfp4_linear's kernels on 32-row slices up to 64 rows (all slices in one
 * launch; the 128-row GEMM tile leaves most CUs idle there), nvfp4_gemm
 * above (row counts measured on MI355X).  All give every row the same bits.
 * Like those calls, calls that use the device workspace must not overlap in
 * time on one device.  Shape contract: nvfp4_gemm's.
 * Errors: those of the calls it makes.
 */
int nvfp4_matmul(const void* x_bf16, const uint8_t* w_packed, const uint8_t* scales_e4m3,
                 float tensor_scale, void* y, int64_t m, int64_t n, int64_t k, int y_dtype,
                 void* stream);

/*
 * Device, asynchronous.  Expands an NVFP4 weight to bf16 w_bf16[N, K]
 * (caller-owned, 16-byte aligned, N * K * 2 bytes), like "Module ops"
 * dequant_nvfp4_to_bf16: with apply_tensor_scale = 1 each element is the
 * exact t * e4m3 * e2m1 rounded once to the nearest bf16 (ties to even); with
 * 0 it is e4m3 * e2m1, exact in bf16 (the weight nvfp4_gemm_expanded takes).
 * w_packed: device, [N, K/2], 4-byte aligned; scales_e4m3: device, [N, K/16].
 * Shape: 1 <= N <= 2^28, 16 <= K <= 2^20, K % 16 == 0.
 * Errors: NULL, SHAPE, ALIGN, DTYPE (apply_tensor_scale not 0 or 1), HIP.
 */
int nvfp4_dequant_bf16(const uint8_t* w_packed, const uint8_t* scales_e4m3, float tensor_scale,
                       int apply_tensor_scale, void* w_bf16, int64_t n, int64_t k, void* stream);

/*
 * Device, asynchronous.  The third regime of "10 Kernels" 10.2 (above about
 * 1,024 rows: expand to BF16 once, then a plain GEMM): nvfp4_gemm reading the
 * weight as w_bf16[N, K] = e4m3 * e2m1 (nvfp4_dequant_bf16 with
 * apply_tensor_scale = 0, 16-byte aligned), with tensor_scale applied once to
 * the fp32 sum, so every row's bits equal nvfp4_gemm's.  Other arguments and
 * errors as nvfp4_gemm.
 */
int nvfp4_gemm_expanded(const void* x_bf16, const void* w_bf16, float tensor_scale, void* y,
                        int64_t m, int64_t n, int64_t k, int y_dtype, void* stream);

/*
 * Device, asynchronous on `stream`.  The third regime of "10 Kernels" 10.2 as
 * the pages run it (expand to BF16 once, then the platform's library GEMM):
 * y = t * x @ w_bf16^T through hipBLASLt, bf16 operands, fp32 accumulation,
 * t applied to the fp32 sum, one rounding to y's type.  Arguments, layouts
 * and the shape contract as nvfp4_gemm_expanded (w_bf16 from
 * nvfp4_dequant_bf16 with apply_tensor_scale = 0).  The library picks its own
 * kernel and K order per shape, so the bits are not nvfp4_gemm's and a row
 * may differ in its last bits between row counts (within the same error
 * bound); repeated calls of one shape give the same bits.  The first call on
 * a device creates the library handle and a 32 MiB workspace (hipMalloc), the
 * first call of each (M, N, K, y_dtype) builds its plan (host only); both are
 * kept until the process ends, so make those calls before capturing a graph.
 * Calls on one device that overlap in time share the workspace: keep them on
 * one stream.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP, DEVICE, LIBRARY.
 */
int nvfp4_gemm_library(const void* x_bf16, const void* w_bf16, float tensor_scale, void* y,
                       int64_t m, int64_t n, int64_t k, int y_dtype, void* stream);

/*
 * Device, asynchronous.  All three regimes of "10 Kernels" 10.2's table over
 * one stored format: nvfp4_matmul below expand_min_m rows (1..32 rows
 * skinny, then the many-row kernels; every row nvfp4_linear's bits), and from
 * expand_min_m rows on the third regime: the weight expanded to bf16 into
 * w_bf16_scratch (device, caller-owned, N * K * 2 bytes, 16-byte aligned; its
 * contents are overwritten) by nvfp4_dequant_bf16 without the tensor scale,
 * then nvfp4_gemm_library (those rows carry the library's bits, within the
 * same error bound).  expand_min_m = 0 takes 768: the pages put the boundary
 * at about 1,024 rows; on MI355X expanding per call is ahead from 768 rows on
 * the decode round's four shapes (mixed at 384..512).  The scratch may be
 * NULL when M stays below the threshold.  A caller that keeps the expanded
 * weight calls nvfp4_gemm_library directly.  Shape contract: nvfp4_gemm's.
 * Errors: SHAPE (also a negative expand_min_m), NULL, and those of the calls
 * it makes.
 */
int nvfp4_matmul_expand(const void* x_bf16, const uint8_t* w_packed, const uint8_t* scales_e4m3,
                        float tensor_scale, void* y, int64_t m, int64_t n, int64_t k, int y_dtype,
                        void* w_bf16_scratch, int64_t expand_min_m, void* stream);

/*
 * Host.  Writes into buf (NUL-terminated) the kernel nvfp4_linear launches for
 * an M x N x K product with this output type on the current device, as its
 * template name reads in a kernel trace, then its grid, block and LDS bytes
 * (and, for the many-row kernel, how many workgroups share a column group);
 * "none" for M = 0.  For profiles, which "CUDA Kernel Engineering" (profiling)
 * and "10 Kernels" 10.7 read per kernel.  Runs nvfp4_init's set-up.
 * Errors: NULL, SHAPE, DTYPE, BUFFER, HIP, DEVICE, TILEFILE.
 */
int nvfp4_launch_info(int64_t m, int64_t n, int64_t k, int y_dtype, char* buf, int64_t buflen);

/*
 * Device, asynchronous on `stream`: reads a_bytes at a and b_bytes at b once
 * with 16-byte loads and nothing else (e.g. a product's packed weights and
 * its scales), a plain-read ceiling to time a product kernel against
 * ("10 Kernels" 10.7 times kernels over working sets larger than the caches).
 * a, b: device, 16-byte aligned, sizes multiples of 16 (either may be 0).
 * sink: device, 4 bytes, written only in the unlikely case that the bytes
 * read XOR to one fixed value.  Errors: NULL, SHAPE, ALIGN, HIP.
 */
int nvfp4_read_probe(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes, void* sink,
                     void* stream);

/* Host.  Static text for a status code; never NULL. */
const char* nvfp4_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_W4A16_H */
