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
 *  - no atomics: a row's output bits do not depend on M or on the other rows
 *    ("10 Kernels", section 10.1).
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
    NVFP4_ERR_TILE = -11      /* nvfp4_linear_tiled: the tile does not fit the shape */
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
 * Host.  Checks that the current HIP device is gfx950, loads the kernels'
 * code objects and the (N, K) tile table once per process (the table may be
 * overridden by the file named in the environment variable NVFP4_TILES, read
 * here only).  Call before capturing nvfp4_linear into a HIP graph; the first
 * nvfp4_linear call runs it otherwise.  Safe to call more than once.
 * Errors: HIP, DEVICE, TILEFILE.
 */
int nvfp4_init(void);

/*
 * Device, asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *   y[M, N] = x[M, K] . Wd[N, K]^T with Wd as at the top of this file.
 * x:           device, bf16 [M, K] row-major (pitch K elements), 16-byte aligned.
 * w_packed:    device, [N, K/2] bytes, 16-byte aligned.
 * scales_e4m3: device, [N, K/16] bytes, 16-byte aligned.
 * tensor_scale: fp32 value; applied once to the fp32 sum, then one rounding.
 * y:           device, [M, N] row-major (pitch N), bf16 (2-byte aligned) or
 *              fp32 (4-byte aligned) by y_dtype.  Must not overlap the inputs.
 * All buffers belong to the caller and must stay alive until the stream has
 * passed this call.  M == 0 returns NVFP4_OK and launches nothing.  Rows
 * r < M of y are written in full; nothing else is written.  The reduction over
 * K runs in an order fixed by (N, K) alone, so a row's bits are the same for
 * every M and every position of the row in x.  No allocation, no host sync.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP, DEVICE, TILEFILE.
 */
int nvfp4_linear(const void* x_bf16, const uint8_t* w_packed,
                 const uint8_t* scales_e4m3, float tensor_scale, void* y,
                 int64_t m, int64_t n, int64_t k, int y_dtype, void* stream);

/*
 * Device, asynchronous: nvfp4_linear with an explicit launch tile instead of
 * the (N, K) table's, for tile sweeps ("10 Kernels", section 10.2: the tables
 * hold the launch settings a sweep picked).  cols: output columns per
 * wavefront (16, 32 or 64); waves: wavefronts per workgroup (1..8), each
 * summing one of `waves` equal K segments, added in segment order; unroll:
 * 128-k blocks per pipeline step (1, 2 or 4), with K a multiple of
 * 128 * unroll * waves.  cols and unroll never change the result's bits;
 * waves does (it is the K segmentation).
 * Errors: those of nvfp4_linear, and TILE for a tile that does not fit.
 */
int nvfp4_linear_tiled(const void* x_bf16, const uint8_t* w_packed,
                       const uint8_t* scales_e4m3, float tensor_scale, void* y,
                       int64_t m, int64_t n, int64_t k, int y_dtype, int cols,
                       int waves, int unroll, void* stream);

/*
 * Host.  Writes a one-line text description of the tile nvfp4_linear uses for
 * an (N, K) weight into buf (NUL-terminated): the table entry, the K split and
 * the grid.  Errors: NULL, SHAPE, BUFFER, TILEFILE.
 */
int nvfp4_tile_info(int64_t n, int64_t k, char* buf, int64_t buflen);

/* Host.  Static text for a status code; never NULL. */
const char* nvfp4_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_W4A16_H */
