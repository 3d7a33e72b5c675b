// Host-side set-up shared by the kernel files of the library.
#pragma once

#include <cstddef>
#include <cstdint>

#include "nvfp4_w4a16.h"

namespace nvfp4 {

// Process-wide and current-device set-up (tile override, kernel attributes);
// allocates nothing.  Returns an NVFP4_* status.
int device_setup();

// Kernel attributes of the many-row GEMM kernels (their LDS beyond 64 KB).
int gemm_setup();

// Kernel attributes of the FP8 (W8A16) kernels.
int w8a16_setup();

// The current device's CU count (after device_setup; 256 if unknown).
int device_cus();

// nvfp4_init's set-up (allocating the device workspace once per device), then
// the current device's buffer for the many-row GEMM's per-group partial sums
// (*part = NULL and *bytes = 0 when it could not be allocated) and its CU count.
int gemm_partials(float** part, size_t* bytes, int* cus);

// y[i] = t * (((part[0][i] + part[1][i]) + part[2][i]) + ...), i < mn, rounded
// once to y_dtype: the group sums of a K-split product added in group order.
// With group > 1 the parts are segment chains, `group` consecutive ones
// forming a group: each group is summed in order first, then the group sums
// (the tile's two-level order).  SHAPE if group does not divide parts.
int launch_ordered_sum(const float* part, int parts, int64_t mn, float t, void* y, int y_dtype, void* stream,
                       int group = 1);

// The many-row kernel on FP8 block-scaled weights (W8A16, at most 32 rows):
// K in `waves` segments, `group` of them per segment group (the FP8 tile),
// wg_waves (2, 4 or 6) wavefronts of 16 columns per workgroup, the segment
// groups meeting through nvfp4_init's workspace, or with `whole` all in one
// workgroup.  *launched is false, and nothing was launched, where it cannot
// run (segments not whole 512-k windows, LDS, no workspace).
int launch_fp8_split(const void* x, const uint8_t* w, const float* s, void* y, int64_t m, int64_t n, int64_t k,
                     int y_dtype, int waves, int group, int wg_waves, bool whole, void* stream, bool* launched);

// Several products of one (N, K) in one launch of the skinny kernels
// (blockIdx.y picks one: a table row, a second weight over the same x, or a
// slice of rows of one product) and the de-interleaved store.
struct MultiLaunch {
    const nvfp4_group_t* table = nullptr;   // device table of `count` products, or NULL
    int count = 1;                          // products in the launch
    const uint8_t* wp1 = nullptr;           // without a table: product 1's weight over the same x
    const uint8_t* sc1 = nullptr;
    void* y1 = nullptr;
    float t1 = 0.0f;
    int omap_parts = 0;                     // de-interleaving parts per group (0: none)
    int omap_width[4] = {0, 0, 0, 0};
    int omap_gwidth = 0;
    int omap_ngroups = 0;
    int slice_rows = 0;                     // row slices of one product: count slices of x and y
    int rows_total = 0;                     // rows of that product (m is then the slice's rows)
    const void* up = nullptr;               // the silu input: x is the gate, this the up activation
};

// launch_multi's answer when a silu-input launch cannot run in one kernel
// (its form would not be the per-tile kernel, or that kernel's LDS would not
// hold the up slice too); nothing was launched.
constexpr int kNotFused = 1;

// nvfp4_linear's dispatch and kernels for such a launch; m bounds every
// product's rows.  Arguments are validated as nvfp4_linear does, except the
// pointers inside a table.
int launch_multi(const void* x, const uint8_t* wp, const uint8_t* sc, float t, void* y, int64_t m, int64_t n,
                 int64_t k, int y_dtype, void* stream, const MultiLaunch& ml);

}  // namespace nvfp4
