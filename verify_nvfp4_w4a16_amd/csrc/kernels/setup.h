// Host-side set-up shared by the kernel files of the library.
#pragma once

#include <cstddef>

namespace nvfp4 {

// Process-wide and current-device set-up (tile override, kernel attributes);
// allocates nothing.  Returns an NVFP4_* status.
int device_setup();

// Kernel attributes of the many-row GEMM kernels (their LDS beyond 64 KB).
int gemm_setup();

// Kernel attributes of the fused and grouped kernels.
int fused_setup();

// Kernel attributes of the FP8 (W8A16) kernels.
int w8a16_setup();

// The current device's CU count (after device_setup; 256 if unknown).
int device_cus();

// nvfp4_init's set-up (allocating the device workspace once per device), then
// the current device's buffer for the many-row GEMM's per-group partial sums
// (*part = NULL and *bytes = 0 when it could not be allocated) and its CU count.
int gemm_partials(float** part, size_t* bytes, int* cus);

}  // namespace nvfp4
