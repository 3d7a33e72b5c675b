// Host-side set-up shared by the kernel files of the library.
#pragma once

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

}  // namespace nvfp4
