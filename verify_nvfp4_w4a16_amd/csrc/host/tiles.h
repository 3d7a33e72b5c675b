// Launch tiles of the NVFP4 skinny product, keyed by the weight shape (N, K).
//
// "10 Kernels", section 10.1: every tile table is keyed by the weight's shape,
// never by the row count, so the reduction over K runs in the same order at 1
// row and at 32; section 10.2 keeps a per-shape table of launch settings that
// a sweep picked.  Here a tile fixes, for one (N, K):
//   cols  - weight rows (output columns) one wavefront owns: 16, 32 or 64;
//   waves - wavefronts of one workgroup, each taking an equal, contiguous
//           share (slice) of K; their partial sums are added in slice order;
//   unroll - 128-k blocks a wavefront loads per step of its software
//           pipeline (1, 2 or 4);
//   split  - groups of consecutive segments (1, 2, 4 or 8, dividing waves):
//           an output is the sum, in group order, of its group sums, each
//           the sum of the group's segment chains in segment order;
//   mwaves - wavefronts per workgroup of the many-row kernel (4, 6 or 8, or 0:
//           chosen by the row count), which runs one segment group per
//           workgroup.
// Only `waves` and `split` enter the arithmetic of an output (how K is cut
// and in which order the pieces are added); `cols`, `unroll` and `mwaves`
// change the launch, never the bits.  The tile is a function of (N, K) only.
#pragma once
#include <cstdint>
#include <string>

namespace nvfp4 {

struct Tile {
    int cols = 16;   // 16 * C, C in {1, 2, 4}
    int waves = 8;   // K segments (wavefronts per workgroup of the one-group kernels), 1..8
    int unroll = 2;  // 128-k blocks per pipeline step: 1, 2 or 4
    int split = 1;   // segment groups: 1, 2, 4 or 8, dividing waves
    int mwaves = 0;  // wavefronts per workgroup of the many-row kernel: 4, 6, 8 or 0 (by row count)
};

// Checks a tile against a shape: cols in {16, 32, 64}; waves in 1..8;
// unroll in {1, 2, 4}; each segment K / waves a whole number of unroll * 128 k;
// split in {1, 2, 4, 8} dividing waves; mwaves in {0, 4, 6, 8}.
bool tile_valid(const Tile& t, int64_t n, int64_t k);

// Segment groups the default rule picks for N output columns: enough
// workgroups of 128 columns x one group each for every one of 256 CUs, at
// most `waves` groups.
int default_split(int64_t n, int waves);

// The tile for (N, K): the override table if one was loaded, else the built-in
// table, else the default rule.  Never depends on M.
Tile tile_for(int64_t n, int64_t k);

// Loads, once per process, the override table from the file named by the
// environment variable NVFP4_TILES (if set), so the table is constant for the
// life of the process.  Lines: "N K cols waves unroll [split [mwaves]]"; '#'
// starts a comment; a missing split is 1 and a missing mwaves 0.
// Returns NVFP4_OK or NVFP4_ERR_TILEFILE (the same status on every call).
int load_tile_override();

std::string tile_text(int64_t n, int64_t k, const Tile& t);

}  // namespace nvfp4
