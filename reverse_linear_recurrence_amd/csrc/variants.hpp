// variants.hpp -- the tiling variants of the scan kernels and the lookup of a
// compiled kernel instance; shared by the host code and the kernel tables.
#pragma once

#include <stdint.h>

namespace rlca {

struct Variant {
  int LPR;  // lanes per row inside a wavefront (64 when WPR > 1)
  int WPR;  // wavefronts per row
};

// Every lane owns K = 4 consecutive steps: one 16-byte vector of each fp32
// array (an 8-byte vector of each bf16 array) and one 16-byte vector of each
// fp32 output, so every load and store instruction of a wavefront covers one
// contiguous span and uses each cache line it touches in full.  (Longer spans
// per lane split each instruction into strided partial lines: 4x the line
// requests for 16 fp32 steps per lane, and partial-line output writes for 8
// bf16 steps per lane.)
constexpr int kStepsPerLane = 4;
constexpr Variant kVariants[] = {
    {16, 1},  // 0: tile    64 steps, 16 rows per 256-thread workgroup
    {32, 1},  // 1: tile   128,  8 rows per workgroup
    {64, 1},  // 2: tile   256,  4 rows per workgroup
    {64, 4},  // 3: tile  1024,  1 row per 256-thread workgroup
    {64, 8},  // 4: tile  2048,  1 row per 512-thread workgroup
    {64, 16}, // 5: tile  4096,  1 row per 1024-thread workgroup
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

inline int64_t tile_steps(const Variant &v) {
  return static_cast<int64_t>(kStepsPerLane) * v.LPR * v.WPR;
}

// Host-side address of the kernel instance for an algorithm (Algo), input
// dtype (rlca_dtype), variant index and stride mode.  plain_kernel: the
// windowed entry points without carries (every Algo but the generic scan);
// window_kernel: carry vector in, carry and carry map out (every Algo).
const void *plain_kernel(int algo, int dtype, int variant, bool uniform);
const void *window_kernel(int algo, int dtype, int variant, bool uniform);
// The policy-table kernels (Retrace, V-trace), 256-thread workgroups: 4
// wavefronts per row (1024-step tiles, one row per workgroup) or 1 (256-step
// tiles, four rows per workgroup).
const void *probs_kernel_for(int algo, int dtype, int waves_per_row, bool window);
constexpr int kProbsBlock = 256;
constexpr int64_t kProbsShortRow = 256;  // rows up to this long: one wavefront each

}  // namespace rlca
