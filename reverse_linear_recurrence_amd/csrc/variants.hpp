// variants.hpp -- the tiling variants of the scan kernels and the lookup of a
// compiled kernel instance; shared by the host code and the kernel tables.
#pragma once

#include <stdint.h>

namespace rlca {

enum Algo : int {
  kReturns = 0, kGae = 1, kTdLambda = 2, kVtrace = 3, kRetrace = 4,
  // forward-time mirrors: A_t = alpha_t + beta_t * A_{t-1}
  kEligibility = 5, kCumsum = 6,
  // the generic segmented scan over caller-given (alpha, beta), reverse and
  // forward in time
  kAffine = 7, kAffineFwd = 8
};

struct Variant {
  int LPR;    // lanes per row inside a wavefront (64 when WPR > 1)
  int WPR;    // wavefronts per row
  bool wide;  // 8 steps per lane on bf16 inputs (see steps_per_lane)
};

constexpr Variant kVariants[] = {
    {16, 1, false},  // 0: tile    64 steps, 16 rows per 256-thread workgroup (window, GAE: 32 per 512)
    {32, 1, false},  // 1: tile   128,  8 rows per workgroup (window, GAE: 16 per 512 threads)
    {64, 1, false},  // 2: tile   256,  4 rows per workgroup
    {64, 4, false},  // 3: tile  1024,  1 row per 256-thread workgroup
    {64, 8, false},  // 4: tile  2048,  1 row per 512-thread workgroup
    {64, 16, false}, // 5: tile  4096,  1 row per 1024-thread workgroup
    {64, 4, true},   // 6: as 3, bf16 tile 2048
    {64, 8, true},   // 7: as 4, bf16 tile 4096
    {64, 16, true},  // 8: as 5, bf16 tile 8192
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);
constexpr int kFirstWide = 6;  // variants kFirstWide + i are variants 3 + i, wide

// Every lane owns K consecutive steps, one 16-byte vector of each input
// array: K = 4 everywhere except the wide variants on bf16 inputs, where
// K = 8 (one 16-byte vector of each bf16 array).  That halves the tiles (and
// the workgroup barriers) per row and doubles the bytes each tile has in
// flight.  V-trace keeps K = 4 there: its 1024-thread instance would spill;
// on fp32 inputs and for V-trace a wide variant is the same kernel as its
// narrow twin.  Each load instruction of a wavefront covers one contiguous
// span, and so does each output store (at K = 8 after staging through LDS).
// (Longer fp32 spans per lane split each instruction into strided partial
// lines: 4x the line requests for 16 fp32 steps per lane.)
constexpr int steps_per_lane(const Variant &v, bool bf16, bool vtrace) {
  return v.wide && bf16 && !vtrace ? 8 : 4;
}

// Wavefronts per workgroup: WPR for rows of whole wavefronts; otherwise 4,
// or 8 for window instances and GAE when rows take part of a wavefront
// (LPR < 64).  Larger workgroups write the per-row carry vectors in longer
// runs: the GAE 4096x128 window call took 3.66 instead of 3.97 us,
// eligibility 2.91 instead of 2.99; with one row per wavefront they were
// slower (TD(lambda) 16384x256 window 11.93 against 11.52 us).  Of the plain
// calls, GAE 4096x128 (two outputs) took 3.29 against 3.31 us with 8, while
// the eligibility trace and the episodic sum at 4096x128 took 2.54 against
// 2.52 us and keep 4 (2 wavefronts: 3.45, 2.53 us).
constexpr int short_row_waves(int WPR, int LPR, bool window, int algo) {
  return WPR > 1 ? WPR : (LPR < 64 && (window || algo == kGae) ? 8 : 4);
}

inline int64_t tile_steps(const Variant &v, bool bf16, bool vtrace) {
  return static_cast<int64_t>(steps_per_lane(v, bf16, vtrace)) * v.LPR * v.WPR;
}

// Host-side address of the kernel instance for an algorithm (Algo), input
// dtype (rlca_dtype), variant index and stride mode.  plain_kernel: the
// windowed entry points without carries (every Algo but the generic scan),
// tiles: 1 or 2 for the instance of rows of exactly that many whole tiles
// (uniform strides only; otherwise, and for 0, the general instance),
// aligned: with every flag row 4-byte aligned (reverse recurrences and the
// generic scan); window_kernel: carry vector in, carry and carry map out
// (every Algo), with the same choices.
const void *plain_kernel(int algo, int dtype, int variant, bool uniform, int tiles, bool aligned);
const void *window_kernel(int algo, int dtype, int variant, bool uniform, int tiles,
                          bool aligned);
// chain_kernel: the chained instance (one-launch split call) for segments of
// `tiles` (1 or 2) whole tiles of a whole-wavefront tiling (variants 3-8,
// uniform row stride); NULL otherwise.
const void *chain_kernel(int algo, int dtype, int variant, int tiles);
// The policy-table kernels (Retrace, V-trace), 256-thread workgroups: 4
// wavefronts per row (1024-step tiles, one row per workgroup) or 1 (256-step
// tiles, four rows per workgroup).
const void *probs_kernel_for(int algo, int dtype, int waves_per_row, bool window);
constexpr int kProbsBlock = 256;
constexpr int64_t kProbsShortRow = 256;  // rows up to this long: one wavefront each

}  // namespace rlca
