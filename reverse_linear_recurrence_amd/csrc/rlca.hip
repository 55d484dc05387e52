// rlca.hip -- host side of librlca.so: argument validation, tiling choice and
// kernel launch for the C ABI declared in include/rlca.h.
//
// Nothing here touches element data: every step of the computation runs in
// the kernels of scan_kernels.hpp (instantiated in kernels_plain.hip and
// kernels_window.hip) and probs_kernels.hpp (kernels_probs.hip).  A call
// validates its arguments, picks a tiling variant, and enqueues one kernel on
// the caller's stream (a window call split over a few long rows: three, see
// below).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "materialized.hpp"
#include "probs_kernels.hpp"
#include "rlca.h"
#include "scan_kernels.hpp"
#include "variants.hpp"

namespace rlca {

// The public algorithm codes of rlca_variant_info are the kernels' own.
constexpr bool same_code(int public_code, int kernel_code) { return public_code == kernel_code; }
static_assert(same_code(RLCA_ALGO_RETURNS, kReturns) && same_code(RLCA_ALGO_GAE, kGae) &&
                  same_code(RLCA_ALGO_TD_LAMBDA, kTdLambda) &&
                  same_code(RLCA_ALGO_VTRACE, kVtrace) && same_code(RLCA_ALGO_RETRACE, kRetrace) &&
                  same_code(RLCA_ALGO_ELIGIBILITY, kEligibility) &&
                  same_code(RLCA_ALGO_CUMSUM, kCumsum) && same_code(RLCA_ALGO_AFFINE, kAffine),
              "rlca_algo and Algo disagree");
namespace {

// Default tiling (measured on MI355X).  Short rows: the smallest
// one-wavefront tile that covers T.  Long rows (tiles loop along T, each
// tile's loads issued while the previous one is computed): about 4096
// wavefronts (16 per CU) -- the most wavefronts per row such that N * WPR
// stays within that and the tile is not longer than the row; from 8192 rows
// on, one wavefront per row.  On bf16 inputs a long-row choice then takes its
// wide twin (8 steps per lane) when the row holds one of its tiles.
int auto_variant(int64_t N, int64_t T, bool bf16, bool vtrace) {
  constexpr int64_t kTargetWaves = 4096;
  auto tile = [&](int v) { return tile_steps(kVariants[v], bf16, vtrace); };
  auto widen = [&](int v) {
    const int w = v - 3 + kFirstWide;
    return steps_per_lane(kVariants[w], bf16, vtrace) == 8 && tile(w) <= T ? w : v;
  };
  for (int v = 0; v <= 2; ++v)
    if (T <= tile(v)) return v;
  if (N >= 2 * kTargetWaves) return 2;
  for (int v = 5; v >= 3; --v)
    if (N * kVariants[v].WPR <= kTargetWaves && tile(v) <= T) return widen(v);
  return tile(3) <= T ? widen(3) : 2;
}

// ------------------------------------------------------------- errors

thread_local std::string t_last_error;
thread_local int t_forced_variant = -1;
thread_local int t_last_variant = -1;
thread_local int t_chained = 1;      // rlca_set_chained
thread_local int t_last_launches = 0;  // rlca_last_launches
thread_local int t_last_segments = 0;  // rlca_last_segments


int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  t_last_error = buf;
  return status;
}

#ifdef RLCA_TIMESTAMPS
// Instrumented build: the wavefronts' wall-clock stamps of the last scan
// kernel launched on each device (see scan_kernels.hpp), and the number of
// wavefronts of the calling thread's last launch.
static __device__ __align__(256) uint64_t stamp_buf[2 * kStampWaves];
std::mutex g_stamp_mutex;
uint64_t *g_stamp_buf[64];
thread_local int64_t t_last_waves = 0;
thread_local int t_last_device = 0;

int stamp_buffer(int *dev_out, uint64_t **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RLCA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(RLCA_EINVAL, "device %d beyond the stamp table", dev);
  std::lock_guard<std::mutex> lock(g_stamp_mutex);
  if (g_stamp_buf[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(stamp_buf));
    if (e != hipSuccess || p == nullptr)
      return fail(RLCA_EHIP, "address of the stamp buffer: %s", hipGetErrorString(e));
    g_stamp_buf[dev] = static_cast<uint64_t *>(p);
  }
  *dev_out = dev;
  *out = g_stamp_buf[dev];
  return RLCA_OK;
}
#endif

// ------------------------------------------------------------- validation

struct Arr {
  const char *name;
  const void *ptr;
  int64_t ld;      // row stride in elements
  int64_t width;   // elements used per row
  int64_t esize;   // bytes per element
  bool required;
  bool output;
  bool one_row = false;  // a single row (the per-row bootstrap vector)
  // Byte span [lo, hi) the call may touch; filled by check_array.
  uintptr_t lo = 0, hi = 0;
};

int check_array(Arr &a, int64_t N) {
  if (a.one_row) N = 1;
  if (a.ptr == nullptr) {
    if (a.required) return fail(RLCA_EINVAL, "%s must not be NULL", a.name);
    return RLCA_OK;
  }
  const uintptr_t p = reinterpret_cast<uintptr_t>(a.ptr);
  if (p % static_cast<uintptr_t>(a.esize) != 0)
    return fail(RLCA_EINVAL, "%s is not aligned to its element size (%lld bytes)", a.name,
                static_cast<long long>(a.esize));
  if (a.ld < a.width)
    return fail(RLCA_EINVAL, "ld_%s = %lld is smaller than the row length %lld", a.name,
                static_cast<long long>(a.ld), static_cast<long long>(a.width));
  if (a.ld > INT32_MAX && !a.one_row)
    return fail(RLCA_EINVAL, "ld_%s = %lld exceeds 2^31-1", a.name, static_cast<long long>(a.ld));
  // Span in elements: (N-1)*ld + width, checked against overflow.
  const int64_t lim = INT64_MAX / a.esize;
  if (N > 1 && a.ld > (lim - a.width) / (N - 1))
    return fail(RLCA_EINVAL, "%s: %lld rows of stride %lld overflow the address space", a.name,
                static_cast<long long>(N), static_cast<long long>(a.ld));
  const int64_t elems = (N - 1) * a.ld + a.width;
  a.lo = p;
  a.hi = p + static_cast<uintptr_t>(elems * a.esize);
  if (a.hi < a.lo) return fail(RLCA_EINVAL, "%s: address range wraps around", a.name);
  return RLCA_OK;
}

int check_aliasing(Arr *arrs, int n) {
  for (int i = 0; i < n; ++i) {
    if (!arrs[i].output || arrs[i].ptr == nullptr) continue;
    for (int j = 0; j < n; ++j) {
      if (i == j || arrs[j].ptr == nullptr) continue;
      if (arrs[j].output && j < i) continue;  // each output pair once
      if (arrs[i].lo < arrs[j].hi && arrs[j].lo < arrs[i].hi)
        return fail(RLCA_EALIAS, "output %s overlaps %s %s", arrs[i].name,
                    arrs[j].output ? "output" : "input", arrs[j].name);
    }
  }
  return RLCA_OK;
}

int check_unit(const char *name, float x) {
  if (!(x >= 0.f && x <= 1.f)) return fail(RLCA_EINVAL, "%s = %g must lie in [0, 1]", name, x);
  return RLCA_OK;
}

int check_clip(const char *name, float x) {
  if (!(x > 0.f)) return fail(RLCA_EINVAL, "%s = %g must be > 0", name, x);
  return RLCA_OK;
}

int check_sizes(int64_t N, int64_t T, int dtype) {
  if (N < 0) return fail(RLCA_EINVAL, "num_envs = %lld must be >= 0", static_cast<long long>(N));
  if (T < 1) return fail(RLCA_EINVAL, "T = %lld must be >= 1", static_cast<long long>(T));
  if (N > INT32_MAX) return fail(RLCA_EINVAL, "num_envs = %lld exceeds 2^31-1", static_cast<long long>(N));
  if (T > INT32_MAX - 1)
    return fail(RLCA_EINVAL, "T = %lld exceeds 2^31-2", static_cast<long long>(T));
  if (dtype != RLCA_F32 && dtype != RLCA_BF16) return fail(RLCA_EDTYPE, "unknown dtype %d", dtype);
  return RLCA_OK;
}

#define RLCA_TRY(expr)            \
  do {                            \
    const int rc_ = (expr);       \
    if (rc_ != RLCA_OK) return rc_; \
  } while (0)

// The hot streams of a launch (see scan_kernels.hpp) and the stride of values
// (or Retrace's truncation switch) in ldx; returns whether the hot [N,T]
// streams share the rewards' row stride (the kUniform instances).
bool hot_streams(int algo, const Args &a, bool dense_tv, const void *(&hot)[5], int64_t *ldx_out) {
  hot[0] = a.r;
  for (int i = 1; i < 5; ++i) hot[i] = nullptr;
  int64_t hld[5] = {a.ld_r, 0, 0, 0, 0};  // stride of each hot [N,T] stream (0: none)
  int64_t ldx = 0;
  switch (algo) {
    case kReturns:
      hot[1] = a.term; hld[1] = a.ld_term;
      hot[2] = a.trunc; hld[2] = a.ld_trunc;
      hot[3] = dense_tv ? a.tv : nullptr; hld[3] = a.ld_tv;
      hot[4] = a.boot;  // a [N] vector: no stride
      break;
    case kGae:
    case kTdLambda:
      hot[1] = a.v; ldx = a.ld_v;
      hot[2] = a.term; hld[2] = a.ld_term;
      hot[3] = a.trunc; hld[3] = a.ld_trunc;
      hot[4] = dense_tv ? a.tv : nullptr; hld[4] = a.ld_tv;
      break;
    case kVtrace:
      hot[1] = a.v; ldx = a.ld_v;
      hot[2] = a.lr; hld[2] = a.ld_lr;
      hot[3] = a.term; hld[3] = a.ld_term;
      hot[4] = a.trunc; hld[4] = a.ld_trunc;
      break;
    case kRetrace:
      hot[1] = a.v; hld[1] = a.ld_v;
      hot[2] = a.eq; hld[2] = a.ld_eq;
      hot[3] = a.lr; hld[3] = a.ld_lr;
      hot[4] = a.term; hld[4] = a.ld_term;
      ldx = a.trunc != nullptr ? 1 : 0;
      break;
    case kAffine:
    case kAffineFwd:
      hot[1] = a.v; hld[1] = a.ld_v;  // beta
      hot[2] = a.term; hld[2] = a.ld_term;  // reset flags
      break;
    default:  // kEligibility, kCumsum
      hot[1] = a.term; hld[1] = a.ld_term;
      hot[2] = a.trunc; hld[2] = a.ld_trunc;
      hot[3] = a.boot;  // initial carry, a [N] vector: no stride
      break;
  }
  bool uniform = true;
  for (int i = 1; i < 5; ++i)
    if (hot[i] != nullptr && hld[i] != 0 && hld[i] != a.ld_r) uniform = false;
  *ldx_out = ldx;
  return uniform;
}

int64_t esize_of(int dtype) { return dtype == RLCA_BF16 ? 2 : 4; }

// A chained split (one pass over the inputs): the tiling, whole tiles per
// segment, segments per row, and the workspace (its epoch word, then the
// words the segments publish).
struct ChainPlan {
  int v = -1;  // < 0: none
  int tiles = 0;
  int64_t S = 0;
  unsigned long long *slots = nullptr;
};

// window: the instance with carry vectors (Args::cin, cout, cmap).
// S > 1: segment view (window instances): each of the args.N rows is cut
// into S segments of args.T steps, segment y taken by grid row y.
// chain: the chained instance for that segment view (S = chain->S).
int launch(int algo, int dtype, const Args &args, void *stream, bool window = false, int S = 1,
           const ChainPlan *chain = nullptr) {
  const int v = chain != nullptr ? chain->v
                : t_forced_variant >= 0
                    ? t_forced_variant
                    : auto_variant(args.N * S, args.T, dtype == RLCA_BF16, algo == kVtrace);
  const Variant var = kVariants[v];
  dim3 grid, block;
  const int waves = short_row_waves(var.WPR, var.LPR, window, algo);
  if (var.WPR > 1) {
    grid = dim3(static_cast<unsigned>(args.N), static_cast<unsigned>(S));
  } else {
    const int64_t rows_per_wg = waves * (64 / var.LPR);
    grid = dim3(static_cast<unsigned>((args.N + rows_per_wg - 1) / rows_per_wg),
                static_cast<unsigned>(S));
  }
  block = dim3(64 * waves);
  Args a = args;
  a.seg_count = S;
  if (chain != nullptr) {
    a.chain = chain->slots;
    if (!(algo == kEligibility || algo == kCumsum || algo == kAffineFwd)) {
      // Reverse recurrences take the segments from the row's end: every row
      // pointer moves to the row's last segment (scan_kernels.hpp).
      const int64_t shift = (S - 1) * args.T;
      const int64_t es = esize_of(dtype);
      auto move = [&](const void *ptr, int64_t esize) -> const void * {
        return ptr == nullptr ? nullptr : static_cast<const char *>(ptr) + shift * esize;
      };
      a.r = move(a.r, es);
      a.v = move(a.v, es);
      a.lr = move(a.lr, es);
      a.eq = move(a.eq, es);
      a.tv = move(a.tv, es);
      a.term = static_cast<const uint8_t *>(move(a.term, 1));
      a.trunc = static_cast<const uint8_t *>(move(a.trunc, 1));
      a.o0 = a.o0 == nullptr ? nullptr : a.o0 + shift;
      a.o1 = a.o1 == nullptr ? nullptr : a.o1 + shift;
    }
  }
#ifdef RLCA_TIMESTAMPS
  int stamp_dev = 0;
  RLCA_TRY(stamp_buffer(&stamp_dev, &a.stamps));
#endif
  // Truncation bootstraps of the whole call: dense reads for small batches.
  const bool dense_tv = args.N * S * args.T <= kDenseTvMaxSteps;
  // Hot streams (see scan_kernels.hpp), passed again as preloaded scalars.
  const void *hot[5];
  int64_t ldx = 0;
  const bool uniform = hot_streams(algo, a, dense_tv, hot, &ldx);
  int N32 = static_cast<int>(a.N);
  int T32 = static_cast<int>(a.T);
  int ldT = static_cast<int>(a.ld_r);
  int ldX = static_cast<int>(ldx);
  void *kargs[] = {&hot[0], &hot[1], &hot[2], &hot[3], &hot[4], &N32, &T32, &ldT, &ldX, &a};
  // Rows of exactly one or two whole tiles take the instance for that many
  // tiles (straight-line code: fewer registers, or no redundant prefetch),
  // and its aligned twin when every flag row the kernel reads is 4-byte
  // aligned: the flag arrays' rows, or, standing in for a missing one, the
  // rewards' rows.
  const int64_t tile = tile_steps(var, dtype == RLCA_BF16, algo == kVtrace);
  const int tiles = args.T == tile ? 1 : (args.T == 2 * tile ? 2 : 0);
  auto rows_aligned = [&](const void *ptr, int64_t ld, int64_t esize) {
    return reinterpret_cast<uintptr_t>(ptr) % 4 == 0 && (args.N <= 1 || (ld * esize) % 4 == 0);
  };
  const int64_t es = dtype == RLCA_BF16 ? 2 : 4;
  const bool flags_aligned =
      (a.term == nullptr || rows_aligned(a.term, a.ld_term, 1)) &&
      (a.trunc == nullptr || rows_aligned(a.trunc, a.ld_trunc, 1)) &&
      ((a.term != nullptr && a.trunc != nullptr) || rows_aligned(a.r, a.ld_r, es));
  const void *kernel = chain != nullptr ? (uniform ? chain_kernel(algo, dtype, v, chain->tiles)
                                                   : nullptr)
                       : window ? window_kernel(algo, dtype, v, uniform, tiles, flags_aligned)
                                : plain_kernel(algo, dtype, v, uniform, tiles, flags_aligned);
  if (kernel == nullptr) return fail(RLCA_EINVAL, "no kernel for algorithm %d", algo);
  const hipError_t e = hipLaunchKernel(kernel, grid, block, kargs, 0,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(RLCA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  t_last_variant = v;
#ifdef RLCA_TIMESTAMPS
  t_last_waves = static_cast<int64_t>(grid.x) * grid.y * waves;
  t_last_device = stamp_dev;
#endif
  return RLCA_OK;
}

// The carry vectors of a window call (all NULL and off for the plain calls),
// and the caller's workspace for a split call (NULL: never split).
struct Window {
  bool on;
  const float *cin;
  float *cout;
  float *cmap;
  void *ws = nullptr;
  int64_t ws_bytes = 0;
  // The materialized doubling scan (materialized.hpp) in ws instead of the
  // fused kernel.
  bool materialized = false;
};
constexpr Window kNoWindow{false, nullptr, nullptr, nullptr};

// The materialized doubling scan: its pairs (two pairs of [N, T] float
// arrays) in the caller's workspace; 2 + ceil(log2 T) launches.
int launch_materialized(int algo, int dtype, const Args &args, float *ws, void *stream) {
  int64_t N = args.N, T = args.T;
  const int64_t NT = N * T;
  float *pa = ws, *pb = ws + NT, *qa = ws + 2 * NT, *qb = ws + 3 * NT;
  const dim3 grid(static_cast<unsigned>((T + kMatBlock - 1) / kMatBlock),
                  static_cast<unsigned>(N < kMatMaxGridRows ? N : kMatMaxGridRows));
  const dim3 block(kMatBlock);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  Args a = args;
  auto go = [&](const void *kernel, void **kargs) {
    if (kernel == nullptr) return fail(RLCA_EINVAL, "no materialized kernel for algorithm %d", algo);
    const hipError_t e = hipLaunchKernel(kernel, grid, block, kargs, 0, s);
    if (e != hipSuccess) return fail(RLCA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return static_cast<int>(RLCA_OK);
  };
  void *k1[] = {&a, &pa, &pb};
  RLCA_TRY(go(mat_coeffs_kernel(algo, dtype), k1));
  for (int64_t off = 1; off < T; off *= 2) {
    void *kd[] = {&pa, &pb, &qa, &qb, &N, &T, &off};
    RLCA_TRY(go(mat_double_kernel(), kd));
    float *ta = pa, *tb = pb;
    pa = qa;
    pb = qb;
    qa = ta;
    qb = tb;
  }
  void *k3[] = {&a, &pa, &pb};
  RLCA_TRY(go(mat_epilogue_kernel(algo, dtype), k3));
  t_last_variant = -1;
  return RLCA_OK;
}

// Room a call's argument table keeps after its own arrays: the window's
// three carry vectors and a split call's workspace.
constexpr int kExtraArrs = 4;

// Append the window's carry vectors to a call's arrays (arrs has room for
// them); returns the new count.
int add_window(Arr *arrs, int n, const Window &w, int64_t N) {
  if (w.on) {
    arrs[n++] = Arr{"carry_in", w.cin, N, N, 4, false, false, true};
    arrs[n++] = Arr{"carry_out", w.cout, N, N, 4, false, true, true};
    arrs[n++] = Arr{"carry_map", w.cmap, 2 * N, 2 * N, 4, false, true, true};
  }
  return n;
}

// ------------------------------------------------------------- split calls
//
// Few long rows leave most CUs idle with one workgroup per row.  A window call
// (or generic scan) given a workspace takes the chained form below where it
// applies; otherwise, with at most kSplitMaxRows rows, it
// cuts every row into S segments of T / S steps and runs them as N * S rows of
// the window kernels, the T-split of the window calls done inside the library:
//   1. every segment from carry 0, writing only its carry map (a, b);
//   2. per row, the maps composed from the row's end (forward mirrors: its
//      start) into the carry entering each segment, and the row's carry out
//      and carry map (compose_carries);
//   3. every segment again from that carry, writing the outputs.
// The inputs are read twice.  Used only by window calls given a workspace of
// at least 3 * N * S floats (rlca_split_workspace_bytes).

constexpr int64_t kSplitMaxRows = 64;    // split calls with at most this many rows
constexpr int64_t kSplitMinRow = 32768;  // and rows at least this long
constexpr int64_t kSplitTarget = 256;    // into about this many segments (one per CU)
constexpr int64_t kSplitMinLen = 4096;   // of at least this many steps

// Segments per row for a call of N rows of T steps (1: no split): the
// smallest power of two with N * S >= kSplitTarget, T % S == 0 and
// T / S >= kSplitMinLen, stopping early where either no longer holds.  Below
// kSplitMinRow steps a row takes one workgroup too little time to repay the
// two extra launches and the second read (bf16 96x16384: 9.9 us unsplit,
// 12.1 us split into 4), and above kSplitMaxRows rows the unsplit call
// already nears the bandwidth the split reaches (bf16 96x32768: 18.5 us
// unsplit, 20.5 us split into 4; 64x65536: 32.4 against 22.8 us).
int64_t split_count(int64_t N, int64_t T) {
  if (N > kSplitMaxRows || T < kSplitMinRow) return 1;
  int64_t S = 1;
  while (N * S < kSplitTarget && T % (2 * S) == 0 && T / (2 * S) >= kSplitMinLen) S *= 2;
  return S;
}

// The chained form of a split call (one pass; see scan_kernels.hpp): the
// segments are one or two whole tiles of a whole-wavefront tiling, at most
// kChainMaxSegments per row, so that each workgroup's segment is scanned in
// registers before its carry is known.  Taken for N rows of T steps with
// T >= kChainMinRow and N <= min(kChainMaxRows, T / kChainStepsPerRow):
// with more rows, one workgroup per row already keeps enough CUs busy for
// long enough that the look-back, a latency the unsplit call does not have,
// costs more than the split saves.  Measured on GAE (us per call, unsplit
// against chained): bf16 240x32768 24.8 / 25.1, 208x49152 34.9 / 31.7, fp32
// 224x32768 28.2 / 29.4; bf16 128x16384 8.9 / 7.9, 200x16384 10.2 / 12.9;
// bf16 64x8192 5.5 / 4.9, 128x8192 5.9 / 6.4; bf16 32x4096 3.8 / 4.6.
//
// Of the plans, the one with the least
//   ceil(N * S / kSplitTarget) * L + ceil(N * S / (kSplitTarget * r)) * kChainSegmentCost
//     + S * kChainLinkCost,
// ties going to the longer segment: the rounds of one segment per CU the
// grid needs times a segment's L steps, plus a fixed cost per segment (its
// start, its look-back and its drain) that a second workgroup resident on
// the same CU hides (r = chain_residency, 1 or 2), plus a cost per link of
// a row's chain (beyond 64 segments a look-back waits for a segment 64
// back to have found its own carry; bf16 2x262144: 7.2 us in 128 segments
// of 2048 steps per row, 6.3 in 64 of 4096).  Measured on GAE (us per call):
// bf16 16x262144 15.4 with two tiles of 8192 per segment, 15.4 with one;
// 176x131072, 74.7 and 68.8; 160x32768, 22.0 and 18.5 (unsplit 22.2); fp32
// 96x32768, 14.6 with two tiles of 4096, 14.1 with two of 2048 (the best),
// 16.2 with one of 4096.  A rule on the segment count alone misses one way
// or the other: the fewer, longer segments win where they fill the CUs
// once, the shorter ones where the longer would leave a second round half
// empty.
constexpr int64_t kChainMaxRows = 224;
constexpr int64_t kChainMinRow = 8192;
constexpr int64_t kChainStepsPerRow = 128;
constexpr int64_t kChainSegmentCost = 4096;
constexpr int64_t kChainLinkCost = 32;

// Workgroups of a chained instance that one CU holds at once, counted up to
// 2.  Every chained instance holds at least two, but for the 16-wavefront
// instances of two tiles that need more than 64 VGPRs (two such workgroups
// put 8 wavefronts on each SIMD, which then has room for fewer): returns,
// GAE and TD(lambda) at 8 steps per lane (70 to 87 VGPRs), V-trace (66),
// and Retrace at 8 steps per lane or on bf16 inputs (67 to 101).  These
// counts are those of the compiled code; a CPU test checks the table
// against it.
int chain_residency(int algo, const Variant &v, int tiles, bool bf16) {
  if (v.WPR != 16 || tiles != 2) return 2;
  const int K = steps_per_lane(v, bf16, algo == kVtrace);
  switch (algo) {
    case kReturns:
    case kGae:
    case kTdLambda:
      return K == 8 ? 1 : 2;
    case kVtrace:
      return 1;
    case kRetrace:
      return K == 8 || bf16 ? 1 : 2;
    default:
      return 2;
  }
}

ChainPlan chain_plan(int64_t N, int64_t T, bool bf16, int algo) {
  ChainPlan best;
  if (N < 1 || N > kChainMaxRows || T < kChainMinRow || N * kChainStepsPerRow > T) return best;
  int64_t best_cost = 0, best_len = 0;
  auto consider = [&](bool wide_only) {
    for (int v = kNumVariants - 1; v >= 0; --v) {
      if (kVariants[v].WPR == 1 || (wide_only && !kVariants[v].wide)) continue;
      for (int tiles = 2; tiles >= 1; --tiles) {
        const int64_t len = tiles * tile_steps(kVariants[v], bf16, algo == kVtrace);
        if (T % len != 0) continue;
        const int64_t S = T / len;
        if (S < 2 || S > kChainMaxSegments) continue;
        const int64_t r = chain_residency(algo, kVariants[v], tiles, bf16);
        const int64_t cost =
            (N * S + kSplitTarget - 1) / kSplitTarget * len +
            (N * S + kSplitTarget * r - 1) / (kSplitTarget * r) * kChainSegmentCost +
            S * kChainLinkCost;
        if (best.v < 0 || cost < best_cost || (cost == best_cost && len > best_len)) {
          best.v = v;
          best.tiles = tiles;
          best.S = S;
          best_cost = cost;
          best_len = len;
        }
      }
    }
  };
  // On bf16 inputs the wide tilings (8 steps per lane: one 16-byte vector
  // per lane and array) come before the narrow ones (8-byte vectors), which
  // serve only rows that no wide tile divides (bf16 GAE 4x65536: 5.2 us in
  // 128 segments of 2048 steps, 5.7 us in 256 of 1024).
  if (bf16 && algo != kVtrace) consider(true);
  if (best.v < 0) consider(false);
  return best;
}

// Workspace bytes of a chained split: the epoch word, then 4 words per
// segment.
int64_t chain_bytes(int64_t N, int64_t S) { return 8 + 32 * N * S; }

// The workspace a split call of N rows of T steps may use: the larger of the
// three-launch split's and the chained form's for any input dtype and algorithm.
int64_t split_workspace_bytes(int64_t N, int64_t T) {
  const int64_t S = split_count(N, T);
  int64_t need = S > 1 ? 12 * N * S : 0;
  for (int bf16 = 0; bf16 < 2; ++bf16) {
    for (int algo = kReturns; algo <= kAffineFwd; ++algo) {
      const ChainPlan c = chain_plan(N, T, bf16 != 0, algo);
      if (c.v >= 0 && chain_bytes(N, c.S) > need) need = chain_bytes(N, c.S);
    }
  }
  return need;
}

// The carry entering each segment, from the segments' maps: reverse
// recurrences compose from the row's last segment, forward ones from its
// first, starting from the caller's carry_in (NULL: 0).  Also the row's
// carry_out (the last segment's outgoing carry in composition order) and its
// carry map (the composite of every segment map).  One wavefront per row.
// Its lanes load the maps of 64 consecutive segments at once (every chunk's
// loads are issued before the first is used), and a shuffle scan composes
// them: lane j ends with the composite of the chunk's maps from its own to
// the chunk's end in composition order.  Chunks are taken in that order, each
// starting from the carry the previous one hands on.
__global__ void __launch_bounds__(64)
compose_carries(const float *__restrict__ map, const float *__restrict__ init,
                float *__restrict__ cin, int S, bool forward, float *__restrict__ cout,
                float *__restrict__ cmap) {
  constexpr int kMaxChunks = 4;
  static_assert(kSplitTarget <= 64 * kMaxChunks, "S <= kSplitTarget segments per row");
  const int64_t n = blockIdx.x;
  const int lane = threadIdx.x;
  const int nchunks = (S + 63) / 64;
  // chunk k, lane j: the segment j-th in composition order within the chunk
  auto seg_of = [&](int k, int j) {
    const int i = 64 * k + j;  // position in composition order
    return forward ? i : S - 1 - i;
  };
  float ma[kMaxChunks], mb[kMaxChunks];
#pragma unroll
  for (int k = 0; k < kMaxChunks; ++k) {
    ma[k] = 0.f;
    mb[k] = 1.f;  // identity past the row's segments
    if (k < nchunks && 64 * k + lane < S) {
      const int64_t e = n * S + seg_of(k, lane);
      ma[k] = map[2 * e];
      mb[k] = map[2 * e + 1];
    }
  }
  float c = init != nullptr ? init[n] : 0.f;
  float ta = 0.f, tb = 1.f;  // the composite of the chunks so far
  for (int k = 0; k < nchunks; ++k) {
    // Inclusive scan in composition order: after it, lane j holds
    // f_j o f_{j-1} o ... o f_0 (f_0 applied first).
    float a = ma[k], b = mb[k];
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
      const float pa = __shfl_up(a, d), pb = __shfl_up(b, d);
      if (lane >= d) {
        a = fmaf(b, pa, a);
        b = b * pb;
      }
    }
    // The carry entering lane j's segment: lanes 0 .. j-1 applied to c.
    float ea = __shfl_up(a, 1), eb = __shfl_up(b, 1);
    if (lane == 0) {
      ea = 0.f;
      eb = 1.f;
    }
    if (64 * k + lane < S) cin[n * S + seg_of(k, lane)] = fmaf(eb, c, ea);
    const float ka = __shfl(a, 63), kb = __shfl(b, 63);
    c = fmaf(kb, c, ka);
    ta = fmaf(kb, ta, ka);
    tb = kb * tb;
  }
  if (lane == 0) {
    if (cout != nullptr) cout[n] = c;
    if (cmap != nullptr) {
      cmap[2 * n] = ta;
      cmap[2 * n + 1] = tb;
    }
  }
}

// Validate the arrays of a call (plus the window's carry vectors and a split
// call's workspace), then fill the window fields of Args and launch.  The
// call's n arrays come first in arrs, which has room for kExtraArrs more.
template <int kCap>
int validate_and_launch(int algo, int dtype, int64_t N, Arr (&arrs)[kCap], int n,
                        const Window &w, Args &a, void *stream) {
  if (n + kExtraArrs > kCap) return fail(RLCA_EINVAL, "internal: argument table too small");
  n = add_window(arrs, n, w, N);
  if (w.ws != nullptr) {
    if (w.ws_bytes < 0)
      return fail(RLCA_EINVAL, "workspace_bytes = %lld is negative",
                  static_cast<long long>(w.ws_bytes));
    if (reinterpret_cast<uintptr_t>(w.ws) % 4 != 0)
      return fail(RLCA_EINVAL, "workspace is not 4-byte aligned");
  }
  if (w.materialized) {
    if (w.ws == nullptr) return fail(RLCA_EINVAL, "the materialized scan needs a workspace");
    if (N == 0) return RLCA_OK;
    if (N > INT64_MAX / 16 / a.T)
      return fail(RLCA_EINVAL, "%lld x %lld steps are too many for the materialized scan",
                  static_cast<long long>(N), static_cast<long long>(a.T));
    const int64_t nt = N * a.T;
    if (w.ws_bytes < 16 * nt)
      return fail(RLCA_EINVAL,
                  "workspace_bytes = %lld is less than the %lld the materialized scan needs "
                  "(rlca_materialized_workspace_bytes)",
                  static_cast<long long>(w.ws_bytes), static_cast<long long>(16 * nt));
    arrs[n++] = Arr{"workspace", w.ws, 4 * nt, 4 * nt, 4, false, true, true};
    for (int i = 0; i < n; ++i) RLCA_TRY(check_array(arrs[i], N));
    RLCA_TRY(check_aliasing(arrs, n));
    RLCA_TRY(launch_materialized(algo, dtype, a, static_cast<float *>(w.ws), stream));
    t_last_launches = 2 + static_cast<int>(std::ceil(std::log2(static_cast<double>(a.T))));
    t_last_segments = 1;
    return RLCA_OK;
  }
  if (N == 0) return RLCA_OK;
  // The chained split (one pass) where it applies: a workspace large
  // enough and 8-byte aligned (its words are 64-bit), rows that share one
  // stride, and chaining not switched off for this thread.  (It wins also
  // where it has fewer segments than the three-launch form: bf16 GAE
  // 1x1048576, 64 against 256 segments, took 11.77 against 12.37 us;
  // 2x524288, 64 against 128, 8.47 against 10.76 us.)
  if (w.ws != nullptr && t_chained) {
    ChainPlan cp = chain_plan(N, a.T, dtype == RLCA_BF16, algo);
    const void *hot[5];
    int64_t ldx = 0;
    if (cp.v >= 0 &&
        reinterpret_cast<uintptr_t>(w.ws) % 8 == 0 &&
        w.ws_bytes >= chain_bytes(N, cp.S) && hot_streams(algo, a, false, hot, &ldx)) {
      const int64_t floats = chain_bytes(N, cp.S) / 4;
      arrs[n++] = Arr{"workspace", w.ws, floats, floats, 4, false, true, true};
      for (int i = 0; i < n; ++i) RLCA_TRY(check_array(arrs[i], N));
      RLCA_TRY(check_aliasing(arrs, n));
      a.cin = w.cin;
      a.cout = w.cout;
      a.cmap = w.cmap;
      cp.slots = static_cast<unsigned long long *>(w.ws);
      Args ac = a;
      ac.T = a.T / cp.S;
      RLCA_TRY(launch(algo, dtype, ac, stream, true, static_cast<int>(cp.S), &cp));
      t_last_launches = 1;
      t_last_segments = static_cast<int>(cp.S);
      return RLCA_OK;
    }
  }
  const int64_t S = split_count(N, a.T);
  const bool split = S > 1 && w.ws != nullptr;
  if (split) {
    if (w.ws_bytes < 12 * N * S)
      return fail(RLCA_EINVAL,
                  "workspace_bytes = %lld is less than the %lld this call's split needs "
                  "(rlca_split_workspace_bytes)",
                  static_cast<long long>(w.ws_bytes), static_cast<long long>(12 * N * S));
    arrs[n++] = Arr{"workspace", w.ws, 3 * N * S, 3 * N * S, 4, false, true, true};
  }
  for (int i = 0; i < n; ++i) RLCA_TRY(check_array(arrs[i], N));
  RLCA_TRY(check_aliasing(arrs, n));
  a.cin = w.cin;
  a.cout = w.cout;
  a.cmap = w.cmap;
  if (!split) {
    RLCA_TRY(launch(algo, dtype, a, stream, w.on));
    t_last_launches = 1;
    t_last_segments = 1;
    return RLCA_OK;
  }

  float *const ws = static_cast<float *>(w.ws);
  float *maps = ws, *cins = ws + 2 * N * S;
  Args a1 = a;  // 1. maps only
  a1.T = a.T / S;
  a1.o0 = nullptr;
  a1.o1 = nullptr;
  a1.cin = nullptr;
  a1.cout = nullptr;
  a1.cmap = maps;
  RLCA_TRY(launch(algo, dtype, a1, stream, true, static_cast<int>(S)));
  // 2. compose, from the caller's carry_in
  bool forward = algo == kEligibility || algo == kCumsum || algo == kAffineFwd;
  const float *cmaps = maps, *init = w.cin;
  float *cout = w.cout, *cmap = w.cmap;
  int S32 = static_cast<int>(S);
  void *kargs[] = {&cmaps, &init, &cins, &S32, &forward, &cout, &cmap};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&compose_carries),
                                       dim3(static_cast<unsigned>(N)), dim3(64), kargs, 0,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RLCA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  Args a2 = a;  // 3. outputs
  a2.T = a.T / S;
  a2.cin = cins;
  a2.cout = nullptr;
  a2.cmap = nullptr;
  RLCA_TRY(launch(algo, dtype, a2, stream, true, static_cast<int>(S)));
  t_last_launches = 3;
  t_last_segments = S32;
  return RLCA_OK;
}

// The policy-table kernels: a 256-thread workgroup per row for long rows,
// one wavefront per row (four per workgroup) for rows of at most 256 steps;
// arguments by value.
int launch_probs(int algo, int dtype, const Args &args, const TableArgs &tables, void *stream,
                 bool window) {
  const int wpr = args.T <= kProbsShortRow ? 1 : 4;
  const void *kernel = probs_kernel_for(algo, dtype, wpr, window);
  if (kernel == nullptr) return fail(RLCA_EINVAL, "no policy-table kernel for algorithm %d", algo);
  Args a = args;
  TableArgs ta = tables;
#ifdef RLCA_TIMESTAMPS
  int stamp_dev = 0;
  RLCA_TRY(stamp_buffer(&stamp_dev, &a.stamps));
#endif
  const int64_t rows_per_block = 4 / wpr;
  const dim3 grid(static_cast<unsigned>((a.N + rows_per_block - 1) / rows_per_block));
  const dim3 block(kProbsBlock);
  void *kargs[] = {&a, &ta};
  const hipError_t e =
      hipLaunchKernel(kernel, grid, block, kargs, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RLCA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  t_last_variant = -1;
  t_last_launches = 1;
  t_last_segments = 1;
#ifdef RLCA_TIMESTAMPS
  t_last_waves = static_cast<int64_t>(grid.x) * (kProbsBlock / 64);
  t_last_device = stamp_dev;
#endif
  return RLCA_OK;
}

constexpr int64_t kMaxActions = 65536;

int check_actions(int64_t A) {
  if (A < 1 || A > kMaxActions)
    return fail(RLCA_EINVAL, "num_actions = %lld must lie in [1, %lld]", static_cast<long long>(A),
                static_cast<long long>(kMaxActions));
  return RLCA_OK;
}

int returns_impl(int64_t num_envs, int64_t T, int dtype, const void *rewards, int64_t ld_rewards,
                 const uint8_t *terminated, int64_t ld_terminated, const uint8_t *truncated,
                 int64_t ld_truncated, const void *trunc_values, int64_t ld_trunc_values,
                 const void *bootstrap, float gamma, float *returns, int64_t ld_returns,
                 const Window &w, void *stream) {
  RLCA_TRY(check_sizes(num_envs, T, dtype));
  RLCA_TRY(check_unit("gamma", gamma));
  if (truncated != nullptr && trunc_values == nullptr)
    return fail(RLCA_EINVAL, "truncated is given but trunc_values is NULL");
  const int64_t es = esize_of(dtype);
  const bool tv_used = truncated != nullptr;
  Arr arrs[6 + kExtraArrs] = {
      {"rewards", rewards, ld_rewards, T, es, true, false},
      {"terminated", terminated, ld_terminated, T, 1, false, false},
      {"truncated", truncated, ld_truncated, T, 1, false, false},
      {"trunc_values", tv_used ? trunc_values : nullptr, ld_trunc_values, T, es, false, false},
      {"bootstrap", bootstrap, num_envs, num_envs, es, false, false, true},
      {"returns", returns, ld_returns, T, 4, true, true},
  };
  Args a{};
  a.N = num_envs; a.T = T;
  a.r = rewards; a.ld_r = ld_rewards;
  a.tv = tv_used ? trunc_values : nullptr; a.ld_tv = ld_trunc_values;
  a.boot = bootstrap;
  a.term = terminated; a.ld_term = ld_terminated;
  a.trunc = truncated; a.ld_trunc = ld_truncated;
  a.o0 = returns; a.ld_o0 = ld_returns;
  a.gamma = gamma; a.lam = 1.f; a.rho_bar = a.c_bar = a.pg_rho_bar = 1.f;
  return validate_and_launch(kReturns, dtype, num_envs, arrs, 6, w, a, stream);
}

int gae_like(int algo, int64_t num_envs, int64_t T, int dtype, const void *rewards,
             int64_t ld_rewards, const void *values, int64_t ld_values,
             const uint8_t *terminated, int64_t ld_terminated, const uint8_t *truncated,
             int64_t ld_truncated, const void *trunc_values, int64_t ld_trunc_values,
             float gamma, float lam, float *out0, int64_t ld_out0, float *out1,
             int64_t ld_out1, const char *name0, const char *name1, const Window &w,
             void *stream) {
  RLCA_TRY(check_sizes(num_envs, T, dtype));
  RLCA_TRY(check_unit("gamma", gamma));
  RLCA_TRY(check_unit("lam", lam));
  if (truncated != nullptr && trunc_values == nullptr)
    return fail(RLCA_EINVAL, "truncated is given but trunc_values is NULL");
  const int64_t es = esize_of(dtype);
  const bool tv_used = truncated != nullptr;
  Arr arrs[7 + kExtraArrs] = {
      {"rewards", rewards, ld_rewards, T, es, true, false},
      {"values", values, ld_values, T + 1, es, true, false},
      {"terminated", terminated, ld_terminated, T, 1, false, false},
      {"truncated", truncated, ld_truncated, T, 1, false, false},
      {"trunc_values", tv_used ? trunc_values : nullptr, ld_trunc_values, T, es, false, false},
      {name0, out0, ld_out0, T, 4, true, true},
      {name1, out1, ld_out1, T, 4, false, true},
  };
  Args a{};
  a.N = num_envs; a.T = T;
  a.r = rewards; a.ld_r = ld_rewards;
  a.v = values; a.ld_v = ld_values;
  a.tv = tv_used ? trunc_values : nullptr; a.ld_tv = ld_trunc_values;
  a.term = terminated; a.ld_term = ld_terminated;
  a.trunc = truncated; a.ld_trunc = ld_truncated;
  a.o0 = out0; a.ld_o0 = ld_out0;
  a.o1 = out1; a.ld_o1 = ld_out1;
  a.gamma = gamma; a.lam = lam; a.rho_bar = a.c_bar = a.pg_rho_bar = 1.f;
  return validate_and_launch(algo, dtype, num_envs, arrs, 7, w, a, stream);
}

int vtrace_impl(int64_t num_envs, int64_t T, int dtype, const void *rewards, int64_t ld_rewards,
                const void *values, int64_t ld_values, const void *log_rhos,
                int64_t ld_log_rhos, const uint8_t *terminated, int64_t ld_terminated,
                const uint8_t *truncated, int64_t ld_truncated, const void *trunc_values,
                int64_t ld_trunc_values, float gamma, float lam, float rho_bar, float c_bar,
                float pg_rho_bar, float *vs, int64_t ld_vs, float *pg_advantages,
                int64_t ld_pg_advantages, const Window &w, void *stream) {
  RLCA_TRY(check_sizes(num_envs, T, dtype));
  RLCA_TRY(check_unit("gamma", gamma));
  RLCA_TRY(check_unit("lam", lam));
  RLCA_TRY(check_clip("rho_bar", rho_bar));
  RLCA_TRY(check_clip("c_bar", c_bar));
  RLCA_TRY(check_clip("pg_rho_bar", pg_rho_bar));
  if (truncated != nullptr && trunc_values == nullptr)
    return fail(RLCA_EINVAL, "truncated is given but trunc_values is NULL");
  const int64_t es = esize_of(dtype);
  const bool tv_used = truncated != nullptr;
  Arr arrs[8 + kExtraArrs] = {
      {"rewards", rewards, ld_rewards, T, es, true, false},
      {"values", values, ld_values, T + 1, es, true, false},
      {"log_rhos", log_rhos, ld_log_rhos, T, es, true, false},
      {"terminated", terminated, ld_terminated, T, 1, false, false},
      {"truncated", truncated, ld_truncated, T, 1, false, false},
      {"trunc_values", tv_used ? trunc_values : nullptr, ld_trunc_values, T, es, false, false},
      {"vs", vs, ld_vs, T, 4, true, true},
      {"pg_advantages", pg_advantages, ld_pg_advantages, T, 4, false, true},
  };
  Args a{};
  a.N = num_envs; a.T = T;
  a.r = rewards; a.ld_r = ld_rewards;
  a.v = values; a.ld_v = ld_values;
  a.lr = log_rhos; a.ld_lr = ld_log_rhos;
  a.tv = tv_used ? trunc_values : nullptr; a.ld_tv = ld_trunc_values;
  a.term = terminated; a.ld_term = ld_terminated;
  a.trunc = truncated; a.ld_trunc = ld_truncated;
  a.o0 = vs; a.ld_o0 = ld_vs;
  a.o1 = pg_advantages; a.ld_o1 = ld_pg_advantages;
  a.gamma = gamma; a.lam = lam; a.rho_bar = rho_bar; a.c_bar = c_bar; a.pg_rho_bar = pg_rho_bar;
  return validate_and_launch(kVtrace, dtype, num_envs, arrs, 8, w, a, stream);
}

int retrace_impl(int64_t num_envs, int64_t T, int dtype, const void *rewards, int64_t ld_rewards,
                 const void *q_taken, int64_t ld_q_taken, const void *exp_q_next,
                 int64_t ld_exp_q_next, const void *log_rhos, int64_t ld_log_rhos,
                 const uint8_t *terminated, int64_t ld_terminated, const uint8_t *truncated,
                 int64_t ld_truncated, float gamma, float lam, float c_bar, float *q_ret,
                 int64_t ld_q_ret, const Window &w, void *stream) {
  RLCA_TRY(check_sizes(num_envs, T, dtype));
  RLCA_TRY(check_unit("gamma", gamma));
  RLCA_TRY(check_unit("lam", lam));
  RLCA_TRY(check_clip("c_bar", c_bar));
  const int64_t es = esize_of(dtype);
  Arr arrs[7 + kExtraArrs] = {
      {"rewards", rewards, ld_rewards, T, es, true, false},
      {"q_taken", q_taken, ld_q_taken, T, es, true, false},
      {"exp_q_next", exp_q_next, ld_exp_q_next, T, es, true, false},
      {"log_rhos", log_rhos, ld_log_rhos, T, es, true, false},
      {"terminated", terminated, ld_terminated, T, 1, false, false},
      {"truncated", truncated, ld_truncated, T, 1, false, false},
      {"q_ret", q_ret, ld_q_ret, T, 4, true, true},
  };
  Args a{};
  a.N = num_envs; a.T = T;
  a.r = rewards; a.ld_r = ld_rewards;
  a.v = q_taken; a.ld_v = ld_q_taken;
  a.eq = exp_q_next; a.ld_eq = ld_exp_q_next;
  a.lr = log_rhos; a.ld_lr = ld_log_rhos;
  a.term = terminated; a.ld_term = ld_terminated;
  a.trunc = truncated; a.ld_trunc = ld_truncated;
  a.o0 = q_ret; a.ld_o0 = ld_q_ret;
  a.gamma = gamma; a.lam = lam; a.rho_bar = 1.f; a.c_bar = c_bar; a.pg_rho_bar = 1.f;
  return validate_and_launch(kRetrace, dtype, num_envs, arrs, 7, w, a, stream);
}

int forward_like(int algo, int64_t num_envs, int64_t T, int dtype, const void *x, int64_t ld_x,
                 const uint8_t *terminated, int64_t ld_terminated, const uint8_t *truncated,
                 int64_t ld_truncated, const void *init, float gamma, float lam, float *out,
                 int64_t ld_out, const char *init_name, const char *out_name, const Window &w,
                 void *stream) {
  RLCA_TRY(check_sizes(num_envs, T, dtype));
  RLCA_TRY(check_unit("gamma", gamma));
  RLCA_TRY(check_unit("lam", lam));
  const int64_t es = esize_of(dtype);
  Arr arrs[5 + kExtraArrs] = {
      {"x", x, ld_x, T, es, true, false},
      {"terminated", terminated, ld_terminated, T, 1, false, false},
      {"truncated", truncated, ld_truncated, T, 1, false, false},
      {init_name, init, num_envs, num_envs, es, false, false, true},
      {out_name, out, ld_out, T, 4, true, true},
  };
  Args a{};
  a.N = num_envs; a.T = T;
  a.r = x; a.ld_r = ld_x;
  a.boot = init;
  a.term = terminated; a.ld_term = ld_terminated;
  a.trunc = truncated; a.ld_trunc = ld_truncated;
  a.o0 = out; a.ld_o0 = ld_out;
  a.gamma = gamma; a.lam = lam; a.rho_bar = a.c_bar = a.pg_rho_bar = 1.f;
  return validate_and_launch(algo, dtype, num_envs, arrs, 5, w, a, stream);
}

int retrace_probs_impl(int64_t num_envs, int64_t T, int64_t num_actions, int dtype,
                       const void *rewards, int64_t ld_rewards, const void *q_values,
                       int64_t ld_q_values, const int32_t *actions, int64_t ld_actions,
                       const void *log_pi, int64_t ld_log_pi, const void *log_mu,
                       int64_t ld_log_mu, int log_mu_taken, const uint8_t *terminated,
                       int64_t ld_terminated, const uint8_t *truncated, int64_t ld_truncated,
                       const void *trunc_eq,
                       int64_t ld_trunc_eq, float gamma, float lam, float c_bar, float *q_ret,
                       int64_t ld_q_ret, const Window &w, void *stream) {
  RLCA_TRY(check_sizes(num_envs, T, dtype));
  RLCA_TRY(check_actions(num_actions));
  if (log_mu_taken != 0 && log_mu_taken != 1)
    return fail(RLCA_EINVAL, "log_mu_taken = %d must be 0 or 1", log_mu_taken);
  RLCA_TRY(check_unit("gamma", gamma));
  RLCA_TRY(check_unit("lam", lam));
  RLCA_TRY(check_clip("c_bar", c_bar));
  if (truncated != nullptr && trunc_eq == nullptr)
    return fail(RLCA_EINVAL, "truncated is given but trunc_eq is NULL");
  const int64_t es = esize_of(dtype);
  const int64_t A = num_actions;
  Arr arrs[12] = {
      {"rewards", rewards, ld_rewards, T, es, true, false},
      {"q_values", q_values, ld_q_values, (T + 1) * A, es, true, false},
      {"actions", actions, ld_actions, T, 4, true, false},
      {"log_pi", log_pi, ld_log_pi, (T + 1) * A, es, true, false},
      {"log_mu", log_mu, ld_log_mu, log_mu_taken ? T : T * A, es, true, false},
      {"terminated", terminated, ld_terminated, T, 1, false, false},
      {"truncated", truncated, ld_truncated, T, 1, false, false},
      {"trunc_eq", truncated != nullptr ? trunc_eq : nullptr, ld_trunc_eq, T, es, false, false},
      {"q_ret", q_ret, ld_q_ret, T, 4, true, true},
  };
  const int n = add_window(arrs, 9, w, num_envs);
  if (num_envs == 0) return RLCA_OK;
  for (int i = 0; i < n; ++i) RLCA_TRY(check_array(arrs[i], num_envs));
  RLCA_TRY(check_aliasing(arrs, n));
  Args a{};
  a.N = num_envs; a.T = T;
  a.r = rewards; a.ld_r = ld_rewards;
  a.term = terminated; a.ld_term = ld_terminated;
  a.trunc = truncated; a.ld_trunc = ld_truncated;
  a.o0 = q_ret; a.ld_o0 = ld_q_ret;
  a.gamma = gamma; a.lam = lam; a.rho_bar = 1.f; a.c_bar = c_bar; a.pg_rho_bar = 1.f;
  TableArgs ta{};
  ta.A = A;
  ta.q = q_values; ta.ld_q = ld_q_values;
  ta.act = actions; ta.ld_act = ld_actions;
  ta.lpi = log_pi; ta.ld_lpi = ld_log_pi;
  ta.lmu = log_mu; ta.ld_lmu = ld_log_mu;
  ta.mu_taken = log_mu_taken;
  ta.teq = truncated != nullptr ? trunc_eq : nullptr; ta.ld_teq = ld_trunc_eq;
  a.cin = w.cin; a.cout = w.cout; a.cmap = w.cmap;
  return launch_probs(kRetrace, dtype, a, ta, stream, w.on);
}

int vtrace_probs_impl(int64_t num_envs, int64_t T, int64_t num_actions, int dtype,
                      const void *rewards, int64_t ld_rewards, const void *values,
                      int64_t ld_values, const int32_t *actions, int64_t ld_actions,
                      const void *log_pi, int64_t ld_log_pi, const void *log_mu,
                      int64_t ld_log_mu, int log_mu_taken, const uint8_t *terminated,
                      int64_t ld_terminated, const uint8_t *truncated, int64_t ld_truncated,
                      const void *trunc_values,
                      int64_t ld_trunc_values, float gamma, float lam, float rho_bar,
                      float c_bar, float pg_rho_bar, float *vs, int64_t ld_vs,
                      float *pg_advantages, int64_t ld_pg_advantages, const Window &w,
                      void *stream) {
  RLCA_TRY(check_sizes(num_envs, T, dtype));
  RLCA_TRY(check_actions(num_actions));
  if (log_mu_taken != 0 && log_mu_taken != 1)
    return fail(RLCA_EINVAL, "log_mu_taken = %d must be 0 or 1", log_mu_taken);
  RLCA_TRY(check_unit("gamma", gamma));
  RLCA_TRY(check_unit("lam", lam));
  RLCA_TRY(check_clip("rho_bar", rho_bar));
  RLCA_TRY(check_clip("c_bar", c_bar));
  RLCA_TRY(check_clip("pg_rho_bar", pg_rho_bar));
  if (truncated != nullptr && trunc_values == nullptr)
    return fail(RLCA_EINVAL, "truncated is given but trunc_values is NULL");
  const int64_t es = esize_of(dtype);
  const int64_t A = num_actions;
  const bool tv_used = truncated != nullptr;
  Arr arrs[13] = {
      {"rewards", rewards, ld_rewards, T, es, true, false},
      {"values", values, ld_values, T + 1, es, true, false},
      {"actions", actions, ld_actions, T, 4, true, false},
      {"log_pi", log_pi, ld_log_pi, T * A, es, true, false},
      {"log_mu", log_mu, ld_log_mu, log_mu_taken ? T : T * A, es, true, false},
      {"terminated", terminated, ld_terminated, T, 1, false, false},
      {"truncated", truncated, ld_truncated, T, 1, false, false},
      {"trunc_values", tv_used ? trunc_values : nullptr, ld_trunc_values, T, es, false, false},
      {"vs", vs, ld_vs, T, 4, true, true},
      {"pg_advantages", pg_advantages, ld_pg_advantages, T, 4, false, true},
  };
  const int n = add_window(arrs, 10, w, num_envs);
  if (num_envs == 0) return RLCA_OK;
  for (int i = 0; i < n; ++i) RLCA_TRY(check_array(arrs[i], num_envs));
  RLCA_TRY(check_aliasing(arrs, n));
  Args a{};
  a.N = num_envs; a.T = T;
  a.r = rewards; a.ld_r = ld_rewards;
  a.v = values; a.ld_v = ld_values;
  a.tv = tv_used ? trunc_values : nullptr; a.ld_tv = ld_trunc_values;
  a.term = terminated; a.ld_term = ld_terminated;
  a.trunc = truncated; a.ld_trunc = ld_truncated;
  a.o0 = vs; a.ld_o0 = ld_vs;
  a.o1 = pg_advantages; a.ld_o1 = ld_pg_advantages;
  a.gamma = gamma; a.lam = lam; a.rho_bar = rho_bar; a.c_bar = c_bar; a.pg_rho_bar = pg_rho_bar;
  TableArgs ta{};
  ta.A = A;
  ta.act = actions; ta.ld_act = ld_actions;
  ta.lpi = log_pi; ta.ld_lpi = ld_log_pi;
  ta.lmu = log_mu; ta.ld_lmu = ld_log_mu;
  ta.mu_taken = log_mu_taken;
  a.cin = w.cin; a.cout = w.cout; a.cmap = w.cmap;
  return launch_probs(kVtrace, dtype, a, ta, stream, w.on);
}

// ------------------------------------------- the no-allocation entry point
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation) take a split call's
// workspace from this file-scope array instead of passing one, and always
// take the three-launch form: 3 floats per segment, room for every such
// split (at most kSplitMaxRows rows, fewer than 2 * kSplitTarget segments in
// all), 6 KB per device,
// held until the process ends.  In host code `scratch` only names the
// symbol; its address on a device comes from hipGetSymbolAddress, made once
// per device (scratch_on) and used for every kernel argument.
constexpr int64_t kScratchSegments = 2 * kSplitTarget;
constexpr int64_t kScratchFloats = 3 * kScratchSegments;
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float *g_scratch[kMaxDevices];  // the array's address on each device, once known

// The device a stream belongs to (the current device for the NULL stream).
int device_of(void *stream, int *dev) {
  hipError_t e;
  if (stream == nullptr) {
    e = hipGetDevice(dev);
  } else {
    hipDevice_t d = 0;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &d);
    *dev = static_cast<int>(d);
  }
  if (e != hipSuccess) return fail(RLCA_EHIP, "device of the stream: %s", hipGetErrorString(e));
  return RLCA_OK;
}

// The scratch array's address on the device of `stream`: looked up on the
// first call on that device, with that device current, then kept.
int scratch_on(void *stream, float **out) {
  int dev = 0;
  RLCA_TRY(device_of(stream, &dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RLCA_EINVAL, "device %d is beyond the %d devices the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    if (e != hipSuccess) return fail(RLCA_EHIP, "selecting device %d: %s", dev, hipGetErrorString(e));
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess || p == nullptr)
      return fail(RLCA_EHIP, "address of the scratch array on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch[dev] = static_cast<float *>(p);
  }
  *out = g_scratch[dev];
  return RLCA_OK;
}

Window window_of(const float *cin, float *cout, float *cmap, void *ws, int64_t ws_bytes) {
  return Window{true, cin, cout, cmap, ws, ws_bytes};
}

Window materialized_in(void *ws, int64_t ws_bytes) {
  return Window{false, nullptr, nullptr, nullptr, ws, ws_bytes, true};
}

}  // namespace
}  // namespace rlca

using namespace rlca;

extern "C" {

int rlca_returns(int64_t num_envs, int64_t T, int dtype, const void *rewards, int64_t ld_rewards,
                 const uint8_t *terminated, int64_t ld_terminated, const uint8_t *truncated,
                 int64_t ld_truncated, const void *trunc_values, int64_t ld_trunc_values,
                 const void *bootstrap, float gamma, float *returns, int64_t ld_returns,
                 void *stream) {
  return returns_impl(num_envs, T, dtype, rewards, ld_rewards, terminated, ld_terminated,
                      truncated, ld_truncated, trunc_values, ld_trunc_values, bootstrap, gamma,
                      returns, ld_returns, kNoWindow, stream);
}

int rlca_gae(int64_t num_envs, int64_t T, int dtype, const void *rewards, int64_t ld_rewards,
             const void *values, int64_t ld_values, const uint8_t *terminated,
             int64_t ld_terminated, const uint8_t *truncated, int64_t ld_truncated,
             const void *trunc_values, int64_t ld_trunc_values, float gamma, float lam,
             float *advantages, int64_t ld_advantages, float *targets, int64_t ld_targets,
             void *stream) {
  return gae_like(kGae, num_envs, T, dtype, rewards, ld_rewards, values, ld_values, terminated,
                  ld_terminated, truncated, ld_truncated, trunc_values, ld_trunc_values, gamma,
                  lam, advantages, ld_advantages, targets, ld_targets, "advantages", "targets",
                  kNoWindow, stream);
}

int rlca_td_lambda(int64_t num_envs, int64_t T, int dtype, const void *rewards,
                   int64_t ld_rewards, const void *values, int64_t ld_values,
                   const uint8_t *terminated, int64_t ld_terminated, const uint8_t *truncated,
                   int64_t ld_truncated, const void *trunc_values, int64_t ld_trunc_values,
                   float gamma, float lam, float *lambda_returns, int64_t ld_lambda_returns,
                   void *stream) {
  return gae_like(kTdLambda, num_envs, T, dtype, rewards, ld_rewards, values, ld_values,
                  terminated, ld_terminated, truncated, ld_truncated, trunc_values,
                  ld_trunc_values, gamma, lam, lambda_returns, ld_lambda_returns, nullptr, 0,
                  "lambda_returns", "unused", kNoWindow, stream);
}

int rlca_vtrace(int64_t num_envs, int64_t T, int dtype, const void *rewards, int64_t ld_rewards,
                const void *values, int64_t ld_values, const void *log_rhos,
                int64_t ld_log_rhos, const uint8_t *terminated, int64_t ld_terminated,
                const uint8_t *truncated, int64_t ld_truncated, const void *trunc_values,
                int64_t ld_trunc_values, float gamma, float lam, float rho_bar, float c_bar,
                float pg_rho_bar, float *vs, int64_t ld_vs, float *pg_advantages,
                int64_t ld_pg_advantages, void *stream) {
  return vtrace_impl(num_envs, T, dtype, rewards, ld_rewards, values, ld_values, log_rhos,
                     ld_log_rhos, terminated, ld_terminated, truncated, ld_truncated,
                     trunc_values, ld_trunc_values, gamma, lam, rho_bar, c_bar, pg_rho_bar, vs,
                     ld_vs, pg_advantages, ld_pg_advantages, kNoWindow, stream);
}

int rlca_retrace(int64_t num_envs, int64_t T, int dtype, const void *rewards, int64_t ld_rewards,
                 const void *q_taken, int64_t ld_q_taken, const void *exp_q_next,
                 int64_t ld_exp_q_next, const void *log_rhos, int64_t ld_log_rhos,
                 const uint8_t *terminated, int64_t ld_terminated, const uint8_t *truncated,
                 int64_t ld_truncated, float gamma, float lam, float c_bar, float *q_ret,
                 int64_t ld_q_ret, void *stream) {
  return retrace_impl(num_envs, T, dtype, rewards, ld_rewards, q_taken, ld_q_taken, exp_q_next,
                      ld_exp_q_next, log_rhos, ld_log_rhos, terminated, ld_terminated,
                      truncated, ld_truncated, gamma, lam, c_bar, q_ret, ld_q_ret, kNoWindow,
                      stream);
}

int rlca_eligibility_trace(int64_t num_envs, int64_t T, int dtype, const void *x, int64_t ld_x,
                           const uint8_t *terminated, int64_t ld_terminated,
                           const uint8_t *truncated, int64_t ld_truncated, const void *z_init,
                           float gamma, float lam, float *traces, int64_t ld_traces,
                           void *stream) {
  return forward_like(kEligibility, num_envs, T, dtype, x, ld_x, terminated, ld_terminated,
                      truncated, ld_truncated, z_init, gamma, lam, traces, ld_traces, "z_init",
                      "traces", kNoWindow, stream);
}

int rlca_episodic_cumsum(int64_t num_envs, int64_t T, int dtype, const void *x, int64_t ld_x,
                         const uint8_t *terminated, int64_t ld_terminated,
                         const uint8_t *truncated, int64_t ld_truncated, const void *s_init,
                         float *sums, int64_t ld_sums, void *stream) {
  return forward_like(kCumsum, num_envs, T, dtype, x, ld_x, terminated, ld_terminated, truncated,
                      ld_truncated, s_init, 1.f, 1.f, sums, ld_sums, "s_init", "sums", kNoWindow,
                      stream);
}

// ------------------------------------------ materialized doubling scan

int64_t rlca_materialized_workspace_bytes(int64_t num_envs, int64_t T) {
  if (num_envs < 0 || T < 1) {
    fail(RLCA_EINVAL, "num_envs must be >= 0 and T >= 1");
    return -1;
  }
  if (num_envs > 0 && num_envs > INT64_MAX / 16 / T) {
    fail(RLCA_EINVAL, "too many steps for the materialized scan");
    return -1;
  }
  return 16 * num_envs * T;
}

int rlca_returns_materialized(int64_t num_envs, int64_t T, int dtype, const void *rewards,
                              int64_t ld_rewards, const uint8_t *terminated,
                              int64_t ld_terminated, const uint8_t *truncated,
                              int64_t ld_truncated, const void *trunc_values,
                              int64_t ld_trunc_values, const void *bootstrap, float gamma,
                              float *returns, int64_t ld_returns, void *workspace,
                              int64_t workspace_bytes, void *stream) {
  return returns_impl(num_envs, T, dtype, rewards, ld_rewards, terminated, ld_terminated,
                      truncated, ld_truncated, trunc_values, ld_trunc_values, bootstrap, gamma,
                      returns, ld_returns, materialized_in(workspace, workspace_bytes), stream);
}

int rlca_gae_materialized(int64_t num_envs, int64_t T, int dtype, const void *rewards,
                          int64_t ld_rewards, const void *values, int64_t ld_values,
                          const uint8_t *terminated, int64_t ld_terminated,
                          const uint8_t *truncated, int64_t ld_truncated,
                          const void *trunc_values, int64_t ld_trunc_values, float gamma,
                          float lam, float *advantages, int64_t ld_advantages, float *targets,
                          int64_t ld_targets, void *workspace, int64_t workspace_bytes,
                          void *stream) {
  return gae_like(kGae, num_envs, T, dtype, rewards, ld_rewards, values, ld_values, terminated,
                  ld_terminated, truncated, ld_truncated, trunc_values, ld_trunc_values, gamma,
                  lam, advantages, ld_advantages, targets, ld_targets, "advantages", "targets",
                  materialized_in(workspace, workspace_bytes), stream);
}

int rlca_td_lambda_materialized(int64_t num_envs, int64_t T, int dtype, const void *rewards,
                                int64_t ld_rewards, const void *values, int64_t ld_values,
                                const uint8_t *terminated, int64_t ld_terminated,
                                const uint8_t *truncated, int64_t ld_truncated,
                                const void *trunc_values, int64_t ld_trunc_values, float gamma,
                                float lam, float *lambda_returns, int64_t ld_lambda_returns,
                                void *workspace, int64_t workspace_bytes, void *stream) {
  return gae_like(kTdLambda, num_envs, T, dtype, rewards, ld_rewards, values, ld_values,
                  terminated, ld_terminated, truncated, ld_truncated, trunc_values,
                  ld_trunc_values, gamma, lam, lambda_returns, ld_lambda_returns, nullptr, 0,
                  "lambda_returns", "unused", materialized_in(workspace, workspace_bytes),
                  stream);
}

int rlca_vtrace_materialized(int64_t num_envs, int64_t T, int dtype, const void *rewards,
                             int64_t ld_rewards, const void *values, int64_t ld_values,
                             const void *log_rhos, int64_t ld_log_rhos,
                             const uint8_t *terminated, int64_t ld_terminated,
                             const uint8_t *truncated, int64_t ld_truncated,
                             const void *trunc_values, int64_t ld_trunc_values, float gamma,
                             float lam, float rho_bar, float c_bar, float pg_rho_bar, float *vs,
                             int64_t ld_vs, float *pg_advantages, int64_t ld_pg_advantages,
                             void *workspace, int64_t workspace_bytes, void *stream) {
  return vtrace_impl(num_envs, T, dtype, rewards, ld_rewards, values, ld_values, log_rhos,
                     ld_log_rhos, terminated, ld_terminated, truncated, ld_truncated,
                     trunc_values, ld_trunc_values, gamma, lam, rho_bar, c_bar, pg_rho_bar, vs,
                     ld_vs, pg_advantages, ld_pg_advantages,
                     materialized_in(workspace, workspace_bytes), stream);
}

int rlca_retrace_materialized(int64_t num_envs, int64_t T, int dtype, const void *rewards,
                              int64_t ld_rewards, const void *q_taken, int64_t ld_q_taken,
                              const void *exp_q_next, int64_t ld_exp_q_next,
                              const void *log_rhos, int64_t ld_log_rhos,
                              const uint8_t *terminated, int64_t ld_terminated,
                              const uint8_t *truncated, int64_t ld_truncated, float gamma,
                              float lam, float c_bar, float *q_ret, int64_t ld_q_ret,
                              void *workspace, int64_t workspace_bytes, void *stream) {
  return retrace_impl(num_envs, T, dtype, rewards, ld_rewards, q_taken, ld_q_taken, exp_q_next,
                      ld_exp_q_next, log_rhos, ld_log_rhos, terminated, ld_terminated,
                      truncated, ld_truncated, gamma, lam, c_bar, q_ret, ld_q_ret,
                      materialized_in(workspace, workspace_bytes), stream);
}

// ------------------------------------------------------ window entry points
//
// `workspace` (nullable) enables the split of few long rows (see
// validate_and_launch); the plain entry points above never split.

int rlca_returns_chunk(int64_t num_envs, int64_t T, int dtype, const void *rewards,
                       int64_t ld_rewards, const uint8_t *terminated, int64_t ld_terminated,
                       const uint8_t *truncated, int64_t ld_truncated, const void *trunc_values,
                       int64_t ld_trunc_values, const float *carry_in, float gamma,
                       float *returns, int64_t ld_returns, float *carry_out, float *carry_map,
                       void *workspace, int64_t workspace_bytes, void *stream) {
  return returns_impl(num_envs, T, dtype, rewards, ld_rewards, terminated, ld_terminated,
                      truncated, ld_truncated, trunc_values, ld_trunc_values, nullptr, gamma,
                      returns, ld_returns,
                      window_of(carry_in, carry_out, carry_map, workspace, workspace_bytes),
                      stream);
}

int rlca_gae_chunk(int64_t num_envs, int64_t T, int dtype, const void *rewards,
                   int64_t ld_rewards, const void *values, int64_t ld_values,
                   const uint8_t *terminated, int64_t ld_terminated, const uint8_t *truncated,
                   int64_t ld_truncated, const void *trunc_values, int64_t ld_trunc_values,
                   float gamma, float lam, float *advantages, int64_t ld_advantages,
                   float *targets, int64_t ld_targets, const float *carry_in, float *carry_out,
                   float *carry_map, void *workspace, int64_t workspace_bytes, void *stream) {
  return gae_like(kGae, num_envs, T, dtype, rewards, ld_rewards, values, ld_values, terminated,
                  ld_terminated, truncated, ld_truncated, trunc_values, ld_trunc_values, gamma,
                  lam, advantages, ld_advantages, targets, ld_targets, "advantages", "targets",
                  window_of(carry_in, carry_out, carry_map, workspace, workspace_bytes), stream);
}

int rlca_gae_chunk_noalloc(int64_t num_envs, int64_t T, int dtype, const void *rewards,
                           int64_t ld_rewards, const void *values, int64_t ld_values,
                           const uint8_t *terminated, int64_t ld_terminated,
                           const uint8_t *truncated, int64_t ld_truncated,
                           const void *trunc_values, int64_t ld_trunc_values, float gamma,
                           float lam, float *advantages, int64_t ld_advantages, float *targets,
                           int64_t ld_targets, const float *carry_in, float *carry_out,
                           float *carry_map, void *stream) {
  RLCA_TRY(check_sizes(num_envs, T, dtype));
  // The library's scratch array replaces the caller's workspace, only for a
  // call that splits.
  float *ws = nullptr;
  const int64_t S = split_count(num_envs, T);
  if (num_envs > 0 && S > 1) {
    if (3 * num_envs * S > kScratchFloats)
      return fail(RLCA_EINVAL, "the split of %lld rows into %lld segments needs %lld bytes, more "
                  "than the %lld of the library's scratch array",
                  static_cast<long long>(num_envs), static_cast<long long>(S),
                  static_cast<long long>(12 * num_envs * S),
                  static_cast<long long>(4 * kScratchFloats));
    RLCA_TRY(scratch_on(stream, &ws));
  }
  // Always the three-launch form of a split (the scratch array is sized for
  // it).
  const int chained = t_chained;
  t_chained = 0;
  const int rc = gae_like(kGae, num_envs, T, dtype, rewards, ld_rewards, values, ld_values,
                          terminated, ld_terminated, truncated, ld_truncated, trunc_values,
                          ld_trunc_values, gamma, lam, advantages, ld_advantages, targets,
                          ld_targets, "advantages", "targets",
                          window_of(carry_in, carry_out, carry_map, ws, 4 * kScratchFloats),
                          stream);
  t_chained = chained;
  return rc;
}

int rlca_td_lambda_chunk(int64_t num_envs, int64_t T, int dtype, const void *rewards,
                         int64_t ld_rewards, const void *values, int64_t ld_values,
                         const uint8_t *terminated, int64_t ld_terminated,
                         const uint8_t *truncated, int64_t ld_truncated,
                         const void *trunc_values, int64_t ld_trunc_values, float gamma,
                         float lam, float *lambda_returns, int64_t ld_lambda_returns,
                         const float *carry_in, float *carry_out, float *carry_map,
                         void *workspace, int64_t workspace_bytes, void *stream) {
  return gae_like(kTdLambda, num_envs, T, dtype, rewards, ld_rewards, values, ld_values,
                  terminated, ld_terminated, truncated, ld_truncated, trunc_values,
                  ld_trunc_values, gamma, lam, lambda_returns, ld_lambda_returns, nullptr, 0,
                  "lambda_returns", "unused",
                  window_of(carry_in, carry_out, carry_map, workspace, workspace_bytes), stream);
}

int rlca_vtrace_chunk(int64_t num_envs, int64_t T, int dtype, const void *rewards,
                      int64_t ld_rewards, const void *values, int64_t ld_values,
                      const void *log_rhos, int64_t ld_log_rhos, const uint8_t *terminated,
                      int64_t ld_terminated, const uint8_t *truncated, int64_t ld_truncated,
                      const void *trunc_values, int64_t ld_trunc_values, float gamma, float lam,
                      float rho_bar, float c_bar, float pg_rho_bar, float *vs, int64_t ld_vs,
                      float *pg_advantages, int64_t ld_pg_advantages, const float *carry_in,
                      float *carry_out, float *carry_map, void *workspace,
                      int64_t workspace_bytes, void *stream) {
  return vtrace_impl(num_envs, T, dtype, rewards, ld_rewards, values, ld_values, log_rhos,
                     ld_log_rhos, terminated, ld_terminated, truncated, ld_truncated,
                     trunc_values, ld_trunc_values, gamma, lam, rho_bar, c_bar, pg_rho_bar, vs,
                     ld_vs, pg_advantages, ld_pg_advantages,
                     window_of(carry_in, carry_out, carry_map, workspace, workspace_bytes),
                     stream);
}

int rlca_retrace_chunk(int64_t num_envs, int64_t T, int dtype, const void *rewards,
                       int64_t ld_rewards, const void *q_taken, int64_t ld_q_taken,
                       const void *exp_q_next, int64_t ld_exp_q_next, const void *log_rhos,
                       int64_t ld_log_rhos, const uint8_t *terminated, int64_t ld_terminated,
                       const uint8_t *truncated, int64_t ld_truncated, float gamma, float lam,
                       float c_bar, float *q_ret, int64_t ld_q_ret, const float *carry_in,
                       float *carry_out, float *carry_map, void *workspace,
                       int64_t workspace_bytes, void *stream) {
  return retrace_impl(num_envs, T, dtype, rewards, ld_rewards, q_taken, ld_q_taken, exp_q_next,
                      ld_exp_q_next, log_rhos, ld_log_rhos, terminated, ld_terminated,
                      truncated, ld_truncated, gamma, lam, c_bar, q_ret, ld_q_ret,
                      window_of(carry_in, carry_out, carry_map, workspace, workspace_bytes),
                      stream);
}

int rlca_eligibility_trace_chunk(int64_t num_envs, int64_t T, int dtype, const void *x,
                                 int64_t ld_x, const uint8_t *terminated, int64_t ld_terminated,
                                 const uint8_t *truncated, int64_t ld_truncated,
                                 const float *carry_in, float gamma, float lam, float *traces,
                                 int64_t ld_traces, float *carry_out, float *carry_map,
                                 void *workspace, int64_t workspace_bytes, void *stream) {
  return forward_like(kEligibility, num_envs, T, dtype, x, ld_x, terminated, ld_terminated,
                      truncated, ld_truncated, nullptr, gamma, lam, traces, ld_traces, "z_init",
                      "traces",
                      window_of(carry_in, carry_out, carry_map, workspace, workspace_bytes),
                      stream);
}

int rlca_episodic_cumsum_chunk(int64_t num_envs, int64_t T, int dtype, const void *x,
                               int64_t ld_x, const uint8_t *terminated, int64_t ld_terminated,
                               const uint8_t *truncated, int64_t ld_truncated,
                               const float *carry_in, float *sums, int64_t ld_sums,
                               float *carry_out, float *carry_map, void *workspace,
                               int64_t workspace_bytes, void *stream) {
  return forward_like(kCumsum, num_envs, T, dtype, x, ld_x, terminated, ld_terminated, truncated,
                      ld_truncated, nullptr, 1.f, 1.f, sums, ld_sums, "s_init", "sums",
                      window_of(carry_in, carry_out, carry_map, workspace, workspace_bytes),
                      stream);
}

int rlca_affine_scan(int64_t num_envs, int64_t T, int dtype, const void *alpha,
                     int64_t ld_alpha, const void *beta, int64_t ld_beta, const uint8_t *reset,
                     int64_t ld_reset, int reverse, const float *carry_in, float *out,
                     int64_t ld_out, float *carry_out, float *carry_map, void *workspace,
                     int64_t workspace_bytes, void *stream) {
  RLCA_TRY(check_sizes(num_envs, T, dtype));
  if (reverse != 0 && reverse != 1)
    return fail(RLCA_EINVAL, "reverse = %d must be 0 or 1", reverse);
  const int64_t es = esize_of(dtype);
  Arr arrs[4 + kExtraArrs] = {
      {"alpha", alpha, ld_alpha, T, es, true, false},
      {"beta", beta, ld_beta, T, es, true, false},
      {"reset", reset, ld_reset, T, 1, false, false},
      {"out", out, ld_out, T, 4, true, true},
  };
  Args a{};
  a.N = num_envs; a.T = T;
  a.r = alpha; a.ld_r = ld_alpha;
  a.v = beta; a.ld_v = ld_beta;
  a.term = reset; a.ld_term = ld_reset;
  a.o0 = out; a.ld_o0 = ld_out;
  a.gamma = a.lam = a.rho_bar = a.c_bar = a.pg_rho_bar = 1.f;
  return validate_and_launch(reverse ? kAffine : kAffineFwd, dtype, num_envs, arrs, 4,
                             window_of(carry_in, carry_out, carry_map, workspace, workspace_bytes),
                             a, stream);
}

// ------------------------------------------------ policy-table entry points

int rlca_retrace_probs(int64_t num_envs, int64_t T, int64_t num_actions, int dtype,
                       const void *rewards, int64_t ld_rewards, const void *q_values,
                       int64_t ld_q_values, const int32_t *actions, int64_t ld_actions,
                       const void *log_pi, int64_t ld_log_pi, const void *log_mu,
                       int64_t ld_log_mu, int log_mu_taken, const uint8_t *terminated,
                       int64_t ld_terminated, const uint8_t *truncated, int64_t ld_truncated,
                       const void *trunc_eq, int64_t ld_trunc_eq, float gamma, float lam,
                       float c_bar, float *q_ret, int64_t ld_q_ret, void *stream) {
  return retrace_probs_impl(num_envs, T, num_actions, dtype, rewards, ld_rewards, q_values,
                            ld_q_values, actions, ld_actions, log_pi, ld_log_pi, log_mu,
                            ld_log_mu, log_mu_taken, terminated, ld_terminated, truncated,
                            ld_truncated, trunc_eq, ld_trunc_eq, gamma, lam, c_bar, q_ret,
                            ld_q_ret, kNoWindow, stream);
}

int rlca_vtrace_probs(int64_t num_envs, int64_t T, int64_t num_actions, int dtype,
                      const void *rewards, int64_t ld_rewards, const void *values,
                      int64_t ld_values, const int32_t *actions, int64_t ld_actions,
                      const void *log_pi, int64_t ld_log_pi, const void *log_mu,
                      int64_t ld_log_mu, int log_mu_taken, const uint8_t *terminated,
                      int64_t ld_terminated, const uint8_t *truncated, int64_t ld_truncated,
                      const void *trunc_values, int64_t ld_trunc_values, float gamma, float lam,
                      float rho_bar, float c_bar, float pg_rho_bar, float *vs, int64_t ld_vs,
                      float *pg_advantages, int64_t ld_pg_advantages, void *stream) {
  return vtrace_probs_impl(num_envs, T, num_actions, dtype, rewards, ld_rewards, values, ld_values,
                           actions, ld_actions, log_pi, ld_log_pi, log_mu, ld_log_mu,
                           log_mu_taken, terminated, ld_terminated, truncated, ld_truncated,
                           trunc_values, ld_trunc_values, gamma, lam, rho_bar, c_bar, pg_rho_bar,
                           vs, ld_vs, pg_advantages, ld_pg_advantages, kNoWindow, stream);
}

int rlca_retrace_probs_chunk(int64_t num_envs, int64_t T, int64_t num_actions, int dtype,
                             const void *rewards, int64_t ld_rewards, const void *q_values,
                             int64_t ld_q_values, const int32_t *actions, int64_t ld_actions,
                             const void *log_pi, int64_t ld_log_pi, const void *log_mu,
                             int64_t ld_log_mu, int log_mu_taken, const uint8_t *terminated,
                             int64_t ld_terminated, const uint8_t *truncated,
                             int64_t ld_truncated, const void *trunc_eq, int64_t ld_trunc_eq,
                             float gamma, float lam, float c_bar, float *q_ret,
                             int64_t ld_q_ret, const float *carry_in, float *carry_out,
                             float *carry_map, void *stream) {
  return retrace_probs_impl(num_envs, T, num_actions, dtype, rewards, ld_rewards, q_values,
                            ld_q_values, actions, ld_actions, log_pi, ld_log_pi, log_mu,
                            ld_log_mu, log_mu_taken, terminated, ld_terminated, truncated,
                            ld_truncated, trunc_eq, ld_trunc_eq, gamma, lam, c_bar, q_ret,
                            ld_q_ret, Window{true, carry_in, carry_out, carry_map}, stream);
}

int rlca_vtrace_probs_chunk(int64_t num_envs, int64_t T, int64_t num_actions, int dtype,
                            const void *rewards, int64_t ld_rewards, const void *values,
                            int64_t ld_values, const int32_t *actions, int64_t ld_actions,
                            const void *log_pi, int64_t ld_log_pi, const void *log_mu,
                            int64_t ld_log_mu, int log_mu_taken, const uint8_t *terminated,
                            int64_t ld_terminated, const uint8_t *truncated,
                            int64_t ld_truncated, const void *trunc_values,
                            int64_t ld_trunc_values, float gamma, float lam, float rho_bar,
                            float c_bar, float pg_rho_bar, float *vs, int64_t ld_vs,
                            float *pg_advantages, int64_t ld_pg_advantages,
                            const float *carry_in, float *carry_out, float *carry_map,
                            void *stream) {
  return vtrace_probs_impl(num_envs, T, num_actions, dtype, rewards, ld_rewards, values, ld_values,
                           actions, ld_actions, log_pi, ld_log_pi, log_mu, ld_log_mu,
                           log_mu_taken, terminated, ld_terminated, truncated, ld_truncated,
                           trunc_values, ld_trunc_values, gamma, lam, rho_bar, c_bar, pg_rho_bar,
                           vs, ld_vs, pg_advantages, ld_pg_advantages,
                           Window{true, carry_in, carry_out, carry_map}, stream);
}

const char *rlca_last_error(void) { return t_last_error.c_str(); }

// 0.5.0: T < 1 is an error; the split calls' workspace is an argument of the
// window calls (no per-thread workspace).  0.5.1: split calls in one pass (the
// chained form), rlca_set_chained, rlca_last_launches.  0.5.2: the chained
// form in one launch (its last workgroup advances the epoch), rlca_last_segments.
int rlca_version(void) { return 520; }

int rlca_split_segments(int64_t num_envs, int64_t T) {
  if (num_envs < 0 || T < 1) {
    fail(RLCA_EINVAL, "num_envs must be >= 0 and T >= 1");
    return -1;
  }
  return static_cast<int>(split_count(num_envs, T));
}

int64_t rlca_split_workspace_bytes(int64_t num_envs, int64_t T) {
  if (num_envs < 0 || T < 1) {
    fail(RLCA_EINVAL, "num_envs must be >= 0 and T >= 1");
    return -1;
  }
  return split_workspace_bytes(num_envs, T);
}

int rlca_timestamps(uint64_t *dst, int64_t max_waves, int64_t *waves) {
#ifdef RLCA_TIMESTAMPS
  if (dst == nullptr || waves == nullptr || max_waves < 0)
    return fail(RLCA_EINVAL, "dst and waves must not be NULL, max_waves >= 0");
  int dev = 0;
  uint64_t *buf = nullptr;
  RLCA_TRY(stamp_buffer(&dev, &buf));
  if (dev != t_last_device) return fail(RLCA_EINVAL, "the last launch ran on another device");
  int64_t n = t_last_waves < kStampWaves ? t_last_waves : kStampWaves;
  if (n > max_waves) n = max_waves;
  const hipError_t e = hipMemcpy(dst, buf, static_cast<size_t>(2 * n) * sizeof(uint64_t),
                                 hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(RLCA_EHIP, "reading the stamps: %s", hipGetErrorString(e));
  *waves = n;
  return RLCA_OK;
#else
  (void)dst;
  (void)max_waves;
  if (waves != nullptr) *waves = 0;
  return fail(RLCA_EINVAL, "this build records no timestamps (the instrumented build does)");
#endif
}

int rlca_num_variants(void) { return kNumVariants; }

int rlca_set_variant(int variant) {
  if (variant < -1 || variant >= kNumVariants) return -2;
  const int prev = t_forced_variant;
  t_forced_variant = variant;
  return prev;
}

int rlca_variant_info(int variant, int algo, int dtype, int *steps_per_lane_out,
                      int *lanes_per_row, int *waves_per_row) {
  if (variant < 0 || variant >= kNumVariants)
    return fail(RLCA_EINVAL, "unknown variant %d", variant);
  if (algo < RLCA_ALGO_RETURNS || algo > RLCA_ALGO_AFFINE)
    return fail(RLCA_EINVAL, "unknown algorithm %d", algo);
  if (dtype != RLCA_F32 && dtype != RLCA_BF16) return fail(RLCA_EDTYPE, "unknown dtype %d", dtype);
  const Variant v = kVariants[variant];
  if (steps_per_lane_out)
    *steps_per_lane_out = steps_per_lane(v, dtype == RLCA_BF16, algo == RLCA_ALGO_VTRACE);
  if (lanes_per_row) *lanes_per_row = v.WPR > 1 ? 64 * v.WPR : v.LPR;
  if (waves_per_row) *waves_per_row = v.WPR;
  return RLCA_OK;
}

int rlca_last_variant(void) { return t_last_variant; }

int rlca_set_chained(int enable) {
  const int prev = t_chained;
  t_chained = enable != 0;
  return prev;
}

int rlca_last_launches(void) { return t_last_launches; }

int rlca_last_segments(void) { return t_last_segments; }

}  // extern "C"
