// scan_kernels.hpp -- gfx950 (CDNA4) kernels for reverse-time affine
// recurrences A_t = alpha_t + beta_t * A_{t+1} over [num_envs, T] rollouts.
//
// Source: the rl-triton explainer pages ("rl-triton: High-Performance Triton
// GPU Kernels for Reinforcement Learning Credit Assignment", Zehnder 2026),
// Technical summary:
//   Method 1  every algorithm is an instance of the recurrence above and is
//             evaluated as an associative scan over (alpha_t, beta_t) with
//             (a_B, b_B) (+) (a_A, b_A) = (a_B + b_B a_A, b_A b_B), B earlier;
//   Method 2  the pairs are built from the raw rollout in registers, scanned
//             on chip, and only the final outputs are written (one read and
//             one write of HBM per element);
//   Method 3  termination zeroes the successor value, truncation bootstraps
//             from a supplied value, both cut the trace; the window bootstrap
//             enters alpha_{T-1} or the carry A_T, never both.
//
// Mapping onto CDNA4 (64-lane wavefronts):
//   * A row is processed in tiles of kTile = kGroup * K steps, where kGroup
//     lanes share the row: LPR lanes of one wavefront (16, 32 or 64), or WPR
//     whole wavefronts of a workgroup.  Tiles are aligned to the row start
//     and visited from the last one (latest in time) to the first, carrying
//     the scalar A at the tile boundary.
//   * Lane g of the group owns the K consecutive steps
//     [tile_start + (kGroup-1-g)*K, +K): lane order is the REVERSE of time
//     order, so the upward DPP prefix scan (row_shr, row_bcast) computes the
//     time-suffix composite that a reverse recurrence needs.  Memory access
//     stays coalesced: a wavefront still reads one contiguous span.
//   * Per lane: vector loads of its K steps (4-byte aligned dwordx4 loads;
//     bf16 and uint8 rows of any alignment are read as aligned dwords and
//     realigned in registers), (alpha, beta) built in VGPRs, folded
//     sequentially (K-1 FMAs), then log2(LPR) DPP levels of the operator
//     across lanes (two DPP instructions each), then (WPR > 1) one LDS
//     exchange of per-wavefront aggregates, scanned across lanes.  Each lane
//     then re-runs its K steps from its incoming value and writes the fused
//     outputs with vector stores.
//   * HBM traffic is one read of every input element the method uses (plus
//     the V_{t+1} / log_rho_{t+1} neighbour, which hits in cache) and one
//     write of every output element.  No intermediate touches HBM.
//   * Window instances (kChunk): the carry entering the window is read from a
//     per-row vector, and the row's outgoing carry and the affine map from
//     the incoming to the outgoing carry (the composite of every step, kept
//     beside the scalar carry from tile to tile) are written per row, so that
//     consecutive windows of one rollout chain exactly (Method 3, rollout
//     windows; the operator is associative).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "variants.hpp"

namespace rlca {

using bf16_t = uint16_t;  // raw bfloat16 bits

// Everything a launch needs, passed by value in the kernel argument segment.
// Row pointers are byte-exact device addresses; ld_* are row strides in
// elements.  Field use per algorithm:
//   r      rewards [N,T]                                  (all)
//   v      values [N,T+1] (gae, td_lambda, vtrace) or q_taken [N,T] (retrace)
//   lr     log importance ratios [N,T]                    (vtrace, retrace)
//   eq     E_pi Q(s_{t+1}, .) [N,T]                        (retrace)
//   tv     truncation bootstrap values [N,T], nullable    (not retrace)
//   boot   window bootstrap [N], nullable                 (returns)
//   o0     returns | advantages | lambda returns | vs | q_ret
//   o1     targets (gae) | pg advantages (vtrace), nullable
// Generic scan: r = alpha, v = beta [N,T], term = reset flags, o0 = A.
// Window instances only: cin [N] incoming carry (nullable: 0), cout [N]
// outgoing carry, cmap [N,2] carry map, both nullable.
struct Args {
  int64_t N, T;
  const void *r;  int64_t ld_r;
  const void *v;  int64_t ld_v;
  const void *lr; int64_t ld_lr;
  const void *eq; int64_t ld_eq;
  const void *tv; int64_t ld_tv;
  const void *boot;
  const uint8_t *term;  int64_t ld_term;
  const uint8_t *trunc; int64_t ld_trunc;
  float *o0; int64_t ld_o0;
  float *o1; int64_t ld_o1;
  float gamma, lam, rho_bar, c_bar, pg_rho_bar;
  const float *cin;
  float *cout;
  float *cmap;
  int seg_count = 1;  // window instances: segments per row (gridDim.y; 1 unless split)
  // Chained instances (split calls in one pass, see chain_lookback): the
  // workspace, its epoch word (the previous call's tag) followed by the segments'
  // published carry maps, 4 words per (row, segment).
  unsigned long long *chain = nullptr;
#ifdef RLCA_TIMESTAMPS
  uint64_t *stamps;   // instrumented build: per-wavefront wall-clock stamps
#endif
};

#ifdef RLCA_TIMESTAMPS
// Instrumented build only (compiled with -DRLCA_TIMESTAMPS into a library of
// its own, never the product library): every wavefront of a scan kernel
// records the 100 MHz wall clock at entry and again once all of its loads and
// stores have completed, as (start, end) at stamps[2 * w], w the wavefront's
// index in the launch (the first kStampWaves wavefronts only).  The launch's
// duration on the GPU is then max(end) - min(start), without the runtime's
// per-launch cost around it.
constexpr int64_t kStampWaves = 1 << 16;

__device__ __forceinline__ uint64_t wall_clock() { return __builtin_amdgcn_s_memrealtime(); }

// Taken at a kernel's entry; its destructor, run at every return, waits for
// the wavefront's loads and stores and records both stamps.
struct WaveStamp {
  uint64_t *stamps;
  uint64_t start;
  __device__ ~WaveStamp() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);  // every load and store of this wavefront done
    const uint64_t end = wall_clock();
    const int waves = static_cast<int>(blockDim.x) >> 6;
    const int64_t w = (static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x) * waves +
                      (threadIdx.x >> 6);
    if ((threadIdx.x & 63) == 0 && w < kStampWaves) {
      stamps[2 * w] = start;
      stamps[2 * w + 1] = end;
    }
  }
};
#endif

// Hot streams: the (up to) five arrays each algorithm reads at the start of a
// tile.  They are passed again as leading scalar kernel arguments h0..h4,
// with N, T and two row strides, 14 dwords that the dispatcher preloads into
// SGPRs: a wavefront issues its loads without first fetching the argument
// block from memory.
//   returns:        h = r, term, trunc, trunc_values, bootstrap
//   gae, td_lambda: h = r, v, term, trunc, trunc_values
//   vtrace:         h = r, v, log_rho, term, trunc     (trunc_values cold)
//   retrace:        h = r, q, eq, log_rho, term        (trunc cold)
//   eligibility, cumsum: h = x (in r), term, trunc, initial carry [N], -
//   affine (both directions): h = alpha, beta, reset, -, -
// ldT is the common row stride of the hot [N,T] streams, ldX the stride of
// values (gae, td_lambda, vtrace) or 1 if truncation flags are given
// (retrace).  When the hot [N,T] streams do not share one stride, the
// kUniform = false instances take every stride from Args instead.

// Batches of at most this many env-steps read trunc_values as whole vectors
// with the other loads, instead of a dependent load at truncated steps after
// the flags arrive: at that size the kernel is latency bound and the extra
// bytes cost less than the extra memory round trip.  The host decides (for
// the whole call, split or not) and passes the hot bootstrap pointer only
// for dense reads; sparse reads take the bootstraps' own pointer from Args.
#ifndef RLCA_DENSE_TV_MAX_STEPS
#define RLCA_DENSE_TV_MAX_STEPS (int64_t(1) << 20)
#endif
constexpr int64_t kDenseTvMaxSteps = RLCA_DENSE_TV_MAX_STEPS;

// ------------------------------------------------------------------ loads

struct __attribute__((aligned(4))) F4 { float x, y, z, w; };
struct __attribute__((aligned(4))) U4 { uint32_t x, y, z, w; };
struct __attribute__((aligned(4))) U2 { uint32_t x, y; };
// Four floats with 4-byte alignment, for non-temporal vector stores.
typedef float V4 __attribute__((ext_vector_type(4), aligned(4)));

// ND consecutive dwords from a 4-byte aligned address, as dwordx4/x2/x1 loads.
// Vector types for the loads below (4-byte alignment is all they assume).
typedef uint32_t NU4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t NU2 __attribute__((ext_vector_type(2), aligned(4)));
typedef float NF4 __attribute__((ext_vector_type(4), aligned(4)));

// kNT: non-temporal loads, for streams that nothing reads again (flags, the
// truncation bootstraps, Retrace's expectations, the policy tables, and the
// values where V_{t0+K} comes from the neighbouring lane).  The rewards,
// log-ratios and otherwise the values stay ordinary loads: the step-(t0+K)
// neighbour of values and log-ratios, and a missing flag array's stand-in
// (the lane's own reward bytes), re-read lines they bring in, and measured
// slower (TD(lambda) 16384x256 +5%) when those streams were non-temporal too.
template <int ND, bool kNT = false>
__device__ __forceinline__ void ld_dwords(const uint32_t *__restrict__ p, uint32_t (&d)[ND]) {
#pragma unroll
  for (int i = 0; i + 4 <= ND; i += 4) {
    NU4 q;
    if constexpr (kNT) q = __builtin_nontemporal_load(reinterpret_cast<const NU4 *>(p + i));
    else q = *reinterpret_cast<const NU4 *>(p + i);
    d[i] = q.x; d[i + 1] = q.y; d[i + 2] = q.z; d[i + 3] = q.w;
  }
  constexpr int done4 = ND / 4 * 4;
  if constexpr (ND - done4 >= 2) {
    NU2 q;
    if constexpr (kNT) q = __builtin_nontemporal_load(reinterpret_cast<const NU2 *>(p + done4));
    else q = *reinterpret_cast<const NU2 *>(p + done4);
    d[done4] = q.x; d[done4 + 1] = q.y;
  }
  if constexpr ((ND - done4) % 2 == 1) {
    if constexpr (kNT) d[ND - 1] = __builtin_nontemporal_load(p + ND - 1);
    else d[ND - 1] = p[ND - 1];
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename InT> struct Ld;

template <> struct Ld<float> {
  // K consecutive values at p (K % 4 == 0; p 4-byte aligned): K/4 dwordx4.
  template <int K, bool kNT = false>
  static __device__ __forceinline__ void vec(const float *__restrict__ p, float (&x)[K]) {
    static_assert(K % 4 == 0, "K must be a multiple of 4");
#pragma unroll
    for (int i = 0; i < K / 4; ++i) {
      NF4 q;
      if constexpr (kNT) q = __builtin_nontemporal_load(reinterpret_cast<const NF4 *>(p) + i);
      else q = reinterpret_cast<const NF4 *>(p)[i];
      x[4 * i] = q.x; x[4 * i + 1] = q.y; x[4 * i + 2] = q.z; x[4 * i + 3] = q.w;
    }
  }
  static __device__ __forceinline__ float one(const float *p) { return *p; }
};

template <> struct Ld<bf16_t> {
  // K consecutive bf16 values at p (K % 4 == 0; p 2-byte aligned).  Reads the
  // K/2 dwords starting at the dword that holds p[0], plus one more dword:
  // the one holding p[K-1] when p is odd-aligned (it is then the dword after
  // the K/2), else the last of the K/2 again.  Every dword read holds a
  // requested element, and there is no branch.
  template <int K, bool kNT = false>
  static __device__ __forceinline__ void vec(const bf16_t *__restrict__ p, float (&x)[K]) {
    static_assert(K % 4 == 0, "K must be a multiple of 4");
    const int odd = static_cast<int>((reinterpret_cast<uintptr_t>(p) >> 1) & 1);
    const uint32_t *base = reinterpret_cast<const uint32_t *>(p - odd);
    uint32_t d[K / 2];
    ld_dwords<K / 2, kNT>(base, d);
    const uint32_t extra = base[K / 2 - 1 + odd];
    // In the byte pair {dn : da} (da = dword e/2 in bytes 0-3, dn = the next
    // dword in bytes 4-7), element e starts at byte 2 * ((e & 1) + odd).
    // One v_perm_b32 moves its two bytes to the top half of the result and
    // zeros the bottom half (selector byte 0x0c), which is the element as a
    // float.
    const uint32_t sel_even = odd ? 0x03020c0cu : 0x01000c0cu;
    const uint32_t sel_odd = odd ? 0x05040c0cu : 0x03020c0cu;
#pragma unroll
    for (int e = 0; e < K; ++e) {
      const uint32_t da = d[e / 2];
      const uint32_t dn = e / 2 + 1 < K / 2 ? d[e / 2 + 1] : extra;
      x[e] = __uint_as_float(__builtin_amdgcn_perm(dn, da, (e & 1) ? sel_odd : sel_even));
    }
  }
  static __device__ __forceinline__ float one(const bf16_t *p) {
    return __uint_as_float(static_cast<uint32_t>(*p) << 16);
  }
};

// K flag bytes at p (any alignment), loaded as raw dwords and realigned
// later (decode), so the loads of a tile are all in flight before any use.
// Same rule as the bf16 loader: K/4 dwords from the dword holding p[0], plus
// the dword holding p[K-1] (a repeat of the last one when p is 4-byte
// aligned).  After decode, byte j of the span is bits [8*(j%4), +8) of w[j/4].
template <int K>
struct FlagWords {
  uint32_t d[K / 4];
  uint32_t extra;
  uint32_t sh;  // misalignment of p in bytes (0-3)
};

// kAligned: p is known to be 4-byte aligned (every flag row of the call is),
// so the span is exactly its K/4 dwords and no further dword is read.
template <int K, bool kAligned = false>
__device__ __forceinline__ void ld_flags_raw(const uint8_t *__restrict__ p, FlagWords<K> &f) {
  static_assert(K % 4 == 0, "K must be a multiple of 4");
  if constexpr (kAligned) {
    ld_dwords<K / 4, true>(reinterpret_cast<const uint32_t *>(p), f.d);
    f.extra = f.d[K / 4 - 1];
    f.sh = 0;
  } else {
    const int mis = static_cast<int>(reinterpret_cast<uintptr_t>(p) & 3);
    const uint32_t *base = reinterpret_cast<const uint32_t *>(p - mis);
    ld_dwords<K / 4, true>(base, f.d);
    f.extra = base[K / 4 - 1 + (mis != 0)];
    f.sh = static_cast<uint32_t>(mis);
  }
}

// Each output dword is the byte pair {hi : lo} moved down by the misalignment,
// one v_alignbyte_b32.  (A 64-bit shift, v_lshrrev_b64, does the same, but
// with its shift amount in the last VGPR of a kernel's allocation it has
// decoded the flags of some wavefronts of 512-thread workgroups unshifted,
// now and then; the byte align takes no such operand pair.)
template <int K>
__device__ __forceinline__ void decode_flags(const FlagWords<K> &f, uint32_t (&w)[K / 4]) {
#pragma unroll
  for (int i = 0; i < K / 4; ++i) {
    const uint32_t hi = i + 1 < K / 4 ? f.d[i + 1] : f.extra;
    w[i] = __builtin_amdgcn_alignbyte(hi, f.d[i], f.sh);
  }
}

template <int K>
__device__ __forceinline__ bool flag(const uint32_t (&w)[K / 4], int j) {
  return ((w[j >> 2] >> ((j & 3) * 8)) & 0xffu) != 0;
}

// Element-wise predicated loads (e < lim) for the ragged last tile of a row.
template <typename InT, int K>
__device__ __forceinline__ void ld_part(const InT *__restrict__ p, int64_t lim, float (&x)[K]) {
#pragma unroll
  for (int e = 0; e < K; ++e) x[e] = e < lim ? Ld<InT>::one(p + e) : 0.f;
}

template <int K>
__device__ __forceinline__ void ld_flags_part(const uint8_t *__restrict__ p, int64_t lim,
                                              uint32_t (&w)[K / 4]) {
#pragma unroll
  for (int i = 0; i < K / 4; ++i) w[i] = 0;
#pragma unroll
  for (int e = 0; e < K; ++e)
    if (e < lim && p[e] != 0) w[e >> 2] |= 1u << ((e & 3) * 8);
}

// ------------------------------------------------------- cross-lane scan

// Value of `src` in the lane selected by the DPP control CTRL (rows enabled by
// ROW_MASK); lanes without a valid source, or in disabled rows, get `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float src, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src),
                                                     CTRL, ROW_MASK, 0xf, false));
}

// One Hillis-Steele level of the affine operator: this lane (earlier in time)
// composes with the aggregate of a lower lane (later in time):
//   (a, b) <- (a + b * a_src, b * b_src).
// Two DPP instructions: v_fmac_f32_dpp (a += a_src * b) and v_mul_f32_dpp
// (b *= b_src).  Without bound_ctrl a lane whose source is outside its row
// (or in a row the mask leaves out) is not written, which is exactly the
// identity (0, 1).  The compiler's hazard check does not see into asm, so the
// block starts with the two wait states a DPP read needs after a VALU write
// of its source; the second DPP read (of b) follows its last write by three.
#define RLCA_SCAN_LEVEL(a, b, CTRL, ROW_MASK)                                          \
  asm("s_nop 1\n\t"                                                                \
      "v_fmac_f32_dpp %0, %0, %1 " CTRL " row_mask:" ROW_MASK " bank_mask:0xf\n\t"   \
      "v_mul_f32_dpp %1, %1, %1 " CTRL " row_mask:" ROW_MASK " bank_mask:0xf"          \
      : "+v"(a), "+v"(b))

// Inclusive scan over aligned groups of LANES lanes (4, 8, 16, 32 or 64):
// afterwards lane i holds f_i o f_{i-1} o ... o f_{group start}.
template <int LANES>
__device__ __forceinline__ void group_scan(float &a, float &b) {
  static_assert(LANES == 4 || LANES == 8 || LANES == 16 || LANES == 32 || LANES == 64,
                "group of 4, 8, 16, 32 or 64 lanes");
  RLCA_SCAN_LEVEL(a, b, "row_shr:1", "0xf");
  RLCA_SCAN_LEVEL(a, b, "row_shr:2", "0xf");
  if constexpr (LANES >= 8) RLCA_SCAN_LEVEL(a, b, "row_shr:4", "0xf");
  if constexpr (LANES >= 16) RLCA_SCAN_LEVEL(a, b, "row_shr:8", "0xf");
  if constexpr (LANES >= 32) RLCA_SCAN_LEVEL(a, b, "row_bcast:15", "0xa");  // -> rows 1, 3
  if constexpr (LANES >= 64) RLCA_SCAN_LEVEL(a, b, "row_bcast:31", "0xc");  // -> rows 2, 3
}

__device__ __forceinline__ float readlane(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

__device__ __forceinline__ float lane_shuffle(float x, int src_lane) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(x)));
}

// ------------------------------------------------------------------ kernel

// Pin a value to this point of the program: nothing computed from the
// result can be hoisted above the (empty, volatile) asm statement.  Applied
// to kernel-argument scalars (late) and to the per-lane row index (late_v)
// where a cold argument is first used, so that the scalar loads of the
// argument block may be issued early but are waited for only after the
// tile's vector loads are in flight.  Pointers are never passed through the
// barrier, so they keep their global address space.
template <typename V>
__device__ __forceinline__ V late(V x) {
  asm volatile("" : "+s"(x));
  return x;
}

__device__ __forceinline__ int64_t late_v(int64_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// A row index pinned the same way, in scalar registers when the whole
// workgroup shares the row (kU: rows of whole wavefronts), so that the
// addresses formed from it stay scalar.
template <bool kU>
__device__ __forceinline__ int64_t late_row(int64_t x) {
  if constexpr (kU) return late(x);
  else return late_v(x);
}

template <int A> struct Uses {
  static constexpr bool forward = A == kEligibility || A == kCumsum || A == kAffineFwd;
  // Reset by the flags of the step before (an episode that ended after step
  // t-1 restarts at t); the generic scan uses the flag of the step itself.
  static constexpr bool prev_flags = A == kEligibility || A == kCumsum;
  static constexpr bool affine = A == kAffine || A == kAffineFwd;  // beta [N,T] in v
  static constexpr bool values = A == kGae || A == kTdLambda || A == kVtrace;  // V [N,T+1]
  static constexpr bool q = A == kRetrace;
  static constexpr bool log_rho = A == kVtrace || A == kRetrace;
  static constexpr bool tv = A == kReturns || A == kGae || A == kTdLambda || A == kVtrace;
  static constexpr bool two_outputs = A == kGae || A == kVtrace;
};

// Row pointers of the hot streams; the cold ones (outputs, and the arrays
// marked cold above) are formed from Args at their first use (see late()).
template <typename InT>
struct RowPtrs {
  const InT *r, *v, *lr, *eq, *tv;
  const uint8_t *te, *tr;
  bool has_te, has_tr, dense_tv;
  int64_t row;      // row index (row 0 for rows past N)
  int64_t src;      // the row of the caller's arrays holding the data (= row)
  int64_t seg_off;  // the offset of the first step there (segment view)
};

// A lane's inputs for its K steps t0 .. t0+K-1.  issue_tile (or load_edge)
// fills the loaded fields; finish_tile adds the decoded flags and the
// sparse bootstraps as new fields, never copying a loaded value, so the
// arithmetic reads the load destinations in place and a tile's loads can be
// in flight while the previous tile is computed.  v and lr carry the
// step-(t0+K) neighbour in slot K; v holds q_taken for Retrace.
template <int K>
struct Tile {
  // as loaded
  FlagWords<K> ftr, fte;
  float r[K], v[K + 1], lr[K + 1], eq[K], tv[K];
  // derived
  uint32_t te[K / 4], tr[K / 4];  // one byte per step, nonzero = flag set
                                  // (forward: the flag of the step before)
  bool at_start;                  // forward: the lane's span starts at t = 0
  float ts[K];                    // bootstraps read at truncated steps (Bits<> form)
  bool dense;                     // tv[] holds the bootstraps (else ts[])
};

// One input element as loaded, widened to a float only at its use (a
// conversion right after the load would wait for it inside the branch).
// bf16 keeps its 16 bits zero-extended in a float register.
template <typename InT> struct Bits;
template <> struct Bits<float> {
  static __device__ __forceinline__ float load(const float *p) { return *p; }
  static __device__ __forceinline__ float to_float(float b) { return b; }
};
template <> struct Bits<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t *p) {
    return __uint_as_float(static_cast<uint32_t>(*p));
  }
  static __device__ __forceinline__ float to_float(float b) {
    return __uint_as_float(__float_as_uint(b) << 16);
  }
};

// The truncation bootstrap of step j; read only where step j is truncated.
template <typename InT, int K>
__device__ __forceinline__ float tv_at(const Tile<K> &x, int j) {
  return x.dense ? x.tv[j] : Bits<InT>::to_float(x.ts[j]);
}

// One read of the raw rollout for a lane of a whole tile (Method 2: on-chip
// construction): unconditional vector loads, all issued before any use.
// kVkNeighbour (one-tile instances only, where a lane's span is its row's
// last exactly when lim <= K): only a wavefront's first lane and a row's
// last span load V_{t0+K}; the others take it from their neighbour
// (vk_from_neighbour).  mid runs between the flag loads and the others.
struct NoMid {
  __device__ void operator()() const {}
};
template <int A, typename InT, int K, bool kAligned = false, bool kVkNeighbour = false,
          typename Mid = NoMid>
__device__ __forceinline__ void issue_tile(const Args &p, const RowPtrs<InT> &rp, int64_t t0,
                                           int64_t lim, Tile<K> &q, Mid mid = Mid()) {
  using U = Uses<A>;
#pragma unroll
  for (int j = 0; j < K; ++j) { q.v[j] = 0.f; q.lr[j] = 0.f; q.eq[j] = 0.f; q.tv[j] = 0.f; }
  q.v[K] = 0.f;
  q.lr[K] = 0.f;
  // Flags first, with no branch: a missing flag array is replaced by the
  // lane's own reward bytes (the address of its reward load, so a cache hit)
  // and masked to zero after decoding.  The truncation test in finish_tile
  // then waits for the flags only, with every other load in flight.
  // Forward recurrences use the flag of the step before each step: read the
  // K bytes from t0 - 1 (from t0 at the row start; finish_tile then shifts
  // in "no boundary" before step 0).
  const int64_t f0 = Uses<A>::prev_flags ? (t0 > 0 ? t0 - 1 : 0) : t0;
  q.at_start = Uses<A>::prev_flags && t0 == 0;
  const uint8_t *own = reinterpret_cast<const uint8_t *>(rp.r + t0);
  const uint8_t *trp = own;
  if constexpr (A == kRetrace) {
    // Cold stream: only a call with truncation flags waits for Args here.
    if (rp.has_tr) trp = p.trunc + late_v(rp.src) * p.ld_trunc + rp.seg_off + t0;
  } else {
    trp = rp.has_tr ? rp.tr + f0 : own;
  }
  if constexpr (kAligned && A == kGae) {
    // GAE's aligned instances: a missing flag array's stand-in load is
    // skipped behind a uniform branch (GAE 4096x128 with the V_{t0+K} form
    // below: 3.42 -> 3.32 us per launch; TD(lambda) 16384x256 with the same
    // two changes: 10.07 -> 10.34 us, so the other algorithms keep the
    // unconditional form).
    auto zero = [](FlagWords<K> &f) {
#pragma unroll
      for (int i = 0; i < K / 4; ++i) f.d[i] = 0u;
      f.extra = 0u;
      f.sh = 0u;
    };
    if (rp.has_tr) ld_flags_raw<K, true>(trp, q.ftr);
    else zero(q.ftr);
    if (rp.has_te) ld_flags_raw<K, true>(rp.te + f0, q.fte);
    else zero(q.fte);
  } else {
    ld_flags_raw<K, kAligned>(trp, q.ftr);
    ld_flags_raw<K, kAligned>(rp.has_te ? rp.te + f0 : own, q.fte);
  }
  mid();
  Ld<InT>::template vec<K>(rp.r + t0, q.r);
  if constexpr (U::values || U::q || U::affine) {
    // Values are non-temporal where most lanes take V_{t0+K} from their
    // neighbour, so that nothing re-reads their lines (GAE 4096x128: 3.355 ->
    // 3.316 us per launch); elsewhere the V_{t0+K} loads re-read them.
    float vk[K];
    Ld<InT>::template vec<K, kVkNeighbour>(rp.v + t0, vk);
#pragma unroll
    for (int j = 0; j < K; ++j) q.v[j] = vk[j];
    if constexpr (kVkNeighbour && U::values) {
      // V_{t0+K} is the next span's first value, which the lane before in the
      // wavefront holds (vk_from_neighbour); only a wavefront's first lane
      // and a row's last span load it.
      if ((threadIdx.x & 63) == 0 || lim <= K) q.v[K] = Ld<InT>::one(rp.v + t0 + K);
    } else if constexpr (U::values) {
      q.v[K] = Ld<InT>::one(rp.v + t0 + K);  // V_{t0+K} (<= V_T)
    }
  }
  if constexpr (U::q) Ld<InT>::template vec<K, true>(rp.eq + t0, q.eq);
  if constexpr (U::log_rho) {
    float lk[K];
    Ld<InT>::template vec<K>(rp.lr + t0, lk);
#pragma unroll
    for (int j = 0; j < K; ++j) q.lr[j] = lk[j];
    if constexpr (A == kRetrace) {
      // log_rho_{t0+K}; at the row end (lim == K) re-read the last step
      // instead, whose value the trace then ignores.
      q.lr[K] = Ld<InT>::one(rp.lr + t0 + (lim > K ? K : K - 1));
    }
  }
  q.dense = false;
  if constexpr (U::tv && A != kVtrace) {
    // Small batches read the bootstraps as whole vectors in flight with the
    // other loads (no dependent round trip after the flags arrive; the extra
    // bytes cost less than the latency there).  Otherwise the lane re-reads
    // its own rewards (a cache hit, unused) and finish_tile reads the
    // bootstraps at truncated steps only.
    float tk[K];
    Ld<InT>::template vec<K, true>(rp.dense_tv ? rp.tv + t0 : rp.r + t0, tk);
#pragma unroll
    for (int j = 0; j < K; ++j) q.tv[j] = tk[j];
    q.dense = rp.dense_tv;
  }
  // Keep every load above ahead of the first use of any loaded value: the
  // scheduler would otherwise pull the flag decoding up and wait for the
  // flags before issuing the remaining loads.
  __builtin_amdgcn_sched_barrier(0);
}

// V_{t0+K} of a lane that did not load it (issue_tile with kVkNeighbour): the
// first value of the lane before it in the wavefront, whose
// span is the next one in time (reverse lane order).  A wavefront's first
// lane and a row's last span (end_span) loaded their own.
template <int K>
__device__ __forceinline__ void vk_from_neighbour(Tile<K> &x, bool end_span) {
  const float nb = dpp<0x138, 0xf>(x.v[0], x.v[K]);  // wave_shr:1
  x.v[K] = ((threadIdx.x & 63) == 0 || end_span) ? x.v[K] : nb;
}

// Truncation bootstraps at truncated steps only (rare), into registers of
// their own.  ts[] is written only when some step of the lane is truncated;
// every read of it is guarded by that step's truncation flag, so on other
// paths it is never read (and not zeroed: a write there would wait for
// loads of earlier tiles).  Flags of steps outside the row are zero.
template <int A, typename InT, int K>
__device__ __forceinline__ void sparse_tv(const Args &p, const RowPtrs<InT> &rp, int64_t t0,
                                          Tile<K> &x) {
  if constexpr (Uses<A>::tv) {
    if (x.dense) return;
    uint32_t any_tr = 0;
#pragma unroll
    for (int i = 0; i < K / 4; ++i) any_tr |= x.tr[i];
    if (any_tr != 0) {
      // The bootstraps' own row pointer (the hot one is null when they are
      // read sparsely).
      const InT *tv_row =
          static_cast<const InT *>(p.tv) + late_v(rp.src) * p.ld_tv + rp.seg_off;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        x.ts[j] = 0.f;
        if (flag<K>(x.tr, j)) x.ts[j] = Bits<InT>::load(tv_row + t0 + j);
      }
    }
  }
}

// Decode an issued tile's flags (the first use of its loads).
template <int A, typename InT, int K>
__device__ __forceinline__ void decode_tile(const RowPtrs<InT> &rp, Tile<K> &x) {
  decode_flags<K>(x.ftr, x.tr);
  decode_flags<K>(x.fte, x.te);
  if constexpr (Uses<A>::prev_flags) {
    if (x.at_start) {  // bytes t0 .. t0+K-1 were read: shift by one step
#pragma unroll
      for (int i = K / 4 - 1; i >= 0; --i) {
        x.tr[i] = (x.tr[i] << 8) | (i > 0 ? x.tr[i - 1] >> 24 : 0u);
        x.te[i] = (x.te[i] << 8) | (i > 0 ? x.te[i - 1] >> 24 : 0u);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < K / 4; ++i) {
    x.tr[i] = rp.has_tr ? x.tr[i] : 0u;
    x.te[i] = rp.has_te ? x.te[i] : 0u;
  }
}

// Decode an issued tile and issue its sparse bootstrap loads.
template <int A, typename InT, int K>
__device__ __forceinline__ void finish_tile(const Args &p, const RowPtrs<InT> &rp, int64_t t0,
                                            Tile<K> &x) {
  decode_tile<A, InT, K>(rp, x);
  sparse_tv<A, InT, K>(p, rp, t0, x);
}

// Move a lane's per-step values d steps down (x[j] <- x[j + d], zero past the
// end), d the same for every field of the lane.
template <int N>
__device__ __forceinline__ void shift_down(float (&x)[N], int d) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    float v = 0.f;
#pragma unroll
    for (int k = 1; j + k < N; ++k) v = d == k ? x[j + k] : v;
    x[j] = d == 0 ? x[j] : v;
  }
}

template <int K>
__device__ __forceinline__ void shift_flags_down(uint32_t (&w)[K / 4], int d) {
  uint32_t out[K / 4];
#pragma unroll
  for (int i = 0; i < K / 4; ++i) out[i] = 0u;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    uint32_t b = 0u;
#pragma unroll
    for (int k = 0; j + k < K; ++k) b = d == k ? (w[(j + k) >> 2] >> (((j + k) & 3) * 8)) & 0xffu : b;
    out[j >> 2] |= b << ((j & 3) * 8);
  }
#pragma unroll
  for (int i = 0; i < K / 4; ++i) w[i] = out[i];
}

// The ragged last tile of a row.  Rows of at least K steps: every lane loads
// K steps as in a whole tile, a lane whose span runs past the row's end the
// row's last K steps [T - K, T), and then moves its values down so that slot
// j holds step t0 + j (slots past the end are zero and masked later).  No
// lane branches, so every load of the tile is in flight together.  Shorter
// rows load the steps e < lim one by one.
template <int A, typename InT, int K>
__device__ __forceinline__ void load_edge(const Args &p, const RowPtrs<InT> &rp, int64_t t0,
                                          int64_t lim, int64_t T, Tile<K> &x) {
  if (T >= K) {
    const int64_t tb = t0 < T - K ? t0 : T - K;
    const int d = static_cast<int>(t0 - tb < K ? t0 - tb : K);
    issue_tile<A, InT, K>(p, rp, tb, T - tb, x);
    decode_tile<A, InT, K>(rp, x);
    shift_down(x.r, d);
    shift_down(x.v, d);
    shift_down(x.lr, d);
    shift_down(x.eq, d);
    shift_down(x.tv, d);
    shift_flags_down<K>(x.te, d);
    shift_flags_down<K>(x.tr, d);
    sparse_tv<A, InT, K>(p, rp, t0, x);
    return;
  }
  using U = Uses<A>;
#pragma unroll
  for (int j = 0; j < K; ++j) { x.r[j] = 0.f; x.v[j] = 0.f; x.lr[j] = 0.f; x.eq[j] = 0.f; x.tv[j] = 0.f; }
  x.v[K] = 0.f;
  x.lr[K] = 0.f;
  x.dense = false;
#pragma unroll
  for (int i = 0; i < K / 4; ++i) { x.te[i] = 0; x.tr[i] = 0; }
  x.at_start = false;
  if (lim > 0) {
    if constexpr (Uses<A>::prev_flags) {
      // The flag of the step before each step (none before t = 0).
#pragma unroll
      for (int e = 0; e < K; ++e) {
        const bool in = e < lim && t0 + e > 0;
        if (in && rp.has_tr && rp.tr[t0 + e - 1] != 0) x.tr[e >> 2] |= 1u << ((e & 3) * 8);
        if (in && rp.has_te && rp.te[t0 + e - 1] != 0) x.te[e >> 2] |= 1u << ((e & 3) * 8);
      }
    } else {
      if (rp.has_tr) {
        const uint8_t *trp;
        if constexpr (A == kRetrace) trp = p.trunc + late_v(rp.src) * p.ld_trunc + rp.seg_off;
        else trp = rp.tr;
        ld_flags_part<K>(trp + t0, lim, x.tr);
      }
      if (rp.has_te) ld_flags_part<K>(rp.te + t0, lim, x.te);
    }
    ld_part<InT, K>(rp.r + t0, lim, x.r);
    if constexpr (U::values) {
#pragma unroll
      for (int e = 0; e <= K; ++e) x.v[e] = e <= lim ? Ld<InT>::one(rp.v + t0 + e) : 0.f;
    }
    if constexpr (U::q || U::affine) {
      float qk[K];
      ld_part<InT, K>(rp.v + t0, lim, qk);
#pragma unroll
      for (int j = 0; j < K; ++j) x.v[j] = qk[j];
      if constexpr (U::q) ld_part<InT, K>(rp.eq + t0, lim, x.eq);
    }
    if constexpr (U::log_rho) {
#pragma unroll
      for (int e = 0; e <= K; ++e) x.lr[e] = e < lim ? Ld<InT>::one(rp.lr + t0 + e) : 0.f;
    }
  }
  sparse_tv<A, InT, K>(p, rp, t0, x);
}

// (alpha_t, beta_t) per step (Method 1 coefficients, Method 3 masks).  Steps
// outside the row get the identity map (0, 1).
template <int A, typename InT, int K, bool kEdge, bool kChunk, bool kEarly = true>
__device__ __forceinline__ void coefficients(const Tile<K> &x, int64_t lim, const Args &p,
                                             float (&al)[K], float (&be)[K], float (&ratio)[K]) {
  const float gamma = late(p.gamma);
  const float lam = late(p.lam);
  const float gl = gamma * lam;
  const float rho_bar = A == kVtrace ? late(p.rho_bar) : 1.f;
  const float c_bar = A == kVtrace || A == kRetrace ? late(p.c_bar) : 1.f;
  if constexpr (kEarly && (A == kReturns || A == kGae || A == kTdLambda || Uses<A>::prev_flags)) {
    // The factors need the flags only, which arrive first: they are formed
    // before the wait for the tile's other loads, and the work left once the
    // data is in is shorter (GAE 4096x128 3.27 -> 3.23 us, TD(lambda)
    // 16384x256 10.07 -> 10.01 us, GAE bf16 256x16384 11.75 -> 11.46 us).
    // Forward mirrors: te, tr are the flags of step t-1, and a boundary there
    // restarts at step t.  (kEarly is off in the general instances' two-buffer
    // tile loop at 8 steps per lane, whose registers would then spill.)
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const bool done = flag<K>(x.te, j) || flag<K>(x.tr, j);
      const float b_j = done ? 0.f : (A == kReturns ? gamma : A == kCumsum ? 1.f : gl);
      be[j] = !kEdge || j < lim ? b_j : 1.f;
      ratio[j] = 0.f;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const bool te = flag<K>(x.te, j);
      const bool tr = flag<K>(x.tr, j);
      float a_j;
      if constexpr (A == kReturns) {
        a_j = (tr && !te) ? fmaf(gamma, tv_at<InT, K>(x, j), x.r[j]) : x.r[j];
      } else if constexpr (A == kGae || A == kTdLambda) {
        const float nv = te ? 0.f : (tr ? tv_at<InT, K>(x, j) : x.v[j + 1]);
        a_j = fmaf(gamma, nv, x.r[j]) - x.v[j];
      } else {  // forward mirrors
        a_j = x.r[j];
      }
      al[j] = !kEdge || j < lim ? a_j : 0.f;
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const bool te = flag<K>(x.te, j);
    const bool tr = flag<K>(x.tr, j);
    const bool done = te || tr;
    float a_j, b_j;
    ratio[j] = 0.f;
    if constexpr (A == kReturns) {
      a_j = (tr && !te) ? fmaf(gamma, tv_at<InT, K>(x, j), x.r[j]) : x.r[j];
      b_j = done ? 0.f : gamma;
    } else if constexpr (A == kGae || A == kTdLambda) {
      const float nv = te ? 0.f : (tr ? tv_at<InT, K>(x, j) : x.v[j + 1]);
      a_j = fmaf(gamma, nv, x.r[j]) - x.v[j];
      b_j = done ? 0.f : gl;
    } else if constexpr (A == kVtrace) {
      const float e = __expf(x.lr[j]);
      ratio[j] = e;
      const float nv = te ? 0.f : (tr ? tv_at<InT, K>(x, j) : x.v[j + 1]);
      a_j = fminf(rho_bar, e) * (fmaf(gamma, nv, x.r[j]) - x.v[j]);
      b_j = done ? 0.f : gamma * (lam * fminf(c_bar, e));
    } else if constexpr (Uses<A>::affine) {
      // te: reset flag of step t itself.
      a_j = x.r[j];
      b_j = te ? 0.f : x.v[j];
    } else if constexpr (Uses<A>::forward) {
      // te, tr: flags of step t-1; a boundary there restarts at step t.
      a_j = x.r[j];
      b_j = done ? 0.f : (A == kCumsum ? 1.f : gl);
    } else {  // kRetrace
      a_j = (te ? x.r[j] : fmaf(gamma, x.eq[j], x.r[j])) - x.v[j];
      const bool has_next = j + 1 < lim;  // step t+1 lies inside the row
      const float c_next = lam * fminf(c_bar, __expf(x.lr[j + 1]));
      if constexpr (kChunk) {
        // Window: the carry is c_T * (Qret_T - Q_T) of the step after the
        // window, so the last step's factor is gamma alone.
        b_j = done ? 0.f : gamma * (has_next ? c_next : 1.f);
      } else {
        b_j = (done || !has_next) ? 0.f : gamma * c_next;
      }
    }
    const bool valid = !kEdge || j < lim;
    al[j] = valid ? a_j : 0.f;
    be[j] = valid ? b_j : 1.f;
  }
}

// The row's carry map (a, b), carry = a + b * (carry entering the window),
// kept beside the scalar carry by the window instances.
struct CarryMap {
  float a, b;
};

// Window instances: what the outgoing carry needs besides the scan, read
// with the carry entering the window once the row's first tile of loads is
// in flight (so that no wait for the argument block or for these loads comes
// before them): Retrace's log_rho_0 and the forward mirrors' flags of step
// T-1.
struct WindowIn {
  float lr0;
  bool done_last;
};

template <int A, typename InT, bool kU = false, bool kReadCarry = true>
__device__ __forceinline__ WindowIn window_in(const Args &p, const RowPtrs<InT> &rp, int64_t T,
                                              float &carry) {
  WindowIn w{0.f, false};
  if constexpr (kReadCarry) {
    // The carry vectors hold one entry per segment (row-major over segments).
    const int64_t row = late_row<kU>(rp.row) * late(p.seg_count) + blockIdx.y;
    if (p.cin != nullptr) carry = p.cin[row];
  }
  if constexpr (A == kRetrace) w.lr0 = Ld<InT>::one(rp.lr);
  if constexpr (Uses<A>::prev_flags)
    w.done_last = (rp.has_te && rp.te[T - 1] != 0) || (rp.has_tr && rp.tr[T - 1] != 0);
  return w;
}

// The arguments the end of a row needs (output rows and strides; the window
// instances' carry vectors and segment count), held in scalar registers from
// here on: placed after a tile's loads are issued, their scalar loads are
// waited for while those loads are in flight instead of just before the
// stores (TD(lambda) 16384x256 10.03 -> 9.98 us, its window call without
// carries 10.12 -> 10.08 us, the GAE 4096x128 one 3.37 -> 3.34 us).
template <bool kChunk>
__device__ __forceinline__ void pin_epilogue_args(const Args &p) {
  asm volatile("" ::"s"(p.o0), "s"(p.o1), "s"(p.ld_o0), "s"(p.ld_o1));
  if constexpr (kChunk) asm volatile("" ::"s"(p.cout), "s"(p.cmap), "s"(p.seg_count));
}

// The window instances' per-row results, written after the row's last tile
// by the group's last lane in scan order: the carry the neighbouring window
// takes and the map from this window's incoming carry to it.  Reverse
// recurrences hand on A_0 (Retrace: c_0 * A_0, the trace factor of step 0
// applied); forward mirrors hand on A_{T-1}, or nothing when an episode ends
// after step T-1; the generic scan hands on its last state unchanged.
// The factor between a window's last scan state and the carry it hands on
// (see window_out).
template <int A>
__device__ __forceinline__ float window_factor(const Args &p, const WindowIn &w) {
  float f = 1.f;
  if constexpr (A == kRetrace) f = p.lam * fminf(p.c_bar, __expf(w.lr0));
  if constexpr (Uses<A>::prev_flags) f = w.done_last ? 0.f : 1.f;
  return f;
}

template <int A, typename InT, bool kU = false>
__device__ __forceinline__ void window_out(const Args &p, const RowPtrs<InT> &rp,
                                           const WindowIn &w, bool write, float carry,
                                           CarryMap m) {
  if (!write) return;
  const float f = window_factor<A>(p, w);
  const int64_t row = late_row<kU>(rp.row) * late(p.seg_count) + blockIdx.y;
  if (p.cout != nullptr) p.cout[row] = f * carry;
  if (p.cmap != nullptr) {
    p.cmap[2 * row] = f * m.a;
    p.cmap[2 * row + 1] = f * m.b;
  }
}

// The end of a tile: re-run the lane's steps from the value entering its span
// (xin) and write the tile's outputs, with the fused epilogue of each
// algorithm.  al, be: the steps' coefficients; ratio: V-trace's e^{log_rho}.
template <int A, typename InT, int K, int WPR, bool kEdge, bool kChunk>
__device__ __forceinline__ void tile_epilogue(const Args &p, const RowPtrs<InT> &rp,
                                              const Tile<K> &x, int64_t t0, int64_t lim,
                                              bool row_ok, int lane, int wave,
                                              const float (&al)[K], const float (&be)[K],
                                              const float (&ratio)[K], float xin) {
  using U = Uses<A>;
  // Re-run the lane's steps from its incoming value; fused epilogue.
  const float gamma = late(p.gamma);
  const float pg_rho_bar = A == kVtrace ? late(p.pg_rho_bar) : 1.f;
  float o0[K], o1[K];
  float xa = xin;
  if constexpr (U::forward) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      xa = fmaf(be[j], xa, al[j]);
      o0[j] = xa;
      o1[j] = 0.f;
    }
  }
#pragma unroll
  for (int j = K - 1; j >= 0; --j) {
    if constexpr (U::forward) break;
    const float xn = xa;  // A_{t+1}
    xa = fmaf(be[j], xa, al[j]);
    o1[j] = 0.f;
    if constexpr (A == kReturns || A == kAffine) {
      o0[j] = xa;
    } else if constexpr (A == kGae) {
      o0[j] = xa;
      o1[j] = xa + x.v[j];
    } else if constexpr (A == kTdLambda) {
      o0[j] = xa + x.v[j];
    } else if constexpr (A == kVtrace) {
      o0[j] = x.v[j] + xa;
      const bool te = flag<K>(x.te, j);
      const bool tr = flag<K>(x.tr, j);
      const float nvs = te ? 0.f : (tr ? tv_at<InT, K>(x, j) : x.v[j + 1] + xn);
      o1[j] = fminf(pg_rho_bar, ratio[j]) * (fmaf(gamma, nvs, x.r[j]) - x.v[j]);
    } else {  // kRetrace
      o0[j] = x.v[j] + xa;
    }
  }

  // One write of the outputs.
  const bool has_o1 = U::two_outputs && late(p.o1) != nullptr;
  const int64_t orow = late_row<(WPR > 1)>(rp.src);
  // Rows and strides are below 2^31: one 32 x 32 -> 64-bit multiply each.
  auto row_off = [&](int64_t ld) {
    return static_cast<int64_t>(static_cast<uint64_t>(static_cast<uint32_t>(orow)) *
                                static_cast<uint32_t>(ld));
  };
  float *o0_row = p.o0 + row_off(p.ld_o0) + rp.seg_off;
  float *o1_row = p.o1 + row_off(p.ld_o1) + rp.seg_off;
  // Window instances with no outputs (the first pass of a split call) write
  // only the carry vectors.
  const bool store = row_ok && (!kChunk || p.o0 != nullptr);
  if constexpr (!kEdge) {
    // Non-temporal (streaming) dwordx4 stores: outputs are written once and
    // not re-read by this kernel.
    if constexpr (K == 8 && WPR > 1) {
      // Eight steps per lane: a lane's 32 output bytes would be two 16-byte
      // stores, each instruction writing every other 16-byte piece of the
      // wavefront's span.  Stage the outputs through this wavefront's part
      // of LDS instead, in time order, and store them back as two
      // instructions that each write one contiguous half of the span.
      // (Whole tiles only: every lane of the wavefront holds K steps.)
      __shared__ float4 s_stage[WPR][2 * 64];
      const int pos = U::forward ? lane : 63 - lane;  // the lane's span in the wavefront's
      const int64_t ws = t0 - static_cast<int64_t>(pos) * K;  // the wavefront's first step
      float4 *st = s_stage[wave];
      auto put = [&](float *row, const float (&o)[K]) {
        st[2 * pos] = make_float4(o[0], o[1], o[2], o[3]);
        st[2 * pos + 1] = make_float4(o[4], o[5], o[6], o[7]);
        // The wavefront's LDS operations complete in order; this keeps the
        // compiler from moving the reads of other lanes' values above.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const float4 lo = st[lane], hi = st[64 + lane];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        V4 *dst = reinterpret_cast<V4 *>(row + ws);
        __builtin_nontemporal_store(V4{lo.x, lo.y, lo.z, lo.w}, dst + lane);
        __builtin_nontemporal_store(V4{hi.x, hi.y, hi.z, hi.w}, dst + 64 + lane);
      };
      if (store) {
        put(o0_row, o0);
        if (has_o1) put(o1_row, o1);
      }
    } else if (store) {
#pragma unroll
      for (int i = 0; i < K / 4; ++i)
        __builtin_nontemporal_store(V4{o0[4 * i], o0[4 * i + 1], o0[4 * i + 2], o0[4 * i + 3]},
                                    reinterpret_cast<V4 *>(o0_row + t0) + i);
      if (has_o1) {
#pragma unroll
        for (int i = 0; i < K / 4; ++i)
          __builtin_nontemporal_store(V4{o1[4 * i], o1[4 * i + 1], o1[4 * i + 2], o1[4 * i + 3]},
                                      reinterpret_cast<V4 *>(o1_row + t0) + i);
      }
    }
  } else if (lim >= K && store) {
    // Ragged tile, a lane whose steps all lie in the row: as above.
#pragma unroll
    for (int i = 0; i < K / 4; ++i)
      __builtin_nontemporal_store(V4{o0[4 * i], o0[4 * i + 1], o0[4 * i + 2], o0[4 * i + 3]},
                                  reinterpret_cast<V4 *>(o0_row + t0) + i);
    if (has_o1) {
#pragma unroll
      for (int i = 0; i < K / 4; ++i)
        __builtin_nontemporal_store(V4{o1[4 * i], o1[4 * i + 1], o1[4 * i + 2], o1[4 * i + 3]},
                                    reinterpret_cast<V4 *>(o1_row + t0) + i);
    }
  } else if (store) {
#pragma unroll
    for (int e = 0; e < K; ++e)
      if (e < lim) {
        o0_row[t0 + e] = o0[e];
        if (has_o1) o1_row[t0 + e] = o1[e];
      }
  }
}

// One tile of one row group, inputs already loaded: build pairs, fold, scan,
// carry, re-run, store.  Returns the carry for the next tile in scan order
// (in every lane when need_carry; need_carry is false for the row's last
// tile).  Window instances also fold the tile's composite into m in the
// group's last lane in scan order, whose inclusive scan is that composite,
// and after the row's last tile that lane writes the window results
// (window_out) before the tile's outputs are stored.
template <int A, typename InT, int K, int LPR, int WPR, bool kEdge, bool kChunk,
          bool kEarly = true>
__device__ __forceinline__ float tile_compute(const Args &p, const RowPtrs<InT> &rp,
                                              const Tile<K> &x, int64_t t0, int64_t lim,
                                              bool row_ok, int64_t c, bool need_carry, int lane,
                                              int wave, float carry, float2 (*s_agg)[WPR],
                                              CarryMap &m, const WindowIn &win,
                                              bool write_window) {
  constexpr int kScanLanes = WPR > 1 ? 64 : LPR;
  using U = Uses<A>;

  float al[K], be[K], ratio[K];
  coefficients<A, InT, K, kEdge, kChunk, kEarly>(x, lim, p, al, be, ratio);

  // Fold the lane's steps into one map of the incoming value: reverse,
  // (a, b) = f_{t0} o ... o f_{t0+K-1}; forward, f_{t0+K-1} o ... o f_{t0}.
  float a, b;
  if constexpr (U::forward) {
    a = al[0];
    b = be[0];
#pragma unroll
    for (int j = 1; j < K; ++j) {
      a = fmaf(be[j], a, al[j]);
      b = be[j] * b;
    }
  } else {
    a = al[K - 1];
    b = be[K - 1];
#pragma unroll
    for (int j = K - 2; j >= 0; --j) {
      a = fmaf(be[j], a, al[j]);
      b = be[j] * b;
    }
  }

  group_scan<kScanLanes>(a, b);

  // Carry into this lane group's span and out of the tile.
  float cin = carry;
  float carry_out = 0.f;
  if constexpr (WPR > 1) {
    const int buf = static_cast<int>(c & 1);
    const float wa = readlane(a, 63), wb = readlane(b, 63);  // whole-wavefront map
    if (lane == 0) s_agg[buf][wave] = make_float2(wa, wb);
    __syncthreads();
    // Wavefront 0 holds the first span of the tile in scan order (reverse:
    // the latest steps; forward: the earliest): compose from it onward.
    // Lane w < WPR of every wavefront takes wavefront w's map, and a scan
    // over those lanes leaves in lane w the composite of wavefronts 0 .. w.
    const float2 ag = lane < WPR ? s_agg[buf][lane] : make_float2(0.f, 1.f);
    float sa = ag.x, sb = ag.y;
    group_scan<WPR>(sa, sb);
    const int w = __builtin_amdgcn_readfirstlane(wave);
    const int wp = w > 0 ? w - 1 : 0;
    const float pa = readlane(sa, wp), pb = readlane(sb, wp);  // wavefronts 0 .. w-1
    if (w > 0) cin = fmaf(pb, carry, pa);
    const float ta = readlane(sa, WPR - 1), tb = readlane(sb, WPR - 1);
    const float xc = fmaf(tb, carry, ta);
    CarryMap tm{ta, tb};  // the tile's composite
    carry_out = xc;
    if constexpr (kChunk) {
      m.a = fmaf(tm.b, m.a, tm.a);
      m.b = tm.b * m.b;
      if (!need_carry) window_out<A, InT, (WPR > 1)>(p, rp, win, write_window, xc, m);
    }
  }
  // A at the far end of this lane's span (reverse: its earliest step;
  // forward: its latest) ...
  const float y = fmaf(b, cin, a);
  // ... and the value entering the lane's span: y of the previous lane in
  // scan order (lane - 1), the next-later (reverse) or next-earlier (forward)
  // span.
  float xin = dpp<0x138, 0xf>(y, cin);  // wave_shr:1
  if ((lane % kScanLanes) == 0) xin = cin;
  if constexpr (WPR == 1) {
    if (need_carry) {
      if constexpr (LPR == 64) carry_out = readlane(y, 63);
      else carry_out = lane_shuffle(y, (lane / LPR) * LPR + LPR - 1);
    }
    if constexpr (kChunk) {
      // Meaningful in the group's last lane only (see above).
      m.a = fmaf(b, m.a, a);
      m.b = b * m.b;
      if (!need_carry) window_out<A, InT, (WPR > 1)>(p, rp, win, write_window, y, m);
    }
  }

  tile_epilogue<A, InT, K, WPR, kEdge, kChunk>(p, rp, x, t0, lim, row_ok, lane, wave, al, be,
                                              ratio, xin);
  return carry_out;
}

// ---------------------------------------------------- chained (one-pass) split
//
// A split call's segments in one pass: workgroup (row, k) takes the k-th
// segment of its row in scan order (from the row's end for reverse
// recurrences, from its start for forward ones), k = blockIdx.y.  It loads
// and scans its segment without a carry (tile_scan), publishes the segment's
// carry map, finds the carry entering its segment from the maps of the
// segments before it in scan order (chain_lookback), publishes the carry map
// from the row's incoming carry to its own outgoing one, then writes its
// outputs (tile_emit).  The inputs are read once; the carry maps are the
// window calls' (window_out), composed as the split calls compose them.
//
// Each published value is one 64-bit word, written and read with relaxed
// device-scope atomics (coherent across the chip's L2 caches): the value's
// bits in the low half and the call's tag in the high half, so a word is
// either wholly this call's or not yet written by it.  The workspace's epoch
// word holds the previous call's tag, and this call's is the next value
// (never 0): every workgroup reads the word once, before it publishes
// anything, and the launch's last workgroup stores the new tag there once no
// workgroup of this call can still read it (chain_advance; also on every
// replay of a captured graph), so that no word an earlier call left is taken
// for one of this call.  (A fresh workspace filled with any one 32-bit
// pattern holds no word with the first call's tag.)  A workgroup reads only
// the words of workgroups with smaller linear ids, which were dispatched no
// later; the poll is bounded all the same (kChainMaxPolls), and a carry not
// found by then is NaN.

constexpr int kChainMaxPolls = 1 << 16;
constexpr int kChainMaxSegments = 256;  // segments per row (look-back: a window of 64)

// A lane's state after the carry-free scan of a whole tile (WPR > 1): its
// inclusive map within the wavefront (a, b), the composite of the wavefronts
// before it in the tile (pa, pb; first: it is the first), and the tile's
// composite (ta, tb).
struct TileScan {
  float a, b, pa, pb, ta, tb;
  bool first;
};

template <int A, typename InT, int K, int WPR>
__device__ __forceinline__ TileScan tile_scan(const Args &p, const Tile<K> &x, int64_t lim,
                                              int64_t c, int lane, int wave,
                                              float2 (*s_agg)[WPR]) {
  using U = Uses<A>;
  float al[K], be[K], ratio[K];
  coefficients<A, InT, K, false, true>(x, lim, p, al, be, ratio);
  float a, b;
  if constexpr (U::forward) {
    a = al[0];
    b = be[0];
#pragma unroll
    for (int j = 1; j < K; ++j) {
      a = fmaf(be[j], a, al[j]);
      b = be[j] * b;
    }
  } else {
    a = al[K - 1];
    b = be[K - 1];
#pragma unroll
    for (int j = K - 2; j >= 0; --j) {
      a = fmaf(be[j], a, al[j]);
      b = be[j] * b;
    }
  }
  group_scan<64>(a, b);
  const int buf = static_cast<int>(c & 1);
  const float wa = readlane(a, 63), wb = readlane(b, 63);
  if (lane == 0) s_agg[buf][wave] = make_float2(wa, wb);
  __syncthreads();
  const float2 ag = lane < WPR ? s_agg[buf][lane] : make_float2(0.f, 1.f);
  float sa = ag.x, sb = ag.y;
  group_scan<WPR>(sa, sb);
  const int w = __builtin_amdgcn_readfirstlane(wave);
  const int wp = w > 0 ? w - 1 : 0;
  TileScan s;
  s.a = a;
  s.b = b;
  s.pa = readlane(sa, wp);
  s.pb = readlane(sb, wp);
  s.ta = readlane(sa, WPR - 1);
  s.tb = readlane(sb, WPR - 1);
  s.first = w == 0;
  return s;
}

// The outputs of a tile scanned by tile_scan, given the carry entering it;
// returns the carry it hands on.
template <int A, typename InT, int K, int WPR>
__device__ __forceinline__ float tile_emit(const Args &p, const RowPtrs<InT> &rp,
                                           const Tile<K> &x, int64_t t0, int64_t lim, bool row_ok,
                                           int lane, int wave, float carry, const TileScan &s) {
  const float cin = s.first ? carry : fmaf(s.pb, carry, s.pa);
  const float y = fmaf(s.b, cin, s.a);
  float xin = dpp<0x138, 0xf>(y, cin);  // wave_shr:1
  if (lane == 0) xin = cin;
  float al[K], be[K], ratio[K];
  coefficients<A, InT, K, false, true>(x, lim, p, al, be, ratio);
  tile_epilogue<A, InT, K, WPR, false, true>(p, rp, x, t0, lim, row_ok, lane, wave, al, be, ratio,
                                             xin);
  return fmaf(s.tb, carry, s.ta);
}

__device__ __forceinline__ unsigned long long chain_word(float v, uint32_t tag) {
  return (static_cast<unsigned long long>(tag) << 32) | __float_as_uint(v);
}

__device__ __forceinline__ void chain_put(unsigned long long *w, float v, uint32_t tag) {
  __hip_atomic_store(w, chain_word(v, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wavefront 0 of workgroup (row, k > 0): the map from the row's incoming carry
// to the carry entering segment k, (ra, rb), from the words of the (at most
// 64) segments before it, k0 = max(0, k - 64) .. k-1 (slots: the row's first
// word).  Per segment j: words 0, 1 the segment's own carry map, words 2, 3
// the map from the row's incoming carry to the carry it hands on (segment 0
// publishes only these).  Lane i reads segment k0 + i's four words; the
// latest segment j0 of the window whose words 2, 3 are this call's, with
// words 0, 1 of every later one, composes the answer in one scan.  Beyond 64
// segments the window holds no segment 0: the words 2, 3 of one of its
// segments must appear first, which each publishes once its own look-back
// has ended (the segments below the window come no later in dispatch, so one
// always does).  Returns false if the words were not all there within
// kChainMaxPolls polls.
__device__ __forceinline__ bool chain_lookback(unsigned long long *slots, uint32_t tag, int k,
                                               int lane, float &ra, float &rb) {
  const int k0 = k > 64 ? k - 64 : 0;
  const int n = k - k0;  // window length, 1 .. 64
  for (int it = 0; it < kChainMaxPolls; ++it) {
    unsigned long long w0 = 0, w1 = 0, w2 = 0, w3 = 0;
    if (lane < n) {
      unsigned long long *s = slots + 4 * (k0 + lane);
      w2 = __hip_atomic_load(s + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      w3 = __hip_atomic_load(s + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      w0 = __hip_atomic_load(s + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      w1 = __hip_atomic_load(s + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    auto mine = [&](unsigned long long w) { return static_cast<uint32_t>(w >> 32) == tag; };
    const bool inc = lane < n && mine(w2) && mine(w3);
    const bool agg = lane < n && mine(w0) && mine(w1);
    const unsigned long long inc_mask = __ballot(inc);
    const unsigned long long agg_mask = __ballot(agg);
    if (inc_mask != 0) {
      const int j0 = 63 - __clzll(static_cast<long long>(inc_mask));  // window lane
      // lanes j0+1 .. n-1 need their own maps
      const unsigned long long below_n = n >= 64 ? ~0ull : (1ull << n) - 1;
      const unsigned long long need = below_n & ~((2ull << j0) - 1);
      if ((agg_mask & need) == need) {
        float a = 0.f, b = 1.f;  // identity below j0
        if (lane == j0) {
          a = __uint_as_float(static_cast<uint32_t>(w2));
          b = __uint_as_float(static_cast<uint32_t>(w3));
        } else if (lane > j0 && lane < n) {
          a = __uint_as_float(static_cast<uint32_t>(w0));
          b = __uint_as_float(static_cast<uint32_t>(w1));
        }
        group_scan<64>(a, b);  // lane i: f_i o ... o f_0
        ra = readlane(a, n - 1);
        rb = readlane(b, n - 1);
        return true;
      }
    }
    __builtin_amdgcn_s_sleep(2);
  }
  ra = __int_as_float(0x7fc00000);
  rb = ra;
  return false;
}

// Wavefront 0 of the launch's last workgroup (row N-1, segment S-1; the
// highest linear id), after its own outputs: waits until the last segment of
// every row (lane i: rows i, i + 64, ... below N) has published its words 2,
// 3 with this call's tag, then stores that tag in the epoch word for the next
// call.  A
// segment publishes words 2, 3 only after its look-back has found words of
// every earlier segment of its row, directly or through the words 2, 3 of a
// segment that had itself found them, so by then every workgroup of the call
// has read the epoch word (each reads it before publishing anything).  Were
// the wait to run out, the epoch advances all the same.
__device__ __forceinline__ void chain_advance(unsigned long long *epoch, uint32_t tag, int N,
                                              int S, int lane) {
  for (int it = 0; it < kChainMaxPolls; ++it) {
    bool done = true;
#pragma unroll
    for (int c = 0; c < 4; ++c) {  // rows lane + 64 c, N <= 256
      const int r = lane + 64 * c;
      if (r < N) {
        const unsigned long long w = __hip_atomic_load(
            epoch + 1 + (static_cast<int64_t>(r) * S + (S - 1)) * 4 + 2, __ATOMIC_RELAXED,
            __HIP_MEMORY_SCOPE_AGENT);
        done = done && static_cast<uint32_t>(w >> 32) == tag;
      }
    }
    if (__ballot(!done) == 0) break;
    __builtin_amdgcn_s_sleep(2);
  }
  if (lane == 0)
    __hip_atomic_store(epoch, static_cast<unsigned long long>(tag), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Algo A, input type InT, K steps per lane, LPR lanes per row inside one
// wavefront (WPR == 1), or WPR wavefronts per row (then LPR must be 64).
// kTiles: 0 for the general instance (any T); 1 or 2 for instances that
// take rows of exactly one or exactly two whole tiles (T == kTiles * K *
// lanes per row) only, as straight-line code.  The one-tile instance holds
// one tile of loads and no tile loop, so it needs far fewer VGPRs than the
// general instance (which sizes its registers for the two-buffer loop), and
// more of its wavefronts fit on a SIMD at once.  The two-tile instance
// issues both tiles' loads up front and no more: the general loop's
// unconditional prefetch would re-read a third tile, half again the loads
// of such a row (GAE bf16 256x16384: 13.1 -> 11.5 us without it).
// kAligned (fixed-tile instances of the reverse recurrences only): every
// flag row the kernel reads (and, for a missing flag array, its stand-in,
// the rewards row) is 4-byte aligned, so a lane's flag span is read as
// exactly its K/4 dwords.
// Workgroup: 64 * short_row_waves(WPR, LPR, kChunk, A) threads.
// h0..h4, N32, T32, ldT, ldX: the preloaded hot arguments (see above); they
// duplicate fields of p.  kChunk: window instance (carry vector in, carry and
// carry map out).
template <int A, typename InT, int K, int LPR, int WPR, bool kUniform, bool kChunk,
          int kTiles = 0, bool kAligned = false, bool kChain = false>
__global__ void __launch_bounds__(64 * short_row_waves(WPR, LPR, kChunk, A))
scan_kernel(const void *h0, const void *h1, const void *h2, const void *h3, const void *h4,
            int N32, int T32, int ldT, int ldX, const Args p) {
  static_assert(WPR == 1 || LPR == 64, "multi-wavefront rows use whole wavefronts");
#ifdef RLCA_TIMESTAMPS
  const WaveStamp stamp{p.stamps, wall_clock()};  // written at every return
#endif
  constexpr int kWaves = short_row_waves(WPR, LPR, kChunk, A);
  constexpr int kGroup = WPR > 1 ? 64 * WPR : LPR;
  constexpr int kTile = kGroup * K;

  __shared__ float2 s_agg[2][WPR];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int64_t row;
  int g;  // lane index within the row group; g = 0 owns the latest steps of a tile
  if constexpr (WPR > 1) {
    row = blockIdx.x;
    g = wave * 64 + lane;
  } else {
    row = (static_cast<int64_t>(blockIdx.x) * kWaves + wave) * (64 / LPR) + lane / LPR;
    g = lane % LPR;
  }
  // Rows past N (last workgroup only) read row 0 and store nothing; their
  // lanes stay active because the DPP scan reads every lane of a group.
  const bool row_ok = row < N32;
  const int64_t rr = row_ok ? row : 0;
  const int64_t T = T32;
  // Segment view (window instances of a split call): the launch has one
  // grid row per segment, and workgroups of grid row y take segment y, T
  // steps long, of their rows (no argument is read before the loads).
  const int64_t src = rr;
  // Chained instances of reverse recurrences take the segments from the
  // row's end: the host passes every row pointer moved to the row's last
  // segment, and segment y starts y segments before it.
  const int64_t seg_off =
      kChunk ? (kChain && !Uses<A>::forward ? -static_cast<int64_t>(blockIdx.y) * T
                                            : static_cast<int64_t>(blockIdx.y) * T)
             : 0;
  // Row stride of a hot stream: the preloaded common stride, or (mixed
  // strides) the stream's own stride from Args.
  auto ld = [&](int64_t own_ld) -> int64_t { return kUniform ? static_cast<int64_t>(ldT) : own_ld; };
  auto in_row = [&](const void *base, int64_t stride) {
    return static_cast<const InT *>(base) + src * stride + seg_off;
  };
  auto flag_row = [&](const void *base, int64_t stride) {
    return static_cast<const uint8_t *>(base) + src * stride + seg_off;
  };

  RowPtrs<InT> rp;
  rp.row = rr;
  rp.src = src;
  rp.seg_off = seg_off;
  rp.r = in_row(h0, ld(p.ld_r));
  rp.tv = nullptr;
  if constexpr (A == kReturns) {
    rp.te = flag_row(h1, ld(p.ld_term));
    rp.tr = flag_row(h2, ld(p.ld_trunc));
    rp.tv = in_row(h3, ld(p.ld_tv));
    rp.has_te = h1 != nullptr;
    rp.has_tr = h2 != nullptr;
    rp.dense_tv = h3 != nullptr;
  } else if constexpr (A == kGae || A == kTdLambda) {
    rp.v = in_row(h1, kUniform ? static_cast<int64_t>(ldX) : p.ld_v);
    rp.te = flag_row(h2, ld(p.ld_term));
    rp.tr = flag_row(h3, ld(p.ld_trunc));
    rp.tv = in_row(h4, ld(p.ld_tv));
    rp.has_te = h2 != nullptr;
    rp.has_tr = h3 != nullptr;
    rp.dense_tv = h4 != nullptr;
  } else if constexpr (A == kVtrace) {
    rp.v = in_row(h1, kUniform ? static_cast<int64_t>(ldX) : p.ld_v);
    rp.lr = in_row(h2, ld(p.ld_lr));
    rp.te = flag_row(h3, ld(p.ld_term));
    rp.tr = flag_row(h4, ld(p.ld_trunc));
    rp.has_te = h3 != nullptr;
    rp.has_tr = h4 != nullptr;
    rp.dense_tv = false;
  } else if constexpr (Uses<A>::affine) {
    rp.v = in_row(h1, ld(p.ld_v));
    rp.te = flag_row(h2, ld(p.ld_term));
    rp.tr = nullptr;
    rp.has_te = h2 != nullptr;
    rp.has_tr = false;
    rp.dense_tv = false;
  } else if constexpr (Uses<A>::forward) {
    rp.te = flag_row(h1, ld(p.ld_term));
    rp.tr = flag_row(h2, ld(p.ld_trunc));
    rp.has_te = h1 != nullptr;
    rp.has_tr = h2 != nullptr;
    rp.dense_tv = false;
  } else {  // kRetrace
    rp.v = in_row(h1, ld(p.ld_v));
    rp.eq = in_row(h2, ld(p.ld_eq));
    rp.lr = in_row(h3, ld(p.ld_lr));
    rp.te = flag_row(h4, ld(p.ld_term));
    rp.tr = nullptr;
    rp.has_te = h4 != nullptr;
    rp.has_tr = ldX != 0;
    rp.dense_tv = false;
  }

  // The value entering the current tile: A_T before the last tile (reverse),
  // A_{-1} before the first (forward).
  float carry = 0.f;
  if constexpr (kChunk) {
    // read by window_in after the first loads are issued
  } else if constexpr (A == kReturns) {
    if (h4 != nullptr) carry = Ld<InT>::one(static_cast<const InT *>(h4) + rr);
  } else if constexpr (Uses<A>::forward) {
    if (h3 != nullptr) carry = Ld<InT>::one(static_cast<const InT *>(h3) + rr);
  }
  CarryMap m{0.f, 1.f};
  WindowIn win{0.f, false};
  const bool write_window = row_ok && g == kGroup - 1;

  // Tiles are visited from the last (latest in time) to the first.  A ragged
  // last tile takes the element-wise path; every whole tile's loads are
  // issued while the tile after it (in time) is being computed.
  const int64_t ntiles = (T + kTile - 1) / kTile;
  // Lane g's span in a tile: reverse recurrences scan lanes against time
  // (g = 0 owns the latest steps), forward ones along it.
  const int64_t lane_off =
      static_cast<int64_t>(Uses<A>::forward ? g : kGroup - 1 - g) * K;
  [[maybe_unused]] auto t0_of = [&](int64_t c) { return c * kTile + lane_off; };

  // The general instances' tile loop forms the factors early (coefficients)
  // at 4 steps per lane only.
  constexpr bool kLoopEarly = K == 4;

  // One whole tile: straight-line code.
  auto one_tile = [&]() {
    // GAE's aligned one-tile instances take V_{t0+K} from the neighbouring
    // lane (with the flag loads of issue_tile: GAE 4096x128 3.42 -> 3.32 us;
    // TD(lambda) 16384x256 measured slower with the same two changes).
    constexpr bool kVk = kTiles == 1 && kAligned && A == kGae;
    Tile<K> x;
    if constexpr (kChunk && LPR < 64 && A == kGae) {
      // GAE's window calls on rows that share a wavefront read the carry
      // entering the window between the flags and the other loads, so that
      // it is not the last load to arrive (GAE 4096x128 window call 3.45 ->
      // 3.36 us; with one row per wavefront, TD(lambda) 16384x256, it cost
      // 1.4 us, and the forward mirrors, whose window_in also reads flags,
      // 0.25 us at 4096x128).
      issue_tile<A, InT, K, kAligned, kVk>(p, rp, lane_off, T - lane_off, x, [&]() {
        win = window_in<A, InT, (WPR > 1)>(p, rp, T, carry);
      });
    } else {
      issue_tile<A, InT, K, kAligned, kVk>(p, rp, lane_off, T - lane_off, x);
      if constexpr (kChunk) win = window_in<A, InT, (WPR > 1)>(p, rp, T, carry);
    }
    pin_epilogue_args<kChunk>(p);
    finish_tile<A, InT, K>(p, rp, lane_off, x);
    if constexpr (kVk) vk_from_neighbour(x, T - lane_off <= K);
    tile_compute<A, InT, K, LPR, WPR, false, kChunk>(p, rp, x, lane_off, T - lane_off, row_ok, 0,
                                                     false, lane, wave, carry, s_agg, m, win,
                                                     write_window);
  };
  if constexpr (kChain) {
    // One segment of a split call (see chain_lookback): its tiles scanned
    // without a carry, the segment's carry map published, the carry entering
    // the segment found, then the outputs.
    static_assert(kChunk && WPR > 1 && (kTiles == 1 || kTiles == 2),
                  "chained instances: whole-wavefront rows of one or two tiles");
    __shared__ float s_chain[2];
    constexpr int64_t kFirst = kTiles == 1 || Uses<A>::forward ? 0 : 1;
    constexpr int64_t kSecond = 1 - kFirst;
    Tile<K> xf, xs;
    float unused = 0.f;
    issue_tile<A, InT, K>(p, rp, t0_of(kFirst), T - t0_of(kFirst), xf);
    win = window_in<A, InT, true, false>(p, rp, T, unused);
    finish_tile<A, InT, K>(p, rp, t0_of(kFirst), xf);
    if constexpr (kTiles == 2) issue_tile<A, InT, K>(p, rp, t0_of(kSecond), T - t0_of(kSecond), xs);
    const TileScan sf = tile_scan<A, InT, K, WPR>(p, xf, T - t0_of(kFirst), kFirst, lane, wave,
                                                  s_agg);
    TileScan ss{};
    if constexpr (kTiles == 2) {
      finish_tile<A, InT, K>(p, rp, t0_of(kSecond), xs);
      ss = tile_scan<A, InT, K, WPR>(p, xs, T - t0_of(kSecond), kSecond, lane, wave, s_agg);
    }
    // The segment's carry map: its tiles' composites in scan order, times
    // the factor between its last scan state and the carry it hands on.
    float ma = sf.ta, mb = sf.tb;
    if constexpr (kTiles == 2) {
      ma = fmaf(ss.tb, ma, ss.ta);
      mb = ss.tb * mb;
    }
    const float f = window_factor<A>(p, win);
    ma *= f;
    mb *= f;
    const int k = static_cast<int>(blockIdx.y);
    const int S = late(p.seg_count);
    unsigned long long *slots = p.chain + 1 + row * 4 * static_cast<int64_t>(S);
    const uint32_t epoch = static_cast<uint32_t>(
        __hip_atomic_load(p.chain, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    const uint32_t tag = epoch + 1 != 0 ? epoch + 1 : 1;
    const float c_row = p.cin != nullptr ? p.cin[row] : 0.f;
    if (wave == 0) {
      // (ra, rb): the row's incoming carry -> the carry entering this segment
      float ra = 0.f, rb = 1.f;
      if (k > 0) {
        if (lane == 0) {
          chain_put(slots + 4 * k, ma, tag);
          chain_put(slots + 4 * k + 1, mb, tag);
        }
        chain_lookback(slots, tag, k, lane, ra, rb);
      }
      const float pa = fmaf(mb, ra, ma), pb = mb * rb;  // ... -> the carry it hands on
      if (lane == 0) {
        chain_put(slots + 4 * k + 2, pa, tag);
        chain_put(slots + 4 * k + 3, pb, tag);
        s_chain[0] = ra;
        s_chain[1] = rb;
        if (k == S - 1) {
          if (p.cout != nullptr) p.cout[row] = fmaf(pb, c_row, pa);
          if (p.cmap != nullptr) {
            p.cmap[2 * row] = pa;
            p.cmap[2 * row + 1] = pb;
          }
        }
      }
    }
    __syncthreads();
    const float c_seg = fmaf(s_chain[1], c_row, s_chain[0]);
    const float c_next = tile_emit<A, InT, K, WPR>(p, rp, xf, t0_of(kFirst), T - t0_of(kFirst),
                                                   row_ok, lane, wave, c_seg, sf);
    if constexpr (kTiles == 2)
      tile_emit<A, InT, K, WPR>(p, rp, xs, t0_of(kSecond), T - t0_of(kSecond), row_ok, lane,
                                wave, c_next, ss);
    (void)c_next;
    if (wave == 0 && k == S - 1 && row == N32 - 1) chain_advance(p.chain, tag, N32, S, lane);
  } else if constexpr (kTiles == 1) {
    one_tile();
  } else if constexpr (kTiles == 2) {
    // Two whole tiles, both tiles' loads in flight: the tile computed first
    // (the later one in time for reverse recurrences, the earlier one for
    // forward ones) hands its carry to the other.
    constexpr int64_t kFirst = Uses<A>::forward ? 0 : 1;
    constexpr int64_t kSecond = 1 - kFirst;
    Tile<K> xf, xs;
    issue_tile<A, InT, K, kAligned>(p, rp, t0_of(kFirst), T - t0_of(kFirst), xf);
    if constexpr (kChunk) win = window_in<A, InT, (WPR > 1)>(p, rp, T, carry);
    pin_epilogue_args<kChunk>(p);
    finish_tile<A, InT, K>(p, rp, t0_of(kFirst), xf);
    issue_tile<A, InT, K, kAligned>(p, rp, t0_of(kSecond), T - t0_of(kSecond), xs);
    carry = tile_compute<A, InT, K, LPR, WPR, false, kChunk>(
        p, rp, xf, t0_of(kFirst), T - t0_of(kFirst), row_ok, kFirst, true, lane, wave, carry,
        s_agg, m, win, write_window);
    finish_tile<A, InT, K>(p, rp, t0_of(kSecond), xs);
    tile_compute<A, InT, K, LPR, WPR, false, kChunk>(p, rp, xs, t0_of(kSecond),
                                                     T - t0_of(kSecond), row_ok, kSecond, false,
                                                     lane, wave, carry, s_agg, m, win,
                                                     write_window);
  } else {
    if (ntiles == 1 && T == kTile) {
      one_tile();
      return;
    }
    {
      const bool ragged = T % kTile != 0;
      if constexpr (Uses<A>::forward) {
        // Tiles from the first to the last; the ragged one comes last.  Same
        // two-buffer pipeline as below, in increasing c.
        const int64_t nwhole = ragged ? ntiles - 1 : ntiles;
        Tile<K> buf_a, buf_b;
        int64_t c = 0;
        if (nwhole > 0) {
          issue_tile<A, InT, K>(p, rp, t0_of(0), T - t0_of(0), buf_a);
          if constexpr (kChunk) win = window_in<A, InT, (WPR > 1)>(p, rp, T, carry);
          for (;;) {
            {
              finish_tile<A, InT, K>(p, rp, t0_of(c), buf_a);
              const int64_t cn = c + 1 < nwhole ? c + 1 : c;
              issue_tile<A, InT, K>(p, rp, t0_of(cn), T - t0_of(cn), buf_b);
              carry = tile_compute<A, InT, K, LPR, WPR, false, kChunk, kLoopEarly>(
                  p, rp, buf_a, t0_of(c), T - t0_of(c), row_ok, c, c + 1 < ntiles, lane, wave, carry,
                  s_agg, m, win, write_window);
            }
            if (++c == nwhole) break;
            {
              finish_tile<A, InT, K>(p, rp, t0_of(c), buf_b);
              const int64_t cn = c + 1 < nwhole ? c + 1 : c;
              issue_tile<A, InT, K>(p, rp, t0_of(cn), T - t0_of(cn), buf_a);
              carry = tile_compute<A, InT, K, LPR, WPR, false, kChunk, kLoopEarly>(
                  p, rp, buf_b, t0_of(c), T - t0_of(c), row_ok, c, c + 1 < ntiles, lane, wave, carry,
                  s_agg, m, win, write_window);
            }
            if (++c == nwhole) break;
          }
        }
        if (ragged) {
          const int64_t te0 = t0_of(ntiles - 1);
          const int64_t lim = row_ok ? (T - te0 > 0 ? T - te0 : 0) : 0;
          Tile<K> x;
          load_edge<A, InT, K>(p, rp, te0, lim, T, x);
          if constexpr (kChunk) {
            if (nwhole == 0) win = window_in<A, InT, (WPR > 1)>(p, rp, T, carry);
          }
          tile_compute<A, InT, K, LPR, WPR, true, kChunk, kLoopEarly>(p, rp, x, te0, lim, row_ok, ntiles - 1,
                                                          false, lane, wave, carry, s_agg, m, win,
                                                          write_window);
        }
        return;
      }
      int64_t c = ragged ? ntiles - 2 : ntiles - 1;  // latest whole tile
      // Two explicit buffers, alternating: tile c is decoded (and its sparse
      // bootstrap loads issued) before tile c-1's loads are issued into the other
      // buffer, then tile c is computed.  In-order load completion then lets the
      // computation of tile c wait for tile c only, and no register copies are
      // needed between iterations.  The prefetch is unconditional (no branch for
      // the wait-count analysis to merge): after tile 0 it re-reads tile 0, which
      // was just loaded (cache hits, never used).
      Tile<K> buf_a, buf_b;
      if (c >= 0) issue_tile<A, InT, K>(p, rp, t0_of(c), T - t0_of(c), buf_a);
      if (ragged) {
        const int64_t te0 = t0_of(ntiles - 1);
        const int64_t lim = row_ok ? (T - te0 > 0 ? T - te0 : 0) : 0;
        Tile<K> x;
        load_edge<A, InT, K>(p, rp, te0, lim, T, x);
        if constexpr (kChunk) win = window_in<A, InT, (WPR > 1)>(p, rp, T, carry);
        carry = tile_compute<A, InT, K, LPR, WPR, true, kChunk, kLoopEarly>(p, rp, x, te0, lim, row_ok,
                                                                ntiles - 1, c >= 0, lane, wave, carry,
                                                                s_agg, m, win, write_window);
      } else {
        if constexpr (kChunk) win = window_in<A, InT, (WPR > 1)>(p, rp, T, carry);
      }
      if (c < 0) return;
      for (;;) {
        {
          finish_tile<A, InT, K>(p, rp, t0_of(c), buf_a);
          const int64_t cn = c > 0 ? c - 1 : 0;
          issue_tile<A, InT, K>(p, rp, t0_of(cn), T - t0_of(cn), buf_b);
          carry = tile_compute<A, InT, K, LPR, WPR, false, kChunk, kLoopEarly>(
              p, rp, buf_a, t0_of(c), T - t0_of(c), row_ok, c, c > 0, lane, wave, carry, s_agg, m,
              win, write_window);
        }
        if (c == 0) break;
        --c;
        {
          finish_tile<A, InT, K>(p, rp, t0_of(c), buf_b);
          const int64_t cn = c > 0 ? c - 1 : 0;
          issue_tile<A, InT, K>(p, rp, t0_of(cn), T - t0_of(cn), buf_a);
          carry = tile_compute<A, InT, K, LPR, WPR, false, kChunk, kLoopEarly>(
              p, rp, buf_b, t0_of(c), T - t0_of(c), row_ok, c, c > 0, lane, wave, carry, s_agg, m,
              win, write_window);
        }
        if (c == 0) break;
        --c;
      }
    }
  }
}

}  // namespace rlca
