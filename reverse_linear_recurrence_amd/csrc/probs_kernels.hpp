// probs_kernels.hpp -- Retrace(lambda) and V-trace from the policies'
// log-probability tables (rl-triton, Results: the heavier Retrace workload
// loads the action probabilities at every step).
//
// The per-step quantities the scan needs are formed on chip from [N, T(+1), A]
// tables, then the scan core of scan_kernels.hpp (tile_compute) runs as for
// rlca_retrace / rlca_vtrace:
//   log_rho_t = log_pi[t][a_t] - log_mu[t][a_t]
//   Retrace: q_taken_t = q[t][a_t] and
//            EQ_t = sum over a of exp(log_pi[t+1][a]) * q[t+1][a]
//            (after a truncation that is not a termination: trunc_eq[t]).
//
// Mapping.  One 256-thread workgroup (4 wavefronts) per row; each thread owns
// K = 4 consecutive steps of a 1024-step tile, tiles visited from the last to
// the first, with the multi-wavefront scan of scan_kernels.hpp.  For each
// tile the workgroup first streams the tables' slices with coalesced 16-byte
// loads (thread i taking elements 4i .. 4i+3, 4(i+256) .., and so on), keeps
// the taken action's entries in LDS and, for Retrace, sums exp(log_pi) * q per
// slice: each lane's parts are combined with its neighbours' across a 16-lane
// row (DPP) and one lane per slice and row adds the result into that slice's
// LDS accumulator.  Streaming whole tables moves fewer bytes than gathering
// one entry per slice would, because every gathered entry costs a whole
// memory line.  Each thread then reads its steps' quantities from LDS.
#pragma once

#include "scan_kernels.hpp"

namespace rlca {

// The tables of the policy-table entry points.  Row strides ld_* are in
// elements; a table row holds its slices contiguously, A entries each.
struct TableArgs {
  int64_t A;
  const void *q;       int64_t ld_q;    // [N, T+1, A]            (Retrace)
  const int32_t *act;  int64_t ld_act;  // [N, T]
  const void *lpi;     int64_t ld_lpi;  // [N, T+1, A] Retrace, [N, T, A] V-trace
  const void *lmu;     int64_t ld_lmu;  // [N, T, A], or [N, T] when mu_taken
  const void *teq;     int64_t ld_teq;  // [N, T], read at truncations (Retrace)
  int mu_taken;                         // log_mu holds the taken actions' entries only
};

constexpr int kProbsK = 4;
constexpr int kProbsThreads = 256;                  // threads per workgroup
constexpr int kProbsUnroll = 2;                     // table chunks in flight per thread
// Two tilings: WPR = 4 wavefronts share one row (1024-step tiles, one row per
// workgroup) for long rows; WPR = 1, one wavefront per row (256-step tiles,
// four rows per workgroup) for rows of at most 256 steps.

// Slice and entry of element e of a tile's table span (A entries per slice):
// a float reciprocal estimate, corrected to the exact quotient.  A span holds
// at most 1025 slices of at most 65536 entries, so e fits in 32 bits; the
// estimate is within one of the quotient.
__device__ __forceinline__ void slice_of(int e, int A, float inv_a, int &sl, int &a) {
  const int q = static_cast<int>((static_cast<float>(e) + 0.5f) * inv_a);
  const int r = e - q * A;
  const bool lo = r < 0, hi = r >= A;
  sl = lo ? q - 1 : (hi ? q + 1 : q);
  a = lo ? r + A : (hi ? r - A : r);
}

// Entry k (0..3) of a chunk of four, k a run-time value, as a select chain.
__device__ __forceinline__ float pick4(float v0, float v1, float v2, float v3, int k) {
  float r = v0;
  r = k == 1 ? v1 : r;
  r = k == 2 ? v2 : r;
  r = k == 3 ? v3 : r;
  return r;
}

// Pass four register values through an empty asm.  The compiler then treats
// them as opaque, so select chains over them stay selects: otherwise a chain
// indexed by a run-time value can become an indexed load from a private
// array, which lives in scratch memory.
__device__ __forceinline__ void opaque4(float &v0, float &v1, float &v2, float &v3) {
  asm("" : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3));
}

// DPP row_shr:D within 16-lane rows: lane l of a row gets lane l - D's
// value, lanes without a source get `old`.
template <int D>
__device__ __forceinline__ float row_shr(float src, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src),
                                                     0x110 + D, 0xf, 0xf, false));
}
template <int D>
__device__ __forceinline__ int row_shr(int src, int old) {
  return __builtin_amdgcn_update_dpp(old, src, 0x110 + D, 0xf, 0xf, false);
}

// One level of the segmented inclusive sum within 16-lane rows: slices never
// decrease across lanes, so a lane D below with the same slice heads a run of
// lanes that all share it.
template <int D>
__device__ __forceinline__ void seg_level(float &run, int key) {
  const float v = row_shr<D>(run, 0.f);
  const int k = row_shr<D>(key, -1);
  run = k == key ? run + v : run;
}

// The vector part of stream_slices: chunks of four consecutive elements.
// Each thread keeps kProbsUnroll chunks in flight: as soon as it has used a
// chunk it issues the load of the chunk one round later into the same
// registers (past the end, a re-read of chunk 0, unused).  Rounds are counted
// per wavefront, so every lane of a wavefront runs every round (lanes past
// the end with nothing to add).
//
// kWide (A >= 4): a chunk holds the end of at most one slice, so it is handled
// without branches per element: the slice sl of its first entry a0 covers
// entries k < A - a0 and slice sl + 1 the rest; each slice's taken entry sits
// at a known position in the chunk (or outside it).  With kSum, a lane's part
// of slice sl + 1 moves to the next lane (which starts in that slice), the
// parts of each slice are summed across the lanes of a 16-lane row (DPP), and
// only the row's last lane of each slice adds into LDS: adjacent lanes share
// slices, and LDS atomics on one address serialize.  Otherwise (A < 4) the
// chunk walks its elements one by one with one LDS atomic per run.
template <int kGroup, typename InT, bool kOther, bool kSum, bool kWide>
__device__ __forceinline__ void stream_chunks(const InT *tab, const InT *other, int nvec, int A,
                                              float inv_a, const int *acts, float *taken,
                                              float *taken_other, float *acc, int tid) {
  if (nvec == 0) return;
  constexpr int kRound = kGroup * kProbsUnroll;  // chunks per round of the workgroup
  const int lane = tid & 63;
  const bool row_end = (lane & 15) == 15;
  float tv[kProbsUnroll][4], ov[kProbsUnroll][4] = {};  // ov: the second table (kOther)
  auto issue = [&](int u, int c) {
    const int idx = c < nvec ? c : 0;  // in range
    Ld<InT>::template vec<4, true>(tab + 4 * static_cast<int64_t>(idx), tv[u]);
    if constexpr (kOther) Ld<InT>::template vec<4, true>(other + 4 * static_cast<int64_t>(idx), ov[u]);
  };
#pragma unroll
  for (int u = 0; u < kProbsUnroll; ++u) issue(u, tid + kGroup * u);
  for (int i0 = tid; i0 - lane < nvec; i0 += kRound) {
#pragma unroll
    for (int u = 0; u < kProbsUnroll; ++u) {
      const int c = i0 + kGroup * u;
      const bool live = c < nvec;
      if constexpr (kWide) {
        int sl = -1, split = 4;
        float run0 = 0.f, run1 = 0.f;
        if (live) {
          int a;
          slice_of(4 * c, A, inv_a, sl, a);
          float t0 = tv[u][0], t1 = tv[u][1], t2 = tv[u][2], t3 = tv[u][3];
          float o0 = ov[u][0], o1 = ov[u][1], o2 = ov[u][2], o3 = ov[u][3];
          opaque4(t0, t1, t2, t3);
          if constexpr (kOther) opaque4(o0, o1, o2, o3);
          split = A - a;               // entries k < split belong to slice sl
          const bool two = split < 4;  // slice sl + 1 starts inside the chunk
          // Position in the chunk of each slice's taken entry; an action
          // outside [0, A) lands outside the slice's range and stores nothing.
          const int k0 = acts[sl] - a;
          int k1 = 4;
          if (two) k1 = split + acts[sl + 1];
          if (k0 >= 0 && k0 < split && k0 < 4) {
            taken[sl] = pick4(t0, t1, t2, t3, k0);
            if constexpr (kOther) taken_other[sl] = pick4(o0, o1, o2, o3, k0);
          }
          if (k1 >= split && k1 < 4) {
            taken[sl + 1] = pick4(t0, t1, t2, t3, k1);
            if constexpr (kOther) taken_other[sl + 1] = pick4(o0, o1, o2, o3, k1);
          }
          if constexpr (kSum) {
            // Each slice's part summed in element order.
            auto add = [&](float t, float o, int k) {
              const float e = __expf(t);
              const float f0 = fmaf(e, o, run0);
              const float f1 = fmaf(e, o, run1);
              const bool first = k < split;
              run0 = first ? f0 : run0;
              run1 = first ? run1 : f1;
            };
            add(t0, o0, 0);
            add(t1, o1, 1);
            add(t2, o2, 2);
            add(t3, o3, 3);
          }
        }
        if constexpr (kSum) {
          // Every lane of the wavefront is active here.  A lane whose chunk
          // ends inside slice sl + 1 hands that part to the next lane, which
          // starts in slice sl + 1, unless the next lane is in the next row
          // or past the end.
          const bool next_live = c + 1 < nvec;
          const bool keep1 = split < 4 && (row_end || !next_live);
          run0 += row_shr<1>(split < 4 ? run1 : 0.f, 0.f);
          if (A + 3 > 4) seg_level<1>(run0, sl);
          if (A + 3 > 8) seg_level<2>(run0, sl);
          if (A + 3 > 16) seg_level<4>(run0, sl);
          if (A + 3 > 32) seg_level<8>(run0, sl);
          // The last lane of its slice in the row adds the row's part.
          const bool tail = live && (split <= 4 || row_end || !next_live);
          if (tail && sl >= 1) atomicAdd(&acc[sl - 1], run0);
          if (live && keep1) atomicAdd(&acc[sl], run1);
        }
      } else if (live) {
        int sl, a;
        slice_of(4 * c, A, inv_a, sl, a);
        int cur = sl;
        float run = 0.f;
        int act = acts[sl];  // the current slice's taken action, read once per slice
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if constexpr (kSum) {
            if (sl != cur) {
              if (cur >= 1) atomicAdd(&acc[cur - 1], run);
              run = 0.f;
              cur = sl;
            }
            run = fmaf(__expf(tv[u][k]), ov[u][k], run);
          }
          if (a == act) {
            taken[sl] = tv[u][k];
            if constexpr (kOther) taken_other[sl] = ov[u][k];
          }
          if (++a == A) {
            a = 0;
            ++sl;
            if (k < 3) act = acts[sl];
          }
        }
        if constexpr (kSum) {
          if (cur >= 1) atomicAdd(&acc[cur - 1], run);
        }
      }
      issue(u, c + kRound);
    }
  }
}

// Stream slices [0, nsl) of one table row span (tile-relative), A entries
// each, with the whole workgroup; kOther: a second table over the same span
// alongside.  Every element whose entry is the slice's taken action is
// stored to taken[slice] (and the second table's to taken_other[slice]);
// with kSum, exp(this table's entry) times the second table's entry is added
// into acc[slice - 1] (the expectation of the step before the slice); the
// parts are combined across lanes first (stream_chunks), so that few LDS
// atomics go out per slice.
template <int kGroup, typename InT, bool kOther, bool kSum>
__device__ __forceinline__ void stream_slices(const InT *tab, const InT *other, int nsl,
                                              int64_t A, float inv_a, const int *acts,
                                              float *taken, float *taken_other, float *acc,
                                              int tid) {
  static_assert(kOther || !kSum, "the sum needs the second table");
  const int A32 = static_cast<int>(A);
  const int nel = nsl * A32;  // at most 1025 * 65536 < 2^31
  const int nvec = nel / 4;
  if (A32 >= 4)
    stream_chunks<kGroup, InT, kOther, kSum, true>(tab, other, nvec, A32, inv_a, acts, taken,
                                                   taken_other, acc, tid);
  else
    stream_chunks<kGroup, InT, kOther, kSum, false>(tab, other, nvec, A32, inv_a, acts, taken,
                                                    taken_other, acc, tid);
  for (int e = 4 * nvec + tid; e < nel; e += kGroup) {
    int sl, a;
    slice_of(e, A32, inv_a, sl, a);
    const float v = Ld<InT>::one(tab + e);
    float o = 0.f;
    if constexpr (kOther) o = Ld<InT>::one(other + e);
    if constexpr (kSum) {
      if (sl >= 1) atomicAdd(&acc[sl - 1], __expf(v) * o);
    }
    if (a == acts[sl]) {
      taken[sl] = v;
      if constexpr (kOther) taken_other[sl] = o;
    }
  }
}

// kChunk: window instance (carry vector in; carry and carry map out, as in
// scan_kernel).
template <int Algo, typename InT, int WPR, bool kChunk>
__global__ void __launch_bounds__(kProbsThreads)
probs_kernel(const Args p, const TableArgs ta) {
  static_assert(Algo == kRetrace || Algo == kVtrace, "policy tables: Retrace or V-trace");
  static_assert(WPR == 1 || WPR == 4, "one or four wavefronts per row");
#ifdef RLCA_TIMESTAMPS
  const WaveStamp stamp{p.stamps, wall_clock()};  // written at every return
#endif
  constexpr int K = kProbsK;
  constexpr int kGroup = 64 * WPR;            // threads per row
  constexpr int kTile = kGroup * K;           // steps per tile
  constexpr int kRows = kProbsThreads / kGroup;  // rows per workgroup
  // Per row and tile slice (slot kTile: the slice after the tile): the
  // expectation, the taken q, log_pi and log_mu, and the action.
  __shared__ float s_eq_all[kRows][kTile + 1];
  __shared__ float s_qt_all[kRows][kTile + 1];
  __shared__ float s_lp_all[kRows][kTile + 1];
  __shared__ float s_lm_all[kRows][kTile + 1];
  __shared__ int s_act_all[kRows][kTile + 1];
  __shared__ float2 s_agg[2][WPR];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tid = WPR > 1 ? static_cast<int>(threadIdx.x) : lane;  // thread within the row
  const int slot = WPR > 1 ? 0 : wave;                               // the row's LDS arrays
  float *s_eq = s_eq_all[slot];
  float *s_qt = s_qt_all[slot];
  float *s_lp = s_lp_all[slot];
  float *s_lm = s_lm_all[slot];
  int *s_act = s_act_all[slot];
  const int64_t N = p.N, T = p.T, A = ta.A;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRows + (WPR > 1 ? 0 : wave);
  // Rows past N (last workgroup) read row 0 and store nothing; they take part
  // in every barrier.
  const bool row_ok = row < N;
  const int64_t rr = row_ok ? row : 0;

  RowPtrs<InT> rp;
  rp.row = rr;
  rp.src = rr;
  rp.seg_off = 0;
  rp.r = static_cast<const InT *>(p.r) + rr * p.ld_r;
  rp.v = Algo == kVtrace ? static_cast<const InT *>(p.v) + rr * p.ld_v : nullptr;
  rp.lr = rp.eq = rp.tv = nullptr;
  rp.te = p.term + rr * p.ld_term;
  rp.tr = p.trunc + rr * p.ld_trunc;
  rp.has_te = p.term != nullptr;
  rp.has_tr = p.trunc != nullptr;
  rp.dense_tv = false;
  const int32_t *act_row = ta.act + rr * ta.ld_act;
  const InT *lpi_row = static_cast<const InT *>(ta.lpi) + rr * ta.ld_lpi;
  const InT *lmu_row = static_cast<const InT *>(ta.lmu) + rr * ta.ld_lmu;
  const InT *q_row = Algo == kRetrace ? static_cast<const InT *>(ta.q) + rr * ta.ld_q : nullptr;
  const float nan = __int_as_float(0x7fc00000);
  const float inv_a = 1.f / static_cast<float>(A);

  const int64_t ntiles = (T + kTile - 1) / kTile;
  const int lane_off = (kGroup - 1 - tid) * K;  // reverse: thread 0 owns the latest steps
  float carry = 0.f;
  if constexpr (kChunk) {
    if (p.cin != nullptr) carry = p.cin[rr];
  }
  CarryMap m{0.f, 1.f};
  WindowIn win{0.f, false};
  // The window results come from the row's last thread in scan order, which
  // owns the row's first steps (its log_rho_0 gives Retrace's c_0).
  const bool write_window = kChunk && row_ok && tid == kGroup - 1;

  for (int64_t c = ntiles - 1; c >= 0; --c) {
    const int64_t ts = c * kTile;
    const int64_t t0 = ts + lane_off;
    const int64_t lim = row_ok ? (T - t0 > 0 ? T - t0 : 0) : 0;
    const bool whole = ts + kTile <= T;
    // Slices of the tile (Retrace: and the slice after it, at most slice T).
    const int nsteps = static_cast<int>(T - ts < kTile ? T - ts : kTile);
    const int nsl = Algo == kRetrace ? nsteps + 1 : nsteps;

    __syncthreads();  // the previous tile's reads of the LDS arrays are done
    for (int i = tid; i < nsl; i += kGroup) {
      const int64_t t = ts + i;
      s_act[i] = t < T ? act_row[t] : -1;
      s_eq[i] = 0.f;
      s_qt[i] = nan;  // taken entries stay NaN for an action outside [0, A)
      s_lp[i] = nan;
      s_lm[i] = nan;
    }
    __syncthreads();
    if constexpr (Algo == kRetrace) {
      stream_slices<kGroup, InT, true, true>(lpi_row + ts * A, q_row + ts * A, nsl, A, inv_a, s_act,
                                     s_lp, s_qt, s_eq, tid);
      // A log_mu table: its slices below T (the slice after the window has
      // no action).
      const int nsl_mu = static_cast<int>(T - ts < nsl ? T - ts : nsl);
      if (!ta.mu_taken)
        stream_slices<kGroup, InT, false, false>(lmu_row + ts * A, nullptr, nsl_mu, A, inv_a, s_act,
                                         s_lm, nullptr, nullptr, tid);
    } else {
      if (ta.mu_taken)
        stream_slices<kGroup, InT, false, false>(lpi_row + ts * A, nullptr, nsl, A, inv_a, s_act, s_lp,
                                         nullptr, nullptr, tid);
      else
        stream_slices<kGroup, InT, true, false>(lpi_row + ts * A, lmu_row + ts * A, nsl, A, inv_a, s_act,
                                        s_lp, s_lm, nullptr, tid);
    }
    __syncthreads();

    // The thread's rewards, flags and (V-trace) values.
    Tile<K> x;
#pragma unroll
    for (int j = 0; j < K; ++j) { x.r[j] = 0.f; x.v[j] = 0.f; x.lr[j] = 0.f; x.eq[j] = 0.f; x.tv[j] = 0.f; }
    x.v[K] = 0.f;
    x.lr[K] = 0.f;
    x.dense = false;
    x.at_start = false;
#pragma unroll
    for (int i = 0; i < K / 4; ++i) { x.te[i] = 0; x.tr[i] = 0; }
    if (whole) {
      Ld<InT>::template vec<K>(rp.r + t0, x.r);
      const uint8_t *own = reinterpret_cast<const uint8_t *>(rp.r + t0);
      ld_flags_raw<K>(rp.has_te ? rp.te + t0 : own, x.fte);
      ld_flags_raw<K>(rp.has_tr ? rp.tr + t0 : own, x.ftr);
      if constexpr (Algo == kVtrace) {
        float vk[K];
        Ld<InT>::template vec<K>(rp.v + t0, vk);
#pragma unroll
        for (int j = 0; j < K; ++j) x.v[j] = vk[j];
        x.v[K] = Ld<InT>::one(rp.v + t0 + K);
      }
      decode_flags<K>(x.fte, x.te);
      decode_flags<K>(x.ftr, x.tr);
#pragma unroll
      for (int i = 0; i < K / 4; ++i) {
        x.te[i] = rp.has_te ? x.te[i] : 0u;
        x.tr[i] = rp.has_tr ? x.tr[i] : 0u;
      }
    } else if (lim > 0) {
      ld_part<InT, K>(rp.r + t0, lim, x.r);
      if (rp.has_te) ld_flags_part<K>(rp.te + t0, lim, x.te);
      if (rp.has_tr) ld_flags_part<K>(rp.tr + t0, lim, x.tr);
      if constexpr (Algo == kVtrace) {
#pragma unroll
        for (int e = 0; e <= K; ++e) x.v[e] = e <= lim ? Ld<InT>::one(rp.v + t0 + e) : 0.f;
      }
    }

    // Behaviour entries given per step (mu_taken): read like the rewards.
    float lmk[K + 1];
#pragma unroll
    for (int j = 0; j <= K; ++j) lmk[j] = 0.f;
    if (ta.mu_taken) {
      if (whole) {
        float v4[K];
        Ld<InT>::template vec<K>(lmu_row + t0, v4);
#pragma unroll
        for (int j = 0; j < K; ++j) lmk[j] = v4[j];
      } else {
        float v4[K];
        ld_part<InT, K>(lmu_row + t0, lim, v4);
#pragma unroll
        for (int j = 0; j < K; ++j) lmk[j] = v4[j];
      }
      if (Algo == kRetrace && lim > K) lmk[K] = Ld<InT>::one(lmu_row + t0 + K);
    }

    // The per-step quantities from LDS: log_rho (and Retrace's neighbour
    // log_rho_{t0+K}, q_taken and the expectation, or the truncation value).
    const int s0 = lane_off;
    const InT *teq_row =
        Algo == kRetrace ? static_cast<const InT *>(ta.teq) + late_v(rr) * ta.ld_teq : nullptr;
#pragma unroll
    for (int j = 0; j <= K; ++j) {
      const bool step = j < lim;
      const bool next = Algo == kRetrace && j == K && lim > K;
      if (step || next) {
        const int s = s0 + j;
        x.lr[j] = s_lp[s] - (ta.mu_taken ? lmk[j] : s_lm[s]);
        if (j < K) {
          if constexpr (Algo == kRetrace) {
            x.v[j] = s_qt[s];
            const bool trunc_only = flag<K>(x.tr, j) && !flag<K>(x.te, j);
            x.eq[j] = trunc_only ? Ld<InT>::one(teq_row + t0 + j) : s_eq[s];
          }
        }
      }
    }
    if constexpr (Algo == kVtrace) sparse_tv<kVtrace, InT, K>(p, rp, t0, x);

    if constexpr (kChunk && Algo == kRetrace) {
      if (c == 0) win.lr0 = x.lr[0];
    }
    if (whole) {
      carry = tile_compute<Algo, InT, K, 64, WPR, false, kChunk>(p, rp, x, t0, T - t0, row_ok, c,
                                                                 c > 0, lane, wave, carry, s_agg,
                                                                 m, win, write_window);
    } else {
      carry = tile_compute<Algo, InT, K, 64, WPR, true, kChunk>(p, rp, x, t0, lim, row_ok, c,
                                                                c > 0, lane, wave, carry, s_agg, m,
                                                                win, write_window);
    }
  }
}

}  // namespace rlca
