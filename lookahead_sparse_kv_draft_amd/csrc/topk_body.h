// The latency-oriented top-k of one unit by one workgroup of NT threads, every
// thread holding at most KPT keys in registers (candidate c lives in slot
// c / NT of thread c % NT).  Shared by the selection kernels (NT = 512 or 1024,
// one workgroup per unit) and by the decode step's first launch when it carries
// another layer's selection (NT = 128, one workgroup per unit).  The ranking is
// the total order (descending score, ascending block index) with -0.0 ranked as
// +0.0; the sink block and the newest block are forced (OasisKV explainer,
// Figure 7 right: the draft query predicts the next step's top-K blocks).
//
// Serial chains and instruction counts are what cost time in a kernel this
// small (two wavefronts per SIMD issue about one instruction each per four
// cycles), so each step is spread over all threads and the bookkeeping that is
// the same for every thread is kept in scalar registers:
//   * the radix digits are 10 bits (1024 histogram bins, 1024 / NT consecutive
//     bins per thread) taken from the highest bit where the keys differ (block
//     min/max), so the first pass already spreads the keys; the search stops as
//     soon as the bin holding the m-th key can be taken whole: when its keys
//     are exactly the ones still needed, or when they fit the winner list
//     beside the keys above it (the ranking then keeps the first m), so one
//     pass is the rule;
//   * winners are appended with one LDS atomic per wavefront (ballot counts);
//     ties at the threshold, when a bin is not taken whole, are ranked in index
//     order with a workgroup scan;
//   * each winner's output position is the number of smaller winners, counted
//     with unrolled broadcast reads of the winner list.
#pragma once

#include "diff_body.h"

namespace oasis {

constexpr int kTkThreads = 1024;  // the selection kernels' workgroup
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkBins = 1024;     // histogram bins of a radix pass (10-bit digits)
constexpr int kTkMaxWin = 512;

template <int NT>
struct TopkFastShared {
  int hist[kTkBins];
  int start[kTkBins + 1];  // first pass: keys in the bins before each bin
  unsigned long long win[kTkMaxWin];
  uint32_t wlo[NT / kWave], whi[NT / kWave];
  int wtot[NT / kWave];
  int bin, before, cnt, nwin;
};

// Inclusive sum over the NT threads and the block total (two barriers; with
// TRAIL = false the second one, which protects wtot for the next call, is left
// to the caller).
template <int NT, bool TRAIL = true>
__device__ __forceinline__ int tk_incl_sum(int v, int* wtot, int* total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_incl_sum(v);
  if (lane == kWave - 1) wtot[w] = v;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int x = wtot[i];
    off += (i < w) ? x : 0;
    tot += x;
  }
  if (TRAIL) __syncthreads();
  *total = tot;
  return v + off;
}

// The bin holding the rem-th key of the histogram (sh.bin, the keys in the
// bins before it sh.before, its own count sh.cnt; exactly one bin qualifies
// when 1 <= rem <= the histogram's total), with each bin's exclusive prefix
// recorded in sh.start when START; the histogram is cleared for a next pass.
// Ends with a barrier.
template <int NT, bool START>
__device__ __forceinline__ void tk_find_bin(TopkFastShared<NT>& sh, int rem) {
  constexpr int BPT = kTkBins / NT;
  const int tid = threadIdx.x;
  int hv[BPT];
  int hsum = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    hv[i] = sh.hist[tid * BPT + i];
    hsum += hv[i];
  }
  int unused_total;
  const int incl = tk_incl_sum<NT, false>(hsum, sh.wtot, &unused_total);  // the barrier below protects wtot
  int excl = incl - hsum;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int bin = tid * BPT + i;
    if (START) sh.start[bin] = excl;
    if (excl < rem && excl + hv[i] >= rem) {
      sh.bin = bin;
      sh.before = excl;
      sh.cnt = hv[i];
    }
    excl += hv[i];
    sh.hist[bin] = 0;
  }
  if (START && tid == NT - 1) sh.start[kTkBins] = incl;
  __syncthreads();
}

// x through an empty asm statement: a value the compiler cannot see through,
// so that indices built from it are recomputed where they are used instead of
// being kept live across the whole selection (with many keys per thread the
// hoisted indices of every key would spill).
template <bool OPAQUE>
__device__ __forceinline__ int fresh_copy(int x) {
  if constexpr (OPAQUE) asm volatile("" : "+v"(x));
  return x;
}

// This thread's candidate scores (candidate c = block c + 1) from the unit's
// score row su.  Issued first by every caller: every index below Nmax is in
// bounds, and the context length, which arrives later, decides which keys take
// part.
template <int NT, int KPT>
__device__ __forceinline__ void topk_fast_load(const float* __restrict__ su, int Nmax, float (&v)[KPT]) {
#pragma unroll
  for (int u = 0; u < KPT; ++u) v[u] = su[min(u * NT + static_cast<int>(threadIdx.x) + 1, Nmax - 1)];
}

// The selection of unit `unit` from the scores topk_fast_load returned and the
// request's context length n (read by the caller before anything else, so its
// round trip overlaps the scores'); written to sel and, in rank order and -1
// padded, to the LDS array selL when it is not null.  With the LDS table
// slot_of (block -> slot, -1 = none; complete on entry) the ranking also
// records what the resident-set diff needs of each selected block, while it
// holds it: slot_keys (one entry per slot) receives the order key of the block
// each slot holds, before any early return (the diff ranks eviction victims by
// the same keys); selS (rank order, -1 padded) the slot of each selected block;
// selF (one byte per slot, cleared by the caller) 1 for each slot that holds a
// selected block.
template <int NT, int KPT>
__device__ __forceinline__ void topk_fast_body(const float (&v)[KPT], int n, int unit, int32_t* __restrict__ sel,
                                               int Nmax, int kb, int32_t* selL, TopkFastShared<NT>& sh,
                                               const int8_t* slot_of = nullptr, uint32_t* slot_keys = nullptr,
                                               int8_t* selS = nullptr, uint8_t* selF = nullptr) {
  constexpr int NW = NT / kWave;
  constexpr int BPT = kTkBins / NT;  // consecutive histogram bins per thread
  static_assert(BPT * NT == kTkBins, "the bins are spread evenly over the threads");
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int N = max(1, min((n + kBlock - 1) / kBlock, Nmax));
  const int F0 = (N == 1) ? 1 : 2;
  const int C = max(0, N - 2);  // candidates are blocks 1 .. N-2
  const int m = min(kb - F0, C);
  int32_t* out = sel + static_cast<size_t>(unit) * kb;
  // a selected block's slot, recorded at rank position pos
  auto note_slot = [&](int pos, int blk) {
    if (selS != nullptr) {
      const int s = slot_of[blk];
      selS[pos] = static_cast<int8_t>(s);
      if (s >= 0) selF[s] = 1;
    }
  };
  // the forced blocks: lane 0 block 0, lane 1 the newest block
  if (tid < F0) {
    const int blk = (tid == 0) ? 0 : N - 1;
    out[tid] = blk;
    if (selL != nullptr) selL[tid] = blk;
    note_slot(tid, blk);
  }
  for (int i = F0 + max(m, 0) + tid; i < kb; i += NT) {
    out[i] = -1;
    if (selL != nullptr) selL[i] = -1;
    if (selS != nullptr) selS[i] = -1;
  }
  // Candidate u * NT + t (t = this thread) takes part when below C; each phase
  // below takes its own copy of t, through which the indices and these tests
  // are recomputed rather than held (with more than 8 keys per thread).
  constexpr bool kFresh = KPT > 8;
  auto valid = [&](int u, int t) { return u * NT + t < C; };
  uint32_t key[KPT];
  {
    const int t = fresh_copy<kFresh>(tid);
#pragma unroll
    for (int u = 0; u < KPT; ++u) key[u] = valid(u, t) ? desc_key(v[u]) : 0xFFFFFFFFu;
  }
  if (slot_keys != nullptr) {
    // table reads four at a time (indices clamped), then their writes
    constexpr int SB = KPT < 4 ? KPT : 4;
    const int t1 = fresh_copy<kFresh>(tid) + 1;
#pragma unroll
    for (int u0 = 0; u0 < KPT; u0 += SB) {
      int so[SB];
#pragma unroll
      for (int j = 0; j < SB; ++j) so[j] = slot_of[min((u0 + j) * NT + t1, Nmax - 1)];
#pragma unroll
      for (int j = 0; j < SB; ++j)
        if ((u0 + j) * NT + t1 < Nmax && so[j] >= 0) slot_keys[so[j]] = key[u0 + j];
    }
  }
  if (m <= 0) return;  // uniform: every thread leaves together

  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  const int tr = fresh_copy<kFresh>(tid);
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    if (valid(u, tr)) {
      lo = min(lo, key[u]);
      hi = max(hi, key[u]);
    }
  }
  {
    uint32_t a0, a1, b0, b1;  // lanes ^ 32 and ^ 16 through the lane swaps
    lane_pair32(lo, a0, a1);
    lane_pair32(hi, b0, b1);
    lo = min(a0, a1);
    hi = max(b0, b1);
    lane_pair16(lo, a0, a1);
    lane_pair16(hi, b0, b1);
    lo = min(a0, a1);
    hi = max(b0, b1);
  }
  // then across each row by DPP (lane ^ 1, ^ 2, the half-row and row mirrors)
  lo = min(lo, static_cast<uint32_t>(dpp_from<0xB1>(static_cast<int>(lo))));
  hi = max(hi, static_cast<uint32_t>(dpp_from<0xB1>(static_cast<int>(hi))));
  lo = min(lo, static_cast<uint32_t>(dpp_from<0x4E>(static_cast<int>(lo))));
  hi = max(hi, static_cast<uint32_t>(dpp_from<0x4E>(static_cast<int>(hi))));
  lo = min(lo, static_cast<uint32_t>(dpp_from<0x141>(static_cast<int>(lo))));
  hi = max(hi, static_cast<uint32_t>(dpp_from<0x141>(static_cast<int>(hi))));
  lo = min(lo, static_cast<uint32_t>(dpp_from<0x140>(static_cast<int>(lo))));
  hi = max(hi, static_cast<uint32_t>(dpp_from<0x140>(static_cast<int>(hi))));
  if (lane == 0) {
    sh.wlo[w] = lo;
    sh.whi[w] = hi;
  }
#pragma unroll
  for (int i = 0; i < BPT; ++i) sh.hist[tid * BPT + i] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    lo = min(lo, sh.wlo[i]);
    hi = max(hi, sh.whi[i]);
  }
  // every lane now holds the workgroup's range: say so to the compiler, so the
  // radix bookkeeping below stays in scalar registers
  lo = __builtin_amdgcn_readfirstlane(lo);
  hi = __builtin_amdgcn_readfirstlane(hi);
  // Radix select on d = key - lo in [0, hi - lo]: the selection is every key
  // with d < base plus `rem` keys of the current bin range.
  const uint32_t range = hi - lo;
  const int width = (range == 0u) ? 0 : 32 - __clz(static_cast<int>(range));
  const int shift0 = max(width - 10, 0);
  // from here on the keys are held as d = key - lo (the same order over the
  // candidates); the winner list holds d << 32 | block, so the original keys
  // need not stay live beside them
  uint32_t(&d)[KPT] = key;
#pragma unroll
  for (int u = 0; u < KPT; ++u) d[u] -= lo;
  // First pass: 1024 bins over the whole range (every d >> shift0 is a bin).
  {
    const int t = fresh_copy<kFresh>(tid);
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      if (valid(u, t)) atomicAdd(&sh.hist[d[u] >> shift0], 1);
  }
  __syncthreads();
  tk_find_bin<NT, true>(sh, m);
  int tbin = __builtin_amdgcn_readfirstlane(sh.bin);
  int rem = m - __builtin_amdgcn_readfirstlane(sh.before);
  int tcnt = __builtin_amdgcn_readfirstlane(sh.cnt);
  const uint64_t below = (1ull << lane) - 1ull;
  // The bin is taken whole when its keys are exactly the ones still needed, or
  // when the winners so far plus the whole bin fit the winner list: the rank
  // counting below then keeps the first m of them (the bin's keys rank after
  // every key above the bin).
  if (tcnt == rem || m - rem + tcnt <= kTkMaxWin) {
    // One pass was enough (the rule): the winners are the keys of bins
    // 0 .. tbin.  Each key goes to its bin's range of the winner list
    // (counting-sort scatter, the cleared histogram as cursors), and its output
    // position is the number of keys in earlier bins plus its rank inside its
    // own bin, so only keys that share a bin are compared.
    const int ncoll = m - rem + tcnt;
    const uint32_t lim = (static_cast<uint32_t>(tbin) << shift0) + ((1u << shift0) - 1u);  // last d of bin tbin
    const int t = fresh_copy<kFresh>(tid);
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      if (valid(u, t) && d[u] <= lim) {
        const int bk = static_cast<int>(d[u] >> shift0);
        sh.win[sh.start[bk] + atomicAdd(&sh.hist[bk], 1)] =
            (static_cast<unsigned long long>(d[u]) << 32) | static_cast<uint32_t>(u * NT + t + 1);
      }
    }
    __syncthreads();
    for (int wi = tid; wi < ncoll; wi += NT) {
      const unsigned long long mine = sh.win[wi];
      const int bk = static_cast<int>(static_cast<uint32_t>(mine >> 32) >> shift0);
      const int b0 = sh.start[bk], b1 = sh.start[bk + 1];
      const int r = b0 + rank_below(sh.win + b0, b1 - b0, mine, 1, 0);
      if (r < m) {
        const int blk = static_cast<int32_t>(mine & 0xFFFFFFFFull);  // block index = candidate + 1
        out[F0 + r] = blk;
        if (selL != nullptr) selL[F0 + r] = blk;
        note_slot(F0 + r, blk);
      }
    }
    return;
  }
  // Further passes of 10-bit digits inside the threshold bin, until its bin can
  // be taken whole or a single key value remains (ties at the threshold).
  uint32_t base = static_cast<uint32_t>(tbin) << shift0;
  int shift = shift0;
  bool exact = false;
  int ncoll = m;  // keys the collection below gathers
  while (shift > 0) {
    shift = max(shift - 10, 0);
    const uint64_t span = 1ull << (shift + 10);
    const int t = fresh_copy<kFresh>(tid);
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      if (valid(u, t) && d[u] >= base && static_cast<uint64_t>(d[u] - base) < span)
        atomicAdd(&sh.hist[static_cast<int>((d[u] - base) >> shift)], 1);
    }
    __syncthreads();
    tk_find_bin<NT, false>(sh, rem);
    tbin = __builtin_amdgcn_readfirstlane(sh.bin);
    rem -= __builtin_amdgcn_readfirstlane(sh.before);
    tcnt = __builtin_amdgcn_readfirstlane(sh.cnt);
    base += static_cast<uint32_t>(tbin) << shift;
    if (tcnt == rem || m - rem + tcnt <= kTkMaxWin) {
      ncoll = m - rem + tcnt;
      base += static_cast<uint32_t>((1ull << shift) - 1ull);
      exact = true;
      break;
    }
  }
  // Collect winners: d < base (d <= base when exact) with one atomic per wavefront.
  if (tid == 0) sh.nwin = 0;
  __syncthreads();
  const int tc = fresh_copy<kFresh>(tid);
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const bool win = valid(u, tc) && (exact ? d[u] <= base : d[u] < base);
    const uint64_t bw = __ballot(win);
    if (bw) {
      int wbase = 0;
      if (lane == 0) wbase = atomicAdd(&sh.nwin, __popcll(bw));
      wbase = __builtin_amdgcn_readlane(wbase, 0);
      if (win)
        sh.win[wbase + __popcll(bw & below)] =
            (static_cast<unsigned long long>(d[u]) << 32) | static_cast<uint32_t>(u * NT + tc + 1);
    }
  }
  if (!exact) {
    // ties at d == base: the first `rem` in index order (u, then thread)
    int taken = 0;
    const int n_lt = m - rem;
    const int te = fresh_copy<kFresh>(tid);
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const bool eq = valid(u, te) && d[u] == base;
      int tot;
      const int r = tk_incl_sum<NT>(eq ? 1 : 0, sh.wtot, &tot) - (eq ? 1 : 0);
      if (eq && taken + r < rem)
        sh.win[n_lt + taken + r] =
            (static_cast<unsigned long long>(d[u]) << 32) | static_cast<uint32_t>(u * NT + te + 1);
      taken += tot;
    }
  }
  __syncthreads();
  // Output position = number of smaller winners (all keys distinct by index),
  // counted by P adjacent threads per winner and summed across their lanes;
  // with more winners than NT / P, in rounds of NT / P winners.
  const int nw = ncoll;  // the m winners, and with a whole threshold bin the rest of its keys
  const int P = (nw * 16 <= NT) ? 16 : (nw * 8 <= NT) ? 8 : (nw * 4 <= NT) ? 4 : (nw * 2 <= NT) ? 2 : 1;
  for (int w0 = 0; w0 < nw; w0 += NT / P) {  // uniform: every lane of a group takes part
    const int wi = w0 + tid / P, part = tid & (P - 1);
    const unsigned long long mine = sh.win[min(wi, nw - 1)];
    const int r = rank_below(sh.win, nw, mine, P, part);
    if (part == 0 && wi < nw && r < m) {
      const int blk = static_cast<int32_t>(mine & 0xFFFFFFFFull);  // block index = candidate + 1
      out[F0 + r] = blk;
      if (selL != nullptr) selL[F0 + r] = blk;
      note_slot(F0 + r, blk);
    }
  }
}

}  // namespace oasis
