// Top-k block selection per (request, KV head): the sink block 0 and the newest
// block are always kept (attention sinks are among the works the OasisKV pages
// build on), then the best-scoring other blocks fill the budget of k blocks
// (OasisKV explainer, Figure 7 right: the draft query predicts the next step's
// top-K blocks).  Ranking is the total order (descending score, ascending block
// index) with -0.0 ranked as +0.0.
//
// One 256-thread workgroup per unit, latency-oriented (the whole launch moves
// well under a megabyte):
//   1. the candidates' 32-bit order keys are staged once in LDS;
//   2. a 3-pass radix select (11, 11, 10-bit digits) finds the key T of the
//      m-th best candidate; each pass counts digits with LDS atomics and one
//      wavefront scans the 2048 bins, so a pass costs two barriers;
//   3. candidates with key < T and those equal to T are collected with LDS
//      atomics (if very many keys equal T, an ordered ballot pass takes the
//      lowest indices instead);
//   4. the rank of each collected (key, index) pair is the number of smaller
//      pairs, which places it directly in the output (rank counting instead of
//      a sorting network); equal keys rank by index, so ties go to the lower
//      index.
//
// Fast path (N <= 8192 blocks, k <= 512): one 1024-thread workgroup per unit,
// every thread holding at most 8 keys in registers (candidate c lives in slot
// c / 1024 of thread c % 1024).  Serial chains are what cost time in a kernel
// this small, so each step is spread over all threads:
//   * the radix digits are 10 bits (one histogram bin per thread) taken from the
//     highest bit where the keys differ (block min/max), so the first pass
//     already spreads the keys; the search stops as soon as the bin holding the
//     m-th key can be taken whole: when its keys are exactly the ones still
//     needed, or when they fit the winner list beside the keys above it (the
//     ranking then keeps the first m), so one pass is the rule;
//   * winners are appended with one LDS atomic per wavefront (ballot counts);
//     ties at the threshold, when a bin is not taken whole, are ranked in index
//     order with a workgroup scan;
//   * each winner's output position is the number of smaller winners, counted
//     with unrolled broadcast reads of the winner list.
#include "block_ops.h"
#include "attn_combine.h"
#include "diff_body.h"
#include "select_wg.h"
#include "topk_body.h"

namespace oasis {
namespace {

constexpr int kBins = 2048;

struct TopkShared {
  int hist[2][kBins];
  int wave_tot[kWavesPerWG];
  int digit, rem, n_lt, n_eq;
};

__global__ __launch_bounds__(256) void topk_wg_kernel(const float* __restrict__ scores,
                                                   const int32_t* __restrict__ ctx_len,
                                                   int32_t* __restrict__ sel, int H, int Nmax,
                                                   int kb, int cap_list, int keys_in_lds) {
  extern __shared__ unsigned long long dyn[];
  unsigned long long* list = dyn;                                 // [cap_list]
  uint32_t* keys = reinterpret_cast<uint32_t*>(list + cap_list);  // [Nmax] if keys_in_lds
  __shared__ TopkShared sh;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  const int n = ctx_len[unit / H];
  const int N = max(1, min((n + kBlock - 1) / kBlock, Nmax));
  const int F0 = (N == 1) ? 1 : 2;
  const int C = max(0, N - 2);  // candidates are blocks 1 .. N-2
  const int m = min(kb - F0, C);
  int32_t* out = sel + static_cast<size_t>(unit) * kb;
  const float* sc = scores + static_cast<size_t>(unit) * Nmax;
  if (tid == 0) {
    out[0] = 0;
    if (N > 1) out[1] = N - 1;
  }
  for (int i = F0 + max(m, 0) + tid; i < kb; i += kWG) out[i] = -1;
  if (m <= 0) return;

  // 1. keys of candidate c = block c + 1, loaded 8 per thread at a time so the
  //    loads are in flight together (indices clamped: no branch around a load)
  if (keys_in_lds) {
    for (int c0 = 0; c0 < C; c0 += 8 * kWG) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = sc[min(c0 + u * kWG + tid, C - 1) + 1];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u * kWG + tid;
        if (c < C) keys[c] = desc_key(v[u]);
      }
    }
  }
  auto key_of = [&](int c) -> uint32_t { return keys_in_lds ? keys[c] : desc_key(sc[c + 1]); };
  for (int i = tid; i < kBins; i += kWG) sh.hist[0][i] = 0;
  __syncthreads();

  // 2. radix select over the digits (11, 11, 10 bits from the top)
  uint32_t prefix = 0u, mask = 0u;
  int rem = m;
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    const int shift = (p == 0) ? 21 : (p == 1) ? 10 : 0;
    const uint32_t dmask = (p == 2) ? 0x3FFu : 0x7FFu;
    int* hist = sh.hist[p & 1];
    int* next = sh.hist[(p + 1) & 1];
    for (int c = tid; c < C; c += kWG) {
      const uint32_t key = key_of(c);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1);
    }
    for (int i = tid; i < kBins; i += kWG) next[i] = 0;  // cleared for the next pass
    __syncthreads();
    if (tid < kWave) {
      // lane covers bins [32 * lane, 32 * lane + 32)
      const int lane = tid;
      int part[32];
      int s = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        part[j] = hist[32 * lane + j];
        s += part[j];
      }
      const int incl = wave_incl_sum(s);  // the whole wavefront takes part
      const int excl = incl - s;
      if (excl < rem && incl >= rem) {  // exactly one lane: the m-th key is in its bins
        int acc = excl;
        bool found = false;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          if (!found && acc + part[j] >= rem) {
            found = true;
            sh.digit = 32 * lane + j;
            sh.rem = rem - acc;
          }
          acc += part[j];
        }
      }
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(sh.digit) << shift;
    mask |= dmask << shift;
    rem = sh.rem;
  }
  const uint32_t Tkey = prefix;
  const int need_eq = rem;       // candidates equal to Tkey to take, lowest index first
  const int n_lt = m - need_eq;  // candidates strictly better than Tkey

  // 3. collect: key < T into list[0 .. n_lt), key == T after them
  if (tid == 0) {
    sh.n_lt = 0;
    sh.n_eq = 0;
  }
  __syncthreads();
  const int eq_room = cap_list - n_lt;
  for (int c = tid; c < C; c += kWG) {
    const uint32_t key = key_of(c);
    if (key < Tkey) {
      const int pos = atomicAdd(&sh.n_lt, 1);
      if (pos < n_lt)
        list[pos] = (static_cast<unsigned long long>(key) << 32) | static_cast<uint32_t>(c + 1);
    } else if (key == Tkey) {
      const int pos = atomicAdd(&sh.n_eq, 1);
      if (pos < eq_room)
        list[n_lt + pos] = (static_cast<unsigned long long>(key) << 32) | static_cast<uint32_t>(c + 1);
    }
  }
  __syncthreads();
  int total = n_lt + min(sh.n_eq, eq_room);
  if (sh.n_eq > eq_room) {
    // Very many ties at T: take the lowest-index ones with an ordered ballot pass.
    int base = 0;
    for (int c0 = 0; c0 < C && base < need_eq; c0 += kWG) {
      const int c = c0 + tid;
      const bool eq = c < C && key_of(c) == Tkey;
      int tot;
      const int rank = wg_rank_of_flag(eq, &tot, sh.wave_tot);
      if (eq && base + rank < need_eq)
        list[n_lt + base + rank] = (static_cast<unsigned long long>(Tkey) << 32) | static_cast<uint32_t>(c + 1);
      base += tot;
    }
    total = m;
    __syncthreads();
  }

  // 4. rank counting: the output position of each pair is the number of smaller pairs
  for (int i = tid; i < total; i += kWG) {
    const unsigned long long v = list[i];
    int r = 0;
    for (int j = 0; j < total; ++j) r += (list[j] < v) ? 1 : 0;
    if (r < m) out[F0 + r] = static_cast<int32_t>(v & 0xFFFFFFFFull);
  }
}



template <int KPT>
__global__ __launch_bounds__(1024) void topk_fast_kernel(const float* __restrict__ scores,
                                                         const int32_t* __restrict__ ctx_len,
                                                         int32_t* __restrict__ sel, int H, int Nmax, int kb) {
  __shared__ TopkFastShared<kTkThreads> sh;
  const int n = ctx_len[blockIdx.x / H];
  float v[KPT];
  topk_fast_load<kTkThreads, KPT>(scores + static_cast<size_t>(blockIdx.x) * Nmax, Nmax, v);
  topk_fast_body<kTkThreads, KPT>(v, n, blockIdx.x, sel, Nmax, kb, nullptr, sh);
}

// Dynamic LDS of the fused selection + diff for budgets above 128 blocks: the
// diff's arrays and the selection (k ints).
inline size_t select_diff_lds_bytes(int kb, int Nmax, int cap) {
  return diff_lds_bytes(kb, Nmax, cap) + static_cast<size_t>(kb) * 4;
}

// Fused selection + diff of one unit by a 1024-thread workgroup, for budgets
// above 128 blocks (select_wg.h covers the rest): the selection's score loads
// go out first, the diff's loads behind them stay in flight through the
// selection, which reaches the diff through LDS; every wavefront takes part in
// the diff (diff_body).
template <int KPT>
__device__ __forceinline__ void select_diff_unit(
    const float* __restrict__ scores, const int32_t* __restrict__ ctx_len, int32_t* __restrict__ sel,
    int32_t* __restrict__ b2s, int32_t* __restrict__ s2b, int32_t* __restrict__ fetch,
    int32_t* __restrict__ n_fetch, int32_t* __restrict__ evict, int32_t* __restrict__ attend,
    int32_t* __restrict__ n_attend, int H, int Nmax, int kb, int cap, unsigned long long* smem_u64,
    TopkFastShared<kTkThreads>& sh, DiffShared& dsh) {
  int32_t* selL = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(smem_u64) + diff_lds_bytes(kb, Nmax, cap));
  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  int32_t* bu = b2s + static_cast<size_t>(unit) * Nmax;
  int32_t* slu = s2b + static_cast<size_t>(unit) * kb;
  const float* su = scores + static_cast<size_t>(unit) * Nmax;
  // Loads in the order that keeps one round trip before the selection starts:
  // the scores and the slot map (independent), then the context length, then
  // the scores of the resident blocks (which need the slot map).
  float v[KPT];
  topk_fast_load<kTkThreads, KPT>(su, Nmax, v);
  const int sb = slu[min(tid, kb - 1)];  // clamped: no branch around the loads
  const int n = ctx_len[unit / H];
  __builtin_amdgcn_sched_barrier(0);
  const bool sok = sb >= 0 && sb < Nmax;
  const float sv = su[sok ? sb : 0];
  topk_fast_body<kTkThreads, KPT>(v, n, unit, sel, Nmax, kb, selL, sh);
  __syncthreads();
  diff_body(unit, kb, Nmax, cap, selL, sb, sv, bu, slu, fetch, n_fetch, evict, attend, n_attend, smem_u64, dsh);
}

template <int KPT>
__global__ __launch_bounds__(1024) void select_diff_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ ctx_len, int32_t* __restrict__ sel,
    int32_t* __restrict__ b2s, int32_t* __restrict__ s2b, int32_t* __restrict__ fetch,
    int32_t* __restrict__ n_fetch, int32_t* __restrict__ evict, int32_t* __restrict__ attend,
    int32_t* __restrict__ n_attend, int H, int Nmax, int kb, int cap) {
  extern __shared__ unsigned long long smem_u64[];
  __shared__ TopkFastShared<kTkThreads> sh;
  __shared__ DiffShared dsh;
  select_diff_unit<KPT>(scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, H, Nmax, kb, cap,
                        smem_u64, sh, dsh);
}

// The same in workgroups [0, units), then the attention's split combine,
// sixteen query rows per workgroup, in the rest.
template <int KPT, int D, int SMAX>
__global__ __launch_bounds__(1024) void select_diff_combine_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ ctx_len, int32_t* __restrict__ sel,
    int32_t* __restrict__ b2s, int32_t* __restrict__ s2b, int32_t* __restrict__ fetch,
    int32_t* __restrict__ n_fetch, int32_t* __restrict__ evict, int32_t* __restrict__ attend,
    int32_t* __restrict__ n_attend, int H, int Nmax, int kb, int cap, int units,
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml, float* __restrict__ out, int arows,
    int splits, int comb_total) {
  if (static_cast<int>(blockIdx.x) >= units) {
    attn_combine_row<D, SMAX>(ws_acc, ws_ml, out, arows, splits, comb_total,
                              (blockIdx.x - units) * kTkWaves + threadIdx.x / kWave, threadIdx.x & (kWave - 1));
    return;
  }
  extern __shared__ unsigned long long smem_u64[];
  __shared__ TopkFastShared<kTkThreads> sh;
  __shared__ DiffShared dsh;
  select_diff_unit<KPT>(scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, H, Nmax, kb, cap,
                        smem_u64, sh, dsh);
}

template <int KPT, int D, int SMAX>
hipError_t sdc_t(const Ctx& c, const float* scores, const int32_t* ctx_len, int32_t* sel, int32_t* b2s,
                 int32_t* s2b, int32_t* fetch, int32_t* n_fetch, int32_t* evict, int32_t* attend,
                 int32_t* n_attend, const float* ws_acc, const float* ws_ml, float* out, hipStream_t st) {
  const int kb = c.s.budget_blocks, cap = c.s.fetch_cap;
  const size_t lds = select_diff_lds_bytes(kb, c.s.max_blocks, cap);
  const int comb_total = c.units * c.rows_attn;
  const int ncomb = (comb_total + kTkWaves - 1) / kTkWaves;
  hipLaunchKernelGGL((select_diff_combine_kernel<KPT, D, SMAX>), dim3(c.units + ncomb), dim3(kTkThreads), lds, st,
                     scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, c.s.kv_heads,
                     c.s.max_blocks, kb, cap, c.units, ws_acc, ws_ml, out, c.rows_attn, c.attn_splits, comb_total);
  return hipGetLastError();
}

template <int KPT, int D>
hipError_t sdc_s(const Ctx& c, const float* scores, const int32_t* ctx_len, int32_t* sel, int32_t* b2s,
                 int32_t* s2b, int32_t* fetch, int32_t* n_fetch, int32_t* evict, int32_t* attend,
                 int32_t* n_attend, const float* ws_acc, const float* ws_ml, float* out, hipStream_t st) {
  const int S = c.attn_splits;
  if (S <= 4) return sdc_t<KPT, D, 4>(c, scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, ws_acc, ws_ml, out, st);
  if (S <= 8) return sdc_t<KPT, D, 8>(c, scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, ws_acc, ws_ml, out, st);
  if (S <= 16) return sdc_t<KPT, D, 16>(c, scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, ws_acc, ws_ml, out, st);
  return sdc_t<KPT, D, 32>(c, scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, ws_acc, ws_ml, out, st);
}

template <int KPT>
hipError_t sdc_d(const Ctx& c, const float* scores, const int32_t* ctx_len, int32_t* sel, int32_t* b2s,
                 int32_t* s2b, int32_t* fetch, int32_t* n_fetch, int32_t* evict, int32_t* attend,
                 int32_t* n_attend, const float* ws_acc, const float* ws_ml, float* out, hipStream_t st) {
  return c.s.head_dim == 128
             ? sdc_s<KPT, 128>(c, scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, ws_acc, ws_ml, out, st)
             : sdc_s<KPT, 64>(c, scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, ws_acc, ws_ml, out, st);
}

// ---- budgets of at most 128 blocks: one workgroup selection per unit ----
// (select_wg.h), alone, or with the attention's split combine (NT / 64 query
// rows per workgroup) in the workgroups after the units'.
template <int NT, int KPT, bool LRU>
__global__ __launch_bounds__(NT) void select_wg_kernel(SelectJob job, int H, int Nmax, int kb, int cap) {
  __shared__ SelectLds<NT> lds;
  select_diff_wg<NT, KPT, LRU>(job, blockIdx.x, H, Nmax, kb, cap, lds);
}

template <int NT, int KPT, bool LRU, int D, int SMAX>
__global__ __launch_bounds__(NT) void select_wg_combine_kernel(SelectJob job, int units, int H, int Nmax, int kb,
                                                               int cap, const float* __restrict__ ws_acc,
                                                               const float* __restrict__ ws_ml,
                                                               float* __restrict__ out, int arows, int splits,
                                                               int comb_total) {
  __shared__ SelectLds<NT> lds;
  if (static_cast<int>(blockIdx.x) < units) {
    select_diff_wg<NT, KPT, LRU>(job, blockIdx.x, H, Nmax, kb, cap, lds);
    return;
  }
  attn_combine_row<D, SMAX>(ws_acc, ws_ml, out, arows, splits, comb_total,
                            (blockIdx.x - units) * (NT / kWave) + threadIdx.x / kWave, threadIdx.x & (kWave - 1));
}

// Workgroup size by keys per unit: 512 threads up to 2048 blocks, 1024 beyond
// (measured in the decode step at 2048 and 8192 blocks).
#define OASIS_SWG_BY_SIZE(LAUNCH)                \
  do {                                           \
    const int N = c.s.max_blocks;                \
    if (N <= 512) { LAUNCH(512, 1); }            \
    if (N <= 1024) { LAUNCH(512, 2); }           \
    if (N <= 2048) { LAUNCH(512, 4); }           \
    if (N <= 4096) { LAUNCH(1024, 4); }          \
    LAUNCH(1024, 8);                             \
  } while (0)

template <bool LRU, int D, int SMAX>
hipError_t swg_t(const Ctx& c, const SelectJob& job, const float* ws_acc, const float* ws_ml, float* out,
                 int comb_total, hipStream_t st) {
#define OASIS_SWGC(NT, KPT)                                                                                     \
  hipLaunchKernelGGL((select_wg_combine_kernel<NT, KPT, LRU, D, SMAX>),                                          \
                     dim3(c.units + (comb_total + NT / kWave - 1) / (NT / kWave)), dim3(NT), 0, st, job, c.units, \
                     c.s.kv_heads, c.s.max_blocks, c.s.budget_blocks, c.s.fetch_cap, ws_acc, ws_ml, out,        \
                     c.rows_attn, c.attn_splits, comb_total);                                                   \
  return hipGetLastError()
  OASIS_SWG_BY_SIZE(OASIS_SWGC);
#undef OASIS_SWGC
}

template <bool LRU>
hipError_t swg_alone(const Ctx& c, const SelectJob& job, hipStream_t st) {
#define OASIS_SWGA(NT, KPT)                                                                                 \
  hipLaunchKernelGGL((select_wg_kernel<NT, KPT, LRU>), dim3(c.units), dim3(NT), 0, st, job, c.s.kv_heads,   \
                     c.s.max_blocks, c.s.budget_blocks, c.s.fetch_cap);                                      \
  return hipGetLastError()
  OASIS_SWG_BY_SIZE(OASIS_SWGA);
#undef OASIS_SWGA
}
#undef OASIS_SWG_BY_SIZE

template <bool LRU>
hipError_t swg_l(const Ctx& c, const SelectJob& job, const void* ws, float* out, bool combine, hipStream_t st) {
  if (!combine) return swg_alone<LRU>(c, job, st);
  const float* ws_acc = static_cast<const float*>(ws);
  const float* ws_ml = reinterpret_cast<const float*>(static_cast<const char*>(ws) + attn_ws_acc_bytes(c));
  const int comb_total = c.units * c.rows_attn;
  const int S = c.attn_splits;
  if (c.s.head_dim == 128) {
    if (S <= 4) return swg_t<LRU, 128, 4>(c, job, ws_acc, ws_ml, out, comb_total, st);
    if (S <= 8) return swg_t<LRU, 128, 8>(c, job, ws_acc, ws_ml, out, comb_total, st);
    if (S <= 16) return swg_t<LRU, 128, 16>(c, job, ws_acc, ws_ml, out, comb_total, st);
    return swg_t<LRU, 128, 32>(c, job, ws_acc, ws_ml, out, comb_total, st);
  }
  if (S <= 4) return swg_t<LRU, 64, 4>(c, job, ws_acc, ws_ml, out, comb_total, st);
  if (S <= 8) return swg_t<LRU, 64, 8>(c, job, ws_acc, ws_ml, out, comb_total, st);
  if (S <= 16) return swg_t<LRU, 64, 16>(c, job, ws_acc, ws_ml, out, comb_total, st);
  return swg_t<LRU, 64, 32>(c, job, ws_acc, ws_ml, out, comb_total, st);
}

hipError_t swg_d(const Ctx& c, const SelectJob& job, const void* ws, float* out, bool combine, hipStream_t st) {
  return job.last_use != nullptr ? swg_l<true>(c, job, ws, out, combine, st)
                                 : swg_l<false>(c, job, ws, out, combine, st);
}

SelectJob job_of(const float* scores, const int32_t* ctx_len, int32_t* sel, int32_t* b2s, int32_t* s2b,
                 int32_t* fetch, int32_t* n_fetch, int32_t* evict, int32_t* attend, int32_t* n_attend,
                 const LruState& lru) {
  SelectJob j;
  j.scores = scores;
  j.ctx_len = ctx_len;
  j.sel = sel;
  j.b2s = b2s;
  j.s2b = s2b;
  j.fetch = fetch;
  j.n_fetch = n_fetch;
  j.evict = evict;
  j.attend = attend;
  j.n_attend = n_attend;
  j.last_use = lru.last_use;
  j.step = lru.step;
  return j;
}

template <int KPT>
hipError_t fast_t(const Ctx& c, const float* scores, const int32_t* ctx_len, int32_t* sel, hipStream_t st) {
  hipLaunchKernelGGL((topk_fast_kernel<KPT>), dim3(c.units), dim3(kTkThreads), 0, st, scores, ctx_len, sel,
                     c.s.kv_heads, c.s.max_blocks, c.s.budget_blocks);
  return hipGetLastError();
}

template <int KPT>
hipError_t select_diff_t(const Ctx& c, const float* scores, const int32_t* ctx_len, int32_t* sel, int32_t* b2s,
                         int32_t* s2b, int32_t* fetch, int32_t* n_fetch, int32_t* evict, int32_t* attend,
                         int32_t* n_attend, hipStream_t st) {
  const int kb = c.s.budget_blocks, cap = c.s.fetch_cap;
  const size_t lds = select_diff_lds_bytes(kb, c.s.max_blocks, cap);
  hipLaunchKernelGGL((select_diff_kernel<KPT>), dim3(c.units), dim3(kTkThreads), lds, st, scores, ctx_len, sel,
                     b2s, s2b, fetch, n_fetch, evict, attend, n_attend, c.s.kv_heads, c.s.max_blocks, kb, cap);
  return hipGetLastError();
}

}  // namespace

bool select_wg_available(const Ctx& c) {
  return c.s.budget_blocks <= kDiffWaveMaxBudget && c.s.max_blocks <= kSelWgMaxBlocks;
}

bool select_diff_fused_available(const Ctx& c) {
  return select_wg_available(c) || (c.s.budget_blocks - 2 <= kTkMaxWin && c.s.max_blocks <= 8 * kTkThreads);
}

bool select_diff_lru_available(const Ctx& c) { return select_wg_available(c); }

hipError_t launch_select_diff(const Ctx& c, const float* scores, const int32_t* ctx_len, int32_t* sel,
                              int32_t* b2s, int32_t* s2b, int32_t* fetch, int32_t* n_fetch, int32_t* evict,
                              int32_t* attend, int32_t* n_attend, hipStream_t st, LruState lru) {
  if (select_wg_available(c))
    return swg_d(c, job_of(scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, lru), nullptr,
                 nullptr, false, st);
  if (lru.last_use != nullptr) return hipErrorInvalidValue;
  const int kpt = (c.s.max_blocks + kTkThreads - 1) / kTkThreads;
  if (kpt <= 1) return select_diff_t<1>(c, scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, st);
  if (kpt <= 2) return select_diff_t<2>(c, scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, st);
  if (kpt <= 4) return select_diff_t<4>(c, scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, st);
  return select_diff_t<8>(c, scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, st);
}

hipError_t launch_select_diff_combine(const Ctx& c, const float* scores, const int32_t* ctx_len, int32_t* sel,
                                      int32_t* b2s, int32_t* s2b, int32_t* fetch, int32_t* n_fetch, int32_t* evict,
                                      int32_t* attend, int32_t* n_attend, const void* ws, float* out,
                                      hipStream_t st, LruState lru) {
  if (select_wg_available(c))
    return swg_d(c, job_of(scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, lru), ws, out,
                 true, st);
  if (lru.last_use != nullptr) return hipErrorInvalidValue;
  const float* ws_acc = static_cast<const float*>(ws);
  const float* ws_ml = reinterpret_cast<const float*>(static_cast<const char*>(ws) + attn_ws_acc_bytes(c));
  const int kpt = (c.s.max_blocks + kTkThreads - 1) / kTkThreads;
  if (kpt <= 1) return sdc_d<1>(c, scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, ws_acc, ws_ml, out, st);
  if (kpt <= 2) return sdc_d<2>(c, scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, ws_acc, ws_ml, out, st);
  if (kpt <= 4) return sdc_d<4>(c, scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, ws_acc, ws_ml, out, st);
  return sdc_d<8>(c, scores, ctx_len, sel, b2s, s2b, fetch, n_fetch, evict, attend, n_attend, ws_acc, ws_ml, out, st);
}

hipError_t launch_topk(const Ctx& c, const float* scores, const int32_t* ctx_len, int32_t* sel,
                       hipStream_t st) {
  if (c.s.budget_blocks - 2 <= kTkMaxWin) {
    const int kpt = (c.s.max_blocks + kTkThreads - 1) / kTkThreads;  // keys per thread
    if (kpt <= 1) return fast_t<1>(c, scores, ctx_len, sel, st);
    if (kpt <= 2) return fast_t<2>(c, scores, ctx_len, sel, st);
    if (kpt <= 4) return fast_t<4>(c, scores, ctx_len, sel, st);
    if (kpt <= 8) return fast_t<8>(c, scores, ctx_len, sel, st);
  }
  int P = 1;
  while (P < c.s.budget_blocks) P <<= 1;
  const int cap_list = 2 * P;  // the m winners plus room for ties at the threshold
  // Stage the keys in LDS when everything fits in 60 KiB; otherwise read scores each pass.
  const size_t fixed = sizeof(int) * (2 * 2048 + 8) + static_cast<size_t>(cap_list) * 8;
  const int keys_in_lds = (fixed + static_cast<size_t>(c.s.max_blocks) * 4 <= 60 * 1024) ? 1 : 0;
  const size_t lds = static_cast<size_t>(cap_list) * sizeof(unsigned long long) +
                     (keys_in_lds ? static_cast<size_t>(c.s.max_blocks) * sizeof(uint32_t) : 0);
  hipLaunchKernelGGL(topk_wg_kernel, dim3(c.units), dim3(kWG), lds, st, scores, ctx_len, sel,
                     c.s.kv_heads, c.s.max_blocks, c.s.budget_blocks, cap_list, keys_in_lds);
  return hipGetLastError();
}

}  // namespace oasis
