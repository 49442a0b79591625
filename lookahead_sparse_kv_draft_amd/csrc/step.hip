// One layer's decode step (OasisKV explainer, Figure 8: at step t the layer's
// attention runs over the resident part of S_t while the draft queries predict
// S_{t+1}; selection, diff and transfer follow).  The attention and the
// lookahead scoring need only step t's inputs and neither reads the other's
// output, so they can share a launch; the attention's split combine is small
// and rides with whatever launch follows the attention.
//
// Two launches (default shape):
//   1. attention (split partials) and scoring in ONE grid: the scoring streams
//      while the attention is in its latency-bound start and tail,
//   2. top-k selection and the resident-set diff, with the split combine in
//      the workgroups after the selection's.
// Three launches (other shapes): attention; combine + scoring; select + diff.
#include "attn_body.h"
#include "attn_combine.h"
#include "score_body.h"

namespace oasis {
namespace {

// Workgroups [0, ncomb_wg) merge four query rows each; the rest are scoring
// workgroups of four wavefronts.
template <int D, int RT, int SMAX>
__global__ __launch_bounds__(256) void combine_score_kernel(
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml, float* __restrict__ out, int arows,
    int splits, int comb_total, int ncomb_wg, const uint16_t* __restrict__ q, const uint16_t* __restrict__ meta,
    const int32_t* __restrict__ ctx_len, float* __restrict__ scores, int H, int G, int T, int ndraft, int rows,
    int Nmax, int wpu, int tpw, int total_waves) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  if (static_cast<int>(blockIdx.x) < ncomb_wg) {
    attn_combine_row<D, SMAX>(ws_acc, ws_ml, out, arows, splits, comb_total, blockIdx.x * 4 + wv, lane);
    return;
  }
  score_wave<D, RT>(q, meta, ctx_len, scores, H, G, T, ndraft, 1, rows, Nmax, wpu, tpw, total_waves,
                    (blockIdx.x - ncomb_wg) * 4 + wv, lane);
}

// One page of another layer's fetch list, copied from the device-mapped pinned
// host tier into that layer's pool by one workgroup of NT threads: all reads of
// a batch issued before its writes.  Entries beyond n_fetch and entries out of
// range are skipped, as in the standalone gather.
template <int NT>
__device__ __forceinline__ void gather_page(const StepGather& g, int Nmax, int kb, int page16, int entry, int unit) {
  constexpr int kBatch = 4;
  const int nf = g.n_fetch[unit];
  if (entry >= nf || entry >= g.cap) return;
  const int b = g.fetch[(static_cast<size_t>(unit) * g.cap + entry) * 2];
  const int s = g.fetch[(static_cast<size_t>(unit) * g.cap + entry) * 2 + 1];
  if (b < 0 || b >= Nmax || s < 0 || s >= kb) return;
  const uint4* src = g.host + (static_cast<size_t>(unit) * Nmax + b) * page16;
  uint4* dst = g.pool + (static_cast<size_t>(unit) * kb + s) * page16;
  for (int c0 = 0; c0 < page16; c0 += NT * kBatch) {
    uint4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = c0 + u * NT + static_cast<int>(threadIdx.x);
      if (c < page16) v[u] = src[c];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = c0 + u * NT + static_cast<int>(threadIdx.x);
      if (c < page16) dst[c] = v[u];
    }
  }
}

// Attention (2-page ring) and scoring workgroups in one grid of workgroups of
// W wavefronts (W = 2, or 4 for up to two attention row tiles), led by
// n_gather_wg workgroups that move another layer's fetched pages (one per
// fetch entry and unit; none without a transfer): the host-link reads start
// with the launch and overlap its HBM-bound work.
// order 0: attention workgroups first; 1: scoring first; 2: interleaved one for
// one while both last.
template <int D, int RTA, int RTS, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu((RTA <= 3 && RTS <= 2) ? 2 : 1))) void attn_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ pool, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ b2s, const int32_t* __restrict__ attend, const int32_t* __restrict__ n_attend,
    const int32_t* __restrict__ ctx_attn, float* __restrict__ ws_acc, float* __restrict__ ws_ml,
    float* __restrict__ out, int H, int arows, int Nmax, int kb, int splits, int run, float scale_log2,
    const uint16_t* __restrict__ meta, const int32_t* __restrict__ ctx_score, float* __restrict__ scores, int G,
    int T, int ndraft, int srows, int wpu, int tpw, int total_waves, int n_attn_wg, int n_score_wg, int order,
    StepGather gather, int n_gather_wg, int page16) {
  if (static_cast<int>(blockIdx.x) < n_gather_wg) {
    const int units = n_gather_wg / gather.cap;
    gather_page<64 * W>(gather, Nmax, kb, page16, blockIdx.x / units, blockIdx.x % units);
    return;
  }
  const int bid = blockIdx.x - n_gather_wg;
  bool is_attn;
  int idx;
  if (order == 0) {
    is_attn = bid < n_attn_wg;
    idx = is_attn ? bid : bid - n_attn_wg;
  } else if (order == 1) {
    is_attn = bid >= n_score_wg;
    idx = is_attn ? bid - n_score_wg : bid;
  } else {
    const int m = min(n_attn_wg, n_score_wg);
    if (bid < 2 * m) {
      is_attn = (bid & 1) == 0;
      idx = bid >> 1;
    } else {
      is_attn = n_attn_wg > m;
      idx = m + (bid - 2 * m);
    }
  }
  if (is_attn) {
    attn_wg<D, RTA, W, 2>(q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, H, arows, Nmax, kb,
                          splits, run, scale_log2, idx);
  } else {
    score_wave<D, RTS>(q, meta, ctx_score, scores, H, G, T, ndraft, 1, srows, Nmax, wpu, tpw, total_waves,
                       idx * W + static_cast<int>(threadIdx.x) / kWave, threadIdx.x & (kWave - 1));
  }
}

template <int D, int RTA, int RTS, int W>
hipError_t as_t(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                const int32_t* attend, const int32_t* n_attend, const int32_t* ctx_attn, float* ws_acc,
                float* ws_ml, float* out, const void* meta, const int32_t* ctx_score, float* scores,
                const StepGather& g, hipStream_t st) {
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  const int n_attn_wg = c.units * c.attn_splits;
  const int wpu = score_waves_per_unit(c);
  const int total = c.units * wpu;
  const int n_score_wg = (total + W - 1) / W;
  const int n_gather_wg = (g.host != nullptr && g.cap > 0) ? g.cap * c.units : 0;
  const int page16 = static_cast<int>(c.page_elems * c.elem_bytes / 16);
  hipLaunchKernelGGL((attn_score_kernel<D, RTA, RTS, W>), dim3(n_gather_wg + n_attn_wg + n_score_wg), dim3(64 * W), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(pool), sel, b2s, attend,
                     n_attend, ctx_attn, ws_acc, ws_ml, out, c.s.kv_heads, c.rows_attn, c.s.max_blocks,
                     c.s.budget_blocks, c.attn_splits, c.attn_run, scale_log2, static_cast<const uint16_t*>(meta),
                     ctx_score, scores, c.s.group, c.T, c.s.n_draft, c.rows_score, wpu, c.score_tpw, total,
                     n_attn_wg, n_score_wg, c.step_order, g, n_gather_wg, page16);
  return hipGetLastError();
}

template <int D, int RTA, int W>
hipError_t as_s(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                const int32_t* attend, const int32_t* n_attend, const int32_t* ctx_attn, float* ws_acc,
                float* ws_ml, float* out, const void* meta, const int32_t* ctx_score, float* scores,
                const StepGather& g, hipStream_t st) {
  switch ((c.rows_score + 15) / 16) {
    case 1: return as_t<D, RTA, 1, W>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, st);
    case 2: return as_t<D, RTA, 2, W>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, st);
    case 3: return as_t<D, RTA, 3, W>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, st);
    default: return as_t<D, RTA, 4, W>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, st);
  }
}

template <int D>
hipError_t as_d(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                const int32_t* attend, const int32_t* n_attend, const int32_t* ctx_attn, float* ws_acc,
                float* ws_ml, float* out, const void* meta, const int32_t* ctx_score, float* scores,
                const StepGather& g, hipStream_t st) {
  const bool w4 = c.attn_waves == 4;
  switch ((c.rows_attn + 15) / 16) {
    case 1: return w4 ? as_s<D, 1, 4>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, st)
                      : as_s<D, 1, 2>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, st);
    case 2: return w4 ? as_s<D, 2, 4>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, st)
                      : as_s<D, 2, 2>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, st);
    default: return as_s<D, 3, 2>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, st);
  }
}

template <int D, int RT, int SMAX>
hipError_t cs_t(const Ctx& c, const float* ws_acc, const float* ws_ml, float* out, const void* q,
                const void* meta, const int32_t* ctx_len, float* scores, hipStream_t st) {
  const int comb_total = c.units * c.rows_attn;
  const int ncomb_wg = (comb_total + 3) / 4;
  const int wpu = score_waves_per_unit(c);
  const int total = c.units * wpu;
  const int grid = ncomb_wg + (total + 3) / 4;
  hipLaunchKernelGGL((combine_score_kernel<D, RT, SMAX>), dim3(grid), dim3(256), 0, st, ws_acc, ws_ml, out,
                     c.rows_attn, c.attn_splits, comb_total, ncomb_wg, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(meta), ctx_len, scores, c.s.kv_heads, c.s.group, c.T,
                     c.s.n_draft, c.rows_score, c.s.max_blocks, wpu, c.score_tpw, total);
  return hipGetLastError();
}

template <int D, int RT>
hipError_t cs_s(const Ctx& c, const float* ws_acc, const float* ws_ml, float* out, const void* q,
                const void* meta, const int32_t* ctx_len, float* scores, hipStream_t st) {
  const int S = c.attn_splits;
  if (S <= 4) return cs_t<D, RT, 4>(c, ws_acc, ws_ml, out, q, meta, ctx_len, scores, st);
  if (S <= 8) return cs_t<D, RT, 8>(c, ws_acc, ws_ml, out, q, meta, ctx_len, scores, st);
  if (S <= 16) return cs_t<D, RT, 16>(c, ws_acc, ws_ml, out, q, meta, ctx_len, scores, st);
  return cs_t<D, RT, 32>(c, ws_acc, ws_ml, out, q, meta, ctx_len, scores, st);
}

template <int D>
hipError_t cs_d(const Ctx& c, const float* ws_acc, const float* ws_ml, float* out, const void* q,
                const void* meta, const int32_t* ctx_len, float* scores, hipStream_t st) {
  switch ((c.rows_score + 15) / 16) {
    case 1: return cs_s<D, 1>(c, ws_acc, ws_ml, out, q, meta, ctx_len, scores, st);
    case 2: return cs_s<D, 2>(c, ws_acc, ws_ml, out, q, meta, ctx_len, scores, st);
    case 3: return cs_s<D, 3>(c, ws_acc, ws_ml, out, q, meta, ctx_len, scores, st);
    default: return cs_s<D, 4>(c, ws_acc, ws_ml, out, q, meta, ctx_len, scores, st);
  }
}

}  // namespace

bool attn_and_score_fused_available(const Ctx& c) {
  return c.s.dtype == OASIS_BF16 && c.attn_pf == 2 && c.rows_attn <= 48 &&
         (c.attn_waves == 2 || (c.attn_waves == 4 && c.rows_attn <= 32));
}

hipError_t launch_attn_and_score(const Ctx& c, const void* q, const void* pool, const int32_t* sel,
                                 const int32_t* b2s, const int32_t* attend, const int32_t* n_attend,
                                 const int32_t* ctx_attn, float* out, void* ws, const void* meta,
                                 const int32_t* ctx_score, float* scores, hipStream_t st, const StepGather& g) {
  if (!attn_and_score_fused_available(c)) return hipErrorInvalidValue;
  float* ws_acc = static_cast<float*>(ws);
  float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + attn_ws_acc_bytes(c));
  return c.s.head_dim == 128
             ? as_d<128>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score,
                         scores, g, st)
             : as_d<64>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score,
                        scores, g, st);
}

hipError_t launch_combine_and_score(const Ctx& c, void* ws, float* out, const void* q, const void* meta,
                                   const int32_t* ctx_len, float* scores, hipStream_t st) {
  if (c.s.dtype != OASIS_BF16) return hipErrorInvalidValue;
  const float* ws_acc = static_cast<const float*>(ws);
  const float* ws_ml = reinterpret_cast<const float*>(static_cast<const char*>(ws) + attn_ws_acc_bytes(c));
  return c.s.head_dim == 128 ? cs_d<128>(c, ws_acc, ws_ml, out, q, meta, ctx_len, scores, st)
                             : cs_d<64>(c, ws_acc, ws_ml, out, q, meta, ctx_len, scores, st);
}

}  // namespace oasis
