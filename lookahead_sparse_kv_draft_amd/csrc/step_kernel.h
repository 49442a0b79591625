// The decode step's first launch (OasisKV explainer, Figure 8: at step t the
// layer's attention runs over the resident part of S_t while the draft queries
// predict S_{t+1}; prediction, selection and transfer of one layer proceed
// while later layers compute): attention workgroups (split partials) and
// lookahead-scoring workgroups in one grid, optionally led by workgroups that
// move another layer's fetched pages and (KPT > 0: keys per selecting thread)
// by workgroups that run another state's top-k selection and resident-set diff
// from scores an earlier launch wrote.  Nothing in the grid waits for anything
// else in it: the carried selection reads and writes only the other state.
#pragma once

#include "attn_body.h"
#include "score_body.h"
#include "select_wg.h"

namespace oasis {
namespace {

// One page of another layer's fetch list, copied from the device-mapped pinned
// host tier into that layer's pool by one workgroup of NT threads, one 16-byte
// read in flight per thread: over the host link, reading two or four chunks
// per thread at once measured slower (more of each step's transfer exposed).
// Entries beyond n_fetch and entries out of range are skipped, as in the
// standalone gather.
template <int NT>
__device__ __forceinline__ void gather_page(const StepGather& g, int Nmax, int kb, int page16, int entry, int unit) {
  const int nf = g.n_fetch[unit];
  if (entry >= nf || entry >= g.cap) return;
  const int b = g.fetch[(static_cast<size_t>(unit) * g.cap + entry) * 2];
  const int s = g.fetch[(static_cast<size_t>(unit) * g.cap + entry) * 2 + 1];
  if (b < 0 || b >= Nmax || s < 0 || s >= kb) return;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(g.host + (static_cast<size_t>(unit) * Nmax + b) * page16);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(g.pool + (static_cast<size_t>(unit) * kb + s) * page16);
#pragma unroll 1
  for (int c = static_cast<int>(threadIdx.x); c < page16; c += NT) dst[c] = src[c];
}

// The LDS of a first-launch workgroup: an attention workgroup's, overlaid with
// a selecting workgroup's when the launch carries a selection.
template <int D, int RT, int W, bool SEL>
struct StepLds {
  AttnLds<D, RT, W> attn;
};
template <int D, int RT, int W>
struct StepLds<D, RT, W, true> {
  union {
    AttnLds<D, RT, W> attn;
    SelectLds<64 * W> sel;
  };
};

// Attention (2-page ring) and scoring workgroups in one grid of workgroups of
// W wavefronts (W = 2, or 4 for up to two attention row tiles), led by
// n_gather_wg workgroups that move another layer's fetched pages (one per
// fetch entry and unit; none without a transfer): the host-link reads start
// with the launch and overlap its HBM-bound work.
// order 0: attention workgroups first; 1: scoring first; 2: interleaved one for
// one while both last.  With KPT > 0, n_select_wg workgroups (one per unit of
// the carried state) follow the transfer's and select.
template <int D, int RTA, int RTS, int W, int KPT>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu((RTA <= 3 && RTS <= 2) ? 2 : 1))) void attn_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ pool, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ b2s, const int32_t* __restrict__ attend, const int32_t* __restrict__ n_attend,
    const int32_t* __restrict__ ctx_attn, float* __restrict__ ws_acc, float* __restrict__ ws_ml,
    float* __restrict__ out, int H, int arows, int Nmax, int kb, int splits, int run, float scale_log2,
    const uint16_t* __restrict__ meta, const int32_t* __restrict__ ctx_score, float* __restrict__ scores, int G,
    int T, int ndraft, int srows, int wpu, int tpw, int total_waves, int n_attn_wg, int n_score_wg, int order,
    StepGather gather, int n_gather_wg, int page16, SelectJob job, int n_select_wg, int cap,
    int32_t* __restrict__ arrive) {
  constexpr bool SEL = KPT > 0;
  __shared__ StepLds<D, RTA, W, SEL> lds;
  if (static_cast<int>(blockIdx.x) < n_gather_wg) {
    const int units = n_gather_wg / gather.cap;
    gather_page<64 * W>(gather, Nmax, kb, page16, blockIdx.x / units, blockIdx.x % units);
    return;
  }
  if constexpr (SEL) {
    if (static_cast<int>(blockIdx.x) < n_gather_wg + n_select_wg) {
      select_diff_wg<64 * W, KPT, false>(job, blockIdx.x - n_gather_wg, H, Nmax, kb, cap, lds.sel);
      return;
    }
  }
  const int bid = blockIdx.x - n_gather_wg - n_select_wg;
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
                          splits, run, scale_log2, idx, lds.attn, arrive);
    return;
  }
  score_wave<D, RTS>(q, meta, ctx_score, scores, H, G, T, ndraft, 1, srows, Nmax, wpu, tpw, total_waves,
                     idx * W + static_cast<int>(threadIdx.x) / kWave, threadIdx.x & (kWave - 1));
}

template <int D, int RTA, int RTS, int W, int KPT>
hipError_t as_t(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                const int32_t* attend, const int32_t* n_attend, const int32_t* ctx_attn, float* ws_acc,
                float* ws_ml, float* out, const void* meta, const int32_t* ctx_score, float* scores,
                const StepGather& g, const SelectJob* job, hipStream_t st) {
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  const int n_attn_wg = c.units * c.attn_splits;
  const int wpu = score_waves_per_unit(c);
  const int total = c.units * wpu;
  const int n_score_wg = (total + W - 1) / W;
  const int n_gather_wg = (g.host != nullptr && g.cap > 0) ? g.cap * c.units : 0;
  const int page16 = static_cast<int>(c.page_elems * c.elem_bytes / 16);
  const int n_select_wg = (KPT > 0 && job != nullptr) ? c.units : 0;
  hipLaunchKernelGGL((attn_score_kernel<D, RTA, RTS, W, KPT>),
                     dim3(n_gather_wg + n_select_wg + n_attn_wg + n_score_wg),
                     dim3(64 * W), 0, st, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(pool), sel,
                     b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, c.s.kv_heads, c.rows_attn,
                     c.s.max_blocks, c.s.budget_blocks, c.attn_splits, c.attn_run, scale_log2,
                     static_cast<const uint16_t*>(meta), ctx_score, scores, c.s.group, c.T, c.s.n_draft,
                     c.rows_score, wpu, c.score_tpw, total, n_attn_wg, n_score_wg, c.step_order, g, n_gather_wg,
                     page16, job != nullptr ? *job : SelectJob(), n_select_wg, c.s.fetch_cap,
                     c.attn_merge ? reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws_acc) + c.ws_arrive_off)
                                  : nullptr);
  return hipGetLastError();
}

template <int D, int RTA, int W, int KPT>
hipError_t as_s(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                const int32_t* attend, const int32_t* n_attend, const int32_t* ctx_attn, float* ws_acc,
                float* ws_ml, float* out, const void* meta, const int32_t* ctx_score, float* scores,
                const StepGather& g, const SelectJob* job, hipStream_t st) {
  switch ((c.rows_score + 15) / 16) {
    case 1: return as_t<D, RTA, 1, W, KPT>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, job, st);
    case 2: return as_t<D, RTA, 2, W, KPT>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, job, st);
    case 3: return as_t<D, RTA, 3, W, KPT>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, job, st);
    default: return as_t<D, RTA, 4, W, KPT>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, job, st);
  }
}

// The first launch for one head dimension: row tiles and wavefronts per
// workgroup from the shape (a carried selection is built for W = 2 only).
template <int D, int KPT>
hipError_t as_d(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                const int32_t* attend, const int32_t* n_attend, const int32_t* ctx_attn, float* ws_acc,
                float* ws_ml, float* out, const void* meta, const int32_t* ctx_score, float* scores,
                const StepGather& g, const SelectJob* job, hipStream_t st) {
  const bool w4 = c.attn_waves == 4;
  if constexpr (KPT > 0) {
    if (w4) return hipErrorInvalidValue;
    switch ((c.rows_attn + 15) / 16) {
      case 1: return as_s<D, 1, 2, KPT>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, job, st);
      case 2: return as_s<D, 2, 2, KPT>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, job, st);
      default: return as_s<D, 3, 2, KPT>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, job, st);
    }
  } else {
    switch ((c.rows_attn + 15) / 16) {
      case 1: return w4 ? as_s<D, 1, 4, 0>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, job, st)
                        : as_s<D, 1, 2, 0>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, job, st);
      case 2: return w4 ? as_s<D, 2, 4, 0>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, job, st)
                        : as_s<D, 2, 2, 0>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, job, st);
      default: return as_s<D, 3, 2, 0>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score, scores, g, job, st);
    }
  }
}

}  // namespace
}  // namespace oasis
