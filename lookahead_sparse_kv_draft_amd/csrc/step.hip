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
#include "attn_combine.h"
#include "step_kernel.h"

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
             ? as_d<128, 0>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score,
                            scores, g, nullptr, st)
             : as_d<64, 0>(c, q, pool, sel, b2s, attend, n_attend, ctx_attn, ws_acc, ws_ml, out, meta, ctx_score,
                           scores, g, nullptr, st);
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
