// Log-sum-exp merge of the attention's split partials (the split-K of the sparse
// decode attention over the resident selected blocks, OasisKV explainer Figure 7
// right).  Used by the attention's own combine kernel and by the launch that
// carries the combine beside the lookahead scoring.
#pragma once

#include "oasis_internal.h"

namespace oasis {

// One wavefront merges one (unit, query row) = id.  Every split's partial row and (max, sum) are loaded in one
// batch (split index clamped to the last split, whose repeats get weight 0),
// then merged: out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
template <int D, int SMAX>
__device__ __forceinline__ void attn_combine_row(const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
                                        float* __restrict__ out, int rows, int splits, int total, int id,
                                        int lane) {
  constexpr int PER = D / kWave;  // output channels per lane (1 or 2)
  if (id >= total) return;  // id = unit * rows + row, wavefront-uniform
  const int unit = id / rows;
  const int row = id - unit * rows;
  float v[SMAX][PER];
  float2 ml[SMAX];
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    const size_t p = (static_cast<size_t>(unit) * splits + min(s, splits - 1)) * rows + row;
    ml[s] = *reinterpret_cast<const float2*>(ws_ml + p * 2);
    if constexpr (PER == 2) {
      const float2 t = *reinterpret_cast<const float2*>(ws_acc + p * D + 2 * lane);
      v[s][0] = t.x;
      v[s][1] = t.y;
    } else {
      v[s][0] = ws_acc[p * D + lane];
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < SMAX; ++s) M = fmaxf(M, ml[s].x);  // repeats do not change the max
  float L = 0.f, a[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) a[j] = 0.f;
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    const float w = (s >= splits || ml[s].x == -INFINITY) ? 0.f : exp2f(ml[s].x - M);
    L += w * ml[s].y;
#pragma unroll
    for (int j = 0; j < PER; ++j) a[j] += w * v[s][j];
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  float* o = out + static_cast<size_t>(id) * D + PER * lane;
#pragma unroll
  for (int j = 0; j < PER; ++j) o[j] = a[j] * inv;
}

// Workspace layout of the attention: partial accumulators [units][splits][rows][D],
// then (max, sum) [units][splits][rows][2], each region 256-byte aligned.
inline size_t attn_ws_acc_bytes(const Ctx& c) {
  const size_t parts = static_cast<size_t>(c.units) * c.attn_splits * c.rows_attn;
  return (parts * c.s.head_dim * sizeof(float) + 255) / 256 * 256;
}
inline size_t attn_ws_ml_bytes(const Ctx& c) {
  const size_t parts = static_cast<size_t>(c.units) * c.attn_splits * c.rows_attn;
  return (parts * 2 * sizeof(float) + 255) / 256 * 256;
}

}  // namespace oasis
