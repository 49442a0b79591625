// Lookahead scoring of every KV block from the draft queries (OasisKV explainer,
// Figure 7 right: the draft queries scan the compressed keys to predict the next
// step's top-K blocks).  The score of block b is the Quest upper bound
//     max over draft rows q of  sum_c max(q_c * kmin_c, q_c * kmax_c),
// which equals q+ . kmax + q- . kmin with q+ = max(q, 0), q- = min(q, 0).
//
// bf16 path: the bound is a dense contraction of the [rows x 2d] matrix
// [q- | q+] with the [2d x blocks] metadata, so it runs on the bf16 MFMA
// (v_mfma_f32_16x16x32_bf16): q+ and q- are exact in bf16, every product is exact
// in fp32 and the sum accumulates in fp32.  One wavefront streams 16-block tiles
// of one (request, KV head): B operand = 16 blocks x 32 metadata elements, each
// lane loading 16 bytes of one contiguous 1 KiB piece per k-step (the metadata
// tiles are stored chunk-major for this), A operand = the
// split query rows held in registers for the whole wavefront.  The next tile's
// loads are issued before the current tile's MFMAs.  Rows are reduced with a max
// inside each lane and two cross-lane exchanges.
//
// f32 path: one thread per block, query rows staged in LDS, plain fp32 VALU.
#include "append_body.h"
#include "score_body.h"

namespace oasis {
namespace {

// n_app_wg workgroups (one per unit, or none) after the scoring's write the
// page row of a token a decode step appends (its metadata row was updated by
// the step's attention launch, before this one).  Placed ahead of the scoring
// they made the step about 1.5 us longer.
template <int D, int RT>
__global__ __launch_bounds__(256) void score_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ meta,
    const int32_t* __restrict__ ctx_len, float* __restrict__ scores, int H, int G, int T,
    int ndraft, int t0, int rows, int Nmax, int waves_per_unit, int tpw, int total_waves, StepAppend app,
    int n_app_wg, int kb) {
  const int n_score_wg = static_cast<int>(gridDim.x) - n_app_wg;
  if (static_cast<int>(blockIdx.x) >= n_score_wg) {
    append_page<uint16_t, D>(static_cast<const uint16_t*>(app.k_new), static_cast<const uint16_t*>(app.v_new),
                             app.ctx_in, static_cast<uint16_t*>(app.pool), app.b2s, blockIdx.x - n_score_wg, H,
                             Nmax, kb, threadIdx.x, 256);
    return;
  }
  score_wave<D, RT>(q, meta, ctx_len, scores, H, G, T, ndraft, t0, rows, Nmax, waves_per_unit, tpw, total_waves,
                    blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave, threadIdx.x & (kWave - 1));
}

template <int D>
__global__ __launch_bounds__(256) void score_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ meta, const int32_t* __restrict__ ctx_len,
    float* __restrict__ scores, int H, int G, int T, int ndraft, int t0, int rows, int Nmax) {
  extern __shared__ float qs[];  // [rows][D]
  const int unit = blockIdx.y;
  const int n = ctx_len[unit / H];
  const int N = min((n + kBlock - 1) / kBlock, Nmax);
  if (static_cast<int>(blockIdx.x) * 256 >= N) return;
  for (int i = threadIdx.x; i < rows * D; i += blockDim.x) {
    const int row = i / D, c = i - (i / D) * D;
    const int g = row / ndraft, t = t0 + (row - g * ndraft);
    qs[i] = q[((static_cast<size_t>(unit) * G + g) * T + t) * D + c];
  }
  __syncthreads();
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= N) return;
  float best = -INFINITY;
  for (int row = 0; row < rows; ++row) {
    float s = 0.f;
    for (int c = 0; c < D; ++c) {
      const float qc = qs[row * D + c];
      s += fmaxf(qc * meta[meta_offset<D, 4>(unit, b, c, Nmax)], qc * meta[meta_offset<D, 4>(unit, b, D + c, Nmax)]);
    }
    best = fmaxf(best, s);
  }
  scores[static_cast<size_t>(unit) * Nmax + b] = best;
}

// Query rows scored: rows t0 .. t0 + nd - 1 of every group member (the drafts:
// t0 = 1, nd = n_draft; the verify query: t0 = 0, nd = 1).
struct ScoreRows {
  int nd, t0, rows;
};

template <int D, int RT>
hipError_t mfma_t(const Ctx& c, const void* q, const void* meta, const int32_t* ctx_len,
                  float* scores, ScoreRows sr, hipStream_t st, const StepAppend* ap) {
  const int wpu = score_waves_per_unit(c);
  const int total = c.units * wpu;
  const int n_app_wg = ap != nullptr ? c.units : 0;
  const int grid = (total + 3) / 4 + n_app_wg;
  hipLaunchKernelGGL((score_mfma_kernel<D, RT>), dim3(grid), dim3(256), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(meta), ctx_len,
                     scores, c.s.kv_heads, c.s.group, c.T, sr.nd, sr.t0, sr.rows,
                     c.s.max_blocks, wpu, c.score_tpw, total, ap != nullptr ? *ap : StepAppend(), n_app_wg,
                     c.s.budget_blocks);
  return hipGetLastError();
}

template <int D>
hipError_t f32_t(const Ctx& c, const void* q, const void* meta, const int32_t* ctx_len,
                 float* scores, ScoreRows sr, hipStream_t st) {
  dim3 grid((c.s.max_blocks + 255) / 256, c.units);
  const size_t lds = static_cast<size_t>(sr.rows) * D * sizeof(float);
  hipLaunchKernelGGL((score_f32_kernel<D>), grid, dim3(256), lds, st,
                     static_cast<const float*>(q), static_cast<const float*>(meta), ctx_len, scores,
                     c.s.kv_heads, c.s.group, c.T, sr.nd, sr.t0, sr.rows, c.s.max_blocks);
  return hipGetLastError();
}

template <int D>
hipError_t mfma_rows(const Ctx& c, const void* q, const void* meta, const int32_t* ctx_len,
                     float* scores, ScoreRows sr, hipStream_t st, const StepAppend* ap) {
  switch ((sr.rows + 15) / 16) {
    case 1: return mfma_t<D, 1>(c, q, meta, ctx_len, scores, sr, st, ap);
    case 2: return mfma_t<D, 2>(c, q, meta, ctx_len, scores, sr, st, ap);
    case 3: return mfma_t<D, 3>(c, q, meta, ctx_len, scores, sr, st, ap);
    default: return mfma_t<D, 4>(c, q, meta, ctx_len, scores, sr, st, ap);
  }
}

}  // namespace

hipError_t launch_score(const Ctx& c0, const void* q, const void* meta, const int32_t* ctx_len,
                        float* scores, hipStream_t st, bool verify, const StepAppend* ap) {
  // a scoring launch of its own: its own run of tiles per wavefront
  Ctx c = c0;
  c.score_tpw = c0.score_tpw_solo;
  const ScoreRows sr = verify ? ScoreRows{1, 0, c.s.group} : ScoreRows{c.s.n_draft, 1, c.rows_score};
  if (c.s.dtype == OASIS_BF16)
    return c.s.head_dim == 128 ? mfma_rows<128>(c, q, meta, ctx_len, scores, sr, st, ap)
                               : mfma_rows<64>(c, q, meta, ctx_len, scores, sr, st, ap);
  if (ap != nullptr) return hipErrorInvalidValue;  // the fp32 kernel carries no append
  return c.s.head_dim == 128 ? f32_t<128>(c, q, meta, ctx_len, scores, sr, st)
                             : f32_t<64>(c, q, meta, ctx_len, scores, sr, st);
}

}  // namespace oasis
