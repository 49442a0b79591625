// Sparse paged GQA decode attention over the resident selected blocks (OasisKV
// explainer, Figure 7 right: the verify query and the draft queries attend
// together over the sparse KV working set held in HBM).
//
// Work unit: one (request, KV head) and one split of its selection list.  All
// T*G query rows of the unit (verify + drafts for each grouped query head) ride
// in the same wavefront, so every KV page is read from HBM once per step.
//
// bf16 path, per 16-token block and per 16-row query tile, on the MFMA units:
//   S^T[tok][row] = K[tok][:] . Q[row][:]   v_mfma_f32_16x16x32_bf16, A = the K
//       page rows (16 contiguous bytes per lane), B = the query rows (registers);
//       the output leaves lane (col, grp) with tokens 4grp..4grp+3 of row col;
//   online softmax in the log2 domain, in registers: block max over the 4
//       tokens of the lane and two cross-lane exchanges, a reference max that
//       moves only on large increases; probabilities rounded to bf16 (the running
//       sum adds the rounded values, so weights and normaliser agree);
//   O^T[ch][row] += V^T[ch][tok] . P^T[tok][row]  v_mfma_f32_16x16x16_bf16, A =
//       the page's channel-major V^T (8 contiguous bytes per lane), B = the
//       lane's own 4 probabilities: P never leaves registers.
// The page layout (K token-major, V channel-major) is what makes both products
// read contiguous lane-sized pieces without an LDS transpose.  A wavefront
// keeps a ring of PF pages in flight: each page's math runs while the next
// pages' loads are outstanding.
//
// f32 path: VALU, query rows and logits in LDS, accumulators in registers.
// Both paths leave one partial per split; a log-sum-exp combine kernel merges
// them.
#include <algorithm>
#include <mutex>

#include "append_body.h"
#include "attn_body.h"
#include "attn_combine.h"

namespace oasis {
namespace {

// n_app_wg workgroups (one per unit, or none) after the attention's update the
// metadata row of a token being appended (the attention reads no metadata; the
// token's page row is written by the scoring launch that follows, which reads
// no pages: written here, beside the attention's reads of the same pages, it
// made the launch several microseconds longer).
template <int D, int RT, int W, int PF>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu((PF <= 2 && RT <= 3) ? 2 : 1))) void attn_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ pool,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ b2s, const int32_t* __restrict__ attend,
    const int32_t* __restrict__ n_attend, const int32_t* __restrict__ ctx_len, float* __restrict__ ws_acc,
    float* __restrict__ ws_ml, float* __restrict__ out, int H, int rows, int Nmax, int kb,
    int splits, int run, float scale_log2, StepAppend app, int n_app_wg) {
  __shared__ AttnLds<D, RT, W> lds;
  const int n_attn_wg = static_cast<int>(gridDim.x) - n_app_wg;
  if (static_cast<int>(blockIdx.x) >= n_attn_wg) {
    append_meta<uint16_t, D>(static_cast<const uint16_t*>(app.k_new), app.ctx_in, app.ctx_out,
                             static_cast<uint16_t*>(app.meta), blockIdx.x - n_attn_wg, H, Nmax, threadIdx.x, 64 * W);
    return;
  }
  attn_wg<D, RT, W, PF>(q, pool, sel, b2s, attend, n_attend, ctx_len, ws_acc, ws_ml, out, H, rows, Nmax, kb, splits,
                        run, scale_log2, blockIdx.x, lds);
}

// fp32 path: workgroup of 256 threads per (unit, split).
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ pool, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ b2s, const int32_t* __restrict__ attend, const int32_t* __restrict__ n_attend,
    const int32_t* __restrict__ ctx_len, float* __restrict__ ws_acc, float* __restrict__ ws_ml, int H, int GT,
    int rows, int Nmax, int kb, int splits, int split_len, float scale_log2) {
  constexpr int PAGE = 2 * kBlock * D;
  constexpr int J = (kMaxRows * D + 255) / 256;  // accumulators per thread (upper bound)
  extern __shared__ float smem[];
  float* qs = smem;                   // [rows][D]
  float* lg = qs + rows * D;          // [rows][16] logits, then probabilities
  float* alpha_s = lg + rows * kBlock;  // [rows]
  float* m_s = alpha_s + rows;        // [rows]
  float* l_s = m_s + rows;            // [rows]
  const int tid = threadIdx.x;
  const int wid = blockIdx.x;
  const int unit = wid / splits;
  const int split = wid - unit * splits;
  const int n = ctx_len[unit / H];
  for (int i = tid; i < rows * D; i += 256) qs[i] = q[static_cast<size_t>(unit) * GT * D + i];
  for (int i = tid; i < rows; i += 256) {
    m_s[i] = -INFINITY;
    l_s[i] = 0.f;
  }
  float acc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) acc[j] = 0.f;
  __syncthreads();
  // the split's entries: of the selection, or an even share of an attended list
  int i0, i1;
  if (attend != nullptr) {
    const int natt = min(max(n_attend[unit], 0), kb);
    const int per = (natt + splits - 1) / splits;
    i0 = min(natt, split * per);
    i1 = min(natt, i0 + per);
  } else {
    i0 = split * split_len;
    i1 = min(kb, i0 + split_len);
  }
  for (int e = i0; e < i1; ++e) {
    int b, slot;
    if (attend != nullptr) {
      const int pk = attend[static_cast<size_t>(unit) * kb + e];
      b = pk >> kAttendSlotBits;
      slot = pk & ((1 << kAttendSlotBits) - 1);
      if (b < 0 || b >= Nmax) continue;
    } else {
      b = sel[static_cast<size_t>(unit) * kb + e];
      if (b < 0 || b >= Nmax) continue;
      slot = b2s[static_cast<size_t>(unit) * Nmax + b];
    }
    const int ntok = min(kBlock, n - kBlock * b);
    if (slot < 0 || slot >= kb || ntok <= 0) continue;
    const float* pg = pool + (static_cast<size_t>(unit) * kb + slot) * PAGE;
    for (int i = tid; i < rows * kBlock; i += 256) {
      const int row = i / kBlock, tok = i - (i / kBlock) * kBlock;
      float s = -INFINITY;
      if (tok < ntok) {
        s = 0.f;
        for (int c = 0; c < D; ++c) s += qs[row * D + c] * pg[tok * D + c];
        s *= scale_log2;
      }
      lg[i] = s;
    }
    __syncthreads();
    for (int row = tid; row < rows; row += 256) {
      float mb = -INFINITY;
      for (int t = 0; t < kBlock; ++t) mb = fmaxf(mb, lg[row * kBlock + t]);
      const float mnew = fmaxf(m_s[row], mb);
      const float a = exp2f(m_s[row] - mnew);
      float ps = 0.f;
      for (int t = 0; t < kBlock; ++t) {
        const float p = exp2f(lg[row * kBlock + t] - mnew);
        lg[row * kBlock + t] = p;
        ps += p;
      }
      l_s[row] = l_s[row] * a + ps;
      m_s[row] = mnew;
      alpha_s[row] = a;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int i = tid + 256 * j;
      if (i < rows * D) {
        const int row = i / D, c = i - (i / D) * D;
        float a = acc[j] * alpha_s[row];
        for (int t = 0; t < ntok; ++t) a += lg[row * kBlock + t] * pg[kBlock * D + c * kBlock + t];
        acc[j] = a;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = tid + 256 * j;
    if (i < rows * D) ws_acc[static_cast<size_t>(wid) * rows * D + i] = acc[j];
  }
  for (int row = tid; row < rows; row += 256) {
    ws_ml[(static_cast<size_t>(wid) * rows + row) * 2] = m_s[row];
    ws_ml[(static_cast<size_t>(wid) * rows + row) * 2 + 1] = l_s[row];
  }
}

template <int D, int SMAX>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ ws_acc,
                                                           const float* __restrict__ ws_ml,
                                                           float* __restrict__ out, int rows,
                                                           int splits, int total) {
  attn_combine_row<D, SMAX>(ws_acc, ws_ml, out, rows, splits, total, blockIdx.x * 4 + threadIdx.x / kWave,
                            threadIdx.x & (kWave - 1));
}

template <int D, int RT, int W, int PF>
hipError_t mfma_wp(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                   const int32_t* attend, const int32_t* n_attend, const int32_t* ctx_len, float* ws_acc,
                   float* ws_ml, float* out, float scale_log2, hipStream_t st, const StepAppend* ap) {
  const int n_app_wg = ap != nullptr ? c.units : 0;
  hipLaunchKernelGGL((attn_mfma_kernel<D, RT, W, PF>), dim3(n_app_wg + c.units * c.attn_splits), dim3(W * kWave), 0,
                     st, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(pool), sel, b2s, attend,
                     n_attend, ctx_len,
                     ws_acc, ws_ml, out, c.s.kv_heads, c.rows_attn, c.s.max_blocks,
                     c.s.budget_blocks, c.attn_splits, c.attn_run, scale_log2,
                     ap != nullptr ? *ap : StepAppend(), n_app_wg);
  return hipGetLastError();
}

template <int D, int RT, int W>
hipError_t mfma_w(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                  const int32_t* attend, const int32_t* n_attend, const int32_t* ctx_len, float* ws_acc,
                  float* ws_ml, float* out, float scale_log2, hipStream_t st, const StepAppend* ap) {
  switch (c.attn_pf) {
    case 2: return mfma_wp<D, RT, W, 2>(c, q, pool, sel, b2s, attend, n_attend, ctx_len, ws_acc, ws_ml, out, scale_log2, st, ap);
    case 4: return mfma_wp<D, RT, W, 4>(c, q, pool, sel, b2s, attend, n_attend, ctx_len, ws_acc, ws_ml, out, scale_log2, st, ap);
    default: return mfma_wp<D, RT, W, 8>(c, q, pool, sel, b2s, attend, n_attend, ctx_len, ws_acc, ws_ml, out, scale_log2, st, ap);
  }
}

template <int D, int RT>
hipError_t mfma_t(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                  const int32_t* attend, const int32_t* n_attend, const int32_t* ctx_len, float* ws_acc,
                  float* ws_ml, float* out, float scale_log2, hipStream_t st, const StepAppend* ap) {
  if (c.attn_waves == 1) return mfma_w<D, RT, 1>(c, q, pool, sel, b2s, attend, n_attend, ctx_len, ws_acc, ws_ml, out, scale_log2, st, ap);
  // at most 2 wavefronts for 3 or 4 row tiles (LDS of the wavefront merge)
  if (RT >= 3 || c.attn_waves == 2)
    return mfma_w<D, RT, 2>(c, q, pool, sel, b2s, attend, n_attend, ctx_len, ws_acc, ws_ml, out, scale_log2, st, ap);
  return mfma_w<D, RT, (RT >= 3 ? 2 : 4)>(c, q, pool, sel, b2s, attend, n_attend, ctx_len, ws_acc, ws_ml, out, scale_log2, st, ap);
}

template <int D>
hipError_t main_t(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                  const int32_t* attend, const int32_t* n_attend, const int32_t* ctx_len, float* ws_acc,
                  float* ws_ml, float* out, hipStream_t st, const StepAppend* ap) {
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  if (c.s.dtype == OASIS_BF16) {
    switch ((c.rows_attn + 15) / 16) {
      case 1: return mfma_t<D, 1>(c, q, pool, sel, b2s, attend, n_attend, ctx_len, ws_acc, ws_ml, out, scale_log2, st, ap);
      case 2: return mfma_t<D, 2>(c, q, pool, sel, b2s, attend, n_attend, ctx_len, ws_acc, ws_ml, out, scale_log2, st, ap);
      case 3: return mfma_t<D, 3>(c, q, pool, sel, b2s, attend, n_attend, ctx_len, ws_acc, ws_ml, out, scale_log2, st, ap);
      default: return mfma_t<D, 4>(c, q, pool, sel, b2s, attend, n_attend, ctx_len, ws_acc, ws_ml, out, scale_log2, st, ap);
    }
  }
  if (ap != nullptr) return hipErrorInvalidValue;  // the fp32 kernel carries no append
  const int rows = c.rows_attn;
  const size_t lds = (static_cast<size_t>(rows) * D + rows * kBlock + 3 * rows) * sizeof(float);
  hipLaunchKernelGGL((attn_f32_kernel<D>), dim3(c.units * c.attn_splits), dim3(256), lds, st,
                     static_cast<const float*>(q), static_cast<const float*>(pool), sel, b2s, attend,
                     n_attend, ctx_len, ws_acc, ws_ml, c.s.kv_heads, c.rows_attn, rows, c.s.max_blocks,
                     c.s.budget_blocks, c.attn_splits, c.attn_split_len, scale_log2);
  return hipGetLastError();
}

template <int D>
hipError_t combine_t(const Ctx& c, const float* ws_acc, const float* ws_ml, float* out, hipStream_t st) {
  const int total = c.units * c.rows_attn;
  const int grid = (total + 3) / 4;
  const int S = c.attn_splits;
#define OASIS_COMBINE(SM)                                                                           \
  hipLaunchKernelGGL((attn_combine_kernel<D, SM>), dim3(grid), dim3(256), 0, st, ws_acc, ws_ml, out, \
                     c.rows_attn, S, total)
  if (S <= 4)
    OASIS_COMBINE(4);
  else if (S <= 8)
    OASIS_COMBINE(8);
  else if (S <= 16)
    OASIS_COMBINE(16);
  else
    OASIS_COMBINE(32);
#undef OASIS_COMBINE
  return hipGetLastError();
}

}  // namespace

size_t attn_ws_partials_bytes(const Ctx& c) {
  Ctx solo = c;
  solo.attn_splits = c.attn_splits_solo;
  return std::max(attn_ws_acc_bytes(c) + attn_ws_ml_bytes(c), attn_ws_acc_bytes(solo) + attn_ws_ml_bytes(solo));
}

size_t attn_workspace_bytes(const Ctx& c) {
  // the partials, then one int32 arrival counter per unit (256-byte aligned)
  return attn_ws_partials_bytes(c) + (static_cast<size_t>(c.units) * 4 + 255) / 256 * 256;
}

bool attn_needs_combine(const Ctx& c) {
  // the bf16 kernel writes the output itself when there is a single split
  return !(c.s.dtype == OASIS_BF16 && c.attn_splits == 1);
}

hipError_t launch_attn_main(const Ctx& c, const void* q, const void* pool, const int32_t* sel,
                            const int32_t* b2s, const int32_t* attend, const int32_t* n_attend,
                            const int32_t* ctx_len, float* out, void* ws, hipStream_t st, const StepAppend* ap) {
  float* ws_acc = static_cast<float*>(ws);
  float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + attn_ws_acc_bytes(c));
  return (c.s.head_dim == 128)
             ? main_t<128>(c, q, pool, sel, b2s, attend, n_attend, ctx_len, ws_acc, ws_ml, out, st, ap)
             : main_t<64>(c, q, pool, sel, b2s, attend, n_attend, ctx_len, ws_acc, ws_ml, out, st, ap);
}

hipError_t launch_attn_combine(const Ctx& c, void* ws, float* out, hipStream_t st) {
  if (!attn_needs_combine(c)) return hipSuccess;
  float* ws_acc = static_cast<float*>(ws);
  float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + attn_ws_acc_bytes(c));
  return (c.s.head_dim == 128) ? combine_t<128>(c, ws_acc, ws_ml, out, st) : combine_t<64>(c, ws_acc, ws_ml, out, st);
}

hipError_t launch_attn(const Ctx& c0, const void* q, const void* pool, const int32_t* sel,
                       const int32_t* b2s, const int32_t* attend, const int32_t* n_attend,
                       const int32_t* ctx_len, float* out, void* ws, hipStream_t st, const StepAppend* ap) {
  // the attention on its own: its own split shape and ring (the workspace fits the larger one)
  Ctx c = c0;
  c.attn_splits = c0.attn_splits_solo;
  c.attn_run = c0.attn_run_solo;
  c.attn_pf = c0.attn_pf_solo;
  c.attn_split_len = c0.attn_waves * c0.attn_run_solo;
  hipError_t e = launch_attn_main(c, q, pool, sel, b2s, attend, n_attend, ctx_len, out, ws, st, ap);
  if (e != hipSuccess || !attn_needs_combine(c)) return e;
  float* ws_acc = static_cast<float*>(ws);
  float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + attn_ws_acc_bytes(c));
  return (c.s.head_dim == 128) ? combine_t<128>(c, ws_acc, ws_ml, out, st)
                               : combine_t<64>(c, ws_acc, ws_ml, out, st);
}

// ---- the attention without a caller workspace ----
// Its split partials live in this file-scope device array: one copy per GPU,
// held until the process ends, shared by every such call on that GPU (calls
// that overlap on one GPU race on it).  Nothing in it must start at zero: every
// split writes its whole partial before the combine reads it.  In host code the
// array's name is only a stand-in; its device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = static_cast<size_t>(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t attn_scratch_bytes() { return kScratchBytes; }

hipError_t launch_attn_noalloc(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                               const int32_t* ctx_len, float* out, hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_scratch_ptr[dev] = p;
    }
    ws = g_scratch_ptr[dev];
  }
  return launch_attn(c, q, pool, sel, b2s, nullptr, nullptr, ctx_len, out, ws, st);
}

}  // namespace oasis
