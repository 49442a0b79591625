// Top-k block selection per (request, KV head): the sink block 0 and the newest
// block are always kept (attention sinks are among the works the OasisKV pages
// build on), then the best-scoring other blocks fill the budget of k blocks
// (OasisKV explainer, Figure 7 right: the draft query predicts the next step's
// top-K blocks).  Ranking is the total order (descending score, ascending block
// index) with -0.0 ranked as +0.0.
//
// One 256-thread workgroup per unit.  A 4-pass, 8-bit radix select over 32-bit
// order keys finds the key T of the m-th best candidate; one ordered pass then
// collects every candidate with key < T (any order) and the lowest-index
// candidates with key == T (workgroup ballot ranks), and a bitonic sort of the
// m (key, index) pairs in LDS produces the rank order.  Scores are read from
// global memory (L2-resident: the score kernel just wrote them).
#include "block_ops.h"

namespace oasis {
namespace {

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ scores,
                                                   const int32_t* __restrict__ ctx_len,
                                                   int32_t* __restrict__ sel, int H, int Nmax,
                                                   int kb, int P) {
  extern __shared__ unsigned long long buf[];  // [P]
  __shared__ int hist[256];
  __shared__ int wave_tot[kWavesPerWG];
  __shared__ int sh_digit, sh_rem, sh_nlt;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  const int n = ctx_len[unit / H];
  const int N = max(1, min((n + kBlock - 1) / kBlock, Nmax));
  const int F0 = (N == 1) ? 1 : 2;
  const int C = max(0, N - 2);
  const int m = min(kb - F0, C);
  int32_t* out = sel + static_cast<size_t>(unit) * kb;
  const float* sc = scores + static_cast<size_t>(unit) * Nmax;
  if (tid == 0) {
    out[0] = 0;
    if (N > 1) out[1] = N - 1;
  }
  for (int i = F0 + max(m, 0) + tid; i < kb; i += kWG) out[i] = -1;
  if (m <= 0) return;

  uint32_t prefix = 0u, mask = 0u;
  int rem = m;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int b = 1 + tid; b < N - 1; b += kWG) {
      const uint32_t key = desc_key(sc[b]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    const int v = hist[tid];
    const int incl = wg_inclusive_sum(v, wave_tot);
    const int excl = incl - v;
    if (excl < rem && incl >= rem) {
      sh_digit = tid;
      sh_rem = rem - excl;
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(sh_digit) << shift;
    mask |= 255u << shift;
    rem = sh_rem;
    __syncthreads();
  }
  const uint32_t Tkey = prefix;
  const int need_eq = rem;     // candidates equal to Tkey to take, lowest index first
  const int n_lt = m - need_eq;  // candidates strictly better than Tkey

  if (tid == 0) sh_nlt = 0;
  __syncthreads();
  int eq_base = 0;  // uniform across the workgroup
  for (int base = 1; base < N - 1; base += kWG) {
    const int b = base + tid;
    const bool valid = b < N - 1;
    const uint32_t key = valid ? desc_key(sc[b]) : 0xFFFFFFFFu;
    if (valid && key < Tkey) {
      const int pos = atomicAdd(&sh_nlt, 1);
      if (pos < P) buf[pos] = (static_cast<unsigned long long>(key) << 32) | static_cast<uint32_t>(b);
    }
    if (eq_base < need_eq) {  // uniform branch: ranks of equal keys in index order
      const bool eq = valid && key == Tkey;
      int tot;
      const int rank = wg_rank_of_flag(eq, &tot, wave_tot);
      if (eq && eq_base + rank < need_eq)
        buf[n_lt + eq_base + rank] =
            (static_cast<unsigned long long>(Tkey) << 32) | static_cast<uint32_t>(b);
      eq_base += tot;
    }
  }
  for (int i = m + tid; i < P; i += kWG) buf[i] = ~0ull;
  __syncthreads();
  wg_bitonic_sort(buf, P);
  for (int i = tid; i < m; i += kWG) out[F0 + i] = static_cast<int32_t>(buf[i] & 0xFFFFFFFFull);
}

}  // namespace

hipError_t launch_topk(const Ctx& c, const float* scores, const int32_t* ctx_len, int32_t* sel,
                       hipStream_t st) {
  int P = 1;
  while (P < c.s.budget_blocks) P <<= 1;
  const size_t lds = static_cast<size_t>(P) * sizeof(unsigned long long);
  hipLaunchKernelGGL(topk_kernel, dim3(c.units), dim3(kWG), lds, st, scores, ctx_len, sel,
                     c.s.kv_heads, c.s.max_blocks, c.s.budget_blocks, P);
  return hipGetLastError();
}

}  // namespace oasis
