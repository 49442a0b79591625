// Selection against the HBM-resident set with a per-step fetch cap and capped
// eviction (OasisKV explainer, "What they did" item 3 and Table 2: only missing
// predicted blocks are fetched, bounded per step; Figure 9: a per-KV-head table
// maps each GPU block slot to a CPU block, kept here with its inverse).
//
// One 256-thread workgroup per (request, KV head):
//   1. mark the selected blocks in an LDS bitmap;
//   2. missing = selected blocks without a slot, in rank order (workgroup ballot
//      ranks); the first min(cap, |missing|) are fetched;
//   3. free slots in ascending order;
//   4. if the free slots do not cover the fetch, the victims are the resident
//      blocks outside the selection with the largest (descending score,
//      ascending index) keys, i.e. lowest score first and the higher index first
//      among equal scores: a bitonic sort of at most k keys in LDS;
//   5. targets = free slots, then the victims' slots; both maps are updated in
//      place after every read of the old state (barrier in between).
#include "block_ops.h"

namespace oasis {
namespace {

__global__ __launch_bounds__(256) void diff_kernel(
    const int32_t* __restrict__ sel, const float* __restrict__ scores, int32_t* __restrict__ b2s,
    int32_t* __restrict__ s2b, int32_t* __restrict__ fetch, int32_t* __restrict__ n_fetch,
    int32_t* __restrict__ evict, int Nmax, int kb, int cap, int P) {
  extern __shared__ unsigned long long smem_u64[];
  unsigned long long* cand = smem_u64;                            // [P]
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(cand + P);       // [(Nmax + 31) / 32]
  const int nwords = (Nmax + 31) / 32;
  int32_t* F = reinterpret_cast<int32_t*>(bitmap + nwords);       // [cap]
  int32_t* tgt = F + cap;                                         // [cap]
  int32_t* freeS = tgt + cap;                                     // [kb]
  __shared__ int wave_tot[kWavesPerWG];
  __shared__ int sh_nc;

  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  const int32_t* su = sel + static_cast<size_t>(unit) * kb;
  int32_t* bu = b2s + static_cast<size_t>(unit) * Nmax;
  int32_t* slu = s2b + static_cast<size_t>(unit) * kb;
  const float* sc = scores + static_cast<size_t>(unit) * Nmax;

  for (int i = tid; i < nwords; i += kWG) bitmap[i] = 0u;
  if (tid == 0) sh_nc = 0;
  __syncthreads();
  for (int i = tid; i < kb; i += kWG) {
    const int b = su[i];
    if (b >= 0 && b < Nmax) atomicOr(&bitmap[b >> 5], 1u << (b & 31));
  }

  // 2. missing blocks in rank order, first `cap` kept
  int nmiss = 0;
  for (int base = 0; base < kb; base += kWG) {
    const int i = base + tid;
    int b = -1;
    bool flag = false;
    if (i < kb) {
      b = su[i];
      flag = (b >= 0 && b < Nmax && bu[b] < 0);
    }
    int tot;
    const int rank = wg_rank_of_flag(flag, &tot, wave_tot);
    if (flag && nmiss + rank < cap) F[nmiss + rank] = b;
    nmiss += tot;
  }
  // 3. free slots, ascending
  int nfree = 0;
  for (int base = 0; base < kb; base += kWG) {
    const int s = base + tid;
    const bool flag = s < kb && slu[s] < 0;
    int tot;
    const int rank = wg_rank_of_flag(flag, &tot, wave_tot);
    if (flag) freeS[nfree + rank] = s;
    nfree += tot;
  }
  int nF = min(cap, nmiss);
  int need = max(0, nF - nfree);

  // 4. victims: resident blocks outside the selection, largest keys first
  if (need > 0) {
    for (int s = tid; s < kb; s += kWG) {
      const int b = slu[s];
      if (b >= 0 && b < Nmax && !((bitmap[b >> 5] >> (b & 31)) & 1u)) {
        const int pos = atomicAdd(&sh_nc, 1);
        cand[pos] = (static_cast<unsigned long long>(desc_key(sc[b])) << 32) | static_cast<uint32_t>(b);
      }
    }
    __syncthreads();
    const int nc = sh_nc;
    for (int i = nc + tid; i < P; i += kWG) cand[i] = 0ull;  // pads sort first
    __syncthreads();
    wg_bitonic_sort(cand, P);
    // Consistent maps with at most k selected blocks always leave enough victims;
    // clamp anyway so inconsistent input cannot evict a padding entry.
    if (need > nc) {
      need = nc;
      nF = nfree + nc;
    }
  }
  // 5. targets from the old state
  for (int i = tid; i < nF; i += kWG) {
    if (i < nfree) {
      tgt[i] = freeS[i];
    } else {
      const int v = static_cast<int>(cand[P - 1 - (i - nfree)] & 0xFFFFFFFFull);
      tgt[i] = (v >= 0 && v < Nmax) ? bu[v] : -1;
    }
  }
  __syncthreads();
  for (int i = tid; i < need; i += kWG) {
    const int v = static_cast<int>(cand[P - 1 - i] & 0xFFFFFFFFull);
    if (v >= 0 && v < Nmax) bu[v] = -1;
  }
  // Targets are valid slots whenever the maps are mutually inverse; a corrupt map
  // cannot make this kernel write outside its buffers.
  for (int i = tid; i < nF; i += kWG) {
    const int s = tgt[i];
    if (s >= 0 && s < kb) {
      slu[s] = F[i];
      bu[F[i]] = s;
    }
  }
  int32_t* fu = fetch + static_cast<size_t>(unit) * cap * 2;
  int32_t* eu = evict + static_cast<size_t>(unit) * cap;
  for (int i = tid; i < cap; i += kWG) {
    fu[2 * i] = (i < nF) ? F[i] : -1;
    fu[2 * i + 1] = (i < nF) ? tgt[i] : -1;
    eu[i] = (i < need) ? static_cast<int32_t>(cand[P - 1 - i] & 0xFFFFFFFFull) : -1;
  }
  if (tid == 0) n_fetch[unit] = nF;
}

}  // namespace

hipError_t launch_diff(const Ctx& c, const int32_t* sel, const float* scores, int32_t* b2s,
                       int32_t* s2b, int32_t* fetch, int32_t* n_fetch, int32_t* evict,
                       hipStream_t st) {
  int P = 1;
  while (P < c.s.budget_blocks) P <<= 1;
  const int nwords = (c.s.max_blocks + 31) / 32;
  const size_t lds = static_cast<size_t>(P) * 8 + static_cast<size_t>(nwords) * 4 +
                     static_cast<size_t>(2 * c.s.fetch_cap + c.s.budget_blocks) * 4;
  hipLaunchKernelGGL(diff_kernel, dim3(c.units), dim3(kWG), lds, st, sel, scores, b2s, s2b, fetch,
                     n_fetch, evict, c.s.max_blocks, c.s.budget_blocks, c.s.fetch_cap, P);
  return hipGetLastError();
}

}  // namespace oasis
