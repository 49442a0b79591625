// Selection against the HBM-resident set with a per-step fetch cap and capped
// eviction (OasisKV explainer, "What they did" item 3 and Table 2: only missing
// predicted blocks are fetched, bounded per step; Figure 9: a per-KV-head table
// maps each GPU block slot to a CPU block, kept here with its inverse).
//
// One workgroup per (request, KV head) with one thread per selection entry and
// per slot (k threads, rounded up to whole wavefronts).  The work is a few
// hundred integers, so the kernel is built for latency: two dependent rounds of
// global loads (selection and slot map; then block map and the residents'
// scores), ordered compaction with ballots plus one cross-wavefront exchange,
// and a handful of barriers:
//   1. missing = selected blocks without a slot, in rank order; the first
//      min(cap, |missing|) are fetched;
//   2. free slots in ascending order;
//   3. if the free slots do not cover the fetch, the victims are the resident
//      blocks outside the selection with the largest (descending score,
//      ascending index) keys, i.e. lowest score first and the higher index first
//      among equal scores; each candidate's place is the number of larger keys;
//   4. targets = free slots, then the victims' slots; both maps are updated in
//      place after every read of the old state.
#include "oasis_internal.h"

namespace oasis {
namespace {

constexpr int kDiffMaxWaves = kMaxBudget / kWave;

struct DiffShared {
  int miss_tot[kDiffMaxWaves], free_tot[kDiffMaxWaves], cand_tot[kDiffMaxWaves];
};

__global__ __launch_bounds__(1024) void diff_kernel(
    const int32_t* __restrict__ sel, const float* __restrict__ scores, int32_t* __restrict__ b2s,
    int32_t* __restrict__ s2b, int32_t* __restrict__ fetch, int32_t* __restrict__ n_fetch,
    int32_t* __restrict__ evict, int Nmax, int kb, int cap) {
  extern __shared__ unsigned long long smem_u64[];
  unsigned long long* ckey = smem_u64;                       // [kb] candidate key per slot (0 = none)
  const int nwords = (Nmax + 31) / 32;
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(ckey + kb);  // [nwords] selected blocks
  int32_t* F = reinterpret_cast<int32_t*>(bitmap + nwords);  // [cap] fetched blocks
  int32_t* tgt = F + cap;                                     // [cap] their target slots
  int32_t* freeS = tgt + cap;                                 // [kb] free slots, ascending
  int32_t* vict = freeS + kb;                                 // [cap] victim blocks
  int32_t* victS = vict + cap;                                // [cap] victim slots
  __shared__ DiffShared sh;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int nw = blockDim.x / kWave;
  const int unit = blockIdx.x;
  const int32_t* su = sel + static_cast<size_t>(unit) * kb;
  int32_t* bu = b2s + static_cast<size_t>(unit) * Nmax;
  int32_t* slu = s2b + static_cast<size_t>(unit) * kb;
  const float* sc = scores + static_cast<size_t>(unit) * Nmax;
  const uint64_t below = (1ull << lane) - 1ull;

  // round 1 (thread i: selection entry i and slot i; index clamped, no branch)
  const int i = tid;
  const bool in = i < kb;
  const int ic = min(i, kb - 1);
  const int b = in ? su[ic] : -1;
  const int sb = in ? slu[ic] : -1;  // block held by slot i
  const bool bok = b >= 0 && b < Nmax;
  const bool sok = sb >= 0 && sb < Nmax;
  for (int j = tid; j < nwords; j += blockDim.x) bitmap[j] = 0u;
  // round 2: slot of the selected block, score of the resident block
  const int res = bu[bok ? b : 0];
  const float sv = sc[sok ? sb : 0];
  __syncthreads();
  if (bok) atomicOr(&bitmap[b >> 5], 1u << (b & 31));

  // 1 + 2: ordered ranks of "missing" (by selection entry) and "free" (by slot)
  const bool miss = bok && res < 0;
  const bool fr = in && sb < 0;
  const uint64_t bm = __ballot(miss), bf = __ballot(fr);
  if (lane == 0) {
    sh.miss_tot[w] = __popcll(bm);
    sh.free_tot[w] = __popcll(bf);
  }
  __syncthreads();
  int moff = 0, foff = 0, nmiss = 0, nfree = 0;
  for (int j = 0; j < nw; ++j) {
    const int a = sh.miss_tot[j], c = sh.free_tot[j];
    moff += (j < w) ? a : 0;
    foff += (j < w) ? c : 0;
    nmiss += a;
    nfree += c;
  }
  const int mrank = moff + __popcll(bm & below);
  if (miss && mrank < cap) F[mrank] = b;
  if (fr) freeS[foff + __popcll(bf & below)] = i;
  int nF = min(cap, nmiss);
  int need = max(0, nF - nfree);  // uniform

  // 3. victims (only when the free slots do not cover the fetch)
  if (need > 0) {
    const bool cnd = sok && !((bitmap[sb >> 5] >> (sb & 31)) & 1u);
    const unsigned long long mykey =
        cnd ? ((static_cast<unsigned long long>(desc_key(sv)) << 32) | static_cast<uint32_t>(sb + 1)) : 0ull;
    if (in) ckey[i] = mykey;
    const uint64_t bc = __ballot(cnd);
    if (lane == 0) sh.cand_tot[w] = __popcll(bc);
    __syncthreads();
    int nc = 0;
    for (int j = 0; j < nw; ++j) nc += sh.cand_tot[j];
    // Consistent maps with at most k selected blocks always leave enough
    // victims; clamp anyway so inconsistent input stays within the buffers.
    if (need > nc) {
      need = nc;
      nF = nfree + nc;
    }
    if (cnd) {
      int r = 0, j = 0;
      for (; j + 8 <= kb; j += 8) {
#pragma unroll
        for (int t = 0; t < 8; ++t) r += (ckey[j + t] > mykey) ? 1 : 0;
      }
      for (; j < kb; ++j) r += (ckey[j] > mykey) ? 1 : 0;
      if (r < need) {
        vict[r] = sb;
        victS[r] = i;
      }
    }
  }
  __syncthreads();

  // 4. targets, then the map updates and the lists
  if (tid < nF) tgt[tid] = (tid < nfree) ? freeS[tid] : victS[tid - nfree];
  __syncthreads();
  if (tid < need) bu[vict[tid]] = -1;
  if (tid < nF) {
    const int s = tgt[tid];
    slu[s] = F[tid];
    bu[F[tid]] = s;
  }
  int32_t* fu = fetch + static_cast<size_t>(unit) * cap * 2;
  int32_t* eu = evict + static_cast<size_t>(unit) * cap;
  for (int j = tid; j < cap; j += blockDim.x) {
    fu[2 * j] = (j < nF) ? F[j] : -1;
    fu[2 * j + 1] = (j < nF) ? tgt[j] : -1;
    eu[j] = (j < need) ? vict[j] : -1;
  }
  if (tid == 0) n_fetch[unit] = nF;
}

}  // namespace

hipError_t launch_diff(const Ctx& c, const int32_t* sel, const float* scores, int32_t* b2s,
                       int32_t* s2b, int32_t* fetch, int32_t* n_fetch, int32_t* evict,
                       hipStream_t st) {
  const int kb = c.s.budget_blocks, cap = c.s.fetch_cap;
  const int nwords = (c.s.max_blocks + 31) / 32;
  const int threads = (kb + kWave - 1) / kWave * kWave;
  const size_t lds = static_cast<size_t>(kb) * 8 + static_cast<size_t>(nwords) * 4 +
                     static_cast<size_t>(kb + 4 * cap) * 4;
  hipLaunchKernelGGL(diff_kernel, dim3(c.units), dim3(threads), lds, st, sel, scores, b2s, s2b, fetch,
                     n_fetch, evict, c.s.max_blocks, kb, cap);
  return hipGetLastError();
}

}  // namespace oasis
