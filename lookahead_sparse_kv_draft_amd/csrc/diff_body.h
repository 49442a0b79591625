// The set-difference / capped-fetch / capped-eviction step shared by the
// standalone diff kernel and the fused select-and-diff kernel (OasisKV
// explainer, "What they did" item 3 and Table 2: only missing predicted blocks
// are fetched, bounded per step; Figure 9: a per-KV-head table maps each GPU
// block slot to a CPU block, kept here with its inverse).
//
// Run by every thread of a workgroup of whole wavefronts with at least k
// threads; thread i handles selection entry i and slot i:
//   1. missing = selected blocks without a slot, in rank order; the first
//      min(cap, |missing|) are fetched;
//   2. free slots in ascending order;
//   3. if the free slots do not cover the fetch, the victims are the resident
//      blocks outside the selection with the largest (descending score,
//      ascending index) keys, i.e. lowest score first and the higher index first
//      among equal scores; each candidate's place is the number of larger keys;
//   4. targets = free slots, then the victims' slots; both maps are updated in
//      place after every read of the old state.
#pragma once

#include "oasis_internal.h"

namespace oasis {

constexpr int kDiffMaxWaves = kMaxBudget / kWave;

struct DiffShared {
  int miss_tot[kDiffMaxWaves], free_tot[kDiffMaxWaves], cand_tot[kDiffMaxWaves], att_tot[kDiffMaxWaves];
};

// Dynamic LDS bytes of diff_body (8-byte aligned start).
__host__ __device__ inline size_t diff_lds_bytes(int kb, int Nmax, int cap) {
  const size_t nwords = static_cast<size_t>(Nmax + 31) / 32;
  return static_cast<size_t>(kb) * 8 + nwords * 4 + static_cast<size_t>(kb + 4 * cap) * 4;
}

// selL: LDS [kb], the selection in rank order (complete and visible on entry).
// sb: block held by slot tid (slot_to_block, -1 = free; any value for tid >= kb);
// sv: that block's score.  bu/slu: this unit's block_to_slot / slot_to_block rows.
// attend / n_attend (optional, both or neither): the attended list the next
// attention needs, i.e. the selected blocks resident once this step's fetch has
// landed, in rank order, packed block << 10 | slot, and its length.
__device__ inline void diff_body(int unit, int kb, int Nmax, int cap, const int32_t* selL, int sb, float sv,
                                 int32_t* __restrict__ bu, int32_t* __restrict__ slu,
                                 int32_t* __restrict__ fetch, int32_t* __restrict__ n_fetch,
                                 int32_t* __restrict__ evict, int32_t* __restrict__ attend,
                                 int32_t* __restrict__ n_attend, unsigned long long* lds, DiffShared& sh) {
  unsigned long long* ckey = lds;                            // [kb] candidate key per slot (0 = none)
  const int nwords = (Nmax + 31) / 32;
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(ckey + kb);  // [nwords] selected blocks
  int32_t* F = reinterpret_cast<int32_t*>(bitmap + nwords);  // [cap] fetched blocks
  int32_t* tgt = F + cap;                                     // [cap] their target slots
  int32_t* freeS = tgt + cap;                                 // [kb] free slots, ascending
  int32_t* vict = freeS + kb;                                 // [cap] victim blocks
  int32_t* victS = vict + cap;                                // [cap] victim slots

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int nw = blockDim.x / kWave;
  const uint64_t below = (1ull << lane) - 1ull;
  const int i = tid;
  const bool in = i < kb;
  const int b = in ? selL[i] : -1;
  if (!in) sb = -1;
  const bool bok = b >= 0 && b < Nmax;
  const bool sok = sb >= 0 && sb < Nmax;
  for (int j = tid; j < nwords; j += blockDim.x) bitmap[j] = 0u;
  const int res = bu[bok ? b : 0];  // slot of the selected block (index clamped: no branch)
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
    // Each candidate's place = number of larger keys (non-candidates hold 0),
    // counted by P adjacent threads per slot and summed across their lanes.
    const int P0 = static_cast<int>(blockDim.x) / kb;
    const int P = (P0 >= 16) ? 16 : (P0 >= 8) ? 8 : (P0 >= 4) ? 4 : (P0 >= 2) ? 2 : 1;
    const int ci = tid / P, part = tid & (P - 1);
    const unsigned long long ck = (ci < kb) ? ckey[ci] : 0ull;
    // (the reads of a batch are unconditional, indices clamped, so they are
    // in flight together)
    constexpr int kBatch = 8;
    int r = 0;
    for (int j = part; j < kb; j += kBatch * P) {
      unsigned long long x[kBatch];
#pragma unroll
      for (int t = 0; t < kBatch; ++t) x[t] = ckey[min(j + t * P, kb - 1)];
#pragma unroll
      for (int t = 0; t < kBatch; ++t) r += static_cast<int>((j + t * P < kb) & (x[t] > ck));
    }
    for (int o = 1; o < P; o <<= 1) r += __shfl_xor(r, o);
    if (part == 0 && ck != 0ull && r < need) {
      vict[r] = static_cast<int32_t>(ck & 0xFFFFFFFFull) - 1;  // the block (stored + 1)
      victS[r] = ci;
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

  // 5. the attended list for the next attention: selected blocks that stay
  // resident (a resident selected block is never a victim) or are fetched now
  if (attend != nullptr) {
    int slot_after = -1;
    if (bok) slot_after = (res >= 0) ? res : ((miss && mrank < nF) ? tgt[mrank] : -1);
    const bool att = in && slot_after >= 0 && slot_after < kb;
    const uint64_t ba = __ballot(att);
    if (lane == 0) sh.att_tot[w] = __popcll(ba);
    __syncthreads();
    int off = 0, tot = 0;
    for (int j = 0; j < nw; ++j) {
      const int a = sh.att_tot[j];
      off += (j < w) ? a : 0;
      tot += a;
    }
    if (att) attend[static_cast<size_t>(unit) * kb + off + __popcll(ba & below)] = (b << kAttendSlotBits) | slot_after;
    if (tid == 0) n_attend[unit] = tot;
  }
}

}  // namespace oasis
