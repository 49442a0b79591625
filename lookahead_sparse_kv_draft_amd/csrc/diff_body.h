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
  return static_cast<size_t>(kb) * 8 + nwords * 4 + static_cast<size_t>(3 * kb + 4 * cap) * 4;
}

// Number of entries of a[0 .. n) below `mine`, counted by P adjacent threads
// (this thread is `part` of them; P <= 16, the group fully active) and summed
// across their lanes.  The reads of
// a batch are unconditional (indices clamped), so they are in flight together.
template <typename K>
__device__ __forceinline__ int rank_below(const K* a, int n, K mine, int P, int part) {
  constexpr int kBatch = 8;
  int r = 0;
  for (int j = part; j < n; j += kBatch * P) {
    K x[kBatch];
#pragma unroll
    for (int t = 0; t < kBatch; ++t) x[t] = a[min(j + t * P, n - 1)];
#pragma unroll
    for (int t = 0; t < kBatch; ++t) r += static_cast<int>((j + t * P < n) & (x[t] < mine));
  }
  return group_sum(r, P);
}

// selL: LDS [kb], the selection in rank order (complete and visible on entry).
// sb: block held by slot tid (slot_to_block, -1 = free; any value for tid >= kb);
// sv: that block's score.  bu/slu: this unit's block_to_slot / slot_to_block rows.
// attend / n_attend (optional, both or neither): the attended list the next
// attention needs, i.e. the selected blocks resident once this step's fetch has
// landed, in rank order, packed block << 10 | slot, and its length.
__device__ __forceinline__ void diff_body(int unit, int kb, int Nmax, int cap, const int32_t* selL, int sb, float sv,
                                 int32_t* __restrict__ bu, int32_t* __restrict__ slu,
                                 int32_t* __restrict__ fetch, int32_t* __restrict__ n_fetch,
                                 int32_t* __restrict__ evict, int32_t* __restrict__ attend,
                                 int32_t* __restrict__ n_attend, unsigned long long* lds, DiffShared& sh) {
  unsigned long long* candK = lds;                           // [kb] complemented keys of the candidates
  const int nwords = (Nmax + 31) / 32;
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(candK + kb);  // [nwords] selected blocks
  int32_t* F = reinterpret_cast<int32_t*>(bitmap + nwords);  // [cap] fetched blocks
  int32_t* tgt = F + cap;                                     // [cap] their target slots
  int32_t* freeS = tgt + cap;                                 // [kb] free slots, ascending
  int32_t* vict = freeS + kb;                                 // [cap] victim blocks
  int32_t* victS = vict + cap;                                // [cap] victim slots
  int32_t* candS = victS + cap;                               // [kb] the candidates' slots

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  // Only the first ceil(k / 64) wavefronts hold selection entries and slots; in
  // a larger workgroup the others skip the per-entry work (wavefront-uniform
  // branches) and only meet the barriers, so they take no issue slots from the
  // wavefronts on the critical path.
  const int nwa = min(static_cast<int>(blockDim.x) / kWave, (kb + kWave - 1) / kWave);
  const bool act = w < nwa;
  const uint64_t below = (1ull << lane) - 1ull;
  const int i = tid;
  const bool in = i < kb;
  if (!in) sb = -1;
  int b = -1, res = -1;
  if (act) {
    b = in ? selL[i] : -1;
    res = bu[(b >= 0 && b < Nmax) ? b : 0];  // slot of the selected block (index clamped: no branch)
  }
  const bool bok = b >= 0 && b < Nmax;
  const bool sok = sb >= 0 && sb < Nmax;
  for (int j = tid; j < nwords; j += blockDim.x) bitmap[j] = 0u;
  __syncthreads();
  if (bok) atomicOr(&bitmap[b >> 5], 1u << (b & 31));

  // 1 + 2: ordered ranks of "missing" (by selection entry) and "free" (by slot)
  const bool miss = bok && res < 0;
  const bool fr = in && sb < 0;
  uint64_t bm = 0ull, bf = 0ull;
  if (act) {
    bm = __ballot(miss);
    bf = __ballot(fr);
    if (lane == 0) {
      sh.miss_tot[w] = __popcll(bm);
      sh.free_tot[w] = __popcll(bf);
    }
  }
  __syncthreads();
  int moff = 0, foff = 0, nmiss = 0, nfree = 0;
  for (int j = 0; j < nwa; ++j) {
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

  // 3. victims (only when the free slots do not cover the fetch): the
  // candidates are compacted (slot order), then each one's place is the number
  // of candidates with a larger key.  Usually few slots are candidates (about
  // as many as blocks are missing), so this is short.
  if (need > 0) {
    bool cnd = false;
    unsigned long long mykey = 0ull;
    uint64_t bc = 0ull;
    if (act) {
      cnd = sok && !((bitmap[sb >> 5] >> (sb & 31)) & 1u);
      mykey = (static_cast<unsigned long long>(desc_key(sv)) << 32) | static_cast<uint32_t>(sb + 1);
      bc = __ballot(cnd);
      if (lane == 0) sh.cand_tot[w] = __popcll(bc);
    }
    __syncthreads();
    int nc = 0, coff = 0;
    for (int j = 0; j < nwa; ++j) {
      const int a = sh.cand_tot[j];
      coff += (j < w) ? a : 0;
      nc += a;
    }
    if (cnd) {
      const int pos = coff + __popcll(bc & below);
      candK[pos] = ~mykey;  // complemented: a larger key ranks first
      candS[pos] = i;
    }
    // Consistent maps with at most k selected blocks always leave enough
    // victims; clamp anyway so inconsistent input stays within the buffers.
    if (need > nc) {
      need = nc;
      nF = nfree + nc;
    }
    __syncthreads();
    const int nthr = static_cast<int>(blockDim.x);
    const int P = (nc * 8 <= nthr) ? 8 : (nc * 4 <= nthr) ? 4 : (nc * 2 <= nthr) ? 2 : 1;
    const int ci = tid / P, part = tid & (P - 1);
    if (ci < nc) {  // whole groups of P adjacent lanes: the shuffles stay inside them
      const unsigned long long ck = candK[ci];
      const int r = rank_below(candK, nc, ck, P, part);
      if (part == 0 && r < need) {
        vict[r] = static_cast<int32_t>(~ck & 0xFFFFFFFFull) - 1;  // the block (stored + 1)
        victS[r] = candS[ci];
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

  // 5. the attended list for the next attention: selected blocks that stay
  // resident (a resident selected block is never a victim) or are fetched now
  if (attend != nullptr) {
    int slot_after = -1;
    if (bok) slot_after = (res >= 0) ? res : ((miss && mrank < nF) ? tgt[mrank] : -1);
    const bool att = in && slot_after >= 0 && slot_after < kb;
    uint64_t ba = 0ull;
    if (act) {
      ba = __ballot(att);
      if (lane == 0) sh.att_tot[w] = __popcll(ba);
    }
    __syncthreads();
    int off = 0, tot = 0;
    for (int j = 0; j < nwa; ++j) {
      const int a = sh.att_tot[j];
      off += (j < w) ? a : 0;
      tot += a;
    }
    if (att) attend[static_cast<size_t>(unit) * kb + off + __popcll(ba & below)] = (b << kAttendSlotBits) | slot_after;
    if (tid == 0) n_attend[unit] = tot;
  }
}

// The same step run by ONE wavefront for k <= 128 (the largest shape of the
// decode step's default path): lane l handles selection entries and slots l and
// l + 64, every rank is a ballot within the wavefront, so there is no barrier at
// all (the wavefront's LDS accesses complete in order).  A lone wavefront issues
// about one instruction every four cycles, so the step is written for few
// instructions and few dependent LDS round trips: the selection arrives with
// what the top-k found out while ranking it, and each lane writes the list
// entries it owns directly.
//   selL: LDS [kb], the selection in rank order (-1 padded);
//   selS: LDS [kb], the slot each selected block held before the step (-1: not
//         resident);
//   selF: LDS [kb], per slot: 1 when the block it holds is selected;
//   sb:   the slot map for slots l and l + 64 (-1 / any for slots >= kb);
//   kd:   the selection's order keys (desc_key of the score) of the blocks in
//         those two slots, read only for resident blocks outside the selection
//         (the diff ranks victims by the same keys as the selection).
// Least-recently-used eviction when lu (this unit's per-slot stamps) is not
// null: luv holds the stamps of slots l and l + 64; victims are taken oldest
// stamp first, then in the lowest-score order, and the slots the next attention
// reads are stamped with `step` ([EXPL] Table 2 runs LRU eviction).
constexpr int kDiffWaveMaxBudget = 2 * kWave;
constexpr int kDiffWavePad = 8;  // the victim ranking reads the candidates 8 at a time
// LDS bytes diff_wave carves: candidate keys and stamps (padded), targets.
constexpr int kDiffWaveLdsBytes = (kDiffWaveMaxBudget + kDiffWavePad) * 12 + kDiffWaveMaxBudget * 4;

__device__ __forceinline__ void diff_wave(int unit, int kb, int Nmax, int cap, const int32_t* selL,
                                          const int8_t* selS, const uint8_t* selF, const int (&sb)[2],
                                          const uint32_t (&kd)[2], const int (&luv)[2], int32_t* __restrict__ lu,
                                          int step, int32_t* __restrict__ bu, int32_t* __restrict__ slu,
                                          int32_t* __restrict__ fetch, int32_t* __restrict__ n_fetch,
                                          int32_t* __restrict__ evict, int32_t* __restrict__ attend,
                                          int32_t* __restrict__ n_attend, unsigned long long* lds) {
  unsigned long long* candK = lds;                                                         // [kb + pad]
  int32_t* tgt = reinterpret_cast<int32_t*>(candK + kDiffWaveMaxBudget + kDiffWavePad);   // [kb]
  int32_t* candA = tgt + kDiffWaveMaxBudget;                                              // [kb + pad] LRU
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t below = (1ull << lane) - 1ull;
  int b[2], res[2];
  bool in[2], bok[2], miss[2], cnd[2];
  uint64_t bm[2], bf[2], bc[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int i = lane + e * kWave;
    const int ic = min(i, kb - 1);  // clamped: no branch around the reads
    in[e] = i < kb;
    const int bl = selL[ic];
    const int rs = selS[ic];
    const bool f = selF[ic] != 0;
    b[e] = in[e] ? bl : -1;
    bok[e] = b[e] >= 0 && b[e] < Nmax;
    res[e] = bok[e] ? rs : -1;
    miss[e] = bok[e] && res[e] < 0;
    cnd[e] = in[e] && sb[e] >= 0 && sb[e] < Nmax && !f;  // resident, outside the selection
    bm[e] = __ballot(miss[e]);
    bf[e] = __ballot(in[e] && sb[e] < 0);
    bc[e] = __ballot(cnd[e]);
  }
  // 1 + 2: missing blocks in selection order, free slots in ascending order
  const int nm0 = __popcll(bm[0]), nf0 = __popcll(bf[0]), nc0 = __popcll(bc[0]);
  const int nmiss = nm0 + __popcll(bm[1]), nfree = nf0 + __popcll(bf[1]), nc = nc0 + __popcll(bc[1]);
  int nF = min(cap, nmiss);
  int need = max(0, nF - nfree);
  // Consistent maps with at most k selected blocks always leave enough
  // victims; clamp anyway so inconsistent input stays within the buffers.
  if (need > nc) {
    need = nc;
    nF = nfree + nc;
  }

  // 3. victims: resident blocks outside the selection, compacted in slot order
  // (sentinels after the last one), each placed by the number of candidates
  // with a larger key
  int r[2] = {need, need};
  if (need > 0) {
    unsigned long long ck[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      ck[e] = ~((static_cast<unsigned long long>(kd[e]) << 32) | static_cast<uint32_t>(sb[e] + 1));
      if (cnd[e]) {
        const int pos = (e ? nc0 : 0) + __popcll(bc[e] & below);
        candK[pos] = ck[e];  // complemented: a larger key ranks first
        if (lu != nullptr) candA[pos] = luv[e];
      }
    }
    if (lane < kDiffWavePad) {
      candK[nc + lane] = ~0ull;  // never below a candidate's key
      if (lu != nullptr) candA[nc + lane] = 0x7FFFFFFF;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    int r0 = 0, r1 = 0;
    if (lu == nullptr) {
      for (int j = 0; j < nc; j += kDiffWavePad) {
        unsigned long long x[kDiffWavePad];
#pragma unroll
        for (int t = 0; t < kDiffWavePad; ++t) x[t] = candK[j + t];
#pragma unroll
        for (int t = 0; t < kDiffWavePad; ++t) {
          r0 += static_cast<int>(x[t] < ck[0]);
          r1 += static_cast<int>(x[t] < ck[1]);
        }
      }
    } else {
      // (older stamp, then the lowest-score order) ranks first
      for (int j = 0; j < nc; j += kDiffWavePad) {
        unsigned long long x[kDiffWavePad];
        int a[kDiffWavePad];
#pragma unroll
        for (int t = 0; t < kDiffWavePad; ++t) {
          x[t] = candK[j + t];
          a[t] = candA[j + t];
        }
#pragma unroll
        for (int t = 0; t < kDiffWavePad; ++t) {
          r0 += static_cast<int>((a[t] < luv[0]) | ((a[t] == luv[0]) & (x[t] < ck[0])));
          r1 += static_cast<int>((a[t] < luv[1]) | ((a[t] == luv[1]) & (x[t] < ck[1])));
        }
      }
    }
    r[0] = cnd[0] ? r0 : need;
    r[1] = cnd[1] ? r1 : need;
  }

  // 4. targets (free slots, then the victims' slots in rank order); each
  // victim's lane writes its evict entry and clears its block's slot
  int32_t* fu = fetch + static_cast<size_t>(unit) * cap * 2;
  int32_t* eu = evict + static_cast<size_t>(unit) * cap;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int slot = lane + e * kWave;
    if ((bf[e] >> lane) & 1ull) {
      const int fr = (e ? nf0 : 0) + __popcll(bf[e] & below);
      if (fr < nF) tgt[fr] = slot;
    }
    if (r[e] < need) {
      tgt[nfree + r[e]] = slot;
      eu[r[e]] = sb[e];
      bu[sb[e]] = -1;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  // 5. each fetched block's lane takes its target: fetch entry and both maps
  int sa[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int mrank = (e ? nm0 : 0) + __popcll(bm[e] & below);
    sa[e] = res[e];
    if (miss[e] && mrank < nF) {
      const int s = tgt[mrank];
      fu[2 * mrank] = b[e];
      fu[2 * mrank + 1] = s;
      slu[s] = b[e];
      bu[b[e]] = s;
      sa[e] = s;
    }
  }
  for (int j = nF + lane; j < cap; j += kWave) {
    fu[2 * j] = -1;
    fu[2 * j + 1] = -1;
  }
  for (int j = need + lane; j < cap; j += kWave) eu[j] = -1;
  if (lane == 0) n_fetch[unit] = nF;

  // 6. the attended list for the next attention (selection order); with LRU
  // its slots take this step's stamp
  if (attend != nullptr || lu != nullptr) {
    uint64_t ba[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      ba[e] = __ballot(in[e] && sa[e] >= 0 && sa[e] < kb);
      if (lu != nullptr && ((ba[e] >> lane) & 1ull)) lu[sa[e]] = step;
    }
    if (attend == nullptr) return;
    const int na0 = __popcll(ba[0]);
    int32_t* au = attend + static_cast<size_t>(unit) * kb;
#pragma unroll
    for (int e = 0; e < 2; ++e)
      if ((ba[e] >> lane) & 1ull) au[(e ? na0 : 0) + __popcll(ba[e] & below)] = (b[e] << kAttendSlotBits) | sa[e];
    if (lane == 0) n_attend[unit] = na0 + __popcll(ba[1]);
  }
}

}  // namespace oasis
