// The top-k selection and resident-set diff of one (request, KV head) by one
// workgroup of NT threads (OasisKV explainer, Figure 7 right: the draft query
// predicts the next step's top-K blocks; "What they did" item 3 and Table 2:
// only missing blocks are fetched, capped, and victims evicted), for budgets of
// at most 128 blocks: the step's second launch (NT = 512 or 1024, one workgroup
// per unit beside the split combine), the selection launch of its own, and the
// first launch that carries another state's selection (NT = 128).
#pragma once

#include "topk_body.h"

namespace oasis {

// Largest block count of a workgroup selection (k <= 128).
constexpr int kSelWgMaxBlocks = 8 * 1024;

template <int NT>
struct SelectLds {
  TopkFastShared<NT> tk;
  int32_t selL[kDiffWaveMaxBudget];                   // the selection in rank order
  uint32_t slot_keys[kDiffWaveMaxBudget];             // order key of the block in each slot
  unsigned long long diff[kDiffWaveLdsBytes / 8];      // diff_wave's arrays
  int8_t selS[kDiffWaveMaxBudget];                     // slot of each selected block (-1: none)
  uint8_t selF[kDiffWaveMaxBudget];                    // per slot: its block is selected
  int8_t slot_of[kSelWgMaxBlocks];                     // block -> slot before the step (-1: none)
};

// The unit's selection and diff: its scores, slot map (and stamps) and
// context length in one round trip of loads; the block -> slot table is built
// in LDS as the inverse of the slot map (every diff keeps block_to_slot its
// inverse, so the block map row itself is not read), and the victims' order
// keys are the selection's own keys of the blocks the slots hold, so no second
// dependent load is issued; then topk_body.h and diff_wave (LRU: least recently
// used eviction with the job's stamps).  Needs k <= 128 and Nmax <= 8192.
template <int NT, int KPT, bool LRU>
__device__ __forceinline__ void select_diff_wg(const SelectJob& job, int unit, int H, int Nmax, int kb, int cap,
                                               SelectLds<NT>& sh) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  int32_t* bu = job.b2s + static_cast<size_t>(unit) * Nmax;
  int32_t* slu = job.s2b + static_cast<size_t>(unit) * kb;
  float v[KPT];
  topk_fast_load<NT, KPT>(job.scores + static_cast<size_t>(unit) * Nmax, Nmax, v);
  int sbw[2], luw[2] = {0, 0};
  int32_t* lu = LRU ? job.last_use + static_cast<size_t>(unit) * kb : nullptr;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int ie = min(lane + e * kWave, kb - 1);  // clamped: no branch around the loads
    sbw[e] = slu[ie];
    if constexpr (LRU) luw[e] = lu[ie];
  }
  const int sb_own = slu[min(tid, kb - 1)];  // slot tid's block, for the table
  const int n = job.ctx_len[unit / H];
  uint32_t* tab = reinterpret_cast<uint32_t*>(sh.slot_of);
  for (int j = tid; j < (Nmax + 3) / 4; j += NT) tab[j] = 0xFFFFFFFFu;  // every entry -1
  if (tid < kDiffWaveMaxBudget / 4) reinterpret_cast<uint32_t*>(sh.selF)[tid] = 0u;
  __syncthreads();
  if (tid < kb && sb_own >= 0 && sb_own < Nmax) sh.slot_of[sb_own] = static_cast<int8_t>(tid);
  __syncthreads();
  topk_fast_body<NT, KPT>(v, n, unit, job.sel, Nmax, kb, sh.selL, sh.tk, sh.slot_of, sh.slot_keys, sh.selS,
                          sh.selF);
  __syncthreads();
  if (tid >= kWave) return;
  uint32_t kd[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) kd[e] = sh.slot_keys[min(lane + e * kWave, kb - 1)];
  diff_wave(unit, kb, Nmax, cap, sh.selL, sh.selS, sh.selF, sbw, kd, luw, lu, job.step, bu, slu, job.fetch,
            job.n_fetch, job.evict, job.attend, job.n_attend, sh.diff);
}

}  // namespace oasis
