// The sparse paged decode attention of one workgroup (one split of one
// unit's attended set): shared by the attention kernel and by the launch that
// carries the attention and the lookahead scoring together.  The algorithm and
// its layout are described in attn.hip (OasisKV explainer, Figure 7 right).
#pragma once

#include "oasis_internal.h"

namespace oasis {

constexpr float kLazyRescale = 8.f;

// Two wavefronts per SIMD for the 2-page ring with up to three row tiles: the
// registers then hold the accumulators too (no spills), and a second wavefront
// hides the first one's MFMA and exchange latencies.
// W wavefronts per workgroup, splits workgroups per unit; each wavefront takes
// an even share (at most `run` entries) of the unit's attended list and streams
// its pages through a ring of PF page buffers in registers (PF pages always in
// flight, every wait exact).  The wavefronts merge in LDS; with one
// split the workgroup writes the output, otherwise its partial (unnormalised
// accumulator, row max, row sum) for the combine kernel.
// The LDS of one attention workgroup: the wavefronts' row statistics and
// accumulator slices for the merge, and the unit's attended list when the
// workgroup builds it from the selection and the block map.  A kernel that also
// runs other kinds of workgroups can overlay this with their LDS.
template <int D, int RT, int W>
struct AttnLds {
  static constexpr int NSLICE = (W > 1) ? W / 2 : 1;
  float m[W][RT * 16];
  float l[W][RT * 16];
  float4 slice[NSLICE][RT][D / 16][kWave];  // wavefront accumulators in register layout
  int att[kMaxBudget];
  int wcnt[4][W];
  int last;  // the in-launch merge: this workgroup arrived last for its unit
};

// Device-coherent (sc1: coherent across the XCDs' L2 caches) 16- and 8-byte
// accesses for the split partials that another workgroup of the same launch
// reads: only these take the coherent path, nothing is written back or
// invalidated wholesale.
constexpr int kCoherentDevice = 16;
typedef unsigned int u32v4_t __attribute__((__vector_size__(16)));
typedef unsigned int u32v2_t __attribute__((__vector_size__(8)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ void store_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32v4_t, v), r, off, 0, kCoherentDevice);
}
__device__ __forceinline__ void store_coherent2(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x2_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32v2_t, v), r, off, 0, kCoherentDevice);
}
__device__ __forceinline__ f32x4_t load_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherentDevice));
}
__device__ __forceinline__ f32x2_t load_coherent2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCoherentDevice));
}

// The split merge inside the attention's launch (arrive: one counter per unit,
// zero before the launch; the merging workgroup leaves it zero again).
// Wavefront 0 writes the workgroup's partial (unnormalised accumulator, row
// max, row sum) with device-coherent stores, waits for them and counts the
// workgroup in with a device-scope atomic; the workgroup that arrives last
// merges every split of its unit from device-coherent loads and writes the
// output.  The arithmetic is the split combine's (attn_combine.h): the rows'
// maximum over the splits first, then sum_s 2^(m_s - M) acc_s and
// sum_s 2^(m_s - M) l_s accumulated over s = 0, 1, ... in that order, so the
// output equals the combine launch's bit for bit.  Wavefront w merges the
// channel tiles w, w + W, ...  Needs splits <= kAttnMergeMaxSplits.
template <int D, int RT, int W>
__device__ __forceinline__ void merge_in_launch(const f32x4_t (&acc)[RT][D / 16], const float (&mrun)[RT],
                                                const float (&Lwg)[RT], float* __restrict__ ws_acc,
                                                float* __restrict__ ws_ml, float* __restrict__ out, int rows,
                                                int splits, int unit, int wid, int32_t* __restrict__ arrive,
                                                AttnLds<D, RT, W>& lds) {
  constexpr int CT = D / 16;
  constexpr int CW = (CT + W - 1) / W;
  constexpr int SM = kAttnMergeMaxSplits;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const __amdgpu_buffer_rsrc_t racc = coherent_rsrc(ws_acc, 0x7FFFFFFF);
  const __amdgpu_buffer_rsrc_t rml = coherent_rsrc(ws_ml, 0x7FFFFFFF);
  if (wv == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = rt * 16 + col;
      if (row < rows) {
        const uint32_t p = static_cast<uint32_t>(wid * rows + row);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) store_coherent4(racc, (p * D + 16 * ct + 4 * grp) * 4u, acc[rt][ct]);
        if (grp == 0) store_coherent2(rml, p * 8u, f32x2_t{mrun[rt], Lwg[rt]});
      }
    }
    // the partial is complete at device scope before the count says so
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    int old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(arrive + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (lane == 0) lds.last = (old == splits - 1) ? 1 : 0;
  }
  __syncthreads();
  if (lds.last == 0) return;
  asm volatile("" ::: "memory");  // the loads below stay after the count

  // Every split's row statistics and the first SB splits' accumulators are
  // requested together, then the rest SB splits at a time (registers allow 4
  // with up to two row tiles, 2 with more): two round trips for 8 splits.
  constexpr int SB = (RT <= 2) ? 4 : 2;
  f32x2_t ml[RT][SM];
  f32x4_t v[SB][RT][CW];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int rr = min(rt * 16 + col, rows - 1);  // padded rows read row rows-1 and write nothing
        const uint32_t p = static_cast<uint32_t>((unit * splits + min(s0 + u, splits - 1)) * rows + rr);
#pragma unroll
        for (int i = 0; i < CW; ++i) {
          const int ct = min(wv + W * i, CT - 1);
          v[u][rt][i] = load_coherent4(racc, (p * D + 16 * ct + 4 * grp) * 4u);
        }
      }
  };
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rr = min(rt * 16 + col, rows - 1);
#pragma unroll
    for (int s = 0; s < SM; ++s) {
      const uint32_t p = static_cast<uint32_t>((unit * splits + min(s, splits - 1)) * rows + rr);
      ml[rt][s] = load_coherent2(rml, p * 8u);
    }
  }
  load_batch(0);
  // the rows' maximum over the splits, then each split's weight and the sum
  float w[RT][SM], L[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < SM; ++s) M = fmaxf(M, ml[rt][s][0]);  // repeats do not change the max
    L[rt] = 0.f;
#pragma unroll
    for (int s = 0; s < SM; ++s) {
      w[rt][s] = (s >= splits || ml[rt][s][0] == -INFINITY) ? 0.f : exp2f(ml[rt][s][0] - M);
      L[rt] += w[rt][s] * ml[rt][s][1];
    }
  }
  f32x4_t a[RT][CW];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < CW; ++i) a[rt][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // accumulated in split order
#pragma unroll
  for (int s0 = 0; s0 < SM; s0 += SB) {
    if (s0 >= splits) break;
    if (s0 > 0) load_batch(s0);
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < CW; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) a[rt][i][j] += w[rt][s0 + u] * v[u][rt][i][j];
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + col;
    if (row >= rows) continue;
    const float inv = (L[rt] > 0.f) ? 1.f / L[rt] : 0.f;
    float* orow = out + (static_cast<size_t>(unit) * rows + row) * D;
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int ct = wv + W * i;
      if (ct < CT)
        *reinterpret_cast<float4*>(orow + 16 * ct + 4 * grp) =
            make_float4(a[rt][i][0] * inv, a[rt][i][1] * inv, a[rt][i][2] * inv, a[rt][i][3] * inv);
    }
  }
  if (tid == 0) __hip_atomic_store(arrive + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int RT, int W, int PF>
__device__ __forceinline__ void attn_wg(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ pool,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ b2s, const int32_t* __restrict__ attend,
    const int32_t* __restrict__ n_attend, const int32_t* __restrict__ ctx_len, float* __restrict__ ws_acc,
    float* __restrict__ ws_ml, float* __restrict__ out, int H, int rows, int Nmax, int kb,
    int splits, int run, float scale_log2, int wid, AttnLds<D, RT, W>& lds, int32_t* __restrict__ arrive = nullptr) {
  constexpr int KS = D / 32;  // QK k-steps of 32 channels
  constexpr int CT = D / 16;  // PV channel tiles
  constexpr int PAGE = 2 * kBlock * D;
  constexpr int NT = 64 * W;
  auto& sm_m = lds.m;
  auto& sm_l = lds.l;
  auto& sm_slice = lds.slice;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int col = lane & 15;
  const int grp = lane >> 4;
  // wid = unit * splits + split
  const int unit = wid / splits;
  const int split = wid - unit * splits;
  const int n = ctx_len[unit / H];

  // Query rows as the B operand of S^T = K Q^T: lane (col, grp) holds row
  // rt*16+col, channels 8*(4s+grp) .. +7 for k-step s.  Issued first: they do
  // not depend on the selection lookups below.
  uint4 Qb[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + col;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      // row clamped so the load is unconditional; padded rows are zeroed below
      Qb[rt][s] = *reinterpret_cast<const uint4*>(q + (static_cast<size_t>(unit) * rows + min(row, rows - 1)) * D +
                                                  8 * (4 * s + grp));
      if (row >= rows) Qb[rt][s] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  // This wavefront's pages: nb entries, slot and token count of entry j in lane j.
  int nb, c_slot, c_ntok;
  if (attend != nullptr) {
    // The attended list a diff left (rank order, block << 10 | slot) and its
    // length; this wavefront takes a contiguous share of an even split over all
    // splits * W wavefronts of the unit.  The share of a full list (length k,
    // the steady state) is loaded beside the length, so the page loads wait for
    // one round trip, not two; a shorter list loads its own share after.
    const int nwv = splits * W;
    const int* au = attend + static_cast<size_t>(unit) * kb;
    const int perk = (kb + nwv - 1) / nwv;
    const int e0k = (split * W + wv) * perk;
    int pk = au[min(e0k + lane, kb - 1)];  // clamped: no branch around the load
    // a compiler-only barrier (no instruction, no wait): the load above is issued
    // here, not merged with the short-list load below into one that waits for
    // the length
    asm volatile("" ::: "memory");
    const int natt = min(max(n_attend[unit], 0), kb);
    const int per = (natt + nwv - 1) / nwv;  // <= run <= 64
    const int e0 = (split * W + wv) * per;
    const int cnt = max(0, min(per, natt - e0));
    if (natt != kb) pk = au[min(e0 + lane, kb - 1)];  // wavefront-uniform
    if (lane >= cnt) pk = 0;
    int my_slot = -1, my_ntok = 0;
    if (lane < cnt) {
      const int b = pk >> kAttendSlotBits;
      const int sl = pk & ((1 << kAttendSlotBits) - 1);
      const int nt = min(kBlock, n - kBlock * b);
      if (b >= 0 && b < Nmax && sl < kb && nt > 0) {
        my_slot = sl;
        my_ntok = nt;
      }
    }
    // compact the usable entries into lanes 0 .. nb-1 (forward lane permute)
    const uint64_t valid = __ballot(my_slot >= 0);
    nb = __popcll(valid);
    const int dst = (my_slot >= 0 ? __popcll(valid & ((1ull << lane) - 1ull)) : 63) * 4;
    c_slot = __builtin_amdgcn_ds_permute(dst, my_slot);
    c_ntok = __builtin_amdgcn_ds_permute(dst, my_ntok);
  } else {
    // The unit's attended entries (selected blocks that are resident and hold
    // tokens below n), in rank order, packed slot | ntok << 16: every workgroup of
    // the unit builds the whole list in LDS (lookups in batches of four entries
    // per thread, all loads of a batch in flight), then takes its wavefronts'
    // shares of an even split over all splits * W wavefronts of the unit, so every
    // wavefront streams the same number of pages (+-1).
    auto& sm_att = lds.att;
    auto& sm_wcnt = lds.wcnt;
    const uint64_t below = (1ull << lane) - 1ull;
    int natt = 0;
    for (int c0 = 0; c0 < kb; c0 += 4 * NT) {
      int bsel[4], slot[4];
  #pragma unroll
      for (int u = 0; u < 4; ++u) bsel[u] = sel[static_cast<size_t>(unit) * kb + min(c0 + u * NT + tid, kb - 1)];
  #pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int b = bsel[u];
        slot[u] = b2s[static_cast<size_t>(unit) * Nmax + ((b >= 0 && b < Nmax) ? b : 0)];
      }
      int v[4];
      uint64_t bal[4];
  #pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = c0 + u * NT + tid;
        const int b = bsel[u];
        const int nt = min(kBlock, n - kBlock * b);
        const bool ok = i < kb && b >= 0 && b < Nmax && slot[u] >= 0 && slot[u] < kb && nt > 0;
        v[u] = ok ? (slot[u] | (nt << 16)) : -1;
        bal[u] = __ballot(ok);
        if (lane == 0) sm_wcnt[u][wv] = __popcll(bal[u]);
      }
      __syncthreads();
  #pragma unroll
      for (int u = 0; u < 4; ++u) {
        int before = 0, tot = 0;
  #pragma unroll
        for (int w = 0; w < W; ++w) {
          const int cw = sm_wcnt[u][w];
          before += (w < wv) ? cw : 0;
          tot += cw;
        }
        if (v[u] >= 0) sm_att[natt + before + __popcll(bal[u] & below)] = v[u];
        natt += tot;
      }
      __syncthreads();  // the list is complete; sm_wcnt may be reused
    }
    // this wavefront's contiguous share, as above
    const int nwv = splits * W;
    const int per = (natt + nwv - 1) / nwv;  // <= run <= 64
    const int e0 = (split * W + wv) * per;
    nb = max(0, min(per, natt - e0));
    const int mine = (lane < nb) ? sm_att[e0 + lane] : 0;
    c_slot = mine & 0xFFFF;
    c_ntok = mine >> 16;
  }

  f32x4_t acc[RT][CT];
  float mrun[RT], lrun[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    mrun[rt] = -INFINITY;
    lrun[rt] = 0.f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const uint16_t* ubase = pool + static_cast<size_t>(unit) * kb * PAGE;
  struct Page {
    uint4 k[KS];
    uint2 v[CT];
  };
  // The page base is wavefront-uniform (scalar registers, read from the entry's
  // lane; entry indices stay below nb <= 64); the lane offsets are the same for
  // every page.
  const uint16_t* kl = ubase + col * D + 8 * grp;
  const uint16_t* vl = ubase + kBlock * D + col * kBlock + 4 * grp;
  auto load = [&](Page& pg, int j) {
    const size_t off = static_cast<size_t>(__builtin_amdgcn_readlane(c_slot, j)) * PAGE;
#pragma unroll
    for (int s = 0; s < KS; ++s) pg.k[s] = load_stream(reinterpret_cast<const uint4*>(kl + off + 32 * s));
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) pg.v[ct] = load_stream(reinterpret_cast<const uint2*>(vl + off + 16 * kBlock * ct));
  };
  auto process = [&](const Page& pg, int ntok) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pg.k[s]), as_bf16x8(Qb[rt][s]), st, 0, 0, 0);
      float x[4];
      float mb = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = (4 * grp + i < ntok) ? st[i] * scale_log2 : -INFINITY;
        mb = fmaxf(mb, x[i]);
      }
      mb = max_xor32(max_xor16(mb));
      // The reference max moves only when a row's block max exceeds it by more
      // than kLazyRescale (log2 units; the first block always moves it), so the
      // accumulators are rescaled rarely; probabilities stay below 2^kLazyRescale.
      if (__ballot(mb > mrun[rt] + kLazyRescale) != 0ull) {
        const float mnew = fmaxf(mrun[rt], mb);
        const float alpha = exp2f(mrun[rt] - mnew);
        mrun[rt] = mnew;
        lrun[rt] *= alpha;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[rt][ct] *= alpha;
      }
      // probabilities rounded to bf16 in pairs by the hardware conversion
      // (round to nearest even); the running sum adds the rounded values
      const f32x2_t p01 = {exp2f(x[0] - mrun[rt]), exp2f(x[1] - mrun[rt])};
      const f32x2_t p23 = {exp2f(x[2] - mrun[rt]), exp2f(x[3] - mrun[rt])};
      const uint2 pw = make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(p01, bf16x2_t)),
                                  __builtin_bit_cast(uint32_t, __builtin_convertvector(p23, bf16x2_t)));
      lrun[rt] += ((__uint_as_float(pw.x << 16) + __uint_as_float(pw.x & 0xFFFF0000u)) +
                   __uint_as_float(pw.y << 16)) + __uint_as_float(pw.y & 0xFFFF0000u);
      const s16x4_t P = as_s16x4(pw);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_s16x4(pg.v[ct]), P, acc[rt][ct], 0, 0, 0);
    }
  };

  // Ring of PF page buffers over the nb attended entries, padded to a multiple
  // of PF: the first PF loads, then groups of PF pages where each processed
  // buffer is refilled with the page PF entries ahead, then the last group.
  // Every load is unconditional (indices clamped: only a padded last group
  // repeats the last page), so each wait covers exactly the older buffers; the
  // processing issues no loads, so skipping padded entries keeps them exact.
  if (nb > 0) {
    Page pg[PF];
    const int npad = (nb + PF - 1) / PF * PF;
#pragma unroll
    for (int j = 0; j < PF; ++j) load(pg[j], min(j, nb - 1));
    __builtin_amdgcn_sched_barrier(0);  // every page request goes out before the math
    for (int j0 = 0; j0 < npad - PF; j0 += PF) {
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        process(pg[j], __builtin_amdgcn_readlane(c_ntok, j0 + j));
        load(pg[j], min(j0 + j + PF, nb - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int j = 0; j < PF; ++j)
      if (npad - PF + j < nb) process(pg[j], __builtin_amdgcn_readlane(c_ntok, npad - PF + j));
  }

  // ---- merge the wavefronts: a fixed-order tree in LDS (deterministic) ----
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float Lw = lrun[rt];
    Lw = add_xor32(add_xor16(Lw));
    if (grp == 0) {
      sm_m[wv][rt * 16 + col] = mrun[rt];
      sm_l[wv][rt * 16 + col] = Lw;
    }
  }
  __syncthreads();
  // workgroup row statistics for this lane's rows: M = max_w m_w,
  // L = sum_w l_w 2^(m_w - M); every wavefront rescales to M
  float Lwg[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + col;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w][row]);
    float Lr = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) Lr += (sm_m[w][row] == -INFINITY) ? 0.f : sm_l[w][row] * exp2f(sm_m[w][row] - M);
    Lwg[rt] = Lr;
    if (W > 1) {
      const float f = (mrun[rt] == -INFINITY) ? 0.f : exp2f(mrun[rt] - M);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[rt][ct] *= f;
    }
    mrun[rt] = M;
  }
#pragma unroll
  for (int half = W / 2; half >= 1; half >>= 1) {
    if (wv >= half && wv < 2 * half) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          sm_slice[wv - half][rt][ct][lane] = make_float4(acc[rt][ct][0], acc[rt][ct][1], acc[rt][ct][2], acc[rt][ct][3]);
    }
    __syncthreads();
    if (wv < half) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const float4 o = sm_slice[wv][rt][ct][lane];
          acc[rt][ct] += f32x4_t{o.x, o.y, o.z, o.w};
        }
    }
    if (half > 1) __syncthreads();
  }
  // wavefront 0 now holds the workgroup's accumulator

  if (arrive != nullptr && splits > 1) {
    merge_in_launch<D, RT, W>(acc, mrun, Lwg, ws_acc, ws_ml, out, rows, splits, unit, wid, arrive, lds);
    return;
  }
  if (wv != 0) return;
  if (splits == 1) {
    float* ou = out + static_cast<size_t>(unit) * rows * D;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = rt * 16 + col;
      if (row < rows) {
        const float inv = (Lwg[rt] > 0.f) ? 1.f / Lwg[rt] : 0.f;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          *reinterpret_cast<float4*>(ou + static_cast<size_t>(row) * D + 16 * ct + 4 * grp) =
              make_float4(acc[rt][ct][0] * inv, acc[rt][ct][1] * inv, acc[rt][ct][2] * inv, acc[rt][ct][3] * inv);
      }
    }
    return;
  }
  float* wa = ws_acc + static_cast<size_t>(wid) * rows * D;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + col;
    if (row < rows) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        *reinterpret_cast<float4*>(wa + static_cast<size_t>(row) * D + 16 * ct + 4 * grp) =
            make_float4(acc[rt][ct][0], acc[rt][ct][1], acc[rt][ct][2], acc[rt][ct][3]);
      if (grp == 0)
        *reinterpret_cast<float2*>(ws_ml + (static_cast<size_t>(wid) * rows + row) * 2) = make_float2(mrun[rt], Lwg[rt]);
    }
  }
}

}  // namespace oasis
