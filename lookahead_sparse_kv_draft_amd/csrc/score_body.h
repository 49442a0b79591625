// One wavefront of the lookahead scoring (the Quest upper bound of every block
// for the draft queries, OasisKV explainer Figure 7 right): shared by the score
// kernel and by the launch that carries the attention's split combine beside it.
// The contraction and its layout are described in score.hip.
#pragma once

#include "oasis_internal.h"

namespace oasis {

// Per-16-bit-lane mask of the negative halves of a packed bf16 pair.
__device__ __forceinline__ uint32_t neg_mask(uint32_t w) {
  return ((w >> 15) & 0x00010001u) * 0xFFFFu;
}

// Wavefronts per (request, KV head): runs of score_tpw 16-block tiles.
inline int score_waves_per_unit(const Ctx& c) {
  const int tiles = (c.s.max_blocks + 15) / 16;
  return (tiles + c.score_tpw - 1) / c.score_tpw;
}

template <int D, int RT>
__device__ inline void score_wave(const uint16_t* __restrict__ q, const uint16_t* __restrict__ meta,
                                  const int32_t* __restrict__ ctx_len, float* __restrict__ scores, int H, int G,
                                  int T, int ndraft, int qt0, int rows, int Nmax, int waves_per_unit, int tpw,
                                  int total_waves, int wave, int lane) {
  constexpr int KSTEPS = D / 16;  // 32-element k-steps over the 2d metadata elements
  constexpr int HALF = KSTEPS / 2;  // steps on the kmin half
  if (wave >= total_waves) return;
  const int unit = wave / waves_per_unit;
  const int chunk = wave - unit * waves_per_unit;
  const int t0 = chunk * tpw;  // this wavefront's first tile (< ceil(Nmax / 16) by the grid)
  const int t1max = min(t0 + tpw, (Nmax + 15) / 16);
  const int col = lane & 15;  // A: query row within the row tile; B/C: block within the tile
  const int grp = lane >> 4;  // k-group of the lane
  // chunk-major metadata tiles (meta_offset): 4d 16-byte chunks per tile, the
  // chunk lane (col, grp) needs at k-step s (chunk 4s + grp of block col) is
  // at 64s + lane, so each k-step is one contiguous 1 KiB load
  constexpr int TILE4 = 4 * D;
  const uint4* mbase = reinterpret_cast<const uint4*>(meta) + static_cast<size_t>(unit) * meta_tiles(Nmax) * TILE4;
  float* sbase = scores + static_cast<size_t>(unit) * Nmax;
  // Loads are unconditional (tile indices clamped; results of blocks past the
  // context are discarded), so every wait below covers exactly the older buffer.
  auto load_c = [&](uint4* Bt, int tile, int nclamp) {
    const int t = min(tile, (nclamp + 15) / 16 - 1);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) Bt[s] = load_stream(mbase + static_cast<size_t>(t) * TILE4 + 64 * s + lane);
  };
  // The first two tiles go out before the context length arrives: every block
  // index below Nmax is in bounds, and the context only decides what is kept.
  uint4 Ba[KSTEPS], Bb[KSTEPS];
  load_c(Ba, t0, Nmax);
  load_c(Bb, min(t0 + 1, t1max - 1), Nmax);
  const int n = ctx_len[unit / H];
  const int N = min((n + kBlock - 1) / kBlock, Nmax);  // context capacity bounds every index
  const int ntiles = (N + 15) / 16;
  if (t0 >= ntiles) return;
  const int t1 = min(t0 + tpw, ntiles);

  // A operands.  Lane (col, grp) at k-step s covers metadata chunk 4s + grp (8
  // elements): kmin channels for s < HALF (paired with q-), kmax channels after
  // (paired with q+).  Both use query channels 8 * (4 * (s mod HALF) + grp) .. +7.
  uint4 A[RT][KSTEPS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + col;
    if (row < rows) {
      const int g = row / ndraft;
      const int t = qt0 + (row - g * ndraft);  // query rows qt0 .. qt0 + ndraft - 1 of each group member
      const uint16_t* qr = q + ((static_cast<size_t>(unit) * G + g) * T + t) * D;
#pragma unroll
      for (int s = 0; s < HALF; ++s) {
        const uint4 raw = *reinterpret_cast<const uint4*>(qr + 8 * (4 * s + grp));
        const uint4 m = make_uint4(neg_mask(raw.x), neg_mask(raw.y), neg_mask(raw.z),
                                   neg_mask(raw.w));
        A[rt][s] = make_uint4(raw.x & m.x, raw.y & m.y, raw.z & m.z, raw.w & m.w);
        A[rt][HALF + s] = make_uint4(raw.x & ~m.x, raw.y & ~m.y, raw.z & ~m.z, raw.w & ~m.w);
      }
    } else {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) A[rt][s] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  auto load = [&](uint4* Bt, int tile) { load_c(Bt, tile, N); };
  auto compute = [&](const uint4* Bt, int tile) {
    float best = -INFINITY;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(A[rt][s]), as_bf16x8(Bt[s]), acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rt * 16 + 4 * grp + i;
        if (row < rows) best = fmaxf(best, acc[i]);
      }
    }
    best = max_xor32(max_xor16(best));
    const int b = tile * 16 + col;
    if (grp == 0 && b < N) sbase[b] = best;
  };
  // Ping-pong over the two tile buffers: each processed buffer is refilled with
  // the tile two ahead, the last one or two tiles without refills.  Indices are
  // clamped and the loop body has no branch (a repeated last tile stores
  // identical scores), so every wait covers exactly the older buffer.
  const int ntl = t1 - t0;
  int j = 0;
  for (; j + 2 < ntl; j += 2) {
    compute(Ba, t0 + j);
    load(Ba, t0 + j + 2);
    __builtin_amdgcn_sched_barrier(0);  // keep the refill ahead of the next math
    compute(Bb, t0 + j + 1);
    load(Bb, t0 + min(j + 3, ntl - 1));
    __builtin_amdgcn_sched_barrier(0);
  }
  // the last one or two tiles, no refills.  Bb holds tile t0 + j + 1 only when
  // that tile is in the run: with a single tile (ntl == 1) it was preloaded
  // from the capacity, past the context, and must not be stored.
  compute(Ba, t0 + j);
  if (j + 1 < ntl) compute(Bb, t0 + j + 1);
}

}  // namespace oasis
