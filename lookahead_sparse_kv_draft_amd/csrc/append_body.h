// Appending one token of one (request, KV head) in long-output decode (OasisKV
// explainer, Figure 7 left: the per-block key min/max the scoring reads stays
// on the GPU; the context grows one token per step).  Shared by the append
// kernel and by the workgroups a decode step's attention launch (metadata) and
// scoring launch (page) carry.
#pragma once

#include "oasis_internal.h"

namespace oasis {

template <typename E> struct Elem;
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(uint16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ uint16_t store(float f) { return f32_to_bf16(f); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(float v) { return v; }
  static __device__ __forceinline__ float store(float f) { return f; }
};

// The token of unit `unit` goes to position p = ctx_in[request], block p / 16:
// its metadata row is set to the token's key (p % 16 == 0) or absorbs it by
// min / max, and ctx_out[request] = p + 1 (written by the request's first KV
// head).  A position outside [0, 16 * Nmax) writes no metadata and leaves the
// context as it was (ctx_out[request] = p), so what reads ctx_out next sees a
// defined length.  Run by nthreads threads (tid = 0 .. nthreads - 1), each
// taking channels tid, tid + nthreads, ...
template <typename E, int D>
__device__ __forceinline__ void append_meta(const E* __restrict__ k_new, const int32_t* __restrict__ ctx_in,
                                            int32_t* __restrict__ ctx_out, E* __restrict__ meta, int unit, int H,
                                            int Nmax, int tid, int nthreads) {
  const int r = unit / H;
  const int h = unit - r * H;
  const int p = ctx_in[r];
  const int b = p / kBlock;
  const int j = p - b * kBlock;
  if (p < 0 || b >= Nmax) {
    if (h == 0 && tid == 0) ctx_out[r] = p;
    return;
  }
  constexpr int CE = 16 / static_cast<int>(sizeof(E));
  const E* kn = k_new + static_cast<size_t>(unit) * D;
  for (int c = tid; c < D; c += nthreads) {
    const E kv = kn[c];
    E* mn = meta + meta_offset<D, CE>(unit, b, c, Nmax);
    E* mx = meta + meta_offset<D, CE>(unit, b, D + c, Nmax);
    if (j == 0) {
      *mn = kv;
      *mx = kv;
    } else {
      const float kf = Elem<E>::load(kv);
      *mn = Elem<E>::store(fminf(Elem<E>::load(*mn), kf));
      *mx = Elem<E>::store(fmaxf(Elem<E>::load(*mx), kf));
    }
  }
  if (h == 0 && tid == 0) ctx_out[r] = p + 1;
}

// The same token's K row and V column into the page of block p / 16 if the
// block holds a slot (b2s); nothing else (nothing at all for a position outside
// the capacity).  Threads as append_meta.
template <typename E, int D>
__device__ __forceinline__ void append_page(const E* __restrict__ k_new, const E* __restrict__ v_new,
                                            const int32_t* __restrict__ ctx_in, E* __restrict__ pool,
                                            const int32_t* __restrict__ b2s, int unit, int H, int Nmax, int kb,
                                            int tid, int nthreads) {
  constexpr int PAGE = 2 * kBlock * D;
  const int p = ctx_in[unit / H];
  const int b = p / kBlock;
  const int j = p - b * kBlock;
  if (p < 0 || b >= Nmax) return;
  const int slot = b2s[static_cast<size_t>(unit) * Nmax + b];
  if (slot < 0 || slot >= kb) return;
  const E* kn = k_new + static_cast<size_t>(unit) * D;
  const E* vn = v_new + static_cast<size_t>(unit) * D;
  E* pg = pool + (static_cast<size_t>(unit) * kb + slot) * PAGE;
  for (int c = tid; c < D; c += nthreads) {
    pg[j * D + c] = kn[c];                    // K row j (token-major)
    pg[kBlock * D + c * kBlock + j] = vn[c];  // V^T column j (channel-major)
  }
}

// Both halves, in one workgroup.
template <typename E, int D>
__device__ __forceinline__ void append_token(const E* __restrict__ k_new, const E* __restrict__ v_new,
                                             const int32_t* __restrict__ ctx_in, int32_t* __restrict__ ctx_out,
                                             E* __restrict__ meta, E* __restrict__ pool,
                                             const int32_t* __restrict__ b2s, int unit, int H, int Nmax, int kb,
                                             int tid, int nthreads) {
  append_meta<E, D>(k_new, ctx_in, ctx_out, meta, unit, H, Nmax, tid, nthreads);
  append_page<E, D>(k_new, v_new, ctx_in, pool, b2s, unit, H, Nmax, kb, tid, nthreads);
}

}  // namespace oasis
