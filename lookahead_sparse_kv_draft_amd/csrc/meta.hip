// Block metadata kernels: per-block, per-channel key min/max ("compressed keys",
// OasisKV explainer, Figure 7 left: per-block min/max pooling kept on the GPU).
//
//  meta_build  - one wavefront per staged page: min/max over the block's tokens
//                below the context length; optionally patches the resident copy.
//  meta_rows   - one wavefront per block of a token range, from key rows.
//  meta_update - one wavefront per (request, KV head): absorbs the appended
//                token into its block's min/max and writes it into the page if
//                the block is resident.
//  admit       - one wavefront per block of a prefill on the device: page into
//                the pinned host tier (and its pool slot if resident) plus the
//                metadata row.
#include "append_body.h"

namespace oasis {
namespace {

template <typename E, int D>
__global__ __launch_bounds__(256) void meta_build_kernel(
    const E* __restrict__ pages, const int32_t* __restrict__ ids, int count,
    const int32_t* __restrict__ ctx_len, E* __restrict__ meta, E* __restrict__ pool,
    const int32_t* __restrict__ b2s, int units, int H, int Nmax, int kb) {
  constexpr int PAGE = 2 * kBlock * D;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (w >= count) return;
  const int id = ids ? ids[w] : w;
  if (id < 0 || id >= units * Nmax) return;
  const int unit = id / Nmax;
  const int b = id - unit * Nmax;
  const int n = ctx_len[unit / H];
  const int N = min((n + kBlock - 1) / kBlock, Nmax);
  if (b >= N) return;
  const int ntok = min(kBlock, n - kBlock * b);
  const E* pg = pages + static_cast<size_t>(w) * PAGE;
  constexpr int CE = 16 / static_cast<int>(sizeof(E));
  for (int c = lane; c < D; c += kWave) {
    float mn = Elem<E>::load(pg[c]);
    float mx = mn;
    for (int j = 1; j < ntok; ++j) {
      const float v = Elem<E>::load(pg[j * D + c]);
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
    meta[meta_offset<D, CE>(unit, b, c, Nmax)] = Elem<E>::store(mn);
    meta[meta_offset<D, CE>(unit, b, D + c, Nmax)] = Elem<E>::store(mx);
  }
  if (pool != nullptr && b2s != nullptr) {
    const int slot = b2s[id];
    if (slot >= 0 && slot < kb) {
      const uint4* src = reinterpret_cast<const uint4*>(pg);
      uint4* dst = reinterpret_cast<uint4*>(pool + (static_cast<size_t>(unit) * kb + slot) * PAGE);
      constexpr int V4 = PAGE * static_cast<int>(sizeof(E)) / 16;
      for (int i = lane; i < V4; i += kWave) dst[i] = src[i];
    }
  }
}

// The metadata of blocks [b0, b1) of every unit from key rows [units][Nmax*16][d]
// (token-major): one wavefront per (unit, block), min/max over the block's
// tokens below the context length; blocks at or past it are not touched.
template <typename E, int D>
__global__ __launch_bounds__(256) void meta_rows_kernel(const E* __restrict__ k_rows,
                                                        const int32_t* __restrict__ ctx_len, E* __restrict__ meta,
                                                        int units, int H, int Nmax, int b0, int b1) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int nb = b1 - b0;
  if (w >= units * nb) return;
  const int unit = w / nb;
  const int b = b0 + (w - unit * nb);
  const int n = ctx_len[unit / H];
  const int N = min((n + kBlock - 1) / kBlock, Nmax);
  if (b >= N) return;
  const int ntok = min(kBlock, n - kBlock * b);
  const E* kr = k_rows + (static_cast<size_t>(unit) * Nmax * kBlock + static_cast<size_t>(b) * kBlock) * D;
  constexpr int CE = 16 / static_cast<int>(sizeof(E));
  for (int c = lane; c < D; c += kWave) {
    float mn = Elem<E>::load(kr[c]);
    float mx = mn;
    for (int j = 1; j < ntok; ++j) {
      const float v = Elem<E>::load(kr[j * D + c]);
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
    meta[meta_offset<D, CE>(unit, b, c, Nmax)] = Elem<E>::store(mn);
    meta[meta_offset<D, CE>(unit, b, D + c, Nmax)] = Elem<E>::store(mx);
  }
}

template <typename E, int D>
hipError_t rows_t(const Ctx& c, const void* k_rows, const int32_t* ctx_len, void* meta, int b0, int b1,
                  hipStream_t st) {
  const long long waves = static_cast<long long>(c.units) * (b1 - b0);
  if (waves <= 0) return hipSuccess;
  hipLaunchKernelGGL((meta_rows_kernel<E, D>), dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), 0, st,
                     static_cast<const E*>(k_rows), ctx_len, static_cast<E*>(meta), c.units, c.s.kv_heads,
                     c.s.max_blocks, b0, b1);
  return hipGetLastError();
}

// The metadata between the library's chunk-major tiles and the logical layout
// [units][Nmax][2][d] (the key min row, then the key max row, per block): one
// thread per 16-byte chunk of a block row; tile padding is neither read nor written.
template <int NC>
__global__ __launch_bounds__(256) void meta_relayout_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                            long long total, int Nmax, int to_logical) {
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const long long per_unit = static_cast<long long>(Nmax) * NC;
  const long long unit = i / per_unit;
  const int rem = static_cast<int>(i - unit * per_unit);
  const int b = rem / NC, c = rem - (rem / NC) * NC;
  const long long tiled = ((unit * meta_tiles(Nmax) + b / kMetaTile) * NC + c) * kMetaTile + (b % kMetaTile);
  if (to_logical)
    dst[i] = src[tiled];
  else
    dst[tiled] = src[i];
}

template <typename E, int D>
__global__ __launch_bounds__(64) void meta_update_kernel(
    const E* __restrict__ k_new, const E* __restrict__ v_new, const int32_t* __restrict__ ctx_in,
    int32_t* __restrict__ ctx_out, E* __restrict__ meta, E* __restrict__ pool,
    const int32_t* __restrict__ b2s, int H, int Nmax, int kb) {
  append_token<E, D>(k_new, v_new, ctx_in, ctx_out, meta, pool, b2s, blockIdx.x, H, Nmax, kb, threadIdx.x, kWave);
}

// Admission of a prefill: one wavefront per (unit, block) below the context.
// Reads the block's 16 key and value rows from the device, writes the page (K
// token-major, V channel-major) into the host tier (pinned, device-mapped: the
// stores go over PCIe) and, if the block is resident, into its pool slot, and
// the block's metadata row.
template <typename E, int D>
__global__ __launch_bounds__(256) void admit_kernel(
    const E* __restrict__ k_rows, const E* __restrict__ v_rows, const int32_t* __restrict__ ctx_len,
    E* __restrict__ host, E* __restrict__ meta, E* __restrict__ pool, const int32_t* __restrict__ b2s, int units,
    int H, int Nmax, int kb) {
  constexpr int PAGE = 2 * kBlock * D;
  constexpr int CE = 16 / static_cast<int>(sizeof(E));
  constexpr int KCH = kBlock * D / CE;  // 16-byte chunks of the K half
  const int lane = threadIdx.x & (kWave - 1);
  const long long w = static_cast<long long>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (w >= static_cast<long long>(units) * Nmax) return;
  const int unit = static_cast<int>(w / Nmax);
  const int b = static_cast<int>(w - static_cast<long long>(unit) * Nmax);
  const int n = ctx_len[unit / H];
  const int N = min((n + kBlock - 1) / kBlock, Nmax);
  if (b >= N) return;
  const int ntok = min(kBlock, n - kBlock * b);
  const size_t row0 = (static_cast<size_t>(unit) * Nmax + b) * kBlock;
  const E* kr = k_rows + row0 * D;
  const E* vr = v_rows + row0 * D;
  const int slot = (pool != nullptr && b2s != nullptr) ? b2s[static_cast<size_t>(unit) * Nmax + b] : -1;
  E* hp = host + (static_cast<size_t>(unit) * Nmax + b) * PAGE;
  E* pp = (slot >= 0 && slot < kb) ? pool + (static_cast<size_t>(unit) * kb + slot) * PAGE : nullptr;
  // K half: the rows as they are
  for (int i = lane; i < KCH; i += kWave) {
    const uint4 x = reinterpret_cast<const uint4*>(kr)[i];
    reinterpret_cast<uint4*>(hp)[i] = x;
    if (pp != nullptr) reinterpret_cast<uint4*>(pp)[i] = x;
  }
  // V half transposed, and the metadata row
  for (int c = lane; c < D; c += kWave) {
    E vt[kBlock];
#pragma unroll
    for (int t = 0; t < kBlock; ++t) vt[t] = vr[static_cast<size_t>(t) * D + c];
#pragma unroll
    for (int t = 0; t < kBlock; ++t) {
      hp[kBlock * D + c * kBlock + t] = vt[t];
      if (pp != nullptr) pp[kBlock * D + c * kBlock + t] = vt[t];
    }
    float mn = Elem<E>::load(kr[c]);
    float mx = mn;
    for (int t = 1; t < ntok; ++t) {
      const float x = Elem<E>::load(kr[static_cast<size_t>(t) * D + c]);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    meta[meta_offset<D, CE>(unit, b, c, Nmax)] = Elem<E>::store(mn);
    meta[meta_offset<D, CE>(unit, b, D + c, Nmax)] = Elem<E>::store(mx);
  }
}

template <typename E, int D>
hipError_t admit_t(const Ctx& c, const void* k_rows, const void* v_rows, const int32_t* ctx_len, void* host_dev,
                   void* meta, void* pool, const int32_t* b2s, hipStream_t st) {
  const long long waves = static_cast<long long>(c.units) * c.s.max_blocks;
  const int grid = static_cast<int>((waves + 3) / 4);
  hipLaunchKernelGGL((admit_kernel<E, D>), dim3(grid), dim3(256), 0, st, static_cast<const E*>(k_rows),
                     static_cast<const E*>(v_rows), ctx_len, static_cast<E*>(host_dev), static_cast<E*>(meta),
                     static_cast<E*>(pool), b2s, c.units, c.s.kv_heads, c.s.max_blocks, c.s.budget_blocks);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t build_t(const Ctx& c, const void* pages, const int32_t* ids, int32_t count,
                   const int32_t* ctx_len, void* meta, void* pool, const int32_t* b2s,
                   hipStream_t st) {
  const int waves_per_wg = 4;
  const int grid = (count + waves_per_wg - 1) / waves_per_wg;
  hipLaunchKernelGGL((meta_build_kernel<E, D>), dim3(grid), dim3(waves_per_wg * kWave), 0, st,
                     static_cast<const E*>(pages), ids, count, ctx_len, static_cast<E*>(meta),
                     static_cast<E*>(pool), b2s, c.units, c.s.kv_heads, c.s.max_blocks,
                     c.s.budget_blocks);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t update_t(const Ctx& c, const void* k_new, const void* v_new, const int32_t* ctx_in,
                    int32_t* ctx_out, void* meta, void* pool, const int32_t* b2s, hipStream_t st) {
  hipLaunchKernelGGL((meta_update_kernel<E, D>), dim3(c.units), dim3(kWave), 0, st,
                     static_cast<const E*>(k_new), static_cast<const E*>(v_new), ctx_in, ctx_out,
                     static_cast<E*>(meta), static_cast<E*>(pool), b2s, c.s.kv_heads,
                     c.s.max_blocks, c.s.budget_blocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_meta_build(const Ctx& c, const void* pages, const int32_t* ids, int32_t count,
                             const int32_t* ctx_len, void* meta, void* pool, const int32_t* b2s,
                             hipStream_t st) {
  if (count <= 0) return hipSuccess;
  const bool bf = c.s.dtype == OASIS_BF16;
  if (c.s.head_dim == 128)
    return bf ? build_t<uint16_t, 128>(c, pages, ids, count, ctx_len, meta, pool, b2s, st)
              : build_t<float, 128>(c, pages, ids, count, ctx_len, meta, pool, b2s, st);
  return bf ? build_t<uint16_t, 64>(c, pages, ids, count, ctx_len, meta, pool, b2s, st)
            : build_t<float, 64>(c, pages, ids, count, ctx_len, meta, pool, b2s, st);
}

hipError_t launch_meta_rows(const Ctx& c, const void* k_rows, int tok_begin, int tok_end, const int32_t* ctx_len,
                            void* meta, hipStream_t st) {
  const int b0 = tok_begin / kBlock, b1 = (tok_end + kBlock - 1) / kBlock;
  const bool bf = c.s.dtype == OASIS_BF16;
  if (c.s.head_dim == 128)
    return bf ? rows_t<uint16_t, 128>(c, k_rows, ctx_len, meta, b0, b1, st)
              : rows_t<float, 128>(c, k_rows, ctx_len, meta, b0, b1, st);
  return bf ? rows_t<uint16_t, 64>(c, k_rows, ctx_len, meta, b0, b1, st)
            : rows_t<float, 64>(c, k_rows, ctx_len, meta, b0, b1, st);
}

hipError_t launch_admit(const Ctx& c, const void* k_rows, const void* v_rows, const int32_t* ctx_len,
                        void* host_dev, void* meta, void* pool, const int32_t* b2s, hipStream_t st) {
  const bool bf = c.s.dtype == OASIS_BF16;
  if (c.s.head_dim == 128)
    return bf ? admit_t<uint16_t, 128>(c, k_rows, v_rows, ctx_len, host_dev, meta, pool, b2s, st)
              : admit_t<float, 128>(c, k_rows, v_rows, ctx_len, host_dev, meta, pool, b2s, st);
  return bf ? admit_t<uint16_t, 64>(c, k_rows, v_rows, ctx_len, host_dev, meta, pool, b2s, st)
            : admit_t<float, 64>(c, k_rows, v_rows, ctx_len, host_dev, meta, pool, b2s, st);
}

hipError_t launch_meta_update(const Ctx& c, const void* k_new, const void* v_new,
                              const int32_t* ctx_in, int32_t* ctx_out, void* meta, void* pool,
                              const int32_t* b2s, hipStream_t st) {
  const bool bf = c.s.dtype == OASIS_BF16;
  if (c.s.head_dim == 128)
    return bf ? update_t<uint16_t, 128>(c, k_new, v_new, ctx_in, ctx_out, meta, pool, b2s, st)
              : update_t<float, 128>(c, k_new, v_new, ctx_in, ctx_out, meta, pool, b2s, st);
  return bf ? update_t<uint16_t, 64>(c, k_new, v_new, ctx_in, ctx_out, meta, pool, b2s, st)
            : update_t<float, 64>(c, k_new, v_new, ctx_in, ctx_out, meta, pool, b2s, st);
}

hipError_t launch_meta_relayout(const Ctx& c, const void* src, void* dst, bool to_logical, hipStream_t st) {
  const int nc = 2 * c.s.head_dim * c.elem_bytes / 16;  // 16-byte chunks per block row
  const long long total = static_cast<long long>(c.units) * c.s.max_blocks * nc;
  if (total == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((total + 255) / 256)), block(256);
  const uint4* s4 = static_cast<const uint4*>(src);
  uint4* d4 = static_cast<uint4*>(dst);
  switch (nc) {
    case 16: hipLaunchKernelGGL((meta_relayout_kernel<16>), grid, block, 0, st, s4, d4, total, c.s.max_blocks, to_logical); break;
    case 32: hipLaunchKernelGGL((meta_relayout_kernel<32>), grid, block, 0, st, s4, d4, total, c.s.max_blocks, to_logical); break;
    case 64: hipLaunchKernelGGL((meta_relayout_kernel<64>), grid, block, 0, st, s4, d4, total, c.s.max_blocks, to_logical); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace oasis
