// Lookahead scoring of every KV block from the draft queries (OasisKV explainer,
// Figure 7 right: the draft queries scan the compressed keys to predict the next
// step's top-K blocks).  The score of block b is the Quest upper bound
//     max over draft rows q of  sum_c max(q_c * kmin_c, q_c * kmax_c),
// which equals q+ . kmax + q- . kmin with q+ = max(q, 0), q- = min(q, 0).
//
// bf16 path: the bound is a dense contraction of the [rows x 2d] matrix
// [q- | q+] with the [2d x blocks] metadata, so it runs on the bf16 MFMA
// (v_mfma_f32_16x16x32_bf16): q+ and q- are exact in bf16, every product is exact
// in fp32 and the sum accumulates in fp32.  One wavefront streams 16-block tiles
// of one (request, KV head): B operand = 16 blocks x 32 metadata elements, each
// lane loading 16 contiguous bytes (a tile is 8 KiB contiguous), A operand = the
// split query rows held in registers for the whole wavefront.  The next tile's
// loads are issued before the current tile's MFMAs.  Rows are reduced with a max
// inside each lane and two cross-lane exchanges.
//
// f32 path: one thread per block, query rows staged in LDS, plain fp32 VALU.
#include "oasis_internal.h"

namespace oasis {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// Per-16-bit-lane mask of the negative halves of a packed bf16 pair.
__device__ __forceinline__ uint32_t neg_mask(uint32_t w) {
  return ((w >> 15) & 0x00010001u) * 0xFFFFu;
}

template <int D, int RT>
__global__ __launch_bounds__(256) void score_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ meta,
    const int32_t* __restrict__ ctx_len, float* __restrict__ scores, int H, int G, int T,
    int ndraft, int rows, int Nmax, int waves_per_unit, int tpw, int total_waves) {
  constexpr int KSTEPS = D / 16;  // 32-element k-steps over the 2d metadata elements
  constexpr int HALF = KSTEPS / 2;  // steps on the kmin half
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (wave >= total_waves) return;
  const int unit = wave / waves_per_unit;
  const int chunk = wave - unit * waves_per_unit;
  const int n = ctx_len[unit / H];
  const int N = min((n + kBlock - 1) / kBlock, Nmax);  // context capacity bounds every index
  const int ntiles = (N + 15) / 16;
  const int t0 = chunk * tpw;
  if (t0 >= ntiles) return;
  const int t1 = min(t0 + tpw, ntiles);
  const int col = lane & 15;  // A: query row within the row tile; B/C: block within the tile
  const int grp = lane >> 4;  // k-group of the lane

  // A operands.  Lane (col, grp) at k-step s covers metadata chunk 4s + grp (8
  // elements): kmin channels for s < HALF (paired with q-), kmax channels after
  // (paired with q+).  Both use query channels 8 * (4 * (s mod HALF) + grp) .. +7.
  uint4 A[RT][KSTEPS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + col;
    if (row < rows) {
      const int g = row / ndraft;
      const int t = 1 + (row - g * ndraft);
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

  const uint4* mbase = reinterpret_cast<const uint4*>(meta + static_cast<size_t>(unit) * Nmax * 2 * D);
  float* sbase = scores + static_cast<size_t>(unit) * Nmax;
  constexpr int CHUNKS = 2 * D / 8;  // 16-byte chunks per block row pair

  // Loads are unconditional (the block index is clamped to N-1; results of
  // blocks >= N are discarded), so the waits below only cover the older buffer.
  auto load = [&](uint4* Bt, int tile) {
    const int b = min(tile * 16 + col, N - 1);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) Bt[s] = mbase[static_cast<size_t>(b) * CHUNKS + 4 * s + grp];
  };
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
    best = fmaxf(best, __shfl_xor(best, 16));
    best = fmaxf(best, __shfl_xor(best, 32));
    const int b = tile * 16 + col;
    if (grp == 0 && b < N) sbase[b] = best;
  };
  // Ping-pong over two tile buffers.  The prefetch index is clamped and the
  // loop body has no branch (an odd count repeats the last tile, whose store is
  // identical), so every wait covers only the older buffer.
  const int ntl = t1 - t0;
  uint4 Ba[KSTEPS], Bb[KSTEPS];
  load(Ba, t0);
  for (int j = 0; j < ntl; j += 2) {
    load(Bb, t0 + min(j + 1, ntl - 1));
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the math
    compute(Ba, t0 + j);
    load(Ba, t0 + min(j + 2, ntl - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(Bb, t0 + min(j + 1, ntl - 1));
  }
}

template <int D>
__global__ __launch_bounds__(256) void score_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ meta, const int32_t* __restrict__ ctx_len,
    float* __restrict__ scores, int H, int G, int T, int ndraft, int rows, int Nmax) {
  extern __shared__ float qs[];  // [rows][D]
  const int unit = blockIdx.y;
  const int n = ctx_len[unit / H];
  const int N = min((n + kBlock - 1) / kBlock, Nmax);
  if (static_cast<int>(blockIdx.x) * 256 >= N) return;
  for (int i = threadIdx.x; i < rows * D; i += blockDim.x) {
    const int row = i / D, c = i - (i / D) * D;
    const int g = row / ndraft, t = 1 + (row - g * ndraft);
    qs[i] = q[((static_cast<size_t>(unit) * G + g) * T + t) * D + c];
  }
  __syncthreads();
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= N) return;
  const float* mr = meta + (static_cast<size_t>(unit) * Nmax + b) * 2 * D;
  float best = -INFINITY;
  for (int row = 0; row < rows; ++row) {
    float s = 0.f;
    for (int c = 0; c < D; ++c) {
      const float qc = qs[row * D + c];
      s += fmaxf(qc * mr[c], qc * mr[D + c]);
    }
    best = fmaxf(best, s);
  }
  scores[static_cast<size_t>(unit) * Nmax + b] = best;
}

template <int D, int RT>
hipError_t mfma_t(const Ctx& c, const void* q, const void* meta, const int32_t* ctx_len,
                  float* scores, hipStream_t st) {
  const int tiles = (c.s.max_blocks + 15) / 16;
  const int wpu = (tiles + c.score_tpw - 1) / c.score_tpw;
  const int total = c.units * wpu;
  const int grid = (total + 3) / 4;
  hipLaunchKernelGGL((score_mfma_kernel<D, RT>), dim3(grid), dim3(256), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(meta), ctx_len,
                     scores, c.s.kv_heads, c.s.group, c.T, c.s.n_draft, c.rows_score,
                     c.s.max_blocks, wpu, c.score_tpw, total);
  return hipGetLastError();
}

template <int D>
hipError_t f32_t(const Ctx& c, const void* q, const void* meta, const int32_t* ctx_len,
                 float* scores, hipStream_t st) {
  dim3 grid((c.s.max_blocks + 255) / 256, c.units);
  const size_t lds = static_cast<size_t>(c.rows_score) * D * sizeof(float);
  hipLaunchKernelGGL((score_f32_kernel<D>), grid, dim3(256), lds, st,
                     static_cast<const float*>(q), static_cast<const float*>(meta), ctx_len, scores,
                     c.s.kv_heads, c.s.group, c.T, c.s.n_draft, c.rows_score, c.s.max_blocks);
  return hipGetLastError();
}

template <int D>
hipError_t mfma_rows(const Ctx& c, const void* q, const void* meta, const int32_t* ctx_len,
                     float* scores, hipStream_t st) {
  switch ((c.rows_score + 15) / 16) {
    case 1: return mfma_t<D, 1>(c, q, meta, ctx_len, scores, st);
    case 2: return mfma_t<D, 2>(c, q, meta, ctx_len, scores, st);
    case 3: return mfma_t<D, 3>(c, q, meta, ctx_len, scores, st);
    default: return mfma_t<D, 4>(c, q, meta, ctx_len, scores, st);
  }
}

}  // namespace

hipError_t launch_score(const Ctx& c, const void* q, const void* meta, const int32_t* ctx_len,
                        float* scores, hipStream_t st) {
  if (c.s.dtype == OASIS_BF16)
    return c.s.head_dim == 128 ? mfma_rows<128>(c, q, meta, ctx_len, scores, st)
                               : mfma_rows<64>(c, q, meta, ctx_len, scores, st);
  return c.s.head_dim == 128 ? f32_t<128>(c, q, meta, ctx_len, scores, st)
                             : f32_t<64>(c, q, meta, ctx_len, scores, st);
}

}  // namespace oasis
