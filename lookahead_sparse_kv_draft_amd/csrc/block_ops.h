// Workgroup-wide primitives for 256-thread (4-wavefront) workgroups.
#pragma once

#include "oasis_internal.h"

namespace oasis {

constexpr int kWG = 256;
constexpr int kWavesPerWG = kWG / kWave;

// Exclusive rank of `flag` among the workgroup's threads in thread order, and the
// total count.  wave_tot: kWavesPerWG ints of LDS.  Contains two barriers.
__device__ __forceinline__ int wg_rank_of_flag(bool flag, int* total, int* wave_tot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const uint64_t bal = __ballot(flag);
  const int within = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) wave_tot[w] = __popcll(bal);
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWavesPerWG; ++i) {
    const int cnt = wave_tot[i];
    off += (i < w) ? cnt : 0;
    tot += cnt;
  }
  __syncthreads();
  *total = tot;
  return off + within;
}

// Inclusive prefix sum of one int per thread over the workgroup.  Two barriers.
__device__ __forceinline__ int wg_inclusive_sum(int v, int* wave_tot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  v = wave_incl_sum(v);
  if (lane == kWave - 1) wave_tot[w] = v;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int i = 0; i < kWavesPerWG; ++i) off += (i < w) ? wave_tot[i] : 0;
  __syncthreads();
  return v + off;
}

// Ascending bitonic sort of P (a power of two) 64-bit keys in LDS.  Callers
// synchronise before; ends with a barrier.
__device__ __forceinline__ void wg_bitonic_sort(unsigned long long* a, int P) {
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (P >> 1); i += blockDim.x) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool asc = (lo & size) == 0;
        const unsigned long long x = a[lo], y = a[hi];
        if ((x > y) == asc) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace oasis
