// Fetch gather (OasisKV explainer, Figure 8 and "What they did" item 2: the
// missing predicted blocks move from the host tier into their HBM slots before
// the layer's attention at the next step; Figure 9: the head-wise table gives
// each fetched block its GPU slot).  The device reads the fetch list the diff
// left in HBM and pulls the pages straight from the pinned host tier over PCIe
// (zero-copy reads), so no host round trip sits between the selection and the
// transfer.  One workgroup per (fetch entry, unit), one 16-byte read in flight
// per thread: over the host link, reading two or four chunks per thread at once
// measured slower (48 against 52 GB/s).
#include "oasis_internal.h"

namespace oasis {
namespace {

constexpr int kGatherThreads = 256;

__global__ __launch_bounds__(kGatherThreads) void fetch_gather_kernel(
    const uint4* __restrict__ host, uint4* __restrict__ pool, const int32_t* __restrict__ fetch,
    const int32_t* __restrict__ n_fetch, int cap, int Nmax, int kb, int page16) {
  const int i = blockIdx.x;     // fetch entry
  const int unit = blockIdx.y;
  const int nf = n_fetch[unit];
  if (i >= nf || i >= cap) return;
  const int b = fetch[(static_cast<size_t>(unit) * cap + i) * 2];
  const int s = fetch[(static_cast<size_t>(unit) * cap + i) * 2 + 1];
  if (b < 0 || b >= Nmax || s < 0 || s >= kb) return;  // never outside the tier or the pool
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(host + (static_cast<size_t>(unit) * Nmax + b) * page16);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(pool + (static_cast<size_t>(unit) * kb + s) * page16);
#pragma unroll 1
  for (int c = static_cast<int>(threadIdx.x); c < page16; c += kGatherThreads) dst[c] = src[c];
}

}  // namespace

hipError_t launch_fetch_gather(const Ctx& c, const void* host_dev, void* pool, const int32_t* fetch,
                               const int32_t* n_fetch, hipStream_t st) {
  const int cap = c.s.fetch_cap;
  if (cap <= 0) return hipSuccess;
  const int page16 = static_cast<int>(c.page_elems * c.elem_bytes / 16);
  hipLaunchKernelGGL(fetch_gather_kernel, dim3(cap, c.units), dim3(kGatherThreads), 0, st,
                     static_cast<const uint4*>(host_dev), static_cast<uint4*>(pool), fetch, n_fetch, cap,
                     c.s.max_blocks, c.s.budget_blocks, page16);
  return hipGetLastError();
}

}  // namespace oasis
