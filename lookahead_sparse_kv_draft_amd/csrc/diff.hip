// Standalone set difference against the HBM-resident set with a per-step fetch
// cap and capped eviction (the step itself is diff_body, diff_body.h).  One
// workgroup per (request, KV head), one thread per selection entry and slot;
// two dependent rounds of global loads: selection and slot map, then the
// resident blocks' scores and the selected blocks' slots.
#include "diff_body.h"

namespace oasis {
namespace {

__global__ __launch_bounds__(1024) void diff_kernel(
    const int32_t* __restrict__ sel, const float* __restrict__ scores, int32_t* __restrict__ b2s,
    int32_t* __restrict__ s2b, int32_t* __restrict__ fetch, int32_t* __restrict__ n_fetch,
    int32_t* __restrict__ evict, int32_t* __restrict__ attend, int32_t* __restrict__ n_attend, int Nmax, int kb,
    int cap) {
  extern __shared__ unsigned long long smem_u64[];
  int32_t* selL = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(smem_u64) + diff_lds_bytes(kb, Nmax, cap));
  __shared__ DiffShared sh;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  const int ic = min(tid, kb - 1);  // clamped: no branch around the loads
  const int b = sel[static_cast<size_t>(unit) * kb + ic];
  const int sb = s2b[static_cast<size_t>(unit) * kb + ic];
  const bool sok = sb >= 0 && sb < Nmax;
  const float sv = scores[static_cast<size_t>(unit) * Nmax + (sok ? sb : 0)];
  if (tid < kb) selL[tid] = b;
  __syncthreads();
  diff_body(unit, kb, Nmax, cap, selL, sb, sv, b2s + static_cast<size_t>(unit) * Nmax,
            s2b + static_cast<size_t>(unit) * kb, fetch, n_fetch, evict, attend, n_attend, smem_u64, sh);
}

}  // namespace

hipError_t launch_diff(const Ctx& c, const int32_t* sel, const float* scores, int32_t* b2s,
                       int32_t* s2b, int32_t* fetch, int32_t* n_fetch, int32_t* evict,
                       int32_t* attend, int32_t* n_attend, hipStream_t st) {
  const int kb = c.s.budget_blocks, cap = c.s.fetch_cap;
  const int threads = (kb + kWave - 1) / kWave * kWave;
  const size_t lds = diff_lds_bytes(kb, c.s.max_blocks, cap) + static_cast<size_t>(kb) * 4;
  hipLaunchKernelGGL(diff_kernel, dim3(c.units), dim3(threads), lds, st, sel, scores, b2s, s2b, fetch,
                     n_fetch, evict, attend, n_attend, c.s.max_blocks, kb, cap);
  return hipGetLastError();
}

}  // namespace oasis
