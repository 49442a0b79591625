// Sparse paged GQA decode attention over the resident selected blocks (OasisKV
// explainer, Figure 7 right: the verify query and the draft queries attend
// together over the sparse KV working set held in HBM).
//
// Work unit: one (request, KV head) and one split of its selection list.  All
// T*G query rows of the unit (verify + drafts for each grouped query head) ride
// in the same wavefront, so every KV page is read from HBM once per step.
//
// bf16 path, per 16-token block and per 16-row query tile, on the MFMA units:
//   S^T[tok][row] = K[tok][:] . Q[row][:]   v_mfma_f32_16x16x32_bf16, A = the K
//       page rows (16 contiguous bytes per lane), B = the query rows (registers);
//       the output leaves lane (col, grp) with tokens 4grp..4grp+3 of row col;
//   online softmax in the log2 domain, in registers: block max over the 4
//       tokens of the lane and two cross-lane exchanges, a reference max that
//       moves only on large increases; probabilities rounded to bf16 (the running
//       sum adds the rounded values, so weights and normaliser agree);
//   O^T[ch][row] += V^T[ch][tok] . P^T[tok][row]  v_mfma_f32_16x16x16_bf16, A =
//       the page's channel-major V^T (8 contiguous bytes per lane), B = the
//       lane's own 4 probabilities: P never leaves registers.
// The page layout (K token-major, V channel-major) is what makes both products
// read contiguous lane-sized pieces without an LDS transpose.  A wavefront
// requests all of its pages before it processes the first.
//
// f32 path: VALU, query rows and logits in LDS, accumulators in registers.
// Both paths leave one partial per split; a log-sum-exp combine kernel merges
// them.
#include "attn_combine.h"

namespace oasis {
namespace {

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
template <int D, int RT, int W, int PF>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu((PF <= 2 && RT <= 3) ? 2 : 1))) void attn_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ pool,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ b2s,
    const int32_t* __restrict__ ctx_len, float* __restrict__ ws_acc, float* __restrict__ ws_ml,
    float* __restrict__ out, int H, int rows, int Nmax, int kb,
    int splits, int run, float scale_log2) {
  constexpr int KS = D / 32;  // QK k-steps of 32 channels
  constexpr int CT = D / 16;  // PV channel tiles
  constexpr int PAGE = 2 * kBlock * D;
  constexpr int NT = 64 * W;
  constexpr int NSLICE = (W > 1) ? W / 2 : 1;
  __shared__ float sm_m[W][RT * 16];
  __shared__ float sm_l[W][RT * 16];
  __shared__ float4 sm_slice[NSLICE][RT][CT][kWave];  // wavefront accumulators in register layout
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int wid = blockIdx.x;  // unit * splits + split
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

  // The unit's attended entries (selected blocks that are resident and hold
  // tokens below n), in rank order, packed slot | ntok << 16: every workgroup of
  // the unit builds the whole list in LDS (lookups in batches of four entries
  // per thread, all loads of a batch in flight), then takes its wavefronts'
  // shares of an even split over all splits * W wavefronts of the unit, so every
  // wavefront streams the same number of pages (+-1).
  __shared__ int sm_att[kMaxBudget];
  __shared__ int sm_wcnt[4][W];
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
  const int nwv = splits * W;
  const int per = (natt + nwv - 1) / nwv;  // <= run <= 64
  const int e0 = (split * W + wv) * per;
  const int nb = max(0, min(per, natt - e0));
  const int mine = (lane < nb) ? sm_att[e0 + lane] : 0;
  const int c_slot = mine & 0xFFFF;
  const int c_ntok = mine >> 16;

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
  // The page base is wavefront-uniform (scalar registers); the lane offsets are
  // the same for every page.
  const uint16_t* kl = ubase + col * D + 8 * grp;
  const uint16_t* vl = ubase + kBlock * D + col * kBlock + 4 * grp;
  auto load = [&](Page& pg, int j) {
    const size_t off = static_cast<size_t>(__builtin_amdgcn_readfirstlane(__shfl(c_slot, j))) * PAGE;
#pragma unroll
    for (int s = 0; s < KS; ++s) pg.k[s] = *reinterpret_cast<const uint4*>(kl + off + 32 * s);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) pg.v[ct] = *reinterpret_cast<const uint2*>(vl + off + 16 * kBlock * ct);
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
      mb = fmaxf(mb, __shfl_xor(mb, 16));
      mb = fmaxf(mb, __shfl_xor(mb, 32));
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
      uint16_t pb[4];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = f32_to_bf16(exp2f(x[i] - mrun[rt]));
        psum += bf16_to_f32(pb[i]);
      }
      lrun[rt] += psum;
      const uint2 pw = make_uint2(static_cast<uint32_t>(pb[0]) | (static_cast<uint32_t>(pb[1]) << 16),
                                  static_cast<uint32_t>(pb[2]) | (static_cast<uint32_t>(pb[3]) << 16));
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
        process(pg[j], __builtin_amdgcn_readfirstlane(__shfl(c_ntok, j0 + j)));
        load(pg[j], min(j0 + j + PF, nb - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int j = 0; j < PF; ++j)
      if (npad - PF + j < nb) process(pg[j], __builtin_amdgcn_readfirstlane(__shfl(c_ntok, npad - PF + j)));
  }

  // ---- merge the wavefronts: a fixed-order tree in LDS (deterministic) ----
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float Lw = lrun[rt];
    Lw += __shfl_xor(Lw, 16);
    Lw += __shfl_xor(Lw, 32);
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

// fp32 path: workgroup of 256 threads per (unit, split).
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ pool, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ b2s, const int32_t* __restrict__ ctx_len,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml, int H, int GT, int rows, int Nmax,
    int kb, int splits, int split_len, float scale_log2) {
  constexpr int PAGE = 2 * kBlock * D;
  constexpr int J = (kMaxRows * D + 255) / 256;  // accumulators per thread (upper bound)
  extern __shared__ float smem[];
  float* qs = smem;                   // [rows][D]
  float* lg = qs + rows * D;          // [rows][16] logits, then probabilities
  float* alpha_s = lg + rows * kBlock;  // [rows]
  float* m_s = alpha_s + rows;        // [rows]
  float* l_s = m_s + rows;            // [rows]
  const int tid = threadIdx.x;
  const int wid = blockIdx.x;
  const int unit = wid / splits;
  const int split = wid - unit * splits;
  const int n = ctx_len[unit / H];
  for (int i = tid; i < rows * D; i += 256) qs[i] = q[static_cast<size_t>(unit) * GT * D + i];
  for (int i = tid; i < rows; i += 256) {
    m_s[i] = -INFINITY;
    l_s[i] = 0.f;
  }
  float acc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) acc[j] = 0.f;
  __syncthreads();
  const int i0 = split * split_len;
  const int i1 = min(kb, i0 + split_len);
  for (int e = i0; e < i1; ++e) {
    const int b = sel[static_cast<size_t>(unit) * kb + e];
    if (b < 0 || b >= Nmax) continue;
    const int slot = b2s[static_cast<size_t>(unit) * Nmax + b];
    const int ntok = min(kBlock, n - kBlock * b);
    if (slot < 0 || slot >= kb || ntok <= 0) continue;
    const float* pg = pool + (static_cast<size_t>(unit) * kb + slot) * PAGE;
    for (int i = tid; i < rows * kBlock; i += 256) {
      const int row = i / kBlock, tok = i - (i / kBlock) * kBlock;
      float s = -INFINITY;
      if (tok < ntok) {
        s = 0.f;
        for (int c = 0; c < D; ++c) s += qs[row * D + c] * pg[tok * D + c];
        s *= scale_log2;
      }
      lg[i] = s;
    }
    __syncthreads();
    for (int row = tid; row < rows; row += 256) {
      float mb = -INFINITY;
      for (int t = 0; t < kBlock; ++t) mb = fmaxf(mb, lg[row * kBlock + t]);
      const float mnew = fmaxf(m_s[row], mb);
      const float a = exp2f(m_s[row] - mnew);
      float ps = 0.f;
      for (int t = 0; t < kBlock; ++t) {
        const float p = exp2f(lg[row * kBlock + t] - mnew);
        lg[row * kBlock + t] = p;
        ps += p;
      }
      l_s[row] = l_s[row] * a + ps;
      m_s[row] = mnew;
      alpha_s[row] = a;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int i = tid + 256 * j;
      if (i < rows * D) {
        const int row = i / D, c = i - (i / D) * D;
        float a = acc[j] * alpha_s[row];
        for (int t = 0; t < ntok; ++t) a += lg[row * kBlock + t] * pg[kBlock * D + c * kBlock + t];
        acc[j] = a;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = tid + 256 * j;
    if (i < rows * D) ws_acc[static_cast<size_t>(wid) * rows * D + i] = acc[j];
  }
  for (int row = tid; row < rows; row += 256) {
    ws_ml[(static_cast<size_t>(wid) * rows + row) * 2] = m_s[row];
    ws_ml[(static_cast<size_t>(wid) * rows + row) * 2 + 1] = l_s[row];
  }
}

template <int D, int SMAX>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ ws_acc,
                                                           const float* __restrict__ ws_ml,
                                                           float* __restrict__ out, int rows,
                                                           int splits, int total) {
  attn_combine_row<D, SMAX>(ws_acc, ws_ml, out, rows, splits, total, blockIdx.x * 4 + threadIdx.x / kWave,
                            threadIdx.x & (kWave - 1));
}

template <int D, int RT, int W, int PF>
hipError_t mfma_wp(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                   const int32_t* ctx_len, float* ws_acc, float* ws_ml, float* out,
                   float scale_log2, hipStream_t st) {
  hipLaunchKernelGGL((attn_mfma_kernel<D, RT, W, PF>), dim3(c.units * c.attn_splits), dim3(W * kWave), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(pool), sel, b2s, ctx_len,
                     ws_acc, ws_ml, out, c.s.kv_heads, c.rows_attn, c.s.max_blocks,
                     c.s.budget_blocks, c.attn_splits, c.attn_run, scale_log2);
  return hipGetLastError();
}

template <int D, int RT, int W>
hipError_t mfma_w(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                  const int32_t* ctx_len, float* ws_acc, float* ws_ml, float* out,
                  float scale_log2, hipStream_t st) {
  switch (c.attn_pf) {
    case 2: return mfma_wp<D, RT, W, 2>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, scale_log2, st);
    case 4: return mfma_wp<D, RT, W, 4>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, scale_log2, st);
    default: return mfma_wp<D, RT, W, 8>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, scale_log2, st);
  }
}

template <int D, int RT>
hipError_t mfma_t(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                  const int32_t* ctx_len, float* ws_acc, float* ws_ml, float* out,
                  float scale_log2, hipStream_t st) {
  if (c.attn_waves == 1) return mfma_w<D, RT, 1>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, scale_log2, st);
  // at most 2 wavefronts for 3 or 4 row tiles (LDS of the wavefront merge)
  if (RT >= 3 || c.attn_waves == 2)
    return mfma_w<D, RT, 2>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, scale_log2, st);
  return mfma_w<D, RT, (RT >= 3 ? 2 : 4)>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, scale_log2, st);
}

template <int D>
hipError_t main_t(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                  const int32_t* ctx_len, float* ws_acc, float* ws_ml, float* out,
                  hipStream_t st) {
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  if (c.s.dtype == OASIS_BF16) {
    switch ((c.rows_attn + 15) / 16) {
      case 1: return mfma_t<D, 1>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, scale_log2, st);
      case 2: return mfma_t<D, 2>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, scale_log2, st);
      case 3: return mfma_t<D, 3>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, scale_log2, st);
      default: return mfma_t<D, 4>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, scale_log2, st);
    }
  }
  const int rows = c.rows_attn;
  const size_t lds = (static_cast<size_t>(rows) * D + rows * kBlock + 3 * rows) * sizeof(float);
  hipLaunchKernelGGL((attn_f32_kernel<D>), dim3(c.units * c.attn_splits), dim3(256), lds, st,
                     static_cast<const float*>(q), static_cast<const float*>(pool), sel, b2s,
                     ctx_len, ws_acc, ws_ml, c.s.kv_heads, c.rows_attn, rows, c.s.max_blocks,
                     c.s.budget_blocks, c.attn_splits, c.attn_split_len, scale_log2);
  return hipGetLastError();
}

template <int D>
hipError_t combine_t(const Ctx& c, const float* ws_acc, const float* ws_ml, float* out, hipStream_t st) {
  const int total = c.units * c.rows_attn;
  const int grid = (total + 3) / 4;
  const int S = c.attn_splits;
#define OASIS_COMBINE(SM)                                                                           \
  hipLaunchKernelGGL((attn_combine_kernel<D, SM>), dim3(grid), dim3(256), 0, st, ws_acc, ws_ml, out, \
                     c.rows_attn, S, total)
  if (S <= 4)
    OASIS_COMBINE(4);
  else if (S <= 8)
    OASIS_COMBINE(8);
  else if (S <= 16)
    OASIS_COMBINE(16);
  else
    OASIS_COMBINE(32);
#undef OASIS_COMBINE
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(const Ctx& c) { return attn_ws_acc_bytes(c) + attn_ws_ml_bytes(c); }

bool attn_needs_combine(const Ctx& c) {
  // the bf16 kernel writes the output itself when there is a single split
  return !(c.s.dtype == OASIS_BF16 && c.attn_splits == 1);
}

hipError_t launch_attn_main(const Ctx& c, const void* q, const void* pool, const int32_t* sel,
                            const int32_t* b2s, const int32_t* ctx_len, float* out, void* ws,
                            hipStream_t st) {
  float* ws_acc = static_cast<float*>(ws);
  float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + attn_ws_acc_bytes(c));
  return (c.s.head_dim == 128) ? main_t<128>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, st)
                               : main_t<64>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, st);
}

hipError_t launch_attn(const Ctx& c, const void* q, const void* pool, const int32_t* sel,
                       const int32_t* b2s, const int32_t* ctx_len, float* out, void* ws,
                       hipStream_t st) {
  hipError_t e = launch_attn_main(c, q, pool, sel, b2s, ctx_len, out, ws, st);
  if (e != hipSuccess || !attn_needs_combine(c)) return e;
  float* ws_acc = static_cast<float*>(ws);
  float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + attn_ws_acc_bytes(c));
  return (c.s.head_dim == 128) ? combine_t<128>(c, ws_acc, ws_ml, out, st)
                               : combine_t<64>(c, ws_acc, ws_ml, out, st);
}

}  // namespace oasis
