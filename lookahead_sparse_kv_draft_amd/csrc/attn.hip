// Sparse paged GQA decode attention over the resident selected blocks (OasisKV
// explainer, Figure 7 right: the verify query and the draft queries attend
// together over the sparse KV working set held in HBM).
//
// Work unit: one (request, KV head) and one split of its selection list; the
// splits are merged by a log-sum-exp combine kernel.  All T*G query rows of the
// unit (verify + drafts for each grouped query head) ride in the same
// wavefront, so every KV page is read from HBM once per step.
//
// bf16 path, per 16-token block and per 16-row query tile, on the MFMA units:
//   S^T[tok][row] = K[tok][:] . Q[row][:]   v_mfma_f32_16x16x32_bf16, A = the K
//       page rows (16 contiguous bytes per lane), B = the query rows (registers);
//       the output leaves lane (col, grp) with tokens 4grp..4grp+3 of row col;
//   online softmax in the log2 domain, in registers: block max over the 4
//       tokens of the lane and two cross-lane exchanges; probabilities rounded
//       to bf16 (the running sum adds the rounded values, so weights and
//       normaliser agree);
//   O^T[ch][row] += V^T[ch][tok] . P^T[tok][row]  v_mfma_f32_16x16x16_bf16, A =
//       the page's channel-major V^T (8 contiguous bytes per lane), B = the
//       lane's own 4 probabilities: P never leaves registers.
// The page layout (K token-major, V channel-major) is what makes both products
// read contiguous lane-sized pieces without an LDS transpose.  The next block's
// page loads are issued before the current block's math.
//
// f32 path: VALU, query rows and logits in LDS, accumulators in registers.
#include "oasis_internal.h"

namespace oasis {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ s16x4_t as_s16x4(const uint2& v) { return __builtin_bit_cast(s16x4_t, v); }

// LDS of the in-workgroup merge: per wave m and l for every row, plus the summed
// accumulator [rows][D].
template <int D, int RT, int W>
struct AttnMergeLds {
  float m[W][RT * 16];
  float l[W][RT * 16];
  float acc[RT * 16][D];
};

// W wavefronts per (unit, split) workgroup; W > 1 merges them in LDS.
template <int D, int RT, int W>
__global__ __launch_bounds__(64 * W) void attn_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ pool,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ b2s,
    const int32_t* __restrict__ ctx_len, float* __restrict__ ws_acc, float* __restrict__ ws_ml,
    float* __restrict__ out, int H, int GT, int rows, int Nmax, int kb, int splits, int split_len,
    float scale_log2) {
  constexpr int KS = D / 32;  // QK k-steps of 32 channels
  constexpr int CT = D / 16;  // PV channel tiles
  constexpr int PAGE = 2 * kBlock * D;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int wid = blockIdx.x;  // unit * splits + split
  const int unit = wid / splits;
  const int split = wid - unit * splits;
  const int n = ctx_len[unit / H];

  // (issued first: independent of the selection lookups below)
  // Query rows as the B operand of S^T = K Q^T: lane (col, grp) holds row
  // rt*16+col, channels 8*(4s+grp) .. +7 for k-step s.
  uint4 Qb[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + col;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      // row clamped so the load is unconditional; padded rows are zeroed below
      Qb[rt][s] = *reinterpret_cast<const uint4*>(q + (static_cast<size_t>(unit) * GT + min(row, rows - 1)) * D +
                                                  8 * (4 * s + grp));
      if (row >= rows) Qb[rt][s] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  // This wavefront's selection entries: i0 + wv, i0 + wv + W, ... (one per lane).
  const int i0 = split * split_len;
  const int cnt = min(split_len, kb - i0);
  const int e = wv + W * lane;
  int my_slot = -1, my_ntok = 0;
  if (e < cnt) {
    const int b = sel[static_cast<size_t>(unit) * kb + i0 + e];
    if (b >= 0 && b < Nmax) {
      const int s = b2s[static_cast<size_t>(unit) * Nmax + b];
      const int nt = min(kBlock, n - kBlock * b);
      if (s >= 0 && s < kb && nt > 0) {
        my_slot = s;
        my_ntok = nt;
      }
    }
  }
  // Compact the valid entries into lanes 0 .. nb-1 (forward lane permute).
  const uint64_t valid = __ballot(my_slot >= 0);
  const int nb = __popcll(valid);
  const int pos = __popcll(valid & ((1ull << lane) - 1ull));
  const int dst = (my_slot >= 0 ? pos : 63) * 4;
  const int c_slot = __builtin_amdgcn_ds_permute(dst, my_slot);
  const int c_ntok = __builtin_amdgcn_ds_permute(dst, my_ntok);

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
  // Issue the loads of compacted entry j (every call loads: no branch around the
  // loads, so each wait below covers only the older buffer).
  auto load = [&](Page& pg, int j) {
    const uint16_t* p = ubase + static_cast<size_t>(__shfl(c_slot, j)) * PAGE;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      pg.k[s] = *reinterpret_cast<const uint4*>(p + col * D + 8 * (4 * s + grp));
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      pg.v[ct] = *reinterpret_cast<const uint2*>(p + kBlock * D + (16 * ct + col) * kBlock + 4 * grp);
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
      const float mnew = fmaxf(mrun[rt], mb);
      const float alpha = exp2f(mrun[rt] - mnew);
      mrun[rt] = mnew;
      uint16_t pb[4];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = f32_to_bf16(exp2f(x[i] - mnew));
        psum += bf16_to_f32(pb[i]);
      }
      lrun[rt] = lrun[rt] * alpha + psum;
      const uint2 pw = make_uint2(static_cast<uint32_t>(pb[0]) | (static_cast<uint32_t>(pb[1]) << 16),
                                  static_cast<uint32_t>(pb[2]) | (static_cast<uint32_t>(pb[3]) << 16));
      const s16x4_t P = as_s16x4(pw);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        acc[rt][ct] *= alpha;
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_s16x4(pg.v[ct]), P, acc[rt][ct], 0, 0, 0);
      }
    }
  };

  // Ping-pong over two page buffers: the next block's loads are in flight while
  // the current block is processed.  Prefetch indices are clamped and an odd
  // count is padded with a zero-token pass (a no-op for the online softmax once
  // a real block has been seen), so the loop body has no branch and every wait
  // covers only the older buffer.
  if (nb > 0) {
    Page pa, pbuf;
    load(pa, 0);
    for (int j = 0; j < nb; j += 2) {
      load(pbuf, min(j + 1, nb - 1));
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the math
      process(pa, __shfl(c_ntok, j));
      load(pa, min(j + 2, nb - 1));
      __builtin_amdgcn_sched_barrier(0);
      process(pbuf, (j + 1 < nb) ? __shfl(c_ntok, j + 1) : 0);
    }
  }

  if constexpr (W == 1) {
    // Single wavefront: the registers hold the whole split.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float L = lrun[rt];
      L += __shfl_xor(L, 16);
      L += __shfl_xor(L, 32);
      const int row = rt * 16 + col;
      if (row < rows) {
        if (splits == 1) {
          const float inv = (mrun[rt] == -INFINITY) ? 0.f : 1.f / L;
          float* o = out + (static_cast<size_t>(unit) * rows + row) * D;
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            *reinterpret_cast<float4*>(o + 16 * ct + 4 * grp) =
                make_float4(acc[rt][ct][0] * inv, acc[rt][ct][1] * inv, acc[rt][ct][2] * inv, acc[rt][ct][3] * inv);
        } else {
          float* wa = ws_acc + (static_cast<size_t>(wid) * rows + row) * D;
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            *reinterpret_cast<float4*>(wa + 16 * ct + 4 * grp) =
                make_float4(acc[rt][ct][0], acc[rt][ct][1], acc[rt][ct][2], acc[rt][ct][3]);
          if (grp == 0) {
            ws_ml[(static_cast<size_t>(wid) * rows + row) * 2] = mrun[rt];
            ws_ml[(static_cast<size_t>(wid) * rows + row) * 2 + 1] = L;
          }
        }
      }
    }
    return;
  } else {
  __shared__ AttnMergeLds<D, RT, W> sm;
  // ---- merge the wavefronts of the workgroup in LDS ----
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float L = lrun[rt];
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    if (grp == 0) {
      sm.m[wv][rt * 16 + col] = mrun[rt];
      sm.l[wv][rt * 16 + col] = L;
    }
  }
  for (int i = threadIdx.x; i < RT * 16 * D; i += blockDim.x) (&sm.acc[0][0])[i] = 0.f;
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + col;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm.m[w][row]);
    const float f = (mrun[rt] == -INFINITY) ? 0.f : exp2f(mrun[rt] - M);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(&sm.acc[row][16 * ct + 4 * grp + i], acc[rt][ct][i] * f);
  }
  __syncthreads();
  // Workgroup result per row: M, L = sum_w l_w * 2^(m_w - M), and sm.acc.
  // One split: write the normalised output; otherwise write the partial.
  const bool final_out = (splits == 1);
  for (int i = threadIdx.x; i < rows * D; i += blockDim.x) {
    const int row = i / D, c = i - row * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm.m[w][row]);
    const float a = sm.acc[row][c];
    if (final_out) {
      float L = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < W; ++w)
          L += (sm.m[w][row] == -INFINITY) ? 0.f : sm.l[w][row] * exp2f(sm.m[w][row] - M);
      }
      out[(static_cast<size_t>(unit) * rows + row) * D + c] = (M == -INFINITY) ? 0.f : a / L;
    } else {
      ws_acc[(static_cast<size_t>(wid) * rows + row) * D + c] = a;
      if (c == 0) {
        float L = 0.f;
        if (M != -INFINITY) {
#pragma unroll
          for (int w = 0; w < W; ++w)
            L += (sm.m[w][row] == -INFINITY) ? 0.f : sm.l[w][row] * exp2f(sm.m[w][row] - M);
        }
        ws_ml[(static_cast<size_t>(wid) * rows + row) * 2] = M;
        ws_ml[(static_cast<size_t>(wid) * rows + row) * 2 + 1] = L;
      }
    }
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

// Log-sum-exp merge of the split partials; one wavefront per (unit, query row),
// four per workgroup.  All partial loads of a row are independent of each other.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ ws_acc,
                                                           const float* __restrict__ ws_ml,
                                                           float* __restrict__ out, int rows,
                                                           int splits, int total) {
  constexpr int PER = D / kWave;
  const int id = blockIdx.x * 4 + threadIdx.x / kWave;  // unit * rows + row
  if (id >= total) return;
  const int unit = id / rows;
  const int row = id - unit * rows;
  const int lane = threadIdx.x & (kWave - 1);
  // lane s < splits holds split s's (m, l)
  float ms = -INFINITY, ls = 0.f;
  if (lane < splits) {
    const size_t p = (static_cast<size_t>(unit) * splits + lane) * rows + row;
    ms = ws_ml[p * 2];
    ls = ws_ml[p * 2 + 1];
  }
  float M = ms;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float* o = out + static_cast<size_t>(id) * D;
  if (M == -INFINITY) {
#pragma unroll
    for (int j = 0; j < PER; ++j) o[lane + kWave * j] = 0.f;
    return;
  }
  const float w_own = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
  float L = w_own * ls;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
  float a[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) a[j] = 0.f;
  // 8 partials at a time so their loads are in flight together (split index
  // clamped; the weight of a clamped repeat is zero)
  for (int s0 = 0; s0 < splits; s0 += 8) {
    float v[8][PER];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = min(s0 + u, splits - 1);
      const float* src = ws_acc + ((static_cast<size_t>(unit) * splits + s) * rows + row) * D;
#pragma unroll
      for (int j = 0; j < PER; ++j) v[u][j] = src[lane + kWave * j];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = (s0 + u < splits) ? __shfl(w_own, s0 + u) : 0.f;
#pragma unroll
      for (int j = 0; j < PER; ++j) a[j] += w * v[u][j];
    }
  }
  const float inv = 1.f / L;
#pragma unroll
  for (int j = 0; j < PER; ++j) o[lane + kWave * j] = a[j] * inv;
}

struct WsLayout {
  size_t acc_floats, ml_floats;
};

WsLayout ws_layout(const Ctx& c) {
  const size_t parts = static_cast<size_t>(c.units) * c.attn_splits * c.rows_attn;
  return {parts * c.s.head_dim, parts * 2};
}

template <int D, int RT, int W>
hipError_t mfma_w(const Ctx& c, const void* q, const void* pool, const int32_t* sel,
                  const int32_t* b2s, const int32_t* ctx_len, float* ws_acc, float* ws_ml,
                  float* out, float scale_log2, hipStream_t st) {
  hipLaunchKernelGGL((attn_mfma_kernel<D, RT, W>), dim3(c.units * c.attn_splits), dim3(W * kWave), 0,
                     st, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(pool), sel, b2s,
                     ctx_len, ws_acc, ws_ml, out, c.s.kv_heads, c.rows_attn, c.rows_attn,
                     c.s.max_blocks, c.s.budget_blocks, c.attn_splits, c.attn_split_len, scale_log2);
  return hipGetLastError();
}

template <int D, int RT>
hipError_t mfma_t(const Ctx& c, const void* q, const void* pool, const int32_t* sel,
                  const int32_t* b2s, const int32_t* ctx_len, float* ws_acc, float* ws_ml,
                  float* out, float scale_log2, hipStream_t st) {
  switch (c.attn_waves) {
    case 1: return mfma_w<D, RT, 1>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, scale_log2, st);
    case 2: return mfma_w<D, RT, 2>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, scale_log2, st);
    default: return mfma_w<D, RT, 4>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, scale_log2, st);
  }
}

template <int D>
hipError_t main_t(const Ctx& c, const void* q, const void* pool, const int32_t* sel,
                  const int32_t* b2s, const int32_t* ctx_len, float* ws_acc, float* ws_ml,
                  float* out, hipStream_t st) {
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

}  // namespace

size_t attn_workspace_bytes(const Ctx& c) {
  const WsLayout w = ws_layout(c);
  const size_t acc_bytes = ((w.acc_floats * sizeof(float)) + 255) / 256 * 256;
  return acc_bytes + w.ml_floats * sizeof(float);
}

hipError_t launch_attn(const Ctx& c, const void* q, const void* pool, const int32_t* sel,
                       const int32_t* b2s, const int32_t* ctx_len, float* out, void* ws,
                       hipStream_t st) {
  const WsLayout w = ws_layout(c);
  float* ws_acc = static_cast<float*>(ws);
  float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                          ((w.acc_floats * sizeof(float)) + 255) / 256 * 256);
  hipError_t e = (c.s.head_dim == 128)
      ? main_t<128>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, st)
      : main_t<64>(c, q, pool, sel, b2s, ctx_len, ws_acc, ws_ml, out, st);
  if (e != hipSuccess) return e;
  // The bf16 kernel writes the output itself when there is a single split.
  if (c.s.dtype == OASIS_BF16 && c.attn_splits == 1) return hipSuccess;
  const int total = c.units * c.rows_attn;
  const int grid = (total + 3) / 4;
  if (c.s.head_dim == 128)
    hipLaunchKernelGGL((attn_combine_kernel<128>), dim3(grid), dim3(256), 0, st, ws_acc, ws_ml,
                       out, c.rows_attn, c.attn_splits, total);
  else
    hipLaunchKernelGGL((attn_combine_kernel<64>), dim3(grid), dim3(256), 0, st, ws_acc, ws_ml,
                       out, c.rows_attn, c.attn_splits, total);
  return hipGetLastError();
}

}  // namespace oasis
