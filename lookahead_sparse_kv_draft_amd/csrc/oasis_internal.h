// Internal declarations shared by the C-ABI layer and the HIP kernels of liboasiskv.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "oasiskv.h"

namespace oasis {

constexpr int kBlock = 16;     // tokens per KV block
constexpr int kWave = 64;      // CDNA wavefront width
constexpr int kMaxRows = 64;   // query rows per unit handled by the kernels (4 MFMA row tiles)
constexpr int kMaxBudget = 1024;
constexpr int kAttendSlotBits = 10;   // attended-list entry = block << 10 | slot (slot < kMaxBudget)

// Block metadata layout.  Per unit, ceil(max_blocks / 16) tiles of 16 blocks;
// in a tile, the 16-byte chunks of the blocks' 2d-element rows (key min, then
// key max) are stored chunk-major: chunk c of block 16t + j at position
// 16c + j.  A 64-lane load of 16 bytes per lane then reads chunks 4s .. 4s+3
// of all 16 blocks, 1 KiB contiguous (the scoring's MFMA operand for k-step s).
constexpr int kMetaTile = 16;
__host__ __device__ inline int meta_tiles(int Nmax) { return (Nmax + kMetaTile - 1) / kMetaTile; }
// Element offset of element e (0 <= e < 2d) of block b of unit `unit`; CE =
// elements per 16-byte chunk (8 for bf16, 4 for fp32).
template <int D, int CE>
__host__ __device__ inline size_t meta_offset(int unit, int b, int e, int Nmax) {
  constexpr int NC = 2 * D / CE;  // chunks per block row
  const int t = b / kMetaTile, j = b - t * kMetaTile;
  const int c = e / CE, o = e - c * CE;
  return ((static_cast<size_t>(unit) * meta_tiles(Nmax) + t) * NC + c) * (kMetaTile * CE) +
         static_cast<size_t>(j) * CE + o;
}
constexpr int kAttnMaxSplits = 32;  // attention splits per unit (merge statistics kept in LDS)
// The split merge inside the fused first launch takes at most this many
// splits (their row statistics stay in registers).
constexpr int kAttnMergeMaxSplits = 8;

struct Ctx {
  oasis_shape s;
  int T;            // 1 + n_draft
  int rows_score;   // n_draft * group
  int rows_attn;    // T * group
  int elem_bytes;   // 2 (bf16) or 4 (f32)
  size_t page_elems;  // 2 * 16 * d
  int units;        // batch * kv_heads
  int attn_splits;  // split-K factor of the attention
  int attn_split_len;  // selection entries per split (attn_waves * attn_run)
  int attn_run;     // selection entries per attention wavefront (<= 64)
  // The attention on its own (not sharing the decode step's launch): its own
  // split count, run (fewer, longer wavefronts are best there) and ring.
  int attn_splits_solo, attn_run_solo, attn_pf_solo;
  int attn_waves;   // wavefronts per attention workgroup (1, 2 or 4)
  int attn_pf;      // pages in flight per attention wavefront (2, 4 or 8)
  int score_tpw;    // 16-block tiles per scoring wave beside the attention in the step's launch
  int score_tpw_solo;  // the same in a scoring launch of its own
  int step_order;   // workgroup order of the fused attention + score launch (0, 1, 2)
  int step_launches;  // launches per decode step: 2 (fused attention + score) or 3
  // The fused first launch merges the attention's splits itself (the last
  // workgroup of a unit to finish), with one arrival counter per unit at
  // ws_arrive_off in the workspace: in the two-launch step (attn_merge) and
  // in the carried step (attn_merge_carry).
  bool attn_merge, attn_merge_carry;
  size_t ws_arrive_off;
};

// ---- kernel launchers (defined in the .hip files); return a hipError_t ----
hipError_t launch_meta_build(const Ctx& c, const void* pages, const int32_t* ids, int32_t count,
                             const int32_t* ctx_len, void* meta, void* pool,
                             const int32_t* b2s, hipStream_t st);
// The metadata from the tiles to [units][Nmax][2][d] (to_logical) or back.
// The metadata of the blocks that tokens [tok_begin, tok_end) fall in, from key
// rows [units][Nmax*16][d].
hipError_t launch_meta_rows(const Ctx& c, const void* k_rows, int tok_begin, int tok_end, const int32_t* ctx_len,
                            void* meta, hipStream_t st);
hipError_t launch_meta_relayout(const Ctx& c, const void* src, void* dst, bool to_logical, hipStream_t st);
hipError_t launch_meta_update(const Ctx& c, const void* k_new, const void* v_new,
                              const int32_t* ctx_in, int32_t* ctx_out, void* meta, void* pool,
                              const int32_t* b2s, hipStream_t st);
// Prefill admission: pages into the host tier (device-mapped pinned memory)
// and resident pool slots, plus the metadata rows.
hipError_t launch_admit(const Ctx& c, const void* k_rows, const void* v_rows, const int32_t* ctx_len,
                        void* host_dev, void* meta, void* pool, const int32_t* b2s, hipStream_t st);
// A token append a decode step's launches carry (bf16): the token's K / V rows
// [B][H][d], its position per request (ctx_in) and ctx_in + 1 (ctx_out), and
// the metadata, pool and block map it updates (as oasis_block_meta_update).
struct StepAppend {
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  const int32_t* ctx_in = nullptr;
  int32_t* ctx_out = nullptr;
  void* meta = nullptr;
  void* pool = nullptr;
  const int32_t* b2s = nullptr;
};
// The lookahead score from the draft rows, or (verify) the same bound from the
// verify query rows.  With `ap` (bf16 only) one workgroup per unit after the
// scoring writes the appended token's page row (the scoring reads no pages).
hipError_t launch_score(const Ctx& c, const void* q, const void* meta, const int32_t* ctx_len,
                        float* scores, hipStream_t st, bool verify = false, const StepAppend* ap = nullptr);
hipError_t launch_topk(const Ctx& c, const float* scores, const int32_t* ctx_len, int32_t* sel,
                       hipStream_t st);
bool select_diff_fused_available(const Ctx& c);
// Least-recently-used eviction (null last_use: lowest-score eviction): the
// per-slot stamps [B][H][k] and this step's stamp.  Supported by the fused
// selection + diff for k <= 128 (select_diff_lru_available).
struct LruState {
  int32_t* last_use = nullptr;
  int step = 0;
};
bool select_diff_lru_available(const Ctx& c);
// Budgets of at most 128 blocks and N_max <= 8192: the selection and diff of a
// unit run in one workgroup (select_wg.h) in every launch that selects.
bool select_wg_available(const Ctx& c);
hipError_t launch_select_diff(const Ctx& c, const float* scores, const int32_t* ctx_len, int32_t* sel,
                              int32_t* b2s, int32_t* s2b, int32_t* fetch, int32_t* n_fetch, int32_t* evict,
                              int32_t* attend, int32_t* n_attend, hipStream_t st, LruState lru = {});
hipError_t launch_diff(const Ctx& c, const int32_t* sel, const float* scores, int32_t* b2s,
                       int32_t* s2b, int32_t* fetch, int32_t* n_fetch, int32_t* evict,
                       int32_t* attend, int32_t* n_attend, hipStream_t st);
// Attention over S ∩ R given either (sel, b2s) or, when attend is not null, the
// attended list a diff produced (sel and b2s are then ignored).  With `ap`
// (bf16 only) one workgroup per unit after the attention updates the appended
// token's metadata row (its page row is left to the scoring launch).
hipError_t launch_attn(const Ctx& c, const void* q, const void* pool, const int32_t* sel,
                       const int32_t* b2s, const int32_t* attend, const int32_t* n_attend,
                       const int32_t* ctx_len, float* out, void* ws, hipStream_t st,
                       const StepAppend* ap = nullptr);
// The attention without its split combine, and whether a combine must follow.
hipError_t launch_attn_main(const Ctx& c, const void* q, const void* pool, const int32_t* sel,
                            const int32_t* b2s, const int32_t* attend, const int32_t* n_attend,
                            const int32_t* ctx_len, float* out, void* ws, hipStream_t st,
                            const StepAppend* ap = nullptr);
bool attn_needs_combine(const Ctx& c);
// The split combine alone (nothing to do when the attention wrote the output).
hipError_t launch_attn_combine(const Ctx& c, void* ws, float* out, hipStream_t st);
// Another layer's page transfer carried by the step's first launch: its host
// tier (device address of the pinned mapping), pool, fetch list and counts
// (host == nullptr: none).
struct StepGather {
  const uint4* host = nullptr;
  uint4* pool = nullptr;
  const int32_t* fetch = nullptr;
  const int32_t* n_fetch = nullptr;
  int cap = 0;
};
// The attention (split partials) and the lookahead score in one launch (bf16,
// 2-wavefront 2-page attention, up to three attention row tiles), optionally
// led by workgroups that carry another layer's transfer.
bool attn_and_score_fused_available(const Ctx& c);
hipError_t launch_attn_and_score(const Ctx& c, const void* q, const void* pool, const int32_t* sel,
                                 const int32_t* b2s, const int32_t* attend, const int32_t* n_attend,
                                 const int32_t* ctx_attn, float* out, void* ws, const void* meta,
                                 const int32_t* ctx_score, float* scores, hipStream_t st,
                                 const StepGather& g = StepGather());
// One state's top-k selection and resident-set diff run by one workgroup per
// unit (select_wg.h): its scores (complete: written by an earlier launch), the
// context length its scoring saw, the state the diff updates, and for
// least-recently-used eviction the per-slot stamps and the step number the diff
// stamps.  Carried by the step's first launch, none of it may be memory that
// launch's own attention or scoring reads or writes (score eviction, k <= 128,
// N_max <= 8192, bf16, head_dim 128, 2 attention wavefronts).
struct SelectJob {
  const float* scores = nullptr;
  const int32_t* ctx_len = nullptr;
  int32_t* sel = nullptr;
  int32_t* b2s = nullptr;
  int32_t* s2b = nullptr;
  int32_t* fetch = nullptr;
  int32_t* n_fetch = nullptr;
  int32_t* evict = nullptr;
  int32_t* attend = nullptr;
  int32_t* n_attend = nullptr;
  int32_t* last_use = nullptr;
  int step = 0;
};
bool attn_score_select_available(const Ctx& c);
// The attention (from the attended list) and the lookahead score in one launch
// (as launch_attn_and_score), led by the transfer's workgroups and, when job is
// not null, by the carried selection's.
hipError_t launch_attn_score_select(const Ctx& c, const void* q, const void* pool, const int32_t* attend,
                                    const int32_t* n_attend, const int32_t* ctx_attn, float* out, void* ws,
                                    const void* meta, const int32_t* ctx_score, float* scores, const SelectJob* job,
                                    hipStream_t st, const StepGather& g = StepGather());
// The fused selection + diff and the attention's split combine in one launch
// (where select_diff_fused_available holds).
hipError_t launch_select_diff_combine(const Ctx& c, const float* scores, const int32_t* ctx_len, int32_t* sel,
                                      int32_t* b2s, int32_t* s2b, int32_t* fetch, int32_t* n_fetch, int32_t* evict,
                                      int32_t* attend, int32_t* n_attend, const void* ws, float* out,
                                      hipStream_t st, LruState lru = {});
// The split combine and the lookahead score in one launch (bf16 only).
hipError_t launch_combine_and_score(const Ctx& c, void* ws, float* out, const void* q, const void* meta,
                                   const int32_t* ctx_len, float* scores, hipStream_t st);
size_t attn_workspace_bytes(const Ctx& c);
// The split partials' part of the workspace (the arrival counters follow it).
size_t attn_ws_partials_bytes(const Ctx& c);
// The attention with its workspace in the library's per-GPU scratch array (no
// allocation); attn_scratch_bytes() is that array's size.
size_t attn_scratch_bytes();
hipError_t launch_attn_noalloc(const Ctx& c, const void* q, const void* pool, const int32_t* sel, const int32_t* b2s,
                               const int32_t* ctx_len, float* out, hipStream_t st);
hipError_t launch_fetch_gather(const Ctx& c, const void* host_dev, void* pool, const int32_t* fetch,
                               const int32_t* n_fetch, hipStream_t st);

// ---- small device helpers ----
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ s16x4_t as_s16x4(const uint2& v) { return __builtin_bit_cast(s16x4_t, v); }

// A value combined with the same value 16 (or 32) lanes away, through the
// gfx950 lane swaps (VALU instructions, no LDS round trip as a shuffle takes):
// swapping a register with itself leaves, in every lane, the lane's own value
// in one result and the value of lane ^ 16 (^ 32) in the other, in an order that
// depends on the lane, so only commutative combinations are formed from them.
__device__ __forceinline__ void lane_pair16(uint32_t x, uint32_t& a, uint32_t& b) {
  const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  a = p[0];
  b = p[1];
}
__device__ __forceinline__ void lane_pair32(uint32_t x, uint32_t& a, uint32_t& b) {
  const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  a = p[0];
  b = p[1];
}
__device__ __forceinline__ float max_xor16(float x) {
  uint32_t a, b;
  lane_pair16(__float_as_uint(x), a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ __forceinline__ float max_xor32(float x) {
  uint32_t a, b;
  lane_pair32(__float_as_uint(x), a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ __forceinline__ float add_xor16(float x) {
  uint32_t a, b;
  lane_pair16(__float_as_uint(x), a, b);
  return __uint_as_float(a) + __uint_as_float(b);
}
__device__ __forceinline__ float add_xor32(float x) {
  uint32_t a, b;
  lane_pair32(__float_as_uint(x), a, b);
  return __uint_as_float(a) + __uint_as_float(b);
}

// DPP moves inside a 16-lane row (VALU, no LDS round trip): lane i takes the
// value of lane ^ 1 (quad_perm [1,0,3,2], 0xB1), lane ^ 2 (quad_perm [2,3,0,1],
// 0x4E), lane 7 - i of its 8 (row_half_mirror, 0x141), lane 15 - i of its row
// (row_mirror, 0x140) or lane i - n of its row (row_shr:n, 0x110 + n; 0 for the
// first n lanes).  The source lane must be active.
template <int CTRL>
__device__ __forceinline__ int dpp_from(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}

// Sum over each group of P adjacent lanes (P = 1, 2, 4, 8 or 16, groups aligned
// to P and fully active); every lane of a group gets the group's sum.
__device__ __forceinline__ int group_sum(int r, int P) {
  if (P >= 2) r += dpp_from<0xB1>(r);
  if (P >= 4) r += dpp_from<0x4E>(r);
  if (P >= 8) r += dpp_from<0x141>(r);
  if (P >= 16) r += dpp_from<0x140>(r);
  return r;
}

// Inclusive prefix sum over the 64 lanes of a wavefront (all lanes active):
// within each row by DPP shifts, then the totals of the rows below from
// lanes 15, 31 and 47.
__device__ __forceinline__ int wave_incl_sum(int v) {
  v += dpp_from<0x111>(v);
  v += dpp_from<0x112>(v);
  v += dpp_from<0x114>(v);
  v += dpp_from<0x118>(v);
  const int row = (threadIdx.x & 63) >> 4;
  const int t0 = __builtin_amdgcn_readlane(v, 15), t1 = __builtin_amdgcn_readlane(v, 31),
            t2 = __builtin_amdgcn_readlane(v, 47);
  return v + (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
}

// Streaming loads of data read once per launch (block metadata tiles, KV
// pages): the non-temporal hint keeps them from displacing cached lines on the
// way in, which measured 4-6 % faster for the bandwidth-bound launches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(w.x, w.y, w.z, w.w);
}
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
  const u32x2_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(w.x, w.y);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// 32-bit key whose ascending order is descending score; -0.0 ranks as +0.0.
__device__ __forceinline__ uint32_t desc_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~ord;
}

}  // namespace oasis
