// C ABI of liboasiskv: argument validation, launch-shape selection and dispatch to
// the HIP kernels; host-side page packing, token append and fetch issue.
// Every entry point validates before enqueuing anything and reports errors through
// a status code plus a thread-local message.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>

#include "oasis_internal.h"

struct oasis_ctx {
  oasis::Ctx c;
};

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return OASIS_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(OASIS_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// [16][d] token-major -> [d][16] channel-major.
template <typename T>
void transpose_block(const T* src, T* dst, int d) {
  for (int t = 0; t < oasis::kBlock; ++t)
    for (int ch = 0; ch < d; ++ch) dst[ch * oasis::kBlock + t] = src[t * d + ch];
}

#define CHECK_HANDLE(h) \
  if ((h) == nullptr) return fail(OASIS_EINVAL, "%s: null handle", __func__)
#define CHECK_PTR(p) \
  if ((p) == nullptr) return fail(OASIS_EINVAL, "%s: %s is null", __func__, #p)
// Device buffers read with 16-byte vector loads.
#define CHECK_ALIGN16(p)                                   \
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)            \
  return fail(OASIS_EINVAL, "%s: %s is not 16-byte aligned", __func__, #p)

}  // namespace

extern "C" {

int oasis_version(void) { return 2; }

const char* oasis_last_error(void) { return g_err.c_str(); }

int oasis_create(const oasis_shape* shape, oasis_handle* out) {
  return oasis_create_with_options(shape, nullptr, out);
}

int oasis_create_with_options(const oasis_shape* shape, const oasis_launch_options* opts, oasis_handle* out) {
  CHECK_PTR(shape);
  CHECK_PTR(out);
  *out = nullptr;
  const oasis_shape& s = *shape;
  if (s.batch < 1 || s.kv_heads < 1 || s.group < 1 || s.max_blocks < 1 || s.n_draft < 1)
    return fail(OASIS_EINVAL, "oasis_create: batch, kv_heads, group, max_blocks, n_draft must be >= 1");
  if (s.budget_blocks < 2 || s.budget_blocks > oasis::kMaxBudget)
    return fail(OASIS_EINVAL, "oasis_create: budget_blocks %d outside [2, %d]", s.budget_blocks,
                oasis::kMaxBudget);
  if (s.fetch_cap < 0) return fail(OASIS_EINVAL, "oasis_create: fetch_cap %d < 0", s.fetch_cap);
  if (s.block_size != oasis::kBlock)
    return fail(OASIS_EUNSUPPORTED, "oasis_create: block_size %d (only 16 is built)", s.block_size);
  if (s.head_dim != 64 && s.head_dim != 128)
    return fail(OASIS_EUNSUPPORTED, "oasis_create: head_dim %d (64 or 128 are built)", s.head_dim);
  if (s.dtype != OASIS_BF16 && s.dtype != OASIS_F32)
    return fail(OASIS_EUNSUPPORTED, "oasis_create: dtype %d", s.dtype);
  if (s.max_blocks > 65536)
    return fail(OASIS_EUNSUPPORTED, "oasis_create: max_blocks %d > 65536", s.max_blocks);
  const long long units = static_cast<long long>(s.batch) * s.kv_heads;
  if (units > (1 << 24)) return fail(OASIS_EUNSUPPORTED, "oasis_create: too many units");
  const int T = 1 + s.n_draft;
  const int rows_score = s.n_draft * s.group;
  const int rows_attn = T * s.group;
  if (rows_attn > oasis::kMaxRows)
    return fail(OASIS_EUNSUPPORTED, "oasis_create: (1 + n_draft) * group = %d query rows > %d",
                rows_attn, oasis::kMaxRows);
  oasis_launch_options o{};
  if (opts != nullptr) o = *opts;
  if (o.attn_waves != 0 && o.attn_waves != 1 && o.attn_waves != 2 && o.attn_waves != 4)
    return fail(OASIS_EINVAL, "oasis_create: attn_waves %d (0, 1, 2 or 4)", o.attn_waves);
  if (o.attn_pf != 0 && o.attn_pf != 2 && o.attn_pf != 4 && o.attn_pf != 8)
    return fail(OASIS_EINVAL, "oasis_create: attn_pf %d (0, 2, 4 or 8)", o.attn_pf);
  if (o.attn_splits < 0 || o.attn_splits > oasis::kAttnMaxSplits)
    return fail(OASIS_EINVAL, "oasis_create: attn_splits %d outside [0, %d]", o.attn_splits, oasis::kAttnMaxSplits);
  if (o.score_tpw < 0 || o.score_tpw > 64)
    return fail(OASIS_EINVAL, "oasis_create: score_tpw %d outside [0, 64]", o.score_tpw);
  if (o.step_order < 0 || o.step_order > 2)
    return fail(OASIS_EINVAL, "oasis_create: step_order %d outside [0, 2]", o.step_order);
  if (o.step_launches != 0 && o.step_launches != 2 && o.step_launches != 3)
    return fail(OASIS_EINVAL, "oasis_create: step_launches %d (0, 2 or 3)", o.step_launches);
  if (o.attn_merge < 0 || o.attn_merge > 3)
    return fail(OASIS_EINVAL, "oasis_create: attn_merge %d (0, 1, 2 or 3)", o.attn_merge);

  oasis_ctx* h = new (std::nothrow) oasis_ctx;
  if (h == nullptr) return fail(OASIS_EINVAL, "oasis_create: out of host memory");
  oasis::Ctx& c = h->c;
  c.s = s;
  c.T = T;
  c.rows_score = rows_score;
  c.rows_attn = rows_attn;
  c.elem_bytes = (s.dtype == OASIS_BF16) ? 2 : 4;
  c.page_elems = static_cast<size_t>(2) * oasis::kBlock * s.head_dim;
  c.units = static_cast<int>(units);

  // Attention: workgroups of W wavefronts, each wavefront streaming a run of
  // consecutive selection entries (at most 64) through a ring of PF page
  // buffers; a workgroup covers W runs (one split).  By default 2 wavefronts,
  // a 2-page ring and about 512 wavefronts per launch, on its own and beside
  // the scoring (fewer, longer-running wavefronts amortise the per-workgroup
  // start-up and write fewer partials).
  const int row_tiles = (rows_attn + 15) / 16;
  const int max_waves = (row_tiles <= 2) ? 4 : 2;  // LDS of the wavefront merge
  const int waves = std::min(o.attn_waves != 0 ? o.attn_waves : 2, max_waves);
  const int kbud = s.budget_blocks;
  // The decode step's first launch (attention beside the scoring, bf16 with the
  // default shape) keeps its own attention and scoring shapes.  With the
  // non-temporal page and metadata loads, about 512 attention wavefronts (as on
  // their own) and runs of 2 scoring tiles measured best: at the 32K-context
  // batch-8 step 34.4 us against 35.3 us with 1024 attention wavefronts, at the
  // 128K-context 8-layer step 40.8 against 42.8 us, within 0.5 % elsewhere.
  const bool step_fused = s.dtype == OASIS_BF16 && rows_attn <= 48 && (waves == 2 || (waves == 4 && row_tiles <= 2));
  // split count for about `target` wavefronts, then the run per wavefront
  auto shape_splits = [&](int target, int* run_out) {
    int sp = o.attn_splits > 0 ? o.attn_splits : (target + c.units * waves - 1) / (c.units * waves);
    const int min_splits = (kbud + 64 * waves - 1) / (64 * waves);  // run <= 64
    const int max_splits = std::min(oasis::kAttnMaxSplits, (kbud + waves - 1) / waves);
    sp = std::max(min_splits, std::min(sp, max_splits));
    const int r = (kbud + sp * waves - 1) / (sp * waves);
    *run_out = r;
    return (kbud + r * waves - 1) / (r * waves);  // no empty split
  };
  // Beside the scoring, the attention's wavefronts scale with its share of
  // the launch's bytes (per unit: k pages of 32 d elements against N_max
  // metadata rows of 2 d): about 512 from an even share up (the 32K-context
  // workloads, where 4 and 2 splits measured best), fewer below it (the
  // 128K-context 8-layer workload, share 0.2: 4 splits, 30.8 us per carried
  // layer step against 31.6 us with 8 splits and 33.7 / 32.3 us with 3 / 5).
  const double share = 16.0 * kbud / (16.0 * kbud + s.max_blocks);
  const int target_fused = std::max(1, static_cast<int>(std::lround(512.0 * std::min(1.0, 2.0 * share))));
  int run = 0, run_solo = 0;
  const int splits = shape_splits(target_fused, &run);
  const int splits_solo = shape_splits(512, &run_solo);
  const int max_pf = (row_tiles <= 2) ? 8 : (row_tiles == 3) ? 4 : 2;  // registers (no spills)
  // measured: a shallow ring keeps the math beside the loads, except where the
  // attention on its own gives each wavefront a whole unit's 64-block run in
  // one split at one wavefront per SIMD: there 4 pages in flight (the batch-64
  // reasoning workload: 60.8 against 62.4-63.3 us alone, the three-launch step
  // 115.3 against 118.4-119.7 us; with 2 to 8 splits of 8- to 32-block runs
  // the 4-page ring was 12-18 % slower)
  const int pf = std::min(o.attn_pf != 0 ? o.attn_pf : 2, max_pf);
  const bool long_runs = splits_solo == 1 && run_solo >= 64 && c.units * waves <= 4 * 256;
  const int pf_solo = std::min(o.attn_pf != 0 ? o.attn_pf : (long_runs ? 4 : 2), max_pf);
  c.attn_waves = waves;
  c.attn_pf = pf;
  c.attn_pf_solo = pf_solo;
  c.attn_run = run;
  c.attn_split_len = waves * run;
  c.attn_splits = splits;
  c.attn_splits_solo = splits_solo;
  c.attn_run_solo = run_solo;

  // Scoring: runs of 16-block tiles per wavefront, for about 4096 wavefronts
  // where the decode step runs it beside the attention (bf16), 2048 in a launch
  // of its own but at most 4 tiles (at the 32K-context batch-8 workload the
  // scoring alone takes 12.6 us with runs of 4 tiles against 13.4 us with 2,
  // while the step's launch is 0.4 us faster with 2; in the batch-64 reasoning
  // step, whose scoring launch reads its metadata cold, 4 tiles beat 8).
  const long long tiles = units * ((s.max_blocks + 15) / 16);
  auto runs_for = [&](long long waves) {
    return o.score_tpw > 0 ? o.score_tpw : static_cast<int>(std::max(1LL, std::min(16LL, tiles / waves)));
  };
  // Beside an attention that moves at least half of the launch's bytes, runs
  // of at most 2 tiles (the 32K-context 8-layer batch-16 workload: 50.6-50.7
  // against 51.9 us per carried layer step with 4; the 32K-context batch-8
  // step already had 2), else for about 4096 wavefronts (the 128K-context
  // 8-layer step: 4 tiles 30.7 against 30.8 us with 2).
  c.score_tpw = !step_fused ? runs_for(2048)
                : (o.score_tpw == 0 && share >= 0.5) ? std::min(2, runs_for(4096)) : runs_for(4096);
  c.score_tpw_solo = o.score_tpw > 0 ? o.score_tpw : std::min(runs_for(2048), 4);
  c.step_order = o.step_order;
  c.step_launches = o.step_launches == 3 ? 3 : 2;
  // The split merge inside the fused first launch, where 2 to 8 splits run
  // beside the scoring (an option; the default combines).  Each attention
  // workgroup then waits for its device-coherent partial and an atomic before
  // it ends, which lengthened the first launch by 2-3.5 us on every workload
  // measured; the carried step saves its combine launch for it, which paid at
  // 8 splits of the 128K-context 8-layer workload (31.7 against 32.5 us per
  // layer step) but not at the 4 splits that shape now takes (31.4 against
  // 30.8 us), nor at the 2 splits of the 32K-context 8-layer batch-16
  // workload (52.3 against 52.2 us); the two-launch step, whose second launch
  // combines beside the selection anyway, lost everywhere (32.7 against
  // 30.1 us at the 32K-context batch-8 step).  Its device-coherent accesses
  // address the partials with 32-bit byte offsets in a view of at most 2 GiB.
  const bool merge_ok = splits >= 2 && splits <= oasis::kAttnMergeMaxSplits && s.dtype == OASIS_BF16 &&
                        oasis::attn_ws_partials_bytes(c) < (static_cast<size_t>(1) << 31);
  const int merge = o.attn_merge != 0 ? o.attn_merge : 1;
  c.attn_merge = merge_ok && merge == 2;
  c.attn_merge_carry = merge_ok && (merge == 2 || merge == 3);
  c.ws_arrive_off = oasis::attn_ws_partials_bytes(c);
  *out = h;
  return ok();
}

int oasis_get_launch_options(oasis_handle h, oasis_launch_options* out) {
  CHECK_HANDLE(h);
  CHECK_PTR(out);
  const oasis::Ctx& c = h->c;
  out->attn_waves = c.attn_waves;
  out->attn_pf = c.attn_pf;
  out->attn_splits = c.attn_splits;
  out->score_tpw = c.score_tpw;
  out->step_order = c.step_order;
  out->attn_merge = c.attn_merge ? 2 : c.attn_merge_carry ? 3 : 1;
  out->step_launches = c.step_launches;
  return ok();
}

int oasis_destroy(oasis_handle h) {
  delete h;
  return ok();
}

size_t oasis_page_bytes(oasis_handle h) {
  return h ? h->c.page_elems * h->c.elem_bytes : 0;
}

size_t oasis_meta_bytes(oasis_handle h) {
  return h ? static_cast<size_t>(h->c.units) * oasis::meta_tiles(h->c.s.max_blocks) * oasis::kMetaTile * 2 *
                 h->c.s.head_dim * h->c.elem_bytes
           : 0;
}

size_t oasis_pool_bytes(oasis_handle h) {
  return h ? static_cast<size_t>(h->c.units) * h->c.s.budget_blocks * oasis_page_bytes(h) : 0;
}

size_t oasis_host_tier_bytes(oasis_handle h) {
  return h ? static_cast<size_t>(h->c.units) * h->c.s.max_blocks * oasis_page_bytes(h) : 0;
}

size_t oasis_workspace_bytes(oasis_handle h) { return h ? oasis::attn_workspace_bytes(h->c) : 0; }

int oasis_pack_pages(oasis_handle h, const void* k, const void* v, const int32_t* blocks,
                     int32_t n_blocks, int32_t unit, void* pages) {
  CHECK_HANDLE(h);
  CHECK_PTR(pages);
  const oasis::Ctx& c = h->c;
  if (n_blocks < 0) return fail(OASIS_EINVAL, "oasis_pack_pages: n_blocks %d < 0", n_blocks);
  if (unit < 0 || unit >= c.units) return fail(OASIS_EINVAL, "oasis_pack_pages: unit %d out of range", unit);
  if (n_blocks > 0 && k == nullptr && v == nullptr)
    return fail(OASIS_EINVAL, "oasis_pack_pages: k and v are both null");
  if (blocks == nullptr && n_blocks > c.s.max_blocks)
    return fail(OASIS_EINVAL, "oasis_pack_pages: n_blocks %d > max_blocks", n_blocks);
  if (blocks != nullptr)
    for (int i = 0; i < n_blocks; ++i)
      if (blocks[i] < 0 || blocks[i] >= c.s.max_blocks)
        return fail(OASIS_EINVAL, "oasis_pack_pages: block %d out of range", blocks[i]);
  const int d = c.s.head_dim;
  const size_t eb = c.elem_bytes;
  const size_t row_bytes = d * eb;
  char* base = static_cast<char*>(pages) + static_cast<size_t>(unit) * c.s.max_blocks * c.page_elems * eb;
  for (int i = 0; i < n_blocks; ++i) {
    const int b = blocks ? blocks[i] : i;
    char* pg = base + static_cast<size_t>(b) * c.page_elems * eb;
    if (k != nullptr)
      memcpy(pg, static_cast<const char*>(k) + static_cast<size_t>(i) * oasis::kBlock * row_bytes,
             oasis::kBlock * row_bytes);
    if (v != nullptr) {
      const char* src = static_cast<const char*>(v) + static_cast<size_t>(i) * oasis::kBlock * row_bytes;
      char* vt = pg + oasis::kBlock * row_bytes;  // V^T [d][16]
      if (eb == 2)
        transpose_block(reinterpret_cast<const uint16_t*>(src), reinterpret_cast<uint16_t*>(vt), d);
      else
        transpose_block(reinterpret_cast<const uint32_t*>(src), reinterpret_cast<uint32_t*>(vt), d);
    }
  }
  return ok();
}

int oasis_host_tier_append(oasis_handle h, const void* k_new, const void* v_new, const int32_t* pos,
                           void* host_tier) {
  CHECK_HANDLE(h);
  CHECK_PTR(k_new);
  CHECK_PTR(v_new);
  CHECK_PTR(pos);
  CHECK_PTR(host_tier);
  const oasis::Ctx& c = h->c;
  for (int r = 0; r < c.s.batch; ++r)
    if (pos[r] < 0 || pos[r] >= c.s.max_blocks * oasis::kBlock)
      return fail(OASIS_EINVAL, "oasis_host_tier_append: position %d of request %d out of range", pos[r], r);
  const int d = c.s.head_dim;
  const size_t eb = c.elem_bytes;
  for (int u = 0; u < c.units; ++u) {
    const int p = pos[u / c.s.kv_heads];
    const int b = p / oasis::kBlock, j = p % oasis::kBlock;
    char* pg = static_cast<char*>(host_tier) + (static_cast<size_t>(u) * c.s.max_blocks + b) * c.page_elems * eb;
    const char* kr = static_cast<const char*>(k_new) + static_cast<size_t>(u) * d * eb;
    const char* vr = static_cast<const char*>(v_new) + static_cast<size_t>(u) * d * eb;
    memcpy(pg + static_cast<size_t>(j) * d * eb, kr, d * eb);
    char* vt = pg + static_cast<size_t>(oasis::kBlock) * d * eb;
    for (int ch = 0; ch < d; ++ch)
      memcpy(vt + (static_cast<size_t>(ch) * oasis::kBlock + j) * eb, vr + static_cast<size_t>(ch) * eb, eb);
  }
  return ok();
}

int oasis_block_meta_build(oasis_handle h, const void* pages, const int32_t* page_ids, int32_t count,
                           const int32_t* ctx_len, void* meta, void* pool,
                           const int32_t* block_to_slot, void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(pages);
  CHECK_PTR(ctx_len);
  CHECK_PTR(meta);
  CHECK_ALIGN16(pages);
  CHECK_ALIGN16(pool);
  const oasis::Ctx& c = h->c;
  if (count < 0) return fail(OASIS_EINVAL, "oasis_block_meta_build: count %d < 0", count);
  if (page_ids == nullptr && static_cast<long long>(count) != static_cast<long long>(c.units) * c.s.max_blocks)
    return fail(OASIS_EINVAL, "oasis_block_meta_build: without page_ids count must be B*H*max_blocks");
  if ((pool == nullptr) != (block_to_slot == nullptr))
    return fail(OASIS_EINVAL, "oasis_block_meta_build: pool and block_to_slot must both be set or both null");
  return hip_status(oasis::launch_meta_build(c, pages, page_ids, count, ctx_len, meta, pool, block_to_slot,
                                             static_cast<hipStream_t>(stream)),
                    "oasis_block_meta_build");
}

int oasis_block_meta_build_rows(oasis_handle h, const void* k_rows, int32_t tok_begin, int32_t tok_end,
                                const int32_t* ctx_len, void* meta, void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(k_rows);
  CHECK_PTR(ctx_len);
  CHECK_PTR(meta);
  CHECK_ALIGN16(k_rows);
  CHECK_ALIGN16(meta);
  const long long ntok = static_cast<long long>(h->c.s.max_blocks) * oasis::kBlock;
  if (tok_begin < 0 || tok_end < tok_begin || tok_end > ntok)
    return fail(OASIS_EINVAL, "oasis_block_meta_build_rows: token range [%d, %d) outside [0, %lld]", tok_begin,
                tok_end, ntok);
  return hip_status(oasis::launch_meta_rows(h->c, k_rows, tok_begin, tok_end, ctx_len, meta,
                                            static_cast<hipStream_t>(stream)),
                    "oasis_block_meta_build_rows");
}

int oasis_block_meta_export(oasis_handle h, const void* meta, void* meta_logical, void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(meta);
  CHECK_PTR(meta_logical);
  CHECK_ALIGN16(meta);
  CHECK_ALIGN16(meta_logical);
  if (meta == meta_logical) return fail(OASIS_EINVAL, "oasis_block_meta_export: in place is not supported");
  return hip_status(oasis::launch_meta_relayout(h->c, meta, meta_logical, true, static_cast<hipStream_t>(stream)),
                    "oasis_block_meta_export");
}

int oasis_block_meta_import(oasis_handle h, const void* meta_logical, void* meta, void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(meta_logical);
  CHECK_PTR(meta);
  CHECK_ALIGN16(meta);
  CHECK_ALIGN16(meta_logical);
  if (meta == meta_logical) return fail(OASIS_EINVAL, "oasis_block_meta_import: in place is not supported");
  return hip_status(oasis::launch_meta_relayout(h->c, meta_logical, meta, false, static_cast<hipStream_t>(stream)),
                    "oasis_block_meta_import");
}

int oasis_block_meta_update(oasis_handle h, const void* k_new, const void* v_new, const int32_t* ctx_len_in,
                            int32_t* ctx_len_out, void* meta, void* pool, const int32_t* block_to_slot,
                            void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(k_new);
  CHECK_PTR(v_new);
  CHECK_PTR(ctx_len_in);
  CHECK_PTR(ctx_len_out);
  CHECK_PTR(meta);
  CHECK_PTR(pool);
  CHECK_PTR(block_to_slot);
  if (static_cast<const void*>(ctx_len_in) == static_cast<const void*>(ctx_len_out))
    return fail(OASIS_EINVAL, "oasis_block_meta_update: ctx_len_out aliases ctx_len_in");
  return hip_status(oasis::launch_meta_update(h->c, k_new, v_new, ctx_len_in, ctx_len_out, meta, pool,
                                              block_to_slot, static_cast<hipStream_t>(stream)),
                    "oasis_block_meta_update");
}

int oasis_lookahead_score(oasis_handle h, const void* q, const void* meta, const int32_t* ctx_len,
                          float* scores, void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(q);
  CHECK_PTR(meta);
  CHECK_PTR(ctx_len);
  CHECK_PTR(scores);
  CHECK_ALIGN16(q);
  CHECK_ALIGN16(meta);
  return hip_status(oasis::launch_score(h->c, q, meta, ctx_len, scores, static_cast<hipStream_t>(stream)),
                    "oasis_lookahead_score");
}

int oasis_verify_score(oasis_handle h, const void* q, const void* meta, const int32_t* ctx_len, float* scores,
                       void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(q);
  CHECK_PTR(meta);
  CHECK_PTR(ctx_len);
  CHECK_PTR(scores);
  CHECK_ALIGN16(q);
  CHECK_ALIGN16(meta);
  return hip_status(oasis::launch_score(h->c, q, meta, ctx_len, scores, static_cast<hipStream_t>(stream), true),
                    "oasis_verify_score");
}

int oasis_topk_select(oasis_handle h, const float* scores, const int32_t* ctx_len, int32_t* sel,
                      void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(scores);
  CHECK_PTR(ctx_len);
  CHECK_PTR(sel);
  return hip_status(oasis::launch_topk(h->c, scores, ctx_len, sel, static_cast<hipStream_t>(stream)),
                    "oasis_topk_select");
}

#define CHECK_ATTEND_PAIR(fn, a, n)                                                                   \
  if (((a) == nullptr) != ((n) == nullptr))                                                           \
    return fail(OASIS_EINVAL, fn ": attend and n_attend must both be given or both be null");

int oasis_resident_diff_cap_evict(oasis_handle h, const int32_t* sel, const float* scores,
                                  int32_t* block_to_slot, int32_t* slot_to_block, int32_t* fetch,
                                  int32_t* n_fetch, int32_t* evict, int32_t* attend, int32_t* n_attend,
                                  void* stream) {
  CHECK_HANDLE(h);
  CHECK_ATTEND_PAIR("oasis_resident_diff_cap_evict", attend, n_attend);
  CHECK_PTR(sel);
  CHECK_PTR(scores);
  CHECK_PTR(block_to_slot);
  CHECK_PTR(slot_to_block);
  CHECK_PTR(n_fetch);
  if (h->c.s.fetch_cap > 0) {
    CHECK_PTR(fetch);
    CHECK_PTR(evict);
  }
  return hip_status(oasis::launch_diff(h->c, sel, scores, block_to_slot, slot_to_block, fetch, n_fetch,
                                       evict, attend, n_attend, static_cast<hipStream_t>(stream)),
                    "oasis_resident_diff_cap_evict");
}

int oasis_select_and_diff(oasis_handle h, const float* scores, const int32_t* ctx_len, int32_t* sel,
                          int32_t* block_to_slot, int32_t* slot_to_block, int32_t* fetch, int32_t* n_fetch,
                          int32_t* evict, int32_t* attend, int32_t* n_attend, void* stream) {
  CHECK_HANDLE(h);
  CHECK_ATTEND_PAIR("oasis_select_and_diff", attend, n_attend);
  CHECK_PTR(scores);
  CHECK_PTR(ctx_len);
  CHECK_PTR(sel);
  CHECK_PTR(block_to_slot);
  CHECK_PTR(slot_to_block);
  CHECK_PTR(n_fetch);
  if (h->c.s.fetch_cap > 0) {
    CHECK_PTR(fetch);
    CHECK_PTR(evict);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (oasis::select_diff_fused_available(h->c))
    return hip_status(oasis::launch_select_diff(h->c, scores, ctx_len, sel, block_to_slot, slot_to_block, fetch,
                                                n_fetch, evict, attend, n_attend, st),
                      "oasis_select_and_diff");
  hipError_t e = oasis::launch_topk(h->c, scores, ctx_len, sel, st);
  if (e == hipSuccess)
    e = oasis::launch_diff(h->c, sel, scores, block_to_slot, slot_to_block, fetch, n_fetch, evict, attend,
                           n_attend, st);
  return hip_status(e, "oasis_select_and_diff");
}

int oasis_fetch_issue(oasis_handle h, const void* host_tier, void* pool, const int32_t* fetch_host,
                      const int32_t* n_fetch_host, void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(host_tier);
  CHECK_PTR(pool);
  CHECK_PTR(n_fetch_host);
  const oasis::Ctx& c = h->c;
  const int cap = c.s.fetch_cap;
  if (cap > 0) CHECK_PTR(fetch_host);
  for (int u = 0; u < c.units; ++u) {
    const int nf = n_fetch_host[u];
    if (nf < 0 || nf > cap) return fail(OASIS_EINVAL, "oasis_fetch_issue: n_fetch %d of unit %d", nf, u);
    for (int i = 0; i < nf; ++i) {
      const int b = fetch_host[(static_cast<size_t>(u) * cap + i) * 2];
      const int s = fetch_host[(static_cast<size_t>(u) * cap + i) * 2 + 1];
      if (b < 0 || b >= c.s.max_blocks || s < 0 || s >= c.s.budget_blocks)
        return fail(OASIS_EINVAL, "oasis_fetch_issue: entry (%d, %d) of unit %d out of range", b, s, u);
    }
  }
  const size_t pb = c.page_elems * c.elem_bytes;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int u = 0; u < c.units; ++u) {
    const int nf = n_fetch_host[u];
    for (int i = 0; i < nf; ++i) {
      const int b = fetch_host[(static_cast<size_t>(u) * cap + i) * 2];
      const int s = fetch_host[(static_cast<size_t>(u) * cap + i) * 2 + 1];
      const char* src = static_cast<const char*>(host_tier) + (static_cast<size_t>(u) * c.s.max_blocks + b) * pb;
      char* dst = static_cast<char*>(pool) + (static_cast<size_t>(u) * c.s.budget_blocks + s) * pb;
      const hipError_t e = hipMemcpyAsync(dst, src, pb, hipMemcpyHostToDevice, st);
      if (e != hipSuccess) return hip_status(e, "oasis_fetch_issue: hipMemcpyAsync");
    }
  }
  return ok();
}

int oasis_sparse_paged_decode_attn(oasis_handle h, const void* q, const void* pool, const int32_t* sel,
                                   const int32_t* block_to_slot, const int32_t* ctx_len, float* out,
                                   void* workspace, void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(q);
  CHECK_PTR(pool);
  CHECK_PTR(sel);
  CHECK_PTR(block_to_slot);
  CHECK_PTR(ctx_len);
  CHECK_PTR(out);
  CHECK_PTR(workspace);
  CHECK_ALIGN16(q);
  CHECK_ALIGN16(pool);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(OASIS_EINVAL, "oasis_sparse_paged_decode_attn: workspace not 256-byte aligned");
  return hip_status(oasis::launch_attn(h->c, q, pool, sel, block_to_slot, nullptr, nullptr, ctx_len, out,
                                       workspace, static_cast<hipStream_t>(stream)),
                    "oasis_sparse_paged_decode_attn");
}

int oasis_sparse_paged_decode_attn_noalloc(oasis_handle h, const void* q, const void* pool, const int32_t* sel,
                                           const int32_t* block_to_slot, const int32_t* ctx_len, float* out,
                                           void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(q);
  CHECK_PTR(pool);
  CHECK_PTR(sel);
  CHECK_PTR(block_to_slot);
  CHECK_PTR(ctx_len);
  CHECK_PTR(out);
  CHECK_ALIGN16(q);
  CHECK_ALIGN16(pool);
  const size_t need = oasis::attn_workspace_bytes(h->c);
  if (need > oasis::attn_scratch_bytes())
    return fail(OASIS_EINVAL,
                "oasis_sparse_paged_decode_attn_noalloc: the shape needs %zu bytes of workspace, more than the "
                "%zu-byte scratch (use oasis_sparse_paged_decode_attn with a workspace)",
                need, oasis::attn_scratch_bytes());
  return hip_status(oasis::launch_attn_noalloc(h->c, q, pool, sel, block_to_slot, ctx_len, out,
                                               static_cast<hipStream_t>(stream)),
                    "oasis_sparse_paged_decode_attn_noalloc");
}

int oasis_sparse_paged_decode_attn_list(oasis_handle h, const void* q, const void* pool, const int32_t* attend,
                                        const int32_t* n_attend, const int32_t* ctx_len, float* out,
                                        void* workspace, void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(q);
  CHECK_PTR(pool);
  CHECK_PTR(attend);
  CHECK_PTR(n_attend);
  CHECK_PTR(ctx_len);
  CHECK_PTR(out);
  CHECK_PTR(workspace);
  CHECK_ALIGN16(q);
  CHECK_ALIGN16(pool);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(OASIS_EINVAL, "oasis_sparse_paged_decode_attn_list: workspace not 256-byte aligned");
  return hip_status(oasis::launch_attn(h->c, q, pool, nullptr, nullptr, attend, n_attend, ctx_len, out,
                                       workspace, static_cast<hipStream_t>(stream)),
                    "oasis_sparse_paged_decode_attn_list");
}

int oasis_admit(oasis_handle h, const void* k_rows, const void* v_rows, const int32_t* ctx_len, void* host_tier,
                void* meta, void* pool, const int32_t* block_to_slot, void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(k_rows);
  CHECK_PTR(v_rows);
  CHECK_PTR(ctx_len);
  CHECK_PTR(host_tier);
  CHECK_PTR(meta);
  CHECK_ALIGN16(k_rows);
  CHECK_ALIGN16(host_tier);
  if ((pool == nullptr) != (block_to_slot == nullptr))
    return fail(OASIS_EINVAL, "oasis_admit: pool and block_to_slot must both be given or both be null");
  if (pool != nullptr) CHECK_ALIGN16(pool);
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, host_tier) != hipSuccess || attr.type != hipMemoryTypeHost ||
      attr.devicePointer == nullptr) {
    (void)hipGetLastError();  // clear the lookup's error state
    return fail(OASIS_EINVAL, "oasis_admit: host_tier is not pinned host memory mapped for the device");
  }
  return hip_status(oasis::launch_admit(h->c, k_rows, v_rows, ctx_len, attr.devicePointer, meta, pool, block_to_slot,
                                        static_cast<hipStream_t>(stream)),
                    "oasis_admit");
}

int oasis_fetch_gather(oasis_handle h, const void* host_tier, void* pool, const int32_t* fetch,
                       const int32_t* n_fetch, void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(host_tier);
  CHECK_PTR(pool);
  CHECK_PTR(n_fetch);
  CHECK_ALIGN16(host_tier);
  CHECK_ALIGN16(pool);
  const oasis::Ctx& c = h->c;
  if (c.s.fetch_cap > 0) CHECK_PTR(fetch);
  // The kernel dereferences the host tier: it must be pinned host memory mapped
  // into the device's address space (hipHostMalloc).
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, host_tier) != hipSuccess || attr.type != hipMemoryTypeHost ||
      attr.devicePointer == nullptr) {
    (void)hipGetLastError();  // clear the lookup's error state
    return fail(OASIS_EINVAL, "oasis_fetch_gather: host_tier is not pinned host memory mapped for the device");
  }
  return hip_status(oasis::launch_fetch_gather(c, attr.devicePointer, pool, fetch, n_fetch,
                                               static_cast<hipStream_t>(stream)),
                    "oasis_fetch_gather");
}

int oasis_attend_and_score(oasis_handle h, const void* q, const void* pool, const void* meta,
                           const int32_t* ctx_attn, const int32_t* ctx_score, const int32_t* sel,
                           const int32_t* block_to_slot, const int32_t* attend, const int32_t* n_attend,
                           float* scores, float* out, void* workspace, void* stream) {
  CHECK_HANDLE(h);
  CHECK_ATTEND_PAIR("oasis_attend_and_score", attend, n_attend);
  CHECK_PTR(q);
  CHECK_PTR(pool);
  CHECK_PTR(meta);
  CHECK_PTR(ctx_attn);
  CHECK_PTR(ctx_score);
  CHECK_PTR(scores);
  CHECK_PTR(out);
  CHECK_PTR(workspace);
  if (attend == nullptr) {
    CHECK_PTR(sel);
    CHECK_PTR(block_to_slot);
  }
  CHECK_ALIGN16(q);
  CHECK_ALIGN16(pool);
  CHECK_ALIGN16(meta);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(OASIS_EINVAL, "oasis_attend_and_score: workspace not 256-byte aligned");
  const oasis::Ctx& c = h->c;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the fp32 reference path attends from the maps when they are given
  const bool list = attend != nullptr && (c.s.dtype == OASIS_BF16 || sel == nullptr);
  hipError_t e;
  if (oasis::attn_and_score_fused_available(c) && c.step_launches == 2) {
    e = oasis::launch_attn_and_score(c, q, pool, sel, block_to_slot, list ? attend : nullptr,
                                     list ? n_attend : nullptr, ctx_attn, out, workspace, meta, ctx_score, scores,
                                     st);
  } else {
    e = oasis::launch_attn_main(c, q, pool, sel, block_to_slot, list ? attend : nullptr, list ? n_attend : nullptr,
                                ctx_attn, out, workspace, st);
    if (e == hipSuccess) e = oasis::launch_score(c, q, meta, ctx_score, scores, st);
  }
  return hip_status(e, "oasis_attend_and_score");
}

int oasis_attn_combine(oasis_handle h, void* workspace, float* out, void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(workspace);
  CHECK_PTR(out);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(OASIS_EINVAL, "oasis_attn_combine: workspace not 256-byte aligned");
  return hip_status(oasis::launch_attn_combine(h->c, workspace, out, static_cast<hipStream_t>(stream)),
                    "oasis_attn_combine");
}

int oasis_select_and_diff_lru(oasis_handle h, const float* scores, const int32_t* ctx_len, int32_t* sel,
                              int32_t* block_to_slot, int32_t* slot_to_block, int32_t* slot_last_use, int32_t step,
                              int32_t* fetch, int32_t* n_fetch, int32_t* evict, int32_t* attend, int32_t* n_attend,
                              void* stream) {
  CHECK_HANDLE(h);
  CHECK_ATTEND_PAIR("oasis_select_and_diff_lru", attend, n_attend);
  CHECK_PTR(scores);
  CHECK_PTR(ctx_len);
  CHECK_PTR(sel);
  CHECK_PTR(block_to_slot);
  CHECK_PTR(slot_to_block);
  CHECK_PTR(slot_last_use);
  CHECK_PTR(n_fetch);
  if (h->c.s.fetch_cap > 0) {
    CHECK_PTR(fetch);
    CHECK_PTR(evict);
  }
  if (!oasis::select_diff_lru_available(h->c))
    return fail(OASIS_EUNSUPPORTED, "oasis_select_and_diff_lru: needs budget_blocks <= 128 and max_blocks <= 8192");
  return hip_status(oasis::launch_select_diff(h->c, scores, ctx_len, sel, block_to_slot, slot_to_block, fetch, n_fetch,
                                              evict, attend, n_attend, static_cast<hipStream_t>(stream),
                                              oasis::LruState{slot_last_use, step}),
                    "oasis_select_and_diff_lru");
}

int oasis_select_diff_combine_lru(oasis_handle h, const float* scores, const int32_t* ctx_score, int32_t* sel,
                                  int32_t* block_to_slot, int32_t* slot_to_block, int32_t* slot_last_use,
                                  int32_t step, int32_t* fetch, int32_t* n_fetch, int32_t* evict, int32_t* attend,
                                  int32_t* n_attend, float* out, void* workspace, void* stream) {
  CHECK_HANDLE(h);
  CHECK_ATTEND_PAIR("oasis_select_diff_combine_lru", attend, n_attend);
  CHECK_PTR(scores);
  CHECK_PTR(ctx_score);
  CHECK_PTR(sel);
  CHECK_PTR(block_to_slot);
  CHECK_PTR(slot_to_block);
  CHECK_PTR(slot_last_use);
  CHECK_PTR(n_fetch);
  CHECK_PTR(out);
  CHECK_PTR(workspace);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(OASIS_EINVAL, "oasis_select_diff_combine_lru: workspace not 256-byte aligned");
  const oasis::Ctx& c = h->c;
  if (c.s.fetch_cap > 0) {
    CHECK_PTR(fetch);
    CHECK_PTR(evict);
  }
  if (!oasis::select_diff_lru_available(c))
    return fail(OASIS_EUNSUPPORTED,
                "oasis_select_diff_combine_lru: needs budget_blocks <= 128 and max_blocks <= 8192");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const oasis::LruState lru{slot_last_use, step};
  hipError_t e;
  if (oasis::attn_needs_combine(c)) {
    e = oasis::launch_select_diff_combine(c, scores, ctx_score, sel, block_to_slot, slot_to_block, fetch, n_fetch,
                                          evict, attend, n_attend, workspace, out, st, lru);
  } else {
    e = oasis::launch_select_diff(c, scores, ctx_score, sel, block_to_slot, slot_to_block, fetch, n_fetch, evict,
                                  attend, n_attend, st, lru);
  }
  return hip_status(e, "oasis_select_diff_combine_lru");
}

int oasis_select_diff_combine(oasis_handle h, const float* scores, const int32_t* ctx_score, int32_t* sel,
                              int32_t* block_to_slot, int32_t* slot_to_block, int32_t* fetch, int32_t* n_fetch,
                              int32_t* evict, int32_t* attend, int32_t* n_attend, float* out, void* workspace,
                              void* stream) {
  CHECK_HANDLE(h);
  CHECK_ATTEND_PAIR("oasis_select_diff_combine", attend, n_attend);
  CHECK_PTR(scores);
  CHECK_PTR(ctx_score);
  CHECK_PTR(sel);
  CHECK_PTR(block_to_slot);
  CHECK_PTR(slot_to_block);
  CHECK_PTR(n_fetch);
  CHECK_PTR(out);
  CHECK_PTR(workspace);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(OASIS_EINVAL, "oasis_select_diff_combine: workspace not 256-byte aligned");
  const oasis::Ctx& c = h->c;
  if (c.s.fetch_cap > 0) {
    CHECK_PTR(fetch);
    CHECK_PTR(evict);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (oasis::select_diff_fused_available(c) && oasis::attn_needs_combine(c)) {
    e = oasis::launch_select_diff_combine(c, scores, ctx_score, sel, block_to_slot, slot_to_block, fetch, n_fetch,
                                          evict, attend, n_attend, workspace, out, st);
  } else {
    e = oasis::launch_attn_combine(c, workspace, out, st);
    if (e == hipSuccess) {
      if (oasis::select_diff_fused_available(c)) {
        e = oasis::launch_select_diff(c, scores, ctx_score, sel, block_to_slot, slot_to_block, fetch, n_fetch, evict,
                                      attend, n_attend, st);
      } else {
        e = oasis::launch_topk(c, scores, ctx_score, sel, st);
        if (e == hipSuccess)
          e = oasis::launch_diff(c, sel, scores, block_to_slot, slot_to_block, fetch, n_fetch, evict, attend,
                                 n_attend, st);
      }
    }
  }
  return hip_status(e, "oasis_select_diff_combine");
}

}  // extern "C"

namespace {

// The decode step of one layer, optionally carrying another layer's transfer
// (g.host != nullptr) in its first launch; arguments already validated.
// ap: a token append the step carries (its scoring then reads the grown
// context ctx_score = ap->ctx_out): where the attention (bf16, its output
// written without a combine) and the scoring are launches of their own, the
// attention launch updates the token's metadata row and the scoring launch
// writes its page row, one workgroup per unit each; otherwise the append
// kernel runs first.
hipError_t decode_step_impl(const oasis::Ctx& c, const void* q, const void* pool, const void* meta,
                            const int32_t* ctx_attn, const int32_t* ctx_score, int32_t* sel, int32_t* block_to_slot,
                            int32_t* slot_to_block, float* scores, float* out, void* workspace, int32_t* fetch,
                            int32_t* n_fetch, int32_t* evict, int32_t* attend, int32_t* n_attend,
                            const oasis::StepGather& g, hipStream_t st, const oasis::StepAppend* ap = nullptr) {
  hipError_t e;
  if (oasis::attn_needs_combine(c) && oasis::attn_and_score_fused_available(c) &&
      oasis::select_diff_fused_available(c) && c.step_launches == 2) {
    // two launches: (the carried transfer,) attention + scoring, then selection + diff + split combine;
    // the scoring reads the appended token's metadata, so an append goes first
    if (ap != nullptr) {
      e = oasis::launch_meta_update(c, ap->k_new, ap->v_new, ap->ctx_in, ap->ctx_out, ap->meta, ap->pool, ap->b2s,
                                    st);
      if (e != hipSuccess) return e;
    }
    e = oasis::launch_attn_and_score(c, q, pool, sel, block_to_slot, attend, n_attend, ctx_attn, out, workspace,
                                     meta, ctx_score, scores, st, g);
    if (e != hipSuccess) return e;
    if (c.attn_merge)  // the first launch merged the splits
      return oasis::launch_select_diff(c, scores, ctx_score, sel, block_to_slot, slot_to_block, fetch, n_fetch, evict,
                                       attend, n_attend, st);
    return oasis::launch_select_diff_combine(c, scores, ctx_score, sel, block_to_slot, slot_to_block, fetch, n_fetch,
                                             evict, attend, n_attend, workspace, out, st);
  }
  // other shapes: the carried transfer as its own launch first
  if (g.host != nullptr) {
    e = oasis::launch_fetch_gather(c, g.host, g.pool, g.fetch, g.n_fetch, st);
    if (e != hipSuccess) return e;
  }
  const bool attn_alone = !(c.s.dtype == OASIS_BF16 && oasis::attn_needs_combine(c));
  const oasis::StepAppend* ride = (ap != nullptr && c.s.dtype == OASIS_BF16 && attn_alone) ? ap : nullptr;
  if (ap != nullptr && ride == nullptr) {
    e = oasis::launch_meta_update(c, ap->k_new, ap->v_new, ap->ctx_in, ap->ctx_out, ap->meta, ap->pool, ap->b2s, st);
    if (e != hipSuccess) return e;
  }
  if (!attn_alone) {
    e = oasis::launch_attn_main(c, q, pool, sel, block_to_slot, attend, n_attend, ctx_attn, out, workspace, st);
    if (e == hipSuccess) e = oasis::launch_combine_and_score(c, workspace, out, q, meta, ctx_score, scores, st);
  } else {
    // the fp32 reference path attends from the maps (the list splits differently)
    e = oasis::launch_attn(c, q, pool, sel, block_to_slot, c.s.dtype == OASIS_BF16 ? attend : nullptr,
                           c.s.dtype == OASIS_BF16 ? n_attend : nullptr, ctx_attn, out, workspace, st, ride);
    if (e == hipSuccess) e = oasis::launch_score(c, q, meta, ctx_score, scores, st, false, ride);
  }
  if (e == hipSuccess) {
    if (oasis::select_diff_fused_available(c)) {
      e = oasis::launch_select_diff(c, scores, ctx_score, sel, block_to_slot, slot_to_block, fetch, n_fetch, evict,
                                    attend, n_attend, st);
    } else {
      e = oasis::launch_topk(c, scores, ctx_score, sel, st);
      if (e == hipSuccess)
        e = oasis::launch_diff(c, sel, scores, block_to_slot, slot_to_block, fetch, n_fetch, evict, attend, n_attend,
                               st);
    }
  }
  return e;
}

#define CHECK_DECODE_STEP_ARGS(fn)                                                              \
  CHECK_HANDLE(h);                                                                              \
  CHECK_ATTEND_PAIR(fn, attend, n_attend);                                                      \
  CHECK_PTR(q);                                                                                 \
  CHECK_PTR(pool);                                                                              \
  CHECK_PTR(meta);                                                                              \
  CHECK_PTR(ctx_attn);                                                                          \
  CHECK_PTR(ctx_score);                                                                         \
  CHECK_PTR(sel);                                                                               \
  CHECK_PTR(block_to_slot);                                                                     \
  CHECK_PTR(slot_to_block);                                                                     \
  CHECK_PTR(scores);                                                                            \
  CHECK_PTR(out);                                                                               \
  CHECK_PTR(workspace);                                                                         \
  CHECK_PTR(n_fetch);                                                                           \
  CHECK_ALIGN16(q);                                                                             \
  CHECK_ALIGN16(pool);                                                                          \
  CHECK_ALIGN16(meta);                                                                          \
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)                                        \
    return fail(OASIS_EINVAL, fn ": workspace not 256-byte aligned");                           \
  if (h->c.s.fetch_cap > 0) {                                                                   \
    CHECK_PTR(fetch);                                                                           \
    CHECK_PTR(evict);                                                                           \
  }

// Another layer's transfer for a step's first launch (none when transfer is
// NULL or the cap is 0): checks and resolves the host tier's device mapping.
int resolve_transfer(oasis_handle h, const void* pool, const oasis_transfer* transfer, oasis::StepGather* g,
                     const char* fn) {
  if (transfer == nullptr || h->c.s.fetch_cap == 0) return OASIS_OK;
  CHECK_PTR(transfer->host_tier);
  CHECK_PTR(transfer->pool);
  CHECK_PTR(transfer->fetch);
  CHECK_PTR(transfer->n_fetch);
  CHECK_ALIGN16(transfer->host_tier);
  CHECK_ALIGN16(transfer->pool);
  if (transfer->pool == pool) return fail(OASIS_EINVAL, "%s: the transfer's pool is this step's pool", fn);
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, transfer->host_tier) != hipSuccess || attr.type != hipMemoryTypeHost ||
      attr.devicePointer == nullptr) {
    (void)hipGetLastError();  // clear the lookup's error state
    return fail(OASIS_EINVAL, "%s: host_tier is not pinned host memory mapped for the device", fn);
  }
  g->host = static_cast<const uint4*>(attr.devicePointer);
  g->pool = static_cast<uint4*>(transfer->pool);
  g->fetch = transfer->fetch;
  g->n_fetch = transfer->n_fetch;
  g->cap = h->c.s.fetch_cap;
  return OASIS_OK;
}

}  // namespace

extern "C" {

int oasis_decode_step_carry(oasis_handle h, const void* q, const void* pool, const void* meta,
                            const int32_t* ctx_attn, const int32_t* ctx_score, const int32_t* attend,
                            const int32_t* n_attend, float* scores, float* out, void* workspace,
                            const oasis_select_job* job, const oasis_transfer* transfer, void* stream) {
  CHECK_HANDLE(h);
  CHECK_PTR(q);
  CHECK_PTR(pool);
  CHECK_PTR(meta);
  CHECK_PTR(ctx_attn);
  CHECK_PTR(ctx_score);
  CHECK_PTR(attend);
  CHECK_PTR(n_attend);
  CHECK_PTR(scores);
  CHECK_PTR(out);
  CHECK_PTR(workspace);
  CHECK_ALIGN16(q);
  CHECK_ALIGN16(pool);
  CHECK_ALIGN16(meta);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(OASIS_EINVAL, "oasis_decode_step_carry: workspace not 256-byte aligned");
  if (!oasis::attn_score_select_available(h->c))
    return fail(OASIS_EUNSUPPORTED,
                "oasis_decode_step_carry: needs bf16, head_dim 128, 2 attention wavefronts, k <= 128 "
                "and max_blocks <= 8192");
  oasis::SelectJob sj;
  if (job != nullptr) {
    CHECK_PTR(job->scores);
    CHECK_PTR(job->ctx_len);
    CHECK_PTR(job->sel);
    CHECK_PTR(job->block_to_slot);
    CHECK_PTR(job->slot_to_block);
    CHECK_PTR(job->n_fetch);
    CHECK_PTR(job->attend);
    CHECK_PTR(job->n_attend);
    if (h->c.s.fetch_cap > 0) {
      CHECK_PTR(job->fetch);
      CHECK_PTR(job->evict);
    }
    // the carried diff must not touch what this launch reads or writes
    if (job->scores == scores || job->attend == attend || job->n_attend == n_attend)
      return fail(OASIS_EINVAL, "oasis_decode_step_carry: the carried selection is this step's own state");
    sj.scores = job->scores;
    sj.ctx_len = job->ctx_len;
    sj.sel = job->sel;
    sj.b2s = job->block_to_slot;
    sj.s2b = job->slot_to_block;
    sj.fetch = job->fetch;
    sj.n_fetch = job->n_fetch;
    sj.evict = job->evict;
    sj.attend = job->attend;
    sj.n_attend = job->n_attend;
  }
  oasis::StepGather g;
  const int rc = resolve_transfer(h, pool, transfer, &g, "oasis_decode_step_carry");
  if (rc != OASIS_OK) return rc;
  if (job != nullptr && g.host != nullptr && (job->fetch == g.fetch || job->n_fetch == g.n_fetch))
    return fail(OASIS_EINVAL, "oasis_decode_step_carry: the transfer reads the fetch list the carried diff writes");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  oasis::Ctx c = h->c;
  c.attn_merge = c.attn_merge_carry;  // the carried step's own choice
  hipError_t e = oasis::launch_attn_score_select(c, q, pool, attend, n_attend, ctx_attn, out, workspace, meta,
                                                 ctx_score, scores, job != nullptr ? &sj : nullptr, st, g);
  if (e == hipSuccess && !c.attn_merge) e = oasis::launch_attn_combine(c, workspace, out, st);
  return hip_status(e, "oasis_decode_step_carry");
}

int oasis_decode_step(oasis_handle h, const void* q, const void* pool, const void* meta,
                      const int32_t* ctx_attn, const int32_t* ctx_score, int32_t* sel, int32_t* block_to_slot,
                      int32_t* slot_to_block, float* scores, float* out, void* workspace, int32_t* fetch,
                      int32_t* n_fetch, int32_t* evict, int32_t* attend, int32_t* n_attend, void* stream) {
  CHECK_DECODE_STEP_ARGS("oasis_decode_step");
  return hip_status(decode_step_impl(h->c, q, pool, meta, ctx_attn, ctx_score, sel, block_to_slot, slot_to_block,
                                     scores, out, workspace, fetch, n_fetch, evict, attend, n_attend,
                                     oasis::StepGather(), static_cast<hipStream_t>(stream)),
                    "oasis_decode_step");
}

int oasis_decode_step_append(oasis_handle h, const void* q, void* pool, void* meta, const int32_t* ctx_in,
                             int32_t* ctx_out, int32_t* sel, int32_t* block_to_slot, int32_t* slot_to_block,
                             float* scores, float* out, void* workspace, int32_t* fetch, int32_t* n_fetch,
                             int32_t* evict, int32_t* attend, int32_t* n_attend, const void* k_new,
                             const void* v_new, void* stream) {
  const int32_t* ctx_attn = ctx_in;
  const int32_t* ctx_score = ctx_out;
  CHECK_DECODE_STEP_ARGS("oasis_decode_step_append");
  CHECK_PTR(k_new);
  CHECK_PTR(v_new);
  if (static_cast<const void*>(ctx_in) == static_cast<const void*>(ctx_out))
    return fail(OASIS_EINVAL, "oasis_decode_step_append: ctx_out aliases ctx_in");
  oasis::StepAppend ap;
  ap.k_new = k_new;
  ap.v_new = v_new;
  ap.ctx_in = ctx_in;
  ap.ctx_out = ctx_out;
  ap.meta = meta;
  ap.pool = pool;
  ap.b2s = block_to_slot;
  return hip_status(decode_step_impl(h->c, q, pool, meta, ctx_attn, ctx_score, sel, block_to_slot, slot_to_block,
                                     scores, out, workspace, fetch, n_fetch, evict, attend, n_attend,
                                     oasis::StepGather(), static_cast<hipStream_t>(stream), &ap),
                    "oasis_decode_step_append");
}

int oasis_decode_step_gather(oasis_handle h, const void* q, const void* pool, const void* meta,
                             const int32_t* ctx_attn, const int32_t* ctx_score, int32_t* sel, int32_t* block_to_slot,
                             int32_t* slot_to_block, float* scores, float* out, void* workspace, int32_t* fetch,
                             int32_t* n_fetch, int32_t* evict, int32_t* attend, int32_t* n_attend,
                             const oasis_transfer* transfer, void* stream) {
  CHECK_DECODE_STEP_ARGS("oasis_decode_step_gather");
  oasis::StepGather g;
  const int rc = resolve_transfer(h, pool, transfer, &g, "oasis_decode_step_gather");
  if (rc != OASIS_OK) return rc;
  return hip_status(decode_step_impl(h->c, q, pool, meta, ctx_attn, ctx_score, sel, block_to_slot, slot_to_block,
                                     scores, out, workspace, fetch, n_fetch, evict, attend, n_attend, g,
                                     static_cast<hipStream_t>(stream)),
                    "oasis_decode_step_gather");
}

}  // extern "C"
