/*
 * oasiskv.h - C ABI of the lookahead sparse-KV decode step for AMD MI355X (gfx950).
 *
 * The per-decode-step hot path of OasisKV's lookahead sparse prefetching, as
 * described by the OasisKV pages:
 *   [EXPL]  METAL MEDIA explainer "OasisKV: Scaling In-Decode KV Cache Beyond
 *           HBM with Lookahead Sparse Prefetching" (arXiv 2608.08097)
 *   [INDEX] mlsanity.com index entry for the same paper ("Builds on" list)
 * Per layer and step: sparse attention of the verify and draft queries over
 * the resident selected KV blocks ([EXPL] Figure 7 right), lookahead scoring of
 * every block from the draft queries against per-block key min/max metadata
 * ([EXPL] Figure 7), top-k selection with the sink and newest block kept,
 * the set difference against the head-wise resident map with a per-step fetch
 * cap and capped eviction ([EXPL] "What they did" item 3, Table 2, Figure 9),
 * and the transfer of the missing blocks from the host tier ([EXPL] Figure 8).
 *
 * Conventions
 *  - Unit = one (request r, KV head h) of one layer; unit index u = r*H + h.
 *    Pointers are per layer: the caller offsets by layer.
 *  - Query head hq = h*G + g serves KV head h (consecutive GQA grouping, [INDEX]
 *    cites GQA).  Queries q are [B][H*G][T][d] with T = 1 + n_draft: row t = 0 is
 *    the verify query, rows 1..n_draft the draft queries of the step.
 *  - Element type (OASIS_BF16 or OASIS_F32) applies to q, block metadata, K/V
 *    pages and appended tokens; scores and attention output are float32.
 *  - Block metadata "meta": per block a row of 2*d elements, the per-channel
 *    key min of the block then the per-channel key max.  Stored per (request,
 *    KV head) in ceil(max_blocks/16) tiles of 16 blocks; inside a tile the rows
 *    are cut into 16-byte chunks stored chunk-major (chunk c of block 16t + j at
 *    chunk position 16c + j), so that each MFMA k-step of the scoring reads one
 *    contiguous KiB.  oasis_block_meta_export / _import convert it to and from
 *    the logical layout [B][H][max_blocks][2][d].
 *  - Page = one block of one unit: K rows [16][d] (token-major) followed by V
 *    transposed [d][16] (channel-major), 2*16*d elements.  The host tier is
 *    [B][H][max_blocks][page] (pinned host memory); the HBM pool is
 *    [B][H][budget_blocks][page]; slot s of unit u is page u*budget_blocks + s.
 *  - Resident maps: slot_to_block [B][H][budget_blocks] and block_to_slot
 *    [B][H][max_blocks], int32, -1 = none; they are kept mutually inverse.
 *  - ctx_len [B] (device, int32): context length per request.  Precondition,
 *    not checked on the host: 1 <= ctx_len[r] <= max_blocks*16 (and < for the
 *    append call).  N = ceil(ctx_len / 16) blocks.
 *  - Ownership: the caller allocates and owns every buffer; the library never
 *    allocates device or host memory.  The handle stores shapes only and is
 *    immutable after creation (safe to share between threads).
 *  - Asynchrony: device entry points only enqueue work on `stream` (a
 *    hipStream_t passed as void*, NULL = default stream) and return.
 *  - Errors: every call returns OASIS_OK or a negative status.  Arguments are
 *    validated before anything is enqueued, so a failed call leaves no partial
 *    work.  oasis_last_error() returns the calling thread's last message.
 */
#ifndef OASISKV_H
#define OASISKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OASIS_OK 0
#define OASIS_EINVAL (-1)        /* null pointer, bad shape field, bad list entry */
#define OASIS_EHIP (-2)          /* a HIP runtime call failed (message kept) */
#define OASIS_EUNSUPPORTED (-3)  /* dtype / head_dim / block_size / row count not built */

#define OASIS_F32 0
#define OASIS_BF16 1

typedef struct oasis_shape {
  int32_t batch;          /* B requests */
  int32_t kv_heads;       /* H */
  int32_t group;          /* G query heads per KV head */
  int32_t head_dim;       /* d: 64 or 128 */
  int32_t block_size;     /* tokens per block: must be 16 */
  int32_t max_blocks;     /* N_max: blocks allocated per unit (context capacity / 16) */
  int32_t budget_blocks;  /* k: selected blocks = HBM slots per unit, 2..1024 */
  int32_t n_draft;        /* D draft queries per step, >= 1 */
  int32_t fetch_cap;      /* blocks fetched per unit per step, >= 0 */
  int32_t dtype;          /* OASIS_BF16 or OASIS_F32 */
} oasis_shape;

typedef struct oasis_ctx* oasis_handle;

/*
 * Launch shapes of the kernels (performance only: every choice computes the
 * same selections, lists and maps; attention outputs differ only by the order
 * of fp32 sums where the split of the attended list changes).  A field left 0
 * takes the default, which the library picks from the shape.
 */
typedef struct oasis_launch_options {
  int32_t attn_waves;     /* wavefronts per attention workgroup: 0, 1, 2 or 4 (default 2;
                             at most 2 with more than 32 attention rows) */
  int32_t attn_pf;        /* pages in flight per attention wavefront: 0, 2, 4 or 8 (default 2;
                             4 for the attention as a launch of its own when it runs one
                             split of 64-block runs per unit at one wavefront per SIMD;
                             capped by the registers the row count needs) */
  int32_t attn_splits;    /* attention workgroups per unit, 0..32 (default: about 512
                             attention wavefronts per launch, beside the scoring fewer
                             where the attention moves under half of that launch's bytes;
                             bounded so that a wavefront streams at most 64 blocks) */
  int32_t score_tpw;      /* 16-block tiles per scoring wavefront, 0..64 (default: about
                             4096 scoring wavefronts beside the attention, 2048 alone) */
  int32_t step_order;     /* workgroup order of the step's first launch: 0 attention first
                             (default), 1 scoring first, 2 interleaved */
  int32_t step_launches;  /* launches per oasis_decode_step: 0 or 2 (attention beside the
                             scoring; selection + diff + split combine), or 3 (attention;
                             combine + scoring; selection + diff) */
  int32_t attn_merge;     /* where the attention's split partials are merged in the steps whose
                             first launch runs the attention beside the scoring: 1 by a combine
                             after that launch (the two-launch step's second launch, the carried
                             step's combine launch); 2 inside that launch in both steps (the
                             last workgroup of each request and KV head to finish merges; only
                             with 2 to 8 splits, else as 1); 3 inside it in the carried step
                             only; 0 default: 1.  The outputs are bit-identical either way. */
} oasis_launch_options;

/* Validates the shape (EINVAL / EUNSUPPORTED) and returns a handle with the
 * default launch options.  No HIP call. */
int oasis_create(const oasis_shape* shape, oasis_handle* out);
/* The same with explicit launch options (opts may be NULL = all defaults);
 * EINVAL on a field outside the ranges above.  The handle stays immutable. */
int oasis_create_with_options(const oasis_shape* shape, const oasis_launch_options* opts,
                              oasis_handle* out);
/* The launch options a handle uses, defaults and caps resolved (score_tpw is
 * the value beside the attention). */
int oasis_get_launch_options(oasis_handle h, oasis_launch_options* out);
int oasis_destroy(oasis_handle h);
/* Last error message of the calling thread ("" if none). */
const char* oasis_last_error(void);
/* ABI version of this library. */
int oasis_version(void);

/* Byte sizes of the caller-allocated buffers of one layer (0 on a bad handle). */
size_t oasis_page_bytes(oasis_handle h);       /* one page: 2*16*d elements */
size_t oasis_meta_bytes(oasis_handle h);       /* B*H*ceil(max_blocks/16)*16*2*d elements */
size_t oasis_pool_bytes(oasis_handle h);       /* B*H*budget_blocks pages */
size_t oasis_host_tier_bytes(oasis_handle h);  /* B*H*max_blocks pages */
/* The attention's workspace (device, 256-byte aligned): its split partials,
 * then one int32 arrival counter per (request, KV head) for the split merge
 * inside the first launch (attn_merge).  Zero the workspace once before its
 * first use; every call leaves the counters zero again. */
size_t oasis_workspace_bytes(oasis_handle h);

/*
 * Host-side page packing (no device work).  Writes n_blocks blocks of unit u
 * into the page layout at `pages` ([B][H][max_blocks][page], host memory).
 * k, v: source rows [n_blocks][16][d] (token-major, element type); either may
 * be NULL to leave that half of the pages unchanged.  blocks: destination
 * block indices [n_blocks] (NULL = 0 .. n_blocks-1).  EINVAL on an index out of
 * range.  This is how the prefill fills the host tier ([EXPL] Figure 7 left:
 * the full KV cache lives in CPU memory).
 */
int oasis_pack_pages(oasis_handle h, const void* k, const void* v, const int32_t* blocks,
                     int32_t n_blocks, int32_t unit, void* pages);

/*
 * Host-side append of one token per unit into the host tier (no device work).
 * k_new, v_new: [B][H][d] host; pos: [B] host, token position per request
 * (= context length before the append).  EINVAL if a position is out of range.
 */
int oasis_host_tier_append(oasis_handle h, const void* k_new, const void* v_new,
                           const int32_t* pos, void* host_tier);

/*
 * Block metadata build (prefill, and rebuild after keys change).  For each of
 * `count` staged pages (device, [count][page]): the page is block b of unit u,
 * id = page_ids[i] = u*max_blocks + b (page_ids NULL: the staged pages are the
 * whole layer, count = B*H*max_blocks, id = i).  Writes meta rows of blocks
 * b < N(ctx_len) as the min and max over the block's tokens below ctx_len
 * ([EXPL] Figure 7 left: per-block min/max pooling).  If pool and
 * block_to_slot are non-NULL, a staged page whose block is resident is also
 * copied into its pool slot.  page_ids entries must be in range (device data,
 * not checked on the host; out-of-range ids are skipped by the kernel).
 */
int oasis_block_meta_build(oasis_handle h, const void* pages, const int32_t* page_ids,
                           int32_t count, const int32_t* ctx_len, void* meta, void* pool,
                           const int32_t* block_to_slot, void* stream);

/*
 * The block metadata from key rows, the form the method states it in ([EXPL]
 * Figure 7 left: per-block min/max pooling of the keys): k_rows
 * [B][H][max_blocks*16][d] token-major on the device (element type, 16-byte
 * aligned).  For every request r, every block b that tokens [tok_begin,
 * tok_end) fall in and that holds tokens below ctx_len[r] gets its metadata
 * row from all of its tokens below ctx_len[r] (also those outside the range).
 * Other blocks are not touched.  EINVAL unless
 * 0 <= tok_begin <= tok_end <= max_blocks*16.
 */
int oasis_block_meta_build_rows(oasis_handle h, const void* k_rows, int32_t tok_begin, int32_t tok_end,
                                const int32_t* ctx_len, void* meta, void* stream);

/*
 * The block metadata in its logical layout ([EXPL] Figure 7 left: per-block,
 * per-channel key min and max): meta_logical is [B][H][max_blocks][2][d]
 * elements (device, 16-byte aligned, oasis_meta_bytes() covers it), block b's
 * key min row then its key max row.  export copies the library's tiles into
 * it; import writes such rows (computed elsewhere) into the tiles.  Blocks at
 * or past a request's context are copied as they are.  Not in place.
 */
int oasis_block_meta_export(oasis_handle h, const void* meta, void* meta_logical, void* stream);
int oasis_block_meta_import(oasis_handle h, const void* meta_logical, void* meta, void* stream);

/*
 * Admission of a prefill computed on the device ([EXPL] Figure 7 left: after the
 * prefill the full KV cache lives in CPU memory and only per-block key min/max
 * stays on the GPU).  k_rows, v_rows: the prefill's keys and values in device
 * memory, [B][H][max_blocks*16][d] token-major (element type; k_rows 16-byte
 * aligned).  For every block b < N(ctx_len) of every unit, one kernel writes the
 * page (K token-major, V channel-major) into host_tier, which must be pinned
 * host memory mapped for the device (the GPU stores it over PCIe; EINVAL
 * otherwise), the block's metadata row (min and max over its tokens below
 * ctx_len) into meta, and, when pool and block_to_slot are given (both or
 * neither) and the block has a slot, the page into that pool slot.  Token rows
 * at or past ctx_len are copied as given.  Blocks >= N are not touched.
 */
int oasis_admit(oasis_handle h, const void* k_rows, const void* v_rows, const int32_t* ctx_len, void* host_tier,
                void* meta, void* pool, const int32_t* block_to_slot, void* stream);

/*
 * Append one token per unit (long-output decode).  k_new, v_new: [B][H][d]
 * device.  The token goes to position p = ctx_len_in[r]: the metadata row of
 * block p/16 is initialised to the token (p % 16 == 0) or absorbs it by
 * min/max; if that block is resident its pool page row is written too.
 * ctx_len_out[r] = p + 1 (ctx_len_out must not alias ctx_len_in).  A position
 * outside [0, 16*max_blocks) is a caller error the device cannot report: that
 * request's metadata and pages are left as they are and ctx_len_out[r] = p
 * (the context does not grow).
 */
int oasis_block_meta_update(oasis_handle h, const void* k_new, const void* v_new,
                            const int32_t* ctx_len_in, int32_t* ctx_len_out, void* meta,
                            void* pool, const int32_t* block_to_slot, void* stream);

/*
 * Lookahead score ([EXPL] Figure 7 right: the draft queries scan the compressed
 * keys to predict the next step's blocks).  For every block b < N of every unit:
 *   scores[u][b] = max over drafts t in 1..D and group heads g of
 *                  sum_c max(q[t][g][c]*kmin[b][c], q[t][g][c]*kmax[b][c])
 * (the Quest upper bound; Quest is in [INDEX] "Builds on").  scores:
 * [B][H][max_blocks] float32; entries b >= N are not written.
 */
int oasis_lookahead_score(oasis_handle h, const void* q, const void* meta, const int32_t* ctx_len,
                          float* scores, void* stream);

/*
 * The same bound from the verify query rows (t = 0) instead of the drafts:
 *   scores[u][b] = max over group heads g of
 *                  sum_c max(q[0][g][c]*kmin[b][c], q[0][g][c]*kmax[b][c]).
 * Selecting the top-k of these scores gives the set the true next-token query
 * picks ([EXPL] Figure 6: the predicted top-K set against the exact set of the
 * true next-token query); the blocks of that set that the lookahead prefetch
 * missed are what a corrective fetch must bring in ([EXPL] "Limits and open
 * work": prediction misses need corrective fetches).  Layout and errors as
 * oasis_lookahead_score.
 */
int oasis_verify_score(oasis_handle h, const void* q, const void* meta, const int32_t* ctx_len, float* scores,
                       void* stream);

/*
 * Top-k selection.  sel [B][H][budget_blocks] int32 in rank order: the sink
 * block 0, then the newest block N-1 (if N > 1), then the other blocks by
 * descending score with ties broken by lower index (-0.0 ranks as +0.0), up to
 * budget_blocks entries; the rest is -1.  With N <= budget_blocks every block
 * is selected.
 */
int oasis_topk_select(oasis_handle h, const float* scores, const int32_t* ctx_len, int32_t* sel,
                      void* stream);

/*
 * Set difference against the resident set, capped fetch, capped eviction
 * ([EXPL] "What they did" item 3; Figure 9).  Per unit:
 *   missing = selected blocks with block_to_slot = -1, in rank order;
 *   fetch   = the first min(fetch_cap, |missing|) of them;
 *   slots   = free slots (slot_to_block = -1) in ascending order, then the
 *             slots of victims: resident blocks outside the selection, taken
 *             lowest score first (equal scores: higher block index first), only
 *             as many as the free slots cannot cover;
 *   both maps are updated in place.
 * fetch [B][H][fetch_cap][2] = (block, slot) pairs, (-1, -1) padded; n_fetch
 * [B][H]; evict [B][H][fetch_cap] victim blocks in eviction order, -1 padded.
 * scores must be the ones sel was made from.
 * attend [B][H][budget_blocks], n_attend [B][H] (optional: both or neither,
 * EINVAL otherwise): the attended set of the next attention, S ∩ R once this
 * step's fetch has landed ([EXPL] Figure 7 right), i.e. the selected blocks
 * that stay resident or are fetched now, in rank order, each entry
 * (block << 10) | slot; entries past n_attend are not written.
 */
int oasis_resident_diff_cap_evict(oasis_handle h, const int32_t* sel, const float* scores,
                                  int32_t* block_to_slot, int32_t* slot_to_block, int32_t* fetch,
                                  int32_t* n_fetch, int32_t* evict, int32_t* attend, int32_t* n_attend,
                                  void* stream);

/*
 * oasis_topk_select followed by oasis_resident_diff_cap_evict on the same
 * arguments, with identical results, in one launch when the shape allows it
 * (max_blocks <= 8192 and budget_blocks <= 514; otherwise the two kernels run
 * back to back).  Saves a launch and a round trip of the selection through
 * global memory on every decode step.  For budget_blocks <= 128 each (request,
 * KV head) is selected and diffed by one workgroup that reads residency from
 * slot_to_block alone: block_to_slot must be its inverse, as every diff,
 * fetch and admission here leaves it (the decode-step calls read it the same
 * way).
 */
int oasis_select_and_diff(oasis_handle h, const float* scores, const int32_t* ctx_len, int32_t* sel,
                          int32_t* block_to_slot, int32_t* slot_to_block, int32_t* fetch,
                          int32_t* n_fetch, int32_t* evict, int32_t* attend, int32_t* n_attend,
                          void* stream);

/*
 * Fetch issue ([EXPL] Figure 8: the transfer lands in HBM before the layer's
 * attention at the next step).  Reads a host-visible copy of fetch / n_fetch
 * (the caller must have synchronised its device-to-host copy) and enqueues one
 * hipMemcpyAsync host-to-device of a page per entry, from host_tier (pinned)
 * to its pool slot, on `stream` (normally a side stream).  All entries are
 * validated before the first copy is enqueued (EINVAL on a bad entry).
 */
int oasis_fetch_issue(oasis_handle h, const void* host_tier, void* pool, const int32_t* fetch_host,
                      const int32_t* n_fetch_host, void* stream);

/*
 * Fetch gather ([EXPL] Figure 8 and "What they did" item 2: the missing
 * predicted blocks move from the host tier into their HBM slots before the
 * layer's attention at the next step).  Device-driven alternative to
 * oasis_fetch_issue: one kernel reads the fetch list and n_fetch where the diff
 * left them (device memory) and copies each page from host_tier (pinned host
 * memory, read by the GPU over PCIe) to its pool slot, on `stream`; no host
 * synchronisation is needed between the diff and the transfer.  host_tier must
 * be pinned host memory mapped for the device (hipHostMalloc / torch
 * pin_memory): checked with hipPointerGetAttributes, EINVAL otherwise.  Entries
 * beyond n_fetch, and entries whose block or slot is out of range, are skipped.
 */
int oasis_fetch_gather(oasis_handle h, const void* host_tier, void* pool, const int32_t* fetch,
                       const int32_t* n_fetch, void* stream);

/*
 * Sparse paged GQA decode attention ([EXPL] Figure 7 right: verify and draft
 * queries attend together over the sparse working set).  For every unit, query
 * row (g, t) and the token set J of the blocks of sel that are resident
 * (block_to_slot >= 0), tokens below ctx_len:
 *   out[r][h*G+g][t] = softmax_j(q . K[j] / sqrt(d)) . V[j]   (0 if J is empty)
 * float32 accumulation, split over the selection with a log-sum-exp merge (a
 * second kernel combines the splits).  out: [B][H*G][T][d] float32.
 * workspace: oasis_workspace_bytes() bytes, not shared by calls that may run at
 * the same time.
 */
int oasis_sparse_paged_decode_attn(oasis_handle h, const void* q, const void* pool,
                                   const int32_t* sel, const int32_t* block_to_slot,
                                   const int32_t* ctx_len, float* out, void* workspace,
                                   void* stream);

/*
 * oasis_sparse_paged_decode_attn for callers that cannot allocate memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without the workspace, the same kernels and
 * the same output.  The split partials live in a scratch array of 16 MiB that
 * the library holds on each GPU it runs on until the process ends; its address
 * is looked up once per device (hipGetSymbolAddress, on the calling thread's
 * current device, which `stream` must belong to).  Nothing is allocated and
 * nothing needs clearing.  EINVAL if the shape needs more workspace than the
 * scratch holds (oasis_workspace_bytes() > 16 MiB).  Every call on a GPU shares
 * that GPU's scratch: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller.
 */
int oasis_sparse_paged_decode_attn_noalloc(oasis_handle h, const void* q, const void* pool,
                                           const int32_t* sel, const int32_t* block_to_slot,
                                           const int32_t* ctx_len, float* out, void* stream);

/*
 * The same attention with S ∩ R given as the attended list a diff produced
 * (attend / n_attend of oasis_resident_diff_cap_evict, oasis_select_and_diff
 * or oasis_decode_step): one load per entry instead of a selection lookup and a
 * map lookup.  Same output and workspace contract; identical results to
 * oasis_sparse_paged_decode_attn on the maps the list was made from.
 */
int oasis_sparse_paged_decode_attn_list(oasis_handle h, const void* q, const void* pool,
                                        const int32_t* attend, const int32_t* n_attend,
                                        const int32_t* ctx_len, float* out, void* workspace,
                                        void* stream);

/*
 * The first launch of a layer's decode step ([EXPL] Figure 8: at step t the
 * attention over the resident part of S_t and the drafts' prediction of S_{t+1}
 * need only step t's inputs): the sparse paged decode attention (as
 * oasis_sparse_paged_decode_attn, or _list when attend is given) and the
 * lookahead scoring (as oasis_lookahead_score with ctx_score) in ONE grid where
 * the shape allows it (bf16, at most 48 attention rows, with the default
 * 2-wavefront attention workgroups, or 4-wavefront ones for at most 32 rows),
 * else back to back.  The attention leaves its split partials
 * in the workspace; `out` is complete after oasis_attn_combine or
 * oasis_select_diff_combine on the same workspace (which do nothing when the
 * attention has a single split and wrote `out` itself), or at once where the
 * handle merges the splits inside this launch (attn_merge 2; a combine after
 * it rewrites the same values).  sel/block_to_slot may be null when attend is
 * given.
 */
int oasis_attend_and_score(oasis_handle h, const void* q, const void* pool, const void* meta,
                           const int32_t* ctx_attn, const int32_t* ctx_score, const int32_t* sel,
                           const int32_t* block_to_slot, const int32_t* attend, const int32_t* n_attend,
                           float* scores, float* out, void* workspace, void* stream);

/* Merges the attention's split partials in `workspace` into `out` (the
 * log-sum-exp combine; nothing to do for a single split). */
int oasis_attn_combine(oasis_handle h, void* workspace, float* out, void* stream);

/*
 * The second launch of a layer's decode step: oasis_select_and_diff (with the
 * attended list when given) and the attention's split combine of `workspace`
 * into `out`, in one grid where the fused selection applies, else back to back.
 */
int oasis_select_diff_combine(oasis_handle h, const float* scores, const int32_t* ctx_score, int32_t* sel,
                              int32_t* block_to_slot, int32_t* slot_to_block, int32_t* fetch, int32_t* n_fetch,
                              int32_t* evict, int32_t* attend, int32_t* n_attend, float* out, void* workspace,
                              void* stream);

/*
 * Least-recently-used eviction variants ([EXPL] Table 2: the fetch-ratio
 * ablation evicts least-recently-used blocks).  As oasis_select_and_diff and
 * oasis_select_diff_combine, except for the victims when the free slots do not
 * cover the fetch: the resident blocks outside the new selection whose slot
 * was read longest ago, i.e. with the smallest stamp in slot_last_use
 * ([B][H][budget_blocks] int32, device, caller-owned; -1 = never read, the
 * caller's initial value), ties in the lowest-score order.  Every slot of the
 * next attention's blocks (the selection after this step's fetch, resident)
 * is stamped with `step` (monotone across calls, chosen by the caller).
 * Available for budget_blocks <= 128 and max_blocks <= 8192, otherwise
 * OASIS_EUNSUPPORTED.
 */
int oasis_select_and_diff_lru(oasis_handle h, const float* scores, const int32_t* ctx_len, int32_t* sel,
                              int32_t* block_to_slot, int32_t* slot_to_block, int32_t* slot_last_use, int32_t step,
                              int32_t* fetch, int32_t* n_fetch, int32_t* evict, int32_t* attend, int32_t* n_attend,
                              void* stream);
int oasis_select_diff_combine_lru(oasis_handle h, const float* scores, const int32_t* ctx_score, int32_t* sel,
                                  int32_t* block_to_slot, int32_t* slot_to_block, int32_t* slot_last_use,
                                  int32_t step, int32_t* fetch, int32_t* n_fetch, int32_t* evict, int32_t* attend,
                                  int32_t* n_attend, float* out, void* workspace, void* stream);

/*
 * One layer's decode step ([EXPL] Figure 8: at step t the layer's attention runs
 * over the resident part of S_t while the draft queries predict S_{t+1}; the
 * selection and the diff that produce the next fetch follow).  Equivalent to,
 * and bit-identical with, the sequence
 *   oasis_sparse_paged_decode_attn(q, pool, sel, block_to_slot, ctx_attn, out, workspace)
 *     (oasis_sparse_paged_decode_attn_list(q, pool, attend, n_attend, ...) when attend is given)
 *   oasis_lookahead_score(q, meta, ctx_score, scores)
 *   oasis_select_and_diff(scores, ctx_score, sel, block_to_slot, slot_to_block, fetch, n_fetch, evict,
 *                         attend, n_attend)
 * with the same arguments, on `stream`: oasis_attend_and_score followed by
 * oasis_select_diff_combine, i.e. two launches for the default shape (three
 * otherwise).  ctx_attn is the context
 * the attention sees (tokens < ctx_attn); ctx_score the context of the scoring
 * and selection (larger by one after an append of this step, which the caller
 * enqueues before this call; the attention does not read what it writes).
 * sel, block_to_slot and slot_to_block (and attend / n_attend when given: the
 * list the previous step's diff left, which this step's diff replaces) are read
 * by the attention and rewritten by the selection/diff afterwards.  Errors as for the three calls; every
 * argument is validated before any launch.
 */
int oasis_decode_step(oasis_handle h, const void* q, const void* pool, const void* meta,
                      const int32_t* ctx_attn, const int32_t* ctx_score, int32_t* sel, int32_t* block_to_slot,
                      int32_t* slot_to_block, float* scores, float* out, void* workspace, int32_t* fetch,
                      int32_t* n_fetch, int32_t* evict, int32_t* attend, int32_t* n_attend, void* stream);

/* The pages a diff chose to fetch for one layer: that layer's pinned host tier
 * (host memory mapped for the device, checked with hipPointerGetAttributes),
 * its HBM pool, and its fetch list and counts (device, as the diff left them). */
typedef struct oasis_transfer {
  const void* host_tier;
  void* pool;
  const int32_t* fetch;    /* [B][H][fetch_cap][2] */
  const int32_t* n_fetch;  /* [B][H] */
} oasis_transfer;

/*
 * oasis_decode_step carrying another layer's transfer inside its first launch
 * ([EXPL] Figure 8: each layer's selection and transfer overlap the compute of
 * the layers after it, and land before that layer's next attention).
 * `transfer` is a layer of the same shape whose diff already ran on this
 * stream; its fetched pages move from its host tier into its pool in workgroups
 * that lead this call's first launch, beside this layer's attention and
 * scoring (the host-link reads overlap the HBM-bound work).  Stream order is
 * the only synchronisation: the move needs no second stream and no event, and
 * everything enqueued later on `stream` sees the pages.  The transfer's pool
 * must not be this call's pool (EINVAL): the attention reads one while the move
 * writes the other.  NULL transfer, or fetch_cap 0: oasis_decode_step.  Where
 * the step's first launch cannot carry it (f32, the three-launch shape) the
 * gather runs as its own launch first.  Results as oasis_decode_step followed by
 * oasis_fetch_gather of the transfer.
 */
int oasis_decode_step_gather(oasis_handle h, const void* q, const void* pool, const void* meta,
                             const int32_t* ctx_attn, const int32_t* ctx_score, int32_t* sel,
                             int32_t* block_to_slot, int32_t* slot_to_block, float* scores, float* out,
                             void* workspace, int32_t* fetch, int32_t* n_fetch, int32_t* evict, int32_t* attend,
                             int32_t* n_attend, const oasis_transfer* transfer, void* stream);

/* One state's top-k selection and resident-set diff, as oasis_select_and_diff
 * takes it: the state's scores (complete: written by an earlier launch), the
 * context length its scoring saw, and the selection, maps, fetch / evict lists
 * and attended list the diff updates (layouts as there; all device). */
typedef struct oasis_select_job {
  const float* scores;
  const int32_t* ctx_len;
  int32_t* sel;
  int32_t* block_to_slot;
  int32_t* slot_to_block;
  int32_t* fetch;
  int32_t* n_fetch;
  int32_t* evict;
  int32_t* attend;
  int32_t* n_attend;
} oasis_select_job;

/*
 * A layer's decode step that also appends this step's token (long-output
 * decode, [EXPL] Figure 7 left and Figure 8): bit-identical with
 *   oasis_block_meta_update(k_new, v_new, ctx_in, ctx_out, meta, pool, block_to_slot)
 *   oasis_decode_step(q, pool, meta, ctx_attn = ctx_in, ctx_score = ctx_out, ...)
 * on `stream`, with one launch fewer where the step's attention and scoring run
 * as launches of their own (bf16 shapes whose attention writes its output
 * without a split combine, e.g. one attention workgroup per (request, KV
 * head)): one workgroup per (request, KV head) after the attention's updates
 * the token's metadata row and ctx_out (the attention reads no metadata), and
 * one after the scoring's writes the token's K / V rows into its block's page
 * when resident (the scoring reads no pages; the next step's attention is the
 * first reader).  Other shapes enqueue the append kernel first.  k_new, v_new:
 * [B][H][d] device; ctx_out (written: ctx_in + 1, or ctx_in for a position
 * outside the capacity, as oasis_block_meta_update) must not alias ctx_in
 * (EINVAL); pool and meta are written.  Other arguments and errors as for
 * oasis_decode_step.
 */
int oasis_decode_step_append(oasis_handle h, const void* q, void* pool, void* meta, const int32_t* ctx_in,
                             int32_t* ctx_out, int32_t* sel, int32_t* block_to_slot, int32_t* slot_to_block,
                             float* scores, float* out, void* workspace, int32_t* fetch, int32_t* n_fetch,
                             int32_t* evict, int32_t* attend, int32_t* n_attend, const void* k_new,
                             const void* v_new, void* stream);

/*
 * A layer's decode step whose first launch carries another state's selection
 * ([EXPL] Figure 8: a layer's prediction, selection and transfer proceed while
 * later layers compute; only that layer's next attention needs them).  Two
 * launches:
 *   1. `job`'s selection and diff (one workgroup per (request, KV head), ahead
 *      of the rest; none when job is NULL), then this layer's attention over
 *      attend / n_attend and the lookahead score of its drafts into `scores`,
 *      led by `transfer`'s page gather when given (as oasis_decode_step_gather);
 *   2. the attention's split combine into `out`.
 * This layer's own selection is not run: the caller carries it, as a job, in
 * a later call (typically the next layer's, the last layer's in the next
 * step's first layer's) or runs it with oasis_select_and_diff; that layer's
 * next attention must follow.  The job's results are identical, bit for bit,
 * to oasis_select_and_diff on the same state.  The job must be another state
 * than this step's: its scores, attended list and fetch list must not be
 * `scores`, `attend` or the transfer's fetch list (EINVAL).  The block map is
 * read only as the inverse of the slot map, as every diff leaves them.
 * EUNSUPPORTED unless bf16, head_dim 128, 2 attention wavefronts per
 * workgroup, budget_blocks <= 128 and max_blocks <= 8192 (score eviction).
 */
int oasis_decode_step_carry(oasis_handle h, const void* q, const void* pool, const void* meta,
                            const int32_t* ctx_attn, const int32_t* ctx_score, const int32_t* attend,
                            const int32_t* n_attend, float* scores, float* out, void* workspace,
                            const oasis_select_job* job, const oasis_transfer* transfer, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* OASISKV_H */
