/*
 * rpa.h -- ragged paged attention with KV append for AMD Instinct MI355X (gfx950).
 *
 * C ABI of librpa.so.  Plain pointers and sizes only.  Device pointers are
 * HIP device addresses; a `stream` argument is a hipStream_t passed as void*.
 *
 * The problem, as the source pages state it
 * -----------------------------------------
 * "Disaggregated prefill and decode" (Perplexity), prefill/decode performance
 * section: each request of a batch step brings qo_len new query tokens and
 * attends over kv_len entries of its KV cache; decode has qo_len = 1, a
 * prefill chunk a large qo_len.  "Accelerating Sonar through speculation"
 * (Perplexity), runtime section: for every step the host allocates KV pages
 * for the new tokens, packs tokens and page information, copies the metadata
 * to the GPU and builds the attention metadata and intermediate buffers once,
 * for prefill, decode and verification alike.  The disaggregation post, KV
 * Messenger section: every layer appends its new KV entries to the cache, and
 * they are valid after the append and before the attention that reads them.
 * Same post, sharded-transfer section: pages use the HND layout (heads before
 * tokens).  "Chunked prefill" (k4i.top), section "correctness": attention
 * over the cache and over the current chunk combine by an online-softmax
 * merge, so chunked prefill equals one-shot prefill.
 *
 * Shape of a step: rpa_plan_create (host) -> rpa_plan_upload (async H2D) ->
 * per layer { rpa_kv_append ; rpa_batch_attention }.  The plan is reused by
 * every layer of the step.  Split form: rpa_plan_create_split ->
 * rpa_plan_upload -> per layer { rpa_split_attention, with rpa_kv_append
 * before, after or beside it }.
 *
 * Notation: request r has n_r = qo_len new tokens, L_r = kv_len keys counting
 * the new ones, c_r = L_r - n_r cached keys, and page size P.  New token t of
 * request r has global row i = qo_indptr[r] + t and absolute position
 * p = c_r + t; with causal = 1 it sees keys 0 .. p (bottom-right alignment).
 * G = num_qo_heads / num_kv_heads; query head h reads KV head h / G.
 *
 * Tensor layouts (elements; last dimension contiguous):
 *   q      [total_q, num_qo_heads, head_dim_qk]      contiguous
 *   k_new  [total_q, num_kv_heads, head_dim_qk]      contiguous
 *   v_new  [total_q, num_kv_heads, head_dim_v]       contiguous
 *   o      [total_q, num_qo_heads, head_dim_v]       contiguous, dtype of q
 *   lse    [total_q, num_qo_heads]                   float32, natural log
 *   pools  element (page, head, slot, d) at
 *          page*page_stride + head*head_stride + slot*token_stride + d
 *          (HND packed: token_stride = d, head_stride = P*d,
 *           page_stride = H*P*d; interleaved K/V pages are expressed by strides)
 *
 * Ownership: the caller owns every device buffer (q, k_new, v_new, pools, o,
 * lse, workspace) and every stream.  The library owns only rpa_plan objects
 * (host memory plus a pinned staging buffer).  No call allocates device
 * memory or synchronises a stream.
 *
 * A plan with no new tokens (total_q == 0) makes rpa_kv_append and
 * rpa_batch_attention return RPA_OK at once; their tensor pointers may then
 * be NULL.
 *
 * Errors: every call returns rpa_status; RPA_OK is 0, failures are negative.
 * Arguments are validated on the host before anything is launched: on an
 * error nothing is launched and no output is touched.  A thread-local message
 * (rpa_last_error_message) describes the last failure.  No C++ exception
 * crosses this interface: every entry point catches them and returns
 * RPA_ERR_HOST_ALLOC (host memory ran out) or RPA_ERR_INTERNAL.
 */
#ifndef RPA_H_
#define RPA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RPA_ABI_VERSION 3

typedef enum rpa_status {
  RPA_OK = 0,
  RPA_ERR_INVALID_ARG = -1,         /* null pointer, bad size, misaligned buffer, bad metadata */
  RPA_ERR_UNSUPPORTED = -2,         /* valid but not implemented: head dims, page size, dtype */
  RPA_ERR_WORKSPACE_TOO_SMALL = -3, /* workspace smaller than rpa_plan_workspace_size */
  RPA_ERR_PAGE_OOB = -4,            /* a page id outside [0, num_pages), or too few pages */
  RPA_ERR_DUPLICATE_WRITE_PAGE = -5,/* a page written by the append is referenced twice */
  RPA_ERR_HIP = -6,                 /* a HIP runtime call failed */
  RPA_ERR_NOT_UPLOADED = -7,        /* the plan has not been uploaded to a workspace */
  RPA_ERR_HOST_ALLOC = -8,          /* host memory ran out inside the call */
  RPA_ERR_INTERNAL = -9             /* any other failure inside the library */
} rpa_status;

typedef enum rpa_dtype {
  RPA_DTYPE_F32 = 0,  /* IEEE binary32 */
  RPA_DTYPE_BF16 = 1  /* bfloat16; arithmetic accumulates in float32 */
} rpa_dtype;

/* Attention configuration, fixed for a plan.
 *   num_qo_heads % num_kv_heads == 0.
 *   (head_dim_qk, head_dim_v) in {(64,64), (128,128), (576,512)}; (576,512) is
 *   the absorbed latent form: one latent KV head whose first 512 dims are the
 *   value (v_cache == k_cache with the same strides).
 *   page_size: a power of two in [1, 256].
 *   causal: 1 = bottom-right causal (query t sees keys 0 .. c_r + t);
 *           0 = every query sees all kv_len keys.  Without causal masking
 *           kv_len may be smaller than qo_len, down to 0: the new tokens then
 *           attend to cached keys only (the cache half of the split execution
 *           in "Chunked prefill", section "correctness"); a request with
 *           kv_len = 0 gets the empty state o = 0, lse = -inf, and a plan
 *           with any kv_len < qo_len cannot append (rpa_kv_append returns
 *           RPA_ERR_INVALID_ARG).
 *   sm_scale: multiplier of q.k (e.g. 1/sqrt(head_dim_qk)); finite and > 0. */
typedef struct rpa_attn_config {
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t head_dim_qk;
  int32_t head_dim_v;
  int32_t page_size;
  int32_t dtype;   /* rpa_dtype */
  int32_t causal;
  float sm_scale;
} rpa_attn_config;

/* Ragged batch of one step.  Host int32 arrays, owned by the caller, read only
 * during rpa_plan_create.
 *   qo_indptr[batch_size+1]: starts at 0, non-decreasing; n_r = qo_indptr[r+1]-qo_indptr[r].
 *   kv_len[batch_size]: L_r >= n_r (the new tokens are the last n_r keys);
 *     with causal = 0, any L_r >= 0 (see rpa_attn_config).
 *   kv_page_indptr[batch_size+1], kv_page_indices[kv_page_indptr[batch_size]]:
 *     CSR page table; request r needs at least ceil(L_r / P) entries, extra
 *     entries are ignored.
 *   num_pages: pool size; every used page id lies in [0, num_pages).
 * A page that the append writes (one holding a position in c_r .. L_r-1) must
 * not be referenced by any other (request, logical page) of the batch. */
typedef struct rpa_batch_desc {
  int32_t batch_size;
  const int32_t* qo_indptr;
  const int32_t* kv_len;
  const int32_t* kv_page_indptr;
  const int32_t* kv_page_indices;
  int32_t num_pages;
} rpa_batch_desc;

/* Strides of a paged pool, in elements; the head dimension is contiguous.
 * All strides must be multiples of 8 elements (16 bytes) for bf16 and of
 * 4 elements for f32; token_stride >= the stored row length. */
typedef struct rpa_cache_strides {
  int64_t page_stride;
  int64_t head_stride;
  int64_t token_stride;
} rpa_cache_strides;

typedef struct rpa_plan rpa_plan;

/* Validate a batch and build its plan on the host: the per-token append map,
 * the attention work items (long kv_len split into pieces so that the GPU's
 * num_cus compute units get balanced work; 0 means 256), and the merge map of
 * the split pieces.
 * Source: "Accelerating Sonar through speculation" (Perplexity), section on
 * inference with speculative decoding: for every step the host allocates KV
 * pages for the new tokens, packs tokens and page information for the GPU and
 * builds the attention metadata once, for prefill, decode and verification
 * alike; "Disaggregated prefill and decode" (Perplexity), performance
 * section: each request has its own qo_len and kv_len, and the work
 * parallelises over requests and over kv_len.
 * Arguments: cfg and batch as described above (read during the call only);
 * num_cus: compute units to balance for (0 = 256); out: receives the plan.
 * No device work; may be called without a GPU.  On success *out receives a
 * plan owned by the library (free with rpa_plan_destroy); on failure *out is
 * NULL.  Errors: INVALID_ARG, UNSUPPORTED, PAGE_OOB, DUPLICATE_WRITE_PAGE,
 * HOST_ALLOC. */
rpa_status rpa_plan_create(const rpa_attn_config* cfg, const rpa_batch_desc* batch,
                           int32_t num_cus, rpa_plan** out);

/* rpa_plan_create for a batch whose speculative drafts form trees
 * ("Accelerating Sonar through speculation", Perplexity: a draft tree is
 * verified in one pass, each draft token attending to the context and to its
 * own ancestors in the tree, under a custom attention mask).  Attention stays
 * causal (cfg->causal must be 1) except among the new tokens of a request
 * that has a mask: there new token t sees new token u iff bit u of its mask
 * row is set, while every cached key stays visible.
 *   tree_indptr[batch_size+1]: word offsets into tree_words, starting at 0;
 *     request r has a mask iff tree_indptr[r+1] > tree_indptr[r], and then
 *     exactly n_r * ceil(n_r/32) words (n_r <= 64);
 *   tree_words: row t of request r is the ceil(n_r/32) words at
 *     tree_indptr[r] + t * ceil(n_r/32); bit u % 32 of word u / 32 is set iff
 *     new token t sees new token u.  Every token must see itself; bits past
 *     n_r must be clear.
 * Both arrays are host memory owned by the caller, read only during the call.
 * A chain mask (row t = bits 0..t) reproduces the causal result.  Requests of
 * the absorbed latent form that carry a mask run on the generic kernel.
 * Errors: as rpa_plan_create; INVALID_ARG for a malformed mask, UNSUPPORTED
 * for a mask over more than 64 new tokens. */
rpa_status rpa_plan_create_tree(const rpa_attn_config* cfg, const rpa_batch_desc* batch,
                                const int32_t* tree_indptr, const uint32_t* tree_words,
                                int32_t num_cus, rpa_plan** out);

/* rpa_plan_create for the split execution of a causal step ("Chunked
 * prefill" (k4i.top), section "correctness": the chunk's attention is the
 * softmax merge of its attention over the cached history and its causal
 * attention over the chunk itself).  The plan has two parts:
 *   cache part: new token t of request r sees all c_r cached keys of its
 *     pages (no mask);
 *   own part:   it sees new tokens 0 .. t of its request, read from the
 *     step's k_new / v_new rows (token-major, the layout table) instead of
 *     the pages;
 * both parts' states are merged per row.  The result equals
 * rpa_batch_attention after rpa_kv_append, and the pages' slots for the new
 * tokens are never read, so the append may run before, after or beside the
 * attention (rpa_kv_append accepts this plan).  Each part is balanced over
 * num_cus compute units on its own; one call runs a constant number of
 * launches whatever the batch: the cache part's kernel classes, the own
 * part's, and one merge.
 * Arguments and ownership as rpa_plan_create; cfg->causal must be 1 and the
 * head dims 64/64 or 128/128.  Errors: as rpa_plan_create; INVALID_ARG for
 * causal = 0, UNSUPPORTED for the 576/512 latent form. */
rpa_status rpa_plan_create_split(const rpa_attn_config* cfg, const rpa_batch_desc* batch,
                                 int32_t num_cus, rpa_plan** out);

/* Device bytes the plan needs in its workspace: metadata plus the float32
 * partial outputs and log-sum-exp values of split pieces.  Host only. */
rpa_status rpa_plan_workspace_size(const rpa_plan* plan, size_t* bytes);

/* Copy the plan's metadata into a caller-owned device workspace (256-byte
 * aligned, at least rpa_plan_workspace_size bytes) with one asynchronous
 * host-to-device copy on `stream`, from a pinned staging buffer the plan
 * owns.  Later calls with this plan use that workspace; it must stay alive
 * and unmodified while they run.  Errors: INVALID_ARG, WORKSPACE_TOO_SMALL, HIP. */
rpa_status rpa_plan_upload(rpa_plan* plan, void* d_workspace, size_t bytes, void* stream);

/* KV append (the per-layer cache update).  For every new token (r, t) and KV
 * head h, copies k_new[i, h, :] into k_cache at page pages_r[(c_r+t)/P],
 * head h, slot (c_r+t)%P, and v_new likewise into v_cache.  A raw copy of the
 * stored elements: no rounding, no other byte of the pools changes.
 * Source: "Disaggregated prefill and decode" (Perplexity), KV Messenger
 * section: each layer appends its new KV entries to the paged cache, and an
 * entry is valid once the append has run and before the attention that reads
 * it; sharded-transfer section: pages hold heads before tokens (HND).
 * Arguments: k_new / v_new token-major device rows as in the layout table;
 * k_cache / v_cache device pools addressed by ks / vs (host structs).  The
 * caller owns every buffer; the call only enqueues work on `stream`.
 * Shared latent (head dims 576/512): pass v_new = NULL and v_cache = NULL or
 * v_cache == k_cache; only k is written.  Pools are in the plan's dtype.
 * Errors: INVALID_ARG, NOT_UPLOADED, HIP. */
rpa_status rpa_kv_append(const rpa_plan* plan, const void* k_new, const void* v_new,
                         void* k_cache, void* v_cache, const rpa_cache_strides* ks,
                         const rpa_cache_strides* vs, void* stream);

/* Batched ragged attention over the paged cache (run after rpa_kv_append of
 * the same step).  For every new token i of request r and query head h:
 *   s_j = sm_scale * <q[i,h,:], K(r, h/G, j)> for visible keys j,
 *   lse[i,h] = ln sum_j exp(s_j),  o[i,h,:] = sum_j exp(s_j - lse) V(r, h/G, j).
 * Split pieces are combined by the log-sum-exp merge inside this call.
 * Source: "Disaggregated prefill and decode" (Perplexity), performance
 * section: requests of one batch differ in qo_len (1 for decode, the chunk
 * for prefill) and kv_len, and attention runs over both in one batch;
 * "Accelerating Sonar through speculation", speculative-decoding section:
 * verification attends n + 1 new tokens; "Chunked prefill" (k4i.top),
 * section "correctness": a chunk's tokens see the whole cache and,
 * causally, the chunk; partial results merge by log-sum-exp.
 * Arguments: q, o token-major device tensors (layout table); pools as in
 * rpa_kv_append; lse device float32 [total_q, num_qo_heads] or NULL.  The
 * caller owns every buffer; the plan's workspace holds the split partials.
 * For the shared latent form pass v_cache == k_cache (or NULL) and vs == ks
 * (or NULL): values are the first head_dim_v elements of each key row.
 * `lse` may be NULL.  Errors: INVALID_ARG, UNSUPPORTED, NOT_UPLOADED, HIP. */
rpa_status rpa_batch_attention(const rpa_plan* plan, const void* q, const void* k_cache,
                               const void* v_cache, const rpa_cache_strides* ks,
                               const rpa_cache_strides* vs, void* o, float* lse,
                               void* stream);

/* Attention of a split plan (rpa_plan_create_split): the same o and lse as
 * rpa_batch_attention over the pages after the append, computed from the
 * cached keys in the pools and the step's own keys in k_new / v_new.
 * Source: "Chunked prefill" (k4i.top), section "correctness": history part
 * and chunk part merge by log-sum-exp into the one-shot result.
 * Arguments: q, o, lse as rpa_batch_attention; k_new / v_new the step's new
 * rows, token-major contiguous [total_q, num_kv_heads, d] (16-byte
 * aligned), the buffers rpa_kv_append copies from; k_cache / v_cache and
 * ks / vs the pools, of which only the first c_r keys of each request are
 * read.  The two parts write their partial states (float32) to the plan's
 * workspace; the merge writes o and lse.  The
 * prefill-sized requests of both parts run in one launch, side by side on
 * shares of the compute units in proportion to their work.  The caller owns
 * every buffer; the call only enqueues work on `stream`.
 * Errors: INVALID_ARG (also for a plan not made by rpa_plan_create_split),
 * NOT_UPLOADED, HIP.  rpa_batch_attention and rpa_batch_attention_noalloc
 * reject a split plan with INVALID_ARG. */
rpa_status rpa_split_attention(const rpa_plan* plan, const void* q, const void* k_new,
                               const void* v_new, const void* k_cache, const void* v_cache,
                               const rpa_cache_strides* ks, const rpa_cache_strides* vs,
                               void* o, float* lse, void* stream);

/* rpa_batch_attention without a workspace, for callers that cannot allocate
 * device memory at the point of the call: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments,
 * same kernels and the same results as rpa_batch_attention; the plan need not
 * be uploaded.  The plan's metadata is copied from its host memory into a
 * static device array of the library (RPA_STATIC_SCRATCH_BYTES, one per GPU,
 * held until the process ends) with one asynchronous copy on `stream`, and
 * the split partials live there too.  The call allocates nothing.
 * Every call on a GPU uses that GPU's one array, so calls whose work may
 * overlap on one GPU (two streams, or two threads) race: order them on one
 * stream.  The plan must stay alive until the call's work has run.
 * Errors: as rpa_batch_attention, and WORKSPACE_TOO_SMALL when the plan's
 * workspace (rpa_plan_workspace_size) exceeds RPA_STATIC_SCRATCH_BYTES. */
#define RPA_STATIC_SCRATCH_BYTES (128u << 20)
rpa_status rpa_batch_attention_noalloc(const rpa_plan* plan, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const rpa_cache_strides* ks,
                                       const rpa_cache_strides* vs, void* o, float* lse,
                                       void* stream);

/* Standalone softmax merge of two attention states over disjoint key sets
 * ("Chunked prefill", section "correctness"):
 *   lse = ln(e^lse_a + e^lse_b),  o = e^(lse_a-lse) o_a + e^(lse_b-lse) o_b.
 * o_a, o_b, o: [rows, heads, dim] in `dtype`; lse_a, lse_b, lse: [rows, heads]
 * float32 (lse may be NULL); dim is a multiple of 8 and the o buffers are
 * 16-byte aligned.  A state with lse = -inf contributes nothing;
 * two -inf states give (-inf, 0).  o may alias o_a or o_b; lse must not alias
 * lse_a or lse_b (INVALID_ARG).  All pointers are device memory the caller
 * owns.  Errors: INVALID_ARG, HIP. */
rpa_status rpa_merge_state(const void* o_a, const float* lse_a, const void* o_b,
                           const float* lse_b, void* o, float* lse, int64_t rows,
                           int32_t heads, int32_t dim, int32_t dtype, void* stream);

/* Page copy between paged pools and transfer buffers.
 * "Disaggregated prefill and decode" (Perplexity), sharded-transfer section:
 * when prefill and decode shard the KV cache differently, pages are split or
 * reconstructed by the shard ratio (a decoder rebuilds full pages from the
 * halves two prefill devices send), and the HND layout keeps a head range of
 * a page contiguous so that it moves as one write.  "Chunked prefill",
 * prefix-cache section: cached prefix blocks are reused; a shared block that
 * is only partly filled must be copied before two requests append to it.
 * For i in [0, num_pages), copies heads [src_head0, src_head0 + num_heads)
 * of page src_pages[i] of `src` into heads [dst_head0, dst_head0 + num_heads)
 * of page dst_pages[i] of `dst`: all page_size slots, `dim` elements per row.
 * A raw copy of the stored bits.
 *   src_pool_pages / dst_pool_pages: pages each side holds; a pair whose
 *     source or destination id lies outside [0, that count) is skipped on
 *     the device (nothing read or written for it); with a NULL page list,
 *     num_pages must not exceed the pool's count (else PAGE_OOB).
 *   src_pool_heads / dst_pool_heads: heads each side holds; the head ranges
 *     must lie inside them (else INVALID_ARG).
 *   src_pages / dst_pages: DEVICE int32 arrays of num_pages page ids, or NULL
 *     for the identity (page i); the caller owns them.
 *   strides (elements, as rpa_cache_strides): any layout, e.g. an HND pool,
 *     an NHD buffer (head_stride = dim, token_stride = heads * dim) or a
 *     packed shard buffer of num_heads heads.
 *   dtype: RPA_DTYPE_F32 or RPA_DTYPE_BF16; dim fills whole 16-byte chunks.
 * The pool counts and strides must describe memory the caller owns; regions
 * written must not overlap regions read.  num_pages = 0 is a no-op.
 * Errors: INVALID_ARG, PAGE_OOB, HIP. */
rpa_status rpa_page_copy(const void* src, const rpa_cache_strides* src_strides,
                         int32_t src_pool_pages, int32_t src_pool_heads, const int32_t* src_pages,
                         void* dst, const rpa_cache_strides* dst_strides, int32_t dst_pool_pages,
                         int32_t dst_pool_heads, const int32_t* dst_pages, int32_t num_pages,
                         int32_t src_head0, int32_t dst_head0, int32_t num_heads,
                         int32_t page_size, int32_t dim, int32_t dtype, void* stream);

/* Free a plan.  Waits for the plan's last upload copy to finish reading the
 * staging buffer.  NULL is ignored. */
void rpa_plan_destroy(rpa_plan* plan);

/* Static description of a status code. */
const char* rpa_status_string(rpa_status status);

/* Message describing the last failure on the calling thread ("" if none). */
const char* rpa_last_error_message(void);

/* RPA_ABI_VERSION of the loaded library. */
int32_t rpa_abi_version(void);

/* Per-kernel timing for profiling.  While enabled (on = 1), the library
 * records a pair of HIP events (timing enabled) on the launch stream around
 * every kernel it launches.  rpa_profile_read waits for the recorded events,
 * folds them into per-kernel totals and returns the total milliseconds and
 * launch count of one kernel: "append", "generic", "decode", "prefill",
 * "mla", "merge", "merge_state" or "page_copy".  rpa_profile_reset clears the totals.
 * Process-wide and thread-safe; off by default.  Errors: INVALID_ARG, HIP. */
rpa_status rpa_profile_enable(int32_t on);
/* Restricts the timing to the kernels named in `kernels`, a comma-separated
 * list of the names above (NULL or "" again times every kernel), so that a
 * timed loop carries events around its dominant kernel only.  Takes effect
 * for later launches; the totals are kept.  Errors: none. */
rpa_status rpa_profile_select(const char* kernels);
rpa_status rpa_profile_read(const char* kernel, double* total_ms, int64_t* launches);
rpa_status rpa_profile_reset(void);

/* Host-only introspection of a plan (for tests and tooling).  Copies up to
 * `cap` int32 values of the named table into `dst` and stores the table's
 * full length in *len.  Names: "items" (8 int32 per work item: request,
 * kv head, first row, end row, first key, end key, split index, kernel
 * class), "splits" (3 int32 per request: number of pieces, keys per piece
 * (0 when the pieces differ in length; the items then give their bounds),
 * first partial row), "append" (2 int32 per new token: page id, slot),
 * "wg_prefill" / "wg_mla" (workgroup b runs items [v[b], v[b + 1]) of that
 * class), "merge_rows" (rows whose pieces are merged), "merge_info" (4 int32
 * per merge row: first partial row, partial-row stride between pieces,
 * pieces holding a key the row sees, 0), "summary" (batch_size,
 * total_q, num items, partial rows, number of items per kernel class 0..3).
 * For a split plan the names give the cache part's tables (it holds the
 * merge and the append map) and "own:<name>" the own part's.
 * Errors: INVALID_ARG for an unknown name. */
rpa_status rpa_plan_debug_dump(const rpa_plan* plan, const char* name, int32_t* dst,
                               int64_t cap, int64_t* len);

#ifdef __cplusplus
}
#endif

#endif /* RPA_H_ */
