/*
 * pkv.h -- batched attention over a paged KV cache on AMD Instinct MI355X (gfx950).
 *
 * A C ABI: plain integers, host or device pointers and sizes.  No C++ or torch
 * types cross it.  The operations follow the documentation pages of the mstar
 * serving engine:
 *   - mstar.engine.resources.attn.wrappers  (FlashInferDecodeWrapper,
 *     FlashInferPrefillWrapper, FlashInferMixedWrapper: plan / run;
 *     check_flashinfer_head_dim)
 *   - mstar.engine.resources.kv.plan         (PagedIndptrs, SequenceView,
 *     KVPlanOutput, PinnedIndexRing)
 *   - mstar.engine.resources.attn.workspace  (Workspace: split-KV partials,
 *     sizing, overflow reporting)
 *   - mstar.engine.resources.attn.dense      (DenseAttentionManager: the
 *     [prefix | fresh] sequence; requires_kv_write: write K/V, then run)
 *
 * Data layout
 * -----------
 * KV cache layer slice (wrappers module docstring; the run methods):
 *     [max_pages, 2, page_size, num_kv_heads, head_dim]  bf16, contiguous.
 *   Index 0 of the "2" axis is K, index 1 is V (a convention: no page fixes it).
 * q, out : [total_q, num_qo_heads, head_dim] bf16, contiguous (decode: total_q = batch).
 * lse    : [total_q, num_qo_heads] float32, natural log of the sum of exp of the
 *          scaled logits.  Optional (NULL: not written).
 * k_new, v_new : [total_q, num_kv_heads, head_dim] bf16, contiguous.
 * Page table (kv.plan, PagedIndptrs), host int32 arrays:
 *   qo_indptr[batch+1]              query tokens of row r are q[qo_indptr[r] : qo_indptr[r+1]]
 *   paged_kv_indptr[batch+1]        pages of row r are paged_kv_indices[indptr[r] : indptr[r+1]]
 *   paged_kv_indices[indptr[batch]] physical page ids in [0, max_pages)
 *   paged_kv_last_page_len[batch]   tokens on row r's last page, in [1, page_size]
 *   so kv_len[r] = (pages(r) - 1) * page_size + last_page_len[r].
 *
 * Semantics
 * ---------
 * Query token t of row r sits at position p = kv_len - q_len + t of the row (the
 * queries are the row's last tokens: a [cached prefix | fresh tokens] sequence,
 * attn.dense).  It attends to keys j with lo <= j <= hi where hi = p when causal
 * (else kv_len - 1) and lo = max(0, p - window_left) when window_left >= 0 (else
 * 0): window_left counts the positions before the query that it still sees
 * (FlashInferPrefillWrapper.plan; the decode plan takes the same argument).
 * Query head h reads KV head h / (num_qo_heads / num_kv_heads).
 *   out = softmax(q k^T / sqrt(head_dim)) v over the visible keys, fp32 accumulation.
 *
 * Call order per step (attn.dense requires_kv_write: the layer stores its K/V
 * before it runs attention):
 *   pkv_plan_create (or pkv_plan_update)    host only; never touches the device
 *   pkv_plan_upload(workspace, stream)      async upload from library-owned pinned memory
 *   per layer: pkv_append_kv(...)           optional; stores this step's K/V
 *              pkv_run(...)                 attention for every planned query
 *          or  pkv_run_append(...)          both in one call
 * One plan serves every layer of a step.  Dense plans (PKV_KIND_DENSE) instead go
 * pkv_dense_plan_create -> pkv_plan_upload -> per layer pkv_dense_gather,
 * pkv_dense_run; pkv_run / pkv_append_kv / pkv_run_append reject them.
 *
 * Ownership: the caller owns every device buffer (q, out, lse, cache, workspace,
 * k_new, v_new).  The library owns the plan handle, which copies what it needs
 * from the host arrays (no pointer is kept after a call returns) and a depth-2
 * ring of page-locked staging buffers (kv.plan, PinnedIndexRing).
 *
 * Errors: every call returns a pkv_status; pkv_last_error() returns a message
 * for the calling thread's last failure (valid until that thread's next call).
 * Device work is enqueued on the given stream and is never synchronised by the
 * library, except that re-using a staging buffer waits for the upload kernel that
 * last read it.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_E_INVALID = 1,      /* malformed page table, bad argument, q_len > kv_len, kv_lens mismatch */
  PKV_E_UNSUPPORTED = 2,  /* head_dim, dtype, page_size or group size this build does not compute,
                             or a page of K and V of 2 GiB or more */
  PKV_E_WORKSPACE = 3,    /* workspace smaller than the plan needs; message gives the bytes */
  PKV_E_CAPACITY = 4,     /* more prompt rows than max_prefill_rows (mixed step) */
  PKV_E_CONFLICT = 5,     /* two appended tokens map to one cache slot */
  PKV_E_DEVICE = 6,       /* a HIP runtime call failed; message gives the HIP error */
  PKV_E_STATE = 7         /* call out of order (e.g. run before upload, or another workspace) */
} pkv_status;

typedef enum pkv_kind {
  PKV_KIND_DECODE = 0,   /* one query token per row; qo_indptr is NULL (FlashInferDecodeWrapper) */
  PKV_KIND_PREFILL = 1,  /* ragged query rows (FlashInferPrefillWrapper) */
  PKV_KIND_MIXED = 2,    /* one-token rows on a decode sub-plan, other rows on a prefill
                            sub-plan (FlashInferMixedWrapper) */
  PKV_KIND_DENSE = 3     /* contiguous [prefix | fresh] K/V per row, cu_q / cu_k offsets
                            (attn.dense DensePlan); built by pkv_dense_plan_create */
} pkv_kind;

typedef enum pkv_dtype { PKV_DTYPE_BF16 = 0 } pkv_dtype;

typedef struct pkv_plan_params {
  int32_t kind;                 /* pkv_kind */
  int32_t num_qo_heads;         /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;         /* Hk */
  int32_t head_dim;             /* 64 or 128 (check_flashinfer_head_dim analogue) */
  int32_t page_size;            /* power of two in [1, 256] */
  int32_t causal;               /* prefill/mixed: nonzero = causal, aligned to the end of KV */
  int32_t window_left;          /* -1 = unbounded, else >= 0 */
  int32_t dtype;                /* PKV_DTYPE_BF16 */
  int32_t max_prefill_rows;     /* mixed only: capacity of the prefill sub-plan */
  int32_t num_cus;              /* compute units the plan balances over; 0 = ask the current HIP
                                   device (the workspace page: plan size depends on the SM count) */
  int64_t max_pages;            /* pages in the layer slice; page ids must be below it */
  int32_t decode_waves_per_cu;  /* decode waves per CU the split-KV partition balances over
                                   (workers = num_cus * this / num_kv_heads, and for a
                                   graph-static plan at most static_max_page_entries); 0 = 4
                                   for group 1, 2, 4 and 16 for group 8 */
  int32_t decode_min_chunk_pages; /* smallest per-worker share of a step's pages; 0 = 8 */
  /* Graph-static mode (attn.wrappers: static buffers for graph capture, sized by
   * batch_size / max_num_pages / max_total_tokens).  All three 0: off.  All three > 0:
   * the workspace is laid out for at most static_max_batch rows, static_max_tokens
   * query tokens and static_max_page_entries page-table entries, every re-plan must
   * fit them (else PKV_E_CAPACITY), and pkv_plan_upload / pkv_append_kv / pkv_run
   * launch the same kernels with the same arguments on every step, so a stream
   * capture of pkv_append_kv / pkv_run can be replayed after each pkv_plan_update +
   * pkv_plan_upload (the upload itself is not captured).  The kernels read the step's
   * work counts from the uploaded workspace; grids are sized for the capacities.
   * Buffers passed to captured calls keep their addresses across replays and hold
   * static_max_tokens rows (only the step's rows are read or written).  Timing
   * (pkv_timing_enable) must be off while capturing.  Not for dense plans. */
  int32_t static_max_batch;
  int32_t static_max_tokens;
  int64_t static_max_page_entries;
} pkv_plan_params;

/* One unit of decode work: a row, a KV head and a contiguous key range.
 * The tile covers keys [kv_start, kv_end) of the row; out_slot < 0 means the tile
 * writes out/lse directly, else it writes split-KV partial number out_slot into
 * the workspace and a merge combines the partials.  Decode work is partitioned
 * over workers, each a group of num_kv_heads waves: a row's visible pages are
 * cut, at page boundaries, into pieces that the same cut gives every KV head;
 * the tiles of a piece are num_kv_heads consecutive entries (kv_head 0, 1, ...),
 * and a worker runs consecutive pieces so that every worker gets about the same
 * number of pages (attn.workspace: the plan depends on the CU count). */
typedef struct pkv_decode_tile {
  int32_t row, kv_head, kv_start, kv_end;
  int32_t page_base;  /* paged_kv_indptr[row] */
  int32_t q_index;    /* token index into q/out */
  int32_t out_slot;   /* -1 or partial slot */
  int32_t kv_len;     /* the row's kv_len */
} pkv_decode_tile;

/* One split-KV merge: partials [slot_base, slot_base + n_chunks) of (q_index, kv_head). */
typedef struct pkv_merge_entry {
  int32_t q_index, kv_head, slot_base, n_chunks;
} pkv_merge_entry;

/* One unit of prefill work: a row, a KV head and a block of that row's query tokens.
 * Query rows of the block are q tokens [q_base + q_start, q_base + q_start + q_count)
 * of every query head of kv_head's group.  Keys [kv_lo, kv_hi] (inclusive) cover the
 * union of the block's visible ranges. */
typedef struct pkv_prefill_tile {
  int32_t row, kv_head, q_start, q_count;
  int32_t kv_lo, kv_hi;
  int32_t page_base;  /* paged_kv_indptr[row] */
  int32_t q_base;     /* qo_indptr[row]: packed token index of the row's first query */
  int32_t kv_len, q_len;
  int32_t pad0, pad1;
} pkv_prefill_tile;

typedef struct pkv_plan pkv_plan;

/* Fill *p with defaults: causal = 1, window_left = -1, dtype = bf16, tuning knobs 0. */
void pkv_plan_params_init(pkv_plan_params* p);

/* Validate the page table and build a plan (FlashInfer*Wrapper.plan analogue).
 * Host only.  qo_indptr must be NULL for PKV_KIND_DECODE and non-NULL otherwise.
 * kv_lens (optional, may be NULL) must equal the lengths the page table implies.
 * On success *out owns a new plan and *workspace_bytes is the exact size of the
 * device workspace the plan needs (plan metadata plus split-KV partials).
 * Errors: PKV_E_INVALID, PKV_E_UNSUPPORTED, PKV_E_CAPACITY, PKV_E_CONFLICT, and
 * PKV_E_DEVICE when num_cus == 0 and the device cannot be queried. */
pkv_status pkv_plan_create(const pkv_plan_params* params, int32_t batch,
                           const int32_t* qo_indptr, const int32_t* paged_kv_indptr,
                           const int32_t* paged_kv_indices,
                           const int32_t* paged_kv_last_page_len, const int32_t* kv_lens,
                           pkv_plan** out, size_t* workspace_bytes);

/* Re-plan an existing handle for a new step with the same params (keeps its staging
 * ring).  Arguments and errors as pkv_plan_create; on error the old plan is kept. */
pkv_status pkv_plan_update(pkv_plan* plan, int32_t batch, const int32_t* qo_indptr,
                           const int32_t* paged_kv_indptr, const int32_t* paged_kv_indices,
                           const int32_t* paged_kv_last_page_len, const int32_t* kv_lens,
                           size_t* workspace_bytes);

void pkv_plan_destroy(pkv_plan* plan);

/* Inspection (host pointers owned by the plan, valid until the next update/destroy). */
pkv_status pkv_plan_decode_tiles(const pkv_plan* plan, const pkv_decode_tile** tiles, int32_t* n);
pkv_status pkv_plan_prefill_tiles(const pkv_plan* plan, const pkv_prefill_tile** tiles, int32_t* n);
pkv_status pkv_plan_merges(const pkv_plan* plan, const pkv_merge_entry** merges, int32_t* n);
/* Flat write slot page * page_size + offset of every planned query token, in q order
 * (decode: the row's last page at offset last_page_len - 1;
 *  FlashInferDecodeWrapper.plan, KVPlanOutput.decode_pages / decode_offsets). */
pkv_status pkv_plan_write_slots(const pkv_plan* plan, const int64_t** slots, int32_t* n);
/* Mixed step: packed q indices of the prompt tokens, prompt rows in ascending order
 * ("moved to the front", FlashInferMixedWrapper).  n = 0 for other kinds. */
pkv_status pkv_plan_permutation(const pkv_plan* plan, const int32_t** perm, int32_t* n);
/* Scalars: [0] total_q, [1] batch, [2] decode rows, [3] prompt rows, [4] decode worker
 * capacity (pages plus per-piece costs of two pages each), [5] partial slots,
 * [6] metadata bytes, [7] workspace bytes, [8] num_cus used, [9] dense key rows
 * (cu_k[batch]; 0 for paged plans), the byte offsets in the workspace of [10] the dense
 * row table, [11] the decode row table, [12] the decode pieces, [13] the merge entries,
 * [14] the prefill tiles, [15] the page-index copy, [16] the decode worker table, and
 * [17] the decode workers (the table has [17] + 1 entries). */
pkv_status pkv_plan_info(const pkv_plan* plan, int64_t info[18]);

/* Write the metadata image pkv_plan_upload copies into the workspace (its first
 * pkv_plan_info[6] bytes) into host memory dst of `bytes` bytes, for inspection or
 * for a caller's own copy: an int64 header [decode pieces, merges, prefill tiles,
 * page indices, write slots, partial slots, query tokens, rows], then the regions
 * at the offsets pkv_plan_info reports (16-byte decode pieces
 * {int32 decode row, int32 piece index within the row, int32 kv_start, int32 kv_end};
 * 32-byte decode rows {page_base, q_index, kv_len, first partial slot or -1, pieces,
 * 3 pad}, a row's partial for KV head h and piece c at first slot + h * pieces + c;
 * the int32 decode worker table, worker w running pieces [table[w], table[w + 1]);
 * 32-byte dense rows {cu_k, cu_q, prefix, fresh, page_base, 3 pad}; merge entries and
 * prefill tiles as declared above; int32 page indices; int64 write slots).  Host only.
 * PKV_E_WORKSPACE if bytes is too small. */
pkv_status pkv_plan_metadata(const pkv_plan* plan, void* dst, size_t bytes);

/* Copy the plan's metadata into the head of `workspace` (device memory of at least
 * the plan's workspace_bytes), enqueued on `stream` (a hipStream_t; NULL = the null
 * stream).  The metadata is serialised into a page-locked, host-coherent staging
 * buffer and a small kernel on `stream` reads it over the host link into the
 * workspace.  The staging buffer is rewritten only after every workgroup of the
 * kernel that last read it has flagged its reads done (a flag in the same
 * host-coherent buffer), so re-planning while earlier steps are in flight is safe
 * (attn.dense force_double_buffer hazard); this call waits for that, up to 60 s,
 * then returns PKV_E_DEVICE.  A plan whose metadata outgrows the staging buffer
 * re-allocates it (page-locked memory, freed with hipHostFree, which waits for the
 * device).  PKV_E_WORKSPACE if workspace_bytes is too small. */
pkv_status pkv_plan_upload(pkv_plan* plan, void* workspace, size_t workspace_bytes, void* stream);

/* Counters of the plan's staging ring (kv.plan PinnedIndexRing: a buffer is reused
 * only after its last reader is done).  stats[0] = uploads launched, stats[1] =
 * uploads that found their staging buffer still being read and waited, stats[2] =
 * nanoseconds spent in those waits.  Host only; PKV_E_INVALID on NULL. */
pkv_status pkv_plan_upload_stats(const pkv_plan* plan, int64_t stats[3]);

/* Attention for every planned query (FlashInfer*Wrapper.run analogue).
 * q, kv_cache_layer, out: device pointers (layouts above); lse may be NULL.
 * workspace must be the buffer of the last pkv_plan_upload (else PKV_E_STATE).
 * Decode rows whose keys span several chunks write fp32 partials into the
 * workspace and a merge kernel combines them by log-sum-exp (attn.workspace).
 * A mixed plan with page_size >= 16 runs its decode rows and prompt rows in one
 * launch (FlashInferMixedWrapper: both sub-plans in one step), the merge after it.
 * One upload serves any number of runs (one per layer); runs that overlap on one
 * workspace (two streams, no ordering) race on its partials.  Enqueued on stream. */
pkv_status pkv_run(const pkv_plan* plan, const void* q, const void* kv_cache_layer, void* out,
                   float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* pkv_plan_upload + pkv_run without a caller workspace and without allocating
 * anything, for callers that cannot allocate device memory: code under stream
 * capture, tight serving loops, harnesses that forbid allocation.  The workspace
 * is a static device array of pkv_noalloc_capacity() bytes (32 MiB), one per GPU,
 * held until the process ends.  q, kv_cache_layer, out and lse are as for
 * pkv_run; the plan's metadata reaches the array through the plan's staging
 * ring, exactly as pkv_plan_upload does.
 * Errors: PKV_E_CAPACITY if the plan's workspace_bytes exceed the array, or if
 *   the plan's staging buffers are smaller than its metadata (pkv_plan_upload
 *   sizes both whenever one grows: upload the plan, or a larger one, once
 *   beforehand; a graph-static plan's metadata never grows); otherwise as
 *   pkv_plan_upload and pkv_run.  Dense plans are PKV_E_INVALID.
 * Every call on one GPU shares its array, which keeps the last call's contents:
 * calls that overlap on one GPU (different streams, or threads without ordering)
 * race.  Calls on one stream are ordered.  The plan's per-kernel timing
 * (pkv_timing_enable) is not recorded for these calls (its events are created on
 * first use). */
pkv_status pkv_run_noalloc(pkv_plan* plan, const void* q, const void* kv_cache_layer, void* out,
                           float* lse, void* stream);
size_t pkv_noalloc_capacity(void);

/* pkv_append_kv followed by pkv_run on the same stream (attn.dense requires_kv_write:
 * the step's K/V are stored before attention reads them).  k_new, v_new: bf16
 * [total_q, Hk, D], 16-byte aligned, not NULL.  Errors as pkv_run and
 * pkv_append_kv; nothing is enqueued when an argument check fails.  Enqueued on stream. */
pkv_status pkv_run_append(const pkv_plan* plan, const void* q, const void* k_new, const void* v_new,
                          void* kv_cache_layer, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Store this step's K and V of every planned query token at its write slot:
 * cache[page, 0, off] = k_new[t], cache[page, 1, off] = v_new[t]
 * (decode: at last_page_len - 1 of the last page; FlashInferDecodeWrapper.plan).
 * Reads the slots from the uploaded workspace.  Enqueued on stream. */
pkv_status pkv_append_kv(const pkv_plan* plan, const void* k_new, const void* v_new,
                         void* kv_cache_layer, void* workspace, size_t workspace_bytes,
                         void* stream);

/* ---- Dense [prefix | fresh] mode (attn.dense: DenseAttentionManager, DensePlan,
 * DenseSegment) ----
 * Row r's K/V are rows [cu_k[r], cu_k[r+1]) of contiguous bf16 tensors k, v
 * [cu_k[batch], Hk, D]: the row's frozen prefix (its first cu_k[r+1] - cu_k[r] -
 * q_len tokens) followed by its q_len = cu_q[r+1] - cu_q[r] fresh tokens, whose
 * queries are rows [cu_q[r], cu_q[r+1]) of q.  Attention is the same as for a paged
 * row of that length (bottom-right causal alignment, window_left).  The fresh K/V
 * never reach the pages (requires_kv_write is False for this backend).
 *
 * pkv_dense_plan_create: params->kind must be PKV_KIND_DENSE; params->page_size and
 * max_pages describe the page pool the prefixes are gathered from.  cu_q, cu_k:
 * host int32 [batch + 1], both starting at 0 and non-decreasing, with
 * q_len <= key count per row and each row's K below 4 GiB.  paged_kv_indptr /
 * paged_kv_indices (both or neither, host int32): each row's pages, which must hold
 * at least its prefix; without them pkv_dense_gather can only copy the fresh tokens.
 * Host only; the handle is freed by pkv_plan_destroy, uploaded by pkv_plan_upload,
 * inspected by pkv_plan_prefill_tiles / pkv_plan_info (info[9] = cu_k[batch]).
 * Errors as pkv_plan_create. */
pkv_status pkv_dense_plan_create(const pkv_plan_params* params, int32_t batch, const int32_t* cu_q,
                                 const int32_t* cu_k, const int32_t* paged_kv_indptr,
                                 const int32_t* paged_kv_indices, pkv_plan** out,
                                 size_t* workspace_bytes);
/* Re-plan a dense handle for a new step (same rules; the upload is invalidated). */
pkv_status pkv_dense_plan_update(pkv_plan* plan, int32_t batch, const int32_t* cu_q,
                                 const int32_t* cu_k, const int32_t* paged_kv_indptr,
                                 const int32_t* paged_kv_indices, size_t* workspace_bytes);
/* Build the contiguous K/V of an uploaded dense plan: k_out / v_out [cu_k[batch], Hk, D]
 * receive, per row, its prefix gathered from kv_cache_layer's pages (only when
 * with_prefix != 0) followed by its fresh tokens k_fresh / v_fresh [cu_q[batch], Hk, D]
 * (DenseAttentionManager gathers the prefix once per stream and layer and
 * concatenates the fresh K/V each step: call with with_prefix = 0 to refresh only the
 * fresh rows of a buffer whose prefixes are already in place).  All device pointers
 * 16-byte aligned.  PKV_E_INVALID if with_prefix is set on a plan without pages.
 * Enqueued on stream; timed as kind [0]. */
pkv_status pkv_dense_gather(const pkv_plan* plan, const void* kv_cache_layer, const void* k_fresh,
                            const void* v_fresh, void* k_out, void* v_out, int32_t with_prefix,
                            void* workspace, size_t workspace_bytes, void* stream);
/* Dense attention of an uploaded dense plan: q [cu_q[batch], Hq, D], k / v
 * [cu_k[batch], Hk, D] bf16, out like q, lse [cu_q[batch], Hq] fp32 or NULL.  Runs the
 * prefill kernel with contiguous addressing; errors as pkv_run.  Enqueued on stream. */
pkv_status pkv_dense_run(const pkv_plan* plan, const void* q, const void* k, const void* v,
                         void* out, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream);

/* The page table of a step's rows without the tokens the step appends
 * (kv.plan context_only_views, for attention over the stored context alone).
 * Row r of the input table (paged_kv_indptr / _indices / _last_page_len, the same
 * CSR arrays pkv_plan_create takes, page_size a power of two in [1, 256]) holds
 * kv_len_r tokens, the last to_compute[r] of them appended this step.  The output
 * row keeps the first kv_len_r - to_compute[r] tokens: its pages are the first
 * ceil(kept / page_size) of the input row's, its last_page_len follows from kept,
 * and out_qo_indptr gives it query_spans[r] query tokens.
 * Plan the result with causal = 0 so that every query sees every kept key (the
 * kept tokens all precede the step's tokens); a row's query count must then
 * still not exceed its kept length.
 * Host only: no device call.  The caller allocates out_indptr[batch + 1],
 * out_indices (at least as many entries as paged_kv_indices), out_last_page_len[batch]
 * and out_qo_indptr[batch + 1].  Errors: PKV_E_INVALID for a malformed table,
 * to_compute[r] outside [0, kv_len_r) (every row keeps a stored token) or a negative
 * query_spans[r]; PKV_E_UNSUPPORTED for a bad page_size.  The outputs are partly
 * written on error. */
pkv_status pkv_context_only_views(int32_t batch, int32_t page_size, const int32_t* paged_kv_indptr,
                                  const int32_t* paged_kv_indices,
                                  const int32_t* paged_kv_last_page_len, const int32_t* to_compute,
                                  const int32_t* query_spans, int32_t* out_indptr,
                                  int32_t* out_indices, int32_t* out_last_page_len,
                                  int32_t* out_qo_indptr);

/* Per-launch timing, a tracing aid (the wrappers' enable_nvtx flag is the pages'
 * counterpart).  While enabled, pkv_run, pkv_run_append and pkv_append_kv record a HIP event on the
 * stream before and after every kernel they launch with this plan.
 * pkv_timing_read waits for those events, returns for each kernel kind
 * ([0] append or dense gather, [1] decode, or the one launch of a mixed plan's decode
 * and prefill work, [2] split-KV merge, [3] prefill or dense attention) the summed
 * milliseconds
 * and the number of launches since the last read, and clears the record.
 * Events come from a pool the plan owns (created on first use, reused after a read). */
pkv_status pkv_timing_enable(pkv_plan* plan, int32_t enable);
pkv_status pkv_timing_read(pkv_plan* plan, double ms[4], int64_t launches[4]);

/* Message for the calling thread's last failed call ("" if none). */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
