// Host-side planner for paged-KV attention: page-table validation, work tiles,
// the balanced split-KV partition of decode work, workspace layout, KV write
// slots and the mixed-step permutation.  No HIP dependency: everything here is
// plain C++ on the host.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "meta.h"
#include "pkv.h"

namespace pkv {

// Byte offsets of the regions of a plan's device workspace.  The metadata
// regions [0, meta_bytes) are filled by the upload; the partial regions are
// scratch written by split decode tiles and read by the merge.
struct WorkspaceLayout {
  size_t off_dense_rows = 0;      // DenseRowMeta per row of a dense plan
  size_t off_decode_rows = 0;     // DecodeRowMeta per decode row
  size_t off_decode_tiles = 0;    // DecodePieceMeta per decode piece
  size_t off_decode_work = 0;     // int32 piece range start per decode worker, plus the end
  size_t off_merges = 0;          // pkv_merge_entry per split (row, KV head)
  size_t off_prefill_tiles = 0;
  size_t off_indices = 0;
  size_t off_slots = 0;
  size_t meta_bytes = 0;
  size_t off_part_o = 0;    // float [n_slots][group][head_dim]
  size_t off_part_lse = 0;  // float [n_slots][group]
  size_t total_bytes = 0;
};

struct PlanData {
  pkv_plan_params params{};
  int32_t batch = 0;
  int32_t total_q = 0;
  int32_t num_cus = 0;
  int32_t group = 1;
  int32_t worker_pages = 0;      // decode balance target: pages (+ overheads) per worker
  int32_t n_workers = 0;         // decode workers of this plan (capacity if graph-static)
  int32_t n_slots = 0;
  int32_t max_merge_chunks = 0;  // largest n_chunks over merges
  int32_t n_decode_rows = 0;
  int32_t n_prompt_rows = 0;
  std::vector<pkv_decode_tile> decode_tiles;
  std::vector<pkv_merge_entry> merges;         // every split (row, KV head)
  std::vector<DecodeRowMeta> decode_rows;      // device form of the decode tiles
  std::vector<DecodePieceMeta> decode_pieces;  // each run by the Hk waves of a worker
  std::vector<int32_t> decode_work;            // n_workers + 1 piece offsets
  std::vector<pkv_prefill_tile> prefill_tiles;
  std::vector<int32_t> indices;  // copy of paged_kv_indices
  std::vector<int64_t> slots;    // flat write slot per query token
  std::vector<int32_t> perm;     // mixed: prompt tokens first
  // graph-static plans: the workspace is laid out for these capacities
  bool is_static = false;
  struct Caps {
    int64_t dec_rows = 0, dec_pieces = 0, dec_workers = 0, merges = 0, n_slots = 0,
            prefill_tiles = 0, indices = 0, tokens = 0;
  } caps;
  // dense plans
  bool dense = false;
  bool dense_pages = false;      // page table given: the gather may copy prefixes
  int64_t total_k = 0;           // cu_k[batch]
  std::vector<DenseRowMeta> dense_rows;
  WorkspaceLayout ws;
};

// Validate the page table and fill `out`.  num_cus must already be resolved
// (> 0).  On failure returns the status and sets `err`.
pkv_status build_plan(const pkv_plan_params& params, int32_t num_cus, int32_t batch,
                      const int32_t* qo_indptr, const int32_t* kv_indptr,
                      const int32_t* kv_indices, const int32_t* last_page_len,
                      const int32_t* kv_lens, PlanData& out, std::string& err);

// Dense plan (kind PKV_KIND_DENSE): rows of contiguous K/V at cu_k offsets with
// queries at cu_q offsets; kv_indptr / kv_indices (both or neither) give each
// row's pages for gathering its prefix (the first cu_k - cu_q tokens).
pkv_status build_dense_plan(const pkv_plan_params& params, int32_t num_cus, int32_t batch,
                            const int32_t* cu_q, const int32_t* cu_k, const int32_t* kv_indptr,
                            const int32_t* kv_indices, PlanData& out, std::string& err);

// Parameter checks that do not need the page table.
pkv_status check_params(const pkv_plan_params& p, std::string& err);

// Copy the metadata regions of `plan` into `dst` (meta_bytes bytes).
void serialize_meta(const PlanData& plan, void* dst);

// Page table of the rows without the step's appended tokens (see
// pkv_context_only_views).
pkv_status context_only_views(int32_t batch, int32_t page_size, const int32_t* kv_indptr,
                              const int32_t* kv_indices, const int32_t* last_page_len,
                              const int32_t* to_compute, const int32_t* query_spans,
                              int32_t* out_indptr, int32_t* out_indices,
                              int32_t* out_last_page_len, int32_t* out_qo_indptr,
                              std::string& err);

}  // namespace pkv
