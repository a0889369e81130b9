// Launchers for the gfx950 kernels.  Plain pointers only; the C ABI in
// capi.cpp validates arguments before it calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "meta.h"
#include "pkv.h"

namespace pkv {

struct DecodeArgs {
  const DecodePieceMeta* pieces;
  const DecodeRowMeta* rows;
  const int32_t* work;      // [n_workers + 1]: worker w runs pieces [work[w], work[w + 1])
  int32_t n_workers;        // each worker is num_kv_heads waves, one per KV head
  const int32_t* indices;   // paged_kv_indices on the device
  const uint16_t* q;        // bf16 [total_q, Hq, D]
  const uint16_t* cache;    // bf16 [max_pages, 2, ps, Hk, D]
  uint16_t* out;            // bf16 [total_q, Hq, D]
  float* lse;               // [total_q, Hq] or null
  float* part_o;            // [n_slots, group, D]
  float* part_lse;          // [n_slots, group]
  int32_t num_qo_heads, num_kv_heads, head_dim, page_size, group;
  float scale_log2;         // log2(e) / sqrt(head_dim)
};

// Graph-static plans: `counts` points at the uploaded counts (workspace header,
// int64 [8]: decode pieces, merges, prefill tiles, indices, slots, partial
// slots, tokens, rows), which replace the n_* arguments; the grids are sized for
// the plan's capacities.  Null otherwise.  (Decode needs no count: its grid is
// the plan's workers and the uploaded worker table gives every worker its
// range, empty for the unused ones.)
struct MergeArgs {
  const pkv_merge_entry* merges;
  int32_t n_merges;
  const int64_t* counts;    // see above
  int32_t max_chunks;       // largest n_chunks of any entry
  const float* part_o;
  const float* part_lse;
  uint16_t* out;
  float* lse;
  int32_t num_qo_heads, head_dim, group;
};

struct AppendArgs {
  const int64_t* slots;     // flat page * ps + offset per token
  int32_t n_tokens;
  const int64_t* counts;    // as in MergeArgs
  const uint16_t* k_new;    // bf16 [n_tokens, Hk, D]
  const uint16_t* v_new;
  uint16_t* cache;
  int32_t num_kv_heads, head_dim, page_size;
};

struct PrefillArgs {
  const pkv_prefill_tile* tiles;
  int32_t n_tiles;
  const int64_t* counts;    // as in MergeArgs
  const int32_t* indices;
  const uint16_t* q;
  const uint16_t* cache;
  // Dense mode (both non-null): contiguous K and V, bf16 [total_k, Hk, D]; a
  // tile's keys start at row page_base (cu_k of its row); cache and indices
  // are unused.
  const uint16_t* k_dense;
  const uint16_t* v_dense;
  uint16_t* out;
  float* lse;
  int32_t num_qo_heads, num_kv_heads, head_dim, page_size, group;
  int32_t causal, window_left;
  float scale_log2;
};

struct GatherArgs {
  const DenseRowMeta* rows;
  int32_t n_rows;
  int32_t with_prefix;      // 0: copy the fresh tokens only
  int64_t total_k;          // dense rows = cu_k of the end
  int32_t total_q;          // fresh tokens = cu_q of the end
  const int32_t* indices;
  const uint16_t* cache;    // bf16 [max_pages, 2, ps, Hk, D]
  const uint16_t* k_fresh;  // bf16 [total_q, Hk, D]
  const uint16_t* v_fresh;
  uint16_t* k_out;          // bf16 [total_k, Hk, D]
  uint16_t* v_out;
  int32_t num_kv_heads, head_dim, page_size;
};

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream);

// Plan metadata upload: the GPU copies n_vec 16-byte vectors from page-locked
// host memory (device-visible pointer) into the workspace.  Workgroup b then
// stores seq into flags[b] (host-coherent memory) to mark its reads done.
struct UploadArgs {
  const uint4* src;
  uint4* dst;
  int64_t n_vec;
  uint32_t* flags;
  uint32_t seq;
  int32_t max_blocks;
};

// *blocks receives the number of workgroups launched (<= a.max_blocks).
hipError_t launch_upload(const UploadArgs& a, hipStream_t stream, int* blocks);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// Decode waves and prefill tiles of a mixed step in one grid (decode
// workgroups first).  Only where mixed_launch_fits: paged K/V with
// page_size >= 16 and one head_dim for both.
bool mixed_launch_fits(const DecodeArgs& da, const PrefillArgs& pa);
hipError_t launch_mixed(const DecodeArgs& da, const PrefillArgs& pa, hipStream_t stream);

}  // namespace pkv
