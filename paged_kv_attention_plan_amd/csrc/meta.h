// Device-side form of a plan's rows and tiles, as uploaded to the workspace.  The public
// structs of pkv.h (pkv_decode_tile, pkv_merge_entry) stay the inspection view;
// this form is what the decode kernel reads: a 16-byte tile plus a per-row
// table, so the per-step upload is about half the size.
#pragma once

#include <cstdint>

namespace pkv {

// One decode row (a row with one query token), in decode-tile order.
struct DecodeRowMeta {
  int32_t page_base;  // paged_kv_indptr[row]
  int32_t q_index;    // token index into q / out / k_new / v_new
  int32_t kv_len;
  int32_t slot0;      // first partial slot of the row (-1: not split)
  int32_t n_chunks;   // key chunks per KV head (1: not split)
  int32_t pad[3];
};

// One decode tile: keys [kv_start, kv_end) of one KV head of one row.
struct DecodeTileMeta {
  int32_t row;        // index into the DecodeRowMeta table
  int16_t kv_head;
  int16_t chunk;      // chunk index within the row
  int32_t kv_start;
  int32_t kv_end;
};

// One row of a dense plan, for the gather: the row's keys are dense rows
// [cu_k, cu_k + prefix + fresh); the prefix comes from the pages
// indices[page_base ..], the fresh part from rows [cu_q, cu_q + fresh) of the
// step's K/V.
struct DenseRowMeta {
  int32_t cu_k, cu_q, prefix, fresh, page_base;
  int32_t pad[3];
};

static_assert(sizeof(DenseRowMeta) == 32, "dense rows are 32 bytes");
static_assert(sizeof(DecodeRowMeta) == 32, "row table entries are 32 bytes");
static_assert(sizeof(DecodeTileMeta) == 16, "decode tiles are 16 bytes");

}  // namespace pkv
