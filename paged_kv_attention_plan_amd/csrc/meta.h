// Device-side form of a plan's rows and tiles, as uploaded to the workspace.  The public
// structs of pkv.h (pkv_decode_tile, pkv_merge_entry) stay the inspection view;
// this form is what the decode kernel reads: 16-byte key-range pieces, a
// per-row table and a per-worker piece range, so the per-step upload stays
// small.
#pragma once

#include <cstdint>

namespace pkv {

// (query head, token) pairs of one prefill tile: the planner cuts each prompt
// row into blocks of kPrefillTilePairs / group query tokens per KV head, and
// the prefill kernel's four waves take 48 pairs each.
constexpr int kPrefillTilePairs = 192;

// One decode row (a row with one query token), in decode-piece order.
struct DecodeRowMeta {
  int32_t page_base;  // paged_kv_indptr[row]
  int32_t q_index;    // token index into q / out / k_new / v_new
  int32_t kv_len;
  int32_t slot0;      // first partial slot of the row (-1: not split)
  int32_t n_chunks;   // pieces of the row, the same for every KV head (1: not split)
  int32_t pad[3];
};

// One decode piece: keys [kv_start, kv_end) of one row, run by every wave of
// a decode worker (one wave per KV head).  Worker w runs the pieces
// [work[w], work[w + 1]) of the worker table in order.
struct DecodePieceMeta {
  int32_t row;        // index into the DecodeRowMeta table
  int32_t chunk;      // piece index within the row
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
static_assert(sizeof(DecodePieceMeta) == 16, "decode pieces are 16 bytes");

}  // namespace pkv
