// Host planner.  The operations it prepares are documented on the mstar pages:
//   kv.plan (PagedIndptrs, SequenceView.last_page_len, KVPlanOutput) for the page
//   table and write locations; attn.wrappers (FlashInferDecodeWrapper.plan,
//   FlashInferPrefillWrapper.plan, FlashInferMixedWrapper) for the plan inputs,
//   window_left and the mixed step; attn.workspace (Workspace) for split-KV
//   partials and a plan size that depends on rows, heads and the CU count.
//
// Tiling policy (ours; the pages leave it open):
//  decode  A row's single query sits at position N-1 and sees keys [lo, N-1],
//          lo = max(0, N-1-window_left) (or 0).  Its visible pages run from
//          lo/ps to (N-1)/ps.  Decode work runs on W workers, each a group of
//          Hk waves (one per KV head) that walk the same key ranges:
//          W = max(1, floor(num_cus * waves_per_cu / Hk)), waves_per_cu 4 for
//          group 1, 2, 4 and 16 for group 8 unless given.  A piece of p pages costs
//          p + kPieceCost (its start-up and epilogue, in page-times).  Rows
//          are taken longest first (ties: lower row index) and poured in that
//          order into workers of capacity C: a worker takes as many of a row's
//          pages as fit (at least one), closes once fewer than one page fits,
//          and the row continues in the next worker.  C is the smallest value
//          >= max(min_chunk_pages, ceil(total / W)) + kPieceCost, total the
//          pages plus one piece cost per row, for which the pour uses at most
//          W workers.  A row cut into n > 1 pieces owns Hk * n consecutive
//          partial slots (head-major) and one merge per head.
//  prefill Query tokens are taken in blocks of kPrefillTilePairs/group (192/group)
//          so a block fills the 192 (head, token) pairs of a kernel tile; a
//          block's keys are [lo of its first token,
//          hi of its last token].  Tiles are ordered by key count, largest first
//          (ties: row, block, KV head), so the longest work is dispatched first.
#include "plan.h"

#include <algorithm>
#include <cstring>
#include <numeric>

namespace pkv {
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Start-up and epilogue of a decode piece, in page-times (the time a wave
// takes to stream one page of its KV head): loading the piece's metadata, its
// query and first keys, and combining and storing its result.
constexpr int64_t kPieceCost = 2;

// Decode workers of a plan: groups of Hk waves.  By default four waves per CU
// (one four-wave workgroup each) for groups up to 4, where the kernel streams
// HBM and one wave per SIMD keeps enough loads in flight; sixteen for group 8,
// where the kernel is bound by its vector ALU and more, shorter pieces keep
// every SIMD busy.  (Measured on MI355X over waves per CU 4, 8, 12 and 16.)
// A graph-static plan has no more workers than page entries (each worker holds
// at least one page), so its capacity grid stays small for small capacities.
int64_t decode_workers(const pkv_plan_params& P, int64_t num_cus) {
  const int64_t g = P.num_qo_heads / P.num_kv_heads;
  const int64_t waves_per_cu = P.decode_waves_per_cu > 0 ? P.decode_waves_per_cu
                               : g == 8                  ? 16
                                                         : 4;
  int64_t w = std::max<int64_t>(1, num_cus * waves_per_cu / P.num_kv_heads);
  if (P.static_max_page_entries > 0) w = std::min(w, P.static_max_page_entries);
  return w;
}

// Pour rows of `pages` (in order) into workers of capacity `cap`; emit(row
// position, first page offset within the row, page count, worker) per piece.
// Returns the number of workers used.
template <class Emit>
int64_t pour(const std::vector<int64_t>& pages, int64_t cap, Emit emit) {
  int64_t w = 0, used = 0;
  bool any = false;
  for (size_t i = 0; i < pages.size(); ++i) {
    for (int64_t done = 0; done < pages[i];) {
      int64_t avail = cap - used - kPieceCost;
      if (avail < 1) {
        ++w;
        used = 0;
        avail = cap - kPieceCost;
      }
      const int64_t take = std::min(pages[i] - done, avail);
      emit(i, done, take, w);
      any = true;
      used += take + kPieceCost;
      done += take;
    }
  }
  return any ? w + 1 : 0;
}

std::string fmt_row(const char* what, int64_t r) {
  return std::string(what) + " (row " + std::to_string(r) + ")";
}

// Prefill tiles of the given rows (FlashInferPrefillWrapper.plan): blocks of
// kPrefillTilePairs / group query tokens per KV head, keys [lo(first token), hi(last token)],
// sorted by key count descending, ties by (row, block, head).  page_base(r) is
// where row r's keys start: its first page-table entry, or its first dense row.
template <class PageBase>
void make_prefill_tiles(const pkv_plan_params& P, const std::vector<int32_t>& rows,
                        const std::vector<int32_t>& kv_len, const std::vector<int32_t>& q_len,
                        const std::vector<int32_t>& q_start, PageBase page_base,
                        std::vector<pkv_prefill_tile>& tiles) {
  if (rows.empty()) return;
  const int32_t Hk = P.num_kv_heads;
  const int64_t bt = kPrefillTilePairs / (P.num_qo_heads / Hk);
  const int64_t w = P.window_left;
  // Every KV head of a query block has the block's key range, and the head is
  // the last tie-breaker: sort the blocks, then emit their heads in order.
  struct Block { int64_t keys; int32_t r, b; int32_t qs, qc, lo, hi; };
  std::vector<Block> blocks;
  for (int32_t r : rows) {
    const int64_t n = kv_len[r], L = q_len[r];
    for (int64_t b = 0; b * bt < L; ++b) {
      const int64_t qs = b * bt, qc = std::min(bt, L - qs);
      const int64_t p0 = n - L + qs, p1 = p0 + qc - 1;
      const int64_t lo = w < 0 ? 0 : std::max<int64_t>(0, p0 - w);
      const int64_t hi = P.causal ? p1 : n - 1;
      blocks.push_back({hi - lo + 1, r, (int32_t)b, (int32_t)qs, (int32_t)qc, (int32_t)lo,
                        (int32_t)hi});
    }
  }
  std::sort(blocks.begin(), blocks.end(), [](const Block& a, const Block& b) {
    if (a.keys != b.keys) return a.keys > b.keys;
    if (a.r != b.r) return a.r < b.r;
    return a.b < b.b;
  });
  tiles.reserve(blocks.size() * Hk);
  for (const Block& bl : blocks) {
    pkv_prefill_tile t{};
    t.row = bl.r;
    t.q_start = bl.qs;
    t.q_count = bl.qc;
    t.kv_lo = bl.lo;
    t.kv_hi = bl.hi;
    t.page_base = page_base(bl.r);
    t.q_base = q_start[bl.r];
    t.kv_len = kv_len[bl.r];
    t.q_len = q_len[bl.r];
    for (int32_t hk = 0; hk < Hk; ++hk) {
      t.kv_head = hk;
      tiles.push_back(t);
    }
  }
}


}  // namespace

pkv_status check_params(const pkv_plan_params& p, std::string& err) {
  if (p.kind < PKV_KIND_DECODE || p.kind > PKV_KIND_DENSE) {
    err = "kind must be PKV_KIND_DECODE, PKV_KIND_PREFILL, PKV_KIND_MIXED or PKV_KIND_DENSE";
    return PKV_E_INVALID;
  }
  if (p.num_qo_heads < 1 || p.num_kv_heads < 1 || p.num_qo_heads % p.num_kv_heads != 0) {
    err = "num_qo_heads must be a positive multiple of num_kv_heads (got " +
          std::to_string(p.num_qo_heads) + ", " + std::to_string(p.num_kv_heads) + ")";
    return PKV_E_INVALID;
  }
  if (p.head_dim != 64 && p.head_dim != 128) {
    err = "head_dim " + std::to_string(p.head_dim) + " is not computed by this library (64 or 128)";
    return PKV_E_UNSUPPORTED;
  }
  if (p.dtype != PKV_DTYPE_BF16) {
    err = "only bf16 q/KV are supported";
    return PKV_E_UNSUPPORTED;
  }
  if (!is_pow2(p.page_size) || p.page_size > 256) {
    err = "page_size must be a power of two in [1, 256] (got " + std::to_string(p.page_size) + ")";
    return PKV_E_UNSUPPORTED;
  }
  // The kernels address K and V inside a page with 32-bit offsets.
  if (2 * (int64_t)p.page_size * p.num_kv_heads * p.head_dim * 2 >= (int64_t(1) << 31)) {
    err = "a page of K and V (2 x page_size x num_kv_heads x head_dim bf16) must stay under 2 GiB "
          "(num_kv_heads " + std::to_string(p.num_kv_heads) + ")";
    return PKV_E_UNSUPPORTED;
  }
  if (p.window_left < -1) {
    err = "window_left must be -1 (unbounded) or >= 0";
    return PKV_E_INVALID;
  }
  if (p.max_pages < 1) {
    err = "max_pages must be >= 1";
    return PKV_E_INVALID;
  }
  const int g = p.num_qo_heads / p.num_kv_heads;
  if ((p.kind == PKV_KIND_DECODE || p.kind == PKV_KIND_MIXED) &&
      !(g == 1 || g == 2 || g == 4 || g == 8)) {
    err = "decode rows need num_qo_heads / num_kv_heads in {1, 2, 4, 8} (got " + std::to_string(g) + ")";
    return PKV_E_UNSUPPORTED;
  }
  if (p.kind != PKV_KIND_DECODE && (kPrefillTilePairs % g) != 0) {
    err = "prefill rows need num_qo_heads / num_kv_heads to divide " +
          std::to_string(kPrefillTilePairs) + " (got " + std::to_string(g) + ")";
    return PKV_E_UNSUPPORTED;
  }
  if (p.kind == PKV_KIND_MIXED && p.max_prefill_rows < 0) {
    err = "max_prefill_rows must be >= 0";
    return PKV_E_INVALID;
  }
  if (p.decode_waves_per_cu < 0 || p.decode_min_chunk_pages < 0) {
    err = "tuning knobs must be >= 0 (0 = default)";
    return PKV_E_INVALID;
  }
  const bool any_static = p.static_max_batch != 0 || p.static_max_tokens != 0 ||
                          p.static_max_page_entries != 0;
  if (any_static) {
    if (p.static_max_batch < 1 || p.static_max_tokens < 1 || p.static_max_page_entries < 1) {
      err = "graph-static capacities must all be >= 1 (or all 0)";
      return PKV_E_INVALID;
    }
    if (p.kind == PKV_KIND_DENSE) {
      err = "dense plans have no graph-static mode";
      return PKV_E_UNSUPPORTED;
    }
  }
  return PKV_OK;
}

// Byte offsets of the workspace regions (256-byte aligned): metadata first,
// then the split-KV partials.
void layout_workspace(PlanData& plan) {
  const pkv_plan_params& P = plan.params;
  const int32_t g = plan.group;
  const PlanData::Caps& c = plan.caps;
  const bool st = plan.is_static;
  // region sizes: this plan's counts, or the capacities of a graph-static plan
  const size_t dec_rows = st ? c.dec_rows : plan.decode_rows.size();
  const size_t dec_pieces = st ? c.dec_pieces : plan.decode_pieces.size();
  const size_t dec_work = plan.decode_work.size();  // capacity + 1 when graph-static
  const size_t merges = st ? c.merges : plan.merges.size();
  const size_t pre_tiles = st ? c.prefill_tiles : plan.prefill_tiles.size();
  const size_t indices = st ? c.indices : plan.indices.size();
  const size_t slots = st ? c.tokens : plan.slots.size();
  const size_t n_slots = st ? c.n_slots : (size_t)plan.n_slots;
  WorkspaceLayout& L = plan.ws;
  size_t off = kAlign;  // first 256 bytes: counts (and the upload's sequence number)
  L.off_dense_rows = off;
  off = align_up(off + plan.dense_rows.size() * sizeof(DenseRowMeta));
  L.off_decode_rows = off;
  off = align_up(off + dec_rows * sizeof(DecodeRowMeta));
  L.off_decode_tiles = off;
  off = align_up(off + dec_pieces * sizeof(DecodePieceMeta));
  L.off_decode_work = off;
  off = align_up(off + dec_work * sizeof(int32_t));
  L.off_merges = off;
  off = align_up(off + merges * sizeof(pkv_merge_entry));
  L.off_prefill_tiles = off;
  off = align_up(off + pre_tiles * sizeof(pkv_prefill_tile));
  L.off_indices = off;
  off = align_up(off + indices * sizeof(int32_t));
  L.off_slots = off;
  off = align_up(off + slots * sizeof(int64_t));
  L.meta_bytes = off;
  L.off_part_o = off;
  off = align_up(off + n_slots * g * P.head_dim * sizeof(float));
  L.off_part_lse = off;
  off = align_up(off + n_slots * g * sizeof(float));
  L.total_bytes = off;
}

// Capacities of a graph-static plan.  Decode: W workers (fixed by the
// parameters); every worker boundary cuts at most one row, so at most
// rows + W - 1 pieces; a split row of n pieces owns Hk * n partial slots, so at
// most Hk * (rows + W) slots; a row splits into at most Hk merges.  Prefill
// tiles: Hk per block of kPrefillTilePairs / group tokens, at most
// Hk * (ceil(tokens / block) + rows).
PlanData::Caps static_caps(const pkv_plan_params& P, int32_t num_cus) {
  PlanData::Caps c;
  const int64_t Hk = P.num_kv_heads, g = P.num_qo_heads / P.num_kv_heads;
  const int64_t B = P.static_max_batch, T = P.static_max_tokens;
  if (P.kind != PKV_KIND_PREFILL) {
    c.dec_rows = B;
    c.dec_workers = decode_workers(P, num_cus);
    c.dec_pieces = B + c.dec_workers;
    c.merges = Hk * B;
    c.n_slots = Hk * c.dec_pieces;
  }
  if (P.kind != PKV_KIND_DECODE) {
    const int64_t bt = kPrefillTilePairs / g;
    const int64_t rows = P.kind == PKV_KIND_MIXED ? std::min<int64_t>(B, P.max_prefill_rows) : B;
    c.prefill_tiles = Hk * ((T + bt - 1) / bt + rows);
  }
  c.indices = P.static_max_page_entries;
  c.tokens = T;
  return c;
}

pkv_status build_plan(const pkv_plan_params& P, int32_t num_cus, int32_t batch,
                      const int32_t* qo_indptr, const int32_t* kv_indptr,
                      const int32_t* kv_indices, const int32_t* last_page_len,
                      const int32_t* kv_lens, PlanData& out, std::string& err) {
  pkv_status st = check_params(P, err);
  if (st != PKV_OK) return st;
  if (num_cus < 1) {
    err = "num_cus must be >= 1";
    return PKV_E_INVALID;
  }
  if (batch < 0) {
    err = "batch must be >= 0";
    return PKV_E_INVALID;
  }
  const bool decode_kind = P.kind == PKV_KIND_DECODE;
  if (decode_kind && qo_indptr != nullptr) {
    err = "qo_indptr must be NULL for a decode plan (one query per row)";
    return PKV_E_INVALID;
  }
  if (!decode_kind && qo_indptr == nullptr) {
    err = "qo_indptr is required for prefill and mixed plans";
    return PKV_E_INVALID;
  }
  if (batch > 0 && (kv_indptr == nullptr || last_page_len == nullptr)) {
    err = "paged_kv_indptr and paged_kv_last_page_len are required";
    return PKV_E_INVALID;
  }
  const int64_t ps = P.page_size;
  const int32_t Hk = P.num_kv_heads;
  const int32_t g = P.num_qo_heads / P.num_kv_heads;
  const int64_t w = P.window_left;

  // ---- page table: kv.plan PagedIndptrs / SequenceView.last_page_len ----
  std::vector<int32_t> kv_len(batch), q_len(batch), q_start(batch);
  if (batch > 0 && kv_indptr[0] != 0) {
    err = "paged_kv_indptr[0] must be 0";
    return PKV_E_INVALID;
  }
  if (!decode_kind && qo_indptr[0] != 0) {
    err = "qo_indptr[0] must be 0";
    return PKV_E_INVALID;
  }
  for (int32_t r = 0; r < batch; ++r) {
    const int64_t np = (int64_t)kv_indptr[r + 1] - kv_indptr[r];
    if (np < 1) {
      err = fmt_row("every row needs at least one page", r);
      return PKV_E_INVALID;
    }
    const int64_t lpl = last_page_len[r];
    if (lpl < 1 || lpl > ps) {
      err = fmt_row("paged_kv_last_page_len must be in [1, page_size]", r);
      return PKV_E_INVALID;
    }
    const int64_t n = (np - 1) * ps + lpl;
    if (n > INT32_MAX) {
      err = fmt_row("kv_len exceeds 2^31-1", r);
      return PKV_E_INVALID;
    }
    kv_len[r] = (int32_t)n;
    if (kv_lens != nullptr && kv_lens[r] != n) {
      err = fmt_row("kv_lens disagrees with the page table", r);
      return PKV_E_INVALID;
    }
    int64_t L = 1, qs = r;
    if (!decode_kind) {
      L = (int64_t)qo_indptr[r + 1] - qo_indptr[r];
      qs = qo_indptr[r];
    }
    if (L < 0 || L > n) {
      err = fmt_row("query count must be in [0, kv_len]", r);
      return PKV_E_INVALID;
    }
    q_len[r] = (int32_t)L;
    q_start[r] = (int32_t)qs;
  }
  const int64_t nnz = batch > 0 ? kv_indptr[batch] : 0;
  if (nnz > 0 && kv_indices == nullptr) {
    err = "paged_kv_indices is required";
    return PKV_E_INVALID;
  }
  for (int64_t i = 0; i < nnz; ++i) {
    if (kv_indices[i] < 0 || kv_indices[i] >= P.max_pages) {
      err = "page id " + std::to_string(kv_indices[i]) + " at index " + std::to_string(i) +
            " outside [0, max_pages)";
      return PKV_E_INVALID;
    }
  }
  const int64_t total_q = decode_kind ? batch : (batch > 0 ? qo_indptr[batch] : 0);
  const bool is_static = P.static_max_batch > 0;
  if (is_static && (batch > P.static_max_batch || total_q > P.static_max_tokens ||
                    nnz > P.static_max_page_entries)) {
    err = "the step exceeds the graph-static capacities (batch " + std::to_string(batch) + " / " +
          std::to_string(P.static_max_batch) + ", tokens " + std::to_string(total_q) + " / " +
          std::to_string(P.static_max_tokens) + ", page entries " + std::to_string(nnz) + " / " +
          std::to_string(P.static_max_page_entries) + ")";
    return PKV_E_CAPACITY;
  }

  PlanData plan;
  plan.params = P;
  plan.batch = batch;
  plan.total_q = (int32_t)total_q;
  plan.num_cus = num_cus;
  plan.group = g;
  plan.indices.assign(kv_indices, kv_indices + nnz);

  // ---- rows per sub-plan (FlashInferMixedWrapper: one-token rows decode) ----
  std::vector<int32_t> dec_rows, pre_rows;
  for (int32_t r = 0; r < batch; ++r) {
    if (P.kind == PKV_KIND_DECODE) dec_rows.push_back(r);
    else if (P.kind == PKV_KIND_PREFILL) { if (q_len[r] >= 1) pre_rows.push_back(r); }
    else if (q_len[r] == 1) dec_rows.push_back(r);
    else if (q_len[r] >= 2) pre_rows.push_back(r);
  }
  if (P.kind == PKV_KIND_MIXED && (int64_t)pre_rows.size() > P.max_prefill_rows) {
    err = std::to_string(pre_rows.size()) + " prompt rows exceed max_prefill_rows=" +
          std::to_string(P.max_prefill_rows);
    return PKV_E_CAPACITY;
  }
  plan.n_decode_rows = (int32_t)dec_rows.size();
  plan.n_prompt_rows = P.kind == PKV_KIND_MIXED ? (int32_t)pre_rows.size() : 0;

  // ---- write slots (FlashInferDecodeWrapper.plan; KVPlanOutput decode_pages/offsets) ----
  plan.slots.resize(total_q);
  for (int32_t r = 0; r < batch; ++r) {
    const int64_t n = kv_len[r], L = q_len[r];
    for (int64_t t = 0; t < L; ++t) {
      const int64_t p = n - L + t;
      const int64_t page = kv_indices[kv_indptr[r] + p / ps];
      plan.slots[q_start[r] + t] = page * ps + p % ps;
    }
  }
  {
    // Every written page entry of a row takes an interval of offsets [lo, hi]
    // of its page; two tokens share a slot exactly when two intervals of the
    // same page overlap.  Sorting the intervals (about T / ps + rows of them)
    // finds that without a set of all T slots.
    struct Iv { int64_t page; int32_t lo, hi; int64_t tok; };
    std::vector<Iv> ivs;
    for (int32_t r = 0; r < batch; ++r) {
      const int64_t n = kv_len[r], L = q_len[r];
      for (int64_t p = n - L; p < n;) {
        const int64_t e = p / ps, pend = std::min(n, (e + 1) * ps);
        ivs.push_back({kv_indices[kv_indptr[r] + e], (int32_t)(p % ps),
                       (int32_t)((pend - 1) % ps), q_start[r] + (p - (n - L))});
        p = pend;
      }
    }
    std::sort(ivs.begin(), ivs.end(), [](const Iv& a, const Iv& b) {
      return a.page != b.page ? a.page < b.page : a.lo < b.lo;
    });
    for (size_t i = 1; i < ivs.size(); ++i) {
      if (ivs[i].page == ivs[i - 1].page && ivs[i].lo <= ivs[i - 1].hi) {
        err = "two appended tokens map to cache slot " +
              std::to_string(ivs[i].page * ps + ivs[i].lo) + " (token " +
              std::to_string(ivs[i].tok) + ")";
        return PKV_E_CONFLICT;
      }
    }
  }

  // ---- mixed permutation: prompt tokens first, rows ascending ----
  if (P.kind == PKV_KIND_MIXED) {
    for (int32_t r : pre_rows)
      for (int32_t t = 0; t < q_len[r]; ++t) plan.perm.push_back(q_start[r] + t);
  }

  // ---- decode pieces, workers and split-KV partials ----
  const int64_t min_chunk = P.decode_min_chunk_pages > 0 ? P.decode_min_chunk_pages : 8;
  const int64_t W = decode_workers(P, num_cus);
  struct DecRow { int32_t r; int64_t lo, fp, lp, vis; };
  std::vector<DecRow> drows;
  drows.reserve(dec_rows.size());
  for (int32_t r : dec_rows) {
    const int64_t n = kv_len[r];
    const int64_t lo = w < 0 ? 0 : std::max<int64_t>(0, n - 1 - w);
    const int64_t fp = lo / ps, lp = (n - 1) / ps;
    drows.push_back({r, lo, fp, lp, lp - fp + 1});
  }
  std::stable_sort(drows.begin(), drows.end(),
                   [](const DecRow& a, const DecRow& b) { return a.vis > b.vis; });
  std::vector<int64_t> vis(drows.size());
  int64_t total = 0;
  for (size_t i = 0; i < drows.size(); ++i) {
    vis[i] = drows[i].vis;
    total += drows[i].vis + kPieceCost;
  }
  int64_t cap = std::max(min_chunk, (total + W - 1) / W) + kPieceCost;
  if (!drows.empty())
    while (pour(vis, cap, [](size_t, int64_t, int64_t, int64_t) {}) > W) ++cap;
  plan.worker_pages = (int32_t)std::min<int64_t>(cap, INT32_MAX);
  // pieces per row (the same for every KV head), then slots and merges
  std::vector<int64_t> n_pieces(drows.size(), 0);
  pour(vis, cap, [&](size_t i, int64_t, int64_t, int64_t) { ++n_pieces[i]; });
  std::vector<int64_t> slot0(drows.size(), -1);
  int64_t slot = 0;
  plan.decode_rows.reserve(drows.size());
  for (size_t i = 0; i < drows.size(); ++i) {
    const DecRow& d = drows[i];
    const int64_t nch = n_pieces[i];
    DecodeRowMeta rm{};
    rm.page_base = kv_indptr[d.r];
    rm.q_index = q_start[d.r];
    rm.kv_len = kv_len[d.r];
    rm.slot0 = nch > 1 ? (int32_t)std::min<int64_t>(slot, INT32_MAX) : -1;
    rm.n_chunks = (int32_t)nch;
    plan.decode_rows.push_back(rm);
    if (nch > 1) {
      slot0[i] = slot;
      for (int32_t hk = 0; hk < Hk; ++hk)
        plan.merges.push_back({q_start[d.r], hk, (int32_t)(slot + hk * nch), (int32_t)nch});
      slot += Hk * nch;
      plan.max_merge_chunks = std::max(plan.max_merge_chunks, (int32_t)nch);
    }
    if (slot > INT32_MAX) {
      err = "too many split-KV partials";
      return PKV_E_INVALID;
    }
  }
  plan.n_slots = (int32_t)slot;
  // the pieces, in pour order, and each worker's piece range
  std::vector<int64_t> chunk_of(drows.size(), 0);
  int64_t last_worker = -1;
  pour(vis, cap, [&](size_t i, int64_t off, int64_t take, int64_t wk) {
    const DecRow& d = drows[i];
    const int64_t n = kv_len[d.r];
    const int64_t p0 = d.fp + off, p1 = p0 + take;
    const int32_t ks = (int32_t)std::max(d.lo, p0 * ps);
    const int32_t ke = (int32_t)std::min(n, p1 * ps);
    const int32_t ch = (int32_t)chunk_of[i]++;
    while (last_worker < wk) {
      plan.decode_work.push_back((int32_t)plan.decode_pieces.size());
      ++last_worker;
    }
    plan.decode_pieces.push_back({(int32_t)i, ch, ks, ke});
    for (int32_t hk = 0; hk < Hk; ++hk) {
      pkv_decode_tile t;
      t.row = d.r;
      t.kv_head = hk;
      t.kv_start = ks;
      t.kv_end = ke;
      t.page_base = kv_indptr[d.r];
      t.q_index = q_start[d.r];
      t.out_slot = slot0[i] >= 0 ? (int32_t)(slot0[i] + hk * n_pieces[i] + ch) : -1;
      t.kv_len = (int32_t)n;
      plan.decode_tiles.push_back(t);
    }
  });
  plan.n_workers = (int32_t)(last_worker + 1);
  plan.decode_work.push_back((int32_t)plan.decode_pieces.size());

  // ---- prefill tiles ----
  make_prefill_tiles(P, pre_rows, kv_len, q_len, q_start,
                     [&](int32_t r) { return kv_indptr[r]; }, plan.prefill_tiles);

  if (is_static) {
    plan.is_static = true;
    plan.caps = static_caps(P, num_cus);
    const PlanData::Caps& c = plan.caps;
    if ((int64_t)plan.decode_rows.size() > c.dec_rows ||
        (int64_t)plan.decode_pieces.size() > c.dec_pieces || plan.n_workers > c.dec_workers ||
        (int64_t)plan.merges.size() > c.merges || plan.n_slots > c.n_slots ||
        (int64_t)plan.prefill_tiles.size() > c.prefill_tiles) {
      err = "internal: a graph-static plan outgrew its capacities";
      return PKV_E_CAPACITY;
    }
    // every worker of the capacity grid reads its range: the unused ones get
    // empty ranges at the end
    plan.decode_work.resize(c.dec_workers + 1, (int32_t)plan.decode_pieces.size());
  }
  layout_workspace(plan);
  out = std::move(plan);
  return PKV_OK;
}

void serialize_meta(const PlanData& plan, void* dst) {
  char* base = static_cast<char*>(dst);
  std::memset(base, 0, plan.ws.meta_bytes);
  const int64_t hdr[8] = {(int64_t)plan.decode_pieces.size(), (int64_t)plan.merges.size(),
                          (int64_t)plan.prefill_tiles.size(), (int64_t)plan.indices.size(),
                          (int64_t)plan.slots.size(), plan.n_slots, plan.total_q, plan.batch};
  std::memcpy(base, hdr, sizeof(hdr));
  auto put = [&](size_t off, const void* src, size_t bytes) {
    if (bytes) std::memcpy(base + off, src, bytes);
  };
  put(plan.ws.off_dense_rows, plan.dense_rows.data(),
      plan.dense_rows.size() * sizeof(DenseRowMeta));
  put(plan.ws.off_decode_rows, plan.decode_rows.data(),
      plan.decode_rows.size() * sizeof(DecodeRowMeta));
  put(plan.ws.off_decode_tiles, plan.decode_pieces.data(),
      plan.decode_pieces.size() * sizeof(DecodePieceMeta));
  put(plan.ws.off_decode_work, plan.decode_work.data(),
      plan.decode_work.size() * sizeof(int32_t));
  put(plan.ws.off_merges, plan.merges.data(), plan.merges.size() * sizeof(pkv_merge_entry));
  put(plan.ws.off_prefill_tiles, plan.prefill_tiles.data(),
      plan.prefill_tiles.size() * sizeof(pkv_prefill_tile));
  put(plan.ws.off_indices, plan.indices.data(), plan.indices.size() * sizeof(int32_t));
  put(plan.ws.off_slots, plan.slots.data(), plan.slots.size() * sizeof(int64_t));
}

// kv.plan context_only_views: each row keeps its first kv_len - to_compute
// tokens (the pages past them dropped) and gets query_spans[r] queries.
pkv_status context_only_views(int32_t batch, int32_t page_size, const int32_t* kv_indptr,
                              const int32_t* kv_indices, const int32_t* last_page_len,
                              const int32_t* to_compute, const int32_t* query_spans,
                              int32_t* out_indptr, int32_t* out_indices,
                              int32_t* out_last_page_len, int32_t* out_qo_indptr,
                              std::string& err) {
  if (batch < 0) {
    err = "batch must be >= 0";
    return PKV_E_INVALID;
  }
  if (!is_pow2(page_size) || page_size > 256) {
    err = "page_size must be a power of two in [1, 256] (got " + std::to_string(page_size) + ")";
    return PKV_E_UNSUPPORTED;
  }
  if (kv_indptr == nullptr || out_indptr == nullptr || out_qo_indptr == nullptr ||
      (batch > 0 && (kv_indices == nullptr || last_page_len == nullptr || to_compute == nullptr ||
                     query_spans == nullptr || out_indices == nullptr ||
                     out_last_page_len == nullptr))) {
    err = "NULL array";
    return PKV_E_INVALID;
  }
  if (kv_indptr[0] != 0) {
    err = "paged_kv_indptr[0] must be 0";
    return PKV_E_INVALID;
  }
  out_indptr[0] = 0;
  out_qo_indptr[0] = 0;
  int64_t nnz = 0, nq = 0;
  for (int32_t r = 0; r < batch; ++r) {
    const int64_t np = (int64_t)kv_indptr[r + 1] - kv_indptr[r];
    if (np < 1) {
      err = fmt_row("every row needs at least one page", r);
      return PKV_E_INVALID;
    }
    const int32_t lpl = last_page_len[r];
    if (lpl < 1 || lpl > page_size) {
      err = fmt_row("paged_kv_last_page_len must be in [1, page_size]", r);
      return PKV_E_INVALID;
    }
    const int64_t n = (np - 1) * page_size + lpl;
    const int64_t tc = to_compute[r], qs = query_spans[r];
    if (tc < 0 || tc >= n) {
      err = fmt_row("to_compute must be in [0, kv_len): a row keeps at least one stored token", r);
      return PKV_E_INVALID;
    }
    if (qs < 0) {
      err = fmt_row("query_spans must be >= 0", r);
      return PKV_E_INVALID;
    }
    const int64_t kept = n - tc;
    const int64_t kp = (kept + page_size - 1) / page_size;
    for (int64_t i = 0; i < kp; ++i) out_indices[nnz + i] = kv_indices[kv_indptr[r] + i];
    nnz += kp;
    nq += qs;
    if (nq > INT32_MAX) {
      err = "more than 2^31 - 1 query tokens";
      return PKV_E_INVALID;
    }
    out_indptr[r + 1] = (int32_t)nnz;
    out_last_page_len[r] = (int32_t)(kept - (kp - 1) * page_size);
    out_qo_indptr[r + 1] = (int32_t)nq;
  }
  return PKV_OK;
}

// attn.dense DensePlan: row r's queries are rows [cu_q[r], cu_q[r+1]) of q and
// its keys rows [cu_k[r], cu_k[r+1]) of the contiguous K/V, the last q_len of
// them fresh (bottom-right causal alignment as for a paged row).
pkv_status build_dense_plan(const pkv_plan_params& P, int32_t num_cus, int32_t batch,
                            const int32_t* cu_q, const int32_t* cu_k, const int32_t* kv_indptr,
                            const int32_t* kv_indices, PlanData& out, std::string& err) {
  pkv_status st = check_params(P, err);
  if (st != PKV_OK) return st;
  if (P.kind != PKV_KIND_DENSE) {
    err = "a dense plan needs kind PKV_KIND_DENSE";
    return PKV_E_INVALID;
  }
  if (num_cus < 1 || batch < 0) {
    err = "num_cus must be >= 1 and batch >= 0";
    return PKV_E_INVALID;
  }
  if (cu_q == nullptr || cu_k == nullptr) {
    err = "cu_q and cu_k are required";
    return PKV_E_INVALID;
  }
  if ((kv_indptr == nullptr) != (kv_indices == nullptr)) {
    err = "paged_kv_indptr and paged_kv_indices must both be given or both be NULL";
    return PKV_E_INVALID;
  }
  if (cu_q[0] != 0 || cu_k[0] != 0) {
    err = "cu_q[0] and cu_k[0] must be 0";
    return PKV_E_INVALID;
  }
  const bool pages = kv_indptr != nullptr;
  if (pages && kv_indptr[0] != 0) {
    err = "paged_kv_indptr[0] must be 0";
    return PKV_E_INVALID;
  }
  const int64_t ps = P.page_size;
  const int64_t row_bytes = (int64_t)P.num_kv_heads * P.head_dim * 2;
  PlanData plan;
  plan.params = P;
  plan.batch = batch;
  plan.num_cus = num_cus;
  plan.group = P.num_qo_heads / P.num_kv_heads;
  plan.dense = true;
  plan.dense_pages = pages;
  std::vector<int32_t> kv_len(batch), q_len(batch), q_start(batch), rows;
  for (int32_t r = 0; r < batch; ++r) {
    const int64_t L = (int64_t)cu_q[r + 1] - cu_q[r], N = (int64_t)cu_k[r + 1] - cu_k[r];
    if (L < 0 || N < 0) {
      err = fmt_row("cu_q and cu_k must be non-decreasing", r);
      return PKV_E_INVALID;
    }
    if (L > N) {
      err = fmt_row("a row's query count must not exceed its key count", r);
      return PKV_E_INVALID;
    }
    // the kernel addresses a row's keys with 32-bit byte offsets
    if ((N + 64) * row_bytes >= (int64_t)1 << 32) {
      err = fmt_row("a row's K (or V) must stay below 4 GiB", r);
      return PKV_E_INVALID;
    }
    const int64_t prefix = N - L;
    DenseRowMeta m{};
    m.cu_k = cu_k[r];
    m.cu_q = cu_q[r];
    m.prefix = (int32_t)prefix;
    m.fresh = (int32_t)L;
    if (pages) {
      const int64_t np = (int64_t)kv_indptr[r + 1] - kv_indptr[r];
      if (np < 0 || np * ps < prefix) {
        err = fmt_row("the row's pages hold fewer tokens than its prefix", r);
        return PKV_E_INVALID;
      }
      for (int64_t i = 0; i < (prefix + ps - 1) / ps; ++i) {
        const int32_t id = kv_indices[kv_indptr[r] + i];
        if (id < 0 || id >= P.max_pages) {
          err = fmt_row("page id outside [0, max_pages)", r);
          return PKV_E_INVALID;
        }
      }
      m.page_base = kv_indptr[r];
    }
    plan.dense_rows.push_back(m);
    kv_len[r] = (int32_t)N;
    q_len[r] = (int32_t)L;
    q_start[r] = cu_q[r];
    if (L >= 1) rows.push_back(r);
  }
  plan.total_q = batch > 0 ? cu_q[batch] : 0;
  plan.total_k = batch > 0 ? cu_k[batch] : 0;
  if (pages) plan.indices.assign(kv_indices, kv_indices + (batch > 0 ? kv_indptr[batch] : 0));
  make_prefill_tiles(P, rows, kv_len, q_len, q_start, [&](int32_t r) { return cu_k[r]; },
                     plan.prefill_tiles);
  layout_workspace(plan);
  out = std::move(plan);
  return PKV_OK;
}

}  // namespace pkv
