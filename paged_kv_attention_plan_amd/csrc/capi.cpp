// The C ABI declared in include/pkv.h: plan handles, the pinned staging ring,
// upload, run and append.  Argument checks happen here, before any launch.
#include <hip/hip_runtime.h>

#include <chrono>
#include <cmath>
#include <cstring>
#include <thread>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"
#include "pkv.h"
#include "handle.h"
#include "plan.h"
#include "stage.h"

namespace {

thread_local std::string g_err;

using pkv::detail::fail;

#define PKV_HIP(expr)                                                                    \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess)                                                                \
      return fail(PKV_E_DEVICE, std::string(#expr) + " failed: " + hipGetErrorString(e_)); \
  } while (0)

constexpr int kUploadBlocks = 256;  // most workgroups one upload launches
// A staging buffer whose readers have not finished after this long counts as
// a failed GPU.
constexpr std::chrono::seconds kStageTimeout(60);

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

namespace {

enum { kAppend = 0, kDecode = 1, kMerge = 2, kPrefill = 3 };

// Record an event on `s` if timing is on; returns the event (or null).
hipError_t timing_mark(const pkv_plan* p, hipStream_t s, int kind, bool begin) {
  Timing& t = p->timing;
  if (!t.enabled) return hipSuccess;
  if (begin) {
    if (t.used + 2 > t.pool.size()) {
      for (int i = 0; i < 2; ++i) {
        hipEvent_t e = nullptr;
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) return err;
        t.pool.push_back(e);
      }
    }
    t.kind.push_back(kind);
    return hipEventRecord(t.pool[t.used], s);
  }
  hipError_t err = hipEventRecord(t.pool[t.used + 1], s);
  t.used += 2;
  return err;
}

}  // namespace

pkv_status pkv::detail::fail(pkv_status s, std::string msg) {
  g_err = std::move(msg);
  return s;
}

void pkv::detail::clear_error() { g_err.clear(); }

extern "C" {

const char* pkv_last_error(void) { return g_err.c_str(); }

const char* pkv_version(void) { return "pkv 0.1 gfx950"; }

void pkv_plan_params_init(pkv_plan_params* p) {
  if (p == nullptr) return;
  std::memset(p, 0, sizeof(*p));
  p->kind = PKV_KIND_DECODE;
  p->causal = 1;
  p->window_left = -1;
  p->dtype = PKV_DTYPE_BF16;
}

static pkv_status resolve_cus(const pkv_plan_params* p, int32_t* cus) {
  if (p->num_cus > 0) {
    *cus = p->num_cus;
    return PKV_OK;
  }
  int dev = 0, n = 0;
  PKV_HIP(hipGetDevice(&dev));
  PKV_HIP(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev));
  *cus = n;
  return PKV_OK;
}

pkv_status pkv_plan_create(const pkv_plan_params* params, int32_t batch, const int32_t* qo_indptr,
                           const int32_t* paged_kv_indptr, const int32_t* paged_kv_indices,
                           const int32_t* paged_kv_last_page_len, const int32_t* kv_lens,
                           pkv_plan** out, size_t* workspace_bytes) {
  g_err.clear();
  if (params == nullptr || out == nullptr || workspace_bytes == nullptr)
    return fail(PKV_E_INVALID, "params, out and workspace_bytes must not be NULL");
  *out = nullptr;
  std::string err;
  pkv_status st = pkv::check_params(*params, err);
  if (st != PKV_OK) return fail(st, err);
  if (params->kind == PKV_KIND_DENSE)
    return fail(PKV_E_INVALID, "dense plans are built by pkv_dense_plan_create");
  int32_t cus = 0;
  st = resolve_cus(params, &cus);
  if (st != PKV_OK) return st;
  pkv_plan* p = new (std::nothrow) pkv_plan;
  if (p == nullptr) return fail(PKV_E_INVALID, "out of host memory");
  st = pkv::build_plan(*params, cus, batch, qo_indptr, paged_kv_indptr, paged_kv_indices,
                       paged_kv_last_page_len, kv_lens, p->d, err);
  if (st != PKV_OK) {
    delete p;
    return fail(st, err);
  }
  *workspace_bytes = p->d.ws.total_bytes;
  *out = p;
  return PKV_OK;
}

pkv_status pkv_plan_update(pkv_plan* plan, int32_t batch, const int32_t* qo_indptr,
                           const int32_t* paged_kv_indptr, const int32_t* paged_kv_indices,
                           const int32_t* paged_kv_last_page_len, const int32_t* kv_lens,
                           size_t* workspace_bytes) {
  g_err.clear();
  if (plan == nullptr || workspace_bytes == nullptr)
    return fail(PKV_E_INVALID, "plan and workspace_bytes must not be NULL");
  if (plan->d.dense) return fail(PKV_E_INVALID, "dense plans are re-planned by pkv_dense_plan_update");
  pkv::PlanData fresh;
  std::string err;
  pkv_status st = pkv::build_plan(plan->d.params, plan->d.num_cus, batch, qo_indptr,
                                  paged_kv_indptr, paged_kv_indices, paged_kv_last_page_len,
                                  kv_lens, fresh, err);
  if (st != PKV_OK) return fail(st, err);
  plan->d = std::move(fresh);
  plan->uploaded_ws = nullptr;
  *workspace_bytes = plan->d.ws.total_bytes;
  return PKV_OK;
}

void pkv_plan_destroy(pkv_plan* plan) {
  if (plan == nullptr) return;
  for (hipEvent_t e : plan->timing.pool) (void)hipEventDestroy(e);
  for (pkv::Stage& s : plan->ring.stage) {
    // A buffer the GPU may still read is not freed (it leaks if the GPU failed).
    if (s.host != nullptr && pkv::wait_stage(s, kStageTimeout)) (void)hipHostFree(s.host);
  }
  delete plan;
}

pkv_status pkv_plan_decode_tiles(const pkv_plan* plan, const pkv_decode_tile** tiles, int32_t* n) {
  if (plan == nullptr || tiles == nullptr || n == nullptr) return fail(PKV_E_INVALID, "NULL argument");
  *tiles = plan->d.decode_tiles.data();
  *n = (int32_t)plan->d.decode_tiles.size();
  return PKV_OK;
}

pkv_status pkv_plan_prefill_tiles(const pkv_plan* plan, const pkv_prefill_tile** tiles, int32_t* n) {
  if (plan == nullptr || tiles == nullptr || n == nullptr) return fail(PKV_E_INVALID, "NULL argument");
  *tiles = plan->d.prefill_tiles.data();
  *n = (int32_t)plan->d.prefill_tiles.size();
  return PKV_OK;
}

pkv_status pkv_plan_merges(const pkv_plan* plan, const pkv_merge_entry** merges, int32_t* n) {
  if (plan == nullptr || merges == nullptr || n == nullptr) return fail(PKV_E_INVALID, "NULL argument");
  *merges = plan->d.merges.data();
  *n = (int32_t)plan->d.merges.size();
  return PKV_OK;
}

pkv_status pkv_plan_write_slots(const pkv_plan* plan, const int64_t** slots, int32_t* n) {
  if (plan == nullptr || slots == nullptr || n == nullptr) return fail(PKV_E_INVALID, "NULL argument");
  *slots = plan->d.slots.data();
  *n = (int32_t)plan->d.slots.size();
  return PKV_OK;
}

pkv_status pkv_plan_metadata(const pkv_plan* plan, void* dst, size_t bytes) {
  g_err.clear();
  if (plan == nullptr || dst == nullptr) return fail(PKV_E_INVALID, "NULL argument");
  if (bytes < plan->d.ws.meta_bytes)
    return fail(PKV_E_WORKSPACE, "the metadata image needs " +
                                     std::to_string(plan->d.ws.meta_bytes) + " bytes");
  pkv::serialize_meta(plan->d, dst);
  return PKV_OK;
}

pkv_status pkv_plan_permutation(const pkv_plan* plan, const int32_t** perm, int32_t* n) {
  if (plan == nullptr || perm == nullptr || n == nullptr) return fail(PKV_E_INVALID, "NULL argument");
  *perm = plan->d.perm.data();
  *n = (int32_t)plan->d.perm.size();
  return PKV_OK;
}

pkv_status pkv_plan_info(const pkv_plan* plan, int64_t info[18]) {
  if (plan == nullptr || info == nullptr) return fail(PKV_E_INVALID, "NULL argument");
  const pkv::PlanData& d = plan->d;
  for (int i = 0; i < 18; ++i) info[i] = 0;
  info[0] = d.total_q;
  info[1] = d.batch;
  info[2] = d.n_decode_rows;
  info[3] = d.n_prompt_rows;
  info[4] = d.worker_pages;
  info[5] = d.n_slots;
  info[6] = (int64_t)d.ws.meta_bytes;
  info[7] = (int64_t)d.ws.total_bytes;
  info[8] = d.num_cus;
  info[9] = d.total_k;
  info[10] = (int64_t)d.ws.off_dense_rows;
  info[11] = (int64_t)d.ws.off_decode_rows;
  info[12] = (int64_t)d.ws.off_decode_tiles;
  info[13] = (int64_t)d.ws.off_merges;
  info[14] = (int64_t)d.ws.off_prefill_tiles;
  info[15] = (int64_t)d.ws.off_indices;
  info[16] = (int64_t)d.ws.off_decode_work;
  info[17] = d.is_static ? d.caps.dec_workers : d.n_workers;
  return PKV_OK;
}

pkv_status pkv_plan_upload_stats(const pkv_plan* plan, int64_t stats[3]) {
  if (plan == nullptr || stats == nullptr) return fail(PKV_E_INVALID, "NULL argument");
  stats[0] = plan->ring.uploads;
  stats[1] = plan->ring.waits;
  stats[2] = plan->ring.wait_ns;
  return PKV_OK;
}

static pkv_status check_paged(const pkv_plan* plan) {
  if (plan != nullptr && plan->d.dense)
    return fail(PKV_E_INVALID, "a dense plan runs through pkv_dense_gather / pkv_dense_run");
  return PKV_OK;
}

static pkv_status check_workspace(const pkv_plan* plan, const void* ws, size_t ws_bytes) {
  const size_t need = plan->d.ws.total_bytes;
  if (ws == nullptr) return fail(PKV_E_INVALID, "workspace must not be NULL");
  if (ws_bytes < need)
    return fail(PKV_E_WORKSPACE,
                "workspace holds " + std::to_string(ws_bytes) + " bytes; this plan needs " +
                    std::to_string(need) + " (plan metadata " + std::to_string(plan->d.ws.meta_bytes) +
                    " + split-KV partials " + std::to_string(need - plan->d.ws.meta_bytes) +
                    "); pass a workspace of at least workspace_bytes");
  return PKV_OK;
}

}  // extern "C"

namespace {

// (Re-)allocate a staging buffer of `cap` bytes plus its completion flags.
// Page-locked and coherent: the upload kernel reads it over the host link,
// never from a stale cache line of an earlier step, and its flag stores reach
// the host.  The buffer must have no reader in flight.
hipError_t grow_stage(pkv::Stage& s, size_t cap) {
  if (s.host != nullptr) {
    hipError_t e = hipHostFree(s.host);
    if (e != hipSuccess) return e;
  }
  s.host = nullptr;
  s.dev = nullptr;
  s.cap = 0;
  hipError_t e = hipHostMalloc(&s.host, cap + kUploadBlocks * sizeof(uint32_t), hipHostMallocCoherent);
  if (e != hipSuccess) return e;
  s.cap = cap;
  e = hipHostGetDevicePointer(&s.dev, s.host, 0);
  if (e != hipSuccess) return e;
  for (int i = 0; i < kUploadBlocks; ++i) s.flags()[i] = s.seq;
  return hipSuccess;
}

}  // namespace

pkv_status pkv::detail::upload_meta(pkv_plan* plan, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream, bool may_allocate) {
  pkv_status st = check_workspace(plan, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  const size_t meta = plan->d.ws.meta_bytes;
  // The buffer this upload rewrites is free once every workgroup of the
  // upload that last read it has stored its completion flag.
  pkv::Stage* sp = plan->ring.acquire(kStageTimeout);
  if (sp == nullptr)
    return fail(PKV_E_DEVICE, "a staging buffer's upload did not finish within 60 s");
  pkv::Stage& s = *sp;
  if (s.cap < meta && !may_allocate)
    return fail(PKV_E_CAPACITY,
                "the plan's staging buffer holds " + std::to_string(s.cap) + " bytes and its metadata needs " +
                    std::to_string(meta) + ": upload the plan (or a larger one) once with pkv_plan_upload, "
                    "which sizes both staging buffers");
  if (s.cap < meta) {
    // Both buffers of the ring grow together (the other one after its last
    // reader is done), so that an upload that may not allocate finds either
    // one large enough.
    pkv::Stage& other = plan->ring.stage[plan->ring.next ^ 1];
    if (!pkv::wait_stage(other, kStageTimeout))
      return fail(PKV_E_DEVICE, "a staging buffer's upload did not finish within 60 s");
    size_t cap = 4096;
    while (cap < meta) cap <<= 1;
    PKV_HIP(grow_stage(s, cap));
    if (other.cap < cap) PKV_HIP(grow_stage(other, cap));
  }
  pkv::serialize_meta(plan->d, s.host);
  hipStream_t st_ = stream;
  pkv::UploadArgs ua{};
  ua.src = static_cast<const uint4*>(s.dev);
  ua.dst = static_cast<uint4*>(workspace);
  ua.n_vec = (int64_t)(meta / 16);  // meta_bytes is a multiple of 256
  ua.flags = reinterpret_cast<uint32_t*>(static_cast<char*>(s.dev) + s.cap);
  ua.seq = plan->ring.next_seq();
  ua.max_blocks = kUploadBlocks;
  int blocks = 0;
  PKV_HIP(pkv::launch_upload(ua, st_, &blocks));
  plan->ring.launched(blocks);
  plan->uploaded_ws = workspace;
  return PKV_OK;
}

extern "C" {

pkv_status pkv_plan_upload(pkv_plan* plan, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (plan == nullptr) return fail(PKV_E_INVALID, "plan must not be NULL");
  return pkv::detail::upload_meta(plan, workspace, workspace_bytes, static_cast<hipStream_t>(stream),
                                  true);
}

namespace {

// Argument checks shared by pkv_run and pkv_run_append.
pkv_status check_run(const pkv_plan* plan, const void* q, const void* kv_cache_layer, void* out,
                     float* lse, void* workspace, size_t workspace_bytes) {
  if (plan == nullptr) return fail(PKV_E_INVALID, "plan must not be NULL");
  if (check_paged(plan) != PKV_OK) return PKV_E_INVALID;
  pkv_status st = check_workspace(plan, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  if (plan->uploaded_ws != workspace)
    return fail(PKV_E_STATE, "the plan was not uploaded to this workspace (call pkv_plan_upload first)");
  if (plan->d.total_q == 0 && !plan->d.is_static) return PKV_OK;
  if (q == nullptr || kv_cache_layer == nullptr || out == nullptr)
    return fail(PKV_E_INVALID, "q, kv_cache_layer and out must not be NULL");
  if (!aligned16(q) || !aligned16(kv_cache_layer) || !aligned16(out) || !aligned16(workspace))
    return fail(PKV_E_INVALID, "q, kv_cache_layer, out and workspace must be 16-byte aligned");
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return fail(PKV_E_INVALID, "lse must be 4-byte aligned");
  return PKV_OK;
}

// Launch the plan's kernels (arguments already checked).  timed: record the
// plan's per-kernel timing events when timing is on (which may create events).
pkv_status run_impl(const pkv_plan* plan, const void* q, const void* kv_cache_layer, void* out,
                    float* lse, void* workspace, void* stream, bool timed = true) {
  const pkv::PlanData& d = plan->d;
  const pkv_plan_params& P = d.params;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto mark = [&](int kind, bool begin) {
    return timed ? timing_mark(plan, s, kind, begin) : hipSuccess;
  };
  const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)P.head_dim));
  const int32_t* indices = reinterpret_cast<const int32_t*>(ws + d.ws.off_indices);
  float* part_o = reinterpret_cast<float*>(ws + d.ws.off_part_o);
  float* part_lse = reinterpret_cast<float*>(ws + d.ws.off_part_lse);
  // A graph-static plan launches every kernel its kind can use, on grids sized
  // for its capacities, and the kernels read the step's counts from the header.
  const bool st = d.is_static;
  const int64_t* counts = st ? reinterpret_cast<const int64_t*>(ws) : nullptr;
  const bool has_dec = st ? d.caps.dec_workers > 0 : d.n_workers > 0;
  const bool has_pre = st ? d.caps.prefill_tiles > 0 : !d.prefill_tiles.empty();
  pkv::DecodeArgs da{};
  if (has_dec) {
    // a graph-static plan's worker table always has its capacity's entries
    da.pieces = reinterpret_cast<const pkv::DecodePieceMeta*>(ws + d.ws.off_decode_tiles);
    da.rows = reinterpret_cast<const pkv::DecodeRowMeta*>(ws + d.ws.off_decode_rows);
    da.work = reinterpret_cast<const int32_t*>(ws + d.ws.off_decode_work);
    da.n_workers = (int32_t)(st ? d.caps.dec_workers : (int64_t)d.n_workers);
    da.indices = indices;
    da.q = static_cast<const uint16_t*>(q);
    da.cache = static_cast<const uint16_t*>(kv_cache_layer);
    da.out = static_cast<uint16_t*>(out);
    da.lse = lse;
    da.part_o = part_o;
    da.part_lse = part_lse;
    da.num_qo_heads = P.num_qo_heads;
    da.num_kv_heads = P.num_kv_heads;
    da.head_dim = P.head_dim;
    da.page_size = P.page_size;
    da.group = d.group;
    da.scale_log2 = scale_log2;
  }
  pkv::PrefillArgs pa{};
  if (has_pre) {
    pa.tiles = reinterpret_cast<const pkv_prefill_tile*>(ws + d.ws.off_prefill_tiles);
    pa.n_tiles = (int32_t)(st ? d.caps.prefill_tiles : (int64_t)d.prefill_tiles.size());
    pa.counts = counts;
    pa.indices = indices;
    pa.q = static_cast<const uint16_t*>(q);
    pa.cache = static_cast<const uint16_t*>(kv_cache_layer);
    pa.out = static_cast<uint16_t*>(out);
    pa.lse = lse;
    pa.num_qo_heads = P.num_qo_heads;
    pa.num_kv_heads = P.num_kv_heads;
    pa.head_dim = P.head_dim;
    pa.page_size = P.page_size;
    pa.group = d.group;
    pa.causal = P.causal ? 1 : 0;
    pa.window_left = P.window_left;
    pa.scale_log2 = scale_log2;
  }
  // A mixed step runs its decode waves and prefill tiles in one launch (the
  // two write disjoint tokens); the merge of split decode rows follows.
  const bool fused = has_dec && has_pre && pkv::mixed_launch_fits(da, pa);
  if (fused) {
    PKV_HIP(mark(kDecode, true));
    PKV_HIP(pkv::launch_mixed(da, pa, s));
    PKV_HIP(mark(kDecode, false));
  } else if (has_dec) {
    PKV_HIP(mark(kDecode, true));
    PKV_HIP(pkv::launch_decode(da, s));
    PKV_HIP(mark(kDecode, false));
  }
  if (st ? d.caps.merges > 0 : !d.merges.empty()) {
    pkv::MergeArgs a{};
    a.merges = reinterpret_cast<const pkv_merge_entry*>(ws + d.ws.off_merges);
    a.n_merges = (int32_t)(st ? d.caps.merges : (int64_t)d.merges.size());
    a.counts = counts;
    // the one-wave-per-pair form serves any chunk count; a static launch must
    // not depend on the step
    a.max_chunks = st ? 0 : d.max_merge_chunks;
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.num_qo_heads = P.num_qo_heads;
    a.head_dim = P.head_dim;
    a.group = d.group;
    PKV_HIP(mark(kMerge, true));
    PKV_HIP(pkv::launch_merge(a, s));
    PKV_HIP(mark(kMerge, false));
  }
  if (has_pre && !fused) {
    PKV_HIP(mark(kPrefill, true));
    PKV_HIP(pkv::launch_prefill(pa, s));
    PKV_HIP(mark(kPrefill, false));
  }
  return PKV_OK;
}

}  // namespace

}  // extern "C"

pkv_status pkv::detail::run_plan(const pkv_plan* plan, const void* q, const void* kv_cache_layer,
                                 void* out, float* lse, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream, bool timed) {
  pkv_status st = check_run(plan, q, kv_cache_layer, out, lse, workspace, workspace_bytes);
  if (st != PKV_OK || (plan->d.total_q == 0 && !plan->d.is_static)) return st;
  return run_impl(plan, q, kv_cache_layer, out, lse, workspace, stream, timed);
}

extern "C" {

pkv_status pkv_run(const pkv_plan* plan, const void* q, const void* kv_cache_layer, void* out,
                   float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  return pkv::detail::run_plan(plan, q, kv_cache_layer, out, lse, workspace, workspace_bytes,
                               static_cast<hipStream_t>(stream), true);
}

pkv_status pkv_run_append(const pkv_plan* plan, const void* q, const void* k_new, const void* v_new,
                          void* kv_cache_layer, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_err.clear();
  pkv_status st = check_run(plan, q, kv_cache_layer, out, lse, workspace, workspace_bytes);
  if (st != PKV_OK || (plan->d.total_q == 0 && !plan->d.is_static)) return st;
  if (k_new == nullptr || v_new == nullptr)
    return fail(PKV_E_INVALID, "k_new and v_new must not be NULL");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_E_INVALID, "k_new and v_new must be 16-byte aligned");
  // Every token is stored before any kernel reads the cache.
  st = pkv_append_kv(plan, k_new, v_new, kv_cache_layer, workspace, workspace_bytes, stream);
  if (st != PKV_OK) return st;
  return run_impl(plan, q, kv_cache_layer, out, lse, workspace, stream);
}

pkv_status pkv_append_kv(const pkv_plan* plan, const void* k_new, const void* v_new,
                         void* kv_cache_layer, void* workspace, size_t workspace_bytes,
                         void* stream) {
  g_err.clear();
  if (plan == nullptr) return fail(PKV_E_INVALID, "plan must not be NULL");
  if (check_paged(plan) != PKV_OK) return PKV_E_INVALID;
  pkv_status st = check_workspace(plan, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  if (plan->uploaded_ws != workspace)
    return fail(PKV_E_STATE, "the plan was not uploaded to this workspace (call pkv_plan_upload first)");
  const pkv::PlanData& d = plan->d;
  if (d.total_q == 0 && !d.is_static) return PKV_OK;
  if (k_new == nullptr || v_new == nullptr || kv_cache_layer == nullptr)
    return fail(PKV_E_INVALID, "k_new, v_new and kv_cache_layer must not be NULL");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(kv_cache_layer))
    return fail(PKV_E_INVALID, "k_new, v_new and kv_cache_layer must be 16-byte aligned");
  pkv::AppendArgs a{};
  a.slots = reinterpret_cast<const int64_t*>(static_cast<char*>(workspace) + d.ws.off_slots);
  a.n_tokens = d.is_static ? (int32_t)d.caps.tokens : d.total_q;
  a.counts = d.is_static ? reinterpret_cast<const int64_t*>(workspace) : nullptr;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.cache = static_cast<uint16_t*>(kv_cache_layer);
  a.num_kv_heads = d.params.num_kv_heads;
  a.head_dim = d.params.head_dim;
  a.page_size = d.params.page_size;
  hipStream_t s = static_cast<hipStream_t>(stream);
  PKV_HIP(timing_mark(plan, s, kAppend, true));
  PKV_HIP(pkv::launch_append(a, s));
  PKV_HIP(timing_mark(plan, s, kAppend, false));
  return PKV_OK;
}

pkv_status pkv_dense_plan_create(const pkv_plan_params* params, int32_t batch, const int32_t* cu_q,
                                 const int32_t* cu_k, const int32_t* paged_kv_indptr,
                                 const int32_t* paged_kv_indices, pkv_plan** out,
                                 size_t* workspace_bytes) {
  g_err.clear();
  if (params == nullptr || out == nullptr || workspace_bytes == nullptr)
    return fail(PKV_E_INVALID, "params, out and workspace_bytes must not be NULL");
  *out = nullptr;
  std::string err;
  pkv_status st = pkv::check_params(*params, err);
  if (st != PKV_OK) return fail(st, err);
  int32_t cus = 0;
  st = resolve_cus(params, &cus);
  if (st != PKV_OK) return st;
  pkv_plan* p = new (std::nothrow) pkv_plan;
  if (p == nullptr) return fail(PKV_E_INVALID, "out of host memory");
  st = pkv::build_dense_plan(*params, cus, batch, cu_q, cu_k, paged_kv_indptr, paged_kv_indices,
                             p->d, err);
  if (st != PKV_OK) {
    delete p;
    return fail(st, err);
  }
  *workspace_bytes = p->d.ws.total_bytes;
  *out = p;
  return PKV_OK;
}

pkv_status pkv_dense_plan_update(pkv_plan* plan, int32_t batch, const int32_t* cu_q,
                                 const int32_t* cu_k, const int32_t* paged_kv_indptr,
                                 const int32_t* paged_kv_indices, size_t* workspace_bytes) {
  g_err.clear();
  if (plan == nullptr || workspace_bytes == nullptr)
    return fail(PKV_E_INVALID, "plan and workspace_bytes must not be NULL");
  if (!plan->d.dense) return fail(PKV_E_INVALID, "not a dense plan (use pkv_plan_update)");
  pkv::PlanData fresh;
  std::string err;
  pkv_status st = pkv::build_dense_plan(plan->d.params, plan->d.num_cus, batch, cu_q, cu_k,
                                        paged_kv_indptr, paged_kv_indices, fresh, err);
  if (st != PKV_OK) return fail(st, err);
  plan->d = std::move(fresh);
  plan->uploaded_ws = nullptr;
  *workspace_bytes = plan->d.ws.total_bytes;
  return PKV_OK;
}

static pkv_status check_dense(const pkv_plan* plan, void* workspace, size_t workspace_bytes) {
  if (plan == nullptr) return fail(PKV_E_INVALID, "plan must not be NULL");
  if (!plan->d.dense) return fail(PKV_E_INVALID, "not a dense plan (use pkv_run)");
  pkv_status st = check_workspace(plan, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  if (plan->uploaded_ws != workspace)
    return fail(PKV_E_STATE, "the plan was not uploaded to this workspace (call pkv_plan_upload first)");
  return PKV_OK;
}

pkv_status pkv_dense_gather(const pkv_plan* plan, const void* kv_cache_layer, const void* k_fresh,
                            const void* v_fresh, void* k_out, void* v_out, int32_t with_prefix,
                            void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  pkv_status st = check_dense(plan, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  const pkv::PlanData& d = plan->d;
  if (d.total_k == 0) return PKV_OK;
  if (k_out == nullptr || v_out == nullptr || !aligned16(k_out) || !aligned16(v_out))
    return fail(PKV_E_INVALID, "k_out and v_out must be non-NULL and 16-byte aligned");
  if (d.total_q > 0 && (k_fresh == nullptr || v_fresh == nullptr || !aligned16(k_fresh) ||
                        !aligned16(v_fresh)))
    return fail(PKV_E_INVALID, "k_fresh and v_fresh must be non-NULL and 16-byte aligned");
  if (with_prefix) {
    if (!d.dense_pages)
      return fail(PKV_E_INVALID, "the plan has no page table: gather with with_prefix = 0");
    if (kv_cache_layer == nullptr || !aligned16(kv_cache_layer))
      return fail(PKV_E_INVALID, "kv_cache_layer must be non-NULL and 16-byte aligned");
  }
  char* ws = static_cast<char*>(workspace);
  pkv::GatherArgs a{};
  a.rows = reinterpret_cast<const pkv::DenseRowMeta*>(ws + d.ws.off_dense_rows);
  a.n_rows = d.batch;
  a.with_prefix = with_prefix ? 1 : 0;
  a.total_k = d.total_k;
  a.total_q = d.total_q;
  a.indices = reinterpret_cast<const int32_t*>(ws + d.ws.off_indices);
  a.cache = static_cast<const uint16_t*>(kv_cache_layer);
  a.k_fresh = static_cast<const uint16_t*>(k_fresh);
  a.v_fresh = static_cast<const uint16_t*>(v_fresh);
  a.k_out = static_cast<uint16_t*>(k_out);
  a.v_out = static_cast<uint16_t*>(v_out);
  a.num_kv_heads = d.params.num_kv_heads;
  a.head_dim = d.params.head_dim;
  a.page_size = d.params.page_size;
  hipStream_t s = static_cast<hipStream_t>(stream);
  PKV_HIP(timing_mark(plan, s, kAppend, true));
  PKV_HIP(pkv::launch_gather(a, s));
  PKV_HIP(timing_mark(plan, s, kAppend, false));
  return PKV_OK;
}

pkv_status pkv_dense_run(const pkv_plan* plan, const void* q, const void* k, const void* v,
                         void* out, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream) {
  g_err.clear();
  pkv_status st = check_dense(plan, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  const pkv::PlanData& d = plan->d;
  if (d.prefill_tiles.empty()) return PKV_OK;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return fail(PKV_E_INVALID, "q, k, v and out must not be NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace))
    return fail(PKV_E_INVALID, "q, k, v, out and workspace must be 16-byte aligned");
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return fail(PKV_E_INVALID, "lse must be 4-byte aligned");
  const pkv_plan_params& P = d.params;
  char* ws = static_cast<char*>(workspace);
  pkv::PrefillArgs a{};
  a.tiles = reinterpret_cast<const pkv_prefill_tile*>(ws + d.ws.off_prefill_tiles);
  a.n_tiles = (int32_t)d.prefill_tiles.size();
  a.q = static_cast<const uint16_t*>(q);
  a.k_dense = static_cast<const uint16_t*>(k);
  a.v_dense = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.num_qo_heads = P.num_qo_heads;
  a.num_kv_heads = P.num_kv_heads;
  a.head_dim = P.head_dim;
  a.page_size = P.page_size;
  a.group = d.group;
  a.causal = P.causal ? 1 : 0;
  a.window_left = P.window_left;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)P.head_dim));
  hipStream_t s = static_cast<hipStream_t>(stream);
  PKV_HIP(timing_mark(plan, s, kPrefill, true));
  PKV_HIP(pkv::launch_prefill(a, s));
  PKV_HIP(timing_mark(plan, s, kPrefill, false));
  return PKV_OK;
}

pkv_status pkv_context_only_views(int32_t batch, int32_t page_size, const int32_t* paged_kv_indptr,
                                  const int32_t* paged_kv_indices,
                                  const int32_t* paged_kv_last_page_len, const int32_t* to_compute,
                                  const int32_t* query_spans, int32_t* out_indptr,
                                  int32_t* out_indices, int32_t* out_last_page_len,
                                  int32_t* out_qo_indptr) {
  g_err.clear();
  std::string err;
  pkv_status st = pkv::context_only_views(batch, page_size, paged_kv_indptr, paged_kv_indices,
                                          paged_kv_last_page_len, to_compute, query_spans,
                                          out_indptr, out_indices, out_last_page_len,
                                          out_qo_indptr, err);
  if (st != PKV_OK) return fail(st, err);
  return PKV_OK;
}

pkv_status pkv_timing_enable(pkv_plan* plan, int32_t enable) {
  g_err.clear();
  if (plan == nullptr) return fail(PKV_E_INVALID, "plan must not be NULL");
  plan->timing.enabled = enable != 0;
  return PKV_OK;
}

pkv_status pkv_timing_read(pkv_plan* plan, double ms[4], int64_t launches[4]) {
  g_err.clear();
  if (plan == nullptr || ms == nullptr || launches == nullptr)
    return fail(PKV_E_INVALID, "NULL argument");
  for (int i = 0; i < 4; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  Timing& t = plan->timing;
  for (size_t i = 0; i < t.used / 2; ++i) {
    PKV_HIP(hipEventSynchronize(t.pool[2 * i + 1]));
    float e = 0.f;
    PKV_HIP(hipEventElapsedTime(&e, t.pool[2 * i], t.pool[2 * i + 1]));
    ms[t.kind[i]] += e;
    launches[t.kind[i]] += 1;
  }
  t.used = 0;
  t.kind.clear();
  return PKV_OK;
}

}  // extern "C"
