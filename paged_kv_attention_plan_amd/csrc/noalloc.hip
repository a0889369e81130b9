// pkv_run_noalloc: pkv_plan_upload + pkv_run for callers that cannot allocate
// device memory (code under stream capture, tight serving loops, harnesses
// that forbid allocation).  The workspace (plan metadata + split-KV partials)
// is a file-scope device array, one per GPU, held until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "handle.h"
#include "pkv.h"

namespace {

// The static workspace.  In host code `scratch` names a host-side stand-in,
// never the device memory: kernels and copies get the address that
// hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of the current device's scratch, looked up once per
// device (with that device current).
pkv_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return pkv::detail::fail(PKV_E_DEVICE, std::string("hipGetDevice failed: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pkv::detail::fail(PKV_E_DEVICE, "device index " + std::to_string(dev) + " beyond " +
                                               std::to_string(kMaxDevices));
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return pkv::detail::fail(PKV_E_DEVICE, std::string("hipGetSymbolAddress(scratch) failed: ") +
                                                 hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

size_t pkv_noalloc_capacity(void) { return kScratchBytes; }

pkv_status pkv_run_noalloc(pkv_plan* plan, const void* q, const void* kv_cache_layer, void* out,
                           float* lse, void* stream) {
  pkv::detail::clear_error();
  if (plan == nullptr) return pkv::detail::fail(PKV_E_INVALID, "plan must not be NULL");
  if (plan->d.dense)
    return pkv::detail::fail(PKV_E_INVALID, "a dense plan runs through pkv_dense_gather / pkv_dense_run");
  const size_t need = plan->d.ws.total_bytes;
  if (need > kScratchBytes)
    return pkv::detail::fail(PKV_E_CAPACITY,
                             "this plan needs a workspace of " + std::to_string(need) +
                                 " bytes; pkv_run_noalloc's static workspace holds " +
                                 std::to_string(kScratchBytes) + " (use pkv_plan_upload + pkv_run)");
  void* ws = nullptr;
  pkv_status st = scratch_address(&ws);
  if (st != PKV_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // Nothing in the workspace must start at zero: the upload rewrites the
  // whole metadata region and every partial is written before it is read.
  st = pkv::detail::upload_meta(plan, ws, kScratchBytes, s, /*may_allocate=*/false);
  if (st != PKV_OK) return st;
  // The plan's per-kernel timing (pkv_timing_enable) is not recorded here: its
  // events are created on first use.
  return pkv::detail::run_plan(plan, q, kv_cache_layer, out, lse, ws, kScratchBytes, s,
                               /*timed=*/false);
}

}  // extern "C"
