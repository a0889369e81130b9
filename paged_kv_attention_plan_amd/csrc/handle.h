// The plan handle behind the opaque pkv_plan of include/pkv.h, and the
// library-internal calls that entry points in other translation units share.
#pragma once

#include <hip/hip_runtime.h>

#include <string>
#include <vector>

#include "pkv.h"
#include "plan.h"
#include "stage.h"

// Event pairs recorded around launches while timing is enabled.
struct Timing {
  bool enabled = false;
  std::vector<hipEvent_t> pool;  // created lazily, reused after a read
  size_t used = 0;
  std::vector<int> kind;         // kernel kind of pair i (events 2i, 2i+1)
};

struct pkv_plan {
  pkv::PlanData d;
  pkv::StageRing ring;  // page-locked, host-coherent staging buffers of the uploads
  void* uploaded_ws = nullptr;
  mutable Timing timing;
};

namespace pkv {
namespace detail {

// Set the thread's error message; returns s.
pkv_status fail(pkv_status s, std::string msg);
// Clear it (at the start of every entry point).
void clear_error();

// Serialise the plan's metadata into its staging ring and enqueue the upload
// kernel that copies it to the head of `workspace` (the body of
// pkv_plan_upload).  With may_allocate false, a staging buffer smaller than
// the metadata is PKV_E_CAPACITY instead of being re-allocated.
pkv_status upload_meta(pkv_plan* plan, void* workspace, size_t workspace_bytes, hipStream_t stream,
                       bool may_allocate);

// Argument checks of pkv_run, then its launches.  timed = false skips the
// plan's per-kernel timing events (their lazy creation allocates).
pkv_status run_plan(const pkv_plan* plan, const void* q, const void* kv_cache_layer, void* out,
                    float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream,
                    bool timed);

}  // namespace detail
}  // namespace pkv
