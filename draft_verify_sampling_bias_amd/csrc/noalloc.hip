// dspark_draft_block_noalloc: dspark_draft_block with the workspace taken
// from a static device array instead of the caller, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Nothing here allocates: the array is a file-scope
// __device__ object that the HIP runtime places on each device the library
// runs on, and it stays there until the process ends.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "dspark.h"
#include "plan.h"

namespace {

// The shared scratch of every dspark_draft_block_noalloc call on a device.
// On the host, `scratch` names a host-side stand-in, not device memory: host
// code uses only the address hipGetSymbolAddress returns for the current
// device (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[DSPARK_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DSPARK_ERR_HIP;
  if (dev >= kMaxDevices) return DSPARK_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return DSPARK_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return DSPARK_OK;
}

}  // namespace

extern "C" int dspark_draft_block_noalloc(const dspark_draft_args* a) {
  dspark::DraftPlan plan;
  int st = dspark::plan_draft(a, &plan);
  if (st != DSPARK_OK) return st;
  // the input checks report through a caller's workspace (dspark_check)
  if (a->flags & DSPARK_CHECK_INPUTS) return DSPARK_ERR_UNSUPPORTED;
  if (plan.total > DSPARK_NOALLOC_SCRATCH_BYTES) return DSPARK_ERR_WORKSPACE;
  if (a->R == 0) return DSPARK_OK;
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != DSPARK_OK) return st;
  dspark_draft_args b = *a;
  b.workspace = ws;
  b.workspace_bytes = DSPARK_NOALLOC_SCRATCH_BYTES;
  return dspark_draft_block(&b);
}
