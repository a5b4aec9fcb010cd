// mo_muon_step_noalloc (include/muon.h): the one-shot Muon step with the
// library's own scratch memory in place of a caller's workspace, for
// callers that cannot allocate device memory.
//
// The scratch is one file-scope device array.  In host code its name is a
// host-side stand-in, not a device address, so the step never uses it
// directly: the first call on each device looks up that device's copy with
// hipGetSymbolAddress (with the device current) and keeps the address, and
// every later call on that device passes the kept address to the kernels,
// exactly as mo_muon_step passes a workspace.
//
// Every kernel of the step writes what it later reads (norm and RMS
// partials, the descriptor table, X_0 with its zero padding, S, P', X'), so
// nothing in the scratch needs clearing between calls.  All calls on one
// GPU share its scratch: calls that overlap on one GPU (different streams,
// or different host threads without ordering) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mo_host.h"
#include "muon.h"

namespace {

constexpr size_t kScratchBytes = size_t{MO_NOALLOC_SCRATCH_MIB} << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch (looked up once per device).
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return mo::fail(MO_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return mo::fail(MO_EUNSUPPORTED, "device ordinal %d is out of range", dev);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return mo::fail(MO_EHIP, "scratch lookup on device %d failed: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MO_OK;
}

}  // namespace

extern "C" {

int mo_muon_step_noalloc(const mo_tensor* tensors, int64_t count, int grad_dtype, int mom_dtype, int ns_dtype,
                         float lr, float wd, float mu, int nesterov, int ns_steps, const float* abc,
                         float rms_scale, float eps, float* update_rms, void* stream) {
  if (count == 0) return MO_OK;
  // size and argument checks need no device: validate before the lookup
  size_t full = 0, mn = 0;
  int rc = mo_muon_workspace_size(tensors, count, ns_dtype, &full, &mn);
  if (rc) return rc;
  if (mn > kScratchBytes)
    return mo::fail(MO_EWORKSPACE, "these matrices need %zu bytes of scratch, more than its %zu bytes", mn,
                    kScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_for_current_device(&ws))) return rc;
  return mo::one_shot_step(tensors, count, grad_dtype, mom_dtype, ns_dtype, lr, wd, mu, nesterov, ns_steps, abc,
                           rms_scale, eps, update_rms, ws, kScratchBytes, stream, "scratch");
}

}  // extern "C"
