// Host-side helpers shared by the library's C-ABI translation units:
// the thread's error message, launch checks, workspace checks and the
// HIP-event timing counters behind mo_profile_*.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "muon.h"

namespace mo {

extern thread_local std::string g_err;
// records the message for mo_last_error and returns `code`
int fail(int code, const char* fmt, ...);
// status of a launch; with MO_DEBUG_SYNC=1 also synchronises the stream
int checked(hipError_t e, hipStream_t s, const char* what);

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }
bool aligned16(const void* p);
int validate_dtype(int dt, const char* what);
int check_workspace(void* ws, size_t ws_bytes, size_t min_bytes);

// Brackets one launch of kernel class `cls` with HIP events on `s` when
// that class's counters are enabled; `work` is its algorithmic work.
class ProfScope {
 public:
  ProfScope(int cls, hipStream_t s, double work);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  int cls_ = -1;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
  hipStream_t s_ = nullptr;
  double work_ = 0.0;
};

// mo_muon_step over a caller's workspace (mo_muon_step) or the library's
// own scratch (mo_muon_step_noalloc: ws_name names it in the error when the
// matrices need more than it holds).
int one_shot_step(const mo_tensor* tensors, int64_t count, int grad_dtype, int mom_dtype, int ns_dtype, float lr,
                  float wd, float mu, int nesterov, int ns_steps, const float* abc, float rms_scale, float eps,
                  float* update_rms, void* workspace, size_t workspace_bytes, void* stream,
                  const char* ws_name);

}  // namespace mo
