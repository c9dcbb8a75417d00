// Per-kernel HIP-event timing of the library's own launches (the diagnostic
// ssd_profile_* entry points). When timing is off, a launch pays one load of
// a flag; when on, each launch is bracketed by two events recorded on the
// stream the kernel is launched on.
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>

namespace ssd {

// Kernel identifiers; the order matches ssd_kernel_id in the public header.
enum KernelId {
  KID_CONV1D = 0,
  KID_CONV_STATE,
  KID_GATED_NORM,
  KID_DECODE,
  KID_CHUNK_STATE,
  KID_STATE_PASS,
  KID_CHUNK_OUT,
  KID_FAST_STATE,
  KID_FAST_PASS,
  KID_FAST_OUT,
  KID_BWD_NORM,
  KID_BWD_CHUNK_Z,
  KID_BWD_REV_PASS,
  KID_BWD_CHUNK,
  KID_BWD_GROUP_SUM,
  KID_BWD_CONV_DU,
  KID_BWD_CONV_DX,
  KID_BWD_Y,
  KID_CHUNK_CB,
  KID_COUNT
};

// switched by ssd_profile_start / _stop, possibly from another thread
extern std::atomic<bool> g_prof_on;
void prof_record(hipStream_t st, int kid, bool begin);

// Brackets the launches in its scope with a pair of events when timing is on.
struct ProfScope {
  hipStream_t st;
  int kid;
  ProfScope(hipStream_t s, int k) : st(s), kid(k) {
    if (g_prof_on.load(std::memory_order_acquire)) prof_record(st, kid, true);
  }
  ~ProfScope() {
    if (g_prof_on.load(std::memory_order_acquire)) prof_record(st, kid, false);
  }
};

}  // namespace ssd
