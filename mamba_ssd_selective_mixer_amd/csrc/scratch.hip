// Allocation-free variant of the whole-prefill entry point, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation). Its scratch memory is one fixed
// device array of this library instead of a caller workspace: each GPU the
// library runs on holds its own copy until the process ends. All calls on
// one GPU share it, so calls that overlap in time on one GPU race; the
// kernels themselves clear what must start at zero (status word, tickets,
// exchange slots), so nothing is reset from the host.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/ssd_mi355x.h"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_addr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The current device's address of `scratch`, looked up once per device with
// that device current (the array's name is a host-side stand-in, never a
// device address).
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SSD_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SSD_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSD_ERR_HIP;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return SSD_OK;
}

}  // namespace

extern "C" int ssd_mixer_prefill_noalloc(const ssd_dims* d, const void* xbc, const void* z,
                                         const void* dt, const float* A, const float* D,
                                         const void* conv_w, const void* conv_b,
                                         const void* norm_w, float eps,
                                         const void* conv_state_in, void* conv_state_out,
                                         const float* ssm_state_in, float* ssm_state_out,
                                         void* out, void* stream) {
  const int rc = ssd_validate(SSD_ENTRY_MIXER_PREFILL, d);
  if (rc) return rc;
  if (ssd_mixer_prefill_workspace_bytes(d) > kScratchBytes) return SSD_ERR_SCRATCH;
  void* ws = nullptr;
  const int ra = scratch_address(&ws);
  if (ra) return ra;
  return ssd_mixer_prefill(d, xbc, z, dt, A, D, conv_w, conv_b, norm_w, eps, conv_state_in,
                           conv_state_out, ssm_state_in, ssm_state_out, out, ws, kScratchBytes,
                           stream);
}
