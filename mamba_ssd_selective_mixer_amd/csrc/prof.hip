// Per-kernel HIP-event timing (ssd_profile_start / _stop / _read /
// ssd_kernel_name). A fixed pool of event pairs is created at start; each
// timed launch takes the next pair, records one event before and one after
// it on its own stream, and reading waits on the recorded events and sums
// the elapsed times per kernel. This is a measurement aid with process-wide
// state: calls from several threads are serialised by a mutex, and timing
// must not be switched on while a stream is being captured into a graph.
#include <mutex>
#include <vector>

#include "../../include/ssd_mi355x.h"
#include "prof.hpp"

namespace ssd {

std::atomic<bool> g_prof_on{false};

namespace {

struct Slot {
  hipEvent_t ev[2];
  int kid;
  bool closed;
};

std::mutex g_mu;
uint64_t g_mask = ~0ull;     // kernels timed: bit k for kernel id k
std::vector<Slot> g_slots;   // the pool; events created once per start
size_t g_used = 0;           // slots taken since start
int g_open[KID_COUNT];       // slot index of the currently open bracket per kernel, or -1
bool g_overflow = false;

const char* kNames[KID_COUNT] = {
    "conv1d_silu",      "conv_state",       "gated_rmsnorm", "decode_step",
    "chunk_state",      "state_pass",       "chunk_out",     "fused_chunk_state",
    "fused_state_pass", "fused_chunk_out_norm", "bwd_gated_norm", "bwd_chunk_z",
    "bwd_rev_pass",     "bwd_chunk",        "bwd_group_sum", "bwd_conv_du",
    "bwd_conv_dx",      "bwd_y",            "chunk_cb",
};

void release() {
  for (Slot& s : g_slots) {
    hipEventDestroy(s.ev[0]);
    hipEventDestroy(s.ev[1]);
  }
  g_slots.clear();
  g_used = 0;
}

}  // namespace

void prof_record(hipStream_t st, int kid, bool begin) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_prof_on.load(std::memory_order_relaxed) || kid < 0 || kid >= KID_COUNT) return;
  if (!((g_mask >> kid) & 1)) return;
  if (begin) {
    if (g_used >= g_slots.size()) {
      g_overflow = true;
      g_open[kid] = -1;
      return;
    }
    const size_t i = g_used++;
    g_slots[i].kid = kid;
    g_slots[i].closed = false;
    g_open[kid] = (int)i;
    hipEventRecord(g_slots[i].ev[0], st);
  } else {
    const int i = g_open[kid];
    if (i < 0) return;
    hipEventRecord(g_slots[i].ev[1], st);
    g_slots[i].closed = true;
    g_open[kid] = -1;
  }
}

}  // namespace ssd

using namespace ssd;

extern "C" {

int ssd_profile_start(int capacity) {
  if (capacity <= 0) return SSD_ERR_SHAPE;
  std::lock_guard<std::mutex> lk(g_mu);
  release();
  g_slots.resize((size_t)capacity);
  for (size_t i = 0; i < g_slots.size(); ++i) {
    if (hipEventCreate(&g_slots[i].ev[0]) != hipSuccess ||
        hipEventCreate(&g_slots[i].ev[1]) != hipSuccess) {
      g_slots.resize(i);  // events of slot i may be half made; drop the pool
      release();
      return SSD_ERR_HIP;
    }
    g_slots[i].kid = -1;
    g_slots[i].closed = false;
  }
  for (int k = 0; k < KID_COUNT; ++k) g_open[k] = -1;
  g_overflow = false;
  g_prof_on.store(true, std::memory_order_release);
  return SSD_OK;
}

int ssd_profile_stop(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_prof_on.store(false, std::memory_order_release);
  return g_overflow ? SSD_ERR_WORKSPACE : SSD_OK;
}

int ssd_profile_read(int kernel, int64_t* launches, double* total_ms) {
  if (!launches || !total_ms) return SSD_ERR_NULL;
  if (kernel < 0 || kernel >= KID_COUNT) return SSD_ERR_SHAPE;
  std::lock_guard<std::mutex> lk(g_mu);
  int64_t n = 0;
  double ms = 0.0;
  for (size_t i = 0; i < g_used; ++i) {
    const Slot& s = g_slots[i];
    if (s.kid != kernel || !s.closed) continue;
    if (hipEventSynchronize(s.ev[1]) != hipSuccess) return SSD_ERR_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, s.ev[0], s.ev[1]) != hipSuccess) return SSD_ERR_HIP;
    ms += t;
    ++n;
  }
  *launches = n;
  *total_ms = ms;
  return SSD_OK;
}

uint64_t ssd_profile_set_mask(uint64_t mask) {
  std::lock_guard<std::mutex> lk(g_mu);
  const uint64_t old = g_mask;
  g_mask = mask;
  return old;
}

const char* ssd_kernel_name(int kernel) {
  return (kernel >= 0 && kernel < KID_COUNT) ? kNames[kernel] : "unknown";
}

}  // extern "C"
