// C ABI of the Mamba-2 mixer core (declared in include/ssd_mi355x.h):
// host-side argument checks, workspace carving and kernel launches. Nothing
// here allocates device memory or keeps mutable global state.
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/ssd_mi355x.h"
#include "launch.hpp"

namespace ssd {
size_t scan_lds_bytes(bool io_bf16, int P, int N, int Q);
}

namespace {

constexpr size_t kLdsPerCU = 160 * 1024;
constexpr size_t kWsAlign = 256;

size_t esize(const ssd_dims* d) { return d->io_dtype == SSD_BF16 ? 2 : 4; }
bool f32op(const ssd_dims* d) { return (d->flags & SSD_FLAG_FP32_OPERANDS) != 0; }

// bound on the polls of the fast path's cross-block norm exchange
std::atomic<int> g_spin_limit{1 << 20};
std::atomic<int> g_bwd_heads{0};  // backward per-chunk workgroup heads; 0: from the shape
// general path's norm: 0 fused into the output kernel from the shape, 1
// fused wherever a norm group fits one workgroup, 2 never (y, then the norm)
std::atomic<int> g_norm_fuse{0};
// fewest (chunk, group) workgroups for which the shape-chosen fusion pays:
// fewer leave the chip idle while each workgroup walks its group's heads
constexpr int64_t kNormFuseBlocks = 512;
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
bool is_one_of(int v, std::initializer_list<int> set) {
  for (int s : set)
    if (v == s) return true;
  return false;
}
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t channels(const ssd_dims* d) {
  return (int64_t)d->nheads * d->headdim + 2 * (int64_t)d->ngroups * d->dstate;
}
// The general path runs 64-token chunks whatever the caller's chunk (the
// result is the same in exact arithmetic; its output kernel is built for 64).
constexpr int kGenChunk = 64;
int64_t gen_chunks(const ssd_dims* d) { return (d->seqlen + kGenChunk - 1) / kGenChunk; }

bool any_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// One buffer of a call: its byte range, whether the call writes it, and the
// slot of the one buffer it may coincide with exactly (an in-place pair such
// as ssm_state_in / ssm_state_out), or -1.
struct Range {
  const void* p;
  size_t n;
  bool written;
  int twin;
};
// Every buffer the call writes must be disjoint from every other buffer it
// touches, except its documented in-place twin at exactly the same address
// and size. Buffers that are only read may overlap each other (x, B and C
// may be views of one tensor).
bool aliased(std::initializer_list<Range> list) {
  const Range* r = list.begin();
  const int n = (int)list.size();
  for (int i = 0; i < n; ++i) {
    if (!r[i].written) continue;
    for (int j = 0; j < n; ++j) {
      if (j == i || (r[j].written && j < i)) continue;
      if (!any_overlap(r[i].p, r[i].n, r[j].p, r[j].n)) continue;
      const bool twins = (r[i].twin == j || r[j].twin == i) && r[i].p == r[j].p && r[i].n == r[j].n;
      if (!twins) return true;
    }
  }
  return false;
}

int check_dims(int entry, const ssd_dims* d) {
  if (!d) return SSD_ERR_NULL;
  if (d->io_dtype != SSD_F32 && d->io_dtype != SSD_BF16) return SSD_ERR_DTYPE;
  if (d->flags & ~SSD_FLAG_FP32_OPERANDS) return SSD_ERR_UNSUPPORTED;
  if (d->batch < 1 || d->seqlen < 1 || d->nheads < 1 || d->headdim < 1 || d->ngroups < 1 ||
      d->dstate < 1)
    return SSD_ERR_SHAPE;
  if (d->nheads % d->ngroups != 0) return SSD_ERR_SHAPE;
  if (!is_one_of(d->headdim, {16, 32, 64, 128})) return SSD_ERR_UNSUPPORTED;
  if (!is_one_of(d->dstate, {16, 32, 64, 128, 256})) return SSD_ERR_UNSUPPORTED;
  if (d->batch > 65535 || d->nheads > 65535) return SSD_ERR_UNSUPPORTED;
  const bool conv = entry == SSD_ENTRY_CONV1D || entry == SSD_ENTRY_DECODE_STEP ||
                    entry == SSD_ENTRY_MIXER_PREFILL;
  const bool scan = entry == SSD_ENTRY_CHUNK_SCAN || entry == SSD_ENTRY_MIXER_PREFILL;
  if (conv) {
    if (d->conv_width < 1) return SSD_ERR_SHAPE;
    if (!is_one_of(d->conv_width, {2, 3, 4})) return SSD_ERR_UNSUPPORTED;
    if ((d->seqlen + 31) / 32 > 65535) return SSD_ERR_UNSUPPORTED;
  }
  if (scan) {
    if (d->chunk < 1) return SSD_ERR_SHAPE;
    if (!is_one_of(d->chunk, {32, 64, 128, 256})) return SSD_ERR_UNSUPPORTED;
    if (ssd::scan_lds_bytes(d->io_dtype == SSD_BF16 && !f32op(d), d->headdim, d->dstate,
                            d->chunk) >
        kLdsPerCU - 8192)
      return SSD_ERR_UNSUPPORTED;
  }
  if (entry == SSD_ENTRY_DECODE_STEP) {
    if (d->seqlen != 1) return SSD_ERR_SHAPE;
    const size_t S = (size_t)d->nheads / d->ngroups * d->headdim;
    if ((2 * S + 2 * (size_t)d->dstate) * 4 > kLdsPerCU - 1024) return SSD_ERR_UNSUPPORTED;
  }
  if (entry < SSD_ENTRY_CONV1D || entry > SSD_ENTRY_MIXER_PREFILL) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

struct ScanWs {
  bool fast;
  int* status;
  float* states;
  float* lam_end;
  float* y32;
  float* cb;  // each chunk's C B^T per group
  unsigned char* conv;
  void* fastws;
  size_t total;
};

bool use_fast(const ssd_dims* d, bool conv) {
  return !f32op(d) && ssd::fast_path_ok(d->io_dtype == SSD_BF16, d->headdim, d->dstate,
                                        d->nheads, d->ngroups, d->chunk, d->conv_width, conv);
}

// Workspace layout for the scan (conv = the scan consumes raw xBC rows).
ScanWs carve(const ssd_dims* d, void* base, bool conv) {
  ScanWs w{};
  const size_t B = d->batch, L = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate;
  const size_t nc = gen_chunks(d);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += round_up(bytes, kWsAlign);
    return o;
  };
  w.fast = use_fast(d, conv);
  const size_t o_status = take(4);  // the call's status word (ssd_workspace_status)
  size_t o_states = 0, o_lam = 0, o_y = 0, o_cb = 0, o_conv = 0, o_fast = 0;
  if (w.fast) {
    o_fast = take(ssd::fast_ws_bytes(d->batch, d->seqlen, d->nheads, d->ngroups, conv));
  } else {
    o_states = take(B * nc * H * P * N * 4);
    o_lam = take(B * H * nc * 4);
    o_y = take(B * L * H * P * 4);
    o_cb = take(ssd::chunk_cb_bytes((int)B, (int)nc, d->ngroups));
    if (conv) o_conv = take(B * L * (size_t)channels(d) * 4);  // fp32 conv output
  }
  w.total = off;
  if (base) {
    unsigned char* p = (unsigned char*)base;
    w.status = (int*)(p + o_status);
    if (w.fast) {
      w.fastws = p + o_fast;
    } else {
      w.states = (float*)(p + o_states);
      w.lam_end = (float*)(p + o_lam);
      w.y32 = (float*)(p + o_y);
      w.cb = (float*)(p + o_cb);
      w.conv = conv ? p + o_conv : nullptr;
    }
  }
  return w;
}

// x_f32: x, B and C are fp32 (the conv's internal copy), else the I/O type.
// dta: dt's token stride and preprocessing (A holds A_log when dta.bias is
// set); zs: z's token stride.
int run_scan(const ssd_dims* d, const void* x, int64_t xs, const void* dt, const DtA& dta,
             const float* A, const float* D, const void* Bm, const void* Cm, int64_t bs,
             bool x_f32, const void* z, int64_t zs, const void* norm_w, float eps,
             const float* s_in, float* s_out, void* y, const ScanWs& ws, hipStream_t st) {
  const bool bf = d->io_dtype == SSD_BF16;
  ssd::ScanShape s{d->batch, d->seqlen, d->nheads, d->headdim, d->ngroups,
                   d->dstate, kGenChunk, (int)gen_chunks(d), dta};
  const bool fo = f32op(d);
  int rc = hip_status(ssd::launch_chunk_state(bf, x_f32, fo, s, x, xs, dt, A, Bm, bs, ws.states,
                                              ws.lam_end, ws.status, st));
  if (rc) return rc;
  rc = hip_status(ssd::launch_state_pass(s, ws.states, ws.lam_end, s_in, s_out, ws.status, st));
  if (rc) return rc;
  const int fuse = g_norm_fuse.load(std::memory_order_relaxed);
  const int64_t blocks = (int64_t)d->batch * s.nc * d->ngroups;
  if (z && ssd::chunk_y_fuses_norm(d->nheads, d->ngroups, d->headdim) &&
      (fuse == 1 || (fuse == 0 && blocks >= kNormFuseBlocks))) {
    // one workgroup holds a whole norm group: the norm runs in the output kernel
    const ssd::YNorm nm{z, zs, norm_w, eps};
    return hip_status(ssd::launch_chunk_y(bf, x_f32, !bf, s, x, xs, Bm, Cm, bs, ws.cb, dt, A, D,
                                          ws.states, y, ws.status, ssd::KID_CHUNK_OUT, st,
                                          &nm));
  }
  const bool fused_norm = z != nullptr;
  void* ydst = fused_norm ? (void*)ws.y32 : y;
  rc = hip_status(ssd::launch_chunk_y(bf, x_f32, fused_norm || !bf, s, x, xs, Bm, Cm, bs, ws.cb,
                                      dt, A, D, ws.states, ydst, ws.status, ssd::KID_CHUNK_OUT,
                                      st));
  if (rc) return rc;
  if (fused_norm)
    rc = hip_status(ssd::launch_gated_norm(bf, true, d->batch * d->seqlen,
                                           d->nheads * d->headdim, d->ngroups, ws.y32, z, zs,
                                           norm_w, eps, y, st));
  return rc;
}

int run_fast(const ssd_dims* d, bool conv, const void* x, const void* Bm, const void* Cm,
             int64_t xs, int64_t bs, const void* dt, const DtA& dta, const float* A,
             const float* D, const void* conv_w, const void* conv_b, const void* conv_in,
             const void* z, int64_t zs, const void* norm_w, float eps, const float* s_in,
             float* s_out, void* y, const ScanWs& ws, hipStream_t st) {
  ssd::FastScanArgs a{};
  a.B = d->batch;
  a.L = d->seqlen;
  a.H = d->nheads;
  a.G = d->ngroups;
  a.x = x;
  a.Bm = Bm;
  a.Cm = Cm;
  a.xs = xs;
  a.bs = bs;
  a.dt = dt;
  a.A = A;
  a.D = D;
  a.dts = dta.dts;
  a.zs = zs;
  a.dt_bias = dta.bias;
  a.conv = conv;
  a.conv_w = conv_w;
  a.conv_b = conv_b;
  a.conv_in = conv_in;
  a.z = z;
  a.norm_w = norm_w;
  a.eps = eps;
  a.s_in = s_in;
  a.s_out = s_out;
  a.y = y;
  a.ws = ws.fastws;
  a.status = ws.status;
  a.spin_max = g_spin_limit.load(std::memory_order_relaxed);
  return hip_status(ssd::launch_fast_scan(a, st));
}

// The launches of a whole prefill (arguments already checked): xbc rows with
// token stride xs, z with token stride zs (or null), dt per dta.
int run_prefill(const ssd_dims* d, const void* xbc, int64_t xs, const void* z, int64_t zs,
                const void* dt, const DtA& dta, const float* A, const float* D,
                const void* conv_w, const void* conv_b, const void* norm_w, float eps,
                const void* conv_state_in, void* conv_state_out, const float* ssm_state_in,
                float* ssm_state_out, void* out, void* workspace, hipStream_t st) {
  const ScanWs ws = carve(d, workspace, true);
  const bool bf = d->io_dtype == SSD_BF16;
  const size_t e = esize(d), C = channels(d), HP = (size_t)d->nheads * d->headdim;
  const int64_t GN = (int64_t)d->ngroups * d->dstate;
  int rc;
  if (ws.fast) {
    // conv recomputed inside the scan kernels; the new conv state is taken
    // after them because they read conv_state_in (which it may overwrite).
    const unsigned char* xb = (const unsigned char*)xbc;
    rc = run_fast(d, true, xbc, xb + HP * e, xb + (HP + GN) * e, xs, xs, dt, dta, A, D, conv_w,
                  conv_b, conv_state_in, z, zs, norm_w, eps, ssm_state_in, ssm_state_out, out,
                  ws, st);
    if (rc || !conv_state_out) return rc;
    return hip_status(ssd::launch_conv_state(bf, d->batch, d->seqlen, (int)C, d->conv_width, xbc,
                                             xs, conv_state_in, conv_state_out, st));
  }
  // the conv output stays fp32 for the scan: with a conv bias, B and C carry
  // a shared offset whose C.B products cancel, so their rounding matters
  rc = hip_status(ssd::launch_conv1d(bf, d->batch, d->seqlen, (int)C, d->conv_width, xbc, xs,
                                     conv_w, conv_b, conv_state_in, ws.conv, C, true, st));
  if (rc) return rc;
  if (conv_state_out) {
    rc = hip_status(ssd::launch_conv_state(bf, d->batch, d->seqlen, (int)C, d->conv_width, xbc,
                                           xs, conv_state_in, conv_state_out, st));
    if (rc) return rc;
  }
  const unsigned char* v = ws.conv;
  return run_scan(d, v, C, dt, dta, A, D, v + HP * 4, v + (HP + GN) * 4, C, true, z, zs, norm_w,
                  eps, ssm_state_in, ssm_state_out, out, ws, st);
}

}  // namespace

extern "C" {

int64_t ssd_conv_channels(const ssd_dims* d) { return d ? channels(d) : 0; }

int64_t ssd_ssm_state_bytes(const ssd_dims* d) {
  if (!d) return 0;
  return (int64_t)d->nheads * d->headdim * d->dstate * 4;
}

int64_t ssd_conv_state_bytes(const ssd_dims* d, int as_fp32) {
  if (!d || d->conv_width < 1) return 0;
  const int64_t e = as_fp32 ? 4 : (int64_t)esize(d);
  return (int64_t)(d->conv_width - 1) * channels(d) * e;
}

int ssd_validate(int entry, const ssd_dims* d) { return check_dims(entry, d); }

const char* ssd_status_str(int status) {
  switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_NULL: return "required pointer is NULL";
    case SSD_ERR_SHAPE: return "invalid or inconsistent sizes";
    case SSD_ERR_UNSUPPORTED: return "shape outside the supported envelope";
    case SSD_ERR_DTYPE: return "unsupported io dtype";
    case SSD_ERR_ALIAS: return "input and output buffers partially overlap";
    case SSD_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case SSD_ERR_HIP: return "HIP runtime error at launch";
    case SSD_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case SSD_ERR_TIMEOUT: return "a cross-workgroup norm exchange gave up waiting";
    case SSD_ERR_NONFINITE: return "an output or the final state is not finite";
    case SSD_ERR_SCRATCH: return "the call needs more scratch than the fixed buffer holds";
    case SSD_ERR_VARLEN: return "ragged-batch offsets or slots are invalid (nothing was computed)";
    default: return "unknown status";
  }
}

int ssd_conv1d(const ssd_dims* d, const void* xbc, int64_t xbc_tok_stride, const void* w,
               const void* bias, const void* conv_state_in, void* conv_state_out, void* out,
               int64_t out_tok_stride, void* stream) {
  int rc = check_dims(SSD_ENTRY_CONV1D, d);
  if (rc) return rc;
  if (!xbc || !w || !out) return SSD_ERR_NULL;
  const int64_t C = channels(d);
  if (xbc_tok_stride < C || out_tok_stride < C) return SSD_ERR_SHAPE;
  const size_t e = esize(d);
  if (!aligned16(xbc) || !aligned16(out) || !aligned16(conv_state_in) ||
      !aligned16(conv_state_out) || (xbc_tok_stride * e) % 16 || (out_tok_stride * e) % 16)
    return SSD_ERR_ALIGN;
  const size_t B = d->batch, L = d->seqlen, R = d->conv_width - 1;
  const size_t nx = ((B * L - 1) * xbc_tok_stride + C) * e;
  const size_t no = ((B * L - 1) * out_tok_stride + C) * e;
  const size_t ns = B * R * C * e;
  if (aliased({{xbc, nx, false, -1},
               {w, C * d->conv_width * e, false, -1},
               {bias, C * e, false, -1},
               {conv_state_in, ns, false, 4},
               {conv_state_out, ns, true, 3},
               {out, no, true, -1}}))
    return SSD_ERR_ALIAS;
  hipStream_t st = (hipStream_t)stream;
  const bool bf = d->io_dtype == SSD_BF16;
  rc = hip_status(ssd::launch_conv1d(bf, d->batch, d->seqlen, (int)C, d->conv_width, xbc,
                                     xbc_tok_stride, w, bias, conv_state_in, out, out_tok_stride,
                                     false, st));
  if (rc || !conv_state_out) return rc;
  return hip_status(ssd::launch_conv_state(bf, d->batch, d->seqlen, (int)C, d->conv_width, xbc,
                                           xbc_tok_stride, conv_state_in, conv_state_out, st));
}

size_t ssd_chunk_scan_workspace_bytes(const ssd_dims* d) {
  if (check_dims(SSD_ENTRY_CHUNK_SCAN, d)) return 0;
  return carve(d, nullptr, false).total;
}

int ssd_chunk_scan(const ssd_dims* d, const void* x, int64_t x_tok_stride, const void* dt,
                   const float* A, const float* D, const void* Bm, const void* Cm,
                   int64_t bc_tok_stride, const void* z, const void* norm_w, float eps,
                   const float* ssm_state_in, float* ssm_state_out, void* y, void* workspace,
                   size_t ws_bytes, void* stream) {
  int rc = check_dims(SSD_ENTRY_CHUNK_SCAN, d);
  if (rc) return rc;
  if (!x || !dt || !A || !Bm || !Cm || !y) return SSD_ERR_NULL;
  if (z && !norm_w) return SSD_ERR_NULL;
  const int64_t HP = (int64_t)d->nheads * d->headdim, GN = (int64_t)d->ngroups * d->dstate;
  if (x_tok_stride < HP || bc_tok_stride < GN) return SSD_ERR_SHAPE;
  const size_t e = esize(d);
  if (!aligned16(x) || !aligned16(dt) || !aligned16(Bm) || !aligned16(Cm) || !aligned16(z) ||
      !aligned16(norm_w) || !aligned16(A) || !aligned16(D) || !aligned16(ssm_state_in) ||
      !aligned16(ssm_state_out) || !aligned16(y) || (x_tok_stride * e) % 16 ||
      (bc_tok_stride * e) % 16)
    return SSD_ERR_ALIGN;
  const ScanWs need = carve(d, nullptr, false);
  if (!workspace || ws_bytes < need.total || ((uintptr_t)workspace % kWsAlign))
    return SSD_ERR_WORKSPACE;
  const size_t T = (size_t)d->batch * d->seqlen;
  const size_t ny = T * HP * e, nst = (size_t)d->batch * HP * d->dstate * 4;
  const size_t nx = ((T - 1) * x_tok_stride + HP) * e, nb = ((T - 1) * bc_tok_stride + GN) * e;
  if (aliased({{x, nx, false, -1},
               {dt, T * d->nheads * e, false, -1},
               {A, (size_t)d->nheads * 4, false, -1},
               {D, (size_t)d->nheads * 4, false, -1},
               {Bm, nb, false, -1},
               {Cm, nb, false, -1},
               {z, ny, false, -1},
               {norm_w, (size_t)HP * e, false, -1},
               {ssm_state_in, nst, false, 9},
               {ssm_state_out, nst, true, 8},
               {y, ny, true, -1},
               {workspace, need.total, true, -1}}))
    return SSD_ERR_ALIAS;
  const ScanWs ws = carve(d, workspace, false);
  const DtA plain{d->nheads, nullptr};
  if (ws.fast)
    return run_fast(d, false, x, Bm, Cm, x_tok_stride, bc_tok_stride, dt, plain, A, D, nullptr,
                    nullptr, nullptr, z, HP, norm_w, eps, ssm_state_in, ssm_state_out, y, ws,
                    (hipStream_t)stream);
  return run_scan(d, x, x_tok_stride, dt, plain, A, D, Bm, Cm, bc_tok_stride, false, z, HP,
                  norm_w, eps, ssm_state_in, ssm_state_out, y, ws, (hipStream_t)stream);
}

int ssd_gated_rmsnorm(const ssd_dims* d, const void* y, const void* z, const void* w, float eps,
                      void* out, void* stream) {
  int rc = check_dims(SSD_ENTRY_GATED_RMSNORM, d);
  if (rc) return rc;
  if (!y || !z || !w || !out) return SSD_ERR_NULL;
  if (!aligned16(y) || !aligned16(z) || !aligned16(w) || !aligned16(out)) return SSD_ERR_ALIGN;
  const size_t n = (size_t)d->batch * d->seqlen * d->nheads * d->headdim * esize(d);
  if (aliased({{y, n, false, 3},
               {z, n, false, -1},
               {w, (size_t)d->nheads * d->headdim * esize(d), false, -1},
               {out, n, true, 0}}))
    return SSD_ERR_ALIAS;
  return hip_status(ssd::launch_gated_norm(d->io_dtype == SSD_BF16, false,
                                           d->batch * d->seqlen, d->nheads * d->headdim,
                                           d->ngroups, y, z, (int64_t)d->nheads * d->headdim, w,
                                           eps, out, (hipStream_t)stream));
}

int ssd_decode_step(const ssd_dims* d, const void* xbc_t, const void* z_t, const void* dt_t,
                    const float* A, const float* D, const void* conv_w, const void* conv_b,
                    const void* norm_w, float eps, void* conv_state, float* ssm_state, void* y_t,
                    void* stream) {
  int rc = check_dims(SSD_ENTRY_DECODE_STEP, d);
  if (rc) return rc;
  if (!xbc_t || !dt_t || !A || !conv_w || !conv_state || !ssm_state || !y_t) return SSD_ERR_NULL;
  if (z_t && !norm_w) return SSD_ERR_NULL;
  if (!aligned16(xbc_t) || !aligned16(z_t) || !aligned16(dt_t) || !aligned16(A) ||
      !aligned16(D) || !aligned16(conv_w) || !aligned16(conv_b) || !aligned16(norm_w) ||
      !aligned16(conv_state) || !aligned16(ssm_state) || !aligned16(y_t))
    return SSD_ERR_ALIGN;
  const size_t e = esize(d), B = d->batch, C = channels(d);
  const size_t HP = (size_t)d->nheads * d->headdim;
  const size_t ny = B * HP * e, ncs = B * (d->conv_width - 1) * C * e,
               nss = B * HP * d->dstate * 4;
  if (aliased({{xbc_t, B * C * e, false, -1},
               {z_t, ny, false, -1},
               {dt_t, B * d->nheads * e, false, -1},
               {A, (size_t)d->nheads * 4, false, -1},
               {D, (size_t)d->nheads * 4, false, -1},
               {conv_w, C * d->conv_width * e, false, -1},
               {conv_b, C * e, false, -1},
               {norm_w, HP * e, false, -1},
               {conv_state, ncs, true, -1},
               {ssm_state, nss, true, -1},
               {y_t, ny, true, -1}}))
    return SSD_ERR_ALIAS;
  return hip_status(ssd::launch_decode(d->io_dtype == SSD_BF16, d->batch, d->nheads,
                                       d->headdim, d->ngroups, d->dstate, d->conv_width, xbc_t,
                                       (int64_t)C, z_t, (int64_t)HP, dt_t,
                                       DtA{d->nheads, nullptr}, A, D, conv_w, conv_b, norm_w, eps,
                                       conv_state, ssm_state, y_t, (hipStream_t)stream));
}

size_t ssd_mixer_prefill_workspace_bytes(const ssd_dims* d) {
  if (check_dims(SSD_ENTRY_MIXER_PREFILL, d)) return 0;
  return carve(d, nullptr, true).total;
}

int ssd_mixer_prefill(const ssd_dims* d, const void* xbc, const void* z, const void* dt,
                      const float* A, const float* D, const void* conv_w, const void* conv_b,
                      const void* norm_w, float eps, const void* conv_state_in,
                      void* conv_state_out, const float* ssm_state_in, float* ssm_state_out,
                      void* out, void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_dims(SSD_ENTRY_MIXER_PREFILL, d);
  if (rc) return rc;
  if (!xbc || !dt || !A || !conv_w || !out) return SSD_ERR_NULL;
  if (z && !norm_w) return SSD_ERR_NULL;
  if (!aligned16(xbc) || !aligned16(z) || !aligned16(dt) || !aligned16(A) || !aligned16(D) ||
      !aligned16(conv_w) || !aligned16(conv_b) || !aligned16(norm_w) ||
      !aligned16(conv_state_in) || !aligned16(conv_state_out) || !aligned16(ssm_state_in) ||
      !aligned16(ssm_state_out) || !aligned16(out))
    return SSD_ERR_ALIGN;
  const ScanWs need = carve(d, nullptr, true);
  if (!workspace || ws_bytes < need.total || ((uintptr_t)workspace % kWsAlign))
    return SSD_ERR_WORKSPACE;
  const size_t e = esize(d), T = (size_t)d->batch * d->seqlen, C = channels(d);
  const size_t HP = (size_t)d->nheads * d->headdim;
  const size_t nx = T * C * e, no = T * HP * e, ncs = (size_t)d->batch * (d->conv_width - 1) * C * e,
               nss = (size_t)d->batch * HP * d->dstate * 4;
  if (aliased({{xbc, nx, false, -1},
               {z, no, false, -1},
               {dt, T * d->nheads * e, false, -1},
               {A, (size_t)d->nheads * 4, false, -1},
               {D, (size_t)d->nheads * 4, false, -1},
               {conv_w, C * d->conv_width * e, false, -1},
               {conv_b, C * e, false, -1},
               {norm_w, HP * e, false, -1},
               {conv_state_in, ncs, false, 9},
               {conv_state_out, ncs, true, 8},
               {ssm_state_in, nss, false, 11},
               {ssm_state_out, nss, true, 10},
               {out, no, true, -1},
               {workspace, need.total, true, -1}}))
    return SSD_ERR_ALIAS;
  return run_prefill(d, xbc, (int64_t)C, z, (int64_t)HP, dt, DtA{d->nheads, nullptr}, A, D,
                     conv_w, conv_b, norm_w, eps, conv_state_in, conv_state_out, ssm_state_in,
                     ssm_state_out, out, workspace, (hipStream_t)stream);
}

int ssd_mixer_prefill_packed(const ssd_dims* d, const void* zxbcdt, int64_t row_stride,
                             const float* dt_bias, const float* A_log, const float* D,
                             const void* conv_w, const void* conv_b, const void* norm_w,
                             float eps, const void* conv_state_in, void* conv_state_out,
                             const float* ssm_state_in, float* ssm_state_out, void* out,
                             void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_dims(SSD_ENTRY_MIXER_PREFILL, d);
  if (rc) return rc;
  if (!zxbcdt || !dt_bias || !A_log || !conv_w || !norm_w || !out) return SSD_ERR_NULL;
  const size_t e = esize(d), T = (size_t)d->batch * d->seqlen, C = channels(d);
  const size_t HP = (size_t)d->nheads * d->headdim, width = HP + C + d->nheads;
  if (row_stride < (int64_t)width) return SSD_ERR_SHAPE;
  if (!aligned16(zxbcdt) || (row_stride * e) % 16 || !aligned16(dt_bias) || !aligned16(A_log) ||
      !aligned16(D) || !aligned16(conv_w) || !aligned16(conv_b) || !aligned16(norm_w) ||
      !aligned16(conv_state_in) || !aligned16(conv_state_out) || !aligned16(ssm_state_in) ||
      !aligned16(ssm_state_out) || !aligned16(out))
    return SSD_ERR_ALIGN;
  const ScanWs need = carve(d, nullptr, true);
  if (!workspace || ws_bytes < need.total || ((uintptr_t)workspace % kWsAlign))
    return SSD_ERR_WORKSPACE;
  const size_t nrow = ((T - 1) * row_stride + width) * e, no = T * HP * e,
               ncs = (size_t)d->batch * (d->conv_width - 1) * C * e,
               nss = (size_t)d->batch * HP * d->dstate * 4, nh = (size_t)d->nheads * 4;
  if (aliased({{zxbcdt, nrow, false, -1},
               {dt_bias, nh, false, -1},
               {A_log, nh, false, -1},
               {D, nh, false, -1},
               {conv_w, C * d->conv_width * e, false, -1},
               {conv_b, C * e, false, -1},
               {norm_w, HP * e, false, -1},
               {conv_state_in, ncs, false, 8},
               {conv_state_out, ncs, true, 7},
               {ssm_state_in, nss, false, 10},
               {ssm_state_out, nss, true, 9},
               {out, no, true, -1},
               {workspace, need.total, true, -1}}))
    return SSD_ERR_ALIAS;
  const unsigned char* row = (const unsigned char*)zxbcdt;
  return run_prefill(d, row + HP * e, row_stride, zxbcdt, row_stride, row + (HP + C) * e,
                     DtA{row_stride, dt_bias}, A_log, D, conv_w, conv_b, norm_w, eps,
                     conv_state_in, conv_state_out, ssm_state_in, ssm_state_out, out, workspace,
                     (hipStream_t)stream);
}

int ssd_decode_step_packed(const ssd_dims* d, const void* zxbcdt_t, int64_t row_stride,
                           const float* dt_bias, const float* A_log, const float* D,
                           const void* conv_w, const void* conv_b, const void* norm_w, float eps,
                           void* conv_state, float* ssm_state, void* y_t, void* stream) {
  int rc = check_dims(SSD_ENTRY_DECODE_STEP, d);
  if (rc) return rc;
  if (!zxbcdt_t || !dt_bias || !A_log || !conv_w || !norm_w || !conv_state || !ssm_state || !y_t)
    return SSD_ERR_NULL;
  const size_t e = esize(d), B = d->batch, C = channels(d);
  const size_t HP = (size_t)d->nheads * d->headdim, width = HP + C + d->nheads;
  if (row_stride < (int64_t)width) return SSD_ERR_SHAPE;
  if (!aligned16(zxbcdt_t) || (row_stride * e) % 16 || !aligned16(dt_bias) ||
      !aligned16(A_log) || !aligned16(D) || !aligned16(conv_w) || !aligned16(conv_b) ||
      !aligned16(norm_w) || !aligned16(conv_state) || !aligned16(ssm_state) || !aligned16(y_t))
    return SSD_ERR_ALIGN;
  const size_t nrow = ((B - 1) * row_stride + width) * e, ny = B * HP * e,
               ncs = B * (d->conv_width - 1) * C * e, nss = B * HP * d->dstate * 4,
               nh = (size_t)d->nheads * 4;
  if (aliased({{zxbcdt_t, nrow, false, -1},
               {dt_bias, nh, false, -1},
               {A_log, nh, false, -1},
               {D, nh, false, -1},
               {conv_w, C * d->conv_width * e, false, -1},
               {conv_b, C * e, false, -1},
               {norm_w, HP * e, false, -1},
               {conv_state, ncs, true, -1},
               {ssm_state, nss, true, -1},
               {y_t, ny, true, -1}}))
    return SSD_ERR_ALIAS;
  const unsigned char* row = (const unsigned char*)zxbcdt_t;
  return hip_status(ssd::launch_decode(d->io_dtype == SSD_BF16, d->batch, d->nheads,
                                       d->headdim, d->ngroups, d->dstate, d->conv_width,
                                       row + HP * e, row_stride, zxbcdt_t, row_stride,
                                       row + (HP + C) * e, DtA{row_stride, dt_bias}, A_log, D,
                                       conv_w, conv_b, norm_w, eps, conv_state, ssm_state, y_t,
                                       (hipStream_t)stream));
}

size_t ssd_mixer_varlen_workspace_bytes(const ssd_dims* d, int32_t num_slots) {
  if (check_dims(SSD_ENTRY_MIXER_PREFILL, d) || num_slots < 1) return 0;
  if (!use_fast(d, true) || d->nheads / d->ngroups > ssd::fast_max_norm_heads()) return 0;
  return round_up(4, kWsAlign) +
         ssd::fast_varlen_ws_bytes(d->batch, d->seqlen, d->nheads, d->ngroups, num_slots);
}

int ssd_mixer_varlen(const ssd_dims* d, const int32_t* cu_seqlens, const int32_t* slots,
                     const uint8_t* has_state, int32_t num_slots, const void* xbc, const void* z,
                     const void* dt, const float* A, const float* D, const void* conv_w,
                     const void* conv_b, const void* norm_w, float eps, void* conv_pool,
                     float* ssm_pool, void* out, void* workspace, size_t ws_bytes,
                     void* stream) {
  int rc = check_dims(SSD_ENTRY_MIXER_PREFILL, d);
  if (rc) return rc;
  if (num_slots < 1) return SSD_ERR_SHAPE;
  if (!use_fast(d, true) || d->nheads / d->ngroups > ssd::fast_max_norm_heads())
    return SSD_ERR_UNSUPPORTED;
  if (!cu_seqlens || !slots || !xbc || !dt || !A || !conv_w || !conv_pool || !ssm_pool || !out)
    return SSD_ERR_NULL;
  if (z && !norm_w) return SSD_ERR_NULL;
  if (!aligned16(xbc) || !aligned16(z) || !aligned16(dt) || !aligned16(A) || !aligned16(D) ||
      !aligned16(conv_w) || !aligned16(conv_b) || !aligned16(norm_w) || !aligned16(conv_pool) ||
      !aligned16(ssm_pool) || !aligned16(out) || ((uintptr_t)cu_seqlens & 3) ||
      ((uintptr_t)slots & 3))
    return SSD_ERR_ALIGN;
  const size_t need = ssd_mixer_varlen_workspace_bytes(d, num_slots);
  if (!workspace || ws_bytes < need || ((uintptr_t)workspace % kWsAlign))
    return SSD_ERR_WORKSPACE;
  const size_t e = esize(d), T = (size_t)d->seqlen, C = channels(d), nseq = d->batch;
  const size_t HP = (size_t)d->nheads * d->headdim, nh = (size_t)d->nheads * 4;
  const size_t ncp = (size_t)num_slots * (d->conv_width - 1) * C * e,
               nsp = (size_t)num_slots * HP * d->dstate * 4;
  if (aliased({{xbc, T * C * e, false, -1},
               {z, T * HP * e, false, -1},
               {dt, T * d->nheads * e, false, -1},
               {A, nh, false, -1},
               {D, nh, false, -1},
               {conv_w, C * d->conv_width * e, false, -1},
               {conv_b, C * e, false, -1},
               {norm_w, HP * e, false, -1},
               {cu_seqlens, (nseq + 1) * 4, false, -1},
               {slots, nseq * 4, false, -1},
               {has_state, nseq, false, -1},
               {conv_pool, ncp, true, -1},
               {ssm_pool, nsp, true, -1},
               {out, T * HP * e, true, -1},
               {workspace, need, true, -1}}))
    return SSD_ERR_ALIAS;
  unsigned char* ws = (unsigned char*)workspace;
  const int64_t GN = (int64_t)d->ngroups * d->dstate;
  const unsigned char* xb = (const unsigned char*)xbc;
  ssd::FastScanArgs a{};
  a.B = d->batch;
  a.L = d->seqlen;
  a.H = d->nheads;
  a.G = d->ngroups;
  a.x = xbc;
  a.Bm = xb + HP * e;
  a.Cm = xb + (HP + GN) * e;
  a.xs = (int64_t)C;
  a.bs = (int64_t)C;
  a.dt = dt;
  a.A = A;
  a.D = D;
  a.dts = d->nheads;
  a.zs = (int64_t)HP;
  a.dt_bias = nullptr;
  a.conv = true;
  a.conv_w = conv_w;
  a.conv_b = conv_b;
  a.conv_in = nullptr;
  a.z = z;
  a.norm_w = norm_w;
  a.eps = eps;
  a.s_in = nullptr;
  a.s_out = nullptr;
  a.y = out;
  a.status = (int*)ws;
  a.ws = ws + round_up(4, kWsAlign);
  a.spin_max = g_spin_limit.load(std::memory_order_relaxed);
  a.q.cu = cu_seqlens;
  a.q.slots = slots;
  a.q.has_state = has_state;
  a.q.conv_pool = conv_pool;
  a.q.ssm_pool = ssm_pool;
  a.num_slots = num_slots;
  return hip_status(ssd::launch_fast_scan(a, (hipStream_t)stream));
}

// The backward kernels' own limits: a norm row spreads over one workgroup,
// at most 64 channels on each of 256 threads (16 on each of 1024 when the row
// is held in registers); norm groups fit a 256-entry table.
constexpr int kBwdMaxHP = 256 * 64, kBwdMaxGroups = 256;

size_t ssd_mixer_backward_workspace_bytes(const ssd_dims* d) {
  if (check_dims(SSD_ENTRY_MIXER_PREFILL, d)) return 0;
  if ((int64_t)d->nheads * d->headdim > kBwdMaxHP || d->ngroups > kBwdMaxGroups) return 0;
  return round_up(4, kWsAlign) + ssd::backward_ws_bytes(d->batch, d->seqlen, d->nheads,
                                                        d->headdim, d->ngroups, d->dstate);
}

int ssd_mixer_backward(const ssd_dims* d, const void* xbc, const void* z, const void* dt,
                       const float* A, const float* D, const void* conv_w, const void* conv_b,
                       const void* norm_w, float eps, const void* conv_state_in,
                       const float* ssm_state_in, const void* d_out,
                       const float* d_ssm_state_out, void* d_xbc, void* d_z, void* d_dt,
                       float* d_A, float* d_D, float* d_conv_w, float* d_conv_b,
                       float* d_norm_w, float* d_conv_state_in, float* d_ssm_state_in,
                       void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_dims(SSD_ENTRY_MIXER_PREFILL, d);
  if (rc) return rc;
  if ((int64_t)d->nheads * d->headdim > kBwdMaxHP || d->ngroups > kBwdMaxGroups)
    return SSD_ERR_UNSUPPORTED;
  // the recomputed forward runs the generic kernels with fp32 operands
  ssd_dims inner = *d;
  inner.flags |= SSD_FLAG_FP32_OPERANDS;
  inner.chunk = 64;
  if ((rc = check_dims(SSD_ENTRY_MIXER_PREFILL, &inner))) return rc;
  if (!xbc || !z || !dt || !A || !conv_w || !norm_w || !d_out || !d_xbc || !d_z || !d_dt ||
      !d_A || !d_conv_w || !d_norm_w)
    return SSD_ERR_NULL;
  if (!aligned16(xbc) || !aligned16(z) || !aligned16(dt) || !aligned16(A) || !aligned16(D) ||
      !aligned16(conv_w) || !aligned16(conv_b) || !aligned16(norm_w) ||
      !aligned16(conv_state_in) || !aligned16(ssm_state_in) || !aligned16(d_out) ||
      !aligned16(d_ssm_state_out) || !aligned16(d_xbc) || !aligned16(d_z) || !aligned16(d_dt) ||
      !aligned16(d_A) || !aligned16(d_D) || !aligned16(d_conv_w) || !aligned16(d_conv_b) ||
      !aligned16(d_norm_w) || !aligned16(d_conv_state_in) || !aligned16(d_ssm_state_in))
    return SSD_ERR_ALIGN;
  const size_t need = ssd_mixer_backward_workspace_bytes(d);
  if (!workspace || ws_bytes < need || ((uintptr_t)workspace % kWsAlign))
    return SSD_ERR_WORKSPACE;
  const size_t e = esize(d), T = (size_t)d->batch * d->seqlen, C = channels(d);
  const size_t HP = (size_t)d->nheads * d->headdim, nh = (size_t)d->nheads * 4;
  const size_t ncs = (size_t)d->batch * (d->conv_width - 1) * C,
               nss = (size_t)d->batch * HP * d->dstate * 4, W = d->conv_width;
  if (aliased({{xbc, T * C * e, false, -1},
               {z, T * HP * e, false, -1},
               {dt, T * d->nheads * e, false, -1},
               {A, nh, false, -1},
               {D, nh, false, -1},
               {conv_w, C * W * e, false, -1},
               {conv_b, C * e, false, -1},
               {norm_w, HP * e, false, -1},
               {conv_state_in, ncs * e, false, -1},
               {ssm_state_in, nss, false, -1},
               {d_out, T * HP * e, false, -1},
               {d_ssm_state_out, nss, false, -1},
               {d_xbc, T * C * e, true, -1},
               {d_z, T * HP * e, true, -1},
               {d_dt, T * d->nheads * e, true, -1},
               {d_A, nh, true, -1},
               {d_D, nh, true, -1},
               {d_conv_w, C * W * 4, true, -1},
               {d_conv_b, C * 4, true, -1},
               {d_norm_w, HP * 4, true, -1},
               {d_conv_state_in, ncs * 4, true, -1},
               {d_ssm_state_in, nss, true, -1},
               {workspace, need, true, -1}}))
    return SSD_ERR_ALIAS;
  ssd::BackwardArgs a{};
  a.io_bf16 = d->io_dtype == SSD_BF16;
  a.B = d->batch;
  a.L = d->seqlen;
  a.H = d->nheads;
  a.P = d->headdim;
  a.G = d->ngroups;
  a.N = d->dstate;
  a.W = d->conv_width;
  a.xbc = xbc;
  a.z = z;
  a.dt = dt;
  a.A = A;
  a.D = D;
  a.conv_w = conv_w;
  a.conv_b = conv_b;
  a.norm_w = norm_w;
  a.eps = eps;
  a.conv_in = conv_state_in;
  a.s_in = ssm_state_in;
  a.d_out = d_out;
  a.d_s_out = d_ssm_state_out;
  a.d_xbc = d_xbc;
  a.d_z = d_z;
  a.d_dt = d_dt;
  a.d_A = d_A;
  a.d_D = d_D;
  a.d_conv_w = d_conv_w;
  a.d_conv_b = d_conv_b;
  a.d_norm_w = d_norm_w;
  a.d_conv_in = d_conv_state_in;
  a.d_s_in = d_ssm_state_in;
  a.status = (int*)workspace;
  a.chunk_heads = g_bwd_heads.load(std::memory_order_relaxed);
  a.ws = (unsigned char*)workspace + round_up(4, kWsAlign);
  return hip_status(ssd::launch_backward(a, (hipStream_t)stream));
}

int ssd_workspace_status(const void* workspace, void* stream) {
  if (!workspace) return SSD_ERR_NULL;
  if ((uintptr_t)workspace % kWsAlign) return SSD_ERR_WORKSPACE;
  int word = 0;
  hipStream_t st = (hipStream_t)stream;
  if (hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return SSD_ERR_HIP;
  if (word & 4) return SSD_ERR_VARLEN;
  if (word & 1) return SSD_ERR_TIMEOUT;
  if (word & 2) return SSD_ERR_NONFINITE;
  return SSD_OK;
}

int ssd_set_exchange_spin_limit(int polls) {
  if (polls < 0) return SSD_ERR_SHAPE;
  return g_spin_limit.exchange(polls);
}

int ssd_set_backward_chunk_heads(int heads) {
  if (heads < 0 || heads > 32 || (heads & (heads - 1))) return SSD_ERR_SHAPE;
  return g_bwd_heads.exchange(heads);
}

int ssd_set_output_norm_fusion(int mode) {
  if (mode < 0 || mode > 2) return SSD_ERR_SHAPE;
  return g_norm_fuse.exchange(mode);
}

}  // extern "C"
