// C ABI of the Mamba-2 mixer core (declared in include/ssd_mi355x.h):
// host-side argument checks, workspace carving and kernel launches. Nothing
// here allocates device memory or keeps mutable global state.
#include <stdint.h>
#include <string.h>

#include "../../include/ssd_mi355x.h"
#include "launch.hpp"

namespace ssd {
size_t scan_lds_bytes(bool io_bf16, int P, int N, int Q);
}

namespace {

constexpr size_t kLdsPerCU = 160 * 1024;
constexpr size_t kWsAlign = 256;

size_t esize(const ssd_dims* d) { return d->io_dtype == SSD_BF16 ? 2 : 4; }
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
int64_t nchunks(const ssd_dims* d) { return (d->seqlen + d->chunk - 1) / d->chunk; }

// Byte ranges: NULL or identical pointers are fine, any other overlap is not.
bool partial_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || a == b) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}
bool any_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int check_dims(int entry, const ssd_dims* d) {
  if (!d) return SSD_ERR_NULL;
  if (d->io_dtype != SSD_F32 && d->io_dtype != SSD_BF16) return SSD_ERR_DTYPE;
  if (d->batch < 1 || d->seqlen < 1 || d->nheads < 1 || d->headdim < 1 || d->ngroups < 1 ||
      d->dstate < 1)
    return SSD_ERR_SHAPE;
  if (d->nheads % d->ngroups != 0) return SSD_ERR_SHAPE;
  if (!is_one_of(d->headdim, {16, 32, 64, 128})) return SSD_ERR_UNSUPPORTED;
  if (!is_one_of(d->dstate, {16, 32, 64, 128})) return SSD_ERR_UNSUPPORTED;
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
    if (ssd::scan_lds_bytes(d->io_dtype == SSD_BF16, d->headdim, d->dstate, d->chunk) >
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
  float* states;
  float* lam_end;
  float* y32;
  unsigned char* conv;
  void* fastws;
  size_t total;
};

bool use_fast(const ssd_dims* d, bool conv) {
  return ssd::fast_path_ok(d->io_dtype == SSD_BF16, d->headdim, d->dstate, d->nheads, d->ngroups,
                           d->chunk, d->conv_width, conv);
}

// Workspace layout for the scan (conv = the scan consumes raw xBC rows).
ScanWs carve(const ssd_dims* d, void* base, bool conv) {
  ScanWs w{};
  const size_t B = d->batch, L = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate;
  const size_t nc = nchunks(d);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += round_up(bytes, kWsAlign);
    return o;
  };
  w.fast = use_fast(d, conv);
  size_t o_states = 0, o_lam = 0, o_y = 0, o_conv = 0, o_fast = 0;
  if (w.fast) {
    o_fast = take(ssd::fast_ws_bytes(d->batch, d->seqlen, d->nheads, d->ngroups, conv));
  } else {
    o_states = take(B * nc * H * P * N * 4);
    o_lam = take(B * H * nc * 4);
    o_y = take(B * L * H * P * 4);
    if (conv) o_conv = take(B * L * (size_t)channels(d) * 4);  // fp32 conv output
  }
  w.total = off;
  if (base) {
    unsigned char* p = (unsigned char*)base;
    if (w.fast) {
      w.fastws = p + o_fast;
    } else {
      w.states = (float*)(p + o_states);
      w.lam_end = (float*)(p + o_lam);
      w.y32 = (float*)(p + o_y);
      w.conv = conv ? p + o_conv : nullptr;
    }
  }
  return w;
}

// x_f32: x, B and C are fp32 (the conv's internal copy), else the I/O type.
int run_scan(const ssd_dims* d, const void* x, int64_t xs, const void* dt, const float* A,
             const float* D, const void* Bm, const void* Cm, int64_t bs, bool x_f32, const void* z,
             const void* norm_w, float eps, const float* s_in, float* s_out, void* y,
             const ScanWs& ws, hipStream_t st) {
  const bool bf = d->io_dtype == SSD_BF16;
  ssd::ScanShape s{d->batch, d->seqlen, d->nheads, d->headdim, d->ngroups,
                   d->dstate, d->chunk, (int)nchunks(d)};
  int rc = hip_status(
      ssd::launch_chunk_state(bf, x_f32, s, x, xs, dt, A, Bm, bs, ws.states, ws.lam_end, st));
  if (rc) return rc;
  rc = hip_status(ssd::launch_state_pass(s, ws.states, ws.lam_end, s_in, s_out, st));
  if (rc) return rc;
  const bool fused_norm = z != nullptr;
  void* ydst = fused_norm ? (void*)ws.y32 : y;
  rc = hip_status(ssd::launch_chunk_out(bf, x_f32, s, x, xs, dt, A, D, Bm, Cm, bs, ws.states, ydst,
                                        fused_norm || !bf, st));
  if (rc) return rc;
  if (fused_norm)
    rc = hip_status(ssd::launch_gated_norm(bf, true, d->batch * d->seqlen,
                                           d->nheads * d->headdim, d->ngroups, ws.y32, z,
                                           norm_w, eps, y, st));
  return rc;
}

int run_fast(const ssd_dims* d, bool conv, const void* x, const void* Bm, const void* Cm,
             int64_t xs, int64_t bs, const void* dt, const float* A, const float* D,
             const void* conv_w, const void* conv_b, const void* conv_in, const void* z,
             const void* norm_w, float eps, const float* s_in, float* s_out, void* y,
             const ScanWs& ws, hipStream_t st) {
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
  return hip_status(ssd::launch_fast_scan(a, st));
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
  if (any_overlap(out, no, xbc, nx) || any_overlap(out, no, conv_state_in, ns) ||
      any_overlap(out, no, conv_state_out, ns) || partial_overlap(conv_state_in, ns, conv_state_out, ns) ||
      any_overlap(conv_state_out, ns, xbc, nx))
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
  if (any_overlap(y, ny, x, nx) || any_overlap(y, ny, Bm, nb) || any_overlap(y, ny, Cm, nb) ||
      any_overlap(y, ny, dt, T * d->nheads * e) || any_overlap(y, ny, z, ny) ||
      any_overlap(y, ny, ssm_state_in, nst) || any_overlap(y, ny, ssm_state_out, nst) ||
      partial_overlap(ssm_state_in, nst, ssm_state_out, nst) ||
      any_overlap(workspace, need.total, y, ny) || any_overlap(workspace, need.total, x, nx))
    return SSD_ERR_ALIAS;
  const ScanWs ws = carve(d, workspace, false);
  if (ws.fast)
    return run_fast(d, false, x, Bm, Cm, x_tok_stride, bc_tok_stride, dt, A, D, nullptr, nullptr,
                    nullptr, z, norm_w, eps, ssm_state_in, ssm_state_out, y, ws,
                    (hipStream_t)stream);
  return run_scan(d, x, x_tok_stride, dt, A, D, Bm, Cm, bc_tok_stride, false, z, norm_w, eps,
                  ssm_state_in, ssm_state_out, y, ws, (hipStream_t)stream);
}

int ssd_gated_rmsnorm(const ssd_dims* d, const void* y, const void* z, const void* w, float eps,
                      void* out, void* stream) {
  int rc = check_dims(SSD_ENTRY_GATED_RMSNORM, d);
  if (rc) return rc;
  if (!y || !z || !w || !out) return SSD_ERR_NULL;
  if (!aligned16(y) || !aligned16(z) || !aligned16(w) || !aligned16(out)) return SSD_ERR_ALIGN;
  const size_t n = (size_t)d->batch * d->seqlen * d->nheads * d->headdim * esize(d);
  if (partial_overlap(out, n, y, n) || any_overlap(out, n, z, n)) return SSD_ERR_ALIAS;
  return hip_status(ssd::launch_gated_norm(d->io_dtype == SSD_BF16, false,
                                           d->batch * d->seqlen, d->nheads * d->headdim,
                                           d->ngroups, y, z, w, eps, out, (hipStream_t)stream));
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
  if (any_overlap(y_t, ny, xbc_t, B * C * e) || any_overlap(y_t, ny, z_t, ny) ||
      any_overlap(y_t, ny, conv_state, ncs) || any_overlap(y_t, ny, ssm_state, nss) ||
      any_overlap(conv_state, ncs, ssm_state, nss) || any_overlap(conv_state, ncs, xbc_t, B * C * e))
    return SSD_ERR_ALIAS;
  return hip_status(ssd::launch_decode(d->io_dtype == SSD_BF16, d->batch, d->nheads,
                                       d->headdim, d->ngroups, d->dstate, d->conv_width, xbc_t,
                                       z_t, dt_t, A, D, conv_w, conv_b, norm_w, eps, conv_state,
                                       ssm_state, y_t, (hipStream_t)stream));
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
  if (any_overlap(out, no, xbc, nx) || any_overlap(out, no, z, no) ||
      any_overlap(out, no, dt, T * d->nheads * e) || any_overlap(out, no, conv_state_in, ncs) ||
      any_overlap(out, no, conv_state_out, ncs) || any_overlap(out, no, ssm_state_in, nss) ||
      any_overlap(out, no, ssm_state_out, nss) ||
      partial_overlap(conv_state_in, ncs, conv_state_out, ncs) ||
      partial_overlap(ssm_state_in, nss, ssm_state_out, nss) ||
      any_overlap(conv_state_out, ncs, xbc, nx) || any_overlap(workspace, need.total, out, no) ||
      any_overlap(workspace, need.total, xbc, nx))
    return SSD_ERR_ALIAS;
  const ScanWs ws = carve(d, workspace, true);
  hipStream_t st = (hipStream_t)stream;
  const bool bf = d->io_dtype == SSD_BF16;
  const int64_t GN = (int64_t)d->ngroups * d->dstate;
  if (ws.fast) {
    // conv recomputed inside the scan kernels; the new conv state is taken
    // after them because they read conv_state_in (which it may overwrite).
    const unsigned char* xb = (const unsigned char*)xbc;
    rc = run_fast(d, true, xbc, xb + HP * e, xb + (HP + GN) * e, C, C, dt, A, D, conv_w, conv_b,
                  conv_state_in, z, norm_w, eps, ssm_state_in, ssm_state_out, out, ws, st);
    if (rc || !conv_state_out) return rc;
    return hip_status(ssd::launch_conv_state(bf, d->batch, d->seqlen, (int)C, d->conv_width, xbc,
                                             C, conv_state_in, conv_state_out, st));
  }
  // the conv output stays fp32 for the scan: with a conv bias, B and C carry
  // a shared offset whose C.B products cancel, so their rounding matters
  rc = hip_status(ssd::launch_conv1d(bf, d->batch, d->seqlen, (int)C, d->conv_width, xbc, C,
                                     conv_w, conv_b, conv_state_in, ws.conv, C, true, st));
  if (rc) return rc;
  if (conv_state_out) {
    rc = hip_status(ssd::launch_conv_state(bf, d->batch, d->seqlen, (int)C, d->conv_width, xbc,
                                           C, conv_state_in, conv_state_out, st));
    if (rc) return rc;
  }
  const unsigned char* v = ws.conv;
  return run_scan(d, v, C, dt, A, D, v + HP * 4, v + (HP + GN) * 4, C, true, z, norm_w, eps,
                  ssm_state_in, ssm_state_out, out, ws, st);
}

}  // extern "C"
