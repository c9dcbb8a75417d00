// Chunked state-space-duality (SSD) scan on gfx950: the block decomposition
// of the selective recurrence ("feat(model): add Nemotron-3 Nano hybrid ..."
// attribution commit: the chunk-parallel SSD block decomposition,
// ssd_minimal_discrete / segsum).
//
// For chunk k = [t0, t0 + Q) of head h (group g = h / (H/G)), with
// a_t = dt_t A_h and the inclusive segment sum Lam_t = sum_{r=t0..t} a_r:
//   chunk state   dS_k[p,n] = sum_s exp(Lam_end - Lam_s) dt_s x_s[p] B_s[n]
//   state passing S_in(0) = S_init, S_in(k+1) = exp(Lam_end,k) S_in(k) + dS_k
//   chunk output  y_t[p] = sum_{s<=t} (C_t . B_s) exp(Lam_t - Lam_s) dt_s x_s[p]
//                          + exp(Lam_t) (S_in(k) C_t)[p] + D_h x_t[p]
// The three dense contractions (B^T (w x), C B^T, and the masked (C B^T) X
// together with C S_in^T) run on 16x16 MFMA tiles with fp32 accumulation:
// fp16 operands for bf16 I/O (inputs converted as they are staged; the norm
// that may follow amplifies operand rounding, and fp16's mantissa is 8x
// finer than bf16's), fp32 operands for fp32 I/O. Decays are always
// formed as exp(Lam_t - Lam_s) of a masked difference, never as a ratio of
// exponentials, so they stay finite for any chunk length.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace ssd {

constexpr int kScanThreads = 256;  // 4 waves
constexpr int kStateSB = 64;       // tokens staged per block in the chunk-state kernel

template <class T> struct Pad { static constexpr int v = 8; };     // fp16 operands: 16 bytes per LDS row
template <> struct Pad<float> { static constexpr int v = 4; };
// MFMA operand type: fp16 for bf16 I/O unless F32OP asks for fp32 operands
// (fp32 range for every intermediate), fp32 for fp32 I/O.
template <class T, bool F32OP>
using OpT = typename std::conditional<F32OP, float, typename OpOf<T>::type>::type;
constexpr int kStatusNonFinite = 2;  // status bit: an output or the final state is not finite

// Inclusive cumulative sum of a_s = dt_s * A over the chunk (s < len; zero
// beyond) into lam[], and dt_s into dts[]. Q <= 256 = blockDim.
template <class T>
__device__ __forceinline__ void chunk_cumsum(const T* __restrict__ dt, const DtA& dta,
                                             int64_t row0, int h, float Ah, int len, float* lam,
                                             float* dts, float* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float d = 0.f;
  if (tid < len) d = dt_of(to_f(dt[(row0 + tid) * dta.dts + h]), dta, h);
  const float v = wave_incl_scan(d * Ah);
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  float add = 0.f;
  for (int w = 0; w < wave; ++w) add += wsum[w];
  lam[tid] = v + add;
  dts[tid] = d;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Phase 1: chunk states dS_k = (w x)^T B per (chunk, head, batch).
// T: I/O type (dt); TX: element type of x and B (T, or fp32 when they come
// from the conv's internal fp32 copy). MAXT: most 16x16 output tiles per wave
// (P N / 1024 rounded up to 16 or 32; d_state 256 with head_dim 128 needs 32).
template <class T, class TX, bool F32OP, int MAXT>
__global__ __launch_bounds__(kScanThreads) void k_chunk_state(
    const TX* __restrict__ x, int64_t xs, const T* __restrict__ dt, const float* __restrict__ A,
    const TX* __restrict__ Bm, int64_t bs, float* __restrict__ states,
    float* __restrict__ lam_end, int* status, DtA dta, int L, int H, int G, int P, int N, int Q,
    int nc) {
  typedef OpT<T, F32OP> O;  // MFMA operand type
  using M = Mfma<O>;
  constexpr int KP = kStateSB + Pad<O>::v;
  extern __shared__ __align__(16) unsigned char smraw[];
  O* XwT = reinterpret_cast<O*>(smraw);  // [P][KP]  x_s[p] * w_s, k = s contiguous
  O* BT = XwT + P * KP;                  // [N][KP]  B_s[n]
  __shared__ float lam[kScanThreads], dts[kScanThreads], wgt[kScanThreads], wsum[4];

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (H / G);
  const int t0 = c * Q, len = min(Q, L - t0);
  const int64_t row0 = (int64_t)b * L + t0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // this call's status word starts clear (later kernels only set bits)
  if ((blockIdx.x | blockIdx.y | blockIdx.z | threadIdx.x) == 0) *status = 0;

  chunk_cumsum<T>(dt, dta, row0, h, a_of(A, dta, h), len, lam, dts, wsum);
  const float lamE = lam[len - 1];
  wgt[tid] = tid < len ? fexp(lamE - lam[tid]) * dts[tid] : 0.f;
  __syncthreads();

  const int ntn = N / 16, tiles = (P / 16) * ntn;
  constexpr int kMaxTPW = MAXT;
  f32x4 acc[kMaxTPW];
#pragma unroll
  for (int i = 0; i < kMaxTPW; ++i) acc[i] = zero4();

  const int P8 = P / 8, N8 = N / 8;
  for (int s0 = 0; s0 < len; s0 += kStateSB) {
    for (int v = tid; v < kStateSB * P8; v += kScanThreads) {
      const int s = v / P8, p0 = (v % P8) * 8;
      float xv[8];
      if (s0 + s < len) {
        load8(x + (row0 + s0 + s) * xs + (int64_t)h * P + p0, xv);
        const float ww = wgt[s0 + s];
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] *= ww;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) XwT[(p0 + j) * KP + s] = from_f<O>(xv[j]);
    }
    for (int v = tid; v < kStateSB * N8; v += kScanThreads) {
      const int s = v / N8, n0 = (v % N8) * 8;
      float bv[8];
      if (s0 + s < len) {
        load8(Bm + (row0 + s0 + s) * bs + (int64_t)g * N + n0, bv);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) bv[j] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) BT[(n0 + j) * KP + s] = from_f<O>(bv[j]);
    }
    __syncthreads();
    const int kk = M::KPL * (lane >> 4), rr = lane & 15;
#pragma unroll
    for (int i = 0; i < kMaxTPW; ++i) {
      const int tile = wave + 4 * i;
      if (tile < tiles) {
        const int tp = tile / ntn, tn = tile % ntn;
        const O* ap = XwT + (tp * 16 + rr) * KP + kk;
        const O* bp = BT + (tn * 16 + rr) * KP + kk;
#pragma unroll
        for (int k = 0; k < kStateSB; k += M::KSTEP)
          acc[i] = M::mma(M::ld(ap + k), M::ld(bp + k), acc[i]);
      }
    }
    __syncthreads();
  }

  float* out = states + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
#pragma unroll
  for (int i = 0; i < kMaxTPW; ++i) {
    const int tile = wave + 4 * i;
    if (tile < tiles) {
      const int tp = tile / ntn, tn = tile % ntn;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = tp * 16 + 4 * (lane >> 4) + r, n = tn * 16 + (lane & 15);
        out[(int64_t)p * N + n] = acc[i][r];
      }
    }
  }
  if (tid == 0) lam_end[((int64_t)b * H + h) * nc + c] = lamE;
}

// ---------------------------------------------------------------------------
// Phase 2: state passing along the chunks, in place: states[k] := S_in(k).
__global__ __launch_bounds__(kScanThreads) void k_state_pass(float* states,
                                                             const float* __restrict__ lam_end,
                                                             const float* s_in, float* s_out,
                                                             int* status, int H, int PN, int nc) {
  const int e = (blockIdx.x * kScanThreads + threadIdx.x) * 4;
  const int h = blockIdx.y, b = blockIdx.z;
  if (e >= PN) return;
  const int64_t bh = (int64_t)b * H + h;
  float4 S = make_float4(0.f, 0.f, 0.f, 0.f);
  if (s_in) S = *reinterpret_cast<const float4*>(s_in + bh * PN + e);
  for (int c = 0; c < nc; ++c) {
    float* p = states + (((int64_t)b * nc + c) * H + h) * PN + e;
    const float4 d = *reinterpret_cast<const float4*>(p);
    *reinterpret_cast<float4*>(p) = S;
    const float al = fexp(lam_end[bh * nc + c]);
    S.x = al * S.x + d.x;
    S.y = al * S.y + d.y;
    S.z = al * S.z + d.z;
    S.w = al * S.w + d.w;
  }
  if (s_out) {
    *reinterpret_cast<float4*>(s_out + bh * PN + e) = S;
    if (S.x * 0.f + S.y * 0.f + S.z * 0.f + S.w * 0.f != 0.f) atomicOr(status, kStatusNonFinite);
  }
}

// ---------------------------------------------------------------------------
// Phase 3: chunk outputs. Each wave owns 16-row tiles of the chunk: it forms
// the causal tiles of M = (C B^T) o exp(Lam_t - Lam_s) in its LDS slab, then
// y = M (dt x) + exp(Lam_t) C S_in^T + D x for every 16-column tile of P.
template <class T, class TX, bool YF32, bool F32OP>
__global__ __launch_bounds__(kScanThreads) void k_chunk_out(
    const TX* __restrict__ x, int64_t xs, const T* __restrict__ dt, const float* __restrict__ A,
    const float* __restrict__ D, const TX* __restrict__ Bm, const TX* __restrict__ Cm, int64_t bs,
    const float* __restrict__ states, void* __restrict__ yout, int* status, DtA dta, int L, int H,
    int G, int P, int N, int Q, int nc) {
  typedef OpT<T, F32OP> O;  // MFMA operand type
  using M = Mfma<O>;
  const int QK = Q + Pad<O>::v;
  extern __shared__ __align__(16) unsigned char smraw[];
  O* XdtT = reinterpret_cast<O*>(smraw);  // [P][QK]  dt_s x_s[p], k = s contiguous
  O* Mall = XdtT + P * QK;                // [4 waves][16][QK]
  __shared__ float lam[kScanThreads], dts[kScanThreads], wsum[4];

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (H / G);
  const int t0 = c * Q, len = min(Q, L - t0);
  const int64_t row0 = (int64_t)b * L + t0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kk = M::KPL * (lane >> 4), rr = lane & 15;

  chunk_cumsum<T>(dt, dta, row0, h, a_of(A, dta, h), len, lam, dts, wsum);

  const int P8 = P / 8;
  for (int v = tid; v < Q * P8; v += kScanThreads) {
    const int s = v / P8, p0 = (v % P8) * 8;
    float xv[8];
    if (s < len) {
      load8(x + (row0 + s) * xs + (int64_t)h * P + p0, xv);
      const float d = dts[s];
#pragma unroll
      for (int j = 0; j < 8; ++j) xv[j] *= d;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) xv[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) XdtT[(p0 + j) * QK + s] = from_f<O>(xv[j]);
  }
  __syncthreads();

  const float* Sin = states + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
  const float Dh = D ? D[h] : 0.f;
  O* Mw = Mall + wave * 16 * QK;
  const TX* Cg = Cm + (int64_t)g * N;
  const TX* Bg = Bm + (int64_t)g * N;
  const int nrt = (len + 15) / 16;
  float chk = 0.f;  // NaN once any output is infinite or NaN
  for (int rt0 = 0; rt0 < nrt; rt0 += 4) {
    const int rt = rt0 + wave;
    const bool active = rt < nrt;
    const int ns = (rt + 1) * 16;
    const int nsr = (ns + M::KSTEP - 1) / M::KSTEP * M::KSTEP;
    const int trow = rt * 16 + rr;  // A-operand row of this lane
    const bool trow_ok = active && trow < len;
    if (active) {
      for (int st = 0; st <= rt; ++st) {
        const int scol = st * 16 + rr;
        const bool scol_ok = scol < len;
        f32x4 gacc = zero4();
        for (int k = 0; k < N; k += M::KSTEP) {
          // a lane's k-slice past N (N = 16 under a 32-deep fp16 MFMA) is zero
          const bool kin = k + kk < N;
          typename M::frag fa, fb;
          if (trow_ok && kin) fa = M::ldg(Cg + (row0 + trow) * bs + k + kk);
          else fa = typename M::frag{};
          if (scol_ok && kin) fb = M::ldg(Bg + (row0 + scol) * bs + k + kk);
          else fb = typename M::frag{};
          gacc = M::mma(fa, fb, gacc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = rt * 16 + 4 * (lane >> 4) + r, s = st * 16 + (lane & 15);
          float m = 0.f;
          if (s <= t && t < len) m = gacc[r] * fexp(lam[t] - lam[s]);
          Mw[(4 * (lane >> 4) + r) * QK + s] = from_f<O>(m);
        }
      }
      for (int s = ns + (lane & 15); s < nsr; s += 16)
        for (int r = 0; r < 4; ++r) Mw[(4 * (lane >> 4) + r) * QK + s] = from_f<O>(0.f);
    }
    __syncthreads();
    if (active) {
      for (int pt = 0; pt < P / 16; ++pt) {
        f32x4 acc = zero4(), acc2 = zero4();
        const O* mp = Mw + rr * QK + kk;
        const O* xp = XdtT + (pt * 16 + rr) * QK + kk;
        for (int k = 0; k < nsr; k += M::KSTEP) acc = M::mma(M::ld(mp + k), M::ld(xp + k), acc);
        const float* sp = Sin + (int64_t)(pt * 16 + rr) * N + kk;
        for (int k = 0; k < N; k += M::KSTEP) {
          const bool kin = k + kk < N;
          typename M::frag fa, fs;
          if (trow_ok && kin) fa = M::ldg(Cg + (row0 + trow) * bs + k + kk);
          else fa = typename M::frag{};
          if (kin) fs = M::cvt(sp + k);
          else fs = typename M::frag{};
          acc2 = M::mma(fa, fs, acc2);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = rt * 16 + 4 * (lane >> 4) + r, p = pt * 16 + (lane & 15);
          if (t < len) {
            const float xv = to_f(x[(row0 + t) * xs + (int64_t)h * P + p]);
            const float yv = acc[r] + fexp(lam[t]) * acc2[r] + Dh * xv;
            chk += yv * 0.f;
            const int64_t o = (row0 + t) * (int64_t)H * P + (int64_t)h * P + p;
            if (YF32) reinterpret_cast<float*>(yout)[o] = yv;
            else reinterpret_cast<T*>(yout)[o] = from_f<T>(yv);
          }
        }
      }
    }
    __syncthreads();
  }
  if (chk != 0.f) atomicOr(status, kStatusNonFinite);
}

// ---------------------------------------------------------------------------
// op16: the MFMA operands are fp16 (else fp32)
static size_t state_lds(bool op16, int P, int N) {
  const int KP = kStateSB + (op16 ? 8 : 4);
  return (size_t)(P + N) * KP * (op16 ? 2 : 4);
}
static size_t out_lds(bool op16, int P, int Q) {
  const int QK = Q + (op16 ? 8 : 4);
  return (size_t)(P + 4 * 16) * QK * (op16 ? 2 : 4);
}

hipError_t launch_chunk_state(bool io_bf16, bool x_f32, bool f32op, const ScanShape& s,
                              const void* x, int64_t xs, const void* dt, const float* A,
                              const void* Bm, int64_t bs, float* states, float* lam_end,
                              int* status, hipStream_t st) {
  ProfScope ps(st, KID_CHUNK_STATE);
  dim3 grid(s.nc, s.H, s.B), block(kScanThreads);
  const size_t lds = state_lds(io_bf16 && !f32op, s.P, s.N);
  const bool t32 = s.P * s.N > 16 * 1024;  // tiles per wave beyond 16
#define SSD_STATE_T(TT, TX, F, T)                                                              \
  hipLaunchKernelGGL((k_chunk_state<TT, TX, F, T>), grid, block, lds, st, (const TX*)x, xs,     \
                     (const TT*)dt, A, (const TX*)Bm, bs, states, lam_end, status, s.dta, s.L,  \
                     s.H, s.G, s.P, s.N, s.Q, s.nc)
#define SSD_STATE(TT, TX, F) \
  if (t32) SSD_STATE_T(TT, TX, F, 32); else SSD_STATE_T(TT, TX, F, 16)
  if (!io_bf16) {
    SSD_STATE(float, float, true);
  } else if (x_f32) {
    if (f32op) { SSD_STATE(bf16, float, true); }
    else { SSD_STATE(bf16, float, false); }
  } else {
    if (f32op) { SSD_STATE(bf16, bf16, true); }
    else { SSD_STATE(bf16, bf16, false); }
  }
#undef SSD_STATE
#undef SSD_STATE_T
  return hipGetLastError();
}

hipError_t launch_state_pass(const ScanShape& s, float* states, const float* lam_end,
                             const float* s_in, float* s_out, int* status, hipStream_t st) {
  ProfScope ps(st, KID_STATE_PASS);
  const int PN = s.P * s.N;
  dim3 grid((PN / 4 + kScanThreads - 1) / kScanThreads, s.H, s.B), block(kScanThreads);
  hipLaunchKernelGGL(k_state_pass, grid, block, 0, st, states, lam_end, s_in, s_out, status, s.H,
                     PN, s.nc);
  return hipGetLastError();
}

hipError_t launch_chunk_out(bool io_bf16, bool x_f32, bool f32op, const ScanShape& s,
                            const void* x, int64_t xs, const void* dt, const float* A,
                            const float* D, const void* Bm, const void* Cm, int64_t bs,
                            const float* states, void* y, bool y_f32, int* status,
                            hipStream_t st) {
  ProfScope ps(st, KID_CHUNK_OUT);
  dim3 grid(s.nc, s.H, s.B), block(kScanThreads);
  const size_t lds = out_lds(io_bf16 && !f32op, s.P, s.Q);
#define SSD_OUT(TT, TX, YF, F)                                                                  \
  hipLaunchKernelGGL((k_chunk_out<TT, TX, YF, F>), grid, block, lds, st, (const TX*)x, xs,      \
                     (const TT*)dt, A, D, (const TX*)Bm, (const TX*)Cm, bs, states, y, status,  \
                     s.dta, s.L, s.H, s.G, s.P, s.N, s.Q, s.nc)
#define SSD_OUT_F(TT, TX, YF) \
  if (f32op) SSD_OUT(TT, TX, YF, true); else SSD_OUT(TT, TX, YF, false)
  if (!io_bf16) SSD_OUT(float, float, true, true);
  else if (x_f32) {
    if (y_f32) { SSD_OUT_F(bf16, float, true); }
    else { SSD_OUT_F(bf16, float, false); }
  } else {
    if (y_f32) { SSD_OUT_F(bf16, bf16, true); }
    else { SSD_OUT_F(bf16, bf16, false); }
  }
#undef SSD_OUT_F
#undef SSD_OUT
  return hipGetLastError();
}

// LDS bytes the two MFMA kernels need for a shape (the host checks these
// against the 160 KiB of one CU before launching).
size_t scan_lds_bytes(bool op16, int P, int N, int Q) {
  const size_t a = state_lds(op16, P, N), b = out_lds(op16, P, Q);
  return a > b ? a : b;
}

}  // namespace ssd
