// Backward pass of the mixer prefill (conv + SiLU, chunked SSD scan, gated
// RMSNorm): given d_out (and optionally the gradient of the final SSM
// state), the gradients with respect to xBC, z, dt, A, D, the conv weight
// and bias, the norm weight and the initial states ("feat(model): add
// Nemotron-3 Nano hybrid ..." section "Testing": gradient flow through the
// mixer; "Caveats": the native backend is activation-memory hungry).
//
// The forward is recomputed first on the general kernels with fp32 MFMA
// operands (conv output v, the carried-in state of every chunk, pre-norm y);
// then, per chunk k of head h with Lam the inclusive cumsum of dt A inside
// the chunk, E[t,s] = exp(Lam_t - Lam_s) (s <= t), G = C B^T, K = dY X^T:
//   dX[s]   = sum_{t>=s} G E dt_s dY[t] + D dY[s] + w_s (dS_out B_s),  w_s = exp(Lam_end - Lam_s) dt_s
//   dC[t]   = sum_{s<=t} K E dt_s B[s] + exp(Lam_t) dY[t] S_in
//   dB[s]   = sum_{t>=s} K E dt_s C[t] + w_s X[s] dS_out
//   dS_in   = exp(Lam_end) dS_out + sum_t exp(Lam_t) dY[t] (outer) C[t]
// with dS_out of chunk k the dS_in of chunk k+1 (a reverse pass over the
// chunks), and dt, A through dLam (reverse cumsum within the chunk). The
// gated norm and the conv are differentiated directly. Everything is fp32;
// dense products are plain loops over L2-resident operands.
#include "common.hpp"
#include "launch.hpp"

namespace ssd {
namespace bwd {

constexpr int kThreads = 256;
constexpr int kNormRows = 8;      // rows per norm-backward workgroup
constexpr int kMaxNormVec = 64;   // H*P / 256 channels per thread at most
constexpr int kMaxGroups = 256;

// zero n floats
__global__ __launch_bounds__(kThreads) void k_zero(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    p[i] = 0.f;
}

// ---------------------------------------------------------------- gated norm
// q = y silu(z), r = (mean_group(q^2) + eps)^-1/2, out = q r w. For each row:
//   dq = w r g - q r^3 mean_group(w g q);  dy = dq silu(z);
//   dz = dq y silu'(z);  dw += g q r  (summed over rows).
// dy overwrites y (each thread reads its channels before writing them).
template <class T>
__global__ __launch_bounds__(kThreads) void k_norm_bwd(float* y, const T* __restrict__ z,
                                                       const T* __restrict__ w,
                                                       const T* __restrict__ g, float eps,
                                                       T* __restrict__ dz, float* dw,
                                                       int64_t rows, int HP, int G) {
  __shared__ float sq[kMaxGroups], sg[kMaxGroups];
  const int tid = threadIdx.x;
  const int S = HP / G;
  float dwp[kMaxNormVec];
#pragma unroll
  for (int i = 0; i < kMaxNormVec; ++i) dwp[i] = 0.f;
  const int nv = (HP + kThreads - 1) / kThreads;
  for (int rr = 0; rr < kNormRows; ++rr) {
    const int64_t row = (int64_t)blockIdx.x * kNormRows + rr;
    if (row >= rows) break;
    for (int j = tid; j < G; j += kThreads) sq[j] = sg[j] = 0.f;
    __syncthreads();
    for (int i = 0; i < nv; ++i) {
      const int c = tid + i * kThreads;
      if (c < HP) {
        const int64_t o = row * HP + c;
        const float zz = to_f(z[o]), q = y[o] * zz / (1.f + __expf(-zz));
        atomicAdd(&sq[c / S], q * q);
        atomicAdd(&sg[c / S], to_f(w[c]) * to_f(g[o]) * q);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMaxNormVec; ++i) {
      const int c = tid + i * kThreads;
      if (i < nv && c < HP) {
        const int64_t o = row * HP + c;
        const int j = c / S;
        const float r = rsqrtf(sq[j] / S + eps), k3 = r * r * r * sg[j] / S;
        const float zz = to_f(z[o]), sig = 1.f / (1.f + __expf(-zz)), s = zz * sig;
        const float yy = y[o], q = yy * s, gg = to_f(g[o]);
        const float dq = to_f(w[c]) * r * gg - q * k3;
        y[o] = dq * s;
        dz[o] = from_f<T>(dq * yy * (sig + s * (1.f - sig)));
        dwp[i] += gg * q * r;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < kMaxNormVec; ++i) {
    const int c = tid + i * kThreads;
    if (i < nv && c < HP) atomicAdd(dw + c, dwp[i]);
  }
}

// ---------------------------------------------------------------- chunk Lam
// Lam (inclusive cumsum of dt A over the chunk, natural log units), dt and
// exp(Lam) of the first len positions into lam / dts / ex (Q <= 64: wave 0).
template <class T>
__device__ __forceinline__ void chunk_lam(const T* __restrict__ dt, const DtA& dta, int64_t row0,
                                          int h, float Ah, int len, float* lam, float* dts,
                                          float* ex) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const float d = tid < len ? dt_of(to_f(dt[(row0 + tid) * dta.dts + h]), dta, h) : 0.f;
    const float v = wave_incl_scan(d * Ah);
    lam[tid] = v;
    dts[tid] = d;
    ex[tid] = __expf(v);
  }
  __syncthreads();
}

// ---------------------------------------------------------------- dS_in part
// Z[p,n] = sum_t exp(Lam_t) dY[t,p] C[t,n] of one (chunk, head), into zb.
template <class T>
__global__ __launch_bounds__(kThreads) void k_chunk_z(const float* __restrict__ v,
                                                      const float* __restrict__ dY,
                                                      const T* __restrict__ dt, DtA dta,
                                                      const float* __restrict__ A, float* zb,
                                                      int L, int H, int G, int P, int N, int Q,
                                                      int nc) {
  __shared__ float lam[64], dts[64], ex[64];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z, g = h / (H / G);
  const int t0 = c * Q, len = min(Q, L - t0);
  const int64_t row0 = (int64_t)b * L + t0;
  const int HP = H * P, C = HP + 2 * G * N, co = HP + G * N + g * N;
  chunk_lam<T>(dt, dta, row0, h, a_of(A, dta, h), len, lam, dts, ex);
  float* out = zb + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
  for (int i = threadIdx.x; i < P * N; i += kThreads) {
    const int p = i / N, n = i % N;
    float acc = 0.f;
    for (int t = 0; t < len; ++t)
      acc += ex[t] * dY[(row0 + t) * HP + h * P + p] * v[(row0 + t) * C + co + n];
    out[i] = acc;
  }
}

// ---------------------------------------------------------------- reverse pass
// dS (adjoint of the state) from the last chunk back: buf[k] holds Z_k on
// entry and dS_out(k) on exit; dS_in(k) = exp(Lam_end,k) dS_out(k) + Z_k,
// dS_out(k - 1) = dS_in(k). The initial state's gradient is dS_in(0).
__global__ __launch_bounds__(kThreads) void k_rev_pass(float* buf, const float* __restrict__ lam_end,
                                                       const float* __restrict__ d_final,
                                                       float* d_init, int H, int PN, int nc) {
  const int e = blockIdx.x * kThreads + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  if (e >= PN) return;
  const int64_t bh = (int64_t)b * H + h;
  float dS = d_final ? d_final[bh * PN + e] : 0.f;
  for (int k = nc - 1; k >= 0; --k) {
    float* p = buf + (((int64_t)b * nc + k) * H + h) * PN + e;
    const float z = *p;
    *p = dS;
    dS = __expf(lam_end[bh * nc + k]) * dS + z;
  }
  if (d_init) d_init[bh * PN + e] = dS;
}

// ---------------------------------------------------------------- chunk grads
// One (chunk, head, batch): dX into dv's x channels, this head's share of dB
// and dC into dBh / dCh [T, H, N], d(dt) into ddt (io dtype), and dA, dD.
// dt and A reach the output through Lam only (a_u = dt_u A feeds Lam_t for
// every t >= u), so d(a_u) is the sum over t >= u of dLam_t. That sum is
// formed term by term, without differences of partial sums:
//   intra-chunk:  sum_{t>=u} sum_{s<u} F[t,s] dt_s,  F = K o G o E
//   state out:    exp(Lam_end) <dS_out, S_in> + sum_{s<u} w_s U_s
//   inter-chunk:  sum_{t>=u} Y_t,  Y_t = dY[t] . (exp(Lam_t) C_t S_in)
// where U_s = B_s . (X[s] dS_out).
template <class T>
__global__ __launch_bounds__(kThreads) void k_chunk_bwd(
    const float* __restrict__ v, const float* __restrict__ dY, const T* __restrict__ dt, DtA dta,
    const float* __restrict__ A, const float* __restrict__ D, const float* __restrict__ Sin,
    const float* __restrict__ dSo, float* __restrict__ dv, float* __restrict__ dBh,
    float* __restrict__ dCh, T* __restrict__ ddt, float* dA, float* dD, int L, int H, int G,
    int P, int N, int Q, int nc) {
  extern __shared__ float sm[];
  const int QS = Q + 1;
  float* Km = sm;               // [Q][QS]: K = dY X^T, then dG = K E dt_s
  float* Gm = sm + Q * QS;      // [Q][QS]: G = C B^T, then M = G E dt_s
  float* Fm = sm + 2 * Q * QS;  // [Q][QS]: F = K G E, then its column suffix sums
  __shared__ float lam[64], dts[64], ex[64], wv[64], colF[64], Yo[64], U[64], dai[64], tmp[64];
  __shared__ float red[4];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z, g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = c * Q, len = min(Q, L - t0);
  const int64_t row0 = (int64_t)b * L + t0;
  const int HP = H * P, C = HP + 2 * G * N;
  const int xo = h * P, bo = HP + g * N, co = HP + G * N + g * N;
  const float Ah = a_of(A, dta, h), Dh = D ? D[h] : 0.f;
  const int64_t sb = (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
  const float* Si = Sin + sb;
  const float* dS = dSo + sb;
  chunk_lam<T>(dt, dta, row0, h, Ah, len, lam, dts, ex);
  const float lamE = lam[len - 1];
  if (tid < 64) {
    wv[tid] = tid < len ? __expf(lamE - lam[tid]) * dts[tid] : 0.f;
    Yo[tid] = 0.f;
    U[tid] = 0.f;
  }
  if (tid < 4) red[tid] = 0.f;
  // K and G over the causal pairs
  for (int i = tid; i < Q * Q; i += kThreads) {
    const int t = i / Q, s = i % Q;
    float k = 0.f, gg = 0.f;
    if (s <= t && t < len) {
      const float* dy = dY + (row0 + t) * HP + xo;
      const float* xs = v + (row0 + s) * C + xo;
      for (int p = 0; p < P; ++p) k += dy[p] * xs[p];
      const float* ct = v + (row0 + t) * C + co;
      const float* bs = v + (row0 + s) * C + bo;
      for (int n = 0; n < N; ++n) gg += ct[n] * bs[n];
    }
    Km[t * QS + s] = k;
    Gm[t * QS + s] = gg;
  }
  __syncthreads();
  // F by columns: thread s walks t down from the chunk's end, keeping
  // R[t,s] = sum_{t' >= t} F[t',s] in place for t > s; colF[s] = R[s,s]
  if (tid < Q) {
    const int s = tid;
    float acc = 0.f;
    for (int t = len - 1; t >= s; --t) {
      acc += Km[t * QS + s] * Gm[t * QS + s] * __expf(lam[t] - lam[s]);
      Fm[t * QS + s] = acc;
    }
    colF[s] = acc;
  }
  __syncthreads();
  // dai[u] = sum_{s<u} dt_s R[u,s] (four lanes per u) and the dt_s E scaling
  {
    const int u = tid >> 2, j = tid & 3;
    float acc = 0.f;
    if (u < len)
      for (int s = j; s < u; s += 4) acc += dts[s] * Fm[u * QS + s];
    acc = group_sum_last<4>(acc);
    if (j == 0 && u < Q) dai[u] = acc;
  }
  for (int i = tid; i < Q * Q; i += kThreads) {
    const int t = i / Q, s = i % Q;
    const float f = (s <= t && t < len) ? __expf(lam[t] - lam[s]) * dts[s] : 0.f;
    Km[t * QS + s] *= f;
    Gm[t * QS + s] *= f;
  }
  __syncthreads();
  // dX[s,p] and dD
  float ddp = 0.f;
  for (int i = tid; i < len * P; i += kThreads) {
    const int s = i / P, p = i % P;
    float acc = 0.f;
    for (int t = s; t < len; ++t) acc += Gm[t * QS + s] * dY[(row0 + t) * HP + xo + p];
    const float dys = dY[(row0 + s) * HP + xo + p];
    const float* bs = v + (row0 + s) * C + bo;
    const float* dsp = dS + (int64_t)p * N;
    float t3 = 0.f;
    for (int n = 0; n < N; ++n) t3 += bs[n] * dsp[n];
    dv[(row0 + s) * C + xo + p] = acc + Dh * dys + wv[s] * t3;
    ddp += dys * v[(row0 + s) * C + xo + p];
  }
  // dC[t,n] (and Y_t)
  for (int i = tid; i < len * N; i += kThreads) {
    const int t = i / N, n = i % N;
    float acc = 0.f;
    for (int s = 0; s <= t; ++s) acc += Km[t * QS + s] * v[(row0 + s) * C + bo + n];
    const float* dy = dY + (row0 + t) * HP + xo;
    float t1 = 0.f;
    for (int p = 0; p < P; ++p) t1 += dy[p] * Si[(int64_t)p * N + n];
    dCh[((row0 + t) * H + h) * N + n] = acc + ex[t] * t1;
    atomicAdd(&Yo[t], ex[t] * v[(row0 + t) * C + co + n] * t1);
  }
  // dB[s,n] (and U_s)
  for (int i = tid; i < len * N; i += kThreads) {
    const int s = i / N, n = i % N;
    float acc = 0.f;
    for (int t = s; t < len; ++t) acc += Km[t * QS + s] * v[(row0 + t) * C + co + n];
    const float* xs = v + (row0 + s) * C + xo;
    float t2 = 0.f;
    for (int p = 0; p < P; ++p) t2 += xs[p] * dS[(int64_t)p * N + n];
    dBh[((row0 + s) * H + h) * N + n] = acc + wv[s] * t2;
    atomicAdd(&U[s], v[(row0 + s) * C + bo + n] * t2);
  }
  // <dS_out, S_in>
  float cst = 0.f;
  for (int i = tid; i < P * N; i += kThreads) cst += dS[i] * Si[i];
  cst = wave_sum(cst);
  ddp = wave_sum(ddp);
  if (lane == 0) {
    atomicAdd(&red[0], cst);
    atomicAdd(&red[1], ddp);
  }
  __syncthreads();
  if (tid == 0 && dD) atomicAdd(dD + h, red[1]);
  // d(a_u), d(dt_u) and dA (wave 0, one lane per position)
  if (wave == 0) {
    const int u = lane;
    // sum_{t >= u} Y_t: an inclusive scan over the reversed positions
    const float ry = wave_incl_scan(63 - u < len ? Yo[63 - u] : 0.f);
    tmp[63 - u] = ry;
    // sum_{s < u} w_s U_s: an inclusive scan of the shifted terms
    const float pw = wave_incl_scan(u > 0 && u - 1 < len ? wv[u - 1] * U[u - 1] : 0.f);
    __builtin_amdgcn_wave_barrier();  // tmp is written and read by one wave
    float da_dt = 0.f;
    if (u < len) {
      const float da = dai[u] + tmp[u] + __expf(lamE) * red[0] + pw;
      const float dd = colF[u] + __expf(lamE - lam[u]) * U[u] + Ah * da;
      ddt[(row0 + u) * (int64_t)H + h] = from_f<T>(dd);
      da_dt = dts[u] * da;
    }
    const float sa = wave_sum(da_dt);
    if (lane == 0) atomicAdd(dA + h, sa);
  }
}

// ---------------------------------------------------------------- group sums
// dv's B and C channels = the sums of dBh / dCh over the heads of each group.
__global__ __launch_bounds__(kThreads) void k_group_sum(const float* __restrict__ dBh,
                                                        const float* __restrict__ dCh,
                                                        float* dv, int64_t T, int H, int G,
                                                        int N, int HP) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= T * G * N) return;
  const int64_t t = i / (G * N);
  const int gn = (int)(i % (G * N)), g = gn / N, n = gn % N, hpg = H / G;
  float sb = 0.f, sc = 0.f;
  for (int k = 0; k < hpg; ++k) {
    const int64_t o = (t * H + g * hpg + k) * N + n;
    sb += dBh[o];
    sc += dCh[o];
  }
  const int64_t C = HP + 2 * (int64_t)G * N;
  dv[t * C + HP + gn] = sb;
  dv[t * C + HP + (int64_t)G * N + gn] = sc;
}

// ---------------------------------------------------------------- conv + SiLU
// du = dv silu'(u) over a range of kConvTok tokens of one channel (u
// recomputed from [conv state ; xbc]); du overwrites dv; dw, db summed.
constexpr int kConvTok = 64;
template <class T>
__global__ __launch_bounds__(kThreads) void k_conv_du(const T* __restrict__ xbc,
                                                      const T* __restrict__ cin,
                                                      const T* __restrict__ w,
                                                      const T* __restrict__ bias, float* dv,
                                                      float* dw, float* db, int L, int C, int W) {
  const int c = blockIdx.x * kThreads + threadIdx.x;
  const int t0 = blockIdx.y * kConvTok, b = blockIdx.z;
  if (c >= C) return;
  float wk[4] = {0.f, 0.f, 0.f, 0.f}, dwp[4] = {0.f, 0.f, 0.f, 0.f}, dbp = 0.f;
  for (int k = 0; k < W; ++k) wk[k] = to_f(w[(int64_t)c * W + k]);
  const float bc = bias ? to_f(bias[c]) : 0.f;
  // ext row e: conv state rows (e < W-1) or token e - (W-1)
  auto ext = [&](int e) -> float {
    if (e >= W - 1) return to_f(xbc[((int64_t)b * L + e - (W - 1)) * C + c]);
    return cin ? to_f(cin[((int64_t)b * (W - 1) + e) * C + c]) : 0.f;
  };
  for (int t = t0; t < min(L, t0 + kConvTok); ++t) {
    float e[4];
    float u = bc;
    for (int k = 0; k < W; ++k) {
      e[k] = ext(t + k);
      u += wk[k] * e[k];
    }
    const float sig = 1.f / (1.f + __expf(-u));
    const int64_t o = ((int64_t)b * L + t) * C + c;
    const float du = dv[o] * (sig + u * sig * (1.f - sig));
    dv[o] = du;
    for (int k = 0; k < W; ++k) dwp[k] += du * e[k];
    dbp += du;
  }
  for (int k = 0; k < W; ++k) atomicAdd(dw + (int64_t)c * W + k, dwp[k]);
  if (db) atomicAdd(db + c, dbp);
}

// Gradient of the conv input rows ext = [conv state ; xbc]: d_ext[e] =
// sum_k w[k] du[e - k] over output tokens e - k in range; rows e >= W-1 go to
// d_xbc, the first W-1 to the initial conv state's gradient (fp32).
template <class T>
__global__ __launch_bounds__(kThreads) void k_conv_dx(const float* __restrict__ du,
                                                      const T* __restrict__ w, T* __restrict__ dx,
                                                      float* dcin, int L, int C, int W) {
  const int c = blockIdx.x * kThreads + threadIdx.x;
  const int e0 = blockIdx.y * kConvTok, b = blockIdx.z;
  if (c >= C) return;
  float wk[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < W; ++k) wk[k] = to_f(w[(int64_t)c * W + k]);
  for (int e = e0; e < min(L + W - 1, e0 + kConvTok); ++e) {
    float acc = 0.f;
    for (int k = 0; k < W; ++k) {
      const int tt = e - k;  // output token whose window puts tap k on row e
      if (tt >= 0 && tt < L) acc += wk[k] * du[((int64_t)b * L + tt) * C + c];
    }
    if (e >= W - 1)
      dx[((int64_t)b * L + e - (W - 1)) * C + c] = from_f<T>(acc);
    else if (dcin)
      dcin[((int64_t)b * (W - 1) + e) * C + c] = acc;
  }
}

}  // namespace bwd

// Workspace of the backward pass: fp32 v, y / dY, carried-in states, Lam_end,
// dS_out, per-head dB / dC and dv, for chunk length Q.
namespace {
size_t bround(size_t b) { return (b + 255) / 256 * 256; }
}
// chunk length of the backward kernels (their [Q][Q+1] tiles live in LDS)
constexpr int kBwdChunk = 64;
size_t backward_ws_bytes(int B, int L, int H, int P, int G, int N) {
  const size_t T = (size_t)B * L, HP = (size_t)H * P, C = HP + 2 * (size_t)G * N;
  const size_t Q = kBwdChunk, nc = (L + Q - 1) / Q;
  const size_t st = (size_t)B * nc * H * P * N * 4;
  return bround(T * C * 4) + bround(T * HP * 4) + 2 * bround(st) + bround((size_t)B * H * nc * 4) +
         2 * bround(T * H * N * 4) + bround(T * C * 4);
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t st) {
  using namespace bwd;
  const bool bf = a.io_bf16;
  const int B = a.B, L = a.L, H = a.H, P = a.P, G = a.G, N = a.N, W = a.W;
  const int64_t T = (int64_t)B * L, HP = (int64_t)H * P, C = HP + 2 * (int64_t)G * N;
  const int Q = kBwdChunk, nc = (L + Q - 1) / Q;
  const size_t sts = (size_t)B * nc * H * P * N * 4;
  unsigned char* w = (unsigned char*)a.ws;
  float* v = (float*)w;
  w += bround(T * C * 4);
  float* y = (float*)w;
  w += bround(T * HP * 4);
  float* states = (float*)w;
  w += bround(sts);
  float* dso = (float*)w;
  w += bround(sts);
  float* lam_end = (float*)w;
  w += bround((size_t)B * H * nc * 4);
  float* dBh = (float*)w;
  w += bround(T * H * N * 4);
  float* dCh = (float*)w;
  w += bround(T * H * N * 4);
  float* dv = (float*)w;
  const DtA plain{H, nullptr};
  hipError_t e;
#define SSD_CHECK()                         \
  if ((e = hipGetLastError()) != hipSuccess) \
    return e;
  // recompute the forward pieces (fp32 operands)
  e = launch_conv1d(bf, B, L, (int)C, W, a.xbc, C, a.conv_w, a.conv_b, a.conv_in, v, C, true, st);
  if (e != hipSuccess) return e;
  ScanShape s{B, L, H, P, G, N, Q, nc, plain};
  const unsigned char* vb = (const unsigned char*)v;
  e = launch_chunk_state(bf, true, true, s, v, C, a.dt, a.A, vb + HP * 4, C, states, lam_end,
                         a.status, st);
  if (e != hipSuccess) return e;
  e = launch_state_pass(s, states, lam_end, a.s_in, nullptr, a.status, st);
  if (e != hipSuccess) return e;
  e = launch_chunk_out(bf, true, true, s, v, C, a.dt, a.A, a.D, vb + HP * 4,
                       vb + (HP + (int64_t)G * N) * 4, C, states, y, true, a.status, st);
  if (e != hipSuccess) return e;
  // zero the summed gradients
  auto zero = [&](float* p, int64_t n) {
    if (p && n > 0)
      hipLaunchKernelGGL(k_zero, dim3((unsigned)std::min<int64_t>((n + kThreads - 1) / kThreads, 4096)),
                         dim3(kThreads), 0, st, p, n);
  };
  zero(a.d_A, H);
  zero(a.d_D, H);
  zero(a.d_conv_w, C * W);
  zero(a.d_conv_b, C);
  zero(a.d_norm_w, HP);
  SSD_CHECK();
  const dim3 gr((unsigned)((T + kNormRows - 1) / kNormRows));
  {
  ProfScope ps(st, KID_BWD_NORM);
  if (bf)
    hipLaunchKernelGGL(k_norm_bwd<bf16>, gr, dim3(kThreads), 0, st, y, (const bf16*)a.z,
                       (const bf16*)a.norm_w, (const bf16*)a.d_out, a.eps, (bf16*)a.d_z,
                       a.d_norm_w, T, (int)HP, G);
  else
    hipLaunchKernelGGL(k_norm_bwd<float>, gr, dim3(kThreads), 0, st, y, (const float*)a.z,
                       (const float*)a.norm_w, (const float*)a.d_out, a.eps, (float*)a.d_z,
                       a.d_norm_w, T, (int)HP, G);
  }
  SSD_CHECK();
  const dim3 gc(nc, H, B);
  {
  ProfScope ps(st, KID_BWD_CHUNK_Z);
  if (bf)
    hipLaunchKernelGGL(k_chunk_z<bf16>, gc, dim3(kThreads), 0, st, v, y, (const bf16*)a.dt, plain,
                       a.A, dso, L, H, G, P, N, Q, nc);
  else
    hipLaunchKernelGGL(k_chunk_z<float>, gc, dim3(kThreads), 0, st, v, y, (const float*)a.dt,
                       plain, a.A, dso, L, H, G, P, N, Q, nc);
  }
  SSD_CHECK();
  {
  ProfScope ps(st, KID_BWD_REV_PASS);
  hipLaunchKernelGGL(k_rev_pass, dim3((P * N + kThreads - 1) / kThreads, H, B), dim3(kThreads), 0,
                     st, dso, lam_end, a.d_s_out, a.d_s_in, H, P * N, nc);
  }
  SSD_CHECK();
  const size_t lds = 3 * (size_t)Q * (Q + 1) * 4;
  {
  ProfScope ps(st, KID_BWD_CHUNK);
  if (bf)
    hipLaunchKernelGGL(k_chunk_bwd<bf16>, gc, dim3(kThreads), lds, st, v, y, (const bf16*)a.dt,
                       plain, a.A, a.D, states, dso, dv, dBh, dCh, (bf16*)a.d_dt, a.d_A, a.d_D, L,
                       H, G, P, N, Q, nc);
  else
    hipLaunchKernelGGL(k_chunk_bwd<float>, gc, dim3(kThreads), lds, st, v, y, (const float*)a.dt,
                       plain, a.A, a.D, states, dso, dv, dBh, dCh, (float*)a.d_dt, a.d_A, a.d_D,
                       L, H, G, P, N, Q, nc);
  }
  SSD_CHECK();
  {
  ProfScope ps(st, KID_BWD_GROUP_SUM);
  hipLaunchKernelGGL(k_group_sum, dim3((unsigned)((T * G * N + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, dBh, dCh, dv, T, H, G, N, (int)HP);
  }
  SSD_CHECK();
  const dim3 gd((unsigned)((C + kThreads - 1) / kThreads), (L + kConvTok - 1) / kConvTok, B);
  {
  ProfScope ps(st, KID_BWD_CONV_DU);
  if (bf)
    hipLaunchKernelGGL(k_conv_du<bf16>, gd, dim3(kThreads), 0, st, (const bf16*)a.xbc,
                       (const bf16*)a.conv_in, (const bf16*)a.conv_w, (const bf16*)a.conv_b, dv,
                       a.d_conv_w, a.d_conv_b, L, (int)C, W);
  else
    hipLaunchKernelGGL(k_conv_du<float>, gd, dim3(kThreads), 0, st, (const float*)a.xbc,
                       (const float*)a.conv_in, (const float*)a.conv_w, (const float*)a.conv_b,
                       dv, a.d_conv_w, a.d_conv_b, L, (int)C, W);
  }
  SSD_CHECK();
  const dim3 gx((unsigned)((C + kThreads - 1) / kThreads), (L + W - 1 + kConvTok - 1) / kConvTok, B);
  {
  ProfScope ps(st, KID_BWD_CONV_DX);
  if (bf)
    hipLaunchKernelGGL(k_conv_dx<bf16>, gx, dim3(kThreads), 0, st, dv, (const bf16*)a.conv_w,
                       (bf16*)a.d_xbc, a.d_conv_in, L, (int)C, W);
  else
    hipLaunchKernelGGL(k_conv_dx<float>, gx, dim3(kThreads), 0, st, dv, (const float*)a.conv_w,
                       (float*)a.d_xbc, a.d_conv_in, L, (int)C, W);
  }
  SSD_CHECK();
#undef SSD_CHECK
  return hipSuccess;
}

}  // namespace ssd
