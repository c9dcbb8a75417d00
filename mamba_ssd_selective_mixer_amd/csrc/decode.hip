// Single-token decode step ("feat(model): Nemotron-H hybrid ... on the CPU",
// section "Validation": token-by-token decode, every Mamba layer resuming
// from its slot). One workgroup per (sequence, group): it
//   1. shifts the conv state of the group's channels (x of its H/G heads,
//      its B and C) by one row and applies conv + SiLU to the new token;
//   2. for each head of the group streams the fp32 [P, N] SSM state once:
//      S = exp(dt*A) * S + dt * x (outer) B,  y[p] = S[p, :] . C + D * x[p];
//   3. applies the gated RMSNorm over the group's H/G*P channels (norm groups
//      and B/C groups coincide) and writes y.
// The state stream dominates: each lane owns 4 consecutive n of a row, so a
// wave reads and writes 1 KiB contiguous per instruction; the row sums over
// n are butterfly reductions inside aligned groups of N/4 lanes.
// VAR: the one-token sequences of a ragged batch (continuous batching):
// workgroup (g, j) takes the j-th listed sequence, its token row from the
// offsets and its states from its pool slot (zeros when it starts fresh).
#include "common.hpp"
#include "launch.hpp"

namespace ssd {

constexpr int kDecThreads = 256;
constexpr int kDecUnroll = 8;  // state float4 loads kept in flight per lane


template <class T, int N, int W, bool VAR>
__global__ __launch_bounds__(kDecThreads) void k_decode(
    const T* __restrict__ xbc, const T* __restrict__ z, const T* __restrict__ dt,
    const float* __restrict__ A, const float* __restrict__ D, const T* __restrict__ cw,
    const T* __restrict__ cb, const T* __restrict__ nw, float eps, T* __restrict__ conv_state,
    float* __restrict__ ssm, T* __restrict__ y, int64_t xrs, int64_t zrs, DtA dta, int H, int P,
    int G, float inv_S, Seqs q, const int32_t* __restrict__ dec) {
  extern __shared__ __align__(16) float sm[];
  const int g = blockIdx.x;
  const int hpg = H / G, S = hpg * P;
  const int HP = H * P, GN = G * N, C = HP + 2 * GN;
  // this workgroup's token row and states
  int64_t row = blockIdx.y;
  T* cst = conv_state + row * (W - 1) * C;
  float* ssm_b = ssm + row * H * (int64_t)(P * N);
  bool fresh = false;
  if constexpr (VAR) {
    if (__builtin_amdgcn_readfirstlane(*q.valid) != 1) return;
    const int j = blockIdx.y;
    if (j >= dec[gridDim.y]) return;
    const int i = dec[j], slot = q.slots[i];
    row = q.cu[i];
    cst = (T*)q.conv_pool + (int64_t)slot * (W - 1) * C;
    ssm_b = q.ssm_pool + (int64_t)slot * H * (int64_t)(P * N);
    fresh = q.has_state && !q.has_state[i];
  }
  float* xs = sm;          // [S] post-conv x of the group's heads
  float* Bs = xs + S;      // [N]
  float* Cs = Bs + N;      // [N]
  float* ys = Cs + N;      // [S]
  __shared__ float red[4];
  const int tid = threadIdx.x;

  // 1. conv state shift + conv + SiLU on the group's S + 2N channels.
  const int nv = (S + 2 * N) / 8;
  for (int v = tid; v < nv; v += kDecThreads) {
    const int o = v * 8;
    int c0;
    float* dst;
    if (o < S) { c0 = g * S + o; dst = xs + o; }
    else if (o < S + N) { c0 = HP + g * N + (o - S); dst = Bs + (o - S); }
    else { c0 = HP + GN + g * N + (o - S - N); dst = Cs + (o - S - N); }
    float win[W][8];
    T* cs = cst + c0;
#pragma unroll
    for (int r = 0; r < W - 1; ++r) {
      if (fresh) {
#pragma unroll
        for (int j = 0; j < 8; ++j) win[r][j] = 0.f;
      } else {
        load8(cs + (int64_t)r * C, win[r]);
      }
    }
    load8(xbc + row * xrs + c0, win[W - 1]);
#pragma unroll
    for (int r = 0; r < W - 1; ++r) store8(cs + (int64_t)r * C, win[r + 1]);
    float wv[W][8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int k = 0; k < W; ++k) wv[k][j] = to_f(cw[(int64_t)(c0 + j) * W + k]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float u = cb ? to_f(cb[c0 + j]) : 0.f;
#pragma unroll
      for (int k = 0; k < W; ++k) u += wv[k][j] * win[k][j];
      dst[j] = silu(u);
    }
  }
  __syncthreads();

  // 2. state update and output, head by head. The state of the next head is
  // loaded before the current head is updated; state loads and stores are
  // non-temporal (each element is touched once per step).
  constexpr int LPR = N / 4;                 // lanes per state row
  const int PN = P * N;
  const int n0 = (4 * tid) % N;
  const float4 Bv = *reinterpret_cast<const float4*>(Bs + n0);
  const float4 Cv = *reinterpret_cast<const float4*>(Cs + n0);
  const int iters = (PN + 4 * kDecThreads - 1) / (4 * kDecThreads);
  float* sb = ssm_b + (int64_t)g * hpg * PN;  // the group's heads
  if (iters <= kDecUnroll) {
    f32x4 cur[kDecUnroll];
    auto load_head = [&](int hl, f32x4 (&dst)[kDecUnroll]) {
      const float* st = sb + (int64_t)hl * PN;
#pragma unroll
      for (int u = 0; u < kDecUnroll; ++u) {
        const int e = 4 * tid + u * 4 * kDecThreads;
        if (u < iters && e < PN) {
          dst[u] = fresh ? zero4()
                         : __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(st + e));
        }
      }
    };
    load_head(0, cur);
    for (int hl = 0; hl < hpg; ++hl) {
      f32x4 nxt[kDecUnroll];
      if (hl + 1 < hpg) load_head(hl + 1, nxt);
      const int h = g * hpg + hl;
      const float dtv = dt_of(to_f(dt[row * dta.dts + h]), dta, h);
      const float al = fexp(dtv * a_of(A, dta, h));
      const float Dh = D ? D[h] : 0.f;
      float* st = sb + (int64_t)hl * PN;
#pragma unroll
      for (int u = 0; u < kDecUnroll; ++u) {
        const int e = 4 * tid + u * 4 * kDecThreads;
        if (u < iters && e < PN) {
          const int p = e / N;
          const float xp = xs[hl * P + p];
          const float dx = dtv * xp;
          f32x4 v = cur[u];
          v[0] = al * v[0] + dx * Bv.x;
          v[1] = al * v[1] + dx * Bv.y;
          v[2] = al * v[2] + dx * Bv.z;
          v[3] = al * v[3] + dx * Bv.w;
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(st + e));
          float part = v[0] * Cv.x + v[1] * Cv.y + v[2] * Cv.z + v[3] * Cv.w;
          part = group_sum_last<LPR>(part);
          if ((tid % LPR) == LPR - 1) ys[hl * P + p] = part + Dh * xp;
        }
      }
#pragma unroll
      for (int u = 0; u < kDecUnroll; ++u) cur[u] = nxt[u];
    }
  } else {
    for (int hl = 0; hl < hpg; ++hl) {
      const int h = g * hpg + hl;
      const float dtv = dt_of(to_f(dt[row * dta.dts + h]), dta, h);
      const float al = fexp(dtv * a_of(A, dta, h));
      const float Dh = D ? D[h] : 0.f;
      float* st = ssm_b + (int64_t)h * PN;
      for (int i0 = 0; i0 < iters; i0 += kDecUnroll) {
        f32x4 s[kDecUnroll];
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
          const int e = 4 * tid + (i0 + u) * 4 * kDecThreads;
          if (i0 + u < iters && e < PN)
            s[u] = fresh ? zero4()
                         : __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(st + e));
        }
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
          const int e = 4 * tid + (i0 + u) * 4 * kDecThreads;
          if (i0 + u < iters && e < PN) {
            const int p = e / N;
            const float xp = xs[hl * P + p];
            const float dx = dtv * xp;
            f32x4 v = s[u];
            v[0] = al * v[0] + dx * Bv.x;
            v[1] = al * v[1] + dx * Bv.y;
            v[2] = al * v[2] + dx * Bv.z;
            v[3] = al * v[3] + dx * Bv.w;
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(st + e));
            float part = v[0] * Cv.x + v[1] * Cv.y + v[2] * Cv.z + v[3] * Cv.w;
            part = group_sum_last<LPR>(part);
            if ((tid % LPR) == LPR - 1) ys[hl * P + p] = part + Dh * xp;
          }
        }
      }
    }
  }
  __syncthreads();

  // 3. gated RMSNorm over the group's S channels (or the plain output).
  T* yo = y + row * HP + (int64_t)g * S;
  if (z) {
    const T* zz = z + row * zrs + (int64_t)g * S;
    float ss = 0.f;
    for (int i = tid; i < S; i += kDecThreads) {
      const float q = ys[i] * silu(to_f(zz[i]));
      ss += q * q;
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const float tot = red[0] + red[1] + red[2] + red[3];
    const float inv = __builtin_amdgcn_rsqf(tot * inv_S + eps);
    for (int i = tid; i < S; i += kDecThreads) {
      const float q = ys[i] * silu(to_f(zz[i]));
      yo[i] = from_f<T>(q * to_f(nw[(int64_t)g * S + i]) * inv);
    }
  } else {
    for (int i = tid; i < S; i += kDecThreads) yo[i] = from_f<T>(ys[i]);
  }
}

template <class T, bool VAR>
static hipError_t decode_dispatch(int B, int H, int P, int G, int N, int W, const void* xbc,
                                  int64_t xrs, const void* z, int64_t zrs, const void* dt,
                                  const DtA& dta, const float* A, const float* D, const void* cw,
                                  const void* cb, const void* nw, float eps, void* conv_state,
                                  float* ssm, void* y, const Seqs& q, const int32_t* dec,
                                  hipStream_t st) {
  const int S = H / G * P;
  const size_t lds = (size_t)(2 * S + 2 * N) * sizeof(float);
  dim3 grid(G, B), block(kDecThreads);
  const float inv_S = 1.0f / (float)S;
#define SSD_DEC(NN, WW)                                                                          \
  hipLaunchKernelGGL((k_decode<T, NN, WW, VAR>), grid, block, lds, st, (const T*)xbc,          \
                     (const T*)z, (const T*)dt, A, D, (const T*)cw, (const T*)cb, (const T*)nw,  \
                     eps, (T*)conv_state, ssm, (T*)y, xrs, zrs, dta, H, P, G, inv_S, q, dec)
#define SSD_DEC_W(NN)                     \
  switch (W) {                            \
    case 2: SSD_DEC(NN, 2); break;        \
    case 3: SSD_DEC(NN, 3); break;        \
    default: SSD_DEC(NN, 4); break;       \
  }
  switch (N) {
    case 16: SSD_DEC_W(16); break;
    case 32: SSD_DEC_W(32); break;
    case 64: SSD_DEC_W(64); break;
    case 128: SSD_DEC_W(128); break;
    default: SSD_DEC_W(256); break;
  }
#undef SSD_DEC_W
#undef SSD_DEC
  return hipGetLastError();
}

hipError_t launch_decode(bool io_bf16, int B, int H, int P, int G, int N, int W,
                         const void* xbc, int64_t xrs, const void* z, int64_t zrs,
                         const void* dt, const DtA& dta, const float* A, const float* D,
                         const void* cw, const void* cb, const void* nw, float eps,
                         void* conv_state, float* ssm_state, void* y, hipStream_t st) {
  ProfScope ps(st, KID_DECODE);
  const Seqs none{};
  return io_bf16 ? decode_dispatch<bf16, false>(B, H, P, G, N, W, xbc, xrs, z, zrs, dt, dta, A,
                                                D, cw, cb, nw, eps, conv_state, ssm_state, y,
                                                none, nullptr, st)
                 : decode_dispatch<float, false>(B, H, P, G, N, W, xbc, xrs, z, zrs, dt, dta, A,
                                                 D, cw, cb, nw, eps, conv_state, ssm_state, y,
                                                 none, nullptr, st);
}

hipError_t launch_decode_varlen(bool io_bf16, int nseq, int H, int P, int G, int N, int W,
                                const void* xbc, int64_t xrs, const void* z, int64_t zrs,
                                const void* dt, const DtA& dta, const float* A, const float* D,
                                const void* cw, const void* cb, const void* nw, float eps,
                                const Seqs& q, const int32_t* dec, void* y, hipStream_t st) {
  ProfScope ps(st, KID_DECODE);
  // a workgroup per (group, listed sequence); those past the list's count
  // return at once
  return io_bf16 ? decode_dispatch<bf16, true>(nseq, H, P, G, N, W, xbc, xrs, z, zrs, dt, dta,
                                               A, D, cw, cb, nw, eps, nullptr, nullptr, y, q,
                                               dec, st)
                 : decode_dispatch<float, true>(nseq, H, P, G, N, W, xbc, xrs, z, zrs, dt, dta,
                                                A, D, cw, cb, nw, eps, nullptr, nullptr, y, q,
                                                dec, st);
}

}  // namespace ssd
