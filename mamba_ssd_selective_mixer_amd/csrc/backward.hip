// Backward pass of the mixer prefill (conv + SiLU, chunked SSD scan, gated
// RMSNorm): given d_out (and optionally the gradient of the final SSM
// state), the gradients with respect to xBC, z, dt, A, D, the conv weight
// and bias, the norm weight and the initial states ("feat(model): add
// Nemotron-3 Nano hybrid ..." section "Testing": gradient flow through the
// mixer; "Caveats": the native backend is activation-memory hungry, so
// nothing of the forward is kept: it is recomputed here).
//
// Per chunk of Q = 64 tokens of head h, with Lam the inclusive cumsum of
// dt A inside the chunk, E[t,s] = exp(Lam_t - Lam_s) (s <= t), G = C B^T,
// K = dY X^T, M = G o E dt_s, dG = K o E dt_s, w_s = exp(Lam_end - Lam_s) dt_s:
//   y       = M X + exp(Lam_t) C S_in^T + D X                (recomputed)
//   dX[s]   = sum_{t>=s} M[t,s] dY[t] + D dY[s] + w_s (B_s dS_out^T)
//   dC[t]   = sum_{s<=t} dG[t,s] B[s] + exp(Lam_t) dY[t] S_in
//   dB[s]   = sum_{t>=s} dG[t,s] C[t] + w_s X[s] dS_out
//   dS_in   = exp(Lam_end) dS_out + sum_t exp(Lam_t) dY[t] (outer) C[t]
// with dS_out of chunk k the dS_in of chunk k+1 (a reverse pass over the
// chunks), and dt, A through dLam. The dense products run on fp32 MFMA
// (16x16x4, fp32 accumulation) with operand slices staged in LDS; the gated
// norm and the conv are differentiated elementwise.
#include "common.hpp"
#include "f32tiles.hpp"
#include "launch.hpp"

namespace ssd {
namespace bwd {

using namespace f32t;
constexpr int kNormBlocks = 1024; // most norm-backward workgroups (one dw part each)
constexpr int kMaxGroups = 256;
constexpr int kMaxNormPieces = 64;  // 256-channel pieces of a row (H*P <= 16384)

// ---------------------------------------------------------------- gated norm
SSD_DEV float sum4(float4 v) { return (v.x + v.y) + (v.z + v.w); }

// q = y silu(z), r = (mean_group(q^2) + eps)^-1/2, out = q r w. For each row:
//   dq = w r g - q r^3 mean_group(w g q);  dy = dq silu(z);
//   dz = dq y silu'(z);  dw += g q r  (summed over rows).
// dy overwrites y (each thread reads its channels before writing them). Each
// thread takes 4 consecutive channels (one norm group: groups are multiples
// of 16 channels). A workgroup takes `rows` consecutive rows and sums its
// share of dw in LDS, then writes it to its row of dw_part [gridDim.x][HP].
// Each 4-channel lane keeps its row sums in LDS; the group sums then add
// them in a fixed order (no atomics: the result does not depend on timing).
// Norm groups of whole 256-channel pieces take k_norm_bwd_wide instead.
template <class T>
__global__ __launch_bounds__(kThreads) void k_norm_bwd(float* y, const T* __restrict__ z,
                                                       const T* __restrict__ w,
                                                       const T* __restrict__ g, float eps,
                                                       T* __restrict__ dz, float* dw_part,
                                                       int64_t nrows, int rows, int HP, int G) {
  extern __shared__ float4 dwl[];  // [HP / 4], then two [HP / 4] lane sums
  __shared__ float sq[kMaxGroups], sg[kMaxGroups];
  const int tid = threadIdx.x;
  const int S = HP / G, HP4 = HP / 4;
  float* p2 = reinterpret_cast<float*>(dwl + HP4);
  float* pw = p2 + HP4;
  const int per = S / 4;
  for (int c = tid; c < HP4; c += kThreads) dwl[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int rr = 0; rr < rows; ++rr) {
    const int64_t row = (int64_t)blockIdx.x * rows + rr;
    if (row >= nrows) break;
#pragma unroll 4
    for (int c0 = 0; c0 < HP4; c0 += kThreads) {
      const int c4 = c0 + tid, c = 4 * c4;
      float q2 = 0.f, wgq = 0.f;
      if (c4 < HP4) {
        const int64_t o = row * HP + c;
        const float4 zz = ld4(z + o), yy = ld4(y + o), ww = ld4(w + c), gg = ld4(g + o);
        const float4 q = make_float4(yy.x * zz.x * frcp(1.f + __expf(-zz.x)),
                                     yy.y * zz.y * frcp(1.f + __expf(-zz.y)),
                                     yy.z * zz.z * frcp(1.f + __expf(-zz.z)),
                                     yy.w * zz.w * frcp(1.f + __expf(-zz.w)));
        q2 = sum4(make_float4(q.x * q.x, q.y * q.y, q.z * q.z, q.w * q.w));
        wgq = sum4(make_float4(ww.x * gg.x * q.x, ww.y * gg.y * q.y, ww.z * gg.z * q.z,
                               ww.w * gg.w * q.w));
      }
      if (c4 < HP4) {
        p2[c4] = q2;
        pw[c4] = wgq;
      }
    }
    __syncthreads();
    for (int j = tid; j < G; j += kThreads) {
      float a = 0.f, b = 0.f;
      for (int k = 0; k < per; ++k) {
        a += p2[j * per + k];
        b += pw[j * per + k];
      }
      sq[j] = a;
      sg[j] = b;
    }
    __syncthreads();
#pragma unroll 4
    for (int c4 = tid; c4 < HP4; c4 += kThreads) {
      const int c = 4 * c4;
      const int64_t o = row * HP + c;
      const int j = c / S;
      const float r = rsqrtf(sq[j] / S + eps), k3 = r * r * r * sg[j] / S;
      const float4 zz = ld4(z + o), yy = ld4(y + o), ww = ld4(w + c), gg = ld4(g + o);
      float zv[4] = {zz.x, zz.y, zz.z, zz.w}, yv[4] = {yy.x, yy.y, yy.z, yy.w};
      float wv4[4] = {ww.x, ww.y, ww.z, ww.w}, gv[4] = {gg.x, gg.y, gg.z, gg.w};
      float dy[4], dzv[4], dwv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sig = frcp(1.f + __expf(-zv[i])), sl = zv[i] * sig;
        const float q = yv[i] * sl;
        const float dq = wv4[i] * r * gv[i] - q * k3;
        dy[i] = dq * sl;
        dzv[i] = dq * yv[i] * (sig + sl * (1.f - sig));
        dwv[i] = gv[i] * q * r;
      }
      st4(y + o, make_float4(dy[0], dy[1], dy[2], dy[3]));
      st4(dz + o, make_float4(dzv[0], dzv[1], dzv[2], dzv[3]));
      float4 acc = dwl[c4];
      acc.x += dwv[0];
      acc.y += dwv[1];
      acc.z += dwv[2];
      acc.w += dwv[3];
      dwl[c4] = acc;
    }
    __syncthreads();
  }
  for (int c4 = tid; c4 < HP4; c4 += kThreads)
    st4(dw_part + (int64_t)blockIdx.x * HP + 4 * c4, dwl[c4]);
}

// The same for bf16 I/O and norm groups of whole 256-channel pieces, with
// each row read once: a 1024-thread workgroup holds a row's channels in
// registers (up to four 4-channel units per thread, z and g as raw bf16;
// unit c4 = tid + 1024 k, so piece k * 16 + wave is one wave's 64 lanes),
// loads the next row meanwhile, and sums its share of dw in LDS (each
// thread its own units). A piece's sums come from its wave (deterministic
// DPP sums) and the group sums add the pieces in a fixed order.
constexpr int kNormWideThreads = 1024;
constexpr int kNormWideBlocks = 256;
SSD_DEV float4 bf4(uint2 u) {
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
__global__ __launch_bounds__(kNormWideThreads) void k_norm_bwd_wide(
    float* y, const bf16* __restrict__ z, const bf16* __restrict__ w, const bf16* __restrict__ g,
    float eps, bf16* __restrict__ dz, float* dw_part, int64_t nrows, int rows, int HP, int G) {
  constexpr int KU = kMaxNormPieces * 64 / kNormWideThreads;
  extern __shared__ float4 dwl[];  // [HP / 4]
  __shared__ float p2[kMaxNormPieces], pw[kMaxNormPieces], sq[kMaxGroups], sg[kMaxGroups];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = HP / G, HP4 = HP / 4, per = S / 256;
  bool on[KU];
  uint2 wr[KU];
#pragma unroll
  for (int k = 0; k < KU; ++k) {
    const int c4 = tid + kNormWideThreads * k;
    on[k] = c4 < HP4;
    wr[k] = on[k] ? *reinterpret_cast<const uint2*>(w + 4 * c4) : make_uint2(0u, 0u);
    if (on[k]) dwl[c4] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int64_t r0 = (int64_t)blockIdx.x * rows;
  const int nr = (int)min((int64_t)rows, nrows - r0);
  float4 yn[KU];
  uint2 zn[KU], gn[KU];
#pragma unroll
  for (int k = 0; k < KU; ++k) {
    yn[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    zn[k] = gn[k] = make_uint2(0u, 0u);
  }
  auto fetch = [&](int64_t row) {
#pragma unroll
    for (int k = 0; k < KU; ++k)
      if (on[k]) {
        const int64_t o = row * HP + 4 * (tid + kNormWideThreads * k);
        yn[k] = ld4(y + o);
        zn[k] = *reinterpret_cast<const uint2*>(z + o);
        gn[k] = *reinterpret_cast<const uint2*>(g + o);
      }
  };
  if (nr > 0) fetch(r0);
  for (int rr = 0; rr < nr; ++rr) {
    const int64_t row = r0 + rr;
    float4 yy[KU];
    uint2 zr[KU], gr[KU];
#pragma unroll
    for (int k = 0; k < KU; ++k) {
      yy[k] = yn[k];
      zr[k] = zn[k];
      gr[k] = gn[k];
    }
    if (rr + 1 < nr) fetch(row + 1);
#pragma unroll
    for (int k = 0; k < KU; ++k) {
      const float4 zz = bf4(zr[k]), gg = bf4(gr[k]), wv = bf4(wr[k]);
      const float4 qk = make_float4(yy[k].x * zz.x * frcp(1.f + __expf(-zz.x)),
                                    yy[k].y * zz.y * frcp(1.f + __expf(-zz.y)),
                                    yy[k].z * zz.z * frcp(1.f + __expf(-zz.z)),
                                    yy[k].w * zz.w * frcp(1.f + __expf(-zz.w)));
      // on[k] is uniform over a wave (HP / 4 is a multiple of 64 here)
      const float q2 = wave_sum(sum4(make_float4(qk.x * qk.x, qk.y * qk.y, qk.z * qk.z,
                                                 qk.w * qk.w)));
      const float wgq = wave_sum(sum4(make_float4(wv.x * gg.x * qk.x, wv.y * gg.y * qk.y,
                                                  wv.z * gg.z * qk.z, wv.w * gg.w * qk.w)));
      if (lane == 0 && on[k]) {
        p2[k * (kNormWideThreads / 64) + wave] = q2;
        pw[k * (kNormWideThreads / 64) + wave] = wgq;
      }
    }
    __syncthreads();
    if (tid < G) {
      float a = 0.f, b = 0.f;
      for (int k = 0; k < per; ++k) {
        a += p2[tid * per + k];
        b += pw[tid * per + k];
      }
      sq[tid] = a;
      sg[tid] = b;
    }
    __syncthreads();
    // the row's values are taken up again from their raw registers (the
    // empty asm hides them from the compiler, which would otherwise keep
    // every value derived in the first pass alive across the barriers)
#pragma unroll
    for (int k = 0; k < KU; ++k)
      asm volatile(""
                   : "+v"(yy[k].x), "+v"(yy[k].y), "+v"(yy[k].z), "+v"(yy[k].w), "+v"(zr[k].x),
                     "+v"(zr[k].y), "+v"(gr[k].x), "+v"(gr[k].y), "+v"(wr[k].x), "+v"(wr[k].y));
#pragma unroll
    for (int k = 0; k < KU; ++k)
      if (on[k]) {
        const int c = 4 * (tid + kNormWideThreads * k);
        const int64_t o = row * HP + c;
        const int j = c / S;
        const float r = rsqrtf(sq[j] / S + eps), k3 = r * r * r * sg[j] / S;
        const float4 zz = bf4(zr[k]), gg = bf4(gr[k]), wv = bf4(wr[k]);
        const float zv[4] = {zz.x, zz.y, zz.z, zz.w};
        const float yv[4] = {yy[k].x, yy[k].y, yy[k].z, yy[k].w};
        const float wq[4] = {wv.x, wv.y, wv.z, wv.w};
        const float gv[4] = {gg.x, gg.y, gg.z, gg.w};
        float dy[4], dzv[4], dwv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sig = frcp(1.f + __expf(-zv[i])), sl = zv[i] * sig;
          const float qq = yv[i] * sl;
          const float dq = wq[i] * r * gv[i] - qq * k3;
          dy[i] = dq * sl;
          dzv[i] = dq * yv[i] * (sig + sl * (1.f - sig));
          dwv[i] = gv[i] * qq * r;
        }
        st4(y + o, make_float4(dy[0], dy[1], dy[2], dy[3]));
        st4(dz + o, make_float4(dzv[0], dzv[1], dzv[2], dzv[3]));
        float4 acc = dwl[c / 4];
        acc.x += dwv[0];
        acc.y += dwv[1];
        acc.z += dwv[2];
        acc.w += dwv[3];
        dwl[c / 4] = acc;
      }
  }
#pragma unroll
  for (int k = 0; k < KU; ++k)
    if (on[k]) {
      const int c4 = tid + kNormWideThreads * k;
      st4(dw_part + (int64_t)blockIdx.x * HP + 4 * c4, dwl[c4]);
    }
}

// out[c] = sum over the parts of part[i * stride + c]. A workgroup takes 64
// columns; its four waves sum the parts i = w mod 4 with four loads in
// flight, then the four partial sums are added in a fixed order (the result
// does not depend on timing).
__global__ __launch_bounds__(kThreads) void k_sum_parts(const float* __restrict__ part,
                                                        int64_t stride, float* __restrict__ out,
                                                        int nparts, int n) {
  __shared__ float red[4][64];
  const int cl = threadIdx.x & 63, j = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + cl;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  if (c < n) {
    int i = j;
    for (; i + 12 < nparts; i += 16) {
      a0 += part[(int64_t)i * stride + c];
      a1 += part[(int64_t)(i + 4) * stride + c];
      a2 += part[(int64_t)(i + 8) * stride + c];
      a3 += part[(int64_t)(i + 12) * stride + c];
    }
    for (; i < nparts; i += 4) a0 += part[(int64_t)i * stride + c];
  }
  red[j][cl] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  if (j == 0 && c < n) out[c] = (red[0][cl] + red[1][cl]) + (red[2][cl] + red[3][cl]);
}

// ---------------------------------------------------------------- dS_in part
// Rows [0, 64) x columns [0, COLS) of a row-major fp32 matrix held in
// registers (rows >= nrows zero), then stored transposed and scaled per row
// (element (r, c) at c * pitch + r, times sc[r]), with stage_cols' mapping.
template <int COLS>
struct ColRegs {
  static constexpr int kItems = kQ * (COLS / 4), kN = (kItems + kThreads - 1) / kThreads;
  float4 v[kN];
  SSD_DEV void load(const float* src, int rs, int nrows) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int idx = threadIdx.x + i * kThreads, r = idx % kQ, c4 = (idx / kQ) * 4;
      v[i] = (idx < kItems && r < nrows) ? ld4(src + (int64_t)r * rs + c4)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  SSD_DEV void store_cols(float* dst, int pitch, const float* sc) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int idx = threadIdx.x + i * kThreads, r = idx % kQ, c4 = (idx / kQ) * 4;
      if (idx < kItems) {
        const float f = sc[r];
        dst[(c4 + 0) * pitch + r] = v[i].x * f;
        dst[(c4 + 1) * pitch + r] = v[i].y * f;
        dst[(c4 + 2) * pitch + r] = v[i].z * f;
        dst[(c4 + 3) * pitch + r] = v[i].w * f;
      }
    }
  }
};

// Z[p,n] = sum_t exp(Lam_t) dY[t,p] C[t,n] of one chunk for hpb heads of one
// group, one after the other, into zb. The chunk's C (shared by the heads)
// and each head's exp(Lam_t) dY are staged transposed in LDS ([n][t],
// [p][t]), so each lane reads four consecutive t of both operands in one
// 16-byte read (k-permuted MFMA steps, as in the chunk-output kernel); work
// items (16-row tile of p, up to 8 tiles of n) go round the waves. The next
// head's dY rows are loaded into registers while a head is computed.
template <class T, int P>
__global__ __launch_bounds__(kThreads) void k_chunk_z(const float* __restrict__ v,
                                                      const float* __restrict__ dY,
                                                      const T* __restrict__ dt, DtA dta,
                                                      const float* __restrict__ A, float* zb,
                                                      int L, int H, int G, int N, int nc,
                                                      int hpb) {
  extern __shared__ __align__(16) float sm[];
  __shared__ float lam[64], dts[64], ex[64];
  constexpr int NPT = P / 16;
  float* Yt = sm;             // [P][kQP]: exp(Lam_t) dY[t, p]
  float* Ct = sm + P * kQP;   // [N][kQP]: C[t, n]
  const int c = blockIdx.x, b = blockIdx.z, g = blockIdx.y * hpb / (H / G);
  const int t0 = c * kQ, len = min(kQ, L - t0);
  const int64_t row0 = (int64_t)b * L + t0;
  const int HP = H * P;
  const int64_t C = HP + 2 * (int64_t)G * N, co = HP + (int64_t)(G + g) * N;
  stage_cols(Ct, kQP, v + row0 * C + co, (int)C, kQ, len, N);
  ColRegs<P> yr;
  yr.load(dY + row0 * HP + (int64_t)blockIdx.y * hpb * P, HP, len);
#pragma unroll 1
  for (int hj = 0; hj < hpb; ++hj) {
    const int h = blockIdx.y * hpb + hj;
    // the thread index is hidden per head, so lane-dependent addresses are not
    // hoisted out of the head loop and held in registers across it
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lk = lane >> 4;
    chunk_lam<T>(dt, dta, row0, h, a_of(A, dta, h), len, lam, dts, ex);
    yr.store_cols(Yt, kQP, ex);
    __syncthreads();
    if (hj + 1 < hpb) yr.load(dY + row0 * HP + (int64_t)(h + 1) * P, HP, len);
    float* out = zb + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
    const int nnt = N / 16, nng = (nnt + 7) / 8;
    const int kend = (len + 15) & ~15;  // rows past len are zero
    for (int item = wave; item < NPT * nng; item += 4) {
      const int pt = item % NPT, nt0 = (item / NPT) * 8, ntn = min(8, nnt - nt0);
      f32x4 acc[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = zero4();
      for (int k0 = 0; k0 < kend; k0 += 16) {
        const int kq = k0 + 4 * lk;
        const float4 a4 = ld4(Yt + (pt * 16 + lr) * kQP + kq);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < ntn) {
            const float4 b4 = ld4(Ct + ((nt0 + j) * 16 + lr) * kQP + kq);
            acc[j] = mma(a4.x, b4.x, acc[j]);
            acc[j] = mma(a4.y, b4.y, acc[j]);
            acc[j] = mma(a4.z, b4.z, acc[j]);
            acc[j] = mma(a4.w, b4.w, acc[j]);
          }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < ntn)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            out[(int64_t)(pt * 16 + 4 * lk + r) * N + (nt0 + j) * 16 + lr] = acc[j][r];
    }
    __syncthreads();  // Yt, lam and ex are restaged for the next head
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
constexpr int kNS = 16;        // width (in n) of the per-chunk gradient kernel's state slices
constexpr int kChunkHeads = 32; // most heads of one group per per-chunk gradient workgroup
constexpr int kZHeads = 8;      // most heads of one group per state-gradient-term workgroup
constexpr int kBP = kNS + 4;   // pitch of such a slice stored as rows

// Rows [0, ROWS) x columns [0, kNS) of a row-major fp32 matrix held in
// registers between their global loads and their LDS stores (the next
// slice's loads in flight while one is computed on); rows >= nrows are
// zero. Stored as rows (element (r, c) at r pitch + c) or transposed (at
// c pitch + r).
template <int ROWS>
struct NSlice {
  static constexpr int kItems = ROWS * (kNS / 4), kN = (kItems + kThreads - 1) / kThreads;
  float4 v[kN];
  SSD_DEV void load(const float* src, int rs, int nrows) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int idx = threadIdx.x + i * kThreads, r = idx / (kNS / 4), c4 = (idx % (kNS / 4)) * 4;
      v[i] = (idx < kItems && r < nrows) ? ld4(src + (int64_t)r * rs + c4)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  SSD_DEV void store_rows(float* dst, int pitch) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int idx = threadIdx.x + i * kThreads, r = idx / (kNS / 4), c4 = (idx % (kNS / 4)) * 4;
      if (idx < kItems) st4(dst + r * pitch + c4, v[i]);
    }
  }
  SSD_DEV void store_cols(float* dst, int pitch) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int idx = threadIdx.x + i * kThreads, r = idx / (kNS / 4), c4 = (idx % (kNS / 4)) * 4;
      if (idx < kItems) {
        dst[(c4 + 0) * pitch + r] = v[i].x;
        dst[(c4 + 1) * pitch + r] = v[i].y;
        dst[(c4 + 2) * pitch + r] = v[i].z;
        dst[(c4 + 3) * pitch + r] = v[i].w;
      }
    }
  }
};

SSD_DEV f32x4 mma4(float4 a, float4 b, f32x4 c) {
  c = mma(a.x, b.x, c);
  c = mma(a.y, b.y, c);
  c = mma(a.z, b.z, c);
  return mma(a.w, b.w, c);
}

// One (chunk, head, batch): dX into dv's x channels, this head's share of dB
// and dC into its workgroup's rows of dBh / dCh [T, H / hpb, N] (written by
// the workgroup's first head, added to by the others), d(dt) into ddt (io
// dtype), and this chunk's parts of dA and dD into dA / dD [B nc, H] (or dD
// null).
// dt and A reach the output through Lam only (a_u = dt_u A feeds Lam_t for
// every t >= u), so d(a_u) is the sum over t >= u of dLam_t. That sum is
// formed term by term, without differences of partial sums:
//   intra-chunk:  sum_{t>=u} sum_{s<u} F[t,s] dt_s,  F = K o G o E
//   state out:    exp(Lam_end) <dS_out, S_in> + sum_{s<u} w_s U_s
//   inter-chunk:  sum_{t>=u} Y_t,  Y_t = exp(Lam_t) dY[t] . (C_t S_in^T)
// where U_s = X[s] . (B_s dS_out^T) and Y_t = C_t . (exp(Lam_t) dY[t] S_in),
// the latter from dC's inter-chunk part. Wave w owns the 16-row tile w of s
// (dX, dB) and of t (dC).
template <class T, int P>
__device__ __forceinline__ void chunk_bwd_head(
    const float* __restrict__ v, const float* __restrict__ dY, const T* __restrict__ dt, DtA dta,
    const float* __restrict__ A, const float* __restrict__ D, const float* __restrict__ Sin,
    const float* __restrict__ dSo, float* __restrict__ dv,
    float* __restrict__ dBh, float* __restrict__ dCh, T* __restrict__ ddt, float* dA, float* dD,
    int L, int H, int G, int N, int nc, int h, int hpb, SliceRegs<kQ>& ry, SliceRegs<kQ>& rx,
    bool fetched, const f32x4 (&gt)[3]) {
  extern __shared__ __align__(16) float sm[];
  float* Mt = sm;                // [Q][kQP]: G, then M = G o E dt_s
  float* Dg = sm + kQ * kQP;     // [Q][kQP]: K, then dG = K o E dt_s
  float* SA = sm + 2 * kQ * kQP; // staging
  __shared__ float lam[64], dts[64], ex[64], wv[64], colF[64], Yo[64], U[64], dai[64], tmp[64];
  __shared__ float red[4][2];  // per wave: its share of <dS_out, S_in> and of dD
  constexpr int NPT = P / 16;
  const int c = blockIdx.x, b = blockIdx.z, g = h / (H / G);
  // the thread index is hidden from the compiler per head, so the many
  // lane-dependent addresses are formed inside the head instead of being
  // hoisted out of the workgroup's head loop and held in registers across it
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lk = lane >> 4;
  const int t0 = c * kQ, len = min(kQ, L - t0);
  const int64_t row0 = (int64_t)b * L + t0;
  const int HP = H * P, Hs = H / hpb;
  const bool first = h % hpb == 0;  // the block's first head writes its dB / dC rows
  const int64_t C = HP + 2 * (int64_t)G * N, xo = (int64_t)h * P, bo = HP + (int64_t)g * N,
                co = HP + (int64_t)(G + g) * N;
  const float Ah = a_of(A, dta, h), Dh = D ? D[h] : 0.f;
  const int64_t sb = (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
  const float* Si = Sin + sb;
  const float* dS = dSo + sb;
  const int sw = wave * 16;
  for (int i = tid; i < 2 * kQ * kQP; i += kThreads) sm[i] = 0.f;
  chunk_lam<T>(dt, dta, row0, h, Ah, len, lam, dts, ex);
  const float lamE = lam[len - 1];
  if (tid < 64) wv[tid] = tid < len ? __expf(lamE - lam[tid]) * dts[tid] : 0.f;

  // (1) K = dY X^T on the causal tiles over slices of p; G (gt) from the
  // group's C B^T, computed once per chunk and group
  {
    int rt[3], st[3];
    bool on[3];
    f32x4 aK[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      on[i] = causal_tile(wave, i, rt[i], st[i]);
      aK[i] = zero4();
    }
    float* Ys = SA;
    float* Xs = SA + kQ * kSP;
    auto fetch = [&](int k0) {
      const int nvp = min(kKS, P - k0);
      ry.load(dY + row0 * HP + xo + k0, HP, len, nvp);
      rx.load(v + row0 * C + xo + k0, (int)C, len, nvp);
    };
    if (!fetched) fetch(0);  // else the previous head loaded the first slice
    for (int k0 = 0; k0 < P; k0 += kKS) {
      const int nvp = min(kKS, P - k0);
      ry.store(Ys);
      rx.store(Xs);
      __syncthreads();
      if (k0 + kKS < P) fetch(k0 + kKS);
      // k-permuted MFMA steps: a lane's four k values of both operands in
      // one 16-byte read (nvp is a multiple of 16)
      for (int kk = 0; kk < nvp; kk += 16)
#pragma unroll
        for (int i = 0; i < 3; ++i)
          if (on[i])
            aK[i] = mma4(ld4(Ys + (rt[i] * 16 + lr) * kSP + kk + 4 * lk),
                         ld4(Xs + (st[i] * 16 + lr) * kSP + kk + 4 * lk), aK[i]);
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (on[i])
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = rt[i] * 16 + 4 * lk + r, s = st[i] * 16 + lr;
          Mt[t * kQP + s] = gt[i][r];
          Dg[t * kQP + s] = aK[i][r];
        }
  }
  __syncthreads();

  // (2) F by columns, R[t,s] = sum_{t' >= t} F[t',s] (s <= t < len): wave q
  // sums its own 16 rows of t from the bottom up (lane s on column s) and
  // keeps its column totals; R is its in-rows sum plus the totals of the
  // later waves. K and G take their E dt_s factor in the same pass.
  {
    constexpr int FP = kQ + 1;
    float* Fm = SA;              // [Q][FP]: sums over the wave's own rows
    float* tot = SA + kQ * FP;   // [4][Q]: column totals of each wave's rows
    {
      const int s = lane;
      const float ls = lam[s], ds = dts[s];
      float acc = 0.f;
#pragma unroll
      for (int i = 15; i >= 0; --i) {
        const int t = sw + i;
        const float e = (s <= t && t < len) ? __expf(lam[t] - ls) : 0.f;
        const float kv = Dg[t * kQP + s], gv = Mt[t * kQP + s];
        acc += kv * gv * e;
        Fm[t * FP + s] = acc;
        const float f = e * ds;
        Dg[t * kQP + s] = kv * f;
        Mt[t * kQP + s] = gv * f;
      }
      tot[wave * kQ + s] = acc;
    }
    __syncthreads();
    // dai[u] = sum_{s<u} dt_s R[u,s] (four lanes per u; row u lies in this
    // wave's rows) and colF[s] = R[s,s]
    {
      const int u = tid >> 2, j = tid & 3;
      float acc = 0.f;
      if (u < len)
        for (int s = j; s < u; s += 4) {
          float r = Fm[u * FP + s];
          for (int q = wave + 1; q < 4; ++q) r += tot[q * kQ + s];
          acc += dts[s] * r;
        }
      acc = group_sum_last<4>(acc);
      if (j == 0) dai[u] = acc;
    }
    if (wave == 0) {
      const int s = lane;
      float r = Fm[s * FP + s];
      for (int q = (s >> 4) + 1; q < 4; ++q) r += tot[q * kQ + s];
      colF[s] = r;
    }
    __syncthreads();
  }

  // (3) dX intra: sum_{t >= s} M[t,s] dY[t,p], the chunk's dY rows staged.
  // dX's two products are formed transposed (rows p, columns s), so lane l
  // holds p = 16 pt + 4 (l / 16) + (0..3) of token s = sw + l % 16: the same
  // elements as its dY and X fragments below.
  f32x4 a1[NPT], a2[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) a1[i] = a2[i] = zero4();
  {
    constexpr int YP = P + 16;
    float* Ys = SA;  // [Q][YP]
    stage_rows(Ys, YP, dY + row0 * HP + xo, HP, kQ, len, P);
    __syncthreads();
    for (int k0 = sw; k0 < kQ; k0 += 4) {
      const int t = k0 + lk;
      const float m = Mt[t * kQP + sw + lr];
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) a1[pt] = mma(Ys[t * YP + pt * 16 + lr], m, a1[pt]);
    }
    __syncthreads();
  }

  // (4) over 16-wide slices of n: B_s dS_out^T of the wave's tokens (a2), and
  // the slice's tiles of dC (rows t) and dB (rows s). Every product takes
  // k-permuted steps (a lane's four k values of both operands in one 16-byte
  // read): B and dS_out are staged both as rows (n contiguous, for a2) and
  // transposed (k contiguous), C and S_in transposed, and dG is copied
  // transposed into the space M held; dY and X of the wave's rows sit in
  // registers, p = 16 j + 4 (l / 16) + (0..3) for lane l.
  float4 ya[NPT], xa[NPT];
  {
    const int r = sw + lr;
    const bool ok = r < len;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      ya[j] = ok ? ld4(dY + (row0 + r) * HP + xo + 16 * j + 4 * lk) : make_float4(0.f, 0.f, 0.f, 0.f);
      xa[j] = ok ? ld4(v + (row0 + r) * C + xo + 16 * j + 4 * lk) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  float* DgT = Mt;  // [Q][kQP]: dG[t, s] at s kQP + t
  for (int i = tid; i < kQ * kQ / 4; i += kThreads) {
    const int t = i >> 4, s4 = (i & 15) * 4;
    const float4 d = ld4(Dg + t * kQP + s4);
    DgT[(s4 + 0) * kQP + t] = d.x;
    DgT[(s4 + 1) * kQP + t] = d.y;
    DgT[(s4 + 2) * kQP + t] = d.z;
    DgT[(s4 + 3) * kQP + t] = d.w;
  }
  float cstp = 0.f;
  float yp[4] = {0.f, 0.f, 0.f, 0.f};  // this lane's share of Y_t, t = sw + 4 lk + r
  {
    constexpr int TP = P + 4;
    float* Bs = SA;               // [Q][kBP]: B[s, n]
    float* Ds = Bs + kQ * kBP;    // [P][kBP]: dS_out[p, n]
    float* Bt = Ds + P * kBP;     // [kNS][kQP]: B[s, n] at n kQP + s
    float* Ct = Bt + kNS * kQP;   // [kNS][kQP]: C[t, n] at n kQP + t
    float* St = Ct + kNS * kQP;   // [kNS][TP]: S_in[p, n] at n TP + p
    float* Dt = St + kNS * TP;    // [kNS][TP]: dS_out[p, n] at n TP + p
    NSlice<kQ> rb, rc;
    NSlice<P> rs, rd;
    auto fetch = [&](int n0) {
      rb.load(v + row0 * C + bo + n0, (int)C, len);
      rc.load(v + row0 * C + co + n0, (int)C, len);
      rs.load(Si + n0, N, P);
      rd.load(dS + n0, N, P);
    };
    fetch(0);
    for (int n0 = 0; n0 < N; n0 += kNS) {  // N is a multiple of 16
      rb.store_rows(Bs, kBP);
      rb.store_cols(Bt, kQP);
      rc.store_cols(Ct, kQP);
      rs.store_cols(St, TP);
      rd.store_rows(Ds, kBP);
      rd.store_cols(Dt, TP);
      __syncthreads();
      if (n0 + kNS < N) fetch(n0 + kNS);
      // the workgroup's earlier heads' sums of this slice's dC / dB rows
      // (written by this lane), loaded while the slice is computed
      float pc[4] = {0.f, 0.f, 0.f, 0.f}, pb[4] = {0.f, 0.f, 0.f, 0.f};
      if (!first)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = sw + 4 * lk + r;
          if (t < len) {
            const int64_t o = ((row0 + t) * Hs + h / hpb) * N + n0 + lr;
            pc[r] = dCh[o];
            pb[r] = dBh[o];
          }
        }
      for (int i = tid; i < kNS * (P / 4); i += kThreads) {
        const int n = i / (P / 4), p4 = (i % (P / 4)) * 4;
        const float4 a = ld4(St + n * TP + p4), d = ld4(Dt + n * TP + p4);
        cstp += (a.x * d.x + a.y * d.y) + (a.z * d.z + a.w * d.w);
      }
      {
        const float4 a4 = ld4(Bs + (sw + lr) * kBP + 4 * lk);
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt)
          a2[pt] = mma4(ld4(Ds + (pt * 16 + lr) * kBP + 4 * lk), a4, a2[pt]);
      }
      f32x4 dc = zero4(), db = zero4();
#pragma unroll
      for (int j = 0; j < NPT; ++j) {
        dc = mma4(ya[j], ld4(St + lr * TP + 16 * j + 4 * lk), dc);
        db = mma4(xa[j], ld4(Dt + lr * TP + 16 * j + 4 * lk), db);
      }
      {
        // Y_t = sum_n C[t,n] (exp(Lam_t) dY[t] S_in)[n]: the inter part of dC
        const float4 c4 = ld4(Ct + lr * kQP + sw + 4 * lk);
        const float cr[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = sw + 4 * lk + r;
          dc[r] *= ex[t];
          db[r] *= wv[t];
          yp[r] += cr[r] * dc[r];
        }
      }
      for (int j = 0; j <= wave; ++j)  // s < sw + 16
        dc = mma4(ld4(Dg + (sw + lr) * kQP + 16 * j + 4 * lk), ld4(Bt + lr * kQP + 16 * j + 4 * lk),
                  dc);
      for (int j = wave; j < 4; ++j)  // t >= sw
        db = mma4(ld4(DgT + (sw + lr) * kQP + 16 * j + 4 * lk),
                  ld4(Ct + lr * kQP + 16 * j + 4 * lk), db);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = sw + 4 * lk + r;
        if (t < len) {
          const int64_t o = ((row0 + t) * Hs + h / hpb) * N + n0 + lr;
          dCh[o] = pc[r] + dc[r];
          dBh[o] = pb[r] + db[r];
        }
      }
      __syncthreads();
    }
  }

  // the next head of the workgroup: its first slice of dY and X, loaded
  // while this head finishes
  if (h % hpb + 1 < hpb) {
    const int nvp = min(kKS, P);
    ry.load(dY + row0 * HP + xo + P, HP, len, nvp);
    rx.load(v + row0 * C + xo + P, (int)C, len, nvp);
  }

  // (5) dX, and the row sums U_s, Y_t; dD and <dS_out, S_in>. Lane l holds
  // four consecutive p of token s = sw + l % 16 in a1, a2, ya and xa.
  {
    const int s = sw + lr;
    float up = 0.f, ddp = 0.f;
    if (s < len) {
      const float ws = wv[s];
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        const float4 xv = xa[pt], dys = ya[pt];
        st4(dv + (row0 + s) * C + xo + 16 * pt + 4 * lk,
            make_float4(a1[pt][0] + ws * a2[pt][0] + Dh * dys.x,
                        a1[pt][1] + ws * a2[pt][1] + Dh * dys.y,
                        a1[pt][2] + ws * a2[pt][2] + Dh * dys.z,
                        a1[pt][3] + ws * a2[pt][3] + Dh * dys.w));
        up += (xv.x * a2[pt][0] + xv.y * a2[pt][1]) + (xv.z * a2[pt][2] + xv.w * a2[pt][3]);
        ddp += (dys.x * xv.x + dys.y * xv.y) + (dys.z * xv.z + dys.w * xv.w);
      }
    }
    // U_s: the lanes l, l + 16, l + 32, l + 48 hold the parts of token s
    up += __shfl_xor(up, 16);
    up += __shfl_xor(up, 32);
    if (lk == 0) U[s] = up;
#pragma unroll
    for (int r = 0; r < 4; ++r) yp[r] = group_sum_last<16>(yp[r]);
    if (lr == 0)
#pragma unroll
      for (int r = 0; r < 4; ++r) Yo[sw + 4 * lk + r] = yp[r];
    cstp = wave_sum(cstp);
    ddp = wave_sum(ddp);
    if (lane == 0) {
      red[wave][0] = cstp;
      red[wave][1] = ddp;
    }
  }
  __syncthreads();
  // this chunk's parts of dD and dA, summed over the chunks later in a fixed
  // order: part[(b nc + c) H + h]
  const int64_t part = ((int64_t)b * nc + c) * H + h;
  const float cst = (red[0][0] + red[1][0]) + (red[2][0] + red[3][0]);
  if (tid == 0 && dD) dD[part] = (red[0][1] + red[1][1]) + (red[2][1] + red[3][1]);
  // (6) d(a_u), d(dt_u) and dA (wave 0, one lane per position)
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
      const float da = dai[u] + tmp[u] + __expf(lamE) * cst + pw;
      const float dd = colF[u] + __expf(lamE - lam[u]) * U[u] + Ah * da;
      ddt[(row0 + u) * (int64_t)H + h] = from_f<T>(dd);
      da_dt = dts[u] * da;
    }
    const float sa = wave_sum(da_dt);
    if (lane == 0) dA[part] = sa;
  }
}

// hpb heads of one group per workgroup, one after the other (MULTI; else
// hpb = 1): their dB and dC rows are summed in place (rows [T, H / hpb, N]).
template <class T, int P, bool MULTI>
__global__ __launch_bounds__(kThreads, 2) void k_chunk_bwd(
    const float* __restrict__ v, const float* __restrict__ dY, const T* __restrict__ dt, DtA dta,
    const float* __restrict__ A, const float* __restrict__ D, const float* __restrict__ Sin,
    const float* __restrict__ dSo, const float* __restrict__ cb, float* __restrict__ dv,
    float* __restrict__ dBh, float* __restrict__ dCh, T* __restrict__ ddt, float* dA, float* dD,
    int L, int H, int G, int N, int nc, int hpb) {
  SliceRegs<kQ> ry, rx;  // the first dY / X slice of a head's K product
  // this wave's causal tiles of the group's C B^T, the same for every head
  // of the workgroup (element (t, s) at t Q + s)
  f32x4 gt[3];
  {
    const int lane = threadIdx.x & 63, lr = lane & 15, lk = lane >> 4;
    const int g = blockIdx.y * hpb / (H / G);
    const float* cbk = cb + (((int64_t)blockIdx.z * nc + blockIdx.x) * G + g) * (kQ * kQ);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      int rt, st;
      const bool on = causal_tile(threadIdx.x >> 6, i, rt, st);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        gt[i][r] = on ? cbk[(rt * 16 + 4 * lk + r) * kQ + st * 16 + lr] : 0.f;
    }
  }
  if constexpr (!MULTI) {
    chunk_bwd_head<T, P>(v, dY, dt, dta, A, D, Sin, dSo, dv, dBh, dCh, ddt, dA, dD, L, H, G, N,
                         nc, blockIdx.y, 1, ry, rx, false, gt);
  } else {
#pragma unroll 1
    for (int j = 0; j < hpb; ++j) {
      chunk_bwd_head<T, P>(v, dY, dt, dta, A, D, Sin, dSo, dv, dBh, dCh, ddt, dA, dD, L, H, G, N,
                           nc, blockIdx.y * hpb + j, hpb, ry, rx, j > 0, gt);
      __syncthreads();  // LDS is reused by the next head
    }
  }
}

// ---------------------------------------------------------------- group sums
// dv's B and C channels = the sums of dBh / dCh over the rows of each group
// (Hs / G rows per group, each already the sum of a workgroup's heads).
__global__ __launch_bounds__(kThreads) void k_group_sum(const float* __restrict__ dBh,
                                                        const float* __restrict__ dCh,
                                                        float* dv, int64_t T, int Hs, int G,
                                                        int N, int HP) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= T * G * N) return;
  const int64_t t = i / (G * N);
  const int gn = (int)(i % (G * N)), g = gn / N, n = gn % N, spg = Hs / G;
  float sb = 0.f, sc = 0.f;
  for (int k = 0; k < spg; ++k) {
    const int64_t o = (t * Hs + g * spg + k) * N + n;
    sb += dBh[o];
    sc += dCh[o];
  }
  const int64_t C = HP + 2 * (int64_t)G * N;
  dv[t * C + HP + gn] = sb;
  dv[t * C + HP + (int64_t)G * N + gn] = sc;
}

// ---------------------------------------------------------------- conv + SiLU
// du = dv silu'(u) over a range of kConvTok tokens of four channels, u
// recomputed from the rows ext = [conv state ; xbc] through a sliding window;
// du overwrites dv. The range's sums for the weight and bias gradients go to
// its row of part: part[range][c * W + k] and part[range][C * W + c]. Each
// thread takes 4 consecutive channels (C is a multiple of 16), so its loads
// and stores are 16-byte (fp32) or 8-byte (bf16) vectors.
constexpr int kConvTok = 64;
SSD_DEV float4 f4mul(float4 a, float4 b) { return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w); }
SSD_DEV float4 f4fma(float4 a, float4 b, float4 c) {
  return make_float4(a.x * b.x + c.x, a.y * b.y + c.y, a.z * b.z + c.z, a.w * b.w + c.w);
}
template <class T, int W>
__global__ __launch_bounds__(kThreads) void k_conv_du(const T* __restrict__ xbc,
                                                      const T* __restrict__ cin,
                                                      const T* __restrict__ w,
                                                      const T* __restrict__ bias, float* dv,
                                                      float* part, int L, int C) {
  const int c = (blockIdx.x * kThreads + threadIdx.x) * 4;
  const int t0 = blockIdx.y * kConvTok, b = blockIdx.z;
  if (c >= C) return;
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 wk[W], dwp[W], win[W], dbp = z4;
#pragma unroll
  for (int k = 0; k < W; ++k) {
    wk[k] = make_float4(to_f(w[(int64_t)c * W + k]), to_f(w[(int64_t)(c + 1) * W + k]),
                        to_f(w[(int64_t)(c + 2) * W + k]), to_f(w[(int64_t)(c + 3) * W + k]));
    dwp[k] = z4;
  }
  const float4 bc = bias ? ld4(bias + c) : z4;
  // ext row e: conv state rows (e < W-1) or token e - (W-1)
  auto ext = [&](int e) -> float4 {
    if (e >= W - 1) return ld4(xbc + ((int64_t)b * L + e - (W - 1)) * C + c);
    return cin ? ld4(cin + ((int64_t)b * (W - 1) + e) * C + c) : z4;
  };
#pragma unroll
  for (int k = 0; k < W - 1; ++k) win[k] = ext(t0 + k);
  const int t1 = min(L, t0 + kConvTok);
  for (int t = t0; t < t1; ++t) {
    win[W - 1] = ext(t + W - 1);
    float4 u = bc;
#pragma unroll
    for (int k = 0; k < W; ++k) u = f4fma(wk[k], win[k], u);
    const float uv[4] = {u.x, u.y, u.z, u.w};
    float g[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sig = frcp(1.f + __expf(-uv[i]));
      g[i] = sig + uv[i] * sig * (1.f - sig);
    }
    const int64_t o = ((int64_t)b * L + t) * C + c;
    const float4 du = f4mul(ld4(dv + o), make_float4(g[0], g[1], g[2], g[3]));
    st4(dv + o, du);
#pragma unroll
    for (int k = 0; k < W; ++k) dwp[k] = f4fma(du, win[k], dwp[k]);
    dbp = make_float4(dbp.x + du.x, dbp.y + du.y, dbp.z + du.z, dbp.w + du.w);
#pragma unroll
    for (int k = 0; k < W - 1; ++k) win[k] = win[k + 1];
  }
  float* pr = part + ((int64_t)b * gridDim.y + blockIdx.y) * ((int64_t)C * (W + 1));
#pragma unroll
  for (int k = 0; k < W; ++k) {
    pr[(int64_t)c * W + k] = dwp[k].x;
    pr[(int64_t)(c + 1) * W + k] = dwp[k].y;
    pr[(int64_t)(c + 2) * W + k] = dwp[k].z;
    pr[(int64_t)(c + 3) * W + k] = dwp[k].w;
  }
  st4(pr + (int64_t)C * W + c, dbp);
}

// Gradient of the conv input rows ext = [conv state ; xbc]: d_ext[e] =
// sum_k w[k] du[e - k] over output tokens e - k in range (a sliding window
// over du); rows e >= W-1 go to d_xbc, the first W-1 to the initial conv
// state's gradient (fp32). Four consecutive channels per thread.
template <class T, int W>
__global__ __launch_bounds__(kThreads) void k_conv_dx(const float* __restrict__ du,
                                                      const T* __restrict__ w, T* __restrict__ dx,
                                                      float* dcin, int L, int C) {
  const int c = (blockIdx.x * kThreads + threadIdx.x) * 4;
  const int e0 = blockIdx.y * kConvTok, b = blockIdx.z;
  if (c >= C) return;
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 wk[W], win[W];  // win[k] = du[e - k]
#pragma unroll
  for (int k = 0; k < W; ++k)
    wk[k] = make_float4(to_f(w[(int64_t)c * W + k]), to_f(w[(int64_t)(c + 1) * W + k]),
                        to_f(w[(int64_t)(c + 2) * W + k]), to_f(w[(int64_t)(c + 3) * W + k]));
  auto dut = [&](int tt) -> float4 {
    return (tt >= 0 && tt < L) ? ld4(du + ((int64_t)b * L + tt) * C + c) : z4;
  };
#pragma unroll
  for (int k = 1; k < W; ++k) win[k] = dut(e0 - k);
  const int e1 = min(L + W - 1, e0 + kConvTok);
  for (int e = e0; e < e1; ++e) {
    win[0] = dut(e);
    float4 acc = z4;
#pragma unroll
    for (int k = 0; k < W; ++k) acc = f4fma(wk[k], win[k], acc);
    if (e >= W - 1)
      st4(dx + ((int64_t)b * L + e - (W - 1)) * C + c, acc);
    else if (dcin)
      st4(dcin + ((int64_t)b * (W - 1) + e) * C + c, acc);
#pragma unroll
    for (int k = W - 1; k > 0; --k) win[k] = win[k - 1];
  }
}

}  // namespace bwd

// Workspace of the backward pass (fp32): conv output v [T, Cch], y then dY
// [T, H*P], carried-in states and their gradients [B, nc, H, P, N], Lam_end
// [B, H, nc], dB / dC rows per per-chunk workgroup [T, H / hpb, N] (sized
// for hpb = 1), dv [T, Cch], the partial sums, and each chunk's C B^T per
// group [B, nc, G, Q, Q]; 64-token chunks.
namespace {
size_t bround(size_t b) { return (b + 255) / 256 * 256; }

// LDS of the per-chunk kernels (the chunk gradients and the state-gradient
// terms)
size_t bwd_chunk_lds(int P) {
  const size_t stage1 = 2 * (size_t)bwd::kQ * bwd::kSP,
               fm = (size_t)bwd::kQ * (bwd::kQ + 1) + 4 * (size_t)bwd::kQ,
               ys = (size_t)bwd::kQ * (P + 16),
               stage4 = (size_t)(bwd::kQ + P) * bwd::kBP + 2 * (size_t)bwd::kNS * bwd::kQP +
                        2 * (size_t)bwd::kNS * (P + 4);
  return (2 * (size_t)bwd::kQ * bwd::kQP + std::max(std::max(stage1, fm), std::max(ys, stage4))) *
         4;
}
size_t bwd_z_lds(int P, int N) { return (size_t)(P + N) * bwd::kQP * 4; }
}  // namespace

size_t backward_ws_bytes(int B, int L, int H, int P, int G, int N) {
  const size_t T = (size_t)B * L, HP = (size_t)H * P, C = HP + 2 * (size_t)G * N;
  const size_t nc = (L + bwd::kQ - 1) / bwd::kQ;
  const size_t st = (size_t)B * nc * H * P * N * 4;
  return bround(T * C * 4) + bround(T * HP * 4) + 2 * bround(st) + bround((size_t)B * H * nc * 4) +
         2 * bround(T * H * N * 4) + bround(T * C * 4) + bround((size_t)bwd::kNormBlocks * HP * 4) +
         bround((size_t)B * ((L + bwd::kConvTok - 1) / bwd::kConvTok) * C * 5 * 4) +
         bround((size_t)2 * B * nc * H * 4) + bround(chunk_cb_bytes(B, (int)nc, G));
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t st) {
  using namespace bwd;
  const bool bf = a.io_bf16;
  const int B = a.B, L = a.L, H = a.H, P = a.P, G = a.G, N = a.N, W = a.W;
  const int64_t T = (int64_t)B * L, HP = (int64_t)H * P, C = HP + 2 * (int64_t)G * N;
  const int nc = (L + kQ - 1) / kQ;
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
  w += bround(T * C * 4);
  float* dw_part = (float*)w;
  w += bround((size_t)kNormBlocks * HP * 4);
  float* conv_part = (float*)w;  // [B * ranges][Cch * (W + 1)]
  w += bround((size_t)B * ((L + kConvTok - 1) / kConvTok) * C * 5 * 4);
  float* dA_part = (float*)w;  // [B nc, H]: each chunk's part of dA, then of dD
  float* dD_part = dA_part + (size_t)B * nc * H;
  w += bround((size_t)2 * B * nc * H * 4);
  float* cb = (float*)w;  // [B nc G][Q][Q]: each chunk's C B^T per group
  const DtA plain{H, nullptr};
  const dim3 gc(nc, H, B), blk(kThreads);
  hipError_t e;
#define SSD_CHECK()                          \
  if ((e = hipGetLastError()) != hipSuccess) \
    return e;
// one launch per head size (the kernels are specialised on P)
#define SSD_BY_P(LAUNCH)               \
  switch (P) {                         \
    case 16: LAUNCH(16); break;        \
    case 32: LAUNCH(32); break;        \
    case 64: LAUNCH(64); break;        \
    default: LAUNCH(128); break;       \
  }
  // recompute the forward: conv output, chunk states passed into carried-in
  // states, y (all fp32)
  e = launch_conv1d(bf, B, L, (int)C, W, a.xbc, C, a.conv_w, a.conv_b, a.conv_in, v, C, true, st);
  if (e != hipSuccess) return e;
  ScanShape s{B, L, H, P, G, N, kQ, nc, plain};  // kQ: 64, as the output kernel needs
  const unsigned char* vb = (const unsigned char*)v;
  e = launch_chunk_state(bf, true, true, s, v, C, a.dt, a.A, vb + HP * 4, C, states, lam_end,
                         a.status, st);
  if (e != hipSuccess) return e;
  e = launch_state_pass(s, states, lam_end, a.s_in, nullptr, a.status, st);
  if (e != hipSuccess) return e;
  e = launch_chunk_y(bf, true, true, s, v, C, vb + HP * 4, vb + (HP + (int64_t)G * N) * 4, C, cb,
                     a.dt, a.A, a.D, states, y, a.status, KID_BWD_Y, st);
  if (e != hipSuccess) return e;
  {
    ProfScope ps(st, KID_BWD_NORM);
    // bf16 I/O with whole 256-channel pieces per norm group: the pieces'
    // sums come from the waves, and a row fits one 1024-thread workgroup's
    // registers; else each 4-channel lane's sums are kept in LDS
    const bool wide = bf && (HP / G) % 256 == 0;
    const int nblk = wide ? kNormWideBlocks : kNormBlocks;
    const int rows = (int)((T + nblk - 1) / nblk);
    const int nb = (int)((T + rows - 1) / rows);
    const size_t lds = (size_t)HP * 4 + (size_t)HP / 4 * 2 * 4;  // k_norm_bwd: dw, lane sums
#define SSD_NORM(TT)                                                                             \
  hipLaunchKernelGGL((k_norm_bwd<TT>), dim3(nb), blk, lds, st, y, (const TT*)a.z,                \
                     (const TT*)a.norm_w, (const TT*)a.d_out, a.eps, (TT*)a.d_z, dw_part, T,    \
                     rows, (int)HP, G)
    if (wide)
      hipLaunchKernelGGL(k_norm_bwd_wide, dim3(nb), dim3(kNormWideThreads), (size_t)HP * 4, st, y,
                         (const bf16*)a.z, (const bf16*)a.norm_w, (const bf16*)a.d_out, a.eps,
                         (bf16*)a.d_z, dw_part, T, rows, (int)HP, G);
    else if (bf)
      SSD_NORM(bf16);
    else
      SSD_NORM(float);
#undef SSD_NORM
    hipLaunchKernelGGL(k_sum_parts, dim3((unsigned)((HP + 63) / 64)), blk, 0, st, dw_part, HP,
                       a.d_norm_w, nb, (int)HP);
  }
  SSD_CHECK();
  {
    ProfScope ps(st, KID_BWD_CHUNK_Z);
    const size_t zl = bwd_z_lds(P, N);
    // heads per workgroup (one C staging for all of them): the most, up to
    // kZHeads, that divide the heads of a group and leave 2048 workgroups
    int zh = kZHeads;
    while (zh > 1 && ((H / G) % zh || (int64_t)B * nc * (H / zh) < 2048)) zh /= 2;
    if (a.chunk_heads > 0 && (H / G) % a.chunk_heads == 0) zh = a.chunk_heads;  // diagnostic
    const dim3 gz(nc, H / zh, B);
#define SSD_Z(PP)                                                                                \
  if (bf)                                                                                        \
    hipLaunchKernelGGL((k_chunk_z<bf16, PP>), gz, blk, zl, st, v, y, (const bf16*)a.dt, plain,   \
                       a.A, dso, L, H, G, N, nc, zh);                                            \
  else                                                                                           \
    hipLaunchKernelGGL((k_chunk_z<float, PP>), gz, blk, zl, st, v, y, (const float*)a.dt, plain, \
                       a.A, dso, L, H, G, N, nc, zh)
    SSD_BY_P(SSD_Z)
#undef SSD_Z
  }
  SSD_CHECK();
  {
    ProfScope ps(st, KID_BWD_REV_PASS);
    hipLaunchKernelGGL(k_rev_pass, dim3((P * N + kThreads - 1) / kThreads, H, B), blk, 0, st,
                       dso, lam_end, a.d_s_out, a.d_s_in, H, P * N, nc);
  }
  SSD_CHECK();
  // heads per workgroup of the per-chunk kernel (their dB / dC rows summed in
  // place): the most, up to kChunkHeads, that divide the heads of a group and
  // leave at least 1024 workgroups; one for head size 128, whose registers
  // do not hold the head loop
  int hpb = P == 128 ? 1 : kChunkHeads;
  while (hpb > 1 && ((H / G) % hpb || (int64_t)B * nc * (H / hpb) < 1024)) hpb /= 2;
  if (a.chunk_heads > 0 && a.chunk_heads <= kChunkHeads && P != 128 && (H / G) % a.chunk_heads == 0)
    hpb = a.chunk_heads;  // a diagnostic setting, where the shape allows it
  {
    ProfScope ps(st, KID_BWD_CHUNK);
    const size_t lds = bwd_chunk_lds(P);
    const dim3 gh(nc, H / hpb, B);
#define SSD_CB_M(TT, PP, MM)                                                                    \
  hipLaunchKernelGGL((k_chunk_bwd<TT, PP, MM>), gh, blk, lds, st, v, y, (const TT*)a.dt, plain, \
                     a.A, a.D, states, dso, cb, dv, dBh, dCh, (TT*)a.d_dt, dA_part,             \
                     a.d_D ? dD_part : nullptr, L, H, G, N, nc, hpb)
#define SSD_CB_T(TT, PP)             \
  {                                  \
    if (PP == 128 || hpb == 1)       \
      SSD_CB_M(TT, PP, false);       \
    else                             \
      SSD_CB_M(TT, PP, PP != 128);   \
  }
#define SSD_CB(PP)      \
  {                     \
    if (bf)             \
      SSD_CB_T(bf16, PP) \
    else                \
      SSD_CB_T(float, PP) \
  }
    SSD_BY_P(SSD_CB)
#undef SSD_CB
#undef SSD_CB_T
#undef SSD_CB_M
    // dA and dD: the chunks' parts added in a fixed order
    hipLaunchKernelGGL(k_sum_parts, dim3((unsigned)((H + 63) / 64)), blk, 0, st, dA_part,
                       (int64_t)H, a.d_A, B * nc, H);
    if (a.d_D)
      hipLaunchKernelGGL(k_sum_parts, dim3((unsigned)((H + 63) / 64)), blk, 0, st, dD_part,
                         (int64_t)H, a.d_D, B * nc, H);
  }
  SSD_CHECK();
  {
    ProfScope ps(st, KID_BWD_GROUP_SUM);
    hipLaunchKernelGGL(k_group_sum, dim3((unsigned)((T * G * N + kThreads - 1) / kThreads)), blk,
                       0, st, dBh, dCh, dv, T, H / hpb, G, N, (int)HP);
  }
  SSD_CHECK();
  {
    ProfScope ps(st, KID_BWD_CONV_DU);
    const int ny = (L + kConvTok - 1) / kConvTok;
    const dim3 gd((unsigned)((C / 4 + kThreads - 1) / kThreads), ny, B);
#define SSD_DU(TT, WW)                                                                       \
  hipLaunchKernelGGL((k_conv_du<TT, WW>), gd, blk, 0, st, (const TT*)a.xbc,                  \
                     (const TT*)a.conv_in, (const TT*)a.conv_w, (const TT*)a.conv_b, dv,     \
                     conv_part, L, (int)C)
#define SSD_DU_W(TT) \
  if (W == 2) SSD_DU(TT, 2); else if (W == 3) SSD_DU(TT, 3); else SSD_DU(TT, 4)
    if (bf) { SSD_DU_W(bf16); } else { SSD_DU_W(float); }
#undef SSD_DU_W
#undef SSD_DU
    const int64_t pst = C * (W + 1);
    hipLaunchKernelGGL(k_sum_parts, dim3((unsigned)((C * W + 63) / 64)), blk, 0, st, conv_part,
                       pst, a.d_conv_w, B * ny, (int)(C * W));
    if (a.d_conv_b)
      hipLaunchKernelGGL(k_sum_parts, dim3((unsigned)((C + 63) / 64)), blk, 0, st,
                         conv_part + C * W, pst, a.d_conv_b, B * ny, (int)C);
  }
  SSD_CHECK();
  {
    ProfScope ps(st, KID_BWD_CONV_DX);
    const dim3 gx((unsigned)((C / 4 + kThreads - 1) / kThreads),
                  (L + W - 1 + kConvTok - 1) / kConvTok, B);
#define SSD_DX(TT, WW)                                                                         \
  hipLaunchKernelGGL((k_conv_dx<TT, WW>), gx, blk, 0, st, dv, (const TT*)a.conv_w,             \
                     (TT*)a.d_xbc, a.d_conv_in, L, (int)C)
#define SSD_DX_W(TT) \
  if (W == 2) SSD_DX(TT, 2); else if (W == 3) SSD_DX(TT, 3); else SSD_DX(TT, 4)
    if (bf) { SSD_DX_W(bf16); } else { SSD_DX_W(float); }
#undef SSD_DX_W
#undef SSD_DX
  }
  SSD_CHECK();
#undef SSD_BY_P
#undef SSD_CHECK
  return hipSuccess;
}

}  // namespace ssd
