// Fast path of the chunked SSD scan for the Mamba-2 layer shape of the
// Nemotron-H models (head_dim 64, d_state 128; "NemotronH-0.3B-A0.3B" card,
// "Configuration Changes": mamba_head_dim 64, n_groups 8), bf16 I/O, with
// the causal conv + SiLU recomputed inside the consumers so the conv output
// never goes to HBM.
//
// Same block decomposition as the generic kernels ("feat(model): add
// Nemotron-3 Nano hybrid ..." attribution commit: ssd_minimal_discrete /
// segsum), blocked in 128-token chunks. Three launches:
//   1. k_fstate  (chunk, batch x head-block): conv+SiLU of x and B for the
//      chunk, dS_h = (x w_h)^T B for 4 heads on bf16 MFMA, written fp32.
//   2. k_fpass   state passing along chunks; S_in(k) written as bf16 (the
//      precision the MFMA consumes), final state fp32.
//   3. k_fout    (chunk, batch x head-block): conv+SiLU of x, B, C; the causal
//      C B^T computed once and shared by the 4 heads; per head
//      y = M' x + exp(Lam_t) C S_in^T + D x with M'[t,s] = (C_t.B_s)
//      exp(Lam_t - Lam_s) dt_s on bf16 MFMA and D x in fp32 (x recomputed at
//      full precision: the norm that follows divides by rms(q), so this
//      largest term of y must not carry bf16 rounding); then the gated
//      RMSNorm over the 4 heads (one norm group) and a coalesced store.
#include "common.hpp"
#include "launch.hpp"

namespace ssd {
namespace fast {

constexpr int P = 64, N = 128, QI = 128, HB = 4, W = 4;
constexpr int NT = 512;       // threads per workgroup (8 waves)
constexpr int RS = QI + 8;    // padded bf16 row of [.][QI] tiles (16 B skew per row)
constexpr int NS = N + 8;     // padded bf16 row of [.][N] tiles
constexpr int OS = HB * P + 8;

// Where the x / B / C rows of one batch come from.
struct Src {
  const bf16* x;      // channel 0 of x  at (batch 0, token 0)
  const bf16* b;      // channel 0 of B
  const bf16* c;      // channel 0 of C
  int64_t xs, bs;     // token strides (elements) of x and of B/C
  const bf16* cw;     // conv weight [Cch][W] (conv mode)
  const bf16* cbias;  // conv bias [Cch] or null
  const bf16* cin;    // conv state in [B][W-1][Cch] or null
  int C, HP, GN;      // conv channels, H*P, G*N
};

SSD_DEV uint32_t pk(float a, float b) { return pack_bf16x2(a, b); }

// Unpack 8 bf16 (one 16-byte row segment) to fp32.
SSD_DEV void unpack8(const uint4 u, float (&v)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Stage 8 tokens x 8 channels of conv+SiLU output (or of the plain input
// when !CONV) into LDS as bf16: TRANS=false writes row i (token) at
// dst + i*ld as one 16-byte vector; TRANS=true writes row j (channel) at
// dst + j*ld with the 8 tokens contiguous. Rows past nvalid are zero; each
// token i is multiplied by scale[i] when scale is non-null.
// src: the channel vector's element at token 0 of this batch; tseq: sequence
// position of the first token; Lm1: last token of the sequence; ch: absolute
// xBC channel (conv weights); cin_b: conv state of this batch or null.
// Every row load is issued before any is used: addresses are clamped into
// the sequence and out-of-range rows are masked afterwards, so the loads
// are not serialised behind per-lane branches.
template <bool CONV, bool TRANS>
SSD_DEV void conv_stage(const bf16* __restrict__ src, int64_t ts, int tseq, int nvalid, int Lm1,
                        const Src& s, int ch, const bf16* cin_b, const float* scale, bf16* dst,
                        int ld) {
  constexpr int R = CONV ? W - 1 : 0;
  uint4 raw[8 + R];
#pragma unroll
  for (int i = 0; i < 8 + R; ++i) {
    const int t = tseq - R + i;
    const bf16* p = (CONV && t < 0 && cin_b) ? cin_b + (int64_t)(W - 1 + t) * s.C + ch
                                             : src + (int64_t)min(max(t, 0), Lm1) * ts;
    raw[i] = *reinterpret_cast<const uint4*>(p);
  }
  float wk[W][8], bi[8];
  if (CONV) {
    const uint4* wp = reinterpret_cast<const uint4*>(s.cw + (int64_t)ch * W);
    // 8 channels x 4 taps = 32 bf16 = 4 x 16 B; element (j, k) at j*W + k
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 u = wp[q];
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx0 = q * 8 + 2 * e;  // element index of the low half
        wk[idx0 % W][idx0 / W] = __uint_as_float(w4[e] << 16);
        wk[(idx0 + 1) % W][(idx0 + 1) / W] = __uint_as_float(w4[e] & 0xffff0000u);
      }
    }
    if (s.cbias) {
      load8(s.cbias + ch, bi);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) bi[j] = 0.f;
    }
  }
  float win[R + 1][8];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    unpack8(raw[i], win[i]);
    if (tseq - R + i < 0 && !cin_b) {
#pragma unroll
      for (int j = 0; j < 8; ++j) win[i][j] = 0.f;
    }
  }
  uint32_t pk8[8][4];  // TRANS: channel j, tokens (2e, 2e+1)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    unpack8(raw[i + R], win[R]);
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float u;
      if (CONV) {
        u = bi[j];
#pragma unroll
        for (int k = 0; k < W; ++k) u += wk[k][j] * win[k][j];
        u = silu(u);
      } else {
        u = win[R][j];
      }
      if (scale) u *= scale[i];
      v[j] = i < nvalid ? u : 0.f;
    }
    if (TRANS) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t hbits = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[j]);
        if (i & 1) pk8[j][i >> 1] |= hbits << 16;
        else pk8[j][i >> 1] = hbits;
      }
    } else {
      *reinterpret_cast<uint4*>(dst + i * ld) =
          make_uint4(pk(v[0], v[1]), pk(v[2], v[3]), pk(v[4], v[5]), pk(v[6], v[7]));
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j) win[r][j] = win[r + 1][j];
  }
  if (TRANS) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<uint4*>(dst + j * ld) = make_uint4(pk8[j][0], pk8[j][1], pk8[j][2], pk8[j][3]);
  }
}

// Inclusive cumsum of dt*A for the HB heads of the workgroup: thread tid
// handles head tid / QI, position tid % QI (two waves per head).
SSD_DEV void heads_cumsum(const bf16* __restrict__ dt, int64_t row0, int H, int h0, int len,
                          const float* __restrict__ A, float (*lam)[QI], float (*dts)[QI],
                          float* wtot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = tid / QI, t = tid % QI;
  const float dr = to_f(dt[(row0 + min(t, len - 1)) * H + h0 + hh]);
  const float d = t < len ? dr : 0.f;
  float v = d * A[h0 + hh];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float n = __shfl_up(v, o, 64);
    if (lane >= o) v += n;
  }
  if (lane == 63) wtot[wave] = v;
  __syncthreads();
  if (wave & 1) v += wtot[wave - 1];
  lam[hh][t] = v;
  dts[hh][t] = d;
  __syncthreads();
}

// x-channel block mapping for transposed staging: within 16 lanes, 2 channel
// vectors x 8 token blocks, so the 16-byte LDS writes of a phase hit 16
// distinct bank groups. Returns (cv, tbi) for block index i of a tile with
// ncv channel vectors and QI/8 = 16 token blocks.
SSD_DEV void tmap(int i, int& cv, int& tbi) {
  tbi = (i >> 1) & 15;
  cv = (i & 1) | ((i >> 5) << 1);
}

// D * x for 4 consecutive tokens (tseq .. tseq+3, nvalid of them inside the
// chunk) of channels ch0 + 16*pt, pt < 4, with x at full fp32 precision: in
// conv mode x is recomputed here from the raw xBC rows (7 rows cover the
// 4 outputs' taps), otherwise it is read from the input.
template <bool CONV>
SSD_DEV void dx_term(const Src& s, int b, int L, int tseq, int nvalid, int ch0, float Dh,
                     const bf16* cin_b, float (&dx)[4][4]) {
  const bf16* xb = s.x + (int64_t)b * L * s.xs;
  constexpr int R = CONV ? W - 1 : 0;
  bf16 raw[4][R + 4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    const int ch = ch0 + pt * 16;
#pragma unroll
    for (int i = 0; i < R + 4; ++i) {
      const int t = tseq - R + i;
      const bf16* p = (CONV && t < 0 && cin_b) ? cin_b + (int64_t)(W - 1 + t) * s.C + ch
                                               : xb + (int64_t)min(max(t, 0), L - 1) * s.xs + ch;
      raw[pt][i] = *p;
    }
  }
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    const int ch = ch0 + pt * 16;
    if (!CONV) {
#pragma unroll
      for (int r = 0; r < 4; ++r) dx[pt][r] = r < nvalid ? Dh * to_f(raw[pt][r]) : 0.f;
      continue;
    }
    float row[R + 4];
#pragma unroll
    for (int i = 0; i < R + 4; ++i) {
      const int t = tseq - R + i;
      row[i] = (t < 0 && !cin_b) ? 0.f : to_f(raw[pt][i]);
    }
    float wk[W];
#pragma unroll
    for (int k = 0; k < W; ++k) wk[k] = to_f(s.cw[(int64_t)ch * W + k]);
    const float bi = s.cbias ? to_f(s.cbias[ch]) : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float u = bi;
#pragma unroll
      for (int k = 0; k < W; ++k) u += wk[k] * row[r + k];
      dx[pt][r] = r < nvalid ? Dh * silu(u) : 0.f;
    }
  }
}

// ---------------------------------------------------------------- phase 1
template <bool CONV>
__global__ __launch_bounds__(NT) void k_fstate(Src s, const bf16* __restrict__ dt,
                                               const float* __restrict__ A,
                                               float* __restrict__ states,
                                               float* __restrict__ lam_end, int L, int H, int G,
                                               int nc) {
  __shared__ __align__(16) bf16 BT[N * RS];        // [n][s]
  __shared__ __align__(16) bf16 XT[HB * P * RS];   // [head][p][s] = x_s[p] w_s
  __shared__ float lam[HB][QI], wv[HB][QI], wtot[NT / 64];
  const int c = blockIdx.x, hpb = H / HB;
  const int b = blockIdx.y / hpb, h0 = (blockIdx.y % hpb) * HB, g = h0 / (H / G);
  const int t0 = c * QI, len = min(QI, L - t0);
  const int64_t row0 = (int64_t)b * L + t0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  heads_cumsum(dt, row0, H, h0, len, A, lam, wv, wtot);
  {
    const int hh = tid / QI, t = tid % QI;
    const float lamE = lam[hh][len - 1];
    const float d = wv[hh][t];
    __syncthreads();
    wv[hh][t] = t < len ? fexp(lamE - lam[hh][t]) * d : 0.f;
  }
  __syncthreads();

  const bf16* cin_b = CONV && s.cin ? s.cin + (int64_t)b * (W - 1) * s.C : nullptr;
  const bf16* xb = s.x + (int64_t)b * L * s.xs;
  const bf16* bb = s.b + (int64_t)b * L * s.bs;
  // x: 32 channel vectors x 16 token blocks; B: 16 x 16.
  for (int blk = tid; blk < 768; blk += NT) {
    int cv, tbi;
    if (blk < 512) {
      tmap(blk, cv, tbi);
      const int hh = cv >> 3, p0 = (cv & 7) * 8;
      const int ch = (h0 + hh) * P + p0;
      conv_stage<CONV, true>(xb + ch, s.xs, t0 + tbi * 8, min(8, max(0, len - tbi * 8)), L - 1, s,
                             ch, cin_b, &wv[hh][tbi * 8], XT + (hh * P + p0) * RS + tbi * 8, RS);
    } else {
      tmap(blk - 512, cv, tbi);
      const int n0 = cv * 8;
      const int ch = s.HP + g * N + n0;
      conv_stage<CONV, true>(bb + g * N + n0, s.bs, t0 + tbi * 8, min(8, max(0, len - tbi * 8)),
                             L - 1, s, ch, cin_b, nullptr, BT + n0 * RS + tbi * 8, RS);
    }
  }
  __syncthreads();

  // dS_h [64 x 128] = XT_h . BT^T over k = s. Wave w: head w/2, p-tiles 2(w%2)..+1.
  const int hh = wave >> 1, pt0 = (wave & 1) * 2;
  const int rr = lane & 15, kk = 8 * (lane >> 4);
  f32x4 acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[i][n] = zero4();
  const bf16* a0p = XT + (hh * P + pt0 * 16 + rr) * RS + kk;
  const bf16* a1p = a0p + 16 * RS;
  const bf16* bp = BT + rr * RS + kk;
#pragma unroll
  for (int k = 0; k < QI; k += 32) {
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(a0p + k);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(a1p + k);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const bf16x8 bf = *reinterpret_cast<const bf16x8*>(bp + n * 16 * RS + k);
      acc[0][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bf, acc[0][n], 0, 0, 0);
      acc[1][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bf, acc[1][n], 0, 0, 0);
    }
  }
  float* out = states + (((int64_t)b * nc + c) * H + h0 + hh) * (int64_t)(P * N);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = (pt0 + i) * 16 + 4 * (lane >> 4) + r, nn = n * 16 + rr;
        out[p * N + nn] = acc[i][n][r];
      }
  if (tid < HB) lam_end[((int64_t)b * H + h0 + tid) * nc + c] = lam[tid][len - 1];
}

// ---------------------------------------------------------------- phase 2
constexpr int kPassDepth = 8;
__global__ __launch_bounds__(256) void k_fpass(const float* __restrict__ dS,
                                               const float* __restrict__ lam_end,
                                               const float* s_in, float* s_out,
                                               bf16* __restrict__ sin_bf, int H, int nc) {
  constexpr int PN = P * N;
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * H + h;
  float4 S = make_float4(0.f, 0.f, 0.f, 0.f);
  if (s_in) S = *reinterpret_cast<const float4*>(s_in + bh * PN + e);
  for (int c0 = 0; c0 < nc; c0 += kPassDepth) {
    float4 d[kPassDepth];
    float al[kPassDepth];
#pragma unroll
    for (int u = 0; u < kPassDepth; ++u) {
      const int c = c0 + u;
      if (c < nc) {
        d[u] = *reinterpret_cast<const float4*>(dS + (((int64_t)b * nc + c) * H + h) * PN + e);
        al[u] = fexp(lam_end[bh * nc + c]);
      }
    }
#pragma unroll
    for (int u = 0; u < kPassDepth; ++u) {
      const int c = c0 + u;
      if (c < nc) {
        uint2 o = make_uint2(pk(S.x, S.y), pk(S.z, S.w));
        *reinterpret_cast<uint2*>(sin_bf + (((int64_t)b * nc + c) * H + h) * PN + e) = o;
        S.x = al[u] * S.x + d[u].x;
        S.y = al[u] * S.y + d[u].y;
        S.z = al[u] * S.z + d[u].z;
        S.w = al[u] * S.w + d[u].w;
      }
    }
  }
  if (s_out) *reinterpret_cast<float4*>(s_out + bh * PN + e) = S;
}

// ---------------------------------------------------------------- phase 3
// YMODE 0: fused gated norm -> bf16 out; 1: y -> bf16 out; 2: y -> fp32 out.
template <bool CONV, int YMODE>
__global__ __launch_bounds__(NT) void k_fout(Src s, const bf16* __restrict__ dt,
                                             const float* __restrict__ A,
                                             const float* __restrict__ D,
                                             const bf16* __restrict__ sin_bf,
                                             const bf16* __restrict__ z,
                                             const bf16* __restrict__ nw, float eps,
                                             void* __restrict__ out, int L, int H, int G, int nc) {
  __shared__ __align__(16) bf16 Cs[QI * NS];      // [t][n]
  __shared__ __align__(16) bf16 Gs[QI * RS];      // [t][s] = C_t . B_s (causal tiles)
  __shared__ __align__(16) bf16 U[HB * P * RS];   // Bs [s][n], then XT [head][p][s], then out tile
  __shared__ float lam[HB][QI], dts[HB][QI], wtot[NT / 64], rss[QI];
  bf16* Bs = U;
  bf16* XT = U;
  bf16* Ot = U;

  const int c = blockIdx.x, hpb = H / HB;
  const int b = blockIdx.y / hpb, h0 = (blockIdx.y % hpb) * HB, g = h0 / (H / G);
  const int t0 = c * QI, len = min(QI, L - t0);
  const int64_t row0 = (int64_t)b * L + t0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rr = lane & 15, kk = 8 * (lane >> 4), r4 = 4 * (lane >> 4);
  const int HP = s.HP;

  if (tid < QI) rss[tid] = 0.f;
  heads_cumsum(dt, row0, H, h0, len, A, lam, dts, wtot);

  const bf16* cin_b = CONV && s.cin ? s.cin + (int64_t)b * (W - 1) * s.C : nullptr;
  // B and C, natural layout: 16 channel vectors x 16 token blocks each.
  {
    const int blk = tid;  // 512 blocks, one per thread
    const bool isC = blk >= 256;
    const int i = blk & 255, cv = i & 15, tbi = i >> 4, n0 = cv * 8;
    const bf16* base = (isC ? s.c : s.b) + (int64_t)b * L * s.bs + g * N + n0;
    const int ch = s.HP + (isC ? s.GN : 0) + g * N + n0;
    conv_stage<CONV, false>(base, s.bs, t0 + tbi * 8, min(8, max(0, len - tbi * 8)), L - 1, s, ch,
                            cin_b, nullptr, (isC ? Cs : Bs) + (tbi * 8) * NS + n0, NS);
  }
  __syncthreads();

  // Causal G tiles (ti >= si), 36 of them, over 8 waves.
  for (int tile = wave; tile < 36; tile += NT / 64) {
    int ti = 0;
    while ((ti + 1) * (ti + 2) / 2 <= tile) ++ti;
    const int si = tile - ti * (ti + 1) / 2;
    f32x4 gacc = zero4();
    const bf16* ap = Cs + (ti * 16 + rr) * NS + kk;
    const bf16* bp = Bs + (si * 16 + rr) * NS + kk;
#pragma unroll
    for (int k = 0; k < N; k += 32)
      gacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(ap + k),
                                                    *reinterpret_cast<const bf16x8*>(bp + k),
                                                    gacc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) Gs[(ti * 16 + r4 + r) * RS + si * 16 + rr] = (bf16)gacc[r];
  }
  __syncthreads();

  // x of the 4 heads, transposed [head][p][s] (overwrites Bs).
  {
    const bf16* xb = s.x + (int64_t)b * L * s.xs;
    int cv, tbi;
    tmap(tid, cv, tbi);
    const int hh = cv >> 3, p0 = (cv & 7) * 8;
    const int ch = (h0 + hh) * P + p0;
    conv_stage<CONV, true>(xb + ch, s.xs, t0 + tbi * 8, min(8, max(0, len - tbi * 8)), L - 1, s, ch,
                           cin_b, nullptr, XT + (hh * P + p0) * RS + tbi * 8, RS);
  }
  __syncthreads();

  // Main products. Wave w: heads 2(w/4), 2(w/4)+1; row tiles w%4 and 7-w%4.
  // Each (row tile, head) unit first issues its global loads (gate inputs and
  // the rows for the exact D x term), then runs its MFMAs, then combines.
  float q[2][2][4][4];  // [row tile][head][p tile][r]: gated output (or y)
  float ssr[2][4];      // per-row sum of squares of this lane's gated values
  const int hsel = 2 * (wave >> 2);
#pragma unroll
  for (int ui = 0; ui < 2; ++ui) {
    const int rt = ui == 0 ? (wave & 3) : 7 - (wave & 3);
    const int trow = rt * 16 + rr;  // A-operand row
    const int nks = (rt * 16 + 16 + 31) / 32;
#pragma unroll
    for (int r = 0; r < 4; ++r) ssr[ui][r] = 0.f;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int hh = hsel + hi;
      bf16 zr[4][4];
      if (YMODE == 0) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = min(rt * 16 + r4 + r, len - 1);
            zr[pt][r] = z[(row0 + t) * HP + (h0 + hh) * P + pt * 16 + rr];
          }
      }
      float dx[4][4];
      dx_term<CONV>(s, b, L, t0 + rt * 16 + r4, len - (rt * 16 + r4), (h0 + hh) * P + rr,
                    D ? D[h0 + hh] : 0.f, cin_b, dx);
      const float lt = lam[hh][trow];
      f32x4 acc[4], acc2[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) { acc[pt] = zero4(); acc2[pt] = zero4(); }
      for (int ks = 0; ks < nks; ++ks) {
        const int sb = ks * 32 + kk;
        const bf16x8 g8 = *reinterpret_cast<const bf16x8*>(Gs + trow * RS + sb);
        const float4 l0 = *reinterpret_cast<const float4*>(&lam[hh][sb]);
        const float4 l1 = *reinterpret_cast<const float4*>(&lam[hh][sb + 4]);
        const float4 d0 = *reinterpret_cast<const float4*>(&dts[hh][sb]);
        const float4 d1 = *reinterpret_cast<const float4*>(&dts[hh][sb + 4]);
        const float ls[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        const float ds[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
        bf16x8 af;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float m = (float)g8[j] * fexp(fminf(lt - ls[j], 0.f)) * ds[j];
          af[j] = (bf16)(sb + j <= trow ? m : 0.f);
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const bf16x8 bf =
              *reinterpret_cast<const bf16x8*>(XT + (hh * P + pt * 16 + rr) * RS + sb);
          acc[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[pt], 0, 0, 0);
        }
      }
      const bf16* sp = sin_bf + (((int64_t)b * nc + c) * H + h0 + hh) * (int64_t)(P * N);
#pragma unroll
      for (int ks = 0; ks < N / 32; ++ks) {
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(Cs + trow * NS + ks * 32 + kk);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const bf16x8 bf =
              *reinterpret_cast<const bf16x8*>(sp + (pt * 16 + rr) * N + ks * 32 + kk);
          acc2[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc2[pt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = rt * 16 + r4 + r;
        const float el = fexp(lam[hh][t]);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const float y = acc[pt][r] + el * acc2[pt][r] + dx[pt][r];
          if (YMODE == 0) {
            const float qq = t < len ? y * silu(to_f(zr[pt][r])) : 0.f;
            q[ui][hi][pt][r] = qq;
            ssr[ui][r] += qq * qq;
          } else if (t < len) {
            const int64_t o = (row0 + t) * HP + (h0 + hh) * P + pt * 16 + rr;
            if (YMODE == 2) reinterpret_cast<float*>(out)[o] = y;
            else reinterpret_cast<bf16*>(out)[o] = (bf16)y;
          }
        }
      }
    }
  }

  if (YMODE == 0) {
    // per-row sum of squares over the 4 heads' 256 channels: 16 lanes x 8
    // values here, the other head pair in another wave (LDS atomics)
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int rt = ui == 0 ? (wave & 3) : 7 - (wave & 3);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float ss = ssr[ui][r];
        ss += __shfl_xor(ss, 1, 64);
        ss += __shfl_xor(ss, 2, 64);
        ss += __shfl_xor(ss, 4, 64);
        ss += __shfl_xor(ss, 8, 64);
        if (rr == 0) atomicAdd(&rss[rt * 16 + r4 + r], ss);
      }
    }
    __syncthreads();  // all XT reads done, row sums complete
    const float invS = 1.0f / (float)(HB * P);
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int rt = ui == 0 ? (wave & 3) : 7 - (wave & 3);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = rt * 16 + r4 + r;
        const float inv = __builtin_amdgcn_rsqf(rss[t] * invS + eps);
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) {
            const int col = (hsel + hi) * P + pt * 16 + rr;
            const float w = to_f(nw[h0 * P + col]);
            Ot[t * OS + col] = (bf16)(q[ui][hi][pt][r] * w * inv);
          }
      }
    }
    __syncthreads();
    bf16* o = reinterpret_cast<bf16*>(out);
    for (int i = tid; i < QI * (HB * P / 8); i += NT) {
      const int t = i / (HB * P / 8), v8 = i % (HB * P / 8);
      if (t < len)
        *reinterpret_cast<uint4*>(o + (row0 + t) * HP + h0 * P + v8 * 8) =
            *reinterpret_cast<const uint4*>(Ot + t * OS + v8 * 8);
    }
  }
}

}  // namespace fast

// ---------------------------------------------------------------------------
bool fast_path_ok(bool io_bf16, int P, int N, int H, int G, int Q, int W, bool conv) {
  return io_bf16 && P == fast::P && N == fast::N && (H / G) % fast::HB == 0 && Q >= 64 &&
         (!conv || W == fast::W);
}

size_t fast_ws_bytes(int B, int L, int H) {
  const size_t nc = (L + fast::QI - 1) / fast::QI;
  const size_t PN = fast::P * fast::N;
  return (size_t)B * nc * H * PN * (4 + 2) + (size_t)B * H * nc * 4 + 3 * 256;
}

hipError_t launch_fast_scan(const FastScanArgs& a, hipStream_t st) {
  using namespace fast;
  const int nc = (a.L + QI - 1) / QI;
  const size_t PN = P * N;
  unsigned char* w = (unsigned char*)a.ws;
  float* dS = (float*)w;
  w += ((size_t)a.B * nc * a.H * PN * 4 + 255) / 256 * 256;
  bf16* sinb = (bf16*)w;
  w += ((size_t)a.B * nc * a.H * PN * 2 + 255) / 256 * 256;
  float* lam_end = (float*)w;

  Src s;
  s.x = (const bf16*)a.x;
  s.b = (const bf16*)a.Bm;
  s.c = (const bf16*)a.Cm;
  s.xs = a.xs;
  s.bs = a.bs;
  s.cw = (const bf16*)a.conv_w;
  s.cbias = (const bf16*)a.conv_b;
  s.cin = (const bf16*)a.conv_in;
  s.C = a.H * P + 2 * a.G * N;
  s.HP = a.H * P;
  s.GN = a.G * N;

  dim3 g1(nc, a.B * (a.H / HB));
  if (a.conv)
    hipLaunchKernelGGL(k_fstate<true>, g1, dim3(NT), 0, st, s, (const bf16*)a.dt, a.A, dS,
                       lam_end, a.L, a.H, a.G, nc);
  else
    hipLaunchKernelGGL(k_fstate<false>, g1, dim3(NT), 0, st, s, (const bf16*)a.dt, a.A, dS,
                       lam_end, a.L, a.H, a.G, nc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_fpass, dim3(PN / 1024, a.H, a.B), dim3(256), 0, st, dS, lam_end, a.s_in,
                     a.s_out, sinb, a.H, nc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 0: fused norm (norm group == head block), 1: y bf16, 2: y fp32 (norm afterwards)
  const int ymode = a.z ? ((a.H / a.G) == HB ? 0 : 2) : 1;
#define SSD_FOUT(CV, YM)                                                                         \
  hipLaunchKernelGGL((k_fout<CV, YM>), g1, dim3(NT), 0, st, s, (const bf16*)a.dt, a.A, a.D,      \
                     sinb, (const bf16*)a.z, (const bf16*)a.norm_w, a.eps,                        \
                     ymode == 2 ? (void*)a.y32 : a.y, a.L, a.H, a.G, nc)
  if (a.conv) {
    if (ymode == 0) SSD_FOUT(true, 0);
    else if (ymode == 1) SSD_FOUT(true, 1);
    else SSD_FOUT(true, 2);
  } else {
    if (ymode == 0) SSD_FOUT(false, 0);
    else if (ymode == 1) SSD_FOUT(false, 1);
    else SSD_FOUT(false, 2);
  }
#undef SSD_FOUT
  e = hipGetLastError();
  if (e != hipSuccess || ymode != 2) return e;
  return launch_gated_norm(true, true, a.B * a.L, a.H * P, a.G, a.y32, a.z, a.norm_w, a.eps, a.y,
                           st);
}

}  // namespace ssd
