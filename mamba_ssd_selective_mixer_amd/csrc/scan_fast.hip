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
//      chunk, dS_h = (x w_h)^T B for 4 heads on fp16 MFMA, written fp16.
//   2. k_fpass   state passing along chunks in fp32; S_in(k) written as fp16
//      (the precision the MFMA consumes), final state fp32.
//   3. k_fout    (chunk, batch x head-block): conv+SiLU of x, B, C; the causal
//      C B^T computed once and shared by the 4 heads; per head
//      y = M' x + exp(Lam_t) C S_in^T + D x with M'[t,s] = (C_t.B_s)
//      exp(Lam_t - Lam_s) dt_s on fp16 MFMA and D x from x kept as an fp16
//      hi + lo pair (the norm that follows divides by rms(q), so this
//      largest term of y must not carry operand rounding); then the gated
//      RMSNorm over the 4 heads (one norm group) and a coalesced store.
#include "common.hpp"
#include "launch.hpp"

namespace ssd {
namespace fast {

constexpr int P = 64, N = 128, QI = 128, HB = 4, W = 4;
constexpr int NT = 256;       // threads per workgroup (4 waves): two workgroups fit a CU
constexpr int RS = QI + 8;    // padded 16-bit row of [.][QI] tiles (16 B skew per row)
constexpr int NS = N + 8;     // padded 16-bit row of [.][N] tiles
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

// Internal MFMA operands are fp16 (11-bit mantissa, 8x finer than bf16):
// conv outputs, C.B^T, the masked decay matrix, chunk states and passed
// states all stay far inside its range for normalised activations.
typedef _Float16 f16;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;

SSD_DEV uint32_t pk(float a, float b) {
  const f16 lo = (f16)a, hi = (f16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}
SSD_DEV float h2f_lo(uint32_t w) { return (float)__builtin_bit_cast(f16, (uint16_t)(w & 0xffffu)); }
SSD_DEV float h2f_hi(uint32_t w) { return (float)__builtin_bit_cast(f16, (uint16_t)(w >> 16)); }
SSD_DEV void load8h(const f16* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = h2f_lo(w[i]);
    v[2 * i + 1] = h2f_hi(w[i]);
  }
}
SSD_DEV f32x4 mma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

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
                        const Src& s, int ch, const bf16* cin_b, const float* scale, f16* dst,
                        int ld, f16* lo = nullptr, int ldlo = 0) {
  constexpr int R = CONV ? W - 1 : 0;
  uint4 raw[8 + R];
#pragma unroll
  for (int i = 0; i < 8 + R; ++i) {
    const int t = tseq - R + i;
    const bf16* p = (CONV && t < 0 && cin_b) ? cin_b + (int64_t)(W - 1 + t) * s.C + ch
                                             : src + (int64_t)min(max(t, 0), Lm1) * ts;
    raw[i] = *reinterpret_cast<const uint4*>(p);
  }
  uint4 wraw[4];  // 8 channels x 4 taps, bf16, element (j, k) at j*W + k
  float bi[8];
  if (CONV) {
    const uint4* wp = reinterpret_cast<const uint4*>(s.cw + (int64_t)ch * W);
#pragma unroll
    for (int q = 0; q < 4; ++q) wraw[q] = wp[q];
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
        for (int k = 0; k < W; ++k) {
          const int e = j * W + k;  // bf16 element of the 32-element weight block
          const uint32_t wd = (&wraw[e >> 3].x)[(e >> 1) & 3];
          u += __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16)) * win[k][j];
        }
        u = silu(u);
      } else {
        u = win[R][j];
      }
      if (scale) u *= scale[i];
      v[j] = i < nvalid ? u : 0.f;
    }
    if (TRANS) {
      float rem[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f16 hv = (f16)v[j];
        rem[j] = v[j] - (float)hv;
        const uint32_t hbits = (uint32_t)__builtin_bit_cast(uint16_t, hv);
        if (i & 1) pk8[j][i >> 1] |= hbits << 16;
        else pk8[j][i >> 1] = hbits;
      }
      if (lo)  // what fp16 dropped, so hi + lo carries ~22 mantissa bits
        *reinterpret_cast<uint4*>(lo + i * ldlo) = make_uint4(
            pk(rem[0], rem[1]), pk(rem[2], rem[3]), pk(rem[4], rem[5]), pk(rem[6], rem[7]));
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

// 4 tokens x 8 channels of conv+SiLU output (or of the plain input), for
// the transposed x staging of the output kernel: fp16(x) goes to
// dst + j*ld (4 tokens contiguous, 8 bytes per channel row) and x - fp16(x)
// to lo + i*ldlo (8 channels contiguous per token row). Same load pattern as
// conv_stage with half the rows in flight.
template <bool CONV>
SSD_DEV void conv_stage4(const bf16* __restrict__ src, int64_t ts, int tseq, int nvalid, int Lm1,
                         const Src& s, int ch, const bf16* cin_b, f16* dst, int ld, f16* lo,
                         int ldlo) {
  constexpr int R = CONV ? W - 1 : 0;
  uint4 raw[4 + R];
#pragma unroll
  for (int i = 0; i < 4 + R; ++i) {
    const int t = tseq - R + i;
    const bf16* p = (CONV && t < 0 && cin_b) ? cin_b + (int64_t)(W - 1 + t) * s.C + ch
                                             : src + (int64_t)min(max(t, 0), Lm1) * ts;
    raw[i] = *reinterpret_cast<const uint4*>(p);
  }
  uint4 wraw[4];
  float bi[8];
  if (CONV) {
    const uint4* wp = reinterpret_cast<const uint4*>(s.cw + (int64_t)ch * W);
#pragma unroll
    for (int q = 0; q < 4; ++q) wraw[q] = wp[q];
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
  uint32_t pk4[8][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    unpack8(raw[i + R], win[R]);
    float v[8], rem[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float u;
      if (CONV) {
        u = bi[j];
#pragma unroll
        for (int k = 0; k < W; ++k) {
          const int e = j * W + k;
          const uint32_t wd = (&wraw[e >> 3].x)[(e >> 1) & 3];
          u += __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16)) * win[k][j];
        }
        u = silu(u);
      } else {
        u = win[R][j];
      }
      v[j] = i < nvalid ? u : 0.f;
      const f16 hv = (f16)v[j];
      rem[j] = v[j] - (float)hv;
      const uint32_t hbits = (uint32_t)__builtin_bit_cast(uint16_t, hv);
      if (i & 1) pk4[j][i >> 1] |= hbits << 16;
      else pk4[j][i >> 1] = hbits;
    }
    *reinterpret_cast<uint4*>(lo + i * ldlo) =
        make_uint4(pk(rem[0], rem[1]), pk(rem[2], rem[3]), pk(rem[4], rem[5]), pk(rem[6], rem[7]));
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j) win[r][j] = win[r + 1][j];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<uint2*>(dst + j * ld) = make_uint2(pk4[j][0], pk4[j][1]);
}

// Inclusive cumsum of dt*A over the chunk for the HB = 4 heads of the
// workgroup: wave w takes head w, lane l positions 2l and 2l+1.
SSD_DEV void heads_cumsum(const bf16* __restrict__ dt, int64_t row0, int H, int h0, int len,
                          const float* __restrict__ A, float (*lam)[QI], float (*dts)[QI]) {
  const int lane = threadIdx.x & 63, hh = threadIdx.x >> 6;
  const int t = 2 * lane;
  const float r0 = to_f(dt[(row0 + min(t, len - 1)) * H + h0 + hh]);
  const float r1 = to_f(dt[(row0 + min(t + 1, len - 1)) * H + h0 + hh]);
  const float d0 = t < len ? r0 : 0.f, d1 = t + 1 < len ? r1 : 0.f;
  const float Ah = A[h0 + hh];
  const float a0 = d0 * Ah, a1 = d1 * Ah;
  float v = a0 + a1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float n = __shfl_up(v, o, 64);
    if (lane >= o) v += n;
  }
  const float excl = v - (a0 + a1);
  lam[hh][t] = excl + a0;
  lam[hh][t + 1] = excl + a0 + a1;
  dts[hh][t] = d0;
  dts[hh][t + 1] = d1;
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

// ---------------------------------------------------------------- phase 1
// dS_h [P x N] = sum_s x_s w_s (outer) B_s for the 4 heads of the workgroup,
// two heads per pass so the LDS stays under half a CU.
template <bool CONV>
__global__ __launch_bounds__(NT, 2) void k_fstate(Src s, const bf16* __restrict__ dt,
                                               const float* __restrict__ A,
                                               f16* __restrict__ states,
                                               float* __restrict__ lam_end, int L, int H, int G,
                                               int nc) {
  static_assert(RS == N + 8, "dS restaging reuses XT rows");
  __shared__ __align__(16) f16 BT[N * RS];         // [n][s]
  __shared__ __align__(16) f16 XT[2 * P * RS];     // [head of pair][p][s] = x_s[p] w_s
  __shared__ float lam[HB][QI], wv[HB][QI];
  const int c = blockIdx.x, hpb = H / HB;
  const int b = blockIdx.y / hpb, h0 = (blockIdx.y % hpb) * HB, g = h0 / (H / G);
  const int t0 = c * QI, len = min(QI, L - t0);
  const int64_t row0 = (int64_t)b * L + t0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  heads_cumsum(dt, row0, H, h0, len, A, lam, wv);
  {
    const int hh = wave, t = 2 * lane;
    const float lamE = lam[hh][len - 1];
    wv[hh][t] = t < len ? fexp(lamE - lam[hh][t]) * wv[hh][t] : 0.f;
    wv[hh][t + 1] = t + 1 < len ? fexp(lamE - lam[hh][t + 1]) * wv[hh][t + 1] : 0.f;
  }

  const bf16* cin_b = CONV && s.cin ? s.cin + (int64_t)b * (W - 1) * s.C : nullptr;
  const bf16* xb = s.x + (int64_t)b * L * s.xs;
  const bf16* bb = s.b + (int64_t)b * L * s.bs;
  int cv, tbi;
  tmap(tid, cv, tbi);  // 16 channel vectors x 16 token blocks, one per thread
  {
    const int n0 = cv * 8;
    conv_stage<CONV, true>(bb + g * N + n0, s.bs, t0 + tbi * 8, min(8, max(0, len - tbi * 8)),
                           L - 1, s, s.HP + g * N + n0, cin_b, nullptr, BT + n0 * RS + tbi * 8,
                           RS);
  }
  __syncthreads();  // also publishes wv

  const int hx = wave >> 1, pt0 = (wave & 1) * 2;
  const int rr = lane & 15, kk = 8 * (lane >> 4);
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    {
      const int hs = cv >> 3, p0 = (cv & 7) * 8, hh = 2 * pass + hs;
      const int ch = (h0 + hh) * P + p0;
      conv_stage<CONV, true>(xb + ch, s.xs, t0 + tbi * 8, min(8, max(0, len - tbi * 8)), L - 1,
                             s, ch, cin_b, &wv[hh][tbi * 8], XT + (hs * P + p0) * RS + tbi * 8,
                             RS);
    }
    __syncthreads();
    // wave w: head w/2 of the pair, p-tiles 2(w%2), 2(w%2)+1, all 8 n-tiles
    f32x4 acc[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int n = 0; n < 8; ++n) acc[i][n] = zero4();
    const f16* a0p = XT + (hx * P + pt0 * 16 + rr) * RS + kk;
    const f16* a1p = a0p + 16 * RS;
    const f16* bp = BT + rr * RS + kk;
#pragma unroll
    for (int k = 0; k < QI; k += 32) {
      const f16x8 a0 = *reinterpret_cast<const f16x8*>(a0p + k);
      const f16x8 a1 = *reinterpret_cast<const f16x8*>(a1p + k);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const f16x8 bf = *reinterpret_cast<const f16x8*>(bp + n * 16 * RS + k);
        acc[0][n] = mma16(a0, bf, acc[0][n]);
        acc[1][n] = mma16(a1, bf, acc[1][n]);
      }
    }
    __syncthreads();  // XT reads done: restage dS there as fp16 [head][p][n]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int p = (pt0 + i) * 16 + 4 * (lane >> 4) + r, nn = n * 16 + rr;
          XT[(hx * P + p) * RS + nn] = (f16)acc[i][n][r];
        }
    __syncthreads();
    f16* out = states + (((int64_t)b * nc + c) * H + h0 + 2 * pass) * (int64_t)(P * N);
    for (int i = tid; i < 2 * P * (N / 8); i += NT) {
      const int row = i / (N / 8), v8 = i % (N / 8);  // row = head of pair * P + p
      *reinterpret_cast<uint4*>(out + (int64_t)row * N + v8 * 8) =
          *reinterpret_cast<const uint4*>(XT + row * RS + v8 * 8);
    }
    __syncthreads();  // restaged rows read before the next pair overwrites XT
  }
  if (tid < HB) lam_end[((int64_t)b * H + h0 + tid) * nc + c] = lam[tid][len - 1];
}

// ---------------------------------------------------------------- phase 2
constexpr int kPassDepth = 8;
__global__ __launch_bounds__(256) void k_fpass(const f16* __restrict__ dS,
                                               const float* __restrict__ lam_end,
                                               const float* s_in, float* s_out,
                                               f16* __restrict__ sin_h, int H, int nc) {
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
        const uint2 raw = *reinterpret_cast<const uint2*>(dS + (((int64_t)b * nc + c) * H + h) * PN + e);
        d[u] = make_float4(h2f_lo(raw.x), h2f_hi(raw.x), h2f_lo(raw.y), h2f_hi(raw.y));
        al[u] = fexp(lam_end[bh * nc + c]);
      }
    }
#pragma unroll
    for (int u = 0; u < kPassDepth; ++u) {
      const int c = c0 + u;
      if (c < nc) {
        uint2 o = make_uint2(pk(S.x, S.y), pk(S.z, S.w));
        *reinterpret_cast<uint2*>(sin_h + (((int64_t)b * nc + c) * H + h) * PN + e) = o;
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
// NORM: fuse the gated RMSNorm (the 4 heads are one norm group); else the
// scan output y is written (bf16).
//
// Wave w owns row tiles w and 7-w of the chunk (equal causal work) for all 4
// heads. It keeps in registers the C.B^T tiles of its rows (computed as
// (B C^T) tiles, whose MFMA output layout is exactly the A-operand layout of
// the next product once that product's 32 k-slots are mapped to the
// sequence positions 4q..4q+3 and 16+4q..16+4q+3 of its two 16-column
// tiles) and its C fragments, so after the first phase the LDS only holds
// x: fp16(x) transposed for the MFMA, plus the part fp16 drops (XL) so D x
// is taken at ~22-bit mantissa precision. Heads go in two passes of 2; the
// wave's y values stay in registers (fp16) until both passes are done, then
// go through an LDS tile to a coalesced epilogue that gates with z,
// normalises each row over its 256 channels and stores 16-byte vectors.
constexpr int XLS = 2 * P + 8;  // padded row of the [t][2 heads x P] low part
template <bool CONV, bool NORM>
__global__ __launch_bounds__(NT, 2) void k_fout(Src s, const bf16* __restrict__ dt,
                                                const float* __restrict__ A,
                                                const float* __restrict__ D,
                                                const f16* __restrict__ sin_h,
                                                const bf16* __restrict__ z,
                                                const bf16* __restrict__ nw, float eps,
                                                bf16* __restrict__ out, int L, int H, int G,
                                                int nc) {
  static_assert(2 * P * RS == QI * NS && QI * XLS == QI * NS, "x hi/lo reuse the B/C space");
  static_assert(QI * OS <= 2 * QI * NS, "output tile must fit");
  __shared__ __align__(16) f16 U[2 * QI * NS];  // Bs | Cs, then XT | XL per head pair, then Ot
  __shared__ float lam[HB][QI], dts[HB][QI];
  f16* Bs = U;
  f16* Cs = U + QI * NS;
  f16* XT = U;                // [head of pair][p][s]: fp16(x)
  f16* XL = U + 2 * P * RS;   // [t][head of pair x p]: x - fp16(x)
  f16* Ot = U;                // [t][4 heads x p]: y

  const int c = blockIdx.x, hpb = H / HB;
  const int b = blockIdx.y / hpb, h0 = (blockIdx.y % hpb) * HB, g = h0 / (H / G);
  const int t0 = c * QI, len = min(QI, L - t0);
  const int64_t row0 = (int64_t)b * L + t0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rr = lane & 15, q4 = lane >> 4, kk = 8 * q4, r4 = 4 * q4;
  const int HP = s.HP;

  heads_cumsum(dt, row0, H, h0, len, A, lam, dts);

  const bf16* cin_b = CONV && s.cin ? s.cin + (int64_t)b * (W - 1) * s.C : nullptr;
  // B and C, natural layout [t][n]: 16 channel vectors x 16 token blocks each.
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int i = tid, cv = i & 15, tbi = i >> 4, n0 = cv * 8;
    const bf16* base = (half ? s.c : s.b) + (int64_t)b * L * s.bs + g * N + n0;
    const int ch = s.HP + (half ? s.GN : 0) + g * N + n0;
    conv_stage<CONV, false>(base, s.bs, t0 + tbi * 8, min(8, max(0, len - tbi * 8)), L - 1, s, ch,
                            cin_b, nullptr, (half ? Cs : Bs) + (tbi * 8) * NS + n0, NS);
  }
  __syncthreads();

  const int rta = wave, rtb = 7 - wave;
  // (B C^T) tiles j <= rt of the wave's two row tiles: lane holds C_t.B_s for
  // t = 16 rt + rr and s = 16 j + 4 q4 + r (fp16, the MFMA operand precision).
  uint2 Ga[4], Gb[8];
  f16x8 Cfa[4], Cfb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    Cfa[ks] = *reinterpret_cast<const f16x8*>(Cs + (rta * 16 + rr) * NS + ks * 32 + kk);
    Cfb[ks] = *reinterpret_cast<const f16x8*>(Cs + (rtb * 16 + rr) * NS + ks * 32 + kk);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    f32x4 ga = zero4(), gb = zero4();
    const f16* bp = Bs + (j * 16 + rr) * NS + kk;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f16x8 bf = *reinterpret_cast<const f16x8*>(bp + ks * 32);
      if (j < 4 && j <= rta) ga = mma16(bf, Cfa[ks], ga);
      if (j <= rtb) gb = mma16(bf, Cfb[ks], gb);
    }
    if (j < 4) Ga[j] = make_uint2(pk(ga[0], ga[1]), pk(ga[2], ga[3]));
    Gb[j] = make_uint2(pk(gb[0], gb[1]), pk(gb[2], gb[3]));
  }
  // y starts as the inter-chunk term exp(Lam_t) C_t S_in^T for all 4 heads,
  // kept as fp16 pairs: [row tile][head][p tile][rows r4+0,1 | r4+2,3].
  uint32_t yk[2][4][4][2];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    const f16* sp = sin_h + (((int64_t)b * nc + c) * H + h0 + hh) * (int64_t)(P * N);
    f32x4 acc2a[4], acc2b[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) { acc2a[pt] = zero4(); acc2b[pt] = zero4(); }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const f16x8 sf = *reinterpret_cast<const f16x8*>(sp + (pt * 16 + rr) * N + ks * 32 + kk);
        acc2a[pt] = mma16(Cfa[ks], sf, acc2a[pt]);
        acc2b[pt] = mma16(Cfb[ks], sf, acc2b[pt]);
      }
    }
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int rt = ui == 0 ? rta : rtb;
      float el[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) el[r] = fexp(lam[hh][rt * 16 + r4 + r]);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const f32x4 a2 = ui == 0 ? acc2a[pt] : acc2b[pt];
        yk[ui][hh][pt][0] = pk(el[0] * a2[0], el[1] * a2[1]);
        yk[ui][hh][pt][1] = pk(el[2] * a2[2], el[3] * a2[3]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // one head's S_in fragments in flight at a time
  }
  __syncthreads();  // B and C no longer read from LDS

  const bf16* xb = s.x + (int64_t)b * L * s.xs;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    // x of heads 2*pass, 2*pass+1: 16 channel vectors x 32 blocks of 4 tokens;
    // within 32 lanes, 2 vectors x 16 blocks hit distinct LDS banks.
#pragma unroll 1
    for (int i = tid; i < 512; i += NT) {
      const int tb = (i >> 1) & 31, cv = (i & 1) | ((i >> 6) << 1);
      const int hs = cv >> 3, p0 = (cv & 7) * 8;
      const int ch = (h0 + 2 * pass + hs) * P + p0;
      conv_stage4<CONV>(xb + ch, s.xs, t0 + tb * 4, min(4, max(0, len - tb * 4)), L - 1, s, ch,
                        cin_b, XT + (hs * P + p0) * RS + tb * 4, RS,
                        XL + (tb * 4) * XLS + hs * P + p0, XLS);
    }
    __syncthreads();
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int hh = 2 * pass + hi;
      const float Dh = D ? D[h0 + hh] : 0.f;
#pragma unroll
      for (int ui = 0; ui < 2; ++ui) {
        const int rt = ui == 0 ? rta : rtb;
        const int trow = rt * 16 + rr;  // A-operand row
        const float lt = lam[hh][trow];
        f32x4 acc[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          if (2 * ks <= rt) {
            // k-slots 8 q4 + r <-> s = 32 ks + 4 q4 + r, 8 q4 + 4 + r <-> s + 16
            const int s0 = ks * 32 + r4;
            const float4 l0 = *reinterpret_cast<const float4*>(&lam[hh][s0]);
            const float4 l1 = *reinterpret_cast<const float4*>(&lam[hh][s0 + 16]);
            const float4 d0 = *reinterpret_cast<const float4*>(&dts[hh][s0]);
            const float4 d1 = *reinterpret_cast<const float4*>(&dts[hh][s0 + 16]);
            const float ls[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
            const float ds[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
            uint2 g0, g1;
            if (ui == 0) {
              g0 = Ga[(2 * ks) & 3];
              g1 = (2 * ks + 1 <= rt) ? Ga[(2 * ks + 1) & 3] : make_uint2(0u, 0u);
            } else {
              g0 = Gb[2 * ks];
              g1 = (2 * ks + 1 <= rt) ? Gb[2 * ks + 1] : make_uint2(0u, 0u);
            }
            const float gv[8] = {h2f_lo(g0.x), h2f_hi(g0.x), h2f_lo(g0.y), h2f_hi(g0.y),
                                 h2f_lo(g1.x), h2f_hi(g1.x), h2f_lo(g1.y), h2f_hi(g1.y)};
            f16x8 af;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int sj = s0 + (j & 3) + (j >> 2) * 16;
              const float m = gv[j] * fexp(fminf(lt - ls[j], 0.f)) * ds[j];
              af[j] = (f16)(sj <= trow ? m : 0.f);
            }
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
              const f16* xr = XT + (hi * P + pt * 16 + rr) * RS + s0;
              const uint2 lo = *reinterpret_cast<const uint2*>(xr);
              const uint2 hi2 = *reinterpret_cast<const uint2*>(xr + 16);
              const uint4 u = make_uint4(lo.x, lo.y, hi2.x, hi2.y);
              acc[pt] = mma16(af, __builtin_bit_cast(f16x8, u), acc[pt]);
            }
          }
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          float yv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = rt * 16 + r4 + r;
            const int p = pt * 16 + rr;
            const float xv = (float)XT[(hi * P + p) * RS + t] + (float)XL[t * XLS + hi * P + p];
            yv[r] = acc[pt][r] + Dh * xv;
          }
          // add to the inter-chunk term; register indices stay static under
          // the runtime pass loop
          uint32_t* w2 = pass == 0 ? yk[ui][hi][pt] : yk[ui][2 + hi][pt];
          const float o0 = h2f_lo(w2[0]), o1 = h2f_hi(w2[0]);
          const float o2 = h2f_lo(w2[1]), o3 = h2f_hi(w2[1]);
          const uint32_t p01 = pk(yv[0] + o0, yv[1] + o1), p23 = pk(yv[2] + o2, yv[3] + o3);
          if (pass == 0) {
            yk[ui][hi][pt][0] = p01;
            yk[ui][hi][pt][1] = p23;
          } else {
            yk[ui][2 + hi][pt][0] = p01;
            yk[ui][2 + hi][pt][1] = p23;
          }
        }
      }
    }
    __syncthreads();  // XT/XL of this pair no longer read (and Ot may follow)
  }

  // y -> Ot [t][4 heads x P]
#pragma unroll
  for (int ui = 0; ui < 2; ++ui) {
    const int rt = ui == 0 ? rta : rtb;
#pragma unroll
    for (int hh = 0; hh < HB; ++hh)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t w2 = yk[ui][hh][pt][r >> 1];
          const uint16_t bits = (r & 1) ? (uint16_t)(w2 >> 16) : (uint16_t)(w2 & 0xffffu);
          Ot[(rt * 16 + r4 + r) * OS + hh * P + pt * 16 + rr] = __builtin_bit_cast(f16, bits);
        }
  }
  __syncthreads();

  // Epilogue: 32 consecutive threads take one row (8 channels each).
  for (int i = tid; i < QI * (HB * P / 8); i += NT) {
    const int t = i >> 5, v8 = i & 31;
    const bool ok = t < len;
    const int64_t go = (row0 + min(t, len - 1)) * HP + h0 * P + v8 * 8;
    float yv[8];
    load8h(Ot + t * OS + v8 * 8, yv);
    if (NORM) {
      float zv[8], wv8[8];
      load8(z + go, zv);
      load8(nw + h0 * P + v8 * 8, wv8);
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        yv[j] *= silu(zv[j]);
        ss += yv[j] * yv[j];
      }
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) ss += __shfl_xor(ss, o, 64);
      const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / (HB * P)) + eps);
#pragma unroll
      for (int j = 0; j < 8; ++j) yv[j] *= wv8[j] * inv;
    }
    if (ok) store8(out + go, yv);
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
  return (size_t)B * nc * H * PN * (2 + 2) + (size_t)B * H * nc * 4 + 3 * 256;
}

hipError_t launch_fast_scan(const FastScanArgs& a, hipStream_t st) {
  using namespace fast;
  const int nc = (a.L + QI - 1) / QI;
  const size_t PN = P * N;
  unsigned char* w = (unsigned char*)a.ws;
  fast::f16* dS = (fast::f16*)w;
  w += ((size_t)a.B * nc * a.H * PN * 2 + 255) / 256 * 256;
  fast::f16* sinb = (fast::f16*)w;
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
  {
  ProfScope ps(st, KID_FAST_STATE);
  if (a.conv)
    hipLaunchKernelGGL(k_fstate<true>, g1, dim3(NT), 0, st, s, (const bf16*)a.dt, a.A, dS,
                       lam_end, a.L, a.H, a.G, nc);
  else
    hipLaunchKernelGGL(k_fstate<false>, g1, dim3(NT), 0, st, s, (const bf16*)a.dt, a.A, dS,
                       lam_end, a.L, a.H, a.G, nc);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
  ProfScope ps(st, KID_FAST_PASS);
  hipLaunchKernelGGL(k_fpass, dim3(PN / 1024, a.H, a.B), dim3(256), 0, st, dS, lam_end, a.s_in,
                     a.s_out, sinb, a.H, nc);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // fused norm when a norm group is exactly the 4-head block; otherwise y
  // (bf16) goes to the output and the grouped norm runs on it in place.
  const bool fused = a.z && (a.H / a.G) == HB;
#define SSD_FOUT(CV, NM)                                                                         \
  hipLaunchKernelGGL((k_fout<CV, NM>), g1, dim3(NT), 0, st, s, (const bf16*)a.dt, a.A, a.D,      \
                     sinb, (const bf16*)a.z, (const bf16*)a.norm_w, a.eps, (bf16*)a.y, a.L, a.H, \
                     a.G, nc)
  {
  ProfScope ps(st, KID_FAST_OUT);
  if (a.conv) {
    if (fused) SSD_FOUT(true, true);
    else SSD_FOUT(true, false);
  } else {
    if (fused) SSD_FOUT(false, true);
    else SSD_FOUT(false, false);
  }
  }
#undef SSD_FOUT
  e = hipGetLastError();
  if (e != hipSuccess || !a.z || fused) return e;
  return launch_gated_norm(true, false, a.B * a.L, a.H * P, a.G, a.y, a.z, a.norm_w, a.eps, a.y,
                           st);
}

}  // namespace ssd
