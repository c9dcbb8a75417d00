// Fast path of the chunked SSD scan for the Mamba-2 layer shape of the
// Nemotron-H models (head_dim 64, d_state 128; "NemotronH-0.3B-A0.3B" card,
// "Configuration Changes": mamba_head_dim 64, n_groups 8), bf16 I/O, with
// the causal conv + SiLU recomputed inside the consumers so the conv output
// never goes to HBM.
//
// Same block decomposition as the generic kernels ("feat(model): add
// Nemotron-3 Nano hybrid ..." attribution commit: ssd_minimal_discrete /
// segsum), blocked in 128-token chunks. Three launches:
//   1. k_fstate  (chunk, batch x group): conv+SiLU of B once and of x per
//      head, dS_h = (x w_h)^T B for every head of the group on fp16 MFMA,
//      written fp16; when a group spans several 4-head blocks it also
//      writes the convolved B and C rows (fp16) for step 3.
//   2. k_fpass   state passing along chunks in fp32; S_in(k) written as fp16
//      (the precision the MFMA consumes), final state fp32.
//   3. k_fout    (chunk, batch x 4-head block): conv+SiLU of x, B, C (B and
//      C read convolved when step 1 wrote them); the causal C B^T computed
//      once and shared by the 4 heads; per head
//      y = M' x + exp(Lam_t) C S_in^T + D x with M'[t,s] = (C_t.B_s)
//      exp(Lam_t - Lam_s) dt_s on fp16 MFMA and D x on the same fp16 x tile
//      (D as an fp16 hi + lo pair); then the gated
//      RMSNorm, within the block when the 4 heads are one norm group, else
//      across the group's blocks (per-token sums of q^2 exchanged through
//      device memory); coalesced stores.
#include "common.hpp"
#include "launch.hpp"

namespace ssd {
namespace fast {

constexpr int P = 64, N = 128, QI = 128, HB = 4, W = 4;
constexpr int NT = 256;       // threads per workgroup (4 waves): two workgroups fit a CU
// LDS row pitches in 16-bit elements. [.][QI] tiles (x, B^T) are read 8
// bytes per lane by 16 consecutive rows: a pitch of 2 mod 32 banks keeps those
// reads (and the 8-byte transposed writes) free of bank conflicts, at the
// price of 8-byte (not 16-byte) row alignment, so every access to them is at
// most 8 bytes wide. [.][N] tiles are read 16 bytes per lane by 8 rows:
// a pitch of 4 mod 32 banks, 16-byte aligned. The output tile [t][4 heads x
// P] is written 8 bytes per lane by 16 rows: 2 mod 32 banks.
constexpr int RS = QI + 4;
constexpr int NS = N + 8;
constexpr int OS = HB * P + 4;

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
  int64_t zs;         // token stride of z (elements)
  DtA dta;            // dt's token stride; raw dt + bias and A_log, or dt and A as given
  Seqs q;             // ragged sequences over a state pool, or a dense batch (q.cu null)
};

// Where one chunk of one sequence lies. Dense batch: chunk c of sequence b,
// all of length L. Ragged: global chunk c of the call's chunk table, whose
// sequence, length and state slot come from the table. False for a chunk
// no sequence owns (the table is padded) or when the table is invalid.
struct ChunkGeo {
  int64_t tok0;     // global token row of the sequence's token 0
  int64_t kg;       // global chunk index: storage of dS / S_in / Lam_end
  int L, t0, len;   // sequence length, chunk start within it, tokens in the chunk
  const bf16* cin;  // the sequence's conv state rows, or null (zeros)
};
SSD_DEV bool chunk_geo(const Src& s, int c, int b, int L, int nc, ChunkGeo& g) {
  if (!s.q.cu) {
    g.tok0 = (int64_t)b * L;
    g.kg = (int64_t)b * nc + c;
    g.L = L;
    g.t0 = c * QI;
    g.len = min(QI, L - g.t0);
    g.cin = s.cin ? s.cin + (int64_t)b * (W - 1) * s.C : nullptr;
    return true;
  }
  if (__builtin_amdgcn_readfirstlane(*s.q.valid) != 1) return false;
  const int seq = __builtin_amdgcn_readfirstlane(s.q.chunk_seq[c]);
  if (seq < 0) return false;
  const int a = s.q.cu[seq];
  g.tok0 = a;
  g.kg = c;
  g.L = s.q.cu[seq + 1] - a;
  g.t0 = (c - s.q.chunk_first[seq]) * QI;
  g.len = min(QI, g.L - g.t0);
  const bool resume = !s.q.has_state || s.q.has_state[seq];
  g.cin = resume ? (const bf16*)s.q.conv_pool + (int64_t)s.q.slots[seq] * (W - 1) * s.C : nullptr;
  return true;
}

// Internal MFMA operands are fp16 (11-bit mantissa, 8x finer than bf16):
// conv outputs, C.B^T, the masked decay matrix, chunk states and passed
// states all stay far inside its range for normalised activations.
typedef _Float16 f16;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
// Native 4 x 32-bit vector: arrays of it stay in registers (arrays of the
// HIP uint4 struct can end up in scratch memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// two fp32 -> one word of two fp16 (round to nearest even; a in the low half)
SSD_DEV f16x2 cvt2(float a, float b) { return __builtin_convertvector(f32x2{a, b}, f16x2); }
SSD_DEV uint32_t pk(float a, float b) { return __builtin_bit_cast(uint32_t, cvt2(a, b)); }
SSD_DEV float h2f_lo(uint32_t w) { return (float)__builtin_bit_cast(f16, (uint16_t)(w & 0xffffu)); }
SSD_DEV float h2f_hi(uint32_t w) { return (float)__builtin_bit_cast(f16, (uint16_t)(w >> 16)); }
// 16 bytes from an 8-byte aligned LDS address, as two 8-byte accesses
SSD_DEV f16x8 lds16(const f16* p) {
  const uint2 a = *reinterpret_cast<const uint2*>(p);
  const uint2 b = *reinterpret_cast<const uint2*>(p + 4);
  return __builtin_bit_cast(f16x8, make_uint4(a.x, a.y, b.x, b.y));
}
SSD_DEV void sts16(f16* p, const u32x4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(v[0], v[1]);
  *reinterpret_cast<uint2*>(p + 4) = make_uint2(v[2], v[3]);
}
// 8 fp16 (four pairs) to fp32
SSD_DEV void unpack8h(const u32x4 u, float (&v)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = h2f_lo(w[i]);
    v[2 * i + 1] = h2f_hi(w[i]);
  }
}
SSD_DEV void load8h(const f16* p, float (&v)[8]) {
  const uint2 a = *reinterpret_cast<const uint2*>(p);
  const uint2 b = *reinterpret_cast<const uint2*>(p + 4);
  unpack8h(u32x4{a.x, a.y, b.x, b.y}, v);
}
// An empty asm that takes the values in registers: the computation of x
// cannot be sunk past this point.
SSD_DEV void pin(uint32_t (&x)[2]) { asm volatile("" : "+v"(x[0]), "+v"(x[1])); }
SSD_DEV f32x4 mma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Unpack 8 bf16 (one 16-byte row segment) to fp32.
SSD_DEV void unpack8(const u32x4 u, float (&v)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// ---- causal conv + SiLU of a tile of T tokens x 8 channels ----------------
// raw[r] holds the 8 bf16 channels of token tseq - R + r (R = W - 1 halo rows
// when CONV). For channel j, the bf16 pair (token r, token r + 1) is built
// with one byte permute and the 4-tap window is two bf16 dot products with
// fp32 accumulation against the weight pairs (w0, w1) and (w2, w3):
// u_i = bias + (x_{i-3}, x_{i-2}).(w0, w1) + (x_{i-1}, x_i).(w2, w3).
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
SSD_DEV float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a),
                                        __builtin_bit_cast(bf16x2v, b), c, false);
}
template <int J>
SSD_DEV uint32_t chan_pair(const u32x4 r0, const u32x4 r1) {
  // low halves (J even) or high halves (J odd) of word J/2 of two rows
  return __builtin_amdgcn_perm(r1[J >> 1], r0[J >> 1], (J & 1) ? 0x07060302u : 0x05040100u);
}
template <int J, int T>
SSD_DEV void conv_chan(const u32x4 (&raw)[T + W - 1], const u32x4 (&wraw)[4], float bias,
                       float (&v)[T][8]) {
  const uint32_t w01 = wraw[J >> 1][(J & 1) * 2], w23 = wraw[J >> 1][(J & 1) * 2 + 1];
  uint32_t pr[T + 2];
#pragma unroll
  for (int r = 0; r < T + 2; ++r) pr[r] = chan_pair<J>(raw[r], raw[r + 1]);
#pragma unroll
  for (int i = 0; i < T; ++i) v[i][J] = silu(dot2bf(pr[i], w01, dot2bf(pr[i + 2], w23, bias)));
}
// Conv weights (8 channels x 4 taps, bf16, element (j, k) at j*W + k) and
// bias (8 bf16, zero without one) of one 8-channel vector. Loaded by the
// caller ahead of the rows they are applied to, so that waiting for those
// rows also covers them and never drains later loads or stores.
template <bool CONV>
struct ConvW {
  u32x4 w[4];
  u32x4 b;
};
template <>
struct ConvW<false> {};
template <bool CONV>
SSD_DEV void convw_load(ConvW<CONV>& cw, const Src& s, int ch) {
  if constexpr (CONV) {
    static_assert(W == 4, "two bf16 pairs per window");
    const u32x4* wp = reinterpret_cast<const u32x4*>(s.cw + (int64_t)ch * W);
#pragma unroll
    for (int q = 0; q < 4; ++q) cw.w[q] = wp[q];
    cw.b = s.cbias ? *reinterpret_cast<const u32x4*>(s.cbias + ch) : u32x4{0u, 0u, 0u, 0u};
  }
}
template <bool CONV, int T>
SSD_DEV void conv_tile(const u32x4 (&raw)[T + (CONV ? W - 1 : 0)], const ConvW<CONV>& cw,
                       float (&v)[T][8]) {
  if constexpr (CONV) {
    const u32x4(&wraw)[4] = cw.w;
    float bi[8];
    unpack8(cw.b, bi);
    conv_chan<0, T>(raw, wraw, bi[0], v);
    conv_chan<1, T>(raw, wraw, bi[1], v);
    conv_chan<2, T>(raw, wraw, bi[2], v);
    conv_chan<3, T>(raw, wraw, bi[3], v);
    conv_chan<4, T>(raw, wraw, bi[4], v);
    conv_chan<5, T>(raw, wraw, bi[5], v);
    conv_chan<6, T>(raw, wraw, bi[6], v);
    conv_chan<7, T>(raw, wraw, bi[7], v);
  } else {
#pragma unroll
    for (int i = 0; i < T; ++i) unpack8(raw[i], v[i]);
  }
}

// silu of the 8 bf16 conv biases of one channel vector
SSD_DEV void bias_silu8(const u32x4 b, float (&o)[8]) {
  unpack8(b, o);
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = silu(o[j]);
}

// Load the T (+ halo) rows of one 8-channel vector: every row load is issued
// before any is used; addresses are clamped into the sequence (the conv
// state supplies rows before token 0 when present, else they are zeroed by
// rows_mask_head), so the loads are not serialised behind per-lane branches.
// NTL: streaming loads, for rows no later kernel reads again
template <bool CONV, int T, bool NTL = false>
SSD_DEV void rows_load(u32x4 (&raw)[T + (CONV ? W - 1 : 0)], const bf16* __restrict__ src,
                       int64_t ts, int tseq, int Lm1, const Src& s, int ch, const bf16* cin_b) {
  constexpr int R = CONV ? W - 1 : 0;
#pragma unroll
  for (int i = 0; i < T + R; ++i) {
    const int t = tseq - R + i;
    const bf16* p = (CONV && t < 0 && cin_b) ? cin_b + (int64_t)(W - 1 + t) * s.C + ch
                                             : src + (int64_t)min(max(t, 0), Lm1) * ts;
    if constexpr (NTL)
      raw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else
      raw[i] = *reinterpret_cast<const u32x4*>(p);
  }
}
template <bool CONV, int T>
SSD_DEV void rows_mask_head(u32x4 (&raw)[T + (CONV ? W - 1 : 0)], int tseq, const bf16* cin_b) {
  if constexpr (CONV) {
    if (tseq < W - 1 && !cin_b) {  // only the first rows of a sequence
#pragma unroll
      for (int i = 0; i < W - 1; ++i)
        if (tseq - (W - 1) + i < 0) raw[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Stage 8 tokens x 8 channels of conv+SiLU output (or of the plain input
// when !CONV) into LDS as fp16: TRANS=false writes row i (token) at
// dst + i*ld as one 16-byte vector; TRANS=true writes row j (channel) at
// dst + j*ld with the 8 tokens contiguous. Rows past nvalid are zero. With
// gdst, rows i < nvalid also go to global memory at gdst + i*gld (16 bytes
// each); without dst, only there.
// src: the channel vector's element at token 0 of this batch; tseq: sequence
// position of the first token; Lm1: last token of the sequence; ch: absolute
// xBC channel (conv weights); cin_b: conv state of this batch or null.
// OFS handles the shared channel offsets of B and C (see the state split
// below), with off = silu(offb) and dw = silu(dwb) from 8 packed bf16 conv
// biases: kOfsSub stores v - off; kOfsDot also gives, per token i, dot[i] =
// v_i . dw on the fp32 values. The subtraction is done as the values are
// packed (a separate pass over the tile costs registers). Rows past nvalid
// are stored as zero and their dots are zero.
template <bool CONV>
using Rows8 = u32x4[8 + (CONV ? W - 1 : 0)];
constexpr int kOfsNone = 0, kOfsDot = 1, kOfsSub = 2;
template <bool CONV, bool TRANS, int OFS = kOfsNone>
SSD_DEV void conv_store(Rows8<CONV>& raw, const ConvW<CONV>& cw, int tseq, int nvalid,
                        const bf16* cin_b, f16* dst, int ld, f16* gdst = nullptr,
                        int64_t gld = 0, u32x4 offb = {}, u32x4 dwb = {},
                        float* dot = nullptr) {
  rows_mask_head<CONV, 8>(raw, tseq, cin_b);
  float v[8][8];
  conv_tile<CONV, 8>(raw, cw, v);
  float off[8] = {};
  if constexpr (OFS != kOfsNone) {
    bias_silu8(offb, off);
    if constexpr (OFS == kOfsDot) {
      float dw[8];
      bias_silu8(dwb, dw);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) d = fmaf(v[i][j], dw[j], d);
        dot[i] = i < nvalid ? d : 0.f;
      }
    }
  }
  if (nvalid < 8) {  // only the tail of a sequence (its stored rows are 0)
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = i < nvalid ? v[i][j] : off[j];
  }
  // token row i less the offsets, as fp16
  auto row = [&](int i) {
    return u32x4{pk(v[i][0] - off[0], v[i][1] - off[1]), pk(v[i][2] - off[2], v[i][3] - off[3]),
                 pk(v[i][4] - off[4], v[i][5] - off[5]), pk(v[i][6] - off[6], v[i][7] - off[7])};
  };
  if (gdst) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < nvalid) *reinterpret_cast<u32x4*>(gdst + i * gld) = row(i);
  }
  if (!dst) return;
  if (TRANS) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float o = off[j];
      sts16(dst + j * ld, u32x4{pk(v[0][j] - o, v[1][j] - o), pk(v[2][j] - o, v[3][j] - o),
                                pk(v[4][j] - o, v[5][j] - o), pk(v[6][j] - o, v[7][j] - o)});
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(dst + i * ld) = row(i);
  }
}
// The same for 4 of the tokens, natural layout, to global memory only (rows
// i < nvalid at gdst + i * gld): half the live tile of the 8-token form.
// raw: the 4 (+ halo) rows of tokens tseq .. tseq + 3.
template <bool CONV, int OFS>
SSD_DEV void conv_store4(const u32x4* raw_p, const ConvW<CONV>& cw, int tseq, int nvalid,
                         const bf16* cin_b, f16* gdst, int64_t gld, u32x4 offb = {},
                         u32x4 dwb = {}, float* dot = nullptr) {
  constexpr int R = 4 + (CONV ? W - 1 : 0);
  u32x4 raw[R];
#pragma unroll
  for (int i = 0; i < R; ++i) raw[i] = raw_p[i];
  rows_mask_head<CONV, 4>(raw, tseq, cin_b);
  float v[4][8];
  conv_tile<CONV, 4>(raw, cw, v);
  float off[8] = {};
  if constexpr (OFS != kOfsNone) {
    bias_silu8(offb, off);
    if constexpr (OFS == kOfsDot) {
      float dw[8];
      bias_silu8(dwb, dw);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) d = fmaf(v[i][j], dw[j], d);
        dot[i] = i < nvalid ? d : 0.f;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < nvalid)
      *reinterpret_cast<u32x4*>(gdst + i * gld) =
          u32x4{pk(v[i][0] - off[0], v[i][1] - off[1]), pk(v[i][2] - off[2], v[i][3] - off[3]),
                pk(v[i][4] - off[4], v[i][5] - off[5]), pk(v[i][6] - off[6], v[i][7] - off[7])};
}

// Raw rows of one x staging item: 4 tokens (+ W-1 halo when CONV) of one
// 8-channel vector, loaded ahead of their use.
template <bool CONV>
struct XRaw {
  u32x4 v[4 + (CONV ? W - 1 : 0)];
};

template <bool CONV, bool NTL = false>
SSD_DEV void x_load(XRaw<CONV>& r, const bf16* __restrict__ src, int64_t ts, int tseq, int Lm1,
                    const Src& s, int ch, const bf16* cin_b) {
  rows_load<CONV, 4, NTL>(r.v, src, ts, tseq, Lm1, s, ch, cin_b);
}

// conv + SiLU (or the plain input) of a loaded item, times scale[i] for
// token i when scale is non-null; fp16(x) goes to hi + j*ld and, when LO,
// x - fp16(x) to lo + j*ld (channel row j, the 4 tokens contiguous: the
// MFMA operand layout [p][s]). Rows past nvalid are zero.
template <bool CONV, bool LO>
SSD_DEV void x_store(XRaw<CONV>& r, const ConvW<CONV>& cw, int tseq, int nvalid,
                     const bf16* cin_b, const float* scale, f16* hi, f16* lo, int ld) {
  rows_mask_head<CONV, 4>(r.v, tseq, cin_b);
  float v[4][8];
  conv_tile<CONV, 4>(r.v, cw, v);
  if (scale) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] *= scale[i];
  }
  if (nvalid < 4) {  // only the tail of a sequence
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = i < nvalid ? v[i][j] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const f16x2 h01 = cvt2(v[0][j], v[1][j]), h23 = cvt2(v[2][j], v[3][j]);
    *reinterpret_cast<uint2*>(hi + j * ld) =
        make_uint2(__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23));
    if (LO)
      *reinterpret_cast<uint2*>(lo + j * ld) =
          make_uint2(pk(v[0][j] - (float)h01[0], v[1][j] - (float)h01[1]),
                     pk(v[2][j] - (float)h23[0], v[3][j] - (float)h23[1]));
  }
}

// ---- the state split ------------------------------------------------------
// With a conv bias, the convolved B and C rows share per-channel offsets
// bbar = silu(b_B) and cbar = silu(b_C), much larger than their variation,
// and x has one too, so the state grows a large rank-one part along bbar
// while C_t . bbar can be far smaller than |C_t| |bbar|: rounding S or C to
// the fp16 operand precision would cost most of the bits of C_t . S. The
// kernels therefore carry S = S' + a bbar^T (the same matrix, split):
//   chunk state   dS' = sum_s x_s w_s (B_s - bbar)^T on the MFMA, and the
//                 fp32 row sums da = sum_s x_s w_s (a ones-row MFMA on the
//                 same fp16 operand);
//   state pass    S' and a in fp32 (the carried-in state split by projecting
//                 its rows on bbar), S'_in in fp16 plus, per row p, a_in and
//                 sc'_in = S'_in . cbar in fp32; the final state S' + a bbar^T;
//   output        C_t . S_in = (C_t - cbar) . S'_in + sc'_in + a_in u_t with
//                 u_t = C_t . bbar in fp32 from the fp32 conv output, and
//                 C_t . B_s = (C_t - cbar) . (B_s - bbar) + u_t + v_s with
//                 v_s = cbar . (B_s - bbar).
// Only the fp16 operands change: S', B - bbar and C - cbar are small, and
// everything that cancels is summed in fp32. Without a bias nothing is split.
// Per (chunk, head) the split keeps kAux x P floats: da, a_in, sc'_in.
constexpr int kAux = 3;
// Sums of dot[i] over the 16 lanes of a row; the lane at position cv of the
// row keeps the sum of token cv (cv < 8).
SSD_DEV float row_dots_pick(float (&dot)[8], int cv) {
  float mine = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = group_sum_last<16>(dot[i]);
    mine = cv == i ? t : mine;
  }
  return mine;
}

// B-channel block mapping for transposed staging: within 16 lanes, 2 channel
// vectors x 8 token blocks, so the 16-byte LDS writes of a phase hit 16
// distinct bank groups. Returns (cv, tbi) for block index i of a tile with
// 16 channel vectors and QI/8 = 16 token blocks.
SSD_DEV void tmap(int i, int& cv, int& tbi) {
  tbi = (i >> 1) & 15;
  cv = (i & 1) | ((i >> 5) << 1);
}

// ---------------------------------------------------------------- phase 1
// dS_h [P x N] = sum_s x_s w_s (outer) B_s, w_s = exp(Lam_end - Lam_s) dt_s,
// for every head of the group, computed transposed (dS_h^T = B^T X'), so
// each lane holds 4 consecutive n of one p; pairs of lanes trade halves
// and store 16 bytes each (a wave's stores per row cover one whole 128-byte
// line). B^T is staged
// once (conv) for the group; x of one head at a time goes through two LDS
// buffers, the rows of later heads loaded two heads ahead. With aux (a conv
// bias: the state split) B^T is staged as B - bbar, da goes to aux and, with
// PRE, the kept rows are B - bbar and C - cbar, with u_t per token in ug.
template <bool CONV, bool PRE>
__global__ __launch_bounds__(NT, 2) void k_fstate(Src s, const bf16* __restrict__ dt,
                                               const float* __restrict__ A,
                                               f16* __restrict__ states,
                                               float* __restrict__ lam_end,
                                               f16* __restrict__ bcv, f16* __restrict__ ccv,
                                               float* __restrict__ aux,
                                               float* __restrict__ ug, int* status, int L,
                                               int H, int G, int nc, int hs) {
  __shared__ __align__(16) f16 BT[N * RS];      // [n][s]
  __shared__ __align__(16) f16 XB[2 * P * RS];  // two [p][s] buffers of x_s w_s
  __shared__ float wv[2][HB][QI];               // w_s of the current / next head block
  // hs workgroups share a (chunk, group), each walking hpg of its heads; the
  // first also keeps the convolved B and C rows for the output kernel
  const int g = blockIdx.y / hs, part = blockIdx.y % hs;
  const int hpg = H / G / hs, hg0 = g * (H / G) + part * hpg;
  const bool keep = PRE && part == 0;
  ChunkGeo cg;
  if (!chunk_geo(s, blockIdx.x, blockIdx.z, L, nc, cg)) return;
  L = cg.L;
  const int t0 = cg.t0, len = cg.len;
  const int64_t row0 = cg.tok0 + t0;
  // the wave index is uniform: read it into a scalar register
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rr = lane & 15, q4 = lane >> 4, kk = 8 * q4, r4 = 4 * q4;
  const int tc = 2 * lane;
  // this call's status word starts clear (the later kernels of the call only
  // set bits in it); with a ragged batch the table kernel cleared it
  if (!s.q.cu && (blockIdx.x | blockIdx.y | blockIdx.z | threadIdx.x) == 0) *status = 0;

  // Lam = inclusive cumsum of dt A over the chunk for head h0 + wave (flat
  // past len, where dt counts as 0), kept in log2 units so every decay is
  // one exp2; w_s = exp(Lam_end - Lam_s) dt_s goes to dst[wave][s].
  auto cumsum = [&](int h0, float dr0, float dr1, float (*dst)[QI]) {
    const float d0 = tc < len ? dr0 : 0.f, d1 = tc + 1 < len ? dr1 : 0.f;
    const float Ah = a_of(A, s.dta, h0 + wave) * kLog2e;
    const float a0 = d0 * Ah, a1 = d1 * Ah;
    const float v = wave_incl_scan(a0 + a1);
    const float l0 = v - a1, l1 = v;
    const float lamE = lane_value(l1, 63);
    dst[wave][tc] = fexp2(lamE - l0) * d0;
    dst[wave][tc + 1] = fexp2(lamE - l1) * d1;
    if (lane == 0) lam_end[cg.kg * H + h0 + wave] = lamE;
  };
  auto dt_at = [&](int h, int t) {
    return dt_of(to_f(dt[(row0 + min(t, len - 1)) * s.dta.dts + h]), s.dta, h);
  };

  // dt of the first head block, fetched before B
  const float dr0 = dt_at(hg0 + wave, tc), dr1 = dt_at(hg0 + wave, tc + 1);

  const bf16* cin_b = CONV ? cg.cin : nullptr;
  const bf16* xb = s.x + cg.tok0 * s.xs;
  const bf16* bb = s.b + cg.tok0 * s.bs;
  // x staging item of this thread (one head): 8 channel vectors x 32 blocks
  // of 4 tokens, 8 consecutive lanes on the 8 vectors of one block, so each
  // row load instruction reads whole 128-byte lines of 8 rows. The rows of
  // the group's heads 0 and 1 are loaded together with those of B; later
  // heads are loaded two heads ahead.
  const int xtb = tid >> 3, xcv = tid & 7, xp0 = xcv * 8;
  const int xnv = min(4, max(0, len - xtb * 4));
  XRaw<CONV> xr[2];
  ConvW<CONV> cwx;  // weights of the next x item to be staged
  // B item of this thread (16 channel vectors x 16 blocks of 8 tokens): with
  // PRE, 16 lanes on the 16 vectors of a row, so the rows kept for the
  // output kernel are stored as whole 256-byte pieces; otherwise the mapping
  // whose transposed LDS writes are conflict-free
  int cv, tbi;
  if constexpr (PRE) {
    cv = tid & 15;
    tbi = tid >> 4;
  } else {
    tmap(tid, cv, tbi);
  }
  const int n0 = cv * 8, tseq = t0 + tbi * 8;
  const int nvb = min(8, max(0, len - tbi * 8));
  const int64_t grow = (row0 + tbi * 8) * s.GN + g * N + n0;  // its row in bcv / ccv
  const bool ofs = CONV && aux;  // uniform: the state split is on
  // conv biases of this thread's 8 B channels (zero without the split)
  u32x4 bbr = {0u, 0u, 0u, 0u};
  {
    const int ch = s.HP + g * N + n0;
    // weights before rows (see ConvW)
    ConvW<CONV> cwb;
    convw_load<CONV>(cwb, s, ch);
    convw_load<CONV>(cwx, s, hg0 * P + xp0);
    Rows8<CONV> rb;
    rows_load<CONV, 8>(rb, bb + g * N + n0, s.bs, tseq, L - 1, s, ch, cin_b);
#pragma unroll
    for (int k = 0; k < 2; ++k)
      x_load<CONV>(xr[k], xb + (hg0 + k) * P + xp0, s.xs, t0 + xtb * 4, L - 1, s,
                   (hg0 + k) * P + xp0, cin_b);
    if constexpr (CONV) {
      if (ofs) bbr = cwb.b;
    }
    // with PRE, conv'd B also kept (natural layout) for the output kernel
    conv_store<CONV, true, CONV ? kOfsSub : kOfsNone>(rb, cwb, tseq, nvb, cin_b,
                                                      BT + n0 * RS + tbi * 8, RS,
                                                      keep ? bcv + grow : nullptr, s.GN, bbr);
  }
  // with PRE, conv'd C too for the output kernel (a group spans several of
  // its 4-head blocks, each of which would otherwise redo the B and C conv):
  // rows fetched now, converted after head 0 is staged
  Rows8<CONV> rc;
  ConvW<CONV> cwc;
  if constexpr (PRE) if (keep) {
    const int ch = s.HP + s.GN + g * N + n0;
    convw_load<CONV>(cwc, s, ch);
    rows_load<CONV, 8>(rc, s.c + cg.tok0 * s.bs + g * N + n0, s.bs, tseq, L - 1, s, ch,
                       cin_b);
  }
  cumsum(hg0, dr0, dr1, wv[0]);
  __syncthreads();

  // wave w: n-tiles 4 (w & 1) .. + 3 (one 128-byte half row of dS^T) and
  // p-tiles 2 (w >> 1), + 1, so each row segment a wave stores is a whole
  // cache line
  const int nt0 = 4 * (wave & 1), pt0 = 2 * (wave >> 1);
  // the split's row sums: wave w takes p-tile pt0 + (w & 1) with an A operand
  // whose row 0 is all ones (lane rr == 0), so output row 0 is sum_s x_s w_s
  f16x8 ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = rr == 0 ? (f16)1.0f : (f16)0.0f;

  x_store<CONV, false>(xr[0], cwx, t0 + xtb * 4, xnv, cin_b, &wv[0][0][xtb * 4],
                       XB + xp0 * RS + xtb * 4, nullptr, RS);
  if constexpr (PRE) if (keep) {
    float ud[8];
    // two halves of 4 tokens (the halo rows of the second are rows 4..)
    constexpr int kOfsC = CONV ? kOfsDot : kOfsNone;
    const u32x4 cbr = ofs ? cwc.b : u32x4{};
    conv_store4<CONV, kOfsC>(rc, cwc, tseq, nvb, cin_b, ccv + grow, s.GN, cbr, bbr, ud);
    conv_store4<CONV, kOfsC>(rc + 4, cwc, tseq + 4, nvb - 4, cin_b, ccv + grow + 4 * s.GN, s.GN,
                             cbr, bbr, ud + 4);
    if (ofs) {
      const float umine = row_dots_pick(ud, cv);
      if (cv < nvb) ug[(row0 + tbi * 8 + cv) * G + g] = umine;
    }
  }
  __syncthreads();

  // heads of the group in blocks of HB; head k = j HB + hh (even HB keeps
  // the buffer parity of head k equal to the parity of hh)
  for (int j = 0; j * HB < hpg; ++j) {
    float(*wcur)[QI] = wv[j & 1];
    float(*wnext)[QI] = wv[(j + 1) & 1];
    const int h0 = hg0 + j * HB;
    const bool more = (j + 1) * HB < hpg;
    // dt of the next block, fetched a block ahead of its cumsum (a load
    // waited on right away would also wait for this block's stores)
    bf16 dn0 = {}, dn1 = {};
    if (more) {
      dn0 = dt[(row0 + min(tc, len - 1)) * s.dta.dts + h0 + HB + wave];
      dn1 = dt[(row0 + min(tc + 1, len - 1)) * s.dta.dts + h0 + HB + wave];
    }
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      const int k = j * HB + hh;
      const f16* XT = XB + (hh & 1) * (P * RS);
      // weights of head k + 1 (staged at the end of this head), issued
      // before the rows of head k + 2
      if (k + 1 < hpg) convw_load<CONV>(cwx, s, (hg0 + k + 1) * P + xp0);
      if (k + 2 < hpg) {
        const int ch = (hg0 + k + 2) * P + xp0;
        x_load<CONV>(xr[hh & 1], xb + ch, s.xs, t0 + xtb * 4, L - 1, s, ch, cin_b);
      }
      // next block's decay weights, published by this iteration's barrier
      if (hh == HB - 2 && more)
        cumsum(h0 + HB, dt_of(to_f(dn0), s.dta, h0 + HB + wave),
               dt_of(to_f(dn1), s.dta, h0 + HB + wave), wnext);
      f32x4 acc[4][2], sa = zero4();
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int pi = 0; pi < 2; ++pi) acc[j][pi] = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        f16x8 xf[2];
#pragma unroll
        for (int pi = 0; pi < 2; ++pi)
          xf[pi] = lds16(XT + ((pt0 + pi) * 16 + rr) * RS + ks * 32 + kk);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // B^T fragment (A operand: row n, k = s)
          const f16x8 bf = lds16(BT + ((nt0 + j) * 16 + rr) * RS + ks * 32 + kk);
#pragma unroll
          for (int pi = 0; pi < 2; ++pi) acc[j][pi] = mma16(bf, xf[pi], acc[j][pi]);
        }
        if (ofs) sa = mma16(ones, (wave & 1) ? xf[1] : xf[0], sa);
      }
      // da of rows p = (pt0 + (w & 1)) 16 + rr: output row 0 (lanes 0..15)
      if (ofs && q4 == 0)
        aux[(cg.kg * H + h0 + hh) * (int64_t)(kAux * P) + (pt0 + (wave & 1)) * 16 + rr] = sa[0];
      // lane: n = (nt0 + j) * 16 + r4 + r, p = (pt0 + pi) * 16 + rr
      f16* o = states + (cg.kg * H + h0 + hh) * (int64_t)(P * N);
      // lanes q4 = 2m, 2m + 1 (16 apart) trade halves (an LDS-crossbar lane
      // swap, lane ^ 16) so each stores 16 bytes: the even one n-tile 2 jp,
      // the odd one n-tile 2 jp + 1. A store instruction then writes 64-byte
      // pieces of 16 rows instead of 32-byte ones.
      const bool evq = (q4 & 1) == 0;
#pragma unroll
      for (int pi = 0; pi < 2; ++pi)
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) {
          const int ja = 2 * jp, jb = ja + 1;
          const uint32_t a0 = pk(acc[ja][pi][0], acc[ja][pi][1]);
          const uint32_t a1 = pk(acc[ja][pi][2], acc[ja][pi][3]);
          const uint32_t b0 = pk(acc[jb][pi][0], acc[jb][pi][1]);
          const uint32_t b1 = pk(acc[jb][pi][2], acc[jb][pi][3]);
          const uint32_t r0 = __builtin_amdgcn_ds_swizzle(evq ? b0 : a0, 0x401F);
          const uint32_t r1 = __builtin_amdgcn_ds_swizzle(evq ? b1 : a1, 0x401F);
          const u32x4 w = evq ? u32x4{a0, a1, r0, r1} : u32x4{r0, r1, b0, b1};
          const int n0 = evq ? (nt0 + ja) * 16 + r4 : (nt0 + jb) * 16 + r4 - 4;
          *reinterpret_cast<u32x4*>(o + ((pt0 + pi) * 16 + rr) * N + n0) = w;
        }
      if (k + 1 < hpg) {
        f16* nx = XB + ((hh + 1) & 1) * (P * RS);
        const float* sc = hh + 1 < HB ? &wcur[hh + 1][xtb * 4] : &wnext[0][xtb * 4];
        x_store<CONV, false>(xr[(hh + 1) & 1], cwx, t0 + xtb * 4, xnv, cin_b, sc,
                             nx + xp0 * RS + xtb * 4, nullptr, RS);
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- phase 2
// S_in(0) = initial state (or 0); S_in(k+1) = exp(Lam_end,k) S_in(k) + dS_k.
// One thread carries V consecutive (p, n) elements of one (batch, head) in
// fp32 through all chunks, reading dS_k 64 / V chunks ahead (256 bytes of
// loads in flight per thread). V = 8 (16-byte accesses) when that gives the
// grid four workgroups per CU; calls with few heads and sequences (one long
// sequence of the tiny layer: 128 workgroups at V = 8) take V = 4 or 2, so
// more lanes stream the buffer, each with a deeper look-ahead along its
// chain of chunks. It also resets the
// state of the output kernel's cross-block norm (this launch always precedes
// that one on the stream): the kParts ticket counters to 0 and the npart
// per-row partial-sum slots to kUnset.
constexpr int kParts = 8;          // ticket partitions: block index mod 8, one per XCD
constexpr float kUnset = -1.0f;    // an unwritten slot: never a sum of squares (nor NaN)
// bits of the call's status word (first word of the workspace)
constexpr int kStatusTimeout = 1;    // a cross-block norm wait gave up
constexpr int kStatusNonFinite = 2;  // an output or the final state is not finite
// V fp16 of one thread: one load or store of 2 V bytes
template <int V> struct PassVec;
template <> struct PassVec<8> { typedef u32x4 T; };
template <> struct PassVec<4> { typedef uint32_t T __attribute__((ext_vector_type(2))); };
template <> struct PassVec<2> { typedef uint32_t T; };
template <int V>
SSD_DEV uint32_t pass_word(const typename PassVec<V>::T& v, int i) {
  if constexpr (V == 2) return v;
  else return v[i];
}
template <int V>
SSD_DEV void pass_ldf(const float* p, float (&v)[V]) {
  if constexpr (V == 8) {
    load8(p, v);
  } else {
#pragma unroll
    for (int j = 0; j < V; j += 2) {
      const float2 f = *reinterpret_cast<const float2*>(p + j);
      v[j] = f.x;
      v[j + 1] = f.y;
    }
  }
}
template <int V>
SSD_DEV void pass_stf(float* p, const float (&v)[V]) {
  if constexpr (V == 8) {
    store8(p, v);
  } else {
#pragma unroll
    for (int j = 0; j < V; j += 2) *reinterpret_cast<float2*>(p + j) = make_float2(v[j], v[j + 1]);
  }
}
// dS and sin_h are one buffer: S_in(k) overwrites dS_k, which this thread
// has loaded before (its own elements only), so neither pointer is restrict.
// With aux (the state split) the carried state is S' (dS holds dS') plus a
// bbar^T: the 16 lanes of a row p hold its 128 elements (V = 8 only), so
// the row sums are row-wide DPP reductions; a_in and sc'_in of chunk k go to
// aux beside da_k, and cbar of each group to cbg (fp16).
template <int V>
__global__ __launch_bounds__(256) void k_fpass(const f16* dS,
                                               const float* __restrict__ lam_end,
                                               const float* s_in, float* s_out,
                                               f16* sin_h, float* __restrict__ aux,
                                               f16* __restrict__ cbg,
                                               const bf16* __restrict__ cbias, int HP, int GN,
                                               int hpg, int* sync, float* part,
                                               int64_t npart, int* status, Seqs q, int H,
                                               int nc) {
  constexpr int PN = P * N;
  typedef typename PassVec<V>::T VT;
  constexpr int kPassDepth = 64 / V;  // chunks of loads in flight
  const int e = (blockIdx.x * 256 + threadIdx.x) * V;
  const int h = blockIdx.y;
  const int p = e / N, n0 = e % N;
  const bool ofs = V == 8 && aux != nullptr;  // the launcher takes V = 8 with the split
  {
    const int64_t gt =
        ((int64_t)(blockIdx.z * H + h) * gridDim.x + blockIdx.x) * 256 + threadIdx.x;
    const int64_t nt = (int64_t)gridDim.x * gridDim.y * gridDim.z * 256;
    if (sync && gt < kParts) sync[gt] = 0;
    for (int64_t i = gt; i < npart; i += nt) part[i] = kUnset;
  }
  // Dense batch: sequence blockIdx.z. Ragged batch: the entries blockIdx.z,
  // blockIdx.z + gridDim.z, ... of the table's list of sequences with two or
  // more tokens (a sequence with none keeps its slot, one token is the decode
  // kernel's), so the grid need not span every sequence of the batch.
  const int nz = !q.cu ? (int)blockIdx.z + 1
                 : __builtin_amdgcn_readfirstlane(*q.valid) == 1
                     ? __builtin_amdgcn_readfirstlane(*q.npre)
                     : 0;
  for (int zi = blockIdx.z; zi < nz; zi += gridDim.z) {
  const int b = !q.cu ? zi : __builtin_amdgcn_readfirstlane(q.pre[zi]);
  // the chunks of sequence b (global chunk k0 onwards) and where its state
  // comes from and goes to
  int64_t k0;
  int ncs = nc;
  const float* sin_p;
  float* sout_p;
  if (!q.cu) {
    const int64_t bh = (int64_t)b * H + h;
    k0 = (int64_t)b * nc;
    sin_p = s_in ? s_in + bh * PN : nullptr;
    sout_p = s_out ? s_out + bh * PN : nullptr;
  } else {
    k0 = q.chunk_first[b];
    ncs = q.chunk_first[b + 1] - q.chunk_first[b];
    float* slot = q.ssm_pool + ((int64_t)q.slots[b] * H + h) * PN;
    sin_p = !q.has_state || q.has_state[b] ? slot : nullptr;
    sout_p = slot;
  }
  float S[V];
  if (sin_p) {
    pass_ldf<V>(sin_p + e, S);
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) S[j] = 0.f;
  }
  // bbar, cbar of this thread's 8 columns; a of its row (0 without the split)
  float bbar[8] = {}, cbar[8] = {};
  float a = 0.f;
  if constexpr (V == 8) if (ofs) {
    const int g = h / hpg;
    load8(cbias + HP + g * N + n0, bbar);
    load8(cbias + HP + GN + g * N + n0, cbar);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bbar[j] = silu(bbar[j]);
      cbar[j] = silu(cbar[j]);
    }
    // cbar of the group in fp16 for the output kernel (row 0 of the group's
    // first head; other batches write the same values)
    if (blockIdx.x == 0 && p == 0 && h % hpg == 0)
      *reinterpret_cast<u32x4*>(cbg + g * N + n0) =
          u32x4{pk(cbar[0], cbar[1]), pk(cbar[2], cbar[3]), pk(cbar[4], cbar[5]),
                pk(cbar[6], cbar[7])};
    // carried-in state: a = (S . bbar) / |bbar|^2 per row, S' = S - a bbar^T
    float sb = 0.f, bq = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sb = fmaf(S[j], bbar[j], sb);
      bq = fmaf(bbar[j], bbar[j], bq);
    }
    sb = group_sum_last<16>(sb);
    bq = group_sum_last<16>(bq);
    a = bq > 0.f ? sb / bq : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) S[j] = fmaf(-a, bbar[j], S[j]);
  }
  for (int c0 = 0; c0 < ncs; c0 += kPassDepth) {
    VT d[kPassDepth];
    float al[kPassDepth], da[kPassDepth];
#pragma unroll
    for (int u = 0; u < kPassDepth; ++u) {
      const int c = min(c0 + u, ncs - 1);
      // each increment is read once: a streaming load
      d[u] = __builtin_nontemporal_load(
          reinterpret_cast<const VT*>(dS + ((k0 + c) * H + h) * PN + e));
      al[u] = fexp2(lam_end[(k0 + c) * H + h]);  // Lam_end in log2 units
      da[u] = ofs ? aux[((k0 + c) * H + h) * (int64_t)(kAux * P) + p] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kPassDepth; ++u) {
      const int c = c0 + u;
      if (c < ncs) {
        VT o;
        if constexpr (V == 2) {
          o = pk(S[0], S[1]);
        } else {
#pragma unroll
          for (int j = 0; j < V / 2; ++j) o[j] = pk(S[2 * j], S[2 * j + 1]);
        }
        *reinterpret_cast<VT*>(sin_h + ((k0 + c) * H + h) * PN + e) = o;
        if constexpr (V == 8) if (ofs) {
          float sc = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) sc = fmaf(S[j], cbar[j], sc);
          sc = group_sum_last<16>(sc);
          if ((threadIdx.x & 15) == 0) {
            float* ap = aux + ((k0 + c) * H + h) * (int64_t)(kAux * P);
            ap[P + p] = a;
            ap[2 * P + p] = sc;
          }
          a = al[u] * a + da[u];
        }
#pragma unroll
        for (int j = 0; j < V / 2; ++j) {
          const uint32_t w = pass_word<V>(d[u], j);
          S[2 * j] = al[u] * S[2 * j] + h2f_lo(w);
          S[2 * j + 1] = al[u] * S[2 * j + 1] + h2f_hi(w);
        }
      }
    }
  }
  if (sout_p) {
    if constexpr (V == 8) if (ofs) {
#pragma unroll
      for (int j = 0; j < 8; ++j) S[j] = fmaf(a, bbar[j], S[j]);
    }
    pass_stf<V>(sout_p + e, S);
    float chk = 0.f;  // NaN when any element is infinite or NaN
#pragma unroll
    for (int j = 0; j < V; ++j) chk += S[j] * 0.f;
    if (chk != 0.f) atomicOr(status, kStatusNonFinite);
  }
  }  // sequences
}

// ---------------------------------------------------------------- phase 3
// NM selects the epilogue: 0 writes the scan output y (bf16); 1 fuses the
// gated RMSNorm when the 4 heads are one norm group; 2 fuses it when a norm
// group spans nb = H/G/4 blocks: each block publishes its per-token sums of
// q^2 over its 256 channels, gathers its partners' sums, and scales its own
// rows (no y round trip through HBM).
//
// Every product is computed transposed, y^T[p, t], so a lane's accumulator
// holds 4 consecutive channels p of one token t (the row t = lane % 16 of
// the wave's row tile): y^T = X^T M'^T + S_in (exp(Lam_t) C_t)^T + D x^T.
// Wave w owns row tiles w and 7-w of the chunk (equal causal work) for all
// 4 heads. The C.B^T tiles of its rows stay in registers (computed as
// (B C^T) tiles, whose MFMA output layout is the B-operand layout of the
// next product once its 32 k-slots are mapped to the sequence positions
// 4q..4q+3 and 16+4q..16+4q+3 of two 16-column tiles). D x runs on the MFMA
// as [x | x] against [D_hi I ; D_lo I]: one MFMA per tile, with x at the
// fp16 precision of the other products (its rounding, at most 2^-12 of |x|,
// is far inside the bf16 output's tolerance) and D to ~22 bits.
// Phases: B, C staged (conv) -> G tiles and C fragments in registers while
// the first head's carried-in states are fetched -> per head: its x tile and
// its carried-in states staged in LDS (the next head's rows and states
// loaded meanwhile), the inter-chunk term, the intra-chunk term and D x
// accumulated in the same fp32 registers (the first two can be large and of
// opposite sign, so no rounding between them), y kept as fp16 pairs -> y
// through an LDS tile to a coalesced epilogue that gates with z
// (prefetched), normalises each row over its 256 channels and stores
// 16-byte vectors. With aux (the state split) B, C and S_in are the split
// operands and u_t, v_s, a_in, sc'_in enter in fp32: u_t + v_s on the C.B^T
// tiles before their fp16 rounding, sc'_in + a_in u_t on the inter-chunk
// accumulators before exp(Lam_t).
template <bool CONV, int NM, bool PREC>
__global__ __launch_bounds__(NT, 2) void k_fout(Src s, const bf16* __restrict__ dt,
                                                const float* __restrict__ A,
                                                const float* __restrict__ D,
                                                const f16* __restrict__ sin_h,
                                                const f16* __restrict__ bcv,
                                                const f16* __restrict__ ccv,
                                                const float* __restrict__ aux,
                                                const float* __restrict__ ug,
                                                const f16* __restrict__ cbg,
                                                const bf16* __restrict__ z,
                                                const bf16* __restrict__ nw, float eps,
                                                bf16* __restrict__ out, float* part, int* sync,
                                                int* status, int spin_max, int L, int H, int G,
                                                int nc) {
  static_assert(P * RS + P * NS + 2 * P * 2 <= 2 * QI * NS,
                "x tile, one head's states and its a_in, sc'_in fit");
  static_assert(QI * OS <= 2 * QI * NS, "output tile must fit");
  __shared__ __align__(16) f16 U[2 * QI * NS];  // Bs | Cs, then x tile + states, then Ot
  __shared__ float lam[HB][QI], dts[HB][QI], csd[HB][QI];
  __shared__ __align__(16) float uvs[2][QI];    // u_t, v_t of the split
  // conv weights ([channel][tap]) and bias of the block's HB * P x channels
  constexpr int kXW = CONV ? HB * P * W / 8 : 1, kXB = CONV ? HB * P / 8 : 1;
  __shared__ __align__(16) u32x4 XWl[kXW], XBl[kXB];
  f16* Bs = U;
  f16* Cs = U + QI * NS;
  f16* XT = U;                // [p][RS]: fp16(x) of the current head
  f16* Sl = U + P * RS;       // [p][NS]: S_in of the current head
  // a_in [P] | sc'_in [P] of the current head (fp32, 16-byte aligned)
  float* aS = reinterpret_cast<float*>(U + P * RS + P * NS);
  f16* Ot = U;                // [t][4 heads x p]: y
  const bool ofs = CONV && aux;  // uniform: the state split is on

  int c, b, h0, tk = 0;
  if constexpr (NM == 2) {
    // A ragged batch's grid covers the padded chunk table. Workgroups past
    // the chunks the table holds (or all, for a refused table) leave here,
    // before taking a ticket, when every ticket partition keeps whole norm
    // groups: the first nact H/HB workgroups by index then hold exactly the
    // tickets of the table's groups. Otherwise they take one and leave below.
    if (s.q.cu) {
      const int nparts0 = (gridDim.x * gridDim.z * G) % kParts == 0 ? kParts : 1;
      const int nact = __builtin_amdgcn_readfirstlane(*s.q.valid) == 1
                           ? __builtin_amdgcn_readfirstlane(*s.q.nchunks)
                           : 0;
      const int64_t lin =
          ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
      if (((int64_t)nact * G) % nparts0 == 0 && lin >= (int64_t)nact * (H / HB)) return;
    }
    // the tile comes from a ticket taken in arrival order. Blocks whose index
    // is v mod kParts (those one XCD receives) take tickets from counter v
    // and serve the norm groups that are v mod kParts, so the blocks of a
    // group share that XCD's L2 (and their B and C rows); a group's blocks
    // hold consecutive tickets of their partition, so a workgroup only waits
    // for partners that have already started, whatever the dispatch order.
    // When the group count is not a multiple of kParts: one partition.
    __shared__ int tk_s;
    const int nb = H / G / HB, nbat = gridDim.z;
    const int ngrp = gridDim.x * nbat * G, nparts = ngrp % kParts == 0 ? kParts : 1;
    const int part_id = ((blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) % nparts;
    if (threadIdx.x == 0)
      tk_s = __hip_atomic_fetch_add(sync + part_id, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int kloc = __builtin_amdgcn_readfirstlane(tk_s);
    // norm group grp = (chunk * batches + batch) * G + group; its j-th block
    // (heads of block j of the group) holds slot tk = grp * nb + j
    const int grp = (kloc / nb) * nparts + part_id;
    tk = grp * nb + kloc % nb;
    h0 = ((grp % G) * nb + tk % nb) * HB;
    b = (grp / G) % nbat;
    c = grp / G / nbat;
  } else {
    c = blockIdx.x;
    b = blockIdx.z;
    h0 = blockIdx.y * HB;
  }
  const int g = h0 / (H / G);
  // with a ragged batch, every block of a chunk no sequence owns returns
  // here, before any exchange: its norm-group partners share the chunk
  ChunkGeo cg;
  if (!chunk_geo(s, c, b, L, nc, cg)) return;
  L = cg.L;
  const int t0 = cg.t0, len = cg.len;
  const int64_t row0 = cg.tok0 + t0;
  // the wave index is uniform: read it into a scalar register
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rr = lane & 15, q4 = lane >> 4, kk = 8 * q4, r4 = 4 * q4;
  const int HP = s.HP;

  // dt of head `wave`, positions 2 lane and 2 lane + 1, fetched before B/C
  const int tc = 2 * lane;
  const float dr0 =
      dt_of(to_f(dt[(row0 + min(tc, len - 1)) * s.dta.dts + h0 + wave]), s.dta, h0 + wave);
  const float dr1 =
      dt_of(to_f(dt[(row0 + min(tc + 1, len - 1)) * s.dta.dts + h0 + wave]), s.dta, h0 + wave);

  const bf16* cin_b = CONV ? cg.cin : nullptr;
  // x staging item of this thread (one head): 8 channel vectors x 32 blocks
  // of 4 tokens, 8 consecutive lanes on the 8 vectors of one block (whole
  // 128-byte lines per row load). The rows of head 0 are loaded with those
  // of B and C. With PREC the x rows (also read by the chunk-state kernel
  // before) are streamed: nothing reads them after this kernel.
  const int xtb = tid >> 3, xcv = tid & 7, xp0 = xcv * 8;
  const bf16* xb = s.x + cg.tok0 * s.xs;
  const int xnv = min(4, max(0, len - xtb * 4));
  XRaw<CONV> xr;
  // this thread's piece of the block's x conv weights / bias, for XWl / XBl
  u32x4 xwp = {0u, 0u, 0u, 0u};
  if constexpr (CONV) {
    if (tid < kXW)
      xwp = reinterpret_cast<const u32x4*>(s.cw + (int64_t)h0 * P * W)[tid];
    else if (tid < kXW + kXB && s.cbias)
      xwp = reinterpret_cast<const u32x4*>(s.cbias + h0 * P)[tid - kXW];
  }
  // conv weights of an x item (local channel lch) from LDS
  auto xw_get = [&](ConvW<CONV>& cw, int lch) {
    if constexpr (CONV) {
#pragma unroll
      for (int q = 0; q < 4; ++q) cw.w[q] = XWl[lch * W / 8 + q];
      cw.b = XBl[lch / 8];
    }
  };
  // B and C, natural layout [t][n]: 16 channel vectors x 16 token blocks
  // each; the rows of both are loaded before either is converted. With PREC
  // both come already convolved, in fp16, from the chunk-state kernel.
  {
    const int cv = tid & 15, tbi = tid >> 4, n0 = cv * 8;
    const int tseq = t0 + tbi * 8, nv = min(8, max(0, len - tbi * 8));
    float ud[8];  // u_t of the split, per token
    const int64_t boff = cg.tok0 * s.bs + g * N + n0;
    const int chb = s.HP + g * N + n0, chc = chb + s.GN;
    // rows of the precomputed buffers, clamped into the sequence
    auto pre_rows = [&](const f16* src, u32x4 (&v)[8]) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = *reinterpret_cast<const u32x4*>(
            src + (cg.tok0 + min(tseq + i, L - 1)) * s.GN + g * N + n0);
    };
    auto pre_put = [&](const u32x4 (&v)[8], f16* dst) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4*>(dst + i * NS) = i < nv ? v[i] : u32x4{0u, 0u, 0u, 0u};
    };
    if constexpr (PREC) {
      // rows of B - bbar and C - cbar, and u_t, from the chunk-state kernel
      u32x4 vb[8], vc[8];
      pre_rows(bcv, vb);
      pre_rows(ccv, vc);
      float u = 0.f;
      if (ofs && tid < QI && tid < len) u = ug[(row0 + tid) * G + g];
      x_load<CONV, PREC>(xr, xb + h0 * P + xp0, s.xs, t0 + xtb * 4, L - 1, s, h0 * P + xp0, cin_b);
      pre_put(vb, Bs + (tbi * 8) * NS + n0);
      pre_put(vc, Cs + (tbi * 8) * NS + n0);
      if (ofs && tid < QI) uvs[0][tid] = u;
    } else {
      // weights before rows (see ConvW)
      ConvW<CONV> cwb, cwc;
      convw_load<CONV>(cwb, s, chb);
      convw_load<CONV>(cwc, s, chc);
      Rows8<CONV> rb, rc;
      rows_load<CONV, 8>(rb, s.b + boff, s.bs, tseq, L - 1, s, chb, cin_b);
      rows_load<CONV, 8>(rc, s.c + boff, s.bs, tseq, L - 1, s, chc, cin_b);
      x_load<CONV, PREC>(xr, xb + h0 * P + xp0, s.xs, t0 + xtb * 4, L - 1, s, h0 * P + xp0, cin_b);
      // conv biases of the 8 B and C channels: the split's offsets (zero without)
      u32x4 bbr = {0u, 0u, 0u, 0u}, cbr = {0u, 0u, 0u, 0u};
      if constexpr (CONV) {
        if (ofs) {
          bbr = cwb.b;
          cbr = cwc.b;
        }
      }
      conv_store<CONV, false, CONV ? kOfsSub : kOfsNone>(
          rb, cwb, tseq, nv, cin_b, Bs + (tbi * 8) * NS + n0, NS, nullptr, 0, bbr);
      conv_store<CONV, false, CONV ? kOfsDot : kOfsNone>(
          rc, cwc, tseq, nv, cin_b, Cs + (tbi * 8) * NS + n0, NS, nullptr, 0, cbr, bbr, ud);
      if (ofs) {
        const float um = row_dots_pick(ud, cv);
        if (cv < 8) uvs[0][tbi * 8 + cv] = um;
      }
    }
    if constexpr (CONV) {
      if (tid < kXW) XWl[tid] = xwp;
      else if (tid < kXW + kXB) XBl[tid - kXW] = xwp;
    }
    if (ofs && tid < QI) uvs[1][tid] = 0.f;  // v_t: two halves are added below
  }
  // Lam (inclusive cumsum of dt A), dt, and csd[s] = exp(Lam_ref - Lam_s) dt_s
  // with Lam_ref the value at the end of s's 32-position block (<= Lam_s).
  {
    const float d0 = tc < len ? dr0 : 0.f, d1 = tc + 1 < len ? dr1 : 0.f;
    const float Ah = a_of(A, s.dta, h0 + wave) * kLog2e;  // Lam in log2 units
    const float a0 = d0 * Ah, a1 = d1 * Ah;
    const float v = wave_incl_scan(a0 + a1);
    const float l0 = v - a1, l1 = v;
    const float lref = row_last(l1);  // lane 16 k + 15 ends the block of 32
    lam[wave][tc] = l0;
    lam[wave][tc + 1] = l1;
    dts[wave][tc] = d0;
    dts[wave][tc + 1] = d1;
    csd[wave][tc] = fexp2(lref - l0) * d0;
    csd[wave][tc + 1] = fexp2(lref - l1) * d1;
  }
  __syncthreads();
  if (ofs) {
    // v_t = cbar . (B_t - bbar) from the staged fp16 rows (fp16 products are
    // exact in the fp32 dot): waves 0, 1 take channels 0..63 and waves 2, 3
    // channels 64..127 of token tid % 128, reading cbar at uniform addresses;
    // the two halves meet in uvs[1] (0 + a + b is the same in either order)
    const int sv = tid & (QI - 1), hv = wave >> 1;
    const f16* bp = Bs + sv * NS + hv * (N / 2);
    const f16* cp = cbg + g * N + hv * (N / 2);
    float d = 0.f;
#pragma unroll
    for (int k = 0; k < N / 16; ++k) {
      const f16x8 b8 = *reinterpret_cast<const f16x8*>(bp + 8 * k);
      const f16x8 c8 = *reinterpret_cast<const f16x8*>(cp + 8 * k);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        d = __builtin_amdgcn_fdot2(f16x2{b8[2 * q], b8[2 * q + 1]}, f16x2{c8[2 * q], c8[2 * q + 1]},
                                   d, false);
    }
    atomicAdd(&uvs[1][sv], d);
    __syncthreads();
  }

  const int rta = wave, rtb = 7 - wave;
  // C fragments of the wave's rows (B operand: column t, k = n)
  f16x8 Cfa[4], Cfb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    Cfa[ks] = *reinterpret_cast<const f16x8*>(Cs + (rta * 16 + rr) * NS + ks * 32 + kk);
    Cfb[ks] = *reinterpret_cast<const f16x8*>(Cs + (rtb * 16 + rr) * NS + ks * 32 + kk);
  }
  // carried-in states of one head (contiguous [p][n], 16 KB): 4 x 16 bytes
  // per thread, loaded a head ahead and staged into LDS with that head's x;
  // with the split, threads 0..31 also carry its a_in | sc'_in (512 bytes)
  const f16* sbase = sin_h + (cg.kg * H + h0) * (int64_t)(P * N);
  u32x4 sreg[4], areg = {0u, 0u, 0u, 0u};
  auto s_load = [&](int hh) {
    const f16* sp = sbase + (int64_t)hh * (P * N);
#pragma unroll
    for (int i = 0; i < 4; ++i)  // read once: streaming loads
      sreg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sp + (tid + NT * i) * 8));
    if (ofs && tid < 2 * P / 4)
      areg = *reinterpret_cast<const u32x4*>(aux + (cg.kg * H + h0 + hh) * (int64_t)(kAux * P) +
                                             P + tid * 4);
  };
  auto s_store = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + NT * i, row = idx >> 4, v = idx & 15;  // row = p
      *reinterpret_cast<u32x4*>(Sl + row * NS + v * 8) = sreg[i];
    }
    if (ofs && tid < 2 * P / 4) *reinterpret_cast<u32x4*>(aS + tid * 4) = areg;
  };
  s_load(0);  // in flight while the G tiles are computed
  // u_t of the lane's tokens in the two row tiles (the split)
  const float ua = ofs ? uvs[0][rta * 16 + rr] : 0.f, ub = ofs ? uvs[0][rtb * 16 + rr] : 0.f;
  // (B C^T) tiles j <= rt of the wave's two row tiles: lane holds C_t.B_s for
  // t = 16 rt + rr and s = 16 j + 4 q4 + r (fp16, the MFMA operand precision).
  uint2 Ga[4], Gb[8];
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
    if (ofs) {
      const float4 v4 = *reinterpret_cast<const float4*>(&uvs[1][j * 16 + r4]);
      const float vs[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ga[r] += ua + vs[r];
        gb[r] += ub + vs[r];
      }
    }
    if (j < 4) Ga[j] = make_uint2(pk(ga[0], ga[1]), pk(ga[2], ga[3]));
    Gb[j] = make_uint2(pk(gb[0], gb[1]), pk(gb[2], gb[3]));
  }
  __syncthreads();  // B and C no longer read from LDS
  {
    ConvW<CONV> cwx;
    xw_get(cwx, xp0);
    x_store<CONV, false>(xr, cwx, t0 + xtb * 4, xnv, cin_b, nullptr, XT + xp0 * RS + xtb * 4,
                         nullptr, RS);
    s_store();
  }
  __syncthreads();

  // y^T of the block: fp16 pairs [row tile][head][p tile][p = r4 + 0,1 |
  // r4 + 2,3] at t = 16 rt + rr.
  uint32_t yk[2][4][4][2];

  // epilogue mapping: 16 consecutive threads take one row (8 channels from
  // each 128-channel half), thread rows t = tid / 16 + 16 e; the z of the
  // first ZPF rows is fetched during the last head
  static_assert(HB * P == 256 && NT == 256, "epilogue mapping");
  const int ev8 = tid & 15, et0 = tid >> 4;
  constexpr int EPI = QI / (NT / 16);  // 8 rows per thread
  constexpr int ZPF = EPI / 2;         // rows whose z is fetched during the last head
  u32x4 zr[NM ? 2 * EPI : 1];
  auto z_fetch = [&](int e) {
    const int t = et0 + 16 * e;
    // z is read once, here: a streaming load does not displace the x, B
    // and C lines (also read by the chunk-state kernel) or the chunk
    // states held in the last-level cache
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      zr[2 * e + hf] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          z + (row0 + min(t, len - 1)) * s.zs + h0 * P + hf * 128 + ev8 * 8));
  };

  // causal mask of the diagonal 16 x 16 tiles, position r of this lane's
  // k-slot quadruple: s = 16 rt + r4 + r against t = 16 rt + rr
  bool dmask[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) dmask[r] = r4 + r <= rr;
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    if (hh + 1 < HB) {
      const int ch = (h0 + hh + 1) * P + xp0;
      x_load<CONV, PREC>(xr, xb + ch, s.xs, t0 + xtb * 4, L - 1, s, ch, cin_b);
      s_load(hh + 1);
    } else if (NM) {
#pragma unroll
      for (int e = 0; e < ZPF; ++e) z_fetch(e);
    }
    const float Dh = D ? D[h0 + hh] : 0.f;
    const f16 dhi = (f16)Dh, dlo = (f16)(Dh - (float)dhi);
    // B operand [D_hi I ; D_lo I]: k-slot 8 q4 + j of column rr is D_hi
    // (k < 16) or D_lo (k >= 16) when (8 q4 + j) mod 16 == rr
    f16x8 df;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool on = ((8 * (q4 & 1) + j) == rr);
      df[j] = on ? (q4 < 2 ? dhi : dlo) : (f16)0.f;
    }
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int rt = ui == 0 ? rta : rtb;
      const int trow = rt * 16 + rr;  // this lane's token (B-operand column)
      const float lt = lam[hh][trow];
      // inter-chunk term S_in (exp(Lam_t) C_t)^T first, in the accumulators
      // the intra-chunk term is added to
      f32x4 acc[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        acc[pt] = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const f16x8 sf =
              *reinterpret_cast<const f16x8*>(Sl + (pt * 16 + rr) * NS + ks * 32 + kk);
          acc[pt] = mma16(sf, ui == 0 ? Cfa[ks] : Cfb[ks], acc[pt]);
        }
      }
      {
        if (ofs) {
          // + sc'_in[p] + a_in[p] u_t, p = 16 pt + r4 + r
          const float ut = ui == 0 ? ua : ub;
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) {
            const float4 a4 = *reinterpret_cast<const float4*>(aS + pt * 16 + r4);
            const float4 s4 = *reinterpret_cast<const float4*>(aS + P + pt * 16 + r4);
            acc[pt][0] = fmaf(a4.x, ut, acc[pt][0] + s4.x);
            acc[pt][1] = fmaf(a4.y, ut, acc[pt][1] + s4.y);
            acc[pt][2] = fmaf(a4.z, ut, acc[pt][2] + s4.z);
            acc[pt][3] = fmaf(a4.w, ut, acc[pt][3] + s4.w);
          }
        }
        const float et = fexp2(lt);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[pt][r] *= et;
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (2 * ks <= rt) {
          // k-slots 8 q4 + r <-> s = 32 ks + 4 q4 + r, 8 q4 + 4 + r <-> s + 16
          const int s0 = ks * 32 + r4;
          uint2 g0, g1;
          if (ui == 0) {
            g0 = Ga[(2 * ks) & 3];
            g1 = (2 * ks + 1 <= rt) ? Ga[(2 * ks + 1) & 3] : make_uint2(0u, 0u);
          } else {
            g0 = Gb[2 * ks];
            g1 = (2 * ks + 1 <= rt) ? Gb[2 * ks + 1] : make_uint2(0u, 0u);
          }
          // decay factors (fp32) -> fp16 pairs, times the fp16 C.B^T pairs
          float dj[8];
          if (2 * ks + 2 <= rt) {
            // whole block before the row tile: exp(Lam_t - Lam_s) dt_s =
            // exp(Lam_t - Lam_ref) csd_s, both factors <= 1
            const float rf = fexp2(lt - lam[hh][ks * 32 + 31]);
            const float4 c0 = *reinterpret_cast<const float4*>(&csd[hh][s0]);
            const float4 c1 = *reinterpret_cast<const float4*>(&csd[hh][s0 + 16]);
            const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) dj[j] = rf * cs[j];
          } else {
            // the block holding the diagonal 16 x 16 tile: for odd rt its
            // first 16 positions all precede the row tile and the tile is its
            // second half; for even rt the tile is its first half and the
            // second half lies after every t. In the tile, s <= t is
            // r4 + r <= rr. Positions with s > t get exponent -inf (exactly
            // 0, no select after a possibly infinite exp2).
            const bool odd = rt & 1;
            const float4 l0 = *reinterpret_cast<const float4*>(&lam[hh][s0]);
            const float4 l1 = *reinterpret_cast<const float4*>(&lam[hh][s0 + 16]);
            const float4 d0 = *reinterpret_cast<const float4*>(&dts[hh][s0]);
            const float4 d1 = *reinterpret_cast<const float4*>(&dts[hh][s0 + 16]);
            const float ls[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
            const float ds[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
            constexpr float kNegInf = -__builtin_huge_valf();
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const bool on0 = odd || dmask[r], on1 = odd && dmask[r];
              dj[r] = fexp2(on0 ? lt - ls[r] : kNegInf) * ds[r];
              dj[4 + r] = fexp2(on1 ? lt - ls[4 + r] : kNegInf) * ds[4 + r];
            }
          }
          const uint32_t gw[4] = {g0.x, g0.y, g1.x, g1.y};
          u32x4 aw;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            aw[q] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, gw[q]) *
                                                     cvt2(dj[2 * q], dj[2 * q + 1]));
          const f16x8 af = __builtin_bit_cast(f16x8, aw);
          f16x8 xa[4];
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) {
            const f16* xr0 = XT + (pt * 16 + rr) * RS + s0;
            const uint2 lo = *reinterpret_cast<const uint2*>(xr0);
            const uint2 hi2 = *reinterpret_cast<const uint2*>(xr0 + 16);
            xa[pt] = __builtin_bit_cast(f16x8, make_uint4(lo.x, lo.y, hi2.x, hi2.y));
          }
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) acc[pt] = mma16(xa[pt], af, acc[pt]);
        }
      }
      // D x: A = [x | x] over the row tile's 16 positions
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const f16x8 xa = lds16(XT + (pt * 16 + rr) * RS + rt * 16 + 8 * (q4 & 1));
        acc[pt] = mma16(xa, df, acc[pt]);
        yk[ui][hh][pt][0] = pk(acc[pt][0], acc[pt][1]);
        yk[ui][hh][pt][1] = pk(acc[pt][2], acc[pt][3]);
        pin(yk[ui][hh][pt]);
      }
    }
    __syncthreads();  // this head's x tile and states no longer read
    if (hh + 1 < HB) {
      ConvW<CONV> cwx;
      xw_get(cwx, (hh + 1) * P + xp0);
      x_store<CONV, false>(xr, cwx, t0 + xtb * 4, xnv, cin_b, nullptr, XT + xp0 * RS + xtb * 4,
                           nullptr, RS);
      s_store();
      __syncthreads();
    }
  }

  // Epilogue: 16 consecutive threads (one DPP row) take one token row, 8
  // channels from each 128-channel half, rows t = tid / 16 + 16 e; the z of
  // the later rows is fetched now, behind the first rows' work
  if constexpr (NM != 0) {
#pragma unroll
    for (int e = ZPF; e < EPI; ++e) z_fetch(e);
  }
  float wv8[2][8];
  if (NM) {
    load8(nw + h0 * P + ev8 * 8, wv8[0]);
    load8(nw + h0 * P + 128 + ev8 * 8, wv8[1]);
  }
  // y -> Ot [t][4 heads x P]: a lane's 4 channels of one token are 8 bytes
#pragma unroll
  for (int ui = 0; ui < 2; ++ui) {
    const int rt = ui == 0 ? rta : rtb;
#pragma unroll
    for (int hh = 0; hh < HB; ++hh)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
        *reinterpret_cast<uint2*>(Ot + (rt * 16 + rr) * OS + hh * P + pt * 16 + r4) =
            make_uint2(yk[ui][hh][pt][0], yk[ui][hh][pt][1]);
  }
  __syncthreads();

  if constexpr (NM == 2) {
    // q = y silu(z) is kept in registers as fp16 pairs (the y registers are
    // free by now) and each row's sum of q^2 over this block's 256 channels
    // is published at device scope
    const int nb = H / G / HB, grp = tk / nb;
    float* inv_s = &csd[0][0];  // per-row sums, then 1 / rms (csd is free by now)
    u32x4 qk[EPI][2];
#pragma unroll
    for (int e = 0; e < EPI; ++e) {
      const int t = et0 + 16 * e;
      float ss = 0.f;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float yv[8], zv[8];
        load8h(Ot + t * OS + hf * 128 + ev8 * 8, yv);
        unpack8(zr[2 * e + hf], zv);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          yv[j] *= silu(zv[j]);
          ss += yv[j] * yv[j];
        }
        qk[e][hf] = u32x4{pk(yv[0], yv[1]), pk(yv[2], yv[3]), pk(yv[4], yv[5]), pk(yv[6], yv[7])};
      }
      ss = group_sum_last<16>(ss);
      if (ev8 == 0) inv_s[t] = ss;
    }
    __syncthreads();
    // one thread per row publishes this block's sum and gathers the group's:
    // a slot still holding kUnset (never a sum of squares, not even NaN) has
    // not been written yet; a wait that runs out poisons the row
    if (tid < QI) {
      const int j = tk % nb;
      const float own = inv_s[tid];
      __hip_atomic_store(part + (int64_t)tk * QI + tid, own, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      const float* gp = part + (int64_t)grp * nb * QI + tid;
      float sq = 0.f;
      bool ok = false;
      for (int it = 0; it < spin_max && !ok; ++it) {
        sq = 0.f;
        ok = true;
#pragma unroll 8
        for (int k = 0; k < nb; ++k) {
          const float v = k == j ? own
                                 : __hip_atomic_load(gp + (int64_t)k * QI, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
          ok = ok && v != kUnset;
          sq += v;
        }
        if (!ok) __builtin_amdgcn_s_sleep(2);
      }
      inv_s[tid] = ok ? __builtin_amdgcn_rsqf(sq * (1.0f / (nb * HB * P)) + eps)
                      : __builtin_nanf("");
      // report a wait that gave up, and rows whose sum of squares is not
      // finite (an input or an intermediate out of range), in the status word
      if (!ok) atomicOr(status, kStatusTimeout);
      else if (tid < len && !(sq < __builtin_huge_valf())) atomicOr(status, kStatusNonFinite);
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPI; ++e) {
      const int t = et0 + 16 * e;
      const float inv = inv_s[t];
      if (t < len) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          float yv[8];
          unpack8h(qk[e][hf], yv);
#pragma unroll
          for (int j = 0; j < 8; ++j) yv[j] *= wv8[hf][j] * inv;
          // streaming store: the normalised output is final
          const u32x4 w = {pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]),
                           pack_bf16x2(yv[4], yv[5]), pack_bf16x2(yv[6], yv[7])};
          __builtin_nontemporal_store(
              w, reinterpret_cast<u32x4*>(out + (row0 + t) * HP + h0 * P + hf * 128 + ev8 * 8));
        }
      }
    }
    return;
  }

#pragma unroll
  for (int e = 0; e < EPI; ++e) {
    const int t = et0 + 16 * e;
    float yv[2][8];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) load8h(Ot + t * OS + hf * 128 + ev8 * 8, yv[hf]);
    if (NM) {
      float ss = 0.f;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float zv[8];
        unpack8(zr[2 * e + hf], zv);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          yv[hf][j] *= silu(zv[j]);
          ss += yv[hf][j] * yv[hf][j];
        }
      }
      ss = group_sum_last<16>(ss);
      if (ev8 == 0 && t < len && !(ss < __builtin_huge_valf()))
        atomicOr(status, kStatusNonFinite);
      const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / (HB * P)) + eps);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 8; ++j) yv[hf][j] *= wv8[hf][j] * inv;
    }
    if (t < len) {
      if (!NM) {
        float chk = 0.f;  // NaN when any value is infinite or NaN
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int j = 0; j < 8; ++j) chk += yv[hf][j] * 0.f;
        if (chk != 0.f) atomicOr(status, kStatusNonFinite);
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        // streaming store: the output is final (for norm groups of more than
        // kMaxNormBlocks blocks the grouped norm streams y back once)
        store8_stream(out + (row0 + t) * HP + h0 * P + hf * 128 + ev8 * 8, yv[hf]);
      }
    }
  }
}

}  // namespace fast

// ---------------------------------------------------------------------------
bool fast_path_ok(bool io_bf16, int P, int N, int H, int G, int Q, int W, bool conv) {
  return io_bf16 && P == fast::P && N == fast::N && (H / G) % fast::HB == 0 && Q >= 64 &&
         (!conv || W == fast::W);
}

// Workspace: chunk-state increments, overwritten in place by the carried-in
// states (fp16), Lam_end; with a conv bias the state split's per-chunk rows
// (da, a_in, sc'_in); when a group spans several 4-head blocks, the per-row
// partial sums and the ticket counters of the cross-block norm and, with the
// conv, the convolved B and C rows in fp16 for the output kernel (and, with
// a bias, u_t per token and group).
namespace {
size_t ws_round(size_t b) { return (b + 255) / 256 * 256; }
bool wide(int H, int G) { return H / G > fast::HB; }
// Most 4-head blocks per norm group normalised across blocks: a waiting
// block holds its slot, and up to (blocks - 1) blocks of one group per ticket
// partition may wait for the rest, so the group must fit well inside one
// XCD's 64 resident workgroups. Wider groups take y and the grouped norm.
constexpr int kMaxNormBlocks = 32;
bool pre_c(int H, int G, bool conv) { return conv && wide(H, G); }
}  // namespace
// Byte offsets of the workspace pieces. Dense batch: B sequences of L
// tokens, B * ceil(L / QI) chunks. Ragged batch (varlen): B sequences, L
// tokens in all, at most ceil(L / QI) + B chunks (a padded table), plus the
// chunk table and a bitmap of the pool's slots.
struct FastLayout {
  int64_t chunks, npart;
  size_t dS, lam, aux, cbg, part, sync, bcv, ccv, uv, valid, first, cseq, bitmap, dec, pre, total;
};
// The split's pieces are reserved whenever the conv is on (the size query
// does not know whether a call brings a bias); a call uses them with one.
FastLayout fast_layout(int B, int L, int H, int G, bool conv, bool varlen, int num_slots) {
  using namespace fast;
  FastLayout f{};
  const size_t PN = P * N;
  f.chunks = varlen ? (int64_t)(L + QI - 1) / QI + B : (int64_t)B * ((L + QI - 1) / QI);
  f.npart = f.chunks * (H / HB) * QI;
  const size_t toks = (size_t)(varlen ? L : (int64_t)B * L);
  const size_t rows = toks * G * N * 2;
  const bool split = conv;
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off += ws_round(n);
    return o;
  };
  f.dS = take((size_t)f.chunks * H * PN * 2);
  f.lam = take((size_t)f.chunks * H * 4);
  if (split) {
    f.aux = take((size_t)f.chunks * H * kAux * P * 4);
    f.cbg = take((size_t)G * N * 2);
  }
  if (wide(H, G)) {
    f.part = take((size_t)f.npart * 4);
    f.sync = take(kParts * 4);
  }
  if (pre_c(H, G, conv)) {
    f.bcv = take(rows);
    f.ccv = take(rows);
    if (split) f.uv = take(toks * G * 4);
  }
  if (varlen) {
    f.valid = take(4);
    f.first = take(((size_t)B + 1) * 4);
    f.cseq = take((size_t)f.chunks * 4);
    f.bitmap = take(((size_t)num_slots + 31) / 32 * 4);
    f.dec = take(((size_t)B + 1) * 4);  // one-token sequences, then their count
    f.pre = take(((size_t)B + 1) * 4);  // sequences of two or more tokens, then their count
  }
  f.total = off;
  return f;
}

size_t fast_ws_bytes(int B, int L, int H, int G, bool conv) {
  return fast_layout(B, L, H, G, conv, false, 0).total;
}
size_t fast_varlen_ws_bytes(int nseq, int T, int H, int G, int num_slots) {
  return fast_layout(nseq, T, H, G, true, true, num_slots).total;
}
int fast_max_norm_heads() { return kMaxNormBlocks * fast::HB; }

namespace fast {
// The chunk table of a ragged batch, built by one workgroup at the start of
// the call: sequence i owns tokens [cu[i], cu[i+1]) and ceil(len_i / QI)
// consecutive global chunks from chunk_first[i]; chunk_seq maps each chunk
// back (-1 past the last). Checks on the device what the host cannot see:
// cu[0] == 0, cu[nseq] == T, no negative length, every slot of a sequence
// with tokens inside the pool and used once (a bitmap). Any failure leaves
// valid = 0 (every later kernel of the call then does nothing: no output,
// no state is written) and sets the call's status bit.
constexpr int kTableThreads = 1024;
constexpr int kStatusVarlen = 4;  // status bit: the ragged batch's metadata is invalid
__global__ __launch_bounds__(kTableThreads) void k_varlen_table(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ slots, int nseq, int T,
    int num_slots, int32_t* chunk_first, int32_t* chunk_seq, int64_t max_chunks,
    uint32_t* bitmap, int32_t* dec, int32_t* pre, int* valid, int* status) {
  __shared__ int bad;
  __shared__ int csum[kTableThreads], dsum[kTableThreads], psum[kTableThreads];
  const int tid = threadIdx.x;
  if (tid == 0) {
    bad = 0;
    *status = 0;  // this call's status word starts clear
    *valid = 0;
  }
  const int nw = (num_slots + 31) / 32;
  for (int i = tid; i < nw; i += kTableThreads) bitmap[i] = 0u;
  __syncthreads();
  // thread tid takes sequences [i0, i1)
  const int per = (nseq + kTableThreads - 1) / kTableThreads;
  const int i0 = min(nseq, tid * per), i1 = min(nseq, i0 + per);
  int cnt = 0, dcnt = 0, pcnt = 0, err = 0;
  if (tid == 0 && (cu[0] != 0 || cu[nseq] != T)) err = 1;
  for (int i = i0; i < i1; ++i) {
    const int len = cu[i + 1] - cu[i];
    if (len < 0) {
      err = 1;
      continue;
    }
    if (len == 0) continue;
    const int sl = slots[i];
    if (sl < 0 || sl >= num_slots) {
      err = 1;
      continue;
    }
    const uint32_t bit = 1u << (sl & 31);
    if (atomicOr(bitmap + (sl >> 5), bit) & bit) err = 1;  // slot used twice
    if (len == 1) {
      ++dcnt;  // a decode step: the decode kernel takes it, it gets no chunk
    } else {
      cnt += (len + QI - 1) / QI;
      ++pcnt;
    }
  }
  if (err) atomicOr(&bad, 1);
  // exclusive scans of the per-thread chunk, decode-step and prefill counts
  csum[tid] = cnt;
  dsum[tid] = dcnt;
  psum[tid] = pcnt;
  __syncthreads();
  for (int d = 1; d < kTableThreads; d <<= 1) {
    const int v = tid >= d ? csum[tid - d] : 0, w = tid >= d ? dsum[tid - d] : 0,
              u = tid >= d ? psum[tid - d] : 0;
    __syncthreads();
    csum[tid] += v;
    dsum[tid] += w;
    psum[tid] += u;
    __syncthreads();
  }
  int base = csum[tid] - cnt, dbase = dsum[tid] - dcnt, pbase = psum[tid] - pcnt;
  const int total = csum[kTableThreads - 1];
  for (int i = i0; i < i1; ++i) {
    chunk_first[i] = base;
    const int len = cu[i + 1] - cu[i];
    const int n = len > 1 ? (len + QI - 1) / QI : 0;
    for (int j = 0; j < n; ++j)  // bounded: garbage offsets only make the call invalid
      if (base + j >= 0 && base + j < max_chunks) chunk_seq[base + j] = i;
    base += n;
    if (len == 1) dec[dbase++] = i;
    else if (len > 1) pre[pbase++] = i;
  }
  if (tid == 0) {
    chunk_first[nseq] = total;
    dec[nseq] = dsum[kTableThreads - 1];
    pre[nseq] = psum[kTableThreads - 1];
  }
  for (int64_t k = max(total, 0) + tid; k < max_chunks; k += kTableThreads) chunk_seq[k] = -1;
  __syncthreads();
  if (tid == 0) {
    if (bad || total > max_chunks) {
      atomicOr(status, kStatusVarlen);
    } else {
      // the table's global writes are ordered before the flag's
      __threadfence();
      *valid = 1;
    }
  }
}

// The new conv state of each sequence of a ragged batch: the last W-1 rows
// of [its slot's rows (or zeros) ; its tokens], written back into the slot
// (in place: a row is read before any row it could overwrite).
__global__ __launch_bounds__(256) void k_varlen_conv_state(const bf16* __restrict__ xbc,
                                                           int64_t xs, Seqs q, int C) {
  const int cv = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (cv * 8 >= C || __builtin_amdgcn_readfirstlane(*q.valid) != 1) return;
  const int a = q.cu[b], L = q.cu[b + 1] - a;
  if (L <= 1) return;  // none, or a decode step (the decode kernel shifts it)
  bf16* slot = (bf16*)q.conv_pool + (int64_t)q.slots[b] * (W - 1) * C + cv * 8;
  const bool resume = !q.has_state || q.has_state[b];
#pragma unroll
  for (int r = 0; r < W - 1; ++r) {
    const int e = L + r;  // row of [state ; tokens]
    u32x4 v = {0u, 0u, 0u, 0u};
    if (e >= W - 1)
      v = *reinterpret_cast<const u32x4*>(xbc + (a + e - (W - 1)) * xs + cv * 8);
    else if (resume)
      v = *reinterpret_cast<const u32x4*>(slot + (int64_t)e * C);
    *reinterpret_cast<u32x4*>(slot + (int64_t)r * C) = v;
  }
}
}  // namespace fast

hipError_t launch_fast_scan(const FastScanArgs& a, hipStream_t st) {
  using namespace fast;
  const bool varlen = a.q.cu != nullptr;
  const bool split = a.conv && a.conv_b;  // the state split: with a conv bias
  const FastLayout f = fast_layout(a.B, a.L, a.H, a.G, a.conv, varlen, a.num_slots);
  // dense: (chunk, ., batch) grids; ragged: (global chunk, ., 1)
  const int nc = varlen ? (int)f.chunks : (a.L + QI - 1) / QI;
  const int gz = varlen ? 1 : a.B;
  const size_t PN = P * N;
  unsigned char* w = (unsigned char*)a.ws;
  // chunk increments, overwritten in place by the carried-in states
  fast::f16* dS = (fast::f16*)(w + f.dS);
  fast::f16* sinb = dS;
  float* lam_end = (float*)(w + f.lam);
  float* part = wide(a.H, a.G) ? (float*)(w + f.part) : nullptr;
  int* sync = wide(a.H, a.G) ? (int*)(w + f.sync) : nullptr;
  const int64_t npart = f.npart;
  // output kernel epilogue: 0 = y, 1 = norm within the block, 2 = norm
  // across the group's blocks (its state is reset by the pass kernel); with
  // more than kMaxNormBlocks blocks per group, y and then the grouped norm
  const bool norm_after = a.z && a.H / a.G > kMaxNormBlocks * HB;
  const int nm = !a.z || norm_after ? 0 : wide(a.H, a.G) ? 2 : 1;
  const bool prec = pre_c(a.H, a.G, a.conv);
  fast::f16* bcv = prec ? (fast::f16*)(w + f.bcv) : nullptr;
  fast::f16* ccv = prec ? (fast::f16*)(w + f.ccv) : nullptr;
  float* aux = split ? (float*)(w + f.aux) : nullptr;
  float* ug = split && prec ? (float*)(w + f.uv) : nullptr;
  fast::f16* cbg = split ? (fast::f16*)(w + f.cbg) : nullptr;
  Seqs q = a.q;
  if (varlen) {
    q.valid = (const int*)(w + f.valid);
    q.chunk_first = (const int32_t*)(w + f.first);
    q.nchunks = q.chunk_first + a.B;
    q.pre = (const int32_t*)(w + f.pre);
    q.npre = q.pre + a.B;
    q.chunk_seq = (const int32_t*)(w + f.cseq);
    hipLaunchKernelGGL(k_varlen_table, dim3(1), dim3(kTableThreads), 0, st, a.q.cu, a.q.slots,
                       a.B, a.L, a.num_slots, (int32_t*)(w + f.first), (int32_t*)(w + f.cseq),
                       f.chunks, (uint32_t*)(w + f.bitmap), (int32_t*)(w + f.dec),
                       (int32_t*)(w + f.pre),
                       (int*)(w + f.valid), a.status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

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
  s.zs = a.zs;
  s.dta = DtA{a.dts, a.dt_bias};
  s.q = q;

  // (chunk, 4-head block, batch): the chunk varies fastest in dispatch order
  const dim3 g1(nc, a.H / HB, gz);
  {
    // one workgroup per (chunk, group, batch): B staged once for the group
    ProfScope ps(st, KID_FAST_STATE);
    // a ragged batch splits each (chunk, group)'s heads over two workgroups
    // when they come in blocks of 8: its chunk count is known only on the
    // device, and one workgroup per (chunk, group) left the serving batch's
    // 552 of them a second, nearly empty round of a 512-workgroup machine
    const int hs = varlen && (a.H / a.G) % (2 * HB) == 0 ? 2 : 1;
    const dim3 g0(nc, a.G * hs, gz);
    const bf16* dt = (const bf16*)a.dt;
    if (prec)
      hipLaunchKernelGGL((k_fstate<true, true>), g0, dim3(NT), 0, st, s, dt, a.A, dS, lam_end,
                         bcv, ccv, aux, ug, a.status, a.L, a.H, a.G, nc, hs);
    else if (a.conv)
      hipLaunchKernelGGL((k_fstate<true, false>), g0, dim3(NT), 0, st, s, dt, a.A, dS, lam_end,
                         nullptr, nullptr, aux, nullptr, a.status, a.L, a.H, a.G, nc, hs);
    else
      hipLaunchKernelGGL((k_fstate<false, false>), g0, dim3(NT), 0, st, s, dt, a.A, dS, lam_end,
                         nullptr, nullptr, nullptr, nullptr, a.status, a.L, a.H, a.G, nc, hs);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps(st, KID_FAST_PASS);
    // 8 elements per thread unless that leaves fewer than four workgroups
    // per CU (the split always takes 8)
    // a ragged batch's workgroups walk the list of its prefills, gridDim.z
    // apart: enough z slices for 2048 workgroups at 8 elements per thread
    const int64_t per_z = (int64_t)a.H * (PN / (256 * 8));
    const int zdim =
        !varlen ? a.B : (int)std::min<int64_t>(a.B, std::max<int64_t>(1, (2048 + per_z - 1) / per_z));
    const int64_t heads = (int64_t)a.H * zdim;
    const int pv = split || heads * (PN / (256 * 8)) >= 1024 ? 8
                   : heads * (PN / (256 * 4)) >= 1024       ? 4
                                                            : 2;
#define SSD_FPASS(V)                                                                           \
  hipLaunchKernelGGL(k_fpass<V>, dim3(PN / (256 * V), a.H, zdim), dim3(256), 0, st, dS, lam_end, \
                     a.s_in, a.s_out, sinb, aux, cbg, (const bf16*)a.conv_b, a.H * P, a.G * N,  \
                     a.H / a.G, nm == 2 ? sync : nullptr, part, nm == 2 ? npart : 0, a.status, q, \
                     a.H, nc)
    if (pv == 8) SSD_FPASS(8);
    else if (pv == 4) SSD_FPASS(4);
    else SSD_FPASS(2);
#undef SSD_FPASS
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // gated norm: within the block when a norm group is exactly the 4-head
  // block, across the group's blocks when it spans several; without z the
  // scan output y is written
#define SSD_FOUT(CV, NM, PC)                                                                  \
  hipLaunchKernelGGL((k_fout<CV, NM, PC>), g1, dim3(NT), 0, st, s, (const bf16*)a.dt, a.A, a.D, \
                     sinb, bcv, ccv, aux, ug, cbg, (const bf16*)a.z, (const bf16*)a.norm_w,     \
                     a.eps, (bf16*)a.y, part, sync, a.status, a.spin_max, a.L, a.H, a.G, nc)
  {
    ProfScope ps(st, KID_FAST_OUT);
    // precomputed B and C exist exactly when the conv is on and a group spans
    // several blocks
    if (a.conv) {
      if (nm == 1) SSD_FOUT(true, 1, false);
      else if (nm == 2) SSD_FOUT(true, 2, true);
      else if (prec) SSD_FOUT(true, 0, true);
      else SSD_FOUT(true, 0, false);
    } else {
      if (nm == 1) SSD_FOUT(false, 1, false);
      else if (nm == 2) SSD_FOUT(false, 2, false);
      else SSD_FOUT(false, 0, false);
    }
  }
#undef SSD_FOUT
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (varlen) {
    // new conv states last: the scan kernels read the slots' old rows
    const int C = a.H * P + 2 * a.G * N;
    hipLaunchKernelGGL(k_varlen_conv_state, dim3((C / 8 + 255) / 256, a.B), dim3(256), 0, st,
                       (const bf16*)a.x, a.xs, q, C);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the one-token sequences: a decode step each, states in their slots
    return launch_decode_varlen(true, a.B, a.H, P, a.G, N, W, a.x, a.xs, a.z, a.zs, a.dt,
                                DtA{a.dts, a.dt_bias}, a.A, a.D, a.conv_w, a.conv_b, a.norm_w,
                                a.eps, q, (const int32_t*)(w + f.dec), a.y, st);
  }
  if (!norm_after) return e;
  return launch_gated_norm(true, false, a.B * a.L, a.H * P, a.G, a.y, a.z, a.zs, a.norm_w, a.eps,
                           a.y, st);
}

}  // namespace ssd
