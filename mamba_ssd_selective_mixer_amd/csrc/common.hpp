// Device helpers shared by the gfx950 kernels of the Mamba-2 mixer core:
// I/O element conversion, vector loads/stores, fast transcendental helpers,
// wave reductions and MFMA fragment wrappers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dta.hpp"

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef _Float16 h16;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 h16x8;

#define SSD_DEV __device__ __forceinline__

SSD_DEV float to_f(float v) { return v; }
SSD_DEV float to_f(bf16 v) { return (float)v; }

template <class T> SSD_DEV T from_f(float v);
template <> SSD_DEV float from_f<float>(float v) { return v; }
template <> SSD_DEV bf16 from_f<bf16>(float v) { return (bf16)v; }  // round to nearest even
template <> SSD_DEV h16 from_f<h16>(float v) { return (h16)v; }     // round to nearest even

// MFMA operand type for an I/O type: fp16 for bf16 I/O (11-bit mantissa, 8x
// finer than bf16 at the same MFMA rate), fp32 for fp32 I/O.
template <class T> struct OpOf { typedef T type; };
template <> struct OpOf<bf16> { typedef h16 type; };

// exp(x) through the hardware base-2 exponential.
SSD_DEV float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
SSD_DEV float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kLog2e = 1.4426950408889634f;
SSD_DEV float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
SSD_DEV float silu(float u) { return u * frcp(1.0f + fexp(-u)); }

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^-|v|), with log1p(e)
// taken as log(u) e / (u - 1), u = 1 + e (exact when u rounds to 1).
SSD_DEV float softplus(float v) {
  const float e = fexp(-__builtin_fabsf(v));
  const float u = 1.0f + e;
  const float l = u == 1.0f ? e : __builtin_amdgcn_logf(u) * 0.6931471805599453f * e * frcp(u - 1.0f);
  return __builtin_fmaxf(v, 0.0f) + l;
}

SSD_DEV float dt_of(float raw, const DtA& p, int h) {
  return p.bias ? softplus(raw + p.bias[h]) : raw;
}
SSD_DEV float a_of(const float* A, const DtA& p, int h) { return p.bias ? -fexp(A[h]) : A[h]; }

// ---- 8-element vector I/O (16 bytes for bf16, 32 bytes for fp32) ---------
SSD_DEV void load8(const float* p, float (&v)[8]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
SSD_DEV void load8(const bf16* p, float (&v)[8]) {
  uint4 a = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
SSD_DEV void store8(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
// two fp32 -> one word of two bf16 (round to nearest even; a in the low
// half), one packed conversion
SSD_DEV uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{a, b}, bf16x2));
}
SSD_DEV void store8(bf16* p, const float (&v)[8]) {
  uint4 a;
  a.x = pack_bf16x2(v[0], v[1]);
  a.y = pack_bf16x2(v[2], v[3]);
  a.z = pack_bf16x2(v[4], v[5]);
  a.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = a;
}

// Streaming (non-temporal) 8-element loads and stores, for data read once or
// not read back: they do not displace cached lines other kernels reuse.
typedef unsigned u32x4s __attribute__((ext_vector_type(4)));
SSD_DEV void load8_stream(const bf16* p, float (&v)[8]) {
  const u32x4s u = __builtin_nontemporal_load(reinterpret_cast<const u32x4s*>(p));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
SSD_DEV void load8_stream(const float* p, float (&v)[8]) { load8(p, v); }
SSD_DEV void store8_stream(bf16* p, const float (&v)[8]) {
  const u32x4s u = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7])};
  __builtin_nontemporal_store(u, reinterpret_cast<u32x4s*>(p));
}
SSD_DEV void store8_stream(float* p, const float (&v)[8]) { store8(p, v); }

// ---- cross-lane sums, scans and broadcasts -------------------------------
// Built on DPP row operations (a row is 16 lanes): each step is one VALU
// instruction reading another lane's register, with no LDS round trip.
// dpp_src<CTRL, ROWS>(v): the value of the lane CTRL selects, 0 where it
// selects no lane (bound_ctrl) or where the row is not in the ROWS mask.
template <int CTRL, int ROWS = 0xF>
SSD_DEV float dpp_src(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, true));
}
// Sum over aligned groups of W lanes (W a power of two <= 64). For W <= 16
// every lane of the group holds the sum; for W = 32 and 64 the group's last
// lane does.
template <int W>
SSD_DEV float group_sum_last(float v) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "group width");
  if constexpr (W >= 2) v += dpp_src<0xB1>(v);        // quad_perm [1,0,3,2]
  if constexpr (W >= 4) v += dpp_src<0x4E>(v);        // quad_perm [2,3,0,1]
  if constexpr (W >= 8) v += dpp_src<0x141>(v);       // row_half_mirror
  if constexpr (W >= 16) v += dpp_src<0x140>(v);      // row_mirror
  if constexpr (W >= 32) v += dpp_src<0x142, 0xA>(v); // row_bcast:15 into rows 1, 3
  if constexpr (W >= 64) v += dpp_src<0x143, 0xC>(v); // row_bcast:31 into rows 2, 3
  return v;
}
// value of lane l (uniform)
SSD_DEV float lane_value(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// sum over the 64 lanes (uniform)
SSD_DEV float wave_sum(float v) { return lane_value(group_sum_last<64>(v), 63); }
// inclusive prefix sum over the 64 lanes
SSD_DEV float wave_incl_scan(float v) {
  v += dpp_src<0x111>(v);       // row_shr:1
  v += dpp_src<0x112>(v);       // row_shr:2
  v += dpp_src<0x114>(v);       // row_shr:4
  v += dpp_src<0x118>(v);       // row_shr:8
  v += dpp_src<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_src<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}
// value of the last lane of this lane's row
SSD_DEV float row_last(float v) { return dpp_src<0x15F>(v); }  // row_newbcast:15

// ---- MFMA fragments ---------------------------------------------------------
// 16x16 output tile, fp32 accumulate. For one MFMA of depth KSTEP, lane l
// holds KPL consecutive k values starting at k = KPL * (l / 16) of row
// (A operand) or column (B operand) l % 16; the output lane l holds rows
// 4 * (l / 16) + r, r < 4, of column l % 16.
template <class T> struct Mfma;
template <> struct Mfma<h16> {
  static constexpr int KPL = 8, KSTEP = 32;
  typedef h16x8 frag;
  static SSD_DEV f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // KPL consecutive operand values from LDS.
  static SSD_DEV frag ld(const h16* p) { return *reinterpret_cast<const h16x8*>(p); }
  // KPL consecutive bf16 values from memory, converted.
  static SSD_DEV frag ldg(const bf16* p) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
    frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (h16)(float)v[j];
    return f;
  }
  // KPL consecutive values converted from fp32.
  static SSD_DEV frag cvt(const float* p) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    frag f;
    f[0] = (h16)a.x; f[1] = (h16)a.y; f[2] = (h16)a.z; f[3] = (h16)a.w;
    f[4] = (h16)b.x; f[5] = (h16)b.y; f[6] = (h16)b.z; f[7] = (h16)b.w;
    return f;
  }
  static SSD_DEV frag ldg(const float* p) { return cvt(p); }
};
template <> struct Mfma<float> {
  static constexpr int KPL = 1, KSTEP = 4;
  typedef float frag;
  static SSD_DEV f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static SSD_DEV frag ld(const float* p) { return *p; }
  static SSD_DEV frag ldg(const float* p) { return *p; }
  static SSD_DEV frag ldg(const bf16* p) { return (float)*p; }
  static SSD_DEV frag cvt(const float* p) { return *p; }
};

SSD_DEV f32x4 zero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }
