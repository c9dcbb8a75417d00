// Device helpers shared by the gfx950 kernels of the Mamba-2 mixer core:
// I/O element conversion, vector loads/stores, fast transcendental helpers,
// wave reductions and MFMA fragment wrappers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

#define SSD_DEV __device__ __forceinline__

SSD_DEV float to_f(float v) { return v; }
SSD_DEV float to_f(bf16 v) { return (float)v; }

template <class T> SSD_DEV T from_f(float v);
template <> SSD_DEV float from_f<float>(float v) { return v; }
template <> SSD_DEV bf16 from_f<bf16>(float v) { return (bf16)v; }  // round to nearest even

// exp(x) through the hardware base-2 exponential.
SSD_DEV float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
SSD_DEV float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kLog2e = 1.4426950408889634f;
SSD_DEV float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
SSD_DEV float silu(float u) { return u * frcp(1.0f + fexp(-u)); }

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
SSD_DEV uint32_t pack_bf16x2(float a, float b) {
  bf16 lo = (bf16)a, hi = (bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}
SSD_DEV void store8(bf16* p, const float (&v)[8]) {
  uint4 a;
  a.x = pack_bf16x2(v[0], v[1]);
  a.y = pack_bf16x2(v[2], v[3]);
  a.z = pack_bf16x2(v[4], v[5]);
  a.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = a;
}

// ---- wave64 reductions ----------------------------------------------------
SSD_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Sum over aligned groups of `width` lanes (width a power of two <= 64).
SSD_DEV float group_sum(float v, int width) {
  for (int o = width >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---- MFMA fragments ---------------------------------------------------------
// 16x16 output tile, fp32 accumulate. For one MFMA of depth KSTEP, lane l
// holds KPL consecutive k values starting at k = KPL * (l / 16) of row
// (A operand) or column (B operand) l % 16; the output lane l holds rows
// 4 * (l / 16) + r, r < 4, of column l % 16.
template <class T> struct Mfma;
template <> struct Mfma<bf16> {
  static constexpr int KPL = 8, KSTEP = 32;
  typedef bf16x8 frag;
  static SSD_DEV f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // KPL consecutive operand values from LDS / memory of the operand type.
  static SSD_DEV frag ld(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  // KPL consecutive values converted from fp32.
  static SSD_DEV frag cvt(const float* p) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    frag f;
    f[0] = (bf16)a.x; f[1] = (bf16)a.y; f[2] = (bf16)a.z; f[3] = (bf16)a.w;
    f[4] = (bf16)b.x; f[5] = (bf16)b.y; f[6] = (bf16)b.z; f[7] = (bf16)b.w;
    return f;
  }
};
template <> struct Mfma<float> {
  static constexpr int KPL = 1, KSTEP = 4;
  typedef float frag;
  static SSD_DEV f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static SSD_DEV frag ld(const float* p) { return *p; }
  static SSD_DEV frag cvt(const float* p) { return *p; }
};

SSD_DEV f32x4 zero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }
