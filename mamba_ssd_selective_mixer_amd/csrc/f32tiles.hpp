// fp32 MFMA tile helpers shared by the kernels that run the chunked scan on
// fp32 operands in 64-token chunks (the general output kernel and the
// backward pass): staging of operand slices through registers into LDS,
// the causal tile split over four waves, and the chunk's Lam.
#pragma once
#include "common.hpp"

namespace ssd {
namespace f32t {

SSD_DEV float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
SSD_DEV float4 ld4(const bf16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
SSD_DEV void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
SSD_DEV void st4(bf16* p, float4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

constexpr int kThreads = 256;
constexpr int kQ = 64;           // chunk length
constexpr int kQP = kQ + 4;      // pitch of the Q x Q tiles (floats)
constexpr int kKS = 32;          // width of a staged operand slice
constexpr int kSP = kKS + 4;     // pitch of a staged slice

// MFMA 16x16x4 fp32. Lane l supplies A[row l%16][k l/16] and B[k l/16][col
// l%16]; acc[r] is C[row 4 (l/16) + r][col l%16].
SSD_DEV f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// One staged slice (rows [0, ROWS) x columns [0, kKS)) held in registers
// between its global loads and its LDS stores, so that the next slice's
// loads are in flight while the current one is computed on.
template <int ROWS>
struct SliceRegs {
  static constexpr int kItems = ROWS * (kKS / 4), kN = (kItems + kThreads - 1) / kThreads;
  float4 v[kN];
  template <class TX>
  SSD_DEV void load(const TX* src, int rs, int nrows, int ncols) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int idx = threadIdx.x + i * kThreads, r = idx / (kKS / 4), c4 = (idx % (kKS / 4)) * 4;
      v[i] = (idx < kItems && r < nrows && c4 < ncols) ? ld4(src + r * rs + c4)
                                                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  SSD_DEV void store(float* dst) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int idx = threadIdx.x + i * kThreads, r = idx / (kKS / 4), c4 = (idx % (kKS / 4)) * 4;
      if (idx < kItems) *reinterpret_cast<float4*>(dst + r * kSP + c4) = v[i];
    }
  }
};

// Rows [0, rows) x columns [0, cols) (a multiple of 4) of a row-major fp32
// or bf16 matrix into dst [rows][pitch] (fp32), scaled per row by sc[r] when sc is given;
// rows >= nrows are zero. A pitch of 16 (mod 64) floats keeps column-wise
// fragment reads (16 columns x 4 rows per wave) free of bank conflicts.
template <class TX>
SSD_DEV void stage_rows(float* dst, int pitch, const TX* src, int rs, int rows, int nrows,
                        int cols, const float* sc = nullptr) {
  const int c4n = cols / 4;
  for (int i = threadIdx.x; i < rows * c4n; i += kThreads) {
    const int r = i / c4n, c4 = (i % c4n) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < nrows) {
      v = ld4(src + r * rs + c4);
      if (sc) {
        const float f = sc[r];
        v.x *= f;
        v.y *= f;
        v.z *= f;
        v.w *= f;
      }
    }
    *reinterpret_cast<float4*>(dst + r * pitch + c4) = v;
  }
}

// The same rows transposed: dst [cols][pitch], element (r, c) at c * pitch +
// r, so a column's consecutive rows are contiguous (k-contiguous operand
// reads for a contraction over the rows); scaled per row by sc[r] when sc
// is given; rows >= nrows are zero.
template <class TX>
SSD_DEV void stage_cols(float* dst, int pitch, const TX* src, int rs, int rows, int nrows,
                        int cols, const float* sc = nullptr) {
  const int c4n = cols / 4;
  for (int i = threadIdx.x; i < rows * c4n; i += kThreads) {
    const int r = i % rows, c4 = (i / rows) * 4;
    float4 v = r < nrows ? ld4(src + r * rs + c4) : make_float4(0.f, 0.f, 0.f, 0.f);
    if (sc && r < nrows) {
      const float f = sc[r];
      v.x *= f;
      v.y *= f;
      v.z *= f;
      v.w *= f;
    }
    dst[(c4 + 0) * pitch + r] = v.x;
    dst[(c4 + 1) * pitch + r] = v.y;
    dst[(c4 + 2) * pitch + r] = v.z;
    dst[(c4 + 3) * pitch + r] = v.w;
  }
}

// The ten causal 16x16 tiles (rt, st), st <= rt, of a 64 x 64 block spread
// over the four waves (at most three each): whether slot i of wave w holds one.
SSD_DEV bool causal_tile(int w, int i, int& rt, int& st) {
  if (w == 3) {
    rt = 3;
    st = 3;
    return i == 0;
  }
  if (w == 0) {
    rt = i == 0 ? 0 : 1;
    st = i == 0 ? 0 : i - 1;
    return true;
  }
  rt = w + 1;
  st = i;
  return true;
}

// chunk Lam
// Lam (inclusive cumsum of dt A over the chunk, natural log units), dt and
// exp(Lam) of the first len positions into lam / dts / ex (wave 0).
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


}  // namespace f32t
}  // namespace ssd
