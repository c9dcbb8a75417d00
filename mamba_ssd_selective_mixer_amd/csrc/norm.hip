// Grouped gated RMSNorm ("feat(model): Nemotron-H hybrid ... on the CPU",
// section "2. feat(model)": GatedRMSNorm after the scan; "feat(model): add
// Nemotron-3 Nano hybrid ..." attribution commit: GatedRMSNorm semantics).
//
// For each row and each of G groups of S = HP/G contiguous channels:
//   q = y * silu(z);  out = q * w / sqrt(mean(q^2) + eps).
// One workgroup per row; each wave takes whole groups. When a group fits in
// kNormVec 8-channel vectors per lane (S <= 64 * 8 * kNormVec), q stays in
// registers between the sum of squares and the scaled store, so y, z and
// the SiLU are touched once; larger groups re-read y and z (from L1/L2).
#include "common.hpp"
#include "launch.hpp"

namespace ssd {

constexpr int kNormVec = 4;

template <class T, class TY>
__global__ __launch_bounds__(256) void k_gated_norm(const TY* y,
                                                    const T* __restrict__ z, int64_t zs,
                                                    const T* __restrict__ w, float eps,
                                                    T* out, int HP, int G) {
  const int64_t row = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int S = HP / G, S8 = S / 8;
  const float inv_S = 1.0f / (float)S;
  if (S8 <= 64 * kNormVec) {
    for (int j = wave; j < G; j += 4) {
      const int64_t base = row * HP + (int64_t)j * S;
      const int64_t zbase = row * zs + (int64_t)j * S;
      float q[kNormVec][8];
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < kNormVec; ++k) {
        const int v = lane + 64 * k;
        if (v < S8) {
          float yv[8], zv[8];
          load8(y + base + v * 8, yv);
          load8_stream(z + zbase + v * 8, zv);  // z is read once
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            q[k][i] = yv[i] * silu(zv[i]);
            ss += q[k][i] * q[k][i];
          }
        }
      }
      ss = wave_sum(ss);
      const float inv = __builtin_amdgcn_rsqf(ss * inv_S + eps);
#pragma unroll
      for (int k = 0; k < kNormVec; ++k) {
        const int v = lane + 64 * k;
        if (v < S8) {
          float wv[8], o[8];
          load8(w + (int64_t)j * S + v * 8, wv);
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] = q[k][i] * wv[i] * inv;
          store8_stream(out + base + v * 8, o);  // final output, not read back
        }
      }
    }
    return;
  }
  for (int j = wave; j < G; j += 4) {
    const int64_t base = row * HP + (int64_t)j * S;
    const int64_t zbase = row * zs + (int64_t)j * S;
    float ss = 0.f;
    for (int v = lane; v < S8; v += 64) {
      float yv[8], zv[8];
      load8(y + base + v * 8, yv);
      load8(z + zbase + v * 8, zv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q = yv[i] * silu(zv[i]);
        ss += q * q;
      }
    }
    ss = wave_sum(ss);
    const float inv = __builtin_amdgcn_rsqf(ss * inv_S + eps);
    for (int v = lane; v < S8; v += 64) {
      float yv[8], zv[8], wv[8], o[8];
      load8(y + base + v * 8, yv);
      load8(z + zbase + v * 8, zv);
      load8(w + (int64_t)j * S + v * 8, wv);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = yv[i] * silu(zv[i]) * wv[i] * inv;
      store8(out + base + v * 8, o);
    }
  }
}

hipError_t launch_gated_norm(bool io_bf16, bool y_f32, int rows, int HP, int G, const void* y,
                             const void* z, int64_t zs, const void* w, float eps, void* out,
                             hipStream_t st) {
  ProfScope ps(st, KID_GATED_NORM);
  dim3 grid(rows), block(256);
  if (io_bf16) {
    if (y_f32)
      hipLaunchKernelGGL((k_gated_norm<bf16, float>), grid, block, 0, st, (const float*)y,
                         (const bf16*)z, zs, (const bf16*)w, eps, (bf16*)out, HP, G);
    else
      hipLaunchKernelGGL((k_gated_norm<bf16, bf16>), grid, block, 0, st, (const bf16*)y,
                         (const bf16*)z, zs, (const bf16*)w, eps, (bf16*)out, HP, G);
  } else {
    hipLaunchKernelGGL((k_gated_norm<float, float>), grid, block, 0, st, (const float*)y,
                       (const float*)z, zs, (const float*)w, eps, (float*)out, HP, G);
  }
  return hipGetLastError();
}

}  // namespace ssd
