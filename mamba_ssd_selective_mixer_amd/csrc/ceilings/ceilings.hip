// Machine ceilings measured on the GPU the benchmark runs on, so the mixer
// kernels' fractions can be read against what this GPU reaches with the
// simplest possible kernel of each kind (a separate library: nothing of the
// mixer path uses it).
//   ceil_copy: a streaming device-to-device copy (16-byte non-temporal loads
//              and stores, grid-stride), the pattern of a kernel that reads
//              and writes each byte once.
//   ceil_mfma: only fp16 16x16x32 MFMA instructions with fp32 accumulation,
//              eight independent chains per wave, no memory traffic besides
//              one store per lane at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_copy(const u32x4* __restrict__ src,
                                              u32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void k_mfma(float* __restrict__ out, int iters) {
  f16x8 a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = (_Float16)(0.001f * (threadIdx.x + j));
    b[j] = (_Float16)(0.002f * (blockIdx.x + j));
  }
  f32x4 acc[kChains];
  for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Copy nbytes (a multiple of 16) from src to dst on `stream` with `blocks`
// workgroups of 256 threads. Returns 0, or -1 for bad arguments / a failed
// launch.
int ceil_copy(const void* src, void* dst, int64_t nbytes, int blocks, void* stream) {
  if (!src || !dst || nbytes <= 0 || nbytes % 16 || blocks <= 0) return -1;
  hipLaunchKernelGGL(k_copy, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, (u32x4*)dst, nbytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// `blocks` workgroups of 256 threads each run `iters` x 8 MFMA per wave;
// out needs blocks * 256 floats. Dense FLOPs issued:
// blocks * 4 waves * iters * 8 * (2 * 16 * 16 * 32).
int ceil_mfma(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(k_mfma, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
