// Depthwise causal conv1d + SiLU over the xBC channels, and the carried conv
// state ("feat(model): Nemotron-H hybrid ... on the CPU", section
// "2. feat(model)": the CausalConv1D op of the Mamba2 mixer).
//
// out[b,t,c] = silu(bias[c] + sum_k w[c,k] * ext[b,t+k,c]) with
// ext[b] = conv_state_in[b] (W-1 rows, oldest first) followed by xbc[b].
// Each thread owns 8 adjacent channels (one 16-byte bf16 vector) over a run
// of kConvTT tokens and keeps the W-1 previous rows in registers, so every
// input row is read once per run (plus a W-1 row halo) with coalesced
// 16/32-byte accesses across the channel dimension.
#include "common.hpp"
#include "launch.hpp"

namespace ssd {

constexpr int kConvTT = 32;   // tokens per thread
constexpr int kConvAhead = 4; // input rows loaded ahead of their use
constexpr int kConvThreads = 256;

// TO: output element type (the I/O type, or fp32 for the scan's internal copy)
template <class T, class TO, int W>
__global__ __launch_bounds__(kConvThreads) void k_conv1d(
    const T* __restrict__ xbc, int64_t xs, const T* __restrict__ w,
    const T* __restrict__ bias, const T* __restrict__ cin, TO* __restrict__ out,
    int64_t os, int L, int C) {
  const int cv = blockIdx.x * kConvThreads + threadIdx.x;
  if (cv * 8 >= C) return;
  const int c0 = cv * 8;
  const int b = blockIdx.z;
  const int t0 = blockIdx.y * kConvTT;
  float wk[W][8], bi[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int k = 0; k < W; ++k) wk[k][j] = to_f(w[(int64_t)(c0 + j) * W + k]);
    bi[j] = bias ? to_f(bias[c0 + j]) : 0.f;
  }
  float win[W][8];  // rows t-W+1 .. t-1 in win[0..W-2]
#pragma unroll
  for (int r = 0; r < W - 1; ++r) {
    const int t = t0 - (W - 1) + r;
    if (t >= 0) {
      load8(xbc + ((int64_t)b * L + t) * xs + c0, win[r]);
    } else if (cin) {
      load8(cin + ((int64_t)b * (W - 1) + (W - 1 + t)) * C + c0, win[r]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) win[r][j] = 0.f;
    }
  }
  const int tend = min(L, t0 + kConvTT);
  // one output row from win[] (its newest row in win[W-1]), then the window
  // slides by one
  auto step = [&](int t) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float u = bi[j];
#pragma unroll
      for (int k = 0; k < W; ++k) u += wk[k][j] * win[k][j];
      v[j] = silu(u);
    }
    store8(out + ((int64_t)b * L + t) * os + c0, v);
#pragma unroll
    for (int r = 0; r < W - 1; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j) win[r][j] = win[r + 1][j];
  };
  // kConvAhead rows are loaded before any of them is used, so a short run
  // does not wait one memory latency per token
  int t = t0;
  for (; t + kConvAhead <= tend; t += kConvAhead) {
    float rows[kConvAhead][8];
#pragma unroll
    for (int q = 0; q < kConvAhead; ++q) load8(xbc + ((int64_t)b * L + t + q) * xs + c0, rows[q]);
#pragma unroll
    for (int q = 0; q < kConvAhead; ++q) {
#pragma unroll
      for (int j = 0; j < 8; ++j) win[W - 1][j] = rows[q][j];
      step(t + q);
    }
  }
  for (; t < tend; ++t) {
    load8(xbc + ((int64_t)b * L + t) * xs + c0, win[W - 1]);
    step(t);
  }
}

// conv_out[b, r] = ext[b, L + r] for r < W-1. Rows are visited in increasing
// r by the thread that owns the channels, so cout == cin is safe: row L + r
// of the old state is read before any row >= L + r is overwritten.
template <class T, int W>
__global__ __launch_bounds__(kConvThreads) void k_conv_state(
    const T* __restrict__ xbc, int64_t xs, const T* cin, T* cout, int L, int C) {
  const int cv = blockIdx.x * kConvThreads + threadIdx.x;
  if (cv * 8 >= C) return;
  const int c0 = cv * 8;
  const int b = blockIdx.y;
#pragma unroll
  for (int r = 0; r < W - 1; ++r) {
    const int e = L + r;
    float v[8];
    if (e >= W - 1) {
      load8(xbc + ((int64_t)b * L + (e - (W - 1))) * xs + c0, v);
    } else if (cin) {
      load8(cin + ((int64_t)b * (W - 1) + e) * C + c0, v);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.f;
    }
    store8(cout + ((int64_t)b * (W - 1) + r) * C + c0, v);
  }
}

template <class T, class TO>
static hipError_t conv_dispatch(int B, int L, int C, int W, const void* xbc, int64_t xs,
                                const void* w, const void* bias, const void* cin, void* out,
                                int64_t os, hipStream_t st) {
  dim3 grid((C / 8 + kConvThreads - 1) / kConvThreads, (L + kConvTT - 1) / kConvTT, B);
  const T* X = (const T*)xbc;
  const T* Wt = (const T*)w;
  const T* Bi = (const T*)bias;
  const T* Ci = (const T*)cin;
  TO* O = (TO*)out;
  const dim3 blk(kConvThreads);
  switch (W) {
    case 2: hipLaunchKernelGGL((k_conv1d<T, TO, 2>), grid, blk, 0, st, X, xs, Wt, Bi, Ci, O, os, L, C); break;
    case 3: hipLaunchKernelGGL((k_conv1d<T, TO, 3>), grid, blk, 0, st, X, xs, Wt, Bi, Ci, O, os, L, C); break;
    default: hipLaunchKernelGGL((k_conv1d<T, TO, 4>), grid, blk, 0, st, X, xs, Wt, Bi, Ci, O, os, L, C); break;
  }
  return hipGetLastError();
}

hipError_t launch_conv1d(bool io_bf16, int B, int L, int C, int W, const void* xbc, int64_t xs,
                         const void* w, const void* bias, const void* cin, void* out, int64_t os,
                         bool out_f32, hipStream_t st) {
  ProfScope ps(st, KID_CONV1D);
  if (!io_bf16) return conv_dispatch<float, float>(B, L, C, W, xbc, xs, w, bias, cin, out, os, st);
  return out_f32 ? conv_dispatch<bf16, float>(B, L, C, W, xbc, xs, w, bias, cin, out, os, st)
                 : conv_dispatch<bf16, bf16>(B, L, C, W, xbc, xs, w, bias, cin, out, os, st);
}

template <class T>
static hipError_t conv_state_dispatch(int B, int L, int C, int W, const void* xbc, int64_t xs,
                                      const void* cin, void* cout, hipStream_t st) {
  dim3 grid((C / 8 + kConvThreads - 1) / kConvThreads, B);
  const T* X = (const T*)xbc;
  const T* Ci = (const T*)cin;
  T* Co = (T*)cout;
  switch (W) {
    case 2: hipLaunchKernelGGL((k_conv_state<T, 2>), grid, dim3(kConvThreads), 0, st, X, xs, Ci, Co, L, C); break;
    case 3: hipLaunchKernelGGL((k_conv_state<T, 3>), grid, dim3(kConvThreads), 0, st, X, xs, Ci, Co, L, C); break;
    default: hipLaunchKernelGGL((k_conv_state<T, 4>), grid, dim3(kConvThreads), 0, st, X, xs, Ci, Co, L, C); break;
  }
  return hipGetLastError();
}

hipError_t launch_conv_state(bool io_bf16, int B, int L, int C, int W, const void* xbc,
                             int64_t xs, const void* cin, void* cout, hipStream_t st) {
  ProfScope ps(st, KID_CONV_STATE);
  return io_bf16 ? conv_state_dispatch<bf16>(B, L, C, W, xbc, xs, cin, cout, st)
                 : conv_state_dispatch<float>(B, L, C, W, xbc, xs, cin, cout, st);
}

}  // namespace ssd
