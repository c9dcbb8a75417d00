// Host-side launchers of the gfx950 kernels (one per kernel family). The
// C-ABI layer validates every argument before it calls any of these.
#pragma once
#include <hip/hip_runtime.h>

#include "prof.hpp"
#include <stdint.h>

namespace ssd {

struct ScanShape {
  int B, L, H, P, G, N, Q, nc;
};

// Depthwise causal conv + SiLU; io_bf16 selects bf16 (else fp32) elements;
// out_f32 writes the output in fp32 whatever the I/O type.
hipError_t launch_conv1d(bool io_bf16, int B, int L, int C, int W, const void* xbc,
                         int64_t xs, const void* w, const void* bias, const void* cin,
                         void* out, int64_t os, bool out_f32, hipStream_t st);
// conv_out[b] = last W-1 rows of [cin[b] ; xbc[b]] (safe when cout == cin).
hipError_t launch_conv_state(bool io_bf16, int B, int L, int C, int W, const void* xbc,
                             int64_t xs, const void* cin, void* cout, hipStream_t st);
// Grouped gated RMSNorm; y_f32 says y is fp32 (else io dtype).
hipError_t launch_gated_norm(bool io_bf16, bool y_f32, int rows, int HP, int G,
                             const void* y, const void* z, const void* w, float eps,
                             void* out, hipStream_t st);
// One decode token per sequence.
hipError_t launch_decode(bool io_bf16, int B, int H, int P, int G, int N, int W,
                         const void* xbc, const void* z, const void* dt, const float* A,
                         const float* D, const void* cw, const void* cb, const void* nw,
                         float eps, void* conv_state, float* ssm_state, void* y,
                         hipStream_t st);
// Chunked scan, three phases: chunk states, state passing, chunk outputs.
// x_f32: x, B and C are fp32 (else the I/O type); dt and y are the I/O type.
hipError_t launch_chunk_state(bool io_bf16, bool x_f32, const ScanShape& s, const void* x,
                              int64_t xs, const void* dt, const float* A, const void* Bm,
                              int64_t bs, float* states, float* lam_end, hipStream_t st);
hipError_t launch_state_pass(const ScanShape& s, float* states, const float* lam_end,
                             const float* s_in, float* s_out, hipStream_t st);
hipError_t launch_chunk_out(bool io_bf16, bool x_f32, const ScanShape& s, const void* x,
                            int64_t xs, const void* dt, const float* A, const float* D,
                            const void* Bm, const void* Cm, int64_t bs, const float* states,
                            void* y, bool y_f32, hipStream_t st);

}  // namespace ssd

namespace ssd {

// Fast path (head_dim 64, d_state 128, bf16, heads per group a multiple of 4).
struct FastScanArgs {
  int B, L, H, G;
  const void* x;      // x rows (conv mode: the raw xBC rows)
  const void* Bm;     // B rows (conv mode: xBC + H*P)
  const void* Cm;     // C rows (conv mode: xBC + H*P + G*N)
  int64_t xs, bs;     // token strides (elements)
  const void* dt;
  const float* A;
  const float* D;
  bool conv;          // recompute conv + SiLU from raw xBC rows
  const void* conv_w;
  const void* conv_b;
  const void* conv_in;
  const void* z;      // null: y is the scan output
  const void* norm_w;
  float eps;
  const float* s_in;
  float* s_out;
  void* y;            // [B, L, H*P] bf16: the normalised output (z given) or y
  void* ws;           // fast_ws_bytes(B, L, H, G, conv) bytes, 256-byte aligned
};
bool fast_path_ok(bool io_bf16, int P, int N, int H, int G, int Q, int W, bool conv);
size_t fast_ws_bytes(int B, int L, int H, int G, bool conv);
hipError_t launch_fast_scan(const FastScanArgs& a, hipStream_t st);

}  // namespace ssd
