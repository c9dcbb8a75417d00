// Host-side launchers of the gfx950 kernels (one per kernel family). The
// C-ABI layer validates every argument before it calls any of these.
#pragma once
#include <hip/hip_runtime.h>

#include "dta.hpp"
#include "prof.hpp"
#include <stdint.h>

namespace ssd {

struct ScanShape {
  int B, L, H, P, G, N, Q, nc;
  DtA dta;  // dt's token stride, and raw dt + bias / A_log or dt / A as given
};

// Depthwise causal conv + SiLU; io_bf16 selects bf16 (else fp32) elements;
// out_f32 writes the output in fp32 whatever the I/O type.
hipError_t launch_conv1d(bool io_bf16, int B, int L, int C, int W, const void* xbc,
                         int64_t xs, const void* w, const void* bias, const void* cin,
                         void* out, int64_t os, bool out_f32, hipStream_t st);
// conv_out[b] = last W-1 rows of [cin[b] ; xbc[b]] (safe when cout == cin).
hipError_t launch_conv_state(bool io_bf16, int B, int L, int C, int W, const void* xbc,
                             int64_t xs, const void* cin, void* cout, hipStream_t st);
// Grouped gated RMSNorm; y_f32 says y is fp32 (else io dtype); zs: token
// stride of z (elements; y and out are dense).
hipError_t launch_gated_norm(bool io_bf16, bool y_f32, int rows, int HP, int G,
                             const void* y, const void* z, int64_t zs, const void* w, float eps,
                             void* out, hipStream_t st);
// One decode token per sequence; xrs, zrs: row strides (elements) of the
// token's xBC and z; dta: dt's row stride and preprocessing.
hipError_t launch_decode(bool io_bf16, int B, int H, int P, int G, int N, int W,
                         const void* xbc, int64_t xrs, const void* z, int64_t zrs,
                         const void* dt, const DtA& dta, const float* A, const float* D,
                         const void* cw, const void* cb, const void* nw, float eps,
                         void* conv_state, float* ssm_state, void* y, hipStream_t st);
// Chunked scan, three phases: chunk states, state passing, chunk outputs
// (the last in launch_chunk_y below).
// x_f32: x, B and C are fp32 (else the I/O type); dt and y are the I/O type.
// f32op: fp32 MFMA operands for bf16 I/O too (else fp16). status: the call's
// status word, cleared by the chunk-state kernel; the others set bits in it.
hipError_t launch_chunk_state(bool io_bf16, bool x_f32, bool f32op, const ScanShape& s,
                              const void* x, int64_t xs, const void* dt, const float* A,
                              const void* Bm, int64_t bs, float* states, float* lam_end,
                              int* status, hipStream_t st);
hipError_t launch_state_pass(const ScanShape& s, float* states, const float* lam_end,
                             const float* s_in, float* s_out, int* status, hipStream_t st);
// The grouped gated RMSNorm fused into the chunk-output kernel: z (I/O
// type, token stride zs), the norm weight w [H P] (I/O type) and eps.
struct YNorm {
  const void* z;
  int64_t zs;
  const void* w;
  float eps;
};
// Whether the output kernel can fuse the norm: a norm group of 1, 2, 4 or
// 8 heads and at most 256 channels (one workgroup holds it in registers).
bool chunk_y_fuses_norm(int H, int G, int P);
// Chunk outputs on fp32 MFMA operands (s.Q must be 64): y = M X + exp(Lam)
// C S_in^T + D X. x_f32: x, B, C fp32 (else the I/O type); y_f32: y fp32
// (else the I/O type). cb: chunk_cb_bytes of workspace, filled first with
// each chunk's C B^T per group (launch_chunk_cb). kid: the kernel id the
// timing aid records the output kernel under. norm: when given (and
// chunk_y_fuses_norm holds), y is the normalised output in the I/O type
// (y_f32 must then say whether the I/O type is fp32).
hipError_t launch_chunk_y(bool io_bf16, bool x_f32, bool y_f32, const ScanShape& s,
                          const void* x, int64_t xs, const void* Bm, const void* Cm, int64_t bs,
                          float* cb, const void* dt, const float* A, const float* D,
                          const float* states, void* y, int* status, int kid, hipStream_t st,
                          const YNorm* norm = nullptr);
// C B^T of each 64-token chunk and group on the causal 16x16 tiles into cb
// [B][nc][G][64][64] (fp32; element (t, s) at t 64 + s). x_bf16: B and C
// are bf16 (else fp32).
hipError_t launch_chunk_cb(bool x_bf16, const ScanShape& s, const void* Bm, const void* Cm,
                           int64_t bs, float* cb, hipStream_t st);
size_t chunk_cb_bytes(int B, int nc, int G);
size_t chunk_y_lds_bytes(int P);

}  // namespace ssd

namespace ssd {

// Ragged sequences over a state pool (continuous batching), or a dense batch
// when cu is null. The chunk table (chunk_seq, chunk_first, valid) is built
// on the device at the start of the call.
struct Seqs {
  const int32_t* cu;           // [nseq + 1] token offsets; null: dense batch
  const int32_t* chunk_seq;    // [chunks] sequence owning each global chunk, -1 none
  const int32_t* chunk_first;  // [nseq + 1] first global chunk of each sequence
  const int32_t* slots;        // [nseq] state slot of each sequence
  const uint8_t* has_state;    // [nseq] resume from the slot (else zeros), or null: all
  const int* valid;            // 1 when the call's metadata passed the device checks
  const int32_t* nchunks;      // [1] chunks the table holds (chunk_first[nseq])
  const int32_t* pre;          // sequences with two or more tokens, in order
  const int32_t* npre;         // [1] their count
  void* conv_pool;             // [slots, W-1, Cch] io dtype
  float* ssm_pool;             // [slots, H, P, N] fp32
};

// Fast path (head_dim 64, d_state 128, bf16, heads per group a multiple of 4).
struct FastScanArgs {
  int B, L, H, G;
  const void* x;      // x rows (conv mode: the raw xBC rows)
  const void* Bm;     // B rows (conv mode: xBC + H*P)
  const void* Cm;     // C rows (conv mode: xBC + H*P + G*N)
  int64_t xs, bs;     // token strides (elements)
  const void* dt;
  const float* A;     // A, or A_log when dt_bias is set
  const float* D;
  int64_t dts, zs;    // token strides of dt and z (elements)
  const float* dt_bias;  // null: dt and A as given; else dt = softplus(dt + bias), A = -exp(A)
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
  int* status;        // the call's status word (cleared by the first kernel)
  int spin_max;       // bound on the cross-block norm's polls
  // ragged batch (q.cu set): B sequences packed back to back (L = total
  // tokens); states in pool slots; the table lives in the workspace
  Seqs q;
  int num_slots;
};
bool fast_path_ok(bool io_bf16, int P, int N, int H, int G, int Q, int W, bool conv);
size_t fast_ws_bytes(int B, int L, int H, int G, bool conv);
// ragged batch of nseq sequences, T tokens in all, over a pool of num_slots
size_t fast_varlen_ws_bytes(int nseq, int T, int H, int G, int num_slots);
// most 4-head blocks per norm group the fused exchange handles
int fast_max_norm_heads();
hipError_t launch_fast_scan(const FastScanArgs& a, hipStream_t st);
// The one-token sequences of a ragged batch, one decode step each: dec lists
// them (dec[nseq] holds their count); token rows from q.cu, states in the
// pool slots (zeros for a fresh sequence); skipped when q.valid is not 1.
hipError_t launch_decode_varlen(bool io_bf16, int nseq, int H, int P, int G, int N, int W,
                                const void* xbc, int64_t xrs, const void* z, int64_t zrs,
                                const void* dt, const DtA& dta, const float* A, const float* D,
                                const void* cw, const void* cb, const void* nw, float eps,
                                const Seqs& q, const int32_t* dec, void* y, hipStream_t st);

}  // namespace ssd

namespace ssd {

// Backward pass of the mixer prefill (conv + SiLU, chunked scan, gated norm).
// Activation gradients in the I/O type, parameter and state gradients fp32.
struct BackwardArgs {
  bool io_bf16;
  int B, L, H, P, G, N, W;
  const void* xbc;      // [B, L, Cch]
  const void* z;        // [B, L, H*P]
  const void* dt;       // [B, L, H] (after softplus)
  const float* A;       // [H] (negative)
  const float* D;       // [H] or null (zero)
  const void* conv_w;   // [Cch, W]
  const void* conv_b;   // [Cch] or null
  const void* norm_w;   // [H*P]
  float eps;
  const void* conv_in;  // [B, W-1, Cch] or null (zeros)
  const float* s_in;    // [B, H, P, N] or null (zeros)
  const void* d_out;    // [B, L, H*P]
  const float* d_s_out; // [B, H, P, N] or null (zero)
  void* d_xbc;          // [B, L, Cch]
  void* d_z;            // [B, L, H*P]
  void* d_dt;           // [B, L, H]
  float* d_A;           // [H]
  float* d_D;           // [H] or null
  float* d_conv_w;      // [Cch, W]
  float* d_conv_b;      // [Cch] or null
  float* d_norm_w;      // [H*P]
  float* d_conv_in;     // [B, W-1, Cch] or null
  float* d_s_in;        // [B, H, P, N] or null
  void* ws;             // backward_ws_bytes(...) bytes, 256-byte aligned
  int* status;          // the call's status word
  int chunk_heads;      // heads per workgroup of the per-chunk kernels; 0: chosen from the shape
};
size_t backward_ws_bytes(int B, int L, int H, int P, int G, int N);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t st);

}  // namespace ssd
