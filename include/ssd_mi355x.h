/*
 * ssd_mi355x.h — C ABI of the MI355X (gfx950) Mamba-2 mixer core.
 *
 * The mixer core every Mamba-2 ("M") layer of a Nemotron-H hybrid runs
 * between its input and output projections: a depthwise causal conv1d with
 * SiLU over xBC, the selective state-space scan (computed by the chunked
 * state-space-duality block decomposition), and a grouped gated RMSNorm,
 * plus a single-token decode update of the per-sequence conv and SSM state.
 * ("feat(model): Nemotron-H hybrid (Mamba2 + attention + MoE) on the CPU",
 * section "2. feat(model): Nemotron-H on the CPU": in_proj, then
 * CausalConv1D, SSMScan and GatedRMSNorm, then out_proj, with the state kept
 * in per-sequence slots.)
 *
 * What is computed (b batch, t token, h head, p < P, n < N, g(h) = h/(H/G)):
 *   conv:  u[b,t,c] = bias[c] + sum_{k<W} w[c,k] * ext[b,t+k,c],
 *          ext[b] = conv_state_in[b] (W-1 rows, oldest first; zeros if NULL)
 *                   followed by xbc[b];  v = u * sigmoid(u).
 *          Channel order of xbc / v: x (H*P) | B (G*N) | C (G*N) (the packed
 *          [z, x, B, C, dt] projection layout of "feat(model): add
 *          Nemotron-3 Nano hybrid ..." attribution commit).
 *   scan:  S_b,h = ssm_state_in (or 0); for each t:
 *            S = exp(dt[t,h]*A[h]) * S + dt[t,h] * x[t,h,:] (outer) B[t,g(h),:]
 *            y[t,h,p] = sum_n S[p,n] * C[t,g(h),n] + D[h] * x[t,h,p]
 *          ssm_state_out = S after the last token. Computed chunk by chunk:
 *          intra-chunk quadratic form masked by the segment-sum decay plus the
 *          state carried across chunks (Modalities PR attribution commit:
 *          ssd_minimal_discrete / segsum); identical in exact arithmetic for
 *          every chunk length.
 *   norm:  for each row and each of G groups of H*P/G contiguous channels:
 *            q = y * silu(z);  out = q * w / sqrt(mean_group(q^2) + eps).
 *   decode: the same chain for one token per sequence, with the conv state
 *          shifted by one row and the SSM state updated in place ("Validation":
 *          token-by-token decode resuming every Mamba layer from its slot).
 *
 * Conventions the pages leave open (stated here, checked against the
 * library's own fp64 reference only): tap w[c][W-1] multiplies the current
 * token; SiLU covers all of xBC; head h reads B/C group h / (H/G); the norm
 * gates first and normalises over contiguous channel groups; dt arrives
 * positive (already softplus-ed) and A negative.
 *
 * Types and layouts. Every pointer is a DEVICE pointer (HBM) except `dims`,
 * which is a host pointer. Tensors are row-major with the innermost
 * dimension contiguous; token strides are in elements. A, D and SSM states
 * are fp32; every other tensor is in dims->io_dtype (fp32 or bf16).
 * All device pointers must be 16-byte aligned, and token strides times the
 * element size must be multiples of 16 bytes.
 *
 * Ownership. The caller owns every buffer and the stream; the library
 * allocates no device memory and keeps no mutable global state apart from
 * the opt-in timing aid declared at the end of this header. Scratch
 * space comes from a caller-provided workspace of at least the size the
 * matching *_workspace_bytes() call returns (256-byte aligned).
 *
 * Errors and asynchrony. Every entry checks its arguments on the host and
 * returns a negative ssd_status before launching anything if one is wrong;
 * unsupported shapes are refused (SSD_ERR_UNSUPPORTED), never computed
 * wrongly. On success the work is enqueued asynchronously on `stream`
 * (a hipStream_t; NULL = the default stream) and SSD_OK is returned. A failed
 * launch returns SSD_ERR_HIP. Calls on one stream run in order; calls that
 * share buffers on different streams race.
 *
 * Supported envelope: batch >= 1, seqlen >= 1 (any length; the last chunk
 * may be short), nheads % ngroups == 0, headdim in {16, 32, 64, 128},
 * dstate in {16, 32, 64, 128}, conv_width in {2, 3, 4},
 * chunk in {32, 64, 128, 256}.
 *
 * Precision. State, decay exponents, sums and the norm are fp32. The dense
 * contractions of the chunked scan run on MFMA with fp32 accumulation: with
 * fp32 operands for fp32 I/O and fp16 operands for bf16 I/O (B, C, x scaled
 * by dt or the decay weights, the decay-masked C B^T and the carried-in
 * states; in the fast path, used for bf16 I/O with headdim 64, dstate 128,
 * heads per group a multiple of 4, dims->chunk >= 64 and conv width 4 when
 * the call includes the conv, also the chunk states, and D x taken from x at
 * fp16 hi + lo precision). Such operands must stay within fp16 range (|v| < 65504):
 * activations after SiLU, dt-weighted states of magnitude beyond that are
 * outside the fast path's envelope. In the fast path the chunk length is an
 * internal choice (128 tokens); the result does not depend on dims->chunk
 * beyond rounding. The fast path fuses the gated norm into its chunk-output
 * kernel, also when a norm group spans several (up to 32) of that kernel's
 * 4-head blocks: their per-token sums of squares are exchanged through the
 * workspace, which needs the group's blocks to run concurrently (a stream
 * with the whole GPU qualifies: 512 resident workgroups, 64 per XCD, against
 * at most 31 waiting per XCD). A wait that cannot complete writes NaN rows
 * after a bounded time instead of hanging. Wider norm groups are normalised
 * by a separate pass over the scan output.
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSD_OK = 0,
  SSD_ERR_NULL = -1,        /* a required pointer is NULL                   */
  SSD_ERR_SHAPE = -2,       /* a size is zero/negative or sizes disagree     */
  SSD_ERR_UNSUPPORTED = -3, /* outside the supported envelope above          */
  SSD_ERR_DTYPE = -4,       /* io_dtype is not SSD_F32 / SSD_BF16            */
  SSD_ERR_ALIAS = -5,       /* input/output buffers partially overlap        */
  SSD_ERR_WORKSPACE = -6,   /* workspace NULL, misaligned or too small       */
  SSD_ERR_HIP = -7,         /* the HIP runtime refused a launch              */
  SSD_ERR_ALIGN = -8        /* pointer or stride breaks the 16-byte rule     */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef struct {
  int32_t batch;      /* B: sequences                                        */
  int32_t seqlen;     /* L: tokens per sequence in this call (1 for decode)  */
  int32_t nheads;     /* H                                                   */
  int32_t headdim;    /* P                                                   */
  int32_t ngroups;    /* G: B/C groups and norm groups                       */
  int32_t dstate;     /* N                                                   */
  int32_t conv_width; /* W                                                   */
  int32_t chunk;      /* Q: chunk length of the block decomposition          */
  int32_t io_dtype;   /* ssd_dtype                                           */
} ssd_dims;

/* Conv channels Cch = H*P + 2*G*N. */
int64_t ssd_conv_channels(const ssd_dims* d);

/* Bytes of one sequence's state slot: SSM state H*P*N fp32, and conv state
 * (W-1)*Cch elements of io_dtype (or fp32 when as_fp32 != 0). Host-only. */
int64_t ssd_ssm_state_bytes(const ssd_dims* d);
int64_t ssd_conv_state_bytes(const ssd_dims* d, int as_fp32);

/* Check dims for one entry (SSD_ENTRY_*) on the host; touches no GPU API. */
enum { SSD_ENTRY_CONV1D = 0, SSD_ENTRY_CHUNK_SCAN = 1, SSD_ENTRY_GATED_RMSNORM = 2,
       SSD_ENTRY_DECODE_STEP = 3, SSD_ENTRY_MIXER_PREFILL = 4 };
int ssd_validate(int entry, const ssd_dims* d);

/* Human-readable name of a status code (static string). */
const char* ssd_status_str(int status);

/*
 * CausalConv1D + SiLU ("2. feat(model)": the CausalConv1D op over xBC).
 *   xbc            [B, L, Cch] (token stride xbc_tok_stride >= Cch)
 *   w              [Cch, W];  bias [Cch] or NULL
 *   conv_state_in  [B, W-1, Cch] or NULL (zeros), oldest row first
 *   conv_state_out [B, W-1, Cch] or NULL; may equal conv_state_in (in place)
 *   out            [B, L, Cch] (token stride out_tok_stride >= Cch); out must
 *                  not overlap xbc.
 */
int ssd_conv1d(const ssd_dims* d, const void* xbc, int64_t xbc_tok_stride,
               const void* w, const void* bias, const void* conv_state_in,
               void* conv_state_out, void* out, int64_t out_tok_stride,
               void* stream);

/*
 * Chunked SSD scan with optional fused gated RMSNorm ("2. feat(model)":
 * SSMScan then GatedRMSNorm; "Validation": resuming from state).
 *   x      [B, L, H, P] (token stride x_tok_stride >= H*P)
 *   dt     [B, L, H] contiguous, > 0;   A [H] fp32 (< 0);   D [H] fp32 or NULL
 *   Bm, Cm [B, L, G, N] (token stride bc_tok_stride >= G*N)
 *   z      [B, L, H*P] contiguous or NULL; when non-NULL, norm_w [H*P] is
 *          required and y receives the gated, normalised output; when NULL,
 *          y receives the scan output itself.
 *   ssm_state_in  [B, H, P, N] fp32 or NULL (zeros)
 *   ssm_state_out [B, H, P, N] fp32 or NULL; may equal ssm_state_in
 *   y      [B, L, H*P] contiguous; must not overlap any input.
 *   workspace of ssd_chunk_scan_workspace_bytes(d) bytes.
 */
size_t ssd_chunk_scan_workspace_bytes(const ssd_dims* d);
int ssd_chunk_scan(const ssd_dims* d, const void* x, int64_t x_tok_stride,
                   const void* dt, const float* A, const float* D,
                   const void* Bm, const void* Cm, int64_t bc_tok_stride,
                   const void* z, const void* norm_w, float eps,
                   const float* ssm_state_in, float* ssm_state_out, void* y,
                   void* workspace, size_t ws_bytes, void* stream);

/*
 * Grouped gated RMSNorm over rows = B*L ("2. feat(model)": GatedRMSNorm).
 *   y, z [B*L, H*P] contiguous (y in io_dtype); w [H*P]; out [B*L, H*P]
 *   (out may equal y).
 */
int ssd_gated_rmsnorm(const ssd_dims* d, const void* y, const void* z,
                      const void* w, float eps, void* out, void* stream);

/*
 * One decode token per sequence, states updated in place ("Validation":
 * token-by-token decode resuming from the sequence's slot). dims->seqlen
 * must be 1.
 *   xbc_t [B, Cch]; z_t [B, H*P] or NULL (then y_t = scan output, norm_w
 *   ignored); dt_t [B, H]; A, D [H] fp32 (D may be NULL); conv_w [Cch, W];
 *   conv_b [Cch] or NULL; norm_w [H*P];
 *   conv_state [B, W-1, Cch] io_dtype (in/out); ssm_state [B, H, P, N] fp32
 *   (in/out); y_t [B, H*P]. No workspace.
 */
int ssd_decode_step(const ssd_dims* d, const void* xbc_t, const void* z_t,
                    const void* dt_t, const float* A, const float* D,
                    const void* conv_w, const void* conv_b,
                    const void* norm_w, float eps, void* conv_state,
                    float* ssm_state, void* y_t, void* stream);

/*
 * The whole prefill path in one call: conv + SiLU over xbc, the chunked scan
 * and the gated norm, with state in and out (the composition of the three
 * calls above, fused where the kernels allow).
 *   xbc [B, L, Cch] contiguous; z [B, L, H*P] or NULL; dt [B, L, H];
 *   conv_state_in / conv_state_out [B, W-1, Cch] or NULL (may be equal);
 *   ssm_state_in / ssm_state_out [B, H, P, N] fp32 or NULL (may be equal);
 *   out [B, L, H*P]; workspace of ssd_mixer_prefill_workspace_bytes(d).
 */
size_t ssd_mixer_prefill_workspace_bytes(const ssd_dims* d);
int ssd_mixer_prefill(const ssd_dims* d, const void* xbc, const void* z,
                      const void* dt, const float* A, const float* D,
                      const void* conv_w, const void* conv_b,
                      const void* norm_w, float eps, const void* conv_state_in,
                      void* conv_state_out, const float* ssm_state_in,
                      float* ssm_state_out, void* out, void* workspace,
                      size_t ws_bytes, void* stream);

/*
 * Per-kernel timing of the library's own launches, a measurement aid (the
 * timing is read on the stream each kernel runs on, so it needs no access
 * to the caller's streams). ssd_profile_start(capacity) creates `capacity`
 * pairs of HIP events and switches timing on: from then on every kernel
 * launch of this library takes the next pair and records one event right
 * before and one right after the kernel on its stream. Launches beyond
 * `capacity` are not timed and ssd_profile_stop() then returns
 * SSD_ERR_WORKSPACE. ssd_profile_read() waits for the recorded events of one
 * kernel and returns how many launches were timed and their summed duration
 * in milliseconds; it can be called any number of times until the next
 * start, which drops the previous pool. The state is process-wide (calls are
 * serialised by a lock); do not switch timing on while a stream is captured
 * into a graph. Kernel identifiers: */
typedef enum {
  SSD_K_CONV1D = 0,          /* conv + SiLU over xBC, standalone      */
  SSD_K_CONV_STATE = 1,      /* conv state out (last W-1 rows)        */
  SSD_K_GATED_NORM = 2,      /* grouped gated RMSNorm, standalone     */
  SSD_K_DECODE = 3,          /* one decode token                      */
  SSD_K_CHUNK_STATE = 4,     /* generic path: chunk states            */
  SSD_K_STATE_PASS = 5,      /* generic path: state passing           */
  SSD_K_CHUNK_OUT = 6,       /* generic path: chunk output            */
  SSD_K_FAST_STATE = 7,      /* fast path: conv + chunk states        */
  SSD_K_FAST_PASS = 8,       /* fast path: state passing              */
  SSD_K_FAST_OUT = 9,        /* fast path: conv + chunk output + norm */
  SSD_K_COUNT = 10
} ssd_kernel_id;
int ssd_profile_start(int capacity);
int ssd_profile_stop(void);
int ssd_profile_read(int kernel, int64_t* launches, double* total_ms);
const char* ssd_kernel_name(int kernel);

#ifdef __cplusplus
}
#endif
#endif /* SSD_MI355X_H */
