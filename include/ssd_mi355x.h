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
 * dstate in {16, 32, 64, 128, 256}, conv_width in {2, 3, 4},
 * chunk in {32, 64, 128, 256}.
 *
 * Precision. State, decay exponents, sums and the norm are fp32. The dense
 * contractions of the chunked scan run on MFMA with fp32 accumulation. The
 * general path (every shape outside the fast path, and fp32 I/O) runs
 * 64-token chunks: its chunk states take fp32 operands for fp32 I/O and
 * fp16 operands for bf16 I/O (x scaled by the decay weights, and B), its
 * carried-in states are fp32 and its chunk outputs (C B^T, the masked decay
 * matrix, C S_in, D x) take fp32 operands. The fast path (bf16 I/O with
 * headdim 64, dstate 128, heads per group a multiple of 4, dims->chunk >= 64
 * and conv width 4 when the call includes the conv) takes fp16 operands
 * throughout (the chunk states and carried-in states are also stored in
 * fp16), with D x taken from the fp16 x operand against D at fp16 hi + lo
 * precision. With a conv bias,
 * B and C (and x) share large per-channel offsets, and the state grows along
 * the B offset bbar, while C . bbar can nearly cancel: the fast path then
 * carries every state as S' + a bbar^T (the same matrix, split), with the
 * fp16 operands only for S', B - bbar and C - cbar (cbar, bbar: SiLU of the
 * conv bias) and everything that cancels (a, C . bbar, S' . cbar) in fp32,
 * so such inputs (slowly decaying heads, A of order -0.01) meet the 2e-2
 * bf16 tolerance on the fast path too. SSD_FLAG_FP32_OPERANDS sends the call
 * to the general path with fp32 operands throughout. The fp16
 * intermediates (activations after SiLU, C B^T, chunk states, carried-in
 * states, the scan output before the norm) must stay within fp16 range
 * (|v| < 65504); a value beyond it becomes infinite, so the output or final
 * state is not finite and ssd_workspace_status() reports SSD_ERR_NONFINITE
 * for the call. With SSD_FLAG_FP32_OPERANDS every intermediate is fp32 (no
 * such limit). The chunk length is an internal choice (128 tokens in the
 * fast path, 64 in the general path); the result does not depend on
 * dims->chunk beyond rounding. The fast path fuses the gated norm into its
 * chunk-output kernel, also when a norm group spans several (up to 32) of that kernel's
 * 4-head blocks: their per-token sums of squares are exchanged through the
 * workspace, which needs the group's blocks to run concurrently (a stream
 * with the whole GPU qualifies: 512 resident workgroups, 64 per XCD, against
 * at most 31 waiting per XCD). A wait that cannot complete writes NaN rows
 * after a bounded time instead of hanging and records SSD_ERR_TIMEOUT for
 * ssd_workspace_status(). Wider norm groups are normalised
 * by a separate pass over the scan output. The general path fuses the norm
 * into its chunk-output kernel when a norm group (1, 2, 4 or 8 heads, at
 * most 256 channels) fits one workgroup and the call is large enough to fill
 * the GPU that way (ssd_set_output_norm_fusion), else it writes the scan
 * output to the workspace and a separate pass normalises it.
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
  SSD_ERR_ALIGN = -8,       /* pointer or stride breaks the 16-byte rule     */
  SSD_ERR_TIMEOUT = -9,     /* (ssd_workspace_status) a cross-workgroup norm
                               exchange gave up waiting; its rows are NaN    */
  SSD_ERR_NONFINITE = -10,  /* (ssd_workspace_status) an output or the final
                               SSM state is infinite or NaN                  */
  SSD_ERR_SCRATCH = -11,    /* (ssd_mixer_prefill_noalloc) the call needs more
                               scratch than the library's fixed buffer holds */
  SSD_ERR_VARLEN = -12      /* (ssd_workspace_status) a ragged batch's offsets
                               or slots failed the device checks; nothing of
                               the call was written                          */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

/* ssd_dims.flags. SSD_FLAG_FP32_OPERANDS: run the chunked scan's dense
 * contractions on fp32 MFMA operands for bf16 I/O as well (every
 * intermediate keeps fp32 range and precision; the general kernels are used,
 * not the fused ones). For inputs whose offsets the fast path's state split
 * does not see (B and C sharing a large offset that does not come from the
 * conv bias, e.g. through ssd_chunk_scan) over slowly decaying heads, the
 * inter-chunk term C . S_in can be a sum of large terms that nearly cancel;
 * fp16 operands resolve each term to 2^-11 of itself (see "Precision"
 * above). Unknown bits are refused (SSD_ERR_UNSUPPORTED). The workspace
 * query takes the flag into account. */
enum { SSD_FLAG_FP32_OPERANDS = 1 };

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
  int32_t flags;      /* SSD_FLAG_* bits, 0 by default                       */
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
 * calls above, fused where the kernels allow). ("feat(model): Nemotron-H
 * hybrid ... on the CPU", section "2. feat(model)": CausalConv1D, SSMScan and
 * GatedRMSNorm in that order; section "Validation": prefill in uneven pieces,
 * the second resuming from state, must match one-shot prefill.)
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
 * The step just before the path, fused: the prefill and decode entries
 * below take the input projection's packed rows and the layer's raw
 * state-space parameters instead of dt and A ("feat(model): Nemotron-H
 * hybrid ... on the CPU", "Supporting changes": in_proj emits [z | xBC | dt]
 * in one row; "feat(model): add Nemotron-3 Nano hybrid ..." attribution
 * commit: packed [z, x, B, C, dt] projection, conv1d / A_log / D / dt_bias
 * parameters). Per token the row holds z (H*P), then xBC (Cch, order
 * x | B | C), then dt_raw (H), in io_dtype; row_stride >= 2*H*P + 2*G*N + H
 * elements separates tokens (row_stride * element size a multiple of 16
 * bytes). The kernels form dt = softplus(dt_raw + dt_bias[h]) =
 * log(1 + exp(dt_raw + dt_bias[h])) and A = -exp(A_log[h]) (no clamp of dt;
 * the pages name the parameters but give no formula: this is the plain
 * reading) and otherwise compute exactly what ssd_mixer_prefill /
 * ssd_decode_step compute with that dt and A and the row's z and xBC.
 *   dt_bias, A_log [H] fp32, required; norm_w required (the row carries z).
 *   ssd_mixer_prefill_packed: zxbcdt [B, L, row_stride]; the workspace is
 *   ssd_mixer_prefill_workspace_bytes(d); states, out and aliasing rules as
 *   ssd_mixer_prefill (the row range is an input).
 *   ssd_decode_step_packed: zxbcdt_t [B, row_stride]; states and y_t as
 *   ssd_decode_step.
 */
int ssd_mixer_prefill_packed(const ssd_dims* d, const void* zxbcdt, int64_t row_stride,
                             const float* dt_bias, const float* A_log, const float* D,
                             const void* conv_w, const void* conv_b, const void* norm_w,
                             float eps, const void* conv_state_in, void* conv_state_out,
                             const float* ssm_state_in, float* ssm_state_out, void* out,
                             void* workspace, size_t ws_bytes, void* stream);
int ssd_decode_step_packed(const ssd_dims* d, const void* zxbcdt_t, int64_t row_stride,
                           const float* dt_bias, const float* A_log, const float* D,
                           const void* conv_w, const void* conv_b, const void* norm_w, float eps,
                           void* conv_state, float* ssm_state, void* y_t, void* stream);

/*
 * Continuous batching over a state pool: ragged sequences, prefilling and
 * decoding, in one call ("feat(model): Nemotron-H hybrid ... on the CPU",
 * section "2. feat(model)": the state lives in the engine's slots; section
 * "Validation": two sequences in one batch on separate slots, one
 * prefilling while the other decodes).
 *   d->batch = number of sequences, d->seqlen = T, their total tokens.
 *   cu_seqlens [batch + 1] int32 (device): sequence i owns tokens
 *     [cu_seqlens[i], cu_seqlens[i+1]) of xbc [T, Cch], z [T, H*P] (or NULL)
 *     and dt [T, H], all contiguous; a one-token sequence is a decode step.
 *   slots [batch] int32 (device): the state slot of each sequence in
 *     conv_pool [num_slots, W-1, Cch] (io_dtype) and ssm_pool
 *     [num_slots, H, P, N] (fp32).
 *   has_state [batch] uint8 (device) or NULL: sequence i resumes from its
 *     slot when has_state[i] != 0 (NULL: every sequence), else starts from
 *     zero states.
 *   Each sequence's output rows go to out [T, H*P] and its final conv and
 *   SSM states are written back into its slot; a sequence with no tokens
 *   leaves its slot as it is. The kernels check on the device that
 *   cu_seqlens starts at 0, ends at T and never decreases, and that every
 *   slot of a sequence with tokens lies in [0, num_slots) and is used once;
 *   a call that fails computes and writes nothing and
 *   ssd_workspace_status() reports SSD_ERR_VARLEN.
 *   Workspace: ssd_mixer_varlen_workspace_bytes(d, num_slots) (0 means the
 *   shape is outside this entry's envelope). Envelope: the fused kernels'
 *   (bf16 I/O, headdim 64, dstate 128, conv width 4, heads per group a
 *   multiple of 4 and at most 128, no flags); otherwise
 *   SSD_ERR_UNSUPPORTED. The pools are read and written in place; every
 *   other buffer must not overlap them, out or the workspace.
 */
size_t ssd_mixer_varlen_workspace_bytes(const ssd_dims* d, int32_t num_slots);
int ssd_mixer_varlen(const ssd_dims* d, const int32_t* cu_seqlens, const int32_t* slots,
                     const uint8_t* has_state, int32_t num_slots, const void* xbc, const void* z,
                     const void* dt, const float* A, const float* D, const void* conv_w,
                     const void* conv_b, const void* norm_w, float eps, void* conv_pool,
                     float* ssm_pool, void* out, void* workspace, size_t ws_bytes,
                     void* stream);

/*
 * ssd_mixer_prefill without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. The call allocates nothing. Its scratch
 * is a fixed 64 MiB device array inside this library, one copy per GPU,
 * held until the process ends; a call whose
 * ssd_mixer_prefill_workspace_bytes(d) exceeds 64 MiB returns
 * SSD_ERR_SCRATCH before any launch (the tiny-model layer, 4 x 2048 tokens
 * at 32 heads, needs 32 MiB). Every call on one GPU shares that array and
 * leaves its contents behind: calls on one stream run in order, calls that
 * overlap in time on one GPU (several streams or threads) race. The kernels
 * clear what must start at zero themselves. Runs on the current device;
 * arguments, layouts, aliasing rules and results are those of
 * ssd_mixer_prefill.
 */
int ssd_mixer_prefill_noalloc(const ssd_dims* d, const void* xbc, const void* z,
                              const void* dt, const float* A, const float* D,
                              const void* conv_w, const void* conv_b, const void* norm_w,
                              float eps, const void* conv_state_in, void* conv_state_out,
                              const float* ssm_state_in, float* ssm_state_out, void* out,
                              void* stream);

/*
 * Backward pass of ssd_mixer_prefill with the gated norm, for training
 * ("feat(model): add Nemotron-3 Nano hybrid ...", section "Testing":
 * gradient flow through the mixer; section "Caveats": the pure-PyTorch
 * backend's activation memory). Given the forward's inputs and d_out (and,
 * optionally, the gradient of the final SSM state), returns the gradients of
 * sum(out * d_out) + sum(ssm_state_out * d_ssm_state_out) with respect to
 * every input and parameter. Nothing from the forward is kept: the call
 * recomputes the conv output, the carried-in state of every 64-token chunk
 * and the scan output before the norm, in fp32.
 *   Inputs as ssd_mixer_prefill: xbc [B, L, Cch], z [B, L, H*P] (required),
 *   dt [B, L, H] (after softplus), A [H], D [H] or NULL (zero),
 *   conv_w [Cch, W], conv_b [Cch] or NULL, norm_w [H*P] (required),
 *   conv_state_in [B, W-1, Cch] or NULL (zeros), ssm_state_in [B, H, P, N]
 *   fp32 or NULL (zeros); d_out [B, L, H*P]; d_ssm_state_out [B, H, P, N]
 *   fp32 or NULL (zero).
 *   Outputs (overwritten, never accumulated into): d_xbc, d_z, d_dt in
 *   io_dtype with the shapes of xbc, z, dt; fp32 d_A [H], d_D [H] (NULL: not
 *   computed), d_conv_w [Cch, W], d_conv_b [Cch] (NULL: not computed),
 *   d_norm_w [H*P], d_conv_state_in [B, W-1, Cch] and d_ssm_state_in
 *   [B, H, P, N] (NULL: not computed).
 *   d->chunk and the FP32_OPERANDS flag are checked as for the forward but
 *   do not change the result. Envelope: the forward's, with H*P <= 16384
 *   and ngroups <= 256 (else ssd_mixer_backward_workspace_bytes returns 0
 *   and the call SSD_ERR_UNSUPPORTED). Every output must be disjoint from
 *   every other buffer. Workspace: ssd_mixer_backward_workspace_bytes(d);
 *   its status word (ssd_workspace_status) reports a non-finite recomputed
 *   scan output.
 */
size_t ssd_mixer_backward_workspace_bytes(const ssd_dims* d);
int ssd_mixer_backward(const ssd_dims* d, const void* xbc, const void* z, const void* dt,
                       const float* A, const float* D, const void* conv_w, const void* conv_b,
                       const void* norm_w, float eps, const void* conv_state_in,
                       const float* ssm_state_in, const void* d_out,
                       const float* d_ssm_state_out, void* d_xbc, void* d_z, void* d_dt,
                       float* d_A, float* d_D, float* d_conv_w, float* d_conv_b,
                       float* d_norm_w, float* d_conv_state_in, float* d_ssm_state_in,
                       void* workspace, size_t ws_bytes, void* stream);

/*
 * Status of the chunk-scan or mixer-prefill call that last used `workspace`
 * (a device pointer, the workspace passed to that call). Conditions that
 * depend on the data, and so cannot be checked before the launch, are
 * recorded by the kernels in the first word of the workspace; this call
 * copies that word to the host on `stream` and waits for the stream, so it
 * sees the call once it has completed. Returns SSD_OK, SSD_ERR_TIMEOUT (a
 * cross-workgroup norm exchange gave up; the affected rows are NaN; see the
 * fast path under "Precision" above) or SSD_ERR_NONFINITE (an output row or
 * the final SSM state is infinite or NaN: a non-finite input, or, in the
 * fused path, an fp16 intermediate beyond its range -- repeat the call with
 * SSD_FLAG_FP32_OPERANDS). SSD_ERR_HIP if the copy fails.
 */
int ssd_workspace_status(const void* workspace, void* stream);

/*
 * Diagnostic: set the bound on the polls of the fused path's cross-workgroup
 * norm exchange (default 2^20) for launches made after the call, process
 * wide. 0 makes every such wait give up at once (every kernel still exits
 * normally, the rows are NaN and the status is SSD_ERR_TIMEOUT). Returns the
 * previous bound, or SSD_ERR_SHAPE for a negative one.
 */
int ssd_set_exchange_spin_limit(int polls);

/*
 * Diagnostic: the number of heads of one group that each workgroup of the
 * backward's per-chunk kernels takes, one after the other: the gradient
 * kernel sums their dB and dC rows in place, the state-gradient-term kernel
 * stages the chunk's C once for them. 0, the default: chosen from the shape
 * (the most, up to 32 and 8, that divide the heads per group and leave at
 * least 1024 and 2048 workgroups; one in the gradient kernel for head size
 * 128). A setting of 1, 2, 4, 8, 16 or 32 is used by later
 * ssd_mixer_backward calls, process wide, wherever it divides the heads per
 * group (and, in the gradient kernel, the head size is below 128; else the
 * default applies); it changes the order in which dB and dC are summed,
 * nothing else. Returns the previous setting, or SSD_ERR_SHAPE for any
 * other value.
 */
int ssd_set_backward_chunk_heads(int heads);

/*
 * Diagnostic: where the general kernels (every shape outside the fused
 * path) apply the grouped gated RMSNorm ("feat(model): Nemotron-H hybrid
 * ... on the CPU", section "2. feat(model)": GatedRMSNorm after the scan).
 * 0, the default: inside the chunk-output kernel when a norm group (1, 2,
 * 4 or 8 heads, at most 256 channels) fits one workgroup and the call has
 * at least 512 (chunk, group) workgroups, else y goes to the workspace and
 * a separate norm kernel follows; 1: inside the output kernel wherever the
 * group fits; 2: always the separate kernel. Either way the same values
 * are computed (the sums run in another order). Process wide, for later
 * calls. Returns the previous mode, or SSD_ERR_SHAPE for any other value.
 */
int ssd_set_output_norm_fusion(int mode);

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
  SSD_K_BWD_NORM = 10,       /* backward: gated norm                  */
  SSD_K_BWD_CHUNK_Z = 11,    /* backward: chunk state-gradient terms  */
  SSD_K_BWD_REV_PASS = 12,   /* backward: reverse state passing       */
  SSD_K_BWD_CHUNK = 13,      /* backward: per-chunk gradients         */
  SSD_K_BWD_GROUP_SUM = 14,  /* backward: B / C gradients per group   */
  SSD_K_BWD_CONV_DU = 15,    /* backward: SiLU + conv weight gradient */
  SSD_K_BWD_CONV_DX = 16,    /* backward: conv input gradient         */
  SSD_K_BWD_Y = 17,          /* backward: scan output recomputed      */
  SSD_K_CHUNK_CB = 18,       /* generic path and backward: C B^T per
                                chunk and group                       */
  SSD_K_COUNT = 19
} ssd_kernel_id;
int ssd_profile_start(int capacity);
int ssd_profile_stop(void);
/* Which kernels the timing brackets: bit k set times kernel id k (all by
 * default); the others launch with no events around them, so the timed
 * stream keeps its ordinary launch-to-launch spacing. Returns the previous
 * mask. Stays in force across starts. */
uint64_t ssd_profile_set_mask(uint64_t mask);
int ssd_profile_read(int kernel, int64_t* launches, double* total_ms);
const char* ssd_kernel_name(int kernel);

#ifdef __cplusplus
}
#endif
#endif /* SSD_MI355X_H */
