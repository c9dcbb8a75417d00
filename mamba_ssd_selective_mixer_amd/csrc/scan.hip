// Chunked state-space-duality (SSD) scan on gfx950: the block decomposition
// of the selective recurrence ("feat(model): add Nemotron-3 Nano hybrid ..."
// attribution commit: the chunk-parallel SSD block decomposition,
// ssd_minimal_discrete / segsum).
//
// For chunk k = [t0, t0 + Q) of head h (group g = h / (H/G)), with
// a_t = dt_t A_h and the inclusive segment sum Lam_t = sum_{r=t0..t} a_r:
//   chunk state   dS_k[p,n] = sum_s exp(Lam_end - Lam_s) dt_s x_s[p] B_s[n]
//   state passing S_in(0) = S_init, S_in(k+1) = exp(Lam_end,k) S_in(k) + dS_k
//   chunk output  y_t[p] = sum_{s<=t} (C_t . B_s) exp(Lam_t - Lam_s) dt_s x_s[p]
//                          + exp(Lam_t) (S_in(k) C_t)[p] + D_h x_t[p]
// The three dense contractions (B^T (w x), C B^T, and the masked (C B^T) X
// together with C S_in^T) run on 16x16 MFMA tiles with fp32 accumulation:
// fp16 operands for bf16 I/O (inputs converted as they are staged; the norm
// that may follow amplifies operand rounding, and fp16's mantissa is 8x
// finer than bf16's), fp32 operands for fp32 I/O. Decays are always
// formed as exp(Lam_t - Lam_s) of a masked difference, never as a ratio of
// exponentials, so they stay finite for any chunk length.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace ssd {

constexpr int kScanThreads = 256;  // 4 waves
constexpr int kStateSB = 64;       // tokens staged per block in the chunk-state kernel
constexpr int kStateHeads = 8;     // most heads of one group per chunk-state workgroup

template <class T> struct Pad { static constexpr int v = 8; };     // fp16 operands: 16 bytes per LDS row
template <> struct Pad<float> { static constexpr int v = 4; };
// MFMA operand type: fp16 for bf16 I/O unless F32OP asks for fp32 operands
// (fp32 range for every intermediate), fp32 for fp32 I/O.
template <class T, bool F32OP>
using OpT = typename std::conditional<F32OP, float, typename OpOf<T>::type>::type;
constexpr int kStatusNonFinite = 2;  // status bit: an output or the final state is not finite

// Inclusive cumulative sum of a_s = dt_s * A over the chunk (s < len; zero
// beyond) into lam[], and dt_s into dts[]. Q <= 256 = blockDim.
template <class T>
__device__ __forceinline__ void chunk_cumsum(const T* __restrict__ dt, const DtA& dta,
                                             int64_t row0, int h, float Ah, int len, float* lam,
                                             float* dts, float* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float d = 0.f;
  if (tid < len) d = dt_of(to_f(dt[(row0 + tid) * dta.dts + h]), dta, h);
  const float v = wave_incl_scan(d * Ah);
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  float add = 0.f;
  for (int w = 0; w < wave; ++w) add += wsum[w];
  lam[tid] = v + add;
  dts[tid] = d;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Phase 1: chunk states dS_k = (w x)^T B per (chunk, head, batch), for hpb
// heads of one group per workgroup, one after the other (a chunk of one
// 64-token slab stages B once for all of them).
// T: I/O type (dt); TX: element type of x and B (T, or fp32 when they come
// from the conv's internal fp32 copy). MAXT: most 16x16 output tiles per wave
// (P N / 1024 rounded up to 16 or 32; d_state 256 with head_dim 128 needs 32).
template <class T, class TX, bool F32OP, int MAXT>
__global__ __launch_bounds__(kScanThreads) void k_chunk_state(
    const TX* __restrict__ x, int64_t xs, const T* __restrict__ dt, const float* __restrict__ A,
    const TX* __restrict__ Bm, int64_t bs, float* __restrict__ states,
    float* __restrict__ lam_end, int* status, DtA dta, int L, int H, int G, int P, int N, int Q,
    int nc, int hpb) {
  typedef OpT<T, F32OP> O;  // MFMA operand type
  using M = Mfma<O>;
  constexpr int KP = kStateSB + Pad<O>::v;
  extern __shared__ __align__(16) unsigned char smraw[];
  O* XwT = reinterpret_cast<O*>(smraw);  // [P][KP]  x_s[p] * w_s, k = s contiguous
  O* BT = XwT + P * KP;                  // [N][KP]  B_s[n]
  __shared__ float lam[kScanThreads], dts[kScanThreads], wgt[kScanThreads], wsum[4];

  const int c = blockIdx.x, b = blockIdx.z;
  const int g = blockIdx.y * hpb / (H / G);
  const int t0 = c * Q, len = min(Q, L - t0);
  const int64_t row0 = (int64_t)b * L + t0;
  // this call's status word starts clear (later kernels only set bits)
  if ((blockIdx.x | blockIdx.y | blockIdx.z | threadIdx.x) == 0) *status = 0;
#pragma unroll 1
  for (int hj = 0; hj < hpb; ++hj) {
    const int h = blockIdx.y * hpb + hj;
    // the thread index is hidden per head, so lane-dependent addresses are not
    // hoisted out of the head loop and held in registers across it
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6;

    chunk_cumsum<T>(dt, dta, row0, h, a_of(A, dta, h), len, lam, dts, wsum);
    const float lamE = lam[len - 1];
    wgt[tid] = tid < len ? fexp(lamE - lam[tid]) * dts[tid] : 0.f;
    __syncthreads();

    const int ntn = N / 16, tiles = (P / 16) * ntn;
    constexpr int kMaxTPW = MAXT;
    f32x4 acc[kMaxTPW];
#pragma unroll
    for (int i = 0; i < kMaxTPW; ++i) acc[i] = zero4();

    // staged transposed ([p][s], [n][s]) with one token per lane, so a wave's
    // LDS stores hit consecutive addresses
    const int P8 = P / 8, N8 = N / 8;
    for (int s0 = 0; s0 < len; s0 += kStateSB) {
      for (int v = tid; v < kStateSB * P8; v += kScanThreads) {
        const int s = v % kStateSB, p0 = (v / kStateSB) * 8;
        float xv[8];
        if (s0 + s < len) {
          load8(x + (row0 + s0 + s) * xs + (int64_t)h * P + p0, xv);
          const float ww = wgt[s0 + s];
#pragma unroll
          for (int j = 0; j < 8; ++j) xv[j] *= ww;
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) xv[j] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) XwT[(p0 + j) * KP + s] = from_f<O>(xv[j]);
      }
      // B is the group's: staged once when the chunk is one slab
      if (hj == 0 || len > kStateSB)
        for (int v = tid; v < kStateSB * N8; v += kScanThreads) {
          const int s = v % kStateSB, n0 = (v / kStateSB) * 8;
          float bv[8];
          if (s0 + s < len) {
            load8(Bm + (row0 + s0 + s) * bs + (int64_t)g * N + n0, bv);
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) bv[j] = 0.f;
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) BT[(n0 + j) * KP + s] = from_f<O>(bv[j]);
        }
      __syncthreads();
      // fp32 operands: k-permuted steps, the MFMA steps of a 16-wide k block
      // taking k = 4 (l / 16) + s for lane l, so a lane's four k values of both
      // operands are one 16-byte read (the contraction order is free)
      constexpr bool kF32 = std::is_same<O, float>::value;
      const int kk = (kF32 ? 4 : M::KPL) * (lane >> 4), rr = lane & 15;
#pragma unroll
      for (int i = 0; i < kMaxTPW; ++i) {
        const int tile = wave + 4 * i;
        if (tile < tiles) {
          const int tp = tile / ntn, tn = tile % ntn;
          const O* ap = XwT + (tp * 16 + rr) * KP + kk;
          const O* bp = BT + (tn * 16 + rr) * KP + kk;
          if constexpr (kF32) {
#pragma unroll
            for (int k = 0; k < kStateSB; k += 16) {
              const float4 a4 = *reinterpret_cast<const float4*>(ap + k);
              const float4 b4 = *reinterpret_cast<const float4*>(bp + k);
              acc[i] = M::mma(a4.x, b4.x, acc[i]);
              acc[i] = M::mma(a4.y, b4.y, acc[i]);
              acc[i] = M::mma(a4.z, b4.z, acc[i]);
              acc[i] = M::mma(a4.w, b4.w, acc[i]);
            }
          } else {
#pragma unroll
            for (int k = 0; k < kStateSB; k += M::KSTEP)
              acc[i] = M::mma(M::ld(ap + k), M::ld(bp + k), acc[i]);
          }
        }
      }
      __syncthreads();
    }

    float* out = states + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
#pragma unroll
    for (int i = 0; i < kMaxTPW; ++i) {
      const int tile = wave + 4 * i;
      if (tile < tiles) {
        const int tp = tile / ntn, tn = tile % ntn;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int p = tp * 16 + 4 * (lane >> 4) + r, n = tn * 16 + (lane & 15);
          out[(int64_t)p * N + n] = acc[i][r];
        }
      }
    }
    if (tid == 0) lam_end[((int64_t)b * H + h) * nc + c] = lamE;
  }
}

// ---------------------------------------------------------------------------
// Phase 2: state passing along the chunks, in place: states[k] := S_in(k).
__global__ __launch_bounds__(kScanThreads) void k_state_pass(float* states,
                                                             const float* __restrict__ lam_end,
                                                             const float* s_in, float* s_out,
                                                             int* status, int H, int PN, int nc) {
  const int e = (blockIdx.x * kScanThreads + threadIdx.x) * 4;
  const int h = blockIdx.y, b = blockIdx.z;
  if (e >= PN) return;
  const int64_t bh = (int64_t)b * H + h;
  float4 S = make_float4(0.f, 0.f, 0.f, 0.f);
  if (s_in) S = *reinterpret_cast<const float4*>(s_in + bh * PN + e);
  for (int c = 0; c < nc; ++c) {
    float* p = states + (((int64_t)b * nc + c) * H + h) * PN + e;
    const float4 d = *reinterpret_cast<const float4*>(p);
    *reinterpret_cast<float4*>(p) = S;
    const float al = fexp(lam_end[bh * nc + c]);
    S.x = al * S.x + d.x;
    S.y = al * S.y + d.y;
    S.z = al * S.z + d.z;
    S.w = al * S.w + d.w;
  }
  if (s_out) {
    *reinterpret_cast<float4*>(s_out + bh * PN + e) = S;
    if (S.x * 0.f + S.y * 0.f + S.z * 0.f + S.w * 0.f != 0.f) atomicOr(status, kStatusNonFinite);
  }
}

// ---------------------------------------------------------------------------
// op16: the MFMA operands are fp16 (else fp32)
static size_t state_lds(bool op16, int P, int N) {
  const int KP = kStateSB + (op16 ? 8 : 4);
  return (size_t)(P + N) * KP * (op16 ? 2 : 4);
}
hipError_t launch_chunk_state(bool io_bf16, bool x_f32, bool f32op, const ScanShape& s,
                              const void* x, int64_t xs, const void* dt, const float* A,
                              const void* Bm, int64_t bs, float* states, float* lam_end,
                              int* status, hipStream_t st) {
  ProfScope ps(st, KID_CHUNK_STATE);
  // heads per workgroup: the most, up to kStateHeads, that divide the heads
  // of a group and leave 2048 workgroups (one slab per chunk: B staged once)
  int hpb = s.Q <= kStateSB ? kStateHeads : 1;
  while (hpb > 1 && ((s.H / s.G) % hpb || (int64_t)s.B * s.nc * (s.H / hpb) < 2048)) hpb /= 2;
  dim3 grid(s.nc, s.H / hpb, s.B), block(kScanThreads);
  const size_t lds = state_lds(io_bf16 && !f32op, s.P, s.N);
  const bool t32 = s.P * s.N > 16 * 1024;  // tiles per wave beyond 16
#define SSD_STATE_T(TT, TX, F, T)                                                              \
  hipLaunchKernelGGL((k_chunk_state<TT, TX, F, T>), grid, block, lds, st, (const TX*)x, xs,     \
                     (const TT*)dt, A, (const TX*)Bm, bs, states, lam_end, status, s.dta, s.L,  \
                     s.H, s.G, s.P, s.N, s.Q, s.nc, hpb)
#define SSD_STATE(TT, TX, F) \
  if (t32) SSD_STATE_T(TT, TX, F, 32); else SSD_STATE_T(TT, TX, F, 16)
  if (!io_bf16) {
    SSD_STATE(float, float, true);
  } else if (x_f32) {
    if (f32op) { SSD_STATE(bf16, float, true); }
    else { SSD_STATE(bf16, float, false); }
  } else {
    if (f32op) { SSD_STATE(bf16, bf16, true); }
    else { SSD_STATE(bf16, bf16, false); }
  }
#undef SSD_STATE
#undef SSD_STATE_T
  return hipGetLastError();
}

hipError_t launch_state_pass(const ScanShape& s, float* states, const float* lam_end,
                             const float* s_in, float* s_out, int* status, hipStream_t st) {
  ProfScope ps(st, KID_STATE_PASS);
  const int PN = s.P * s.N;
  dim3 grid((PN / 4 + kScanThreads - 1) / kScanThreads, s.H, s.B), block(kScanThreads);
  hipLaunchKernelGGL(k_state_pass, grid, block, 0, st, states, lam_end, s_in, s_out, status, s.H,
                     PN, s.nc);
  return hipGetLastError();
}

// LDS bytes the general path's two MFMA kernels need for a shape: the
// chunk-state kernel and the fp32 output kernel (64-token chunks); the host
// checks them against the 160 KiB of one CU before launching.
size_t scan_lds_bytes(bool op16, int P, int N, int Q) {
  (void)Q;  // the general path runs 64-token chunks whatever the caller's chunk
  const size_t a = state_lds(op16, P, N), b = chunk_y_lds_bytes(P);
  return a > b ? a : b;
}

}  // namespace ssd
