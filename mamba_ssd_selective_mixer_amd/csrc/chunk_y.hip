// Chunk outputs of the chunked scan on fp32 MFMA operands, 64-token chunks
// ("feat(model): add Nemotron-3 Nano hybrid ..." attribution commit: the SSD
// block decomposition, diagonal blocks and off-diagonal state terms):
//   y = M X + exp(Lam_t) C S_in^T + D X,  M = (C B^T) o exp(Lam_t - Lam_s) dt_s (s <= t)
// per (chunk, head), with S_in the chunk's carried-in state (fp32). C B^T
// depends on the group only, so it is formed once per chunk and group (a
// kernel of its own) and read by every head of the group. These are the
// general path's output kernels (every shape, fp32 or bf16 I/O) and the
// backward pass's recompute of y. x, B, C are read as fp32 or bf16 rows of
// any token stride; y is written as fp32 or the I/O type.
#include <type_traits>

#include "common.hpp"
#include "f32tiles.hpp"
#include "launch.hpp"

namespace ssd {
namespace f32t {

constexpr int kStatusNonFinite = 2;  // status bit: an output is not finite
constexpr int kYHeads = 8;           // most heads of one group per output workgroup
constexpr int kNormCh = 256;         // most channels of a norm group fused into the output kernel
constexpr int kPieceCh = 128;        // channels of the fused norm's LDS pieces

// G = C B^T of one chunk and group on the ten causal 16x16 tiles (three per
// wave at most), shared by every head of the group: cb [B][nc][G][Q][Q],
// element (t, s) at t Q + s; rows past the chunk's end are zero and the
// tiles above the diagonal are not written. B and C go through LDS in
// 32-wide slices of n (the next slice's loads in flight while one is
// computed). The contraction order is free, so within each 16-wide block
// of k the four MFMA steps take k = 16 j + 4 (l / 16) + s (s = 0..3) for
// lane l: each lane reads its four k values of both operands as one
// 16-byte LDS read.
template <class TX>
__global__ __launch_bounds__(kThreads) void k_chunk_cb(const TX* __restrict__ Bm,
                                                       const TX* __restrict__ Cm, int64_t bs,
                                                       float* __restrict__ cb, int L, int G,
                                                       int N, int nc) {
  extern __shared__ __align__(16) float sm[];
  float* Bs = sm;              // [Q][kSP]
  float* Cs = sm + kQ * kSP;   // [Q][kSP]
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lr = lane & 15, lk = lane >> 4;
  const int t0 = c * kQ, len = min(kQ, L - t0);
  const int64_t row0 = (int64_t)b * L + t0;
  const int bsi = (int)bs;
  const TX* br = Bm + row0 * bs + (int64_t)g * N;
  const TX* cr = Cm + row0 * bs + (int64_t)g * N;
  int rt[3], st[3];
  bool on[3];
  f32x4 aG[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    on[i] = causal_tile(wave, i, rt[i], st[i]);
    aG[i] = zero4();
  }
  SliceRegs<kQ> rb, rc;
  auto fetch = [&](int n0) {
    const int nv = min(kKS, N - n0);
    rb.load(br + n0, bsi, len, nv);
    rc.load(cr + n0, bsi, len, nv);
  };
  fetch(0);
  for (int n0 = 0; n0 < N; n0 += kKS) {
    const int nv = min(kKS, N - n0);
    rb.store(Bs);
    rc.store(Cs);
    __syncthreads();
    if (n0 + kKS < N) fetch(n0 + kKS);
    for (int kk = 0; kk < nv; kk += 16) {  // nv is a multiple of 16 (so is every supported N)
      const int kq = kk + 4 * lk;
#pragma unroll
      for (int i = 0; i < 3; ++i)
        if (on[i]) {
          const float4 a4 = ld4(Cs + (rt[i] * 16 + lr) * kSP + kq);
          const float4 b4 = ld4(Bs + (st[i] * 16 + lr) * kSP + kq);
          aG[i] = mma(a4.x, b4.x, aG[i]);
          aG[i] = mma(a4.y, b4.y, aG[i]);
          aG[i] = mma(a4.z, b4.z, aG[i]);
          aG[i] = mma(a4.w, b4.w, aG[i]);
        }
    }
    __syncthreads();
  }
  float* o = cb + (((int64_t)b * nc + c) * G + g) * (kQ * kQ);
#pragma unroll
  for (int i = 0; i < 3; ++i)
    if (on[i])
#pragma unroll
      for (int r = 0; r < 4; ++r) o[(rt[i] * 16 + 4 * lk + r) * kQ + st[i] * 16 + lr] = aG[i][r];
}

// Wave w owns rows 16 w .. 16 w + 15 of the chunk: its causal tiles of G
// (from the group's C B^T), C S_in^T on its rows over 32-wide slices of n
// (the next slice's loads in flight while one is computed), M into LDS,
// then M X over its rows from the chunk's x staged transposed in LDS; the
// k-permuted MFMA steps as in k_chunk_cb. A workgroup takes hpb heads of
// one group, one after the other; the G tiles are read once for all.
//
// NH > 0 fuses the grouped gated RMSNorm ("feat(model): Nemotron-H hybrid
// ... on the CPU", section "2. feat(model)": GatedRMSNorm after the scan):
// the workgroup takes the NH = hpb heads of one whole norm group (NH P <=
// kNormCh channels), keeps q = y silu(z) of its rows in registers (a lane
// holds 4 tokens x P/16 channels per head; the 16 lanes of one DPP row
// hold one token's channels), sums q^2 per token over the group and writes
// out = q w / rms directly, so y never goes to memory.
template <class T, class TX, class TY, int P, int NH>
__global__ __launch_bounds__(kThreads, 2) void k_chunk_y(
    const TX* __restrict__ x, int64_t xs, const TX* __restrict__ Cm, int64_t bs,
    const float* __restrict__ cb, const T* __restrict__ dt, DtA dta, const float* __restrict__ A,
    const float* __restrict__ D, const float* __restrict__ Sin, TY* __restrict__ y, int* status,
    int L, int H, int G, int N, int nc, int hpb, const T* __restrict__ z, int64_t zs,
    const T* __restrict__ nw, float eps) {
  extern __shared__ __align__(16) float sm[];
  float* Mt = sm;                 // [Q][kQP]: M
  float* Cs = sm + kQ * kQP;      // [Q][kSP]
  float* Ss = Cs + kQ * kSP;      // [P][kSP]
  __shared__ float lam[64], dts[64], ex[64];
  constexpr int NPT = P / 16;
  constexpr bool kNorm = NH > 0;
  static_assert(NH * P <= kNormCh, "q of the norm group held in registers");
  // y of the group's heads on the lane's 4 tokens (norm only)
  float q[kNorm ? NH : 1][NPT][4];
  const int c = blockIdx.x, b = blockIdx.z, g = blockIdx.y * hpb / (H / G);
  const int t0 = c * kQ, len = min(kQ, L - t0);
  const int64_t row0 = (int64_t)b * L + t0;
  const int HP = H * P;
  const int xsi = (int)xs, bsi = (int)bs;
  const TX* cr = Cm + row0 * bs + (int64_t)g * N;
  int rt[3], st[3];
  bool on[3];
  f32x4 aG[3];
  {
    const int lane = threadIdx.x & 63, lr = lane & 15, lk = lane >> 4;
    const float* cbk = cb + (((int64_t)b * nc + c) * G + g) * (kQ * kQ);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      on[i] = causal_tile(threadIdx.x >> 6, i, rt[i], st[i]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        aG[i][r] = on[i] ? cbk[(rt[i] * 16 + 4 * lk + r) * kQ + st[i] * 16 + lr] : 0.f;
    }
  }
  // the fused norm needs q of every head in registers: its head loop is
  // unrolled (NH is a compile-time count); else one head at a time
  constexpr int kUnroll = kNorm ? NH : 1;
  const int nh = kNorm ? NH : hpb;
#pragma unroll kUnroll
  for (int hj = 0; hj < nh; ++hj) {
    const int h = blockIdx.y * nh + hj;
    // the thread index is hidden per head, so lane-dependent addresses are
    // not hoisted out of the head loop and held in registers across it
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lk = lane >> 4;
    const TX* xr = x + row0 * xs + (int64_t)h * P;
    const float Ah = a_of(A, dta, h), Dh = D ? D[h] : 0.f;
    const float* Si = Sin + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
    chunk_lam<T>(dt, dta, row0, h, Ah, len, lam, dts, ex);
    f32x4 aY[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i) aY[i] = zero4();
    const int sw = wave * 16;
    SliceRegs<kQ> rc;
    SliceRegs<P> rs;
    auto fetch = [&](int n0) {
      const int nv = min(kKS, N - n0);
      rc.load(cr + n0, bsi, len, nv);
      rs.load(Si + n0, N, P, nv);
    };
    fetch(0);
    for (int n0 = 0; n0 < N; n0 += kKS) {
      const int nv = min(kKS, N - n0);
      rc.store(Cs);
      rs.store(Ss);
      __syncthreads();
      if (n0 + kKS < N) fetch(n0 + kKS);
      // nv is a multiple of 16 (so is every supported N)
      for (int kk = 0; kk < nv; kk += 16) {
        const int kq = kk + 4 * lk;
        const float4 a4 = ld4(Cs + (sw + lr) * kSP + kq);
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const float4 b4 = ld4(Ss + (pt * 16 + lr) * kSP + kq);
          aY[pt] = mma(a4.x, b4.x, aY[pt]);
          aY[pt] = mma(a4.y, b4.y, aY[pt]);
          aY[pt] = mma(a4.z, b4.z, aY[pt]);
          aY[pt] = mma(a4.w, b4.w, aY[pt]);
        }
      }
      __syncthreads();
    }
    // M = G o E dt_s on the causal tiles (rows and columns past the chunk: 0)
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (on[i])
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = rt[i] * 16 + 4 * lk + r, s = st[i] * 16 + lr;
          const float f = (s <= t && t < len) ? __expf(lam[t] - lam[s]) * dts[s] : 0.f;
          Mt[t * kQP + s] = aG[i][r] * f;
        }
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
      for (int r = 0; r < 4; ++r) aY[pt][r] *= ex[sw + 4 * lk + r];
    // the chunk's x transposed, [p][t], where C and S_in were staged
    float* Xt = Cs;
    stage_cols(Xt, kQP, xr, xsi, kQ, len, P);
    __syncthreads();
    // + M X over s <= t (the wave's rows reach s < sw + 16)
    for (int k0 = 0; k0 < sw + 16; k0 += 16) {
      const int kq = k0 + 4 * lk;
      const float4 a4 = ld4(Mt + (sw + lr) * kQP + kq);
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        const float4 b4 = ld4(Xt + (pt * 16 + lr) * kQP + kq);
        aY[pt] = mma(a4.x, b4.x, aY[pt]);
        aY[pt] = mma(a4.y, b4.y, aY[pt]);
        aY[pt] = mma(a4.z, b4.z, aY[pt]);
        aY[pt] = mma(a4.w, b4.w, aY[pt]);
      }
    }
    if constexpr (kNorm) {
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = sw + 4 * lk + r, p = pt * 16 + lr;
          q[hj][pt][r] = aY[pt][r] + Dh * Xt[p * kQP + t];
        }
    } else {
      float chk = 0.f;  // NaN once an output is infinite or NaN
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = sw + 4 * lk + r, p = pt * 16 + lr;
          if (t < len) {
            const float yv = aY[pt][r] + Dh * Xt[p * kQP + t];
            chk += yv * 0.f;
            y[(row0 + t) * HP + (int64_t)h * P + p] = from_f<TY>(yv);
          }
        }
      if (status && chk != 0.f) atomicOr(status, kStatusNonFinite);
    }
    __syncthreads();  // LDS and lam are reused by the next head
  }
  if constexpr (kNorm) {
    // The group's channels go through LDS in pieces of at most kPieceCh
    // (the head loop's tiles are free by now), so that z is read and the
    // output written as 8-channel vectors: nv lanes (one aligned group)
    // take the nv vectors of one token, each thread the same vector of
    // kTok tokens in every piece. Per token: q = y silu(z), the mean of q^2
    // over the group's NH P channels, then out = q w / rms.
    constexpr int NC = NH * P, PC = NC < kPieceCh ? NC : kPieceCh, NPC = NC / PC;
    constexpr int HPC = PC / P;       // heads per piece
    constexpr int nv = PC / 8;        // lanes per token
    // tokens per thread; with fewer than 4 lanes per token the threads past
    // the chunk's 64 tokens read row 63 and write nothing
    constexpr int kTok = kQ * nv >= kThreads ? kQ * nv / kThreads : 1;
    constexpr int YP = PC + 4;        // LDS pitch (floats)
    static_assert(nv >= 2 && nv <= 16, "epilogue mapping");
    float* Yt = sm;                   // [kQ][YP]
    const int lane = threadIdx.x & 63, lr = lane & 15, lk = lane >> 4;
    const int tw = (threadIdx.x >> 6) * 16 + 4 * lk;
    const int v = threadIdx.x % nv, tr = threadIdx.x / nv;  // token tr + i kThreads / nv
    const int64_t c0 = (int64_t)blockIdx.y * NC + v * 8;    // channel of vector v in piece 0
    float qv[NPC][kTok][8], ss[kTok];
#pragma unroll
    for (int i = 0; i < kTok; ++i) ss[i] = 0.f;
#pragma unroll
    for (int pc = 0; pc < NPC; ++pc) {
      // this piece's heads, from the MFMA layout into [t][c]
#pragma unroll
      for (int hk = 0; hk < HPC; ++hk)
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Yt[(tw + r) * YP + hk * P + pt * 16 + lr] = q[pc * HPC + hk][pt][r];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kTok; ++i) {
        const int t = min(tr + i * (kThreads / nv), kQ - 1);
        float zv[8];
        load8(z + (row0 + min(t, len - 1)) * zs + c0 + pc * PC, zv);
        const float4 a = ld4(Yt + t * YP + v * 8), b = ld4(Yt + t * YP + v * 8 + 4);
        const float yv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          qv[pc][i][j] = yv[j] * silu(zv[j]);
          ss[i] = fmaf(qv[pc][i][j], qv[pc][i][j], ss[i]);
        }
      }
      if (pc + 1 < NPC) __syncthreads();  // the tile takes the next piece
    }
#pragma unroll
    for (int i = 0; i < kTok; ++i) {
      const int t = tr + i * (kThreads / nv);  // rows from len on are not written
      const float sq = group_sum_last<nv>(ss[i]);
      if (t < len) {
        if (status && v == 0 && !(sq < __builtin_huge_valf())) atomicOr(status, kStatusNonFinite);
        const float inv = __builtin_amdgcn_rsqf(sq * (1.0f / NC) + eps);
#pragma unroll
        for (int pc = 0; pc < NPC; ++pc) {
          float wv[8], o[8];
          load8(nw + c0 + pc * PC, wv);
#pragma unroll
          for (int j = 0; j < 8; ++j) o[j] = qv[pc][i][j] * wv[j] * inv;
          store8(y + (row0 + t) * HP + c0 + pc * PC, o);
        }
      }
    }
  }
}

size_t chunk_y_lds(int P, bool norm = false) {
  const size_t slices = (size_t)(kQ + P) * kSP, xcols = (size_t)P * kQP;
  const size_t tiles = (size_t)kQ * kQP + std::max(slices, xcols);
  // the fused norm's [t][c] piece reuses the tiles
  return std::max(tiles, norm ? (size_t)kQ * (kPieceCh + 4) : 0) * 4;
}

}  // namespace f32t

size_t chunk_y_lds_bytes(int P) { return f32t::chunk_y_lds(P); }

size_t chunk_cb_bytes(int B, int nc, int G) {
  return (size_t)B * nc * G * f32t::kQ * f32t::kQ * 4;
}

hipError_t launch_chunk_cb(bool x_bf16, const ScanShape& s, const void* Bm, const void* Cm,
                           int64_t bs, float* cb, hipStream_t st) {
  using namespace f32t;
  if (s.Q != kQ) return hipErrorInvalidValue;
  ProfScope ps(st, KID_CHUNK_CB);
  const dim3 grid(s.nc, s.G, s.B), blk(kThreads);
  const size_t lds = 2 * (size_t)kQ * kSP * 4;
  if (x_bf16)
    hipLaunchKernelGGL((k_chunk_cb<bf16>), grid, blk, lds, st, (const bf16*)Bm, (const bf16*)Cm, bs,
                       cb, s.L, s.G, s.N, s.nc);
  else
    hipLaunchKernelGGL((k_chunk_cb<float>), grid, blk, lds, st, (const float*)Bm,
                       (const float*)Cm, bs, cb, s.L, s.G, s.N, s.nc);
  return hipGetLastError();
}

namespace {
// Launch of the norm-fused output kernel with NH = heads per norm group
// (only the counts whose channels fit kNormCh are instantiated).
template <class TT, class TX, int PP>
hipError_t launch_y_norm(int nh, dim3 grid, size_t lds, hipStream_t st, const void* x,
                         int64_t xs, const void* Cm, int64_t bs, const float* cb, const void* dt,
                         const ScanShape& s, const float* A, const float* D,
                         const float* states, void* out, int* status, const YNorm& nm) {
  using namespace f32t;
  hipError_t e = hipErrorInvalidValue;
  auto go = [&](auto nhc) {
    constexpr int NH = decltype(nhc)::value;
    if constexpr (NH * PP <= kNormCh) {
      hipLaunchKernelGGL((k_chunk_y<TT, TX, TT, PP, NH>), grid, dim3(kThreads), lds, st,
                         (const TX*)x, xs, (const TX*)Cm, bs, cb, (const TT*)dt, s.dta, A, D,
                         states, (TT*)out, status, s.L, s.H, s.G, s.N, s.nc, NH,
                         (const TT*)nm.z, nm.zs, (const TT*)nm.w, nm.eps);
      e = hipGetLastError();
    }
  };
  switch (nh) {
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    case 8: go(std::integral_constant<int, 8>{}); break;
    default: break;
  }
  return e;
}
}  // namespace

bool chunk_y_fuses_norm(int H, int G, int P) {
  const int hg = H / G;
  return (hg == 1 || hg == 2 || hg == 4 || hg == 8) && hg * P <= f32t::kNormCh &&
         (P == 16 || P == 32 || P == 64 || P == 128);
}

hipError_t launch_chunk_y(bool io_bf16, bool x_f32, bool y_f32, const ScanShape& s,
                          const void* x, int64_t xs, const void* Bm, const void* Cm, int64_t bs,
                          float* cb, const void* dt, const float* A, const float* D,
                          const float* states, void* y, int* status, int kid, hipStream_t st,
                          const YNorm* norm) {
  using namespace f32t;
  if (s.Q != kQ) return hipErrorInvalidValue;
  if (norm && (!chunk_y_fuses_norm(s.H, s.G, s.P) || y_f32 != !io_bf16))
    return hipErrorInvalidValue;
  hipError_t e = launch_chunk_cb(io_bf16 && !x_f32, s, Bm, Cm, bs, cb, st);
  if (e != hipSuccess) return e;
  ProfScope ps(st, kid);
  const size_t lds = chunk_y_lds(s.P, norm != nullptr);
  if (norm) {
    // one workgroup per norm group and chunk: the group's heads, one after
    // the other, and its rows normalised at the end
    const int hg = s.H / s.G;
    const dim3 grid(s.nc, s.G, s.B);
#define SSD_YN(TT, TX)                                                                             \
  switch (s.P) {                                                                                  \
    case 16: return launch_y_norm<TT, TX, 16>(hg, grid, lds, st, x, xs, Cm, bs, cb, dt, s, A, D,  \
                                              states, y, status, *norm);                          \
    case 32: return launch_y_norm<TT, TX, 32>(hg, grid, lds, st, x, xs, Cm, bs, cb, dt, s, A, D,  \
                                              states, y, status, *norm);                          \
    case 64: return launch_y_norm<TT, TX, 64>(hg, grid, lds, st, x, xs, Cm, bs, cb, dt, s, A, D,  \
                                              states, y, status, *norm);                          \
    default: return launch_y_norm<TT, TX, 128>(hg, grid, lds, st, x, xs, Cm, bs, cb, dt, s, A, D, \
                                               states, y, status, *norm);                         \
  }
    if (!io_bf16) { SSD_YN(float, float); }
    else if (x_f32) { SSD_YN(bf16, float); }
    else { SSD_YN(bf16, bf16); }
#undef SSD_YN
  }
  // heads per workgroup (the group's C B^T tiles read once for them): the
  // most, up to kYHeads, that divide the heads of a group and leave 2048
  // workgroups
  int hpb = kYHeads;
  while (hpb > 1 && ((s.H / s.G) % hpb || (int64_t)s.B * s.nc * (s.H / hpb) < 2048)) hpb /= 2;
  const dim3 grid(s.nc, s.H / hpb, s.B), blk(kThreads);
#define SSD_Y(TT, TX, TY, PP)                                                                   \
  hipLaunchKernelGGL((k_chunk_y<TT, TX, TY, PP, 0>), grid, blk, lds, st, (const TX*)x, xs,      \
                     (const TX*)Cm, bs, cb, (const TT*)dt, s.dta, A, D, states, (TY*)y, status, \
                     s.L, s.H, s.G, s.N, s.nc, hpb, nullptr, 0, nullptr, 0.f)
#define SSD_Y_P(TT, TX, TY)                  \
  switch (s.P) {                             \
    case 16: SSD_Y(TT, TX, TY, 16); break;   \
    case 32: SSD_Y(TT, TX, TY, 32); break;   \
    case 64: SSD_Y(TT, TX, TY, 64); break;   \
    default: SSD_Y(TT, TX, TY, 128); break;  \
  }
  if (!io_bf16) {
    SSD_Y_P(float, float, float);
  } else if (x_f32) {
    if (y_f32) { SSD_Y_P(bf16, float, float); }
    else { SSD_Y_P(bf16, float, bf16); }
  } else {
    if (y_f32) { SSD_Y_P(bf16, bf16, float); }
    else { SSD_Y_P(bf16, bf16, bf16); }
  }
#undef SSD_Y_P
#undef SSD_Y
  return hipGetLastError();
}

}  // namespace ssd
