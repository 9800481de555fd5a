// Backward of the selective scan (S6) for gfx950, with recomputation.
//
// What is differentiated ("Mamba 논문 리뷰 ... Selective State Space Model",
// tildalice.io: 이산화, Selection Mechanism; the backward pass of
// 하드웨어 인식 병렬 알고리즘 recomputes the states instead of storing them):
//   h_t = Abar_t h_{t-1} + cbar_t B_t x_t,  Abar = exp(delta A),
//   cbar = expm1(delta A)/A (zero-order hold) or delta (simplified),
//   o_t = C_t.h_t + D x_t,  y_t = o_t silu(z_t).
// The reverse pass carries the adjoint of the state,
//   lam_t = C_t g_t + Abar_{t+1} lam_{t+1},  g_t = dy_t silu(z_t),
// and every input gradient is a sum of lam_t, g_t, h_{t-1} and h_t terms.
//
// Work split (the forward kernel's layout): a 256-thread workgroup owns 16
// channels of one batch row, each channel one 16-lane row of a wave, each
// lane N/16 states; the sequence is walked in tiles of 16 steps and lane j
// of a row holds step j's per-channel values (delta, x, z, dy), broadcast to
// the row with DPP row broadcasts.
//  1. ckpt_kernel runs the recurrence forward and stores the state before
//     every tile: 1/16 of the states, the rest is recomputed.
//  2. bwd_kernel walks the tiles backwards.  Per tile it recomputes the 16
//     states of each lane from the tile's checkpoint (kept in registers) with
//     the readout C.h, forms g_t and dz_t, then steps the adjoint back through
//     the tile, accumulating dx and ddelta (sums over the lane's states, then
//     over the row through LDS), dB and dC (sums over the workgroup's 16
//     channels: DPP-free lane shuffles across the 4 rows of a wave, then
//     LDS across the 4 waves) and dA, dD, ddelta_bias in registers.
//  3. reduce kernels add the per-workgroup partial sums of dB, dC over the
//     channel blocks and of dA, dD, ddelta_bias over the batch, in a fixed
//     order.
#include <hip/hip_runtime.h>

#include <utility>

#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int G = 16;    // lanes per channel
constexpr int CH = 16;   // channels per workgroup
constexpr int TT = 16;   // steps per tile
constexpr int NT = 256;  // threads
constexpr int TP = TT + 1;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int T>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + T, 0xF, 0xF, true));
}

template <bool BF16>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
  if constexpr (BF16) return __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16);
  else return ((const float*)p)[i];
}

__device__ __forceinline__ void st(void* p, int64_t i, float v, bool f32) {
  if (f32) ((float*)p)[i] = v;
  else ((__bf16*)p)[i] = (__bf16)v;
}

__device__ __forceinline__ float sigmoid_f32(float v) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-v * kLog2e));
}

// softplus(v) = max(v, 0) + log1p(e^-|v|), log1p(w) = log(u) * w / (u - 1),
// u = 1 + w (u - 1 is exact)
__device__ __forceinline__ float softplus_f32(float v) {
  const float w = __builtin_amdgcn_exp2f(-fabsf(v) * kLog2e);
  const float u = 1.f + w;
  const float lp = u == 1.f ? w : (__builtin_amdgcn_logf(u) * kLn2) * (w * __builtin_amdgcn_rcpf(u - 1.f));
  return fmaxf(v, 0.f) + lp;
}

template <int... S, class F>
__device__ __forceinline__ void for_steps(std::integer_sequence<int, S...>, F&& f) {
  (f(std::integral_constant<int, S>{}), ...);
}

template <int... S, class F>
__device__ __forceinline__ void for_steps_rev(std::integer_sequence<int, S...>, F&& f) {
  (f(std::integral_constant<int, TT - 1 - S>{}), ...);
}

// The per-channel, per-step values of one tile and the (B, C) pairs.
template <int KS>
struct TileSmem {
  float dt[CH][TP];   // step size used (after the softplus); 0 on padding steps
  float dv[CH][TP];   // softplus argument delta + bias
  float x[CH][TP];
  float z[CH][TP];
  float gy[CH][TP];   // dy
  float2 bc[TT][G * KS];
};

template <int KS>
struct BwdSmem {
  TileSmem<KS> t;
  float part[2][NT][TP];          // per-lane partial sums over states, by step
  float red[4][TT][2][G * KS];    // per-wave sums of dB, dC over the wave's 4 channels
};

// Lane constants of its KS states.
template <int KS>
struct LaneA {
  float a[KS], A2[KS], iA[KS];
};

// Stage tile `it` of the workgroup's 16 channels into LDS (zeros past the
// sequence and the channels; delta 0 there so the state does not change).
template <bool BF16, int KS, bool FULL>
__device__ __forceinline__ void stage_tile(TileSmem<KS>& s, const ScanBwdParams& p, int64_t b, int64_t d0, int it) {
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)it * TT;
  for (int i = tid; i < CH * TT; i += NT) {
    const int c = i / TT, j = i % TT;
    const int64_t t = t0 + j, d = d0 + c;
    const bool ok = t < p.L && d < p.D;
    const float xv = ok ? ld<BF16>(p.x, b * p.xs_b + t * p.xs_t + d) : 0.f;
    const float raw = ok ? ld<BF16>(p.delta, b * p.ds_b + t * p.ds_t + d) : 0.f;
    float dt = raw, v = raw;
    if (p.dsoftplus) {
      v = raw + ((p.dbias && d < p.D) ? p.dbias[d * p.dbs_d] : 0.f);
      dt = ok ? softplus_f32(v) : 0.f;
    }
    s.x[c][j] = xv;
    s.dt[c][j] = dt;
    if constexpr (FULL) {
      s.dv[c][j] = v;
      s.z[c][j] = (ok && p.z) ? ld<BF16>(p.z, b * p.zs_b + t * p.zs_t + d) : 0.f;
      const int64_t gi = b * p.gs_b + t * p.gs_t + d;
      s.gy[c][j] = ok ? (p.dy_f32 ? ((const float*)p.dy)[gi] : ld<true>(p.dy, gi)) : 0.f;
    }
  }
  for (int i = tid; i < TT * G * KS; i += NT) {
    const int j = i / (G * KS), n = i % (G * KS);
    const int64_t t = t0 + j;
    const bool ok = t < p.L && n < p.N;
    const float Bv = ok ? ld<BF16>(p.B, b * p.Bs_b + t * p.Bs_t + n * p.Bs_n) : 0.f;
    const float Cv = (FULL && ok) ? ld<BF16>(p.C, b * p.Cs_b + t * p.Cs_t + n * p.Cs_n) : 0.f;
    s.bc[j][n] = make_float2(Bv, Cv);
  }
}

// cbar for one state: expm1(u)/a as Abar/a - 1/a (delta where a == 0), or delta.
__device__ __forceinline__ float cbar(float Ab, float a, float iA, float dt, bool euler) {
  if (euler) return dt;
  return a != 0.f ? __builtin_fmaf(Ab, iA, -iA) : dt;
}

template <bool BF16, int KS>
__device__ __forceinline__ LaneA<KS> lane_a(const ScanBwdParams& p, int64_t d, int sg) {
  LaneA<KS> la;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int n = sg * KS + k;
    float a = -1.f;  // padding states and channels: any A != 0 (B = C = 0 there)
    if (d < p.D && n < p.N) a = p.A[d * p.As_d + n * p.As_n];
    la.a[k] = a;
    la.A2[k] = a * kLog2e;
    la.iA[k] = a != 0.f ? 1.f / a : 0.f;
  }
  return la;
}

// ---------------------------------------------------------- checkpoints

template <bool BF16, int KS>
__global__ __launch_bounds__(NT) void ckpt_kernel(ScanBwdParams p, int64_t n_dblk) {
  __shared__ TileSmem<KS> s;
  const int tid = threadIdx.x, c = tid / G, sg = tid % G;
  const int64_t dblk = blockIdx.x % n_dblk, b = blockIdx.x / n_dblk;
  const int64_t d0 = dblk * CH, d = d0 + c;
  const bool euler = p.euler != 0;
  const LaneA<KS> la = lane_a<BF16, KS>(p, d, sg);
  const int ntiles = (int)((p.L + TT - 1) / TT);
  float h[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int n = sg * KS + k;
    h[k] = (p.h0 && d < p.D && n < p.N) ? p.h0[(b * p.D + d) * p.N + n] : 0.f;
  }
  for (int it = 0; it < ntiles; ++it) {
    if (d < p.D) {
      float* ck = p.ckpt + (((b * ntiles + it) * p.D + d) * p.N);
#pragma unroll
      for (int k = 0; k < KS; ++k)
        if (sg * KS + k < p.N) ck[sg * KS + k] = h[k];
    }
    stage_tile<BF16, KS, false>(s, p, b, d0, it);
    __syncthreads();
    const float hdt = s.dt[c][sg], hx = s.x[c][sg];
    for_steps(std::make_integer_sequence<int, TT>{}, [&](auto S) {
      constexpr int T = decltype(S)::value;
      const float dt = row_bcast<T>(hdt), xv = row_bcast<T>(hx);
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const float Ab = __builtin_amdgcn_exp2f(dt * la.A2[k]);
        const float Bv = s.bc[T][sg * KS + k].x;
        h[k] = __builtin_fmaf(Ab, h[k], cbar(Ab, la.a[k], la.iA[k], dt, euler) * (Bv * xv));
      }
    });
    __syncthreads();
  }
}

// -------------------------------------------------------------- backward

template <bool BF16, int KS>
__global__ __launch_bounds__(NT) void bwd_kernel(ScanBwdParams p, int64_t n_dblk) {
  __shared__ BwdSmem<KS> s;
  const int tid = threadIdx.x, c = tid / G, sg = tid % G;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int64_t dblk = blockIdx.x % n_dblk, b = blockIdx.x / n_dblk;
  const int64_t d0 = dblk * CH, d = d0 + c;
  const bool d_ok = d < p.D;
  const bool euler = p.euler != 0, has_z = p.z != nullptr;
  const LaneA<KS> la = lane_a<BF16, KS>(p, d, sg);
  const float Dk = (p.Dskip && d_ok) ? p.Dskip[d * p.Ds_d] : 0.f;
  const int ntiles = (int)((p.L + TT - 1) / TT);
  float carry[KS], dA[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) carry[k] = dA[k] = 0.f;
  float dD = 0.f, dbias = 0.f;  // this lane's steps of its channel
  float* prow = &s.part[0][tid][0];

  for (int it = ntiles - 1; it >= 0; --it) {
    const int64_t t0 = (int64_t)it * TT;
    stage_tile<BF16, KS, true>(s.t, p, b, d0, it);
    float h0t[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int n = sg * KS + k;
      h0t[k] = (d_ok && n < p.N) ? p.ckpt[((b * ntiles + it) * p.D + d) * p.N + n] : 0.f;
    }
    __syncthreads();
    const float hdt = s.t.dt[c][sg], hx = s.t.x[c][sg];

    // recompute the tile's states and the readout partials
    float hh[TT][KS];
    {
      float h[KS];
#pragma unroll
      for (int k = 0; k < KS; ++k) h[k] = h0t[k];
      for_steps(std::make_integer_sequence<int, TT>{}, [&](auto S) {
        constexpr int T = decltype(S)::value;
        const float dt = row_bcast<T>(hdt), xv = row_bcast<T>(hx);
        float yp = 0.f;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          const float2 bcv = s.t.bc[T][sg * KS + k];
          const float Ab = __builtin_amdgcn_exp2f(dt * la.A2[k]);
          h[k] = __builtin_fmaf(Ab, h[k], cbar(Ab, la.a[k], la.iA[k], dt, euler) * (bcv.x * xv));
          hh[T][k] = h[k];
          yp = __builtin_fmaf(bcv.y, h[k], yp);
        }
        prow[T] = yp;
      });
    }
    // lane sg takes step sg of its channel: o, g, dz
    const int64_t tj = t0 + sg;
    const bool j_ok = d_ok && tj < p.L;
    float o = 0.f;
#pragma unroll
    for (int l = 0; l < G; ++l) o += s.part[0][c * G + l][sg];
    const float xj = hx, zj = s.t.z[c][sg], gyj = s.t.gy[c][sg];
    o = __builtin_fmaf(Dk, xj, o);
    float g = gyj;
    if (has_z) {
      const float sgm = sigmoid_f32(zj);
      g = gyj * zj * sgm;
      const float dz = gyj * o * sgm * __builtin_fmaf(zj, 1.f - sgm, 1.f);
      if (j_ok) st(p.dz, b * p.dzs_b + tj * p.dzs_t + d, dz, p.dz_f32);
    }
    dD = __builtin_fmaf(g, xj, dD);

    // reverse through the tile
    for_steps_rev(std::make_integer_sequence<int, TT>{}, [&](auto S) {
      constexpr int T = decltype(S)::value;
      const float dt = row_bcast<T>(hdt), xv = row_bcast<T>(hx), gs = row_bcast<T>(g);
      float dxp = 0.f, dtp = 0.f;
      float vB[KS], vC[KS];
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const float2 bcv = s.t.bc[T][sg * KS + k];
        const float a = la.a[k];
        const float Ab = __builtin_amdgcn_exp2f(dt * la.A2[k]);
        const float cb = cbar(Ab, a, la.iA[k], dt, euler);
        const float hp = T > 0 ? hh[T > 0 ? T - 1 : 0][k] : h0t[k];
        const float l = __builtin_fmaf(bcv.y, gs, carry[k]);
        const float bx = bcv.x * xv;
        vC[k] = gs * hh[T][k];
        vB[k] = l * cb * xv;
        dxp = __builtin_fmaf(l * cb, bcv.x, dxp);
        const float dc_ddt = euler ? 1.f : Ab;
        const float dc_da = euler ? 0.f : (a != 0.f ? (dt * Ab - cb) * la.iA[k] : 0.5f * dt * dt);
        dtp = __builtin_fmaf(l, __builtin_fmaf(a * Ab, hp, dc_ddt * bx), dtp);
        dA[k] = __builtin_fmaf(l, __builtin_fmaf(dt * Ab, hp, dc_da * bx), dA[k]);
        carry[k] = Ab * l;
      }
      s.part[0][tid][T] = dxp;
      s.part[1][tid][T] = dtp;
      // dB, dC: sum over the wave's 4 channels (rows), then one row writes
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        float vb = vB[k], vc = vC[k];
        vb += __shfl_xor(vb, 16);
        vc += __shfl_xor(vc, 16);
        vb += __shfl_xor(vb, 32);
        vc += __shfl_xor(vc, 32);
        if (lane < G) {
          s.red[wave][T][0][sg * KS + k] = vb;
          s.red[wave][T][1][sg * KS + k] = vc;
        }
      }
    });
    // lane sg: dx and ddelta of step sg
    float dxs = 0.f, dts = 0.f;
#pragma unroll
    for (int l = 0; l < G; ++l) {
      dxs += s.part[0][c * G + l][sg];
      dts += s.part[1][c * G + l][sg];
    }
    dxs = __builtin_fmaf(Dk, g, dxs);
    if (p.dsoftplus) {
      dts *= sigmoid_f32(s.t.dv[c][sg]);
      if (j_ok) dbias += dts;
    }
    if (j_ok) {
      st(p.dx, b * p.dxs_b + tj * p.dxs_t + d, dxs, p.dx_f32);
      st(p.ddelta, b * p.dds_b + tj * p.dds_t + d, dts, p.dd_f32);
    }
    __syncthreads();
    // dB, dC of the tile: sum over the 4 waves, store the workgroup's partial
    for (int i = tid; i < TT * 2 * G * KS; i += NT) {
      const int j = i / (2 * G * KS), q = (i / (G * KS)) % 2, n = i % (G * KS);
      const int64_t t = t0 + j;
      if (t < p.L && n < p.N) {
        const float v = s.red[0][j][q][n] + s.red[1][j][q][n] + s.red[2][j][q][n] + s.red[3][j][q][n];
        float* dst = q == 0 ? p.pdB : p.pdC;
        dst[((dblk * p.batch + b) * p.L + t) * p.N + n] = v;
      }
    }
    __syncthreads();
  }
  // per-channel and per-state sums of this batch row
  if (d_ok) {
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int n = sg * KS + k;
      if (n < p.N) {
        p.pdA[(b * p.D + d) * p.N + n] = dA[k];
        if (p.dh0) p.dh0[(b * p.D + d) * p.N + n] = carry[k];
      }
    }
  }
  // dD and ddelta_bias: sum over the row's 16 lanes (their steps)
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) {
    dD += __shfl_xor(dD, m, G);
    dbias += __shfl_xor(dbias, m, G);
  }
  if (sg == 0 && d_ok) {
    if (p.pdD) p.pdD[b * p.D + d] = dD;
    if (p.pdbias) p.pdbias[b * p.D + d] = dbias;
  }
}

// dst[i] = sum_k src[k * stride + i], k = 0 .. parts-1 in order
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                     int64_t count, int64_t parts, int64_t stride) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  float acc = 0.f;
  for (int64_t k = 0; k < parts; ++k) acc += src[k * stride + i];
  dst[i] = acc;
}

void reduce(const float* src, float* dst, int64_t count, int64_t parts, int64_t stride, hipStream_t stream) {
  const unsigned nb = (unsigned)((count + 255) / 256);
  hipLaunchKernelGGL(reduce_kernel, dim3(nb), dim3(256), 0, stream, src, dst, count, parts, stride);
}

template <bool BF16, int KS>
void launch_ks(const ScanBwdParams& p, hipStream_t stream) {
  const int64_t n_dblk = (p.D + CH - 1) / CH;
  const dim3 grid((unsigned)(n_dblk * p.batch));
  hipLaunchKernelGGL((ckpt_kernel<BF16, KS>), grid, dim3(NT), 0, stream, p, n_dblk);
  hipLaunchKernelGGL((bwd_kernel<BF16, KS>), grid, dim3(NT), 0, stream, p, n_dblk);
  const int64_t bln = p.batch * p.L * p.N;
  reduce(p.pdB, p.dB, bln, n_dblk, bln, stream);
  reduce(p.pdC, p.dC, bln, n_dblk, bln, stream);
  reduce(p.pdA, p.dA, p.D * p.N, p.batch, p.D * p.N, stream);
  if (p.dD) reduce(p.pdD, p.dD, p.D, p.batch, p.D, stream);
  if (p.ddbias) reduce(p.pdbias, p.ddbias, p.D, p.batch, p.D, stream);
}

template <bool BF16>
void launch_io(const ScanBwdParams& p, hipStream_t stream) {
  if (p.N <= 16) launch_ks<BF16, 1>(p, stream);
  else if (p.N <= 32) launch_ks<BF16, 2>(p, stream);
  else launch_ks<BF16, 4>(p, stream);
}

}  // namespace

hipError_t launch_selective_scan_bwd(const ScanBwdParams& p, hipStream_t stream) {
  if (p.io_bf16) launch_io<true>(p, stream);
  else launch_io<false>(p, stream);
  return hipGetLastError();
}

}  // namespace ssm
