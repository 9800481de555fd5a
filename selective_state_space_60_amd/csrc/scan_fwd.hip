// Selective scan (S6) forward for gfx950.
//
// What is computed ("Mamba 논문 리뷰 ... Selective State Space Model",
// tildalice.io: 이산화, Selection Mechanism, 하드웨어 인식 병렬 알고리즘; skip term
// D from the yongggg.tistory.com review, State Space Model section):
//   Abar = exp(delta*A),  Bbar = (exp(delta*A) - 1)/A * B   (zero-order hold)
//   h_t = Abar h_{t-1} + Bbar x_t,   y_t = (C_t . h_t + D x_t) * silu(z_t)
// The pages' recipe -- discretise, scan and multiply by C in one kernel, with
// no (batch, L, D, N) tensor in HBM -- is kept; the blocking is MI355X's own:
//
//  * A 256-thread workgroup owns 32 channels of one batch row and one stretch
//    of the sequence.  Each channel is spread over 8 lanes; a lane keeps N/8
//    states in registers for the whole walk, so the N-wide state never leaves
//    the register file.
//  * The sequence is walked in tiles of 32 steps.  x, delta, z (32 x 32) and
//    B, C (32 x N) of the next tile are fetched with coalesced loads into
//    registers while the current tile is being scanned, then converted to fp32
//    and staged in LDS.  Each lane reads its channel's delta/x and its states'
//    B/C from LDS (broadcast reads).
//  * Per step and state: u = delta*A*log2(e) (1 mul), Abar = v_exp_f32(u)
//    (a half-rate transcendental on gfx950), c = Abar/A - 1/A (1 fma),
//    h = Abar*h + c*(B*x) (3 ops), y += C*h (1 fma).  The 8 lanes of a channel
//    add their partial readouts with three DPP adds.
//  * The readout sums of a tile go to LDS; the whole workgroup then applies
//    the D skip and the SiLU(z) gate, rounds to the output type and writes the
//    tile with coalesced stores.
//  * When the batch x channel count alone cannot fill the 1024 SIMDs (long,
//    narrow problems), the sequence is cut into segments: (1) every segment
//    but the last is scanned from h = 0 for its end state and its sum of
//    delta, (2) a small kernel chains those into the state entering each
//    segment, (3) every segment is scanned again from that state and writes y.
//    This is the associative combine of (Abar, Bbar x) pairs (tildalice.io,
//    병렬 스캔) applied at segment granularity.
#include <hip/hip_runtime.h>

#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int G = kScanLanesPerChannel;
constexpr int CH = kScanChannelsPerBlock;
constexpr int TT = kScanTileSteps;
constexpr int NT = kScanThreads;
constexpr float kLog2e = 1.4426950408889634f;

enum : uint32_t { kHasZ = 1u, kHasD = 2u, kEuler = 4u, kHasH0 = 8u, kWantHLast = 16u };

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

template <bool BF16>
__device__ __forceinline__ float ld_io(const void* p, int64_t i) {
  if constexpr (BF16) return bf2f(((const uint16_t*)p)[i]);
  else return ((const float*)p)[i];
}

// Sum over the 8 lanes of a channel (lanes 8k..8k+7): xor-1, xor-2 within
// quads, then the two quads of each 8-lane half-row.
__device__ __forceinline__ float sum8(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  return v;
}

// Logical block index -> (dblk, seg, b), with blocks of neighbouring
// channels placed on the same XCD (the hardware deals consecutive block ids
// round-robin over the 8 XCDs), so that the 128-byte lines two blocks share
// are fetched into one L2.
__device__ __forceinline__ int64_t logical_block(int64_t nblocks_padded) {
  int64_t i = blockIdx.x;
  return (i & 7) * (nblocks_padded >> 3) + (i >> 3);
}

template <int KS>
struct alignas(16) ScanSmem {
  float x[2][TT][CH];
  float dl[2][TT][CH];
  float z[2][TT][CH];
  float Bt[2][TT][G * KS];
  float Ct[2][TT][G * KS];
  float ysum[TT][CH];
  float Dk[CH];
  int any_zero_A;
};

// Registers holding one tile's global loads while the previous tile is scanned.
template <int KS>
struct TileRegs {
  float x[4], dl[4], z[4];
  float B[KS], C[KS];
};

template <bool BF16, bool VEC>
__device__ __forceinline__ void load4(const void* base, int64_t off, bool row_ok, int dleft, float out[4]) {
  // 4 consecutive channels starting at element `off`; dleft = channels left in D.
  if (VEC && row_ok && dleft >= 4) {
    if constexpr (BF16) {
      uint2 v = *(const uint2*)((const uint16_t*)base + off);
      out[0] = bf2f(v.x & 0xFFFF); out[1] = bf2f(v.x >> 16);
      out[2] = bf2f(v.y & 0xFFFF); out[3] = bf2f(v.y >> 16);
    } else {
      float4 v = *(const float4*)((const float*)base + off);
      out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = (row_ok && j < dleft) ? ld_io<BF16>(base, off + j) : 0.f;
  }
}

template <bool BF16, bool VEC, int KS, bool WANT_Z>
__device__ __forceinline__ void load_tile(const ScanParams& p, int64_t b, int64_t d0, int64_t t0, int64_t t_end,
                                          TileRegs<KS>& r) {
  const int tid = threadIdx.x;
  const int row = tid >> 3, c0 = (tid & 7) * 4;
  const int64_t t = t0 + row;
  const bool row_ok = t < t_end;
  const int dleft = (int)(p.D - (d0 + c0));
  load4<BF16, VEC>(p.x, b * p.xs_b + t * p.xs_t + d0 + c0, row_ok, dleft, r.x);
  load4<BF16, VEC>(p.delta, b * p.ds_b + t * p.ds_t + d0 + c0, row_ok, dleft, r.dl);
  if (WANT_Z) load4<BF16, VEC>(p.z, b * p.zs_b + t * p.zs_t + d0 + c0, row_ok, dleft, r.z);
  // B, C tile: TT x (G*KS) values, KS per thread.
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int e = tid * KS + k;
    const int rr = e / (G * KS), n = e % (G * KS);
    const int64_t tt = t0 + rr;
    const bool ok = tt < t_end && n < p.N;
    r.B[k] = ok ? ld_io<BF16>(p.B, b * p.Bs_b + tt * p.Bs_t + n * p.Bs_n) : 0.f;
    r.C[k] = ok ? ld_io<BF16>(p.C, b * p.Cs_b + tt * p.Cs_t + n * p.Cs_n) : 0.f;
  }
}

template <int KS, bool WANT_Z>
__device__ __forceinline__ void store_tile(ScanSmem<KS>& s, int buf, const TileRegs<KS>& r) {
  const int tid = threadIdx.x;
  const int row = tid >> 3, c0 = (tid & 7) * 4;
  *(float4*)&s.x[buf][row][c0] = make_float4(r.x[0], r.x[1], r.x[2], r.x[3]);
  *(float4*)&s.dl[buf][row][c0] = make_float4(r.dl[0], r.dl[1], r.dl[2], r.dl[3]);
  if (WANT_Z) *(float4*)&s.z[buf][row][c0] = make_float4(r.z[0], r.z[1], r.z[2], r.z[3]);
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int e = threadIdx.x * KS + k;
    (&s.Bt[buf][0][0])[e] = r.B[k];
    (&s.Ct[buf][0][0])[e] = r.C[k];
  }
}

// Discretisation + state update for one step of one lane's KS states.
// DISC: 0 = zero-order hold with A != 0, 1 = zero-order hold allowing A == 0,
// 2 = Bbar = delta*B.   Returns the lane's partial readout sum_k C_k h_k.
template <int KS, int DISC, bool READOUT>
__device__ __forceinline__ float step(float (&h)[KS], const float (&A2)[KS], const float (&iA)[KS],
                                      const float (&ez)[KS], float dt, float xt, const float* Bv,
                                      const float* Cv) {
  float yp = 0.f;
  const float dtx = dt * xt;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const float Ab = __builtin_amdgcn_exp2f(dt * A2[k]);
    if constexpr (DISC == 2) {
      h[k] = __builtin_fmaf(Ab, h[k], Bv[k] * dtx);
    } else {
      // (Abar - 1)/A as Abar*(1/A) - 1/A in one rounding; for A == 0 the
      // factor is 0 and ez*delta supplies the limit delta.
      float c = __builtin_fmaf(Ab, iA[k], -iA[k]);
      if constexpr (DISC == 1) c = __builtin_fmaf(ez[k], dt, c);
      h[k] = __builtin_fmaf(Ab, h[k], c * (Bv[k] * xt));
    }
    if constexpr (READOUT) yp = __builtin_fmaf(Cv[k], h[k], yp);
  }
  return yp;
}

// Scan one tile of `nt` steps held in LDS buffer `buf`.
template <int KS, int DISC, bool READOUT>
__device__ __forceinline__ void scan_tile(ScanSmem<KS>& s, int buf, int nt, float (&h)[KS], const float (&A2)[KS],
                                          const float (&iA)[KS], const float (&ez)[KS], float& sum_dt) {
  const int tid = threadIdx.x;
  const int ch = tid >> 3, sg = tid & 7;
  auto one = [&](int t) {
    const float dt = s.dl[buf][t][ch];
    const float xt = s.x[buf][t][ch];
    float Bv[KS], Cv[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      Bv[k] = s.Bt[buf][t][sg * KS + k];
      if (READOUT) Cv[k] = s.Ct[buf][t][sg * KS + k];
    }
    float yp = step<KS, DISC, READOUT>(h, A2, iA, ez, dt, xt, Bv, Cv);
    if (READOUT) {
      yp = sum8(yp);
      if (sg == (t & 7)) s.ysum[t][ch] = yp;
    } else {
      sum_dt += dt;
    }
  };
  if (nt == TT) {
#pragma unroll 4
    for (int t = 0; t < TT; ++t) one(t);
  } else {
    for (int t = 0; t < nt; ++t) one(t);
  }
}

// MODE 0: write y (and h_last / use h_in).  MODE 1: segment aggregates only.
template <bool BF16, bool VEC, int KS, int MODE>
__global__ __launch_bounds__(NT) void scan_kernel(ScanParams p, int64_t n_dblk, int64_t nseg_run,
                                                  int64_t nblocks_padded) {
  __shared__ ScanSmem<KS> s;
  constexpr int NP = G * KS;
  const int tid = threadIdx.x;
  const int ch = tid >> 3, sg = tid & 7;

  const int64_t lb = logical_block(nblocks_padded);
  if (lb >= n_dblk * nseg_run * p.batch) return;
  const int64_t dblk = lb % n_dblk;
  const int64_t seg = (lb / n_dblk) % nseg_run;
  const int64_t b = lb / (n_dblk * nseg_run);
  const int64_t d0 = dblk * CH;
  const int64_t d = d0 + ch;
  const bool d_ok = d < p.D;
  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = (t_begin + p.seg_len < p.L) ? t_begin + p.seg_len : p.L;
  const bool want_z = MODE == 0 && (p.flags & kHasZ);

  // Per-lane constants: log2(e)*A, 1/A, (A == 0) for this lane's KS states.
  float A2[KS], iA[KS], ez[KS], h[KS];
  int zero_A = 0;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int n = sg * KS + k;
    float a = -1.f;  // padding states (n >= N) and channels (d >= D): any A != 0, B = C = 0
    if (d_ok && n < p.N) a = p.A[d * p.As_d + n * p.As_n];
    zero_A |= (a == 0.f);
    A2[k] = a * kLog2e;
    iA[k] = a != 0.f ? 1.f / a : 0.f;
    ez[k] = a == 0.f ? 1.f : 0.f;
    h[k] = 0.f;
  }
  if (MODE == 0) {
    const float* src = nullptr;
    if (p.n_seg > 1) src = p.h_in + ((b * p.n_seg + seg) * p.D) * p.N;
    else if (p.flags & kHasH0) src = p.h0 + (b * p.D) * p.N;
    if (src && d_ok) {
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const int n = sg * KS + k;
        if (n < p.N) h[k] = src[d * p.N + n];
      }
    }
  }
  if (tid == 0) s.any_zero_A = 0;
  if (tid < CH) s.Dk[tid] = (MODE == 0 && (p.flags & kHasD) && d0 + tid < p.D) ? p.Dskip[(d0 + tid) * p.Ds_d] : 0.f;
  __syncthreads();
  if (zero_A) s.any_zero_A = 1;
  __syncthreads();
  const int disc = (p.flags & kEuler) ? 2 : (s.any_zero_A ? 1 : 0);

  TileRegs<KS> r;
  const int64_t ntiles = (t_end - t_begin + TT - 1) / TT;
  if (want_z) load_tile<BF16, VEC, KS, true>(p, b, d0, t_begin, t_end, r);
  else load_tile<BF16, VEC, KS, false>(p, b, d0, t_begin, t_end, r);
  if (want_z) store_tile<KS, true>(s, 0, r);
  else store_tile<KS, false>(s, 0, r);
  __syncthreads();

  float sum_dt = 0.f;
  for (int64_t it = 0; it < ntiles; ++it) {
    const int buf = (int)(it & 1);
    const int64_t t0 = t_begin + it * TT;
    const int nt = (int)((t_end - t0) < TT ? (t_end - t0) : TT);
    const bool more = it + 1 < ntiles;
    if (more) {
      if (want_z) load_tile<BF16, VEC, KS, true>(p, b, d0, t0 + TT, t_end, r);
      else load_tile<BF16, VEC, KS, false>(p, b, d0, t0 + TT, t_end, r);
    }
    if (MODE == 0) {
      if (disc == 0) scan_tile<KS, 0, true>(s, buf, nt, h, A2, iA, ez, sum_dt);
      else if (disc == 1) scan_tile<KS, 1, true>(s, buf, nt, h, A2, iA, ez, sum_dt);
      else scan_tile<KS, 2, true>(s, buf, nt, h, A2, iA, ez, sum_dt);
      __syncthreads();
      // Finalize the tile: y = (ysum + D x) * silu(z), 4 channels per thread.
      const int row = tid >> 3, c0 = (tid & 7) * 4;
      const int64_t t = t0 + row;
      if (row < nt) {
        float yv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float v = __builtin_fmaf(s.Dk[c0 + j], s.x[buf][row][c0 + j], s.ysum[row][c0 + j]);
          if (want_z) {
            const float zf = s.z[buf][row][c0 + j];
            v *= zf * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-zf * kLog2e));
          }
          yv[j] = v;
        }
        const int dleft = (int)(p.D - (d0 + c0));
        const int64_t off = b * p.ys_b + t * p.ys_t + d0 + c0;
        if (p.y_f32) {
          float* yp = (float*)p.y;
          if (VEC && dleft >= 4) *(float4*)(yp + off) = make_float4(yv[0], yv[1], yv[2], yv[3]);
          else
            for (int j = 0; j < 4; ++j)
              if (j < dleft) yp[off + j] = yv[j];
        } else if (BF16) {
          uint16_t* yp = (uint16_t*)p.y;
          if (VEC && dleft >= 4) {
            uint2 v;
            v.x = (uint32_t)f2bf(yv[0]) | ((uint32_t)f2bf(yv[1]) << 16);
            v.y = (uint32_t)f2bf(yv[2]) | ((uint32_t)f2bf(yv[3]) << 16);
            *(uint2*)(yp + off) = v;
          } else {
            for (int j = 0; j < 4; ++j)
              if (j < dleft) yp[off + j] = f2bf(yv[j]);
          }
        } else {
          float* yp = (float*)p.y;
          if (VEC && dleft >= 4) *(float4*)(yp + off) = make_float4(yv[0], yv[1], yv[2], yv[3]);
          else
            for (int j = 0; j < 4; ++j)
              if (j < dleft) yp[off + j] = yv[j];
        }
      }
    } else {
      if (disc == 0) scan_tile<KS, 0, false>(s, buf, nt, h, A2, iA, ez, sum_dt);
      else if (disc == 1) scan_tile<KS, 1, false>(s, buf, nt, h, A2, iA, ez, sum_dt);
      else scan_tile<KS, 2, false>(s, buf, nt, h, A2, iA, ez, sum_dt);
    }
    if (more) {
      if (want_z) store_tile<KS, true>(s, buf ^ 1, r);
      else store_tile<KS, false>(s, buf ^ 1, r);
    }
    __syncthreads();
  }

  if (!d_ok) return;
  if (MODE == 0) {
    const bool last = seg == p.n_seg - 1;
    if (last && (p.flags & kWantHLast)) {
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const int n = sg * KS + k;
        if (n < p.N) p.h_last[(b * p.D + d) * p.N + n] = h[k];
      }
    }
  } else {
    float* H = p.agg_H + ((b * (p.n_seg - 1) + seg) * p.D + d) * p.N;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int n = sg * KS + k;
      if (n < p.N) H[n] = h[k];
    }
    if (sg == 0) p.agg_S[(b * (p.n_seg - 1) + seg) * p.D + d] = sum_dt;
  }
}

// Chain segment aggregates: h_in[0] = h0 or 0; h_in[s+1] = exp(A*S_s) h_in[s] + H_s.
__global__ __launch_bounds__(256) void scan_combine_kernel(ScanParams p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // over batch*D*N
  if (i >= p.batch * p.D * p.N) return;
  const int64_t n = i % p.N, d = (i / p.N) % p.D, b = i / (p.N * p.D);
  const float a2 = p.A[d * p.As_d + n * p.As_n] * kLog2e;
  float h = (p.flags & kHasH0) ? p.h0[i] : 0.f;
  p.h_in[((b * p.n_seg + 0) * p.D + d) * p.N + n] = h;
  for (int s = 0; s + 1 < p.n_seg; ++s) {
    const float S = p.agg_S[(b * (p.n_seg - 1) + s) * p.D + d];
    const float H = p.agg_H[((b * (p.n_seg - 1) + s) * p.D + d) * p.N + n];
    h = __builtin_fmaf(__builtin_amdgcn_exp2f(a2 * S), h, H);
    p.h_in[((b * p.n_seg + s + 1) * p.D + d) * p.N + n] = h;
  }
}

template <bool BF16, bool VEC, int KS>
hipError_t launch_ks(const ScanParams& p, hipStream_t stream) {
  const int64_t n_dblk = (p.D + CH - 1) / CH;
  auto padded = [](int64_t n) { return (n + 7) / 8 * 8; };
  if (p.n_seg > 1) {
    const int64_t nb = n_dblk * (p.n_seg - 1) * p.batch;
    hipLaunchKernelGGL((scan_kernel<BF16, VEC, KS, 1>), dim3((unsigned)padded(nb)), dim3(NT), 0, stream, p, n_dblk,
                       (int64_t)(p.n_seg - 1), padded(nb));
    const int64_t ncomb = p.batch * p.D * p.N;
    hipLaunchKernelGGL(scan_combine_kernel, dim3((unsigned)((ncomb + 255) / 256)), dim3(256), 0, stream, p);
  }
  const int64_t nb = n_dblk * p.n_seg * p.batch;
  hipLaunchKernelGGL((scan_kernel<BF16, VEC, KS, 0>), dim3((unsigned)padded(nb)), dim3(NT), 0, stream, p, n_dblk,
                     (int64_t)p.n_seg, padded(nb));
  return hipGetLastError();
}

template <bool BF16, bool VEC>
hipError_t launch_io(const ScanParams& p, hipStream_t stream) {
  if (p.N <= G * 1) return launch_ks<BF16, VEC, 1>(p, stream);
  if (p.N <= G * 2) return launch_ks<BF16, VEC, 2>(p, stream);
  if (p.N <= G * 4) return launch_ks<BF16, VEC, 4>(p, stream);
  return launch_ks<BF16, VEC, 8>(p, stream);
}

}  // namespace

hipError_t launch_selective_scan(const ScanParams& p, hipStream_t stream) {
  // Vector tile loads/stores need 4 consecutive channels to be 8-byte (bf16)
  // or 16-byte (fp32) aligned for every (b, t).
  const int64_t e = p.io_bf16 ? 2 : 4;
  const int64_t ye = p.y_f32 ? 4 : e;
  auto al = [](const void* q, int64_t bytes) { return q == nullptr || ((uintptr_t)q % (uintptr_t)bytes) == 0; };
  bool vec = al(p.x, 4 * e) && al(p.delta, 4 * e) && al(p.y, 4 * ye) && p.xs_b % 4 == 0 && p.xs_t % 4 == 0 &&
             p.ds_b % 4 == 0 && p.ds_t % 4 == 0 && p.ys_b % 4 == 0 && p.ys_t % 4 == 0;
  if (p.flags & kHasZ) vec = vec && al(p.z, 4 * e) && p.zs_b % 4 == 0 && p.zs_t % 4 == 0;
  if (p.io_bf16) return vec ? launch_io<true, true>(p, stream) : launch_io<true, false>(p, stream);
  return vec ? launch_io<false, true>(p, stream) : launch_io<false, false>(p, stream);
}

}  // namespace ssm
