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
//     every tile: 1/16 of the states, the rest is recomputed.  (A training
//     forward can store the same states itself; then this pass is skipped.)
//  2. bwd_kernel walks the tiles backwards.  Per tile it recomputes the 16
//     states of each lane from the tile's checkpoint (kept in registers) with
//     the readout C.h, forms g_t and dz_t, then steps the adjoint back through
//     the tile, accumulating dx and ddelta (sums over the lane's states, then
//     over the row through LDS), dB and dC (sums over the workgroup's 16
//     channels: cross-row lane swaps over the 4 rows of a wave, then LDS
//     across the 4 waves) and dA, dD, ddelta_bias in registers.
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

// Sums over the 4 rows (16-lane groups) of a wave, for the dB and dC terms
// of two steps at once, in two gfx950 lane swaps (lane layouts checked on the
// device).  permlane32 swap of (u, v) returns (u's lower half-wave | v's
// lower) and (u's upper | v's upper): their sum holds u's two half-sums (rows
// 0+2, 1+3) in the lower half-wave and v's in the upper.  permlane16 swap of
// (a, b) returns rows (a0, b0, a2, b2) and (a1, b1, a3, b3): their sum is
// (a0+a1, b0+b1, a2+a3, b2+b3).
__device__ __forceinline__ float half_sums(float u, float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(u), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float row_sums(float a, float b) {
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <int... S, class F>
__device__ __forceinline__ void for_steps(std::integer_sequence<int, S...>, F&& f) {
  (f(std::integral_constant<int, S>{}), ...);
}

template <int... S, class F>
__device__ __forceinline__ void for_steps_rev(std::integer_sequence<int, S...>, F&& f) {
  (f(std::integral_constant<int, TT - 1 - S>{}), ...);
}

static_assert(CH * TT == NT, "one (channel, step) of a tile per thread");

// Logical block index: the hardware deals consecutive block ids round-robin
// over the 8 XCDs, each with its own L2.  A tile row of 16 channels is 32
// bytes of a 128-byte line, so neighbouring channel blocks are put on the
// same XCD, where they share each line's one fetch from HBM.
__device__ __forceinline__ int64_t logical_block(int64_t nblocks_padded) {
  const int64_t i = blockIdx.x;
  return (i & 7) * (nblocks_padded >> 3) + (i >> 3);
}

// Update forms (uniform per workgroup): zero-order hold with A != 0, zero-order
// hold with some A == 0 (limit delta), and the simplified Bbar = delta B.
enum Form : int { kZoh = 0, kZohZero = 1, kEuler = 2 };

// The (B, C) pairs of one tile, and per-lane sums of the backward.
template <int KS>
struct BwdSmem {
  float2 bc[TT][G * KS];
  float part[2][NT][TP];          // per-lane partial sums over states, by step
  float red[4][TT][2][G * KS];    // per-wave sums of dB, dC over the wave's 4 channels
};

template <int KS>
struct CkptSmem {
  float2 bc[TT][G * KS];
};

// Lane constants of its KS states.
template <int KS>
struct LaneA {
  float a[KS], A2[KS], iA[KS];
};

// What a thread reads of one tile: step (tid % 16) of channel (tid / 16) --
// the values its lane holds -- and KS (B, C) pairs for the shared staging.
template <int KS>
struct Fetch {
  float x, dr, z;
  uint32_t gy;  // dy as loaded: fp32 bits, or bf16 bits in the low half (converted where it is used)
  float B[KS], C[KS];
};

// One tensor walked tile by tile through a per-lane pointer (VGPRs: the
// strides are needed only here, which keeps the scalar registers free).
struct LanePtr {
  const char* p;     // this lane's element in the current tile
  int64_t step;      // bytes from one tile to the next
  const char* safe;  // a valid element, read in place of one past the end
};

// (batch, L, width) tensor, element (b, t, col) at b*sb + t*st + col*sc:
// lane reads step j, column col of tile `it`.
__device__ __forceinline__ LanePtr lane_ptr(const void* p, int64_t es, int64_t b, int64_t sb, int64_t st, int64_t sc,
                                            int64_t col, int j, int it) {
  LanePtr r;
  r.safe = (const char*)p;
  r.step = TT * st * es;
  r.p = (const char*)p + (b * sb + ((int64_t)it * TT + j) * st + col * sc) * es;
  return r;
}

template <bool BF16>
__device__ __forceinline__ float lload(const LanePtr& w, bool ok) {
  const char* a = ok ? w.p : w.safe;
  if constexpr (BF16) return __uint_as_float((uint32_t)(*(const uint16_t*)a) << 16);
  else return *(const float*)a;
}

template <int KS>
struct LanePtrs {
  LanePtr x, dr, z, gy;
  LanePtr B[KS], C[KS];
};

template <bool BF16, int KS>
__device__ __forceinline__ LanePtrs<KS> lane_ptrs(const ScanBwdParams& p, int64_t b, int64_t d0, int it) {
  const int tid = threadIdx.x;
  const int j = tid % TT;
  const int64_t d = d0 + tid / TT;
  const int64_t e = BF16 ? 2 : 4;
  LanePtrs<KS> w;
  w.x = lane_ptr(p.x, e, b, p.xs_b, p.xs_t, 1, d, j, it);
  w.dr = lane_ptr(p.delta, e, b, p.ds_b, p.ds_t, 1, d, j, it);
  w.z = p.z ? lane_ptr(p.z, e, b, p.zs_b, p.zs_t, 1, d, j, it) : w.x;
  w.gy = lane_ptr(p.dy, p.dy_f32 ? 4 : 2, b, p.gs_b, p.gs_t, 1, d, j, it);
#pragma unroll
  for (int r = 0; r < KS; ++r) {
    const int i = tid + r * NT;
    w.B[r] = lane_ptr(p.B, e, b, p.Bs_b, p.Bs_t, p.Bs_n, i % (G * KS), i / (G * KS), it);
    w.C[r] = lane_ptr(p.C, e, b, p.Cs_b, p.Cs_t, p.Cs_n, i % (G * KS), i / (G * KS), it);
  }
  return w;
}

// Read tile `it` at the pointers, then move them `dir` tiles on.  Loads are
// unconditional (steps, channels and states past the end read a valid
// element, zeroed afterwards).
template <bool BF16, int KS, bool FULL>
__device__ __forceinline__ Fetch<KS> fetch(const ScanBwdParams& p, LanePtrs<KS>& w, int64_t d0, int it, int dir) {
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)it * TT;
  const bool tile_ok = it >= 0;  // tile -1 (after the first) and tiles past the end read nothing
  const bool ok = tile_ok && d0 + tid / TT < p.D && t0 + tid % TT < p.L;
  Fetch<KS> f;
  f.x = lload<BF16>(w.x, ok);
  f.dr = lload<BF16>(w.dr, ok);
  // No conversion behind a branch on p.z or p.dy_f32: converting there makes
  // the compiler wait for these loads (and all before them) at once, while
  // they are meant to be in flight for a whole tile.
  if constexpr (FULL) {
    f.z = lload<BF16>(w.z, ok);  // without z, w.z reads x's element (unused)
    const char* a = ok ? w.gy.p : w.gy.safe;
    f.gy = p.dy_f32 ? *(const uint32_t*)a : (uint32_t)*(const uint16_t*)a;
  }
  if (!ok) {
    f.x = f.dr = f.z = 0.f;
    f.gy = 0u;
  }
  w.x.p += dir * w.x.step;
  w.dr.p += dir * w.dr.step;
  w.z.p += dir * w.z.step;
  w.gy.p += dir * w.gy.step;
#pragma unroll
  for (int r = 0; r < KS; ++r) {
    const int i = tid + r * NT;
    const bool okb = tile_ok && i % (G * KS) < p.N && t0 + i / (G * KS) < p.L;
    f.B[r] = lload<BF16>(w.B[r], okb);
    f.C[r] = FULL ? lload<BF16>(w.C[r], okb) : 0.f;
    if (!okb) f.B[r] = f.C[r] = 0.f;
    w.B[r].p += dir * w.B[r].step;
    w.C[r].p += dir * w.C[r].step;
  }
  return f;
}

template <int KS>
__device__ __forceinline__ void put_bc(float2 (&bc)[TT][G * KS], const Fetch<KS>& f) {
#pragma unroll
  for (int r = 0; r < KS; ++r) {
    const int i = threadIdx.x + r * NT;
    bc[i / (G * KS)][i % (G * KS)] = make_float2(f.B[r], f.C[r]);
  }
}

// The lane's step size for its step: softplus(delta + bias) inside the
// sequence, 0 on padding steps (no change of the state).
__device__ __forceinline__ float step_size(const ScanBwdParams& p, float raw, float bias, bool ok, float& v) {
  v = raw + bias;
  if (!p.dsoftplus) return raw;
  return ok ? softplus_f32(v) : 0.f;
}

// cbar = Bbar / B for one state.
template <int FORM>
__device__ __forceinline__ float cbar(float Ab, float a, float iA, float dt) {
  if constexpr (FORM == kEuler) return dt;
  else if constexpr (FORM == kZoh) return __builtin_fmaf(Ab, iA, -iA);
  else return a != 0.f ? __builtin_fmaf(Ab, iA, -iA) : dt;
}

template <bool BF16, int KS>
__device__ __forceinline__ LaneA<KS> lane_a(const ScanBwdParams& p, int64_t d, int sg, int& zero_a) {
  LaneA<KS> la;
  zero_a = 0;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int n = sg * KS + k;
    float a = -1.f;  // padding states and channels: any A != 0 (B = C = 0 there)
    if (d < p.D && n < p.N) a = p.A[d * p.As_d + n * p.As_n];
    zero_a |= a == 0.f;
    la.a[k] = a;
    la.A2[k] = a * kLog2e;
    la.iA[k] = a != 0.f ? 1.f / a : 0.f;
  }
  return la;
}

// ---------------------------------------------------------- checkpoints

template <bool BF16, int KS, int FORM>
__device__ __forceinline__ void ckpt_walk(CkptSmem<KS>& s, const ScanBwdParams& p, int64_t b, int64_t d0,
                                          const LaneA<KS>& la, float (&h)[KS]) {
  const int tid = threadIdx.x, c = tid / G, sg = tid % G;
  const int64_t d = d0 + c;
  const int ntiles = (int)((p.L + TT - 1) / TT);
  const float bias = (p.dbias && d < p.D) ? p.dbias[d * p.dbs_d] : 0.f;
  LanePtrs<KS> w = lane_ptrs<BF16, KS>(p, b, d0, 0);
  Fetch<KS> cur = fetch<BF16, KS, false>(p, w, d0, 0, 1);
  for (int it = 0; it < ntiles; ++it) {
    if (d < p.D) {
      float* ck = p.ckpt + (((b * ntiles + it) * p.D + d) * p.N);
#pragma unroll
      for (int k = 0; k < KS; ++k)
        if (sg * KS + k < p.N) ck[sg * KS + k] = h[k];
    }
    put_bc<KS>(s.bc, cur);
    float v;
    const float hdt = step_size(p, cur.dr, bias, (int64_t)it * TT + sg < p.L && d < p.D, v), hx = cur.x;
    __syncthreads();
    cur = fetch<BF16, KS, false>(p, w, d0, it + 1, 1);  // past the last tile: masked
    for_steps(std::make_integer_sequence<int, TT>{}, [&](auto S) {
#pragma clang fp contract(off)
      constexpr int T = decltype(S)::value;
      const float dt = row_bcast<T>(hdt), xv = row_bcast<T>(hx);
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const float Ab = __builtin_amdgcn_exp2f(dt * la.A2[k]);
        const float Bv = s.bc[T][sg * KS + k].x;
        h[k] = __builtin_fmaf(Ab, h[k], cbar<FORM>(Ab, la.a[k], la.iA[k], dt) * (Bv * xv));
      }
    });
    __syncthreads();
  }
}

template <bool BF16, int KS, bool EULER>
__global__ __launch_bounds__(NT) void ckpt_kernel(ScanBwdParams p, int64_t n_dblk, int64_t nblocks_padded) {
  __shared__ CkptSmem<KS> s;
  const int tid = threadIdx.x, c = tid / G, sg = tid % G;
  const int64_t lb = logical_block(nblocks_padded);
  if (lb >= n_dblk * p.batch) return;
  const int64_t dblk = lb % n_dblk, b = lb / n_dblk;
  const int64_t d0 = dblk * CH, d = d0 + c;
  int zero_a;
  const LaneA<KS> la = lane_a<BF16, KS>(p, d, sg, zero_a);
  float h[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int n = sg * KS + k;
    h[k] = (p.h0 && d < p.D && n < p.N) ? p.h0[(b * p.D + d) * p.N + n] : 0.f;
  }
  if constexpr (EULER) {
    ckpt_walk<BF16, KS, kEuler>(s, p, b, d0, la, h);
  } else {
    if (__syncthreads_or(zero_a)) ckpt_walk<BF16, KS, kZohZero>(s, p, b, d0, la, h);
    else ckpt_walk<BF16, KS, kZoh>(s, p, b, d0, la, h);
  }
}

// -------------------------------------------------------------- backward

template <bool BF16, int KS, int FORM>
__device__ __forceinline__ void bwd_walk(BwdSmem<KS>& s, const ScanBwdParams& p, int64_t b, int64_t dblk,
                                         int64_t seg, const LaneA<KS>& la) {
  const int tid = threadIdx.x, c = tid / G, sg = tid % G;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int64_t d0 = dblk * CH, d = d0 + c;
  const bool d_ok = d < p.D;
  const bool has_z = p.z != nullptr;
  const float Dk = (p.Dskip && d_ok) ? p.Dskip[d * p.Ds_d] : 0.f;
  const float bias = (p.dbias && d_ok) ? p.dbias[d * p.dbs_d] : 0.f;
  const int ntiles = (int)((p.L + TT - 1) / TT);
  // this workgroup's tiles: its segment's (the whole sequence unless split)
  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = p.n_seg > 1 && t_begin + p.seg_len < p.L ? t_begin + p.seg_len : p.L;
  const int it_lo = (int)(t_begin / TT), it_hi = (int)((t_end - 1) / TT);
  float carry[KS], dA[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int n = sg * KS + k;
    // the adjoint carried in from the later segments (zero for the last)
    carry[k] = (p.n_seg > 1 && d_ok && n < p.N) ? p.cin[((b * p.n_seg + seg) * p.D + d) * p.N + n] : 0.f;
    dA[k] = 0.f;
  }
  float dD = 0.f, dbias = 0.f;  // this lane's steps of its channel
  float* prow = &s.part[0][tid][0];
  static_assert(TT % 2 == 0, "dB, dC row sums pair the steps");
  // this lane's store of the paired row sums: row r of the wave holds step
  // T + 1 - (r & 1) (T even) of dB (r < 2) or dC (r >= 2)
  const int wrow = c % 4;
  float* red_lane = &s.red[wave][0][0][0] + (1 - (wrow & 1)) * 2 * G * KS + (wrow >> 1) * G * KS + sg * KS;

  // Per-lane pointers, set up once and moved one tile per iteration (the
  // loop then needs no strides: fewer live scalar registers).
  const int64_t dd = d_ok ? d : 0;
  const float* ckp = p.ckpt + ((b * ntiles + it_hi) * p.D + dd) * p.N;  // tile it_hi
  const int64_t ck_step = p.D * p.N;
  const int64_t e_dx = p.dx_f32 ? 4 : 2, e_dd = p.dd_f32 ? 4 : 2, e_dz = p.dz_f32 ? 4 : 2;
  char* pdx = (char*)p.dx + (b * p.dxs_b + ((int64_t)it_hi * TT + sg) * p.dxs_t + dd) * e_dx;
  char* pdd = (char*)p.ddelta + (b * p.dds_b + ((int64_t)it_hi * TT + sg) * p.dds_t + dd) * e_dd;
  char* pdz = p.dz ? (char*)p.dz + (b * p.dzs_b + ((int64_t)it_hi * TT + sg) * p.dzs_t + dd) * e_dz : nullptr;
  const int64_t sdx = TT * p.dxs_t * e_dx, sdd = TT * p.dds_t * e_dd, sdz = TT * p.dzs_t * e_dz;
  const bool dx_f32 = p.dx_f32, dd_f32 = p.dd_f32, dz_f32 = p.dz_f32;
  // dB, dC partials: element (j, q, n) of a tile per thread (2 * KS of them)
  constexpr int RED = TT * 2 * G * KS / NT;
  static_assert(RED * NT == TT * 2 * G * KS, "whole tiles of dB, dC partials");
  float* pred[RED];
  bool red_n_ok[RED];
  int red_j[RED];
  const int64_t red_step = (int64_t)TT * p.N;
#pragma unroll
  for (int r = 0; r < RED; ++r) {
    const int i = tid + r * NT;
    const int j = i / (2 * G * KS), q = (i / (G * KS)) % 2, n = i % (G * KS);
    red_j[r] = j;
    red_n_ok[r] = n < p.N;
    pred[r] = (q == 0 ? p.pdB : p.pdC) + ((dblk * p.batch + b) * p.L + (int64_t)it_hi * TT + j) * p.N +
              (n < p.N ? n : 0);
  }
  const int64_t L = p.L;
  const int N = (int)p.N;
  auto ckpt_of = [&](float (&h)[KS]) {
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int n = sg * KS + k;
      const bool ok = d_ok && n < N;
      const float v = ckp[ok ? n : 0];
      h[k] = ok ? v : 0.f;
    }
  };
  LanePtrs<KS> w = lane_ptrs<BF16, KS>(p, b, d0, it_hi);
  Fetch<KS> cur = fetch<BF16, KS, true>(p, w, d0, it_hi, -1);
  float h0n[KS];
  ckpt_of(h0n);
  for (int it = it_hi; it >= it_lo; --it) {
    const int64_t t0 = (int64_t)it * TT;
    const bool j_ok = d_ok && t0 + sg < L;
    put_bc<KS>(s.bc, cur);
    float dv;
    float hdt = step_size(p, cur.dr, bias, j_ok, dv), hx = cur.x;
    const float zj = cur.z, gyj = __uint_as_float(p.dy_f32 ? cur.gy : cur.gy << 16);
    float h0t[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) h0t[k] = h0n[k];
    __syncthreads();
    // the previous tile's inputs are in flight during this tile (before the
    // first tile of the sequence: masked; before a later segment's first
    // tile: read, unused)
    cur = fetch<BF16, KS, true>(p, w, d0, it - 1, -1);
    if (it > 0) ckp -= ck_step;
    ckpt_of(h0n);

    // recompute the tile's states (and Abar) and the readout partials
    float hh[TT][KS], AA[TT][KS];
    {
      float h[KS];
      float2 bc_next[KS];  // the next step's (B, C), read one step ahead
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        h[k] = h0t[k];
        bc_next[k] = s.bc[0][sg * KS + k];
      }
      for_steps(std::make_integer_sequence<int, TT>{}, [&](auto S) {
#pragma clang fp contract(off)
        constexpr int T = decltype(S)::value;
        const float dt = row_bcast<T>(hdt), xv = row_bcast<T>(hx);
        float2 bc_cur[KS];
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          bc_cur[k] = bc_next[k];
          if constexpr (T + 1 < TT) bc_next[k] = s.bc[T + 1][sg * KS + k];
        }
        float yp = 0.f;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          const float2 bcv = bc_cur[k];
          const float Ab = __builtin_amdgcn_exp2f(dt * la.A2[k]);
          h[k] = __builtin_fmaf(Ab, h[k], cbar<FORM>(Ab, la.a[k], la.iA[k], dt) * (bcv.x * xv));
          hh[T][k] = h[k];
          AA[T][k] = Ab;
          yp = __builtin_fmaf(bcv.y, h[k], yp);
        }
        prow[T] = yp;
        __builtin_amdgcn_sched_barrier(0);  // one step at a time: bounded live registers
      });
    }
    // lane sg takes step sg of its channel: o, g, dz
    float o = 0.f;
#pragma unroll
    for (int l = 0; l < G; ++l) o += s.part[0][c * G + l][sg];
    o = __builtin_fmaf(Dk, hx, o);
    float g = gyj;
    if (has_z) {
      const float sgm = sigmoid_f32(zj);
      g = gyj * zj * sgm;
      const float dz = gyj * o * sgm * __builtin_fmaf(zj, 1.f - sgm, 1.f);
      if (j_ok) st(pdz, 0, dz, dz_f32);
    }
    dD = __builtin_fmaf(g, hx, dD);
    // the reverse recomputes its per-step values instead of keeping the
    // recompute phase's (fewer live registers)
    asm volatile("" : "+v"(hdt), "+v"(hx));

    // reverse through the tile
    float held[KS];
    float2 bc_next[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) bc_next[k] = s.bc[TT - 1][sg * KS + k];
    for_steps_rev(std::make_integer_sequence<int, TT>{}, [&](auto S) {
#pragma clang fp contract(off)
      constexpr int T = decltype(S)::value;
      const float dt = row_bcast<T>(hdt), xv = row_bcast<T>(hx), gs = row_bcast<T>(g);
      float dxp = 0.f, dtp = 0.f;
      float vB[KS], vC[KS];
      float2 bc_cur[KS];
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        bc_cur[k] = bc_next[k];
        if constexpr (T > 0) bc_next[k] = s.bc[T - 1][sg * KS + k];
      }
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const float2 bcv = bc_cur[k];
        const float a = la.a[k];
        const float Ab = AA[T][k];
        const float cb = cbar<FORM>(Ab, a, la.iA[k], dt);
        const float hp = T > 0 ? hh[T > 0 ? T - 1 : 0][k] : h0t[k];
        const float l = __builtin_fmaf(bcv.y, gs, carry[k]);
        const float bx = bcv.x * xv;
        vC[k] = gs * hh[T][k];
        const float lc = l * cb;
        vB[k] = lc * xv;
        dxp = __builtin_fmaf(lc, bcv.x, dxp);
        const float la_ = Ab * l;  // Abar lam: the next (earlier) step's carry
        if constexpr (FORM == kEuler) {
          // dh/ddelta = a Abar h_{t-1} + B x;  dh/da = delta Abar h_{t-1}
          dtp = __builtin_fmaf(la_, a * hp, __builtin_fmaf(l, bx, dtp));
          dA[k] = __builtin_fmaf(la_, dt * hp, dA[k]);
        } else {
          // dh/ddelta = Abar (a h_{t-1} + B x);  dh/da = delta Abar h_{t-1} + dcbar/da B x,
          // dcbar/da = (delta Abar - cbar)/a (delta^2/2 at a = 0)
          dtp = __builtin_fmaf(la_, __builtin_fmaf(a, hp, bx), dtp);
          float dc_da = __builtin_fmaf(dt, Ab, -cb) * la.iA[k];
          if constexpr (FORM == kZohZero) dc_da = a != 0.f ? dc_da : 0.5f * dt * dt;
          dA[k] = __builtin_fmaf(la_, dt * hp, __builtin_fmaf(l * dc_da, bx, dA[k]));
        }
        carry[k] = la_;
        // pin the accumulation to this step: left free, the compiler sinks
        // every step's dA terms past the tile and keeps their operands live
        asm volatile("" : "+v"(dA[k]));
      }
      s.part[0][tid][T] = dxp;
      s.part[1][tid][T] = dtp;
      // dB, dC: sums over the wave's 4 channels (rows), two steps at a time.
      // Odd step T keeps its half-sums; at step T - 1 the row sums give row 0
      // dB and row 2 dC of step T, rows 1 and 3 those of step T - 1, and each
      // lane stores its own (a store in every lane: none is left divergent).
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const float u = half_sums(vB[k], vC[k]);
        if constexpr (T % 2 == 1) {
          held[k] = u;
        } else {
          red_lane[T * 2 * G * KS + k] = row_sums(held[k], u);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
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
      dts *= sigmoid_f32(dv);
      if (j_ok) dbias += dts;
    }
    if (j_ok) {
      st(pdx, 0, dxs, dx_f32);
      st(pdd, 0, dts, dd_f32);
    }
    __syncthreads();
    // dB, dC of the tile: sum over the 4 waves, store the workgroup's partial
#pragma unroll
    for (int r = 0; r < RED; ++r) {
      const int i = tid + r * NT;
      const int j = i / (2 * G * KS), q = (i / (G * KS)) % 2, n = i % (G * KS);
      const float v = s.red[0][j][q][n] + s.red[1][j][q][n] + s.red[2][j][q][n] + s.red[3][j][q][n];
      // written once, read back only by the reduction kernel: non-temporal,
      // so these 2 KB per tile do not displace the input lines that the
      // neighbouring workgroups share in L2
      if (t0 + red_j[r] < L && red_n_ok[r]) __builtin_nontemporal_store(v, pred[r]);
      pred[r] -= red_step;
    }
    pdx -= sdx;
    pdd -= sdd;
    if (pdz) pdz -= sdz;
    __syncthreads();
  }
  // per-channel and per-state sums of this batch row (and segment)
  const int64_t bs = b * p.n_seg + seg;
  if (d_ok) {
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int n = sg * KS + k;
      if (n < p.N) {
        p.pdA[(bs * p.D + d) * p.N + n] = dA[k];
        if (p.dh0 && seg == 0) p.dh0[(b * p.D + d) * p.N + n] = carry[k];
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
    if (p.pdD) p.pdD[bs * p.D + d] = dD;
    if (p.pdbias) p.pdbias[bs * p.D + d] = dbias;
  }
}

template <bool BF16, int KS, bool EULER>
__device__ __forceinline__ void bwd_block(BwdSmem<KS>& s, const ScanBwdParams& p, int64_t n_dblk,
                                          int64_t nblocks_padded) {
  const int tid = threadIdx.x;
  const int64_t lb = logical_block(nblocks_padded);
  if (lb >= n_dblk * p.n_seg * p.batch) return;
  const int64_t dblk = lb % n_dblk, seg = (lb / n_dblk) % p.n_seg, b = lb / (n_dblk * p.n_seg);
  int zero_a;
  const LaneA<KS> la = lane_a<BF16, KS>(p, dblk * CH + tid / G, tid % G, zero_a);
  if constexpr (EULER) {
    bwd_walk<BF16, KS, kEuler>(s, p, b, dblk, seg, la);
  } else {
    if (__syncthreads_or(zero_a)) bwd_walk<BF16, KS, kZohZero>(s, p, b, dblk, seg, la);
    else bwd_walk<BF16, KS, kZoh>(s, p, b, dblk, seg, la);
  }
}

template <bool BF16, int KS, bool EULER>
__global__ __launch_bounds__(NT) void bwd_kernel(ScanBwdParams p, int64_t n_dblk, int64_t nblocks_padded) {
  __shared__ BwdSmem<KS> s;
  bwd_block<BF16, KS, EULER>(s, p, n_dblk, nblocks_padded);
}

// One state per lane: capped at 168 VGPRs, three waves per SIMD (at 169 the
// 8-register allocation granule leaves room for two).
template <bool BF16, bool EULER>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_num_vgpr(168))) void bwd_kernel_1(ScanBwdParams p,
                                                                                        int64_t n_dblk,
                                                                                        int64_t nblocks_padded) {
  __shared__ BwdSmem<1> s;
  bwd_block<BF16, 1, EULER>(s, p, n_dblk, nblocks_padded);
}

// ------------------------------------------------- sequence split: carries

// The adjoint recurrence alone, lam_t = C_t g_t + Abar_{t+1} lam_{t+1}, over
// segment s = 1 + (its index) from a zero carry: it needs no state, so it is
// a few operations per state and step.  Writes the carry out of the
// segment's first step, Abar lam (cH), and the segment's sum of delta (cS).
template <bool BF16, int KS>
__global__ __launch_bounds__(NT) void bwd_carry_kernel(ScanBwdParams p, int64_t n_dblk, int64_t nblocks_padded) {
  __shared__ float Cs[TT][G * KS];
  const int tid = threadIdx.x, c = tid / G, sg = tid % G;
  const int64_t lb = logical_block(nblocks_padded);
  if (lb >= n_dblk * (p.n_seg - 1) * p.batch) return;
  const int64_t dblk = lb % n_dblk, seg = 1 + (lb / n_dblk) % (p.n_seg - 1), b = lb / (n_dblk * (p.n_seg - 1));
  const int64_t d0 = dblk * CH, d = d0 + c;
  const bool d_ok = d < p.D;
  const bool has_z = p.z != nullptr;
  const float bias = (p.dbias && d_ok) ? p.dbias[d * p.dbs_d] : 0.f;
  int zero_a;
  const LaneA<KS> la = lane_a<BF16, KS>(p, d, sg, zero_a);
  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = t_begin + p.seg_len < p.L ? t_begin + p.seg_len : p.L;
  const int it_lo = (int)(t_begin / TT), it_hi = (int)((t_end - 1) / TT);
  float carry[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) carry[k] = 0.f;
  float sum_dt = 0.f;
  LanePtrs<KS> w = lane_ptrs<BF16, KS>(p, b, d0, it_hi);
  Fetch<KS> cur = fetch<BF16, KS, true>(p, w, d0, it_hi, -1);
  for (int it = it_hi; it >= it_lo; --it) {
    const bool j_ok = d_ok && (int64_t)it * TT + sg < p.L;
#pragma unroll
    for (int r = 0; r < KS; ++r) {
      const int i = tid + r * NT;
      Cs[i / (G * KS)][i % (G * KS)] = cur.C[r];
    }
    float dv;
    const float hdt = step_size(p, cur.dr, bias, j_ok, dv);
    const float zj = cur.z, gyj = __uint_as_float(p.dy_f32 ? cur.gy : cur.gy << 16);
    const float g = has_z ? gyj * zj * sigmoid_f32(zj) : gyj;
    sum_dt += hdt;
    __syncthreads();
    cur = fetch<BF16, KS, true>(p, w, d0, it - 1, -1);  // before the segment: read, unused
    for_steps_rev(std::make_integer_sequence<int, TT>{}, [&](auto S) {
#pragma clang fp contract(off)
      constexpr int T = decltype(S)::value;
      const float dt = row_bcast<T>(hdt), gs = row_bcast<T>(g);
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const float Ab = __builtin_amdgcn_exp2f(dt * la.A2[k]);
        carry[k] = Ab * __builtin_fmaf(Cs[T][sg * KS + k], gs, carry[k]);
      }
    });
    __syncthreads();
  }
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) sum_dt += __shfl_xor(sum_dt, m, G);
  if (!d_ok) return;
  const int64_t bs = b * p.n_seg + seg;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int n = sg * KS + k;
    if (n < p.N) p.cH[(bs * p.D + d) * p.N + n] = carry[k];
  }
  if (sg == 0) p.cS[bs * p.D + d] = sum_dt;
}

// The carry into each segment's last step, from the last segment back:
// cin[n_seg-1] = 0;  cin[s-1] = cH[s] + exp(A * cS[s]) cin[s].
__global__ __launch_bounds__(256) void bwd_combine_kernel(ScanBwdParams p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // over batch*D*N
  if (i >= p.batch * p.D * p.N) return;
  const int64_t n = i % p.N, d = (i / p.N) % p.D, b = i / (p.N * p.D);
  const float a2 = p.A[d * p.As_d + n * p.As_n] * kLog2e;
  float c = 0.f;
  p.cin[((b * p.n_seg + p.n_seg - 1) * p.D + d) * p.N + n] = 0.f;
  for (int64_t sgm = p.n_seg - 1; sgm >= 1; --sgm) {
    const int64_t bs = b * p.n_seg + sgm;
    c = __builtin_fmaf(__builtin_amdgcn_exp2f(a2 * p.cS[bs * p.D + d]), c, p.cH[(bs * p.D + d) * p.N + n]);
    p.cin[((bs - 1) * p.D + d) * p.N + n] = c;
  }
}

// dst[i] = sum_k src[k * stride + i] over k = 0 .. parts-1, in a fixed order:
// the RG waves of a workgroup each add one run of consecutive parts in order
// (run r holds parts [r*parts/RG, (r+1)*parts/RG)), then the run sums are
// added in run order.  V consecutive elements per lane (V = 4: 16-byte
// loads, for 16-byte aligned buffers, count and stride).  RG loads in flight
// per column keep the partial sums streaming from HBM.
constexpr int RG = 4;

template <int V>
struct Vec {
  float v[V];
};

template <int V>
__device__ __forceinline__ Vec<V> vload(const float* p) {
  Vec<V> r;
  if constexpr (V == 4) {
    const float4 q = *(const float4*)p;
    r.v[0] = q.x, r.v[1] = q.y, r.v[2] = q.z, r.v[3] = q.w;
  } else {
    r.v[0] = *p;
  }
  return r;
}

template <int V>
__global__ __launch_bounds__(64 * RG) void reduce_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                         int64_t count, int64_t parts, int64_t stride) {
  __shared__ float run_sum[RG - 1][64 * V];
  const int c = threadIdx.x % 64, r = threadIdx.x / 64;
  const int64_t i = ((int64_t)blockIdx.x * 64 + c) * V;
  const bool ok = i < count;
  const int64_t k0 = r * parts / RG, k1 = (r + 1) * parts / RG;
  float acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = 0.f;
  if (ok) {
    const float* q = src + k0 * stride + i;
    int64_t k = k0;
    for (; k + 4 <= k1; k += 4, q += 4 * stride) {
      const Vec<V> a = vload<V>(q), b = vload<V>(q + stride), d = vload<V>(q + 2 * stride),
                   e4 = vload<V>(q + 3 * stride);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = ((acc[e] + a.v[e]) + b.v[e] + d.v[e]) + e4.v[e];
    }
    for (; k < k1; ++k, q += stride) {
      const Vec<V> a = vload<V>(q);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += a.v[e];
    }
  }
  if (r > 0) {
#pragma unroll
    for (int e = 0; e < V; ++e) run_sum[r - 1][c * V + e] = acc[e];
  }
  __syncthreads();
  if (r == 0 && ok) {
#pragma unroll
    for (int g = 0; g < RG - 1; ++g)
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += run_sum[g][c * V + e];
    if constexpr (V == 4) *(float4*)(dst + i) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    else dst[i] = acc[0];
  }
}

void reduce(const float* src, float* dst, int64_t count, int64_t parts, int64_t stride, hipStream_t stream) {
  const bool v4 = count % 4 == 0 && stride % 4 == 0 && ((uintptr_t)src | (uintptr_t)dst) % 16 == 0;
  if (v4) {
    const unsigned nb = (unsigned)((count / 4 + 63) / 64);
    hipLaunchKernelGGL(reduce_kernel<4>, dim3(nb), dim3(64 * RG), 0, stream, src, dst, count, parts, stride);
  } else {
    const unsigned nb = (unsigned)((count + 63) / 64);
    hipLaunchKernelGGL(reduce_kernel<1>, dim3(nb), dim3(64 * RG), 0, stream, src, dst, count, parts, stride);
  }
}

template <bool BF16, int KS>
void launch_ks(const ScanBwdParams& p, hipStream_t stream) {
  const int64_t n_dblk = (p.D + CH - 1) / CH;
  auto pad8 = [](int64_t n) { return (n + 7) / 8 * 8; };  // blocks past the end exit at once
  const int64_t npad = pad8(n_dblk * p.batch);
  const dim3 grid((unsigned)npad);
  // unsplit, the checkpoint pass (the split path's checkpoints come from the
  // forward's split kernels, run by the caller)
  if (!p.ckpt_given) {
    if (p.euler) hipLaunchKernelGGL((ckpt_kernel<BF16, KS, true>), grid, dim3(NT), 0, stream, p, n_dblk, npad);
    else hipLaunchKernelGGL((ckpt_kernel<BF16, KS, false>), grid, dim3(NT), 0, stream, p, n_dblk, npad);
  }
  if (p.n_seg > 1) {
    const int64_t nc = pad8(n_dblk * (p.n_seg - 1) * p.batch);
    hipLaunchKernelGGL((bwd_carry_kernel<BF16, KS>), dim3((unsigned)nc), dim3(NT), 0, stream, p, n_dblk, nc);
    const int64_t ncomb = p.batch * p.D * p.N;
    hipLaunchKernelGGL(bwd_combine_kernel, dim3((unsigned)((ncomb + 255) / 256)), dim3(256), 0, stream, p);
  }
  const int64_t nb = pad8(n_dblk * p.n_seg * p.batch);
  const dim3 gb((unsigned)nb);
  if constexpr (KS == 1) {
    if (p.euler) hipLaunchKernelGGL((bwd_kernel_1<BF16, true>), gb, dim3(NT), 0, stream, p, n_dblk, nb);
    else hipLaunchKernelGGL((bwd_kernel_1<BF16, false>), gb, dim3(NT), 0, stream, p, n_dblk, nb);
  } else {
    if (p.euler) hipLaunchKernelGGL((bwd_kernel<BF16, KS, true>), gb, dim3(NT), 0, stream, p, n_dblk, nb);
    else hipLaunchKernelGGL((bwd_kernel<BF16, KS, false>), gb, dim3(NT), 0, stream, p, n_dblk, nb);
  }
  const int64_t bln = p.batch * p.L * p.N;
  const int64_t nbs = p.batch * p.n_seg;  // parts of the per-row sums: batch rows x segments
  reduce(p.pdB, p.dB, bln, n_dblk, bln, stream);
  reduce(p.pdC, p.dC, bln, n_dblk, bln, stream);
  reduce(p.pdA, p.dA, p.D * p.N, nbs, p.D * p.N, stream);
  if (p.dD) reduce(p.pdD, p.dD, p.D, nbs, p.D, stream);
  if (p.ddbias) reduce(p.pdbias, p.ddbias, p.D, nbs, p.D, stream);
}

template <bool BF16>
void launch_io(const ScanBwdParams& p, hipStream_t stream) {
  if (p.N <= 16) launch_ks<BF16, 1>(p, stream);
  else if (p.N <= 32) launch_ks<BF16, 2>(p, stream);
  else launch_ks<BF16, 4>(p, stream);
}

}  // namespace

void launch_fixed_order_sum(const float* src, float* dst, int64_t count, int64_t parts, int64_t stride,
                            hipStream_t stream) {
  reduce(src, dst, count, parts, stride, stream);
}

hipError_t launch_selective_scan_bwd(const ScanBwdParams& p, hipStream_t stream) {
  if (p.io_bf16) launch_io<true>(p, stream);
  else launch_io<false>(p, stream);
  return hipGetLastError();
}

}  // namespace ssm
