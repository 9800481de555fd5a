// Selective scan (S6) forward for gfx950.
//
// What is computed ("Mamba 논문 리뷰 ... Selective State Space Model",
// tildalice.io: 이산화, Selection Mechanism, 하드웨어 인식 병렬 알고리즘; skip term
// D from the yongggg.tistory.com review, State Space Model section):
//   Abar = exp(delta*A),  Bbar = (exp(delta*A) - 1)/A * B   (zero-order hold)
//   h_t = Abar h_{t-1} + Bbar x_t,   y_t = (C_t . h_t + D x_t) * silu(z_t)
// The pages' recipe -- discretise, scan and multiply by C in one kernel, with
// no (batch, L, D, N) tensor in HBM -- is kept; the blocking is MI355X's own.
//
// On gfx950 this path is bound by VALU issue and LDS bandwidth, not by HBM:
// every state of every token*channel costs one v_exp_f32 (half rate) and
// several fp32 ops, against ~8 bytes of HBM traffic per token*channel.
// Everything else is arranged to add as little as possible on top:
//
//  * A 256-thread workgroup owns 16 channels of one batch row and one stretch
//    of the sequence.  Each channel is one 16-lane row of a wave; a lane keeps
//    N/16 states in registers for the whole walk (one state at N = 16), so the
//    N-wide state never leaves the register file.  With 16 lanes per channel a
//    wide layer gives thousands of equal waves.
//  * The sequence is walked in tiles of 16 steps, and lane j of a channel's
//    row also holds step j of the tile: its delta, x and z.  A step broadcasts
//    delta and x from that lane to the row with a DPP row broadcast folded
//    into the multiply that consumes them, so they cost no extra instruction
//    and no LDS traffic.  B and C (16 x N per tile, shared by the 16 channels)
//    are staged in LDS as (B, C) pairs; a lane reads two steps' worth with one
//    16-byte read.
//  * Global memory is touched in whole rows of the workgroup's 16 channels
//    (32 bytes in bf16): thread (t, c) = (tid/16, tid%16) loads x, delta, z
//    of step t, channel c and stores y the same way; a small LDS transpose
//    hands them to and from the lanes that hold them.  Loads run two tiles
//    ahead, into registers, as buffer loads: each lane's byte offset inside a
//    tile is fixed and the buffer base advances in SGPRs; in the last tile of
//    a stretch the descriptor's range ends at the last element that belongs
//    to it, so reads past the end return zero without touching memory.
//  * Per step and state, with A != 0 and one state per lane, the kernel
//    carries g = A*h instead of h:  g_t = Abar*(g_{t-1} + B x) - B x, the
//    zero-order-hold update multiplied through by A.  That is one exp2, two
//    multiplies (delta*A*log2(e) and B*x), an add and an fma; the factor 1/A
//    moves out of the recurrence into the readout sum.  Workgroups with
//    several states per lane, with A == 0 somewhere (limit delta*B), or with
//    the simplified discretisation (Bbar = delta*B) carry h itself.
//  * Each lane writes its partial readout (C*g, or C.h over its states) to
//    LDS; after every tile lane j of a channel's row sums the 16 partials of
//    step j -- weighted by 1/A of the state in the g form -- adds D*x and
//    applies SiLU(z).  The partials are wave-private, so this needs no
//    workgroup barrier; the results go through LDS to the row-wise stores of
//    the next tile.
//  * When batch x channels cannot fill the GPU (long, narrow problems), the
//    sequence is cut into segments: (1) each segment but the last is scanned
//    from h = 0 for its end state and its sum of delta, (2) a small kernel
//    chains those into the state entering each segment (the associative
//    combine of (Abar, Bbar x) pairs -- tildalice.io, 병렬 스캔 -- at segment
//    granularity), (3) every segment is scanned from its entering state and
//    writes y.
#include <hip/hip_runtime.h>

#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int G = kScanLanesPerChannel;    // 16 lanes per channel (one DPP row)
constexpr int CH = kScanChannelsPerBlock;  // 16 channels per workgroup
constexpr int TT = kScanTileSteps;         // 16 steps per tile (one per lane of a row)
constexpr int NT = kScanThreads;           // 256 threads
constexpr int UB = 4;                      // steps per register block
constexpr int TP = TT + 2;                 // time pitch (float2) of the staged B/C; even keeps 16-byte reads aligned
constexpr int PN = TT * (64 / G) + 4;      // pitch (floats) of one state's row of partials
constexpr int HP = TT + 1;                 // pitch of the per-channel step arrays of the LDS transpose
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // buffer descriptor word 3 for raw (unformatted) access on gfx9

static_assert(G == 16 && TT == G && CH * G == NT && UB == 4, "tiling");

enum : uint32_t { kHasZ = 1u, kHasD = 2u, kEuler = 4u, kHasH0 = 8u, kWantHLast = 16u };

// Update forms (uniform per workgroup):
//   kFormG     : g = A*h, zero-order hold, A != 0 everywhere, one state per lane
//   kFormH     : h, zero-order hold, A != 0
//   kFormHZero : h, zero-order hold, some A == 0 (limit delta*B)
//   kFormEuler : h, Bbar = delta*B
enum Form : int { kFormG = 0, kFormH = 1, kFormHZero = 2, kFormEuler = 3 };

// Logical block index with blocks of neighbouring channels placed on the same
// XCD (the hardware deals consecutive block ids round-robin over the 8 XCDs),
// so the cache lines several blocks share are fetched into one L2.
__device__ __forceinline__ int64_t logical_block(int64_t nblocks_padded) {
  const int64_t i = blockIdx.x;
  return (i & 7) * (nblocks_padded >> 3) + (i >> 3);
}

// Value of lane T of this lane's 16-lane row (DPP row broadcast).
template <int T>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + T, 0xF, 0xF, true));
}

// A wave-uniform walk over a tensor: the address of the current tile's first
// element (b, t0, d0), the bytes from one tile to the next, and the byte
// range of the stretch's last tile (up to and including its last element).
// Accesses go through a raw buffer descriptor at that address; reads at or
// beyond the range return zero and touch no memory.
struct Span {
  const char* p;
  int32_t step;
  uint32_t last_range;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const Span& s, bool last) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)s.p, (short)0, (int)(last ? s.last_range : 0xFFFFFFFFu),
                                           (int)kRsrcWord3);
}

__device__ __forceinline__ void advance(Span& s) { s.p += s.step; }

template <bool BF16>
__device__ __forceinline__ uint32_t bload(const Span& s, bool last, uint32_t voff) {
  if constexpr (BF16) return __builtin_amdgcn_raw_buffer_load_b16(rsrc(s, last), (int)voff, 0, 0);
  else return __builtin_amdgcn_raw_buffer_load_b32(rsrc(s, last), (int)voff, 0, 0);
}

template <bool BF16>
__device__ __forceinline__ float raw2f(uint32_t v) {
  if constexpr (BF16) return __uint_as_float(v << 16);
  else return __uint_as_float(v);
}

template <int KS>
struct alignas(16) ScanSmem {
  float2 bc[2][G * KS][TP];  // (B_n, C_n), time-major per state, double-buffered
  // Partial readouts, wave-private: part[wave][state lane][16*(channel of wave) + step]
  float part[NT / 64][G][PN];
  float2 hx[2][CH][HP];      // (delta, x) per channel and step, double-buffered
  uint32_t hz[2][CH][HP];    // z (raw bits)
  float yb[2][CH][HP];       // finalized y, stored row-wise one tile later
};

// One tile's global loads, held as raw bits until the tile is staged: they
// are issued two tiles ahead of use, and converting them at load time would
// make the wave wait for them right away.
template <int KS>
struct Raw {
  uint32_t x, dl, z;
  uint32_t B[KS], C[KS];
};

// The current tile's per-channel values held by this lane (step lane%16).
struct Hold {
  float dt, x, xs;  // delta, x, and the value broadcast as x (x, or delta*x in the Euler form)
  uint32_t z;       // raw bits
};

// Per-lane byte offsets inside a tile (fixed for the whole walk).
template <int KS>
struct Offs {
  uint32_t x, dl, z, y;
  uint32_t B[KS], C[KS];
  bool bc_ok[KS];  // the staged state exists (n < N)
};

// Everything one workgroup needs while walking its stretch of the sequence.
template <int KS>
struct Walk {
  Span x, dl, z, B, C;  // load heads (advance as tiles are loaded)
  Span y;               // store head (advances as tiles are finalized)
  Offs<KS> o;
  int ntiles;           // tiles in the stretch
  int last_rows;        // rows of the last tile that belong to the stretch (1..TT)
  int st_t;             // row-wise role: step (tid/16) of this thread's loads and stores
  bool st_ch_ok;        // row-wise role: channel tid%16 exists
  bool y_f32;
};

// Per-lane constants of this lane's KS states.
template <int KS>
struct Lane {
  float A2[KS];  // log2(e) * A
  float iA[KS];  // 1/A (0 where A == 0)
  float ez[KS];  // 1 where A == 0, else 0
};

template <bool BF16, int KS, bool WANT_Z>
__device__ __forceinline__ void load_tile(Walk<KS>& w, int it, Raw<KS>& r) {
  const bool last = it == w.ntiles - 1;
  r.x = bload<BF16>(w.x, last, w.o.x);
  r.dl = bload<BF16>(w.dl, last, w.o.dl);
  if constexpr (WANT_Z) r.z = bload<BF16>(w.z, last, w.o.z);
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    r.B[k] = bload<BF16>(w.B, last, w.o.B[k]);
    r.C[k] = bload<BF16>(w.C, last, w.o.C[k]);
  }
  advance(w.x);
  advance(w.dl);
  if constexpr (WANT_Z) advance(w.z);
  advance(w.B);
  advance(w.C);
}

// Make tile `it` (raw registers r) current: B/C into LDS buffer `buf`, this
// lane's step into registers.  Rows at or past the end of the stretch are
// zeroed: delta = x = 0 leaves every state unchanged, so a partial last tile
// is scanned like a full one.
template <bool BF16, int KS>
__device__ __forceinline__ void stage_tile(ScanSmem<KS>& s, int buf, const Walk<KS>& w, int it, const Raw<KS>& r) {
  const int tid = threadIdx.x;
  float dt = raw2f<BF16>(r.dl), xv = raw2f<BF16>(r.x);
  float Bv[KS], Cv[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    Bv[k] = w.o.bc_ok[k] ? raw2f<BF16>(r.B[k]) : 0.f;
    Cv[k] = w.o.bc_ok[k] ? raw2f<BF16>(r.C[k]) : 0.f;
  }
  if (it == w.ntiles - 1) {  // uniform: only the last tile
    const bool st_ok = w.st_t < w.last_rows;
    dt = st_ok ? dt : 0.f;
    xv = st_ok ? xv : 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      Bv[k] = st_ok ? Bv[k] : 0.f;
      Cv[k] = st_ok ? Cv[k] : 0.f;
    }
  }
#pragma unroll
  for (int k = 0; k < KS; ++k) s.bc[buf][(tid % G) + G * k][w.st_t] = make_float2(Bv[k], Cv[k]);
  s.hx[buf][tid % G][w.st_t] = make_float2(dt, xv);
  s.hz[buf][tid % G][w.st_t] = r.z;
}

// This lane's step (lane%16) of its channel (tid/16) for the tile in `buf`.
template <int KS, int FORM>
__device__ __forceinline__ void take_hold(const ScanSmem<KS>& s, int buf, bool want_z, Hold& hd) {
  const int tid = threadIdx.x;
  const float2 v = s.hx[buf][tid / G][tid % G];
  hd.dt = v.x;
  hd.x = v.y;
  hd.xs = FORM == kFormEuler ? v.x * v.y : v.y;
  hd.z = want_z ? s.hz[buf][tid / G][tid % G] : 0u;
}

// One step (step T of the tile) of one lane's KS states; returns the lane's
// partial readout.  delta and x come from lane T of the row.  No implicit
// fusing of multiplies into adds here: that would turn the broadcast
// multiplies into fmas, which cannot take the DPP operand.
template <int KS, int FORM, bool READOUT, int T>
__device__ __forceinline__ float step(float (&h)[KS], const Lane<KS>& ln, const Hold& hd, const float4 (&bc)[KS],
                                      bool hi) {
#pragma clang fp contract(off)
  float yp = 0.f;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const float Bv = hi ? bc[k].z : bc[k].x;
    const float Cv = hi ? bc[k].w : bc[k].y;
    const float Ab = __builtin_amdgcn_exp2f(row_bcast<T>(hd.dt) * ln.A2[k]);
    const float q = row_bcast<T>(hd.xs) * Bv;  // B*x (B*delta*x in the Euler form)
    if constexpr (FORM == kFormG) {
      h[k] = __builtin_fmaf(Ab, h[k] + q, -q);
    } else if constexpr (FORM == kFormEuler) {
      h[k] = __builtin_fmaf(Ab, h[k], q);
    } else {
      // (Abar - 1)/A as Abar*(1/A) - 1/A with one rounding; with A == 0 the
      // factor is 0 and ez*delta supplies the limit delta.
      float c = __builtin_fmaf(Ab, ln.iA[k], -ln.iA[k]);
      if constexpr (FORM == kFormHZero) c = __builtin_fmaf(ln.ez[k], row_bcast<T>(hd.dt), c);
      h[k] = __builtin_fmaf(Ab, h[k], c * q);
    }
    if constexpr (READOUT) yp = k == 0 ? Cv * h[k] : __builtin_fmaf(Cv, h[k], yp);
  }
  return yp;
}

// B/C of steps t0 .. t0+3 for this lane's states: o[u][k] = (B_t, C_t, B_t+1, C_t+1), t = t0 + 2u.
template <int KS>
__device__ __forceinline__ void read_block(const ScanSmem<KS>& s, int buf, int t0, int sg, float4 (&o)[2][KS]) {
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int k = 0; k < KS; ++k) o[u][k] = *(const float4*)&s.bc[buf][sg * KS + k][t0 + 2 * u];
}

// Blocks BLK.. of one tile: operands of block BLK+1 are read while block BLK
// is scanned.  prow: this lane's row of partials (column 16*channel).
template <int KS, int FORM, bool READOUT, int BLK>
__device__ __forceinline__ void scan_blocks(const ScanSmem<KS>& s, float* prow, int buf, int sg, float (&h)[KS],
                                            const Lane<KS>& ln, const Hold& hd, float4 (&o)[2][2][KS]) {
  if constexpr (BLK < TT / UB) {
    if constexpr (BLK + 1 < TT / UB) read_block<KS>(s, buf, (BLK + 1) * UB, sg, o[(BLK + 1) & 1]);
    const float4(&c)[2][KS] = o[BLK & 1];
    float yp[UB];
    yp[0] = step<KS, FORM, READOUT, UB * BLK + 0>(h, ln, hd, c[0], false);
    yp[1] = step<KS, FORM, READOUT, UB * BLK + 1>(h, ln, hd, c[0], true);
    yp[2] = step<KS, FORM, READOUT, UB * BLK + 2>(h, ln, hd, c[1], false);
    yp[3] = step<KS, FORM, READOUT, UB * BLK + 3>(h, ln, hd, c[1], true);
    if (READOUT) *(float4*)&prow[UB * BLK] = make_float4(yp[0], yp[1], yp[2], yp[3]);
    scan_blocks<KS, FORM, READOUT, BLK + 1>(s, prow, buf, sg, h, ln, hd, o);
  }
}

// Finalize a tile: lane j of the row takes step j: y = (sum_n w_n partial_n +
// D x) * silu(z), w_n = 1/A_n in the g form, else 1.  pcol: the lane's
// (channel, step) column in state row 0 of the partials.
template <bool BF16, int KS, int FORM>
__device__ __forceinline__ void finalize_tile(ScanSmem<KS>& s, int buf, const float* pcol, const float (&fA)[G],
                                              float Dk, const Hold& hd, bool want_z) {
  float acc = 0.f;
#pragma unroll
  for (int n = 0; n < G; ++n) {
    const float v = pcol[n * PN];
    if constexpr (FORM == kFormG) acc = __builtin_fmaf(fA[n], v, acc);
    else acc += v;
  }
  float v = __builtin_fmaf(Dk, hd.x, acc);
  if (want_z) {
    const float zf = raw2f<BF16>(hd.z);
    v *= zf * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-zf * kLog2e));
  }
  s.yb[buf][threadIdx.x / G][threadIdx.x % G] = v;
}

// Store tile `it` (finalized into yb[buf] before the last barrier) row-wise:
// thread (t, c) = (tid/16, tid%16) stores step t of channel c.
template <bool BF16, int KS>
__device__ __forceinline__ void store_y(const ScanSmem<KS>& s, int buf, Walk<KS>& w, int it) {
  const float v = s.yb[buf][threadIdx.x % G][w.st_t];
  const bool row_ok = it < w.ntiles - 1 || w.st_t < w.last_rows;
  if (row_ok && w.st_ch_ok) {
    if (w.y_f32 || !BF16)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rsrc(w.y, false), (int)w.o.y, 0, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)v), rsrc(w.y, false), (int)w.o.y,
                                            0, 0);
  }
  advance(w.y);
}

// The walk over the stretch, for one update form.  MODE 0 writes y;
// MODE 1 only carries the state (from 0) and this lane's share of the sum of
// delta (the steps it holds).
template <bool BF16, int KS, int MODE, int FORM>
__device__ __forceinline__ void walk(ScanSmem<KS>& s, Walk<KS>& w, float (&h)[KS], const Lane<KS>& ln,
                                     const float (&fA)[G], float Dk, bool want_z, float& sum_dt) {
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, sg = tid % G;
  float* prow = &s.part[wave][sg][G * (lane / G)];
  const float* pcol = &s.part[wave][0][lane];
  // Loads run two tiles ahead of use: ra/rb hold the tiles with it & 1 == 0/1.
  Raw<KS> ra, rb;
  Hold hd;
  auto load = [&](int it, Raw<KS>& r) {
    if (want_z) load_tile<BF16, KS, true>(w, it, r);
    else load_tile<BF16, KS, false>(w, it, r);
  };
  load(0, ra);
  stage_tile<BF16, KS>(s, 0, w, 0, ra);
  if (w.ntiles > 1) load(1, rb);
  if (w.ntiles > 2) load(2, ra);
  __syncthreads();
  // One tile: take this lane's step, scan, finalize into yb, store the
  // previous tile's y, stage tile it+1 (held in rn) and refill rn with tile
  // it+3.
  auto body = [&](int it, Raw<KS>& rn) {
    const int buf = it & 1;
    take_hold<KS, FORM>(s, buf, want_z, hd);
    float4 o[2][2][KS];
    read_block<KS>(s, buf, 0, sg, o[0]);
    scan_blocks<KS, FORM, MODE == 0, 0>(s, prow, buf, sg, h, ln, hd, o);
    if (MODE == 0) {
      finalize_tile<BF16, KS, FORM>(s, buf, pcol, fA, Dk, hd, want_z);
      if (it > 0) store_y<BF16, KS>(s, buf ^ 1, w, it - 1);
    } else {
      sum_dt += hd.dt;
    }
    if (it + 1 < w.ntiles) {
      stage_tile<BF16, KS>(s, buf ^ 1, w, it + 1, rn);
      if (it + 3 < w.ntiles) load(it + 3, rn);
    }
    __syncthreads();
  };
  for (int it = 0; it < w.ntiles; it += 2) {
    body(it, rb);
    if (it + 1 < w.ntiles) body(it + 1, ra);
  }
  if (MODE == 0) store_y<BF16, KS>(s, (w.ntiles - 1) & 1, w, w.ntiles - 1);
}

// MODE 0: write y (and h_last / start from h_in).  MODE 1: segment aggregates.
template <bool BF16, int KS, int MODE>
__global__ __launch_bounds__(NT) void scan_kernel(ScanParams p, int64_t n_dblk, int64_t nseg_run,
                                                  int64_t nblocks_padded) {
  __shared__ ScanSmem<KS> s;
  const int tid = threadIdx.x;
  const int chb = tid / G, sg = tid % G;

  const int64_t lb = logical_block(nblocks_padded);
  if (lb >= n_dblk * nseg_run * p.batch) return;
  const int64_t dblk = lb % n_dblk;
  const int64_t seg = (lb / n_dblk) % nseg_run;
  const int64_t b = lb / (n_dblk * nseg_run);
  const int64_t d0 = dblk * CH;
  const int64_t d = d0 + chb;  // this lane's channel (scan and finalize)
  const bool d_ok = d < p.D;
  const bool want_z = MODE == 0 && (p.flags & kHasZ);
  const int64_t esz = BF16 ? 2 : 4;

  Walk<KS> w;
  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = (t_begin + p.seg_len < p.L) ? t_begin + p.seg_len : p.L;
  w.ntiles = (int)((t_end - t_begin + TT - 1) / TT);
  w.last_rows = (int)(t_end - t_begin - (int64_t)(w.ntiles - 1) * TT);
  w.y_f32 = p.y_f32 != 0;

  // Per-lane constants of this lane's KS states.
  Lane<KS> ln;
  float Av[KS], h[KS];
  int zero_A = 0;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int n = sg * KS + k;
    float a = -1.f;  // padding states (n >= N) and channels (d >= D): any A != 0, B = C = 0
    if (d_ok && n < p.N) a = p.A[d * p.As_d + n * p.As_n];
    zero_A |= (a == 0.f);
    Av[k] = a;
    ln.A2[k] = a * kLog2e;
    ln.iA[k] = a != 0.f ? 1.f / a : 0.f;
    ln.ez[k] = a == 0.f ? 1.f : 0.f;
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
  const bool any_zero_A = __syncthreads_or(zero_A) != 0;

  float Dk = 0.f;
  if (MODE == 0 && (p.flags & kHasD) && d_ok) Dk = p.Dskip[d * p.Ds_d];

  // Streams: each starts at element (b, t_begin, d0) (state 0 for B, C) and
  // advances one tile of rows at a time.  The last tile's range ends at its
  // last row's last element (channel D-1 or state N-1): lanes of rows past
  // the stretch, or of channels / states past the end of the tensor's last
  // row, read zeros.  (Rows past the stretch inside the tensor may also be
  // read; stage_tile discards them.)
  const int64_t rows_last = w.last_rows;
  auto span = [&](const void* base, int64_t sb, int64_t st, int64_t sw, int64_t width, int64_t e, int64_t inner) {
    Span sp;
    sp.p = (const char*)base + (b * sb + t_begin * st + inner) * e;
    sp.step = (int32_t)(TT * st * e);
    sp.last_range = (uint32_t)(((rows_last - 1) * st + (width - 1) * sw + 1) * e);
    return sp;
  };
  w.x = span(p.x, p.xs_b, p.xs_t, 1, p.D - d0, esz, d0);
  w.dl = span(p.delta, p.ds_b, p.ds_t, 1, p.D - d0, esz, d0);
  w.z = want_z ? span(p.z, p.zs_b, p.zs_t, 1, p.D - d0, esz, d0) : w.x;
  w.B = span(p.B, p.Bs_b, p.Bs_t, p.Bs_n, p.N, esz, 0);
  w.C = span(p.C, p.Cs_b, p.Cs_t, p.Cs_n, p.N, esz, 0);
  const int64_t yesz = (p.y_f32 || !BF16) ? 4 : 2;
  w.y = MODE == 0 ? span(p.y, p.ys_b, p.ys_t, 1, p.D - d0, yesz, d0) : w.x;

  // Row-wise role: thread (t, c) = (tid/16, tid%16) loads x, delta, z of
  // step t, channel c and stores y the same way; for B and C it loads state
  // c + 16k of step t (states >= N read state 0 and are zeroed when staged).
  w.st_t = tid / G;
  w.st_ch_ok = d0 + sg < p.D;
  w.o.x = (uint32_t)((w.st_t * p.xs_t + sg) * esz);
  w.o.dl = (uint32_t)((w.st_t * p.ds_t + sg) * esz);
  w.o.z = want_z ? (uint32_t)((w.st_t * p.zs_t + sg) * esz) : 0u;
  w.o.y = MODE == 0 ? (uint32_t)((w.st_t * p.ys_t + sg) * yesz) : 0u;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int n = sg + G * k;
    w.o.bc_ok[k] = n < p.N;
    const int64_t nn = n < p.N ? n : 0;
    w.o.B[k] = (uint32_t)((w.st_t * p.Bs_t + nn * p.Bs_n) * esz);
    w.o.C[k] = (uint32_t)((w.st_t * p.Cs_t + nn * p.Cs_n) * esz);
  }

  int form;
  if (p.flags & kEuler) form = kFormEuler;
  else if (any_zero_A) form = kFormHZero;
  else form = (KS == 1) ? kFormG : kFormH;

  float fA[G];
#pragma unroll
  for (int n = 0; n < G; ++n) fA[n] = 1.f;
  float sum_dt = 0.f;
  if (KS == 1 && form == kFormG) {
    // g form: the finalize weighs the partial of state n by 1/A of the lane's channel.
    if (MODE == 0) {
#pragma unroll
      for (int n = 0; n < G; ++n) {
        float a = -1.f;
        if (d_ok && n < p.N) a = p.A[d * p.As_d + n * p.As_n];
        fA[n] = 1.f / a;
      }
    }
#pragma unroll
    for (int k = 0; k < KS; ++k) h[k] *= Av[k];  // g = A h
    walk<BF16, KS, MODE, kFormG>(s, w, h, ln, fA, Dk, want_z, sum_dt);
#pragma unroll
    for (int k = 0; k < KS; ++k) h[k] *= ln.iA[k];  // h = g / A
  } else if (form == kFormEuler) {
    walk<BF16, KS, MODE, kFormEuler>(s, w, h, ln, fA, Dk, want_z, sum_dt);
  } else if (form == kFormHZero) {
    walk<BF16, KS, MODE, kFormHZero>(s, w, h, ln, fA, Dk, want_z, sum_dt);
  } else {
    walk<BF16, KS, MODE, kFormH>(s, w, h, ln, fA, Dk, want_z, sum_dt);
  }

  if (MODE == 1) {
    // the row's 16 lanes each summed the steps they hold
#pragma unroll
    for (int m = 1; m < G; m <<= 1) sum_dt += __shfl_xor(sum_dt, m, G);
  }
  if (!d_ok) return;
  if (MODE == 0) {
    if (seg == p.n_seg - 1 && (p.flags & kWantHLast)) {
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

template <bool BF16, int KS>
hipError_t launch_ks(const ScanParams& p, hipStream_t stream) {
  const int64_t n_dblk = (p.D + CH - 1) / CH;
  auto padded = [](int64_t n) { return (n + 7) / 8 * 8; };
  if (p.n_seg > 1) {
    const int64_t nb = n_dblk * (p.n_seg - 1) * p.batch;
    hipLaunchKernelGGL((scan_kernel<BF16, KS, 1>), dim3((unsigned)padded(nb)), dim3(NT), 0, stream, p, n_dblk,
                       (int64_t)(p.n_seg - 1), padded(nb));
    const int64_t ncomb = p.batch * p.D * p.N;
    hipLaunchKernelGGL(scan_combine_kernel, dim3((unsigned)((ncomb + 255) / 256)), dim3(256), 0, stream, p);
  }
  const int64_t nb = n_dblk * p.n_seg * p.batch;
  hipLaunchKernelGGL((scan_kernel<BF16, KS, 0>), dim3((unsigned)padded(nb)), dim3(NT), 0, stream, p, n_dblk,
                     (int64_t)p.n_seg, padded(nb));
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_io(const ScanParams& p, hipStream_t stream) {
  if (p.N <= G * 1) return launch_ks<BF16, 1>(p, stream);
  if (p.N <= G * 2) return launch_ks<BF16, 2>(p, stream);
  return launch_ks<BF16, 4>(p, stream);
}

}  // namespace

hipError_t launch_selective_scan(const ScanParams& p, hipStream_t stream) {
  return p.io_bf16 ? launch_io<true>(p, stream) : launch_io<false>(p, stream);
}

}  // namespace ssm
