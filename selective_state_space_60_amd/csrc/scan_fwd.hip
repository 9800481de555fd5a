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
//  * Global memory is read and written in whole tiles: when the layout allows
//    (rows aligned to 4 elements), each wave loads one or two of the tile's
//    16 x 16 pieces -- x, delta, z, and 16 states of B or C -- with one 8- or
//    16-byte load per lane, two tiles ahead of use, and one wave stores y the
//    same way; an LDS transpose hands the values to and from the lanes that
//    hold them.  Other layouts load element by element, one tile ahead.
//    Loads are buffer loads: each lane's byte offset inside a tile is fixed
//    and the buffer base advances in SGPRs; in the last tile of a stretch the
//    descriptor's range ends at the last element that belongs to it, so reads
//    past the end return zero without touching memory.
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
//    workgroup barrier; the results go through LDS to the stores of the next
//    tile.
//  * When batch x channels cannot fill the GPU (long, narrow problems), the
//    sequence is cut into segments: (1) every segment is scanned from h = 0
//    (the first from h0) and writes y, and each but the last also its end
//    state and its sum of delta; (2) a small kernel chains those into the
//    state entering each segment (the associative combine of (Abar, Bbar x)
//    pairs -- tildalice.io, 병렬 스캔 -- at segment granularity); (3) each
//    later segment is scanned again from its entering state, next to a twin
//    of the first pass's states from zero.  The two differ by the entering
//    state times the running product of Abar, which decays; once every state
//    equals its twin bit for bit (checked at the end of each tile), the rest
//    of the first pass's output is exactly what the rescan would write, and
//    the rescan stops.  A decaying model rescans a short prefix of each
//    segment; with no decay the rescan runs to the segment's end.
#include <hip/hip_runtime.h>

#include <mutex>

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

static_assert(G == 16 && TT == G && CH == 16 && CH * G == NT && UB == 4, "tiling");

enum : uint32_t { kHasZ = 1u, kHasD = 2u, kEuler = 4u, kHasH0 = 8u, kWantHLast = 16u };

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
// element, the bytes from one tile to the next, and the descriptor range for
// the tiles before the last (all of memory, or 0 for an unused stream) and
// for the last tile (up to and including its last element).  Accesses go
// through a raw buffer descriptor at that address; reads at or beyond the
// range return zero and touch no memory.
struct Span {
  const char* p;
  int32_t step;
  uint32_t full_range;
  uint32_t last_range;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const Span& s, uint32_t range) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)s.p, (short)0, (int)range, (int)kRsrcWord3);
}

__device__ __forceinline__ void advance(Span& s) { s.p += s.step; }

// Geometry of a workgroup's stretch, in tiles.
struct Tiles {
  int ntiles;     // tiles that hold rows of the stretch
  int last_rows;  // rows of the last of them that belong to it (1..TT)
  // Descriptor range for tile `it` (tiles past the stretch read nothing).
  __device__ __forceinline__ uint32_t range(const Span& s, int it) const {
    return it < ntiles - 1 ? s.full_range : (it == ntiles - 1 ? s.last_range : 0u);
  }
  __device__ __forceinline__ bool row_ok(int it, int r) const {
    return it < ntiles - 1 || (it == ntiles - 1 && r < last_rows);
  }
};

// A span over rows of a tensor starting at element offset `off`: `st` is the
// row stride, the last tile's range ends at element (rows_last - 1, width - 1)
// of the span (elements of a row `sw` apart).
__device__ __forceinline__ Span make_span(const void* base, int64_t off, int64_t st, int64_t sw, int64_t width,
                                          int64_t e, int rows_last, bool live) {
  Span sp;
  sp.p = (const char*)base + off * e;
  sp.step = (int32_t)(TT * st * e);
  sp.full_range = live ? 0xFFFFFFFFu : 0u;
  sp.last_range = live && width > 0 ? (uint32_t)(((int64_t)(rows_last - 1) * st + (width - 1) * sw + 1) * e) : 0u;
  return sp;
}

// Two floats to a bf16 pair (a in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 (converting each float alone and merging the halves
// takes four instructions).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
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
  float2 hx[2][CH][HP];  // (delta, x) per channel and step, double-buffered
  float hz[2][CH][HP];   // z
  float yb[2][CH][HP];   // finalized y, stored one tile later
};

// ---------------------------------------------------------------- loaders
//
// A loader moves one tile of x, delta, z, B, C from global memory into LDS
// (load: into registers, `kDepth` tiles ahead; stage: registers -> LDS) and
// y from LDS to global memory.  Rows past the stretch are staged as zeros:
// delta = x = 0 leaves every state unchanged, so a partial last tile (and
// the padding tile that evens out the two-ahead loop) is scanned like a full
// one.

// Element-wise loader for any layout: thread (t, c) = (tid/16, tid%16) loads
// x, delta, z of step t, channel c and states c + 16k of B and C, and stores
// y of step t, channel c.
template <bool BF16, int KS>
struct ElemLoader {
  static constexpr int kDepth = 1;
  struct Set {
    uint32_t x, dl, z;
    uint32_t B[KS], C[KS];
  };
  Span x, dl, z, B, C, y;
  uint32_t ox, odl, oz, oy, oB[KS], oC[KS];
  bool bc_ok[KS];  // state c + 16k exists
  bool ch_ok;      // channel c exists
  bool y_f32;
  int t;

  __device__ __forceinline__ uint32_t ld(const Span& s, uint32_t range, uint32_t voff) const {
    if constexpr (BF16) return __builtin_amdgcn_raw_buffer_load_b16(rsrc(s, range), (int)voff, 0, 0);
    else return __builtin_amdgcn_raw_buffer_load_b32(rsrc(s, range), (int)voff, 0, 0);
  }

  __device__ __forceinline__ void load(const Tiles& tl, int it, Set& r) {
    r.x = ld(x, tl.range(x, it), ox);
    r.dl = ld(dl, tl.range(dl, it), odl);
    r.z = ld(z, tl.range(z, it), oz);
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      r.B[k] = ld(B, tl.range(B, it), oB[k]);
      r.C[k] = ld(C, tl.range(C, it), oC[k]);
    }
    advance(x);
    advance(dl);
    advance(z);
    advance(B);
    advance(C);
  }

  __device__ __forceinline__ void stage(ScanSmem<KS>& s, const Tiles& tl, int buf, int it, const Set& r) const {
    const int c = threadIdx.x % G;
    const bool ok = tl.row_ok(it, t);
    const float dt = raw2f<BF16>(r.dl), xv = raw2f<BF16>(r.x);
    s.hx[buf][c][t] = make_float2(ok ? dt : 0.f, ok ? xv : 0.f);
    s.hz[buf][c][t] = raw2f<BF16>(r.z);
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const bool okk = ok && bc_ok[k];
      s.bc[buf][c + G * k][t] = make_float2(okk ? raw2f<BF16>(r.B[k]) : 0.f, okk ? raw2f<BF16>(r.C[k]) : 0.f);
    }
  }

  __device__ __forceinline__ void store_y(const ScanSmem<KS>& s, const Tiles& tl, int buf, int it) {
    const int c = threadIdx.x % G;
    const float v = s.yb[buf][c][t];
    if (tl.row_ok(it, t) && ch_ok) {
      if (y_f32 || !BF16)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rsrc(y, 0xFFFFFFFFu), (int)oy, 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)v), rsrc(y, 0xFFFFFFFFu),
                                              (int)oy, 0, 0);
    }
    advance(y);
  }
};

// Tile-piece loader for layouts whose rows are aligned to 4 elements (x,
// delta, z, y with D % 4 == 0; B, C contiguous over states with N % 4 == 0).
// The tile is cut into 16 x 16 pieces -- x, delta, z, then B and C in groups
// of 16 states -- dealt round-robin to the 4 waves; lane (r, q) = (lane/4,
// lane%4) of a wave loads row r, elements 4q..4q+3 of each of its pieces.
// Wave 3 also stores y.
template <bool BF16, int KS>
struct VecLoader {
  static constexpr int kDepth = 2;
  static constexpr int kPieces = 3 + 2 * KS;
  static constexpr int kSlots = (kPieces + 3) / 4;
  static constexpr int kYWave = 3;
  using Word = typename std::conditional<BF16, u32x2, u32x4>::type;  // 4 elements
  struct Set {
    Word v[kSlots];
  };
  Span sp[kSlots];
  bool used[kSlots];     // the slot holds a piece
  uint32_t voff[kSlots];  // byte offset of this lane's 4 elements in the piece
  // Where the slot's 4 elements go in LDS: element i of tile buffer `buf` at
  // dst[j] + buf * dbuf[j] + i * dpitch[j] (floats).  A lane whose 4 states
  // lie past N (N % 4 == 0 on this path, so a piece is all in or all out)
  // stores nothing: those rows of B and C are cleared once (clear_rows).
  float* dst[kSlots];
  int dbuf[kSlots], dpitch[kSlots];
  bool st_ok[kSlots];
  Span y;
  uint32_t oy;
  bool y_ok;  // this lane's 4 channels exist
  bool y_f32;
  int r, q;

  __device__ __forceinline__ Word ld(const Span& s, uint32_t range, uint32_t off) const {
    if constexpr (BF16) return __builtin_amdgcn_raw_buffer_load_b64(rsrc(s, range), (int)off, 0, 0);
    else return __builtin_amdgcn_raw_buffer_load_b128(rsrc(s, range), (int)off, 0, 0);
  }

  __device__ __forceinline__ void load(const Tiles& tl, int it, Set& st) {
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      st.v[j] = ld(sp[j], tl.range(sp[j], it), voff[j]);
      advance(sp[j]);
    }
  }

  __device__ __forceinline__ static void unpack(const Word& w, float (&e)[4]) {
    if constexpr (BF16) {
      e[0] = __uint_as_float(w.x << 16);
      e[1] = __uint_as_float(w.x & 0xFFFF0000u);
      e[2] = __uint_as_float(w.y << 16);
      e[3] = __uint_as_float(w.y & 0xFFFF0000u);
    } else {
      e[0] = __uint_as_float(w.x);
      e[1] = __uint_as_float(w.y);
      e[2] = __uint_as_float(w.z);
      e[3] = __uint_as_float(w.w);
    }
  }

  // Rows past the stretch need no mask: their loads lie past the descriptor
  // range of the stretch's last tile (or of a tile past it) and return zeros.
  // (A mask per element costs a lane mask per element and slot, more than
  // the scalar registers hold.)
  __device__ __forceinline__ void stage(ScanSmem<KS>&, const Tiles&, int buf, int, const Set& st) const {
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      if (!used[j] || !st_ok[j]) continue;
      float e[4];
      unpack(st.v[j], e);
      float* d = dst[j] + buf * dbuf[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i * dpitch[j]] = e[i];
    }
  }

  // Zeros into the B and C rows of states n_states .. G*KS-1 of both tile
  // buffers (never staged); ordered before their first read by the barrier
  // that follows the first stage.
  __device__ __forceinline__ static void clear_rows(ScanSmem<KS>& s, int n_states) {
    const int n0 = n_states < G * KS ? n_states : G * KS;
    const int per_buf = (G * KS - n0) * TP;
    for (int i = threadIdx.x; i < 2 * per_buf; i += NT) {
      const int b = i / per_buf, k = i % per_buf;
      s.bc[b][n0 + k / TP][k % TP] = make_float2(0.f, 0.f);
    }
  }

  // Set slot j up for piece `kd` (see VecLoader); `s` gives the LDS layout.
  __device__ __forceinline__ void place(ScanSmem<KS>& s, int j, int kd, int n_states) {
    used[j] = kd < kPieces;
    st_ok[j] = true;
    if (kd == 0 || kd == 1) {
      dst[j] = kd == 0 ? &s.hx[0][4 * q][r].y : &s.hx[0][4 * q][r].x;
      dpitch[j] = 2 * HP;
      dbuf[j] = 2 * CH * HP;
    } else if (kd == 2) {
      dst[j] = &s.hz[0][4 * q][r];
      dpitch[j] = HP;
      dbuf[j] = CH * HP;
    } else {
      const bool isC = kd >= 3 + KS;
      const int n0 = 16 * (kd - 3 - (isC ? KS : 0)) + 4 * q;
      const int nk = n0 < G * KS ? n0 : 0;
      dst[j] = isC ? &s.bc[0][nk][r].y : &s.bc[0][nk][r].x;
      dpitch[j] = 2 * TP;
      dbuf[j] = 2 * G * KS * TP;
      const int left = n_states - n0;
      st_ok[j] = left >= 4;
    }
  }

  __device__ __forceinline__ void store_y(const ScanSmem<KS>& s, const Tiles& tl, int buf, int it) {
    if (__builtin_amdgcn_readfirstlane(threadIdx.x / 64) == kYWave) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = s.yb[buf][4 * q + i][r];
      if (tl.row_ok(it, r) && y_ok) {
        if (y_f32 || !BF16) {
          u32x4 w;
          w.x = __float_as_uint(v[0]);
          w.y = __float_as_uint(v[1]);
          w.z = __float_as_uint(v[2]);
          w.w = __float_as_uint(v[3]);
          __builtin_amdgcn_raw_buffer_store_b128(w, rsrc(y, 0xFFFFFFFFu), (int)oy, 0, 0);
        } else {
          u32x2 w;
          w.x = pack2(v[0], v[1]);
          w.y = pack2(v[2], v[3]);
          __builtin_amdgcn_raw_buffer_store_b64(w, rsrc(y, 0xFFFFFFFFu), (int)oy, 0, 0);
        }
      }
    }
    advance(y);
  }
};

// ------------------------------------------------------------- the scan

// The current tile's per-channel values held by this lane (step lane%16).
struct Hold {
  float dt, x, xs;  // delta, x, and the value broadcast as x (x, or delta*x in the Euler form)
  float z;
};

// Per-lane constants of this lane's KS states.
template <int KS>
struct Lane {
  float A2[KS];  // log2(e) * A
  float iA[KS];  // 1/A (0 where A == 0)
  float ez[KS];  // 1 where A == 0, else 0
};

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^-|v|); log1p(w) is taken
// as log(u) * w / (u - 1) with u = 1 + w (u - 1 is exact), which keeps its
// relative accuracy for small w.
__device__ __forceinline__ float softplus_f32(float v) {
  constexpr float kLn2 = 0.6931471805599453f;
  const float w = __builtin_amdgcn_exp2f(-fabsf(v) * kLog2e);
  const float u = 1.f + w;
  const float lp = u == 1.f ? w : (__builtin_amdgcn_logf(u) * kLn2) * (w * __builtin_amdgcn_rcpf(u - 1.f));
  return fmaxf(v, 0.f) + lp;
}

// Step-size transform of a lane: delta <- softplus(delta + bias) on the
// lane's steps inside the sequence; padding steps keep delta = 0 (no change
// of the state).
struct DeltaXform {
  bool on;
  float bias;
};

// This lane's step (lane%16) of its channel (tid/16) for the tile in `buf`;
// `valid`: that step lies inside the stretch.
template <int KS, int FORM>
__device__ __forceinline__ void take_hold(const ScanSmem<KS>& s, int buf, bool want_z, Hold& hd,
                                          const DeltaXform& dx, bool valid) {
  const int tid = threadIdx.x;
  const float2 v = s.hx[buf][tid / G][tid % G];
  float dt = v.x;
  if (dx.on) dt = valid ? softplus_f32(dt + dx.bias) : 0.f;
  hd.dt = dt;
  hd.x = v.y;
  hd.xs = FORM == kFormEuler ? dt * v.y : v.y;
  hd.z = want_z ? s.hz[buf][tid / G][tid % G] : 0.f;
}

// One state update of the form FORM with the step's factors.
template <int FORM>
__device__ __forceinline__ float update(float h, float Ab, float q, float c) {
  if constexpr (FORM == kFormG) return __builtin_fmaf(Ab, h + q, -q);
  else if constexpr (FORM == kFormEuler) return __builtin_fmaf(Ab, h, q);
  else return __builtin_fmaf(Ab, h, c * q);
}

// One step (step T of the tile) of one lane's KS states; returns the lane's
// partial readout.  delta and x come from lane T of the row.  No implicit
// fusing of multiplies into adds here: that would turn the broadcast
// multiplies into fmas, which cannot take the DPP operand.  With TWIN, a
// second set of states h2 takes the same step (same factors, same
// operations, so the same roundings), and only h is read out.
template <int KS, int FORM, bool TWIN, int T>
__device__ __forceinline__ float step(float (&h)[KS], float (&h2)[KS], const Lane<KS>& ln, const Hold& hd,
                                      const float4 (&bc)[KS], bool hi) {
#pragma clang fp contract(off)
  float yp = 0.f;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const float Bv = hi ? bc[k].z : bc[k].x;
    const float Cv = hi ? bc[k].w : bc[k].y;
    const float Ab = __builtin_amdgcn_exp2f(row_bcast<T>(hd.dt) * ln.A2[k]);
    const float q = row_bcast<T>(hd.xs) * Bv;  // B*x (B*delta*x in the Euler form)
    float c = 0.f;
    if constexpr (FORM == kFormH || FORM == kFormHZero) {
      // (Abar - 1)/A as Abar*(1/A) - 1/A with one rounding; with A == 0 the
      // factor is 0 and ez*delta supplies the limit delta.
      c = __builtin_fmaf(Ab, ln.iA[k], -ln.iA[k]);
      if constexpr (FORM == kFormHZero) c = __builtin_fmaf(ln.ez[k], row_bcast<T>(hd.dt), c);
    }
    h[k] = update<FORM>(h[k], Ab, q, c);
    if constexpr (TWIN) h2[k] = update<FORM>(h2[k], Ab, q, c);
    yp = k == 0 ? Cv * h[k] : __builtin_fmaf(Cv, h[k], yp);
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
template <int KS, int FORM, bool TWIN, int BLK>
__device__ __forceinline__ void scan_blocks(const ScanSmem<KS>& s, float* prow, int buf, int sg, float (&h)[KS],
                                            float (&h2)[KS], const Lane<KS>& ln, const Hold& hd,
                                            float4 (&o)[2][2][KS]) {
  if constexpr (BLK < TT / UB) {
    if constexpr (BLK + 1 < TT / UB) read_block<KS>(s, buf, (BLK + 1) * UB, sg, o[(BLK + 1) & 1]);
    const float4(&c)[2][KS] = o[BLK & 1];
    float yp[UB];
    yp[0] = step<KS, FORM, TWIN, UB * BLK + 0>(h, h2, ln, hd, c[0], false);
    yp[1] = step<KS, FORM, TWIN, UB * BLK + 1>(h, h2, ln, hd, c[0], true);
    yp[2] = step<KS, FORM, TWIN, UB * BLK + 2>(h, h2, ln, hd, c[1], false);
    yp[3] = step<KS, FORM, TWIN, UB * BLK + 3>(h, h2, ln, hd, c[1], true);
    *(float4*)&prow[UB * BLK] = make_float4(yp[0], yp[1], yp[2], yp[3]);
    scan_blocks<KS, FORM, TWIN, BLK + 1>(s, prow, buf, sg, h, h2, ln, hd, o);
  }
}

// Finalize a tile: lane j of the row takes step j: y = (sum_n w_n partial_n +
// D x) * silu(z), w_n = 1/A_n in the g form, else 1, into yb[buf].  pcol: the
// lane's (channel, step) column in state row 0 of the partials.
template <int KS, int FORM>
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
  if (want_z) v *= hd.z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-hd.z * kLog2e));
  s.yb[buf][threadIdx.x / G][threadIdx.x % G] = v;
}

// Where a walk stores the state before each of its tiles (the backward's
// checkpoints): `p` points at the lane's first state of the stretch's first
// tile, `step` is one tile's stride, `nk` the lane's states below N.
struct CkptOut {
  float* p;  // null: no checkpoints
  int64_t step;
  int nk;
};

// The walk over the stretch, for one update form; writes y and the
// checkpoints.  MODE 0 also sums this lane's share of delta (the steps it
// holds).  MODE 2 carries a twin of the states, h2, started where the first
// pass over the stretch started (zero), and ends the walk after the first
// tile at whose end every state of the workgroup equals its twin bit for bit:
// from there on, the first pass's states, y and checkpoints are exactly the
// ones this walk would produce.  Returns whether the walk ended that way.
template <class L, int KS, int MODE, int FORM>
__device__ __forceinline__ bool walk(ScanSmem<KS>& s, L& ld, const Tiles& tl, float (&h)[KS], float (&h2)[KS],
                                     const Lane<KS>& ln, const float (&fA)[G], float Dk, bool want_z, float& sum_dt,
                                     const DeltaXform& dx, const CkptOut& ck) {
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, sg = tid % G;
  float* prow = &s.part[wave][sg][G * (lane / G)];
  const float* pcol = &s.part[wave][0][lane];
  typename L::Set ra, rb;
  Hold hd;
  // Tiles walked: with two tiles in flight the loop is unrolled by two, so
  // the count is evened out with an all-padding tile.
  const int nrun = L::kDepth == 2 ? (tl.ntiles + 1) & ~1 : tl.ntiles;
  ld.load(tl, 0, ra);
  ld.stage(s, tl, 0, 0, ra);
  if constexpr (L::kDepth == 2) {
    ld.load(tl, 1, rb);
    ld.load(tl, 2, ra);
  } else {
    ld.load(tl, 1, ra);
  }
  __syncthreads();
  // One tile: take this lane's step, scan, finalize into yb, store the
  // previous tile's y, stage tile it+1 (held in rn) and refill rn.  Loads
  // are issued whatever `it` (past the stretch they read nothing): a branch
  // around them would make the compiler wait for them at once.  Returns
  // (MODE 2) whether the states and their twins now agree.
  auto body = [&](int it, typename L::Set& rn) -> bool {
    const int buf = it & 1;
    const int rows = it < tl.ntiles - 1 ? TT : (it == tl.ntiles - 1 ? tl.last_rows : 0);
    if (ck.p && it < tl.ntiles) {
#pragma unroll
      for (int k = 0; k < KS; ++k)  // the g form carries A h
        if (k < ck.nk) ck.p[it * ck.step + k] = FORM == kFormG ? h[k] * ln.iA[k] : h[k];
    }
    take_hold<KS, FORM>(s, buf, want_z, hd, dx, sg < rows);
    float4 o[2][2][KS];
    read_block<KS>(s, buf, 0, sg, o[0]);
    scan_blocks<KS, FORM, MODE == 2, 0>(s, prow, buf, sg, h, h2, ln, hd, o);
    finalize_tile<KS, FORM>(s, buf, pcol, fA, Dk, hd, want_z);
    if (it > 0) ld.store_y(s, tl, buf ^ 1, it - 1);
    if (MODE == 0) sum_dt += hd.dt;
    if (it + 1 < nrun) ld.stage(s, tl, buf ^ 1, it + 1, rn);
    ld.load(tl, it + 1 + L::kDepth, rn);
    if constexpr (MODE == 2) {
      bool same = true;
#pragma unroll
      for (int k = 0; k < KS; ++k) same = same && (__float_as_uint(h[k]) == __float_as_uint(h2[k]));
      return __syncthreads_and(same) != 0;
    } else {
      __syncthreads();
      return false;
    }
  };
  int last = nrun - 1;
  bool met = false;
  if constexpr (L::kDepth == 2) {
    for (int it = 0; it < nrun; it += 2) {
      if (body(it, rb)) { last = it; met = true; break; }
      if (body(it + 1, ra)) { last = it + 1; met = true; break; }
    }
  } else {
    for (int it = 0; it < nrun; ++it)
      if (body(it, ra)) { last = it; met = true; break; }
  }
  ld.store_y(s, tl, last & 1, last);
  return met;
}

// MODE 0: scan the stretch and write y (and h_last, the checkpoints).  With
// the sequence split, every segment starts from zero (segment 0 from h0) and
// each segment but the last writes its aggregate (end state, sum of delta).
// MODE 2 (split only; segments 1..n_seg-1): rescan a segment from the state
// entering it, next to a twin started from zero, until the two agree.
// (The fp32 single-state first pass is held to five waves per SIMD, the
// occupancy the planner's segment count assumes.)
template <bool BF16, bool VEC, int KS, int MODE>
__global__ __launch_bounds__(NT, (!BF16 && KS == 1 && MODE == 0) ? 5 : 1) void scan_kernel(
    ScanParams p, int64_t n_dblk, int64_t nseg_run, int64_t nblocks_padded) {
  __shared__ ScanSmem<KS> s;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;  // wave: uniform (SGPR)
  const int chb = tid / G, sg = tid % G;

  const int64_t lb = logical_block(nblocks_padded);
  if (lb >= n_dblk * nseg_run * p.batch) return;
  const int64_t dblk = lb % n_dblk;
  const int64_t seg = (MODE == 2 ? 1 : 0) + (lb / n_dblk) % nseg_run;
  const int64_t b = lb / (n_dblk * nseg_run);
  const int64_t d0 = dblk * CH;
  const int64_t d = d0 + chb;  // this lane's channel (scan and finalize)
  const bool d_ok = d < p.D;
  const bool want_z = (p.flags & kHasZ) != 0;
  const int64_t esz = BF16 ? 2 : 4;
  const int64_t yesz = (p.y_f32 || !BF16) ? 4 : 2;

  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = (t_begin + p.seg_len < p.L) ? t_begin + p.seg_len : p.L;
  Tiles tl;
  tl.ntiles = (int)((t_end - t_begin + TT - 1) / TT);
  tl.last_rows = (int)(t_end - t_begin - (int64_t)(tl.ntiles - 1) * TT);

  // Per-lane constants of this lane's KS states.
  Lane<KS> ln;
  float Av[KS], h[KS], h2[KS];
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
    h2[k] = 0.f;
  }
  {
    const float* src = nullptr;
    if (MODE == 2) src = p.h_in + ((b * p.n_seg + seg) * p.D) * p.N;
    else if (seg == 0 && (p.flags & kHasH0)) src = p.h0 + (b * p.D) * p.N;
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
  if ((p.flags & kHasD) && d_ok) Dk = p.Dskip[d * p.Ds_d];

  // Streams: each starts at row t_begin of batch row b and advances one tile
  // of rows at a time.  The last tile's range ends at its last row's last
  // element (channel D-1 or state N-1 of the span): lanes of rows past the
  // stretch, or of channels / states past the end of the tensor's last row,
  // read zeros.  (With rows that overlap in memory, rows past the stretch
  // can lie inside that range: the element loader, which such layouts take,
  // stages them as zeros.)
  const int rows_last = tl.last_rows;
  typename std::conditional<VEC, VecLoader<BF16, KS>, ElemLoader<BF16, KS>>::type ld;
  if constexpr (VEC) {
    ld.r = lane / 4;
    ld.q = lane % 4;
    ld.y_f32 = p.y_f32 != 0;
#pragma unroll
    for (int j = 0; j < ld.kSlots; ++j) {
      const int kd = wave + 4 * j;
      ld.place(s, j, kd, (int)p.N);
      const void* base = p.x;
      int64_t sb = 0, st = 0, col0 = 0, width = 0;
      bool live = kd < ld.kPieces;
      if (kd == 0) { base = p.x; sb = p.xs_b; st = p.xs_t; col0 = d0; width = p.D - d0; }
      else if (kd == 1) { base = p.delta; sb = p.ds_b; st = p.ds_t; col0 = d0; width = p.D - d0; }
      else if (kd == 2) { base = want_z ? p.z : p.x; sb = p.zs_b; st = p.zs_t; col0 = d0; width = p.D - d0; live = want_z; }
      else if (kd < 3 + KS) { base = p.B; sb = p.Bs_b; st = p.Bs_t; col0 = 16 * (kd - 3); width = p.N - col0; }
      else if (kd < ld.kPieces) { base = p.C; sb = p.Cs_b; st = p.Cs_t; col0 = 16 * (kd - 3 - KS); width = p.N - col0; }
      width = width < 16 ? width : 16;
      live = live && width > 0;
      ld.sp[j] = make_span(base, b * sb + t_begin * st + col0, st, 1, width, esz, rows_last, live);
      ld.voff[j] = (uint32_t)((ld.r * st + 4 * ld.q) * esz);
    }
    ld.y = make_span(p.y, b * p.ys_b + t_begin * p.ys_t + d0, p.ys_t, 1, p.D - d0, yesz, rows_last, true);
    ld.oy = (uint32_t)((ld.r * p.ys_t + 4 * ld.q) * yesz);
    ld.y_ok = d0 + 4 * ld.q < p.D;
    ld.clear_rows(s, (int)p.N);
  } else {
    ld.t = tid / G;
    ld.ch_ok = d0 + sg < p.D;
    ld.y_f32 = p.y_f32 != 0;
    ld.x = make_span(p.x, b * p.xs_b + t_begin * p.xs_t + d0, p.xs_t, 1, p.D - d0, esz, rows_last, true);
    ld.dl = make_span(p.delta, b * p.ds_b + t_begin * p.ds_t + d0, p.ds_t, 1, p.D - d0, esz, rows_last, true);
    ld.z = make_span(want_z ? p.z : p.x, b * p.zs_b + t_begin * p.zs_t + d0, p.zs_t, 1, p.D - d0, esz, rows_last,
                     want_z);
    ld.B = make_span(p.B, b * p.Bs_b + t_begin * p.Bs_t, p.Bs_t, p.Bs_n, p.N, esz, rows_last, true);
    ld.C = make_span(p.C, b * p.Cs_b + t_begin * p.Cs_t, p.Cs_t, p.Cs_n, p.N, esz, rows_last, true);
    ld.y = make_span(p.y, b * p.ys_b + t_begin * p.ys_t + d0, p.ys_t, 1, p.D - d0, yesz, rows_last, true);
    ld.ox = (uint32_t)((ld.t * p.xs_t + sg) * esz);
    ld.odl = (uint32_t)((ld.t * p.ds_t + sg) * esz);
    ld.oz = (uint32_t)((ld.t * p.zs_t + sg) * esz);
    ld.oy = (uint32_t)((ld.t * p.ys_t + sg) * yesz);
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int n = sg + G * k;
      ld.bc_ok[k] = n < p.N;
      const int64_t nn = n < p.N ? n : 0;
      ld.oB[k] = (uint32_t)((ld.t * p.Bs_t + nn * p.Bs_n) * esz);
      ld.oC[k] = (uint32_t)((ld.t * p.Cs_t + nn * p.Cs_n) * esz);
    }
  }

  int form;
  if (p.flags & kEuler) form = kFormEuler;
  else if (any_zero_A) form = kFormHZero;
  else form = (KS == 1) ? kFormG : kFormH;

  float fA[G];
#pragma unroll
  for (int n = 0; n < G; ++n) fA[n] = 1.f;
  float sum_dt = 0.f;
  CkptOut ck;
  ck.p = nullptr;
  ck.step = p.D * p.N;
  ck.nk = 0;
  if (p.ckpt && d_ok) {
    const int64_t n0 = sg * KS;
    ck.nk = n0 >= p.N ? 0 : (p.N - n0 < KS ? (int)(p.N - n0) : KS);
    ck.p = p.ckpt + ((b * ((p.L + TT - 1) / TT) + t_begin / TT) * p.D + d) * p.N + (n0 < p.N ? n0 : 0);
  }
  DeltaXform dx;
  dx.on = p.dsoftplus != 0;
  dx.bias = (dx.on && p.dbias && d_ok) ? p.dbias[d * p.dbs_d] : 0.f;
  bool met = false;
  if (KS == 1 && form == kFormG) {
    // g form: the finalize weighs the partial of state n by 1/A of the lane's channel.
#pragma unroll
    for (int n = 0; n < G; ++n) {
      float a = -1.f;
      if (d_ok && n < p.N) a = p.A[d * p.As_d + n * p.As_n];
      fA[n] = 1.f / a;
    }
#pragma unroll
    for (int k = 0; k < KS; ++k) h[k] *= Av[k];  // g = A h (the twin starts at 0)
    met = walk<decltype(ld), KS, MODE, kFormG>(s, ld, tl, h, h2, ln, fA, Dk, want_z, sum_dt, dx, ck);
#pragma unroll
    for (int k = 0; k < KS; ++k) h[k] *= ln.iA[k];  // h = g / A
  } else if (form == kFormEuler) {
    met = walk<decltype(ld), KS, MODE, kFormEuler>(s, ld, tl, h, h2, ln, fA, Dk, want_z, sum_dt, dx, ck);
  } else if (form == kFormHZero) {
    met = walk<decltype(ld), KS, MODE, kFormHZero>(s, ld, tl, h, h2, ln, fA, Dk, want_z, sum_dt, dx, ck);
  } else {
    met = walk<decltype(ld), KS, MODE, kFormH>(s, ld, tl, h, h2, ln, fA, Dk, want_z, sum_dt, dx, ck);
  }

  const bool split = p.n_seg > 1;
  if (MODE == 0 && split) {
    // the row's 16 lanes each summed the steps they hold
#pragma unroll
    for (int m = 1; m < G; m <<= 1) sum_dt += __shfl_xor(sum_dt, m, G);
  }
  if (!d_ok) return;
  // h_last: the last segment's end state.  A MODE 2 walk that met its twin
  // leaves the first pass's (equal) one in place.
  if (seg == p.n_seg - 1 && (p.flags & kWantHLast) && !met) {
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int n = sg * KS + k;
      if (n < p.N) p.h_last[(b * p.D + d) * p.N + n] = h[k];
    }
  }
  if (MODE == 0 && split && seg < p.n_seg - 1) {
    float* H = p.agg_H + ((b * (p.n_seg - 1) + seg) * p.D + d) * p.N;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int n = sg * KS + k;
      if (n < p.N) H[n] = h[k];
    }
    if (sg == 0) p.agg_S[(b * (p.n_seg - 1) + seg) * p.D + d] = sum_dt;
  }
}

// States entering segments 1..n_seg-1 from the first pass's aggregates
// (segment 0's includes h0):  h_in[1] = H_0;  h_in[s+1] = exp(A*S_s) h_in[s] + H_s.
__global__ __launch_bounds__(256) void scan_combine_kernel(ScanParams p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // over batch*D*N
  if (i >= p.batch * p.D * p.N) return;
  const int64_t n = i % p.N, d = (i / p.N) % p.D, b = i / (p.N * p.D);
  const float a2 = p.A[d * p.As_d + n * p.As_n] * kLog2e;
  float h = p.agg_H[((b * (p.n_seg - 1) + 0) * p.D + d) * p.N + n];
  for (int s = 1; s < p.n_seg; ++s) {
    p.h_in[((b * p.n_seg + s) * p.D + d) * p.N + n] = h;
    if (s + 1 < p.n_seg) {
      const float S = p.agg_S[(b * (p.n_seg - 1) + s) * p.D + d];
      const float H = p.agg_H[((b * (p.n_seg - 1) + s) * p.D + d) * p.N + n];
      h = __builtin_fmaf(__builtin_amdgcn_exp2f(a2 * S), h, H);
    }
  }
}

template <bool BF16, bool VEC, int KS>
hipError_t launch_ks(const ScanParams& p, hipStream_t stream) {
  const int64_t n_dblk = (p.D + CH - 1) / CH;
  auto padded = [](int64_t n) { return (n + 7) / 8 * 8; };
  // pass 1: every segment from zero (segment 0 from h0)
  const int64_t nb = n_dblk * p.n_seg * p.batch;
  hipLaunchKernelGGL((scan_kernel<BF16, VEC, KS, 0>), dim3((unsigned)padded(nb)), dim3(NT), 0, stream, p, n_dblk,
                     (int64_t)p.n_seg, padded(nb));
  if (p.n_seg > 1) {
    // the states entering the segments, then each segment's correction
    const int64_t ncomb = p.batch * p.D * p.N;
    hipLaunchKernelGGL(scan_combine_kernel, dim3((unsigned)((ncomb + 255) / 256)), dim3(256), 0, stream, p);
    const int64_t nb2 = n_dblk * (p.n_seg - 1) * p.batch;
    hipLaunchKernelGGL((scan_kernel<BF16, VEC, KS, 2>), dim3((unsigned)padded(nb2)), dim3(NT), 0, stream, p,
                       n_dblk, (int64_t)(p.n_seg - 1), padded(nb2));
  }
  return hipGetLastError();
}

template <bool BF16, bool VEC>
hipError_t launch_io(const ScanParams& p, hipStream_t stream) {
  if (p.N <= G * 1) return launch_ks<BF16, VEC, 1>(p, stream);
  if (p.N <= G * 2) return launch_ks<BF16, VEC, 2>(p, stream);
  return launch_ks<BF16, VEC, 4>(p, stream);
}

}  // namespace

// Workspace of the allocation-free entry point: one copy per GPU, alive until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// the device array: kernels are given the address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[kScanStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null: not looked up yet)
}  // namespace

hipError_t scan_static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_selective_scan(const ScanParams& p, hipStream_t stream) {
  // Tile pieces load 4 consecutive elements per lane: every row of x, delta,
  // z, y must start 4-element aligned, and B, C must be contiguous over states.
  const int64_t e = p.io_bf16 ? 2 : 4;
  const int64_t ye = (p.y_f32 || !p.io_bf16) ? 4 : 2;
  auto al = [](const void* q, int64_t bytes) { return q == nullptr || ((uintptr_t)q % (uintptr_t)bytes) == 0; };
  bool vec = p.D % 4 == 0 && p.N % 4 == 0 && al(p.x, 4 * e) && al(p.delta, 4 * e) && al(p.y, 4 * ye) &&
             al(p.B, 4 * e) && al(p.C, 4 * e) && p.xs_b % 4 == 0 && p.xs_t % 4 == 0 && p.ds_b % 4 == 0 &&
             p.ds_t % 4 == 0 && p.ys_b % 4 == 0 && p.ys_t % 4 == 0 && p.Bs_n == 1 && p.Cs_n == 1 &&
             p.Bs_b % 4 == 0 && p.Bs_t % 4 == 0 && p.Cs_b % 4 == 0 && p.Cs_t % 4 == 0 &&
             // rows apart by at least their width: the last tile's descriptor
             // range then ends before any row past the stretch
             p.xs_t >= p.D && p.ds_t >= p.D && p.Bs_t >= p.N && p.Cs_t >= p.N &&
             // (y strides 0: one scratch row takes every store, y not wanted)
             (p.ys_t >= p.D || (p.ys_t == 0 && p.ys_b == 0));
  if (p.flags & kHasZ) vec = vec && al(p.z, 4 * e) && p.zs_b % 4 == 0 && p.zs_t % 4 == 0 && p.zs_t >= p.D;
  if (p.io_bf16) return vec ? launch_io<true, true>(p, stream) : launch_io<true, false>(p, stream);
  return vec ? launch_io<false, true>(p, stream) : launch_io<false, false>(p, stream);
}

}  // namespace ssm
