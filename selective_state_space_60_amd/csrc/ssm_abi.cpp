// Host side of libssm: descriptor validation, workspace planning and
// dispatch to the gfx950 kernels.  Every check runs before any HIP call, so a
// rejected call has no side effects (and the checks run without a GPU).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "../../include/ssm.h"
#include "ssm_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr uint32_t kScanFlags = SSM_HAS_Z | SSM_HAS_D | SSM_DISC_EULER | SSM_HAS_H0 | SSM_WANT_HLAST |
                                SSM_DELTA_SOFTPLUS | SSM_HAS_DELTA_BIAS | SSM_WANT_CKPT;
constexpr uint32_t kSSDFlags = SSM_HAS_D | SSM_DISC_EULER | SSM_HAS_H0 | SSM_WANT_HLAST;
constexpr uint32_t kUpdateFlags = SSM_HAS_Z | SSM_HAS_D | SSM_DISC_EULER | SSM_DELTA_SOFTPLUS | SSM_HAS_DELTA_BIAS;
constexpr uint32_t kConvFlags = SSM_HAS_BIAS | SSM_SILU;
constexpr uint32_t kScanBwdFlags = SSM_HAS_Z | SSM_HAS_D | SSM_DISC_EULER | SSM_HAS_H0 | SSM_DELTA_SOFTPLUS |
                                   SSM_HAS_DELTA_BIAS | SSM_HAS_CKPT;

// Shape of the scan checkpoints: the state before every 16-step tile.
void ckpt_shape(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t (&sh)[4]) {
  sh[0] = batch;
  sh[1] = (seqlen + 15) / 16;
  sh[2] = dim;
  sh[3] = dstate;
}
constexpr int kSimds = 256 * 4;  // MI355X: 256 compute units x 4 SIMDs

int64_t esize(int32_t dt) { return dt == SSM_BF16 || dt == SSM_F16 ? 2 : 4; }

struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi)
  bool valid = false;
};

Span span_of(const ssm_tensor_desc& t, const void* ptr) {
  Span s;
  if (!ptr) return s;
  int64_t last = 0;
  for (int i = 0; i < t.ndim; ++i) last += (t.shape[i] - 1) * t.stride[i];
  s.lo = (uintptr_t)ptr;
  s.hi = s.lo + (uintptr_t)((last + 1) * esize(t.dtype));
  s.valid = true;
  return s;
}

// The bytes [ptr, ptr + bytes) of a plain contiguous buffer.
Span span_bytes(const void* ptr, int64_t bytes) {
  Span s;
  if (!ptr) return s;
  s.lo = (uintptr_t)ptr;
  s.hi = s.lo + (uintptr_t)bytes;
  s.valid = true;
  return s;
}

bool overlap(const Span& a, const Span& b) { return a.valid && b.valid && a.lo < b.hi && b.lo < a.hi; }

// Shape, dtype and stride checks of one tensor.
ssm_status check_tensor(const ssm_tensor_desc& t, int ndim, const int64_t* shape, bool dtype_ok, bool inner_unit,
                        bool contiguous) {
  if (!dtype_ok) return SSM_ERR_DTYPE;
  if (t.ndim != ndim) return SSM_ERR_SHAPE;
  for (int i = 0; i < ndim; ++i)
    if (t.shape[i] != shape[i]) return SSM_ERR_SHAPE;
  for (int i = 0; i < ndim; ++i)
    if (t.stride[i] < 0) return SSM_ERR_STRIDE;
  if (inner_unit && t.stride[ndim - 1] != 1 && t.shape[ndim - 1] > 1) return SSM_ERR_STRIDE;
  if (contiguous) {
    int64_t expect = 1;
    for (int i = ndim - 1; i >= 0; --i) {
      if (t.shape[i] > 1 && t.stride[i] != expect) return SSM_ERR_STRIDE;
      expect *= t.shape[i];
    }
  }
  return SSM_OK;
}

// An output must not write one element twice: with dimensions sorted by
// stride, each stride must be at least the extent of the smaller ones.
bool non_overlapping(const ssm_tensor_desc& t) {
  int idx[SSM_MAX_DIMS];
  int n = 0;
  for (int i = 0; i < t.ndim; ++i)
    if (t.shape[i] > 1) idx[n++] = i;
  std::sort(idx, idx + n, [&](int a, int b) { return t.stride[a] < t.stride[b]; });
  int64_t extent = 1;
  for (int k = 0; k < n; ++k) {
    if (t.stride[idx[k]] < extent) return false;
    extent = t.stride[idx[k]] * (t.shape[idx[k]] - 1) + extent;
  }
  return true;
}

bool aligned(const void* p, int64_t bytes) { return ((uintptr_t)p % (uintptr_t)bytes) == 0; }

int64_t round256(int64_t n) { return (n + 255) / 256 * 256; }

// ------------------------------------------------------------------ scan

struct ScanPlan {
  int n_seg = 1;
  int64_t seg_len = 0;
  int64_t ws_H = 0, ws_S = 0, ws_hin = 0, ws_total = 0;
};

// Segments of a sequence split: only when batch x channels cannot give every
// SIMD a wave, into about `target` waves per SIMD, segments at least 2048
// steps long and a whole number of 16-step tiles.
void split_seq(int64_t batch, int64_t seqlen, int64_t dim, int64_t target, int& n_seg_out, int64_t& seg_len_out) {
  const int64_t blocks = batch * ((dim + ssm::kScanChannelsPerBlock - 1) / ssm::kScanChannelsPerBlock);
  const int64_t waves = blocks * (ssm::kScanThreads / 64);
  int64_t n_seg = 1;
  if (waves < kSimds) {
    n_seg = std::max<int64_t>(1, (target * kSimds + waves / 2) / waves);
    n_seg = std::min<int64_t>(n_seg, std::max<int64_t>(1, seqlen / 2048));
  }
  int64_t seg_len = (seqlen + n_seg - 1) / n_seg;
  seg_len = (seg_len + ssm::kScanTileSteps - 1) / ssm::kScanTileSteps * ssm::kScanTileSteps;
  n_seg_out = (int)((seqlen + seg_len - 1) / seg_len);
  seg_len_out = seg_len;
}

// The forward's split targets five waves per SIMD (its first pass runs at
// five).
ScanPlan plan_scan_dims(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  ScanPlan pl;
  split_seq(batch, seqlen, dim, 5, pl.n_seg, pl.seg_len);
  const int64_t n_seg = pl.n_seg;
  if (n_seg > 1) {
    pl.ws_H = round256(batch * (n_seg - 1) * dim * dstate * 4);
    pl.ws_S = round256(batch * (n_seg - 1) * dim * 4);
    pl.ws_hin = round256(batch * n_seg * dim * dstate * 4);
  }
  pl.ws_total = pl.ws_H + pl.ws_S + pl.ws_hin;
  return pl;
}

ScanPlan plan_scan(const ssm_scan_desc& d) { return plan_scan_dims(d.batch, d.seqlen, d.dim, d.dstate); }

ssm_status validate_scan_desc(const ssm_scan_desc* d) {
  if (!d) return SSM_ERR_NULL;
  if (d->batch <= 0 || d->seqlen <= 0 || d->dim <= 0 || d->dstate <= 0) return SSM_ERR_SHAPE;
  if (d->flags & ~kScanFlags) return SSM_ERR_UNSUPPORTED;
  if ((d->flags & SSM_HAS_DELTA_BIAS) && !(d->flags & SSM_DELTA_SOFTPLUS)) return SSM_ERR_UNSUPPORTED;
  if (d->dstate > SSM_SCAN_MAX_DSTATE) return SSM_ERR_UNSUPPORTED;
  const int32_t io = d->x.dtype;
  if (io == SSM_F16) return SSM_ERR_UNSUPPORTED;
  const bool io_ok = io == SSM_F32 || io == SSM_BF16;
  const int64_t bld[3] = {d->batch, d->seqlen, d->dim};
  const int64_t bln[3] = {d->batch, d->seqlen, d->dstate};
  const int64_t dn[2] = {d->dim, d->dstate};
  const int64_t dd[1] = {d->dim};
  const int64_t bdn[3] = {d->batch, d->dim, d->dstate};
  ssm_status s;
  if ((s = check_tensor(d->x, 3, bld, io_ok, true, false))) return s;
  if ((s = check_tensor(d->delta, 3, bld, d->delta.dtype == io, true, false))) return s;
  if ((s = check_tensor(d->B, 3, bln, d->B.dtype == io, false, false))) return s;
  if ((s = check_tensor(d->C, 3, bln, d->C.dtype == io, false, false))) return s;
  if ((s = check_tensor(d->A, 2, dn, d->A.dtype == SSM_F32, false, false))) return s;
  if ((s = check_tensor(d->y, 3, bld, d->y.dtype == io || d->y.dtype == SSM_F32, true, false))) return s;
  if (!non_overlapping(d->y)) return SSM_ERR_STRIDE;
  if (d->flags & SSM_HAS_Z)
    if ((s = check_tensor(d->z, 3, bld, d->z.dtype == io, true, false))) return s;
  if (d->flags & SSM_HAS_D)
    if ((s = check_tensor(d->D, 1, dd, d->D.dtype == SSM_F32, false, false))) return s;
  if (d->flags & SSM_HAS_H0)
    if ((s = check_tensor(d->h0, 3, bdn, d->h0.dtype == SSM_F32, false, true))) return s;
  if (d->flags & SSM_WANT_HLAST)
    if ((s = check_tensor(d->h_last, 3, bdn, d->h_last.dtype == SSM_F32, false, true))) return s;
  if (d->flags & SSM_HAS_DELTA_BIAS)
    if ((s = check_tensor(d->delta_bias, 1, dd, d->delta_bias.dtype == SSM_F32, false, false))) return s;
  if (d->flags & SSM_WANT_CKPT) {
    int64_t ck[4];
    ckpt_shape(d->batch, d->seqlen, d->dim, d->dstate, ck);
    if ((s = check_tensor(d->ckpt, 4, ck, d->ckpt.dtype == SSM_F32, false, true))) return s;
  }
  // The kernel addresses one tile of rows (and, for B and C, all N states of
  // a row) with 32-bit byte offsets from the tile's first element.
  const int64_t e = esize(io), ey = esize(d->y.dtype);
  const int64_t rows = ssm::kScanTileSteps;
  auto fits = [&](const ssm_tensor_desc& t, int64_t width, int64_t es) {
    return (rows * t.stride[1] + width * t.stride[2]) * es < ((int64_t)1 << 31);
  };
  if (!fits(d->x, ssm::kScanChannelsPerBlock, e) || !fits(d->delta, ssm::kScanChannelsPerBlock, e) ||
      !fits(d->y, ssm::kScanChannelsPerBlock, ey) || !fits(d->B, d->dstate, e) || !fits(d->C, d->dstate, e) ||
      ((d->flags & SSM_HAS_Z) && !fits(d->z, ssm::kScanChannelsPerBlock, e)))
    return SSM_ERR_UNSUPPORTED;
  return SSM_OK;
}

ssm_status validate_scan_ptrs(const ssm_scan_desc* d, const ssm_scan_ptrs* p) {
  if (!p) return SSM_ERR_NULL;
  const uint32_t f = d->flags;
  if (!p->x || !p->delta || !p->A || !p->B || !p->C || !p->y) return SSM_ERR_NULL;
  if ((f & SSM_HAS_Z) && !p->z) return SSM_ERR_NULL;
  if ((f & SSM_HAS_D) && !p->D) return SSM_ERR_NULL;
  if ((f & SSM_HAS_H0) && !p->h0) return SSM_ERR_NULL;
  if ((f & SSM_WANT_HLAST) && !p->h_last) return SSM_ERR_NULL;
  if ((f & SSM_HAS_DELTA_BIAS) && !p->delta_bias) return SSM_ERR_NULL;
  if ((f & SSM_HAS_DELTA_BIAS) && !aligned(p->delta_bias, 4)) return SSM_ERR_ALIGN;
  if ((f & SSM_WANT_CKPT) && !p->ckpt) return SSM_ERR_NULL;
  if ((f & SSM_WANT_CKPT) && !aligned(p->ckpt, 4)) return SSM_ERR_ALIGN;
  const int64_t io = esize(d->x.dtype);
  if (!aligned(p->x, io) || !aligned(p->delta, io) || !aligned(p->B, io) || !aligned(p->C, io) ||
      !aligned(p->A, 4) || !aligned(p->y, esize(d->y.dtype)))
    return SSM_ERR_ALIGN;
  if (((f & SSM_HAS_Z) && !aligned(p->z, io)) || ((f & SSM_HAS_D) && !aligned(p->D, 4)) ||
      ((f & SSM_HAS_H0) && !aligned(p->h0, 4)) || ((f & SSM_WANT_HLAST) && !aligned(p->h_last, 4)))
    return SSM_ERR_ALIGN;
  const Span ins[] = {span_of(d->x, p->x),
                      span_of(d->delta, p->delta),
                      span_of(d->A, p->A),
                      span_of(d->B, p->B),
                      span_of(d->C, p->C),
                      (f & SSM_HAS_D) ? span_of(d->D, p->D) : Span(),
                      (f & SSM_HAS_Z) ? span_of(d->z, p->z) : Span(),
                      (f & SSM_HAS_H0) ? span_of(d->h0, p->h0) : Span(),
                      (f & SSM_HAS_DELTA_BIAS) ? span_of(d->delta_bias, p->delta_bias) : Span()};
  const Span ys = span_of(d->y, p->y);
  const Span hl = (f & SSM_WANT_HLAST) ? span_of(d->h_last, p->h_last) : Span();
  const Span ck = (f & SSM_WANT_CKPT) ? span_of(d->ckpt, p->ckpt) : Span();
  for (const Span& s : ins)
    if (overlap(ys, s) || overlap(hl, s) || overlap(ck, s)) return SSM_ERR_ALIAS;
  if (overlap(ys, hl) || overlap(ys, ck) || overlap(hl, ck)) return SSM_ERR_ALIAS;
  return SSM_OK;
}

// ------------------------------------------------------------------- SSD

struct SSDPlan {
  int64_t nchunks = 0, Lp = 0;
  int64_t ws_acum = 0, ws_beta = 0, ws_states = 0, ws_sin = 0, ws_total = 0;
};

SSDPlan plan_ssd(const ssm_ssd_desc& d) {
  SSDPlan pl;
  pl.nchunks = (d.seqlen + d.chunk - 1) / d.chunk;
  pl.Lp = pl.nchunks * d.chunk;
  pl.ws_acum = round256(d.batch * d.nheads * pl.Lp * 4);
  pl.ws_beta = pl.ws_acum;
  pl.ws_states = round256(d.batch * pl.nchunks * d.nheads * d.headdim * d.dstate * 4);
  pl.ws_sin = round256(d.batch * pl.nchunks * d.nheads * d.headdim * d.dstate * 2);
  pl.ws_total = pl.ws_acum + pl.ws_beta + pl.ws_states + pl.ws_sin;
  return pl;
}

ssm_status validate_ssd_desc(const ssm_ssd_desc* d) {
  if (!d) return SSM_ERR_NULL;
  if (d->batch <= 0 || d->seqlen <= 0 || d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0 || d->ngroups <= 0 ||
      d->chunk <= 0)
    return SSM_ERR_SHAPE;
  if (d->nheads % d->ngroups) return SSM_ERR_SHAPE;
  if (d->flags & ~kSSDFlags) return SSM_ERR_UNSUPPORTED;
  if (d->headdim != 64 || (d->dstate != 64 && d->dstate != 128 && d->dstate != 256) ||
      (d->chunk != 64 && d->chunk != 128 && d->chunk != 256) || (d->dstate == 256 && d->chunk == 256))
    return SSM_ERR_UNSUPPORTED;
  if (d->x.dtype == SSM_F32 || d->x.dtype == SSM_F16) return SSM_ERR_UNSUPPORTED;
  const int64_t blhp[4] = {d->batch, d->seqlen, d->nheads, d->headdim};
  const int64_t blh[3] = {d->batch, d->seqlen, d->nheads};
  const int64_t blgn[4] = {d->batch, d->seqlen, d->ngroups, d->dstate};
  const int64_t h1[1] = {d->nheads};
  const int64_t bhpn[4] = {d->batch, d->nheads, d->headdim, d->dstate};
  ssm_status s;
  if ((s = check_tensor(d->x, 4, blhp, d->x.dtype == SSM_BF16, true, false))) return s;
  if ((s = check_tensor(d->delta, 3, blh, d->delta.dtype == SSM_BF16, true, false))) return s;
  if ((s = check_tensor(d->B, 4, blgn, d->B.dtype == SSM_BF16, true, false))) return s;
  if ((s = check_tensor(d->C, 4, blgn, d->C.dtype == SSM_BF16, true, false))) return s;
  if ((s = check_tensor(d->A, 1, h1, d->A.dtype == SSM_F32, false, false))) return s;
  if ((s = check_tensor(d->y, 4, blhp, d->y.dtype == SSM_BF16 || d->y.dtype == SSM_F32, true, false))) return s;
  if (!non_overlapping(d->y)) return SSM_ERR_STRIDE;
  if (d->flags & SSM_HAS_D)
    if ((s = check_tensor(d->D, 1, h1, d->D.dtype == SSM_F32, false, false))) return s;
  if (d->flags & SSM_HAS_H0)
    if ((s = check_tensor(d->h0, 4, bhpn, d->h0.dtype == SSM_F32, false, true))) return s;
  if (d->flags & SSM_WANT_HLAST)
    if ((s = check_tensor(d->h_last, 4, bhpn, d->h_last.dtype == SSM_F32, false, true))) return s;
  return SSM_OK;
}

// Which pointers a step reads or writes.
enum : unsigned { kNeedX = 1, kNeedDelta = 2, kNeedB = 4, kNeedC = 8, kNeedY = 16, kNeedAll = 31 };

// The SSD kernels move whole 16-byte groups of a row (8 bf16 / 4 fp32): each
// (batch, step, head or group) row must start 16-byte aligned.
bool rows_aligned16(const ssm_tensor_desc& t, const void* ptr, int outer_dims) {
  if (!ptr) return true;
  const int64_t e = esize(t.dtype);
  if ((uintptr_t)ptr % 16) return false;
  for (int i = 0; i < outer_dims; ++i)
    if (t.shape[i] > 1 && (t.stride[i] * e) % 16) return false;
  return true;
}

ssm_status validate_ssd_ptrs(const ssm_ssd_desc* d, const ssm_ssd_ptrs* p, unsigned need) {
  if (!p) return SSM_ERR_NULL;
  const uint32_t f = d->flags;
  if (!p->A) return SSM_ERR_NULL;
  if (((need & kNeedX) && !p->x) || ((need & kNeedDelta) && !p->delta) || ((need & kNeedB) && !p->B) ||
      ((need & kNeedC) && !p->C) || ((need & kNeedY) && !p->y))
    return SSM_ERR_NULL;
  if ((need & kNeedY) && (f & SSM_HAS_D) && !p->D) return SSM_ERR_NULL;
  if ((f & SSM_HAS_H0) && !p->h0) return SSM_ERR_NULL;
  if ((f & SSM_WANT_HLAST) && !p->h_last) return SSM_ERR_NULL;
  if ((p->x && !aligned(p->x, 2)) || (p->delta && !aligned(p->delta, 2)) || (p->B && !aligned(p->B, 2)) ||
      (p->C && !aligned(p->C, 2)) || !aligned(p->A, 4) || (p->y && !aligned(p->y, esize(d->y.dtype))) ||
      (p->D && !aligned(p->D, 4)) || (p->h0 && !aligned(p->h0, 4)) || (p->h_last && !aligned(p->h_last, 4)))
    return SSM_ERR_ALIGN;
  if (!rows_aligned16(d->x, (need & kNeedX) ? p->x : nullptr, 3) ||
      !rows_aligned16(d->B, (need & kNeedB) ? p->B : nullptr, 3) ||
      !rows_aligned16(d->C, (need & kNeedC) ? p->C : nullptr, 3) ||
      !rows_aligned16(d->y, (need & kNeedY) ? p->y : nullptr, 3) || (p->h0 && !aligned(p->h0, 16)) ||
      (p->h_last && !aligned(p->h_last, 16)))
    return SSM_ERR_ALIGN;
  const Span ins[] = {span_of(d->x, p->x),
                      span_of(d->delta, p->delta),
                      span_of(d->A, p->A),
                      span_of(d->B, p->B),
                      span_of(d->C, p->C),
                      (f & SSM_HAS_D) ? span_of(d->D, p->D) : Span(),
                      (f & SSM_HAS_H0) ? span_of(d->h0, p->h0) : Span()};
  const Span ys = (need & kNeedY) ? span_of(d->y, p->y) : Span();
  const Span hl = (f & SSM_WANT_HLAST) ? span_of(d->h_last, p->h_last) : Span();
  for (const Span& s : ins)
    if (overlap(ys, s) || overlap(hl, s)) return SSM_ERR_ALIAS;
  if (overlap(ys, hl)) return SSM_ERR_ALIAS;
  return SSM_OK;
}

ssm::SSDParams make_ssd_params(const ssm_ssd_desc* d, const ssm_ssd_ptrs* p, const SSDPlan& pl) {
  ssm::SSDParams q;
  std::memset(&q, 0, sizeof(q));
  q.x = p->x; q.delta = p->delta; q.A = p->A; q.B = p->B; q.C = p->C;
  q.Dskip = (d->flags & SSM_HAS_D) ? p->D : nullptr;
  q.y = p->y;
  q.h0 = (d->flags & SSM_HAS_H0) ? p->h0 : nullptr;
  q.h_last = (d->flags & SSM_WANT_HLAST) ? p->h_last : nullptr;
  q.batch = d->batch; q.L = d->seqlen; q.H = d->nheads; q.P = d->headdim; q.N = d->dstate;
  q.G = d->ngroups; q.Q = d->chunk; q.nchunks = pl.nchunks; q.Lp = pl.Lp;
  q.xs_b = d->x.stride[0]; q.xs_t = d->x.stride[1]; q.xs_h = d->x.stride[2];
  q.ds_b = d->delta.stride[0]; q.ds_t = d->delta.stride[1]; q.ds_h = d->delta.stride[2];
  q.Bs_b = d->B.stride[0]; q.Bs_t = d->B.stride[1]; q.Bs_g = d->B.stride[2];
  q.Cs_b = d->C.stride[0]; q.Cs_t = d->C.stride[1]; q.Cs_g = d->C.stride[2];
  q.ys_b = d->y.stride[0]; q.ys_t = d->y.stride[1]; q.ys_h = d->y.stride[2];
  q.As_h = d->A.stride[0];
  q.Ds_h = (d->flags & SSM_HAS_D) ? d->D.stride[0] : 0;
  q.euler = (d->flags & SSM_DISC_EULER) ? 1 : 0;
  q.y_f32 = d->y.dtype == SSM_F32;
  return q;
}

// ---------------------------------------------------------- SSD backward

constexpr uint32_t kSSDBwdFlags = SSM_HAS_D | SSM_DISC_EULER | SSM_HAS_H0 | SSM_HAS_SSD_FWD;

struct SSDBwdPlan {
  SSDPlan f;
  int HB = 1, nhb = 1;
  int64_t ws_state = 0, ws_s32 = 0, ws_half = 0, ws_aend = 0, ws_step = 0, ws_acA = 0, ws_part = 0, ws_pdb = 0,
          ws_total = 0;
  bool own_fwd = true;  // A_cum, beta and states are recomputed into the workspace
};

// The forward problem of a backward descriptor (dx stands in for y: both are
// (batch, seqlen, nheads, headdim) BF16 or F32 with unit innermost stride).
ssm_ssd_desc ssd_fwd_of(const ssm_ssd_bwd_desc& d) {
  ssm_ssd_desc f;
  std::memset(&f, 0, sizeof(f));
  f.batch = d.batch; f.seqlen = d.seqlen; f.nheads = d.nheads; f.headdim = d.headdim; f.dstate = d.dstate;
  f.ngroups = d.ngroups; f.chunk = d.chunk; f.flags = d.flags & ~SSM_HAS_SSD_FWD;
  f.x = d.x; f.delta = d.delta; f.A = d.A; f.B = d.B; f.C = d.C; f.D = d.D; f.y = d.dx; f.h0 = d.h0;
  return f;
}

SSDBwdPlan plan_ssd_bwd(const ssm_ssd_bwd_desc& d) {
  SSDBwdPlan pl;
  const ssm_ssd_desc f = ssd_fwd_of(d);
  pl.f = plan_ssd(f);
  const int64_t nc = pl.f.nchunks, hpg = d.nheads / d.ngroups;
  // heads per workgroup of the dC / dx passes: as few rounds of workgroups
  // as the heads allow (ssd_heads_per_block), counted for the dx pass, which
  // sets the time and runs one workgroup per compute unit (20 heads and one
  // round at the 2.7B layer with chunk 256; 40 at chunk 128)
  pl.HB = ssm::ssd_heads_per_block(hpg, d.batch * nc * d.ngroups, kSimds / 4);
  pl.nhb = (int)((hpg + pl.HB - 1) / pl.HB);
  const int64_t E = d.batch * nc * d.nheads * d.headdim * d.dstate;
  pl.ws_state = round256(E * 4);
  // the entering states in fp32 for the state pass's backward sweep: kept in
  // registers when the chunk-parallel kernel runs (up to 32 chunks)
  pl.ws_s32 = nc <= 32 ? 0 : pl.ws_state;
  pl.ws_half = round256(E * 2);
  pl.ws_aend = round256(d.batch * d.nheads * nc * ((64 / ssm::ssd_bwd_state_rows(nc)) * (d.dstate / 64)) * 4);
  pl.ws_step = round256(d.batch * d.nheads * pl.f.Lp * 4);
  pl.ws_acA = round256((d.dstate / 64) * d.batch * d.nheads * pl.f.Lp * 4);  // one per 64-wide block of the states
  pl.ws_part = round256(d.batch * nc * d.nheads * 4);
  pl.ws_pdb = round256((int64_t)pl.nhb * d.batch * d.seqlen * d.ngroups * d.dstate * 4);
  // A_cum, beta | states, dS, S32 | SinT, dSl, dSlT | pAend | dAcA | dAcB, dbeta, Tj, dDj | pA, pD | pdB, pdC;
  // with SSM_HAS_SSD_FWD the caller's A_cum, beta and states take the place of the first three
  pl.own_fwd = !(d.flags & SSM_HAS_SSD_FWD);
  pl.ws_total = (pl.own_fwd ? pl.f.ws_acum + pl.f.ws_beta + pl.ws_state : 0) + pl.ws_state + pl.ws_s32 + 3 * pl.ws_half +
                pl.ws_aend + pl.ws_acA + 4 * pl.ws_step + 2 * pl.ws_part + 2 * pl.ws_pdb;
  return pl;
}

ssm_status validate_ssd_bwd_desc(const ssm_ssd_bwd_desc* d) {
  if (!d) return SSM_ERR_NULL;
  if (d->flags & ~kSSDBwdFlags) return SSM_ERR_UNSUPPORTED;
  const ssm_ssd_desc f = ssd_fwd_of(*d);
  ssm_status s = validate_ssd_desc(&f);
  if (s) return s;
  const int64_t blhp[4] = {d->batch, d->seqlen, d->nheads, d->headdim};
  const int64_t blh[3] = {d->batch, d->seqlen, d->nheads};
  const int64_t blgn[4] = {d->batch, d->seqlen, d->ngroups, d->dstate};
  const int64_t h1[1] = {d->nheads};
  const int64_t bhpn[4] = {d->batch, d->nheads, d->headdim, d->dstate};
  if ((s = check_tensor(d->dy, 4, blhp, d->dy.dtype == SSM_BF16, true, false))) return s;
  if ((s = check_tensor(d->ddelta, 3, blh, d->ddelta.dtype == SSM_F32, true, false))) return s;
  if (!non_overlapping(d->ddelta)) return SSM_ERR_STRIDE;
  if ((s = check_tensor(d->dA, 1, h1, d->dA.dtype == SSM_F32, false, true))) return s;
  if ((s = check_tensor(d->dB, 4, blgn, d->dB.dtype == SSM_F32, false, true))) return s;
  if ((s = check_tensor(d->dC, 4, blgn, d->dC.dtype == SSM_F32, false, true))) return s;
  if (d->flags & SSM_HAS_D)
    if ((s = check_tensor(d->dD, 1, h1, d->dD.dtype == SSM_F32, false, true))) return s;
  if (d->flags & SSM_HAS_H0)
    if ((s = check_tensor(d->dh0, 4, bhpn, d->dh0.dtype == SSM_F32, false, true))) return s;
  const SSDBwdPlan pl = plan_ssd_bwd(*d);
  if (d->batch * pl.f.nchunks * d->ngroups * pl.nhb >= ((int64_t)1 << 31) ||
      d->batch * d->nheads * pl.f.nchunks * 4 >= ((int64_t)1 << 31))
    return SSM_ERR_UNSUPPORTED;
  // The dx pass loads a chunk's rows of x and dy with 32-bit byte offsets
  // from the chunk's first row.
  if (d->chunk * d->x.stride[1] * 2 >= ((int64_t)1 << 31) || d->chunk * d->dy.stride[1] * 2 >= ((int64_t)1 << 31))
    return SSM_ERR_UNSUPPORTED;
  return SSM_OK;
}

// `ws`: the workspace the call will write (invalid span: none given); it may
// not overlap any input, output or the forward's intermediates.
ssm_status validate_ssd_bwd_ptrs(const ssm_ssd_bwd_desc* d, const ssm_ssd_bwd_ptrs* p, Span ws = Span()) {
  if (!p) return SSM_ERR_NULL;
  const uint32_t f = d->flags;
  if (!p->x || !p->delta || !p->A || !p->B || !p->C || !p->dy || !p->dx || !p->ddelta || !p->dA || !p->dB ||
      !p->dC)
    return SSM_ERR_NULL;
  if ((f & SSM_HAS_D) && (!p->D || !p->dD)) return SSM_ERR_NULL;
  if ((f & SSM_HAS_H0) && (!p->h0 || !p->dh0)) return SSM_ERR_NULL;
  const bool fwd = f & SSM_HAS_SSD_FWD;
  if (fwd && (!p->A_cum || !p->beta || !p->states)) return SSM_ERR_NULL;
  if (fwd && (!aligned(p->A_cum, 16) || !aligned(p->beta, 16) || !aligned(p->states, 16))) return SSM_ERR_ALIGN;
  if (!aligned(p->delta, 2) || !aligned(p->A, 4) || !aligned(p->ddelta, 4) || !aligned(p->dA, 4) ||
      !aligned(p->dB, 4) || !aligned(p->dC, 4) || (p->D && !aligned(p->D, 4)) || (p->dD && !aligned(p->dD, 4)))
    return SSM_ERR_ALIGN;
  if (!rows_aligned16(d->x, p->x, 3) || !rows_aligned16(d->dy, p->dy, 3) || !rows_aligned16(d->B, p->B, 3) ||
      !rows_aligned16(d->C, p->C, 3) || !rows_aligned16(d->dx, p->dx, 3) ||
      ((f & SSM_HAS_H0) && (!aligned(p->h0, 16) || !aligned(p->dh0, 16))))
    return SSM_ERR_ALIGN;
  // sizes of the forward's intermediates: (batch, nheads, Lp) and (batch, nchunks, nheads, headdim, dstate) F32
  const int64_t nc = (d->seqlen + d->chunk - 1) / d->chunk;
  const int64_t acum_bytes = d->batch * d->nheads * nc * d->chunk * 4;
  const int64_t state_bytes = d->batch * nc * d->nheads * d->headdim * d->dstate * 4;
  const Span ins[] = {span_of(d->x, p->x),  span_of(d->delta, p->delta), span_of(d->A, p->A),
                      span_of(d->B, p->B),  span_of(d->C, p->C),         span_of(d->dy, p->dy),
                      (f & SSM_HAS_D) ? span_of(d->D, p->D) : Span(),
                      (f & SSM_HAS_H0) ? span_of(d->h0, p->h0) : Span(),
                      fwd ? span_bytes(p->A_cum, acum_bytes) : Span(),
                      fwd ? span_bytes(p->beta, acum_bytes) : Span(),
                      fwd ? span_bytes(p->states, state_bytes) : Span()};
  const Span outs[] = {span_of(d->dx, p->dx), span_of(d->ddelta, p->ddelta), span_of(d->dA, p->dA),
                       span_of(d->dB, p->dB), span_of(d->dC, p->dC),
                       (f & SSM_HAS_D) ? span_of(d->dD, p->dD) : Span(),
                       (f & SSM_HAS_H0) ? span_of(d->dh0, p->dh0) : Span()};
  const int no = sizeof(outs) / sizeof(outs[0]);
  for (int i = 0; i < no; ++i) {
    for (const Span& s : ins)
      if (overlap(outs[i], s)) return SSM_ERR_ALIAS;
    for (int j = i + 1; j < no; ++j)
      if (overlap(outs[i], outs[j])) return SSM_ERR_ALIAS;
    if (overlap(outs[i], ws)) return SSM_ERR_ALIAS;
  }
  for (const Span& s : ins)
    if (overlap(ws, s)) return SSM_ERR_ALIAS;
  return SSM_OK;
}

// ---------------------------------------------------------------- decode

ssm_status validate_update(const ssm_update_desc* d, const ssm_update_ptrs* p) {
  if (!d || !p) return SSM_ERR_NULL;
  if (d->batch <= 0 || d->dim <= 0 || d->dstate <= 0) return SSM_ERR_SHAPE;
  if (d->flags & ~kUpdateFlags) return SSM_ERR_UNSUPPORTED;
  if ((d->flags & SSM_HAS_DELTA_BIAS) && !(d->flags & SSM_DELTA_SOFTPLUS)) return SSM_ERR_UNSUPPORTED;
  if (d->dstate > SSM_SCAN_MAX_DSTATE) return SSM_ERR_UNSUPPORTED;
  // one workgroup per (batch element, 16..256 channels): the grid is 1-D
  if (d->dim > (1 << 30) || d->batch * ((d->dim + 15) / 16) >= ((int64_t)1 << 31)) return SSM_ERR_UNSUPPORTED;
  const int32_t io = d->x.dtype;
  if (io == SSM_F16) return SSM_ERR_UNSUPPORTED;
  const bool io_ok = io == SSM_F32 || io == SSM_BF16;
  const uint32_t f = d->flags;
  const int64_t bd[2] = {d->batch, d->dim};
  const int64_t bn[2] = {d->batch, d->dstate};
  const int64_t dn[2] = {d->dim, d->dstate};
  const int64_t dd[1] = {d->dim};
  const int64_t bdn[3] = {d->batch, d->dim, d->dstate};
  ssm_status s;
  if ((s = check_tensor(d->x, 2, bd, io_ok, true, false))) return s;
  if ((s = check_tensor(d->delta, 2, bd, d->delta.dtype == io, true, false))) return s;
  if ((s = check_tensor(d->B, 2, bn, d->B.dtype == io, false, false))) return s;
  if ((s = check_tensor(d->C, 2, bn, d->C.dtype == io, false, false))) return s;
  if ((s = check_tensor(d->A, 2, dn, d->A.dtype == SSM_F32, false, false))) return s;
  if ((s = check_tensor(d->y, 2, bd, d->y.dtype == io || d->y.dtype == SSM_F32, true, false))) return s;
  if (!non_overlapping(d->y)) return SSM_ERR_STRIDE;
  if ((s = check_tensor(d->state, 3, bdn, d->state.dtype == SSM_F32, false, true))) return s;
  if (f & SSM_HAS_Z)
    if ((s = check_tensor(d->z, 2, bd, d->z.dtype == io, true, false))) return s;
  if (f & SSM_HAS_D)
    if ((s = check_tensor(d->D, 1, dd, d->D.dtype == SSM_F32, false, false))) return s;
  if (f & SSM_HAS_DELTA_BIAS)
    if ((s = check_tensor(d->delta_bias, 1, dd, d->delta_bias.dtype == SSM_F32, false, false))) return s;
  if (!p->x || !p->delta || !p->A || !p->B || !p->C || !p->y || !p->state) return SSM_ERR_NULL;
  if ((f & SSM_HAS_DELTA_BIAS) && (!p->delta_bias)) return SSM_ERR_NULL;
  if ((f & SSM_HAS_DELTA_BIAS) && !aligned(p->delta_bias, 4)) return SSM_ERR_ALIGN;
  if ((f & SSM_HAS_Z) && !p->z) return SSM_ERR_NULL;
  if ((f & SSM_HAS_D) && !p->D) return SSM_ERR_NULL;
  const int64_t e = esize(io);
  if (!aligned(p->x, e) || !aligned(p->delta, e) || !aligned(p->B, e) || !aligned(p->C, e) || !aligned(p->A, 4) ||
      !aligned(p->y, esize(d->y.dtype)) || !aligned(p->state, 4))
    return SSM_ERR_ALIGN;
  if (((f & SSM_HAS_Z) && !aligned(p->z, e)) || ((f & SSM_HAS_D) && !aligned(p->D, 4))) return SSM_ERR_ALIGN;
  const Span ins[] = {span_of(d->x, p->x),
                      span_of(d->delta, p->delta),
                      span_of(d->A, p->A),
                      span_of(d->B, p->B),
                      span_of(d->C, p->C),
                      (f & SSM_HAS_D) ? span_of(d->D, p->D) : Span(),
                      (f & SSM_HAS_Z) ? span_of(d->z, p->z) : Span(),
                      (f & SSM_HAS_DELTA_BIAS) ? span_of(d->delta_bias, p->delta_bias) : Span()};
  const Span ys = span_of(d->y, p->y);
  const Span st = span_of(d->state, p->state);
  for (const Span& sp : ins)
    if (overlap(ys, sp) || overlap(st, sp)) return SSM_ERR_ALIAS;
  if (overlap(ys, st)) return SSM_ERR_ALIAS;
  return SSM_OK;
}

// --------------------------------------------------------- scan backward

// Workspace of the backward, in this order: checkpoints (unless given), the
// per-channel-block partials of dB and dC, the per-(batch row, segment)
// partials of dA, dD and dbias, and with the sequence split the segment
// carries cH, cS, cin.  When the split backward computes its own
// checkpoints, the forward's split aggregates (agg_H, agg_S, h_in, which fit)
// reuse the carry buffers: the forward is done with them before the carry
// pass starts.
struct BwdPlan {
  int64_t ntiles = 0, n_dblk = 0;
  int n_seg = 1;
  int64_t seg_len = 0;
  ScanPlan fwd;  // the split forward that writes the checkpoints (fwd.n_seg > 1)
  int64_t ws_ckpt = 0, ws_pdB = 0, ws_pdA = 0, ws_pdD = 0, ws_cH = 0, ws_cS = 0, ws_yrow = 0, ws_total = 0;
};

BwdPlan plan_bwd(const ssm_scan_bwd_desc& d) {
  BwdPlan pl;
  pl.ntiles = (d.seqlen + 15) / 16;
  pl.n_dblk = (d.dim + 15) / 16;
  // the backward's walk holds three waves per SIMD
  split_seq(d.batch, d.seqlen, d.dim, 3, pl.n_seg, pl.seg_len);
  const int64_t ns = pl.n_seg;
  if (ns > 1 && !(d.flags & SSM_HAS_CKPT)) {
    pl.fwd = plan_scan_dims(d.batch, d.seqlen, d.dim, d.dstate);
    pl.ws_yrow = round256(d.dim * 4);  // the checkpoint forward's y: one fp32 row, overwritten
  }
  pl.ws_ckpt = (d.flags & SSM_HAS_CKPT) ? 0 : round256(d.batch * pl.ntiles * d.dim * d.dstate * 4);
  pl.ws_pdB = round256(pl.n_dblk * d.batch * d.seqlen * d.dstate * 4);
  pl.ws_pdA = round256(d.batch * ns * d.dim * d.dstate * 4);
  pl.ws_pdD = round256(d.batch * ns * d.dim * 4);
  if (ns > 1) {
    // cH and cin are (batch, n_seg, D, N) like pdA, cS (batch, n_seg, D) like pdD
    pl.ws_cH = std::max(pl.ws_pdA, std::max(pl.fwd.ws_H, pl.fwd.ws_hin));
    pl.ws_cS = std::max(pl.ws_pdD, pl.fwd.ws_S);
  }
  pl.ws_total = pl.ws_ckpt + 2 * pl.ws_pdB + pl.ws_pdA + 2 * pl.ws_pdD + 2 * pl.ws_cH + pl.ws_cS + pl.ws_yrow;
  return pl;
}

ssm_status validate_bwd_desc(const ssm_scan_bwd_desc* d) {
  if (!d) return SSM_ERR_NULL;
  if (d->batch <= 0 || d->seqlen <= 0 || d->dim <= 0 || d->dstate <= 0) return SSM_ERR_SHAPE;
  const uint32_t f = d->flags;
  if (f & ~kScanBwdFlags) return SSM_ERR_UNSUPPORTED;
  if ((f & SSM_HAS_DELTA_BIAS) && !(f & SSM_DELTA_SOFTPLUS)) return SSM_ERR_UNSUPPORTED;
  if (d->dstate > SSM_SCAN_MAX_DSTATE) return SSM_ERR_UNSUPPORTED;
  if (d->batch * ((d->dim + 15) / 16) >= ((int64_t)1 << 31)) return SSM_ERR_UNSUPPORTED;
  const int32_t io = d->x.dtype;
  if (io == SSM_F16) return SSM_ERR_UNSUPPORTED;
  const bool io_ok = io == SSM_F32 || io == SSM_BF16;
  auto out_ok = [&](int32_t dt) { return dt == io || dt == SSM_F32; };
  const int64_t bld[3] = {d->batch, d->seqlen, d->dim};
  const int64_t bln[3] = {d->batch, d->seqlen, d->dstate};
  const int64_t dn[2] = {d->dim, d->dstate};
  const int64_t dd[1] = {d->dim};
  const int64_t bdn[3] = {d->batch, d->dim, d->dstate};
  ssm_status s;
  if ((s = check_tensor(d->x, 3, bld, io_ok, true, false))) return s;
  if ((s = check_tensor(d->delta, 3, bld, d->delta.dtype == io, true, false))) return s;
  if ((s = check_tensor(d->B, 3, bln, d->B.dtype == io, false, false))) return s;
  if ((s = check_tensor(d->C, 3, bln, d->C.dtype == io, false, false))) return s;
  if ((s = check_tensor(d->A, 2, dn, d->A.dtype == SSM_F32, false, false))) return s;
  if ((s = check_tensor(d->dy, 3, bld, out_ok(d->dy.dtype), true, false))) return s;
  if ((s = check_tensor(d->dx, 3, bld, out_ok(d->dx.dtype), true, false))) return s;
  if ((s = check_tensor(d->ddelta, 3, bld, out_ok(d->ddelta.dtype), true, false))) return s;
  if ((s = check_tensor(d->dA, 2, dn, d->dA.dtype == SSM_F32, false, true))) return s;
  if ((s = check_tensor(d->dB, 3, bln, d->dB.dtype == SSM_F32, false, true))) return s;
  if ((s = check_tensor(d->dC, 3, bln, d->dC.dtype == SSM_F32, false, true))) return s;
  if (!non_overlapping(d->dx) || !non_overlapping(d->ddelta)) return SSM_ERR_STRIDE;
  if (f & SSM_HAS_Z) {
    if ((s = check_tensor(d->z, 3, bld, d->z.dtype == io, true, false))) return s;
    if ((s = check_tensor(d->dz, 3, bld, out_ok(d->dz.dtype), true, false))) return s;
    if (!non_overlapping(d->dz)) return SSM_ERR_STRIDE;
  }
  if (f & SSM_HAS_D) {
    if ((s = check_tensor(d->D, 1, dd, d->D.dtype == SSM_F32, false, false))) return s;
    if ((s = check_tensor(d->dD, 1, dd, d->dD.dtype == SSM_F32, false, true))) return s;
  }
  if (f & SSM_HAS_H0) {
    if ((s = check_tensor(d->h0, 3, bdn, d->h0.dtype == SSM_F32, false, true))) return s;
    if ((s = check_tensor(d->dh0, 3, bdn, d->dh0.dtype == SSM_F32, false, true))) return s;
  }
  if (f & SSM_HAS_DELTA_BIAS) {
    if ((s = check_tensor(d->delta_bias, 1, dd, d->delta_bias.dtype == SSM_F32, false, false))) return s;
    if ((s = check_tensor(d->ddelta_bias, 1, dd, d->ddelta_bias.dtype == SSM_F32, false, true))) return s;
  }
  if (f & SSM_HAS_CKPT) {
    int64_t ck[4];
    ckpt_shape(d->batch, d->seqlen, d->dim, d->dstate, ck);
    if ((s = check_tensor(d->ckpt, 4, ck, d->ckpt.dtype == SSM_F32, false, true))) return s;
  }
  // The kernels address one 16-step tile of 16 channels (or of all dstate
  // states of B and C) with 32-bit byte offsets.
  const int64_t e = esize(io);
  auto fits = [&](const ssm_tensor_desc& t, int64_t width, int64_t es) {
    return (16 * t.stride[1] + width * t.stride[2]) * es < ((int64_t)1 << 31);
  };
  if (!fits(d->x, 16, e) || !fits(d->delta, 16, e) || !fits(d->dy, 16, esize(d->dy.dtype)) ||
      !fits(d->B, d->dstate, e) || !fits(d->C, d->dstate, e) || ((f & SSM_HAS_Z) && !fits(d->z, 16, e)))
    return SSM_ERR_UNSUPPORTED;
  return SSM_OK;
}

ssm_status validate_bwd_ptrs(const ssm_scan_bwd_desc* d, const ssm_scan_bwd_ptrs* p) {
  if (!p) return SSM_ERR_NULL;
  const uint32_t f = d->flags;
  if (!p->x || !p->delta || !p->A || !p->B || !p->C || !p->dy || !p->dx || !p->ddelta || !p->dA || !p->dB ||
      !p->dC)
    return SSM_ERR_NULL;
  if ((f & SSM_HAS_Z) && (!p->z || !p->dz)) return SSM_ERR_NULL;
  if ((f & SSM_HAS_D) && (!p->D || !p->dD)) return SSM_ERR_NULL;
  if ((f & SSM_HAS_H0) && (!p->h0 || !p->dh0)) return SSM_ERR_NULL;
  if ((f & SSM_HAS_DELTA_BIAS) && (!p->delta_bias || !p->ddelta_bias)) return SSM_ERR_NULL;
  if ((f & SSM_HAS_CKPT) && !p->ckpt) return SSM_ERR_NULL;
  if ((f & SSM_HAS_CKPT) && !aligned(p->ckpt, 4)) return SSM_ERR_ALIGN;
  const int64_t e = esize(d->x.dtype);
  if (!aligned(p->x, e) || !aligned(p->delta, e) || !aligned(p->B, e) || !aligned(p->C, e) || !aligned(p->A, 4) ||
      !aligned(p->dy, esize(d->dy.dtype)) || !aligned(p->dx, esize(d->dx.dtype)) ||
      !aligned(p->ddelta, esize(d->ddelta.dtype)) || !aligned(p->dA, 4) || !aligned(p->dB, 4) || !aligned(p->dC, 4))
    return SSM_ERR_ALIGN;
  if ((f & SSM_HAS_Z) && (!aligned(p->z, e) || !aligned(p->dz, esize(d->dz.dtype)))) return SSM_ERR_ALIGN;
  if ((f & SSM_HAS_D) && (!aligned(p->D, 4) || !aligned(p->dD, 4))) return SSM_ERR_ALIGN;
  if ((f & SSM_HAS_H0) && (!aligned(p->h0, 4) || !aligned(p->dh0, 4))) return SSM_ERR_ALIGN;
  if ((f & SSM_HAS_DELTA_BIAS) && (!aligned(p->delta_bias, 4) || !aligned(p->ddelta_bias, 4))) return SSM_ERR_ALIGN;
  const Span ins[] = {span_of(d->x, p->x),
                      span_of(d->delta, p->delta),
                      span_of(d->A, p->A),
                      span_of(d->B, p->B),
                      span_of(d->C, p->C),
                      span_of(d->dy, p->dy),
                      (f & SSM_HAS_D) ? span_of(d->D, p->D) : Span(),
                      (f & SSM_HAS_Z) ? span_of(d->z, p->z) : Span(),
                      (f & SSM_HAS_H0) ? span_of(d->h0, p->h0) : Span(),
                      (f & SSM_HAS_DELTA_BIAS) ? span_of(d->delta_bias, p->delta_bias) : Span(),
                      (f & SSM_HAS_CKPT) ? span_of(d->ckpt, p->ckpt) : Span()};
  const Span outs[] = {span_of(d->dx, p->dx),
                       span_of(d->ddelta, p->ddelta),
                       span_of(d->dA, p->dA),
                       span_of(d->dB, p->dB),
                       span_of(d->dC, p->dC),
                       (f & SSM_HAS_Z) ? span_of(d->dz, p->dz) : Span(),
                       (f & SSM_HAS_D) ? span_of(d->dD, p->dD) : Span(),
                       (f & SSM_HAS_H0) ? span_of(d->dh0, p->dh0) : Span(),
                       (f & SSM_HAS_DELTA_BIAS) ? span_of(d->ddelta_bias, p->ddelta_bias) : Span()};
  const int nout = (int)(sizeof(outs) / sizeof(outs[0]));
  for (int i = 0; i < nout; ++i) {
    for (const Span& sp : ins)
      if (overlap(outs[i], sp)) return SSM_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

// ------------------------------------------------------------------ conv

ssm_status validate_conv(const ssm_conv_desc* d, const ssm_conv_ptrs* p) {
  if (!d || !p) return SSM_ERR_NULL;
  if (d->batch <= 0 || d->seqlen <= 0 || d->dim <= 0 || d->width <= 0) return SSM_ERR_SHAPE;
  if (d->flags & ~kConvFlags) return SSM_ERR_UNSUPPORTED;
  if (d->width > ssm::kConvMaxWidth) return SSM_ERR_UNSUPPORTED;
  // grid: (channel blocks) x (32-step runs) x batch workgroups, 1-D
  if (d->batch * ((d->seqlen + 31) / 32) * ((d->dim + 255) / 256) >= ((int64_t)1 << 31)) return SSM_ERR_UNSUPPORTED;
  const int32_t io = d->x.dtype;
  if (io == SSM_F16) return SSM_ERR_UNSUPPORTED;
  const bool io_ok = io == SSM_F32 || io == SSM_BF16;
  const uint32_t f = d->flags;
  const int64_t bld[3] = {d->batch, d->seqlen, d->dim};
  const int64_t dw[2] = {d->dim, d->width};
  const int64_t dd[1] = {d->dim};
  ssm_status s;
  if ((s = check_tensor(d->x, 3, bld, io_ok, true, false))) return s;
  if ((s = check_tensor(d->y, 3, bld, d->y.dtype == io || d->y.dtype == SSM_F32, true, false))) return s;
  if (!non_overlapping(d->y)) return SSM_ERR_STRIDE;
  if ((s = check_tensor(d->weight, 2, dw, d->weight.dtype == SSM_F32, false, false))) return s;
  if (f & SSM_HAS_BIAS)
    if ((s = check_tensor(d->bias, 1, dd, d->bias.dtype == SSM_F32, false, false))) return s;
  if (!p->x || !p->weight || !p->y) return SSM_ERR_NULL;
  if ((f & SSM_HAS_BIAS) && !p->bias) return SSM_ERR_NULL;
  if (!aligned(p->x, esize(io)) || !aligned(p->y, esize(d->y.dtype)) || !aligned(p->weight, 4)) return SSM_ERR_ALIGN;
  if ((f & SSM_HAS_BIAS) && !aligned(p->bias, 4)) return SSM_ERR_ALIGN;
  // the kernel addresses a run of 32 + width rows of 1024 channels with
  // 32-bit byte offsets below 2^29
  if ((32 + ssm::kConvMaxWidth) * std::max(d->x.stride[1], d->y.stride[1]) * 4 + 1024 * 4 >= ((int64_t)1 << 29))
    return SSM_ERR_UNSUPPORTED;
  const Span ys = span_of(d->y, p->y);
  if (overlap(ys, span_of(d->x, p->x)) || overlap(ys, span_of(d->weight, p->weight)) ||
      ((f & SSM_HAS_BIAS) && overlap(ys, span_of(d->bias, p->bias))))
    return SSM_ERR_ALIAS;
  return SSM_OK;
}

ssm_status hip_status(hipError_t e) {
  if (e == hipSuccess) return SSM_OK;
  g_last_hip_error = (int)e;
  return SSM_ERR_HIP;
}

// Fills the kernel parameters of a validated scan and launches it; the
// workspace (pl.ws_total bytes, 256-byte aligned) is the caller's or the
// static scratch.
ssm_status launch_scan_fwd(const ssm_scan_desc* d, const ssm_scan_ptrs* p, const ScanPlan& pl, void* workspace,
                           void* hip_stream) {
  ssm::ScanParams q;
  std::memset(&q, 0, sizeof(q));
  const uint32_t f = d->flags;
  q.x = p->x; q.delta = p->delta; q.z = (f & SSM_HAS_Z) ? p->z : nullptr; q.y = p->y;
  q.B = p->B; q.C = p->C; q.A = p->A; q.Dskip = (f & SSM_HAS_D) ? p->D : nullptr;
  q.h0 = (f & SSM_HAS_H0) ? p->h0 : nullptr;
  q.h_last = (f & SSM_WANT_HLAST) ? p->h_last : nullptr;
  q.batch = d->batch; q.L = d->seqlen; q.D = d->dim; q.N = d->dstate;
  q.xs_b = d->x.stride[0]; q.xs_t = d->x.stride[1];
  q.ds_b = d->delta.stride[0]; q.ds_t = d->delta.stride[1];
  if (f & SSM_HAS_Z) { q.zs_b = d->z.stride[0]; q.zs_t = d->z.stride[1]; }
  q.ys_b = d->y.stride[0]; q.ys_t = d->y.stride[1];
  q.Bs_b = d->B.stride[0]; q.Bs_t = d->B.stride[1]; q.Bs_n = d->B.stride[2];
  q.Cs_b = d->C.stride[0]; q.Cs_t = d->C.stride[1]; q.Cs_n = d->C.stride[2];
  q.As_d = d->A.stride[0]; q.As_n = d->A.stride[1];
  q.Ds_d = (f & SSM_HAS_D) ? d->D.stride[0] : 0;
  q.flags = f;
  q.io_bf16 = d->x.dtype == SSM_BF16;
  q.y_f32 = d->y.dtype == SSM_F32;
  q.dsoftplus = (f & SSM_DELTA_SOFTPLUS) ? 1 : 0;
  q.dbias = (f & SSM_HAS_DELTA_BIAS) ? p->delta_bias : nullptr;
  q.dbs_d = (f & SSM_HAS_DELTA_BIAS) ? d->delta_bias.stride[0] : 0;
  q.ckpt = (f & SSM_WANT_CKPT) ? p->ckpt : nullptr;
  q.n_seg = pl.n_seg;
  q.seg_len = pl.seg_len;
  if (pl.n_seg > 1) {
    char* w = (char*)workspace;
    q.agg_H = (float*)w;
    q.agg_S = (float*)(w + pl.ws_H);
    q.h_in = (float*)(w + pl.ws_H + pl.ws_S);
  }
  return hip_status(ssm::launch_selective_scan(q, (hipStream_t)hip_stream));
}

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_status_string(ssm_status s) {
  switch (s) {
    case SSM_OK: return "SSM_OK";
    case SSM_ERR_NULL: return "SSM_ERR_NULL: a required pointer is NULL";
    case SSM_ERR_SHAPE: return "SSM_ERR_SHAPE: a size is <= 0 or a tensor shape does not match";
    case SSM_ERR_DTYPE: return "SSM_ERR_DTYPE: dtype not allowed for this tensor";
    case SSM_ERR_STRIDE: return "SSM_ERR_STRIDE: negative, non-unit innermost or self-overlapping strides";
    case SSM_ERR_ALIGN: return "SSM_ERR_ALIGN: pointer not aligned";
    case SSM_ERR_ALIAS: return "SSM_ERR_ALIAS: an output overlaps another tensor";
    case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED: valid but not implemented";
    case SSM_ERR_WORKSPACE: return "SSM_ERR_WORKSPACE: workspace missing or too small";
    case SSM_ERR_HIP: return "SSM_ERR_HIP: a HIP call failed";
  }
  return "unknown ssm_status";
}

int ssm_last_hip_error(void) { return g_last_hip_error; }

ssm_status ssm_selective_scan_workspace_size(const ssm_scan_desc* d, size_t* bytes) {
  if (!bytes) return SSM_ERR_NULL;
  ssm_status s = validate_scan_desc(d);
  if (s) return s;
  *bytes = (size_t)plan_scan(*d).ws_total;
  return SSM_OK;
}

ssm_status ssm_selective_scan_fwd(const ssm_scan_desc* d, const ssm_scan_ptrs* p, void* workspace,
                                  size_t workspace_bytes, void* hip_stream) {
  ssm_status s = validate_scan_desc(d);
  if (s) return s;
  if ((s = validate_scan_ptrs(d, p))) return s;
  const ScanPlan pl = plan_scan(*d);
  if (pl.ws_total > 0) {
    if (!workspace || workspace_bytes < (size_t)pl.ws_total) return SSM_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SSM_ERR_ALIGN;
  }
  return launch_scan_fwd(d, p, pl, workspace, hip_stream);
}

ssm_status ssm_selective_scan_fwd_noalloc(const ssm_scan_desc* d, const ssm_scan_ptrs* p, void* hip_stream) {
  ssm_status s = validate_scan_desc(d);
  if (s) return s;
  if ((s = validate_scan_ptrs(d, p))) return s;
  const ScanPlan pl = plan_scan(*d);
  static_assert(SSM_SCAN_STATIC_SCRATCH_BYTES == ssm::kScanStaticScratchBytes, "scratch size");
  if ((size_t)pl.ws_total > SSM_SCAN_STATIC_SCRATCH_BYTES) return SSM_ERR_WORKSPACE;
  void* ws = nullptr;
  if (pl.ws_total > 0) {
    hipError_t e = ssm::scan_static_scratch(&ws);
    if (e != hipSuccess) return hip_status(e);
  }
  return launch_scan_fwd(d, p, pl, ws, hip_stream);
}

ssm_status ssm_ssd_chunk_workspace_size(const ssm_ssd_desc* d, size_t* bytes) {
  if (!bytes) return SSM_ERR_NULL;
  ssm_status s = validate_ssd_desc(d);
  if (s) return s;
  *bytes = (size_t)plan_ssd(*d).ws_total;
  return SSM_OK;
}

ssm_status ssm_ssd_chunk_fwd(const ssm_ssd_desc* d, const ssm_ssd_ptrs* p, void* workspace, size_t workspace_bytes,
                             void* hip_stream) {
  ssm_status s = validate_ssd_desc(d);
  if (s) return s;
  if ((s = validate_ssd_ptrs(d, p, kNeedAll))) return s;
  const SSDPlan pl = plan_ssd(*d);
  if (!workspace || workspace_bytes < (size_t)pl.ws_total) return SSM_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return SSM_ERR_ALIGN;
  ssm::SSDParams q = make_ssd_params(d, p, pl);
  char* w = (char*)workspace;
  q.A_cum = (float*)w;
  q.beta = (float*)(w + pl.ws_acum);
  q.states = (float*)(w + pl.ws_acum + pl.ws_beta);
  q.S_in = (void*)(w + pl.ws_acum + pl.ws_beta + pl.ws_states);
  hipStream_t st = (hipStream_t)hip_stream;
  hipError_t e;
  if ((e = ssm::launch_ssd_chunk_cumsum(q, st)) != hipSuccess) return hip_status(e);
  if ((e = ssm::launch_ssd_chunk_state(q, st)) != hipSuccess) return hip_status(e);
  if ((e = ssm::launch_ssd_state_passing(q, st)) != hipSuccess) return hip_status(e);
  return hip_status(ssm::launch_ssd_chunk_scan(q, st));
}

ssm_status ssm_ssd_chunk_cumsum(const ssm_ssd_desc* d, const ssm_ssd_ptrs* p, float* A_cum, float* beta,
                                void* hip_stream) {
  ssm_status s = validate_ssd_desc(d);
  if (s) return s;
  if ((s = validate_ssd_ptrs(d, p, kNeedDelta))) return s;
  if (!A_cum || !beta) return SSM_ERR_NULL;
  if (!aligned(A_cum, 16) || !aligned(beta, 16)) return SSM_ERR_ALIGN;
  const SSDPlan pl = plan_ssd(*d);
  ssm::SSDParams q = make_ssd_params(d, p, pl);
  q.A_cum = A_cum;
  q.beta = beta;
  return hip_status(ssm::launch_ssd_chunk_cumsum(q, (hipStream_t)hip_stream));
}

ssm_status ssm_ssd_chunk_state(const ssm_ssd_desc* d, const ssm_ssd_ptrs* p, const float* A_cum,
                               const float* beta, float* states, void* hip_stream) {
  ssm_status s = validate_ssd_desc(d);
  if (s) return s;
  if ((s = validate_ssd_ptrs(d, p, kNeedX | kNeedB))) return s;
  if (!A_cum || !beta || !states) return SSM_ERR_NULL;
  if (!aligned(A_cum, 16) || !aligned(beta, 16) || !aligned(states, 16)) return SSM_ERR_ALIGN;
  const SSDPlan pl = plan_ssd(*d);
  ssm::SSDParams q = make_ssd_params(d, p, pl);
  q.A_cum = (float*)A_cum;
  q.beta = (float*)beta;
  q.states = states;
  return hip_status(ssm::launch_ssd_chunk_state(q, (hipStream_t)hip_stream));
}

ssm_status ssm_ssd_state_passing(const ssm_ssd_desc* d, const ssm_ssd_ptrs* p, const float* A_cum,
                                 const float* states, void* S_in, void* hip_stream) {
  ssm_status s = validate_ssd_desc(d);
  if (s) return s;
  if ((s = validate_ssd_ptrs(d, p, 0))) return s;
  if (!A_cum || !states || !S_in) return SSM_ERR_NULL;
  if (!aligned(A_cum, 16) || !aligned(states, 16) || !aligned(S_in, 16)) return SSM_ERR_ALIGN;
  const SSDPlan pl = plan_ssd(*d);
  ssm::SSDParams q = make_ssd_params(d, p, pl);
  q.A_cum = (float*)A_cum;
  q.states = (float*)states;
  q.S_in = S_in;
  return hip_status(ssm::launch_ssd_state_passing(q, (hipStream_t)hip_stream));
}

ssm_status ssm_ssd_chunk_scan(const ssm_ssd_desc* d, const ssm_ssd_ptrs* p, const float* A_cum, const float* beta,
                              const void* S_in, void* hip_stream) {
  ssm_status s = validate_ssd_desc(d);
  if (s) return s;
  if ((s = validate_ssd_ptrs(d, p, kNeedX | kNeedB | kNeedC | kNeedY))) return s;
  if (!A_cum || !beta || !S_in) return SSM_ERR_NULL;
  if (!aligned(A_cum, 16) || !aligned(beta, 16) || !aligned(S_in, 16)) return SSM_ERR_ALIGN;
  const SSDPlan pl = plan_ssd(*d);
  ssm::SSDParams q = make_ssd_params(d, p, pl);
  q.A_cum = (float*)A_cum;
  q.beta = (float*)beta;
  q.S_in = (void*)S_in;
  return hip_status(ssm::launch_ssd_chunk_scan(q, (hipStream_t)hip_stream));
}

ssm_status ssm_selective_scan_bwd_workspace_size(const ssm_scan_bwd_desc* d, size_t* bytes) {
  if (!bytes) return SSM_ERR_NULL;
  ssm_status s = validate_bwd_desc(d);
  if (s) return s;
  *bytes = (size_t)plan_bwd(*d).ws_total;
  return SSM_OK;
}

ssm_status ssm_selective_scan_bwd(const ssm_scan_bwd_desc* d, const ssm_scan_bwd_ptrs* p, void* workspace,
                                  size_t workspace_bytes, void* hip_stream) {
  ssm_status s = validate_bwd_desc(d);
  if (s) return s;
  if ((s = validate_bwd_ptrs(d, p))) return s;
  const BwdPlan pl = plan_bwd(*d);
  if (!workspace || workspace_bytes < (size_t)pl.ws_total) return SSM_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return SSM_ERR_ALIGN;
  const uint32_t f = d->flags;
  ssm::ScanBwdParams q;
  std::memset(&q, 0, sizeof(q));
  q.x = p->x; q.delta = p->delta; q.z = (f & SSM_HAS_Z) ? p->z : nullptr; q.dy = p->dy;
  q.B = p->B; q.C = p->C; q.A = p->A; q.Dskip = (f & SSM_HAS_D) ? p->D : nullptr;
  q.h0 = (f & SSM_HAS_H0) ? p->h0 : nullptr;
  q.dbias = (f & SSM_HAS_DELTA_BIAS) ? p->delta_bias : nullptr;
  q.dx = p->dx; q.ddelta = p->ddelta; q.dz = (f & SSM_HAS_Z) ? p->dz : nullptr;
  q.dA = p->dA; q.dB = p->dB; q.dC = p->dC;
  q.dD = (f & SSM_HAS_D) ? p->dD : nullptr;
  q.dh0 = (f & SSM_HAS_H0) ? p->dh0 : nullptr;
  q.ddbias = (f & SSM_HAS_DELTA_BIAS) ? p->ddelta_bias : nullptr;
  char* w = (char*)workspace;
  q.ckpt = (f & SSM_HAS_CKPT) ? (float*)p->ckpt : (float*)w;  // the given checkpoints are only read
  q.ckpt_given = (f & SSM_HAS_CKPT) ? 1 : 0;
  q.pdB = (float*)(w + pl.ws_ckpt);
  q.pdC = (float*)(w + pl.ws_ckpt + pl.ws_pdB);
  q.pdA = (float*)(w + pl.ws_ckpt + 2 * pl.ws_pdB);
  q.pdD = (f & SSM_HAS_D) ? (float*)(w + pl.ws_ckpt + 2 * pl.ws_pdB + pl.ws_pdA) : nullptr;
  q.pdbias = (f & SSM_HAS_DELTA_BIAS) ? (float*)(w + pl.ws_ckpt + 2 * pl.ws_pdB + pl.ws_pdA + pl.ws_pdD) : nullptr;
  q.batch = d->batch; q.L = d->seqlen; q.D = d->dim; q.N = d->dstate;
  q.xs_b = d->x.stride[0]; q.xs_t = d->x.stride[1];
  q.ds_b = d->delta.stride[0]; q.ds_t = d->delta.stride[1];
  if (f & SSM_HAS_Z) {
    q.zs_b = d->z.stride[0]; q.zs_t = d->z.stride[1];
    q.dzs_b = d->dz.stride[0]; q.dzs_t = d->dz.stride[1];
    q.dz_f32 = d->dz.dtype == SSM_F32;
  }
  q.gs_b = d->dy.stride[0]; q.gs_t = d->dy.stride[1];
  q.dxs_b = d->dx.stride[0]; q.dxs_t = d->dx.stride[1];
  q.dds_b = d->ddelta.stride[0]; q.dds_t = d->ddelta.stride[1];
  q.Bs_b = d->B.stride[0]; q.Bs_t = d->B.stride[1]; q.Bs_n = d->B.stride[2];
  q.Cs_b = d->C.stride[0]; q.Cs_t = d->C.stride[1]; q.Cs_n = d->C.stride[2];
  q.As_d = d->A.stride[0]; q.As_n = d->A.stride[1];
  q.Ds_d = (f & SSM_HAS_D) ? d->D.stride[0] : 0;
  q.dbs_d = (f & SSM_HAS_DELTA_BIAS) ? d->delta_bias.stride[0] : 0;
  q.io_bf16 = d->x.dtype == SSM_BF16;
  q.dy_f32 = d->dy.dtype == SSM_F32;
  q.dx_f32 = d->dx.dtype == SSM_F32;
  q.dd_f32 = d->ddelta.dtype == SSM_F32;
  q.euler = (f & SSM_DISC_EULER) ? 1 : 0;
  q.dsoftplus = (f & SSM_DELTA_SOFTPLUS) ? 1 : 0;
  q.n_seg = pl.n_seg;
  q.seg_len = pl.seg_len;
  hipStream_t st = (hipStream_t)hip_stream;
  if (pl.n_seg > 1) {
    char* c = w + pl.ws_ckpt + 2 * pl.ws_pdB + pl.ws_pdA + 2 * pl.ws_pdD;
    q.cH = (float*)c;
    q.cin = (float*)(c + pl.ws_cH);
    q.cS = (float*)(c + 2 * pl.ws_cH);
    if (!q.ckpt_given) {
      // The checkpoints from the forward's split kernels; y goes to a
      // scratch row (strides 0) and is not used.
      ssm::ScanParams fq;
      std::memset(&fq, 0, sizeof(fq));
      fq.x = q.x; fq.delta = q.delta; fq.B = q.B; fq.C = q.C; fq.A = q.A; fq.h0 = q.h0;
      fq.batch = q.batch; fq.L = q.L; fq.D = q.D; fq.N = q.N;
      fq.xs_b = q.xs_b; fq.xs_t = q.xs_t; fq.ds_b = q.ds_b; fq.ds_t = q.ds_t;
      fq.y = c + 2 * pl.ws_cH + pl.ws_cS;
      fq.ys_b = 0; fq.ys_t = 0;
      fq.Bs_b = q.Bs_b; fq.Bs_t = q.Bs_t; fq.Bs_n = q.Bs_n;
      fq.Cs_b = q.Cs_b; fq.Cs_t = q.Cs_t; fq.Cs_n = q.Cs_n;
      fq.As_d = q.As_d; fq.As_n = q.As_n;
      fq.flags = f & (SSM_DISC_EULER | SSM_HAS_H0);
      fq.io_bf16 = q.io_bf16;
      fq.y_f32 = 1;
      fq.dbias = q.dbias; fq.dbs_d = q.dbs_d; fq.dsoftplus = q.dsoftplus;
      fq.ckpt = q.ckpt;
      fq.n_seg = pl.fwd.n_seg;
      fq.seg_len = pl.fwd.seg_len;
      if (fq.n_seg > 1) {
        fq.agg_H = q.cH;
        fq.agg_S = q.cS;
        fq.h_in = q.cin;
      }
      hipError_t e = ssm::launch_selective_scan(fq, st);
      if (e != hipSuccess) return hip_status(e);
      q.ckpt_given = 1;
    }
  }
  return hip_status(ssm::launch_selective_scan_bwd(q, st));
}

ssm_status ssm_ssd_bwd_workspace_size(const ssm_ssd_bwd_desc* d, size_t* bytes) {
  if (!bytes) return SSM_ERR_NULL;
  ssm_status s = validate_ssd_bwd_desc(d);
  if (s) return s;
  *bytes = (size_t)plan_ssd_bwd(*d).ws_total;
  return SSM_OK;
}

ssm_status ssm_ssd_bwd(const ssm_ssd_bwd_desc* d, const ssm_ssd_bwd_ptrs* p, void* workspace, size_t workspace_bytes,
                       void* hip_stream) {
  ssm_status s = validate_ssd_bwd_desc(d);
  if (s) return s;
  const SSDBwdPlan pl = plan_ssd_bwd(*d);
  if ((s = validate_ssd_bwd_ptrs(d, p, span_bytes(workspace, pl.ws_total)))) return s;
  if (!workspace || workspace_bytes < (size_t)pl.ws_total) return SSM_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return SSM_ERR_ALIGN;
  const uint32_t f = d->flags;
  const ssm_ssd_desc fd = ssd_fwd_of(*d);
  ssm_ssd_ptrs fp;
  std::memset(&fp, 0, sizeof(fp));
  fp.x = p->x; fp.delta = p->delta; fp.A = p->A; fp.B = p->B; fp.C = p->C;
  fp.D = (f & SSM_HAS_D) ? p->D : nullptr;
  fp.h0 = (f & SSM_HAS_H0) ? p->h0 : nullptr;
  ssm::SSDBwdParams q;
  std::memset(&q, 0, sizeof(q));
  q.f = make_ssd_params(&fd, &fp, pl.f);
  q.f.y = nullptr;
  char* w = (char*)workspace;
  auto take = [&](int64_t bytes) {
    char* r = w;
    w += bytes;
    return r;
  };
  if (pl.own_fwd) {
    q.f.A_cum = (float*)take(pl.f.ws_acum);
    q.f.beta = (float*)take(pl.f.ws_beta);
    q.f.states = (float*)take(pl.ws_state);
  } else {  // read only by the backward's kernels
    q.f.A_cum = const_cast<float*>(p->A_cum);
    q.f.beta = const_cast<float*>(p->beta);
    q.f.states = const_cast<float*>(p->states);
  }
  q.dS = (float*)take(pl.ws_state);
  q.S32 = pl.ws_s32 ? (float*)take(pl.ws_s32) : nullptr;
  q.SinT = (uint16_t*)take(pl.ws_half);
  q.dSl = (uint16_t*)take(pl.ws_half);
  q.dSlT = (uint16_t*)take(pl.ws_half);
  q.pAend = (float*)take(pl.ws_aend);
  q.dAcA = (float*)take(pl.ws_acA);
  q.dAcB = (float*)take(pl.ws_step);
  q.dbeta = (float*)take(pl.ws_step);
  q.Tj = (float*)take(pl.ws_step);
  q.dDj = (float*)take(pl.ws_step);
  q.pA = (float*)take(pl.ws_part);
  q.pD = (float*)take(pl.ws_part);
  q.pdB = (float*)take(pl.ws_pdb);
  q.pdC = (float*)take(pl.ws_pdb);
  q.dy = p->dy;
  q.dys_b = d->dy.stride[0]; q.dys_t = d->dy.stride[1]; q.dys_h = d->dy.stride[2];
  q.dx = p->dx;
  q.dxs_b = d->dx.stride[0]; q.dxs_t = d->dx.stride[1]; q.dxs_h = d->dx.stride[2];
  q.dx_f32 = d->dx.dtype == SSM_F32;
  q.ddelta = p->ddelta;
  q.dds_b = d->ddelta.stride[0]; q.dds_t = d->ddelta.stride[1]; q.dds_h = d->ddelta.stride[2];
  q.dh0 = (f & SSM_HAS_H0) ? p->dh0 : nullptr;
  q.HB = pl.HB;
  q.nhb = pl.nhb;
  q.aend_parts = (64 / ssm::ssd_bwd_state_rows(q.f.nchunks)) * (int)(d->dstate / 64);
  const hipStream_t st = (hipStream_t)hip_stream;
  if (pl.own_fwd) {  // recompute the forward's A_cum, beta and chunk states
    hipError_t e = ssm::launch_ssd_chunk_cumsum(q.f, st);
    if (e == hipSuccess) e = ssm::launch_ssd_chunk_state(q.f, st);
    if (e != hipSuccess) return hip_status(e);
  }
  return hip_status(ssm::launch_ssd_bwd(q, p->dA, p->dB, p->dC, (f & SSM_HAS_D) ? p->dD : nullptr,
                                        (hipStream_t)hip_stream));
}

ssm_status ssm_causal_conv1d_fwd(const ssm_conv_desc* d, const ssm_conv_ptrs* p, void* hip_stream) {
  ssm_status s = validate_conv(d, p);
  if (s) return s;
  ssm::ConvParams q;
  std::memset(&q, 0, sizeof(q));
  q.x = p->x; q.w = p->weight; q.bias = (d->flags & SSM_HAS_BIAS) ? p->bias : nullptr; q.y = p->y;
  q.batch = d->batch; q.L = d->seqlen; q.D = d->dim; q.W = d->width;
  q.xs_b = d->x.stride[0]; q.xs_t = d->x.stride[1];
  q.ys_b = d->y.stride[0]; q.ys_t = d->y.stride[1];
  // the kernel drops stores past row L-1 by a range check that needs a row
  // stride of at least dim; a single row's stride is arbitrary, so give it one
  if (d->seqlen == 1) { q.xs_t = d->dim; q.ys_t = d->dim; }
  q.ws_d = d->weight.stride[0]; q.ws_k = d->weight.stride[1];
  q.bs_d = (d->flags & SSM_HAS_BIAS) ? d->bias.stride[0] : 0;
  q.io_bf16 = d->x.dtype == SSM_BF16;
  q.y_f32 = d->y.dtype == SSM_F32;
  q.silu = (d->flags & SSM_SILU) ? 1 : 0;
  return hip_status(ssm::launch_causal_conv1d(q, (hipStream_t)hip_stream));
}

ssm_status ssm_selective_state_update(const ssm_update_desc* d, const ssm_update_ptrs* p, void* hip_stream) {
  ssm_status s = validate_update(d, p);
  if (s) return s;
  ssm::UpdateParams q;
  std::memset(&q, 0, sizeof(q));
  const uint32_t f = d->flags;
  q.x = p->x; q.delta = p->delta; q.z = (f & SSM_HAS_Z) ? p->z : nullptr; q.y = p->y;
  q.B = p->B; q.C = p->C; q.A = p->A; q.Dskip = (f & SSM_HAS_D) ? p->D : nullptr; q.state = p->state;
  q.batch = d->batch; q.D = d->dim; q.N = d->dstate;
  q.xs_b = d->x.stride[0]; q.ds_b = d->delta.stride[0];
  q.zs_b = (f & SSM_HAS_Z) ? d->z.stride[0] : 0; q.ys_b = d->y.stride[0];
  q.Bs_b = d->B.stride[0]; q.Bs_n = d->B.stride[1];
  q.Cs_b = d->C.stride[0]; q.Cs_n = d->C.stride[1];
  q.As_d = d->A.stride[0]; q.As_n = d->A.stride[1];
  q.Ds_d = (f & SSM_HAS_D) ? d->D.stride[0] : 0;
  q.euler = (f & SSM_DISC_EULER) ? 1 : 0;
  q.io_bf16 = d->x.dtype == SSM_BF16;
  q.y_f32 = d->y.dtype == SSM_F32;
  q.dsoftplus = (f & SSM_DELTA_SOFTPLUS) ? 1 : 0;
  q.dbias = (f & SSM_HAS_DELTA_BIAS) ? p->delta_bias : nullptr;
  q.dbs_d = (f & SSM_HAS_DELTA_BIAS) ? d->delta_bias.stride[0] : 0;
  return hip_status(ssm::launch_selective_state_update(q, (hipStream_t)hip_stream));
}

}  // extern "C"
