// Internal declarations shared by the host dispatch (ssm_abi.cpp) and the
// gfx950 kernels (scan_fwd.hip, ssd_fwd.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// ----------------------------------------------------------- selective scan
struct ScanParams {
  const void* x;
  const void* delta;
  const void* z;
  void* y;
  const void* B;
  const void* C;
  const float* A;
  const float* Dskip;
  const float* h0;
  float* h_last;
  int64_t batch, L, D, N;
  // element strides; ys_b = ys_t = 0 makes y one scratch row of D elements
  // that every store lands in (when only the checkpoints are wanted)
  int64_t xs_b, xs_t, ds_b, ds_t, zs_b, zs_t, ys_b, ys_t;
  int64_t Bs_b, Bs_t, Bs_n, Cs_b, Cs_t, Cs_n;
  int64_t As_d, As_n, Ds_d;
  uint32_t flags;
  int io_bf16;  // x, delta, z, B, C are bf16 (1) or fp32 (0)
  int y_f32;    // y stored as fp32 (1) or in the io type (0)
  // Sequence split: segment s covers [s*seg_len, min(L, (s+1)*seg_len)).
  int n_seg;
  int64_t seg_len;
  float* agg_H;  // (batch, n_seg-1, D, N): end state of segment s in the first pass (from 0; segment 0 from h0)
  float* agg_S;  // (batch, n_seg-1, D): sum of delta over segment s
  float* h_in;   // (batch, n_seg, D, N): state entering segment s (s >= 1)
  // Step-size transform: delta <- softplus(delta + dbias[d * dbs_d]) when
  // dsoftplus (dbias may be null: bias 0).
  const float* dbias;
  int64_t dbs_d;
  int dsoftplus;
  // Optional (batch, ceil(L/16), D, N) fp32: the state before every 16-step
  // tile, as the backward's checkpoints (null: not written).
  float* ckpt;
};

// Tiling of the scan kernels (also used by the host planner).
constexpr int kScanLanesPerChannel = 16;
constexpr int kScanChannelsPerBlock = 16;
constexpr int kScanTileSteps = 16;
constexpr int kScanThreads = kScanLanesPerChannel * kScanChannelsPerBlock;

hipError_t launch_selective_scan(const ScanParams& p, hipStream_t stream);

// Device address of the current device's static scan scratch (the workspace
// of the allocation-free scan entry point), looked up once per device.
constexpr size_t kScanStaticScratchBytes = (size_t)4 << 20;
hipError_t scan_static_scratch(void** ptr);

// ------------------------------------------------------------------- decode
struct UpdateParams {
  const void* x;      // (batch, D)
  const void* delta;  // (batch, D)
  const void* z;      // (batch, D) or null
  void* y;            // (batch, D)
  const void* B;      // (batch, N)
  const void* C;
  const float* A;      // (D, N)
  const float* Dskip;  // (D) or null
  float* state;        // (batch, D, N) contiguous
  int64_t batch, D, N;
  int64_t xs_b, ds_b, zs_b, ys_b, Bs_b, Bs_n, Cs_b, Cs_n, As_d, As_n, Ds_d;
  int euler;
  int io_bf16;
  int y_f32;
  const float* dbias;  // delta <- softplus(delta + dbias[d * dbs_d]) when dsoftplus
  int64_t dbs_d;
  int dsoftplus;
};

hipError_t launch_selective_state_update(const UpdateParams& p, hipStream_t stream);

// ------------------------------------------------------------ scan backward
struct ScanBwdParams {
  const void* x;
  const void* delta;
  const void* z;       // or null
  const void* dy;
  const void* B;
  const void* C;
  const float* A;
  const float* Dskip;  // or null
  const float* h0;     // or null
  const float* dbias;  // or null
  void* dx;
  void* ddelta;
  void* dz;            // or null
  float* dA;           // (D, N)
  float* dB;           // (batch, L, N)
  float* dC;
  float* dD;           // or null
  float* dh0;          // or null
  float* ddbias;       // or null
  // workspace
  float* ckpt;         // (batch, ntiles, D, N): state before each 16-step tile
  int ckpt_given;      // the caller supplied ckpt (the forward's): no checkpoint pass
  float* pdB;          // (n_dblk, batch, L, N): sums over each workgroup's channels
  float* pdC;
  float* pdA;          // (batch, n_seg, D, N): sums over each segment's time
  float* pdD;          // (batch, n_seg, D)
  float* pdbias;       // (batch, n_seg, D)
  // Sequence split (n_seg > 1 when batch x channels cannot fill the GPU):
  // segment s covers [s*seg_len, min(L, (s+1)*seg_len)), seg_len a multiple
  // of 16.  The adjoint carried into each segment's last step comes from a
  // pass that runs the adjoint recurrence alone over every later segment.
  int n_seg;
  int64_t seg_len;
  float* cH;           // (batch, n_seg, D, N): carry out of segment s (s >= 1) from a zero carry in
  float* cS;           // (batch, n_seg, D): sum of delta over segment s
  float* cin;          // (batch, n_seg, D, N): carry into segment s at its last step
  int64_t batch, L, D, N;
  int64_t xs_b, xs_t, ds_b, ds_t, zs_b, zs_t, gs_b, gs_t;  // x, delta, z, dy
  int64_t dxs_b, dxs_t, dds_b, dds_t, dzs_b, dzs_t;        // dx, ddelta, dz
  int64_t Bs_b, Bs_t, Bs_n, Cs_b, Cs_t, Cs_n;
  int64_t As_d, As_n, Ds_d, dbs_d;
  int io_bf16;    // x, delta, z, B, C
  int dy_f32;     // dy fp32 (1) or io (0)
  int dx_f32, dd_f32, dz_f32;
  int euler, dsoftplus;
};

hipError_t launch_selective_scan_bwd(const ScanBwdParams& p, hipStream_t stream);

// --------------------------------------------------------------------- conv
struct ConvParams {
  const void* x;       // (batch, L, D), innermost stride 1
  const float* w;      // (D, W)
  const float* bias;   // (D) or null
  void* y;             // (batch, L, D), innermost stride 1
  int64_t batch, L, D, W;
  int64_t xs_b, xs_t, ys_b, ys_t, ws_d, ws_k, bs_d;  // element strides
  int io_bf16;
  int y_f32;
  int silu;
};

constexpr int kConvMaxWidth = 8;

hipError_t launch_causal_conv1d(const ConvParams& p, hipStream_t stream);

// ---------------------------------------------------------------------- SSD
struct SSDParams {
  const void* x;      // (batch, L, H, P) bf16
  const void* delta;  // (batch, L, H) bf16
  const float* A;     // (H)
  const void* B;      // (batch, L, G, N) bf16
  const void* C;
  const float* Dskip;  // (H) or null
  void* y;             // (batch, L, H, P) bf16 or fp32
  const float* h0;     // (batch, H, P, N) or null
  float* h_last;       // (batch, H, P, N) or null
  int64_t batch, L, H, P, N, G, Q, nchunks, Lp;
  int64_t xs_b, xs_t, xs_h;  // x strides (p stride 1)
  int64_t ds_b, ds_t, ds_h;  // delta strides
  int64_t Bs_b, Bs_t, Bs_g, Cs_b, Cs_t, Cs_g;  // B, C strides (n stride 1)
  int64_t ys_b, ys_t, ys_h;
  int64_t As_h, Ds_h;
  int euler;
  int y_f32;
  float* A_cum;   // (batch, H, Lp)
  float* beta;    // (batch, H, Lp)
  float* states;  // (batch, nchunks, H, P, N)
  void* S_in;     // (batch, nchunks, H, P, N) bf16
  // chunk_state weights: 0 = exp(A_cum_end - A_cum_j) beta_j (the chunk's own
  // state), 1 = exp(A_cum_j) (the backward's sum_i exp(A_cum_i) dy_i C_i^T,
  // with x <- dy and B <- C)
  int state_coef;
};

// SSD backward (P = 64, N = 64).  f holds the forward problem and the
// recomputed forward intermediates (A_cum, beta, states).
struct SSDBwdParams {
  SSDParams f;
  const void* dy;  // (batch, L, H, P) bf16
  int64_t dys_b, dys_t, dys_h;
  void* dx;        // (batch, L, H, P) bf16 or fp32
  int64_t dxs_b, dxs_t, dxs_h;
  int dx_f32;
  float* ddelta;   // (batch, L, H) fp32
  int64_t dds_b, dds_t, dds_h;
  float* dh0;      // (batch, H, P, N) or null
  // workspace
  float* dS;       // (batch, nchunks, H, P, N): sum_i exp(A_cum_i) dy_i C_i^T
  float* S32;      // (batch, nchunks, H, P, N): state entering each chunk (more than 32 chunks; else null)
  uint16_t* SinT;  // (batch, nchunks, H) tiles of N x P bf16, the same transposed: [p / 8][n][p % 8]
  uint16_t* dSl;   // (batch, nchunks, H, P, N) bf16: gradient of each chunk's own state
  uint16_t* dSlT;  // (batch, nchunks, H) tiles of N x P bf16, the same transposed: [p / 8][n][p % 8]
  float* pAend;    // (batch, H, nchunks, aend_parts): chunk-end decay gradient, partial sums
  int aend_parts;  // partial sums per (batch, head, chunk): one per workgroup of the state pass
  float* dAcA;     // (batch, H, Lp): row sums of W = E o C B^T, + C_i . (inter-chunk dC_i)
  float* dAcB;     // (batch, H, Lp): -(column sums of W) - T_j
  float* dbeta;    // (batch, H, Lp)
  float* Tj;       // (batch, H, Lp): chunk-state terms of the chunk-end gradient
  float* dDj;      // (batch, H, Lp): dy_i . x_i
  float* pA;       // (batch, nchunks, H) partial dA
  float* pD;       // (batch, nchunks, H) partial dD
  float* pdB;      // (nhb, batch, L, G, N) partial dB per head block
  float* pdC;      // (nhb, batch, L, G, N)
  int HB, nhb;     // heads per workgroup, head blocks per group
};

hipError_t launch_ssd_bwd(const SSDBwdParams& p, float* dA, float* dB, float* dC, float* dD, hipStream_t stream);

// dst[i] = sum_k src[k * stride + i] over k = 0 .. parts-1 in a fixed order
// (deterministic partial-sum reduction).
void launch_fixed_order_sum(const float* src, float* dst, int64_t count, int64_t parts, int64_t stride,
                            hipStream_t stream);

// Heads per workgroup for the SSD kernels whose workgroup takes a block of one
// group's heads in turn (chunk_scan, and the backward's dC and dx passes):
// the count that minimises (rounds of workgroups) x (heads + 1), where `base`
// workgroups share each head block (batch x chunks x groups), `slots`
// workgroups are resident at once, and one head's time stands for a
// workgroup's set-up (staging B and C, its first head's loads, which nothing
// overlaps).  Ties go to fewer workgroups.
inline int ssd_heads_per_block(int64_t hpg, int64_t base, int64_t slots) {
  int64_t best = 1, best_cost = -1;
  for (int64_t hb = 1; hb <= hpg; ++hb) {
    const int64_t nhb = (hpg + hb - 1) / hb;
    const int64_t cost = ((base * nhb + slots - 1) / slots) * (hb + 1);
    if (best_cost < 0 || cost <= best_cost) {
      best_cost = cost;
      best = hb;
    }
  }
  return (int)best;
}

// Rows of the 64 x N state per workgroup of the SSD backward's state pass:
// 8 for the chunk-parallel kernel (up to 32 chunks), 16 for the one that
// walks the chunks.  The pass writes (64 / rows) (N / 64) partial sums of the
// chunk-end decay gradient per (batch, head, chunk).
inline int ssd_bwd_state_rows(int64_t nchunks) { return nchunks <= 32 ? 8 : 16; }

hipError_t launch_ssd_chunk_cumsum(const SSDParams& p, hipStream_t stream);
hipError_t launch_ssd_chunk_state(const SSDParams& p, hipStream_t stream);
hipError_t launch_ssd_state_passing(const SSDParams& p, hipStream_t stream);
hipError_t launch_ssd_chunk_scan(const SSDParams& p, hipStream_t stream);

}  // namespace ssm
