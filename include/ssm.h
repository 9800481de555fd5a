/*
 * ssm.h -- C ABI of libssm: the selective state-space scan (S6) and its
 * Mamba-2 SSD chunked form, forward pass, on AMD Instinct MI355X (gfx950).
 *
 * The operations (pages cited by title and section):
 *
 *  Selective scan -- "Mamba 논문 리뷰: 선형 시간복잡도로 Transformer에 도전하는
 *  Selective State Space Model" (tildalice.io), sections 이산화, Selection
 *  Mechanism, 하드웨어 인식 병렬 알고리즘 and the SelectiveSSM listing; the skip
 *  term D from "[yongggg's] Mamba ... (Review)", section State Space Model.
 *  For every batch element b and channel d, with N-wide state h:
 *      u        = delta[b,t,d] * A[d,n]
 *      Abar     = exp(u)
 *      Bbar     = (exp(u) - 1) / A[d,n] * B[b,t,n]     (zero-order hold;
 *                 delta*B[b,t,n] when A[d,n] == 0)
 *               | delta[b,t,d] * B[b,t,n]               (SSM_DISC_EULER)
 *      h[n]     = Abar * h[n] + Bbar * x[b,t,d]          h starts at h0 or 0
 *      y[b,t,d] = (sum_n C[b,t,n] h[n] + D[d] x[b,t,d]) * silu(z[b,t,d])
 *  silu(v) = v / (1 + exp(-v)).  D and z are optional (SSM_HAS_D, SSM_HAS_Z).
 *  delta is taken as given (already positive); A is real, normally negative.
 *
 *  SSD -- "Mamba-2: 상태 공간 기반 시퀀스 모델" (obsidian-dorae222), sections
 *  1-세미분리 행렬, SSM-Attention 동치성 and SSD 타일링 알고리즘: the same
 *  recurrence with one scalar A per head, computed by chunks of `chunk` steps:
 *  inside a chunk y = (L o C B^T)(beta x) (L the decay mask), across chunks the
 *  state is passed on; every channel (h, p) of head h shares delta[b,t,h],
 *  A[h] and the B, C of the head's group g = h / (nheads / ngroups).
 *
 * Conventions
 *  - Shapes are outermost first; strides are in ELEMENTS and must be >= 0
 *    (0 = broadcast).  Unless stated, the innermost dimension of x, delta, z,
 *    y must have stride 1 (SSM_ERR_STRIDE otherwise).
 *  - Ownership: the caller owns every buffer, the workspace included.  The
 *    library never allocates, frees, retains pointers or synchronises.  Work
 *    is enqueued on `hip_stream` (a hipStream_t, NULL = default stream) and
 *    the call returns at once; buffers must stay alive until the stream has
 *    run it.  Descriptors are read during the call only.
 *  - Errors: every entry point returns an ssm_status.  All checks except
 *    SSM_ERR_HIP happen on the host before any HIP call, so a rejected call
 *    has no side effects.  Values are never inspected: NaN/Inf propagate.
 *  - Thread safety: no mutable global state; calls may come from any thread
 *    (except ssm_selective_scan_fwd_noalloc, whose device scratch is shared by
 *    all calls on one GPU).
 */
#ifndef SSM_H
#define SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 5
#define SSM_MAX_DIMS 5
#define SSM_SCAN_MAX_DSTATE 64 /* selective scan: N <= 64 */

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL = 1,        /* a required pointer is NULL                       */
  SSM_ERR_SHAPE = 2,       /* sizes <= 0 or tensor shape != required shape    */
  SSM_ERR_DTYPE = 3,       /* dtype not allowed for that tensor                */
  SSM_ERR_STRIDE = 4,      /* negative stride, or innermost stride != 1       */
  SSM_ERR_ALIGN = 5,       /* base pointer not aligned to its element size    */
  SSM_ERR_ALIAS = 6,       /* an output overlaps an input or another output   */
  SSM_ERR_UNSUPPORTED = 7, /* valid but not implemented (e.g. N > 64)         */
  SSM_ERR_WORKSPACE = 8,   /* workspace NULL or smaller than required         */
  SSM_ERR_HIP = 9          /* a HIP call failed; see ssm_last_hip_error()     */
} ssm_status;

typedef enum { SSM_F32 = 0, SSM_BF16 = 1, SSM_F16 = 2 /* reserved */ } ssm_dtype;

typedef struct {
  int32_t dtype; /* ssm_dtype */
  int32_t ndim;
  int64_t shape[SSM_MAX_DIMS];
  int64_t stride[SSM_MAX_DIMS]; /* elements */
} ssm_tensor_desc;

/* descriptor flags */
#define SSM_HAS_Z 1u       /* gate y by silu(z)               (scan, decode) */
#define SSM_HAS_D 2u       /* add D * x                                       */
#define SSM_DISC_EULER 4u  /* Bbar = delta * B instead of zero-order hold     */
#define SSM_HAS_H0 8u      /* start from h0 instead of 0                      */
#define SSM_WANT_HLAST 16u /* write the final state to h_last                 */
#define SSM_DELTA_SOFTPLUS 32u /* delta <- softplus(delta [+ delta_bias[d]])  (scan, decode) */
#define SSM_HAS_DELTA_BIAS 64u /* with SSM_DELTA_SOFTPLUS: add delta_bias first (scan, decode) */
#define SSM_HAS_BIAS 128u      /* conv: add bias[d]                                   */
#define SSM_SILU 256u          /* conv: apply SiLU to the output                      */
#define SSM_WANT_CKPT 512u     /* scan: also write the state before every 16-step tile */
#define SSM_HAS_CKPT 1024u     /* scan backward: read those states, do not recompute them */
#define SSM_HAS_SSD_FWD 2048u  /* SSD backward: read the forward's A_cum, beta and chunk states */

/* ------------------------------------------------------------------ scan */

/* Selective scan problem.  Required tensors (shape, dtype):
 *   x, delta : (batch, seqlen, dim)  io          innermost stride 1
 *   z        : (batch, seqlen, dim)  io          if SSM_HAS_Z, innermost stride 1
 *   y        : (batch, seqlen, dim)  io or F32   innermost stride 1
 *   B, C     : (batch, seqlen, dstate) io        any strides
 *   A        : (dim, dstate)  F32                any strides (0 = shared)
 *   D        : (dim)          F32                if SSM_HAS_D, any stride
 *   h0       : (batch, dim, dstate) F32 contiguous   if SSM_HAS_H0
 *   h_last   : (batch, dim, dstate) F32 contiguous   if SSM_WANT_HLAST
 *   delta_bias: (dim)         F32                if SSM_HAS_DELTA_BIAS, any stride
 *   ckpt     : (batch, ceil(seqlen/16), dim, dstate) F32 contiguous   if SSM_WANT_CKPT:
 *              ckpt[b, k] = the state before step 16k (h0 or 0 for k = 0) --
 *              the checkpoints ssm_selective_scan_bwd takes with SSM_HAS_CKPT,
 *              so that a training step's backward need not rerun the recurrence
 * io is SSM_F32 or SSM_BF16 and is the same for x, delta, z, B, C.
 * SSM_DELTA_SOFTPLUS: the step size used is softplus(delta + delta_bias[d])
 * (softplus(v) = log(1 + e^v); delta_bias taken as 0 without
 * SSM_HAS_DELTA_BIAS) -- the Mamba block computes delta as the softplus of a
 * projection with a bias ("Mamba 논문 리뷰", tildalice.io, SelectiveSSM
 * listing).
 * Descriptors of tensors a flag turns off are ignored.
 * Limit: for x, delta, z, y, (16 * stride[1] + 16 * stride[2]) elements, and
 * for B, C, (16 * stride[1] + dstate * stride[2]) elements, must span less
 * than 2 GiB (SSM_ERR_UNSUPPORTED otherwise). */
typedef struct {
  int64_t batch, seqlen, dim, dstate;
  uint32_t flags;
  ssm_tensor_desc x, delta, A, B, C, D, z, y, h0, h_last, delta_bias, ckpt;
} ssm_scan_desc;

typedef struct {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;   /* NULL unless SSM_HAS_D      */
  const void* z;    /* NULL unless SSM_HAS_Z      */
  void* y;
  const float* h0;  /* NULL unless SSM_HAS_H0     */
  float* h_last;    /* NULL unless SSM_WANT_HLAST */
  const float* delta_bias; /* NULL unless SSM_HAS_DELTA_BIAS */
  float* ckpt;             /* NULL unless SSM_WANT_CKPT      */
} ssm_scan_ptrs;

/* -------------------------------------------------------- scan backward */

/* Backward of the selective scan with recomputation ("Mamba 논문 리뷰",
 * tildalice.io, 하드웨어 인식 병렬 알고리즘 / 역전파 시 재계산: the states are not
 * kept from the forward pass; the backward recomputes them).  Given the
 * forward inputs and dy = dLoss/dy it writes the gradients of every input:
 *   g_t   = dy_t silu(z_t) (dy_t without SSM_HAS_Z), dz_t = dy_t o_t silu'(z_t)
 *           with o_t = C_t.h_t + D x_t
 *   lam_t = C_t g_t + Abar_{t+1} lam_{t+1}        (adjoint of h_t, lam past the end = 0)
 *   dx_t  = D g_t + sum_n lam_t Bbar_t;   dB_t += lam_t cbar_t x_t;   dC_t += g_t h_t
 *   ddelta_t, dA: through Abar = exp(delta A) and Bbar = cbar B (cbar =
 *   expm1(delta A)/A, or delta with SSM_DISC_EULER); dD += g_t x_t;
 *   dh0 = Abar_0 lam_0; with SSM_DELTA_SOFTPLUS ddelta is taken through the
 *   softplus (ddelta_in = ddelta * sigmoid(delta_in + bias)) and ddelta_bias
 *   sums it over batch and time.
 * Tensors (shape, dtype):
 *   x, delta, z, h0, delta_bias, A, B, C, D : as in ssm_scan_desc
 *   dy          : (batch, seqlen, dim)  io or F32   innermost stride 1
 *   dx, ddelta  : (batch, seqlen, dim)  io or F32   innermost stride 1
 *   dz          : (batch, seqlen, dim)  io or F32   if SSM_HAS_Z, innermost stride 1
 *   dA          : (dim, dstate) F32 contiguous
 *   dB, dC      : (batch, seqlen, dstate) F32 contiguous
 *   dD          : (dim) F32 contiguous  if SSM_HAS_D
 *   dh0         : (batch, dim, dstate) F32 contiguous   if SSM_HAS_H0
 *   ddelta_bias : (dim) F32 contiguous  if SSM_HAS_DELTA_BIAS
 *   ckpt        : (batch, ceil(seqlen/16), dim, dstate) F32 contiguous  if SSM_HAS_CKPT:
 *                 the forward's checkpoints (SSM_WANT_CKPT) of the same inputs;
 *                 read only; without the flag they are recomputed in the workspace
 * Flags as in the forward except SSM_WANT_HLAST and SSM_WANT_CKPT (not
 * accepted), plus SSM_HAS_CKPT.  The sums
 * over channels (dB, dC) and over batch and time (dA, dD, ddelta_bias) are
 * formed from per-workgroup fp32 partial sums added in a fixed order, so the
 * results are deterministic.  Outputs may not overlap inputs or each other.
 * Workspace: ssm_selective_scan_bwd_workspace_size bytes (the state at every
 * 16th step and the partial sums), 256-byte aligned.
 * Limit: the forward's span limit, applied to x, delta, z, dy, B and C. */
typedef struct {
  int64_t batch, seqlen, dim, dstate;
  uint32_t flags;
  ssm_tensor_desc x, delta, A, B, C, D, z, h0, delta_bias, dy;
  ssm_tensor_desc dx, ddelta, dz, dA, dB, dC, dD, dh0, ddelta_bias, ckpt;
} ssm_scan_bwd_desc;

typedef struct {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;          /* NULL unless SSM_HAS_D          */
  const void* z;           /* NULL unless SSM_HAS_Z          */
  const float* h0;         /* NULL unless SSM_HAS_H0         */
  const float* delta_bias; /* NULL unless SSM_HAS_DELTA_BIAS */
  const void* dy;
  void* dx;
  void* ddelta;
  void* dz;                /* NULL unless SSM_HAS_Z          */
  float* dA;
  float* dB;
  float* dC;
  float* dD;               /* NULL unless SSM_HAS_D          */
  float* dh0;              /* NULL unless SSM_HAS_H0         */
  float* ddelta_bias;      /* NULL unless SSM_HAS_DELTA_BIAS */
  const float* ckpt;       /* NULL unless SSM_HAS_CKPT       */
} ssm_scan_bwd_ptrs;

/* ------------------------------------------------------------------- SSD */

/* SSD problem.  Required tensors (shape, dtype), all innermost stride 1:
 *   x, y     : (batch, seqlen, nheads, headdim)   BF16 (y may be F32)
 *   delta    : (batch, seqlen, nheads)            BF16
 *   B, C     : (batch, seqlen, ngroups, dstate)   BF16
 *   A        : (nheads)  F32, any stride
 *   D        : (nheads)  F32, any stride          if SSM_HAS_D (one skip weight per head)
 *   h0       : (batch, nheads, headdim, dstate) F32 contiguous  if SSM_HAS_H0
 *   h_last   : (batch, nheads, headdim, dstate) F32 contiguous  if SSM_WANT_HLAST
 * Supported: headdim == 64, dstate in {64, 128, 256}, chunk in {64, 128,
 * 256} except dstate 256 with chunk 256 (its staging exceeds the LDS),
 * nheads % ngroups == 0; seqlen need not be a multiple of chunk (the last
 * chunk is shorter).  SSM_HAS_Z is not accepted.  Every (batch, step, head or
 * group) row of x, B, C and y, and h0 / h_last, must start 16-byte aligned
 * (SSM_ERR_ALIGN otherwise). */
typedef struct {
  int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
  uint32_t flags;
  ssm_tensor_desc x, delta, A, B, C, D, y, h0, h_last;
} ssm_ssd_desc;

typedef struct {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;  /* NULL unless SSM_HAS_D      */
  void* y;
  const float* h0; /* NULL unless SSM_HAS_H0     */
  float* h_last;   /* NULL unless SSM_WANT_HLAST */
} ssm_ssd_ptrs;

/* ---------------------------------------------------------- SSD backward */

/* Backward of the SSD ("Mamba-2: 상태 공간 기반 시퀀스 모델", obsidian-dorae222,
 * SSD 타일링 알고리즘, each chunked step differentiated).  Given the forward
 * inputs and dy = dLoss/dy it writes the gradients of x, delta, A, B, C, D
 * and h0 (no gradient flows in through the final state).  With A_cum, beta,
 * S_in as in the forward steps below, decay_ij = exp(A_cum_i - A_cum_j) for
 * j <= i in a chunk, w_j = exp(A_cum_end - A_cum_j) and, per (batch, head),
 *   G[c]     = sum_{i in c} exp(A_cum_i) dy_i C_i^T + exp(A_cum_end[c]) G[c+1]
 *              (G past the last chunk = 0; G[0] = dh0; G[c+1] is the gradient
 *              of chunk c's own state, dS_loc)
 *   dC_i     = sum_j decay_ij beta_j (dy_i . x_j) B_j + exp(A_cum_i) S_in^T dy_i
 *   R_j      = sum_i decay_ij (C_i . B_j) dy_i + w_j dS_loc B_j
 *   dx_j     = beta_j R_j + D dy_j;   dbeta_j = x_j . R_j
 *   dB_j     = sum_i decay_ij beta_j (dy_i . x_j) C_i + w_j beta_j dS_loc^T x_j
 *   dA_cum_i = sum_j W_ij - sum_k W_ki + exp(A_cum_i) C_i . (S_in^T dy_i) - T_i
 *              with W_ij = decay_ij beta_j (dy_i . x_j)(C_i . B_j) and
 *              T_i = w_i beta_i x_i . (dS_loc B_i), plus at the chunk end
 *              sum_j T_j + exp(A_cum_end) <S_in, G[c+1]>
 *   da       = reverse cumulative sum of dA_cum inside each chunk
 *   ddelta   = A da + dbeta dbeta/ddelta,  dA = sum (delta da + dbeta dbeta/dA)
 *   dD       = sum dy . x;  dB, dC summed over the heads of each group.
 * Tensors (shape, dtype):
 *   x, delta, A, B, C, D, h0 : as in ssm_ssd_desc (SSM_HAS_D, SSM_HAS_H0)
 *   dy     : (batch, seqlen, nheads, headdim) BF16, innermost stride 1
 *   dx     : (batch, seqlen, nheads, headdim) BF16 or F32, innermost stride 1
 *   ddelta : (batch, seqlen, nheads) F32, innermost stride 1
 *   dA     : (nheads) F32 contiguous
 *   dB, dC : (batch, seqlen, ngroups, dstate) F32 contiguous
 *   dD     : (nheads) F32 contiguous                          if SSM_HAS_D
 *   dh0    : (batch, nheads, headdim, dstate) F32 contiguous  if SSM_HAS_H0
 * Flags: SSM_HAS_D, SSM_DISC_EULER, SSM_HAS_H0, SSM_HAS_SSD_FWD.  Supported: as the forward
 * (headdim 64, dstate in {64, 128, 256}, chunk in {64, 128, 256} except
 * dstate 256 with chunk 256, nheads % ngroups == 0).  Every (batch,
 * step, head or group) row of x, dy, B, C and dx, and h0 / dh0, must start
 * 16-byte aligned (SSM_ERR_ALIGN otherwise), and chunk x the step stride of
 * x and of dy must stay below 2^30 elements (SSM_ERR_UNSUPPORTED otherwise).
 * The sums over heads (dB, dC)
 * and over batch and time (dA, dD) are fixed-order sums of per-workgroup
 * partial sums, so the results are deterministic.  Outputs may not overlap
 * inputs or each other.  Workspace: ssm_ssd_bwd_workspace_size bytes
 * (the recomputed forward intermediates and the partial sums), 256-byte
 * aligned.
 * With SSM_HAS_SSD_FWD the caller passes A_cum, beta and states as written
 * by ssm_ssd_chunk_cumsum and ssm_ssd_chunk_state on the same inputs (layouts
 * below ssm_ssd_chunk_fwd; contiguous, 16-byte aligned, read only): the
 * backward then skips those two steps, and its workspace drops their space.
 * A training step that ran the four forward steps keeps them for this. */
typedef struct {
  int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
  uint32_t flags;
  ssm_tensor_desc x, delta, A, B, C, D, h0, dy;
  ssm_tensor_desc dx, ddelta, dA, dB, dC, dD, dh0;
} ssm_ssd_bwd_desc;

typedef struct {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;   /* NULL unless SSM_HAS_D  */
  const float* h0;  /* NULL unless SSM_HAS_H0 */
  const void* dy;
  void* dx;
  float* ddelta;
  float* dA;
  float* dB;
  float* dC;
  float* dD;        /* NULL unless SSM_HAS_D  */
  float* dh0;       /* NULL unless SSM_HAS_H0 */
  const float* A_cum;  /* NULL unless SSM_HAS_SSD_FWD */
  const float* beta;   /* NULL unless SSM_HAS_SSD_FWD */
  const float* states; /* NULL unless SSM_HAS_SSD_FWD */
} ssm_ssd_bwd_ptrs;

/* ---------------------------------------------------------------- decode */

/* One recurrent step (autoregressive decode): the recurrent mode of the
 * discretised SSM ("Mamba 논문 리뷰 ...", tildalice.io, sections SSM의 이중 연산
 * 모드, 추론 속도 and Mamba의 강점 / 고정 크기 상태로 효율적 추론: generation
 * keeps only the fixed (dim x dstate) state).  For every batch element b and
 * channel d,
 *      state[b,d,n] <- Abar * state[b,d,n] + Bbar * x[b,d]      (in place)
 *      y[b,d]        = (sum_n C[b,n] state[b,d,n] + D[d] x[b,d]) * silu(z[b,d])
 * with Abar, Bbar as in the selective scan (delta[b,d], A[d,n], B[b,n]); it
 * equals ssm_selective_scan_fwd with seqlen 1, h0 = h_last = state.
 * Required tensors (shape, dtype):
 *   x, delta : (batch, dim)  io           innermost stride 1
 *   z        : (batch, dim)  io           if SSM_HAS_Z, innermost stride 1
 *   y        : (batch, dim)  io or F32    innermost stride 1
 *   B, C     : (batch, dstate) io         any strides
 *   A        : (dim, dstate) F32          any strides (0 = shared)
 *   D        : (dim) F32                  if SSM_HAS_D, any stride
 *   state    : (batch, dim, dstate) F32 contiguous, read and overwritten
 *   delta_bias: (dim) F32                 if SSM_HAS_DELTA_BIAS, any stride
 * Flags: SSM_HAS_Z, SSM_HAS_D, SSM_DISC_EULER, SSM_DELTA_SOFTPLUS,
 * SSM_HAS_DELTA_BIAS (as in the scan); SSM_HAS_H0 / SSM_WANT_HLAST are not
 * accepted: the state is both.  y and state may not overlap each
 * other or any input.  dstate <= SSM_SCAN_MAX_DSTATE. */
typedef struct {
  int64_t batch, dim, dstate;
  uint32_t flags;
  ssm_tensor_desc x, delta, A, B, C, D, z, y, state, delta_bias;
} ssm_update_desc;

typedef struct {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;  /* NULL unless SSM_HAS_D */
  const void* z;   /* NULL unless SSM_HAS_Z */
  void* y;
  float* state;
  const float* delta_bias; /* NULL unless SSM_HAS_DELTA_BIAS */
} ssm_update_ptrs;

/* ------------------------------------------------------------------ conv */

/* Causal depthwise convolution in front of the scan: the Mamba block's
 * per-channel Conv1D of width k with k - 1 steps of zero padding, cut back to
 * the first seqlen outputs, then SiLU ("Mamba 논문 리뷰", tildalice.io, Mamba
 * 블록 아키텍처 and the SelectiveSSM listing).  For every b, t, d:
 *     y[b,t,d] = bias[d] + sum_{k=0}^{width-1} weight[d,k] * x[b, t-width+1+k, d]
 * with x = 0 before t = 0; then y <- y * sigmoid(y) if SSM_SILU.
 * Required tensors (shape, dtype):
 *   x      : (batch, seqlen, dim)  io (F32 or BF16)   innermost stride 1
 *   y      : (batch, seqlen, dim)  io or F32           innermost stride 1
 *   weight : (dim, width) F32                          any strides
 *   bias   : (dim) F32            if SSM_HAS_BIAS,     any stride
 * Flags: SSM_HAS_BIAS, SSM_SILU.  1 <= width <= 8.  y may not overlap x
 * (the convolution is not computed in place) nor the weights.
 * Limit: 160 * max(x.stride[1], y.stride[1]) + 4096 must be below 2^29
 * (SSM_ERR_UNSUPPORTED otherwise). */
typedef struct {
  int64_t batch, seqlen, dim, width;
  uint32_t flags;
  ssm_tensor_desc x, weight, bias, y;
} ssm_conv_desc;

typedef struct {
  const void* x;
  const float* weight;
  const float* bias; /* NULL unless SSM_HAS_BIAS */
  void* y;
} ssm_conv_ptrs;

/* --------------------------------------------------------------- entries */

/* SSM_ABI_VERSION of the library that is loaded. */
int ssm_abi_version(void);

/* Static text for a status code (never NULL). */
const char* ssm_status_string(ssm_status s);

/* hipError_t of the last SSM_ERR_HIP returned on this thread (0 if none). */
int ssm_last_hip_error(void);

/* Bytes of device workspace ssm_selective_scan_fwd needs for `d` (may be 0).
 * Depends only on the descriptor. */
ssm_status ssm_selective_scan_workspace_size(const ssm_scan_desc* d, size_t* bytes);

/* Selective scan forward (definition at the top of this file).  `workspace`
 * is device memory of at least the queried size, 256-byte aligned (may be
 * NULL when the size is 0); its contents need not be initialised and are
 * overwritten.  Outputs: y, and h_last if SSM_WANT_HLAST. */
ssm_status ssm_selective_scan_fwd(const ssm_scan_desc* d, const ssm_scan_ptrs* p, void* workspace,
                                  size_t workspace_bytes, void* hip_stream);

/* Largest workspace (bytes) ssm_selective_scan_fwd_noalloc can serve. */
#define SSM_SCAN_STATIC_SCRATCH_BYTES ((size_t)4 << 20)

/* ssm_selective_scan_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the workspace taken from a
 * static device array of SSM_SCAN_STATIC_SCRATCH_BYTES that the library holds
 * on each GPU it runs on until the process ends.  The caller still passes
 * every input and output.  Never allocates or frees.
 *  - Returns SSM_ERR_WORKSPACE, before any HIP call, when the workspace that
 *    ssm_selective_scan_workspace_size reports for `d` exceeds
 *    SSM_SCAN_STATIC_SCRATCH_BYTES (long, narrow problems whose sequence is
 *    cut into many segments); other errors as ssm_selective_scan_fwd.
 *  - The first call on a device looks up the array's device address (one
 *    hipGetSymbolAddress, with that device current).
 *  - Every call on a GPU shares that GPU's array: calls that overlap on one
 *    GPU (different streams, or threads) race and must be serialised by the
 *    caller.  Nothing in the array needs clearing between calls. */
ssm_status ssm_selective_scan_fwd_noalloc(const ssm_scan_desc* d, const ssm_scan_ptrs* p, void* hip_stream);

/* Bytes of device workspace ssm_ssd_chunk_fwd needs for `d`. */
ssm_status ssm_ssd_chunk_workspace_size(const ssm_ssd_desc* d, size_t* bytes);

/* SSD forward: the four steps below in order on `hip_stream`, with their
 * intermediates placed in `workspace` (256-byte aligned). */
ssm_status ssm_ssd_chunk_fwd(const ssm_ssd_desc* d, const ssm_ssd_ptrs* p, void* workspace, size_t workspace_bytes,
                             void* hip_stream);

/* The four SSD steps, each one kernel launch, exposed so that each can be
 * checked and timed on its own.  nchunks = ceil(seqlen / chunk); Lp =
 * nchunks * chunk.  Intermediates are contiguous device buffers, 16-byte
 * aligned (SSM_ERR_ALIGN otherwise):
 *   A_cum  : (batch, nheads, Lp) F32  -- inclusive cumulative sum of
 *            delta*A inside each chunk (entries past seqlen unspecified)
 *   beta   : (batch, nheads, Lp) F32  -- expm1(delta*A)/A (delta if A == 0),
 *            or delta with SSM_DISC_EULER
 *   states : (batch, nchunks, nheads, headdim, dstate) F32 -- state each
 *            chunk builds from zero: sum_j exp(A_cum_end - A_cum_j) beta_j x_j B_j^T
 *   S_in   : (batch, nchunks, nheads, headdim, dstate) BF16 -- state entering
 *            each chunk, rounded to bf16 as the chunk-scan operand
 * Step 1 (s1): A_cum, beta from delta and A.
 * Step 2 (s2): states from x, B, A_cum, beta (bf16 matrix cores, fp32 sums).
 * Step 3 (s3): S_in[0] = h0 or 0; S_in[c+1] = exp(A_cum_end[c]) S_in[c] + states[c]
 *              (fp32 recurrence); h_last if SSM_WANT_HLAST.
 * Step 4 (s4): y = (L o C B^T)(beta x) + diag(exp(A_cum)) C S_in^T + D x
 *              with L_ij = exp(A_cum_i - A_cum_j) for j <= i, else 0. */
ssm_status ssm_ssd_chunk_cumsum(const ssm_ssd_desc* d, const ssm_ssd_ptrs* p, float* A_cum, float* beta,
                                void* hip_stream);
ssm_status ssm_ssd_chunk_state(const ssm_ssd_desc* d, const ssm_ssd_ptrs* p, const float* A_cum,
                               const float* beta, float* states, void* hip_stream);
ssm_status ssm_ssd_state_passing(const ssm_ssd_desc* d, const ssm_ssd_ptrs* p, const float* A_cum,
                                 const float* states, void* S_in, void* hip_stream);
ssm_status ssm_ssd_chunk_scan(const ssm_ssd_desc* d, const ssm_ssd_ptrs* p, const float* A_cum, const float* beta,
                              const void* S_in, void* hip_stream);

/* One decode step (definition above ssm_update_desc).  No workspace. */
ssm_status ssm_selective_state_update(const ssm_update_desc* d, const ssm_update_ptrs* p, void* hip_stream);

/* Workspace bytes for ssm_selective_scan_bwd. */
ssm_status ssm_selective_scan_bwd_workspace_size(const ssm_scan_bwd_desc* d, size_t* bytes);

/* Backward of the selective scan (definition above ssm_scan_bwd_desc). */
ssm_status ssm_selective_scan_bwd(const ssm_scan_bwd_desc* d, const ssm_scan_bwd_ptrs* p, void* workspace,
                                  size_t workspace_bytes, void* hip_stream);

/* Workspace bytes for ssm_ssd_bwd. */
ssm_status ssm_ssd_bwd_workspace_size(const ssm_ssd_bwd_desc* d, size_t* bytes);

/* Backward of the SSD (definition above ssm_ssd_bwd_desc). */
ssm_status ssm_ssd_bwd(const ssm_ssd_bwd_desc* d, const ssm_ssd_bwd_ptrs* p, void* workspace, size_t workspace_bytes,
                       void* hip_stream);

/* Causal depthwise convolution (+ bias, + SiLU) (definition above
 * ssm_conv_desc).  No workspace. */
ssm_status ssm_causal_conv1d_fwd(const ssm_conv_desc* d, const ssm_conv_ptrs* p, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H */
