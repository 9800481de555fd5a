/*
 * CPU oracle for the selective state-space scan (S6) and its SSD form.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, fp64 definition the
 * GPU path is checked against.  Only the tests, the smoke check and the
 * bench's CPU-baseline leg may load it.  It shares no code with the GPU path.
 *
 * What it computes, per independent row (one channel of one batch element),
 * following the pages:
 *
 *   Discretisation (tildalice.io "Mamba 논문 리뷰", section 이산화):
 *       Abar = exp(delta * A)
 *       Bbar = (delta*A)^-1 (exp(delta*A) - 1) * delta * B
 *     For a diagonal A this is elementwise: Bbar_n = expm1(delta*a_n) / a_n * B_n,
 *     with the limit delta*B_n when a_n = 0.
 *     The simplified variant Bbar = delta * B (same page, section on the
 *     intuition of delta, and the page's SelectiveSSM listing) is selected by
 *     `euler`.
 *   Recurrence and readout (same page, 이산화 / 연속 시간 SSM):
 *       h_t = Abar_t h_{t-1} + Bbar_t x_t,    h_{-1} = h0 or 0
 *       y_t = C_t . h_t
 *   Skip term (yongggg.tistory.com review, section State Space Model: the
 *   matrix D feeds the input straight to the output):  y_t += D x_t
 *   Gate (tildalice.io, Mamba 블록 아키텍처 and the SelectiveSSM listing:
 *   the scan output is multiplied by SiLU(z)):  y_t *= z_t * sigmoid(z_t)
 *   Optional step-size transform (same listing: delta is the softplus of a
 *   projection, and its delta projection carries a bias):
 *       delta_t <- softplus(delta_t + bias_d),  softplus(v) = log(1 + e^v)
 *
 * The causal depthwise convolution in front of the scan (tildalice.io, Mamba
 * 블록 아키텍처 and the SelectiveSSM listing: a per-channel Conv1D of width k
 * with k - 1 steps of zero padding, cut back to the first L outputs, then
 * SiLU) is oracle_causal_conv1d below.
 *
 * The SSD form (obsidian-dorae222 "Mamba-2", sections on the semiseparable
 * matrix and SSD tiling) is the same recurrence with one scalar A per head:
 * row (b, h, p) scans x[b,:,h,p] with delta[b,:,h], A[h] and the B, C of the
 * head's group.  The oracle computes it as exactly that expanded scan.
 *
 * All arithmetic is fp64 with exp/expm1 from libm.  Inputs stored as bf16, fp32
 * or fp64 are widened exactly.  Rows are independent and are spread over threads.
 *
 * `mutation` (tests only) plants a deliberate mistake so that the tests can
 * show their pins catch it; 0 means the definition above.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Read element i of an input stored as float32 (mode 0), bf16 bit patterns
 * (mode 1) or float64 (mode 2). */
static double rd(const void* p, int mode, int64_t i) {
  if (mode == 2) return ((const double*)p)[i];
  return mode ? bf16_to_double(((const uint16_t*)p)[i]) : (double)((const float*)p)[i];
}

/* log(1 + e^v) without overflow or cancellation. */
static double softplus(double v) { return v > 0 ? v + log1p(exp(-v)) : log1p(exp(v)); }

/* One row of the scan.  All offsets/strides are in elements. */
typedef struct {
  int64_t L, N;
  int io_mode, euler, mutation;
  const void *x, *delta, *B, *C, *z;   /* io dtype */
  const float *A, *Dskip;              /* fp32 */
  const float* dbias;                  /* delta bias (fp32), used with dsoftplus */
  int dsoftplus;                       /* delta <- softplus(delta + dbias) */
  const double* h0;                    /* fp64, may be null */
  int64_t x_off, x_st;                 /* x[t] = x[x_off + t*x_st], same for z */
  int64_t d_off, d_st;                 /* delta[t] */
  int64_t bc_off, bc_st;               /* B[t][n] = B[bc_off + t*bc_st + n], same for C */
  int64_t a_off, a_st;                 /* A[n] = A[a_off + n*a_st] */
  int64_t D_off;                       /* Dskip[D_off] */
  double* y;                           /* y[t], contiguous, length L */
  double* h_last;                      /* length N, may be null */
} row_t;

static void scan_row(const row_t* r, double* h) {
  const int64_t N = r->N;
  for (int64_t n = 0; n < N; ++n) h[n] = r->h0 ? r->h0[n] : 0.0;
  for (int64_t t = 0; t < r->L; ++t) {
    int64_t tx = r->x_off + t * r->x_st;
    if (r->mutation == 4 && t > 0) tx -= r->x_st;          /* off-by-one in time */
    double xt = rd(r->x, r->io_mode, tx);
    double dt = rd(r->delta, r->io_mode, r->d_off + t * r->d_st);
    if (r->dsoftplus) dt = softplus(dt + (r->dbias ? (double)r->dbias[r->D_off] : 0.0));
    double y = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      double a = (double)r->A[r->a_off + n * r->a_st];
      int64_t ib = r->bc_off + t * r->bc_st + n;
      double Bn = rd(r->B, r->io_mode, ib);
      double Cn = rd(r->C, r->io_mode, ib);
      if (r->mutation == 3) { double tmp = Bn; Bn = Cn; Cn = tmp; }   /* B and C swapped */
      double u = dt * a;
      if (r->mutation == 2) u = -u;                                  /* sign of the exponent */
      double Abar = exp(u);
      double Bbar;
      if (r->euler || r->mutation == 5) Bbar = dt * Bn;              /* mutation 5: Euler instead of ZOH */
      else Bbar = (a != 0.0 ? expm1(u) / a : dt) * Bn;
      h[n] = Abar * h[n] + Bbar * xt;
      if (r->mutation == 6 && n + 1 < N) y += Cn * h[n + 1];         /* wrong state index */
      else y += Cn * h[n];
    }
    if (r->Dskip && r->mutation != 1) y += (double)r->Dskip[r->D_off] * xt;   /* mutation 1: skip dropped */
    if (r->z) {
      double zt = rd(r->z, r->io_mode, tx);
      double g = zt / (1.0 + exp(-zt));
      if (r->mutation == 7) g = 1.0 / (1.0 + exp(-zt));            /* sigmoid instead of SiLU */
      y *= g;
    }
    r->y[t] = y;
  }
  if (r->h_last)
    for (int64_t n = 0; n < N; ++n) r->h_last[n] = h[n];
}

/* ---------------------------------------------------------------- threads */

typedef struct {
  int kind; /* 0 scan, 1 ssd */
  /* shapes */
  int64_t batch, L, D, N;            /* scan: D channels; ssd: D = H*P      */
  int64_t H, P, G;                   /* ssd only                             */
  int io_mode, euler, mutation;
  const void *x, *delta, *B, *C, *z;
  const float *A, *Dskip;
  const float* dbias;
  int dsoftplus;
  const double* h0;
  const int64_t* rows;               /* flat row ids: b*D + d                */
  int64_t nrows;
  double *y, *h_last;                /* y: (nrows, L); h_last: (nrows, N)    */
  int64_t next;                      /* work counter                         */
  pthread_mutex_t mu;
} problem_t;

static void make_row(const problem_t* p, int64_t r, row_t* rw) {
  int64_t id = p->rows ? p->rows[r] : r;
  int64_t b = id / p->D, d = id % p->D;
  memset(rw, 0, sizeof(*rw));
  rw->L = p->L; rw->N = p->N;
  rw->io_mode = p->io_mode; rw->euler = p->euler; rw->mutation = p->mutation;
  rw->x = p->x; rw->delta = p->delta; rw->B = p->B; rw->C = p->C; rw->z = p->z;
  rw->A = p->A; rw->Dskip = p->Dskip; rw->dbias = p->dbias; rw->dsoftplus = p->dsoftplus;
  rw->h0 = p->h0 ? p->h0 + id * p->N : 0;
  rw->y = p->y + r * p->L;
  rw->h_last = p->h_last ? p->h_last + r * p->N : 0;
  if (p->kind == 0) {
    /* x, delta, z: (batch, L, D); B, C: (batch, L, N); A: (D, N); Dskip: (D) */
    rw->x_off = b * p->L * p->D + d; rw->x_st = p->D;
    rw->d_off = rw->x_off; rw->d_st = p->D;
    rw->bc_off = b * p->L * p->N; rw->bc_st = p->N;
    rw->a_off = d * p->N; rw->a_st = 1;
    rw->D_off = d;
  } else {
    /* x: (batch, L, H, P); delta: (batch, L, H); A: (H); B, C: (batch, L, G, N);
     * Dskip: (H).  Row d = h*P + p; head h reads group h / (H/G). */
    int64_t h = d / p->P, pp = d % p->P, g = h / (p->H / p->G);
    rw->x_off = b * p->L * p->D + d; rw->x_st = p->D;
    rw->d_off = b * p->L * p->H + h; rw->d_st = p->H;
    rw->bc_off = b * p->L * p->G * p->N + g * p->N; rw->bc_st = p->G * p->N;
    rw->a_off = h; rw->a_st = 0;
    rw->D_off = h;
    (void)pp;
  }
}

static void* worker(void* arg) {
  problem_t* p = (problem_t*)arg;
  double hbuf[4096];
  for (;;) {
    pthread_mutex_lock(&p->mu);
    int64_t r = p->next++;
    pthread_mutex_unlock(&p->mu);
    if (r >= p->nrows) break;
    row_t rw;
    make_row(p, r, &rw);
    scan_row(&rw, hbuf);
  }
  return 0;
}

static int run(problem_t* p, int nthreads) {
  if (p->N > 4096 || p->N < 1) return -1;
  pthread_mutex_init(&p->mu, 0);
  p->next = 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  int started = 0;
  for (int i = 1; i < nthreads; ++i) {
    if (pthread_create(&th[started], 0, worker, p)) break;
    ++started;
  }
  worker(p);
  for (int i = 0; i < started; ++i) pthread_join(th[i], 0);
  pthread_mutex_destroy(&p->mu);
  return 0;
}

/*
 * Selective scan.  Contiguous inputs:
 *   x, delta, z: (batch, L, D)   B, C: (batch, L, N)   A: (D, N)   Dskip: (D)
 *   h0: (batch, D, N) fp64 or NULL.  Dskip / z NULL when off.
 * dsoftplus: delta <- softplus(delta + dbias[d]) (dbias (D) fp32 or NULL = 0).
 * rows: flat ids b*D + d to compute (NULL = all batch*D rows, nrows = batch*D).
 * Outputs: y (nrows, L) and h_last (nrows, N) or NULL, fp64.
 */
int oracle_selective_scan(int64_t batch, int64_t L, int64_t D, int64_t N, int io_mode, int euler,
                          const void* x, const void* delta, const float* A, const void* B, const void* C,
                          const float* Dskip, const void* z, const double* h0, const int64_t* rows,
                          int64_t nrows, double* y, double* h_last, int nthreads, int mutation, int dsoftplus,
                          const float* dbias) {
  problem_t p;
  memset(&p, 0, sizeof(p));
  p.kind = 0; p.batch = batch; p.L = L; p.D = D; p.N = N;
  p.io_mode = io_mode; p.euler = euler; p.mutation = mutation;
  p.dsoftplus = dsoftplus; p.dbias = dbias;
  p.x = x; p.delta = delta; p.A = A; p.B = B; p.C = C; p.Dskip = Dskip; p.z = z; p.h0 = h0;
  p.rows = rows; p.nrows = nrows; p.y = y; p.h_last = h_last;
  return run(&p, nthreads);
}

/*
 * SSD as the expanded selective scan.  Contiguous inputs:
 *   x: (batch, L, H, P)  delta: (batch, L, H)  A: (H)  B, C: (batch, L, G, N)
 *   Dskip: (H) or NULL   h0: (batch, H, P, N) fp64 or NULL
 * rows: flat ids b*(H*P) + h*P + p.  Outputs y (nrows, L), h_last (nrows, N).
 */
int oracle_ssd(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int io_mode, int euler,
               const void* x, const void* delta, const float* A, const void* B, const void* C,
               const float* Dskip, const double* h0, const int64_t* rows, int64_t nrows, double* y,
               double* h_last, int nthreads, int mutation) {
  if (G < 1 || H % G) return -1;
  problem_t p;
  memset(&p, 0, sizeof(p));
  p.kind = 1; p.batch = batch; p.L = L; p.D = H * P; p.N = N; p.H = H; p.P = P; p.G = G;
  p.io_mode = io_mode; p.euler = euler; p.mutation = mutation;
  p.x = x; p.delta = delta; p.A = A; p.B = B; p.C = C; p.Dskip = Dskip; p.z = 0; p.h0 = h0;
  p.rows = rows; p.nrows = nrows; p.y = y; p.h_last = h_last;
  return run(&p, nthreads);
}

/*
 * Causal depthwise convolution, per channel d of batch element b:
 *     out[b,t,d] = bias[d] + sum_{k=0}^{W-1} w[d,k] * x[b, t - (W-1) + k, d]
 * with x = 0 before t = 0 (the W - 1 steps of left padding of the page's
 * Conv1D, whose output is cut back to the first L steps), then SiLU if silu:
 * out <- out * sigmoid(out).  x: (batch, L, D) contiguous in the io dtype;
 * w: (D, W) fp32; bias: (D) fp32 or NULL.  out: (batch, L, D) fp64.
 * `mutation` (tests only): 1 taps reversed, 2 window one step late,
 * 3 SiLU replaced by sigmoid.
 */
int oracle_causal_conv1d(int64_t batch, int64_t L, int64_t D, int64_t W, int io_mode, const void* x, const float* w,
                         const float* bias, int silu, double* out, int mutation) {
  if (W < 1) return -1;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t t = 0; t < L; ++t)
      for (int64_t d = 0; d < D; ++d) {
        double acc = bias ? (double)bias[d] : 0.0;
        for (int64_t k = 0; k < W; ++k) {
          int64_t src = t - (W - 1) + k;
          if (mutation == 2) src -= 1;
          if (src < 0) continue;
          double wk = (double)w[d * W + (mutation == 1 ? W - 1 - k : k)];
          acc += wk * rd(x, io_mode, (b * L + src) * D + d);
        }
        if (silu) acc = mutation == 3 ? 1.0 / (1.0 + exp(-acc)) : acc / (1.0 + exp(-acc));
        out[(b * L + t) * D + d] = acc;
      }
  return 0;
}
