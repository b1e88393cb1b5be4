/*
 * ssm_oracle.c -- plain, sequential, double-precision reference for the
 * selective state-space scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it is used by the tests, by the smoke check and by the CPU
 * baseline leg of the benchmark.  It shares no code, header, table or helper
 * with the HIP library; it has its own bf16 widening and its own softplus.
 *
 * What it computes (sources are the five web pages on state-space models):
 *
 *  - discretization by zero-order hold, Abar = exp(delta*A) elementwise for
 *    a diagonal A, with either the exact ZOH input matrix
 *    Bbar = A^-1 (exp(delta*A) - 1) B  or the simplified Bbar = delta*B
 *    ("State-space models", section "Discretization" (ZOH rule) and the
 *    closing paragraph of "Implementation", which says the official
 *    package uses Bbar = delta*B; "State Space Models: Mamba and Beyond",
 *    section "Discretization: zero-order hold");
 *  - the recurrence h_t = Abar_t h_{t-1} + Bbar_t u_t from h_{-1} = 0 (or a
 *    caller-given h0) and the readout y_t = C_t . h_t + D u_t
 *    ("State-space models", section "Recurrence and convolution";
 *    "Structured State Space Models and Mamba ...", section "Discretization
 *    Mechanics: Zero-Order Hold and Bilinear Transforms");
 *  - selection: delta_t = softplus(raw_t + bias), B_t and C_t shared by all
 *    channels of a sequence, A and delta per channel ("State-space models",
 *    section "Mamba: selection"; "Structured State Space Models and Mamba
 *    ...", section "The Linear Time-Invariance Bottleneck and the Selective
 *    State Space (S6)", the delta_t formula with its bias parameter);
 *  - the block's output gate y * silu(z) ("State-space models", section
 *    "Mamba: selection", paragraph on the Mamba block);
 *  - the time-invariant kernel K_k = C Abar^k Bbar and the causal convolution
 *    y_t = sum_{k<=t} K_k u_{t-k} + D u_t ("State-space models", section
 *    "Recurrence and convolution").
 *
 * The loop is the definition, in time order, one channel at a time.  The
 * only parallelism is over independent channels (b, d), which does not
 * change any channel's arithmetic.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_F64 = 2 };
enum { OR_BBAR_DELTA_B = 0, OR_BBAR_ZOH_EXACT = 1, OR_DISC_EULER = 2, OR_DISC_BILINEAR = 3 };

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double or_widen(const void* p, int dtype, int64_t i) {
  if (dtype == OR_F64) return ((const double*)p)[i];
  if (dtype == OR_F32) return (double)((const float*)p)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* softplus(x) = log(1 + e^x), written in the overflow-free form. */
static double or_softplus(double x) {
  return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

/* silu(z) = z * sigmoid(z). */
static double or_silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * The discretization rules of "State-space models", section
 * "Discretization": zero-order hold (Abar = exp(delta a), with Bbar = delta b
 * as the official package takes it, or the exact A^-1 (exp(delta a) - 1) b),
 * Euler (Abar = 1 + delta a, Bbar = delta b) and bilinear / Tustin
 * (Abar = (1 - delta a/2)^-1 (1 + delta a/2), Bbar = (1 - delta a/2)^-1 delta b);
 * "Structured State Space Models and Mamba ...", section "Discretization
 * Mechanics: Zero-Order Hold and Bilinear Transforms" prints the same
 * bilinear pair.  For a diagonal A each is elementwise.
 */
static double or_abar(double dt, double a, int mode) {
  if (mode == OR_DISC_EULER) return 1.0 + dt * a;
  if (mode == OR_DISC_BILINEAR) return (1.0 + 0.5 * dt * a) / (1.0 - 0.5 * dt * a);
  return exp(dt * a);
}

/* Input coefficient Bbar/B for one (delta, a) pair under the chosen rule. */
static double or_bbar_factor(double dt, double a, int bbar_mode) {
  if (bbar_mode == OR_BBAR_DELTA_B || bbar_mode == OR_DISC_EULER) return dt;
  if (bbar_mode == OR_DISC_BILINEAR) return dt / (1.0 - 0.5 * dt * a);
  /* exact ZOH: (exp(dt*a) - 1) / a, whose limit at a = 0 is dt */
  if (a == 0.0) return dt;
  return expm1(dt * a) / a;
}

/* Channels a worker claims at a time: enough steps per claim that the lock
 * is rare (decode steps are one step each), few enough that the threads
 * stay balanced.  Which thread runs a channel changes no arithmetic. */
static int64_t or_claim_block(int64_t n_channels, int64_t seqlen, int n_threads) {
  int64_t blk = 16384 / (seqlen > 0 ? seqlen : 1);
  const int64_t fair = n_channels / (8 * (int64_t)(n_threads > 0 ? n_threads : 1));
  if (blk > fair) blk = fair;
  return blk < 1 ? 1 : blk;
}

typedef struct {
  int io_dtype;
  const void *u, *delta, *Bm, *Cm, *z;
  const double *A, *Dskip, *delta_bias;
  int delta_softplus, bbar_mode;
  const double* h0;
  int64_t batch, dim, dstate, seqlen;
  const int64_t* channels;
  int64_t n_channels;
  double *y, *final_state;
  /* work distribution */
  int n_threads;
  int64_t next;
  pthread_mutex_t lock;
  int status;
} or_scan_job;

/* The recurrence for one channel c = b*dim + d, written straight from the
 * definition: discretize, update every state, read out, skip, gate. */
static void or_scan_one(const or_scan_job* j, int64_t sel, double* h) {
  const int64_t c = j->channels ? j->channels[sel] : sel;
  const int64_t b = c / j->dim, d = c % j->dim;
  const int64_t N = j->dstate, L = j->seqlen;
  const int64_t row = c * L;            /* u, delta, z: [batch, dim, L] */
  const int64_t bc_base = b * N * L;    /* B, C: [batch, N, L] */
  for (int64_t n = 0; n < N; ++n) h[n] = j->h0 ? j->h0[sel * N + n] : 0.0;
  const double bias = j->delta_bias ? j->delta_bias[d] : 0.0;
  const double Dd = j->Dskip ? j->Dskip[d] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    const double ut = or_widen(j->u, j->io_dtype, row + t);
    const double raw = or_widen(j->delta, j->io_dtype, row + t) + bias;
    const double dt = j->delta_softplus ? or_softplus(raw) : raw;
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double a = j->A[d * N + n];
      const double abar = or_abar(dt, a, j->bbar_mode);
      const double bt = or_widen(j->Bm, j->io_dtype, bc_base + n * L + t);
      const double ct = or_widen(j->Cm, j->io_dtype, bc_base + n * L + t);
      h[n] = abar * h[n] + or_bbar_factor(dt, a, j->bbar_mode) * bt * ut;
      acc += ct * h[n];
    }
    double yt = acc + Dd * ut;
    if (j->z) yt *= or_silu(or_widen(j->z, j->io_dtype, row + t));
    if (j->y) j->y[sel * L + t] = yt;
  }
  if (j->final_state)
    for (int64_t n = 0; n < N; ++n) j->final_state[sel * N + n] = h[n];
}

static void* or_scan_worker(void* arg) {
  or_scan_job* j = (or_scan_job*)arg;
  double* h = (double*)malloc(sizeof(double) * (size_t)j->dstate);
  if (!h) {
    pthread_mutex_lock(&j->lock);
    j->status = 2;
    pthread_mutex_unlock(&j->lock);
    return NULL;
  }
  const int64_t blk = or_claim_block(j->n_channels, j->seqlen, j->n_threads);
  for (;;) {
    pthread_mutex_lock(&j->lock);
    const int64_t first = j->next;
    j->next += blk;
    pthread_mutex_unlock(&j->lock);
    if (first >= j->n_channels) break;
    const int64_t last = first + blk < j->n_channels ? first + blk : j->n_channels;
    for (int64_t sel = first; sel < last; ++sel) or_scan_one(j, sel, h);
  }
  free(h);
  return NULL;
}

/*
 * Selective scan over the channels listed in `channels` (flat index
 * b*dim + d; NULL means all batch*dim channels in order).
 *
 *   u, delta, z : [batch, dim, seqlen]   io_dtype (0 = float32, 1 = bf16 bits)
 *   Bm, Cm      : [batch, dstate, seqlen] io_dtype
 *   A           : [dim, dstate] double
 *   Dskip, delta_bias : [dim] double or NULL (= 0)
 *   z           : NULL = no gate
 *   h0          : [n_channels, dstate] double or NULL (= 0); may equal
 *                 final_state (each channel reads h0 before writing)
 *   y           : [n_channels, seqlen] double out (may be NULL)
 *   final_state : [n_channels, dstate] double out (may be NULL)
 *
 * Returns 0, or 1 on bad arguments, 2 on allocation failure.
 */
int ssm_oracle_selective_scan(int io_dtype, const void* u, const void* delta, const void* Bm,
                              const void* Cm, const void* z, const double* A, const double* Dskip,
                              const double* delta_bias, int delta_softplus, int bbar_mode,
                              const double* h0, int64_t batch, int64_t dim, int64_t dstate,
                              int64_t seqlen, const int64_t* channels, int64_t n_channels,
                              double* y, double* final_state, int n_threads) {
  if (!u || !delta || !Bm || !Cm || !A) return 1;
  if (batch <= 0 || dim <= 0 || dstate <= 0 || seqlen <= 0) return 1;
  if (io_dtype != OR_F32 && io_dtype != OR_BF16 && io_dtype != OR_F64) return 1;
  if (bbar_mode < OR_BBAR_DELTA_B || bbar_mode > OR_DISC_BILINEAR) return 1;
  if (!channels) n_channels = batch * dim;
  for (int64_t i = 0; channels && i < n_channels; ++i)
    if (channels[i] < 0 || channels[i] >= batch * dim) return 1;
  or_scan_job j;
  memset(&j, 0, sizeof j);
  j.io_dtype = io_dtype;
  j.u = u;
  j.delta = delta;
  j.Bm = Bm;
  j.Cm = Cm;
  j.z = z;
  j.A = A;
  j.Dskip = Dskip;
  j.delta_bias = delta_bias;
  j.delta_softplus = delta_softplus;
  j.bbar_mode = bbar_mode;
  j.h0 = h0;
  j.batch = batch;
  j.dim = dim;
  j.dstate = dstate;
  j.seqlen = seqlen;
  j.channels = channels;
  j.n_channels = n_channels;
  j.y = y;
  j.final_state = final_state;
  j.next = 0;
  j.status = 0;
  pthread_mutex_init(&j.lock, NULL);
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  if ((int64_t)n_threads > n_channels) n_threads = (int)n_channels;
  j.n_threads = n_threads;
  pthread_t tid[256];
  int started = 0;
  for (int i = 1; i < n_threads; ++i)
    if (pthread_create(&tid[started], NULL, or_scan_worker, &j) == 0) ++started;
  or_scan_worker(&j);
  for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
  pthread_mutex_destroy(&j.lock);
  return j.status;
}

/*
 * One decode step: the recurrence advanced by a single token per sequence
 * ("State-space models", section "Recurrence and convolution": generation
 * advances the N-dimensional state by one token at constant cost).
 *
 *   state : [n_channels, dstate] double, read and written in place
 *   u, delta, z : [batch, dim] io_dtype;  Bm, Cm : [batch, dstate] io_dtype
 *   y     : [n_channels] double out
 *
 * It is the scan above with seqlen = 1 and h0 = final_state = state.
 */
int ssm_oracle_state_update(int io_dtype, double* state, const void* u, const void* delta,
                            const void* Bm, const void* Cm, const void* z, const double* A,
                            const double* Dskip, const double* delta_bias, int delta_softplus,
                            int bbar_mode, int64_t batch, int64_t dim, int64_t dstate,
                            const int64_t* channels, int64_t n_channels, double* y,
                            int n_threads) {
  if (!state) return 1;
  return ssm_oracle_selective_scan(io_dtype, u, delta, Bm, Cm, z, A, Dskip, delta_bias,
                                   delta_softplus, bbar_mode, state, batch, dim, dstate, 1,
                                   channels, n_channels, y, state, n_threads);
}

/*
 * Time-invariant convolution kernel K[d, k] = sum_n C[d,n] Abar[d,n]^k Bbar[d,n]
 * for k in [0, L) ("State-space models", section "Recurrence and
 * convolution": K_k = C Abar^k Bbar; section "S4: a structured state matrix":
 * with a diagonal A the powers are elementwise).
 *
 *   A : [dim, dstate];  Bv, Cv : rows of length dstate, row d at d*stride
 *   (stride 0 = one row shared by every channel);  delta : [dim]
 *   method 0 : Abar^k directly: exp(k * delta * A) for the exp rules,
 *              pow(Abar, k) for Euler and bilinear
 *   method 1 : Abar^k by repeated multiplication (k successive products)
 *   K : [dim, L] out
 */
int ssm_oracle_lti_kernel(const double* A, const double* Bv, const double* Cv,
                          const double* delta, int64_t dim, int64_t dstate, int64_t L,
                          int64_t b_row_stride, int64_t c_row_stride, int bbar_mode, int method,
                          double* K) {
  if (!A || !Bv || !Cv || !delta || !K || dim <= 0 || dstate <= 0 || L <= 0) return 1;
  if (bbar_mode < OR_BBAR_DELTA_B || bbar_mode > OR_DISC_BILINEAR) return 1;
  for (int64_t d = 0; d < dim; ++d) {
    const double dt = delta[d];
    for (int64_t k = 0; k < L; ++k) K[d * L + k] = 0.0;
    for (int64_t n = 0; n < dstate; ++n) {
      const double a = A[d * dstate + n];
      const double abar = or_abar(dt, a, bbar_mode);
      const double bbar = or_bbar_factor(dt, a, bbar_mode) * Bv[d * b_row_stride + n];
      const double cn = Cv[d * c_row_stride + n];
      double p = 1.0; /* Abar^k for method 1 */
      for (int64_t k = 0; k < L; ++k) {
        const double pk = method == 1 ? p
                          : bbar_mode <= OR_BBAR_ZOH_EXACT ? exp((double)k * dt * a)
                                                           : pow(abar, (double)k);
        K[d * L + k] += cn * pk * bbar;
        p *= abar;
      }
    }
  }
  return 0;
}

/*
 * Causal linear convolution y[t] = sum_{k=0..t} K[k] u[t-k] + D u[t]: the
 * output sees no future input ("State-space models", section "Recurrence and
 * convolution", and the left-padded convolution in "Implementation").
 * Direct O(L^2) sum.
 */
int ssm_oracle_causal_conv(const double* K, const double* u, double Dskip, int64_t L, double* y) {
  if (!K || !u || !y || L <= 0) return 1;
  for (int64_t t = 0; t < L; ++t) {
    double acc = 0.0;
    for (int64_t k = 0; k <= t; ++k) acc += K[k] * u[t - k];
    y[t] = acc + Dskip * u[t];
  }
  return 0;
}

/* ------------------------------------------------------------------ backward
 *
 * Gradients of the selective scan by reverse-mode differentiation of the
 * recurrence above (the backward pass that the fused kernel recomputes the
 * state for: "State-space models", section "The parallel scan").  With
 * g = dL/dy and the final-state gradient dL/dh_{L-1}:
 *
 *   yc_t = C_t . h_t + D u_t,  y_t = yc_t s_t,  s_t = silu(z_t)
 *   dyc_t = g_t s_t,  dz_t = g_t yc_t silu'(z_t)
 *   lambda_t = dyc_t C_t + Abar_{t+1} lambda_{t+1}   (dL/dh_t; the final-state
 *                                                    gradient enters at L-1)
 *   dC_t += dyc_t h_t,  dAbar_t = lambda_t h_{t-1},  dBbar_t = lambda_t B_t u_t
 *   dB_t += lambda_t bbar_t u_t,  du_t = dyc_t D + sum_n lambda_t bbar_t B_t
 *   ddt_t = sum_n [dAbar_t Abar_t A + dBbar_t dbbar/ddt]
 *   dA += dAbar_t Abar_t dt_t + dBbar_t dbbar/dA
 *   draw_t = ddt_t softplus'(raw_t + bias) = ddt_t sigmoid(raw_t + bias)
 *   dh0 = Abar_0 lambda_0
 *
 * For the gradients that are sums over steps or channels (dA, dB, dC, dD,
 * dbias) the oracle can also return, element by element, the sum of the
 * absolute values of the terms written above (ddt expanded into its
 * per-state terms for dbias): the scale against which the rounding of a
 * float32 accumulation of the same terms, in any order, is measured.
 *
 * with bbar = dt (delta*B rule: dbbar/ddt = 1, dbbar/dA = 0) or
 * bbar = (exp(dt A) - 1)/A (exact ZOH: dbbar/ddt = Abar,
 * dbbar/dA = (dt Abar - bbar)/A, limit dt^2/2 at A = 0).
 */

static double or_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

typedef struct {
  int io_dtype;
  const void *u, *delta, *Bm, *Cm, *z;
  const double *A, *Dskip, *delta_bias, *h0, *dy, *dfinal;
  int delta_softplus, bbar_mode;
  int64_t batch, dim, dstate, seqlen;
  const int64_t* channels;
  int64_t n_channels;
  double *du, *ddelta, *dz, *dh0;            /* per selected channel */
  double *dA, *dB, *dC, *dD, *dbias;         /* shared sums (per-thread copies) */
  double *aA, *aB, *aC, *aD, *abias;         /* sums of |term| (optional, all or none) */
  int n_threads;
  int64_t next;
  pthread_mutex_t lock;
  int status;
} or_bwd_job;

typedef struct {
  double *dA, *dB, *dC, *dD, *dbias;
  double *aA, *aB, *aC, *aD, *abias;  /* NULL unless the job asks for them */
} or_bwd_acc;

static void or_bwd_one(const or_bwd_job* j, int64_t sel, double* hs, double* lam, or_bwd_acc* acc) {
  const int64_t c = j->channels ? j->channels[sel] : sel;
  const int64_t b = c / j->dim, d = c % j->dim;
  const int64_t N = j->dstate, L = j->seqlen;
  const int64_t row = c * L, bc_base = b * N * L;
  const double bias = j->delta_bias ? j->delta_bias[d] : 0.0;
  const double Dd = j->Dskip ? j->Dskip[d] : 0.0;
  /* forward: hs[(t + 1) * N + n] = h_t, hs[n] = h_{-1} */
  for (int64_t n = 0; n < N; ++n) hs[n] = j->h0 ? j->h0[sel * N + n] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    const double ut = or_widen(j->u, j->io_dtype, row + t);
    const double raw = or_widen(j->delta, j->io_dtype, row + t) + bias;
    const double dt = j->delta_softplus ? or_softplus(raw) : raw;
    for (int64_t n = 0; n < N; ++n) {
      const double a = j->A[d * N + n];
      const double bt = or_widen(j->Bm, j->io_dtype, bc_base + n * L + t);
      hs[(t + 1) * N + n] =
          exp(dt * a) * hs[t * N + n] + or_bbar_factor(dt, a, j->bbar_mode) * bt * ut;
    }
  }
  /* reverse: lam[n] holds Abar_{t+1} lambda_{t+1} (the final-state gradient at t = L-1) */
  for (int64_t n = 0; n < N; ++n) lam[n] = j->dfinal ? j->dfinal[sel * N + n] : 0.0;
  for (int64_t t = L - 1; t >= 0; --t) {
    const double ut = or_widen(j->u, j->io_dtype, row + t);
    const double raw = or_widen(j->delta, j->io_dtype, row + t) + bias;
    const double dt = j->delta_softplus ? or_softplus(raw) : raw;
    double yc = Dd * ut;
    for (int64_t n = 0; n < N; ++n)
      yc += or_widen(j->Cm, j->io_dtype, bc_base + n * L + t) * hs[(t + 1) * N + n];
    const double g = j->dy[row + t];
    double dyc = g;
    if (j->z) {
      const double zz = or_widen(j->z, j->io_dtype, row + t);
      const double sg = or_sigmoid(zz);
      dyc = g * zz * sg;
      if (j->dz) j->dz[sel * L + t] = g * yc * sg * (1.0 + zz * (1.0 - sg));
    }
    acc->dD[d] += dyc * ut;
    if (acc->aD) acc->aD[d] += fabs(dyc * ut);
    double du = dyc * Dd, ddt = 0.0, addt = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double a = j->A[d * N + n];
      const double abar = exp(dt * a);
      const double bbar = or_bbar_factor(dt, a, j->bbar_mode);
      const double bt = or_widen(j->Bm, j->io_dtype, bc_base + n * L + t);
      const double ct = or_widen(j->Cm, j->io_dtype, bc_base + n * L + t);
      const double l = dyc * ct + lam[n];
      const double dabar = l * hs[t * N + n];
      const double dbbar = l * bt * ut;
      acc->dC[bc_base + n * L + t] += dyc * hs[(t + 1) * N + n];
      acc->dB[bc_base + n * L + t] += l * bbar * ut;
      if (acc->aC) {
        acc->aC[bc_base + n * L + t] += fabs(dyc * hs[(t + 1) * N + n]);
        acc->aB[bc_base + n * L + t] += fabs(l * bbar * ut);
      }
      du += l * bbar * bt;
      double dbbar_ddt, dbbar_dA;
      if (j->bbar_mode == OR_BBAR_DELTA_B) {
        dbbar_ddt = 1.0;
        dbbar_dA = 0.0;
      } else {
        dbbar_ddt = abar;
        dbbar_dA = a != 0.0 ? (dt * abar - bbar) / a : 0.5 * dt * dt;
      }
      ddt += dabar * abar * a + dbbar * dbbar_ddt;
      acc->dA[d * N + n] += dabar * abar * dt + dbbar * dbbar_dA;
      if (acc->aA) {
        addt += fabs(dabar * abar * a) + fabs(dbbar * dbbar_ddt);
        acc->aA[d * N + n] += fabs(dabar * abar * dt) + fabs(dbbar * dbbar_dA);
      }
      lam[n] = abar * l;
    }
    const double dr = j->delta_softplus ? ddt * or_sigmoid(raw) : ddt;
    j->du[sel * L + t] = du;
    j->ddelta[sel * L + t] = dr;
    acc->dbias[d] += dr;
    if (acc->abias) acc->abias[d] += j->delta_softplus ? addt * or_sigmoid(raw) : addt;
  }
  if (j->dh0)
    for (int64_t n = 0; n < N; ++n) j->dh0[sel * N + n] = lam[n];
}

static void* or_bwd_worker(void* arg) {
  or_bwd_job* j = (or_bwd_job*)arg;
  const int64_t N = j->dstate, L = j->seqlen, D = j->dim, Bt = j->batch;
  double* hs = (double*)malloc(sizeof(double) * (size_t)((L + 1) * N));
  double* lam = (double*)malloc(sizeof(double) * (size_t)N);
  or_bwd_acc acc;
  acc.dA = (double*)calloc((size_t)(D * N), sizeof(double));
  acc.dD = (double*)calloc((size_t)D, sizeof(double));
  acc.dbias = (double*)calloc((size_t)D, sizeof(double));
  acc.dB = (double*)calloc((size_t)(Bt * N * L), sizeof(double));
  acc.dC = (double*)calloc((size_t)(Bt * N * L), sizeof(double));
  acc.aA = acc.aB = acc.aC = acc.aD = acc.abias = NULL;
  int ok = hs && lam && acc.dA && acc.dD && acc.dbias && acc.dB && acc.dC;
  if (j->aA) {
    acc.aA = (double*)calloc((size_t)(D * N), sizeof(double));
    acc.aD = (double*)calloc((size_t)D, sizeof(double));
    acc.abias = (double*)calloc((size_t)D, sizeof(double));
    acc.aB = (double*)calloc((size_t)(Bt * N * L), sizeof(double));
    acc.aC = (double*)calloc((size_t)(Bt * N * L), sizeof(double));
    ok = ok && acc.aA && acc.aD && acc.abias && acc.aB && acc.aC;
  }
  const int64_t blk = or_claim_block(j->n_channels, L, j->n_threads);
  for (; ok;) {
    pthread_mutex_lock(&j->lock);
    const int64_t first = j->next;
    j->next += blk;
    pthread_mutex_unlock(&j->lock);
    if (first >= j->n_channels) break;
    const int64_t last = first + blk < j->n_channels ? first + blk : j->n_channels;
    for (int64_t sel = first; sel < last; ++sel) or_bwd_one(j, sel, hs, lam, &acc);
  }
  pthread_mutex_lock(&j->lock);
  if (!ok) {
    j->status = 2;
  } else {
    for (int64_t i = 0; i < D * N; ++i) j->dA[i] += acc.dA[i];
    for (int64_t i = 0; i < D; ++i) j->dD[i] += acc.dD[i];
    for (int64_t i = 0; i < D; ++i) j->dbias[i] += acc.dbias[i];
    for (int64_t i = 0; i < Bt * N * L; ++i) j->dB[i] += acc.dB[i];
    for (int64_t i = 0; i < Bt * N * L; ++i) j->dC[i] += acc.dC[i];
    if (j->aA) {
      for (int64_t i = 0; i < D * N; ++i) j->aA[i] += acc.aA[i];
      for (int64_t i = 0; i < D; ++i) j->aD[i] += acc.aD[i];
      for (int64_t i = 0; i < D; ++i) j->abias[i] += acc.abias[i];
      for (int64_t i = 0; i < Bt * N * L; ++i) j->aB[i] += acc.aB[i];
      for (int64_t i = 0; i < Bt * N * L; ++i) j->aC[i] += acc.aC[i];
    }
  }
  pthread_mutex_unlock(&j->lock);
  free(hs);
  free(lam);
  free(acc.dA);
  free(acc.dD);
  free(acc.dbias);
  free(acc.dB);
  free(acc.dC);
  free(acc.aA);
  free(acc.aD);
  free(acc.abias);
  free(acc.aB);
  free(acc.aC);
  return NULL;
}

/*
 * Backward of ssm_oracle_selective_scan over the selected channels.
 *   dy          : [batch, dim, seqlen] double, gradient of y
 *   dfinal      : [n_channels, dstate] double or NULL, gradient of the final state
 *   h0          : [n_channels, dstate] double or NULL
 * Outputs (double; the sums add the selected channels' contributions):
 *   du, ddelta  : [n_channels, seqlen] (ddelta is the gradient of the raw step)
 *   dz          : [n_channels, seqlen] or NULL
 *   dh0         : [n_channels, dstate] or NULL
 *   dA          : [dim, dstate];  dB, dC : [batch, dstate, seqlen];  dD, dbias : [dim]
 *   aA, aB, aC, aD, abias : NULL, or all five: the sums of |term| of dA, dB,
 *                 dC, dD, dbias, same shapes
 * The sums are overwritten (zeroed first).  Returns 0, 1 on bad arguments,
 * 2 on allocation failure.
 */
int ssm_oracle_selective_scan_bwd(int io_dtype, const void* u, const void* delta, const void* Bm,
                                  const void* Cm, const void* z, const double* A,
                                  const double* Dskip, const double* delta_bias,
                                  int delta_softplus, int bbar_mode, const double* h0,
                                  const double* dy, const double* dfinal, int64_t batch,
                                  int64_t dim, int64_t dstate, int64_t seqlen,
                                  const int64_t* channels, int64_t n_channels, double* du,
                                  double* ddelta, double* dA, double* dB, double* dC, double* dD,
                                  double* dz, double* dbias, double* dh0, double* aA,
                                  double* aB, double* aC, double* aD, double* abias,
                                  int n_threads) {
  if (!u || !delta || !Bm || !Cm || !A || !dy || !du || !ddelta || !dA || !dB || !dC || !dD ||
      !dbias)
    return 1;
  const int any_abs = aA || aB || aC || aD || abias;
  if (any_abs && !(aA && aB && aC && aD && abias)) return 1;
  if (batch <= 0 || dim <= 0 || dstate <= 0 || seqlen <= 0) return 1;
  if (io_dtype != OR_F32 && io_dtype != OR_BF16 && io_dtype != OR_F64) return 1;
  if (bbar_mode != OR_BBAR_DELTA_B && bbar_mode != OR_BBAR_ZOH_EXACT) return 1;
  if (!channels) n_channels = batch * dim;
  for (int64_t i = 0; channels && i < n_channels; ++i)
    if (channels[i] < 0 || channels[i] >= batch * dim) return 1;
  memset(dA, 0, sizeof(double) * (size_t)(dim * dstate));
  memset(dD, 0, sizeof(double) * (size_t)dim);
  memset(dbias, 0, sizeof(double) * (size_t)dim);
  memset(dB, 0, sizeof(double) * (size_t)(batch * dstate * seqlen));
  memset(dC, 0, sizeof(double) * (size_t)(batch * dstate * seqlen));
  if (any_abs) {
    memset(aA, 0, sizeof(double) * (size_t)(dim * dstate));
    memset(aD, 0, sizeof(double) * (size_t)dim);
    memset(abias, 0, sizeof(double) * (size_t)dim);
    memset(aB, 0, sizeof(double) * (size_t)(batch * dstate * seqlen));
    memset(aC, 0, sizeof(double) * (size_t)(batch * dstate * seqlen));
  }
  or_bwd_job j;
  memset(&j, 0, sizeof j);
  j.io_dtype = io_dtype;
  j.u = u;
  j.delta = delta;
  j.Bm = Bm;
  j.Cm = Cm;
  j.z = z;
  j.A = A;
  j.Dskip = Dskip;
  j.delta_bias = delta_bias;
  j.h0 = h0;
  j.dy = dy;
  j.dfinal = dfinal;
  j.delta_softplus = delta_softplus;
  j.bbar_mode = bbar_mode;
  j.batch = batch;
  j.dim = dim;
  j.dstate = dstate;
  j.seqlen = seqlen;
  j.channels = channels;
  j.n_channels = n_channels;
  j.du = du;
  j.ddelta = ddelta;
  j.dz = dz;
  j.dh0 = dh0;
  j.dA = dA;
  j.dB = dB;
  j.dC = dC;
  j.dD = dD;
  j.dbias = dbias;
  j.aA = aA;
  j.aB = aB;
  j.aC = aC;
  j.aD = aD;
  j.abias = abias;
  pthread_mutex_init(&j.lock, NULL);
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  if ((int64_t)n_threads > n_channels) n_threads = (int)n_channels;
  j.n_threads = n_threads;
  pthread_t tid[256];
  int started = 0;
  for (int i = 1; i < n_threads; ++i)
    if (pthread_create(&tid[started], NULL, or_bwd_worker, &j) == 0) ++started;
  or_bwd_worker(&j);
  for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
  pthread_mutex_destroy(&j.lock);
  return j.status;
}

/*
 * Depthwise causal convolution of width W with an optional silu, the step in
 * front of the scan in the Mamba block ("State-space models", section
 * "Mamba: selection", the paragraph on the block: a depthwise causal
 * convolution of width 4 and a silu on one half of the projection).  Per
 * sequence b and channel d:
 *
 *   pre_t = bias_d + sum_{k=0}^{W-1} w_{d,k} x_{t-(W-1)+k},   out_t = silu(pre_t) or pre_t
 *
 * i.e. the cross-correlation of the sequence padded on the left, as the
 * page's F.conv1d snippet computes it ("State-space models", section
 * "Implementation": left padding so that no output sees the future).  The
 * W-1 inputs before t = 0 come from state_in ([batch, dim, W-1], oldest
 * first) or are zero.  state_out (optional) receives the last W-1 inputs of
 * the extended sequence, oldest first: with L = 1 this is the one-token
 * decode step.  Inputs are io dtype bits (0 f32, 1 bf16, 2 f64); weights,
 * bias and states are double; out is double [batch, dim, L].
 */
static double or_conv_x(const void* x, int io_dtype, const double* st, int64_t row, int64_t sbase,
                        int64_t W, int64_t t) {
  if (t >= 0) return or_widen(x, io_dtype, row + t);
  return st ? st[sbase + (W - 1) + t] : 0.0; /* t in [-(W-1), -1] */
}

int ssm_oracle_conv1d(int io_dtype, const void* x, const double* w, const double* bias,
                      const double* state_in, int64_t batch, int64_t dim, int64_t L, int64_t W,
                      int silu, double* out, double* state_out) {
  if (!x || !w || !out || batch <= 0 || dim <= 0 || L <= 0 || W <= 0) return 1;
  for (int64_t c = 0; c < batch * dim; ++c) {
    const int64_t d = c % dim, row = c * L, sb = c * (W - 1);
    for (int64_t t = 0; t < L; ++t) {
      double pre = bias ? bias[d] : 0.0;
      for (int64_t k = 0; k < W; ++k)
        pre += w[d * W + k] * or_conv_x(x, io_dtype, state_in, row, sb, W, t - (W - 1) + k);
      out[row + t] = silu ? or_silu(pre) : pre;
    }
    if (state_out)
      for (int64_t j = 0; j < W - 1; ++j)
        state_out[sb + j] = or_conv_x(x, io_dtype, state_in, row, sb, W, L - (W - 1) + j);
  }
  return 0;
}

/*
 * Gradients of ssm_oracle_conv1d for the loss sum(dout * out): with
 * g_t = dout_t silu'(pre_t) (or dout_t without the silu),
 *   dx_s     = sum_k w_k g_{s+(W-1)-k}          (terms with 0 <= s+(W-1)-k < L)
 *   dw_{d,k} = sum_{b,t} g_t x_{t-(W-1)+k}      dbias_d = sum_{b,t} g_t
 *   dstate_j = the dx of the pre-start input at time j-(W-1).
 * dx and dout are double [batch, dim, L]; dw [dim, W], dbias [dim] are
 * overwritten; dstate_in [batch, dim, W-1] may be NULL.  aw [dim, W] and
 * abias [dim] (both or neither) receive the sums of |term| of dw and dbias.
 */
int ssm_oracle_conv1d_bwd(int io_dtype, const void* x, const double* w, const double* bias,
                          const double* state_in, const double* dout, int64_t batch, int64_t dim,
                          int64_t L, int64_t W, int silu, double* dx, double* dw, double* dbias,
                          double* dstate_in, double* aw, double* abias) {
  if (!x || !w || !dout || !dx || !dw || !dbias || batch <= 0 || dim <= 0 || L <= 0 || W <= 0)
    return 1;
  if (!aw != !abias) return 1;
  memset(dw, 0, sizeof(double) * (size_t)(dim * W));
  memset(dbias, 0, sizeof(double) * (size_t)dim);
  if (aw) {
    memset(aw, 0, sizeof(double) * (size_t)(dim * W));
    memset(abias, 0, sizeof(double) * (size_t)dim);
  }
  double* g = (double*)malloc(sizeof(double) * (size_t)L);
  if (!g) return 2;
  for (int64_t c = 0; c < batch * dim; ++c) {
    const int64_t d = c % dim, row = c * L, sb = c * (W - 1);
    for (int64_t t = 0; t < L; ++t) {
      double pre = bias ? bias[d] : 0.0;
      for (int64_t k = 0; k < W; ++k)
        pre += w[d * W + k] * or_conv_x(x, io_dtype, state_in, row, sb, W, t - (W - 1) + k);
      const double s = or_sigmoid(pre);
      g[t] = silu ? dout[row + t] * s * (1.0 + pre * (1.0 - s)) : dout[row + t];
      dbias[d] += g[t];
      if (abias) abias[d] += fabs(g[t]);
      for (int64_t k = 0; k < W; ++k) {
        const double term = g[t] * or_conv_x(x, io_dtype, state_in, row, sb, W, t - (W - 1) + k);
        dw[d * W + k] += term;
        if (aw) aw[d * W + k] += fabs(term);
      }
    }
    /* input at time s (s >= -(W-1)) feeds outputs t = s + (W-1) - k */
    for (int64_t s = -(W - 1); s < L; ++s) {
      double acc = 0.0;
      for (int64_t k = 0; k < W; ++k) {
        const int64_t t = s + (W - 1) - k;
        if (t >= 0 && t < L) acc += w[d * W + k] * g[t];
      }
      if (s >= 0)
        dx[row + s] = acc;
      else if (dstate_in)
        dstate_in[sb + (W - 1) + s] = acc;
    }
  }
  free(g);
  return 0;
}

/*
 * Mamba-2 selective scan with a scalar A per head ("State-space models",
 * section "The parallel scan", last sentences: A restricted to a scalar times
 * the identity per head; "Structured State Space Models and Mamba ...",
 * section "State Space Duality and Mamba-2").  Per sequence b, head h, head
 * channel p and state n, with group g = h / (nheads / ngroups):
 *
 *   dt_t      = softplus(dt_raw_t + dt_bias_h)   (or dt_raw_t + dt_bias_h)
 *   h_t[p,n]  = exp(dt_t A_h) h_{t-1}[p,n] + dt_t B_t[g,n] x_t[h,p]
 *   y_t[h,p]  = sum_n C_t[g,n] h_t[p,n] + D_h x_t[h,p],   then * silu(z) if z
 *
 * Layouts (channel-major, as for the diagonal scan): x, z [batch, nheads *
 * headdim, L]; dt [batch, nheads, L]; B, C [batch, ngroups * dstate, L];
 * A, D, dt_bias [nheads]; h0 and final_state [batch, nheads, headdim,
 * dstate].  y is double [batch, nheads * headdim, L].  Threads split
 * (b, h) pairs.
 */
typedef struct {
  int io_dtype;
  const void *x, *dt, *Bm, *Cm, *z;
  const double *A, *Dskip, *dt_bias, *h0;
  int softplus;
  int64_t batch, L, H, P, G, N;
  double *y, *final_state;
  int64_t next;
  pthread_mutex_t lock;
} or_ssd_job;

static void or_ssd_one(const or_ssd_job* j, int64_t bh, double* st) {
  const int64_t b = bh / j->H, h = bh % j->H, L = j->L, P = j->P, N = j->N;
  const int64_t g = h / (j->H / j->G);
  for (int64_t i = 0; i < P * N; ++i) st[i] = j->h0 ? j->h0[bh * P * N + i] : 0.0;
  const double bias = j->dt_bias ? j->dt_bias[h] : 0.0;
  const double Dh = j->Dskip ? j->Dskip[h] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    const double raw = or_widen(j->dt, j->io_dtype, (b * j->H + h) * L + t) + bias;
    const double dt = j->softplus ? or_softplus(raw) : raw;
    const double a = exp(dt * j->A[h]);
    for (int64_t p = 0; p < P; ++p) {
      const int64_t xrow = (b * j->H * P + h * P + p) * L;
      const double xt = or_widen(j->x, j->io_dtype, xrow + t);
      double yt = Dh * xt;
      for (int64_t n = 0; n < N; ++n) {
        const int64_t bcrow = (b * j->G * N + g * N + n) * L;
        const double bt = or_widen(j->Bm, j->io_dtype, bcrow + t);
        const double ct = or_widen(j->Cm, j->io_dtype, bcrow + t);
        double* s = st + p * N + n;
        *s = a * *s + dt * bt * xt;
        yt += ct * *s;
      }
      if (j->z) yt *= or_silu(or_widen(j->z, j->io_dtype, xrow + t));
      j->y[xrow + t] = yt;
    }
  }
  if (j->final_state)
    for (int64_t i = 0; i < P * N; ++i) j->final_state[bh * P * N + i] = st[i];
}

static void* or_ssd_worker(void* arg) {
  or_ssd_job* j = (or_ssd_job*)arg;
  double* st = (double*)malloc(sizeof(double) * (size_t)(j->P * j->N));
  if (!st) return (void*)1;
  for (;;) {
    pthread_mutex_lock(&j->lock);
    const int64_t bh = j->next++;
    pthread_mutex_unlock(&j->lock);
    if (bh >= j->batch * j->H) break;
    or_ssd_one(j, bh, st);
  }
  free(st);
  return NULL;
}

int ssm_oracle_ssd(int io_dtype, const void* x, const void* dt, const void* Bm, const void* Cm,
                   const void* z, const double* A, const double* Dskip, const double* dt_bias,
                   int dt_softplus, const double* h0, int64_t batch, int64_t L, int64_t nheads,
                   int64_t headdim, int64_t ngroups, int64_t dstate, double* y,
                   double* final_state, int n_threads) {
  if (!x || !dt || !Bm || !Cm || !A || !y) return 1;
  if (batch <= 0 || L <= 0 || nheads <= 0 || headdim <= 0 || ngroups <= 0 || dstate <= 0) return 1;
  if (nheads % ngroups) return 1;
  if (io_dtype != OR_F32 && io_dtype != OR_BF16 && io_dtype != OR_F64) return 1;
  or_ssd_job j;
  memset(&j, 0, sizeof j);
  j.io_dtype = io_dtype;
  j.x = x; j.dt = dt; j.Bm = Bm; j.Cm = Cm; j.z = z;
  j.A = A; j.Dskip = Dskip; j.dt_bias = dt_bias; j.h0 = h0; j.softplus = dt_softplus;
  j.batch = batch; j.L = L; j.H = nheads; j.P = headdim; j.G = ngroups; j.N = dstate;
  j.y = y; j.final_state = final_state;
  pthread_mutex_init(&j.lock, NULL);
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  if ((int64_t)n_threads > batch * nheads) n_threads = (int)(batch * nheads);
  pthread_t tid[256];
  int started = 0, rc = 0;
  for (int i = 1; i < n_threads; ++i)
    if (pthread_create(&tid[started], NULL, or_ssd_worker, &j) == 0) ++started;
  if (or_ssd_worker(&j)) rc = 2;
  for (int i = 0; i < started; ++i) {
    void* r = NULL;
    pthread_join(tid[i], &r);
    if (r) rc = 2;
  }
  pthread_mutex_destroy(&j.lock);
  return rc;
}
