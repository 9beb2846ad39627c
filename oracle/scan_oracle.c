/*
 * scan_oracle.c -- fp64 CPU oracle for Mamba's selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP kernels.
 *
 * What it computes is the plain definition, written out in double precision,
 * strictly sequential in time for each (batch, channel):
 *
 *   A[n]   = -exp(A_log[d,n])                     diagonal, real, negative
 *            (Mamba notes, awesome.papernotes.org: "训练策略", A = -exp(A_log);
 *             State space models and Mamba, jonathanding.github.io: §1.5)
 *   Delta  = softplus(delta[b,d,t] + bias[d])     (Mamba notes, 设计 1, the
 *            selection formula and its pseudo-code; same notes, 训练策略,
 *            "softplus + bias"; State space models and Mamba, §4)
 *   Abar   = exp(Delta*A[n])                      zero-order hold
 *   Bbar   = A[n]^-1 (exp(Delta*A[n]) - 1) B[b,n,t]
 *            (State space models and Mamba, §2, the ZOH formula; Mamba notes,
 *             设计 1, the same discretization written with (Delta A)^-1 Delta B)
 *   h[n]   = Abar h[n] + Bbar u[b,d,t]            (Mamba notes, 设计 1, the
 *            recurrence; starting state zero: MAMBA walkthrough,
 *            x-humanoid.csdn.net, §3 scan pseudo-code)
 *   y      = sum_n C[b,n,t] h[n] + D[d] u[b,d,t]  readout of the UPDATED state
 *            (Mamba notes, 设计 1 recurrence y_t = C_t h_t and the D skip in its
 *             pseudo-code; State space models and Mamba, §3: y_0 = C Bbar u_0)
 *   out    = y * SiLU(z[b,d,t])                   (Mamba notes, 设计 3 block
 *            pseudo-code and the 整体框架 figure: out = y * SiLU(z))
 *
 * The single-token step is exactly one iteration of the time loop applied to a
 * caller-held state (State space models and Mamba, §3, recurrence mode;
 * Mamba notes, 设计 2: only a (d, N) state is kept at inference).
 *
 * Layouts (all row-major, float64):
 *   u, delta, z, y : (batch, dim, seqlen)      B, C : (batch, dstate, seqlen)
 *   A_log          : (dim, dstate)             D, delta_bias : (dim)
 *   initial_state, final_state : (batch, dim, dstate)
 * Optional pointers may be NULL: D -> 0, z -> no gate, delta_bias -> 0,
 * initial_state -> 0, final_state -> not written.
 *
 * Numerical notes (choices of evaluation, not of definition):
 *   softplus(x) = log(1 + e^x) is evaluated as max(x,0) + log1p(exp(-|x|)),
 *   the same function without overflow.  exp(x) - 1 is evaluated with
 *   expm1(x), the same function without cancellation.  If A[n] == 0 (only
 *   possible for A_log = -inf) Bbar takes its limit Delta * B.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double oracle_softplus(double x) {
  /* log(1 + e^x) */
  return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

static double oracle_silu(double z) {
  /* z * sigmoid(z) */
  return z / (1.0 + exp(-z));
}

/* One time step of one (batch, channel) recurrence: updates h[0..N) in place
 * and returns the gated output for this token. */
static double oracle_one_token(double* h, int64_t N, const double* A, double u, double dlt, double bias,
                               int softplus_on, const double* Bt, int64_t b_stride, const double* Ct,
                               int64_t c_stride, double Dd, const double* zt) {
  double x = dlt + bias;
  double Delta = softplus_on ? oracle_softplus(x) : x;
  double acc = 0.0;
  for (int64_t n = 0; n < N; ++n) {
    double dA = Delta * A[n];
    double Abar = exp(dA);
    double Bn = Bt[n * b_stride];
    double Bbar = (A[n] != 0.0) ? expm1(dA) / A[n] * Bn : Delta * Bn;
    h[n] = Abar * h[n] + Bbar * u;
    acc += Ct[n * c_stride] * h[n];
  }
  double y = acc + Dd * u;
  if (zt) y = y * oracle_silu(*zt);
  return y;
}

int oracle_scan_fwd(const double* u, const double* delta, const double* A_log, const double* B,
                    const double* C, const double* D, const double* z, const double* delta_bias,
                    const double* initial_state, double* final_state, double* y, int64_t batch,
                    int64_t dim, int64_t dstate, int64_t seqlen, int delta_softplus, int nthreads) {
  if (!u || !delta || !A_log || !B || !C || !y) return 1;
  if (batch < 0 || dim < 0 || dstate < 1 || seqlen < 0) return 2;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const int64_t BD = batch * dim;
#pragma omp parallel for schedule(static)
  for (int64_t bd = 0; bd < BD; ++bd) {
    const int64_t b = bd / dim, d = bd % dim;
    double* h = (double*)malloc(sizeof(double) * (size_t)(2 * dstate));
    double* A = h + dstate;
    for (int64_t n = 0; n < dstate; ++n) {
      A[n] = -exp(A_log[d * dstate + n]);
      h[n] = initial_state ? initial_state[bd * dstate + n] : 0.0;
    }
    const double bias = delta_bias ? delta_bias[d] : 0.0;
    const double Dd = D ? D[d] : 0.0;
    const int64_t row = bd * seqlen;                 /* (b, d, :) */
    const int64_t bcrow = b * dstate * seqlen;       /* (b, 0, :) */
    for (int64_t t = 0; t < seqlen; ++t) {
      y[row + t] = oracle_one_token(h, dstate, A, u[row + t], delta[row + t], bias, delta_softplus,
                                    B + bcrow + t, seqlen, C + bcrow + t, seqlen, Dd,
                                    z ? z + row + t : NULL);
    }
    if (final_state)
      for (int64_t n = 0; n < dstate; ++n) final_state[bd * dstate + n] = h[n];
    free(h);
  }
  return 0;
}

int oracle_scan_step(double* state, const double* x, const double* dt, const double* A_log,
                     const double* B, const double* C, const double* D, const double* z,
                     const double* dt_bias, int dt_softplus, double* y, int64_t batch, int64_t dim,
                     int64_t dstate, int nthreads) {
  if (!state || !x || !dt || !A_log || !B || !C || !y) return 1;
  if (batch < 0 || dim < 0 || dstate < 1) return 2;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const int64_t BD = batch * dim;
#pragma omp parallel for schedule(static)
  for (int64_t bd = 0; bd < BD; ++bd) {
    const int64_t b = bd / dim, d = bd % dim;
    double* A = (double*)malloc(sizeof(double) * (size_t)dstate);
    for (int64_t n = 0; n < dstate; ++n) A[n] = -exp(A_log[d * dstate + n]);
    y[bd] = oracle_one_token(state + bd * dstate, dstate, A, x[bd], dt[bd], dt_bias ? dt_bias[d] : 0.0,
                             dt_softplus, B + b * dstate, 1, C + b * dstate, 1, D ? D[d] : 0.0,
                             z ? z + bd : NULL);
    free(A);
  }
  return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
