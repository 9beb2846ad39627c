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
 * Variant (flag `euler`): Bbar = Delta * B[b,n,t], the first-order (Euler)
 * input term that the Mamba notes' 设计 1 pseudo-code writes as Delta B x;
 * Abar stays exp(Delta*A[n]).
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
                               int softplus_on, int euler, const double* Bt, int64_t b_stride,
                               const double* Ct, int64_t c_stride, double Dd, const double* zt) {
  double x = dlt + bias;
  double Delta = softplus_on ? oracle_softplus(x) : x;
  double acc = 0.0;
  for (int64_t n = 0; n < N; ++n) {
    double dA = Delta * A[n];
    double Abar = exp(dA);
    double Bn = Bt[n * b_stride];
    double Bbar;
    if (euler)
      Bbar = Delta * Bn;                                            /* Euler input term */
    else
      Bbar = (A[n] != 0.0) ? expm1(dA) / A[n] * Bn : Delta * Bn;    /* zero-order hold */
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
                    int64_t dim, int64_t dstate, int64_t seqlen, int delta_softplus, int euler,
                    int nthreads) {
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
      y[row + t] = oracle_one_token(h, dstate, A, u[row + t], delta[row + t], bias, delta_softplus, euler,
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
                     const double* dt_bias, int dt_softplus, int euler, double* y, int64_t batch,
                     int64_t dim, int64_t dstate, int nthreads) {
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
                             dt_softplus, euler, B + b * dstate, 1, C + b * dstate, 1, D ? D[d] : 0.0,
                             z ? z + bd : NULL);
    free(A);
  }
  return 0;
}

/*
 * Variable-length batch: nseq sequences packed one after another along the
 * time axis of a single row per channel, sequence s covering tokens
 * [cu_seqlens[s], cu_seqlens[s+1]).  Each sequence is its own scan of the
 * definition above, from its own initial state (or zero), with its own final
 * state; nothing carries across a boundary.  (The pages define the scan of
 * one sequence; packing several into one row is how batches of unequal
 * lengths are laid out without padding -- the plain reading is that the
 * recurrence restarts at each sequence start.)
 *
 *   u, delta, z, y : (dim, total)     B, C : (dstate, total)
 *   initial_states, final_states : (nseq, dim, dstate)
 * cu_seqlens must be non-decreasing from 0 to total (checked: returns 3).
 */
int oracle_scan_fwd_varlen(const double* u, const double* delta, const double* A_log, const double* B,
                           const double* C, const double* D, const double* z, const double* delta_bias,
                           const int64_t* cu_seqlens, const double* initial_states, double* final_states,
                           double* y, int64_t nseq, int64_t dim, int64_t dstate, int64_t total,
                           int delta_softplus, int euler, int nthreads) {
  if (!A_log || !cu_seqlens || !y || (total > 0 && (!u || !delta || !B || !C))) return 1;
  if (nseq < 1 || dim < 0 || dstate < 1 || total < 0) return 2;
  if (cu_seqlens[0] != 0 || cu_seqlens[nseq] != total) return 3;
  for (int64_t s = 0; s < nseq; ++s)
    if (cu_seqlens[s + 1] < cu_seqlens[s]) return 3;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const int64_t SD = nseq * dim;
#pragma omp parallel for schedule(dynamic)
  for (int64_t sd = 0; sd < SD; ++sd) {
    const int64_t s = sd / dim, d = sd % dim;
    double* h = (double*)malloc(sizeof(double) * (size_t)(2 * dstate));
    double* A = h + dstate;
    for (int64_t n = 0; n < dstate; ++n) {
      A[n] = -exp(A_log[d * dstate + n]);
      h[n] = initial_states ? initial_states[sd * dstate + n] : 0.0;   /* restart at the sequence start */
    }
    const double bias = delta_bias ? delta_bias[d] : 0.0;
    const double Dd = D ? D[d] : 0.0;
    const int64_t row = d * total;
    for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
      y[row + t] = oracle_one_token(h, dstate, A, u[row + t], delta[row + t], bias, delta_softplus, euler,
                                    B + t, total, C + t, total, Dd, z ? z + row + t : NULL);
    }
    if (final_states)
      for (int64_t n = 0; n < dstate; ++n) final_states[sd * dstate + n] = h[n];
    free(h);
  }
  return 0;
}

/*
 * Multi-head SSM with a scalar decay per head (the state-space-duality form;
 * State space models and Mamba, jonathanding.github.io, §5: head dim P > 1,
 * the P channels of a head share A, and the dual matrix has
 * Lambda_ij = prod_{t=j+1..i} a_t).  Per batch row b, head h, head channel p
 * and state n, with A_h = -exp(A_log[h]):
 *
 *   Delta_t = softplus(dt[b,t,h] + dt_bias[h])        (or without softplus)
 *   a_t     = exp(Delta_t A_h)                        scalar per (b, t, h)
 *   w_t     = (a_t - 1) / A_h   zero-order hold       (or Delta_t: Euler, flag)
 *   h_t[p,n]= a_t h_{t-1}[p,n] + w_t B[b,t,n] x[b,t,h,p]
 *   y[b,t,h,p] = sum_n C[b,t,n] h_t[p,n] + D[h] x[b,t,h,p]   (times SiLU(z) if z)
 *
 * This is the selective scan above with A and Delta shared by the P channels
 * of a head (B and C are shared by all heads, as they are by all channels
 * there).  Token-major layouts (the layout of the projections that feed it):
 *   x, z, y : (batch, L, H, P)    dt : (batch, L, H)    B, C : (batch, L, N)
 *   A_log, D, dt_bias : (H)       initial_state, final_state : (batch, H, P, N)
 */
int oracle_ssd_fwd(const double* x, const double* dt, const double* A_log, const double* B, const double* C,
                   const double* D, const double* z, const double* dt_bias, const double* initial_state,
                   double* final_state, double* y, int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                   int64_t dstate, int dt_softplus, int euler, int nthreads) {
  if (!A_log || !y || (seqlen > 0 && (!x || !dt || !B || !C))) return 1;
  if (batch < 0 || seqlen < 0 || nheads < 1 || headdim < 1 || dstate < 1) return 2;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const int64_t HP = nheads * headdim;
  const int64_t BHP = batch * HP;
#pragma omp parallel for schedule(static)
  for (int64_t bhp = 0; bhp < BHP; ++bhp) {
    const int64_t b = bhp / HP, hp = bhp % HP, hh = hp / headdim, p = hp % headdim;
    double* h = (double*)malloc(sizeof(double) * (size_t)dstate);
    const double A = -exp(A_log[hh]);
    for (int64_t n = 0; n < dstate; ++n)
      h[n] = initial_state ? initial_state[((b * nheads + hh) * headdim + p) * dstate + n] : 0.0;
    const double bias = dt_bias ? dt_bias[hh] : 0.0;
    const double Dh = D ? D[hh] : 0.0;
    for (int64_t t = 0; t < seqlen; ++t) {
      const double xv = dt[(b * seqlen + t) * nheads + hh] + bias;
      const double Delta = dt_softplus ? oracle_softplus(xv) : xv;
      const double a = exp(Delta * A);
      const double w = euler ? Delta : ((A != 0.0) ? expm1(Delta * A) / A : Delta);
      const int64_t xi = (b * seqlen + t) * HP + hp;      /* (b, t, h, p) */
      const double* Bt = B + (b * seqlen + t) * dstate;
      const double* Ct = C + (b * seqlen + t) * dstate;
      double acc = 0.0;
      for (int64_t n = 0; n < dstate; ++n) {
        h[n] = a * h[n] + w * Bt[n] * x[xi];
        acc += Ct[n] * h[n];
      }
      double yv = acc + Dh * x[xi];
      if (z) yv *= oracle_silu(z[xi]);
      y[xi] = yv;
    }
    if (final_state)
      for (int64_t n = 0; n < dstate; ++n) final_state[((b * nheads + hh) * headdim + p) * dstate + n] = h[n];
    free(h);
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

/*
 * Backward pass (gradients of a scalar loss through the forward above, given
 * dL/dy and optionally dL/d(final_state)).
 *
 * The pages describe the backward pass only as a strategy -- the fused kernel
 * keeps no intermediate states and recomputes them when gradients are needed
 * (State space models and Mamba, jonathanding.github.io, Parallel Scan; Mamba
 * notes, awesome.papernotes.org, 设计 2).  What it must compute is the
 * gradient of the function defined above, obtained here by the chain rule
 * through each step, in reverse time order.  With ytil_t = sum_n C h_t + D u
 * the pre-gate output, s(z) = SiLU(z) and lam_t[n] = dL/dh_t[n] (total):
 *
 *   dytil_t  = dy_t s(z_t);      dz_t = dy_t ytil_t s'(z_t),
 *              s'(z) = sigma(z) (1 + z (1 - sigma(z)))
 *   lam_t    = dytil_t C_t + Abar_{t+1} lam_{t+1}   (lam_{L-1} adds dL/d(final))
 *   dC_t[n] += dytil_t h_t[n]                       (summed over channels)
 *   dB_t[n] += lam_t[n] u_t (Abar_t[n] - 1) / A[n]  (Delta u_t if A = 0)
 *   du_t     = dytil_t D + sum_n lam_t[n] Bbar_t[n]
 *   dDelta_t = sum_n lam_t[n] Abar_t[n] (A[n] h_{t-1}[n] + B_t[n] u_t)
 *   dA[n]   += lam_t[n] (Delta_t Abar_t h_{t-1} + u_t B_t (Delta_t Abar_t A - (Abar_t - 1)) / A^2)
 *              (limit Delta^2 B u / 2 if A = 0)
 *   dA_log   = dA * A                               (A = -exp(A_log))
 *   ddelta_t = dDelta_t sigma(delta_t + bias)       (dDelta_t without softplus)
 *   dbias   += ddelta_t;  dD += dytil_t u_t;  d(initial state) = Abar_0 lam_0
 *
 * With the Euler input term (euler != 0: Bbar = Delta B, the pages' simplified
 * form) the terms that differ are dB_t[n] += lam u Delta, Bbar = Delta B in du,
 * dDelta_t = sum_n lam (A Abar h_{t-1} + B u) and dA[n] += lam Delta Abar h_{t-1}.
 *
 * Outputs (float64, row-major like the inputs): du, ddelta, dz (batch, dim, L);
 * dB, dC (batch, dstate, L); dA_log (dim, dstate); dD, ddelta_bias (dim);
 * d_initial_state (batch, dim, dstate).  dz, dD, ddelta_bias and
 * d_initial_state may be NULL (not computed); d_final_state may be NULL (0).
 * The forward states are kept in full, per (batch, channel), for the reverse
 * sweep.  Channels run in parallel within a batch row; the sums over channels
 * (dB, dC) go through per-thread buffers added in a fixed order, and the sums
 * over batch rows (dA_log, dD, ddelta_bias) run over batch rows in order.
 */
static double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

int oracle_scan_bwd(const double* u, const double* delta, const double* A_log, const double* B,
                    const double* C, const double* D, const double* z, const double* delta_bias,
                    const double* initial_state, const double* dy, const double* d_final_state,
                    double* du, double* ddelta, double* dA_log, double* dB, double* dC, double* dD,
                    double* dz, double* ddelta_bias, double* d_initial_state, int64_t batch, int64_t dim,
                    int64_t dstate, int64_t seqlen, int delta_softplus, int euler, int nthreads) {
  if (!u || !delta || !A_log || !B || !C || !dy || !du || !ddelta || !dA_log || !dB || !dC) return 1;
  if (batch < 0 || dim < 0 || dstate < 1 || seqlen < 0) return 2;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
  const int nthr = omp_get_max_threads();
#else
  (void)nthreads;
  const int nthr = 1;
#endif
  const int64_t N = dstate, L = seqlen;
  for (int64_t i = 0; i < dim * N; ++i) dA_log[i] = 0.0;
  if (dD)
    for (int64_t i = 0; i < dim; ++i) dD[i] = 0.0;
  if (ddelta_bias)
    for (int64_t i = 0; i < dim; ++i) ddelta_bias[i] = 0.0;
  double* part = (double*)calloc((size_t)nthr * (size_t)(2 * N * L + 1), sizeof(double));   /* per-thread dB, dC */
  double* pdim = (double*)calloc((size_t)dim * (size_t)(N + 2), sizeof(double));            /* per-channel sums of one row */
  if (!part || !pdim) {
    free(part);
    free(pdim);
    return 3;
  }
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t i = 0; i < (int64_t)nthr * (2 * N * L + 1); ++i) part[i] = 0.0;
#pragma omp parallel for schedule(static)
    for (int64_t d = 0; d < dim; ++d) {
#ifdef _OPENMP
      const int tid = omp_get_thread_num();
#else
      const int tid = 0;
#endif
      double* pB = part + (int64_t)tid * (2 * N * L + 1);
      double* pC = pB + N * L;
      const int64_t bd = b * dim + d;
      const int64_t row = bd * L, bcrow = b * N * L;
      double* A = (double*)malloc(sizeof(double) * (size_t)(N * (L + 3) + 2 * L));
      double* H = A + N;             /* H[(t + 1) N + n] = h_t[n], H[n] = initial state */
      double* lam = H + N * (L + 1); /* running lam_t[n] */
      double* Dl = lam + N;          /* Delta_t */
      double* yt = Dl + L;           /* ytil_t */
      const double bias = delta_bias ? delta_bias[d] : 0.0;
      const double Dd = D ? D[d] : 0.0;
      for (int64_t n = 0; n < N; ++n) {
        A[n] = -exp(A_log[d * N + n]);
        H[n] = initial_state ? initial_state[bd * N + n] : 0.0;
      }
      /* forward, keeping every state */
      for (int64_t t = 0; t < L; ++t) {
        const double x = delta[row + t] + bias;
        const double Delta = delta_softplus ? oracle_softplus(x) : x;
        Dl[t] = Delta;
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          const double dA = Delta * A[n];
          const double Bn = B[bcrow + n * L + t];
          const double Bbar = euler ? Delta * Bn : ((A[n] != 0.0) ? expm1(dA) / A[n] * Bn : Delta * Bn);
          const double hn = exp(dA) * H[t * N + n] + Bbar * u[row + t];
          H[(t + 1) * N + n] = hn;
          acc += C[bcrow + n * L + t] * hn;
        }
        yt[t] = acc + Dd * u[row + t];
      }
      /* reverse */
      double dDacc = 0.0, dbacc = 0.0;
      double* dAn = pdim + d * (N + 2);
      for (int64_t n = 0; n < N; ++n) lam[n] = d_final_state ? d_final_state[bd * N + n] : 0.0;
      for (int64_t t = L - 1; t >= 0; --t) {
        const double ut = u[row + t], Delta = Dl[t];
        double dyt = dy[row + t];
        if (z) {
          const double zz = z[row + t], sg = oracle_sigmoid(zz);
          if (dz) dz[row + t] = dyt * yt[t] * sg * (1.0 + zz * (1.0 - sg));
          dyt *= zz * sg;
        } else if (dz) {
          dz[row + t] = 0.0;
        }
        dDacc += dyt * ut;
        double dut = dyt * Dd, dDelta = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          const double Bn = B[bcrow + n * L + t], Cn = C[bcrow + n * L + t];
          const double dA = Delta * A[n], Abar = exp(dA), em1 = expm1(dA);
          const double hprev = H[t * N + n];
          /* lam currently holds Abar_{t+1} lam_{t+1} (or dL/d final state) */
          const double l = lam[n] + dyt * Cn;
          pC[n * L + t] += dyt * H[(t + 1) * N + n];
          /* Bbar / B and its derivative in A: (e^{Delta A} - 1) / A for the zero-order hold, Delta
             (independent of A) for the Euler input term */
          const double bq = euler ? Delta : ((A[n] != 0.0) ? em1 / A[n] : Delta);     /* Bbar / B */
          pB[n * L + t] += l * ut * bq;
          dut += l * bq * Bn;
          if (euler)
            dDelta += l * (Abar * A[n] * hprev + Bn * ut);   /* dh/dDelta = A Abar h_{t-1} + B u */
          else
            dDelta += l * Abar * (A[n] * hprev + Bn * ut);
          const double dbq = euler ? 0.0 : ((A[n] != 0.0) ? (Delta * Abar * A[n] - em1) / (A[n] * A[n]) : 0.5 * Delta * Delta);
          dAn[n] += l * (Delta * Abar * hprev + ut * Bn * dbq);
          lam[n] = Abar * l;
        }
        du[row + t] = dut;
        const double dd = delta_softplus ? dDelta * oracle_sigmoid(delta[row + t] + bias) : dDelta;
        ddelta[row + t] = dd;
        dbacc += dd;
      }
      if (d_initial_state)
        for (int64_t n = 0; n < N; ++n) d_initial_state[bd * N + n] = lam[n];
      dAn[N] += dDacc;
      dAn[N + 1] += dbacc;
      free(A);
    }
    /* channel sums for this batch row, threads added in order */
    for (int64_t i = 0; i < N * L; ++i) {
      double sb = 0.0, sc = 0.0;
      for (int k = 0; k < nthr; ++k) {
        sb += part[(int64_t)k * (2 * N * L + 1) + i];
        sc += part[(int64_t)k * (2 * N * L + 1) + N * L + i];
      }
      dB[b * N * L + i] = sb;
      dC[b * N * L + i] = sc;
    }
  }
  for (int64_t d = 0; d < dim; ++d) {
    for (int64_t n = 0; n < N; ++n) dA_log[d * N + n] = pdim[d * (N + 2) + n] * (-exp(A_log[d * N + n]));
    if (dD) dD[d] = pdim[d * (N + 2) + N];
    if (ddelta_bias) ddelta_bias[d] = pdim[d * (N + 2) + N + 1];
  }
  free(part);
  free(pdim);
  return 0;
}

/*
 * Causal depthwise 1-D convolution followed by SiLU, the step in front of the
 * scan in the Mamba block.  Order: the conv, then SiLU, then the SSM, as the
 * Mamba concept page (compassingai.com, §3.3 flow) and State space models and
 * Mamba (jonathanding.github.io, Mamba block architecture) draw it; the Mamba
 * notes' block pseudo-code (awesome.papernotes.org, 设计 3) applies SiLU before
 * the conv, a minority reading not followed.  Kernel size 4: the notes' 设计 3
 * and the layer configuration of the MAMBA walkthrough (x-humanoid.csdn.net,
 * §6: d_conv=4).
 * Per (batch, channel) with K taps:
 *
 *   a[t] = bias[d] + sum_{k=0}^{K-1} w[d,k] * x[t - (K-1) + k]
 *   u[t] = a[t] * sigmoid(a[t])     (or a[t] without the activation)
 *
 * where x at negative times is the caller's initial conv state
 * (batch, dim, K-1), oldest first, or zero.  The final conv state is the last
 * K-1 inputs of the sequence (older ones from the initial state when
 * L < K-1).  Layouts: x, u (batch, dim, L); w (dim, K); bias (dim).
 */
int oracle_conv1d_fwd(const double* x, const double* w, const double* bias, const double* conv_state_in,
                      double* conv_state_out, double* u, int64_t batch, int64_t dim, int64_t seqlen, int64_t K,
                      int silu_on, int nthreads) {
  if (!x || !w || !u) return 1;
  if (batch < 0 || dim < 0 || seqlen < 0 || K < 1) return 2;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const int64_t BD = batch * dim, S = K - 1;
#pragma omp parallel for schedule(static)
  for (int64_t bd = 0; bd < BD; ++bd) {
    const int64_t d = bd % dim;
    const double* xr = x + bd * seqlen;
    for (int64_t t = 0; t < seqlen; ++t) {
      double acc = bias ? bias[d] : 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const int64_t tt = t - S + k;   /* input time of tap k */
        double xv;
        if (tt >= 0)
          xv = xr[tt];
        else
          xv = conv_state_in ? conv_state_in[bd * S + (S + tt)] : 0.0;
        acc += w[d * K + k] * xv;
      }
      u[bd * seqlen + t] = silu_on ? acc * oracle_sigmoid(acc) : acc;
    }
    if (conv_state_out) {
      for (int64_t i = 0; i < S; ++i) {
        const int64_t tt = seqlen - S + i;
        conv_state_out[bd * S + i] = tt >= 0 ? xr[tt] : (conv_state_in ? conv_state_in[bd * S + (S + tt)] : 0.0);
      }
    }
  }
  return 0;
}
