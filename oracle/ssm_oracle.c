/*
 * ssm_oracle.c -- TEST INFRASTRUCTURE ONLY.  CPU fp64 oracle of the Mamba
 * selective state-space (S6) scan and of its single-token state update.
 *
 * Only tests, the smoke check and the benchmark's CPU-baseline leg use this
 * file.  It shares no code, header, table or helper with the GPU library, and
 * the GPU library never calls it.
 *
 * What it computes (plain definition, one channel at a time, sequential in t;
 * page references are to the five web pages about Mamba this project follows):
 *
 *   Delta_t   = softplus(delta_t + dt_bias[d])    (or delta_t + dt_bias[d]
 *               when softplus is off); softplus(x) = log(1 + e^x)
 *   Abar_t[n] = exp(Delta_t * A[d,n])              ZOH transition: "Mamba
 *               close reading" (jsqmd.com) §1.2; mlqm.cn tutorial §3.2
 *   h_t[n]    = Abar_t[n] * h_{t-1}[n] + Delta_t * B_t[n] * u_t
 *               recurrence h_k = Abar h_{k-1} + Bbar x_k with the first-order
 *               input term Bbar = Delta*B: mlqm.cn tutorial §3.2 and §9.2
 *               (dA = exp(dt*A), dB = dt*B, h = dA*h + dB*x); the
 *               tech.kj168168.com essay §二.1
 *   y_t       = (sum_n C_t[n] * h_t[n] + D[d] * u_t) * silu(z_t)
 *               readout plus skip D*x: the essay §二.1 and tutorial §9.2;
 *               SiLU gate on the SSM branch: junchaoiu.github.io summary
 *               (方法, third step) and tutorial §7.1; silu(z) = z/(1+e^-z)
 *   last[n]   = h_{L-1}[n]
 *
 * h_{-1} = 0 unless an initial state is given.  The decode step is the same
 * update for one t, starting from the caller's state ("AI inference series
 * (14)", wiblog.cn: decode is a single-step recurrent update of a per-request
 * state that is updated in place).
 *
 * Readings where the pages are silent (listed with the others in the design
 * notes): softplus and dt_bias appear on no page -- the exact log(1+e^x) is
 * used and dt_bias is added whether or not softplus is on; D and z are
 * optional (NULL = term absent); the gate multiplies the sum including D*u.
 *
 * Numerics: every input value (fp32, or bf16 widened exactly) is converted to
 * double and all arithmetic is IEEE double with libm exp/log1p.  No
 * -ffast-math.  Channels (b, d) are independent and run in parallel (OpenMP);
 * each channel's loop is sequential, so the result does not depend on the
 * thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Element types of u, delta, z, B, C: 0 = IEEE fp32, 1 = bfloat16 (the upper
 * half of an fp32 word, so widening is exact). */
static double elem(const void* p, int64_t i, int dtype) {
  if (dtype == 0) return (double)((const float*)p)[i];
  uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* softplus(x) = log(1 + e^x), written so that e^x never overflows. */
static double softplus(double x) { return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x)); }

/* silu(z) = z * sigmoid(z) = z / (1 + e^-z); for z << 0, e^-z = inf gives -0. */
static double silu(double z) { return z / (1.0 + exp(-z)); }

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Full-sequence scan.  Layouts (row-major, contiguous): u, delta, z [B,D,L];
 * B, C [B,N,L]; A [D,N]; D, dt_bias [D]; h0, last [.,N].
 *
 * chans: NULL = every channel in order (nchans must be B*D); otherwise a list
 * of flat channel indices b*D + d.  Row k of every per-channel array belongs
 * to channel chans[k]: y[k*L + t], last[k*N + n] (last may be NULL) and the
 * initial state h0[k*N + n] (h0 NULL = zeros).
 */
int oracle_scan(const void* u, const void* delta, const float* A, const void* B, const void* C,
                const float* D, const void* z, const float* dt_bias, int softplus_on, const double* h0,
                int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                const int64_t* chans, int64_t nchans, double* y, double* last, int nthreads) {
  if (batch < 0 || dim < 0 || dstate <= 0 || seqlen < 0 || dstate > 1024) return -2;
  if (!chans && nchans != batch * dim) return -2;
  set_threads(nthreads);
  const int64_t L = seqlen, N = dstate;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t k = 0; k < nchans; ++k) {
    const int64_t ch = chans ? chans[k] : k;
    const int64_t b = ch / dim, d = ch % dim;
    double h[1024];
    for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[k * N + n] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
      const int64_t i = ch * L + t; /* (b*D + d)*L + t */
      const double x = elem(delta, i, dtype) + (dt_bias ? (double)dt_bias[d] : 0.0);
      const double dt = softplus_on ? softplus(x) : x;
      const double ut = elem(u, i, dtype);
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        const int64_t j = (b * N + n) * L + t;
        const double abar = exp(dt * (double)A[d * N + n]);
        h[n] = abar * h[n] + dt * elem(B, j, dtype) * ut;
        acc += elem(C, j, dtype) * h[n];
      }
      double yt = acc + (D ? (double)D[d] * ut : 0.0);
      if (z) yt *= silu(elem(z, i, dtype));
      y[k * L + t] = yt;
    }
    if (last)
      for (int64_t n = 0; n < N; ++n) last[k * N + n] = h[n];
  }
  return 0;
}

/*
 * One decode step.  state_in/state_out [rows,N] double (may alias: the update
 * is in place per channel); u, delta, z [B,D]; B, C [B,N]; y [rows].  Softplus
 * is always applied.  chans as in oracle_scan: row k of y, state_in and
 * state_out belongs to channel chans[k] (NULL: row k is channel k).
 */
int oracle_step(const double* state_in, const void* u, const void* delta, const float* A, const void* B,
                const void* C, const float* D, const void* z, const float* dt_bias, int64_t batch, int64_t dim,
                int64_t dstate, int dtype, const int64_t* chans, int64_t nchans, double* y, double* state_out,
                int nthreads) {
  if (batch < 0 || dim < 0 || dstate <= 0 || dstate > 1024) return -2;
  if (!chans && nchans != batch * dim) return -2;
  set_threads(nthreads);
  const int64_t N = dstate;
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < nchans; ++k) {
    const int64_t ch = chans ? chans[k] : k;
    const int64_t b = ch / dim, d = ch % dim;
    const double x = elem(delta, ch, dtype) + (dt_bias ? (double)dt_bias[d] : 0.0);
    const double dt = softplus(x);
    const double ut = elem(u, ch, dtype);
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double abar = exp(dt * (double)A[d * N + n]);
      const double hn = abar * state_in[k * N + n] + dt * elem(B, b * N + n, dtype) * ut;
      state_out[k * N + n] = hn;
      acc += elem(C, b * N + n, dtype) * hn;
    }
    double yt = acc + (D ? (double)D[d] * ut : 0.0);
    if (z) yt *= silu(elem(z, ch, dtype));
    y[k] = yt;
  }
  return 0;
}

/*
 * Causal depthwise 1-D convolution with an optional SiLU, the step just before the
 * selective SSM in the Mamba block ("Mamba: Linear-Time Sequence Modeling ..."
 * summary (junchaoiu.github.io), 方法 third step: linear expansion, 1-D convolution
 * for local features, SiLU; mlqm.cn tutorial §7.1: causal 1-D convolution then SiLU
 * ahead of the selective SSM).  Per channel (b, d) and step t, with width K:
 *
 *   v_t   = bias[d] + sum_{k=0..K-1} w[d,k] * x[t - (K-1) + k]
 *   out_t = silu(v_t) if silu_on else v_t
 *
 * where x at steps before 0 comes from the caller's convolution state: the K-1
 * inputs preceding this sequence, oldest first (state_in[row*(K-1) + j] is the input
 * at step j - (K-1)); state_in NULL = zeros.  The decode path keeps exactly that
 * window per request ("AI inference series (14)" (wiblog.cn): a decode step keeps
 * only the updated state and the little history the local convolution needs).
 * state_out (may be NULL) receives the K-1 inputs ending at step L-1 -- the state a
 * following call continues from.  Layouts: x, out [B,D,L] (x of `dtype`); w [D,K],
 * bias [D] fp32; states [B*D, K-1] double.  state_in and state_out may alias.
 */
int oracle_conv1d(const void* x, const float* w, const float* bias, const double* state_in, int silu_on,
                  int64_t batch, int64_t dim, int64_t seqlen, int64_t width, int dtype, double* out,
                  double* state_out, int nthreads) {
  if (batch < 0 || dim < 0 || seqlen < 0 || width < 1 || width > 64) return -2;
  set_threads(nthreads);
  const int64_t L = seqlen, K = width, rows = batch * dim;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t d = r % dim;
    double hist[64]; /* inputs at steps -(K-1) .. -1 */
    for (int64_t j = 0; j < K - 1; ++j) hist[j] = state_in ? state_in[r * (K - 1) + j] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
      double v = bias ? (double)bias[d] : 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const int64_t s = t - (K - 1) + k; /* input step */
        const double xs = s >= 0 ? elem(x, r * L + s, dtype) : hist[K - 1 + s];
        v += (double)w[d * K + k] * xs;
      }
      out[r * L + t] = silu_on ? silu(v) : v;
    }
    if (state_out) {
      double nw[64];
      for (int64_t j = 0; j < K - 1; ++j) {
        const int64_t s = L - (K - 1) + j;
        nw[j] = s >= 0 ? elem(x, r * L + s, dtype) : hist[K - 1 + s];
      }
      for (int64_t j = 0; j < K - 1; ++j) state_out[r * (K - 1) + j] = nw[j];
    }
  }
  return 0;
}

/*
 * Backward of the forward scan: the gradients of L = sum dy * y with respect to every
 * input, by the adjoint method ("Mamba close reading" (jsqmd.com), gradient analysis: dL/dA
 * as a sum over t of (dh_t/dA)^T dL/dh_t, computed with the adjoint; the Mamba summary,
 * 方法 second step: the backward pass recomputes the states instead of storing them).
 * Per channel (b, d) and state n, with g_t = silu(z_t) (1 without z) and
 * s_t = sum_n C_t[n] h_t[n] + D u_t (y_t = s_t g_t):
 *
 *   ds_t      = dy_t g_t                       dz_t = dy_t s_t silu'(z_t)
 *   lam_t[n]  = ds_t C_t[n] + Abar_{t+1}[n] lam_{t+1}[n]     (lam after the last step = 0)
 *   du_t      = ds_t D + sum_n lam_t[n] Delta_t B_t[n]
 *   dDelta_t  = sum_n lam_t[n] (h_{t-1}[n] Abar_t[n] A[n] + B_t[n] u_t)
 *   ddelta_t  = dDelta_t * (softplus ? sigmoid(delta_t + dt_bias) : 1)
 *   dA[d,n]  += lam_t[n] h_{t-1}[n] Abar_t[n] Delta_t       dD[d] += ds_t u_t
 *   ddt_bias[d] += ddelta_t                                  dh0[n] = Abar_0[n] lam_0[n]
 *   dB[b,n,t] += lam_t[n] Delta_t u_t            dC[b,n,t] += ds_t h_t[n]   (sums over d)
 *
 * Inputs as oracle_scan plus dy [B,D,L] (dtype).  Outputs (double, any may be NULL except
 * du and ddelta): du, ddelta, dz [B,D,L]; dB, dC [B,N,L]; dA [D,N]; dD, ddt_bias [D];
 * dh0 [B,D,N].  Sums over b and d are taken in index order, so the result does not
 * depend on the thread count.  Sequences up to 2^22 steps.
 */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

int oracle_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                    const float* D, const void* z, const float* dt_bias, int softplus_on, const double* h0,
                    const void* dy, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                    double* du, double* ddelta, double* dz, double* dA, double* dB, double* dC, double* dD,
                    double* ddt_bias, double* dh0, int nthreads) {
  if (batch < 0 || dim < 0 || dstate <= 0 || seqlen < 0 || dstate > 1024 || seqlen > (1 << 22)) return -2;
  if (!du || !ddelta) return -2;
  set_threads(nthreads);
  const int64_t L = seqlen, N = dstate, rows = batch * dim;
  int fail = 0;
  /* per channel: du, ddelta, dz, dh0 and the channel's share of dA, dD, ddt_bias */
  double* pA = (double*)calloc((size_t)(rows * N > 0 ? rows * N : 1), sizeof(double));
  double* pD = (double*)calloc((size_t)(rows > 0 ? rows : 1), sizeof(double));
  double* pb = (double*)calloc((size_t)(rows > 0 ? rows : 1), sizeof(double));
  if (!pA || !pD || !pb) fail = 1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < rows; ++r) {
    if (fail) continue;
    const int64_t b = r / dim, d = r % dim;
    double* H = (double*)malloc((size_t)((L + 1) * N > 0 ? (L + 1) * N : 1) * sizeof(double)); /* h_{t-1} at row t */
    double* DT = (double*)malloc((size_t)(L > 0 ? L : 1) * sizeof(double));
    double* lam = (double*)malloc((size_t)N * sizeof(double));
    if (!H || !DT || !lam) { fail = 1; free(H); free(DT); free(lam); continue; }
    for (int64_t n = 0; n < N; ++n) H[n] = h0 ? h0[r * N + n] : 0.0;
    for (int64_t t = 0; t < L; ++t) { /* forward, keeping every state */
      const int64_t i = r * L + t;
      const double x = elem(delta, i, dtype) + (dt_bias ? (double)dt_bias[d] : 0.0);
      const double dt = softplus_on ? softplus(x) : x;
      DT[t] = dt;
      const double ut = elem(u, i, dtype);
      for (int64_t n = 0; n < N; ++n)
        H[(t + 1) * N + n] = exp(dt * (double)A[d * N + n]) * H[t * N + n] + dt * elem(B, (b * N + n) * L + t, dtype) * ut;
    }
    for (int64_t n = 0; n < N; ++n) lam[n] = 0.0;
    double aD = 0.0, ab = 0.0;
    for (int64_t t = L - 1; t >= 0; --t) { /* adjoint, last step first */
      const int64_t i = r * L + t;
      const double ut = elem(u, i, dtype), dyt = elem(dy, i, dtype), dt = DT[t];
      double s = D ? (double)D[d] * ut : 0.0;
      for (int64_t n = 0; n < N; ++n) s += elem(C, (b * N + n) * L + t, dtype) * H[(t + 1) * N + n];
      double g = 1.0, gp = 0.0;
      if (z) {
        const double zz = elem(z, i, dtype), sg = sigmoid(zz);
        g = zz * sg;
        gp = sg * (1.0 + zz * (1.0 - sg));
      }
      const double ds = dyt * g;
      if (dz) dz[i] = z ? dyt * s * gp : 0.0;
      double dut = D ? ds * (double)D[d] : 0.0, dDt = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        const int64_t j = (b * N + n) * L + t;
        const double an = (double)A[d * N + n], abar = exp(dt * an), bt = elem(B, j, dtype);
        /* lam[n] holds Abar_{t+1} lam_{t+1} here */
        lam[n] = ds * elem(C, j, dtype) + lam[n];
        dut += lam[n] * dt * bt;
        dDt += lam[n] * (H[t * N + n] * abar * an + bt * ut);
        pA[r * N + n] += lam[n] * H[t * N + n] * abar * dt;
        lam[n] *= abar; /* -> Abar_t lam_t for the step before */
      }
      const double x = elem(delta, i, dtype) + (dt_bias ? (double)dt_bias[d] : 0.0);
      const double dx = dDt * (softplus_on ? sigmoid(x) : 1.0);
      du[i] = dut;
      ddelta[i] = dx;
      aD += ds * ut;
      ab += dx;
    }
    if (dh0)
      for (int64_t n = 0; n < N; ++n) dh0[r * N + n] = lam[n];
    pD[r] = aD;
    pb[r] = ab;
    free(H);
    free(DT);
    free(lam);
  }
  if (!fail) {
    for (int64_t d = 0; d < dim; ++d) {
      double sD = 0.0, sb = 0.0;
      for (int64_t b = 0; b < batch; ++b) { sD += pD[b * dim + d]; sb += pb[b * dim + d]; }
      if (dD) dD[d] = sD;
      if (ddt_bias) ddt_bias[d] = sb;
      for (int64_t n = 0; n < N; ++n) {
        double sa = 0.0;
        for (int64_t b = 0; b < batch; ++b) sa += pA[(b * dim + d) * N + n];
        if (dA) dA[d * N + n] = sa;
      }
    }
  }
  free(pA);
  free(pD);
  free(pb);
  if (fail) return -3;
  if (!dB && !dC) return 0;
  /* dB, dC: one task per (b, n); state n alone is a scalar recurrence, summed over d in order */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bn = 0; bn < batch * N; ++bn) {
    if (fail) continue;
    const int64_t b = bn / N, n = bn % N;
    double* hs = (double*)malloc((size_t)((L + 1) > 0 ? (L + 1) : 1) * sizeof(double));
    double* DT = (double*)malloc((size_t)(L > 0 ? L : 1) * sizeof(double));
    if (!hs || !DT) { fail = 1; free(hs); free(DT); continue; }
    for (int64_t t = 0; t < L; ++t) {
      if (dB) dB[(b * N + n) * L + t] = 0.0;
      if (dC) dC[(b * N + n) * L + t] = 0.0;
    }
    for (int64_t d = 0; d < dim; ++d) {
      const int64_t r = b * dim + d;
      const double an = (double)A[d * N + n];
      hs[0] = h0 ? h0[r * N + n] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        const int64_t i = r * L + t;
        const double x = elem(delta, i, dtype) + (dt_bias ? (double)dt_bias[d] : 0.0);
        const double dt = softplus_on ? softplus(x) : x;
        DT[t] = dt;
        hs[t + 1] = exp(dt * an) * hs[t] + dt * elem(B, (b * N + n) * L + t, dtype) * elem(u, i, dtype);
      }
      double lam = 0.0;
      for (int64_t t = L - 1; t >= 0; --t) {
        const int64_t i = r * L + t, j = (b * N + n) * L + t;
        const double dyt = elem(dy, i, dtype);
        double g = 1.0;
        if (z) { const double zz = elem(z, i, dtype); g = zz * sigmoid(zz); }
        const double ds = dyt * g;
        lam = ds * elem(C, j, dtype) + lam;
        if (dB) dB[j] += lam * DT[t] * elem(u, i, dtype);
        if (dC) dC[j] += ds * hs[t + 1];
        lam *= exp(DT[t] * an);
      }
    }
    free(hs);
    free(DT);
  }
  return fail ? -3 : 0;
}
