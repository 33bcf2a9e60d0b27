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
