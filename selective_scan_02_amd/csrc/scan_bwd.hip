// scan_bwd.hip -- backward of the selective scan on gfx950: the gradients of a scalar
// loss through y, given dy = dLoss/dy.
//
// The pages describe the forward scan and note that the fused kernel recomputes the
// intermediate states in the backward pass instead of storing them (Mamba summary
// (junchaoiu.github.io), 方法 step 2: hardware-aware algorithm, recomputation; mlqm.cn
// tutorial §6).  The gradients themselves follow from the recurrence by the adjoint
// (reverse-mode) method; with ds_t = dy_t * silu(z_t) and the adjoint
//   lam_t[n] = ds_t C_t[n] + Abar_{t+1}[n] lam_{t+1}[n]          (lam_L = 0)
// they are
//   du_t     = ds_t D + Delta_t sum_n lam_t[n] B_t[n]
//   dDelta_t = sum_n lam_t[n] (Abar_t[n] h_{t-1}[n] A[n] + B_t[n] u_t)
//   ddelta_t = dDelta_t * sigmoid(delta_t + dt_bias)  (softplus on; else dDelta_t)
//   dz_t     = dy_t s_t silu'(z_t),  s_t = sum_n C_t[n] h_t[n] + D u_t
//   dA[n]   += lam_t[n] Abar_t[n] h_{t-1}[n] Delta_t   dD += ds_t u_t   ddt_bias += ddelta_t
//   dB_t[n]  = sum over channels of lam_t[n] Delta_t u_t
//   dC_t[n]  = sum over channels of ds_t h_t[n]
//   dh_{-1}  = Abar_0 lam_0.
//
// Work decomposition (one wave = 64 consecutive channels of one batch row, one channel
// per lane, all dstate states in registers, as in the generic forward kernels):
//   1. checkpoint pass: each sequence segment runs the forward recurrence from h = 0 and
//      stores its state (and running sum of Delta) at the start of every chunk of T
//      steps, plus the segment's end state and total sum of Delta;
//   2. carry pass: the segment end states become each segment's incoming state (the
//      same combination as the forward's segment carry);
//   3. adjoint aggregate pass and reverse carry (only with several segments): each
//      segment but the first runs the adjoint from zero, right to left; a reverse carry
//      turns these into the adjoint entering each segment from its right.  The adjoint
//      recurrence is linear, so a segment's contribution combines as
//      Abar-product * incoming + local, the product being exp(A * sum Delta);
//   4. main pass: each segment walks its chunks right to left.  A chunk's starting state
//      is local checkpoint + exp(A * local sum Delta) * segment incoming state; the chunk
//      reruns the forward over its T steps keeping every h_{t-1} in registers, then runs
//      the adjoint back over them.  Per-channel gradients are written directly; the
//      sums over channels (dB, dC) are reduced across the wave's 64 lanes through LDS
//      and written as one partial per (channel group, batch row, n, t); the sums over
//      time and batch (dA, dD, ddt_bias) are kept per (segment, channel);
//   5. reduction passes: partials are summed in a fixed order (deterministic).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {
namespace {

constexpr int kWave = 64;

// Steps per chunk: the chunk's h_{t-1} for every state stays in registers (T * N of them).
template <int N>
struct Chunk {
  static constexpr int T = N <= 8 ? 16 : N == 16 ? 8 : N == 32 ? 2 : 1;
};

struct BwdArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* dt_bias;
  const float* h0;
  const void* dy;
  void* du;
  void* ddelta;
  void* dz;
  float* dh0;
  float* ck_h;    // [chunks, chans, N]  local state at each chunk start (segment-relative)
  float* ck_dt;   // [chunks, chans]     local sum of Delta before each chunk
  float* seg_h;   // [S, chans, N]       segment end state from 0, then incoming state
  float* seg_dt;  // [S, chans]          sum of Delta over the segment
  float* seg_l;   // [S, chans, N]       adjoint aggregate, then adjoint entering from the right
  float* pB;      // [groups, batch, N, L]  dB summed over one channel group
  float* pC;      // [groups, batch, N, L]
  float* pA;      // [S, chans, N]
  float* pD;      // [S, chans]
  float* pbias;   // [S, chans]
  int64_t batch, dim, seqlen, seg_len, chans;
  int groups, nseg, softplus;
  int ddelta_f32;  // ddelta is written in fp32 whatever the input dtype (for callers that sum it)
  // main pass on the interval plan (iunits > 0)
  int* ticket;    // 1 counter
  int* flags;     // [chains, scanner waves] hand-over flags
  float* hand_l;  // [chains, N, 64] the adjoint handed over at a split point
  int64_t wlen;   // chunks per interval
  int iunits;     // intervals (workgroups); 0: the segment plan
  int max_polls;  // bound of a hand-over wait
  int publish;    // 0 only under the test hook: split points never publish
  float* clear;        // the checkpoint pass zeroes [clear, clear + clear_n) (the main pass's ticket and
  int64_t clear_n;     // flags) on its way, so no launch of its own clears them before the main pass
};

// Hand-over waits of the main pass that gave up (bwd_handover_failures).
static __device__ unsigned int bwd_handover_giveups;

struct Lane {
  int lane;
  int64_t b, d, dd, ch;
  bool active;
};

__device__ __forceinline__ Lane lane_of(const BwdArgs& a) {
  Lane l;
  l.lane = threadIdx.x;
  l.b = blockIdx.x / a.groups;
  l.d = (int64_t)(blockIdx.x % a.groups) * kWave + l.lane;
  l.active = l.d < a.dim;
  l.dd = l.active ? l.d : a.dim - 1;
  l.ch = l.b * a.dim + l.dd;
  return l;
}

__device__ __forceinline__ float step_size(float x, int sp) { return sp ? softplus(x) : x; }

// sigmoid(x) = 1 / (1 + e^-x); e^-x = inf for x << 0 gives 0.
__device__ __forceinline__ float sigmoid(float x) { return rcp(1.0f + ex2(-x * kLog2e)); }

// 1. Checkpoint pass.
template <int N, typename T>
__global__ __launch_bounds__(kWave) void bwd_checkpoint_kernel(BwdArgs a) {
  constexpr int CT = Chunk<N>::T;
  const Lane l = lane_of(a);
  const int seg = blockIdx.y;
  const int64_t L = a.seqlen;
  const int64_t t0 = (int64_t)seg * a.seg_len;
  const int64_t t1 = std::min(t0 + a.seg_len, L);
  const T* __restrict__ u = (const T*)a.u + l.ch * L;
  const T* __restrict__ dl = (const T*)a.delta + l.ch * L;
  const T* __restrict__ Bp = (const T*)a.B + l.b * N * L;
  float A2[N], h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    A2[n] = a.A[l.dd * N + n] * kLog2e;
    h[n] = 0.0f;
  }
  const float bias = a.dt_bias ? a.dt_bias[l.dd] : 0.0f;
  float cum = 0.0f;
  for (int64_t t = t0; t < t1; ++t) {
    if (t > t0 && (t - t0) % CT == 0 && l.active) {
      const int64_t kg = t / CT;
#pragma unroll
      for (int n = 0; n < N; ++n) a.ck_h[(kg * a.chans + l.ch) * N + n] = h[n];
      a.ck_dt[kg * a.chans + l.ch] = cum;
    }
    const float dt = step_size(ld(dl, t) + bias, a.softplus);
    const float du = dt * ld(u, t);
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = __builtin_fmaf(ex2(dt * A2[n]), h[n], du * ld(Bp, (int64_t)n * L + t));
    cum += dt;
  }
  if (!l.active) return;
#pragma unroll
  for (int n = 0; n < N; ++n) a.seg_h[((int64_t)seg * a.chans + l.ch) * N + n] = h[n];
  a.seg_dt[(int64_t)seg * a.chans + l.ch] = cum;
}

constexpr int kCarryBatch = 16;

// 2. Forward carry, one thread per (channel, n), in place over seg_h.
__global__ __launch_bounds__(256) void bwd_fwd_carry_kernel(float* seg_h, const float* seg_dt, const float* A,
                                                            const float* h0, int64_t chans, int64_t dim, int N,
                                                            int nseg) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= chans * N) return;
  const int64_t ch = i / N;
  const float A2 = A[(ch % dim) * N + (i % N)] * kLog2e;
  float h = h0 ? h0[i] : 0.0f;
  // 16 segments at a time, their loads all in flight before the first is used
  for (int s0 = 0; s0 < nseg; s0 += kCarryBatch) {
    const int nb = nseg - s0 < kCarryBatch ? nseg - s0 : kCarryBatch;
    float agg[kCarryBatch], sdt[kCarryBatch];
#pragma unroll
    for (int k = 0; k < kCarryBatch; ++k)
      if (k < nb) {
        agg[k] = seg_h[(int64_t)(s0 + k) * chans * N + i];
        sdt[k] = seg_dt[(int64_t)(s0 + k) * chans + ch];
      }
#pragma unroll
    for (int k = 0; k < kCarryBatch; ++k)
      if (k < nb) {
        seg_h[(int64_t)(s0 + k) * chans * N + i] = h;
        h = __builtin_fmaf(ex2(A2 * sdt[k]), h, agg[k]);
      }
  }
}

// 3a. Adjoint aggregate of segments 1 .. S-1 (blockIdx.y + 1): the adjoint from zero at the
// segment's right end, carried through the segment's first transition, Abar_{t0} lam_{t0}.
template <int N, typename T>
__global__ __launch_bounds__(kWave) void bwd_adjoint_aggregate_kernel(BwdArgs a) {
  const Lane l = lane_of(a);
  const int seg = blockIdx.y + 1;
  const int64_t L = a.seqlen;
  const int64_t t0 = (int64_t)seg * a.seg_len;
  const int64_t t1 = std::min(t0 + a.seg_len, L);
  const T* __restrict__ dl = (const T*)a.delta + l.ch * L;
  const T* __restrict__ dy = (const T*)a.dy + l.ch * L;
  const T* __restrict__ zz = a.z ? (const T*)a.z + l.ch * L : nullptr;
  const T* __restrict__ Cp = (const T*)a.C + l.b * N * L;
  float A2[N], lam[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    A2[n] = a.A[l.dd * N + n] * kLog2e;
    lam[n] = 0.0f;
  }
  const float bias = a.dt_bias ? a.dt_bias[l.dd] : 0.0f;
  for (int64_t t = t1 - 1; t >= t0; --t) {
    const float dt = step_size(ld(dl, t) + bias, a.softplus);
    float ds = ld(dy, t);
    if (zz) ds *= silu(ld(zz, t));
#pragma unroll
    for (int n = 0; n < N; ++n)
      lam[n] = ex2(dt * A2[n]) * __builtin_fmaf(ds, ld(Cp, (int64_t)n * L + t), lam[n]);
  }
  if (!l.active) return;
#pragma unroll
  for (int n = 0; n < N; ++n) a.seg_l[((int64_t)seg * a.chans + l.ch) * N + n] = lam[n];
}

// 3b. Reverse carry, one thread per (channel, n): seg_l[s] becomes the adjoint term that
// enters segment s from the right (zero for the last segment).
__global__ __launch_bounds__(256) void bwd_adjoint_carry_kernel(float* seg_l, const float* seg_dt, const float* A,
                                                                int64_t chans, int64_t dim, int N, int nseg) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= chans * N) return;
  const int64_t ch = i / N;
  const float A2 = A[(ch % dim) * N + (i % N)] * kLog2e;
  float mu = 0.0f;
  // 16 segments at a time (last first), their loads all in flight before the first is used
  for (int s0 = nseg - 1; s0 >= 0; s0 -= kCarryBatch) {
    const int nb = s0 + 1 < kCarryBatch ? s0 + 1 : kCarryBatch;
    float loc[kCarryBatch], sdt[kCarryBatch];
#pragma unroll
    for (int k = 0; k < kCarryBatch; ++k)
      if (k < nb) {
        const int s = s0 - k;
        loc[k] = s > 0 ? seg_l[(int64_t)s * chans * N + i] : 0.0f;
        sdt[k] = seg_dt[(int64_t)s * chans + ch];
      }
#pragma unroll
    for (int k = 0; k < kCarryBatch; ++k)
      if (k < nb) {
        seg_l[(int64_t)(s0 - k) * chans * N + i] = mu;
        mu = __builtin_fmaf(ex2(A2 * sdt[k]), mu, loc[k]);
      }
  }
}

// Sum of v[n] over the wave's 64 lanes, for every n.  Each lane writes its N values into
// red[n][lane]; lane (n = lane / P, part q = lane % P), P = 64 / N lanes per value, then
// adds N consecutive entries of row n and the P parts are combined across lanes.  Every
// lane of value n's group returns its sum.
template <int N>
__device__ __forceinline__ float wave_sum(const float (&v)[N], float* red) {
  constexpr int P = kWave / N;
  const int lane = threadIdx.x;
#pragma unroll
  for (int n = 0; n < N; ++n) red[n * kWave + lane] = v[n];
  __syncthreads();
  const float* row = red + (lane / P) * kWave + (lane % P) * N;
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) s += row[i];
#pragma unroll
  for (int m = 1; m < P; m <<= 1) s += __shfl_xor(s, m);
  __syncthreads();
  return s;
}

// 4. Main pass: one wave per (channel group, batch row) and segment.
template <int N, typename T>
__global__ __launch_bounds__(kWave) void bwd_main_kernel(BwdArgs a) {
  constexpr int CT = Chunk<N>::T;
  constexpr int P = kWave / N;
  __shared__ float red[N * kWave];
  const Lane l = lane_of(a);
  const int seg = blockIdx.y;
  const int64_t L = a.seqlen;
  const int64_t t0 = (int64_t)seg * a.seg_len;
  const int64_t t1 = std::min(t0 + a.seg_len, L);
  const int64_t grp = blockIdx.x % a.groups;
  const T* __restrict__ u = (const T*)a.u + l.ch * L;
  const T* __restrict__ dl = (const T*)a.delta + l.ch * L;
  const T* __restrict__ dy = (const T*)a.dy + l.ch * L;
  const T* __restrict__ zz = a.z ? (const T*)a.z + l.ch * L : nullptr;
  const T* __restrict__ Bp = (const T*)a.B + l.b * N * L;
  const T* __restrict__ Cp = (const T*)a.C + l.b * N * L;
  T* __restrict__ du_o = (T*)a.du + l.ch * L;
  T* __restrict__ dl_o = (T*)a.ddelta + l.ch * L;
  float* __restrict__ dl_of = (float*)a.ddelta + l.ch * L;  // the same row when ddelta is fp32
  T* __restrict__ dz_o = a.z ? (T*)a.dz + l.ch * L : nullptr;
  // this lane's slot in the reduced sums: value n_red, stored by the group's first lane
  const int n_red = l.lane / P;
  const bool red_store = (l.lane % P) == 0;
  float* __restrict__ pB = a.pB + ((grp * a.batch + l.b) * N + n_red) * L;
  float* __restrict__ pC = a.pC + ((grp * a.batch + l.b) * N + n_red) * L;

  float A2[N], hin[N], lam[N], dA[N];
  const bool multi = a.nseg > 1;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    A2[n] = a.A[l.dd * N + n] * kLog2e;
    const int64_t k = ((int64_t)seg * a.chans + l.ch) * N + n;
    hin[n] = multi ? a.seg_h[k] : (a.h0 ? a.h0[l.ch * N + n] : 0.0f);
    lam[n] = (multi && l.active) ? a.seg_l[k] : 0.0f;
    dA[n] = 0.0f;
  }
  const float bias = a.dt_bias ? a.dt_bias[l.dd] : 0.0f;
  const float Dd = a.D ? a.D[l.dd] : 0.0f;
  float accD = 0.0f, accbias = 0.0f;

  const int nck = (int)((t1 - t0 + CT - 1) / CT);
  for (int k = nck - 1; k >= 0; --k) {
    const int64_t tc = t0 + (int64_t)k * CT;
    const int tl = (int)std::min<int64_t>(CT, t1 - tc);
    float h[N];
    if (k == 0) {
#pragma unroll
      for (int n = 0; n < N; ++n) h[n] = hin[n];
    } else {
      const int64_t kg = tc / CT;
      const float c = a.ck_dt[kg * a.chans + l.ch];
#pragma unroll
      for (int n = 0; n < N; ++n)
        h[n] = __builtin_fmaf(ex2(A2[n] * c), hin[n], a.ck_h[(kg * a.chans + l.ch) * N + n]);
    }
    float hp[CT][N], dts[CT], us[CT], dss[CT], sgx[CT];
    // forward over the chunk: states, readout, gate gradient, dC partials
#pragma unroll
    for (int i = 0; i < CT; ++i) {
      if (i < tl) {
        const int64_t t = tc + i;
        const float x = ld(dl, t) + bias;
        const float dt = step_size(x, a.softplus);
        const float ut = ld(u, t);
        const float dut = dt * ut;
        float s = 0.0f;
#pragma unroll
        for (int n = 0; n < N; ++n) {
          hp[i][n] = h[n];
          h[n] = __builtin_fmaf(ex2(dt * A2[n]), h[n], dut * ld(Bp, (int64_t)n * L + t));
          s = __builtin_fmaf(ld(Cp, (int64_t)n * L + t), h[n], s);
        }
        s = __builtin_fmaf(Dd, ut, s);
        const float g = ld(dy, t);
        float ds = g;
        if (zz) {
          const float zv = ld(zz, t);
          const float sg = sigmoid(zv);
          ds = g * zv * sg;
          if (l.active) st(dz_o, t, g * s * sg * __builtin_fmaf(zv, 1.0f - sg, 1.0f));
        }
        if (!l.active) ds = 0.0f;
        dts[i] = dt;
        us[i] = ut;
        dss[i] = ds;
        sgx[i] = a.softplus ? sigmoid(x) : 1.0f;
        float v[N];
#pragma unroll
        for (int n = 0; n < N; ++n) v[n] = ds * h[n];
        const float r = wave_sum<N>(v, red);
        if (red_store) pC[t] = r;
      }
    }
    // adjoint back over the chunk
#pragma unroll
    for (int i = CT - 1; i >= 0; --i) {
      if (i < tl) {
        const int64_t t = tc + i;
        const float dt = dts[i], ut = us[i], ds = dss[i];
        const float dut = dt * ut;
        float accB = 0.0f, accQ = 0.0f, v[N];
#pragma unroll
        for (int n = 0; n < N; ++n) {
          const float lt = __builtin_fmaf(ds, ld(Cp, (int64_t)n * L + t), lam[n]);
          accB = __builtin_fmaf(lt, ld(Bp, (int64_t)n * L + t), accB);
          v[n] = lt * dut;
          const float lp = ex2(dt * A2[n]) * lt;  // Abar_t lam_t, carried to step t-1
          const float q = lp * hp[i][n];
          accQ = __builtin_fmaf(q, A2[n], accQ);
          dA[n] = __builtin_fmaf(q, dt, dA[n]);
          lam[n] = lp;
        }
        const float r = wave_sum<N>(v, red);
        if (red_store) pB[t] = r;
        const float dDelta = __builtin_fmaf(accQ, kLn2, ut * accB);
        const float ddl = dDelta * sgx[i];
        if (l.active) {
          st(du_o, t, __builtin_fmaf(dt, accB, ds * Dd));
          if (a.ddelta_f32)
            dl_of[t] = ddl;
          else
            st(dl_o, t, ddl);
        }
        accD = __builtin_fmaf(ds, ut, accD);
        accbias += ddl;
      }
    }
  }
  if (!l.active) return;
#pragma unroll
  for (int n = 0; n < N; ++n) a.pA[((int64_t)seg * a.chans + l.ch) * N + n] = dA[n];
  a.pD[(int64_t)seg * a.chans + l.ch] = accD;
  a.pbias[(int64_t)seg * a.chans + l.ch] = accbias;
  if (seg == 0 && a.dh0) {
#pragma unroll
    for (int n = 0; n < N; ++n) a.dh0[l.ch * N + n] = lam[n];
  }
}

// 5a. dB, dC: sum of the channel-group partials, one thread per (batch row, n, t).
template <typename T>
__global__ __launch_bounds__(256) void bwd_bc_reduce_kernel(const float* pB, const float* pC, T* dB, T* dC,
                                                            int64_t count, int groups) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= count) return;
  float sb = 0.0f, sc = 0.0f;
  for (int g = 0; g < groups; ++g) {
    sb += pB[(int64_t)g * count + i];
    sc += pC[(int64_t)g * count + i];
  }
  st(dB, i, sb);
  st(dC, i, sc);
}

// 5a'. The same with 16-byte loads when count is a multiple of 4: a thread sums 4 consecutive
// outputs over a quarter of the groups (g = quarter, quarter + 4, ...), and the quarters' sums meet
// in LDS in a fixed order, so the result is still reproducible bit for bit.
template <typename T>
__device__ __forceinline__ void bc_reduce4(const float* pB, const float* pC, T* dB, T* dC, int64_t count, int groups,
                                           int64_t blk) {
  __shared__ float4 sb[4][64], sc[4][64];
  const int qd = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int64_t i4 = (blk * 64 + lane) * 4;
  float4 b = make_float4(0.f, 0.f, 0.f, 0.f), c = b;
  if (i4 < count) {
    for (int g = qd; g < groups; g += 4) {
      const float4 vb = *(const float4*)(pB + (int64_t)g * count + i4);
      const float4 vc = *(const float4*)(pC + (int64_t)g * count + i4);
      b.x += vb.x; b.y += vb.y; b.z += vb.z; b.w += vb.w;
      c.x += vc.x; c.y += vc.y; c.z += vc.z; c.w += vc.w;
    }
  }
  sb[qd][lane] = b;
  sc[qd][lane] = c;
  __syncthreads();
  if (qd != 0 || i4 >= count) return;
  float ob[4] = {b.x, b.y, b.z, b.w}, oc[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int k = 1; k < 4; ++k) {
    const float4 xb = sb[k][lane], xc = sc[k][lane];
    ob[0] += xb.x; ob[1] += xb.y; ob[2] += xb.z; ob[3] += xb.w;
    oc[0] += xc.x; oc[1] += xc.y; oc[2] += xc.z; oc[3] += xc.w;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    st(dB, i4 + j, ob[j]);
    st(dC, i4 + j, oc[j]);
  }
}

// 5b. dA, dD, ddt_bias: sum over segments and batch rows, one thread per (d, n).
__device__ __forceinline__ void param_reduce(const float* pA, const float* pD, const float* pbias, float* dA,
                                             float* dD, float* dbias, int64_t batch, int64_t dim, int N, int nseg,
                                             int64_t blk) {
  const int64_t i = blk * 256 + threadIdx.x;
  if (i >= dim * N) return;
  const int64_t d = i / N;
  const int n = (int)(i % N);
  const int64_t chans = batch * dim;
  float sa = 0.0f, sd = 0.0f, sb = 0.0f;
  for (int s = 0; s < nseg; ++s)
    for (int64_t b = 0; b < batch; ++b) {
      const int64_t ch = (int64_t)s * chans + b * dim + d;
      sa += pA[ch * N + n];
      if (n == 0) {
        sd += pD[ch];
        sb += pbias[ch];
      }
    }
  dA[i] = sa;
  if (n == 0) {
    if (dD) dD[d] = sd;
    if (dbias) dbias[d] = sb;
  }
}

__global__ __launch_bounds__(256) void bwd_param_reduce_kernel(const float* pA, const float* pD, const float* pbias,
                                                               float* dA, float* dD, float* dbias, int64_t batch,
                                                               int64_t dim, int N, int nseg) {
  param_reduce(pA, pD, pbias, dA, dD, dbias, batch, dim, N, nseg, blockIdx.x);
}

// 5a' and 5b in one grid: blocks 0 .. nbc-1 sum dB and dC, the rest dA, dD and ddt_bias (the two need
// nothing of each other; one launch fewer after the main pass).
template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float* pB, const float* pC, T* dB, T* dC, int64_t count,
                                                         int groups, int64_t nbc, const float* pA, const float* pD,
                                                         const float* pbias, float* dA, float* dD, float* dbias,
                                                         int64_t batch, int64_t dim, int N, int nseg) {
  if ((int64_t)blockIdx.x < nbc)
    bc_reduce4(pB, pC, dB, dC, count, groups, blockIdx.x);
  else
    param_reduce(pA, pD, pbias, dA, dD, dbias, batch, dim, N, nseg, (int64_t)blockIdx.x - nbc);
}

// Zero-length sequence: every gradient is zero.  A fill kernel rather than a memset node.
__global__ __launch_bounds__(256) void bwd_zero_kernel(float* p, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// ---------------------------------------------------------------- fast path
// Rows that are whole 16-byte pieces (seqlen a multiple of 8, 16-byte aligned tensors) and
// dstate in {8, 16, 32, 64}.  Each lane moves the 8 steps of its channel's chunk with one or
// two 16-byte loads and stores; B and C are staged per chunk in LDS and read back as
// broadcasts.  The main pass splits the states over N/8 waves of 8 states each (a workgroup
// per channel group), which halves the registers a lane needs for the chunk's states; the
// per-channel sums over n are combined across the waves through LDS.
#ifndef SSM_BWD_WAVES_PER_SIMD
#define SSM_BWD_WAVES_PER_SIMD 1
#endif
#ifndef SSM_BWD_RECOMPUTE_ABAR
#define SSM_BWD_RECOMPUTE_ABAR 1
#endif
constexpr int kCT = 8;   // steps per chunk
constexpr int kSPW = 8;  // states per wave in the main pass

template <typename T>
struct Row8;
template <>
struct Row8<__bf16> {
  struct Raw {
    uint4 v;
  };
  static __device__ __forceinline__ Raw fetch(const __bf16* p) { return Raw{*(const uint4*)p}; }
  static __device__ __forceinline__ void unpack(const Raw& r, float (&v)[8]) {
    const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(__bf16* p, const float (&v)[8]) {
    __bf16 t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = (__bf16)v[i];
    uint4 r;
    __builtin_memcpy(&r, t, sizeof r);
    *(uint4*)p = r;
  }
};
template <>
struct Row8<float> {
  struct Raw {
    float4 a, b;
  };
  static __device__ __forceinline__ Raw fetch(const float* p) {
    return Raw{((const float4*)p)[0], ((const float4*)p)[1]};
  }
  static __device__ __forceinline__ void unpack(const Raw& r, float (&v)[8]) {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w; v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[8]) {
    ((float4*)p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    ((float4*)p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// Per-channel input rows are staged through LDS in tiles of kSC steps for the 64 channels of a
// group: consecutive threads take consecutive 16-byte pieces along a row, so every row segment
// is read once and whole (a lane reading only its own row, 16 bytes at a time, leaves most of
// each cache line to be fetched again by later chunks once other rows have evicted it).
#ifndef SSM_BWD_PRE_TILE
#define SSM_BWD_PRE_TILE 32
#endif
#ifndef SSM_BWD_MAIN_TILE
#define SSM_BWD_MAIN_TILE 32
#endif
constexpr int kSC = SSM_BWD_PRE_TILE;    // steps per staged tile of the pre-passes
constexpr int kSCM = SSM_BWD_MAIN_TILE;  // and of the main pass
constexpr int kSCG = kSC > kSCM ? kSC : kSCM;  // segments are whole tiles of both
static_assert(kSC % 8 == 0 && kSCM % 8 == 0 && kSCG % kSC == 0 && kSCG % kSCM == 0, "tiles of whole chunks");
template <typename T, int SC = kSC>
struct Tile {
  static constexpr int kPiece = 16 / (int)sizeof(T);              // elements per 16-byte piece
  static constexpr int kRow = SC + kPiece;                        // padded row (elements)
  static constexpr int kPieces = SC / kPiece;                     // pieces per row
};

// Stage steps [ts0, ts1) (a multiple of 8, at most kSC) of the first `nt` of the NT tensors: rows
// of the 64 channels of group `grp` of batch row `b` (channels past the end repeat the last one).
// NTH threads take a tensor's pieces in rounds of up to 4 per thread; a round's loads are all issued
// before the first is written to LDS.
template <typename T, int NTH, int NT, int SC = kSC>
__device__ __forceinline__ void stage_rows(T (*tile)[kWave][SC + 16 / sizeof(T)], const T* const (&bases)[NT], int nt,
                                           const BwdArgs& a, int64_t b, int64_t grp, int64_t ts0, int64_t ts1,
                                           int tid) {
  constexpr int P = Tile<T, SC>::kPieces, E = Tile<T, SC>::kPiece, PER = kWave * P;
  constexpr int R = (PER + NTH - 1) / NTH < 4 ? (PER + NTH - 1) / NTH : 4;
  asm volatile("" : "+v"(tid));  // addresses are recomputed per call, not held across the caller's loop
#pragma unroll
  for (int kk = 0; kk < NT; ++kk) {
    if (kk >= nt) break;
#pragma unroll 1
    for (int base = 0; base < PER; base += NTH * R) {
      uint4 v[R];
      bool ok[R];
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const int pc = base + k * NTH + tid;
        const int r = (pc / P) % kWave, pi = pc % P;
        const int64_t ts = ts0 + (int64_t)pi * E;
        ok[k] = pc < PER && ts < ts1;
        const int64_t ch = b * a.dim + std::min<int64_t>(grp * kWave + r, a.dim - 1);
        v[k] = *(const uint4*)(bases[kk] + ch * a.seqlen + (ok[k] ? ts : ts0));
      }
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const int pc = base + k * NTH + tid;
        if (ok[k]) *(uint4*)&tile[kk][(pc / P) % kWave][(pc % P) * E] = v[k];
      }
    }
  }
}

// The same tiles taken in two halves, for the single-wave passes: fetch() loads the next tile's
// pieces into registers while the current tile is computed, store() writes them to LDS when the
// tile starts, so the loads' latency is hidden behind a tile of work.
template <typename T, int NT>
struct TilePrefetch {
  static constexpr int P = Tile<T>::kPieces, E = Tile<T>::kPiece, PER = kWave * P, R = PER / kWave;
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  u32x4 v[NT][R];
  __device__ __forceinline__ void fetch(const T* const (&bases)[NT], int nt, const BwdArgs& a, int64_t b,
                                        int64_t grp, int64_t ts0, int64_t ts1, int lane) {
    asm volatile("" : "+v"(lane));  // addresses are recomputed per call, not held across the caller's loop
#pragma unroll
    for (int kk = 0; kk < NT; ++kk) {
      if (kk >= nt) break;
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const int pc = k * kWave + lane;
        const int r = pc / P, pi = pc % P;
        const int64_t ts = ts0 + (int64_t)pi * E;
        const int64_t ch = b * a.dim + std::min<int64_t>(grp * kWave + r, a.dim - 1);
        v[kk][k] = *(const u32x4*)(bases[kk] + ch * a.seqlen + (ts < ts1 ? ts : ts0));
      }
    }
  }
  __device__ __forceinline__ void store(T (*tile)[kWave][Tile<T>::kRow], int nt, int64_t ts0, int64_t ts1,
                                        int lane) const {
#pragma unroll
    for (int kk = 0; kk < NT; ++kk) {
      if (kk >= nt) break;
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const int pc = k * kWave + lane;
        if (ts0 + (int64_t)(pc % P) * E < ts1) *(u32x4*)&tile[kk][pc / P][(pc % P) * E] = v[kk][k];
      }
    }
  }
};

// Cross-lane sums without LDS.  v_permlane32_swap exchanges lanes 32..63 of its first operand
// with lanes 0..31 of its second, v_permlane16_swap the odd 16-lane rows of the first with the
// even rows of the second; adding the two swapped registers halves the lanes a sum spans.
__device__ __forceinline__ float swap_sum32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_sum16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum of v[j] over the 64 lanes for j = 0..7, as a reduce-scatter: two swaps fold the halves
// and the rows, a select plus a row rotation by 8 folds the half-rows, and three DPP adds
// (half-row mirror, quad swaps by 2 and by 1) finish inside groups of 8 lanes.  Lane l ends
// with the sum of v[j], j = 4 * bit3(l) + 2 * bit4(l) + bit5(l).
__device__ __forceinline__ int reduce8_index(int lane) {
  return ((lane >> 3) & 1) * 4 + ((lane >> 4) & 1) * 2 + ((lane >> 5) & 1);
}
__device__ __forceinline__ float reduce8(const float (&v)[8], bool hi8) {
  const float x0 = swap_sum32(v[0], v[1]), x1 = swap_sum32(v[2], v[3]);
  const float x2 = swap_sum32(v[4], v[5]), x3 = swap_sum32(v[6], v[7]);
  const float y0 = swap_sum16(x0, x1), y1 = swap_sum16(x2, x3);
  const float keep = hi8 ? y1 : y0, send = hi8 ? y0 : y1;
  float z = keep + dpp<0x128>(send);  // row_ror:8
  z += dpp<0x141>(z);                 // row_half_mirror
  z += dpp<0x4E>(z);                  // quad_perm [2,3,0,1]
  z += dpp<0xB1>(z);                  // quad_perm [1,0,3,2]
  return z;
}

// LDS of the fast pre-passes, which run in one launch: the checkpoint pass takes B rows and
// two input tiles (u, delta), the adjoint aggregate C rows and three (delta, dy, z).
template <int N, typename T>
struct PreLds {
  static constexpr int kRows = kCT * N * (int)sizeof(float);
  static constexpr int kTile = kWave * Tile<T>::kRow * (int)sizeof(T);
  static constexpr int kBytes = kRows + 3 * kTile;
};

// 1'. Checkpoint pass, 16-byte rows: segment `seg` of this workgroup's channel group.
// UNI: every channel's A row holds one value (the SSD form), so a step's Abar is one exp for all states
// (the same values as the general form computes).
template <int N, typename T, bool UNI = false>
__device__ __forceinline__ void fbwd_checkpoint(const BwdArgs& a, int seg, unsigned char* lds) {
  using TL = Tile<T>;
  float(*sB)[N] = reinterpret_cast<float(*)[N]>(lds);
  T(*sIn)[kWave][TL::kRow] = reinterpret_cast<T(*)[kWave][TL::kRow]>(lds + PreLds<N, T>::kRows);  // u, delta
  const Lane l = lane_of(a);
  const int64_t grp = blockIdx.x % a.groups;
  const int64_t L = a.seqlen;
  const int64_t t0 = (int64_t)seg * a.seg_len;
  const int64_t t1 = std::min(t0 + a.seg_len, L);
  const T* __restrict__ Bp = (const T*)a.B + l.b * N * L;
  const T* const bases[2] = {(const T*)a.u, (const T*)a.delta};
  float A2[N], h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    A2[n] = a.A[l.dd * N + n] * kLog2e;
    h[n] = 0.0f;
  }
  const float bias = a.dt_bias ? a.dt_bias[l.dd] : 0.0f;
  float cum = 0.0f;
  // the next chunk's B rows are fetched while the current one is computed
  using Raw = typename Row8<T>::Raw;
  Raw nb{};
  const T* brow = Bp + (int64_t)(l.lane < N ? l.lane : 0) * L;
  if (l.lane < N) nb = Row8<T>::fetch(brow + t0);
  // bf16 tiles are prefetched a tile ahead in registers (fp32 tiles would take twice the registers)
  constexpr bool kPre = sizeof(T) == 2;
  TilePrefetch<T, 2> pre;
  if constexpr (kPre) pre.fetch(bases, 2, a, l.b, grp, t0, std::min(t0 + kSC, t1), l.lane);
  for (int64_t tc = t0; tc < t1; tc += kCT) {
    if ((tc - t0) % kSC == 0) {
      if constexpr (kPre) {
        pre.store(sIn, 2, tc, std::min(tc + kSC, t1), l.lane);
        if (tc + kSC < t1) pre.fetch(bases, 2, a, l.b, grp, tc + kSC, std::min(tc + 2 * kSC, t1), l.lane);
      } else {
        stage_rows<T, kWave, 2>(sIn, bases, 2, a, l.b, grp, tc, std::min(tc + kSC, t1), l.lane);
      }
    }
    const Raw rb = nb;
    if (tc + kCT < t1 && l.lane < N) nb = Row8<T>::fetch(brow + tc + kCT);
    if (tc > t0 && l.active) {
      const int64_t kg = tc / kCT;
      float4* ck = (float4*)(a.ck_h + (kg * a.chans + l.ch) * N);
#pragma unroll
      for (int n = 0; n < N; n += 4) ck[n / 4] = make_float4(h[n], h[n + 1], h[n + 2], h[n + 3]);
      a.ck_dt[kg * a.chans + l.ch] = cum;
    }
    if (l.lane < N) {
      float bv[kCT];
      Row8<T>::unpack(rb, bv);
#pragma unroll
      for (int i = 0; i < kCT; ++i) sB[i][l.lane] = bv[i];
    }
    __syncthreads();
    const int off = (int)((tc - t0) % kSC);
    float uv[kCT], dv[kCT];
    Row8<T>::unpack(Row8<T>::fetch(&sIn[0][l.lane][off]), uv);
    Row8<T>::unpack(Row8<T>::fetch(&sIn[1][l.lane][off]), dv);
#pragma unroll
    for (int i = 0; i < kCT; ++i) {
      const float dt = step_size(dv[i] + bias, a.softplus);
      const float du = dt * uv[i];
      const float4* br = (const float4*)sB[i];
      const float e = UNI ? ex2(dt * A2[0]) : 0.0f;
#pragma unroll
      for (int n = 0; n < N; n += 4) {
        const float4 bq = br[n / 4];
        h[n] = __builtin_fmaf(UNI ? e : ex2(dt * A2[n]), h[n], du * bq.x);
        h[n + 1] = __builtin_fmaf(UNI ? e : ex2(dt * A2[n + 1]), h[n + 1], du * bq.y);
        h[n + 2] = __builtin_fmaf(UNI ? e : ex2(dt * A2[n + 2]), h[n + 2], du * bq.z);
        h[n + 3] = __builtin_fmaf(UNI ? e : ex2(dt * A2[n + 3]), h[n + 3], du * bq.w);
      }
      cum += dt;
    }
    __syncthreads();
  }
  if (!l.active) return;
  float4* sh = (float4*)(a.seg_h + ((int64_t)seg * a.chans + l.ch) * N);
#pragma unroll
  for (int n = 0; n < N; n += 4) sh[n / 4] = make_float4(h[n], h[n + 1], h[n + 2], h[n + 3]);
  a.seg_dt[(int64_t)seg * a.chans + l.ch] = cum;
}

// 3a'. Adjoint aggregate, 16-byte rows: segment `seg` (>= 1) of this workgroup's channel group.
template <int N, typename T>
__device__ __forceinline__ void fbwd_adjoint_aggregate(const BwdArgs& a, int seg, unsigned char* lds) {
  using TL = Tile<T>;
  float(*sC)[N] = reinterpret_cast<float(*)[N]>(lds);
  T(*sIn)[kWave][TL::kRow] = reinterpret_cast<T(*)[kWave][TL::kRow]>(lds + PreLds<N, T>::kRows);  // delta, dy, z
  const Lane l = lane_of(a);
  const int64_t grp = blockIdx.x % a.groups;
  const int64_t L = a.seqlen;
  const int64_t t0 = (int64_t)seg * a.seg_len;
  const int64_t t1 = std::min(t0 + a.seg_len, L);
  const bool gated = a.z != nullptr;
  const T* __restrict__ Cp = (const T*)a.C + l.b * N * L;
  const T* const bases[3] = {(const T*)a.delta, (const T*)a.dy, (const T*)a.z};
  float A2[N], lam[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    A2[n] = a.A[l.dd * N + n] * kLog2e;
    lam[n] = 0.0f;
  }
  const float bias = a.dt_bias ? a.dt_bias[l.dd] : 0.0f;
  using Raw = typename Row8<T>::Raw;
  Raw nc{};
  const T* crow = Cp + (int64_t)(l.lane < N ? l.lane : 0) * L;
  if (l.lane < N) nc = Row8<T>::fetch(crow + t1 - kCT);
  // bf16 tiles are prefetched a tile ahead (to the left) in registers
  constexpr bool kPre = sizeof(T) == 2;
  const int nt = gated ? 3 : 2;
  TilePrefetch<T, 3> pre;
  if constexpr (kPre) {
    const int64_t j0 = t0 + (t1 - kCT - t0) / kSC * kSC;
    pre.fetch(bases, nt, a, l.b, grp, j0, std::min(j0 + kSC, t1), l.lane);
  }
  for (int64_t tc = t1 - kCT; tc >= t0; tc -= kCT) {
    const int64_t j0 = t0 + (tc - t0) / kSC * kSC;  // start of this chunk's tile
    if (tc == t1 - kCT || tc + kCT == j0 + kSC) {
      if constexpr (kPre) {
        pre.store(sIn, nt, j0, std::min(j0 + kSC, t1), l.lane);
        if (j0 > t0) pre.fetch(bases, nt, a, l.b, grp, j0 - kSC, j0, l.lane);
      } else {
        stage_rows<T, kWave, 3>(sIn, bases, nt, a, l.b, grp, j0, std::min(j0 + kSC, t1), l.lane);
      }
    }
    const Raw rc = nc;
    if (tc - kCT >= t0 && l.lane < N) nc = Row8<T>::fetch(crow + tc - kCT);
    if (l.lane < N) {
      float cv[kCT];
      Row8<T>::unpack(rc, cv);
#pragma unroll
      for (int i = 0; i < kCT; ++i) sC[i][l.lane] = cv[i];
    }
    __syncthreads();
    const int off = (int)(tc - j0);
    float dv[kCT], gv[kCT], zv[kCT];
    Row8<T>::unpack(Row8<T>::fetch(&sIn[0][l.lane][off]), dv);
    Row8<T>::unpack(Row8<T>::fetch(&sIn[1][l.lane][off]), gv);
    if (gated) Row8<T>::unpack(Row8<T>::fetch(&sIn[2][l.lane][off]), zv);
#pragma unroll
    for (int i = kCT - 1; i >= 0; --i) {
      const float dt = step_size(dv[i] + bias, a.softplus);
      const float ds = gated ? gv[i] * silu(zv[i]) : gv[i];
      const float4* cr = (const float4*)sC[i];
#pragma unroll
      for (int n = 0; n < N; n += 4) {
        const float4 cq = cr[n / 4];
        lam[n] = ex2(dt * A2[n]) * __builtin_fmaf(ds, cq.x, lam[n]);
        lam[n + 1] = ex2(dt * A2[n + 1]) * __builtin_fmaf(ds, cq.y, lam[n + 1]);
        lam[n + 2] = ex2(dt * A2[n + 2]) * __builtin_fmaf(ds, cq.z, lam[n + 2]);
        lam[n + 3] = ex2(dt * A2[n + 3]) * __builtin_fmaf(ds, cq.w, lam[n + 3]);
      }
    }
    __syncthreads();
  }
  if (!l.active) return;
  float4* sl = (float4*)(a.seg_l + ((int64_t)seg * a.chans + l.ch) * N);
#pragma unroll
  for (int n = 0; n < N; n += 4) sl[n / 4] = make_float4(lam[n], lam[n + 1], lam[n + 2], lam[n + 3]);
}

// 1' and 3a' in one launch: rows 0 .. nseg-1 of the grid are the checkpoint pass of each segment,
// rows nseg .. 2 nseg-2 the adjoint aggregate of segments 1 .. nseg-1.  The two need nothing of each
// other, and one grid of both keeps twice the waves resident to hide each other's latency.
template <int N, typename T, bool UNI = false>
__global__ __launch_bounds__(kWave) void fbwd_pre_kernel(BwdArgs a) {
  __shared__ __align__(16) unsigned char lds[PreLds<N, T>::kBytes];
  if (a.clear) {
    const int64_t stride = (int64_t)gridDim.x * gridDim.y * kWave;
    for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * kWave + threadIdx.x; i < a.clear_n; i += stride)
      a.clear[i] = 0.0f;
  }
  const int y = blockIdx.y;
  if (y < a.nseg)
    fbwd_checkpoint<N, T, UNI>(a, y, lds);
  else
    fbwd_adjoint_aggregate<N, T>(a, y - a.nseg + 1, lds);
}

// 4'. Main pass, 16-byte rows: a workgroup of N/8 waves per (channel group, batch row) and
// segment; wave w holds states 8w .. 8w+7 of the group's 64 channels.  Per chunk: stage B and
// C; rerun the forward keeping h_{t-1} (readout partials to LDS, dC partials reduced across
// lanes); run the adjoint back (partials of sum lam B and sum q A to LDS, dB partials); after
// one barrier wave 0 writes dz while the last wave writes du and ddelta.  Two barriers per chunk.
template <int N, typename T>
__global__ __launch_bounds__(kWave * (N / kSPW), SSM_BWD_WAVES_PER_SIMD) void fbwd_main_kernel(BwdArgs a) {
  constexpr int W = N / kSPW;
  __shared__ __align__(16) float sBC[W][2][kCT][kSPW];
  __shared__ float sS[W][kCT][kWave];
  __shared__ float sP[W][2][kCT][kWave];
  __shared__ __align__(16) T sIn[4][kWave][Tile<T, kSCM>::kRow];  // u, delta, dy, z
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t b = blockIdx.x / a.groups;
  const int64_t grp = blockIdx.x % a.groups;
  const int64_t d = grp * kWave + lane;
  const bool active = d < a.dim;
  const int64_t dd = active ? d : a.dim - 1;
  const int64_t ch = b * a.dim + dd;
  const int seg = blockIdx.y;
  const int64_t L = a.seqlen;
  const int64_t t0 = (int64_t)seg * a.seg_len;
  const int64_t t1 = std::min(t0 + a.seg_len, L);
  const int n0 = w * kSPW;
  const bool zz = a.z != nullptr;  // gated
  const T* __restrict__ Bp = (const T*)a.B + b * N * L;
  const T* __restrict__ Cp = (const T*)a.C + b * N * L;
  const int jr = reduce8_index(lane);
  const bool hi8 = (lane & 8) != 0;
  float* __restrict__ pB = a.pB + ((grp * a.batch + b) * N + n0 + jr) * L + (lane & 7);
  float* __restrict__ pC = a.pC + ((grp * a.batch + b) * N + n0 + jr) * L + (lane & 7);

  float A2[kSPW], hin[kSPW], lam[kSPW], dA[kSPW];
  const bool multi = a.nseg > 1;
  {
    const int64_t k = ((int64_t)seg * a.chans + ch) * N + n0;
#pragma unroll
    for (int j = 0; j < kSPW; ++j) {
      A2[j] = a.A[dd * N + n0 + j] * kLog2e;
      hin[j] = multi ? a.seg_h[k + j] : (a.h0 ? a.h0[ch * N + n0 + j] : 0.0f);
      lam[j] = (multi && active) ? a.seg_l[k + j] : 0.0f;
      dA[j] = 0.0f;
    }
  }
  const float bias = a.dt_bias ? a.dt_bias[dd] : 0.0f;
  const float Dd = a.D ? a.D[dd] : 0.0f;
  float accD = 0.0f, accbias = 0.0f;

  // the next chunk's rows and checkpoint are fetched while the current one is computed
  using Raw = typename Row8<T>::Raw;
  const T* bcrow = (lane < kSPW ? Bp : Cp) + (int64_t)(n0 + (lane & 7)) * L;
  Raw nbc{};
  const T* const bases[4] = {(const T*)a.u, (const T*)a.delta, (const T*)a.dy, (const T*)a.z};
  float4 nk0 = make_float4(0.f, 0.f, 0.f, 0.f), nk1 = nk0;
  float nkd = 0.0f;
  auto fetch = [&](int64_t tc) {
    if (lane < 2 * kSPW) nbc = Row8<T>::fetch(bcrow + tc);
    if (tc > t0) {
      const int64_t kg = tc / kCT;
      const float4* ck = (const float4*)(a.ck_h + (kg * a.chans + ch) * N + n0);
      nk0 = ck[0];
      nk1 = ck[1];
      nkd = a.ck_dt[kg * a.chans + ch];
    }
  };
  fetch(t1 - kCT);
  for (int64_t tc = t1 - kCT; tc >= t0; tc -= kCT) {
    const int64_t j0 = t0 + (tc - t0) / kSCM * kSCM;  // start of this chunk's tile
    if (tc == t1 - kCT || tc + kCT == j0 + kSCM)
      stage_rows<T, kWave * W, 4, kSCM>(sIn, bases, zz ? 4 : 3, a, b, grp, j0, std::min(j0 + kSCM, t1), threadIdx.x);
    const Raw rbc = nbc;
    const float4 k0 = nk0, k1 = nk1;
    const float kd = nkd;
    if (tc - kCT >= t0) fetch(tc - kCT);
    float h[kSPW];
    if (tc == t0) {
#pragma unroll
      for (int j = 0; j < kSPW; ++j) h[j] = hin[j];
    } else {
      const float cv[kSPW] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
      for (int j = 0; j < kSPW; ++j) h[j] = __builtin_fmaf(ex2(A2[j] * kd), hin[j], cv[j]);
    }
    if (lane < 2 * kSPW) {
      float bv[kCT];
      Row8<T>::unpack(rbc, bv);
#pragma unroll
      for (int i = 0; i < kCT; ++i) sBC[w][lane >> 3][i][lane & 7] = bv[i];
    }
    __syncthreads();
    const int off = (int)(tc - j0);
    float uv[kCT], dv[kCT], gv[kCT], zv[kCT];
    Row8<T>::unpack(Row8<T>::fetch(&sIn[0][lane][off]), uv);
    Row8<T>::unpack(Row8<T>::fetch(&sIn[1][lane][off]), dv);
    Row8<T>::unpack(Row8<T>::fetch(&sIn[2][lane][off]), gv);
    if (zz) Row8<T>::unpack(Row8<T>::fetch(&sIn[3][lane][off]), zv);
    float dt[kCT], dut[kCT], ds[kCT];
#pragma unroll
    for (int i = 0; i < kCT; ++i) {
      dt[i] = step_size(dv[i] + bias, a.softplus);
      dut[i] = dt[i] * uv[i];
      ds[i] = zz ? gv[i] * silu(zv[i]) : gv[i];
      if (!active) ds[i] = 0.0f;
    }
    // forward over the chunk
    float hp[kCT][kSPW];
    float keepC = 0.0f;
#pragma unroll
    for (int i = 0; i < kCT; ++i) {
      const float4* br = (const float4*)sBC[w][0][i];
      const float4* cr = (const float4*)sBC[w][1][i];
      const float4 b0 = br[0], b1 = br[1], c0 = cr[0], c1 = cr[1];
      const float Bv[kSPW] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      const float Cv[kSPW] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      float s = 0.0f, v[kSPW];
#pragma unroll
      for (int j = 0; j < kSPW; ++j) {
        hp[i][j] = h[j];
        h[j] = __builtin_fmaf(ex2(dt[i] * A2[j]), h[j], dut[i] * Bv[j]);
        s = __builtin_fmaf(Cv[j], h[j], s);
        v[j] = ds[i] * h[j];
      }
      sS[w][i][lane] = s;
      const float r = reduce8(v, hi8);
      if ((lane & 7) == i) keepC = r;
    }
    pC[tc] = keepC;
    // adjoint back over the chunk (no barrier: it reads only this wave's B and C rows; the
    // readout partials in sS are read after the next barrier)
    float keepB = 0.0f;
#pragma unroll
    for (int i = kCT - 1; i >= 0; --i) {
      const float4* br = (const float4*)sBC[w][0][i];
      const float4* cr = (const float4*)sBC[w][1][i];
      const float4 b0 = br[0], b1 = br[1], c0 = cr[0], c1 = cr[1];
      const float Bv[kSPW] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      const float Cv[kSPW] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      float accB = 0.0f, accQ = 0.0f, v[kSPW];
#if SSM_BWD_RECOMPUTE_ABAR
      // an opaque copy of the step keeps the compiler from holding the forward's Abar values
      // in registers across the chunk; they are recomputed instead
      float dtb = dt[i];
      asm volatile("" : "+v"(dtb));
#else
      const float dtb = dt[i];
#endif
#pragma unroll
      for (int j = 0; j < kSPW; ++j) {
        const float lt = __builtin_fmaf(ds[i], Cv[j], lam[j]);
        accB = __builtin_fmaf(lt, Bv[j], accB);
        v[j] = lt * dut[i];
        const float lp = ex2(dtb * A2[j]) * lt;
        const float q = lp * hp[i][j];
        accQ = __builtin_fmaf(q, A2[j], accQ);
        dA[j] = __builtin_fmaf(q, dt[i], dA[j]);
        lam[j] = lp;
      }
      sP[w][0][i][lane] = accB;
      sP[w][1][i][lane] = accQ;
      const float r = reduce8(v, hi8);
      if ((lane & 7) == i) keepB = r;
    }
    pB[tc] = keepB;
    __syncthreads();
    // dz (wave 0) and du, ddelta (the last wave) run side by side; sS is not rewritten before the
    // next chunk's first barrier
    if (w == 0 && zz) {
      float out[kCT];
#pragma unroll
      for (int i = 0; i < kCT; ++i) {
        float s = Dd * uv[i];
#pragma unroll
        for (int q = 0; q < W; ++q) s += sS[q][i][lane];
        const float sg = sigmoid(zv[i]);
        out[i] = gv[i] * s * sg * __builtin_fmaf(zv[i], 1.0f - sg, 1.0f);
      }
      if (active) Row8<T>::store((T*)a.dz + ch * L + tc, out);
    }
    if (w == W - 1) {
      float o_du[kCT], o_dl[kCT];
#pragma unroll
      for (int i = 0; i < kCT; ++i) {
        float sb = 0.0f, sq = 0.0f;
#pragma unroll
        for (int q = 0; q < W; ++q) {
          sb += sP[q][0][i][lane];
          sq += sP[q][1][i][lane];
        }
        o_du[i] = __builtin_fmaf(dt[i], sb, ds[i] * Dd);
        const float dDelta = __builtin_fmaf(sq, kLn2, uv[i] * sb);
        o_dl[i] = a.softplus ? dDelta * sigmoid(dv[i] + bias) : dDelta;
        accD = __builtin_fmaf(ds[i], uv[i], accD);
        accbias += o_dl[i];
      }
      if (active) {
        Row8<T>::store((T*)a.du + ch * L + tc, o_du);
        if (a.ddelta_f32)
          Row8<float>::store((float*)a.ddelta + ch * L + tc, o_dl);
        else
          Row8<T>::store((T*)a.ddelta + ch * L + tc, o_dl);
      }
    }
  }
  if (!active) return;
  {
    const int64_t k = ((int64_t)seg * a.chans + ch) * N + n0;
#pragma unroll
    for (int j = 0; j < kSPW; ++j) a.pA[k + j] = dA[j];
    if (seg == 0 && a.dh0) {
#pragma unroll
      for (int j = 0; j < kSPW; ++j) a.dh0[ch * N + n0 + j] = lam[j];
    }
  }
  if (w == W - 1) {
    a.pD[(int64_t)seg * a.chans + ch] = accD;
    a.pbias[(int64_t)seg * a.chans + ch] = accbias;
  }
}

// 4''. Main pass with roles, 16-byte rows, dstate 8, 16 or 32: a workgroup of 8 waves per
// (channel group, batch row) and segment.  Scanner waves 0-3 hold N/4 states each of the group's
// 64 channels; per chunk of 8 steps (right to left) a scanner reruns the forward from the
// chunk's checkpoint keeping Abar and h_{t-1} of every step in registers, then runs the adjoint
// back over them, reduces its dB and dC contributions across the wave's lanes and leaves three
// partial sums over its states per element in LDS.  Helper waves 4-7 own 2 steps of every chunk:
// they stage the input rows (u, delta, dy, z) in 64-byte tiles, compute the per-element terms the
// scanners read (Delta, Delta u, ds) and keep those the epilogue needs, stage B and C, and one
// chunk behind the scanners sum the four partials in a fixed order into dz, du and ddelta, which
// the next iteration stores as 16-byte row pieces.  One workgroup barrier per chunk: iteration k
// scans chunk k, preps chunk k+1, finishes chunk k-1 and stores chunk k-2.
#ifndef SSM_BWD_ROLES
#define SSM_BWD_ROLES 1
#endif
#ifndef SSM_BWD_INTERVALS
#define SSM_BWD_INTERVALS 1
#endif
// Scanner waves: 4 (one per SIMD).  Eight (two per SIMD, N/8 states each; bf16 up to dstate 16
// only, where LDS holds eight scanners' partial sums) measured no faster on the 2.8B-shaped layer:
// the scanners alone ran 13% faster, but together with the helpers no faster than four.
#ifndef SSM_BWD_SCANNERS_BF16
#define SSM_BWD_SCANNERS_BF16 4
#endif
template <typename T, int N>
constexpr int roles_scanners() { return sizeof(T) == 2 && N <= 16 ? SSM_BWD_SCANNERS_BF16 : 4; }
constexpr int kRH = 4;                      // helper waves, 2 steps of each chunk apiece
template <typename T, int N>
constexpr int roles_threads() { return (roles_scanners<T, N>() + kRH) * kWave; }
constexpr int kRItems = 7;                  // per-element terms: Delta, Delta u, ds, u, sg, gz, gz D u

// Staged input tiles: P 16-byte pieces of each row (64 bytes with four scanners, 32 with eight).
template <typename T, int P>
struct RTile {
  static constexpr int kPieces = P;
  static constexpr int kPiece = 16 / (int)sizeof(T);      // elements per 16-byte piece
  static constexpr int kSteps = P * kPiece;               // steps per tile
  static constexpr int kRow = kSteps + kPiece;            // padded row (elements)
};
template <typename T, int N>
using RTileOf = RTile<T, roles_scanners<T, N>() == 4 ? 4 : 2>;

// Output rings of the main pass: chunk c of a row in slot c % kRing(slot bytes).  A ring holds the
// chunks of one 128-byte line still to be stored plus the one being finished.
constexpr int kOutRingBytes = 160;
constexpr int kBcRing = 5;
template <int SB>
constexpr int out_ring() { return SB == 16 ? 9 : 5; }
static_assert(9 * 16 <= kOutRingBytes && 5 * 32 <= kOutRingBytes, "ring slots fit a row");

template <int N, typename T>
struct RolesSmem {
  static constexpr int S = roles_scanners<T, N>();
  T tile[2][4][kWave][RTileOf<T, N>::kRow];      // u, delta, dy, z; tile m in buffer m % 2
  float prep[2][kRItems][kCT][kWave];         // chunk c in slot c % 2
  float part[2][3][S][kCT][kWave];            // readout, sum lam B, sum q A per scanner
  float bcs[S][2][kCT][N / S];                // each scanner's B and C rows of its chunk, [t][n]
  // dz, du, ddelta rows of the chunks finished and not yet stored, in a ring of chunk slots per
  // row (9 slots of 16 bytes, or 5 of 32 for fp32 rows), so that a row's 128-byte line is stored
  // in one burst once its last chunk is done
  unsigned char ring[3][kWave][kOutRingBytes];
  float dbc[kBcRing][2][N][kCT];              // dB and dC partials of chunk c (this channel group) in slot c % 5
  int ticket;                                 // interval plan: this workgroup's interval
};

template <int K>
__device__ __forceinline__ void lds_vec(const float* p, float (&v)[K]) {
  if constexpr (K % 4 == 0) {
#pragma unroll
    for (int k = 0; k < K; k += 4) {
      const float4 q = *(const float4*)(p + k);
      v[k] = q.x; v[k + 1] = q.y; v[k + 2] = q.z; v[k + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < K; k += 2) {
      const float2 q = *(const float2*)(p + k);
      v[k] = q.x; v[k + 1] = q.y;
    }
  }
}

// Two consecutive elements of a tile row / an output row.
__device__ __forceinline__ void lds_pair(const __bf16* p, float& x, float& y) {
  const uint32_t w = *(const uint32_t*)p;
  x = __uint_as_float(w << 16);
  y = __uint_as_float(w & 0xffff0000u);
}
__device__ __forceinline__ void lds_pair(const float* p, float& x, float& y) {
  const float2 q = *(const float2*)p;
  x = q.x; y = q.y;
}
__device__ __forceinline__ void lds_put_pair(__bf16* p, float x, float y) {
  __bf16 t[2] = {(__bf16)x, (__bf16)y};
  uint32_t w;
  __builtin_memcpy(&w, t, sizeof w);
  *(uint32_t*)p = w;
}
__device__ __forceinline__ void lds_put_pair(float* p, float x, float y) { *(float2*)p = make_float2(x, y); }

template <int N, typename T, bool UNI = false>
__global__ __launch_bounds__((roles_threads<T, N>())) void fbwd_main_roles_kernel(BwdArgs a) {
  constexpr int kRS = roles_scanners<T, N>();
  constexpr int NPW = N / kRS;           // states per scanner
  constexpr int SPG = kCT / NPW < 1 ? 1 : kCT / NPW;  // steps per 8-value lane reduction
  static_assert(N % kRS == 0 && NPW * SPG == 8, "a lane reduction takes 8 values: whole steps of NPW states");
  using RT = RTileOf<T, N>;
  __shared__ __align__(16) RolesSmem<N, T> sm;
  const int wv = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t L = a.seqlen;
  const int64_t tchn = L / kCT;  // chunks per chain
  const bool gated = a.z != nullptr;
  const bool multi = a.nseg > 1;  // checkpoints relative to segments with a carried incoming state

  // The pieces this workgroup runs.  Segment plan: one, segment blockIdx.y of chain blockIdx.x,
  // with the adjoint entering from the right taken from the reverse carry.  Interval plan: the
  // chains (batch row x channel group) laid end to end in processing order, right to left, cut
  // into one interval of wlen chunks per workgroup (wlen >= a chain, so a chain is split at most
  // once); the interval comes from a ticket.  Its pieces run in the order: the right part of its
  // last chain first (it waits for nothing, and the next interval's workgroup waits for the
  // adjoint it hands over at its left end), then the whole chains, then the left part of its
  // first chain, which starts from the adjoint the previous interval's workgroup handed over.
  int64_t is = 0, ie = 0, cf = 0, cl = 0;
  bool itail = false, ihead = false;
  int npieces = 1;
  if (a.iunits > 0) {
    if (threadIdx.x == 0) sm.ticket = atomicAdd(a.ticket, 1);
    __syncthreads();
    const int ival = __builtin_amdgcn_readfirstlane(sm.ticket);
    if (ival >= a.iunits) return;  // uniform: the whole workgroup leaves
    const int64_t total = a.batch * a.groups * tchn;
    is = (int64_t)ival * a.wlen;
    ie = is + a.wlen < total ? is + a.wlen : total;
    cf = is / tchn;
    cl = (ie - 1) / tchn;
    itail = is > cf * tchn;
    ihead = ie < (cl + 1) * tchn;
    npieces = (int)(cl - cf + 1);
  }
  // One piece: its chain cid, its chunks [k0, k1) in processing order (chunk 0: the last 8 steps;
  // chunk k of the piece covers steps [t1 - 8(k+1), t1 - 8k)) and the slot its sums over time go to
  // (pA, pD, pbias).  wait_in: the adjoint comes from another workgroup; hand_out: and goes to
  // another one; whole: the chain's slot 1 stays zero.  Each role runs its own loop over the
  // pieces, so that the compiler keeps the two roles' registers apart.
#define SSM_BWD_PIECE \
  int64_t cid, k0, k1; \
  int slot; \
  if (a.iunits > 0) { \
    if (ihead && pc == 0) { \
      cid = cl; \
    } else { \
      const int q = pc - (ihead ? 1 : 0); \
      const int nfull = npieces - (ihead ? 1 : 0) - (itail ? 1 : 0); \
      cid = q < nfull ? cf + (itail ? 1 : 0) + q : cf; \
    } \
    const int64_t p0 = cid * tchn > is ? cid * tchn : is; \
    const int64_t p1 = (cid + 1) * tchn < ie ? (cid + 1) * tchn : ie; \
    k0 = p0 - cid * tchn; \
    k1 = p1 - cid * tchn; \
    slot = k0 > 0 ? 1 : 0; \
  } else { \
    cid = blockIdx.x; \
    slot = blockIdx.y; \
    const int64_t s0 = (int64_t)blockIdx.y * a.seg_len; \
    const int64_t s1 = s0 + a.seg_len < L ? s0 + a.seg_len : L; \
    k0 = (L - s1) / kCT; \
    k1 = (L - s0) / kCT; \
  } \
  const bool wait_in = a.iunits > 0 && k0 > 0; \
  const bool hand_out = a.iunits > 0 && k1 < tchn; \
  const bool whole = a.iunits > 0 && k0 == 0 && k1 == tchn; \
  const int64_t b = cid / a.groups; \
  const int64_t grp = cid % a.groups; \
  const int64_t d = grp * kWave + lane; \
  const bool active = d < a.dim; \
  const int64_t dd = active ? d : a.dim - 1; \
  const int64_t ch = b * a.dim + dd; \
  const int64_t t0 = L - kCT * k1; \
  const int64_t t1 = L - kCT * k0; \
  const int nch = (int)(k1 - k0); \
  auto chunk_t = [&](int k) { return t1 - (int64_t)kCT * (k + 1); }; \
  auto tile_of = [&](int k) { return (int)((chunk_t(k) - t0) / RT::kSteps); };
  if (wv < kRS) {
  for (int pc = 0; pc < npieces; ++pc) {
  SSM_BWD_PIECE
    // ------------------------------------------------------------------ scanner
    const int n0 = wv * NPW;
    float A2[NPW], lam[NPW], dA[NPW];
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      A2[j] = a.A[dd * N + n0 + j] * kLog2e;
      dA[j] = 0.0f;
    }
    if (wait_in) {
      // Hand-over (interval plan): wait for the flag of the matching scanner wave of the
      // chain's right part, then read its rows of the adjoint.  Flag and adjoint are device-scope
      // atomics, coherent across the XCDs' L2 caches; the loads are issued only after the flag
      // has been seen.  The wait is bounded; if it runs out the piece is poisoned with NaN and
      // counted, so that a broken hand-over cannot pass for numbers.
      const int* f = a.flags + cid * kRS + wv;
      bool arrived = true;
      for (int spin = 0;
           __builtin_amdgcn_readfirstlane(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0;
           ++spin) {
        if (spin >= a.max_polls) {
          arrived = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      const float* hp0 = a.hand_l + cid * N * kWave;
#pragma unroll
      for (int j = 0; j < NPW; ++j)
        lam[j] = arrived ? __hip_atomic_load(hp0 + (n0 + j) * kWave + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : __builtin_nanf("");
      if (!arrived && lane == 0) atomicAdd(&bwd_handover_giveups, 1u);
    } else {
      const int64_t k = ((int64_t)slot * a.chans + ch) * N + n0;
#pragma unroll
      for (int j = 0; j < NPW; ++j) lam[j] = (a.iunits == 0 && multi && active) ? a.seg_l[k + j] : 0.0f;
    }
    // dB / dC partial of this group: after the 8-value reduction lane l holds value
    // reduce8_index(l) of reduction (l & 7); NPW * SPG = 8 values per reduction, NPW reductions
    const int jr = reduce8_index(lane);
    const bool hi8 = (lane & 8) != 0;
    const int rsel = lane & 7;
    const bool rkeep = rsel < NPW;
    const int ri = (rkeep ? rsel : 0) * SPG + jr / NPW, rj = jr % NPW;  // (step, state) of the kept value
    // a chunk's starting state: its checkpoint (relative to the checkpoint pass's segment) plus
    // exp(A * sum Delta) times that segment's incoming state, or the incoming state itself when
    // the chunk starts the segment
    float nk[NPW], nhin[NPW], nkd = 0.0f;
    bool nat = false;
    auto fetch_ck = [&](int k) {
      const int64_t tc = chunk_t(k);
      const int64_t s = tc / a.seg_len;
      nat = tc == s * a.seg_len;
      if (!nat) {
        const int64_t kg = tc / kCT;
        const float* ck = a.ck_h + (kg * a.chans + ch) * N + n0;
#pragma unroll
        for (int j = 0; j < NPW; ++j) nk[j] = ck[j];
        nkd = a.ck_dt[kg * a.chans + ch];
      }
      const int64_t ks = (s * a.chans + ch) * N + n0;
#pragma unroll
      for (int j = 0; j < NPW; ++j) nhin[j] = multi ? a.seg_h[ks + j] : (a.h0 ? a.h0[ch * N + n0 + j] : 0.0f);
    };
#pragma unroll
    for (int j = 0; j < NPW; ++j) nk[j] = nhin[j] = 0.0f;
    // this scanner's B and C rows (its states, the chunk's 8 steps) are loaded a chunk ahead, in
    // 16-byte pieces, and written to its own LDS rows when the chunk starts: with the checkpoint
    // they are the scanner's only memory traffic, all loads, waited for a whole chunk later
    constexpr int kPPR = (int)sizeof(T) * kCT / 16;  // pieces per row (1 bf16, 2 fp32)
    constexpr int kE = 16 / (int)sizeof(T);           // steps per piece
    static_assert(2 * NPW * kPPR <= kWave, "one B/C piece per lane");
    const bool sbl = lane < 2 * NPW * kPPR;
    const int sbw = lane / (NPW * kPPR), sbn = (lane / kPPR) % NPW, sbq = lane % kPPR;
    const T* sbrow = (sbw == 0 ? (const T*)a.B : (const T*)a.C) + (b * N + n0 + (sbl ? sbn : 0)) * L + sbq * kE;
    typedef unsigned u32x4s __attribute__((ext_vector_type(4)));
    u32x4s sbv = {0, 0, 0, 0};
    auto sb_load = [&](int k) {
      if (sbl) sbv = *(const u32x4s*)(sbrow + chunk_t(k));
    };
    auto sb_store = [&]() {
      if (!sbl) return;
      float v[kE];
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = __uint_as_float(sbv[i] << 16);
          v[2 * i + 1] = __uint_as_float(sbv[i] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(sbv[i]);
      }
#pragma unroll
      for (int i = 0; i < kE; ++i) sm.bcs[wv][sbw][sbq * kE + i][sbn] = v[i];
    };
    if (nch > 0) {
      fetch_ck(0);
      sb_load(0);
    }
    __syncthreads();  // prologue: tiles staged
    __syncthreads();  // prologue: chunk 0 prepared
    for (int k = 0; k < nch + 2; ++k) {
      if (k < nch) {
        const int64_t tc = chunk_t(k);
        const int sl = k & 1;
        float h[NPW];
        if (nat) {
#pragma unroll
          for (int j = 0; j < NPW; ++j) h[j] = nhin[j];
        } else {
#pragma unroll
          for (int j = 0; j < NPW; ++j) h[j] = __builtin_fmaf(ex2(A2[j] * nkd), nhin[j], nk[j]);
        }
        sb_store();
        if (k + 1 < nch) {
          sb_load(k + 1);
          fetch_ck(k + 1);
        }
        float dt[kCT], dut[kCT], ds[kCT];
#pragma unroll
        for (int i = 0; i < kCT; ++i) {
          dt[i] = sm.prep[sl][0][i][lane];
          dut[i] = sm.prep[sl][1][i][lane];
          ds[i] = sm.prep[sl][2][i][lane];
        }
        // forward over the chunk: Abar and h_{t-1} kept for the adjoint
        float ab[kCT][NPW], hp[kCT][NPW];
        float keepC = 0.0f, vals[8];
#pragma unroll
        for (int i = 0; i < kCT; ++i) {
          float Bv[NPW], Cv[NPW];
          lds_vec<NPW>(&sm.bcs[wv][0][i][0], Bv);
          lds_vec<NPW>(&sm.bcs[wv][1][i][0], Cv);
          float s = 0.0f;
          const float e1 = UNI ? ex2(dt[i] * A2[0]) : 0.0f;  // the SSD form: one exp for the step
#pragma unroll
          for (int j = 0; j < NPW; ++j) {
            ab[i][j] = UNI ? e1 : ex2(dt[i] * A2[j]);
            hp[i][j] = h[j];
            h[j] = __builtin_fmaf(ab[i][j], h[j], dut[i] * Bv[j]);
            s = __builtin_fmaf(Cv[j], h[j], s);
            vals[(i % SPG) * NPW + j] = ds[i] * h[j];
          }
          sm.part[sl][0][wv][i][lane] = s;
          if (i % SPG == SPG - 1) {
            const float r = reduce8(vals, hi8);
            if (rsel == i / SPG) keepC = r;
          }
        }
        if (rkeep) sm.dbc[k % kBcRing][1][n0 + rj][ri] = keepC;
        // adjoint back over the chunk
        float keepB = 0.0f;
#pragma unroll
        for (int i = kCT - 1; i >= 0; --i) {
          float Bv[NPW], Cv[NPW];
          lds_vec<NPW>(&sm.bcs[wv][0][i][0], Bv);
          lds_vec<NPW>(&sm.bcs[wv][1][i][0], Cv);
          float accB = 0.0f, accQ = 0.0f;
#pragma unroll
          for (int j = 0; j < NPW; ++j) {
            const float lt = __builtin_fmaf(ds[i], Cv[j], lam[j]);
            accB = __builtin_fmaf(lt, Bv[j], accB);
            vals[(i % SPG) * NPW + j] = lt * dut[i];
            const float lp = ab[i][j] * lt;
            const float q = lp * hp[i][j];
            accQ = __builtin_fmaf(q, A2[j], accQ);
            dA[j] = __builtin_fmaf(q, dt[i], dA[j]);
            lam[j] = lp;
          }
          sm.part[sl][1][wv][i][lane] = accB;
          sm.part[sl][2][wv][i][lane] = accQ;
          if (i % SPG == 0) {
            const float r = reduce8(vals, hi8);
            if (rsel == i / SPG) keepB = r;
          }
        }
        if (rkeep) sm.dbc[k % kBcRing][0][n0 + rj][ri] = keepB;
      }
      __syncthreads();
    }
    if (hand_out) {
      // the adjoint at the piece's left end, for the workgroup that runs the rest of the chain;
      // the flag is set once every store of it is acknowledged (the signal fences keep the
      // compiler from moving memory operations across the wait)
      float* hp0 = a.hand_l + cid * N * kWave;
#pragma unroll
      for (int j = 0; j < NPW; ++j)
        __hip_atomic_store(hp0 + (n0 + j) * kWave + lane, lam[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (a.publish) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0) __hip_atomic_store(a.flags + cid * kRS + wv, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();  // the helpers' sums
    if (active) {
      const int64_t k = ((int64_t)slot * a.chans + ch) * N + n0;
#pragma unroll
      for (int j = 0; j < NPW; ++j) a.pA[k + j] = dA[j];
      if (whole) {
#pragma unroll
        for (int j = 0; j < NPW; ++j) a.pA[k + a.chans * N + j] = 0.0f;
      }
      if (t0 == 0 && a.dh0) {
#pragma unroll
        for (int j = 0; j < NPW; ++j) a.dh0[ch * N + n0 + j] = lam[j];
      }
    }
  }  // pieces (scanner)
  } else {
  for (int pc = 0; pc < npieces; ++pc) {
  SSM_BWD_PIECE

  // -------------------------------------------------------------------- helper
  const int hw = wv - kRS;       // this thread's steps of a chunk: 2 hw and 2 hw + 1
  const int htid = threadIdx.x - kRS * kWave;
  const float bias = a.dt_bias ? a.dt_bias[dd] : 0.0f;
  const float Dd = a.D ? a.D[dd] : 0.0f;
  const int ntens = gated ? 4 : 3;
  const T* const bases[4] = {(const T*)a.u, (const T*)a.delta, (const T*)a.dy, (const T*)a.z};
  float accD = 0.0f, accbias = 0.0f;
  // tile pieces: helper waves 0 and 1 load them (64 rows x P pieces of each tensor, P/2 per thread)
  // a whole tile ahead; loads are all these two waves issue, so their waits cover nothing else
  constexpr int TP = RT::kPieces, TPT = TP / 2;
  const bool tl = hw < 2;
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  u32x4 tv[TPT][4];
  auto piece = [&](int j, int& row, int& pc) {
    const int p = htid + j * 2 * kWave;
    row = p / TP;
    pc = p % TP;
  };
  auto tile_load = [&](int m) {
    if (!tl) return;
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      int row, pc;
      piece(j, row, pc);
      const int64_t tch = b * a.dim + std::min<int64_t>(grp * kWave + row, a.dim - 1);
      const int64_t ts = t0 + (int64_t)m * RT::kSteps + pc * RT::kPiece;
      const int64_t tsl = ts < t1 ? ts : t0 + (int64_t)m * RT::kSteps;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q < ntens) tv[j][q] = *(const u32x4*)(bases[q] + tch * L + tsl);
    }
  };
  auto tile_store = [&](int m) {
    if (!tl) return;
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      int row, pc;
      piece(j, row, pc);
      const int64_t ts = t0 + (int64_t)m * RT::kSteps + pc * RT::kPiece;
      if (ts < t1) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q < ntens) *(u32x4*)&sm.tile[m & 1][q][row][pc * RT::kPiece] = tv[j][q];
      }
    }
  };
  // the per-element terms of chunk k for this thread's two steps
  auto prep = [&](int k) {
    const int sl = k & 1;
    const int64_t tc = chunk_t(k);
    const int m = tile_of(k);
    const int off = (int)(tc - (t0 + (int64_t)m * RT::kSteps)) + 2 * hw;
    float uu[2], dl[2], gy[2], zz[2] = {0.0f, 0.0f};
    lds_pair(&sm.tile[m & 1][0][lane][off], uu[0], uu[1]);
    lds_pair(&sm.tile[m & 1][1][lane][off], dl[0], dl[1]);
    lds_pair(&sm.tile[m & 1][2][lane][off], gy[0], gy[1]);
    if (gated) lds_pair(&sm.tile[m & 1][3][lane][off], zz[0], zz[1]);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 2 * hw + e;
      const float x = dl[e] + bias;
      const float dt = step_size(x, a.softplus);
      float ds = gy[e], gz = 0.0f;
      if (gated) {
        const float sz = sigmoid(zz[e]);
        ds = gy[e] * zz[e] * sz;
        gz = gy[e] * sz * __builtin_fmaf(zz[e], 1.0f - sz, 1.0f);
      }
      if (!active) ds = 0.0f;
      accD = __builtin_fmaf(ds, uu[e], accD);
      sm.prep[sl][0][i][lane] = dt;
      sm.prep[sl][1][i][lane] = dt * uu[e];
      sm.prep[sl][2][i][lane] = ds;
      sm.prep[sl][3][i][lane] = uu[e];
      sm.prep[sl][4][i][lane] = a.softplus ? sigmoid(x) : 1.0f;
      sm.prep[sl][5][i][lane] = gz;
      sm.prep[sl][6][i][lane] = gz * Dd * uu[e];
    }
  };
  // dz, du, ddelta of chunk k for this thread's two steps, into the output tile
  auto finish = [&](int k) {
    const int sl = k & 1;
    float o[3][2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 2 * hw + e;
      float s = 0.0f, sb = 0.0f, sq = 0.0f;
#pragma unroll
      for (int w = 0; w < kRS; ++w) {
        s += sm.part[sl][0][w][i][lane];
        sb += sm.part[sl][1][w][i][lane];
        sq += sm.part[sl][2][w][i][lane];
      }
      const float dt = sm.prep[sl][0][i][lane], ds = sm.prep[sl][2][i][lane];
      const float uu = sm.prep[sl][3][i][lane], sg = sm.prep[sl][4][i][lane];
      o[0][e] = __builtin_fmaf(sm.prep[sl][5][i][lane], s, sm.prep[sl][6][i][lane]);
      o[1][e] = __builtin_fmaf(dt, sb, ds * Dd);
      o[2][e] = __builtin_fmaf(sq, kLn2, uu * sb) * sg;
      accbias += o[2][e];
    }
    constexpr int RT_ = out_ring<kCT * sizeof(T)>();
#pragma unroll
    for (int q = 0; q < 2; ++q)
      lds_put_pair((T*)&sm.ring[q][lane][(k % RT_) * kCT * sizeof(T)] + 2 * hw, o[q][0], o[q][1]);
    if (a.ddelta_f32)
      lds_put_pair((float*)&sm.ring[2][lane][(k % 5) * kCT * 4] + 2 * hw, o[2][0], o[2][1]);
    else
      lds_put_pair((T*)&sm.ring[2][lane][(k % RT_) * kCT * sizeof(T)] + 2 * hw, o[2][0], o[2][1]);
  };
  T* const outs[3] = {(T*)a.dz, (T*)a.du, (T*)a.ddelta};
  // all global stores come from the last helper wave (dz, du, ddelta rows here, the dB and dC
  // partials below): reusing a register a store reads waits for the store to complete, and only
  // this wave should pay for that
  //
  // A row's chunks wait in its ring until the chunk that starts a 128-byte line (in address) is
  // done, or the piece's last chunk, and are then stored together: the line is written whole
  // within one iteration instead of a piece per chunk over eight.  A ring never holds more than
  // its size less one (the slot being finished), which the pending count also enforces.
  int pend[3] = {0, 0, 0};
  auto flush_row = [&](auto sbc, const unsigned char* ring_row, char* g, int c, int& np) {
    constexpr int SB = decltype(sbc)::value, R = out_ring<SB>();
    ++np;
    if (((uintptr_t)g & 127) >= (uintptr_t)SB && c != nch - 1 && np < R - 1) return;
#pragma unroll
    for (int j = 0; j < R - 1; ++j) {
      if (j < np) {
        const int slot = (c - j) % R;
#pragma unroll
        for (int h = 0; h < SB / 16; ++h)
          *(uint4*)(g + j * SB + 16 * h) = *(const uint4*)(ring_row + slot * SB + 16 * h);
      }
    }
    np = 0;
  };
  auto store = [&](int c) {
    if (hw != kRH - 1 || !active) return;
    constexpr int SBT = kCT * (int)sizeof(T);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      if (q == 0 && !gated) continue;
      if (q == 2 && a.ddelta_f32)
        flush_row(std::integral_constant<int, kCT * 4>{}, sm.ring[2][lane],
                  (char*)((float*)a.ddelta + ch * L + chunk_t(c)), c, pend[2]);
      else
        flush_row(std::integral_constant<int, SBT>{}, sm.ring[q][lane], (char*)(outs[q] + ch * L + chunk_t(c)), c,
                  pend[q]);
    }
  };

  // the dB and dC partials of chunk c (4 steps per 16-byte piece) by helper wave 3, from the
  // scanners' ring in LDS, stored the same way: a row's chunks together once a line is complete
  constexpr int kBcPer = (4 * N + kWave - 1) / kWave;
  int pendbc[kBcPer];
#pragma unroll
  for (int i = 0; i < kBcPer; ++i) pendbc[i] = 0;
  auto store_bc = [&](int c) {
    if (hw != kRH - 1) return;
    const int64_t tc = chunk_t(c);
#pragma unroll
    for (int p0 = 0; p0 < 4 * N; p0 += kWave) {
      const int q = p0 + lane;
      if (q < 4 * N) {
        const int w = q / (2 * N), n = (q / 2) % N, hf = q % 2;
        float* row = (w == 0 ? a.pB : a.pC) + ((grp * a.batch + b) * N + n) * L + tc;
        int& np = pendbc[p0 / kWave];
        ++np;
        if (((uintptr_t)row & 127) < 32 || c == nch - 1 || np == kBcRing - 1) {
#pragma unroll
          for (int j = 0; j < kBcRing - 1; ++j)
            if (j < np) *(float4*)(row + kCT * j + 4 * hf) = *(const float4*)&sm.dbc[(c - j) % kBcRing][w][n][4 * hf];
          np = 0;
        }
      }
    }
  };

  // Helper waves 0 and 1 only load (tiles, a whole tile ahead), wave 3 only stores: on this GPU
  // one counter tracks a wave's loads and stores together, and reusing a register a store reads
  // waits for the store to complete, so a wave that mixed them would wait for its stores too.
  int tnext = -1;  // the tile whose pieces are in flight in tv
  if (nch > 0) {  // prologue: the tiles of chunks 0 and 1 (they differ when chunk 0 ends a short last tile)
    int last = tile_of(0);
    tile_load(last);
    tile_store(last);
    if (nch > 1 && tile_of(1) != last) {
      last = tile_of(1);
      tile_load(last);
      tile_store(last);
    }
    if (last > 0) {
      tnext = last - 1;
      tile_load(tnext);
    }
  }
  __syncthreads();
  if (nch > 0) prep(0);
  __syncthreads();
  // the storing wave runs its own copy of the loop, so that the waits its stores need are not
  // compiled into the loaders' code
  auto loop = [&](auto storer) {
    for (int k = 0; k < nch + 2; ++k) {
      if constexpr (decltype(storer)::value) {
        if (k >= 2) store(k - 2);
        if (k >= 1 && k - 1 < nch) store_bc(k - 1);
      }
      if (k >= 1 && k - 1 < nch) finish(k - 1);
      if (k + 1 < nch) prep(k + 1);
      if constexpr (!decltype(storer)::value) {
        // chunk k+2 starts the tile in flight: it goes to LDS now, and the next one is requested
        if (k + 2 < nch && tile_of(k + 2) != tile_of(k + 1)) {
          tile_store(tnext);
          tnext = tnext > 0 ? tnext - 1 : -1;
          if (tnext >= 0) tile_load(tnext);
        }
      }
      __syncthreads();
    }
  };
  if (hw == kRH - 1)
    loop(std::true_type{});
  else
    loop(std::false_type{});
  // the helpers' dD and ddt_bias sums, through the partials' LDS (no longer in use)
  float(*acc)[2][kWave] = reinterpret_cast<float(*)[2][kWave]>(&sm.part[0][0][0][0][0]);
  static_assert(sizeof(sm.part) >= sizeof(float) * kRH * 2 * kWave, "room for the helpers' sums");
  acc[hw][0][lane] = accD;
  acc[hw][1][lane] = accbias;
  __syncthreads();
  if (hw == 0 && active) {
    float sD = 0.0f, sb = 0.0f;
#pragma unroll
    for (int w = 0; w < kRH; ++w) {
      sD += acc[w][0][lane];
      sb += acc[w][1][lane];
    }
    a.pD[(int64_t)slot * a.chans + ch] = sD;
    a.pbias[(int64_t)slot * a.chans + ch] = sb;
    if (whole) {
      a.pD[(int64_t)(slot + 1) * a.chans + ch] = 0.0f;
      a.pbias[(int64_t)(slot + 1) * a.chans + ch] = 0.0f;
    }
  }
  }  // pieces (helper)
  }
#undef SSM_BWD_PIECE
}

hipError_t zero(float* p, int64_t n, hipStream_t s) {
  if (!p || n == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

unsigned blocks_of(int64_t n) { return (unsigned)((n + 255) / 256); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int bwd_cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

// Workgroups of `threads` threads of `kernel` resident per CU (at least 1).
template <typename K>
int resident_blocks(K kernel, int threads) {
  int b = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kernel, threads, 0) != hipSuccess || b < 1) b = 1;
  return b;
}

// The fast kernels need whole chunks of 8 steps in 16-byte pieces and at least 8 states.
bool fast_ok(const BwdParams& p) {
  if (p.dstate < kSPW || p.seqlen % kCT != 0) return false;
  const void* ptrs[] = {p.u, p.delta, p.z, p.dy, p.du, p.ddelta, p.dz, p.B, p.C};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return false;
  return true;
}

template <int N, typename T, bool FAST>
hipError_t run(const BwdParams& p, hipStream_t stream) {
  // the main pass with scanner and helper roles (dstate 8, 16, 32), else the symmetric one
  constexpr bool ROLES = FAST && SSM_BWD_ROLES && (N == 8 || N == 16 || N == 32);
  constexpr int CT = FAST ? kCT : Chunk<N>::T;
  constexpr int GR = FAST ? kSCG : CT;    // segment lengths are multiples of this (whole staged tiles)
  constexpr int W = FAST ? N / kSPW : 1;  // waves per workgroup of the main pass
  BwdArgs a{};
  a.u = p.u; a.delta = p.delta; a.A = p.A; a.B = p.B; a.C = p.C; a.D = p.D; a.z = p.z; a.dt_bias = p.dt_bias;
  a.h0 = p.h0; a.dy = p.dy; a.du = p.du; a.ddelta = p.ddelta; a.dz = p.dz; a.dh0 = p.dh0;
  a.ddelta_f32 = p.ddelta_f32 ? 1 : 0;
  // the SSD form's A (one value per channel) takes the kernels that compute one exp per step; above
  // dstate 16 their second copy would crowd the registers, so those take the general kernels
  constexpr bool UNIF = FAST && N <= 16;
  const bool uni = UNIF && p.a_uniform;
  a.batch = p.batch; a.dim = p.dim; a.seqlen = p.seqlen; a.softplus = p.softplus;
  a.chans = p.batch * p.dim;
  a.groups = (int)((p.dim + kWave - 1) / kWave);
  const int64_t L = p.seqlen, chans = a.chans;
  const int64_t units = p.batch * a.groups;  // workgroups per segment
  // Segment count from a cost model: each pass takes (rounds of resident workgroups) x (steps
  // per segment + a start-up cost), with the resident count from the kernels' occupancy on this
  // device; the main pass weighs twice a pre-pass.  Segments are at least 4 chunks long.
  struct Slots {
    int64_t main, ck, adj;
  };
  static const Slots sl = [] {
    const int64_t cus = bwd_cu_count();
    if constexpr (FAST) {
      int64_t m;
      if constexpr (ROLES)
        m = cus * resident_blocks(fbwd_main_roles_kernel<N, T>, roles_threads<T, N>());
      else
        m = cus * resident_blocks(fbwd_main_kernel<N, T>, kWave * W);
      return Slots{m, cus * resident_blocks(fbwd_pre_kernel<N, T>, kWave),
                   cus * resident_blocks(fbwd_pre_kernel<N, T>, kWave)};
    } else {
      return Slots{cus * resident_blocks(bwd_main_kernel<N, T>, kWave),
                   cus * resident_blocks(bwd_checkpoint_kernel<N, T>, kWave),
                   cus * resident_blocks(bwd_adjoint_aggregate_kernel<N, T>, kWave)};
    }
  }();
  const int64_t slots_main = sl.main, slots_ck = sl.ck, slots_adj = sl.adj;
  // Interval plan for the main pass when there are at least as many chains (batch row x channel
  // group) as resident main-pass workgroups: no adjoint aggregate, no reverse carry; the
  // checkpoint pass keeps segments of its own.
  const bool IV = ROLES && SSM_BWD_INTERVALS && units >= slots_main;
  int64_t nseg = 1, seg_len = (L + GR - 1) / GR * GR;
  {
    const int64_t max_seg = std::max<int64_t>(1, std::min<int64_t>(8192, L / (4 * CT)));
    int64_t best = -1;
    const auto rounds = [](int64_t wgs, int64_t slots) { return (wgs + slots - 1) / slots; };
    const auto consider = [&](int64_t k) {
      if (k < 1 || k > max_seg) return;
      const int64_t len = ((L + k - 1) / k + GR - 1) / GR * GR;
      const int64_t real = (L + len - 1) / len;
      // a workgroup's start (first loads, checkpoint, carries) costs about 4 chunks
      // (the fast path runs the two pre-passes as one grid)
      const int64_t pre = FAST ? rounds(units * (IV ? real : 2 * real - 1), slots_ck)
                               : rounds(units * real, slots_ck) + (real > 1 ? rounds(units * (real - 1), slots_adj) : 0);
      // on the interval plan the main pass does not depend on the segment count
      const int64_t cost = (len + 4 * CT) * ((IV ? 0 : 2 * rounds(units * real, slots_main)) + pre);
      if (best < 0 || cost < best || (cost == best && real < nseg)) {
        best = cost;
        nseg = real;
        seg_len = len;
      }
    };
    // every count up to 64, and the counts that fill whole rounds of the main pass or the checkpoint pass
    for (int64_t k = 1; k <= 64; ++k) consider(k);
    for (int64_t m = 1; m <= 64; ++m) {
      consider(m * slots_main / units);
      consider(m * slots_ck / units);
    }
  }
  a.seg_len = seg_len;
  a.nseg = (int)nseg;
  const int64_t nchunks = (L + CT - 1) / CT;
  // sums over time per (slot, channel): one slot per segment, or on the interval plan two per chain
  // (its right part or whole, and its left part)
  const int64_t pslots = IV ? 2 : nseg;
  const int kRSc = ROLES ? roles_scanners<T, N>() : 1;
  const size_t fl[] = {(size_t)(nchunks * chans * N), (size_t)(nchunks * chans), (size_t)(nseg * chans * N),
                       (size_t)(nseg * chans), (size_t)(nseg * chans * N), (size_t)(a.groups * p.batch * N * L),
                       (size_t)(a.groups * p.batch * N * L), (size_t)(pslots * chans * N), (size_t)(pslots * chans),
                       (size_t)(pslots * chans), (size_t)(IV ? units * N * kWave : 0),
                       (size_t)(IV ? 64 + units * kRSc : 0)};
  size_t total = 0;
  for (size_t f : fl) total += (f + 63) / 64 * 64;  // 256-byte aligned pieces
  void* scratch = nullptr;
  bool kept = false;
  hipError_t err = call_scratch(stream, 4, total * sizeof(float), &scratch, &kept);
  if (err != hipSuccess) return err;
  float* q = (float*)scratch;
  float* ctl = nullptr;
  float** dst[] = {&a.ck_h, &a.ck_dt, &a.seg_h, &a.seg_dt, &a.seg_l, &a.pB, &a.pC, &a.pA, &a.pD, &a.pbias, &a.hand_l, &ctl};
  for (int i = 0; i < 12; ++i) {
    *dst[i] = q;
    q += (fl[i] + 63) / 64 * 64;
  }
  if (IV) {
    a.ticket = (int*)ctl;
    a.flags = a.ticket + 64;
    const int64_t work = units * (L / kCT);
    a.wlen = (work + slots_main - 1) / slots_main;  // >= a chain, since units >= slots_main
    a.iunits = (int)((work + a.wlen - 1) / a.wlen);
    handover_wait(&a.max_polls, &a.publish);
  }
  const dim3 grid((unsigned)units, (unsigned)nseg);
  if (FAST && IV) {  // the main pass's ticket and flags (0.0f is all zero bits), cleared by the checkpoint pass
    a.clear = ctl;
    a.clear_n = 64 + units * kRSc;
  }
  if constexpr (FAST) {  // checkpoints (and, on the segment plan, adjoint aggregates) in one grid
    if (uni)
      hipLaunchKernelGGL((fbwd_pre_kernel<N, T, UNIF>), dim3((unsigned)units, (unsigned)(IV ? nseg : 2 * nseg - 1)),
                         dim3(kWave), 0, stream, a);
    else
      hipLaunchKernelGGL((fbwd_pre_kernel<N, T>), dim3((unsigned)units, (unsigned)(IV ? nseg : 2 * nseg - 1)),
                         dim3(kWave), 0, stream, a);
  } else
    hipLaunchKernelGGL((bwd_checkpoint_kernel<N, T>), grid, dim3(kWave), 0, stream, a);
  err = hipGetLastError();
  if (err == hipSuccess && nseg > 1) {
    hipLaunchKernelGGL(bwd_fwd_carry_kernel, dim3(blocks_of(chans * N)), dim3(256), 0, stream, a.seg_h, a.seg_dt,
                       p.A, p.h0, chans, p.dim, N, (int)nseg);
    err = hipGetLastError();
    if (err == hipSuccess && !FAST) {
      const dim3 g1((unsigned)units, (unsigned)(nseg - 1));
      hipLaunchKernelGGL((bwd_adjoint_aggregate_kernel<N, T>), g1, dim3(kWave), 0, stream, a);
      err = hipGetLastError();
    }
    if (err == hipSuccess && !IV) {
      hipLaunchKernelGGL(bwd_adjoint_carry_kernel, dim3(blocks_of(chans * N)), dim3(256), 0, stream, a.seg_l,
                         a.seg_dt, p.A, chans, p.dim, N, (int)nseg);
      err = hipGetLastError();
    }
  }
  if (err == hipSuccess && IV && !FAST) err = zero(ctl, 64 + units * kRSc, stream);  // ticket and flags
  if (err == hipSuccess) {
    if constexpr (ROLES) {
      if (uni)
        hipLaunchKernelGGL((fbwd_main_roles_kernel<N, T, UNIF>), IV ? dim3((unsigned)a.iunits) : grid,
                           dim3(roles_threads<T, N>()), 0, stream, a);
      else
        hipLaunchKernelGGL((fbwd_main_roles_kernel<N, T>), IV ? dim3((unsigned)a.iunits) : grid,
                           dim3(roles_threads<T, N>()), 0, stream, a);
    }
    else if constexpr (FAST)
      hipLaunchKernelGGL((fbwd_main_kernel<N, T>), grid, dim3(kWave * W), 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_main_kernel<N, T>), grid, dim3(kWave), 0, stream, a);
    err = hipGetLastError();
  }
  if (err == hipSuccess) {
    const int64_t count = p.batch * N * L;
    if (count % 4 == 0) {
      const int64_t nbc = (count / 4 + 63) / 64;
      hipLaunchKernelGGL((bwd_reduce_kernel<T>), dim3((unsigned)(nbc + blocks_of(p.dim * N))), dim3(256), 0, stream,
                         a.pB, a.pC, (T*)p.dB, (T*)p.dC, count, a.groups, nbc, a.pA, a.pD, a.pbias, p.dA, p.dD,
                         p.ddt_bias, p.batch, p.dim, N, (int)pslots);
      err = hipGetLastError();
    } else {
      hipLaunchKernelGGL((bwd_bc_reduce_kernel<T>), dim3(blocks_of(count)), dim3(256), 0, stream, a.pB, a.pC,
                         (T*)p.dB, (T*)p.dC, count, a.groups);
      err = hipGetLastError();
      if (err == hipSuccess) {
        hipLaunchKernelGGL(bwd_param_reduce_kernel, dim3(blocks_of(p.dim * N)), dim3(256), 0, stream, a.pA, a.pD,
                           a.pbias, p.dA, p.dD, p.ddt_bias, p.batch, p.dim, N, (int)pslots);
        err = hipGetLastError();
      }
    }
  }
  const hipError_t ferr = call_scratch_release(scratch, kept, stream);
  return err != hipSuccess ? err : ferr;
}

template <typename T>
hipError_t dispatch_n(const BwdParams& p, hipStream_t s) {
  const bool fast = fast_ok(p);
  switch (p.dstate) {
    case 1: return run<1, T, false>(p, s);
    case 2: return run<2, T, false>(p, s);
    case 4: return run<4, T, false>(p, s);
    case 8: return fast ? run<8, T, true>(p, s) : run<8, T, false>(p, s);
    case 16: return fast ? run<16, T, true>(p, s) : run<16, T, false>(p, s);
    case 32: return fast ? run<32, T, true>(p, s) : run<32, T, false>(p, s);
    case 64: return fast ? run<64, T, true>(p, s) : run<64, T, false>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t bwd_handover_failures(uint64_t* count, bool reset) {
  unsigned int v = 0;
  hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(bwd_handover_giveups), sizeof v, 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  *count = v;
  if (reset) {
    const unsigned int zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(bwd_handover_giveups), &zero, sizeof zero, 0, hipMemcpyHostToDevice);
  }
  return e;
}

hipError_t launch_scan_bwd(const BwdParams& p, hipStream_t stream) {
  if (p.seqlen == 0) {
    hipError_t e = zero(p.dA, p.dim * p.dstate, stream);
    if (e == hipSuccess) e = zero(p.dD, p.dim, stream);
    if (e == hipSuccess) e = zero(p.ddt_bias, p.dim, stream);
    if (e == hipSuccess) e = zero(p.dh0, p.batch * p.dim * p.dstate, stream);
    return e;
  }
  return p.dtype == kBF16 ? dispatch_n<__bf16>(p, stream) : dispatch_n<float>(p, stream);
}

}  // namespace ssm
