// scan_fwd.hip -- generic forward selective scan on gfx950, and the dispatcher.
//
// The fast path is scan_chunked.hip; it needs 16-byte aligned rows
// (seqlen * element size a multiple of 16) and 16-byte aligned u, delta, z, y.
// Every other shape runs through the generic kernels below.
//
// Work decomposition.  Each (batch row b, channel d) is an independent
// recurrence over t with dstate diagonal states.  A wavefront holds 64
// consecutive channels of one batch row, one channel per lane, all dstate
// states of that channel in registers.  B_t and C_t are shared by every channel
// of a batch row, so within a wave their addresses are uniform.
//
// Sequence splitting.  The recurrence h_t = Abar_t h_{t-1} + b_t is an
// associative scan over (Abar, b) pairs ("Mamba close reading" (jsqmd.com)
// §2.2 and the chunked sketch of §7; mlqm.cn tutorial §6; tech.kj168168.com
// essay §二.3), so the sequence is cut into S segments processed in parallel:
//   1. aggregate pass: every segment but the last runs the recurrence from
//      h = 0 and stores its end state and sum(Delta) -- the segment's
//      transition product is exp(A * sum(Delta)), since the ZOH factors of a
//      diagonal system multiply by adding exponents;
//   2. carry pass: one thread per (b, d, n) walks the S segment aggregates in
//      order, turning them into each segment's incoming state;
//   3. output pass: every segment reruns its recurrence from its incoming
//      state and writes y (and the final state).
// With S = 1 only the output pass runs.  Softplus, discretisation, recurrence,
// readout, skip and gate are fused in one loop; only y and the final state
// reach HBM (the fused, on-chip-intermediates design the Mamba summary
// (junchaoiu.github.io) describes in 方法 step 2).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {
namespace {

constexpr int kWave = 64;

struct SegArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* dt_bias;
  void* y;
  float* last_state;
  const float* h0;
  float* seg_h;    // [S, batch*dim, N]: aggregate end states, then incoming states
  float* seg_dt;   // [S, batch*dim]: sum of Delta over the segment
  int64_t batch, dim, seqlen, seg_len;
  int groups;      // channel groups of 64 per batch row
  int nseg;
  int softplus;
};

// MODE 0: output pass (y, last_state).  MODE 1: aggregate pass (seg_h, seg_dt).
template <int N, typename T, int MODE>
__global__ __launch_bounds__(kWave) void scan_segment_kernel(SegArgs a) {
  const int lane = threadIdx.x;
  const int64_t b = blockIdx.x / a.groups;
  const int64_t d = (int64_t)(blockIdx.x % a.groups) * kWave + lane;
  const int seg = blockIdx.y;
  const bool active = d < a.dim;
  const int64_t dd = active ? d : a.dim - 1;
  const int64_t ch = b * a.dim + dd;
  const int64_t L = a.seqlen;
  const int64_t t0 = (int64_t)seg * a.seg_len;
  const int64_t t1 = t0 + a.seg_len < L ? t0 + a.seg_len : L;

  const T* __restrict__ u = (const T*)a.u + ch * L;
  const T* __restrict__ dl = (const T*)a.delta + ch * L;
  const T* __restrict__ zz = a.z ? (const T*)a.z + ch * L : nullptr;
  const T* __restrict__ Bp = (const T*)a.B + b * N * L;
  const T* __restrict__ Cp = (const T*)a.C + b * N * L;

  float A2[N], h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) A2[n] = a.A[dd * N + n] * kLog2e;
  // With several segments every output segment, the first included, starts from the carry
  // pass's incoming state (seg_h[0] = initial state): the initial state is then read only by
  // the carry pass, so it may be the same buffer as last_state, which this pass writes.
  if (MODE == 0 && a.seg_h) {
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = a.seg_h[((int64_t)seg * a.batch * a.dim + ch) * N + n];
  } else if (MODE == 0 && a.h0) {
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = a.h0[ch * N + n];
  } else {
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = 0.0f;
  }
  const float bias = a.dt_bias ? a.dt_bias[dd] : 0.0f;
  const float Dd = a.D ? a.D[dd] : 0.0f;
  float sum_dt = 0.0f;

  for (int64_t t = t0; t < t1; ++t) {
    const float x = ld(dl, t) + bias;
    const float dt = a.softplus ? softplus(x) : x;
    const float ut = ld(u, t);
    const float du = dt * ut;
    float acc = 0.0f;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const float abar = ex2(dt * A2[n]);
      h[n] = __builtin_fmaf(abar, h[n], du * ld(Bp, (int64_t)n * L + t));
      if (MODE == 0) acc = __builtin_fmaf(ld(Cp, (int64_t)n * L + t), h[n], acc);
    }
    if (MODE == 0) {
      float yt = __builtin_fmaf(Dd, ut, acc);
      if (zz) yt *= silu(ld(zz, t));
      if (active) st((T*)a.y + ch * L, t, yt);
    } else {
      sum_dt += dt;
    }
  }
  if (!active) return;
  if (MODE == 1) {
    float* sh = a.seg_h + ((int64_t)seg * a.batch * a.dim + ch) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) sh[n] = h[n];
    a.seg_dt[(int64_t)seg * a.batch * a.dim + ch] = sum_dt;
  } else if (a.last_state && t1 == L) {
#pragma unroll
    for (int n = 0; n < N; ++n) a.last_state[ch * N + n] = h[n];
  }
}

// last_state for an empty sequence: the initial state (or zeros), by a kernel rather than a
// memset or copy node, so the call stays safe to capture in a graph.
__global__ __launch_bounds__(256) void empty_sequence_state(float* last, const float* h0, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) last[i] = h0 ? h0[i] : 0.0f;
}

// One thread per (channel, n): turn segment aggregates into incoming states, in place.
// seg_h[s] holds segment s's end state from h = 0; afterwards it holds the state
// entering segment s (seg_h[0] = initial state).
__global__ __launch_bounds__(256) void scan_carry_kernel(float* seg_h, const float* seg_dt, const float* A,
                                                         const float* h0, int64_t chans, int64_t dim, int N,
                                                         int nseg) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= chans * N) return;
  const int64_t ch = i / N;
  const int n = (int)(i % N);
  const float A2 = A[(ch % dim) * N + n] * kLog2e;
  float h = h0 ? h0[i] : 0.0f;
  // 16 segments at a time, their loads all in flight before the first is used
  constexpr int kBatch = 16;
  for (int s0 = 0; s0 < nseg; s0 += kBatch) {
    const int nb = nseg - s0 < kBatch ? nseg - s0 : kBatch;
    float agg[kBatch], sdt[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (k < nb) {
        agg[k] = seg_h[(int64_t)(s0 + k) * chans * N + i];
        sdt[k] = seg_dt[(int64_t)(s0 + k) * chans + ch];
      }
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (k < nb) {
        seg_h[(int64_t)(s0 + k) * chans * N + i] = h;
        h = __builtin_fmaf(ex2(A2 * sdt[k]), h, agg[k]);
      }
  }
}

// Segments of the generic scan: enough waves to fill 256 CUs x 4 SIMDs several times over.
void generic_segments(const ScanParams& p, int64_t* nseg_out, int64_t* seg_len_out) {
  const int64_t waves = p.batch * ((p.dim + kWave - 1) / kWave);
  const int64_t target = 4096;
  int64_t nseg = std::max<int64_t>(1, (target + waves - 1) / waves);
  nseg = std::min<int64_t>(nseg, std::max<int64_t>(1, p.seqlen / 64));
  int64_t seg_len = (p.seqlen + nseg - 1) / nseg;
  seg_len = (seg_len + 7) / 8 * 8;
  nseg = std::max<int64_t>(1, (p.seqlen + seg_len - 1) / seg_len);
  *nseg_out = nseg;
  *seg_len_out = seg_len;
}

template <int N, typename T>
hipError_t run(const ScanParams& p, hipStream_t stream) {
  SegArgs a{};
  a.u = p.u; a.delta = p.delta; a.A = p.A; a.B = p.B; a.C = p.C; a.D = p.D; a.z = p.z;
  a.dt_bias = p.dt_bias; a.y = p.y; a.last_state = p.last_state; a.h0 = p.h0;
  a.batch = p.batch; a.dim = p.dim; a.seqlen = p.seqlen; a.softplus = p.softplus;
  a.groups = (int)((p.dim + kWave - 1) / kWave);
  const int64_t waves = p.batch * a.groups;
  int64_t nseg, seg_len;
  generic_segments(p, &nseg, &seg_len);
  a.seg_len = seg_len;
  a.nseg = (int)nseg;
  const int64_t chans = p.batch * p.dim;
  hipError_t err = hipSuccess;
  if (nseg > 1) {
    const size_t bytes = (size_t)nseg * chans * (N + 1) * sizeof(float);
    void* scratch = nullptr;
    err = scratch_acquire(p, &scratch, bytes, stream);
    if (err != hipSuccess) return err;
    a.seg_h = (float*)scratch;
    a.seg_dt = a.seg_h + (size_t)nseg * chans * N;
    // aggregate pass over segments 0 .. S-2
    hipLaunchKernelGGL((scan_segment_kernel<N, T, 1>), dim3((unsigned)waves, (unsigned)(nseg - 1)), dim3(kWave),
                       0, stream, a);
    err = hipGetLastError();
    if (err == hipSuccess) {
      const int64_t threads = chans * N;
      hipLaunchKernelGGL(scan_carry_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a.seg_h,
                         a.seg_dt, p.A, p.h0, chans, p.dim, N, (int)nseg);
      err = hipGetLastError();
    }
    if (err == hipSuccess) {
      hipLaunchKernelGGL((scan_segment_kernel<N, T, 0>), dim3((unsigned)waves, (unsigned)nseg), dim3(kWave), 0,
                         stream, a);
      err = hipGetLastError();
    }
    hipError_t ferr = scratch_release(p, scratch, stream);
    return err != hipSuccess ? err : ferr;
  }
  hipLaunchKernelGGL((scan_segment_kernel<N, T, 0>), dim3((unsigned)waves, 1), dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_n(const ScanParams& p, hipStream_t s) {
  switch (p.dstate) {
    case 1: return run<1, T>(p, s);
    case 2: return run<2, T>(p, s);
    case 4: return run<4, T>(p, s);
    case 8: return run<8, T>(p, s);
    case 16: return run<16, T>(p, s);
    case 32: return run<32, T>(p, s);
    case 64: return run<64, T>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool dstate_supported(int64_t n) { return n == 1 || n == 2 || n == 4 || n == 8 || n == 16 || n == 32 || n == 64; }

size_t generic_scratch_bytes(const ScanParams& p) {
  if (p.seqlen == 0) return 0;
  int64_t nseg, seg_len;
  generic_segments(p, &nseg, &seg_len);
  return nseg > 1 ? (size_t)nseg * (size_t)(p.batch * p.dim) * (size_t)(p.dstate + 1) * sizeof(float) : 0;
}

size_t scan_scratch_bytes(const ScanParams& p, int cus) {
  if (p.seqlen > 0 && chunked_supported(p)) return chunked_scratch_bytes(p, cus);
  return generic_scratch_bytes(p);
}

hipError_t launch_scan_generic(const ScanParams& p, hipStream_t stream) {
  if (p.seqlen == 0) {
    if (p.last_state && p.last_state != p.h0) {
      const int64_t n = p.batch * p.dim * p.dstate;
      hipLaunchKernelGGL(empty_sequence_state, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p.last_state,
                         p.h0, n);
      return hipGetLastError();
    }
    return hipSuccess;
  }
  return p.dtype == kBF16 ? dispatch_n<__bf16>(p, stream) : dispatch_n<float>(p, stream);
}

// Causal conv1d + SiLU and the scan in one call (p.cw set, p.u = x).  On the fast path the
// convolution runs inside the scan kernels (u never reaches memory); otherwise the convolution
// kernel writes u to scratch and the scan reads it.  Either way the convolution state is written
// as causal_conv1d_fwd writes it.
static hipError_t launch_scan_fwd_conv(const ScanParams& p, hipStream_t stream) {
  ConvParams c{p.u, p.cw, p.cb, p.cst, 1, nullptr, p.cst_out, p.batch, p.dim, p.seqlen, p.ck, p.dtype};
  ScanParams q = p;
  q.cw = nullptr; q.cb = nullptr; q.cst = nullptr; q.cst_out = nullptr; q.ck = 0;
  q.ws = nullptr; q.ws_bytes = 0;
  if (p.seqlen == 0) {
    hipError_t e = launch_conv1d_fwd(c, stream);  // state in -> state out
    return e != hipSuccess ? e : launch_scan_generic(q, stream);
  }
  if (chunked_conv_supported(p)) {
    hipError_t e = launch_scan_chunked(p, stream);
    return e != hipSuccess ? e : launch_conv1d_state_out(c, stream);
  }
  const size_t bytes = (size_t)(p.batch * p.dim * p.seqlen) * (p.dtype == kBF16 ? 2 : 4);
  void* u = nullptr;
  const bool kept = stream_scratch(stream, 1, bytes, &u);
  hipError_t e = kept ? hipSuccess : scratch_alloc(&u, bytes, stream);
  if (e != hipSuccess) return e;
  c.out = u;
  e = launch_conv1d_fwd(c, stream);
  if (e == hipSuccess) {
    q.u = u;
    e = launch_scan_fwd(q, stream);
  }
  const hipError_t f = kept ? hipSuccess : hipFreeAsync(u, stream);
  return e != hipSuccess ? e : f;
}

hipError_t launch_scan_fwd(const ScanParams& p, hipStream_t stream) {
  if (p.cw) return launch_scan_fwd_conv(p, stream);
  if (p.seqlen > 0 && chunked_supported(p)) return launch_scan_chunked(p, stream);
  return launch_scan_generic(p, stream);
}

}  // namespace ssm
