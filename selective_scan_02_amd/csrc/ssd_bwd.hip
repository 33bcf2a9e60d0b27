// ssd_bwd.hip -- backward of the Mamba-2 SSD form (one decay rate and one step size per head).
//
// The SSD layer (mlqm.cn tutorial §8; "AI inference series (14)", the part on how Mamba-2
// reorganises the SSM into matrix computation) is the selective recurrence with A[d, n] =
// A_heads[h] for every state n and delta[b, d, t] = dt[b, h, t] for every channel d of head h
// (dt_bias likewise per head).  Its gradients are therefore those of the selective scan's
// backward on the broadcast parameters, with each broadcast parameter's gradient summed back over
// what it was broadcast to (the chain rule):
//   ddt[b, h, t]  = sum over the head's channels p of ddelta[b, h*P + p, t]
//   dA[h]         = sum over the head's channels and all states of dA[h*P + p, n]
//   ddt_bias[h]   = sum over the head's channels of ddt_bias[h*P + p]
// and every other gradient (dx, dz, dB, dC, dD, dh0) is the scan's own.  So this runs: one kernel
// that broadcasts dt (and A, dt_bias) to the channels, the backward scan's kernels
// (scan_bwd.hip) on the broadcast problem, and one kernel that sums the head gradients in a fixed
// order (results reproducible bit for bit).  The per-channel step-size gradients are kept in fp32
// (the backward scan writes them so on request): summed from the I/O dtype, 64 rounded terms per
// head put the head gradient 3% off on the 2.8B-shaped layer.  The broadcast step sizes (dtype of
// x) and those gradients (fp32) live in pool scratch, batch x heads*headdim x L of each.
#include <hip/hip_runtime.h>

#include "ssm_launch.h"

namespace ssm {
namespace {

// delta[b, d, t] = dt[b, d / P, t], E elements per thread (16 bytes when rows allow).
template <typename T, int E>
__device__ __forceinline__ void bcast_dt(const T* __restrict__ dt, T* __restrict__ delta, int64_t rows, int64_t dim,
                                         int64_t heads, int64_t P, int64_t L, int64_t blk) {
  const int64_t per_row = L / E;
  const int64_t i = blk * 256 + threadIdx.x;
  if (i >= rows * per_row) return;
  const int64_t r = i / per_row, q = i - r * per_row;
  const int64_t b = r / dim, d = r - b * dim;
  const T* src = dt + (b * heads + d / P) * L + q * E;
  T* dst = delta + r * L + q * E;
  if constexpr (E * sizeof(T) == 16) {
    *(uint4*)dst = *(const uint4*)src;
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e] = src[e];
  }
}

// A_full[d, n] = A[d / P]; bias_full[d] = dt_bias[d / P].
__device__ __forceinline__ void bcast_param(const float* A, const float* dt_bias, float* A_full, float* bias_full,
                                            int64_t dim, int64_t P, int64_t N, int64_t blk) {
  const int64_t i = blk * 256 + threadIdx.x;
  if (i >= dim * N) return;
  const int64_t d = i / N;
  A_full[i] = A[d / P];
  if (bias_full && i % N == 0) bias_full[d] = dt_bias[d / P];
}

// ddt[b, h, t] = sum_{p < P} ddelta[b, h*P + p, t], in fp32, p ascending (ddelta is fp32).  A thread
// takes E consecutive steps (16-byte loads when rows allow), and the p loop is unrolled so that
// several rows' loads are in flight at once; each step's sum keeps the same order either way.
template <typename T, int E>
__device__ __forceinline__ void sum_dt(const float* __restrict__ ddelta, T* __restrict__ ddt, int64_t batch,
                                       int64_t heads, int64_t P, int64_t L, int64_t blk) {
  const int64_t per_row = L / E;
  const int64_t i = blk * 256 + threadIdx.x;
  if (i >= batch * heads * per_row) return;
  const int64_t bh = i / per_row, t = (i - bh * per_row) * E;
  const float* src = ddelta + bh * P * L + t;  // rows b*dim + h*P + p = (b*heads + h)*P + p
  float s[E];
#pragma unroll
  for (int e = 0; e < E; ++e) s[e] = 0.0f;
#pragma unroll 8
  for (int64_t p = 0; p < P; ++p) {
    if constexpr (E == 4) {
      const float4 v = *(const float4*)(src + p * L);
      s[0] += v.x; s[1] += v.y; s[2] += v.z; s[3] += v.w;
    } else {
      s[0] += src[p * L];
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) ddt[bh * L + t + e] = (T)s[e];
}

// dA[h] = sum_{p, n} dA_full[h*P + p, n]; ddt_bias[h] = sum_p dbias_full[h*P + p].  One workgroup per
// head: thread j sums terms j, j + 256, ... in order, then a fixed pairwise tree in LDS (results
// reproducible bit for bit).
__device__ __forceinline__ void sum_param(const float* dA_full, const float* dbias_full, float* dA, float* ddt_bias,
                                          int64_t P, int64_t N, int64_t h) {
  __shared__ float red[2][256];
  const int j = threadIdx.x;
  float s = 0.0f, sb = 0.0f;
  for (int64_t k = j; k < P * N; k += 256) s += dA_full[h * P * N + k];
  if (dbias_full)
    for (int64_t p = j; p < P; p += 256) sb += dbias_full[h * P + p];
  red[0][j] = s;
  red[1][j] = sb;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (j < w) {
      red[0][j] += red[0][j + w];
      red[1][j] += red[1][j + w];
    }
    __syncthreads();
  }
  if (j == 0) {
    dA[h] = red[0][0];
    if (ddt_bias) ddt_bias[h] = red[1][0];
  }
}

// The per-head parameters broadcast to every channel (step sizes: blocks 0 .. nb-1; A and the step
// bias: the rest), in one grid ahead of the backward scan.
template <typename T, int E>
__global__ __launch_bounds__(256) void ssd_bcast_kernel(const T* dt, T* delta, int64_t rows, int64_t dim, int64_t heads,
                                                        int64_t P, int64_t L, int64_t nb, const float* A,
                                                        const float* dt_bias, float* A_full, float* bias_full,
                                                        int64_t N) {
  if ((int64_t)blockIdx.x < nb)
    bcast_dt<T, E>(dt, delta, rows, dim, heads, P, L, blockIdx.x);
  else
    bcast_param(A, dt_bias, A_full, bias_full, dim, P, N, (int64_t)blockIdx.x - nb);
}

// The per-head sums after it (step-size gradients: blocks 0 .. nb-1; dA and the step-bias gradient: one
// block per head after them), in one grid.
template <typename T, int E>
__global__ __launch_bounds__(256) void ssd_sum_kernel(const float* ddelta, T* ddt, int64_t batch, int64_t heads,
                                                      int64_t P, int64_t L, int64_t nb, const float* dA_full,
                                                      const float* dbias_full, float* dA, float* ddt_bias, int64_t N) {
  if ((int64_t)blockIdx.x < nb)
    sum_dt<T, E>(ddelta, ddt, batch, heads, P, L, blockIdx.x);
  else
    sum_param(dA_full, dbias_full, dA, ddt_bias, P, N, (int64_t)blockIdx.x - nb);
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }
size_t aligned(size_t bytes) { return (bytes + 255) / 256 * 256; }

template <typename T>
hipError_t run(const SsdBwdParams& q, hipStream_t stream) {
  const SsdParams& f = q.f;
  const int64_t P = f.headdim, H = f.heads, N = f.dstate, L = f.seqlen, dim = H * P;
  const int64_t rows = f.batch * dim;
  const size_t nfull = (size_t)rows * (size_t)L;
  const size_t sz[] = {aligned(nfull * sizeof(T)), aligned(nfull * sizeof(float)), aligned((size_t)dim * N * 4),
                       aligned((size_t)dim * N * 4), aligned((size_t)dim * 4), aligned((size_t)dim * 4)};
  size_t total = 0;
  for (size_t v : sz) total += v;
  void* scratch = nullptr;
  bool kept = false;
  hipError_t err = call_scratch(stream, 3, total, &scratch, &kept);
  if (err != hipSuccess) return err;
  char* c = (char*)scratch;
  T* delta = (T*)c;            c += sz[0];
  float* ddelta = (float*)c;   c += sz[1];  // per-channel gradients kept in fp32 for the head sums
  float* A_full = (float*)c;   c += sz[2];
  float* dA_full = (float*)c;  c += sz[3];
  float* bias_full = (float*)c; c += sz[4];
  float* dbias_full = (float*)c;
  const bool with_bias = f.dt_bias != nullptr;

  {
    constexpr int E = 16 / (int)sizeof(T);
    const bool vec = L % E == 0 && ((uintptr_t)f.dt & 15) == 0;
    const int64_t nb = L > 0 ? (int64_t)blocks_for(rows * (vec ? L / E : L)) : 0;
    const dim3 g((unsigned)(nb + blocks_for(dim * N)));
    if (vec)
      hipLaunchKernelGGL((ssd_bcast_kernel<T, E>), g, dim3(256), 0, stream, (const T*)f.dt, delta, rows, dim, H, P, L,
                         nb, f.A, f.dt_bias, A_full, with_bias ? bias_full : nullptr, N);
    else
      hipLaunchKernelGGL((ssd_bcast_kernel<T, 1>), g, dim3(256), 0, stream, (const T*)f.dt, delta, rows, dim, H, P, L,
                         nb, f.A, f.dt_bias, A_full, with_bias ? bias_full : nullptr, N);
    err = hipGetLastError();
  }
  if (err == hipSuccess) {
    BwdParams b{};
    b.u = f.x; b.delta = delta; b.A = A_full; b.B = f.B; b.C = f.C; b.D = f.D; b.z = f.z;
    b.dt_bias = with_bias ? bias_full : nullptr; b.softplus = f.softplus; b.h0 = f.h0; b.dy = q.dy;
    b.du = q.dx; b.ddelta = ddelta; b.dA = dA_full; b.dB = q.dB; b.dC = q.dC; b.dD = q.dD; b.dz = q.dz;
    b.ddt_bias = q.ddt_bias ? dbias_full : nullptr; b.dh0 = q.dh0;
    b.batch = f.batch; b.dim = dim; b.dstate = N; b.seqlen = L; b.dtype = q.dtype;
    b.ddelta_f32 = true;
    b.a_uniform = true;
    err = launch_scan_bwd(b, stream);
  }
  if (err == hipSuccess) {
    const bool v4 = L % 4 == 0;
    const int64_t nb = L > 0 ? (int64_t)blocks_for(f.batch * H * (v4 ? L / 4 : L)) : 0;
    const dim3 g((unsigned)(nb + H));
    if (v4)
      hipLaunchKernelGGL((ssd_sum_kernel<T, 4>), g, dim3(256), 0, stream, ddelta, (T*)q.ddt, f.batch, H, P, L, nb,
                         dA_full, q.ddt_bias ? dbias_full : nullptr, q.dA, q.ddt_bias, N);
    else
      hipLaunchKernelGGL((ssd_sum_kernel<T, 1>), g, dim3(256), 0, stream, ddelta, (T*)q.ddt, f.batch, H, P, L, nb,
                         dA_full, q.ddt_bias ? dbias_full : nullptr, q.dA, q.ddt_bias, N);
    err = hipGetLastError();
  }
  const hipError_t ferr = call_scratch_release(scratch, kept, stream);
  return err != hipSuccess ? err : ferr;
}

}  // namespace

hipError_t launch_ssd_bwd(const SsdBwdParams& p, hipStream_t stream) {
  return p.dtype == kBF16 ? run<__bf16>(p, stream) : run<float>(p, stream);
}

}  // namespace ssm
