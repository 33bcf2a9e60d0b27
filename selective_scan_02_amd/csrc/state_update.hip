// state_update.hip -- single-token selective state update (decode) on gfx950.
//
// One autoregressive step for every (request b, channel d): the fixed-size
// state h[b, d, :] is read, advanced by one step of the recurrence and written
// back in place, and y[b, d] is produced ("AI inference series (14)",
// wiblog.cn: decode is a single-step recurrent update of a per-request state
// updated in place; mlqm.cn tutorial §9.2: dA = exp(dt*A), dB = dt*B,
// h = dA*h + dB*x, y = sum(C*h) + D*x).
//
// The step is bound by HBM: 2*dstate*4 bytes of state traffic per (b, d)
// against a few bytes of inputs.  Layout: each lane owns 4 consecutive states
// of one (b, d) row (one 16-byte load and store), so a wave reads a contiguous
// 1 KiB of state per instruction; the dstate/4 lanes of a row combine their
// partial readouts with cross-lane adds.
#include <hip/hip_runtime.h>

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {
namespace {

struct StepArgs {
  float* state;
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* dt_bias;
  void* y;
  int64_t rows, dim;
};

template <int N, typename T>
__global__ __launch_bounds__(256) void state_update_kernel(StepArgs a) {
  constexpr int LPR = N >= 4 ? N / 4 : 1;  // lanes per (b, d) row
  constexpr int SPL = N / LPR;             // states per lane
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / LPR;
  const int q = (int)(gid % LPR);
  const bool active = row < a.rows;
  const int64_t r = active ? row : a.rows - 1;
  const int64_t b = r / a.dim, d = r % a.dim;

  float* sp = a.state + r * N + q * SPL;
  float h[SPL];
  if constexpr (SPL == 4) {
    const float4 v = *reinterpret_cast<const float4*>(sp);
    h[0] = v.x; h[1] = v.y; h[2] = v.z; h[3] = v.w;
  } else {
#pragma unroll
    for (int j = 0; j < SPL; ++j) h[j] = sp[j];
  }
  const float x = ld((const T*)a.delta, r) + (a.dt_bias ? a.dt_bias[d] : 0.0f);
  const float dt = softplus(x);
  const float ut = ld((const T*)a.u, r);
  const float du = dt * ut;
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    const int n = q * SPL + j;
    const float abar = ex2(dt * (a.A[d * N + n] * kLog2e));
    h[j] = __builtin_fmaf(abar, h[j], du * ld((const T*)a.B, b * N + n));
    acc = __builtin_fmaf(ld((const T*)a.C, b * N + n), h[j], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (!active) return;
  if constexpr (SPL == 4) {
    *reinterpret_cast<float4*>(sp) = make_float4(h[0], h[1], h[2], h[3]);
  } else {
#pragma unroll
    for (int j = 0; j < SPL; ++j) sp[j] = h[j];
  }
  if (q == 0) {
    float yt = __builtin_fmaf(a.D ? a.D[d] : 0.0f, ut, acc);
    if (a.z) yt *= silu(ld((const T*)a.z, r));
    st((T*)a.y, r, yt);
  }
}

template <int N, typename T>
hipError_t run(const StepParams& p, hipStream_t stream) {
  StepArgs a{p.state, p.u, p.delta, p.A, p.B, p.C, p.D, p.z, p.dt_bias, p.y, p.batch * p.dim, p.dim};
  constexpr int LPR = N >= 4 ? N / 4 : 1;
  const int64_t threads = a.rows * LPR;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((state_update_kernel<N, T>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_n(const StepParams& p, hipStream_t s) {
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

hipError_t launch_state_update(const StepParams& p, hipStream_t stream) {
  return p.dtype == kBF16 ? dispatch_n<__bf16>(p, stream) : dispatch_n<float>(p, stream);
}

}  // namespace ssm
