// conv1d.hip -- causal depthwise 1-D convolution (+ SiLU) and its decode step, gfx950.
//
// The step just before the selective SSM in the Mamba block: a short causal
// convolution along the sequence, one filter per channel, then SiLU (Mamba
// summary (junchaoiu.github.io), 方法 third step; mlqm.cn tutorial §7.1).  A
// request in decode keeps the K-1 most recent inputs of every channel as its
// convolution state next to the SSM state ("AI inference series (14)",
// wiblog.cn: per-request conv state and SSM state, updated in place).
//
//   v_t = bias[d] + sum_{k<K} w[d,k] * x[t-(K-1)+k],   out_t = silu(v_t) (or v_t)
//
// Both kernels are bound by HBM: K FMAs and one SiLU per element against
// 2 x (element size) bytes.  conv1d_fwd_kernel: a wave covers 512 consecutive
// steps of one row, 8 per lane, loaded and stored as 16-byte pieces; the K-1
// inputs before a lane's first step come from the previous lane by a cross-lane
// shift (lane 0 reads them from memory, or from the state before step 0).
// conv1d_update_kernel: one thread per row shifts the window in place.
#include <hip/hip_runtime.h>

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {
namespace {

constexpr int kEPT = 8;               // steps per lane
constexpr int kWaveSteps = 64 * kEPT;  // steps per wave

struct ConvArgs {
  const void* x;
  const float* w;
  const float* bias;
  const float* st_in;   // [rows, K-1] or NULL
  void* out;
  float* st_out;        // [rows, K-1] or NULL
  int64_t rows, dim, L, nseg;
  int silu;
  int vec;              // rows are whole 16-byte pieces and x, out are 16-byte aligned
};

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[kEPT]) {
  if constexpr (sizeof(T) == 2) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __builtin_bit_cast(float, w4[i] << 16);
      v[2 * i + 1] = __builtin_bit_cast(float, w4[i] & 0xffff0000u);
    }
  } else {
    const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&o)[kEPT]) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)o[2 * i]);
      const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)o[2 * i + 1]);
      w4[i] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(p) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  } else {
    reinterpret_cast<float4*>(p)[0] = make_float4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(o[4], o[5], o[6], o[7]);
  }
}

template <int K, typename T>
__global__ __launch_bounds__(256) void conv1d_fwd_kernel(const ConvArgs a) {
  constexpr int H = K > 1 ? K - 1 : 1;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= a.rows * a.nseg) return;  // uniform per wave
  const int64_t row = wave / a.nseg;
  const int64_t t0 = (wave - row * a.nseg) * kWaveSteps + (int64_t)lane * kEPT;
  const int64_t L = a.L;
  const int64_t d = row % a.dim;
  const T* xr = (const T*)a.x + row * L;
  const bool full = a.vec && t0 + kEPT <= L;

  float v[kEPT];
  if (full) {
    load8(xr + t0, v);
  } else {
#pragma unroll
    for (int e = 0; e < kEPT; ++e) v[e] = t0 + e < L ? ld(xr, t0 + e) : 0.0f;
  }
  // inputs at steps t0-(K-1) .. t0-1: the previous lane's last K-1 values
  float hst[H];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) hst[j] = __shfl_up(v[kEPT - (K - 1) + j], 1, 64);
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      const int64_t s = t0 - (K - 1) + j;
      hst[j] = s >= 0 ? ld(xr, s) : (a.st_in ? a.st_in[row * (K - 1) + (K - 1) + s] : 0.0f);
    }
  }
  float w[K];
#pragma unroll
  for (int k = 0; k < K; ++k) w[k] = a.w[d * K + k];
  const float bias = a.bias ? a.bias[d] : 0.0f;

  float o[kEPT];
#pragma unroll
  for (int e = 0; e < kEPT; ++e) {
    float acc = bias;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int s = e - (K - 1) + k;  // step relative to t0
      acc = __builtin_fmaf(w[k], s >= 0 ? v[s >= 0 ? s : 0] : hst[s >= 0 ? 0 : K - 1 + s], acc);
    }
    o[e] = a.silu ? silu(acc) : acc;
  }
  T* orow = (T*)a.out + row * L;
  if (full) {
    store8(orow + t0, o);
  } else {
#pragma unroll
    for (int e = 0; e < kEPT; ++e)
      if (t0 + e < L) st(orow, t0 + e, o[e]);
  }
  // the lane holding step L-1 writes the state a following call continues from
  if (a.st_out && K > 1 && t0 <= L - 1 && L - 1 < t0 + kEPT) {
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      const int64_t s = L - (K - 1) + j;  // input step; >= t0 - (K-1)
      const int r = (int)(s - t0);
      a.st_out[row * (K - 1) + j] = r >= 0 ? v[r >= 0 ? r : 0] : hst[r >= 0 ? 0 : K - 1 + r];
    }
  }
}

// seqlen == 0: the state out is the state in (or zeros)
__global__ __launch_bounds__(256) void conv1d_copy_state(float* dst, const float* src, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}

struct UpdArgs {
  float* state;
  const void* x;
  const float* w;
  const float* bias;
  void* out;
  int64_t rows, dim;
  int silu;
};

template <int K, typename T>
__global__ __launch_bounds__(256) void conv1d_update_kernel(const UpdArgs a) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= a.rows) return;
  const int64_t d = r % a.dim;
  float win[K];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) win[j] = a.state[r * (K - 1) + j];
  win[K - 1] = ld((const T*)a.x, r);
  float acc = a.bias ? a.bias[d] : 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) acc = __builtin_fmaf(a.w[d * K + k], win[k], acc);
  st((T*)a.out, r, a.silu ? silu(acc) : acc);
#pragma unroll
  for (int j = 0; j < K - 1; ++j) a.state[r * (K - 1) + j] = win[j + 1];
}

template <int K, typename T>
hipError_t run_fwd(const ConvParams& p, hipStream_t stream) {
  ConvArgs a{p.x, p.weight, p.bias, p.state_in, p.out, p.state_out, p.batch * p.dim, p.dim, p.seqlen,
             (p.seqlen + kWaveSteps - 1) / kWaveSteps, p.silu, 0};
  const int64_t es = sizeof(T);
  a.vec = (p.seqlen * es) % 16 == 0 && ((uintptr_t)p.x % 16) == 0 && ((uintptr_t)p.out % 16) == 0;
  const int64_t waves = a.rows * a.nseg;
  hipLaunchKernelGGL((conv1d_fwd_kernel<K, T>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int K, typename T>
hipError_t run_update(const ConvStepParams& p, hipStream_t stream) {
  UpdArgs a{p.state, p.x, p.weight, p.bias, p.out, p.batch * p.dim, p.dim, p.silu};
  hipLaunchKernelGGL((conv1d_update_kernel<K, T>), dim3((unsigned)((a.rows + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_fwd(const ConvParams& p, hipStream_t s) {
  switch (p.width) {
    case 1: return run_fwd<1, T>(p, s);
    case 2: return run_fwd<2, T>(p, s);
    case 3: return run_fwd<3, T>(p, s);
    case 4: return run_fwd<4, T>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t dispatch_update(const ConvStepParams& p, hipStream_t s) {
  switch (p.width) {
    case 1: return run_update<1, T>(p, s);
    case 2: return run_update<2, T>(p, s);
    case 3: return run_update<3, T>(p, s);
    case 4: return run_update<4, T>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_conv1d_fwd(const ConvParams& p, hipStream_t stream) {
  if (p.seqlen == 0) {
    if (p.state_out && p.width > 1 && p.state_out != p.state_in) {
      const int64_t n = p.batch * p.dim * (p.width - 1);
      hipLaunchKernelGGL(conv1d_copy_state, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p.state_out,
                         p.state_in, n);
      return hipGetLastError();
    }
    return hipSuccess;
  }
  return p.dtype == kBF16 ? dispatch_fwd<__bf16>(p, stream) : dispatch_fwd<float>(p, stream);
}

hipError_t launch_conv1d_update(const ConvStepParams& p, hipStream_t stream) {
  return p.dtype == kBF16 ? dispatch_update<__bf16>(p, stream) : dispatch_update<float>(p, stream);
}

}  // namespace ssm
