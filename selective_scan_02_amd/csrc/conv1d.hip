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
// 2 x (element size) bytes.  conv1d_fwd_kernel: a wave covers 4 runs of 64
// lanes x 16 bytes of consecutive steps of one row (each load or store
// instruction moves one contiguous kilobyte); the K-1 inputs before a lane's
// piece come from the previous lane by a cross-lane shift, lane 0 taking them
// from lane 63 of the previous run, or from memory (or the state before step 0)
// at the wave's start.
// conv1d_update_kernel: one thread per row shifts the window in place.
#include <hip/hip_runtime.h>

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {
namespace {

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

// A wave covers kRuns consecutive runs of 64 lanes x 16 bytes of one row: every load and
// store instruction moves one contiguous kilobyte, and each lane keeps kRuns pieces in flight.
constexpr int kRuns = 4;
template <typename T> constexpr int kPS = 16 / sizeof(T);  // steps per 16-byte piece

// One wave's runs.  FULL (uniform per wave): every piece lies inside the row and rows are
// 16-byte aligned, so the pieces move as 16-byte vectors; otherwise element by element with
// bounds checks.  The two cases are separate code, so the values stay in registers.
template <int K, typename T, bool FULL>
__device__ __forceinline__ void conv_wave(const ConvArgs& a, int64_t row, int64_t w0, int lane) {
  constexpr int H = K > 1 ? K - 1 : 1;
  constexpr int PS = kPS<T>;
  constexpr int kRunSteps = 64 * PS;
  const int64_t L = a.L;
  const int64_t d = row % a.dim;
  const T* xr = (const T*)a.x + row * L;
  T* orow = (T*)a.out + row * L;

  float v[kRuns][PS];
  if constexpr (FULL) {
    uint4 q[kRuns];
#pragma unroll
    for (int r = 0; r < kRuns; ++r) q[r] = *reinterpret_cast<const uint4*>(xr + w0 + r * kRunSteps + lane * PS);
#pragma unroll
    for (int r = 0; r < kRuns; ++r) {
      const uint32_t w4[4] = {q[r].x, q[r].y, q[r].z, q[r].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (sizeof(T) == 2) {
          v[r][2 * j] = __builtin_bit_cast(float, w4[j] << 16);
          v[r][2 * j + 1] = __builtin_bit_cast(float, w4[j] & 0xffff0000u);
        } else {
          v[r][j] = __builtin_bit_cast(float, w4[j]);
        }
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < kRuns; ++r) {
      const int64_t t0 = w0 + r * kRunSteps + lane * PS;
#pragma unroll
      for (int e = 0; e < PS; ++e) v[r][e] = t0 + e < L ? ld(xr, t0 + e) : 0.0f;
    }
  }
  float w[K];
#pragma unroll
  for (int k = 0; k < K; ++k) w[k] = a.w[d * K + k];
  const float bias = a.bias ? a.bias[d] : 0.0f;
  // inputs at the K-1 steps before the wave: from memory, or the state before step 0
  float h0[H];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int64_t s = w0 - (K - 1) + j;
    h0[j] = s >= 0 ? ld(xr, s) : (a.st_in ? a.st_in[row * (K - 1) + (K - 1) + s] : 0.0f);
  }

#pragma unroll
  for (int r = 0; r < kRuns; ++r) {
    const int64_t t0 = w0 + r * kRunSteps + lane * PS;
    // inputs at steps t0-(K-1) .. t0-1: the previous lane's last K-1 values; lane 0 takes
    // them from lane 63 of the previous run (or from before the wave)
    float hst[H];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      const float up = __shfl_up(v[r][PS - (K - 1) + j], 1, 64);
      const float wrap = r > 0 ? __shfl(v[r > 0 ? r - 1 : 0][PS - (K - 1) + j], 63, 64) : h0[j];
      hst[j] = lane == 0 ? wrap : up;
    }
    float o[PS];
#pragma unroll
    for (int e = 0; e < PS; ++e) {
      float acc = bias;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int s = e - (K - 1) + k;  // step relative to t0
        acc = __builtin_fmaf(w[k], s >= 0 ? v[r][s >= 0 ? s : 0] : hst[s >= 0 ? 0 : K - 1 + s], acc);
      }
      o[e] = a.silu ? silu(acc) : acc;
    }
    if constexpr (FULL) {
      uint32_t w4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (sizeof(T) == 2) {
          const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)o[2 * j]);
          const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)o[2 * j + 1]);
          w4[j] = lo | (hi << 16);
        } else {
          w4[j] = __builtin_bit_cast(uint32_t, o[j]);
        }
      }
      *reinterpret_cast<uint4*>(orow + t0) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    } else {
#pragma unroll
      for (int e = 0; e < PS; ++e)
        if (t0 + e < L) st(orow, t0 + e, o[e]);
    }
    // the lane holding step L-1 writes the state a following call continues from
    if (a.st_out && K > 1 && t0 <= L - 1 && L - 1 < t0 + PS) {
#pragma unroll
      for (int j = 0; j < K - 1; ++j) {
        const int64_t s = L - (K - 1) + j;  // input step; >= t0 - (K-1)
        const int qq = (int)(s - t0);  // in -(K-1) .. PS-1; selected with constant indices only
        float val = 0.0f;
#pragma unroll
        for (int e = 0; e < PS; ++e) val = qq == e ? v[r][e] : val;
#pragma unroll
        for (int m = 0; m < K - 1; ++m) val = qq == m - (K - 1) ? hst[m] : val;
        a.st_out[row * (K - 1) + j] = val;
      }
    }
  }
}

template <int K, typename T>
__global__ __launch_bounds__(256) void conv1d_fwd_kernel(const ConvArgs a) {
  constexpr int64_t kWaveSteps = kRuns * 64 * kPS<T>;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= a.rows * a.nseg) return;  // uniform per wave
  const int64_t row = wave / a.nseg;
  const int64_t w0 = (wave - row * a.nseg) * kWaveSteps;  // first step of the wave
  if (a.vec && w0 + kWaveSteps <= a.L) conv_wave<K, T, true>(a, row, w0, lane);
  else conv_wave<K, T, false>(a, row, w0, lane);
}

// seqlen == 0: the state out is the state in (or zeros)
__global__ __launch_bounds__(256) void conv1d_copy_state(float* dst, const float* src, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}

// The last K-1 inputs of every row (oldest first), reaching into the state before step 0 when
// the row is shorter: the state causal_conv1d_fwd leaves, for callers that fuse the convolution.
template <typename T>
__global__ __launch_bounds__(256) void conv1d_state_tail(const T* x, const float* st_in, float* st_out, int64_t rows,
                                                         int64_t L, int K) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= rows * (K - 1)) return;
  const int64_t row = i / (K - 1);
  const int j = (int)(i - row * (K - 1));
  const int64_t s = L - (K - 1) + j;
  st_out[i] = s >= 0 ? ld(x, row * L + s) : (st_in ? st_in[row * (K - 1) + (K - 1) + s] : 0.0f);
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
  constexpr int64_t kWaveSteps = kRuns * 64 * kPS<T>;
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

hipError_t launch_conv1d_state_out(const ConvParams& p, hipStream_t stream) {
  if (!p.state_out || p.width <= 1) return hipSuccess;
  const int64_t n = p.batch * p.dim * (p.width - 1);
  const dim3 g((unsigned)((n + 255) / 256));
  if (p.dtype == kBF16)
    hipLaunchKernelGGL(conv1d_state_tail<__bf16>, g, dim3(256), 0, stream, (const __bf16*)p.x, p.state_in, p.state_out,
                       p.batch * p.dim, p.seqlen, (int)p.width);
  else
    hipLaunchKernelGGL(conv1d_state_tail<float>, g, dim3(256), 0, stream, (const float*)p.x, p.state_in, p.state_out,
                       p.batch * p.dim, p.seqlen, (int)p.width);
  return hipGetLastError();
}

hipError_t launch_conv1d_update(const ConvStepParams& p, hipStream_t stream) {
  return p.dtype == kBF16 ? dispatch_update<__bf16>(p, stream) : dispatch_update<float>(p, stream);
}

}  // namespace ssm
