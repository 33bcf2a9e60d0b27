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
// against a few bytes of inputs.  Layout: each lane owns 8 consecutive states
// of one (b, d) row (two 16-byte loads and stores), so a wave reads contiguous
// state with every instruction; the dstate/8 lanes of a row combine their
// partial readouts with cross-lane adds.
#include <hip/hip_runtime.h>

#include <algorithm>

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
  int64_t batch, dim;
};

// A block covers 256 / LPR consecutive channels d (LPR lanes per (b, d) row) of kRPT consecutive
// batch rows: the channel's parameters (its row of A, dt_bias, D) are loaded once for the kRPT
// rows, every state load or store instruction of a wave moves one contiguous kilobyte, and each
// lane keeps all its rows' state loads in flight.  (b, d) come from the block's coordinates, with
// no division.  Grids taller than the launch limit walk the batch groups with a stride.  Two rows
// per thread measured best on the 2.8B-shaped serving batch (256 x 5120, dstate 16): 29.7 / 38.0 us
// back to back / cache flushed, against 30.2 / 39.8 for one row and 29.3 / 39.6 for four.
constexpr int kRPT = 2;
// States per lane (all of them when dstate is smaller): a lane moves two 16-byte pieces of its row.
// On the same batch, 8 states per lane with 2 rows measured 28.0 / 37.2 us, 4 per lane 29.6 / 37.6,
// 16 per lane 35.9 / 47.1.
constexpr int kSPL = 8;

template <int N, typename T>
__global__ __launch_bounds__(256) void state_update_kernel(StepArgs a) {
  constexpr int SPL = N >= kSPL ? kSPL : N;  // states per lane
  constexpr int LPR = N / SPL;               // lanes per (b, d) row
  constexpr bool kVec = SPL % 4 == 0;        // states, A, B and C moved 4 at a time
  constexpr int kCh = 256 / LPR;           // channels per block
  const int q = (int)(threadIdx.x % LPR);
  const int64_t dr = (int64_t)blockIdx.x * kCh + threadIdx.x / LPR;
  const bool dok = dr < a.dim;
  const int64_t d = dok ? dr : a.dim - 1;

  // this lane's SPL consecutive entries of A[d], premultiplied by log2(e); dt_bias and D of d
  float a2[SPL];
  if constexpr (kVec) {
#pragma unroll
    for (int k = 0; k < SPL; k += 4) {
      const float4 a4 = *reinterpret_cast<const float4*>(a.A + d * N + q * SPL + k);
      a2[k] = a4.x * kLog2e; a2[k + 1] = a4.y * kLog2e; a2[k + 2] = a4.z * kLog2e; a2[k + 3] = a4.w * kLog2e;
    }
  } else {
#pragma unroll
    for (int j = 0; j < SPL; ++j) a2[j] = a.A[d * N + q * SPL + j] * kLog2e;
  }
  const float bias = a.dt_bias ? a.dt_bias[d] : 0.0f;
  const float Dd = a.D ? a.D[d] : 0.0f;

  const int64_t groups = (a.batch + kRPT - 1) / kRPT;
  for (int64_t g = blockIdx.y; g < groups; g += gridDim.y) {
    const int64_t b0 = g * kRPT;
    float h[kRPT][SPL];
    int64_t rr[kRPT], bb[kRPT];
#pragma unroll
    for (int i = 0; i < kRPT; ++i) {
      bb[i] = b0 + i < a.batch ? b0 + i : a.batch - 1;
      rr[i] = bb[i] * a.dim + d;
      const float* sp = a.state + rr[i] * N + q * SPL;
      if constexpr (kVec) {
#pragma unroll
        for (int k = 0; k < SPL; k += 4) {
          const float4 v = *reinterpret_cast<const float4*>(sp + k);
          h[i][k] = v.x; h[i][k + 1] = v.y; h[i][k + 2] = v.z; h[i][k + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < SPL; ++j) h[i][j] = sp[j];
      }
    }
#pragma unroll
    for (int i = 0; i < kRPT; ++i) {
      const int64_t r = rr[i], b = bb[i];
      const bool active = dok && b0 + i < a.batch;
      const float dt = softplus(ld((const T*)a.delta, r) + bias);
      const float ut = ld((const T*)a.u, r);
      const float du = dt * ut;
      // this lane's SPL consecutive entries of B[b] and C[b], 4 per vector load
      float bv[SPL], cv[SPL];
      if constexpr (kVec && sizeof(T) == 2) {
#pragma unroll
        for (int k = 0; k < SPL; k += 4) {
          const uint2 b2 = *reinterpret_cast<const uint2*>((const T*)a.B + b * N + q * SPL + k);
          const uint2 c2 = *reinterpret_cast<const uint2*>((const T*)a.C + b * N + q * SPL + k);
          bv[k] = __builtin_bit_cast(float, b2.x << 16); bv[k + 1] = __builtin_bit_cast(float, b2.x & 0xffff0000u);
          bv[k + 2] = __builtin_bit_cast(float, b2.y << 16); bv[k + 3] = __builtin_bit_cast(float, b2.y & 0xffff0000u);
          cv[k] = __builtin_bit_cast(float, c2.x << 16); cv[k + 1] = __builtin_bit_cast(float, c2.x & 0xffff0000u);
          cv[k + 2] = __builtin_bit_cast(float, c2.y << 16); cv[k + 3] = __builtin_bit_cast(float, c2.y & 0xffff0000u);
        }
      } else if constexpr (kVec) {
#pragma unroll
        for (int k = 0; k < SPL; k += 4) {
          const float4 b4 = *reinterpret_cast<const float4*>((const T*)a.B + b * N + q * SPL + k);
          const float4 c4 = *reinterpret_cast<const float4*>((const T*)a.C + b * N + q * SPL + k);
          bv[k] = b4.x; bv[k + 1] = b4.y; bv[k + 2] = b4.z; bv[k + 3] = b4.w;
          cv[k] = c4.x; cv[k + 1] = c4.y; cv[k + 2] = c4.z; cv[k + 3] = c4.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
          bv[j] = ld((const T*)a.B, b * N + q * SPL + j);
          cv[j] = ld((const T*)a.C, b * N + q * SPL + j);
        }
      }
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const float abar = ex2(dt * a2[j]);
        h[i][j] = __builtin_fmaf(abar, h[i][j], du * bv[j]);
        acc = __builtin_fmaf(cv[j], h[i][j], acc);
      }
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
      if (active) {
        float* sp = a.state + r * N + q * SPL;
        if constexpr (kVec) {
#pragma unroll
          for (int k = 0; k < SPL; k += 4)
            *reinterpret_cast<float4*>(sp + k) = make_float4(h[i][k], h[i][k + 1], h[i][k + 2], h[i][k + 3]);
        } else {
#pragma unroll
          for (int j = 0; j < SPL; ++j) sp[j] = h[i][j];
        }
        if (q == 0) {
          float yt = __builtin_fmaf(Dd, ut, acc);
          if (a.z) yt *= silu(ld((const T*)a.z, r));
          st((T*)a.y, r, yt);
        }
      }
    }
  }
}

template <int N, typename T>
hipError_t run(const StepParams& p, hipStream_t stream) {
  StepArgs a{p.state, p.u, p.delta, p.A, p.B, p.C, p.D, p.z, p.dt_bias, p.y, p.batch, p.dim};
  constexpr int LPR = N / (N >= kSPL ? kSPL : N);
  constexpr int64_t kCh = 256 / LPR;
  const int64_t gx = (p.dim + kCh - 1) / kCh;
  const int64_t gy = std::min<int64_t>((p.batch + kRPT - 1) / kRPT, 65535);
  hipLaunchKernelGGL((state_update_kernel<N, T>), dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream, a);
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
