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
// of one (b, d) row (one 16-byte load and store), so a wave reads contiguous
// state with every instruction; the dstate/4 lanes of a row combine their
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
// batch rows, and every lane moves SPL = 4 consecutive states of a row with one 16-byte load and
// store, so each state load or store instruction of a wave moves one contiguous kilobyte.  All of a
// lane's loads -- its rows' states first, then their inputs, then the channel's parameters -- are
// issued before any arithmetic, so a wave waits for memory once.  (b, d) come from the block's
// coordinates, with no division.  Grids taller than the launch limit walk the batch groups with a
// stride.  On the 2.8B-shaped serving batch (256 x 5120, dstate 16; HIP events around each step,
// cache flushed before it / back to back): 4 states per lane with 2 rows per thread measured
// 32.4 / 27.3 us, against 36.2 / 28.5 with 8 states per lane and 37.3 / 27.6 for the layout before
// it (8 states per lane, the channel's parameters waited for before the state loads were issued);
// persistent blocks walking several units, with or without the next unit's loads issued ahead,
// measured 36.6-50 us.
#ifndef SSM_DECODE_RPT
#define SSM_DECODE_RPT 2
#endif
constexpr int kRPT = SSM_DECODE_RPT;
constexpr int kSPL = 4;

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

  // optional inputs are loaded from a valid stand-in address and selected away afterwards: a load
  // issued on only some paths makes the compiler wait for every load in flight before going on
  const bool gated = a.z != nullptr, biased = a.dt_bias != nullptr, skip = a.D != nullptr;
  const T* zp = gated ? (const T*)a.z : (const T*)a.u;
  const float* biasp = biased ? a.dt_bias : a.A;
  const float* Dp = skip ? a.D : a.A;
  const int64_t groups = (a.batch + kRPT - 1) / kRPT;
  for (int64_t g = blockIdx.y; g < groups; g += gridDim.y) {
    const int64_t b0 = g * kRPT;
    float h[kRPT][SPL], bv[kRPT][SPL], cv[kRPT][SPL], dl[kRPT], ut[kRPT], zt[kRPT];
    int64_t rr[kRPT], bb[kRPT];
    // loads: the rows' states, then their inputs, then the channel's parameters
#pragma unroll
    for (int i = 0; i < kRPT; ++i) {
      bb[i] = b0 + i < a.batch ? b0 + i : a.batch - 1;
      rr[i] = bb[i] * a.dim + d;
      const float* sp = a.state + rr[i] * N + q * SPL;
      if constexpr (kVec) {
        const float4 v = *reinterpret_cast<const float4*>(sp);
        h[i][0] = v.x; h[i][1] = v.y; h[i][2] = v.z; h[i][3] = v.w;
      } else {
#pragma unroll
        for (int j = 0; j < SPL; ++j) h[i][j] = sp[j];
      }
    }
#pragma unroll
    for (int i = 0; i < kRPT; ++i) {
      const int64_t r = rr[i], b = bb[i];
      dl[i] = ld((const T*)a.delta, r);
      ut[i] = ld((const T*)a.u, r);
      zt[i] = ld(zp, r);
      // this lane's SPL consecutive entries of B[b] and C[b]
      if constexpr (kVec && sizeof(T) == 2) {
        const uint2 b2 = *reinterpret_cast<const uint2*>((const T*)a.B + b * N + q * SPL);
        const uint2 c2 = *reinterpret_cast<const uint2*>((const T*)a.C + b * N + q * SPL);
        bv[i][0] = __builtin_bit_cast(float, b2.x << 16); bv[i][1] = __builtin_bit_cast(float, b2.x & 0xffff0000u);
        bv[i][2] = __builtin_bit_cast(float, b2.y << 16); bv[i][3] = __builtin_bit_cast(float, b2.y & 0xffff0000u);
        cv[i][0] = __builtin_bit_cast(float, c2.x << 16); cv[i][1] = __builtin_bit_cast(float, c2.x & 0xffff0000u);
        cv[i][2] = __builtin_bit_cast(float, c2.y << 16); cv[i][3] = __builtin_bit_cast(float, c2.y & 0xffff0000u);
      } else if constexpr (kVec) {
        const float4 b4 = *reinterpret_cast<const float4*>((const T*)a.B + b * N + q * SPL);
        const float4 c4 = *reinterpret_cast<const float4*>((const T*)a.C + b * N + q * SPL);
        bv[i][0] = b4.x; bv[i][1] = b4.y; bv[i][2] = b4.z; bv[i][3] = b4.w;
        cv[i][0] = c4.x; cv[i][1] = c4.y; cv[i][2] = c4.z; cv[i][3] = c4.w;
      } else {
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
          bv[i][j] = ld((const T*)a.B, b * N + q * SPL + j);
          cv[i][j] = ld((const T*)a.C, b * N + q * SPL + j);
        }
      }
    }
    // this lane's SPL consecutive entries of A[d], premultiplied by log2(e); dt_bias and D of d
    float a2[SPL];
    if constexpr (kVec) {
      const float4 a4 = *reinterpret_cast<const float4*>(a.A + d * N + q * SPL);
      a2[0] = a4.x * kLog2e; a2[1] = a4.y * kLog2e; a2[2] = a4.z * kLog2e; a2[3] = a4.w * kLog2e;
    } else {
#pragma unroll
      for (int j = 0; j < SPL; ++j) a2[j] = a.A[d * N + q * SPL + j] * kLog2e;
    }
    float bias = biasp[d], Dd = Dp[d];
    asm volatile("" : "+v"(bias), "+v"(Dd));  // keeps both loads unconditional
    bias = biased ? bias : 0.0f;
    Dd = skip ? Dd : 0.0f;
#pragma unroll
    for (int i = 0; i < kRPT; ++i) {
      const int64_t r = rr[i];
      const bool active = dok && b0 + i < a.batch;
      const float dt = softplus(dl[i] + bias);
      const float du = dt * ut[i];
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const float abar = ex2(dt * a2[j]);
        h[i][j] = __builtin_fmaf(abar, h[i][j], du * bv[i][j]);
        acc = __builtin_fmaf(cv[i][j], h[i][j], acc);
      }
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
      if (active) {
        float* sp = a.state + r * N + q * SPL;
        if constexpr (kVec) {
          *reinterpret_cast<float4*>(sp) = make_float4(h[i][0], h[i][1], h[i][2], h[i][3]);
        } else {
#pragma unroll
          for (int j = 0; j < SPL; ++j) sp[j] = h[i][j];
        }
        if (q == 0) {
          float yt = __builtin_fmaf(Dd, ut[i], acc);
          if (gated) yt *= silu(zt[i]);
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
