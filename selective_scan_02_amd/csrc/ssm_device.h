// ssm_device.h -- device-side helpers of the gfx950 selective-scan kernels.
//
// Transcendentals use the hardware instructions directly: v_exp_f32 (2^x),
// v_log_f32 (log2 x) and v_rcp_f32 (1/x), each about 1 ulp.  On gfx950 they
// issue at half the fp32 FMA rate and do not overlap with FMAs, so the kernels
// count them as two VALU slots each.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;  // 1 / ln 2
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^-|x|), in fp32 to ~1e-7 relative.
// The step sizes of interest are small (Delta ~ 1e-3), where log(fl(1 + e)) alone
// loses ~2^-24/e in relative terms.  Instead: s = fl(1 + e) and its rounding error
// c = e - (s - 1) are computed exactly (Fast2Sum; 1 >= e), and
// log1p(e) = log(s) + log1p(c/s) ~= log(s) + c.  The dropped part, c(1 - 1/s), is
// below |c| (s-1)/s <= 2^-24 * log(s), i.e. under one ulp of the result.
__device__ __forceinline__ float softplus(float x) {
  const float e = ex2(-__builtin_fabsf(x) * kLog2e);  // e^-|x| in (0, 1]
  const float s = 1.0f + e;
  const float c = e - (s - 1.0f);
  return __builtin_fmaxf(x, 0.0f) + __builtin_fmaf(lg2(s), kLn2, c);
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z).  e^-z overflows to +inf for z << 0,
// and rcp(inf) = 0 gives the correct limit (-0).
__device__ __forceinline__ float silu(float z) { return z * rcp(1.0f + ex2(-z * kLog2e)); }

// Element load / store for the two I/O types.  bf16 -> fp32 is exact (a shift);
// fp32 -> bf16 rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <typename T> __device__ __forceinline__ float ld(const T* p, int64_t i);
template <> __device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<__bf16>(const __bf16* p, int64_t i) { return (float)p[i]; }

template <typename T> __device__ __forceinline__ void st(T* p, int64_t i, float v);
template <> __device__ __forceinline__ void st<float>(float* p, int64_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st<__bf16>(__bf16* p, int64_t i, float v) { p[i] = (__bf16)v; }

}  // namespace ssm
