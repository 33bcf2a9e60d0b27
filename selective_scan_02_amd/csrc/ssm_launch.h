// ssm_launch.h -- internal interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

enum IoType { kF32 = 0, kBF16 = 1 };

struct ScanParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;        // nullable
  const void* z;         // nullable
  const float* dt_bias;  // nullable
  int softplus;
  void* y;
  float* last_state;  // nullable
  const float* h0;    // nullable initial state [batch, dim, dstate]
  int64_t batch, dim, dstate, seqlen;
  int dtype;
};

struct StepParams {
  float* state;
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;        // nullable
  const void* z;         // nullable
  const float* dt_bias;  // nullable
  void* y;
  int64_t batch, dim, dstate;
  int dtype;
};

struct ConvParams {
  const void* x;
  const float* weight;     // [dim, width]
  const float* bias;       // nullable [dim]
  const float* state_in;   // nullable [batch, dim, width-1]
  int silu;
  void* out;
  float* state_out;        // nullable [batch, dim, width-1]
  int64_t batch, dim, seqlen, width;
  int dtype;
};

struct ConvStepParams {
  float* state;            // [batch, dim, width-1], updated in place
  const void* x;           // [batch, dim]
  const float* weight;
  const float* bias;
  int silu;
  void* out;               // [batch, dim]
  int64_t batch, dim, width;
  int dtype;
};

struct BwdParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;        // nullable
  const void* z;         // nullable
  const float* dt_bias;  // nullable
  int softplus;
  const float* h0;       // nullable initial state [batch, dim, dstate]
  const void* dy;
  void* du;
  void* ddelta;
  float* dA;
  void* dB;
  void* dC;
  float* dD;             // nullable
  void* dz;              // written when z is given
  float* ddt_bias;       // nullable
  float* dh0;            // nullable
  int64_t batch, dim, dstate, seqlen;
  int dtype;
};

struct SsdParams {
  const void* x;         // [batch, heads*headdim, L] bf16
  const void* dt;        // [batch, heads, L] bf16
  const float* A;        // [heads]
  const void* B;         // [batch, dstate, L] bf16
  const void* C;
  const float* D;        // [heads*headdim] or null
  const void* z;         // or null
  const float* dt_bias;  // [heads] or null
  int softplus;
  const float* h0;       // [batch, heads*headdim, dstate] or null
  void* y;
  float* last_state;     // or null
  int64_t batch, heads, headdim, dstate, seqlen;
};

struct ScanPlan {
  int mode;          // 0 intervals, 1 one pass, 2 aggregate/carry/output
  int64_t groups;    // channel groups of 64
  int64_t nseg;      // segments per group (modes 1, 2); intervals (mode 0)
  int64_t seg_len;   // steps per segment or per interval
  int64_t units;     // workgroups of the output pass
};
ScanPlan plan_scan(int64_t batch, int64_t dim, int64_t seqlen, int cus);

// Stream-ordered scratch memory from a pool the library owns, one per device.  The pool keeps
// what it has reserved between calls (no return to the system at synchronisation points), so
// the carries and flags of one call reuse the memory of the previous one.
hipError_t scratch_alloc(void** p, size_t bytes, hipStream_t stream);

bool dstate_supported(int64_t n);
hipError_t launch_scan_fwd(const ScanParams& p, hipStream_t stream);      // dispatcher
hipError_t launch_scan_generic(const ScanParams& p, hipStream_t stream);  // any shape / alignment
bool chunked_supported(const ScanParams& p);
hipError_t launch_scan_chunked(const ScanParams& p, hipStream_t stream);  // fast path
hipError_t launch_scan_bwd(const BwdParams& p, hipStream_t stream);
bool ssd_supported(int64_t headdim, int64_t dstate);
hipError_t launch_ssd_fwd(const SsdParams& p, hipStream_t stream);
hipError_t launch_state_update(const StepParams& p, hipStream_t stream);
hipError_t launch_conv1d_fwd(const ConvParams& p, hipStream_t stream);
hipError_t launch_conv1d_update(const ConvStepParams& p, hipStream_t stream);

}  // namespace ssm
