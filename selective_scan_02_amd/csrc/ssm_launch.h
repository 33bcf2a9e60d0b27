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
  // Scratch supplied by the caller (device memory of ws_bytes bytes); NULL = taken from the
  // library's stream-ordered pool and returned to it.  With a workspace nothing is allocated.
  void* ws = nullptr;
  size_t ws_bytes = 0;
  // Causal conv1d + SiLU ahead of the scan (cw non-NULL): u = silu(conv(x)) is computed from
  // x, which `u` then points to; cst = the inputs before step 0, cst_out receives the last ck-1.
  const float* cw = nullptr;   // [dim, ck]
  const float* cb = nullptr;   // [dim] or NULL
  const float* cst = nullptr;  // [batch, dim, ck-1] or NULL
  float* cst_out = nullptr;    // [batch, dim, ck-1] or NULL
  int64_t ck = 0;
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
  bool ddelta_f32 = false;  // ddelta in fp32 whatever dtype is (its row stride is still seqlen)
  bool a_uniform = false;   // A[d, n] is the same for every n of each channel d (the SSD form)
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
  int64_t out_stride;  // mode 2: aggregate segments per output-pass workgroup
};
ScanPlan plan_scan(int64_t batch, int64_t dim, int64_t seqlen, int cus);

// Stream-ordered scratch memory from a pool the library owns, one per device.  The pool keeps
// what it has reserved between calls (no return to the system at synchronisation points), so
// the carries and flags of one call reuse the memory of the previous one.
hipError_t scratch_alloc(void** p, size_t bytes, hipStream_t stream);

// Scratch kept per (device, stream, slot) between calls, grow-only: the calls on one stream run in
// order, so each reuses the buffer without allocating (a stream-ordered pool allocation and free
// per call put a few microseconds between consecutive kernels).  False under graph capture, where
// a pool allocation becomes part of the graph, or when the buffer cannot be made.  Slot 0 is the
// forward scan's scratch, slot 1 the convolution output of the two-kernel convolution + scan, slot 2 the
// SSD forward's chunk states, slot 3 the SSD backward's broadcast parameters and gradients, slot 4 the
// backward scan's checkpoints, carries and partial sums.
bool stream_scratch(hipStream_t stream, int slot, size_t bytes, void** out);
bool is_stream_scratch(const void* ptr);
// Frees every slot kept for the stream on the current device (the stream must have drained).
void stream_scratch_release(hipStream_t stream);
// The stream's slot when it can be kept, else pool memory; call_scratch_release frees only the latter.
hipError_t call_scratch(hipStream_t stream, int slot, size_t bytes, void** ptr, bool* kept);
hipError_t call_scratch_release(void* ptr, bool kept, hipStream_t stream);

// Scratch of one scan call: from the caller's workspace when the parameters carry one (which
// must hold `bytes`, else hipErrorInvalidValue), otherwise the stream's slot-0 scratch, else the
// pool.  scratch_release returns pool memory on the stream and does nothing for the others.
hipError_t scratch_acquire(const ScanParams& p, void** ptr, size_t bytes, hipStream_t stream);
hipError_t scratch_release(const ScanParams& p, void* ptr, hipStream_t stream);

// Scratch bytes selective_scan_fwd needs for these parameters on a GPU with `cus` compute
// units (host-only, mirrors the launch plan: carries and flags of the interval schedule,
// segment aggregates of the two-pass plans; 0 for one pass).
size_t scan_scratch_bytes(const ScanParams& p, int cus);

// The allocation-free scan: a fixed device array per GPU (noalloc.hip), 16 MiB.
constexpr int kMaxDevices = 256;
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
// Address and size of this GPU's copy of that array (the current device's); the address is
// looked up on the first call per device and kept.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);
size_t chunked_scratch_bytes(const ScanParams& p, int cus);
size_t generic_scratch_bytes(const ScanParams& p);
int device_cu_count();

// Interval-schedule hand-over diagnostics: waits that gave up (their pieces poisoned with NaN)
// on the current device since the last reset; and the test hook that bounds the wait and can
// suppress the head pieces' flags.
hipError_t handover_failures(uint64_t* count, bool reset);
// The stream's persistent interval control block (ticket and hand-over flags that need no clearing
// per call): this call's ticket base and flag generation.  False under graph capture or when the
// block cannot be made; the caller then clears a ticket and flags of its own.
bool interval_ctl(hipStream_t s, int64_t nflags, int64_t units, unsigned long long** ticket,
                  unsigned long long** flags, unsigned long long* base, unsigned long long* gen);
void interval_ctl_invalidate(hipStream_t s);  // after a failed launch: the next call makes a new block
// Frees the stream's control block (the stream must have drained); the next call makes a new one.
void interval_ctl_release(hipStream_t s);
hipError_t bwd_handover_failures(uint64_t* count, bool reset);  // the backward main pass's
void set_handover_wait(int max_polls, int publish);
void handover_wait(int* max_polls, int* publish);  // the current settings

bool dstate_supported(int64_t n);
hipError_t launch_scan_fwd(const ScanParams& p, hipStream_t stream);      // dispatcher
hipError_t launch_scan_generic(const ScanParams& p, hipStream_t stream);  // any shape / alignment
bool chunked_supported(const ScanParams& p);
bool chunked_conv_supported(const ScanParams& p);  // the fused convolution path (dstate 16, fp32 rows)
hipError_t launch_scan_chunked(const ScanParams& p, hipStream_t stream);  // fast path
hipError_t launch_scan_bwd(const BwdParams& p, hipStream_t stream);
bool ssd_supported(int64_t headdim, int64_t dstate);
hipError_t launch_ssd_fwd(const SsdParams& p, hipStream_t stream);

// Backward of the SSD form: gradients of sum(dy * y).  Shapes as SsdParams; outputs dx, dz like
// x, ddt like dt (dtype of x), dA [heads], ddt_bias [heads], dD [heads*headdim], dB, dC like B,
// dh0 like h0.  bf16 or fp32 (dtype), any headdim >= 1 and the backward scan's dstates.
struct SsdBwdParams {
  SsdParams f;  // forward inputs (f.y, f.last_state unused)
  int dtype;    // kF32 or kBF16
  const void* dy;
  void* dx;
  void* ddt;
  float* dA;
  void* dB;
  void* dC;
  float* dD;        // nullable
  void* dz;         // written when z is given
  float* ddt_bias;  // nullable
  float* dh0;       // nullable
};
hipError_t launch_ssd_bwd(const SsdBwdParams& p, hipStream_t stream);
hipError_t launch_state_update(const StepParams& p, hipStream_t stream);
hipError_t launch_conv1d_fwd(const ConvParams& p, hipStream_t stream);
hipError_t launch_conv1d_update(const ConvStepParams& p, hipStream_t stream);
// The convolution state a sequence leaves (its last width-1 inputs, from the state before it
// where the sequence is shorter), as causal_conv1d_fwd writes it.
hipError_t launch_conv1d_state_out(const ConvParams& p, hipStream_t stream);

}  // namespace ssm
