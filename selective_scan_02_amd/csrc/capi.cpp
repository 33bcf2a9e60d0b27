// capi.cpp -- the extern "C" boundary: argument validation, error reporting and
// dispatch to the gfx950 kernels.  Validation happens entirely on the host and
// before any HIP call, so a rejected call touches no output.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "../../include/ssm_scan.h"
#include "ssm_launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

struct Range {
  const char* name;
  const void* p;
  uint64_t bytes;
  uint64_t align;
};

bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

int check_aligned(const Range& r) {
  if (r.p && ((uintptr_t)r.p % r.align) != 0)
    return fail(SSM_ERR_MISALIGNED, "%s is not %llu-byte aligned", r.name, (unsigned long long)r.align);
  return SSM_OK;
}

// Product of sizes with an overflow guard: every tensor must stay below 2^40 elements.
bool too_big(int64_t a, int64_t b, int64_t c) {
  const double e = (double)a * (double)b * (double)c;
  return e >= 1099511627776.0;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SSM_OK;
  return fail(SSM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace ssm {

hipError_t scratch_alloc(void** p, size_t bytes, hipStream_t stream) {
  static std::mutex mu;
  static hipMemPool_t pools[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  hipMemPool_t pool;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!pools[dev]) {
      hipMemPoolProps props{};
      props.allocType = hipMemAllocationTypePinned;  // device memory, not migratable
      props.handleTypes = hipMemHandleTypeNone;
      props.location.type = hipMemLocationTypeDevice;
      props.location.id = dev;
      hipMemPool_t np = nullptr;
      if ((e = hipMemPoolCreate(&np, &props)) != hipSuccess) return e;
      uint64_t keep = UINT64_MAX;  // never hand reserved memory back between calls
      if ((e = hipMemPoolSetAttribute(np, hipMemPoolAttrReleaseThreshold, &keep)) != hipSuccess) return e;
      pools[dev] = np;
    }
    pool = pools[dev];
  }
  return hipMallocFromPoolAsync(p, bytes, pool, stream);
}

namespace {
struct StreamWs {
  void* p = nullptr;
  size_t cap = 0;
};
std::mutex g_ws_mu;
std::map<std::tuple<int, hipStream_t, int>, StreamWs> g_ws;
}  // namespace

bool stream_scratch(hipStream_t stream, int slot, size_t bytes, void** out) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) != hipSuccess || st != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();
    return false;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  StreamWs& w = g_ws[{dev, stream, slot}];
  if (w.cap < bytes) {
    constexpr size_t kGrain = (size_t)2 << 20;
    const size_t cap = (std::max(bytes, 2 * w.cap) + kGrain - 1) / kGrain * kGrain;
    void* m = nullptr;
    if (hipMalloc(&m, cap) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    w.p = m;  // the outgrown buffer is dropped, not freed: work queued before may still use it
    w.cap = cap;
    // Keep as much reserved in the pool: a call under stream capture takes its scratch from the
    // pool (a graph cannot share this buffer with the stream's later calls), and capture does not
    // allow the pool to make new memory.
    void* t = nullptr;
    if (scratch_alloc(&t, cap + kGrain, stream) == hipSuccess) (void)hipFreeAsync(t, stream);
    (void)hipGetLastError();
  }
  *out = w.p;
  return true;
}

hipError_t call_scratch(hipStream_t stream, int slot, size_t bytes, void** ptr, bool* kept) {
  *kept = stream_scratch(stream, slot, bytes, ptr);
  return *kept ? hipSuccess : scratch_alloc(ptr, bytes, stream);
}

hipError_t call_scratch_release(void* ptr, bool kept, hipStream_t stream) {
  return kept ? hipSuccess : hipFreeAsync(ptr, stream);
}

void stream_scratch_release(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  for (auto it = g_ws.begin(); it != g_ws.end();) {
    if (std::get<0>(it->first) == dev && std::get<1>(it->first) == stream) {
      if (it->second.p) (void)hipFree(it->second.p);
      it = g_ws.erase(it);
    } else {
      ++it;
    }
  }
}

bool is_stream_scratch(const void* ptr) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  for (const auto& kv : g_ws)
    if (kv.second.p == ptr) return true;
  return false;
}

hipError_t scratch_acquire(const ScanParams& p, void** ptr, size_t bytes, hipStream_t stream) {
  if (p.ws) {
    if (bytes > p.ws_bytes) return hipErrorInvalidValue;
    *ptr = p.ws;
    return hipSuccess;
  }
  if (stream_scratch(stream, 0, bytes, ptr)) return hipSuccess;
  return scratch_alloc(ptr, bytes, stream);
}

hipError_t scratch_release(const ScanParams& p, void* ptr, hipStream_t stream) {
  if (p.ws || is_stream_scratch(ptr)) return hipSuccess;
  return hipFreeAsync(ptr, stream);
}

}  // namespace ssm

extern "C" {

const char* ssm_last_error(void) { return g_last_error.c_str(); }

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

int ssm_release_stream(void* stream) {
  const hipStream_t s = (hipStream_t)stream;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (int rc = hip_status(hipStreamIsCapturing(s, &st), "ssm_release_stream")) return rc;
  if (st != hipStreamCaptureStatusNone) return fail(SSM_ERR_UNSUPPORTED, "ssm_release_stream: the stream is capturing");
  if (int rc = hip_status(hipStreamSynchronize(s), "ssm_release_stream")) return rc;
  ssm::stream_scratch_release(s);
  ssm::interval_ctl_release(s);
  return hip_status(hipGetLastError(), "ssm_release_stream");
}

int ssm_handover_failures(int64_t* count, int reset) {
  g_last_error.clear();
  if (!count) return fail(SSM_ERR_NULL_ARG, "count is NULL");
  uint64_t v = 0, w = 0;
  if (int rc = hip_status(ssm::handover_failures(&v, reset != 0), "ssm_handover_failures")) return rc;
  if (int rc = hip_status(ssm::bwd_handover_failures(&w, reset != 0), "ssm_handover_failures")) return rc;
  *count = (int64_t)(v + w);
  return SSM_OK;
}

int ssm_test_handover_wait(int max_polls, int publish) {
  g_last_error.clear();
  ssm::set_handover_wait(max_polls, publish);
  return SSM_OK;
}

int ssm_scan_plan(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype, int num_cus,
                  int64_t* out) {
  g_last_error.clear();
  if (!out) return fail(SSM_ERR_NULL_ARG, "out is NULL");
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d is not SSM_F32/SSM_BF16", dtype);
  if (batch < 1 || dim < 1 || dstate < 1 || seqlen < 0 || num_cus < 1)
    return fail(SSM_ERR_BAD_SHAPE, "bad sizes");
  if (!ssm::dstate_supported(dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate=%lld not in {1,2,4,8,16,32,64}", (long long)dstate);
  const int64_t es = dtype == SSM_BF16 ? 2 : 4;
  // the chunked kernels need dstate >= 4 and rows that are a whole number of 16-byte pieces
  // (pointer alignment is checked per call); everything else takes the generic kernels
  const bool chunked = dstate >= 4 && (seqlen * es) % 16 == 0 && seqlen > 0;
  if (!chunked) {
    out[0] = 3; out[1] = 0; out[2] = 0; out[3] = 0; out[4] = 0;
    return SSM_OK;
  }
  const ssm::ScanPlan pl = ssm::plan_scan(batch, dim, seqlen, num_cus);
  out[0] = pl.mode; out[1] = pl.groups; out[2] = pl.nseg; out[3] = pl.seg_len; out[4] = pl.units;
  return SSM_OK;
}

}  // extern "C"

namespace {

// The causal conv1d + SiLU fused ahead of the scan: u is computed from x.
struct ConvIn {
  const float* weight = nullptr;  // NULL: no convolution, the first tensor is u
  const float* bias = nullptr;
  const float* state_in = nullptr;
  float* state_out = nullptr;
  int64_t width = 0;
};

int scan_impl(const char* who, const void* u, const void* delta, const float* A, const void* B, const void* C,
              const float* D, const void* z, const float* dt_bias, int softplus, const float* h0, void* y,
              float* last_state, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
              void* stream, bool noalloc = false, const ConvIn& cv = ConvIn()) {
  g_last_error.clear();
  const bool conv = cv.weight != nullptr;
  const char* uname = conv ? "x" : "u";
  // With seqlen == 0 the sequence tensors are empty and may be NULL.
  if (seqlen != 0) {
    if (!u) return fail(SSM_ERR_NULL_ARG, "%s is NULL", uname);
    if (!delta) return fail(SSM_ERR_NULL_ARG, "delta is NULL");
    if (!B) return fail(SSM_ERR_NULL_ARG, "B is NULL");
    if (!C) return fail(SSM_ERR_NULL_ARG, "C is NULL");
    if (!y) return fail(SSM_ERR_NULL_ARG, "y is NULL");
  }
  if (!A) return fail(SSM_ERR_NULL_ARG, "A is NULL");
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d is not SSM_F32/SSM_BF16", dtype);
  if (batch < 1 || dim < 1 || dstate < 1 || seqlen < 0)
    return fail(SSM_ERR_BAD_SHAPE, "bad sizes batch=%lld dim=%lld dstate=%lld seqlen=%lld", (long long)batch,
                (long long)dim, (long long)dstate, (long long)seqlen);
  if (too_big(batch, dim, seqlen) || too_big(batch, dstate, seqlen) || too_big(batch, dim, dstate) ||
      batch * ((dim + 63) / 64) > 0x7fffffffLL)
    return fail(SSM_ERR_BAD_SHAPE, "sizes too large");
  if (!ssm::dstate_supported(dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate=%lld not in {1,2,4,8,16,32,64}", (long long)dstate);
  if (softplus != 0 && softplus != 1) return fail(SSM_ERR_BAD_SHAPE, "softplus must be 0 or 1");
  if (conv && (cv.width < 1 || cv.width > 4))
    return fail(SSM_ERR_UNSUPPORTED, "width=%lld not in 1..4", (long long)cv.width);
  const uint64_t es = dtype == SSM_BF16 ? 2 : 4;
  const uint64_t nx = (uint64_t)batch * dim * seqlen, nbc = (uint64_t)batch * dstate * seqlen;
  const uint64_t nst = (uint64_t)batch * dim * dstate * 4;
  const uint64_t ncs = conv ? (uint64_t)batch * dim * (cv.width - 1) * 4 : 0;
  const Range cins[] = {{"conv_weight", cv.weight, conv ? (uint64_t)dim * cv.width * 4 : 0, 4},
                        {"conv_bias", cv.bias, conv ? (uint64_t)dim * 4 : 0, 4},
                        {"conv_state_in", cv.state_in, ncs, 4}};
  const Range rcs{"conv_state_out", cv.state_out, ncs, 4};
  for (const Range& r : cins)
    if (int rc = check_aligned(r)) return rc;
  if (int rc = check_aligned(rcs)) return rc;
  const Range ins[] = {{uname, u, nx * es, es},
                       {"delta", delta, nx * es, es},
                       {"z", z, nx * es, es},
                       {"B", B, nbc * es, es},
                       {"C", C, nbc * es, es},
                       {"A", A, (uint64_t)dim * dstate * 4, 4},
                       {"D", D, (uint64_t)dim * 4, 4},
                       {"dt_bias", dt_bias, (uint64_t)dim * 4, 4},
                       {"initial_state", h0, nst, 4}};
  const Range ry{"y", y, nx * es, es}, rl{"last_state", last_state, nst, 4};
  for (const Range& r : ins)
    if (int rc = check_aligned(r)) return rc;
  if (int rc = check_aligned(ry)) return rc;
  if (int rc = check_aligned(rl)) return rc;
  for (const Range& r : ins) {
    if (overlap(ry, r)) return fail(SSM_ERR_ALIAS, "y overlaps %s", r.name);
    // the state may be advanced in place: last_state == initial_state exactly
    if (overlap(rl, r) && !(r.p == h0 && last_state == h0)) return fail(SSM_ERR_ALIAS, "last_state overlaps %s", r.name);
  }
  if (overlap(ry, rl)) return fail(SSM_ERR_ALIAS, "y overlaps last_state");
  for (const Range& r : cins) {
    if (overlap(ry, r)) return fail(SSM_ERR_ALIAS, "y overlaps %s", r.name);
    if (overlap(rl, r)) return fail(SSM_ERR_ALIAS, "last_state overlaps %s", r.name);
    if (overlap(rcs, r)) return fail(SSM_ERR_ALIAS, "conv_state_out overlaps %s", r.name);
  }
  for (const Range& r : ins)
    if (overlap(rcs, r)) return fail(SSM_ERR_ALIAS, "conv_state_out overlaps %s", r.name);
  if (overlap(rcs, ry)) return fail(SSM_ERR_ALIAS, "conv_state_out overlaps y");
  if (overlap(rcs, rl)) return fail(SSM_ERR_ALIAS, "conv_state_out overlaps last_state");

  ssm::ScanParams p{};
  p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.dt_bias = dt_bias;
  p.softplus = softplus; p.y = y; p.last_state = last_state; p.h0 = h0;
  p.batch = batch; p.dim = dim; p.dstate = dstate; p.seqlen = seqlen; p.dtype = dtype;
  if (conv) {
    p.cw = cv.weight; p.cb = cv.bias; p.cst = cv.state_in; p.cst_out = cv.state_out; p.ck = cv.width;
  }
  if (noalloc) {
    // scratch from the fixed per-GPU array: refuse what it cannot hold, before any launch
    const size_t need = ssm::scan_scratch_bytes(p, ssm::device_cu_count());
    if (need > ssm::kNoAllocScratchBytes)
      return fail(SSM_ERR_UNSUPPORTED, "%s: this scan needs %zu bytes of scratch; the fixed scratch array holds %zu",
                  who, need, ssm::kNoAllocScratchBytes);
    // always the array (also when the plan needs none): a launch path then never reaches the pool
    if (int rc = hip_status(ssm::noalloc_scratch(&p.ws, &p.ws_bytes), who)) return rc;
  }
  return hip_status(ssm::launch_scan_fwd(p, (hipStream_t)stream), who);
}

}  // namespace

extern "C" {

int selective_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, const void* z, const float* dt_bias, int softplus, void* y,
                       float* last_state, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                       void* stream) {
  return scan_impl("selective_scan_fwd launch", u, delta, A, B, C, D, z, dt_bias, softplus, nullptr, y, last_state,
                   batch, dim, dstate, seqlen, dtype, stream);
}

int selective_scan_fwd_resume(const void* u, const void* delta, const float* A, const void* B, const void* C,
                              const float* D, const void* z, const float* dt_bias, int softplus,
                              const float* initial_state, void* y, float* last_state, int64_t batch,
                              int64_t dim, int64_t dstate, int64_t seqlen, int dtype, void* stream) {
  return scan_impl("selective_scan_fwd_resume launch", u, delta, A, B, C, D, z, dt_bias, softplus, initial_state,
                   y, last_state, batch, dim, dstate, seqlen, dtype, stream);
}

int selective_scan_fwd_conv(const void* x, const float* conv_weight, const float* conv_bias,
                            const float* conv_state_in, float* conv_state_out, int64_t width, const void* delta,
                            const float* A, const void* B, const void* C, const float* D, const void* z,
                            const float* dt_bias, int softplus, const float* initial_state, void* y,
                            float* last_state, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                            int dtype, void* stream) {
  if (!conv_weight) {
    g_last_error.clear();
    return fail(SSM_ERR_NULL_ARG, "conv_weight is NULL");
  }
  ConvIn cv;
  cv.weight = conv_weight; cv.bias = conv_bias; cv.state_in = conv_state_in; cv.state_out = conv_state_out;
  cv.width = width;
  return scan_impl("selective_scan_fwd_conv launch", x, delta, A, B, C, D, z, dt_bias, softplus, initial_state, y,
                   last_state, batch, dim, dstate, seqlen, dtype, stream, false, cv);
}

int selective_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* dt_bias, int softplus,
                               const float* initial_state, void* y, float* last_state, int64_t batch,
                               int64_t dim, int64_t dstate, int64_t seqlen, int dtype, void* stream) {
  return scan_impl("selective_scan_fwd_noalloc", u, delta, A, B, C, D, z, dt_bias, softplus, initial_state, y,
                   last_state, batch, dim, dstate, seqlen, dtype, stream, true);
}

int selective_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, const void* z, const float* dt_bias, int softplus,
                       const float* initial_state, const void* dy, void* du, void* ddelta, float* dA, void* dB,
                       void* dC, float* dD, void* dz, float* ddt_bias, float* dinitial_state, int64_t batch,
                       int64_t dim, int64_t dstate, int64_t seqlen, int dtype, void* stream) {
  g_last_error.clear();
  if (seqlen != 0) {
    if (!u) return fail(SSM_ERR_NULL_ARG, "u is NULL");
    if (!delta) return fail(SSM_ERR_NULL_ARG, "delta is NULL");
    if (!B) return fail(SSM_ERR_NULL_ARG, "B is NULL");
    if (!C) return fail(SSM_ERR_NULL_ARG, "C is NULL");
    if (!dy) return fail(SSM_ERR_NULL_ARG, "dy is NULL");
    if (!du) return fail(SSM_ERR_NULL_ARG, "du is NULL");
    if (!ddelta) return fail(SSM_ERR_NULL_ARG, "ddelta is NULL");
    if (!dB) return fail(SSM_ERR_NULL_ARG, "dB is NULL");
    if (!dC) return fail(SSM_ERR_NULL_ARG, "dC is NULL");
    if (z && !dz) return fail(SSM_ERR_NULL_ARG, "dz is NULL while z is given");
  }
  if (!A) return fail(SSM_ERR_NULL_ARG, "A is NULL");
  if (!dA) return fail(SSM_ERR_NULL_ARG, "dA is NULL");
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d is not SSM_F32/SSM_BF16", dtype);
  if (batch < 1 || dim < 1 || dstate < 1 || seqlen < 0)
    return fail(SSM_ERR_BAD_SHAPE, "bad sizes batch=%lld dim=%lld dstate=%lld seqlen=%lld", (long long)batch,
                (long long)dim, (long long)dstate, (long long)seqlen);
  if (too_big(batch, dim, seqlen) || too_big(batch, dstate, seqlen) || too_big(batch, dim, dstate) ||
      batch * ((dim + 63) / 64) > 0x7fffffffLL)
    return fail(SSM_ERR_BAD_SHAPE, "sizes too large");
  if (!ssm::dstate_supported(dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate=%lld not in {1,2,4,8,16,32,64}", (long long)dstate);
  if (softplus != 0 && softplus != 1) return fail(SSM_ERR_BAD_SHAPE, "softplus must be 0 or 1");
  if (!z) dz = nullptr;  // not written without a gate
  const uint64_t es = dtype == SSM_BF16 ? 2 : 4;
  const uint64_t nx = (uint64_t)batch * dim * seqlen, nbc = (uint64_t)batch * dstate * seqlen;
  const uint64_t nst = (uint64_t)batch * dim * dstate * 4;
  const Range ins[] = {{"u", u, nx * es, es},
                       {"delta", delta, nx * es, es},
                       {"z", z, nx * es, es},
                       {"dy", dy, nx * es, es},
                       {"B", B, nbc * es, es},
                       {"C", C, nbc * es, es},
                       {"A", A, (uint64_t)dim * dstate * 4, 4},
                       {"D", D, (uint64_t)dim * 4, 4},
                       {"dt_bias", dt_bias, (uint64_t)dim * 4, 4},
                       {"initial_state", initial_state, nst, 4}};
  const Range outs[] = {{"du", du, nx * es, es},
                        {"ddelta", ddelta, nx * es, es},
                        {"dz", dz, nx * es, es},
                        {"dB", dB, nbc * es, es},
                        {"dC", dC, nbc * es, es},
                        {"dA", dA, (uint64_t)dim * dstate * 4, 4},
                        {"dD", dD, (uint64_t)dim * 4, 4},
                        {"ddt_bias", ddt_bias, (uint64_t)dim * 4, 4},
                        {"dinitial_state", dinitial_state, nst, 4}};
  for (const Range& r : ins)
    if (int rc = check_aligned(r)) return rc;
  for (const Range& r : outs)
    if (int rc = check_aligned(r)) return rc;
  for (size_t i = 0; i < sizeof outs / sizeof outs[0]; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return fail(SSM_ERR_ALIAS, "%s overlaps %s", outs[i].name, r.name);
    for (size_t j = 0; j < i; ++j)
      if (overlap(outs[i], outs[j])) return fail(SSM_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  ssm::BwdParams p{};
  p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.dt_bias = dt_bias;
  p.softplus = softplus; p.h0 = initial_state; p.dy = dy;
  p.du = du; p.ddelta = ddelta; p.dA = dA; p.dB = dB; p.dC = dC; p.dD = dD; p.dz = dz; p.ddt_bias = ddt_bias;
  p.dh0 = dinitial_state;
  p.batch = batch; p.dim = dim; p.dstate = dstate; p.seqlen = seqlen; p.dtype = dtype;
  return hip_status(ssm::launch_scan_bwd(p, (hipStream_t)stream), "selective_scan_bwd launch");
}

int ssd_scan_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                 const void* z, const float* dt_bias, int softplus, const float* initial_state, void* y,
                 float* last_state, int64_t batch, int64_t heads, int64_t headdim, int64_t dstate, int64_t seqlen,
                 int dtype, void* stream) {
  g_last_error.clear();
  if (seqlen != 0) {
    if (!x) return fail(SSM_ERR_NULL_ARG, "x is NULL");
    if (!dt) return fail(SSM_ERR_NULL_ARG, "dt is NULL");
    if (!B) return fail(SSM_ERR_NULL_ARG, "B is NULL");
    if (!C) return fail(SSM_ERR_NULL_ARG, "C is NULL");
    if (!y) return fail(SSM_ERR_NULL_ARG, "y is NULL");
  }
  if (!A) return fail(SSM_ERR_NULL_ARG, "A is NULL");
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d is not SSM_F32/SSM_BF16", dtype);
  if (batch < 1 || heads < 1 || headdim < 1 || dstate < 1 || seqlen < 0)
    return fail(SSM_ERR_BAD_SHAPE, "bad sizes batch=%lld heads=%lld headdim=%lld dstate=%lld seqlen=%lld",
                (long long)batch, (long long)heads, (long long)headdim, (long long)dstate, (long long)seqlen);
  if (too_big(batch, heads * headdim, seqlen) || too_big(batch, dstate, seqlen) || too_big(batch, heads, seqlen) ||
      too_big(batch, heads * headdim, dstate) || batch * heads > 65535)
    return fail(SSM_ERR_BAD_SHAPE, "sizes too large");
  if (softplus != 0 && softplus != 1) return fail(SSM_ERR_BAD_SHAPE, "softplus must be 0 or 1");
  if (dtype != SSM_BF16) return fail(SSM_ERR_UNSUPPORTED, "the SSD kernels take bf16 inputs only");
  if (!ssm::ssd_supported(headdim, dstate))
    return fail(SSM_ERR_UNSUPPORTED,
                "headdim=%lld dstate=%lld: need headdim in {32,64,128} and dstate in {16,32,64} (dstate <= 32 with "
                "headdim 128)",
                (long long)headdim, (long long)dstate);
  if (seqlen % 8 != 0) return fail(SSM_ERR_UNSUPPORTED, "seqlen=%lld is not a multiple of 8", (long long)seqlen);
  if ((seqlen + 63) / 64 > 0x7fffffffLL) return fail(SSM_ERR_BAD_SHAPE, "sizes too large");
  const uint64_t dim = (uint64_t)heads * headdim;
  const uint64_t nx = (uint64_t)batch * dim * seqlen * 2, nbc = (uint64_t)batch * dstate * seqlen * 2;
  const uint64_t ndt = (uint64_t)batch * heads * seqlen * 2, nst = (uint64_t)batch * dim * dstate * 4;
  const Range ins[] = {{"x", x, nx, 16},
                       {"dt", dt, ndt, 16},
                       {"z", z, nx, 16},
                       {"B", B, nbc, 16},
                       {"C", C, nbc, 16},
                       {"A", A, (uint64_t)heads * 4, 4},
                       {"D", D, dim * 4, 4},
                       {"dt_bias", dt_bias, (uint64_t)heads * 4, 4},
                       {"initial_state", initial_state, nst, 4}};
  const Range ry{"y", y, nx, 16}, rl{"last_state", last_state, nst, 4};
  for (const Range& r : ins)
    if (int rc = check_aligned(r)) return rc;
  if (int rc = check_aligned(ry)) return rc;
  if (int rc = check_aligned(rl)) return rc;
  for (const Range& r : ins) {
    if (overlap(ry, r)) return fail(SSM_ERR_ALIAS, "y overlaps %s", r.name);
    if (overlap(rl, r) && !(r.p == initial_state && last_state == initial_state))
      return fail(SSM_ERR_ALIAS, "last_state overlaps %s", r.name);
  }
  if (overlap(ry, rl)) return fail(SSM_ERR_ALIAS, "y overlaps last_state");
  ssm::SsdParams p{};
  p.x = x; p.dt = dt; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.dt_bias = dt_bias; p.softplus = softplus;
  p.h0 = initial_state; p.y = y; p.last_state = last_state;
  p.batch = batch; p.heads = heads; p.headdim = headdim; p.dstate = dstate; p.seqlen = seqlen;
  return hip_status(ssm::launch_ssd_fwd(p, (hipStream_t)stream), "ssd_scan_fwd launch");
}

int ssd_scan_bwd(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                 const void* z, const float* dt_bias, int softplus, const float* initial_state, const void* dy,
                 void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD, void* dz, float* ddt_bias,
                 float* dinitial_state, int64_t batch, int64_t heads, int64_t headdim, int64_t dstate,
                 int64_t seqlen, int dtype, void* stream) {
  g_last_error.clear();
  if (seqlen != 0) {
    if (!x) return fail(SSM_ERR_NULL_ARG, "x is NULL");
    if (!dt) return fail(SSM_ERR_NULL_ARG, "dt is NULL");
    if (!B) return fail(SSM_ERR_NULL_ARG, "B is NULL");
    if (!C) return fail(SSM_ERR_NULL_ARG, "C is NULL");
    if (!dy) return fail(SSM_ERR_NULL_ARG, "dy is NULL");
    if (!dx) return fail(SSM_ERR_NULL_ARG, "dx is NULL");
    if (!ddt) return fail(SSM_ERR_NULL_ARG, "ddt is NULL");
    if (!dB) return fail(SSM_ERR_NULL_ARG, "dB is NULL");
    if (!dC) return fail(SSM_ERR_NULL_ARG, "dC is NULL");
    if (z && !dz) return fail(SSM_ERR_NULL_ARG, "dz is NULL while z is given");
  }
  if (!A) return fail(SSM_ERR_NULL_ARG, "A is NULL");
  if (!dA) return fail(SSM_ERR_NULL_ARG, "dA is NULL");
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d is not SSM_F32/SSM_BF16", dtype);
  if (batch < 1 || heads < 1 || headdim < 1 || dstate < 1 || seqlen < 0)
    return fail(SSM_ERR_BAD_SHAPE, "bad sizes batch=%lld heads=%lld headdim=%lld dstate=%lld seqlen=%lld",
                (long long)batch, (long long)heads, (long long)headdim, (long long)dstate, (long long)seqlen);
  const int64_t dim = heads * headdim;
  if (heads > (1LL << 40) / headdim || too_big(batch, dim, seqlen) || too_big(batch, dstate, seqlen) ||
      too_big(batch, dim, dstate) || batch * ((dim + 63) / 64) > 0x7fffffffLL)
    return fail(SSM_ERR_BAD_SHAPE, "sizes too large");
  if (!ssm::dstate_supported(dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate=%lld not in {1,2,4,8,16,32,64}", (long long)dstate);
  if (softplus != 0 && softplus != 1) return fail(SSM_ERR_BAD_SHAPE, "softplus must be 0 or 1");
  if (!z) dz = nullptr;  // not written without a gate
  const uint64_t es = dtype == SSM_BF16 ? 2 : 4;
  const uint64_t nx = (uint64_t)batch * dim * seqlen, nbc = (uint64_t)batch * dstate * seqlen;
  const uint64_t ndt = (uint64_t)batch * heads * seqlen, nst = (uint64_t)batch * dim * dstate * 4;
  const Range ins[] = {{"x", x, nx * es, es},
                       {"dt", dt, ndt * es, es},
                       {"z", z, nx * es, es},
                       {"dy", dy, nx * es, es},
                       {"B", B, nbc * es, es},
                       {"C", C, nbc * es, es},
                       {"A", A, (uint64_t)heads * 4, 4},
                       {"D", D, (uint64_t)dim * 4, 4},
                       {"dt_bias", dt_bias, (uint64_t)heads * 4, 4},
                       {"initial_state", initial_state, nst, 4}};
  const Range outs[] = {{"dx", dx, nx * es, es},
                        {"ddt", ddt, ndt * es, es},
                        {"dz", dz, nx * es, es},
                        {"dB", dB, nbc * es, es},
                        {"dC", dC, nbc * es, es},
                        {"dA", dA, (uint64_t)heads * 4, 4},
                        {"dD", dD, (uint64_t)dim * 4, 4},
                        {"ddt_bias", ddt_bias, (uint64_t)heads * 4, 4},
                        {"dinitial_state", dinitial_state, nst, 4}};
  for (const Range& r : ins)
    if (int rc = check_aligned(r)) return rc;
  for (const Range& r : outs)
    if (int rc = check_aligned(r)) return rc;
  for (size_t i = 0; i < sizeof outs / sizeof outs[0]; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return fail(SSM_ERR_ALIAS, "%s overlaps %s", outs[i].name, r.name);
    for (size_t j = 0; j < i; ++j)
      if (overlap(outs[i], outs[j])) return fail(SSM_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  ssm::SsdBwdParams p{};
  p.f.x = x; p.f.dt = dt; p.f.A = A; p.f.B = B; p.f.C = C; p.f.D = D; p.f.z = z; p.f.dt_bias = dt_bias;
  p.f.softplus = softplus; p.f.h0 = initial_state;
  p.f.batch = batch; p.f.heads = heads; p.f.headdim = headdim; p.f.dstate = dstate; p.f.seqlen = seqlen;
  p.dtype = dtype; p.dy = dy; p.dx = dx; p.ddt = ddt; p.dA = dA; p.dB = dB; p.dC = dC; p.dD = dD; p.dz = dz;
  p.ddt_bias = ddt_bias; p.dh0 = dinitial_state;
  return hip_status(ssm::launch_ssd_bwd(p, (hipStream_t)stream), "ssd_scan_bwd launch");
}

int selective_state_update(float* state, const void* u, const void* delta, const float* A, const void* B,
                           const void* C, const float* D, const void* z, const float* dt_bias, void* y,
                           int64_t batch, int64_t dim, int64_t dstate, int dtype, void* stream) {
  g_last_error.clear();
  if (!state) return fail(SSM_ERR_NULL_ARG, "state is NULL");
  if (!u) return fail(SSM_ERR_NULL_ARG, "u is NULL");
  if (!delta) return fail(SSM_ERR_NULL_ARG, "delta is NULL");
  if (!A) return fail(SSM_ERR_NULL_ARG, "A is NULL");
  if (!B) return fail(SSM_ERR_NULL_ARG, "B is NULL");
  if (!C) return fail(SSM_ERR_NULL_ARG, "C is NULL");
  if (!y) return fail(SSM_ERR_NULL_ARG, "y is NULL");
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d is not SSM_F32/SSM_BF16", dtype);
  if (batch < 1 || dim < 1 || dstate < 1)
    return fail(SSM_ERR_BAD_SHAPE, "bad sizes batch=%lld dim=%lld dstate=%lld", (long long)batch, (long long)dim,
                (long long)dstate);
  if (too_big(batch, dim, dstate) || dim >= (1LL << 34)) return fail(SSM_ERR_BAD_SHAPE, "sizes too large");
  if (!ssm::dstate_supported(dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate=%lld not in {1,2,4,8,16,32,64}", (long long)dstate);
  const uint64_t es = dtype == SSM_BF16 ? 2 : 4;
  const uint64_t nx = (uint64_t)batch * dim, nbc = (uint64_t)batch * dstate;
  // with dstate >= 4 a lane moves its states and its A, B and C entries 4 at a time, as vectors
  const uint64_t v4 = dstate >= 4 ? 4 : 1;
  const Range ins[] = {{"u", u, nx * es, es},
                       {"delta", delta, nx * es, es},
                       {"z", z, nx * es, es},
                       {"B", B, nbc * es, v4 * es},
                       {"C", C, nbc * es, v4 * es},
                       {"A", A, (uint64_t)dim * dstate * 4, v4 * 4},
                       {"D", D, (uint64_t)dim * 4, 4},
                       {"dt_bias", dt_bias, (uint64_t)dim * 4, 4}};
  const Range rs{"state", state, nx * dstate * 4, v4 * 4}, ry{"y", y, nx * es, es};
  for (const Range& r : ins)
    if (int rc = check_aligned(r)) return rc;
  if (int rc = check_aligned(rs)) return rc;
  if (int rc = check_aligned(ry)) return rc;
  for (const Range& r : ins) {
    if (overlap(rs, r)) return fail(SSM_ERR_ALIAS, "state overlaps %s", r.name);
    if (overlap(ry, r)) return fail(SSM_ERR_ALIAS, "y overlaps %s", r.name);
  }
  if (overlap(ry, rs)) return fail(SSM_ERR_ALIAS, "y overlaps state");

  ssm::StepParams p{state, u, delta, A, B, C, D, z, dt_bias, y, batch, dim, dstate, dtype};
  return hip_status(ssm::launch_state_update(p, (hipStream_t)stream), "selective_state_update launch");
}

int causal_conv1d_fwd(const void* x, const float* weight, const float* bias, const float* conv_state_in,
                      int silu, void* out, float* conv_state_out, int64_t batch, int64_t dim, int64_t seqlen,
                      int64_t width, int dtype, void* stream) {
  g_last_error.clear();
  if (seqlen != 0) {
    if (!x) return fail(SSM_ERR_NULL_ARG, "x is NULL");
    if (!out) return fail(SSM_ERR_NULL_ARG, "out is NULL");
  }
  if (!weight) return fail(SSM_ERR_NULL_ARG, "weight is NULL");
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d is not SSM_F32/SSM_BF16", dtype);
  if (batch < 1 || dim < 1 || seqlen < 0 || width < 1)
    return fail(SSM_ERR_BAD_SHAPE, "bad sizes batch=%lld dim=%lld seqlen=%lld width=%lld", (long long)batch,
                (long long)dim, (long long)seqlen, (long long)width);
  if (width > 4) return fail(SSM_ERR_UNSUPPORTED, "width=%lld not in 1..4", (long long)width);
  if (too_big(batch, dim, seqlen) || too_big(batch, dim, width)) return fail(SSM_ERR_BAD_SHAPE, "sizes too large");
  if (silu != 0 && silu != 1) return fail(SSM_ERR_BAD_SHAPE, "silu must be 0 or 1");
  const uint64_t es = dtype == SSM_BF16 ? 2 : 4;
  const uint64_t nx = (uint64_t)batch * dim * seqlen, nst = (uint64_t)batch * dim * (width - 1) * 4;
  const Range ins[] = {{"x", x, nx * es, es},
                       {"weight", weight, (uint64_t)dim * width * 4, 4},
                       {"bias", bias, (uint64_t)dim * 4, 4},
                       {"conv_state_in", conv_state_in, nst, 4}};
  const Range ro{"out", out, nx * es, es}, rs{"conv_state_out", conv_state_out, nst, 4};
  for (const Range& r : ins)
    if (int rc = check_aligned(r)) return rc;
  if (int rc = check_aligned(ro)) return rc;
  if (int rc = check_aligned(rs)) return rc;
  for (const Range& r : ins) {
    if (overlap(ro, r)) return fail(SSM_ERR_ALIAS, "out overlaps %s", r.name);
    if (overlap(rs, r)) return fail(SSM_ERR_ALIAS, "conv_state_out overlaps %s", r.name);
  }
  if (overlap(ro, rs)) return fail(SSM_ERR_ALIAS, "out overlaps conv_state_out");
  ssm::ConvParams p{x, weight, bias, conv_state_in, silu, out, conv_state_out, batch, dim, seqlen, width, dtype};
  return hip_status(ssm::launch_conv1d_fwd(p, (hipStream_t)stream), "causal_conv1d_fwd launch");
}

int causal_conv1d_update(float* conv_state, const void* x, const float* weight, const float* bias, int silu,
                         void* out, int64_t batch, int64_t dim, int64_t width, int dtype, void* stream) {
  g_last_error.clear();
  if (!conv_state && width > 1) return fail(SSM_ERR_NULL_ARG, "conv_state is NULL");
  if (!x) return fail(SSM_ERR_NULL_ARG, "x is NULL");
  if (!weight) return fail(SSM_ERR_NULL_ARG, "weight is NULL");
  if (!out) return fail(SSM_ERR_NULL_ARG, "out is NULL");
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d is not SSM_F32/SSM_BF16", dtype);
  if (batch < 1 || dim < 1 || width < 1)
    return fail(SSM_ERR_BAD_SHAPE, "bad sizes batch=%lld dim=%lld width=%lld", (long long)batch, (long long)dim,
                (long long)width);
  if (width > 4) return fail(SSM_ERR_UNSUPPORTED, "width=%lld not in 1..4", (long long)width);
  if (too_big(batch, dim, width)) return fail(SSM_ERR_BAD_SHAPE, "sizes too large");
  if (silu != 0 && silu != 1) return fail(SSM_ERR_BAD_SHAPE, "silu must be 0 or 1");
  const uint64_t es = dtype == SSM_BF16 ? 2 : 4;
  const uint64_t nx = (uint64_t)batch * dim;
  const Range ins[] = {{"x", x, nx * es, es},
                       {"weight", weight, (uint64_t)dim * width * 4, 4},
                       {"bias", bias, (uint64_t)dim * 4, 4}};
  const Range rs{"conv_state", conv_state, nx * (width - 1) * 4, 4}, ro{"out", out, nx * es, es};
  for (const Range& r : ins)
    if (int rc = check_aligned(r)) return rc;
  if (int rc = check_aligned(rs)) return rc;
  if (int rc = check_aligned(ro)) return rc;
  for (const Range& r : ins) {
    if (overlap(rs, r)) return fail(SSM_ERR_ALIAS, "conv_state overlaps %s", r.name);
    if (overlap(ro, r)) return fail(SSM_ERR_ALIAS, "out overlaps %s", r.name);
  }
  if (overlap(ro, rs)) return fail(SSM_ERR_ALIAS, "out overlaps conv_state");
  ssm::ConvStepParams p{conv_state, x, weight, bias, silu, out, batch, dim, width, dtype};
  return hip_status(ssm::launch_conv1d_update(p, (hipStream_t)stream), "causal_conv1d_update launch");
}

}  // extern "C"
