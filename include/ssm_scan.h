/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective state-space scan library.
 *
 * Operations of the Mamba selective SSM ("S6"), as described on the pages this
 * library follows (plus the convolution ahead of it, below):
 *
 *   selective_scan_fwd      the whole-sequence forward scan (training / prefill):
 *                           "Selective Scan 如何兼顾训练与 Decode" in "AI inference
 *                           series (14)" (wiblog.cn) -- prefill runs the parallel
 *                           selective scan and writes the final state; the
 *                           hardware-aware chunked scan of the Mamba summary
 *                           (junchaoiu.github.io, 方法 step 2) and of the mlqm.cn
 *                           tutorial §6.
 *   selective_scan_bwd      gradients of the forward scan (training), states recomputed.
 *   ssd_scan_fwd            the Mamba-2 SSD form (scalar decay per head) on the matrix cores.
 *   ssd_scan_bwd            its backward (every gradient for a given dy).
 *   selective_state_update  one autoregressive decode step: a single-step
 *                           recurrent update of a fixed-size per-request state,
 *                           updated in place (same wiblog.cn page, table of the
 *                           two execution forms and the part on managing per-request state;
 *                           mlqm.cn tutorial §9.2, the single-step update).
 *
 * Per channel d, state n and step t (h_{-1} = 0 for the scan unless resumed from a state):
 *   Delta_t   = softplus(delta_t + dt_bias[d])   (softplus flag off: delta_t + dt_bias[d])
 *   Abar_t[n] = exp(Delta_t * A[d,n])            ZOH transition (mlqm.cn §3.2;
 *                                                "Mamba close reading" (jsqmd.com) §1.2)
 *   h_t[n]    = Abar_t[n] * h_{t-1}[n] + Delta_t * B_t[n] * u_t
 *                                                first-order input term Delta*B (mlqm.cn §3.2, §9.2)
 *   y_t       = (sum_n C_t[n] h_t[n] + D[d] u_t) * silu(z_t),  silu(z) = z * sigmoid(z)
 *                                                readout and D skip (tech.kj168168.com essay §二.1,
 *                                                mlqm.cn §9.2); SiLU gate (Mamba summary 方法 step 3)
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA memory on the
 *    current device), row-major and contiguous (last dimension fastest).
 *  - `dtype` (ssm_dtype_t) is the element type of u, delta, z, B, C and y.  A, D,
 *    dt_bias and the state are always fp32.  Arithmetic is fp32 throughout.
 *  - Ownership: the caller owns every buffer.  The library keeps no pointer to them
 *    after a call returns.  Scratch memory (segment carries, checkpoints, chunk states) is
 *    kept per (device, stream) between calls and held until the process exits: the calls on
 *    one stream run in order and reuse it, calls on different streams never share it.  Under
 *    graph capture it is taken instead, stream-ordered on `stream`, from a memory pool the
 *    library creates per device, and returned to that pool on `stream`; a captured call needs
 *    the pool to hold as much already (an earlier call of that size on any stream reserves it),
 *    since capture does not let the pool make new memory.
 *  - Calls are asynchronous on `stream` (hipStream_t; NULL = the null stream) and
 *    never synchronise the device.
 *  - Errors: the return value is an ssm_status_t.  Arguments are validated before
 *    any HIP call; a validation error leaves every output untouched.  Launch errors
 *    return SSM_ERR_HIP; faults inside a kernel surface at the caller's next
 *    synchronisation.  Non-finite inputs propagate; they are not checked.
 *    ssm_last_error() gives a text for the calling thread's last non-OK status.
 *  - Thread safety: calls on different streams may run concurrently.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype_t;

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL_ARG = -1,     /* a required pointer is NULL                         */
  SSM_ERR_BAD_SHAPE = -2,    /* a size is negative / zero where not allowed / too big */
  SSM_ERR_BAD_DTYPE = -3,    /* dtype is not SSM_F32 or SSM_BF16                   */
  SSM_ERR_MISALIGNED = -4,   /* a pointer is not aligned to its element size (or to the
                                vector width an entry point documents)              */
  SSM_ERR_ALIAS = -5,        /* an output overlaps an input or another output      */
  SSM_ERR_UNSUPPORTED = -6,  /* dstate not in the compiled set {1,2,4,8,16,32,64}  */
  SSM_ERR_HIP = -7           /* a HIP runtime call or kernel launch failed         */
} ssm_status_t;

/*
 * Forward selective scan over a whole sequence.
 *
 *   u, delta, z : [batch, dim, seqlen]  (dtype)   u = input x_t, delta = raw step before bias/softplus
 *   A           : [dim, dstate] fp32             (= -exp(A_log); sign is not checked)
 *   B, C        : [batch, dstate, seqlen] (dtype)  input-dependent, shared by all channels of a batch row
 *   D, dt_bias  : [dim] fp32                     NULL = no skip term / zero bias
 *   z           : NULL = no gate
 *   softplus    : 0 or 1
 *   y           : [batch, dim, seqlen] (dtype) output; must not overlap any input
 *   last_state  : [batch, dim, dstate] fp32 output h_{L-1}; NULL = not written;
 *                 seqlen == 0 writes zeros
 * Required: u, delta, A, B, C, y (all but A may be NULL when seqlen == 0, as
 * the sequence tensors are then empty).  batch, dim, dstate >= 1 and seqlen >= 0;
 * batch * dim * max(seqlen, dstate) < 2^40 elements.
 */
int selective_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, const void* z, const float* dt_bias, int softplus, void* y,
                       float* last_state, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                       int dtype, void* stream);

/*
 * Forward selective scan resumed from a given state: h_{-1} = initial_state instead of 0.
 * This is prefill in pieces -- the state a prefill writes is the state the next piece (or
 * the decode steps) continues from ("AI inference series (14)", wiblog.cn: prefill runs
 * the whole-sequence scan and writes the final state; the request state is then carried
 * forward).  A scan of a+b steps equals a scan of the first a steps followed by this call
 * on the next b steps from its last_state.
 *
 *   initial_state : [batch, dim, dstate] fp32, NULL = zeros (then identical to
 *                   selective_scan_fwd).  It may be the very same buffer as last_state
 *                   (the state is advanced in place); any other overlap with an output
 *                   is SSM_ERR_ALIAS.  seqlen == 0 copies it to last_state.
 * Every other argument, requirement and error is as for selective_scan_fwd.
 */
int selective_scan_fwd_resume(const void* u, const void* delta, const float* A, const void* B, const void* C,
                              const float* D, const void* z, const float* dt_bias, int softplus,
                              const float* initial_state, void* y, float* last_state, int64_t batch,
                              int64_t dim, int64_t dstate, int64_t seqlen, int dtype, void* stream);

/*
 * The causal conv1d + SiLU of the Mamba block and the scan after it, in one call:
 *   u_t = silu(conv_bias[d] + sum_{k<width} conv_weight[d,k] * x[t-(width-1)+k])
 * (Mamba summary (junchaoiu.github.io), 方法 third step: 1-D convolution for local features, then
 * SiLU, then the selective SSM; mlqm.cn tutorial §7.1), and then exactly the scan of
 * selective_scan_fwd_resume on that u.  The call takes whichever route measured faster: for fp32
 * rows (dstate 16) the convolution runs inside the scan kernels and u never reaches memory; for
 * bf16 rows the convolution kernel writes u to scratch kept for the stream and the scan reads it.
 * (A model that also feeds u to other layers needs causal_conv1d_fwd for it.)
 *
 *   x               : [batch, dim, seqlen] (dtype), the convolution's input
 *   conv_weight     : [dim, width] fp32, width in 1..4 (required); conv_bias : [dim] fp32, NULL = 0
 *   conv_state_in   : [batch, dim, width-1] fp32, the inputs before step 0, oldest first; NULL = zeros
 *   conv_state_out  : [batch, dim, width-1] fp32 output, the last width-1 inputs (the state the next
 *                     piece or causal_conv1d_update continues from); NULL = not written.  Must not
 *                     overlap any other argument.
 *   delta, A, B, C, D, z, dt_bias, softplus, initial_state, y, last_state, sizes, dtype, stream:
 *                     as for selective_scan_fwd_resume.
 * On the fused route u is kept in fp32 between the convolution and the scan, as
 * causal_conv1d_fwd followed by the scan does with fp32 rows, so the two agree bit for bit there;
 * on the other route u is rounded to the rows' dtype, as causal_conv1d_fwd stores it.  Other
 * dstates, rows that are not whole 16-byte pieces and unaligned tensors take the second route
 * too.  Errors as for
 * selective_scan_fwd; width outside 1..4 is SSM_ERR_UNSUPPORTED, a NULL conv_weight
 * SSM_ERR_NULL_ARG.
 */
int selective_scan_fwd_conv(const void* x, const float* conv_weight, const float* conv_bias,
                            const float* conv_state_in, float* conv_state_out, int64_t width, const void* delta,
                            const float* A, const void* B, const void* C, const float* D, const void* z,
                            const float* dt_bias, int softplus, const float* initial_state, void* y,
                            float* last_state, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                            int dtype, void* stream);

/*
 * selective_scan_fwd_resume without any memory allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The scan's scratch (carries and hand-over flags of the interval schedule,
 * segment aggregates of the two-pass plans) lives in a fixed 16 MiB device array, one copy
 * per GPU, held from the first call on that GPU until the process exits; nothing is taken
 * from the pool, and no hipMalloc / hipFree is made.  Arguments, results, launch plan and
 * errors are exactly those of selective_scan_fwd_resume (initial_state NULL = zeros), plus:
 * a call whose plan needs more scratch than the array holds returns SSM_ERR_UNSUPPORTED
 * (ssm_last_error() gives both sizes) and touches no output.  The array keeps the last
 * call's contents; what must start at zero is cleared by a kernel at the start of each call.
 * Every call on one GPU shares its array: two calls that overlap in time on the same GPU
 * (on different streams, or from different host threads) race on it and give undefined
 * results, so such callers must order their calls.
 */
int selective_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* dt_bias, int softplus,
                               const float* initial_state, void* y, float* last_state, int64_t batch,
                               int64_t dim, int64_t dstate, int64_t seqlen, int dtype, void* stream);

/*
 * Backward of the forward scan: the gradients of a scalar loss through y, given
 * dy = dLoss/dy.  The pages have the fused kernel recompute the intermediate states in
 * the backward pass rather than store them (Mamba summary (junchaoiu.github.io), 方法
 * step 2; mlqm.cn tutorial §6); the gradients follow from the recurrence above by the
 * adjoint method.  With ds_t = dy_t * silu(z_t) (dy_t without a gate) and
 *   lam_t[n] = ds_t C_t[n] + Abar_{t+1}[n] lam_{t+1}[n],  lam_L = 0,
 *   du_t      = ds_t D[d] + Delta_t sum_n lam_t[n] B_t[n]
 *   ddelta_t  = sigmoid(delta_t + dt_bias[d]) * sum_n lam_t[n] (Abar_t[n] h_{t-1}[n] A[d,n] + B_t[n] u_t)
 *               (without the sigmoid factor when softplus is off)
 *   dz_t      = dy_t * (sum_n C_t[n] h_t[n] + D[d] u_t) * silu'(z_t)
 *   dA[d,n]   = sum over b, t of lam_t[n] Abar_t[n] h_{t-1}[n] Delta_t
 *   dB_t[n]   = sum over d of lam_t[n] Delta_t u_t      dC_t[n] = sum over d of ds_t h_t[n]
 *   dD[d]     = sum over b, t of ds_t u_t               ddt_bias[d] = sum over b, t of ddelta_t
 *   dinitial_state = Abar_0 lam_0
 *
 *   u, delta, A, B, C, D, z, dt_bias, softplus, initial_state : the forward call's inputs,
 *                 as for selective_scan_fwd_resume (initial_state NULL = zeros)
 *   dy          : [batch, dim, seqlen] (dtype)
 *   du, ddelta  : [batch, dim, seqlen] (dtype) outputs
 *   dz          : [batch, dim, seqlen] (dtype) output, required when z is given; not written
 *                 (and may be NULL) without z
 *   dB, dC      : [batch, dstate, seqlen] (dtype) outputs
 *   dA          : [dim, dstate] fp32 output
 *   dD, ddt_bias: [dim] fp32 outputs; NULL = not computed (they are computed whether or not
 *                 D / dt_bias is given: the gradient at zero)
 *   dinitial_state : [batch, dim, dstate] fp32 output; NULL = not computed
 * Sums over channels, batch rows and time are reduced in a fixed order: the result is
 * deterministic.  Every output must not overlap an input or another output.  seqlen == 0
 * writes zeros to dA, dD, ddt_bias and dinitial_state.  Required: u, delta, A, B, C, dy,
 * du, ddelta, dA, dB, dC (all but A and dA may be NULL when seqlen == 0).  Scratch memory
 * (kept for the stream, as above): about (4 * dstate / T + 1) * 4 bytes per (batch, dim, step),
 * T = 16, 8, 2, 1 steps per chunk for dstate <= 8, 16, 32, 64, plus the per-channel-group
 * partials of dB and dC.  Errors as for selective_scan_fwd.
 */
int selective_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, const void* z, const float* dt_bias, int softplus,
                       const float* initial_state, const void* dy, void* du, void* ddelta, float* dA, void* dB,
                       void* dC, float* dD, void* dz, float* ddt_bias, float* dinitial_state, int64_t batch,
                       int64_t dim, int64_t dstate, int64_t seqlen, int dtype, void* stream);

/*
 * The Mamba-2 "state space duality" (SSD) form of the scan: one decay rate and one step size
 * per head of `headdim` channels, evaluated as chunked matrix products on the matrix cores.
 * The pages describe Mamba-2 as showing that the selective scan is dual to multiplication by
 * a structured (semiseparable) matrix, so that the work can be reorganised in chunks onto
 * matrix-multiply units (mlqm.cn tutorial §8; AI inference series (14), the part on
 * reorganising the SSM into matrix computation).  With head h = d / headdim, it computes the
 * recurrence above with A[d, n] = A[h] for every n and delta[b, d, t] = dt[b, h, t]
 * (dt_bias[h] likewise), that is, per head:
 *   y_t = (sum_{s<=t} (C_t . B_s) exp(A[h] (cs_t - cs_s)) Delta_s x_s + D x_t) * silu(z_t),
 *   cs_t = Delta_0 + ... + Delta_t.
 *
 *   x, z, y       : [batch, heads*headdim, seqlen] bf16; z NULL = no gate
 *   dt            : [batch, heads, seqlen] bf16, raw step before bias / softplus
 *   A             : [heads] fp32;  dt_bias : [heads] fp32, NULL = 0
 *   B, C          : [batch, dstate, seqlen] bf16, shared by all heads
 *   D             : [heads*headdim] fp32, NULL = no skip
 *   initial_state : [batch, heads*headdim, dstate] fp32, NULL = zeros; may be the same buffer
 *                   as last_state (advanced in place)
 *   last_state    : [batch, heads*headdim, dstate] fp32 output, NULL = not written
 * Supported: dtype SSM_BF16, headdim 32, 64 or 128, dstate in {16, 32, 64} (at most 32 with
 * headdim 128), seqlen a multiple of 8, and
 * x, dt, z, y, B, C 16-byte aligned; anything else is SSM_ERR_UNSUPPORTED (or
 * SSM_ERR_MISALIGNED).  The matrix-core products take bf16 operands with fp32 accumulation;
 * operands computed in fp32 (the decay-weighted matrices, the carried state) enter as hi + lo
 * bf16 pairs.  Results match the recurrence within the bf16 tolerance; they are not bit-equal
 * to selective_scan_fwd on the broadcast parameters.  Scratch:
 * 4 * dstate * headdim bytes per (batch, head, 64-step chunk).  Errors as for selective_scan_fwd.
 */
int ssd_scan_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                 const void* z, const float* dt_bias, int softplus, const float* initial_state, void* y,
                 float* last_state, int64_t batch, int64_t heads, int64_t headdim, int64_t dstate, int64_t seqlen,
                 int dtype, void* stream);

/*
 * Backward of ssd_scan_fwd: the gradients of a scalar loss through y, given dy = dLoss/dy
 * (the Mamba-2 form's training half; mlqm.cn tutorial §8).  The SSD layer is the selective
 * recurrence with one decay rate and one step size per head, broadcast to the head's channels,
 * so its gradients are selective_scan_bwd's on the broadcast parameters with the broadcast
 * parameters' gradients summed back per head (the chain rule):
 *   ddt[b, h, t] = sum over the head's channels of ddelta;  dA[h] = sum over the head's
 *   channels and all states of dA;  ddt_bias[h] = sum over the head's channels;
 * dx, dz, dB, dC, dD and dinitial_state are the scan's own.  Computed by the backward scan's
 * kernels on the broadcast step sizes, in fp32 state, with every sum in a fixed order (results
 * reproducible bit for bit); not on the matrix cores.
 *   x, z, dy, dx, dz : [batch, heads*headdim, seqlen] (dtype)
 *   dt, ddt          : [batch, heads, seqlen] (dtype)
 *   A, dA            : [heads] fp32;  dt_bias, ddt_bias : [heads] fp32, NULL = absent / not wanted
 *   B, C, dB, dC     : [batch, dstate, seqlen] (dtype)
 *   D, dD            : [heads*headdim] fp32, NULL = absent / not wanted
 *   initial_state, dinitial_state : [batch, heads*headdim, dstate] fp32, NULL = zero / not wanted
 * Supported: SSM_F32 or SSM_BF16, any headdim >= 1, dstate in {1, 2, 4, 8, 16, 32, 64}.
 * Required: x, dt, A, B, C, dy, dx, ddt, dA, dB, dC (and dz when z is given); outputs must not
 * overlap inputs or each other.  Scratch: batch x heads*headdim x seqlen elements of dtype (the
 * broadcast step sizes) and as many fp32 (their gradients, summed per head in fp32), plus the
 * backward scan's.  Errors as for selective_scan_bwd.
 */
int ssd_scan_bwd(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                 const void* z, const float* dt_bias, int softplus, const float* initial_state, const void* dy,
                 void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD, void* dz, float* ddt_bias,
                 float* dinitial_state, int64_t batch, int64_t heads, int64_t headdim, int64_t dstate,
                 int64_t seqlen, int dtype, void* stream);

/*
 * One decode step for `batch` independent requests, state updated IN PLACE.
 *
 *   state       : [batch, dim, dstate] fp32, read as h_{t-1} and overwritten with h_t
 *   u, delta, z : [batch, dim] (dtype); z NULL = no gate
 *   A           : [dim, dstate] fp32
 *   B, C        : [batch, dstate] (dtype)
 *   D, dt_bias  : [dim] fp32, NULL = absent / zero
 *   y           : [batch, dim] (dtype) output
 * With dstate >= 4, state and A must be 16-byte aligned and B, C aligned to 4 elements
 * (lanes move 4 consecutive entries at once); otherwise SSM_ERR_MISALIGNED.
 * Softplus is always applied to delta + dt_bias.  Required: state, u, delta, A,
 * B, C, y; state and y must not overlap an input or each other.
 */
int selective_state_update(float* state, const void* u, const void* delta, const float* A, const void* B,
                           const void* C, const float* D, const void* z, const float* dt_bias, void* y,
                           int64_t batch, int64_t dim, int64_t dstate, int dtype, void* stream);

/*
 * Causal depthwise 1-D convolution with an optional SiLU: the step before the selective
 * SSM in the Mamba block (Mamba summary (junchaoiu.github.io), 方法 third step: linear
 * expansion, 1-D convolution for local features, SiLU; mlqm.cn tutorial §7.1: causal
 * 1-D convolution then SiLU ahead of the selective SSM).  Per row (b, d), step t:
 *
 *   v_t = bias[d] + sum_{k=0..width-1} weight[d,k] * x[t-(width-1)+k]
 *   out_t = silu(v_t) if silu else v_t
 *
 *   x, out        : [batch, dim, seqlen] (dtype); out must not overlap an input
 *   weight        : [dim, width] fp32, width in 1..4;  bias : [dim] fp32, NULL = 0
 *   conv_state_in : [batch, dim, width-1] fp32, the width-1 inputs before step 0,
 *                   oldest first; NULL = zeros
 *   conv_state_out: [batch, dim, width-1] fp32 output, the last width-1 inputs (the
 *                   state the next piece or the decode steps continue from); NULL = not
 *                   written.  Must not overlap conv_state_in or any other argument.
 * A request keeps this window next to its SSM state ("AI inference series (14)",
 * wiblog.cn: per-request conv state and SSM state).  Required: x, weight, out (x and
 * out may be NULL when seqlen == 0).  Errors as for selective_scan_fwd; width outside
 * 1..4 is SSM_ERR_UNSUPPORTED.
 */
int causal_conv1d_fwd(const void* x, const float* weight, const float* bias, const float* conv_state_in,
                      int silu, void* out, float* conv_state_out, int64_t batch, int64_t dim, int64_t seqlen,
                      int64_t width, int dtype, void* stream);

/*
 * One decode step of the convolution for every row, the window advanced in place:
 * out = silu(bias + weight . [conv_state, x]) and conv_state <- [conv_state[1:], x].
 *
 *   conv_state : [batch, dim, width-1] fp32, read and UPDATED IN PLACE
 *   x, out     : [batch, dim] (dtype);  weight, bias, silu, width as above
 * Required: conv_state (unless width == 1), x, weight, out; out must not overlap an input
 * or the state.
 */
int causal_conv1d_update(float* conv_state, const void* x, const float* weight, const float* bias, int silu,
                         void* out, int64_t batch, int64_t dim, int64_t width, int dtype, void* stream);

/*
 * Launch plan selective_scan_fwd would use for these sizes on a GPU with `num_cus`
 * compute units (host-only; no GPU needed).  Writes 5 int64 values to `out`:
 *   out[0] mode: 0 intervals (the channel groups' sequences laid end to end and cut into
 *                one equal interval per workgroup; a sequence split between two
 *                workgroups hands its state on), 1 one pass per channel group,
 *                2 aggregate + carry + output passes, 3 generic kernels (dstate < 4 or
 *                rows not a whole number of 16 bytes)
 *   out[1] channel groups of 64;
 *   out[2] segments per group (modes 1, 2) or intervals (mode 0);
 *   out[3] steps per segment or per interval;
 *   out[4] workgroups of the output pass.
 * Pointer alignment, checked per call, can also route a call to the generic kernels.
 */
int ssm_scan_plan(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype, int num_cus,
                  int64_t* out);

/*
 * Hand-over waits that gave up.  When a scan is cut into intervals (launch plan mode 0), a
 * sequence split between two workgroups continues from the state its first piece hands
 * over; the wait for it is bounded (2^26 polls) so that no launch can hang.  A wait that
 * runs out means that state never arrived: the waiting piece then computes from NaN, so
 * its outputs and the final state are visibly invalid, and a device-side counter is
 * incremented (once per waiting wave, four per sequence).  The backward's main pass, when
 * it runs on intervals (chains, batch row x channel group, at least as many as resident
 * workgroups), hands the adjoint on the same way, right to left, and counts its give-ups
 * in a second counter (a give-up poisons the adjoint, hence the gradients of that part of
 * the sequence and the parameter gradients).  This call copies the sum of the current
 * device's counters to *count (a synchronous device read) and, with reset != 0, sets them
 * to zero.  Required: count.  Errors: SSM_ERR_NULL_ARG, SSM_ERR_HIP.
 */
int ssm_handover_failures(int64_t* count, int reset);

/*
 * Test hook for the give-up path above (scan and backward), process-wide, for the launches that follow:
 * max_polls bounds the wait (<= 0 restores 2^26) and publish = 0 makes the first pieces
 * skip setting their hand-over flags, so that every waiting piece gives up after max_polls
 * polls while every kernel still runs to its end.  (max_polls <= 0, publish = 1) is the
 * normal setting.  Not for production use; not synchronised with calls in flight.
 * Always SSM_OK.
 */
int ssm_test_handover_wait(int max_polls, int publish);

/* Text describing the calling thread's most recent non-OK status ("" if none). */
const char* ssm_last_error(void);

/*
 * Frees the memory the library keeps for `stream` on the current device: the scratch of the
 * scans on that stream (carries, checkpoints, chunk states, the convolution's output) and the
 * interval schedule's control block.  For callers that retire a stream, or a serving loop that
 * wants the memory back between phases.  It first waits for the work queued on the stream;
 * the caller must not queue new work on that stream from another thread while it runs.  The
 * next call on the stream makes what it needs again.  A capturing stream is refused with
 * SSM_ERR_UNSUPPORTED.  Memory the library's pool holds in reserve for captured calls is kept.
 */
int ssm_release_stream(void* stream);

/* ABI version of this header (incremented whenever an entry point is added or changed). */
int ssm_abi_version(void);

#define SSM_ABI_VERSION 10

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
