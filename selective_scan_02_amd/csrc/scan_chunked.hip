// scan_chunked.hip -- the main forward selective-scan kernel for gfx950.
//
// Why this shape.  At dstate = 16 the scan costs ~110 VALU issue slots per
// element (16 exps at half rate plus 4 FMA-class ops per state, softplus and
// SiLU) against ~8 bytes of HBM traffic, so on MI355X it is bound by the
// vector ALUs, not by HBM.  The design spends no VALU work that the plain
// recurrence does not need and finds parallelism without recomputation.
//
//  * Workgroup = 64 consecutive channels (b, d0..d0+63), one channel per lane,
//    and 8 waves in two roles.  Waves 0..3 are SCANNERS: scanner s owns states
//    n in [s*N/4, (s+1)*N/4) of all 64 channels and runs only the recurrence
//    and the partial readout of its states -- a long stream of independent
//    VALU work.  Waves 4..7 are HELPERS: they load u, delta, z, B, C, compute
//    Delta = softplus(delta + dt_bias), Delta*u, D*u and SiLU(z) once per
//    element, sum the four partial readouts, gate, round and store y.  A SIMD
//    hosts one scanner and one helper, so the helper's latency-bound work hides
//    under the scanner's arithmetic.
//  * B_t[n] and C_t[n] are uniform across a scanner wave.  A scanner holds them
//    in VGPRs, lane l carrying step (l mod 16) -- every 16-lane row holds the
//    same 16 values -- and the consuming VALU instruction reads "lane t of my
//    row" through the DPP row_newbcast source modifier: a free broadcast.
//  * The sequence is processed in chunks of kT = 16 steps through a three-stage
//    pipeline -- prep(j) | scan(j-1) | finalize(j-2) -- with one workgroup
//    barrier per chunk.  u, delta, z, B, C are fetched with 16-byte loads two
//    chunks ahead and staged through LDS; y leaves through an LDS tile as
//    16-byte coalesced stores.  Only y and the final state reach HBM (fusion
//    with on-chip intermediates: Mamba summary (junchaoiu.github.io), 方法 step
//    2; tech.kj168168.com essay §二.3).
//
// Sequence parallelism (chunked two-level scan: "Mamba close reading"
// (jsqmd.com) §2.2 and the sketch of §7; mlqm.cn tutorial §6).  The sequence is
// cut into segments that run in parallel, with exact carries between them.
//  MODE 0 (intervals), when there are at least as many channel groups as CUs:
//    the chains of the G channel groups (tch chunks each) are laid end to end and
//    cut into one interval of W = ceil(G * tch / CUs) chunks per workgroup.
//    W >= tch, so an interval holds whole chains plus at most a tail piece of its
//    first chain and a head piece of its last: a chain is split at most once.  A
//    workgroup takes its interval from an atomic ticket and runs the head piece
//    first, then the whole chains, then the tail piece, which starts from the
//    state the previous interval's workgroup hands over at the split point,
//    through global memory, with one flag per scanner wave.  That head was the
//    first piece its workgroup ran, finished at least W - tch chunk-times
//    before the tail starts, so the wait is normally over: no recomputation,
//    exact sequential carry, and a workgroup pays the pipeline's fill and drain
//    once per piece (two or three pieces).  The hand-over uses device-scope
//    atomic loads and stores only (no agent-scope fences: on this multi-XCD
//    part those write back or invalidate whole L2 caches).
//  MODE 1 (output) with K = 1: one segment per group, no carry at all.
//  MODE 2 (aggregate) + carry kernel + MODE 1 (output): for few channel groups
//    (very long sequences).  Every segment but the last first computes its end
//    state from h = 0 and its sum of Delta (the segment's transition is
//    exp(A * sum Delta)); a carry kernel turns these into incoming states; the
//    output pass reruns each segment from its incoming state.
//
// Deadlock freedom of MODE 0: a tail piece waits only for the head piece of the
// interval with the previous ticket.  That workgroup took its ticket earlier, so
// it is running or done, and it runs its head first, which waits for nothing.
// The wait is additionally bounded (it gives up after 2^26 polls), so every
// wave always reaches the exit.  A wait that gives up means the state at the split
// point never arrived: the piece's state is set to NaN, so its outputs and the final
// state visibly fail instead of passing as numbers, and a device counter records it
// (ssm_handover_failures).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <utility>

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {
namespace chunked {

#ifndef SSM_SPLIT_UNITS_PER_CU
// workgroups per CU in the two-pass split; on the 2^20-step sequence 2, 4, 8, 12 and 16 measured
// 2.71, 2.65, 2.45-2.56, 2.46 and 2.62 ms
#define SSM_SPLIT_UNITS_PER_CU 8
#endif
#ifndef SSM_SPLIT_OUT_PER_CU
// output-pass workgroups per CU in the two-pass split: each continues through several
// aggregate segments, so the pipeline fills and drains once per output unit (2^20-step fp32
// sequence, 512 segments: 1, 2 and 8 output units per CU measured 2.44, 2.75-2.79, 2.50 ms)
#define SSM_SPLIT_OUT_PER_CU 1
#endif
#ifndef SSM_HELPER_PRIO
#define SSM_HELPER_PRIO 1
#endif
#ifndef SSM_PREFETCH
#define SSM_PREFETCH 3  // chunks of loads in flight per helper thread (1..3)
#endif
#ifndef SSM_GATE_BLEND
#define SSM_GATE_BLEND 1
#endif

#ifndef SSM_SCAN_SG
#define SSM_SCAN_SG 0  // 0: by states per scanner wave
#endif
#ifndef SSM_HELPERS
// helper waves of the output kernels: 8 (two per SIMD next to its scanner) measured 5% faster
// than 4 on the 2.8B-shaped layer (0.229-0.232 against 0.241-0.246 ms, same box) and about 2%
// on the 2^20-step sequence.  The kernels with the fused convolution (fp32 rows only) also take
// 8: with the channel's taps waited for ahead of the chunk loop they measured 260 against 270 us
// with 4 on the 2.8B-shaped layer in fp32, and 629 against 651 us on 2^18 fp32 steps.
#define SSM_HELPERS 8
#endif

constexpr int kT = 16;  // time steps per chunk (= lanes of a DPP row)
constexpr int kW = 64;  // channels per group = lanes per wave
constexpr int kS = 4;   // scanner waves

// Helper waves per workgroup: 4 in the aggregate pass and above dstate 16 (twelve waves leave 168
// registers per lane, and those scanners need more), otherwise SSM_HELPERS.
template <int MODE, bool CONV, int N>
constexpr int helpers() {
  return MODE == 2 || N > 16 ? 4 : SSM_HELPERS;
}
template <int MODE, bool CONV, int N>
constexpr int threads() {
  return (kS + helpers<MODE, CONV, N>()) * kW;
}

struct Args {
  const void* u;
  const void* delta;
  const void* z;
  const void* B;
  const void* C;
  const float* A;
  const float* D;
  const float* dt_bias;
  const float* h0;
  void* y;
  float* last_state;
  float* seg_h;   // MODE 1/2: [K, batch*dim, N]
  float* seg_dt;  // MODE 2:   [K, batch*dim]
  float* carry;   // MODE 0:   [groups, N, 64] state at a chain's split point
  unsigned long long* flags;   // MODE 0: [groups, kS] one per chain and scanner wave: the call's `gen` once set
  unsigned long long* ticket;  // MODE 0: interval counter; this call's tickets are tbase, tbase + 1, ...
  unsigned long long tbase, gen;
  int64_t batch, dim, L, seg_len;
  int64_t tch;    // MODE 0: chunks per chain (ceil(L / kT))
  int64_t wlen;   // MODE 0: chunks per interval
  int seg_stride;  // MODE 1 after MODE 2: aggregate segments per output unit (seg_h index step)
  int gpr;     // channel groups per batch row
  int groups;  // batch * gpr
  int nseg;    // K
  int units;   // MODE 1/2: K * groups; MODE 0: intervals (workgroups)
  int softplus;
  int max_polls;  // MODE 0: bound of a tail piece's wait for its hand-over flag
  int publish;    // MODE 0: head pieces set their hand-over flags (0 only under the test hook)
  // CONV kernels: u = silu(conv(x)) is computed in place of loading u (`u` above points to x)
  const float* cw;   // [dim, ck] causal depthwise filter
  const float* cb;   // [dim] its bias, or NULL
  const float* cst;  // [batch*dim, ck-1] inputs before step 0 (oldest first), or NULL = zeros
  int ck;            // filter width, 1..4
};

// Hand-over waits that gave up since the counter was last reset (see the MODE 0 wait).
static __device__ unsigned int handover_giveups;

template <typename TI>
__device__ __forceinline__ float lds_elem(const unsigned char* row, int e) {
  if constexpr (sizeof(TI) == 2) {
    const uint16_t v = *reinterpret_cast<const uint16_t*>(row + 2 * e);
    return __builtin_bit_cast(float, (uint32_t)v << 16);
  } else {
    return *reinterpret_cast<const float*>(row + 4 * e);
  }
}

template <typename TI>
__device__ __forceinline__ void lds_store_elem(unsigned char* row, int e, float v) {
  if constexpr (sizeof(TI) == 2) {
    *reinterpret_cast<__bf16*>(row + 2 * e) = (__bf16)v;
  } else {
    *reinterpret_cast<float*>(row + 4 * e) = v;
  }
}

// Source of loader piece p of a chunk-0 view of unit (b, d0, t_begin): u, delta, z rows of the
// group's channels (XT tensors), then the batch row's B (and C) rows; NULL when the piece is
// unused or the channel lies past dim.
template <typename TI, int N, int XT, int PPR, int EPP>
__device__ __forceinline__ const TI* piece_src(const Args& a, int p, int b, int d0, int64_t t_begin) {
  constexpr int XPIECES = XT * kW * PPR;
  constexpr int PIECES = XPIECES + (XT == 3 ? 2 : 1) * N * PPR;
  const int q = p % PPR;
  if (p < XPIECES) {
    const int tensor = p / (kW * PPR), row = (p / PPR) % kW;
    const TI* base = tensor == 0 ? (const TI*)a.u : tensor == 1 ? (const TI*)a.delta : (const TI*)a.z;
    if (base && d0 + row < a.dim) return base + ((int64_t)b * a.dim + d0 + row) * a.L + t_begin + q * EPP;
  } else if (p < PIECES) {
    const int pp = p - XPIECES, tensor = pp / (N * PPR), n = (pp / PPR) % N;
    return (tensor == 0 ? (const TI*)a.B : (const TI*)a.C) + ((int64_t)b * N + n) * a.L + t_begin + q * EPP;
  }
  return nullptr;
}

// LDS of one workgroup.
template <int N, typename TI, bool OUT>
struct Smem {
  static constexpr int ROWB = kT * sizeof(TI) + 4;  // padded row stride (bytes): conflict-free column access
  // u, delta, z of a chunk, [channel][t].  4-deep ring: chunk c is staged in iteration c-1,
  // read by prep in iteration c and by finalize in iteration c+2, and its slot is reused for
  // chunk c+4 in iteration c+3 -- always after a barrier that follows its last read.
  unsigned char tile[4][OUT ? 3 : 2][kW * ROWB];
  float2 dtdu[2][kT][kW];                            // (Delta, Delta*u), [t][channel]
  float part[OUT ? 2 : 1][OUT ? kS : 1][kT][kW];     // partial readouts of the scanners
  unsigned char ytile[OUT ? 2 : 1][kW * ROWB];       // y of one chunk, [channel][t]
  alignas(16) float bc[4][2][N][kT];                 // B, C of a chunk in fp32 (ring, as tile)
  float red[OUT ? 1 : 4][kW];                         // aggregate pass: the helpers' sums of Delta
  float xh[kW][4];   // CONV: the 3 inputs before the unit's first step, per channel (fp32)
  int unit;     // MODE 0: this workgroup's interval
};

// The DPP broadcast operands of the scanners are read from LDS (bc above), so a
// DPP source register is only ever written by an LDS load, never by a VALU
// instruction: a VALU write followed within two instructions by a DPP read of
// the same register is a hazard the compiler does not see through inline
// assembly (tests/test_isa.py checks the generated code for it).
#define SSM_DPP_MUL(dst, bc, other, T) \
  asm("v_mul_f32_dpp %0, %1, %2 row_newbcast:" #T " row_mask:0xf bank_mask:0xf" : "=v"(dst) : "v"(bc), "v"(other))
#define SSM_DPP_FMAC(acc, bc, other, T) \
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:" #T " row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(bc), "v"(other))

// Every 16-byte piece of u, delta, z, y, B and C is either entirely before the
// end of the unit or entirely after it: the fast path requires seqlen to be a
// multiple of the piece length, and segments are multiples of kT.  So tails
// need only whole-piece predicates.
// The aggregate pass (MODE 2) is held to 128 VGPRs, so two of its workgroups share a CU (its LDS
// allows it): on the 2^20-step fp32 sequence that made the two-pass scan 7% faster.  N = 64 would
// spill under that cap and keeps one.
template <int N, typename TI, int MODE, bool CONV>
__global__ __launch_bounds__((threads<MODE, CONV, N>()))
__attribute__((amdgpu_waves_per_eu(MODE == 2 && N <= 32 ? 4 : 1)))
void scan_chunked_kernel(const Args a) {
  constexpr int NPW = N / kS;        // states per scanner
  // Helper waves raise their issue priority in the split modes (on the 2^20-step fp32 sequence
  // 2.44 ms against 2.59 at equal priority); in the interval schedule equal priority measured
  // better (2.8B-shaped layer: 201 us against 217).
  constexpr int kHelperPrio = MODE == 0 ? 0 : SSM_HELPER_PRIO;
  constexpr int kH = helpers<MODE, CONV, N>();  // helper waves
  constexpr int kHT = kH * kW;             // helper threads
  constexpr int kTPH = kT / kH;            // steps per helper thread per chunk
  static_assert(kT % kH == 0, "helpers split a chunk's steps evenly");
  constexpr int ES = sizeof(TI);     // I/O element bytes
  constexpr int EPP = 16 / ES;       // elements per 16-byte piece
  constexpr int PPR = kT / EPP;      // pieces per tile row
  constexpr bool OUT = MODE != 2;
  constexpr int XT = OUT ? 3 : 2;                // staged tiles: u, delta (and z for the output)
  constexpr int XPIECES = XT * kW * PPR;         // pieces of those tiles in one chunk
  constexpr int PIECES = XPIECES + (OUT ? 2 : 1) * N * PPR;  // ... and the B (and C) rows
  constexpr int LPT = (PIECES + kHT - 1) / kHT;  // pieces per helper thread
  constexpr int ROWB = Smem<N, TI, OUT>::ROWB;
  // steps per group of the scanner's exp-ahead / recurrence split (bounds the registers)
  constexpr int SG = SSM_SCAN_SG > 0 ? SSM_SCAN_SG : NPW <= 2 ? 16 : NPW <= 4 ? 8 : 4;
  static_assert(N % kS == 0 && NPW >= 1, "dstate must be a multiple of 4");
  static_assert(kW * PPR <= kHT, "one y piece per helper thread");

  __shared__ Smem<N, TI, OUT> sm;

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid / kW);  // wave index (uniform)
  const bool scanner = wv < kS;
  const int lane = tid % kW;
  const int lt = lane & (kT - 1);            // the step this lane carries in the B/C vectors
  const int hw = wv - kS;                    // helper index (helpers only)
  const int htid = tid - kS * kW;            // helper thread index (helpers only)

  uint4 rs[4][LPT];       // helpers: loader pieces of chunks in flight (chunk c in rs[c % 4])

  // Set this scanner wave's hand-over flag of chain U: every store of its state must be
  // acknowledged first (s_waitcnt 0), so the flag can only become visible after the state.  The
  // signal fences keep the compiler from moving memory operations across the wait.
#define SSM_PUBLISH(U)                                                                            \
  {                                                                                               \
    __atomic_signal_fence(__ATOMIC_SEQ_CST);                                                      \
    __builtin_amdgcn_s_waitcnt(0);                                                                \
    __atomic_signal_fence(__ATOMIC_SEQ_CST);                                                      \
    if (lane == 0)                                                                                \
      __hip_atomic_store(a.flags + (int64_t)(U) * kS + wv, a.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); \
  }

  // MODE 0: this workgroup's interval [is, ie) of the chains laid end to end (chunk units),
  // taken from a ticket, and how it splits into pieces (see the launch notes above).
  int64_t is = 0, ie = 0, cf = 0, cl = 0;
  bool itail = false, ihead = false;
  int npieces = 1;
  if (MODE == 0) {
    if (tid == 0) sm.unit = (int)(atomicAdd(a.ticket, 1ull) - a.tbase);
    __syncthreads();
    const int ival = __builtin_amdgcn_readfirstlane(sm.unit);
    if (ival >= a.units) return;  // uniform: the whole workgroup leaves
    is = (int64_t)ival * a.wlen;
    ie = is + a.wlen < (int64_t)a.groups * a.tch ? is + a.wlen : (int64_t)a.groups * a.tch;
    cf = is / a.tch;
    cl = (ie - 1) / a.tch;
    itail = is > cf * a.tch;        // the first chain starts before the interval: wait for its head
    ihead = ie < (cl + 1) * a.tch;  // the last chain goes on after it: hand its state over
    npieces = (int)(cl - cf + 1);
  }

  for (int iter = 0;; ++iter) {
    int grp, k = 0;
    int64_t t_begin;
    int len;
    bool wait_in = false, hand_out = false;  // MODE 0: state from / to another workgroup
    const int64_t L = a.L;
    if (MODE == 0) {
      if (iter >= npieces) break;
      // order: the head of the last chain first (it never waits, and the next interval's
      // workgroup waits for it), then the whole chains, then the tail of the first chain
      int64_t cid;
      if (ihead && iter == 0) cid = cl;
      else {
        const int q = iter - (ihead ? 1 : 0);
        const int nfullc = npieces - (ihead ? 1 : 0) - (itail ? 1 : 0);
        cid = q < nfullc ? cf + (itail ? 1 : 0) + q : cf;
      }
      const int64_t c0 = cid * a.tch > is ? cid * a.tch : is;
      const int64_t c1 = (cid + 1) * a.tch < ie ? (cid + 1) * a.tch : ie;
      grp = (int)cid;
      t_begin = (c0 - cid * a.tch) * kT;
      const int64_t t_end = (c1 - cid * a.tch) * kT < L ? (c1 - cid * a.tch) * kT : L;
      len = (int)(t_end - t_begin);
      wait_in = c0 > cid * a.tch;
      hand_out = c1 < (cid + 1) * a.tch;
    } else {
      const int unit = iter == 0 ? (int)blockIdx.x : a.units;
      if (unit >= a.units) break;
      k = unit / a.groups;
      grp = unit - k * a.groups;
      t_begin = (int64_t)k * a.seg_len;
      len = (int)((t_begin + a.seg_len < L ? a.seg_len : L - t_begin));  // steps in this unit
    }
    const int b = grp / a.gpr;
    const int d0 = (grp - b * a.gpr) * kW;
    const int nch = (len + kT - 1) / kT;
    const int nfull = len / kT;

    // this lane's channel
    const int c = d0 + lane;
    const bool active = c < a.dim;
    const int cc = active ? c : (int)a.dim - 1;
    const int64_t ch = (int64_t)b * a.dim + cc;

    // ---- scanner state --------------------------------------------------
    float A2[NPW], h[NPW];
    if (scanner) {
#pragma unroll
      for (int j = 0; j < NPW; ++j) A2[j] = a.A[(int64_t)cc * N + wv * NPW + j] * kLog2e;
    }
    // incoming state.  MODE 0 tail piece: each scanner wave waits for the flag of the matching
    // scanner wave of the chain's head piece and loads its own rows of the hand-over state; the
    // helpers meanwhile start loading the piece's first chunks.
    if (MODE == 0 && wait_in) {
      if (scanner) {
        const unsigned long long* f = a.flags + (int64_t)grp * kS + wv;
        bool arrived = true;  // wave-uniform: the comparison is read through readfirstlane
        for (int spin = 0;
             __builtin_amdgcn_readfirstlane(
                 (int)(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.gen)) == 0;
             ++spin) {
          if (spin >= a.max_polls) {  // bounded: never hang (only a broken launch could get here)
            arrived = false;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if (arrived) {
          // Hand-over protocol (the writer is at the unit end): flag and state are device-scope
          // atomics, coherent across the XCDs' L2 caches without any cache-wide write-back or
          // invalidation; the state loads are issued only after the flag has been observed.
          const float* cp = a.carry + (int64_t)grp * N * kW;
#pragma unroll
          for (int j = 0; j < NPW; ++j)
            h[j] = __hip_atomic_load(cp + (wv * NPW + j) * kW + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          // the state at the split point never arrived: poison the piece rather than go on from
          // whatever the carry buffer holds
#pragma unroll
          for (int j = 0; j < NPW; ++j) h[j] = __builtin_nanf("");
          if (lane == 0) atomicAdd(&handover_giveups, 1u);
        }
      }
    } else if (scanner) {
      if (MODE == 1 && a.seg_h) {
        const int64_t ks = (int64_t)k * a.seg_stride;  // the aggregate segment this unit starts at
#pragma unroll
        for (int j = 0; j < NPW; ++j) h[j] = a.seg_h[(ks * a.batch * a.dim + ch) * N + wv * NPW + j];
      } else if (MODE != 2 && t_begin == 0 && a.h0) {
#pragma unroll
        for (int j = 0; j < NPW; ++j) h[j] = a.h0[ch * N + wv * NPW + j];
      } else {
#pragma unroll
        for (int j = 0; j < NPW; ++j) h[j] = 0.0f;
      }
    }

    // ---- helper state -----------------------------------------------------
    const float bias = a.dt_bias ? a.dt_bias[cc] : 0.0f;
    const float Dd = a.D ? a.D[cc] : 0.0f;
    const bool gated = a.z != nullptr;
    uint32_t gmask = gated ? 0xffffffffu : 0u;
    asm volatile("" : "+v"(gmask));  // opaque: the gate select below stays a bit blend, not a branch
    const bool sp = a.softplus != 0;
    float sdt = 0.0f;
    // CONV: taps of this channel's filter on the window t-3 .. t (width K fills the last K
    // positions); positions before the window are never read (selected to 0, not weighted by 0,
    // so that a non-finite input there cannot leak in)
    float cwv[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cbias = 0.0f;
    int cskip = 0;  // window positions before the filter's first tap
    if constexpr (CONV) {
      cskip = 4 - a.ck;
#pragma unroll
      for (int m = 0; m < 4; ++m) cwv[m] = m >= cskip ? a.cw[(int64_t)cc * a.ck + (m - cskip)] : 0.0f;
      cbias = a.cb ? a.cb[cc] : 0.0f;
    }
    // the channel's parameters loaded above are waited for here, once: left pending into the
    // chunk loop, their first use there would wait for every load and store in flight, in every
    // iteration (vmcnt(0) only; the other counters are left at their maximum)
    if constexpr (CONV) __builtin_amdgcn_s_waitcnt(0x0F70);
    // CONV: u of a chunk from its prep to its finalize, two iterations later (slot = chunk % 2:
    // an iteration finalizes chunk J-2 before it preps chunk J into the same slot)
    float ukeep[2][kTPH];
    const TI* lsrc[LPT];               // NULL: piece unused or past a tensor's rows
    const TI* lsrc_f[LPT];             // unconditional-load version (a harmless valid address)
    int lstep[LPT];                    // first step of the piece within a chunk
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int p = htid + i * kHT;
      const int q = p % PPR;
      const TI* src = piece_src<TI, N, XT, PPR, EPP>(a, p, b, d0, t_begin);
      lsrc[i] = src;
      lstep[i] = q * EPP;
      lsrc_f[i] = src ? src : (const TI*)a.u + t_begin + q * EPP;
    }
    const int yrow = htid / PPR, yq = htid % PPR;
    TI* ydst = (OUT && !scanner && htid < kW * PPR && d0 + yrow < a.dim)
                   ? (TI*)a.y + ((int64_t)b * a.dim + d0 + yrow) * L + t_begin + yq * EPP
                   : nullptr;

    // ---------------- helper stages (TB: LDS double-buffer index of the chunk) -------------
    // global -> registers: pieces of chunk CJ (zero past the end)
    // The steady-state version loads unconditionally (lanes without a piece read a valid
    // address of u): a load issued on only some paths would make the compiler wait for every
    // load in flight before the next use, which would undo the prefetch.
#define SSM_LOAD_CHUNK(R, CJ)                                                                       \
  _Pragma("unroll") for (int i = 0; i < LPT; ++i) {                                                 \
    const int st0 = (CJ) * kT + lstep[i];                                                           \
    R[i] = (lsrc[i] && st0 < len) ? *reinterpret_cast<const uint4*>(lsrc[i] + (CJ) * kT)           \
                                  : make_uint4(0, 0, 0, 0);                                         \
  }
#define SSM_LOAD_CHUNK_FULL(R, CJ)                                                                  \
  _Pragma("unroll") for (int i = 0; i < LPT; ++i) R[i] = *reinterpret_cast<const uint4*>(lsrc_f[i] + (CJ) * kT);
    // registers -> LDS: the u/delta/z tile of chunk CJ, and its B/C rows as fp32
#define SSM_STORE_TILE(CJ, TB, R)                                                                    \
  _Pragma("unroll") for (int i = 0; i < LPT; ++i) {                                                  \
    const int p = htid + i * kHT;                                                                    \
    const int q = p % PPR;                                                                           \
    if (p < XPIECES) {                                                                               \
      const int tensor = p / (kW * PPR), row = (p / PPR) % kW;                                       \
      uint32_t* dst = reinterpret_cast<uint32_t*>(&sm.tile[(CJ) & 3][tensor][row * ROWB + q * 16]); \
      dst[0] = R[i].x; dst[1] = R[i].y; dst[2] = R[i].z; dst[3] = R[i].w;                            \
    } else if (p < PIECES) {                                                                         \
      const int pp = p - XPIECES, tensor = pp / (N * PPR), n = (pp / PPR) % N;                       \
      float* dst = &sm.bc[(CJ) & 3][tensor][n][q * EPP];                                             \
      const uint32_t w[4] = {R[i].x, R[i].y, R[i].z, R[i].w};                                        \
      _Pragma("unroll") for (int e = 0; e < EPP; ++e) {                                              \
        if constexpr (ES == 2) dst[e] = (e & 1) ? __builtin_bit_cast(float, w[e >> 1] & 0xffff0000u)  \
                                                : __builtin_bit_cast(float, w[e >> 1] << 16);        \
        else dst[e] = __builtin_bit_cast(float, w[e]);                                               \
      }                                                                                              \
    }                                                                                                \
  }
    // prep chunk J: Delta, Delta*u to LDS; D*u and silu(z) kept in registers for finalize.
    // TAIL: steps past the end of the unit become identity steps (Delta = 0).
#define SSM_PREP(J, TB, TAIL, US)                                                                 \
  {                                                                                               \
    const unsigned char* ru = &sm.tile[(J) & 3][0][lane * ROWB];                                  \
    const unsigned char* rd = &sm.tile[(J) & 3][1][lane * ROWB];                                  \
    float xv[kTPH], uv[kTPH];                                                                     \
    _Pragma("unroll") for (int i = 0; i < kTPH; ++i) {                                            \
      xv[i] = lds_elem<TI>(rd, hw * kTPH + i);                                                    \
      uv[i] = lds_elem<TI>(ru, hw * kTPH + i);                                                    \
    }                                                                                             \
    if constexpr (CONV) {                                                                         \
      /* the tile holds x: u = silu(bias + taps . x[t-3 .. t]), the 3 inputs before this       */ \
      /* thread's first step from the same row, the previous chunk's row, or the unit's halo   */ \
      float xw[kTPH + 3];                                                                         \
      _Pragma("unroll") for (int i = 0; i < kTPH; ++i) xw[3 + i] = uv[i];                        \
      /* the 3 inputs before this thread's first step: this chunk's row where they lie in it,  \
         else the previous chunk's row, or before the unit's first chunk the saved inputs */    \
      _Pragma("unroll") for (int m = 0; m < 3; ++m) {                                             \
        const int ix = hw * kTPH - 3 + m;                                                         \
        if (ix >= 0)                                                                              \
          xw[m] = lds_elem<TI>(ru, ix);                                                           \
        else if ((J) == 0)                                                                        \
          xw[m] = sm.xh[lane][3 + ix];                                                            \
        else                                                                                      \
          xw[m] = lds_elem<TI>(&sm.tile[((J) - 1) & 3][0][lane * ROWB], kT + ix);                \
      }                                                                                           \
      _Pragma("unroll") for (int i = 0; i < kTPH; ++i) {                                          \
        float v = cbias;                                                                          \
        _Pragma("unroll") for (int m = 0; m < 4; ++m)                                             \
          v = __builtin_fmaf(cwv[m], m >= cskip ? xw[i + m] : 0.0f, v);                           \
        uv[i] = silu(v);                                                                          \
        ukeep[US][i] = uv[i];                                                                     \
      }                                                                                           \
    }                                                                                             \
    _Pragma("unroll") for (int i = 0; i < kTPH; ++i) {                                            \
      const int tl = hw * kTPH + i;                                                               \
      const float x = xv[i] + bias;                                                               \
      float dt = softplus(x);                  /* branch-free: the flag selects, no branch */     \
      dt = sp ? dt : x;                                                                           \
      if (TAIL) dt = (J) * kT + tl < len ? dt : 0.0f;                                             \
      sm.dtdu[TB][tl][lane] = make_float2(dt, dt * uv[i]);                                        \
      if (MODE == 2) sdt += dt;                                                                   \
    }                                                                                             \
  }
    // finalize a chunk (LDS buffer TB): sum the partial readouts, add D*u, gate, round into the y tile
#define SSM_FINALIZE(J, TB, US)                                                                   \
  if (OUT) {                                                                                      \
    unsigned char* ry = &sm.ytile[OUT ? (TB) : 0][lane * ROWB];                                   \
    const unsigned char* ru = &sm.tile[(J) & 3][0][lane * ROWB];                                  \
    const unsigned char* rz = &sm.tile[(J) & 3][OUT ? 2 : 0][lane * ROWB];                         \
    float pp[kTPH][kS], uv[kTPH], zv[kTPH];                                                       \
    _Pragma("unroll") for (int i = 0; i < kTPH; ++i) {                                            \
      _Pragma("unroll") for (int w = 0; w < kS; ++w) pp[i][w] = sm.part[OUT ? (TB) : 0][w][hw * kTPH + i][lane]; \
      uv[i] = CONV ? ukeep[US][i] : lds_elem<TI>(ru, hw * kTPH + i);                              \
      zv[i] = lds_elem<TI>(rz, hw * kTPH + i);                                                    \
    }                                                                                             \
    _Pragma("unroll") for (int i = 0; i < kTPH; ++i) {                                            \
      const float acc = (pp[i][0] + pp[i][1]) + (pp[i][2] + pp[i][3]);                            \
      const float g = SSM_GATE_BLEND                                                              \
          ? __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, silu(zv[i])) & gmask) | (0x3f800000u & ~gmask)) \
          : (gated ? silu(zv[i]) : 1.0f);                                                         \
      lds_store_elem<TI>(ry, hw * kTPH + i, (acc + Dd * uv[i]) * g);                              \
    }                                                                                             \
  }
    // y tile of chunk CJ (LDS buffer TB) -> global, 16-byte pieces
#define SSM_STORE_Y(CJ, TB, TAIL)                                                                  \
  if (OUT && ydst && (!(TAIL) || (CJ) * kT + yq * EPP < len)) {                                    \
    const uint32_t* src = reinterpret_cast<const uint32_t*>(&sm.ytile[OUT ? (TB) : 0][yrow * ROWB + yq * 16]); \
    *reinterpret_cast<uint4*>(ydst + (CJ) * kT) = make_uint4(src[0], src[1], src[2], src[3]);       \
  }

    // ---------------- scanner stage ---------------------------------------------------------
    // step T, first part: Abar = exp(Delta*A) and Delta*u*B_t[n] (independent of h)
#define SSM_PRE(T)                                                                                \
  _Pragma("unroll") for (int jj = 0; jj < NPW; ++jj) {                                            \
    abv[(T) % SG][jj] = ex2(ddv[T].x * A2[jj]);                                                   \
    SSM_DPP_MUL(buv[(T) % SG][jj], bB[jj], ddv[T].y, T);                                          \
  }
    // step T, second part: the recurrence and the readout C_t . h_t
#define SSM_CHAIN(T)                                                                              \
  {                                                                                               \
    float p = 0.0f;                                                                               \
    _Pragma("unroll") for (int jj = 0; jj < NPW; ++jj) {                                          \
      h[jj] = __builtin_fmaf(abv[(T) % SG][jj], h[jj], buv[(T) % SG][jj]);                        \
      if (OUT) {                                                                                  \
        if (jj == 0) SSM_DPP_MUL(p, bC[jj], h[jj], T);                                            \
        else SSM_DPP_FMAC(p, bC[jj], h[jj], T);                                                   \
      }                                                                                           \
    }                                                                                             \
    if (OUT) pv[T] = p;                                                                           \
  }
#define SSM_PRE4(T0) SSM_PRE(T0) SSM_PRE(T0 + 1) SSM_PRE(T0 + 2) SSM_PRE(T0 + 3)
#define SSM_CHAIN4(T0) SSM_CHAIN(T0) SSM_CHAIN(T0 + 1) SSM_CHAIN(T0 + 2) SSM_CHAIN(T0 + 3)
    // scan chunk CJ (LDS buffer TB) over this scanner's states
#define SSM_SCAN(CJ, TB)                                                                          \
  {                                                                                               \
    float bB[NPW], bC[NPW];                                                                       \
    _Pragma("unroll") for (int jj = 0; jj < NPW; ++jj) {                                          \
      bB[jj] = sm.bc[(CJ) & 3][0][wv * NPW + jj][lt];                                             \
      bC[jj] = sm.bc[(CJ) & 3][1][wv * NPW + jj][lt];                                             \
    }                                                                                             \
    float2 ddv[kT];                                                                               \
    _Pragma("unroll") for (int t = 0; t < kT; ++t) ddv[t] = sm.dtdu[TB][t][lane];                 \
    float abv[SG][NPW], buv[SG][NPW], pv[OUT ? kT : 1];                                           \
    /* exps and products of a group of steps first, then that group's recurrence */               \
    if constexpr (SG == 16) {                                                                     \
      SSM_PRE4(0) SSM_PRE4(4) SSM_PRE4(8) SSM_PRE4(12)                                            \
      SSM_CHAIN4(0) SSM_CHAIN4(4) SSM_CHAIN4(8) SSM_CHAIN4(12)                                    \
    } else if constexpr (SG == 8) {                                                               \
      SSM_PRE4(0) SSM_PRE4(4) SSM_CHAIN4(0) SSM_CHAIN4(4)                                         \
      SSM_PRE4(8) SSM_PRE4(12) SSM_CHAIN4(8) SSM_CHAIN4(12)                                       \
    } else {                                                                                      \
      SSM_PRE4(0) SSM_CHAIN4(0) SSM_PRE4(4) SSM_CHAIN4(4)                                         \
      SSM_PRE4(8) SSM_CHAIN4(8) SSM_PRE4(12) SSM_CHAIN4(12)                                       \
    }                                                                                             \
    if (OUT) {                                                                                    \
      _Pragma("unroll") for (int t = 0; t < kT; ++t) sm.part[OUT ? (TB) : 0][wv][t][lane] = pv[t]; \
    }                                                                                             \
  }

    // ---------------- iterations ------------------------------------------------------------
    // Iteration J: helpers prefetch chunk J+2, store y(J-3), finalize(J-2), prep(J) and stage
    // chunk J+1 into LDS; scanners scan(J-1).  One workgroup barrier per iteration.  The two
    // roles run separate loops with the same barrier sequence, so their registers never
    // overlap.  Steady-state iterations (all stages active, full chunks) use compile-time LDS
    // buffer indices and no stage predicates.
    const int last_j = nch + (OUT ? 3 : 1);
    if (scanner) {
      __syncthreads();  // prologue
      int j = 0;
      for (; j < 3 && j < last_j; ++j) {
        if (j >= 1 && j <= nch) SSM_SCAN(j - 1, (j - 1) & 1)
        __syncthreads();
      }
      for (; j + 3 < nfull; j += 2) {
        SSM_SCAN(j - 1, 0)  // j odd: chunk j-1 is even
        __syncthreads();
        SSM_SCAN(j, 1)
        __syncthreads();
      }
      for (; j < last_j; ++j) {
        if (j >= 1 && j <= nch) SSM_SCAN(j - 1, (j - 1) & 1)
        __syncthreads();
      }
    } else {
    // Loads run SSM_PREFETCH iterations ahead: iteration J stages chunk J+1 (from register
    // slot (J+1) % 4) into LDS and issues the loads of chunk J+1+SSM_PREFETCH into another
    // slot, so up to SSM_PREFETCH chunks are in flight.  Iterations are unrolled by 4 so every
    // slot and LDS buffer index is a compile-time constant (S4 = J % 4).
#define SSM_HELPER_ITER(J, S4)                                                                    \
  {                                                                                               \
    if ((J) >= 3) SSM_STORE_Y((J) - 3, ((S4) + 1) & 1, true)                                      \
    if ((J) >= 2 && (J) <= nch + 1) SSM_FINALIZE((J) - 2, (S4) & 1, (S4) & 1)                     \
    if ((J) < nch) SSM_PREP(J, (S4) & 1, true, (S4) & 1)                                          \
    if ((J) + 1 < nch) SSM_STORE_TILE((J) + 1, 0, rs[((S4) + 1) % 4])                              \
    if ((J) + 1 + SSM_PREFETCH < nch) SSM_LOAD_CHUNK(rs[((S4) + 1 + SSM_PREFETCH) % 4], (J) + 1 + SSM_PREFETCH) \
    __syncthreads();                                                                              \
  }
#define SSM_HELPER_STEADY(J, S4)                                                                  \
  {                                                                                               \
    SSM_STORE_Y((J) - 3, ((S4) + 1) & 1, false)                                                   \
    SSM_FINALIZE((J) - 2, (S4) & 1, (S4) & 1)                                                     \
    SSM_PREP(J, (S4) & 1, false, (S4) & 1)                                                        \
    SSM_STORE_TILE((J) + 1, 0, rs[((S4) + 1) % 4])                                                \
    SSM_LOAD_CHUNK_FULL(rs[((S4) + 1 + SSM_PREFETCH) % 4], (J) + 1 + SSM_PREFETCH)                \
    __syncthreads();                                                                              \
  }
      if constexpr (kHelperPrio != 0) __builtin_amdgcn_s_setprio(kHelperPrio);
      // prologue: chunk 0 into LDS, chunks 1..SSM_PREFETCH in flight
      SSM_LOAD_CHUNK(rs[0], 0)
      _Pragma("unroll") for (int c = 1; c <= SSM_PREFETCH; ++c) {
        if (c < nch) SSM_LOAD_CHUNK(rs[c], c)
      }
      SSM_STORE_TILE(0, 0, rs[0])
      if constexpr (CONV) {
        // the 3 inputs before the unit's first step: from x, or (at step 0) from the state
        // the caller passes, oldest first, zeros where it has none
        if (htid < 3 * kW) {
          const int r = htid % kW, m = htid / kW;
          const int64_t pos = t_begin - 3 + m;
          float v = 0.0f;
          if (d0 + r < a.dim) {
            const int64_t row = (int64_t)b * a.dim + d0 + r;
            if (pos >= 0) v = ld<TI>((const TI*)a.u, row * L + pos);
            else if (a.cst && a.ck - 1 + pos >= 0) v = a.cst[row * (a.ck - 1) + (a.ck - 1 + pos)];
          }
          sm.xh[r][m] = v;
        }
      }
      __syncthreads();
      SSM_HELPER_ITER(0, 0)
      if (1 < last_j) SSM_HELPER_ITER(1, 1)
      if (2 < last_j) SSM_HELPER_ITER(2, 2)
      int j = 3;
      for (; j + 4 + SSM_PREFETCH < nfull; j += 4) {  // every chunk loaded here is full
        SSM_HELPER_STEADY(j, 3)
        SSM_HELPER_STEADY(j + 1, 0)
        SSM_HELPER_STEADY(j + 2, 1)
        SSM_HELPER_STEADY(j + 3, 2)
      }
      for (; j < last_j; j += 4) {
        SSM_HELPER_ITER(j, 3)
        if (j + 1 < last_j) SSM_HELPER_ITER(j + 1, 0)
        if (j + 2 < last_j) SSM_HELPER_ITER(j + 2, 1)
        if (j + 3 < last_j) SSM_HELPER_ITER(j + 3, 2)
      }
      if constexpr (kHelperPrio != 0) __builtin_amdgcn_s_setprio(0);
#undef SSM_HELPER_ITER
#undef SSM_HELPER_STEADY
    }
#undef SSM_LOAD_CHUNK
#undef SSM_LOAD_CHUNK_FULL
#undef SSM_STORE_TILE
#undef SSM_PREP
#undef SSM_FINALIZE
#undef SSM_STORE_Y
#undef SSM_PRE
#undef SSM_CHAIN
#undef SSM_PRE4
#undef SSM_CHAIN4
#undef SSM_SCAN

    // ---- unit end: hand the state on ----
    if constexpr (MODE == 2) {
      if (scanner && active) {
#pragma unroll
        for (int j2 = 0; j2 < NPW; ++j2) a.seg_h[((int64_t)k * a.batch * a.dim + ch) * N + wv * NPW + j2] = h[j2];
      }
      if (!scanner) sm.red[hw][lane] = sdt;
      __syncthreads();
      if (wv == kS && active) {
        float s2 = sm.red[0][lane];
        for (int w = 1; w < kH; ++w) s2 += sm.red[w][lane];
        a.seg_dt[(int64_t)k * a.batch * a.dim + ch] = s2;
      }
    } else if (MODE == 0 && hand_out) {
      // A head piece: store the state at the split point (device-scope atomics, coherent
      // across the XCDs' L2 caches without cache-wide write-back or invalidation), then set
      // the flags once the stores are acknowledged.
      if (scanner) {
        float* cp = a.carry + (int64_t)grp * N * kW;
#pragma unroll
        for (int j2 = 0; j2 < NPW; ++j2)
          __hip_atomic_store(cp + (wv * NPW + j2) * kW + lane, h[j2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (a.publish) SSM_PUBLISH(grp)
      }
    } else if (MODE == 0 || k == a.nseg - 1) {
      // the piece ends the chain: final state
      if (scanner && a.last_state && active) {
#pragma unroll
        for (int j2 = 0; j2 < NPW; ++j2) a.last_state[ch * N + wv * NPW + j2] = h[j2];
      }
    }
    if (MODE != 0) break;
  }
#undef SSM_PUBLISH
}

__global__ void zero_ints(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Segment carry: turn per-segment end states (from h = 0) into incoming states, in place:
// seg_h[s] <- state entering segment s.  A workgroup of kCW waves takes 64 consecutive (channel, n)
// pairs, one per lane (so every load is coalesced), and wave w walks segments [w P, (w+1) P).
// Each wave first folds its part from zero into (summed step, end state); the parts' folds meet
// in LDS, where each wave combines those before it into the state entering its part; then it
// walks its part again writing the incoming states.  The chain a lane walks is 2P segments long
// instead of nseg.  The last segment's aggregate is never written, and only read where unused.
constexpr int kCW = 16;
__global__ __launch_bounds__(kCW * 64) void carry_split_kernel(float* seg_h, const float* seg_dt, const float* A,
                                                               const float* h0, int64_t chans, int64_t dim, int N,
                                                               int nseg) {
  __shared__ float sD[kCW][64], sE[kCW][64];
  const int lane = threadIdx.x % 64, w = threadIdx.x / 64;
  const int64_t pairs = chans * N;
  const int64_t i0 = blockIdx.x * 64LL + lane;
  const bool ok = i0 < pairs;
  const int64_t i = ok ? i0 : pairs - 1;
  const int64_t chn = i / N;
  const int n = (int)(i % N);
  const float A2 = A[(chn % dim) * N + n] * kLog2e;
  const int P = (nseg + kCW - 1) / kCW;
  const int s0 = min(nseg, w * P), s1 = min(nseg, s0 + P);
  const int s1a = min(s1, nseg - 1);  // aggregates exist for segments 0 .. nseg-2
  constexpr int kB = 8;               // loads in flight per lane
  float e = 0.0f, dsum = 0.0f;
  for (int sb = s0; sb < s1a; sb += kB) {
    float agg[kB], sdt[kB];
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const int s = min(sb + k, s1a - 1);
      agg[k] = seg_h[(int64_t)s * pairs + i];
      sdt[k] = seg_dt[(int64_t)s * chans + chn];
    }
#pragma unroll
    for (int k = 0; k < kB; ++k)
      if (sb + k < s1a) {
        e = __builtin_fmaf(ex2(A2 * sdt[k]), e, agg[k]);
        dsum += sdt[k];
      }
  }
  sD[w][lane] = dsum;
  sE[w][lane] = e;
  __syncthreads();
  float h = h0 ? h0[i] : 0.0f;
  for (int v = 0; v < w; ++v) h = __builtin_fmaf(ex2(A2 * sD[v][lane]), h, sE[v][lane]);
  for (int sb = s0; sb < s1; sb += kB) {
    float agg[kB], sdt[kB];
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const int s = min(sb + k, s1a);  // the last segment reads its predecessor's entry (unused)
      agg[k] = seg_h[(int64_t)s * pairs + i];
      sdt[k] = seg_dt[(int64_t)s * chans + chn];
    }
#pragma unroll
    for (int k = 0; k < kB; ++k)
      if (sb + k < s1) {
        if (ok) seg_h[(int64_t)(sb + k) * pairs + i] = h;
        h = __builtin_fmaf(ex2(A2 * sdt[k]), h, agg[k]);
      }
  }
}

// Hand-over wait bound and flag publication for the launches that follow; changed only by the
// test hook ssm_test_handover_wait.
std::atomic<int> g_max_polls{1 << 26};
std::atomic<int> g_publish{1};

int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

}  // namespace chunked

// Launch shape of the chunked scan for a given problem and CU count.
//  * groups >= CUs: intervals (mode 0): one workgroup per interval of the chains laid end to
//    end, W = ceil(groups * chunks / CUs) chunks each (every workgroup gets the same work;
//    a chain is split at most once).
//  * CUs/2 <= groups < CUs: one pass per group (mode 1) -- splitting a chain cannot shorten
//    it when every chain already has a CU of its own.
//  * fewer groups (long sequences): aggregate / carry / output passes (mode 2) over enough
//    parallel segments to fill the GPU (SSM_SPLIT_UNITS_PER_CU per CU).
ScanPlan plan_scan(int64_t batch, int64_t dim, int64_t seqlen, int cus) {
  using namespace chunked;
  ScanPlan pl{};
  pl.groups = batch * ((dim + kW - 1) / kW);
  const int64_t nch_total = std::max<int64_t>(1, (seqlen + kT - 1) / kT);
  if (pl.groups >= cus) {
    const int64_t total = pl.groups * nch_total;
    const int64_t w = (total + cus - 1) / cus;
    pl.mode = 0;
    pl.units = (total + w - 1) / w;
    pl.nseg = pl.units;
    pl.seg_len = w * kT;
    return pl;
  }
  int64_t K = 1;
  if (2 * pl.groups < cus) {
    const int64_t target_units = (int64_t)SSM_SPLIT_UNITS_PER_CU * cus;
    K = std::max<int64_t>(1, std::min<int64_t>(nch_total, (target_units + pl.groups - 1) / pl.groups));
  }
  pl.seg_len = ((nch_total + K - 1) / K) * kT;
  pl.nseg = std::max<int64_t>(1, (seqlen + pl.seg_len - 1) / pl.seg_len);
  pl.mode = pl.nseg == 1 ? 1 : 2;
  pl.out_stride = 1;
  if (pl.mode == 2) {
    const int64_t out_target = (int64_t)SSM_SPLIT_OUT_PER_CU * cus;
    pl.out_stride = std::max<int64_t>(1, pl.nseg * pl.groups / std::max<int64_t>(1, out_target));
  }
  pl.units = ((pl.nseg + pl.out_stride - 1) / pl.out_stride) * pl.groups;
  return pl;
}

int device_cu_count() { return chunked::cu_count(); }

// Scratch of the chunked scan, from the same plan and formulas the launch below uses.
size_t chunked_scratch_bytes(const ScanParams& p, int cus) {
  using namespace chunked;
  const ScanPlan pl = plan_scan(p.batch, p.dim, p.seqlen, cus);
  const size_t N = (size_t)p.dstate;
  if (pl.mode == 0)
    return (size_t)pl.groups * N * kW * sizeof(float) + ((size_t)pl.groups * kS + 8) * sizeof(unsigned long long);
  if (pl.nseg > 1) return (size_t)pl.nseg * (size_t)(p.batch * p.dim) * (N + 1) * sizeof(float);
  return 0;
}

namespace chunked {

template <int N, typename TI, bool CONV>
hipError_t run(const ScanParams& p, hipStream_t stream) {
  Args a{};
  a.u = p.u; a.delta = p.delta; a.z = p.z; a.B = p.B; a.C = p.C; a.A = p.A; a.D = p.D; a.dt_bias = p.dt_bias;
  a.h0 = p.h0; a.y = p.y; a.last_state = p.last_state;
  a.batch = p.batch; a.dim = p.dim; a.L = p.seqlen; a.softplus = p.softplus;
  a.max_polls = g_max_polls.load();
  a.publish = g_publish.load();
  if constexpr (CONV) {  // p.u is x
    a.cw = p.cw; a.cb = p.cb; a.cst = p.cst; a.ck = (int)p.ck;
  }
  a.gpr = (int)((p.dim + kW - 1) / kW);
  const int cus = cu_count();
  const ScanPlan pl = plan_scan(p.batch, p.dim, p.seqlen, cus);
  a.groups = (int)pl.groups;
  a.seg_len = pl.seg_len;
  a.nseg = (int)pl.nseg;
  a.units = (int)pl.units;
  a.seg_stride = 1;
  const int64_t K = pl.nseg;
  const int64_t chans = p.batch * p.dim;
  hipError_t err = hipSuccess;
  void* scratch = nullptr;
  if (pl.mode == 0) {
    a.tch = (p.seqlen + kT - 1) / kT;
    a.wlen = pl.seg_len / kT;
    const size_t carry_bytes = (size_t)a.groups * N * kW * sizeof(float);
    // The ticket and the flags: the stream's persistent control block when there is one (no
    // clearing per call), else in this call's scratch behind the carry, cleared by a fill kernel
    // (under graph capture, and with a caller's workspace).
    const bool ctl = p.ws == nullptr && interval_ctl(stream, (int64_t)a.groups * kS, a.units, &a.ticket, &a.flags,
                                                     &a.tbase, &a.gen);
    const size_t bytes = carry_bytes + (ctl ? 0 : ((size_t)a.groups * kS + 8) * sizeof(unsigned long long));
    if ((err = scratch_acquire(p, &scratch, bytes, stream)) != hipSuccess) {
      if (ctl) interval_ctl_invalidate(stream);
      return err;
    }
    a.carry = (float*)scratch;
    if (!ctl) {
      a.ticket = (unsigned long long*)((char*)scratch + carry_bytes);
      a.flags = a.ticket + 8;
      a.tbase = 0;
      a.gen = 1;
      const int nints = (a.groups * kS + 8) * 2;
      hipLaunchKernelGGL(zero_ints, dim3((nints + 255) / 256), dim3(256), 0, stream, (int*)a.ticket, nints);
      err = hipGetLastError();
    }
    if (err == hipSuccess) {
      hipLaunchKernelGGL((scan_chunked_kernel<N, TI, 0, CONV>), dim3(a.units), dim3(threads<0, CONV, N>()), 0, stream, a);
      err = hipGetLastError();
    }
    if (err != hipSuccess && ctl) interval_ctl_invalidate(stream);
  } else if (K > 1) {
    const size_t bytes = (size_t)K * chans * (N + 1) * sizeof(float);
    if ((err = scratch_acquire(p, &scratch, bytes, stream)) != hipSuccess) return err;
    a.seg_h = (float*)scratch;
    a.seg_dt = a.seg_h + (size_t)K * chans * N;
    Args agg = a;
    agg.units = (int)((K - 1) * a.groups);  // the last segment's aggregate is never needed
    // the output pass: units of seg_stride consecutive segments, each from the carry at its start
    a.seg_stride = (int)pl.out_stride;
    a.seg_len = pl.seg_len * pl.out_stride;
    a.nseg = (int)((K + pl.out_stride - 1) / pl.out_stride);
    hipLaunchKernelGGL((scan_chunked_kernel<N, TI, 2, CONV>), dim3(agg.units), dim3(threads<2, CONV, N>()), 0, stream, agg);
    err = hipGetLastError();
    if (err == hipSuccess) {
      const int64_t pairs = chans * N;
      hipLaunchKernelGGL(carry_split_kernel, dim3((unsigned)((pairs + 63) / 64)), dim3(kCW * 64), 0, stream,
                         a.seg_h, a.seg_dt, p.A, p.h0, chans, p.dim, N, (int)K);
      err = hipGetLastError();
    }
    if (err == hipSuccess) {
      hipLaunchKernelGGL((scan_chunked_kernel<N, TI, 1, CONV>), dim3(a.units), dim3(threads<1, CONV, N>()), 0, stream, a);
      err = hipGetLastError();
    }
  } else {
    // one segment: a plain output pass from h0 / zeros
    a.nseg = 1;
    hipLaunchKernelGGL((scan_chunked_kernel<N, TI, 1, CONV>), dim3(a.units), dim3(threads<1, CONV, N>()), 0, stream, a);
    err = hipGetLastError();
  }
  if (scratch) {
    hipError_t ferr = scratch_release(p, scratch, stream);
    if (err == hipSuccess) err = ferr;
  }
  return err;
}

template <typename TI>
hipError_t dispatch_n(const ScanParams& p, hipStream_t s) {
  switch (p.dstate) {
    case 4: return run<4, TI, false>(p, s);
    case 8: return run<8, TI, false>(p, s);
    case 16: return run<16, TI, false>(p, s);
    case 32: return run<32, TI, false>(p, s);
    case 64: return run<64, TI, false>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace chunked

// Persistent interval control blocks, one per (device, stream): a 64-bit ticket counter that only
// grows and the hand-over flags, each holding the generation of the call that set it last.  A call
// takes tickets base .. base + units - 1 and sets its flags to its own generation, so nothing needs
// clearing between calls: the calls on one stream run in order, and the host counts the tickets and
// generations they use.  A block is cleared once, when made; one that is outgrown or whose launch
// failed is dropped but never freed (work queued before may still use it).
namespace {
struct IntervalCtl {
  unsigned long long* mem = nullptr;  // [ticket, 7 spare, flags ...]
  int64_t cap = 0;                    // flags held
  unsigned long long tickets = 0;     // tickets of the calls launched so far
  unsigned long long gen = 0;         // generation of the last call
};
std::mutex g_ctl_mutex;
std::map<std::pair<int, hipStream_t>, IntervalCtl> g_ctl;
}  // namespace

bool interval_ctl(hipStream_t s, int64_t nflags, int64_t units, unsigned long long** ticket,
                  unsigned long long** flags, unsigned long long* base, unsigned long long* gen) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess || st != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();
    return false;  // a captured launch would replay one generation: clear flags per call instead
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lk(g_ctl_mutex);
  IntervalCtl& c = g_ctl[{dev, s}];
  if (c.mem == nullptr || c.cap < nflags) {
    const int64_t cap = std::max<int64_t>(nflags, 4096);
    void* m = nullptr;
    if (hipMalloc(&m, (size_t)(cap + 8) * sizeof(unsigned long long)) != hipSuccess) {
      (void)hipGetLastError();
      c.mem = nullptr;
      return false;
    }
    const int nints = (int)((cap + 8) * 2);
    hipLaunchKernelGGL(chunked::zero_ints, dim3((nints + 255) / 256), dim3(256), 0, s, (int*)m, nints);
    if (hipGetLastError() != hipSuccess) {
      c.mem = nullptr;  // m is dropped: the fill may or may not have been queued
      return false;
    }
    c.mem = (unsigned long long*)m;
    c.cap = cap;
    c.tickets = 0;
    c.gen = 0;
  }
  *ticket = c.mem;
  *flags = c.mem + 8;
  *base = c.tickets;
  c.tickets += (unsigned long long)units;
  *gen = ++c.gen;
  return true;
}

void interval_ctl_release(hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  std::lock_guard<std::mutex> lk(g_ctl_mutex);
  auto it = g_ctl.find({dev, s});
  if (it == g_ctl.end()) return;
  if (it->second.mem) (void)hipFree(it->second.mem);  // the stream has drained (the caller synchronised it)
  g_ctl.erase(it);
}

void interval_ctl_invalidate(hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  std::lock_guard<std::mutex> lk(g_ctl_mutex);
  auto it = g_ctl.find({dev, s});
  if (it != g_ctl.end()) it->second.mem = nullptr;
}

hipError_t handover_failures(uint64_t* count, bool reset) {
  unsigned int v = 0;
  hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(chunked::handover_giveups), sizeof v, 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  *count = v;
  if (reset) {
    const unsigned int zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(chunked::handover_giveups), &zero, sizeof zero, 0, hipMemcpyHostToDevice);
  }
  return e;
}

void handover_wait(int* max_polls, int* publish) {
  *max_polls = chunked::g_max_polls.load();
  *publish = chunked::g_publish.load();
}
void set_handover_wait(int max_polls, int publish) {
  chunked::g_max_polls.store(max_polls > 0 ? max_polls : 1 << 26);
  chunked::g_publish.store(publish ? 1 : 0);
}

bool chunked_supported(const ScanParams& p) {
  const int es = p.dtype == kBF16 ? 2 : 4;
  auto al16 = [](const void* q) { return q == nullptr || ((uintptr_t)q % 16) == 0; };
  return p.dstate >= 4 && (p.seqlen * es) % 16 == 0 && p.seqlen < (1LL << 31) && p.dim < (1LL << 30) &&
         p.batch < (1LL << 30) && al16(p.u) && al16(p.delta) && al16(p.z) && al16(p.y) && al16(p.B) && al16(p.C);
}

// The fused convolution runs for fp32 rows.  For bf16 rows the convolution kernel followed by the
// scan measured faster on every shape tried (2.8B-shaped layer 221 against 239 us; 8 x 1536 x 2048
// even; 2 x 2048 x 4096 170 against 179 us; 1024 channels x 2^17 steps 1056 against 1067 us),
// while for fp32 rows the fused kernels were (260 against 276 us; 2^18 steps 629 against 635 us).
bool chunked_conv_supported(const ScanParams& p) {
  return p.dstate == 16 && p.dtype != kBF16 && chunked_supported(p);
}

hipError_t launch_scan_chunked(const ScanParams& p, hipStream_t stream) {
  if (p.cw) {  // fused convolution: dstate 16, fp32 rows (the others take the convolution kernel, then the scan)
    if (!chunked_conv_supported(p)) return hipErrorInvalidValue;
    return chunked::run<16, float, true>(p, stream);
  }
  return p.dtype == kBF16 ? chunked::dispatch_n<__bf16>(p, stream) : chunked::dispatch_n<float>(p, stream);
}

}  // namespace ssm
