// scan_chunked.hip -- the main forward selective-scan kernel for gfx950.
//
// Why this shape.  At dstate = 16 the scan costs ~110 VALU issue slots per
// element (16 exps at half rate plus 4 FMA-class ops per state, softplus and
// SiLU) against ~8 bytes of HBM traffic, so on MI355X it is bound by the
// vector ALUs, not by HBM.  The design therefore spends no VALU work that the
// plain recurrence does not need, and finds parallelism without recomputation:
//
//  * Workgroup = 64 consecutive channels (b, d0..d0+63) x G waves.  Wave g owns
//    states n in [g*N/G, (g+1)*N/G) of all 64 channels, one channel per lane.
//    B_t[n] and C_t[n] are then uniform across the wave and live in SGPRs
//    (scalar loads straight from global memory), so they cost no VALU or LDS
//    bandwidth.  The readout sum over n is split across waves and combined
//    through LDS.
//  * Per element work that does not depend on n (softplus of the step, Delta*u,
//    D*u, SiLU(z), the partial-sum reduction, the bf16 conversions) is done once,
//    spread over all G waves by time step ("prep" and "finalize").
//  * The sequence is processed in chunks of kT steps through a three-stage
//    pipeline -- prep(j+1) | scan(j) | finalize(j-1) -- with one workgroup
//    barrier per chunk.  Waves 0..G/2-1 run the scan stage first and waves
//    G/2..G-1 last, so the two waves sharing a SIMD overlap VALU-heavy and
//    LDS-heavy stages.  u, delta, z are fetched with 16-byte coalesced loads two
//    chunks ahead and staged through LDS; y leaves through an LDS tile as
//    16-byte coalesced stores.  Only y and the final state are written to HBM
//    (fusion with on-chip intermediates: Mamba summary (junchaoiu.github.io),
//    方法 step 2; tech.kj168168.com essay §二.3).
//
// Sequence parallelism (chunked two-level scan: "Mamba close reading"
// (jsqmd.com) §2.2 and the sketch of §7; mlqm.cn tutorial §6).  The sequence is
// cut into K segments; work unit (k, group) scans segment k of a channel group.
//  MODE 0 (chained): persistent workgroups take units in order from an atomic
//    ticket; unit (k, grp) starts from the end state of unit (k-1, grp), handed
//    over through global memory with a release/acquire flag.  Units are ordered
//    k-major, so a unit's predecessor was taken at least `groups` tickets
//    earlier and has normally finished: no recomputation, full sequential
//    exactness of the carry.  Used when there are enough channel groups to
//    occupy the GPU.  The hand-over uses device-scope atomic loads and stores
//    only (no agent-scope fences: on this multi-XCD part those write back or
//    invalidate whole L2 caches).
//  MODE 1 (output) with K = 1: one segment per group, no carry at all.
//  MODE 2 (aggregate) + carry kernel + MODE 1 (output): for few channel groups
//    (very long sequences).  Every segment but the last first computes its end
//    state from h = 0 and its sum of Delta (the segment's transition is
//    exp(A * sum Delta)); a carry kernel turns these into incoming states; the
//    output pass reruns each segment from its incoming state.
//
// Deadlock freedom of MODE 0: a unit waits only on a unit with a smaller
// ticket, which was taken by a workgroup that is already running; the oldest
// unfinished unit never waits.  The wait is additionally bounded (it gives up
// after ~2^26 polls), so every wave always reaches the exit.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {
namespace chunked {

#ifndef SSM_CHAINED_UNITS_PER_CU
#define SSM_CHAINED_UNITS_PER_CU 8
#endif
#ifndef SSM_SPLIT_UNITS_PER_CU
#define SSM_SPLIT_UNITS_PER_CU 4
#endif

constexpr int kT = 16;  // time steps per chunk
constexpr int kW = 64;  // channels per group = lanes per wave


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
  float* carry;   // MODE 0:   [groups, N, 64]
  int* flags;     // MODE 0:   [units]
  int* ticket;    // MODE 0:   1 counter
  int64_t batch, dim, L, seg_len;
  int gpr;     // channel groups per batch row
  int groups;  // batch * gpr
  int nseg;    // K
  int units;   // K * groups
  int softplus;
};

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

// LDS of one workgroup.
template <int N, int G, typename TI, bool OUT>
struct Smem {
  static constexpr int ROWB = kT * sizeof(TI) + 4;  // padded row stride (bytes): conflict-free column access
  unsigned char tile[2][3][kW * ROWB];               // u, delta, z of one chunk, [channel][t]
  float2 dtdu[2][kT][kW];                            // (Delta, Delta*u), [t][channel]
  float part[OUT ? 2 : 1][OUT ? G : 1][kT][kW];      // per-wave partial readouts
  unsigned char ytile[OUT ? 2 : 1][kW * ROWB];       // y of one chunk, [channel][t]
  float bc[3][2][N][kT];                             // B, C of a chunk in fp32 (3-deep ring)
  float red[G][kW];
  int unit;
};

// B_t[n] and C_t[n] are uniform across a wave.  For each chunk of kT = 16 steps
// a wave holds them in VGPRs, lane l carrying step (l mod 16) -- every 16-lane
// row holds the same 16 values -- and the consuming VALU instruction reads
// "lane t of my row" through the DPP row_newbcast source modifier.  The
// broadcast is free (part of the multiply / FMA) and needs no scalar registers.
// The loader threads stage each chunk's B and C rows into LDS as fp32 and every
// wave reads its vectors with one LDS load each, so a DPP source register is
// only ever written by an LDS load, never by a VALU instruction (a VALU write
// followed within two instructions by a DPP read of the same register is a
// hazard the compiler does not see through inline assembly).
#define SSM_DPP_MUL(dst, bc, other, T) \
  asm("v_mul_f32_dpp %0, %1, %2 row_newbcast:" #T " row_mask:0xf bank_mask:0xf" : "=v"(dst) : "v"(bc), "v"(other))
#define SSM_DPP_FMAC(acc, bc, other, T) \
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:" #T " row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(bc), "v"(other))

// Every 16-byte piece of u, delta, z, y and every 16-step group of B and C is
// either entirely before the end of the unit or entirely after it: the fast
// path requires seqlen to be a multiple of the piece length, and segments are
// multiples of kT.  So tails need only whole-piece predicates.
template <int N, int G, typename TI, int MODE>
__global__ __launch_bounds__(kW* G) void scan_chunked_kernel(const Args a) {
  constexpr int NPW = N / G;         // states per wave
  constexpr int ES = sizeof(TI);     // I/O element bytes
  constexpr int EPP = 16 / ES;       // elements per 16-byte piece
  constexpr int PPR = kT / EPP;      // pieces per tile row
  constexpr int NTHR = kW * G;
  constexpr int XPIECES = 3 * kW * PPR;          // u, delta, z tiles of one chunk
  constexpr int PIECES = XPIECES + 2 * N * PPR;  // ... and the B, C rows of the chunk
  constexpr int LPT = (PIECES + NTHR - 1) / NTHR;
  constexpr int TPG = kT / G;  // prep / finalize steps per thread
  constexpr bool OUT = MODE != 2;
  constexpr int ROWB = Smem<N, G, TI, OUT>::ROWB;
  static_assert(kT == 16, "the DPP broadcast addresses the 16 lanes of a row");
  static_assert(kT % G == 0 && N % G == 0, "bad split");
  static_assert(kW * PPR <= NTHR, "one y piece per thread");

  __shared__ Smem<N, G, TI, OUT> sm;

  const int tid = threadIdx.x;
  const int g = __builtin_amdgcn_readfirstlane(tid / kW);  // wave index (uniform)
  const int lane = tid % kW;
  const int lt = lane & (kT - 1);  // the step this lane carries in the B/C vectors

  for (int iter = 0;; ++iter) {
    int unit;
    if (MODE == 0) {
      if (tid == 0) sm.unit = atomicAdd(a.ticket, 1);
      __syncthreads();
      unit = __builtin_amdgcn_readfirstlane(sm.unit);
    } else {
      unit = iter == 0 ? (int)blockIdx.x : a.units;
    }
    if (unit >= a.units) break;
    const int k = unit / a.groups;
    const int grp = unit - k * a.groups;
    const int b = grp / a.gpr;
    const int d0 = (grp - b * a.gpr) * kW;
    const int64_t L = a.L;
    const int64_t t_begin = (int64_t)k * a.seg_len;
    const int len = (int)((t_begin + a.seg_len < L ? a.seg_len : L - t_begin));  // steps in this unit
    const int nch = (len + kT - 1) / kT;

    // this lane's channel (scan, prep and finalize all use channel d0 + lane)
    const int c = d0 + lane;
    const bool active = c < a.dim;
    const int cc = active ? c : (int)a.dim - 1;
    const int64_t ch = (int64_t)b * a.dim + cc;
    const float bias = a.dt_bias ? a.dt_bias[cc] : 0.0f;
    const float Dd = a.D ? a.D[cc] : 0.0f;
    const bool gated = a.z != nullptr;
    const bool sp = a.softplus != 0;
    float A2[NPW], h[NPW];
#pragma unroll
    for (int j = 0; j < NPW; ++j) A2[j] = a.A[(int64_t)cc * N + g * NPW + j] * kLog2e;

    // per-thread global pointers of this unit: loader pieces, the y piece, B/C elements
    const TI* lsrc[LPT];
    int lstep[LPT];  // first step (relative to t_begin) of each loader piece within a chunk
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int p = tid + i * NTHR;
      const int q = p % PPR;
      const TI* src = nullptr;
      if (p < XPIECES) {
        const int tensor = p / (kW * PPR), row = (p / PPR) % kW;
        const TI* base = tensor == 0 ? (const TI*)a.u : tensor == 1 ? (const TI*)a.delta : (const TI*)a.z;
        if (base && d0 + row < a.dim) src = base + ((int64_t)b * a.dim + d0 + row) * L + t_begin + q * EPP;
      } else if (p < PIECES) {
        const int pp = p - XPIECES, tensor = pp / (N * PPR), n = (pp / PPR) % N;
        src = (tensor == 0 ? (const TI*)a.B : (const TI*)a.C) + ((int64_t)b * N + n) * L + t_begin + q * EPP;
      }
      lsrc[i] = src;
      lstep[i] = q * EPP;
    }
    const int yrow = tid / PPR, yq = tid % PPR;
    TI* ydst = (OUT && tid < kW * PPR && d0 + yrow < a.dim)
                   ? (TI*)a.y + ((int64_t)b * a.dim + d0 + yrow) * L + t_begin + yq * EPP
                   : nullptr;

    // ---- incoming state -------------------------------------------------
    if (MODE == 0 && k > 0) {
      // Hand-over protocol (see the writer at the unit end): flag and state are
      // device-scope atomics, coherent across the XCDs' L2 caches without any
      // cache-wide write-back or invalidation; the state loads are issued only
      // after the flag has been observed (thread 0) and a workgroup barrier.
      if (tid == 0) {
        const int* f = a.flags + (unit - a.groups);
        for (int spin = 0; __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0; ++spin) {
          if (spin > (1 << 26)) break;  // bounded: never hang (only a broken launch could get here)
          __builtin_amdgcn_s_sleep(1);
        }
      }
      __syncthreads();
      const float* cp = a.carry + (int64_t)grp * N * kW;
#pragma unroll
      for (int j = 0; j < NPW; ++j)
        h[j] = __hip_atomic_load(cp + (g * NPW + j) * kW + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (MODE == 1 && a.seg_h) {
#pragma unroll
      for (int j = 0; j < NPW; ++j) h[j] = a.seg_h[((int64_t)k * a.batch * a.dim + ch) * N + g * NPW + j];
    } else if (MODE != 2 && k == 0 && a.h0) {
#pragma unroll
      for (int j = 0; j < NPW; ++j) h[j] = a.h0[ch * N + g * NPW + j];
    } else {
#pragma unroll
      for (int j = 0; j < NPW; ++j) h[j] = 0.0f;
    }

    float sdt = 0.0f;
    float dsk[3][TPG], gat[3][TPG];  // D*u and silu(z) of chunks j-2, j-1, j (this thread's steps)
    uint4 rs[2][LPT];                // u/delta/z/B/C pieces of chunks in flight (chunk c in rs[c & 1])
    // unconditional-load pointers for full chunks: an unused piece reads a harmless valid address
    const TI* lsrc_f[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) lsrc_f[i] = lsrc[i] ? lsrc[i] : (const TI*)a.u + t_begin + lstep[i];

    // ---------------- pipeline stages (TB: LDS double-buffer index of the chunk) --------------
    // global -> registers: 16-byte pieces of chunk CJ (zero past the end)
#define SSM_LOAD_CHUNK(R, CJ)                                                                       \
  _Pragma("unroll") for (int i = 0; i < LPT; ++i) {                                                 \
    const int st0 = (CJ) * kT + lstep[i];                                                           \
    R[i] = (lsrc[i] && st0 < len) ? *reinterpret_cast<const uint4*>(lsrc[i] + (CJ) * kT)           \
                                  : make_uint4(0, 0, 0, 0);                                         \
  }
    // same for a chunk known to be full: no predicates
#define SSM_LOAD_CHUNK_FULL(R, CJ)                                                                  \
  _Pragma("unroll") for (int i = 0; i < LPT; ++i) R[i] = *reinterpret_cast<const uint4*>(lsrc_f[i] + (CJ) * kT);
    // registers -> LDS: the u/delta/z tile of chunk CJ, and its B/C rows as fp32
#define SSM_STORE_TILE(CJ, TB, R)                                                                    \
  _Pragma("unroll") for (int i = 0; i < LPT; ++i) {                                                  \
    const int p = tid + i * NTHR;                                                                    \
    const int q = p % PPR;                                                                           \
    if (p < XPIECES) {                                                                               \
      const int tensor = p / (kW * PPR), row = (p / PPR) % kW;                                       \
      uint32_t* dst = reinterpret_cast<uint32_t*>(&sm.tile[TB][tensor][row * ROWB + q * 16]);       \
      dst[0] = R[i].x; dst[1] = R[i].y; dst[2] = R[i].z; dst[3] = R[i].w;                            \
    } else if (p < PIECES) {                                                                         \
      const int pp = p - XPIECES, tensor = pp / (N * PPR), n = (pp / PPR) % N;                       \
      float* dst = &sm.bc[(CJ) % 3][tensor][n][q * EPP];                                             \
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
#define SSM_PREP(J, TB, TAIL)                                                                     \
  {                                                                                               \
    const unsigned char* ru = &sm.tile[TB][0][lane * ROWB];                                       \
    const unsigned char* rd = &sm.tile[TB][1][lane * ROWB];                                       \
    const unsigned char* rz = &sm.tile[TB][2][lane * ROWB];                                       \
    float xv[TPG], uv[TPG], zv[TPG];                                                              \
    _Pragma("unroll") for (int i = 0; i < TPG; ++i) {                                             \
      xv[i] = lds_elem<TI>(rd, g * TPG + i);                                                      \
      uv[i] = lds_elem<TI>(ru, g * TPG + i);                                                      \
      zv[i] = lds_elem<TI>(rz, g * TPG + i);                                                      \
    }                                                                                             \
    _Pragma("unroll") for (int i = 0; i < TPG; ++i) {                                             \
      const int tl = g * TPG + i;                                                                 \
      const float x = xv[i] + bias;                                                               \
      float dt = sp ? softplus(x) : x;                                                            \
      if (TAIL && (J) * kT + tl >= len) dt = 0.0f;                                                \
      sm.dtdu[TB][tl][lane] = make_float2(dt, dt * uv[i]);                                        \
      if (MODE == 2) sdt += dt;                                                                   \
      if (OUT) {                                                                                  \
        dsk[2][i] = Dd * uv[i];                                                                   \
        gat[2][i] = gated ? silu(zv[i]) : 1.0f;                                                   \
      }                                                                                           \
    }                                                                                             \
  }
    // finalize chunk J: sum the G partial readouts, add D*u, gate, round into the y tile
#define SSM_FINALIZE(TB)                                                                          \
  if (OUT) {                                                                                      \
    unsigned char* ry = &sm.ytile[OUT ? (TB) : 0][lane * ROWB];                                   \
    float pp[TPG][G];                                                                             \
    _Pragma("unroll") for (int i = 0; i < TPG; ++i)                                               \
      _Pragma("unroll") for (int w = 0; w < G; ++w) pp[i][w] = sm.part[OUT ? (TB) : 0][w][g * TPG + i][lane]; \
    _Pragma("unroll") for (int i = 0; i < TPG; ++i) {                                             \
      float acc = pp[i][0];                                                                       \
      _Pragma("unroll") for (int w = 1; w < G; ++w) acc += pp[i][w];                              \
      lds_store_elem<TI>(ry, g * TPG + i, (acc + dsk[0][i]) * gat[0][i]);                         \
    }                                                                                             \
  }
    // scan, first part: for step T, Abar = exp(Delta*A) and Delta*u*B_t[n] (independent of h)
#define SSM_PRE(T)                                                                                \
  _Pragma("unroll") for (int jj = 0; jj < NPW; ++jj) {                                            \
    abv[T][jj] = ex2(ddv[T].x * A2[jj]);                                                          \
    SSM_DPP_MUL(buv[T][jj], bB[jj], ddv[T].y, T);                                                 \
  }
    // scan, second part: the recurrence and the readout C_t . h_t of step T
#define SSM_CHAIN(T)                                                                              \
  {                                                                                               \
    float p = 0.0f;                                                                               \
    _Pragma("unroll") for (int jj = 0; jj < NPW; ++jj) {                                          \
      h[jj] = __builtin_fmaf(abv[T][jj], h[jj], buv[T][jj]);                                      \
      if (OUT) {                                                                                  \
        if (jj == 0) SSM_DPP_MUL(p, bC[jj], h[jj], T);                                            \
        else SSM_DPP_FMAC(p, bC[jj], h[jj], T);                                                   \
      }                                                                                           \
    }                                                                                             \
    if (OUT) pv[T] = p;                                                                           \
  }
    // scan chunk CJ (LDS buffer TB) over this wave's states
#define SSM_SCAN(CJ, TB)                                                                          \
  {                                                                                               \
    float bB[NPW], bC[NPW];                                                                       \
    _Pragma("unroll") for (int jj = 0; jj < NPW; ++jj) {                                          \
      bB[jj] = sm.bc[(CJ) % 3][0][g * NPW + jj][lt];                                              \
      bC[jj] = sm.bc[(CJ) % 3][1][g * NPW + jj][lt];                                              \
    }                                                                                             \
    float2 ddv[kT];                                                                               \
    _Pragma("unroll") for (int t = 0; t < kT; ++t) ddv[t] = sm.dtdu[TB][t][lane];                 \
    float abv[kT][NPW], buv[kT][NPW], pv[OUT ? kT : 1];                                           \
    /* exps and products of a group of steps first, then that group's recurrence; the group */    \
    /* shrinks with the states per wave so that the registers stay bounded                   */    \
    if constexpr (NPW <= 2) {                                                                     \
      SSM_PRE(0) SSM_PRE(1) SSM_PRE(2) SSM_PRE(3) SSM_PRE(4) SSM_PRE(5) SSM_PRE(6) SSM_PRE(7)      \
      SSM_PRE(8) SSM_PRE(9) SSM_PRE(10) SSM_PRE(11) SSM_PRE(12) SSM_PRE(13) SSM_PRE(14) SSM_PRE(15) \
      SSM_CHAIN(0) SSM_CHAIN(1) SSM_CHAIN(2) SSM_CHAIN(3) SSM_CHAIN(4) SSM_CHAIN(5) SSM_CHAIN(6)   \
      SSM_CHAIN(7) SSM_CHAIN(8) SSM_CHAIN(9) SSM_CHAIN(10) SSM_CHAIN(11) SSM_CHAIN(12)            \
      SSM_CHAIN(13) SSM_CHAIN(14) SSM_CHAIN(15)                                                   \
    } else if constexpr (NPW <= 4) {                                                              \
      SSM_PRE(0) SSM_PRE(1) SSM_PRE(2) SSM_PRE(3) SSM_PRE(4) SSM_PRE(5) SSM_PRE(6) SSM_PRE(7)      \
      SSM_CHAIN(0) SSM_CHAIN(1) SSM_CHAIN(2) SSM_CHAIN(3) SSM_CHAIN(4) SSM_CHAIN(5) SSM_CHAIN(6)   \
      SSM_CHAIN(7)                                                                                \
      SSM_PRE(8) SSM_PRE(9) SSM_PRE(10) SSM_PRE(11) SSM_PRE(12) SSM_PRE(13) SSM_PRE(14) SSM_PRE(15) \
      SSM_CHAIN(8) SSM_CHAIN(9) SSM_CHAIN(10) SSM_CHAIN(11) SSM_CHAIN(12) SSM_CHAIN(13)           \
      SSM_CHAIN(14) SSM_CHAIN(15)                                                                 \
    } else {                                                                                      \
      SSM_PRE(0) SSM_PRE(1) SSM_PRE(2) SSM_PRE(3) SSM_CHAIN(0) SSM_CHAIN(1) SSM_CHAIN(2) SSM_CHAIN(3) \
      SSM_PRE(4) SSM_PRE(5) SSM_PRE(6) SSM_PRE(7) SSM_CHAIN(4) SSM_CHAIN(5) SSM_CHAIN(6) SSM_CHAIN(7) \
      SSM_PRE(8) SSM_PRE(9) SSM_PRE(10) SSM_PRE(11) SSM_CHAIN(8) SSM_CHAIN(9) SSM_CHAIN(10)       \
      SSM_CHAIN(11)                                                                               \
      SSM_PRE(12) SSM_PRE(13) SSM_PRE(14) SSM_PRE(15) SSM_CHAIN(12) SSM_CHAIN(13) SSM_CHAIN(14)   \
      SSM_CHAIN(15)                                                                               \
    }                                                                                             \
    if (OUT) {                                                                                    \
      _Pragma("unroll") for (int t = 0; t < kT; ++t) sm.part[OUT ? (TB) : 0][g][t][lane] = pv[t]; \
    }                                                                                             \
  }
    // y tile of chunk CJ (LDS buffer TB) -> global, 16-byte pieces
#define SSM_STORE_Y(CJ, TB, TAIL)                                                                  \
  if (OUT && ydst && (!(TAIL) || (CJ) * kT + yq * EPP < len)) {                                    \
    const uint32_t* src = reinterpret_cast<const uint32_t*>(&sm.ytile[OUT ? (TB) : 0][yrow * ROWB + yq * 16]); \
    *reinterpret_cast<uint4*>(ydst + (CJ) * kT) = make_uint4(src[0], src[1], src[2], src[3]);       \
  }
#define SSM_ROTATE                                                                                \
  _Pragma("unroll") for (int i = 0; i < TPG; ++i) {                                               \
    dsk[0][i] = dsk[1][i]; dsk[1][i] = dsk[2][i];                                                 \
    gat[0][i] = gat[1][i]; gat[1][i] = gat[2][i];                                                 \
  }
    // general iteration J (register parity PP = J & 1): every stage checks its range
#define SSM_ITER(J, PP)                                                                           \
  {                                                                                               \
    SSM_LOAD_CHUNK(rs[PP], (J) + 2)                                                               \
    if ((J) >= 3) SSM_STORE_Y((J) - 3, ((J) - 3) & 1, true)                                       \
    if ((J) < nch) SSM_PREP(J, (J) & 1, true)                                                     \
    if ((J) >= 1 && (J) <= nch) SSM_SCAN((J) - 1, ((J) - 1) & 1)                                  \
    if ((J) >= 2 && (J) <= nch + 1) SSM_FINALIZE(((J) - 2) & 1)                                   \
    if ((J) + 1 < nch) SSM_STORE_TILE((J) + 1, ((J) + 1) & 1, rs[1 - (PP)])                       \
    __syncthreads();                                                                              \
    SSM_ROTATE                                                                                    \
  }
    // steady-state iteration: all stages active, all chunks full, compile-time buffers; prep,
    // scan and finalize form one straight-line block the compiler can interleave
#define SSM_ITER_STEADY(J, PP)                                                                    \
  {                                                                                               \
    SSM_LOAD_CHUNK_FULL(rs[PP], (J) + 2)                                                          \
    SSM_STORE_Y((J) - 3, 1 - (PP), false)                                                         \
    SSM_PREP(J, PP, false)                                                                        \
    SSM_SCAN((J) - 1, 1 - (PP))                                                                   \
    SSM_FINALIZE(PP)                                                                              \
    SSM_STORE_TILE((J) + 1, 1 - (PP), rs[1 - (PP)])                                               \
    __syncthreads();                                                                              \
    SSM_ROTATE                                                                                    \
  }

    // prologue: chunk 0 into LDS, chunk 1 into registers
    SSM_LOAD_CHUNK(rs[0], 0)
    SSM_LOAD_CHUNK(rs[1], 1)
    SSM_STORE_TILE(0, 0, rs[0])
    __syncthreads();

    const int last_j = nch + (OUT ? 3 : 1);
    SSM_ITER(0, 0)
    if (1 < last_j) SSM_ITER(1, 1)
    if (2 < last_j) SSM_ITER(2, 0)
    int j = 3;
    const int nfull = len / kT;
    for (; j + 3 < nfull; j += 2) {
      SSM_ITER_STEADY(j, 1)
      SSM_ITER_STEADY(j + 1, 0)
    }
    for (; j < last_j; j += 2) {
      SSM_ITER(j, 1)
      if (j + 1 < last_j) SSM_ITER(j + 1, 0)
    }
#undef SSM_LOAD_CHUNK
#undef SSM_LOAD_CHUNK_FULL
#undef SSM_STORE_TILE
#undef SSM_PREP
#undef SSM_FINALIZE
#undef SSM_PRE
#undef SSM_CHAIN
#undef SSM_SCAN
#undef SSM_STORE_Y
#undef SSM_ROTATE
#undef SSM_ITER
#undef SSM_ITER_STEADY

    // ---- unit end: hand the state on ----
    if (MODE == 2) {
      if (active) {
#pragma unroll
        for (int j = 0; j < NPW; ++j) a.seg_h[((int64_t)k * a.batch * a.dim + ch) * N + g * NPW + j] = h[j];
      }
      sm.red[g][lane] = sdt;
      __syncthreads();
      if (g == 0 && active) {
        float s2 = sm.red[0][lane];
        for (int w = 1; w < G; ++w) s2 += sm.red[w][lane];
        a.seg_dt[(int64_t)k * a.batch * a.dim + ch] = s2;
      }
    } else {
      if (k == a.nseg - 1) {
        if (a.last_state && active) {
#pragma unroll
          for (int j = 0; j < NPW; ++j) a.last_state[ch * N + g * NPW + j] = h[j];
        }
      } else if (MODE == 0) {
        // Publish the end state: device-scope stores, then wait until every one of
        // them is acknowledged (s_waitcnt 0: all counters drained) before the
        // barrier, so the flag -- stored after the barrier -- can only become
        // visible after the state.  The signal fences keep the compiler from
        // moving the stores across the wait.
        float* cp = a.carry + (int64_t)grp * N * kW;
#pragma unroll
        for (int j = 0; j < NPW; ++j)
          __hip_atomic_store(cp + (g * NPW + j) * kW + lane, h[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __syncthreads();
        if (tid == 0) __hip_atomic_store(a.flags + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (MODE != 0) break;
  }
}

__global__ void zero_ints(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// One thread per (channel, n): turn per-segment end states (from h = 0) into
// incoming states, in place: seg_h[s] <- state entering segment s.
__global__ __launch_bounds__(256) void carry_kernel(float* seg_h, const float* seg_dt, const float* A,
                                                    const float* h0, int64_t chans, int64_t dim, int N, int nseg) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= chans * N) return;
  const int64_t chn = i / N;
  const int n = (int)(i % N);
  const float A2 = A[(chn % dim) * N + n] * kLog2e;
  float h = h0 ? h0[i] : 0.0f;
  for (int s = 0; s < nseg; ++s) {
    const int64_t kk = (int64_t)s * chans * N + i;
    const float agg = seg_h[kk];
    seg_h[kk] = h;
    h = __builtin_fmaf(ex2(A2 * seg_dt[(int64_t)s * chans + chn]), h, agg);
  }
}

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

template <int N, typename TI>
hipError_t run(const ScanParams& p, hipStream_t stream) {
  constexpr int G = N >= 8 ? 8 : N;
  Args a{};
  a.u = p.u; a.delta = p.delta; a.z = p.z; a.B = p.B; a.C = p.C; a.A = p.A; a.D = p.D; a.dt_bias = p.dt_bias;
  a.h0 = p.h0; a.y = p.y; a.last_state = p.last_state;
  a.batch = p.batch; a.dim = p.dim; a.L = p.seqlen; a.softplus = p.softplus;
  a.gpr = (int)((p.dim + kW - 1) / kW);
  a.groups = (int)(p.batch * a.gpr);
  const int64_t nch_total = (p.seqlen + kT - 1) / kT;
  const int cus = cu_count();
  const bool chained = a.groups >= cus / 2;
  // work units per CU: chained -> enough units for balance, few enough that the per-unit
  // pipeline fill and drain stay small; two-pass -> enough parallel segments to fill the GPU
  const int64_t target_units = chained ? (int64_t)SSM_CHAINED_UNITS_PER_CU * cus : (int64_t)SSM_SPLIT_UNITS_PER_CU * cus;
  int64_t K = std::max<int64_t>(1, std::min<int64_t>(nch_total, (target_units + a.groups - 1) / a.groups));
  int64_t seg_chunks = (nch_total + K - 1) / K;
  a.seg_len = seg_chunks * kT;
  K = (p.seqlen + a.seg_len - 1) / a.seg_len;
  a.nseg = (int)K;
  a.units = (int)(K * a.groups);
  const int64_t chans = p.batch * p.dim;
  hipError_t err = hipSuccess;
  void* scratch = nullptr;
  if (chained && K > 1) {
    const size_t carry_bytes = (size_t)a.groups * N * kW * sizeof(float);
    const size_t bytes = carry_bytes + (size_t)(a.units + 64) * sizeof(int);
    if ((err = hipMallocAsync(&scratch, bytes, stream)) != hipSuccess) return err;
    a.carry = (float*)scratch;
    a.ticket = (int*)((char*)scratch + carry_bytes);
    a.flags = a.ticket + 64;
    const int nints = a.units + 64;
    hipLaunchKernelGGL(zero_ints, dim3((nints + 255) / 256), dim3(256), 0, stream, a.ticket, nints);
    err = hipGetLastError();
    if (err == hipSuccess) {
      const int grid = std::min(a.units, cus);
      hipLaunchKernelGGL((scan_chunked_kernel<N, G, TI, 0>), dim3(grid), dim3(kW * G), 0, stream, a);
      err = hipGetLastError();
    }
  } else if (K > 1) {
    const size_t bytes = (size_t)K * chans * (N + 1) * sizeof(float);
    if ((err = hipMallocAsync(&scratch, bytes, stream)) != hipSuccess) return err;
    a.seg_h = (float*)scratch;
    a.seg_dt = a.seg_h + (size_t)K * chans * N;
    Args agg = a;
    agg.units = (int)((K - 1) * a.groups);  // the last segment's aggregate is never needed
    hipLaunchKernelGGL((scan_chunked_kernel<N, G, TI, 2>), dim3(agg.units), dim3(kW * G), 0, stream, agg);
    err = hipGetLastError();
    if (err == hipSuccess) {
      const int64_t threads = chans * N;
      hipLaunchKernelGGL(carry_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a.seg_h,
                         a.seg_dt, p.A, p.h0, chans, p.dim, N, (int)K);
      err = hipGetLastError();
    }
    if (err == hipSuccess) {
      hipLaunchKernelGGL((scan_chunked_kernel<N, G, TI, 1>), dim3(a.units), dim3(kW * G), 0, stream, a);
      err = hipGetLastError();
    }
  } else {
    // one segment: a plain output pass from h0 / zeros
    a.nseg = 1;
    hipLaunchKernelGGL((scan_chunked_kernel<N, G, TI, 1>), dim3(a.units), dim3(kW * G), 0, stream, a);
    err = hipGetLastError();
  }
  if (scratch) {
    hipError_t ferr = hipFreeAsync(scratch, stream);
    if (err == hipSuccess) err = ferr;
  }
  return err;
}

template <typename TI>
hipError_t dispatch_n(const ScanParams& p, hipStream_t s) {
  switch (p.dstate) {
    case 4: return run<4, TI>(p, s);
    case 8: return run<8, TI>(p, s);
    case 16: return run<16, TI>(p, s);
    case 32: return run<32, TI>(p, s);
    case 64: return run<64, TI>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace chunked

bool chunked_supported(const ScanParams& p) {
  const int es = p.dtype == kBF16 ? 2 : 4;
  auto al16 = [](const void* q) { return q == nullptr || ((uintptr_t)q % 16) == 0; };
  return p.dstate >= 4 && (p.seqlen * es) % 16 == 0 && p.seqlen < (1LL << 31) && p.dim < (1LL << 30) && p.batch < (1LL << 30) &&
         al16(p.u) && al16(p.delta) && al16(p.z) && al16(p.y) && al16(p.B) && al16(p.C);
}

hipError_t launch_scan_chunked(const ScanParams& p, hipStream_t stream) {
  return p.dtype == kBF16 ? chunked::dispatch_n<__bf16>(p, stream) : chunked::dispatch_n<float>(p, stream);
}

}  // namespace ssm
