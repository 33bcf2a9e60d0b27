// ssd.hip -- the Mamba-2 "state space duality" (SSD) form of the scan on gfx950 MFMA.
//
// With one decay rate a_h and one step size Delta_t per head (every channel of head h
// uses A[d, n] = a_h for all n), the recurrence of the S6 scan is a multiplication by a
// lower-triangular semiseparable matrix (mlqm.cn tutorial §8; AI inference series (14),
// the part on reorganising the SSM into matrix computation): per head,
//   y_t = sum_{s <= t} (C_t . B_s) exp(a (cs_t - cs_s)) Delta_s x_s,   cs_t = sum_{r <= t} Delta_r.
// Cut into chunks of Q = 64 steps, this is three dense products per chunk plus a short
// recurrence over chunks, in two kernels:
//   1. chunk states and state passing (ssd_state_kernel): S_c = sum_s B_s w_s x_s^T,
//      w_s = exp(a (cs_end - cs_s)) Delta_s -- [N x Q] x [Q x 16] on MFMA per 16-column tile -- and
//      H_c = exp(a cs_end,c) H_{c-1} + S_c, the chunks of a head walked in order, H in registers;
//      the state entering each chunk is written out;
//   2. chunk output (ssd_chunk_scan_kernel): Y = (G o decay o Delta) X + diag(exp(a cs_t)) C H_{c-1},
//      G = C B^T -- [Q x N] x [N x Q], [Q x Q] x [Q x P] and [Q x N] x [N x P] on MFMA; then the
//      D skip and the SiLU gate.
// MFMA operands are bf16 with fp32 accumulation.  x, B and C are the bf16 inputs themselves.  The
// operands computed in fp32 -- the decay-weighted matrices and the carried state -- enter as a
// pair of bf16 values, v = hi + lo with hi = bf16(v) and lo = bf16(v - hi), and each product is
// taken twice (hi, then lo): the operand then carries about 16 bits instead of 8, at twice the
// matrix-core work of those products.  Step sizes, cumulative sums, decays and the state passing
// are fp32.
//
// MFMA lane layout of v_mfma_f32_16x16x16_bf16 (checked on the device with an in-bounds probe):
// lane l supplies A[l % 16][4 (l / 16) + j] and B[4 (l / 16) + j][l % 16], j = 0..3, and receives
// D[4 (l / 16) + j][l % 16].  v_mfma_f32_16x16x32_bf16 is the same with 8 (l / 16) + j, j = 0..7, for
// the reduction index.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {
namespace {

constexpr int kQ = 64;  // steps per chunk
// channels per head: the kernels are templates over it (32, 64 or 128: whole 16-channel tiles, and
// the output kernel's 256 threads move a head's 64-step x tile in whole 16-byte pieces)

typedef short bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct SsdArgs {
  const __bf16* x;
  const __bf16* dt;
  const float* A;        // [H]
  const __bf16* B;
  const __bf16* C;
  const float* D;        // [H*P] or null
  const __bf16* z;       // or null
  const float* dt_bias;  // [H] or null
  const float* h0;       // [batch, H*P, N] or null
  __bf16* y;
  float* last;           // [batch, H*P, N] or null
  float* S;  // the state entering each chunk, 16 bytes per (lane, 16-state tile): bf16 hi x4, lo x4;
             // [batch*H, chunks, P/16, N/16, 64 lanes]
  int64_t batch, heads, seqlen;
  int chunks, softplus;
};

__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v = hi + lo to about 16 significant bits: hi = bf16(v), lo = bf16(v - hi).
__device__ __forceinline__ void split_bf16(float v, __bf16& hi, __bf16& lo) {
  hi = (__bf16)v;
  lo = (__bf16)(v - (float)hi);
}

// Inclusive prefix sum over the 64 lanes with DPP (the gfx9 wave scan): four row shifts scan each
// 16-lane row, then row broadcasts of lanes 15 and 31 carry the row totals forward.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_src(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x += dpp_src<0x111, 0xF>(x);  // row_shr:1
  x += dpp_src<0x112, 0xF>(x);  // row_shr:2
  x += dpp_src<0x114, 0xF>(x);  // row_shr:4
  x += dpp_src<0x118, 0xF>(x);  // row_shr:8
  x += dpp_src<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_src<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// 1+2. Chunk states and state passing: one wave per (batch row x head, 16-channel column tile),
// walking the chunks in order with the running state H[n][p] of its 16 columns in registers --
// in the accumulator layout of the chunk-state product, lane (q, r) holding n = 4 q + j (+ 16 nt)
// of column p = 16 tile + r.  Per chunk: S_c = sum_s B_s w_s x_s^T on MFMA, the incoming state is
// written out for the output kernel, then H <- exp(a cs_end) H + S_c.  The following chunks' B, x
// and steps are in flight while one is combined.
template <int N, int kP>
__global__ __launch_bounds__(64) void ssd_state_kernel(SsdArgs a) {
  constexpr int kDepth = 4;  // chunks whose loads are in flight (2, 4 and 8 measured within 3%)
  // decay weights of the chunks in flight, one row per ring slot.  The block is one wave, whose LDS
  // accesses execute in order, so no barrier stands between writing a row and reading it: the
  // combines of consecutive chunks are independent up to the state update and may interleave.
  __shared__ __align__(16) float sw[kDepth][kQ];
  const int lane = threadIdx.x;
  const int pt = blockIdx.x;  // column tile
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / a.heads, h = bh % a.heads;
  const int64_t L = a.seqlen;
  const int r = lane % 16, q = lane / 16;
  const int p = 16 * pt + r;
  const float A2 = a.A[h] * kLog2e;
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  const __bf16* xrow = a.x + (b * a.heads * kP + h * kP + p) * L;  // this lane's B-operand column
  const __bf16* Bb = a.B + b * N * L;
  const __bf16* dtr = a.dt + bh * L;
  const int64_t sidx0 = ((b * a.heads + h) * kP + p) * N;  // [batch, H*P, N] row of column p
  float H[N / 16][4];
#pragma unroll
  for (int nt = 0; nt < N / 16; ++nt)
#pragma unroll
    for (int j = 0; j < 4; ++j) H[nt][j] = a.h0 ? a.h0[sidx0 + 16 * nt + 4 * q + j] : 0.0f;

  // loads of one chunk: x[p][s..s+7] and B[n][s..s+7] for s = 32 kt + 8 q, n = 16 nt + r (16 bytes
  // each), and the step of lane s.  The loads of the next kDepth - 1 chunks are in flight while one
  // is combined.  The loads are unconditional (lanes past the sequence end read step t0 of the chunk
  // instead) and their values are masked where they are used, so no load sits in a branch that must
  // wait for it.
  struct Loads {
    uint4 x[kQ / 32];
    uint4 b[N / 16][kQ / 32];
    unsigned short dt;
  };
  const auto fetch = [&](int c, Loads& ld) {
    const int64_t t0 = (int64_t)c * kQ;
    const int len = (int)std::min<int64_t>(kQ, L - t0);
#pragma unroll
    for (int kt = 0; kt < kQ / 32; ++kt) {
      const int s = 32 * kt + 8 * q;
      const int sv = s < len ? s : 0;  // len is a multiple of 8: a lane's 8 steps are all in or all out
      ld.x[kt] = *(const uint4*)(xrow + t0 + sv);
#pragma unroll
      for (int nt = 0; nt < N / 16; ++nt) ld.b[nt][kt] = *(const uint4*)(Bb + (int64_t)(16 * nt + r) * L + t0 + sv);
    }
    ld.dt = ((const unsigned short*)dtr)[t0 + (lane < len ? lane : 0)];
  };
  const auto combine = [&](int c, const Loads& ld, float* swk) {
    const int64_t t0 = (int64_t)c * kQ;
    const int len = (int)std::min<int64_t>(kQ, L - t0);
    // step sizes and their prefix sums (lane = step)
    const float raw = __uint_as_float((uint32_t)ld.dt << 16) + bias;
    const float dl = lane < len ? (a.softplus ? softplus(raw) : raw) : 0.0f;
    const float cs = wave_prefix_sum(dl);
    const float cs_end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), kQ - 1));
    swk[lane] = ex2(A2 * (cs_end - cs)) * dl;
    // S_c, with the decay-weighted B as hi/lo bf16 A operands
    f32x4 sc[N / 16];
#pragma unroll
    for (int nt = 0; nt < N / 16; ++nt) {
      // hi and lo products accumulate separately: two independent MFMA chains
      f32x4 shi = {0.0f, 0.0f, 0.0f, 0.0f}, slo = shi;
#pragma unroll
      for (int kt = 0; kt < kQ / 32; ++kt) {
        const bool in = 32 * kt + 8 * q < len;
        const float4 w0 = *(const float4*)&swk[32 * kt + 8 * q];  // zero past the sequence end (Delta = 0)
        const float4 w1 = *(const float4*)&swk[32 * kt + 8 * q + 4];
        const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        const uint4 rb = ld.b[nt][kt];
        const uint32_t bw2[4] = {rb.x, rb.y, rb.z, rb.w};
        const uint4 rx = in ? ld.x[kt] : make_uint4(0, 0, 0, 0);
        bf16x8 ahi, alo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t bits = j % 2 ? bw2[j / 2] & 0xffff0000u : bw2[j / 2] << 16;
          __bf16 hi, lo;
          split_bf16(__uint_as_float(bits) * wv[j], hi, lo);
          ahi[j] = hi;
          alo[j] = lo;
        }
        const bf16x8 xv = __builtin_bit_cast(bf16x8, rx);
        shi = mfma32(ahi, xv, shi);
        slo = mfma32(alo, xv, slo);
      }
      sc[nt] = shi + slo;
    }
    // hand the incoming state to the output kernel, already split into the hi/lo bf16 operands it
    // takes, then advance it over the chunk
    uint4* Sin = (uint4*)a.S + ((bh * a.chunks + c) * (kP / 16) + pt) * (N / 16) * 64 + lane;
    const float decay = ex2(A2 * cs_end);
#pragma unroll
    for (int nt = 0; nt < N / 16; ++nt) {
      bf16x4 hhi, hlo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        __bf16 hi, lo;
        split_bf16(H[nt][j], hi, lo);
        hhi[j] = __builtin_bit_cast(short, hi);
        hlo[j] = __builtin_bit_cast(short, lo);
        H[nt][j] = __builtin_fmaf(decay, H[nt][j], sc[nt][j]);
      }
      const uint2 uh = __builtin_bit_cast(uint2, hhi), ul = __builtin_bit_cast(uint2, hlo);
      Sin[nt * 64] = make_uint4(uh.x, uh.y, ul.x, ul.y);
    }
  };
  // kDepth register sets in a ring; the loop is unrolled over the ring so that every set has a
  // fixed register home
  // Past the last chunk a fetch reloads the last chunk (unused), so that whole rounds of kDepth
  // chunks are straight-line code.
  Loads ld[kDepth];
  const int last_c = a.chunks - 1;
#pragma unroll
  for (int k = 0; k < kDepth; ++k) fetch(std::min(k, last_c), ld[k]);
  int c0 = 0;
  for (; c0 + kDepth <= a.chunks; c0 += kDepth) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      combine(c0 + k, ld[k], sw[k]);
      fetch(std::min(c0 + k + kDepth, last_c), ld[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < kDepth - 1; ++k)
    if (c0 + k < a.chunks) combine(c0 + k, ld[k], sw[k]);
  if (a.last) {
#pragma unroll
    for (int nt = 0; nt < N / 16; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) a.last[sidx0 + 16 * nt + 4 * q + j] = H[nt][j];
  }
}

// 3. Chunk outputs: four waves per (chunk, batch row x head); wave w owns output rows
// t = 16 w .. 16 w + 15 (all 64 channels).  The decay-weighted matrix is formed transposed,
// G^T = B C^T, whose accumulator layout (rows s, columns t) is exactly the A-operand layout
// of the next product M x (rows t, reduction index s): it never leaves the registers.
template <int N, int kP>
__global__ __launch_bounds__(256) void ssd_chunk_scan_kernel(SsdArgs a) {
  static_assert(kP % 32 == 0 && kP * kQ / 8 % 256 == 0, "whole x-tile pieces per thread");
  constexpr int XS = kQ + 4;  // padded row of the x tile (bf16): 34 banks, so 16 rows' 8-byte reads miss each other
  constexpr int NS = N + 4;   // padded row of the step-major B and C tiles
  __shared__ __align__(16) __bf16 sX[kP][XS];   // x[p][s]
  __shared__ __align__(16) __bf16 sCt[kQ][NS];  // C[t][n]
  __shared__ __align__(16) __bf16 sBt[kQ][NS];  // B[s][n]
  __shared__ float scs[kQ], sdl[kQ];
  __shared__ __align__(16) float sY[kP][kQ + 4];  // y before the gate, [p][t]
  const int tid = threadIdx.x, w = tid / 64, lane = tid % 64;
  const int c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / a.heads, h = bh % a.heads;
  const int64_t L = a.seqlen;
  const int64_t t0 = (int64_t)c * kQ;
  const int len = (int)std::min<int64_t>(kQ, L - t0);
  const float A2 = a.A[h] * kLog2e;
  const int64_t ch0 = b * a.heads * kP + h * kP;  // first channel of the head
  const __bf16* xh = a.x + ch0 * L + t0;
  const int r = lane % 16, q = lane / 16;
  const int tq = 16 * w + 4 * q;  // first output step of this lane's accumulators
  // Every global load of the block is issued before the first is waited for.  Pieces past the
  // sequence end load step 0 of the chunk instead and are masked where they are used.
  // x tile: 64 rows x 64 steps, 8 steps (16 bytes) per piece
  constexpr int kPieces = kP * kQ / 8 / 256;
  uint4 xraw[kPieces], zraw[kPieces];
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int pc = tid + 256 * i, row = pc / (kQ / 8), s8 = 8 * (pc % (kQ / 8));
    xraw[i] = *(const uint4*)(xh + (int64_t)row * L + (s8 < len ? s8 : 0));
  }
  // B and C rows, 4 steps per piece
  constexpr int kBC = N * kQ / 4 / 256;
  const __bf16* Bb = a.B + b * N * L + t0;
  const __bf16* Cb = a.C + b * N * L + t0;
  uint2 braw[kBC], craw[kBC];
#pragma unroll
  for (int i = 0; i < kBC; ++i) {
    const int pc = tid + 256 * i, n = pc / (kQ / 4), s4 = 4 * (pc % (kQ / 4));
    const int64_t off = (int64_t)n * L + (s4 < len ? s4 : 0);
    braw[i] = *(const uint2*)(Bb + off);
    craw[i] = *(const uint2*)(Cb + off);
  }
  // the step of lane t (wave 0)
  const unsigned short dtraw = ((const unsigned short*)a.dt)[bh * L + t0 + (lane < len ? lane : 0)];
  // gate inputs of this thread's output pieces
  if (a.z) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int pc = tid + 256 * i, row = pc / (kQ / 8), s8 = 8 * (pc % (kQ / 8));
      zraw[i] = *(const uint4*)(a.z + (ch0 + row) * L + t0 + (s8 < len ? s8 : 0));
    }
  }
  float Dv[kP / 16];
#pragma unroll
  for (int pt = 0; pt < kP / 16; ++pt) Dv[pt] = a.D ? a.D[h * kP + 16 * pt + r] : 0.0f;
  // B operand of C H_in: H[n][p] for n = 16 kt + 4 q + j, p = 16 pt + r, one float4 per (pt, kt)
  const uint4* Hin = (const uint4*)a.S + (bh * a.chunks + c) * (kP / 16) * (N / 16) * 64 + lane;
  uint4 hv[N / 16][kP / 16];
#pragma unroll
  for (int pt = 0; pt < kP / 16; ++pt)
#pragma unroll
    for (int kt = 0; kt < N / 16; ++kt) hv[kt][pt] = Hin[(pt * (N / 16) + kt) * 64];

  if (w == 0) {
    const float raw = __uint_as_float((uint32_t)dtraw << 16) + (a.dt_bias ? a.dt_bias[h] : 0.0f);
    const float dl = lane < len ? (a.softplus ? softplus(raw) : raw) : 0.0f;
    scs[lane] = A2 * wave_prefix_sum(dl);  // a cs_t, in log2 units
    sdl[lane] = dl;
  }
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int pc = tid + 256 * i, row = pc / (kQ / 8), s8 = 8 * (pc % (kQ / 8));
    const uint4 v = s8 < len ? xraw[i] : make_uint4(0, 0, 0, 0);
    *(uint2*)&sX[row][s8] = make_uint2(v.x, v.y);
    *(uint2*)&sX[row][s8 + 4] = make_uint2(v.z, v.w);
  }
  // B, C transposed to step-major
#pragma unroll
  for (int i = 0; i < kBC; ++i) {
    const int pc = tid + 256 * i, n = pc / (kQ / 4), s4 = 4 * (pc % (kQ / 4));
    const bool in = s4 < len;
    const uint32_t wb[2] = {in ? braw[i].x : 0u, in ? braw[i].y : 0u};
    const uint32_t wc[2] = {in ? craw[i].x : 0u, in ? craw[i].y : 0u};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint16_t bj = (uint16_t)(wb[jj / 2] >> (16 * (jj % 2))), cj = (uint16_t)(wc[jj / 2] >> (16 * (jj % 2)));
      sBt[s4 + jj][n] = __builtin_bit_cast(__bf16, bj);
      sCt[s4 + jj][n] = __builtin_bit_cast(__bf16, cj);
    }
  }
  __syncthreads();

  const int t = 16 * w + r;  // the step of this lane's A-operand row
  const float cst = scs[t];
  f32x4 acc[kP / 16];
#pragma unroll
  for (int pt = 0; pt < kP / 16; ++pt) acc[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // one 16-step block of the causal product; only the diagonal block (st == w) needs the mask
  const auto block = [&](int st, bool diag) {
    // G^T[s][t] = sum_n B[s][n] C[t][n]: lane holds s = 16 st + 4 q + j, t = 16 w + r
    f32x4 g = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kt = 0; kt < N / 16; ++kt) {
      const bf16x4 av = *(const bf16x4*)&sBt[16 * st + r][16 * kt + 4 * q];
      const bf16x4 bv = *(const bf16x4*)&sCt[t][16 * kt + 4 * q];
      g = mfma16(av, bv, g);
    }
    // M[t][s] = G[t][s] exp(a (cs_t - cs_s)) Delta_s for s <= t, as hi/lo bf16 A operands
    bf16x4 mhi, mlo;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int sj = 16 * st + 4 * q + jj;
      const float v = g[jj] * ex2(cst - scs[sj]) * sdl[sj];
      const float m = diag && sj > t ? 0.0f : v;
      __bf16 hi, lo;
      split_bf16(m, hi, lo);
      mhi[jj] = __builtin_bit_cast(short, hi);
      mlo[jj] = __builtin_bit_cast(short, lo);
    }
#pragma unroll
    for (int pt = 0; pt < kP / 16; ++pt) {
      const bf16x4 bv = *(const bf16x4*)&sX[16 * pt + r][16 * st + 4 * q];
      acc[pt] = mfma16(mhi, bv, acc[pt]);
      acc[pt] = mfma16(mlo, bv, acc[pt]);
    }
  };
  for (int st = 0; st < w; ++st) block(st, false);
  block(w, true);
  // + diag(exp(a cs_t)) C H_in (accumulator rows are t = 16 w + 4 q + j)
  float dec[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) dec[jj] = ex2(scs[tq + jj]);
#pragma unroll
  for (int pt = 0; pt < kP / 16; ++pt) {
    f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kt = 0; kt < N / 16; ++kt) {
      const bf16x4 av = *(const bf16x4*)&sCt[t][16 * kt + 4 * q];
      const bf16x4 hhi = __builtin_bit_cast(bf16x4, make_uint2(hv[kt][pt].x, hv[kt][pt].y));
      const bf16x4 hlo = __builtin_bit_cast(bf16x4, make_uint2(hv[kt][pt].z, hv[kt][pt].w));
      o = mfma16(av, hhi, o);
      o = mfma16(av, hlo, o);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[pt][jj] = __builtin_fmaf(dec[jj], o[jj], acc[pt][jj]);
  }
  // skip: this lane holds steps t = 16 w + 4 q + j of channel p = 16 pt + r; y before the gate
  // goes through LDS so that the gate and the store run on whole 16-byte row pieces
#pragma unroll
  for (int pt = 0; pt < kP / 16; ++pt) {
    const int p = 16 * pt + r;
    float4 v;
    const uint2 xw = *(const uint2*)&sX[p][tq];
    v.x = __builtin_fmaf(Dv[pt], __uint_as_float(xw.x << 16), acc[pt][0]);
    v.y = __builtin_fmaf(Dv[pt], __uint_as_float(xw.x & 0xffff0000u), acc[pt][1]);
    v.z = __builtin_fmaf(Dv[pt], __uint_as_float(xw.y << 16), acc[pt][2]);
    v.w = __builtin_fmaf(Dv[pt], __uint_as_float(xw.y & 0xffff0000u), acc[pt][3]);
    *(float4*)&sY[p][tq] = v;
  }
  __syncthreads();
  // gate and store, 8 steps of one channel per piece
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int pc = tid + 256 * i, row = pc / (kQ / 8), s8 = 8 * (pc % (kQ / 8));
    if (s8 >= len) continue;
    const float4 v0 = *(const float4*)&sY[row][s8], v1 = *(const float4*)&sY[row][s8 + 4];
    float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    if (a.z) {
      const uint32_t zw[4] = {zraw[i].x, zraw[i].y, zraw[i].z, zraw[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] *= silu(__uint_as_float(zw[k] << 16));
        v[2 * k + 1] *= silu(__uint_as_float(zw[k] & 0xffff0000u));
      }
    }
    __bf16 out[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) out[k] = (__bf16)v[k];
    uint4 o;
    __builtin_memcpy(&o, out, sizeof o);
    *(uint4*)(a.y + (ch0 + row) * L + t0 + s8) = o;
  }
}

template <int N, int kP>
hipError_t run(const SsdParams& p, hipStream_t stream) {
  SsdArgs a{};
  a.x = (const __bf16*)p.x; a.dt = (const __bf16*)p.dt; a.A = p.A; a.B = (const __bf16*)p.B;
  a.C = (const __bf16*)p.C; a.D = p.D; a.z = (const __bf16*)p.z; a.dt_bias = p.dt_bias; a.h0 = p.h0;
  a.y = (__bf16*)p.y; a.last = p.last_state;
  a.batch = p.batch; a.heads = p.heads; a.seqlen = p.seqlen; a.softplus = p.softplus;
  a.chunks = (int)((p.seqlen + kQ - 1) / kQ);
  const int64_t bh = p.batch * p.heads;
  const size_t nS = (size_t)bh * a.chunks * N * kP;
  void* scratch = nullptr;
  bool kept = false;
  hipError_t err = call_scratch(stream, 2, nS * sizeof(float), &scratch, &kept);
  if (err != hipSuccess) return err;
  a.S = (float*)scratch;
  hipLaunchKernelGGL((ssd_state_kernel<N, kP>), dim3(kP / 16, (unsigned)bh), dim3(64), 0, stream, a);
  err = hipGetLastError();
  if (err == hipSuccess) {
    hipLaunchKernelGGL((ssd_chunk_scan_kernel<N, kP>), dim3((unsigned)a.chunks, (unsigned)bh), dim3(256), 0, stream,
                       a);
    err = hipGetLastError();
  }
  const hipError_t ferr = call_scratch_release(scratch, kept, stream);
  return err != hipSuccess ? err : ferr;
}

__global__ __launch_bounds__(256) void ssd_empty_state(float* last, const float* h0, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) last[i] = h0 ? h0[i] : 0.0f;
}

}  // namespace

bool ssd_supported(int64_t headdim, int64_t dstate) {
  const bool n_ok = dstate == 16 || dstate == 32 || dstate == 64;
  // heads of 128 channels hold 8 x (dstate / 16) incoming-state tiles per lane: dstate 64 would spill
  return n_ok && (headdim == 32 || headdim == 64 || (headdim == 128 && dstate <= 32));
}

hipError_t launch_ssd_fwd(const SsdParams& p, hipStream_t stream) {
  if (p.seqlen == 0) {
    if (p.last_state && p.last_state != p.h0) {
      const int64_t n = p.batch * p.heads * p.headdim * p.dstate;
      hipLaunchKernelGGL(ssd_empty_state, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p.last_state,
                         p.h0, n);
      return hipGetLastError();
    }
    return hipSuccess;
  }
  if (!ssd_supported(p.headdim, p.dstate)) return hipErrorInvalidValue;
  switch (p.headdim * 1000 + p.dstate) {
    case 32016: return run<16, 32>(p, stream);
    case 32032: return run<32, 32>(p, stream);
    case 32064: return run<64, 32>(p, stream);
    case 64016: return run<16, 64>(p, stream);
    case 64032: return run<32, 64>(p, stream);
    case 64064: return run<64, 64>(p, stream);
    case 128016: return run<16, 128>(p, stream);
    case 128032: return run<32, 128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssm
