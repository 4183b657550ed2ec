// Device bodies of the router: the float32 interleaved router matrix, the fixed-order logits and
// the top-k with softmax renormalisation, each for one explicit block of work, shared by the router
// kernels and the persistent forward.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

// logits[t, e] = (((0 + x[t,0] w[e,0]) + x[t,1] w[e,1]) + ...) + bias[e], float32, one fused
// multiply-add per step. A bf16 x bf16 product is exact in float32, so each step rounds once and
// the order is the written left-to-right one: no split over h, no tree. Bound by the float32 FMA
// rate, 2*T*h*E flop. Each lane owns one expert; the router matrix is first staged once as float32
// (exact), interleaved by 8 columns, so a wave's loads of a step are 64 experts x 32 contiguous
// bytes (one line per lane would thrash the vector L1: a lane's row is revisited 8 steps later).

// The router matrix as float32, 8 columns of every expert side by side: wi[v][e][0..7] =
// w[e][8v .. 8v+7], [h/8][E][8]. One thread per (e, v); 32 contiguous bytes written per thread.
__device__ __forceinline__ void w_interleave_one(const uint16_t* __restrict__ w, int E, int h,
                                                 float* __restrict__ wi, int e, int v) {
  if (e >= E) return;
  const uint4 x = *reinterpret_cast<const uint4*>(w + (size_t)e * h + 8 * v);
  f32x4_t* d = reinterpret_cast<f32x4_t*>(wi + ((size_t)v * E + e) * 8);
  d[0] = (f32x4_t){bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y)};
  d[1] = (f32x4_t){bf16_lo(x.z), bf16_hi(x.z), bf16_lo(x.w), bf16_hi(x.w)};
}

// x is staged through LDS (no float32 copy of it in HBM): a workgroup owns a block of tokens
// and 256 experts (one per lane); x is brought in kRouterCols-column chunks,
// converted to float32 (exact) and stored per 8 columns as [8 columns][tokens] with 16 floats of
// padding after each 8-column block (the 16-lane groups that store one block fill distinct banks),
// double buffered. A step of 8 columns reads each column's token values with 16-byte
// LDS reads at a wave-uniform address (broadcast) and the lane's 8 router weights from the
// float32 interleaved copy, requested two steps ahead. Every logit's sum keeps the order i = 0,
// 1, ..., h-1.
constexpr int kRouterLdsTokens = 8;  // tokens per workgroup of the router kernel
constexpr int kRouterCols = 256;
// floats per 8-column block of TOK tokens, padded
__host__ __device__ constexpr int router_blk(int tok) { return 8 * tok + 16; }

// LDS floats of both buffers for TOK tokens
__host__ __device__ constexpr int router_lds_floats(int tok) {
  return 2 * (kRouterCols / 8) * router_blk(tok);
}

// Tokens [bx * TOK, +TOK) x experts [by * NT * EPL, +NT * EPL) by one workgroup of NT threads,
// through router_lds_floats(TOK) floats of LDS at xs_lds. Thread l owns experts
// by * NT * EPL + l + NT * u (u < EPL): each x value read from LDS feeds EPL fused multiply-adds
// (one float of LDS per FMA would need 256 bytes per clock per CU at the FMA rate; the LDS
// returns about 100-190). The router kernel takes 8 tokens and two experts per thread (0.44 ms on
// the GLM-5.2-shaped layer against 0.50 with 16 tokens and one expert, 0.70 with 16 and two: its
// grid then has only two waves per SIMD).
template <int TOK, int NT = 256, int EPL = 1>
__device__ __forceinline__ void router_logits_tile(const uint16_t* __restrict__ x,
                                                   const float* __restrict__ wi,
                                                   const float* __restrict__ bias,
                                                   float* __restrict__ logits, int T, int h, int E,
                                                   int bx, int by, float* xs_lds) {
  constexpr int CC = kRouterCols;
  constexpr int BLK = router_blk(TOK);
  constexpr int NBLK = CC / 8;                  // 8-column blocks per chunk
  constexpr int PIECES = TOK * NBLK / NT;       // 16-byte x pieces per thread per chunk
  static_assert(PIECES * NT == TOK * NBLK, "whole pieces per thread");
  static_assert((CC / 8) % 2 == 0, "chunks of an even number of steps");
  static_assert(TOK % 8 == 0, "tokens in groups of 8");
  auto xs = [&](int buf) { return xs_lds + buf * (NBLK * BLK); };
  const int tid = threadIdx.x;
  int e[EPL], e_ld[EPL];
#pragma unroll
  for (int u = 0; u < EPL; ++u) {
    e[u] = by * NT * EPL + tid + NT * u;
    e_ld[u] = e[u] < E ? e[u] : E - 1;  // idle lanes read a valid row and store nothing
  }
  const int t0 = bx * TOK;
  const int nch = (h + CC - 1) / CC;
  const int nsteps = h / 8;

  // piece p = tid + NT i: token p % TOK, 8-column block p / TOK (consecutive lanes: consecutive
  // tokens of one block, so the stores of a 16-lane group land in 16 consecutive banks)
  uint4 raw[PIECES];
  auto fetch = [&](int c) {
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int p = tid + NT * i, tt = p % TOK, b8 = p / TOK;
      const int col = c * CC + 8 * b8, t = t0 + tt;
      raw[i] = (t < T && col < h) ? *reinterpret_cast<const uint4*>(x + (size_t)t * h + col)
                                  : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int p = tid + NT * i, tt = p % TOK, b8 = p / TOK;
      float* d = xs(buf) + b8 * BLK + tt;
      const uint4 r = raw[i];
      d[0 * TOK] = bf16_lo(r.x); d[1 * TOK] = bf16_hi(r.x);
      d[2 * TOK] = bf16_lo(r.y); d[3 * TOK] = bf16_hi(r.y);
      d[4 * TOK] = bf16_lo(r.z); d[5 * TOK] = bf16_hi(r.z);
      d[6 * TOK] = bf16_lo(r.w); d[7 * TOK] = bf16_hi(r.w);
    }
  };
  // the 8 router weights of step v for each owned expert
  auto wrow = [&](int v, f32x4_t (&w)[EPL][2]) {
#pragma unroll
    for (int u = 0; u < EPL; ++u) {
      const f32x4_t* wp = reinterpret_cast<const f32x4_t*>(wi + ((size_t)v * E + e_ld[u]) * 8);
      w[u][0] = wp[0];
      w[u][1] = wp[1];
    }
  };

  float acc[EPL][TOK];
#pragma unroll
  for (int u = 0; u < EPL; ++u)
#pragma unroll
    for (int tt = 0; tt < TOK; ++tt) acc[u][tt] = 0.0f;
  // step v (8 columns) from the LDS block at xb with the weights w of step v, which are then
  // reloaded with those of step v + 2; the x values of column q + 1 are read while column q's
  // multiply-adds run
  auto step = [&](int v, const float* xb, f32x4_t (&w)[EPL][2]) {
    float wf[EPL][8];
#pragma unroll
    for (int u = 0; u < EPL; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wf[u][q] = w[u][0][q];
        wf[u][4 + q] = w[u][1][q];
      }
    if (v + 2 < nsteps) wrow(v + 2, w);
    f32x4_t xa[TOK / 4], xn[TOK / 4];
#pragma unroll
    for (int i = 0; i < TOK / 4; ++i) xa[i] = *reinterpret_cast<const f32x4_t*>(xb + 4 * i);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q + 1 < 8) {
#pragma unroll
        for (int i = 0; i < TOK / 4; ++i)
          xn[i] = *reinterpret_cast<const f32x4_t*>(xb + (q + 1) * TOK + 4 * i);
      }
#pragma unroll
      for (int u = 0; u < EPL; ++u)
#pragma unroll
        for (int tt = 0; tt < TOK; ++tt)
          acc[u][tt] = __builtin_fmaf(xa[tt / 4][tt % 4], wf[u][q], acc[u][tt]);
#pragma unroll
      for (int i = 0; i < TOK / 4; ++i) xa[i] = xn[i];
      // this column's multiply-adds stay here and no LDS read moves above (or merges across)
      // them: two columns of x in registers
#pragma unroll
      for (int u = 0; u < EPL; ++u)
#pragma unroll
        for (int tt = 0; tt < TOK; tt += 8)
          asm volatile("" : "+v"(acc[u][tt]), "+v"(acc[u][tt + 1]), "+v"(acc[u][tt + 2]),
                       "+v"(acc[u][tt + 3]), "+v"(acc[u][tt + 4]), "+v"(acc[u][tt + 5]),
                       "+v"(acc[u][tt + 6]), "+v"(acc[u][tt + 7])::"memory");
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  fetch(0);
  put(0);
  __syncthreads();
  // router weights of the even steps in wa, of the odd steps in wb (each reloaded two steps
  // ahead, so no register copies wait on a load just issued)
  f32x4_t wa[EPL][2], wb[EPL][2];
  wrow(0, wa);
  if (nsteps > 1) wrow(1, wb);
  int v = 0;
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    if (c + 1 < nch) fetch(c + 1);
    const int vend = min(nsteps, (c + 1) * CC / 8);
    const int v0 = c * (CC / 8);  // the chunk's first step: its block 0 in the buffer
    // a chunk starts at an even step (CC / 8 is even), so pairs never straddle chunks; an odd
    // last step is even-numbered
    for (; v + 1 < vend; v += 2) {
      step(v, xs(buf) + (v - v0) * BLK, wa);
      step(v + 1, xs(buf) + (v + 1 - v0) * BLK, wb);
    }
    if (v < vend) {
      step(v, xs(buf) + (v - v0) * BLK, wa);
      ++v;
    }
    if (c + 1 < nch) {
      put(buf ^ 1);  // the other buffer was last read in chunk c - 1, before this chunk's barrier
      __syncthreads();
    }
  }
#pragma unroll
  for (int u = 0; u < EPL; ++u) {
    if (e[u] < E) {
      const float b = bias ? bias[e[u]] : 0.0f;
#pragma unroll
      for (int tt = 0; tt < TOK; ++tt)
        if (t0 + tt < T)
          logits[(size_t)(t0 + tt) * E + e[u]] = bias ? acc[u][tt] + b : acc[u][tt];
    }
  }
}

__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

constexpr int kTopkMaxPerLane = 16;  // E <= 1024

// One wave per token. Each lane holds the logits of experts lane, lane+64, ...; k rounds of a
// wave-wide arg-max under (logit desc, index asc) pick the experts in rank order. -0.0 is made
// +0.0 on load so both zeros tie. Weights: softmax over the k selected logits,
// w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), summed in slot order.
__device__ __forceinline__ void topk_softmax_token(const float* __restrict__ logits,
                                                   int32_t* __restrict__ idx,
                                                   float* __restrict__ wout, int E, int k, int t) {
  const int lane = threadIdx.x & 63;
  const float* row = logits + (size_t)t * E;
  float v[kTopkMaxPerLane];
  const int per_lane = (E + 63) / 64;
#pragma unroll
  for (int q = 0; q < kTopkMaxPerLane; ++q) {
    const int e = lane + 64 * q;
    v[q] = (q < per_lane && e < E) ? row[e] + 0.0f : -__builtin_inff();
  }
  unsigned taken = 0u;  // bit q: v[q] already selected (or absent)
#pragma unroll
  for (int q = 0; q < kTopkMaxPerLane; ++q)
    if (!(q < per_lane && lane + 64 * q < E)) taken |= 1u << q;

  float sel_v = 0.0f;  // lane j < k ends up holding the j-th selected logit
  int sel_i = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < kTopkMaxPerLane; ++q) {
      if (!(taken & (1u << q)) && ranks_before(v[q], lane + 64 * q, bv, bi)) {
        bv = v[q];
        bi = lane + 64 * q;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ranks_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    // every lane now holds the winner (bv, bi)
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) {
      sel_v = bv;
      sel_i = bi;
    }
  }
  const float l0 = __shfl(sel_v, 0);
  const float ex = lane < k ? expf(sel_v - l0) : 0.0f;
  // fixed-order sum over the k slots (slot 0 first), identical in every lane
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += __shfl(ex, j);
  if (lane < k) {
    idx[(size_t)t * k + lane] = sel_i;
    wout[(size_t)t * k + lane] = ex / sum;
  }
}

}  // namespace
}  // namespace moe
