// Device bodies of the router: the interleaved router matrix, the fixed-order logits and the top-k
// with softmax renormalisation, each for one explicit block of work, shared by the router kernels
// and the persistent forward.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

// logits[t, e] = (((0 + x[t,0] w[e,0]) + x[t,1] w[e,1]) + ...) + bias[e], float32, one rounding
// per step in the written left-to-right order: no split over h, no tree. 2*T*h*E flop.
//
// The chain runs on the matrix cores. v_mfma_f32_32x32x1_2b_f32 adds one product to each of its
// 2 x 32 x 32 accumulators per instruction (block b: 32 rows of A from lanes 32b .. 32b+31 times
// 32 columns of B from the same lanes), and the product of two bf16 values is exact in float32, so
// each instruction is, per logit, the same single rounding round(acc + x w) as a fused
// multiply-add of the written order, at twice the vector FMA rate.

// The router matrix as bf16 interleaved by 8 columns: wi[v][e][0..7] = w[e][8v .. 8v+7],
// [h/8][E][8] (a wave's 64 experts of one 8-column block are 1 KB contiguous). One thread per
// (e, v), 16 contiguous bytes.
__device__ __forceinline__ void w_interleave_bf16_one(const uint16_t* __restrict__ w, int E, int h,
                                                      uint16_t* __restrict__ wi, int e, int v) {
  if (e >= E) return;
  *reinterpret_cast<uint4*>(wi + ((size_t)v * E + e) * 8) =
      *reinterpret_cast<const uint4*>(w + (size_t)e * h + 8 * v);
}

typedef __attribute__((__vector_size__(32 * sizeof(float)))) float f32x32_t;
constexpr int kRouterTileTokens = 32;   // tokens of a router tile (the MFMA rows)
constexpr int kRouterTileExperts = 256; // experts of a router tile (four waves of 64)
constexpr int kRouterDepth = 4;         // 8-step blocks loaded ahead

// Tokens [bx * 32, +32) x experts [by * 256, +256) by the calling workgroup's four waves (the
// first 256 threads): a wave owns the 32 tokens (the rows, the same in both blocks) and 64 experts
// (block b: experts 32b ..). Lane l reads token l % 32's row of x and expert l's 8-column slices of
// the interleaved router matrix, 16 bytes of each per 8 steps, kRouterDepth blocks ahead.
// Accumulator k of lane l is block k / 16, row 8 ((k % 16) / 4) + 4 (l / 32) + k % 4, column
// l % 32. No barrier: a wave with no expert returns at once.
__device__ __forceinline__ void router_logits_mfma_tile(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ wi,
                                                        const float* __restrict__ bias,
                                                        float* __restrict__ logits, int T, int h,
                                                        int E, int bx, int by) {
  const int lane = threadIdx.x & 63;
  const int t0 = bx * kRouterTileTokens;
  const int eb = by * kRouterTileExperts + 64 * (threadIdx.x >> 6);  // the wave's first expert
  if (eb >= E) return;
  const int t = min(t0 + (lane & 31), T - 1);  // rows past T read a valid row, store nothing
  const int e = min(eb + lane, E - 1);
  const uint16_t* xp = x + (size_t)t * h;
  const uint16_t* wp = wi + (size_t)e * 8;
  const size_t wstep = (size_t)E * 8;  // elements between 8-column blocks
  const int nb = h / 8;
  f32x32_t acc;
#pragma unroll
  for (int k = 0; k < 32; ++k) acc[k] = 0.0f;
  uint4 xq[kRouterDepth], wq[kRouterDepth];
#pragma unroll
  for (int d = 0; d < kRouterDepth; ++d)
    if (d < nb) {
      xq[d] = *reinterpret_cast<const uint4*>(xp + 8 * d);
      wq[d] = *reinterpret_cast<const uint4*>(wp + d * wstep);
    }
  // block v (8 steps): its values as float32 first, so its registers are free for block
  // v + depth's loads (no copy of a register a load is still writing), then its 8 MFMAs
  auto block = [&](int d, bool reload, int vnext) {
    const uint32_t xs[4] = {xq[d].x, xq[d].y, xq[d].z, xq[d].w};
    const uint32_t ws[4] = {wq[d].x, wq[d].y, wq[d].z, wq[d].w};
    float a[8], b[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[2 * q] = bf16_lo(xs[q]);
      a[2 * q + 1] = bf16_hi(xs[q]);
      b[2 * q] = bf16_lo(ws[q]);
      b[2 * q + 1] = bf16_hi(ws[q]);
    }
    // converted before the registers are reloaded (no load moves above this point)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (reload) {
      xq[d] = *reinterpret_cast<const uint4*>(xp + 8 * vnext);
      wq[d] = *reinterpret_cast<const uint4*>(wp + vnext * wstep);
    }
    // the reloads stay ahead of this block's MFMAs (the scheduler would otherwise sink them to
    // the end of the loop body and wait for them at the top of the next iteration)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x1f32(a[q], b[q], acc, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // steady state: every block's reload exists (branch-free, so each prefetch register is simply
  // overwritten); then the last blocks
  int v0 = 0;
  for (; v0 + 2 * kRouterDepth <= nb; v0 += kRouterDepth) {
#pragma unroll
    for (int d = 0; d < kRouterDepth; ++d) block(d, true, v0 + d + kRouterDepth);
  }
  for (; v0 < nb; v0 += kRouterDepth) {
#pragma unroll
    for (int d = 0; d < kRouterDepth; ++d) {
      const int v = v0 + d;
      if (v < nb) block(d, v + kRouterDepth < nb, v + kRouterDepth);
    }
  }
  float bv[2] = {0.0f, 0.0f};  // the bias of the lane's column in either block
  if (bias) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) bv[blk] = bias[min(eb + 32 * blk + (lane & 31), E - 1)];
  }
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int row = 8 * ((k & 15) >> 2) + 4 * (lane >> 5) + (k & 3);
    const int tt = t0 + row, ee = eb + 32 * (k >> 4) + (lane & 31);
    if (tt < T && ee < E) logits[(size_t)tt * E + ee] = bias ? acc[k] + bv[k >> 4] : acc[k];
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
