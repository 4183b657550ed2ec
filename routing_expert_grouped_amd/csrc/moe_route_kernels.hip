// Router: logits in one fixed float32 order, then top-k and softmax renormalisation.
//
// Token routing is one of the parts the Mixture-of-Kittens megakernel fuses (companion news
// digest, Merged summary; Mixture-of-Kittens page, TL;DR). The workloads define it as softmax over
// the router logits, top-k, renormalise; the lower expert index wins a tie.
#include "moe_route_body.h"

namespace moe {
namespace {

// The router matrix as bf16 interleaved by 8 columns: wi[v][e][0..7] = w[e][8v .. 8v+7],
// [h/8][E][8]. One thread per (e, v), 16 contiguous bytes per thread.
__global__ __launch_bounds__(256) void w_interleave_bf16_kernel(const uint16_t* __restrict__ w,
                                                                int E, int h,
                                                                uint16_t* __restrict__ wi) {
  const int e = blockIdx.x * 256 + threadIdx.x, v = blockIdx.y;
  if (e >= E) return;
  *reinterpret_cast<uint4*>(wi + ((size_t)v * E + e) * 8) =
      *reinterpret_cast<const uint4*>(w + (size_t)e * h + 8 * v);
}

// Logits on the matrix cores in the same fixed order. v_mfma_f32_32x32x1_2b_f32 adds one product
// to each of its 2 x 32 x 32 accumulators per instruction (block b: 32 rows of A from lanes 32b ..
// 32b+31 times 32 columns of B from the same lanes), so a chain of them over i = 0, 1, ..., h-1 is
// acc = round(acc + x[t,i] w[e,i]) per step: the product of two bf16 values is exact in float32,
// so each step is the same single rounding as the fused multiply-add of the written order, at
// twice the vector FMA rate. A wave owns 32 tokens (rows; both blocks take the same tokens) and 64
// experts (block b: experts 32b ..); a workgroup of four waves owns 32 tokens x 256 experts. Lane l
// reads token t0 + l % 32's row of x and expert l's interleaved router weights, 16 bytes each per 8
// steps, kRouterDepth 8-step blocks ahead. Accumulator k of lane l is block k / 16, row
// 8 ((k % 16) / 4) + 4 (l / 32) + k % 4, column l % 32.
typedef __attribute__((__vector_size__(32 * sizeof(float)))) float f32x32_t;
constexpr int kRouterDepth = 4;
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ wi,
                                                                 const float* __restrict__ bias,
                                                                 float* __restrict__ logits,
                                                                 int T, int h, int E) {
  const int lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * 32;
  const int eb = blockIdx.y * 256 + 64 * (threadIdx.x >> 6);  // the wave's first expert
  if (eb >= E) return;  // a wave with no expert (no barrier follows)
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

// one wave per token
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits,
                                                           int32_t* __restrict__ idx,
                                                           float* __restrict__ wout, int T, int E,
                                                           int k) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits together
  topk_softmax_token(logits, idx, wout, E, k, t);
}

}  // namespace

size_t router_xf_bytes(int T, int h, int E) {
  (void)T;
  return (size_t)E * h * 4;  // the router matrix as float32, interleaved by 8 columns
}

hipError_t launch_router_logits_xf(const uint16_t* x, const uint16_t* w_router, const float* bias,
                                   float* logits, int T, int h, int E, float* scratch,
                                   hipStream_t st) {
  uint16_t* wi = reinterpret_cast<uint16_t*>(scratch);
  hipLaunchKernelGGL(w_interleave_bf16_kernel, dim3((E + 255) / 256, h / 8), dim3(256), 0, st,
                     w_router, E, h, wi);
  dim3 grid((T + 31) / 32, (E + 255) / 256);
  hipLaunchKernelGGL(router_logits_mfma_kernel, grid, dim3(256), 0, st, x, wi, bias, logits, T, h,
                     E);
  return hipGetLastError();
}

hipError_t launch_topk_softmax(const float* logits, int32_t* idx, float* w, int T, int E, int k,
                               hipStream_t st) {
  hipLaunchKernelGGL(topk_softmax_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, idx, w, T,
                     E, k);
  return hipGetLastError();
}

}  // namespace moe
