// Router: logits in one fixed float32 order, then top-k and softmax renormalisation.
//
// Token routing is one of the parts the Mixture-of-Kittens megakernel fuses (companion news
// digest, Merged summary; Mixture-of-Kittens page, TL;DR). The workloads define it as softmax over
// the router logits, top-k, renormalise; the lower expert index wins a tie.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouterTokens = 8;     // tokens per wave (held in scalar registers)
constexpr int kRouterThreads = 256;  // one expert per lane

// logits[t, e] = (((0 + x[t,0] w[e,0]) + x[t,1] w[e,1]) + ...) + bias[e], float32, one fused
// multiply-add per step. A bf16 x bf16 product is exact in float32, so each step rounds once and
// the order is the written left-to-right one: no split over h, no tree. Bound by the float32 FMA
// rate, 2*T*h*E flop.
//
// Layout: each lane owns one expert; each workgroup owns kRouterTokens tokens whose x values are
// wave-uniform, so they are fetched with scalar loads and fed to the FMAs as scalar operands.
// Both operands are first staged once as float32 (exact):

// x as float32, 8 tokens interleaved: xf[g][i][j] = x[8g + j][i] (zeros past T), [ceil(T/8)][h][8].
// One thread per (group g, 8 columns): 8 16-byte loads (one per token), 256 contiguous bytes out.
__global__ __launch_bounds__(256) void x_interleave_kernel(const uint16_t* __restrict__ x, int T,
                                                           int h, float* __restrict__ xf) {
  const int i8 = blockIdx.x * 256 + threadIdx.x;  // columns 8 i8 .. 8 i8 + 7
  const int g = blockIdx.y;
  if (8 * i8 >= h) return;
  uint4 raw[kRouterTokens];
#pragma unroll
  for (int j = 0; j < kRouterTokens; ++j) {
    const int t = g * kRouterTokens + j;
    raw[j] = t < T ? *reinterpret_cast<const uint4*>(x + (size_t)t * h + 8 * i8)
                   : make_uint4(0u, 0u, 0u, 0u);
  }
  f32x4_t* d = reinterpret_cast<f32x4_t*>(xf + ((size_t)g * h + 8 * i8) * kRouterTokens);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float v[kRouterTokens];
#pragma unroll
    for (int j = 0; j < kRouterTokens; ++j) {
      const uint32_t wd = c < 2 ? raw[j].x : c < 4 ? raw[j].y : c < 6 ? raw[j].z : raw[j].w;
      v[j] = (c & 1) ? bf16_hi(wd) : bf16_lo(wd);
    }
    d[2 * c] = (f32x4_t){v[0], v[1], v[2], v[3]};
    d[2 * c + 1] = (f32x4_t){v[4], v[5], v[6], v[7]};
  }
}

// The router matrix as float32, 8 columns of every expert side by side: wi[v][e][0..7] =
// w[e][8v .. 8v+7], [h/8][E][8]. One thread per (e, v); 32 contiguous bytes written per thread.
__global__ __launch_bounds__(256) void w_interleave_kernel(const uint16_t* __restrict__ w, int E,
                                                           int h, float* __restrict__ wi) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int v = blockIdx.y;
  if (e >= E) return;
  const uint4 x = *reinterpret_cast<const uint4*>(w + (size_t)e * h + 8 * v);
  f32x4_t* d = reinterpret_cast<f32x4_t*>(wi + ((size_t)v * E + e) * 8);
  d[0] = (f32x4_t){bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y)};
  d[1] = (f32x4_t){bf16_lo(x.z), bf16_hi(x.z), bf16_lo(x.w), bf16_hi(x.w)};
}

// The same logits, in the same order, from the interleaved float32 x and router matrix:
//  - the 64 scalar operands of a step of 8 columns are 256 contiguous bytes (scalar loads, no
//    conversion on the scalar unit, which otherwise issues as many instructions as the FMAs);
//  - a wave's router-matrix loads of a step are 64 experts x 32 bytes, contiguous (16 cache
//    lines instead of one line per lane, which thrashed the vector L1: a lane's row is revisited
//    only 8 steps later).
__global__ __launch_bounds__(kRouterThreads) void router_logits_xf_kernel(
    const float* __restrict__ xf, const float* __restrict__ wi, const float* __restrict__ bias,
    float* __restrict__ logits, int T, int h, int E) {
  const int e = blockIdx.y * kRouterThreads + threadIdx.x;
  const int t0 = blockIdx.x * kRouterTokens;
  const int e_ld = e < E ? e : E - 1;  // idle lanes read a valid row and store nothing
  const float* xg = xf + (size_t)blockIdx.x * h * kRouterTokens;
  float acc[kRouterTokens];
#pragma unroll
  for (int tt = 0; tt < kRouterTokens; ++tt) acc[tt] = 0.0f;

  const int nvec = h / 8;
  for (int v = 0; v < nvec; ++v) {
    const f32x4_t* wp = reinterpret_cast<const f32x4_t*>(wi + ((size_t)v * E + e_ld) * 8);
    const f32x4_t w0 = wp[0], w1 = wp[1];
    const float wf[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
    const float* xs = xg + (size_t)v * 8 * kRouterTokens;
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int tt = 0; tt < kRouterTokens; ++tt)
        acc[tt] = __builtin_fmaf(xs[q * kRouterTokens + tt], wf[q], acc[tt]);
  }
  if (e < E) {
    const float b = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int tt = 0; tt < kRouterTokens; ++tt) {
      if (t0 + tt < T) logits[(size_t)(t0 + tt) * E + e] = bias ? acc[tt] + b : acc[tt];
    }
  }
}

// "a ranks before b": larger logit first, then the lower expert index.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

constexpr int kTopkMaxPerLane = 16;  // E <= 1024

// One wave per token. Each lane holds the logits of experts lane, lane+64, ...; k rounds of a
// wave-wide arg-max under (logit desc, index asc) pick the experts in rank order. -0.0 is made
// +0.0 on load so both zeros tie. Weights: softmax over the k selected logits,
// w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), summed in slot order.
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits,
                                                           int32_t* __restrict__ idx,
                                                           float* __restrict__ wout, int T, int E,
                                                           int k) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits together
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

size_t router_xf_bytes(int T, int h, int E) {
  const size_t xf = (size_t)((T + kRouterTokens - 1) / kRouterTokens) * kRouterTokens * h * 4;
  return align_up(xf) + (size_t)E * h * 4;
}

hipError_t launch_router_logits_xf(const uint16_t* x, const uint16_t* w_router, const float* bias,
                                   float* logits, int T, int h, int E, float* scratch,
                                   hipStream_t st) {
  const int groups = (T + kRouterTokens - 1) / kRouterTokens;
  float* xf = scratch;
  float* wi = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(scratch) +
                                       align_up((size_t)groups * kRouterTokens * h * 4));
  hipLaunchKernelGGL(x_interleave_kernel, dim3((h / 8 + 255) / 256, groups), dim3(256), 0, st, x,
                     T, h, xf);
  hipLaunchKernelGGL(w_interleave_kernel, dim3((E + 255) / 256, h / 8), dim3(256), 0, st, w_router,
                     E, h, wi);
  dim3 grid(groups, (E + kRouterThreads - 1) / kRouterThreads);
  hipLaunchKernelGGL(router_logits_xf_kernel, grid, dim3(kRouterThreads), 0, st, xf, wi, bias,
                     logits, T, h, E);
  return hipGetLastError();
}

hipError_t launch_topk_softmax(const float* logits, int32_t* idx, float* w, int T, int E, int k,
                               hipStream_t st) {
  hipLaunchKernelGGL(topk_softmax_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, idx, w, T,
                     E, k);
  return hipGetLastError();
}

}  // namespace moe
