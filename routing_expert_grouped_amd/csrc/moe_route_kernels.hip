// Router: logits in one fixed float32 order, then top-k and softmax renormalisation.
//
// Token routing is one of the parts the Mixture-of-Kittens megakernel fuses (companion news
// digest, Merged summary; Mixture-of-Kittens page, TL;DR). The workloads define it as softmax over
// the router logits, top-k, renormalise; the lower expert index wins a tie.
#include "moe_route_body.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void w_interleave_kernel(const uint16_t* __restrict__ w, int E,
                                                           int h, float* __restrict__ wi) {
  w_interleave_one(w, E, h, wi, blockIdx.x * 256 + threadIdx.x, blockIdx.y);
}

// 128 threads, two experts per thread: 256 experts per workgroup
constexpr int kRouterThreads = 128;
constexpr int kRouterEpl = 2;
__global__ __launch_bounds__(kRouterThreads) void router_logits_lds_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wi, const float* __restrict__ bias,
    float* __restrict__ logits, int T, int h, int E) {
  __shared__ __attribute__((aligned(16))) float xs[router_lds_floats(kRouterLdsTokens)];
  router_logits_tile<kRouterLdsTokens, kRouterThreads, kRouterEpl>(x, wi, bias, logits, T, h, E,
                                                                    blockIdx.x, blockIdx.y, xs);
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
  float* wi = scratch;
  hipLaunchKernelGGL(w_interleave_kernel, dim3((E + 255) / 256, h / 8), dim3(256), 0, st, w_router,
                     E, h, wi);
  constexpr int ew = kRouterThreads * kRouterEpl;  // experts per workgroup
  dim3 grid((T + kRouterLdsTokens - 1) / kRouterLdsTokens, (E + ew - 1) / ew);
  hipLaunchKernelGGL(router_logits_lds_kernel, grid, dim3(kRouterThreads), 0, st, x, wi, bias,
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
