// Router: logits in one fixed float32 order, then top-k and softmax renormalisation.
//
// Token routing is one of the parts the Mixture-of-Kittens megakernel fuses (companion news
// digest, Merged summary; Mixture-of-Kittens page, TL;DR). The workloads define it as softmax over
// the router logits, top-k, renormalise; the lower expert index wins a tie.
#include "moe_route_body.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void w_interleave_bf16_kernel(const uint16_t* __restrict__ w,
                                                                int E, int h,
                                                                uint16_t* __restrict__ wi) {
  w_interleave_bf16_one(w, E, h, wi, blockIdx.x * 256 + threadIdx.x, blockIdx.y);
}

// a router tile (32 tokens x 256 experts) per workgroup of four waves
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ wi,
                                                                 const float* __restrict__ bias,
                                                                 float* __restrict__ logits,
                                                                 int T, int h, int E) {
  router_logits_mfma_tile(x, wi, bias, logits, T, h, E, blockIdx.x, blockIdx.y);
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
  dim3 grid((T + kRouterTileTokens - 1) / kRouterTileTokens,
            (E + kRouterTileExperts - 1) / kRouterTileExperts);
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
