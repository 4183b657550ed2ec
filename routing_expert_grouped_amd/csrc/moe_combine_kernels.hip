// Weighted combine back to token order, in one fixed floating-point order.
//
// The Mixture-of-Kittens page makes bitwise determinism a headline property (TL;DR, Key claims):
// the order of floating-point operations is fixed. Here every output element is
//   y[t, c] = bf16( fma(w[t,k-1], O[inv[t*k+k-1], c], ... fma(w[t,0], O[inv[t*k], c], S[t, c]) ) )
// with slots j ascending, float32 accumulation starting from the shared-expert output (or +0.0)
// and one rounding to bf16 at the end. It is a gather (each token reads its k rows), so there are
// no atomics and nothing depends on scheduling. One workgroup per token, 16-byte accesses.
#include "moe_combine_body.h"

namespace moe {
namespace {

// one workgroup per token
template <int KMAX, int VPT, bool ROUTER>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ out_rows,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w,
                                                      const uint16_t* __restrict__ shared_out,
                                                      uint16_t* __restrict__ y, int h, int k,
                                                      const uint16_t* __restrict__ w_router,
                                                      const int32_t* __restrict__ assign,
                                                      const float* __restrict__ dl, int E) {
  combine_token<KMAX, VPT, ROUTER>(out_rows, inv, w, shared_out, y, h, k, w_router, assign, dl, E,
                                   blockIdx.x);
}

}  // namespace

hipError_t launch_combine(const uint16_t* out_rows, const int32_t* inv, const float* w,
                          const uint16_t* shared_out, uint16_t* y, int T, int h, int k,
                          hipStream_t st, const uint16_t* w_router, const int32_t* assign,
                          const float* dl, int E) {
  const dim3 g(T), b(256);
  // vectors per thread: every 16-byte vector of the row in one round when it fits the registers
  const int rounds = (h / 8 + 255) / 256;
#define MOE_COMBINE(KM, VP, RT)                                                                 \
  hipLaunchKernelGGL((combine_kernel<KM, VP, RT>), g, b, 0, st, out_rows, inv, w, shared_out, y, \
                     h, k, w_router, assign, dl, E)
  if (w_router) {
    if (k <= 8) MOE_COMBINE(8, 1, true);
    else MOE_COMBINE(16, 1, true);
  } else if (k <= 8) {
    if (rounds <= 1) MOE_COMBINE(8, 1, false);
    else if (rounds == 2) MOE_COMBINE(8, 2, false);
    else if (rounds == 3) MOE_COMBINE(8, 3, false);
    else MOE_COMBINE(8, 4, false);
  } else {
    if (rounds <= 1) MOE_COMBINE(16, 1, false);
    else MOE_COMBINE(16, 2, false);
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
