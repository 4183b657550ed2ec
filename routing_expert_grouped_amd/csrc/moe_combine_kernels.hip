// Weighted combine back to token order, in one fixed floating-point order.
//
// The Mixture-of-Kittens page makes bitwise determinism a headline property (TL;DR, Key claims):
// the order of floating-point operations is fixed. Here every output element is
//   y[t, c] = bf16( fma(w[t,k-1], O[inv[t*k+k-1], c], ... fma(w[t,0], O[inv[t*k], c], S[t, c]) ) )
// with slots j ascending, float32 accumulation starting from the shared-expert output (or +0.0)
// and one rounding to bf16 at the end. It is a gather (each token reads its k rows), so there are
// no atomics and nothing depends on scheduling. One workgroup per token, 16-byte accesses.
#include "moe_internal.h"

namespace moe {
namespace {

// KMAX: a bound on k known at compile time, so that the k row loads of a vector are all issued
// before the first fma (a dropped slot loads a valid row and skips its fma).
template <int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ out_rows,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w,
                                                      const uint16_t* __restrict__ shared_out,
                                                      uint16_t* __restrict__ y, int h, int k) {
  const int t = blockIdx.x;
  int src[KMAX];
  float wt[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    src[j] = j < k ? inv[(size_t)t * k + j] : -1;
    wt[j] = j < k ? (w ? w[(size_t)t * k + j] : 1.0f) : 0.0f;  // fma(1, o, acc) is the plain sum
  }
  const int nv = h / 8;
  for (int v = threadIdx.x; v < nv; v += 256) {
    uint4 o[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) o[j] = reinterpret_cast<const uint4*>(out_rows + (size_t)max(src[j], 0) * h)[v];
    float acc[8];
    if (shared_out) {
      const uint4 s = reinterpret_cast<const uint4*>(shared_out + (size_t)t * h)[v];
      acc[0] = bf16_lo(s.x); acc[1] = bf16_hi(s.x); acc[2] = bf16_lo(s.y); acc[3] = bf16_hi(s.y);
      acc[4] = bf16_lo(s.z); acc[5] = bf16_hi(s.z); acc[6] = bf16_lo(s.w); acc[7] = bf16_hi(s.w);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= k || src[j] < 0) continue;  // a dropped assignment contributes nothing
      const float of[8] = {bf16_lo(o[j].x), bf16_hi(o[j].x), bf16_lo(o[j].y), bf16_hi(o[j].y),
                           bf16_lo(o[j].z), bf16_hi(o[j].z), bf16_lo(o[j].w), bf16_hi(o[j].w)};
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(wt[j], of[q], acc[q]);
    }
    uint4 r;
    r.x = pack_bf16x2(acc[0], acc[1]);
    r.y = pack_bf16x2(acc[2], acc[3]);
    r.z = pack_bf16x2(acc[4], acc[5]);
    r.w = pack_bf16x2(acc[6], acc[7]);
    reinterpret_cast<uint4*>(y + (size_t)t * h)[v] = r;
  }
}

}  // namespace

hipError_t launch_combine(const uint16_t* out_rows, const int32_t* inv, const float* w,
                          const uint16_t* shared_out, uint16_t* y, int T, int h, int k,
                          hipStream_t st) {
  if (k <= 8)
    hipLaunchKernelGGL(combine_kernel<8>, dim3(T), dim3(256), 0, st, out_rows, inv, w, shared_out,
                       y, h, k);
  else
    hipLaunchKernelGGL(combine_kernel<16>, dim3(T), dim3(256), 0, st, out_rows, inv, w,
                       shared_out, y, h, k);
  return hipGetLastError();
}

}  // namespace moe
