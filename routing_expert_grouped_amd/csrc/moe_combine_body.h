// Device body of the fixed-order weighted combine (one token per call by 256 threads), shared by
// the combine kernel and the persistent forward.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

// KMAX: a bound on k known at compile time, so that the k row loads of a vector are all issued
// before the first fma (a dropped slot loads a valid row and skips its fma).
// ROUTER (the backward's un-permute of a router layer): after the k rows, the router's part of
// the input gradient is added in the same fixed order, acc = fma(dl[t k + j], W_r[e_j], acc) for
// j ascending (e_j = assign[t k + j], skipped when outside [0, E)), before the one rounding.
template <int KMAX, int VPT, bool ROUTER>
__device__ __forceinline__ void combine_token(const uint16_t* __restrict__ out_rows,
                                              const int32_t* __restrict__ inv,
                                              const float* __restrict__ w,
                                              const uint16_t* __restrict__ shared_out,
                                              uint16_t* __restrict__ y, int h, int k,
                                              const uint16_t* __restrict__ w_router,
                                              const int32_t* __restrict__ assign,
                                              const float* __restrict__ dl, int E, int t) {
  int src[KMAX];
  float wt[KMAX];
  int re[KMAX];
  float rg[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    src[j] = j < k ? inv[(size_t)t * k + j] : -1;
    wt[j] = j < k ? (w ? w[(size_t)t * k + j] : 1.0f) : 0.0f;  // fma(1, o, acc) is the plain sum
    if constexpr (ROUTER) {
      const int e = j < k ? assign[(size_t)t * k + j] : -1;
      re[j] = (unsigned)e < (unsigned)E ? e : -1;
      rg[j] = j < k ? dl[(size_t)t * k + j] : 0.0f;
    }
  }
  const int nv = h / 8;
  // each thread takes VPT 16-byte vectors v0, v0 + 256, ... of the row and requests every row's
  // vectors (k of them per v, plus the shared expert's) before the first fma
  for (int v0 = threadIdx.x; v0 < nv; v0 += 256 * VPT) {
    uint4 o[VPT][KMAX];
    uint4 sh[VPT];
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int v = v0 + 256 * u;
      if (v >= nv) continue;
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < k) o[u][j] = reinterpret_cast<const uint4*>(out_rows + (size_t)max(src[j], 0) * h)[v];
      if (shared_out) sh[u] = reinterpret_cast<const uint4*>(shared_out + (size_t)t * h)[v];
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int v = v0 + 256 * u;
      if (v >= nv) continue;
      float acc[8];
      if (shared_out) {
        const uint4 s = sh[u];
        acc[0] = bf16_lo(s.x); acc[1] = bf16_hi(s.x); acc[2] = bf16_lo(s.y); acc[3] = bf16_hi(s.y);
        acc[4] = bf16_lo(s.z); acc[5] = bf16_hi(s.z); acc[6] = bf16_lo(s.w); acc[7] = bf16_hi(s.w);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
      }
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j >= k || src[j] < 0) continue;  // a dropped assignment contributes nothing
        const uint4 oj = o[u][j];
        const float of[8] = {bf16_lo(oj.x), bf16_hi(oj.x), bf16_lo(oj.y), bf16_hi(oj.y),
                             bf16_lo(oj.z), bf16_hi(oj.z), bf16_lo(oj.w), bf16_hi(oj.w)};
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(wt[j], of[q], acc[q]);
      }
      if constexpr (ROUTER) {
        uint4 wr[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (j < k) wr[j] = reinterpret_cast<const uint4*>(w_router + (size_t)max(re[j], 0) * h)[v];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (j >= k || re[j] < 0) continue;
          const float rf[8] = {bf16_lo(wr[j].x), bf16_hi(wr[j].x), bf16_lo(wr[j].y),
                               bf16_hi(wr[j].y), bf16_lo(wr[j].z), bf16_hi(wr[j].z),
                               bf16_lo(wr[j].w), bf16_hi(wr[j].w)};
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(rg[j], rf[q], acc[q]);
        }
      }
      uint4 r;
      r.x = pack_bf16x2(acc[0], acc[1]);
      r.y = pack_bf16x2(acc[2], acc[3]);
      r.z = pack_bf16x2(acc[4], acc[5]);
      r.w = pack_bf16x2(acc[6], acc[7]);
      reinterpret_cast<uint4*>(y + (size_t)t * h)[v] = r;
    }
  }
}

}  // namespace
}  // namespace moe
