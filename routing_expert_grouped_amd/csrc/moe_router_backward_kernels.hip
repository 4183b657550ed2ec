// Backward through the gate weights and the router.
//
// The forward combines y[t] = S[t] + sum_j w[t, j] * O[inv[t k + j]], so each gate weight's
// gradient is a dot product of the token's output gradient with the expert output row it scaled:
//   dgate[t, j] = <dY[t], O[inv[t k + j]]>                      (0 for a dropped assignment)
// For a layer with its own router the gate weights are the softmax of the k selected logits, and
// the selection is piecewise constant, so only the selected logits get a gradient:
//   dl[t, j] = w[t, j] * (dgate[t, j] - sum_i w[t, i] dgate[t, i])
// which reaches the router matrix, its bias and the input as
//   dW_r[e] = sum over the assignments (t, j) of expert e of dl[t, j] x[t],   db[e] = sum dl,
//   dX_router[t] = sum_j dl[t, j] W_r[idx[t, j]]            (added in the un-permute).
// The Mixture-of-Kittens page (Key claims) measures the whole layer's backward; its flowchart's
// reverse combine pulls the output gradients this starts from.
//
// Every sum has a fixed order: dot products by a fixed per-thread split of h and a fixed
// reduction tree; dW_r and db over each expert's rows in schedule order (assignments ascending),
// in chunks of kRouterChunk rows whose partial sums are then added chunk by chunk.
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ void unpack8f(const uint4 v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// One workgroup per token: its k dot products over h (each thread takes 8-element vectors
// tid, tid + 256, ... in order; then a fixed xor tree in each wave and the four waves in order),
// then, for a router layer, the softmax Jacobian over the token's selected logits.
template <int KMAX, bool ROUTER>
__global__ __launch_bounds__(256) void gate_grad_kernel(const uint16_t* __restrict__ dy,
                                                        const uint16_t* __restrict__ O,
                                                        const int32_t* __restrict__ inv,
                                                        const float* __restrict__ w,
                                                        float* __restrict__ dgate,
                                                        float* __restrict__ dl, int h, int k) {
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int src[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) src[j] = j < k ? inv[(size_t)t * k + j] : -1;
  float part[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) part[j] = 0.0f;
  const int nv = h / 8;
  const uint4* dyv = reinterpret_cast<const uint4*>(dy + (size_t)t * h);
  for (int v = tid; v < nv; v += 256) {
    float d[8];
    unpack8f(dyv[v], d);
    uint4 o[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) o[j] = reinterpret_cast<const uint4*>(O + (size_t)max(src[j], 0) * h)[v];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= k || src[j] < 0) continue;
      float of[8];
      unpack8f(o[j], of);
#pragma unroll
      for (int q = 0; q < 8; ++q) part[j] = __builtin_fmaf(d[q], of[q], part[j]);
    }
  }
  __shared__ float red[4][KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    float v = part[j];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) red[wid][j] = v;
  }
  __syncthreads();
  if (tid == 0) {
    float g[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      g[j] = (j < k && src[j] >= 0) ? ((red[0][j] + red[1][j]) + red[2][j]) + red[3][j] : 0.0f;
      if (j < k) dgate[(size_t)t * k + j] = g[j];
    }
    if constexpr (ROUTER) {
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < k) s = __builtin_fmaf(w[(size_t)t * k + j], g[j], s);
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < k) dl[(size_t)t * k + j] = w[(size_t)t * k + j] * (g[j] - s);
    }
  }
}

// Partial router-matrix gradients: one workgroup per (chunk of up to kRouterChunk rows of one
// expert, 2048 columns). partial[chunk][c] = sum over the chunk's rows r ascending of
// dl[perm[r]] * x[perm[r] / k][c]; partial_db[chunk] = the plain sum of those dl. Eight rows'
// loads are requested before their eight fmas.
__global__ __launch_bounds__(256) void router_wgrad_partial_kernel(
    const int2* __restrict__ tiles, const int* __restrict__ tile_count,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    const float* __restrict__ dl, const uint16_t* __restrict__ x, int h, int k,
    float* __restrict__ partial, float* __restrict__ partial_db) {
  const int ti = blockIdx.x;
  if (ti >= *tile_count) return;  // no barrier in this kernel: surplus workgroups just leave
  const int2 te = tiles[ti];
  const int r0 = te.y;
  const int r1 = min(r0 + kRouterChunk, offsets[te.x + 1]);
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (c >= h) return;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
  float sdl = 0.0f;
  for (int r = r0; r < r1; r += 8) {
    int a[8];
    float g[8];
    uint4 xv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = r + u < r1 ? perm[r + u] : -1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      g[u] = a[u] >= 0 ? dl[a[u]] : 0.0f;
      xv[u] = a[u] >= 0 ? *reinterpret_cast<const uint4*>(x + (size_t)(a[u] / k) * h + c)
                        : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (a[u] < 0) continue;
      float xf[8];
      unpack8f(xv[u], xf);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(g[u], xf[q], acc[q]);
      sdl += g[u];
    }
  }
  float* p = partial + (size_t)ti * h + c;
  *reinterpret_cast<f32x4_t*>(p) = (f32x4_t){acc[0], acc[1], acc[2], acc[3]};
  *reinterpret_cast<f32x4_t*>(p + 4) = (f32x4_t){acc[4], acc[5], acc[6], acc[7]};
  if (blockIdx.y == 0 && threadIdx.x == 0) partial_db[ti] = sdl;
}

// dW_r[e][c] = sum over expert e's chunks in order of partial[chunk][c]; db[e] likewise. One
// workgroup per (expert, 2048 columns); the expert's first chunk is the count of chunks of the
// experts before it (an integer sum, order-free).
__global__ __launch_bounds__(256) void router_wgrad_reduce_kernel(
    const int32_t* __restrict__ offsets, const float* __restrict__ partial,
    const float* __restrict__ partial_db, int h, float* __restrict__ dw_router,
    float* __restrict__ dbias) {
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ int first_s;
  if (tid == 0) first_s = 0;
  __syncthreads();
  int mine = 0;
  for (int i = tid; i < e; i += 256)
    mine += (offsets[i + 1] - offsets[i] + kRouterChunk - 1) / kRouterChunk;
  if (mine) atomicAdd(&first_s, mine);
  __syncthreads();
  const int first = first_s;
  const int n = (offsets[e + 1] - offsets[e] + kRouterChunk - 1) / kRouterChunk;
  const int c = (blockIdx.y * 256 + tid) * 8;
  if (c < h) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    for (int i = 0; i < n; ++i) {
      const float* p = partial + (size_t)(first + i) * h + c;
      const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(p);
      const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[q] += lo[q];
        acc[4 + q] += hi[q];
      }
    }
    float* d = dw_router + (size_t)e * h + c;
    *reinterpret_cast<f32x4_t*>(d) = (f32x4_t){acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4_t*>(d + 4) = (f32x4_t){acc[4], acc[5], acc[6], acc[7]};
  }
  if (dbias && blockIdx.y == 0 && tid == 0) {
    float s = 0.0f;
    for (int i = 0; i < n; ++i) s += partial_db[first + i];
    dbias[e] = s;
  }
}

}  // namespace

hipError_t launch_gate_grads(const uint16_t* dy, const uint16_t* O, const int32_t* inv,
                             const float* w, float* dgate, float* dl, int T, int h, int k,
                             hipStream_t st) {
  const bool router = dl != nullptr;
  if (k <= 8) {
    if (router)
      hipLaunchKernelGGL((gate_grad_kernel<8, true>), dim3(T), dim3(256), 0, st, dy, O, inv, w,
                         dgate, dl, h, k);
    else
      hipLaunchKernelGGL((gate_grad_kernel<8, false>), dim3(T), dim3(256), 0, st, dy, O, inv, w,
                         dgate, dl, h, k);
  } else {
    if (router)
      hipLaunchKernelGGL((gate_grad_kernel<16, true>), dim3(T), dim3(256), 0, st, dy, O, inv, w,
                         dgate, dl, h, k);
    else
      hipLaunchKernelGGL((gate_grad_kernel<16, false>), dim3(T), dim3(256), 0, st, dy, O, inv,
                         w, dgate, dl, h, k);
  }
  return hipGetLastError();
}

size_t router_wgrad_tiles(int R, int E) { return (size_t)(R + kRouterChunk - 1) / kRouterChunk + E; }

hipError_t launch_router_wgrad(const int2* tiles, const int* tile_count, int max_tiles,
                               const int32_t* offsets, const int32_t* perm, const float* dl,
                               const uint16_t* x, int h, int k, int E, float* partial,
                               float* partial_db, float* dw_router, float* dbias,
                               hipStream_t st) {
  const int cb = (h / 8 + 255) / 256;  // column blocks of 2048
  hipLaunchKernelGGL(router_wgrad_partial_kernel, dim3(max_tiles, cb), dim3(256), 0, st, tiles,
                     tile_count, offsets, perm, dl, x, h, k, partial, partial_db);
  hipLaunchKernelGGL(router_wgrad_reduce_kernel, dim3(E, cb), dim3(256), 0, st, offsets, partial,
                     partial_db, h, dw_router, dbias);
  return hipGetLastError();
}

}  // namespace moe
