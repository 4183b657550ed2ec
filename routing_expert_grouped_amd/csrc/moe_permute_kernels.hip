// Device-side schedule and gather: group the routed rows by expert with no host synchronisation,
// then copy (BF16) or quantise (MXFP8) each token into its k routed rows.
//
// The Mixture-of-Kittens flowchart and Key claims describe a schedule computed on the GPU that
// never talks to the host, and a fixed-size buffer that absorbs the dynamic per-expert counts
// without dropping tokens; activation quantisation is fused into the dispatch. On one GPU the
// buffer is the routed-row array of capacity R = T*k, and the schedule is a stable counting sort
// of the assignments a = t*k + j by expert:
//   1. count:  per chunk of 256 assignments, a histogram over the local experts (LDS integer
//              atomics; integer counts do not depend on their order);
//   2. scan:   one exclusive scan over the (expert, chunk) matrix in expert-major order gives the
//              first row of every (expert, chunk) pair, the expert offsets and counts. It runs as
//              a scan over each expert's chunks (one wave per expert, relative to the expert's
//              first row) and a scan over the expert totals (one workgroup);
//   3. rank:   each assignment's row = its (expert, chunk) base + the number of earlier
//              assignments of the same expert in its chunk (wave ballots, then a prefix over the
//              chunk's four waves), so rows inside an expert follow the assignment order and the
//              result never depends on scheduling.
// Assignments with an expert id outside [0, E_loc) are dropped: they get inv = -1 and no row.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kChunk = kSchedChunk;

__global__ __launch_bounds__(kChunk) void sched_count_kernel(const int32_t* __restrict__ assign,
                                                             int R, int E_loc, int nchunks,
                                                             int32_t* __restrict__ cc) {
  extern __shared__ int hist[];
  const int tid = threadIdx.x;
  for (int e = tid; e < E_loc; e += kChunk) hist[e] = 0;
  __syncthreads();
  const int a = blockIdx.x * kChunk + tid;
  if (a < R) {
    const int e = assign[a];
    if ((unsigned)e < (unsigned)E_loc) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E_loc; e += kChunk) cc[(size_t)e * nchunks + blockIdx.x] = hist[e];
}

// Per expert e (one wave each): the exclusive prefix of its chunk counts, in place (cc ->
// first row of (e, chunk) relative to the expert's first row), and its total.
__global__ __launch_bounds__(64) void sched_expert_scan_kernel(int32_t* __restrict__ cc,
                                                                int nchunks,
                                                                int32_t* __restrict__ counts) {
  const int e = blockIdx.x;
  const int lane = threadIdx.x;
  int32_t* row = cc + (size_t)e * nchunks;
  int run = 0;
  for (int c0 = 0; c0 < nchunks; c0 += 64) {
    const int c = c0 + lane;
    const int x = c < nchunks ? row[c] : 0;
    int v = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(v, off);
      if (lane >= off) v += o;
    }
    if (c < nchunks) row[c] = run + v - x;
    run += __shfl(v, 63);
  }
  if (lane == 0) counts[e] = run;
}

// Exclusive scan of the E_loc <= 1024 expert counts: offsets[0..E_loc], one workgroup of 1024.
__global__ __launch_bounds__(1024) void sched_scan_kernel(const int32_t* __restrict__ counts,
                                                          int E_loc,
                                                          int32_t* __restrict__ offsets) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  const int x = tid < E_loc ? counts[tid] : 0;
  int v = x;
  const int lane = tid & 63, wid = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int t = wsum[w];
      wsum[w] = run;
      run += t;
    }
  }
  __syncthreads();
  const int incl = v + wsum[wid];
  if (tid < E_loc) offsets[tid] = incl - x;
  if (tid == E_loc - 1) offsets[E_loc] = incl;
}

__global__ __launch_bounds__(kChunk) void sched_rank_kernel(const int32_t* __restrict__ assign,
                                                            int R, int E_loc, int nchunks,
                                                            const int32_t* __restrict__ base,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ inv) {
  extern __shared__ int wcnt[];  // [4][E_loc]: rows of expert e taken by each wave of the chunk
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  for (int i = tid; i < 4 * E_loc; i += kChunk) wcnt[i] = 0;
  __syncthreads();
  const int a = blockIdx.x * kChunk + tid;
  int e = -1;
  if (a < R) {
    e = assign[a];
    if ((unsigned)e >= (unsigned)E_loc) e = -1;
  }
  // rank among the lanes of this wave with the same expert, by ballots over the distinct experts
  unsigned long long todo = __ballot(e >= 0);
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank_w = 0;
  while (todo) {
    const int leader = __builtin_ctzll(todo);
    const int e0 = __shfl(e, leader);
    const unsigned long long same = __ballot(e == e0);
    if (e == e0) rank_w = __builtin_popcountll(same & below);
    if (lane == leader) wcnt[wid * E_loc + e0] = __builtin_popcountll(same);
    todo &= ~same;
  }
  __syncthreads();
  if (a < R) {
    if (e >= 0) {
      int r = offsets[e] + base[(size_t)e * nchunks + blockIdx.x] + rank_w;
      for (int w = 0; w < wid; ++w) r += wcnt[w * E_loc + e];
      perm[r] = a;
      inv[a] = r;
    } else {
      inv[a] = -1;
    }
  }
}

// BF16 gather, one workgroup per token: x[t] is read once and written to its k rows.
__global__ __launch_bounds__(256) void gather_bf16_kernel(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ inv,
                                                          uint16_t* __restrict__ rows, int h,
                                                          int k) {
  const int t = blockIdx.x;
  const int nv = h / 8;
  const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * h);
  int dst[16];
  for (int j = 0; j < k; ++j) dst[j] = inv[(size_t)t * k + j];
  for (int v = threadIdx.x; v < nv; v += 256) {
    const uint4 val = src[v];
    for (int j = 0; j < k; ++j)
      if (dst[j] >= 0) reinterpret_cast<uint4*>(rows + (size_t)dst[j] * h)[v] = val;
  }
}

// MXFP8 gather, one workgroup per token: each thread quantises one block of 32 values of x[t]
// once (amax, E8M0 exponent, E4M3 codes) and writes the codes and the scale to the k rows.
// inv == nullptr: one copy, to row t (the tokens quantised in place of the routed rows, for a
// GEMM that gathers them itself). sc_cm_rows > 0: scales chunk-major [h/256][sc_cm_rows][8].
__global__ __launch_bounds__(256) void gather_mxfp8_kernel(const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ inv,
                                                           uint8_t* __restrict__ rows,
                                                           uint8_t* __restrict__ scales, int h,
                                                           int k, int sc_cm_rows) {
  const int t = blockIdx.x;
  const int nb = h / kMxBlock;
  int dst[16];
  if (!inv) k = 1;
  for (int j = 0; j < k; ++j) dst[j] = inv ? inv[(size_t)t * k + j] : t;
  for (int b = threadIdx.x; b < nb; b += 256) {
    const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * h + (size_t)b * kMxBlock);
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 w = src[q];
      v[8 * q + 0] = bf16_lo(w.x);
      v[8 * q + 1] = bf16_hi(w.x);
      v[8 * q + 2] = bf16_lo(w.y);
      v[8 * q + 3] = bf16_hi(w.y);
      v[8 * q + 4] = bf16_lo(w.z);
      v[8 * q + 5] = bf16_hi(w.z);
      v[8 * q + 6] = bf16_lo(w.w);
      v[8 * q + 7] = bf16_hi(w.w);
    }
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(v[q]));
    const int s = mx_block_exponent(amax);
    const float inv_s = mx_inv_scale(s);
    uint32_t c[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      c[q] = e4m3_encode(v[4 * q] * inv_s) | (e4m3_encode(v[4 * q + 1] * inv_s) << 8) |
             (e4m3_encode(v[4 * q + 2] * inv_s) << 16) | (e4m3_encode(v[4 * q + 3] * inv_s) << 24);
    const uint4 lo = make_uint4(c[0], c[1], c[2], c[3]);
    const uint4 hi = make_uint4(c[4], c[5], c[6], c[7]);
    for (int j = 0; j < k; ++j) {
      if (dst[j] < 0) continue;
      uint4* d = reinterpret_cast<uint4*>(rows + (size_t)dst[j] * h + (size_t)b * kMxBlock);
      d[0] = lo;
      d[1] = hi;
      const size_t so = sc_cm_rows > 0 ? ((size_t)(b >> 3) * sc_cm_rows + dst[j]) * 8 + (b & 7)
                                       : (size_t)dst[j] * nb + b;
      scales[so] = (uint8_t)(s + 127);
    }
  }
}

}  // namespace

size_t sched_workspace_bytes(int R, int E_loc) {
  const int nchunks = (R + kChunk - 1) / kChunk;
  return align_up((size_t)nchunks * E_loc * sizeof(int32_t));
}

hipError_t launch_schedule(const int32_t* assign, int R, int E_loc, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                           hipStream_t st) {
  const int nchunks = (R + kChunk - 1) / kChunk;
  int32_t* cc = reinterpret_cast<int32_t*>(ws);
  hipLaunchKernelGGL(sched_count_kernel, dim3(nchunks), dim3(kChunk), E_loc * sizeof(int), st,
                     assign, R, E_loc, nchunks, cc);
  hipLaunchKernelGGL(sched_expert_scan_kernel, dim3(E_loc), dim3(64), 0, st, cc, nchunks, counts);
  hipLaunchKernelGGL(sched_scan_kernel, dim3(1), dim3(1024), 0, st, counts, E_loc, offsets);
  hipLaunchKernelGGL(sched_rank_kernel, dim3(nchunks), dim3(kChunk), 4 * E_loc * sizeof(int), st,
                     assign, R, E_loc, nchunks, cc, offsets, perm, inv);
  return hipGetLastError();
}

hipError_t launch_gather_bf16(const uint16_t* x, const int32_t* inv, uint16_t* rows, int T, int h,
                              int k, hipStream_t st) {
  hipLaunchKernelGGL(gather_bf16_kernel, dim3(T), dim3(256), 0, st, x, inv, rows, h, k);
  return hipGetLastError();
}

hipError_t launch_gather_mxfp8(const uint16_t* x, const int32_t* inv, uint8_t* rows,
                               uint8_t* scales, int T, int h, int k, hipStream_t st) {
  hipLaunchKernelGGL(gather_mxfp8_kernel, dim3(T), dim3(256), 0, st, x, inv, rows, scales, h, k,
                     0);
  return hipGetLastError();
}

hipError_t launch_quantize_tokens_mxfp8(const uint16_t* x, uint8_t* codes, uint8_t* scales_cm,
                                        int T, int h, hipStream_t st) {
  hipLaunchKernelGGL(gather_mxfp8_kernel, dim3(T), dim3(256), 0, st, x, nullptr, codes,
                     scales_cm, h, 1, T);
  return hipGetLastError();
}

}  // namespace moe
