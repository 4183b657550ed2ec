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
#include "moe_sched_body.h"

namespace moe {
namespace {

__global__ __launch_bounds__(kChunk) void sched_count_kernel(const int32_t* __restrict__ assign,
                                                             int R, int E_loc, int nchunks,
                                                             int32_t* __restrict__ cc) {
  extern __shared__ int hist[];
  sched_count_chunk(assign, R, E_loc, nchunks, cc, blockIdx.x, hist);
}

__global__ __launch_bounds__(64) void sched_expert_scan_kernel(int32_t* __restrict__ cc,
                                                                int nchunks,
                                                                int32_t* __restrict__ counts) {
  sched_expert_scan_wave(cc, nchunks, counts, blockIdx.x);
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
  extern __shared__ int wcnt[];
  sched_rank_chunk(assign, R, E_loc, nchunks, base, offsets, perm, inv, blockIdx.x, wcnt);
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

__global__ __launch_bounds__(256) void gather_mxfp8_kernel(const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ inv,
                                                           uint8_t* __restrict__ rows,
                                                           uint8_t* __restrict__ scales, int h,
                                                           int k, int sc_cm_rows) {
  gather_mxfp8_token(x, inv, rows, scales, h, k, sc_cm_rows, blockIdx.x);
}

__global__ void zero_i64_kernel(int64_t* p) { *p = 0; }

// every float32 with bits in [lo, lo + n), both signs
__global__ __launch_bounds__(256) void check_e4m3_kernel(uint32_t lo, uint32_t n,
                                                         int64_t* mismatches) {
  int64_t bad = 0;
  for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    for (int s = 0; s < 2; ++s) {
      const float y = __uint_as_float((lo + i) | (s ? 0x80000000u : 0u));
      const uint32_t q = e4m3_encode_rule(y) | (e4m3_encode_rule(-y) << 8) |
                         (e4m3_encode_rule(0.5f * y) << 16) | (e4m3_encode_rule(2.0f * y) << 24);
      bad += (e4m3_encode(y) != e4m3_encode_rule(y)) + (e4m3_pack4(y, -y, 0.5f * y, 2.0f * y) != q);
    }
  }
  if (bad) atomicAdd(reinterpret_cast<unsigned long long*>(mismatches), (unsigned long long)bad);
}

}  // namespace

hipError_t launch_check_e4m3(int64_t* mismatches, hipStream_t st) {
  hipLaunchKernelGGL(zero_i64_kernel, dim3(1), dim3(1), 0, st, mismatches);
  const uint32_t ranges[][2] = {{0x00000000u, 0x00800000u}, {0x00800000u, 0x32000000u},
                                {0x32000000u, 0x44000000u}, {0x44000000u, 0x48000000u}};
  for (const auto& r : ranges)
    hipLaunchKernelGGL(check_e4m3_kernel, dim3(4096), dim3(256), 0, st, r[0], r[1] - r[0],
                       mismatches);
  return hipGetLastError();
}

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
  // one workgroup per token (measured faster here than one flat list of blocks, which the
  // persistent forward uses for its four-wave workgroups)
  hipLaunchKernelGGL(gather_mxfp8_kernel, dim3(T), dim3(256), 0, st, x, nullptr, codes,
                     scales_cm, h, 1, T);
  return hipGetLastError();
}

}  // namespace moe
