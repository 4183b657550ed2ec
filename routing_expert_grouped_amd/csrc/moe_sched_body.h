// Device bodies of the schedule (per-chunk expert histogram, per-expert chunk scan, per-chunk
// ranks) and of the MXFP8 quantisation (the gather of one token; every token once), each for one
// explicit block of work, shared by the schedule kernels and the persistent forward.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kChunk = kSchedChunk;

// chunk `chunk` of kChunk assignments by kChunk threads; hist: E_loc ints of LDS
__device__ __forceinline__ void sched_count_chunk(const int32_t* __restrict__ assign, int R,
                                                  int E_loc, int nchunks, int32_t* __restrict__ cc,
                                                  int chunk, int* hist) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E_loc; e += kChunk) hist[e] = 0;
  __syncthreads();
  const int a = chunk * kChunk + tid;
  if (a < R) {
    const int e = assign[a];
    if ((unsigned)e < (unsigned)E_loc) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E_loc; e += kChunk) cc[(size_t)e * nchunks + chunk] = hist[e];
}

// Per expert e (one wave each): the exclusive prefix of its chunk counts, in place (cc ->
// first row of (e, chunk) relative to the expert's first row), and its total.
__device__ __forceinline__ void sched_expert_scan_wave(int32_t* __restrict__ cc, int nchunks,
                                                       int32_t* __restrict__ counts, int e) {
  const int lane = threadIdx.x & 63;
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


// chunk `chunk` by kChunk threads; wcnt: 4 * E_loc ints of LDS
__device__ __forceinline__ void sched_rank_chunk(const int32_t* __restrict__ assign, int R,
                                                 int E_loc, int nchunks,
                                                 const int32_t* __restrict__ base,
                                                 const int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ perm,
                                                 int32_t* __restrict__ inv, int chunk,
                                                 int* wcnt) {
  // wcnt[w][e]: rows of expert e taken by wave w of the chunk
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  for (int i = tid; i < 4 * E_loc; i += kChunk) wcnt[i] = 0;
  __syncthreads();
  const int a = chunk * kChunk + tid;
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
      int r = offsets[e] + base[(size_t)e * nchunks + chunk] + rank_w;
      for (int w = 0; w < wid; ++w) r += wcnt[w * E_loc + e];
      perm[r] = a;
      inv[a] = r;
    } else {
      inv[a] = -1;
    }
  }
}


// One MX block of 32 bf16 values (four 16-byte pieces) -> 32 E4M3 codes (lo, hi) and the block's
// E8M0 exponent s (the scale byte is s + 127): amax, s = floor(log2 amax) - 8 clamped, values
// divided by 2^s with round-to-nearest-even and saturation.
__device__ __forceinline__ int mx_quantize_block32(const uint4 (&w)[4], uint4& lo, uint4& hi) {
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[8 * q + 0] = bf16_lo(w[q].x);
    v[8 * q + 1] = bf16_hi(w[q].x);
    v[8 * q + 2] = bf16_lo(w[q].y);
    v[8 * q + 3] = bf16_hi(w[q].y);
    v[8 * q + 4] = bf16_lo(w[q].z);
    v[8 * q + 5] = bf16_hi(w[q].z);
    v[8 * q + 6] = bf16_lo(w[q].w);
    v[8 * q + 7] = bf16_hi(w[q].w);
  }
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(v[q]));
  const int s = mx_block_exponent(amax);
  const float inv_s = mx_inv_scale(s);
  uint32_t c[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    c[q] = e4m3_pack4(v[4 * q] * inv_s, v[4 * q + 1] * inv_s,
                      v[4 * q + 2] * inv_s, v[4 * q + 3] * inv_s);
  lo = make_uint4(c[0], c[1], c[2], c[3]);
  hi = make_uint4(c[4], c[5], c[6], c[7]);
  return s;
}

// MXFP8 gather of token t by one workgroup: each thread quantises one block of 32 values of x[t]
// once and writes the codes and the scale to the token's k rows (inv == nullptr: one copy, to row
// t). sc_cm_rows > 0: scales chunk-major [h/256][sc_cm_rows][8], else [rows][h/32].
__device__ __forceinline__ void gather_mxfp8_token(const uint16_t* __restrict__ x,
                                                   const int32_t* __restrict__ inv,
                                                   uint8_t* __restrict__ rows,
                                                   uint8_t* __restrict__ scales, int h, int k,
                                                   int sc_cm_rows, int t) {
  const int nb = h / kMxBlock;
  int dst[16];
  if (!inv) k = 1;
  for (int j = 0; j < k; ++j) dst[j] = inv ? inv[(size_t)t * k + j] : t;
  for (int b = threadIdx.x; b < nb; b += 256) {
    const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * h + (size_t)b * kMxBlock);
    uint4 w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = src[q];
    uint4 lo, hi;
    const int s = mx_quantize_block32(w, lo, hi);
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

// Each token of x[T][h] quantised once into codes[T][h] and chunk-major scales
// [h/256][T][8]: the blocks of all tokens as one flat list, block f = (token f / (h/32), block
// f % (h/32)); this workgroup's 256 threads take blocks base + tid + 256 i, i < J, and request all
// J blocks' loads before quantising any.
template <int J>
__device__ __forceinline__ void quantize_token_blocks(const uint16_t* __restrict__ x,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales_cm, int h,
                                                      int T, long long base) {
  const int nb = h / kMxBlock;
  const long long total = (long long)T * nb;
  uint4 w[J][4];
#pragma unroll
  for (int i = 0; i < J; ++i) {
    const long long f = base + threadIdx.x + 256 * i;
    if (f < total) {
      const uint4* src = reinterpret_cast<const uint4*>(x + f * kMxBlock);  // token-major blocks
#pragma unroll
      for (int q = 0; q < 4; ++q) w[i][q] = src[q];
    }
  }
#pragma unroll
  for (int i = 0; i < J; ++i) {
    const long long f = base + threadIdx.x + 256 * i;
    if (f >= total) continue;
    const int t = (int)(f / nb), b = (int)(f % nb);
    uint4 lo, hi;
    const int s = mx_quantize_block32(w[i], lo, hi);
    uint4* d = reinterpret_cast<uint4*>(codes + f * kMxBlock);
    d[0] = lo;
    d[1] = hi;
    scales_cm[((size_t)(b >> 3) * T + t) * 8 + (b & 7)] = (uint8_t)(s + 127);
  }
}

}  // namespace
}  // namespace moe
