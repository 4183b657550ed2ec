// Data movement of the expert-path backward: backward weight layouts, the un-combine that forms
// each routed row's output gradient, and the per-expert transposes that feed the weight-gradient
// GEMMs.
//
// The Mixture-of-Kittens page (Key claims) runs the MXFP8 backward with the same fused
// quantisation as the forward, and its flowchart mirrors dispatch and combine in the backward
// (the reverse combine pulls output gradients, the reverse dispatch pushes input gradients back).
// Here, with routing weights held fixed:
//   dO[r] = w[a] * dY[a / k]               (a = perm[r]; the un-combine)
//   dH = dO W_down^T, dG = dH * U * silu'(G), dU = dH * silu(G)         (GEMM + epilogue)
// (G and U are the forward's float32 values, kept in the saved buffer; dG and dU are also kept in
// float32, so every MX quantisation below starts from a float32 value)
//   dA = dG W_gate^T + dU W_up^T                                          (GEMM)
//   dX[t] = sum over slots j ascending of dA[inv[t k + j]]                (un-permute)
//   dW_gate_e = A_e^T dG_e, dW_up_e = A_e^T dU_e, dW_down_e = H_e^T dO_e  (GEMMs over rows)
// Every GEMM operand is MX-quantised along that GEMM's reduction axis: h for dH, m for dA, and an
// expert's routed rows for the weight gradients. For the last, each expert's rows are padded with
// zeros to a multiple of the GEMM's K step and stored transposed, [C][kpad_e], at offset
// koff[e] * C, with E8M0 scales per 32 rows; blocks start at the expert's first row.
// Every MX scale array the GEMMs read here is chunk-major: the 8 block scales of one 256-element
// chunk of the reduction axis of each row side by side, [K/256][rows][8] (per expert for weights
// and per expert segment for the transposed operands).
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ void unpack8(const uint4 v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// ------------------------------------------------------------------------------------------------
// Backward weight layouts. Each source row (K contiguous) is copied block by block: source block b
// (32 elements) of row n lands at K position b * bstride + boff of row n, MX-quantised per 32.
//   W_down rows [e][m][h] stay as they are (K = h for dH = dO W_down^T);
//   W_gate and W_up rows [e][h][m] are interleaved per 32 into [e][h][2m] (K = 2m for dA), gate
//   blocks at 64 b, up blocks at 64 b + 32, the same order as the dG | dU columns.
// One thread per block of 32. N: rows per expert (for the chunk-major scales).
// ------------------------------------------------------------------------------------------------
template <bool MX>
__global__ __launch_bounds__(256) void prep_rows_kernel(const uint16_t* __restrict__ src,
                                                        long long nblocks, int Ks, int Kd,
                                                        int bstride, int boff, int N,
                                                        uint8_t* __restrict__ dst,
                                                        uint8_t* __restrict__ dst_s) {
  const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
  if (id >= nblocks) return;
  const int nb = Ks / kMxBlock;
  const long long row = id / nb;  // e * N + n
  const int b = (int)(id % nb);
  const uint4* s = reinterpret_cast<const uint4*>(src + row * Ks + (long long)b * kMxBlock);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) unpack8(s[q], v + 8 * q);
  const long long kd = row * Kd + (long long)b * bstride + boff;
  if constexpr (MX) {
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(v[q]));
    const int sx = mx_block_exponent(amax);
    const float inv = mx_inv_scale(sx);
    uint32_t c[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      c[q] = e4m3_pack4(v[4 * q] * inv, v[4 * q + 1] * inv, v[4 * q + 2] * inv, v[4 * q + 3] * inv);
    uint4* d = reinterpret_cast<uint4*>(dst + kd);
    d[0] = make_uint4(c[0], c[1], c[2], c[3]);
    d[1] = make_uint4(c[4], c[5], c[6], c[7]);
    const long long e = row / N, n = row % N;
    const int kb = (b * bstride + boff) / kMxBlock;  // block along the destination K
    dst_s[e * N * (Kd / kMxBlock) + ((long long)(kb >> 3) * N + n) * 8 + (kb & 7)] =
        (uint8_t)(sx + 127);
  } else {
    uint4* d = reinterpret_cast<uint4*>(dst + 2 * kd);
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = s[q];
  }
}

// ------------------------------------------------------------------------------------------------
// koff[e] = sum over e' < e of ceil(count_e' / align) * align (one workgroup, E_loc <= 1024)
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void kpad_table_kernel(const int32_t* __restrict__ offsets,
                                                          int E_loc, int align,
                                                          int32_t* __restrict__ koff) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  int v = 0;
  if (tid < E_loc) v = (offsets[tid + 1] - offsets[tid] + align - 1) / align * align;
  const int own = v;
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
  if (tid < E_loc) koff[tid] = incl - own;
  if (tid == E_loc - 1) koff[E_loc] = incl;
}

// ------------------------------------------------------------------------------------------------
// Un-combine: dO[r] = w[a] * dY[a / k], a = perm[r], for the rows offsets[0] .. offsets[E_loc]-1.
// BF16: rounded to bf16. MX: quantised per 32 along h from the float32 product (each routed row
// on its own: its gate weight scales the token's gradient). One workgroup per routed row.
// ------------------------------------------------------------------------------------------------
template <bool MX>
__global__ __launch_bounds__(256) void uncombine_kernel(const uint16_t* __restrict__ dy,
                                                        const int32_t* __restrict__ perm,
                                                        const float* __restrict__ w,
                                                        const int32_t* __restrict__ offsets,
                                                        int E_loc, uint8_t* __restrict__ dO,
                                                        uint8_t* __restrict__ dO_s, int R, int h,
                                                        int k) {
  const int r = blockIdx.x;
  if (r >= offsets[E_loc]) return;
  const int a = perm[r];
  const float wt = w[a];
  const uint16_t* src = dy + (size_t)(a / k) * h;
  if constexpr (MX) {
    const int nb = h / kMxBlock;
    for (int b = threadIdx.x; b < nb; b += 256) {
      const uint4* s = reinterpret_cast<const uint4*>(src + b * kMxBlock);
      float v[32];
#pragma unroll
      for (int q = 0; q < 4; ++q) unpack8(s[q], v + 8 * q);
      float amax = 0.0f;
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        v[q] *= wt;
        amax = fmaxf(amax, fabsf(v[q]));
      }
      const int sx = mx_block_exponent(amax);
      const float inv = mx_inv_scale(sx);
      uint32_t c[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        c[q] = e4m3_pack4(v[4 * q] * inv, v[4 * q + 1] * inv,
                          v[4 * q + 2] * inv, v[4 * q + 3] * inv);
      uint4* d = reinterpret_cast<uint4*>(dO + (size_t)r * h + b * kMxBlock);
      d[0] = make_uint4(c[0], c[1], c[2], c[3]);
      d[1] = make_uint4(c[4], c[5], c[6], c[7]);
      dO_s[((size_t)(b >> 3) * R + r) * 8 + (b & 7)] = (uint8_t)(sx + 127);
    }
  } else {
    uint16_t* d = reinterpret_cast<uint16_t*>(dO) + (size_t)r * h;
    for (int c = threadIdx.x; c < h / 8; c += 256) {
      float v[8];
      unpack8(reinterpret_cast<const uint4*>(src)[c], v);
      uint4 o;
      o.x = pack_bf16x2(v[0] * wt, v[1] * wt);
      o.y = pack_bf16x2(v[2] * wt, v[3] * wt);
      o.z = pack_bf16x2(v[4] * wt, v[5] * wt);
      o.w = pack_bf16x2(v[6] * wt, v[7] * wt);
      reinterpret_cast<uint4*>(d)[c] = o;
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Per-expert transpose: a block of RBT rows (of one expert's padded segment) x 64 columns goes
// through LDS; rows past the expert's count are zeros. MX: one thread per (column, 32 rows)
// quantises its block and writes 32 bytes; BF16: one thread per (column, 16 rows).
// ------------------------------------------------------------------------------------------------
template <int SRC, bool MX>
__global__ __launch_bounds__(256) void bwd_transpose_kernel(
    const void* __restrict__ src_, const int32_t* __restrict__ perm,
    const float* __restrict__ w, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ koff, int E_loc, int C, int k, uint8_t* __restrict__ dst,
    uint8_t* __restrict__ dst_s) {
  constexpr int RBT = MX ? 128 : 64;
  __shared__ float tile[RBT][65];
  // rows 64 and up keep their columns XOR 16 (the MX column reads of blocks 64 rows apart would
  // share banks); the BF16 tile has 64 rows and no skew
  auto tile_skew = [](int row) { return 16 * ((row >> 6) & 1); };
  const int kk0 = blockIdx.y * RBT;
  if (kk0 >= koff[E_loc]) return;  // uniform: past the last segment
  // the expert whose segment holds kk0 (exactly one: koff[e] <= kk0 < koff[e+1]), found by the
  // block's threads in parallel: one round of loads instead of a chain of dependent ones
  __shared__ int e_s;
  for (int i = threadIdx.x; i < E_loc; i += 256)
    if (koff[i] <= kk0 && kk0 < koff[i + 1]) e_s = i;
  __syncthreads();
  const int e = e_s;
  const int kbase = koff[e];
  const int kpad = koff[e + 1] - kbase;
  const int q0 = kk0 - kbase;
  const int r0 = offsets[e];
  const int n_e = offsets[e + 1] - r0;
  const int c0 = blockIdx.x * 64;
  const int tid = threadIdx.x;
  const int cq = (tid & 7) * 8;

  // each thread fills rows t0 + 32 i of the tile (RBT / 32 of them): all their source indices
  // are requested first, then all their loads, so a block waits for two memory round trips
  // rather than two per row
  constexpr int RPT = RBT / 32;
  const int t0 = tid >> 3;
  int src_row[RPT];  // routed row (or token for the gathered sources) of each row, -1: zero pad
  float wt[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int q = q0 + t0 + 32 * i;
    src_row[i] = q < n_e ? r0 + q : -1;
    wt[i] = 1.0f;
  }
  if constexpr (SRC == kTrX || SRC == kTrDO) {
    int a[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) a[i] = src_row[i] >= 0 ? perm[src_row[i]] : -1;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      if (a[i] >= 0) {
        if constexpr (SRC == kTrDO) wt[i] = w[a[i]];
        src_row[i] = a[i] / k;  // the token
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int t = t0 + 32 * i;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (src_row[i] >= 0) {
      const int r = src_row[i];
      if constexpr (SRC == kTrX || SRC == kTrDO) {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(src_);
        unpack8(*reinterpret_cast<const uint4*>(src + (size_t)r * C + c0 + cq), v);
        if constexpr (SRC == kTrDO) {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] *= wt[i];
        }
      } else if constexpr (SRC == kTrH) {
        const float* gu = reinterpret_cast<const float*>(src_) + (size_t)r * 2 * C;
        const int c = c0 + cq;
        const size_t gcol = (size_t)64 * (c >> 5) + (c & 31);
        const f32x4_t g0 = *reinterpret_cast<const f32x4_t*>(gu + gcol);
        const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(gu + gcol + 4);
        const f32x4_t u0 = *reinterpret_cast<const f32x4_t*>(gu + gcol + 32);
        const f32x4_t u1 = *reinterpret_cast<const f32x4_t*>(gu + gcol + 36);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] = silu_f(g0[j]) * u0[j];
          v[4 + j] = silu_f(g1[j]) * u1[j];
        }
      } else {
        const float* sp = reinterpret_cast<const float*>(src_) + (size_t)r * C + c0 + cq;
        const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(sp);
        const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(sp + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] = a0[j];
          v[4 + j] = a1[j];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[t][(cq + j) ^ tile_skew(t)] = v[j];
  }
  __syncthreads();

  // MX: wave w takes columns 16 w .. 16 w + 15, four lanes per column (one per 32-row block), so
  // each store instruction writes 64 bytes into each of 16 lines; the column skew of rows 64 and
  // up puts a wave's column reads on 64 distinct banks. BF16: column tid & 63
  const int wv = tid >> 6, ln = tid & 63;
  const int c = MX ? 16 * wv + (ln >> 2) : ln;
  const size_t col_at = (size_t)kbase * C + (size_t)(c0 + c) * kpad + q0;  // element index
  if constexpr (MX) {
    const int b = ln & 3;  // rows 32 b .. 32 b + 31
    const int cs = c ^ tile_skew(32 * b);  // the column's place in rows 32 b .. 32 b + 31
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(tile[32 * b + q][cs]));
    const int sx = mx_block_exponent(amax);
    const float inv = mx_inv_scale(sx);
    uint32_t cw[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      cw[q] = e4m3_pack4(tile[32 * b + 4 * q][cs] * inv, tile[32 * b + 4 * q + 1][cs] * inv,
                         tile[32 * b + 4 * q + 2][cs] * inv, tile[32 * b + 4 * q + 3][cs] * inv);
    uint4* d = reinterpret_cast<uint4*>(dst + col_at + 32 * b);
    d[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    d[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
    const int kb = (q0 + 32 * b) / kMxBlock;  // block along the segment's K
    dst_s[(size_t)kbase * C / kMxBlock + ((size_t)(kb >> 3) * C + c0 + c) * 8 + (kb & 7)] =
        (uint8_t)(sx + 127);
  } else {
    const int b = wv;  // rows 16 b .. 16 b + 15
    uint32_t pw[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) pw[q] = pack_bf16x2(tile[16 * b + 2 * q][c], tile[16 * b + 2 * q + 1][c]);
    uint4* d = reinterpret_cast<uint4*>(dst + 2 * (col_at + 16 * b));
    d[0] = make_uint4(pw[0], pw[1], pw[2], pw[3]);
    d[1] = make_uint4(pw[4], pw[5], pw[6], pw[7]);
  }
}

struct BwdLayout {
  size_t w1b, w1b_s, w2b, w2b_s, total;
};

BwdLayout bwd_layout(int E_loc, int h, int m, bool mx) {
  BwdLayout L{};
  const size_t el = mx ? 1 : 2;
  size_t off = 0;
  L.w1b = off;
  off = align_up(off + (size_t)E_loc * h * 2 * m * el);
  if (mx) {
    L.w1b_s = off;
    off = align_up(off + (size_t)E_loc * h * (2 * m / kMxBlock));
  }
  L.w2b = off;
  off = align_up(off + (size_t)E_loc * m * h * el);
  if (mx) {
    L.w2b_s = off;
    off = align_up(off + (size_t)E_loc * m * (h / kMxBlock));
  }
  L.total = off;
  return L;
}

}  // namespace

size_t prepared_bwd_bytes(int E_loc, int h, int m, bool mx) {
  return bwd_layout(E_loc, h, m, mx).total;
}

PreparedBwd prepared_bwd_views(const void* prepared_bwd, int E_loc, int h, int m, bool mx) {
  const BwdLayout L = bwd_layout(E_loc, h, m, mx);
  const uint8_t* b = reinterpret_cast<const uint8_t*>(prepared_bwd);
  return PreparedBwd{b + L.w1b, mx ? b + L.w1b_s : nullptr, b + L.w2b, mx ? b + L.w2b_s : nullptr};
}

hipError_t launch_prepare_bwd_weights(const uint16_t* w_gate, const uint16_t* w_up,
                                      const uint16_t* w_down, void* prepared_bwd, int E_loc,
                                      int h, int m, bool mx, hipStream_t st) {
  const BwdLayout L = bwd_layout(E_loc, h, m, mx);
  uint8_t* b = reinterpret_cast<uint8_t*>(prepared_bwd);
  const long long n1 = (long long)E_loc * h * (m / kMxBlock);  // blocks of W_gate (and W_up)
  const long long n2 = (long long)E_loc * m * (h / kMxBlock);  // blocks of W_down
  const dim3 g1((unsigned)((n1 + 255) / 256)), g2((unsigned)((n2 + 255) / 256));
  if (mx) {
    hipLaunchKernelGGL(prep_rows_kernel<true>, g1, dim3(256), 0, st, w_gate, n1, m, 2 * m, 64, 0,
                       h, b + L.w1b, b + L.w1b_s);
    hipLaunchKernelGGL(prep_rows_kernel<true>, g1, dim3(256), 0, st, w_up, n1, m, 2 * m, 64, 32,
                       h, b + L.w1b, b + L.w1b_s);
    hipLaunchKernelGGL(prep_rows_kernel<true>, g2, dim3(256), 0, st, w_down, n2, h, h, 32, 0, m,
                       b + L.w2b, b + L.w2b_s);
  } else {
    hipLaunchKernelGGL(prep_rows_kernel<false>, g1, dim3(256), 0, st, w_gate, n1, m, 2 * m, 64, 0,
                       h, b + L.w1b, nullptr);
    hipLaunchKernelGGL(prep_rows_kernel<false>, g1, dim3(256), 0, st, w_up, n1, m, 2 * m, 64, 32,
                       h, b + L.w1b, nullptr);
    hipLaunchKernelGGL(prep_rows_kernel<false>, g2, dim3(256), 0, st, w_down, n2, h, h, 32, 0, m,
                       b + L.w2b, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_kpad_table(const int32_t* offsets, int E_loc, int align, int32_t* koff,
                             hipStream_t st) {
  hipLaunchKernelGGL(kpad_table_kernel, dim3(1), dim3(1024), 0, st, offsets, E_loc, align, koff);
  return hipGetLastError();
}

hipError_t launch_uncombine(const uint16_t* dy, const int32_t* perm, const float* w,
                            const int32_t* offsets, int E_loc, void* dO, uint8_t* dO_s, int R,
                            int h, int k, bool mx, hipStream_t st) {
  uint8_t* d = reinterpret_cast<uint8_t*>(dO);
  if (mx)
    hipLaunchKernelGGL(uncombine_kernel<true>, dim3(R), dim3(256), 0, st, dy, perm, w, offsets,
                       E_loc, d, dO_s, R, h, k);
  else
    hipLaunchKernelGGL(uncombine_kernel<false>, dim3(R), dim3(256), 0, st, dy, perm, w, offsets,
                       E_loc, d, nullptr, R, h, k);
  return hipGetLastError();
}

hipError_t launch_bwd_transpose(int src_kind, const void* src, const int32_t* perm,
                                const float* w, const int32_t* offsets, const int32_t* koff,
                                int E_loc, int C, int k, int rows_max, uint8_t* dst,
                                uint8_t* dst_s, bool mx, hipStream_t st) {
  const int rbt = mx ? 128 : 64;
  const dim3 grid(C / 64, (rows_max + rbt - 1) / rbt);
#define MOE_TR(S)                                                                                \
  do {                                                                                           \
    if (mx)                                                                                      \
      hipLaunchKernelGGL((bwd_transpose_kernel<S, true>), grid, dim3(256), 0, st, src, perm, w,  \
                         offsets, koff, E_loc, C, k, dst, dst_s);                                \
    else                                                                                         \
      hipLaunchKernelGGL((bwd_transpose_kernel<S, false>), grid, dim3(256), 0, st, src, perm, w, \
                         offsets, koff, E_loc, C, k, dst, dst_s);                                \
  } while (0)
  switch (src_kind) {
    case kTrX: MOE_TR(kTrX); break;
    case kTrDO: MOE_TR(kTrDO); break;
    case kTrH: MOE_TR(kTrH); break;
    case kTrRows: MOE_TR(kTrRows); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_TR
  return hipGetLastError();
}

}  // namespace moe
