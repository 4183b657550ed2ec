// Expert SwiGLU FFNs as grouped GEMMs on gfx950 matrix cores, BF16 and MXFP8.
//
// The Mixture-of-Kittens page (flowchart and Key claims) runs the experts as grouped GEMMs in
// MXFP8 with SwiGLU and the activation quantisation fused; BF16 is its other measured precision.
// Here, per local expert e over its routed rows [offsets[e], offsets[e+1]):
//   GEMM-1: [G | U] = rows * W1[e]^T (W1 holds W_gate and W_up columns interleaved per 32),
//           epilogue H = silu(G) * U, stored as bf16 or MX-quantised per 32 along m;
//   GEMM-2: O = H * W2[e]^T, stored as bf16.
//
// Tiling. A workgroup of 4 waves computes a 128 (weight rows n) x 128 (routed rows) output tile;
// each wave a 64 x 64 quarter as 2 x 2 MFMA tiles of 32 x 32. The weight tile is the MFMA's A
// operand and the routed rows its B operand, so each lane ends up holding one routed row and 16
// output columns (four runs of four consecutive columns): the SwiGLU pairs a gate and an up
// register of the same lane, and an MX block of 32 columns of one row lives in one lane and its
// partner lane 32 apart, so its amax needs a single cross-lane step.
//
// K is staged 128 bytes per row at a time (64 bf16 or 128 E4M3) through LDS, double-buffered, with
// the next stage's global loads in flight while the current stage feeds the MFMAs. Rows of 128
// bytes are split into eight 16-byte slots, XOR-swizzled by row so the fragment reads of eight
// consecutive rows hit eight different bank groups.
//
// MXFP8 K order. v_mfma_scale_f32_32x32x64_f8f6f4 multiplies two 32-element MX blocks per lane
// pair: bytes 0-15 of lanes i and i+32 form the first block (scaled by lane i's scale byte),
// bytes 16-31 the second block (scaled by lane i+32's). The K loop walks chunks of 256 elements
// (8 MX blocks) and lets step s in 0..3 of a chunk take blocks s and 4+s, so lane group 0 needs
// the scale bytes of blocks 0..3 and group 1 those of 4..7: each is one aligned 32-bit word of
// the natural [row][K/32] scale layout, and the instruction's byte select picks step s. The sum
// over K is unchanged by this order; it is the same for the weight and the row operand.
//
// Tile table. A small kernel turns the device-side offsets into a list of (expert, first row) M
// tiles; the GEMM grid is sized for the worst case (ceil(R/128) + E_loc tiles) and surplus
// workgroups find an empty entry and exit, so the host never reads the counts.
#include "moe_gemm_big.h"

namespace moe {
namespace {

constexpr int kBM = 128;       // routed rows per tile
constexpr int kBN = 128;       // weight rows (output columns) per tile
constexpr int kThreads = 256;  // 4 waves, 2 x 2
constexpr int kRowBytes = 128; // K bytes per row per stage
constexpr int kStageBytes = (kBM + kBN) * kRowBytes;

__device__ __forceinline__ int swz(int row, int slot) { return slot ^ (row & 7); }

// Byte offset inside a row of the 16-byte slot `c` (0..7) of stage kt.
template <bool MX>
__device__ __forceinline__ int stage_slot_offset(int kt, int c) {
  if constexpr (MX) {
    // stage kt is half (kt & 1) of chunk kt >> 1: K bytes [64h, 64h+64) and [128+64h, 128+64h+64)
    return 256 * (kt >> 1) + 64 * (kt & 1) + (c < 4 ? 16 * c : 128 + 16 * (c - 4));
  } else {
    return kRowBytes * kt + 16 * c;
  }
}

template <bool MX, bool SWIGLU>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs p) {
  const int2 te = p.tiles[blockIdx.x];
  if (te.x < 0) return;  // surplus workgroup: the whole block leaves before any barrier
  const int e = te.x;
  const int row0 = te.y;
  const int row_end = p.offsets[e + 1];
  const int n0 = blockIdx.y * kBN;

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave >> 1;  // weight-row half of the tile
  const int wm = wave & 1;   // routed-row half of the tile
  const int li = lane & 31;
  const int g = lane >> 5;

  const size_t elem = MX ? 1 : 2;
  const size_t ldk = (size_t)p.K * elem;  // bytes per row
  const uint8_t* wexp = p.w + (size_t)e * p.w_stride;

  // global -> LDS loader: thread copies slot (tid & 7) of rows (tid >> 3) + 32 q
  const int lrow = tid >> 3;
  const int lc = tid & 7;
  const uint8_t* gr[4];
  const uint8_t* gw[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int r = row0 + lrow + 32 * q;
    r = r < row_end ? r : row_end - 1;  // rows past the expert's end are never stored
    gr[q] = p.rows + (size_t)r * ldk;
    gw[q] = wexp + (size_t)(n0 + lrow + 32 * q) * ldk;
  }
  uint4 ra[4], rw[4];
  auto gload = [&](int kt) {
    const int off = stage_slot_offset<MX>(kt, lc);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ra[q] = *reinterpret_cast<const uint4*>(gr[q] + off);
      rw[q] = *reinterpret_cast<const uint4*>(gw[q] + off);
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* base = lds + buf * kStageBytes;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = lrow + 32 * q;
      *reinterpret_cast<uint4*>(base + r * kRowBytes + 16 * swz(r, lc)) = ra[q];
      *reinterpret_cast<uint4*>(base + (kBM + r) * kRowBytes + 16 * swz(r, lc)) = rw[q];
    }
  };

  // MX scale words: per chunk c, lane (li, g) needs byte block [8c + 4g, 8c + 4g + 4) of its rows
  const uint8_t* srow[2] = {nullptr, nullptr};
  const uint8_t* sw[2] = {nullptr, nullptr};
  int sc_r[2] = {0, 0}, sc_w[2] = {0, 0};
  const size_t lds_s = (size_t)p.K / kMxBlock;  // scale bytes per row
  if constexpr (MX) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int r = row0 + wm * 64 + i * 32 + li;
      r = r < row_end ? r : row_end - 1;
      srow[i] = p.row_scales + (size_t)r * lds_s + 4 * g;
      sw[i] = p.w_scales + (size_t)e * p.ws_stride + (size_t)(n0 + wn * 64 + i * 32 + li) * lds_s +
              4 * g;
    }
  }
  auto sload = [&](int c) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      sc_r[i] = *reinterpret_cast<const int*>(srow[i] + 8 * c);
      sc_w[i] = *reinterpret_cast<const int*>(sw[i] + 8 * c);
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)(ldk / kRowBytes);  // stages
  gload(0);
  lstore(0);
  if constexpr (MX) sload(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    int nsc_r[2] = {sc_r[0], sc_r[1]}, nsc_w[2] = {sc_w[0], sc_w[1]};
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* A = lds + buf * kStageBytes + kBM * kRowBytes;  // weight rows (MFMA A)
    const uint8_t* B = lds + buf * kStageBytes;                    // routed rows (MFMA B)
    if constexpr (!MX) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8_t af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int ra_ = wn * 64 + i * 32 + li;
          const int rb_ = wm * 64 + i * 32 + li;
          af[i] = *reinterpret_cast<const bf16x8_t*>(A + ra_ * kRowBytes + 16 * swz(ra_, 2 * kk + g));
          bfr[i] = *reinterpret_cast<const bf16x8_t*>(B + rb_ * kRowBytes + 16 * swz(rb_, 2 * kk + g));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    } else {
      // the next chunk's scale words, fetched while this stage computes
      if ((kt & 1) && kt + 1 < nk) {
        sload((kt + 1) >> 1);
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        i32x8_t af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int ra_ = wn * 64 + i * 32 + li;
          const int rb_ = wm * 64 + i * 32 + li;
          const i32x4_t a0 = *reinterpret_cast<const i32x4_t*>(A + ra_ * kRowBytes + 16 * swz(ra_, 2 * s2 + g));
          const i32x4_t a1 = *reinterpret_cast<const i32x4_t*>(A + ra_ * kRowBytes + 16 * swz(ra_, 4 + 2 * s2 + g));
          const i32x4_t b0 = *reinterpret_cast<const i32x4_t*>(B + rb_ * kRowBytes + 16 * swz(rb_, 2 * s2 + g));
          const i32x4_t b1 = *reinterpret_cast<const i32x4_t*>(B + rb_ * kRowBytes + 16 * swz(rb_, 4 + 2 * s2 + g));
          af[i] = (i32x8_t){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          bfr[i] = (i32x8_t){b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        }
        // step s = 2 * (kt & 1) + s2 of the chunk selects scale byte s
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if (kt & 1) {
              acc[i][j] = s2 == 0 ? mfma_mx<2>(af[i], bfr[j], acc[i][j], nsc_w[i], nsc_r[j])
                                  : mfma_mx<3>(af[i], bfr[j], acc[i][j], nsc_w[i], nsc_r[j]);
            } else {
              acc[i][j] = s2 == 0 ? mfma_mx<0>(af[i], bfr[j], acc[i][j], nsc_w[i], nsc_r[j])
                                  : mfma_mx<1>(af[i], bfr[j], acc[i][j], nsc_w[i], nsc_r[j]);
            }
          }
      }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------------------- epilogue
  // acc[i][j][q]: weight row n = n0 + wn*64 + i*32 + (q/4)*8 + g*4 + (q%4),
  //               routed row r = row0 + wm*64 + j*32 + li.
  if constexpr (SWIGLU) {
    // tile columns n0 + wn*64 + [0, 32) are gate columns, [32, 64) the up columns of the same
    // 32 H columns: col0 = (n0 + wn*64) / 2
    const int col0 = (n0 + wn * 64) >> 1;
    const int Hn = p.N >> 1;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = row0 + wm * 64 + j * 32 + li;
      float hv[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) hv[q] = silu_f(acc[0][j][q]) * acc[1][j][q];
      if constexpr (!MX) {
        if (r < row_end) {
          uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + (size_t)r * Hn + col0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            uint2 v;
            v.x = pack_bf16x2(hv[4 * b + 0], hv[4 * b + 1]);
            v.y = pack_bf16x2(hv[4 * b + 2], hv[4 * b + 3]);
            *reinterpret_cast<uint2*>(out + b * 8 + g * 4) = v;
          }
        }
      } else {
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 16; ++q) amax = fmaxf(amax, fabsf(hv[q]));
        amax = fmaxf(amax, __shfl_xor(amax, 32));  // the other 16 columns of the block
        const int s = mx_block_exponent(amax);
        const float inv = mx_inv_scale(s);
        if (r < row_end) {
          uint8_t* out = reinterpret_cast<uint8_t*>(p.out) + (size_t)r * Hn + col0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            uint32_t w4 = e4m3_pack4(hv[4 * b + 0] * inv, hv[4 * b + 1] * inv,
                                     hv[4 * b + 2] * inv, hv[4 * b + 3] * inv);
            *reinterpret_cast<uint32_t*>(out + b * 8 + g * 4) = w4;
          }
          if (g == 0) p.out_scales[(size_t)r * (Hn / kMxBlock) + (col0 >> 5)] = (uint8_t)(s + 127);
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = row0 + wm * 64 + j * 32 + li;
      if (r >= row_end) continue;
      uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + (size_t)r * p.N + n0 + wn * 64;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          uint2 v;
          v.x = pack_bf16x2(acc[i][j][4 * b + 0], acc[i][j][4 * b + 1]);
          v.y = pack_bf16x2(acc[i][j][4 * b + 2], acc[i][j][4 * b + 3]);
          *reinterpret_cast<uint2*>(out + i * 32 + b * 8 + g * 4) = v;
        }
    }
  }
}


// one large tile per workgroup; workgroup L runs on XCD L % 8
template <int MODE, bool MX, int BM, int RB, int NS, int NSR>
__global__ __launch_bounds__(256, 1) void grouped_gemm_big_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[big_lds_bytes(BM, RB, NS, NSR)];
  big_tile<MODE, MX, BM, RB, NS, NSR>(p, blockIdx.x & 7, blockIdx.x >> 3, lds);
}

// The same with two workgroups per CU (at most 80 KB of LDS and 256 registers each, fragments
// read per k-step): the weight gradients, whose tiles reduce over a short K and end in a large
// float32 store, so one workgroup's stores drain while the other's loads and MFMAs run.
template <int MODE, bool MX, int BM, int RB, int NS, int NSR>
__global__ __launch_bounds__(256, 2) void grouped_gemm_big_kernel_occ2(GemmArgs p) {
  static_assert(big_lds_bytes(BM, RB, NS, NSR) <= 80 * 1024, "two workgroups per CU");
  __shared__ __attribute__((aligned(16))) uint8_t lds[big_lds_bytes(BM, RB, NS, NSR)];
  big_tile<MODE, MX, BM, RB, NS, NSR, false>(p, blockIdx.x & 7, blockIdx.x >> 3, lds);
}

// One workgroup: M tiles of bm rows per expert from the device-side offsets, written as
// (expert, first row) entries; entries past the total are (-1, 0).
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* __restrict__ offsets,
                                                          int E_loc, int bm, int max_tiles,
                                                          int2* __restrict__ tiles,
                                                          int* __restrict__ tile_count) {
  __shared__ int sbase[1025];
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  // experts per thread: E_loc <= 1024
  int nt = 0;
  if (tid < E_loc) nt = (offsets[tid + 1] - offsets[tid] + bm - 1) / bm;
  // inclusive scan over 1024 threads (wave scan + wave totals)
  int v = nt;
  const int lane = tid & 63, wid = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      int t = wsum[w];
      wsum[w] = run;
      run += t;
    }
    sbase[1024] = run;
  }
  __syncthreads();
  const int incl = v + wsum[wid];
  const int base = incl - nt;
  if (tid < E_loc) {
    const int r0 = offsets[tid];
    for (int t = 0; t < nt; ++t) tiles[base + t] = make_int2(tid, r0 + t * bm);
  }
  const int total = sbase[1024];
  if (tid == 0) *tile_count = total;
  for (int i = total + tid; i < max_tiles; i += 1024) tiles[i] = make_int2(-1, 0);
}

// ------------------------------------------------------------------------------------------------
// Weight preparation: transpose [K][Ns] source columns into weight rows [Nout][K], placing source
// column n at row (n / 32) * row_stride + row_off + n % 32; MX variant quantises each row per 32
// along K. One workgroup per 64 (K) x 64 (n) tile.
// ------------------------------------------------------------------------------------------------
template <bool MX>
__global__ __launch_bounds__(256) void prep_transpose_kernel(const uint16_t* __restrict__ src,
                                                             int K, int Ns, size_t src_stride,
                                                             uint8_t* __restrict__ dst,
                                                             uint8_t* __restrict__ dst_scales,
                                                             size_t dst_stride,
                                                             size_t dsts_stride, int row_stride,
                                                             int row_off, int sc_cm, int n_rows,
                                                             int tiled) {
  __shared__ float tile[64][65];
  const int e = blockIdx.z;
  const int k0 = blockIdx.y * 64;
  const int c0 = blockIdx.x * 64;
  const uint16_t* s = src + (size_t)e * src_stride;
  const int tid = threadIdx.x;
  for (int i = tid; i < 64 * 64; i += 256) {
    const int kk = i >> 6, cc = i & 63;
    tile[kk][cc] = bf16_to_f32(s[(size_t)(k0 + kk) * Ns + c0 + cc]);
  }
  __syncthreads();
  // byte address of byte kb of destination row orow: natural orow * K bytes + kb, or K-tiled
  // (256-row panels, 128-byte stages; n_rows % 256 == 0 and the row's bytes % 128 == 0)
  const size_t rowb = (size_t)K * (MX ? 1 : 2);
  auto at = [&](int orow, size_t kb) -> size_t {
    if (!tiled) return (size_t)orow * rowb + kb;
    return (((size_t)(orow >> 8) * (rowb >> 7) + (kb >> 7)) * 256 + (orow & 255)) * 128 + (kb & 127);
  };
  if constexpr (!MX) {
    uint8_t* d = dst + (size_t)e * dst_stride;
    for (int i = tid; i < 64 * 64; i += 256) {
      const int cc = i >> 6, kk = i & 63;
      const int n = c0 + cc;
      const int orow = (n >> 5) * row_stride + row_off + (n & 31);
      *reinterpret_cast<uint16_t*>(d + at(orow, (size_t)2 * (k0 + kk))) =
          (uint16_t)f32_to_bf16_bits(tile[kk][cc]);
    }
  } else {
    if (tid < 128) {
      const int cc = tid >> 1, half = tid & 1;
      const int n = c0 + cc;
      const int orow = (n >> 5) * row_stride + row_off + (n & 31);
      float amax = 0.0f;
      for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(tile[half * 32 + q][cc]));
      const int sx = mx_block_exponent(amax);
      const float inv = mx_inv_scale(sx);
      uint8_t* d = dst + (size_t)e * dst_stride + at(orow, (size_t)k0 + half * 32);
      for (int q = 0; q < 32; ++q) d[q] = (uint8_t)e4m3_encode(tile[half * 32 + q][cc] * inv);
      const int kb = (k0 >> 5) + half;  // MX block along K
      const size_t so = sc_cm ? ((size_t)(kb >> 3) * n_rows + orow) * 8 + (kb & 7)
                              : (size_t)orow * (K / kMxBlock) + kb;
      dst_scales[(size_t)e * dsts_stride + so] = (uint8_t)(sx + 127);
    }
  }
}

struct PreparedLayout {
  size_t w1, w1s, w2, w2s, total;
};

PreparedLayout prepared_layout(int E_loc, int h, int m, bool mx) {
  PreparedLayout L{};
  const size_t el = mx ? 1 : 2;
  size_t off = 0;
  L.w1 = off;
  off = align_up(off + (size_t)E_loc * 2 * m * h * el);
  if (mx) {
    L.w1s = off;
    off = align_up(off + (size_t)E_loc * 2 * m * (h / kMxBlock));
  }
  L.w2 = off;
  off = align_up(off + (size_t)E_loc * h * m * el);
  if (mx) {
    L.w2s = off;
    off = align_up(off + (size_t)E_loc * h * (m / kMxBlock));
  }
  L.total = off;
  return L;
}

struct FfnLayout {
  size_t count, tiles, H, Hs, Rs, total;
  int max_tiles;
};

// rows per M tile: the large-tile kernel (h % 256 == 0, m % 128 == 0) takes 256 rows (BF16) when
// the experts hold 224 rows or more on average and there are enough tiles, 192 rows (MXFP8) from
// 128 rows on average, else 128; the small-tile kernel always 128
int ffn_tile_rows(int R, int h, int m, int E_loc, bool mx) {
  if (h % kBigBN || (2 * m) % kBigBN) return kBM;
  // MXFP8: a 256-row tile does not fit the register file; 192 rows (three 32-row fragments per
  // wave) does, and wastes less on experts of a few hundred rows than two 128-row tiles
  if (mx) return (R / E_loc >= 128) ? 192 : 128;
  // BF16: 256 rows when the experts are large enough and the 256-row tiles still give every CU
  // a tile (a launch of fewer tiles than CUs, e.g. the shared expert over 2048 tokens, runs
  // faster as twice as many 128-row tiles)
  const long long tiles256 = (long long)((R + 255) / 256) * ((2 * m) / kBigBN);
  return (R / E_loc >= 224 && tiles256 >= 256) ? 256 : 128;
}

// natural [R][K/32] scales -> chunk-major [K/256][R][8]; one thread per (row, chunk), rows fastest
// so the writes are contiguous (K % 256 == 0)
__global__ __launch_bounds__(256) void scales_chunk_major_kernel(const uint8_t* __restrict__ src,
                                                                 int R, int K,
                                                                 uint8_t* __restrict__ dst) {
  const int nc = K / 256;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)R * nc) return;
  const int r = (int)(i % R), cc = (int)(i / R);
  const uint2 v = *reinterpret_cast<const uint2*>(src + (size_t)r * (K / kMxBlock) + 8 * cc);
  *reinterpret_cast<uint2*>(dst + ((size_t)cc * R + r) * 8) = v;
}

FfnLayout ffn_layout(int R, int h, int m, int E_loc, bool mx) {
  FfnLayout L{};
  // room for 128-row tiles, the smallest any launch takes
  L.max_tiles = (R + kBM - 1) / kBM + E_loc;
  size_t off = 0;
  L.count = off;
  off = align_up(off + sizeof(int));
  L.tiles = off;
  off = align_up(off + (size_t)L.max_tiles * sizeof(int2));
  L.H = off;
  off = align_up(off + (size_t)R * m * (mx ? 1 : 2));
  if (mx) {
    L.Hs = off;
    off = align_up(off + (size_t)R * (m / kMxBlock));
    L.Rs = off;  // the routed rows' scales, chunk-major (large-tile kernel)
    off = align_up(off + (size_t)R * (h / kMxBlock));
  }
  L.total = off;
  return L;
}

}  // namespace

bool ffn_big(int h, int m) { return h % kBigBN == 0 && (2 * m) % kBigBN == 0; }


size_t prepared_bytes(int E_loc, int h, int m, bool mx) {
  return prepared_layout(E_loc, h, m, mx).total;
}

size_t ffn_workspace_bytes(int R, int h, int m, int E_loc, bool mx) {
  return ffn_layout(R, h, m, E_loc, mx).total;
}

hipError_t launch_prepare_weights(const uint16_t* w_gate, const uint16_t* w_up,
                                  const uint16_t* w_down, void* prepared, int E_loc, int h, int m,
                                  bool mx, hipStream_t st) {
  const PreparedLayout L = prepared_layout(E_loc, h, m, mx);
  uint8_t* base = reinterpret_cast<uint8_t*>(prepared);
  const size_t el = mx ? 1 : 2;
  // W1 rows: gate column n -> 64 (n/32) + n%32, up column n -> 64 (n/32) + 32 + n%32; K = h
  dim3 g1(m / 64, h / 64, E_loc);
  const size_t s1 = (size_t)h * m;
  const size_t d1 = (size_t)2 * m * h * el, d1s = (size_t)2 * m * (h / kMxBlock);
  dim3 g2(h / 64, m / 64, E_loc);
  const size_t s2 = (size_t)m * h;
  const size_t d2 = (size_t)h * m * el, d2s = (size_t)h * (m / kMxBlock);
  // the large-tile kernel reads K-tiled codes and chunk-major scales, the small one natural ones
  const int big = ffn_big(h, m) ? 1 : 0;
  if (mx) {
    hipLaunchKernelGGL(prep_transpose_kernel<true>, g1, dim3(256), 0, st, w_gate, h, m, s1,
                       base + L.w1, base + L.w1s, d1, d1s, 64, 0, big, 2 * m, big);
    hipLaunchKernelGGL(prep_transpose_kernel<true>, g1, dim3(256), 0, st, w_up, h, m, s1,
                       base + L.w1, base + L.w1s, d1, d1s, 64, 32, big, 2 * m, big);
    hipLaunchKernelGGL(prep_transpose_kernel<true>, g2, dim3(256), 0, st, w_down, m, h, s2,
                       base + L.w2, base + L.w2s, d2, d2s, 32, 0, big, h, big);
  } else {
    hipLaunchKernelGGL(prep_transpose_kernel<false>, g1, dim3(256), 0, st, w_gate, h, m, s1,
                       base + L.w1, nullptr, d1, 0, 64, 0, 0, 0, big);
    hipLaunchKernelGGL(prep_transpose_kernel<false>, g1, dim3(256), 0, st, w_up, h, m, s1,
                       base + L.w1, nullptr, d1, 0, 64, 32, 0, 0, big);
    hipLaunchKernelGGL(prep_transpose_kernel<false>, g2, dim3(256), 0, st, w_down, m, h, s2,
                       base + L.w2, nullptr, d2, 0, 32, 0, 0, 0, big);
  }
  return hipGetLastError();
}

// kernels launched by name in non-template functions, so that each instantiation is compiled for
// the device
#define MOE_BIG(MODEV, MXV, BMV, G, A)                                                          \
  hipLaunchKernelGGL((grouped_gemm_big_kernel<MODEV, MXV, BMV, kBigRB, big_ns(MXV, BMV),        \
                                              big_nsr(MXV, BMV)>),                              \
                     G, dim3(256), 0, st, A)

// weight gradients: 64-row tiles, two-deep rings, two workgroups per CU (moe_gemm_plan.h)
#define MOE_BIG_OCC2(MODEV, MXV, G, A)                                                          \
  hipLaunchKernelGGL((grouped_gemm_big_kernel_occ2<MODEV, MXV, kWgradRows, kBigRB, kWgradNS,    \
                                                   kWgradNSR>),                                 \
                     G, dim3(256), 0, st, A)

// grid of the large-tile kernel for at most max_mt M tiles and nt N tiles: per XCD at most
// ceil(tiles / 8) plus one per band, and a multiple of 8 for the XCD remap
static dim3 big_grid(int max_mt, int nt) {
  return dim3(8 * big_grid_per_xcd(max_mt, nt));
}

// the fields of the forward FFN's two GEMMs common to both kernels
static void ffn_gemm_args(const void* rows, const uint8_t* row_scales, const int32_t* offsets,
                          const void* prepared, uint16_t* out_rows, void* ws, int R, int h, int m,
                          int E_loc, bool mx, GemmArgs& a1, GemmArgs& a2) {
  const PreparedLayout P = prepared_layout(E_loc, h, m, mx);
  const FfnLayout F = ffn_layout(R, h, m, E_loc, mx);
  const uint8_t* pw = reinterpret_cast<const uint8_t*>(prepared);
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  const size_t el = mx ? 1 : 2;
  a1 = GemmArgs{};
  a1.rows = reinterpret_cast<const uint8_t*>(rows);
  a1.row_scales = row_scales;
  a1.w = pw + P.w1;
  a1.w_scales = mx ? pw + P.w1s : nullptr;
  a1.w_stride = (size_t)2 * m * h * el;
  a1.ws_stride = (size_t)2 * m * (h / kMxBlock);
  a1.offsets = offsets;
  a1.tiles = reinterpret_cast<int2*>(w + F.tiles);
  a1.tile_count = reinterpret_cast<int*>(w + F.count);
  a1.K = h;
  a1.N = 2 * m;
  a1.out = w + F.H;
  a1.out_scales = mx ? w + F.Hs : nullptr;

  a2 = GemmArgs{};
  a2.rows = w + F.H;
  a2.row_scales = mx ? w + F.Hs : nullptr;
  a2.w = pw + P.w2;
  a2.w_scales = mx ? pw + P.w2s : nullptr;
  a2.w_stride = (size_t)h * m * el;
  a2.ws_stride = (size_t)h * (m / kMxBlock);
  a2.offsets = offsets;
  a2.tiles = a1.tiles;
  a2.tile_count = a1.tile_count;
  a2.K = m;
  a2.N = h;
  a2.out = out_rows;
  a2.out_scales = nullptr;
}

// the large-tile kernel's fields: K-tiled weights, GEMM-1 rows through row_src, MX scales
// chunk-major (the input's over n_src rows)
static void big_gemm_args(const uint8_t* row_scales_cm, int n_src, int R, bool mx,
                          const int32_t* row_src, int row_div, GemmArgs& a1, GemmArgs& a2) {
  a1.w_tiled = a2.w_tiled = 1;
  a1.row_src = row_src;  // GEMM-1 may read its rows through an index (GEMM-2 reads H)
  a1.row_div = row_div;
  if (mx) {
    a1.row_scales = row_scales_cm;
    a1.w_sc_cm = a1.r_sc_cm = a1.out_sc_cm = 1;
    a1.sc_rows = n_src;
    a1.out_sc_rows = R;
    a2.w_sc_cm = a2.r_sc_cm = 1;
    a2.sc_rows = R;
  }
}

int ffn_big_gemm_args(const void* rows, const uint8_t* row_scales, int row_scales_rows,
                      const int32_t* offsets, const void* prepared, uint16_t* out_rows, void* ws,
                      int R, int h, int m, int E_loc, bool mx, const int32_t* row_src,
                      int row_div, int bm, GemmArgs& a1, GemmArgs& a2) {
  ffn_gemm_args(rows, row_scales, offsets, prepared, out_rows, ws, R, h, m, E_loc, mx, a1, a2);
  big_gemm_args(row_scales, row_scales_rows, R, mx, row_src, row_div, a1, a2);
  return (R + bm - 1) / bm + E_loc;  // at most ffn_layout's capacity for bm >= 128
}

hipError_t launch_expert_ffn(const void* rows, const uint8_t* row_scales, const int32_t* offsets,
                             const void* prepared, uint16_t* out_rows, void* ws, int R, int h,
                             int m, int E_loc, bool mx, hipStream_t st, const hipEvent_t* ev,
                             float* gu_out, const int32_t* row_src, int row_div, int src_rows,
                             bool scales_cm) {
  const bool save = gu_out != nullptr;
  // a forward that keeps G and U takes 128-row tiles (the 256-row BF16 variant with the extra
  // stores does not fit the register file)
  const int bm = save ? kBM : ffn_tile_rows(R, h, m, E_loc, mx);
  const int max_tiles = (R + bm - 1) / bm + E_loc;
  const FfnLayout F = ffn_layout(R, h, m, E_loc, mx);
  const bool big = ffn_big(h, m);
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  GemmArgs a1{}, a2{};
  ffn_gemm_args(rows, row_scales, offsets, prepared, out_rows, ws, R, h, m, E_loc, mx, a1, a2);
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, st, offsets, E_loc, bm,
                     max_tiles, reinterpret_cast<int2*>(w + F.tiles),
                     reinterpret_cast<int*>(w + F.count));
  if (ev) (void)hipEventRecord(ev[0], st);

  if (big) {
    const dim3 g1 = big_grid(max_tiles, (2 * m) / kBigBN);
    const dim3 g2 = big_grid(max_tiles, h / kBigBN);
    const int n_src = row_src ? src_rows : R;  // rows of `rows` and of its scales
    const uint8_t* rs = row_scales;
    if (mx && !scales_cm) {  // chunk-major scales throughout: weights (prepared so), rows, and H
      const long long units = (long long)n_src * (h / 256);
      hipLaunchKernelGGL(scales_chunk_major_kernel, dim3((unsigned)((units + 255) / 256)),
                         dim3(256), 0, st, row_scales, n_src, h, w + F.Rs);
      rs = w + F.Rs;
    }
    big_gemm_args(rs, n_src, R, mx, row_src, row_div, a1, a2);
    a1.gu_out = gu_out;
    a1.band_gm = band_groups_for((2 * m) / kBigBN, bm, R / E_loc);
    a2.band_gm = band_groups_for(h / kBigBN, bm, R / E_loc);
    if (mx && bm == 192) {  // never with save
      MOE_BIG(kEpiSwiglu, true, 192, g1, a1);
      if (ev) (void)hipEventRecord(ev[1], st);
      MOE_BIG(kEpiStore, true, 192, g2, a2);
    } else if (mx) {
      if (save) MOE_BIG(kEpiSwigluSave, true, 128, g1, a1);
      else MOE_BIG(kEpiSwiglu, true, 128, g1, a1);
      if (ev) (void)hipEventRecord(ev[1], st);
      MOE_BIG(kEpiStore, true, 128, g2, a2);
    } else if (bm == 256) {  // never with save
      MOE_BIG(kEpiSwiglu, false, 256, g1, a1);
      if (ev) (void)hipEventRecord(ev[1], st);
      MOE_BIG(kEpiStore, false, 256, g2, a2);
    } else {
      if (save) MOE_BIG(kEpiSwigluSave, false, 128, g1, a1);
      else MOE_BIG(kEpiSwiglu, false, 128, g1, a1);
      if (ev) (void)hipEventRecord(ev[1], st);
      MOE_BIG(kEpiStore, false, 128, g2, a2);
    }
    if (ev) (void)hipEventRecord(ev[2], st);
    return hipGetLastError();
  }
  // G and U are only kept, rows only gathered through an index, by the large-tile kernel
  if (gu_out || row_src) return hipErrorInvalidValue;
  dim3 grid1(max_tiles, (2 * m) / kBN);
  dim3 grid2(max_tiles, h / kBN);
  if (mx)
    hipLaunchKernelGGL((grouped_gemm_kernel<true, true>), grid1, dim3(kThreads), 0, st, a1);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<false, true>), grid1, dim3(kThreads), 0, st, a1);
  if (ev) (void)hipEventRecord(ev[1], st);
  if (mx)
    hipLaunchKernelGGL((grouped_gemm_kernel<true, false>), grid2, dim3(kThreads), 0, st, a2);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<false, false>), grid2, dim3(kThreads), 0, st, a2);
  if (ev) (void)hipEventRecord(ev[2], st);
  return hipGetLastError();
}

hipError_t launch_tile_table(const int32_t* offsets, int E_loc, int bm, int max_tiles,
                             int2* tiles, int* tile_count, hipStream_t st) {
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, st, offsets, E_loc, bm, max_tiles,
                     tiles, tile_count);
  return hipGetLastError();
}

// the backward's routed-row GEMMs (dH with the SwiGLU-backward epilogue, dA with the store
// epilogue) take the forward GEMM-2's 192-row MXFP8 tile when the experts hold 128 rows or more on
// average, else 128-row tiles (BF16 always: its 256-row tile leaves no room for the
// SwiGLU-backward epilogue beside the accumulators)
constexpr int kBwdBM = 128;

static int bwd_tile_rows(int R, int E_loc, bool mx) {
  return (mx && R / E_loc >= 128) ? 192 : kBwdBM;
}

// the tile table: the count, then room for (R / 128 + E_loc) entries (any tile height >= 128)
size_t gemm_tiles_bytes(int R, int E_loc) {
  return align_up(sizeof(int)) + (size_t)((R + kBwdBM - 1) / kBwdBM + E_loc) * sizeof(int2);
}

hipError_t launch_gemm_tiles(const int32_t* offsets, void* tiles_ws, int R, int E_loc,
                             bool mx, hipStream_t st) {
  const int bm = bwd_tile_rows(R, E_loc, mx);
  const int max_tiles = (R + bm - 1) / bm + E_loc;
  uint8_t* tw = reinterpret_cast<uint8_t*>(tiles_ws);
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, st, offsets, E_loc, bm, max_tiles,
                     reinterpret_cast<int2*>(tw + align_up(sizeof(int))),
                     reinterpret_cast<int*>(tw));
  return hipGetLastError();
}

hipError_t launch_bwd_dgrad(const void* dO, const uint8_t* dO_s, const int32_t* offsets,
                            const uint8_t* w2b, const uint8_t* w2b_s, const uint8_t* w1b,
                            const uint8_t* w1b_s, const float* gu, void* dgu, uint8_t* dgu_s,
                            float* dgu_f32, uint16_t* dA, const void* tiles_ws, int R, int h,
                            int m, int E_loc, bool mx, hipStream_t st, hipEvent_t ev_mid) {
  if (!ffn_big(h, m) || m % kBigBN) return hipErrorInvalidValue;
  const int bm = bwd_tile_rows(R, E_loc, mx);
  const int max_tiles = (R + bm - 1) / bm + E_loc;
  const uint8_t* tw = reinterpret_cast<const uint8_t*>(tiles_ws);
  const int* tile_count = reinterpret_cast<const int*>(tw);
  const int2* tiles = reinterpret_cast<const int2*>(tw + align_up(sizeof(int)));
  const size_t el = mx ? 1 : 2;

  // dH = dO W_down^T (K = h, N = m) with the SwiGLU backward in the epilogue -> dG | dU
  GemmArgs a{};
  a.rows = reinterpret_cast<const uint8_t*>(dO);
  a.row_scales = dO_s;
  a.w = w2b;
  a.w_scales = w2b_s;
  a.w_stride = (size_t)m * h * el;
  a.ws_stride = (size_t)m * (h / kMxBlock);
  a.offsets = offsets;
  a.tiles = tiles;
  a.tile_count = tile_count;
  a.K = h;
  a.N = m;
  a.out = dgu;
  a.out_scales = dgu_s;
  a.gu_in = gu;
  a.d_f32 = dgu_f32;
  // MX: every scale array chunk-major (dO from the un-combine, the backward weights, dG | dU)
  a.w_sc_cm = a.r_sc_cm = a.out_sc_cm = mx ? 1 : 0;
  a.sc_rows = a.out_sc_rows = R;

  // dA = [dG | dU] [W_gate | W_up]^T (K = 2m, interleaved per 32 on both sides, N = h)
  GemmArgs b{};
  b.rows = reinterpret_cast<const uint8_t*>(dgu);
  b.row_scales = dgu_s;
  b.w = w1b;
  b.w_scales = w1b_s;
  b.w_sc_cm = b.r_sc_cm = mx ? 1 : 0;
  b.sc_rows = R;
  b.w_stride = (size_t)h * 2 * m * el;
  b.ws_stride = (size_t)h * (2 * m / kMxBlock);
  b.offsets = offsets;
  b.tiles = tiles;
  b.tile_count = tile_count;
  b.K = 2 * m;
  b.N = h;
  b.out = dA;

  a.band_gm = band_groups_for(m / kBigBN, bm, R / E_loc);
  b.band_gm = band_groups_for(h / kBigBN, bm, R / E_loc);
  const dim3 ga = big_grid(max_tiles, m / kBigBN), gb = big_grid(max_tiles, h / kBigBN);
  if (mx && bm == 192) MOE_BIG(kEpiDSwiglu, true, 192, ga, a);
  else if (mx) MOE_BIG(kEpiDSwiglu, true, kBwdBM, ga, a);
  else MOE_BIG(kEpiDSwiglu, false, kBwdBM, ga, a);
  if (ev_mid) (void)hipEventRecord(ev_mid, st);
  if (mx && bm == 192) MOE_BIG(kEpiStore, true, 192, gb, b);
  else if (mx) MOE_BIG(kEpiStore, true, kBwdBM, gb, b);
  else MOE_BIG(kEpiStore, false, kBwdBM, gb, b);
  return hipGetLastError();
}

hipError_t launch_bwd_wgrad(const uint8_t* At, const uint8_t* At_s, const uint8_t* dGUt,
                            const uint8_t* dGUt_s, const uint8_t* Ht, const uint8_t* Ht_s,
                            const uint8_t* dOt, const uint8_t* dOt_s, const int32_t* koff,
                            void* dw_gate, void* dw_up, void* dw_down, bool out_f32, int h, int m,
                            int E_loc, bool mx, hipStream_t st, hipEvent_t ev_mid) {
  if (h % kBigBN || m % kBigBN) return hipErrorInvalidValue;
  const int bm = kWgradRows;
  // dW_gate | dW_up [e] (h x 2m) = A_e^T [dG | dU]_e: M side A^T (h rows), N side [dG | dU]^T
  GemmArgs a{};
  a.rows = At;
  a.row_scales = At_s;
  a.w = dGUt;
  a.w_scales = dGUt_s;
  a.koff = koff;
  a.M = h;
  a.N = 2 * m;
  a.tiles_total = E_loc * (h / bm);
  a.split_gate_up = 1;
  a.out_f32 = out_f32;
  a.out = dw_gate;
  a.out2 = dw_up;
  a.w_sc_cm = a.r_sc_cm = mx ? 1 : 0;  // per expert segment, [kpad_e/256][C][8]
  a.sc_rows = h;
  // dW_down [e] (m x h) = H_e^T dO_e: M side H^T (m rows), N side dO^T (h rows)
  GemmArgs b{};
  b.rows = Ht;
  b.row_scales = Ht_s;
  b.w = dOt;
  b.w_scales = dOt_s;
  b.koff = koff;
  b.M = m;
  b.N = h;
  b.tiles_total = E_loc * (m / bm);
  b.split_gate_up = 0;
  b.out_f32 = out_f32;
  b.out = dw_down;
  b.w_sc_cm = b.r_sc_cm = mx ? 1 : 0;
  b.sc_rows = m;
  const dim3 ga = big_grid(a.tiles_total, a.N / kBigBN), gb = big_grid(b.tiles_total, b.N / kBigBN);
  if (mx) MOE_BIG_OCC2(kEpiWgrad, true, ga, a);
  else MOE_BIG_OCC2(kEpiWgrad, false, ga, a);
  if (ev_mid) (void)hipEventRecord(ev_mid, st);
  if (mx) MOE_BIG_OCC2(kEpiWgrad, true, gb, b);
  else MOE_BIG_OCC2(kEpiWgrad, false, gb, b);
  return hipGetLastError();
}

#undef MOE_BIG
#undef MOE_BIG_OCC2

}  // namespace moe
