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
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBM = 128;       // routed rows per tile
constexpr int kBN = 128;       // weight rows (output columns) per tile
constexpr int kThreads = 256;  // 4 waves, 2 x 2
constexpr int kRowBytes = 128; // K bytes per row per stage
constexpr int kStageBytes = (kBM + kBN) * kRowBytes;

struct GemmArgs {
  const uint8_t* rows;          // [R][K] bf16 or E4M3 (routed rows)
  const uint8_t* row_scales;    // [R][K/32] (MX)
  const uint8_t* w;             // expert 0 of [E][N][K] weight rows
  const uint8_t* w_scales;      // expert 0 of [E][N][K/32] (MX)
  size_t w_stride;              // bytes between experts (codes / bf16)
  size_t ws_stride;             // bytes between experts (scales)
  const int32_t* offsets;       // [E_loc+1]
  const int2* tiles;            // (expert, first row) per M tile; expert < 0: none
  const int* tile_count;        // number of valid M tiles (large-tile kernel)
  int K;                        // reduction length (elements)
  int N;                        // output columns of this GEMM (weight rows per expert)
  void* out;                    // GEMM-1: H [R][N/2] (bf16 or E4M3); GEMM-2: O [R][N] bf16
  uint8_t* out_scales;          // GEMM-1 MX: H scales [R][N/64]
};

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

template <int OPSEL>
__device__ __forceinline__ f32x16_t mfma_mx(const i32x8_t& a, const i32x8_t& b, f32x16_t c,
                                            int sa, int sb) {
  // format 0 = FP8 E4M3 for both operands; OPSEL picks the scale byte of this step
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPSEL, sa, OPSEL, sb);
}

// the same with the scale byte picked by a value that is constant after unrolling
__device__ __forceinline__ f32x16_t mfma_mx_sel(int sel, const i32x8_t& a, const i32x8_t& b,
                                                f32x16_t c, int sa, int sb) {
  switch (sel) {
    case 0: return mfma_mx<0>(a, b, c, sa, sb);
    case 1: return mfma_mx<1>(a, b, c, sa, sb);
    case 2: return mfma_mx<2>(a, b, c, sa, sb);
    default: return mfma_mx<3>(a, b, c, sa, sb);
  }
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

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
            uint32_t w4 = e4m3_encode(hv[4 * b + 0] * inv) | (e4m3_encode(hv[4 * b + 1] * inv) << 8) |
                          (e4m3_encode(hv[4 * b + 2] * inv) << 16) |
                          (e4m3_encode(hv[4 * b + 3] * inv) << 24);
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


// ------------------------------------------------------------------------------------------------
// Large-tile grouped GEMM: 256 weight rows x BM routed rows (BM = 256 or 128) per workgroup of 4
// waves, each wave 128 x BM/2 as 4 x BM/64 MFMA tiles of 32 x 32 (accumulators live in the
// AccVGPR file). K advances RB bytes per stage (RB = 64 or 128: 32/64 bf16 or 64/128 E4M3).
//
// Operands go global -> LDS directly (global_load_lds_dwordx4), NS stages deep, so no VGPRs hold
// staged data. The compiler does not order these asynchronous LDS writes against the LDS reads, so
// the pipeline waits explicitly: before stage kt is read, s_waitcnt vmcnt(n) with n the exact
// number of loads this wave issued after stage kt's (vmcnt(0) near the end, which is always safe),
// then a barrier so every wave's part of the stage is in LDS and no wave still reads the buffer the
// next load overwrites.
//
// LDS rows are RB bytes, split into 16-byte slots; slot p of row r holds logical chunk p ^ f(r)
// (f(r) = ((r >> 1) ^ (r >> 2)) & 3 for RB = 64, (r ^ (r >> 3)) & 7 for RB = 128), which spreads
// the lanes that read one logical chunk of consecutive rows over distinct bank groups for both
// 8-lane and 16-lane LDS phases. The swizzle is applied on the global side: the DMA writes a
// wave's 64 lanes to 1 KB of consecutive LDS, and each lane fetches the global chunk that belongs
// in its slot.
//
// Work order: workgroup L runs on XCD L % 8; the valid tiles are split into 8 contiguous ranges,
// one per XCD, and inside a range the order walks 4 consecutive M tiles for each N tile, so the 32
// workgroups an XCD runs at once share 4 row panels and 8 weight panels in its L2.
// ------------------------------------------------------------------------------------------------
constexpr int kBigBN = 256;
constexpr int kGroupM = 4;

template <int RB>
__device__ __forceinline__ int big_swz(int row) {
  if constexpr (RB == 64) return ((row >> 1) ^ (row >> 2)) & 3;
  else return (row ^ (row >> 3)) & 7;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_fenced() {
  asm volatile("" ::: "memory");  // no load moves across the count
  wait_vmcnt<N>();
}

// every LDS read of this wave has returned, then all waves meet; no memory access moves across
// 16-byte global -> LDS DMA of one lane (the wave's 64 lanes fill 1 KB of consecutive LDS from
// `l`). The builtin only exists in the device pass; the host pass, which only needs the kernel's
// launch stub, must not see it (it would drop the stub).
__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* l) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
#else
  (void)g;
  (void)l;
#endif
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// stage width and depth per precision (LDS: NS * (256 + BM) * RB bytes, at most 160 KB)
#ifndef MOE_BIG_RB_BF16
#define MOE_BIG_RB_BF16 128
#endif
#ifndef MOE_BIG_NS_BF16
#define MOE_BIG_NS_BF16 2
#endif
#ifndef MOE_BIG_RB_MX
#define MOE_BIG_RB_MX 128
#endif
#ifndef MOE_BIG_NS_MX
#define MOE_BIG_NS_MX 2
#endif
template <bool MX, int BM>
struct BigCfg {
  static constexpr int RB = MX ? MOE_BIG_RB_MX : MOE_BIG_RB_BF16;
  static constexpr int NS = MX ? MOE_BIG_NS_MX : MOE_BIG_NS_BF16;
  static_assert(NS * (kBigBN + BM) * RB <= 160 * 1024, "LDS budget");
};

template <bool MX, bool SWIGLU, int BM, int RB, int NS>
__global__ __launch_bounds__(256, 1) void grouped_gemm_big_kernel(GemmArgs p) {
  constexpr int BN = kBigBN;
  constexpr int ROWS = BN + BM;
  constexpr int STAGE = ROWS * RB;
  constexpr int NI = 4;                          // weight fragments per wave
  constexpr int NJ = BM / 64;                    // row fragments per wave
  constexpr int LOADS = ROWS * RB / 16 / 256;    // 16-byte DMA loads per thread per stage
  constexpr int SLOTS = RB / 16;
  constexpr int SPS = MX ? RB / 64 : RB / 32;    // MFMA k-steps per stage
  constexpr int PER_CHUNK = MX ? 4 / SPS : 1;    // stages per 256-element MX chunk
  constexpr int NSC = MX ? NI + NJ : 0;          // scale loads per chunk
  static_assert(LOADS * (NS - 2) + NSC < 64, "vmcnt range");
  static_assert(!MX || NS - 1 <= PER_CHUNK, "scale prefetch distance");
  __shared__ __attribute__((aligned(16))) uint8_t lds[NS * STAGE];

  // ---- which tile: XCD-contiguous ranges, grouped M order
  const int mt_total = *p.tile_count;
  const int Nt = p.N / BN;
  const int total = mt_total * Nt;
  const int per_xcd = (total + 7) >> 3;
  const int L = blockIdx.x;
  if ((L >> 3) >= per_xcd) return;
  const int logical = (L & 7) * per_xcd + (L >> 3);
  if (logical >= total) return;
  const int gm0 = (logical / (kGroupM * Nt)) * kGroupM;
  const int gsz = min(kGroupM, mt_total - gm0);
  const int rr = logical - gm0 * Nt;
  const int nt = rr / gsz;
  const int2 te = p.tiles[gm0 + rr % gsz];
  const int e = te.x;
  const int row0 = te.y;
  const int row_end = p.offsets[e + 1];
  const int n0 = nt * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave >> 1;
  const int wm = wave & 1;
  const int li = lane & 31;
  const int g = lane >> 5;

  const size_t ldk = (size_t)p.K * (MX ? 1 : 2);
  const uint8_t* wexp = p.w + (size_t)e * p.w_stride;

  // ---- DMA sources: unit id = q * 256 + tid lands at stage byte id * 16 = LDS row id / SLOTS,
  //      physical slot id % SLOTS, and must carry logical chunk slot ^ f(row)
  const uint8_t* src[LOADS];
#pragma unroll
  for (int q = 0; q < LOADS; ++q) {
    const int id = q * 256 + tid;
    const int row = id / SLOTS;
    const int c = (id % SLOTS) ^ big_swz<RB>(row);
    const uint8_t* base;
    if (row < BN) {
      base = wexp + (size_t)(n0 + row) * ldk;
    } else {
      int r = row0 + row - BN;
      r = r < row_end ? r : row_end - 1;  // rows past the expert's end are never stored
      base = p.rows + (size_t)r * ldk;
    }
    if constexpr (MX) src[q] = base + (c < SLOTS / 2 ? 16 * c : 128 + 16 * (c - SLOTS / 2));
    else src[q] = base + 16 * c;
  }
  auto stage_off = [&](int kt) -> size_t {
    // MX: stage kt holds steps s0 .. s0+SPS-1 of chunk kt / PER_CHUNK, i.e. K bytes
    // [256 cc + 32 s0, + 32 SPS) and [256 cc + 128 + 32 s0, + 32 SPS)
    if constexpr (MX) return (size_t)256 * (kt / PER_CHUNK) + 32 * SPS * (kt % PER_CHUNK);
    else return (size_t)RB * kt;
  };
  auto issue = [&](int kt, int buf) {
    const size_t off = stage_off(kt);
#pragma unroll
    for (int q = 0; q < LOADS; ++q)
      dma16(src[q] + off, lds + buf * STAGE + q * 4096 + wave * 1024);
  };

  // ---- MX scale words: one 32-bit word (scale bytes of blocks 4g .. 4g+3 of the chunk) per
  //      fragment row and chunk
  const uint8_t* sw_ptr[NI];
  const uint8_t* sr_ptr[NJ];
  int scw[NI], scr[NJ], nscw[NI], nscr[NJ];
  if constexpr (MX) {
    const size_t nsb = (size_t)p.K / kMxBlock;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      sw_ptr[i] = p.w_scales + (size_t)e * p.ws_stride +
                  (size_t)(n0 + 128 * wn + 32 * i + li) * nsb + 4 * g;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      int r = row0 + (BM / 2) * wm + 32 * j + li;
      r = r < row_end ? r : row_end - 1;
      sr_ptr[j] = p.row_scales + (size_t)r * nsb + 4 * g;
    }
  }
  auto sload = [&](int cc, int (&w)[NI], int (&r)[NJ]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) w[i] = *reinterpret_cast<const int*>(sw_ptr[i] + 8 * cc);
#pragma unroll
    for (int j = 0; j < NJ; ++j) r[j] = *reinterpret_cast<const int*>(sr_ptr[j] + 8 * cc);
  };

  // ---- fragment byte offsets inside a stage: row * RB + 16 * (c ^ f(row)) == fb ^ (16 c)
  int fbw[NI], fbr[NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = 128 * wn + 32 * i + li;
    fbw[i] = row * RB + 16 * big_swz<RB>(row);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int row = BN + (BM / 2) * wm + 32 * j + li;
    fbr[j] = row * RB + 16 * big_swz<RB>(row);
  }

  f32x16_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // MFMAs of one stage; S0 = the MX chunk step of the stage's first k-step
  auto compute = [&](const uint8_t* b, auto s0_tag) {
    constexpr int S0 = decltype(s0_tag)::value;
#pragma unroll
    for (int t = 0; t < SPS; ++t) {
      if constexpr (!MX) {
        bf16x8_t wf[NI], rf[NJ];
#pragma unroll
        for (int i = 0; i < NI; ++i)
          wf[i] = *reinterpret_cast<const bf16x8_t*>(b + (fbw[i] ^ (16 * (2 * t + g))));
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          rf[j] = *reinterpret_cast<const bf16x8_t*>(b + (fbr[j] ^ (16 * (2 * t + g))));
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], rf[j], acc[i][j], 0, 0, 0);
      } else {
        i32x8_t wf[NI], rf[NJ];
        const int c0 = 16 * (2 * t + g), c1 = 16 * (SLOTS / 2 + 2 * t + g);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const i32x4_t a0 = *reinterpret_cast<const i32x4_t*>(b + (fbw[i] ^ c0));
          const i32x4_t a1 = *reinterpret_cast<const i32x4_t*>(b + (fbw[i] ^ c1));
          wf[i] = (i32x8_t){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const i32x4_t b0 = *reinterpret_cast<const i32x4_t*>(b + (fbr[j] ^ c0));
          const i32x4_t b1 = *reinterpret_cast<const i32x4_t*>(b + (fbr[j] ^ c1));
          rf[j] = (i32x8_t){b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = mfma_mx_sel(S0 + t, wf[i], rf[j], acc[i][j], scw[i], scr[j]);
      }
    }
  };

  const int nk = (int)(ldk / RB);
  const int nchunks = MX ? nk / PER_CHUNK : 0;
  if constexpr (MX) sload(0, scw, scr);
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s, s);

  // one stage at position P of its MX chunk (P = 0 for BF16)
  auto step = [&](int kt, auto p_tag) {
    constexpr int P = decltype(p_tag)::value;
    const int cc = MX ? kt / PER_CHUNK : 0;
    // wait until this wave's loads of stage kt have landed: at most the loads issued after them
    // may be outstanding, i.e. the next NS - 2 stages and, at chunk positions 1 .. NS - 2, the
    // next chunk's scale words (issued at position 0, after that stage's wait). Near the end
    // fewer loads follow, and vmcnt(0) is used.
    if (kt + NS - 2 < nk) {
      if constexpr (MX && P >= 1 && P <= NS - 2) {
        if (cc + 1 < nchunks) wait_vmcnt_fenced<LOADS * (NS - 2) + NSC>();
        else wait_vmcnt_fenced<LOADS * (NS - 2)>();
      } else {
        wait_vmcnt_fenced<LOADS * (NS - 2)>();
      }
    } else {
      wait_vmcnt_fenced<0>();
    }
    lds_barrier();
    if constexpr (MX) {
      if (P == 0 && cc + 1 < nchunks) sload(cc + 1, nscw, nscr);
    }
    if (kt + NS - 1 < nk) issue(kt + NS - 1, (kt + NS - 1) % NS);
    compute(lds + (kt % NS) * STAGE, std::integral_constant<int, P * SPS>{});
    if constexpr (MX) {
      if (P == PER_CHUNK - 1) {
#pragma unroll
        for (int i = 0; i < NI; ++i) scw[i] = nscw[i];
#pragma unroll
        for (int j = 0; j < NJ; ++j) scr[j] = nscr[j];
      }
    }
  };
  if constexpr (MX) {
    static_assert(PER_CHUNK == 2 || PER_CHUNK == 4, "chunk split");
    for (int kt = 0; kt < nk; kt += PER_CHUNK) {
      step(kt + 0, std::integral_constant<int, 0>{});
      step(kt + 1, std::integral_constant<int, 1>{});
      if constexpr (PER_CHUNK == 4) {
        step(kt + 2, std::integral_constant<int, 2>{});
        step(kt + 3, std::integral_constant<int, 3>{});
      }
    }
  } else {
    for (int kt = 0; kt < nk; ++kt) step(kt, std::integral_constant<int, 0>{});
  }

  // ---- epilogue. acc[i][j][q]: weight row n0 + 128 wn + 32 i + 8 (q / 4) + 4 g + q % 4,
  //      routed row row0 + (BM/2) wm + 32 j + li
  if constexpr (SWIGLU) {
    const int Hn = p.N >> 1;
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      // weight rows n0 + 128 wn + 64 pr + [0, 32) are gate columns, + [32, 64) the up columns
      const int col0 = (n0 + 128 * wn + 64 * pr) >> 1;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int r = row0 + (BM / 2) * wm + 32 * j + li;
        float hv[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) hv[q] = silu_f(acc[2 * pr][j][q]) * acc[2 * pr + 1][j][q];
        if constexpr (!MX) {
          if (r < row_end) {
            uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + (size_t)r * Hn + col0;
#pragma unroll
            for (int b4 = 0; b4 < 4; ++b4) {
              uint2 v;
              v.x = pack_bf16x2(hv[4 * b4 + 0], hv[4 * b4 + 1]);
              v.y = pack_bf16x2(hv[4 * b4 + 2], hv[4 * b4 + 3]);
              *reinterpret_cast<uint2*>(out + b4 * 8 + g * 4) = v;
            }
          }
        } else {
          float amax = 0.0f;
#pragma unroll
          for (int q = 0; q < 16; ++q) amax = fmaxf(amax, fabsf(hv[q]));
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          const int sx = mx_block_exponent(amax);
          const float inv = mx_inv_scale(sx);
          if (r < row_end) {
            uint8_t* out = reinterpret_cast<uint8_t*>(p.out) + (size_t)r * Hn + col0;
#pragma unroll
            for (int b4 = 0; b4 < 4; ++b4) {
              const uint32_t w4 = e4m3_encode(hv[4 * b4 + 0] * inv) |
                                  (e4m3_encode(hv[4 * b4 + 1] * inv) << 8) |
                                  (e4m3_encode(hv[4 * b4 + 2] * inv) << 16) |
                                  (e4m3_encode(hv[4 * b4 + 3] * inv) << 24);
              *reinterpret_cast<uint32_t*>(out + b4 * 8 + g * 4) = w4;
            }
            if (g == 0) p.out_scales[(size_t)r * (Hn / kMxBlock) + (col0 >> 5)] = (uint8_t)(sx + 127);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = row0 + (BM / 2) * wm + 32 * j + li;
      if (r >= row_end) continue;
      uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + (size_t)r * p.N + n0 + 128 * wn;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          uint2 v;
          v.x = pack_bf16x2(acc[i][j][4 * b4 + 0], acc[i][j][4 * b4 + 1]);
          v.y = pack_bf16x2(acc[i][j][4 * b4 + 2], acc[i][j][4 * b4 + 3]);
          *reinterpret_cast<uint2*>(out + 32 * i + b4 * 8 + g * 4) = v;
        }
    }
  }
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
                                                             int row_off) {
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
  if constexpr (!MX) {
    uint16_t* d = reinterpret_cast<uint16_t*>(dst + (size_t)e * dst_stride);
    for (int i = tid; i < 64 * 64; i += 256) {
      const int cc = i >> 6, kk = i & 63;
      const int n = c0 + cc;
      const int orow = (n >> 5) * row_stride + row_off + (n & 31);
      d[(size_t)orow * K + k0 + kk] = (uint16_t)f32_to_bf16_bits(tile[kk][cc]);
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
      uint8_t* d = dst + (size_t)e * dst_stride + (size_t)orow * K + k0 + half * 32;
      for (int q = 0; q < 32; ++q) d[q] = (uint8_t)e4m3_encode(tile[half * 32 + q][cc] * inv);
      dst_scales[(size_t)e * dsts_stride + (size_t)orow * (K / kMxBlock) + (k0 >> 5) + half] =
          (uint8_t)(sx + 127);
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
  size_t count, tiles, H, Hs, total;
  int max_tiles;
};

// rows per M tile: the large-tile kernel (h % 256 == 0, m % 128 == 0) takes 256 rows when the
// experts hold 224 rows or more on average, else 128; the small-tile kernel always 128
int ffn_tile_rows(int R, int h, int m, int E_loc) {
  if (h % kBigBN || (2 * m) % kBigBN) return kBM;
  return (R / E_loc >= 224) ? 256 : 128;
}
bool ffn_big(int h, int m) { return h % kBigBN == 0 && (2 * m) % kBigBN == 0; }

FfnLayout ffn_layout(int R, int h, int m, int E_loc, bool mx) {
  FfnLayout L{};
  const int bm = ffn_tile_rows(R, h, m, E_loc);
  L.max_tiles = (R + bm - 1) / bm + E_loc;
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
  }
  L.total = off;
  return L;
}

}  // namespace

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
  if (mx) {
    hipLaunchKernelGGL(prep_transpose_kernel<true>, g1, dim3(256), 0, st, w_gate, h, m, s1,
                       base + L.w1, base + L.w1s, d1, d1s, 64, 0);
    hipLaunchKernelGGL(prep_transpose_kernel<true>, g1, dim3(256), 0, st, w_up, h, m, s1,
                       base + L.w1, base + L.w1s, d1, d1s, 64, 32);
    hipLaunchKernelGGL(prep_transpose_kernel<true>, g2, dim3(256), 0, st, w_down, m, h, s2,
                       base + L.w2, base + L.w2s, d2, d2s, 32, 0);
  } else {
    hipLaunchKernelGGL(prep_transpose_kernel<false>, g1, dim3(256), 0, st, w_gate, h, m, s1,
                       base + L.w1, nullptr, d1, 0, 64, 0);
    hipLaunchKernelGGL(prep_transpose_kernel<false>, g1, dim3(256), 0, st, w_up, h, m, s1,
                       base + L.w1, nullptr, d1, 0, 64, 32);
    hipLaunchKernelGGL(prep_transpose_kernel<false>, g2, dim3(256), 0, st, w_down, m, h, s2,
                       base + L.w2, nullptr, d2, 0, 32, 0);
  }
  return hipGetLastError();
}

hipError_t launch_expert_ffn(const void* rows, const uint8_t* row_scales, const int32_t* offsets,
                             const void* prepared, uint16_t* out_rows, void* ws, int R, int h,
                             int m, int E_loc, bool mx, hipStream_t st, const hipEvent_t* ev) {
  const PreparedLayout P = prepared_layout(E_loc, h, m, mx);
  const FfnLayout F = ffn_layout(R, h, m, E_loc, mx);
  const int bm = ffn_tile_rows(R, h, m, E_loc);
  const bool big = ffn_big(h, m);
  const uint8_t* pw = reinterpret_cast<const uint8_t*>(prepared);
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  int2* tiles = reinterpret_cast<int2*>(w + F.tiles);
  int* tile_count = reinterpret_cast<int*>(w + F.count);
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, st, offsets, E_loc, bm,
                     F.max_tiles, tiles, tile_count);
  if (ev) (void)hipEventRecord(ev[0], st);
  const size_t el = mx ? 1 : 2;

  GemmArgs a1{};
  a1.rows = reinterpret_cast<const uint8_t*>(rows);
  a1.row_scales = row_scales;
  a1.w = pw + P.w1;
  a1.w_scales = mx ? pw + P.w1s : nullptr;
  a1.w_stride = (size_t)2 * m * h * el;
  a1.ws_stride = (size_t)2 * m * (h / kMxBlock);
  a1.offsets = offsets;
  a1.tiles = tiles;
  a1.tile_count = tile_count;
  a1.K = h;
  a1.N = 2 * m;
  a1.out = w + F.H;
  a1.out_scales = mx ? w + F.Hs : nullptr;

  GemmArgs a2{};
  a2.rows = w + F.H;
  a2.row_scales = mx ? w + F.Hs : nullptr;
  a2.w = pw + P.w2;
  a2.w_scales = mx ? pw + P.w2s : nullptr;
  a2.w_stride = (size_t)h * m * el;
  a2.ws_stride = (size_t)h * (m / kMxBlock);
  a2.offsets = offsets;
  a2.tiles = tiles;
  a2.tile_count = tile_count;
  a2.K = m;
  a2.N = h;
  a2.out = out_rows;
  a2.out_scales = nullptr;

  if (big) {
    // the XCD remap needs the grid rounded up to a multiple of 8
    const dim3 g1((F.max_tiles * ((2 * m) / kBigBN) + 7) / 8 * 8);
    const dim3 g2((F.max_tiles * (h / kBigBN) + 7) / 8 * 8);
    // kernels launched by name here so that each instantiation is compiled for the device
#define MOE_BIG(MXV, SW, BMV, G, A)                                                             \
    hipLaunchKernelGGL((grouped_gemm_big_kernel<MXV, SW, BMV, (MXV ? MOE_BIG_RB_MX : MOE_BIG_RB_BF16), \
                                                (MXV ? MOE_BIG_NS_MX : MOE_BIG_NS_BF16)>),      \
                       G, dim3(256), 0, st, A)
    if (bm == 256) {
      if (mx) MOE_BIG(true, true, 256, g1, a1); else MOE_BIG(false, true, 256, g1, a1);
      if (ev) (void)hipEventRecord(ev[1], st);
      if (mx) MOE_BIG(true, false, 256, g2, a2); else MOE_BIG(false, false, 256, g2, a2);
    } else {
      if (mx) MOE_BIG(true, true, 128, g1, a1); else MOE_BIG(false, true, 128, g1, a1);
      if (ev) (void)hipEventRecord(ev[1], st);
      if (mx) MOE_BIG(true, false, 128, g2, a2); else MOE_BIG(false, false, 128, g2, a2);
    }
#undef MOE_BIG
    if (ev) (void)hipEventRecord(ev[2], st);
    return hipGetLastError();
  }
  dim3 grid1(F.max_tiles, (2 * m) / kBN);
  dim3 grid2(F.max_tiles, h / kBN);
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

}  // namespace moe
