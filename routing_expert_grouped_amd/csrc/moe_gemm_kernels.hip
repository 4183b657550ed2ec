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

#include "moe_gemm_plan.h"
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
  // large-tile kernel only, by epilogue mode (see EpiMode)
  float* gu_out;                // kEpiSwiglu: G and U, float32 [R][N] in weight-row order, or null
  const float* gu_in;           // kEpiDSwiglu: the forward's G and U, float32 [R][2N]
  float* d_f32;                 // kEpiDSwiglu: dG and dU also as float32 [R][2N], or null
  const int32_t* koff;          // kEpiWgrad: [E_loc+1] first K element of each expert's segment
  int M;                        // kEpiWgrad: rows of the M-side operand per expert
  int tiles_total;              // kEpiWgrad: E_loc * M / BM
  int split_gate_up;            // kEpiWgrad: N is the gate/up-interleaved index (out, out2)
  int out_f32;                  // kEpiWgrad: float32 outputs (else bf16)
  void* out2;                   // kEpiWgrad with split_gate_up: the up half
  // large-tile kernel, MX scale layouts: 0 = natural [rows][K/32]; 1 = chunk-major
  // [K/256][rows][8] (the 8 scale bytes of one 256-element chunk of every row side by side, so a
  // wave's scale words of a chunk are a few cache lines). Weights: rows = N per expert; routed
  // rows (input and the H scales GEMM-1 writes): rows = sc_rows.
  int w_sc_cm;
  int r_sc_cm;
  int out_sc_cm;
  int sc_rows;      // rows of the chunk-major routed-row (input) scale array
  int out_sc_rows;  // rows of the chunk-major output scale array
  // large-tile kernel, routed-row operand gathered on the fly: routed row r reads row
  // row_src[r] / row_div of `rows` (and of its scales), e.g. token perm[r] / k of x; null: row r
  const int32_t* row_src;
  int row_div;
  // large-tile kernel: weight codes K-tiled, [E][N/256][K bytes/128][256][128 bytes] (each stage
  // of a 256-row weight panel is one contiguous 32 KB block), else natural [E][N][K]
  int w_tiled;
};

// Epilogue (and grouping) modes of the large-tile kernel.
//   kEpiSwiglu : GEMM-1 of the forward, H = silu(G) * U
//   kEpiSwigluSave: the same, and G, U stored in float32 (gu_out) for a backward pass
//   kEpiStore  : the accumulators as bf16 (GEMM-2 of the forward, dA of the backward)
//   kEpiDSwiglu: dH of the backward -> dG = dH * U * silu'(G), dU = dH * silu(G) from the saved
//                G, U; stored gate/up-interleaved per 32 (bf16, or MX per 32), plus optionally
//                in float32 (the values the weight gradients quantise along rows)
//   kEpiWgrad  : weight gradients. Each expert is an M x N output reduced over its own padded
//                segment of K (its routed rows); both operands are [rows][K] per expert at the
//                segment's offset. Tiles are (expert, M tile), N tiles as usual.
enum EpiMode : int {
  kEpiSwiglu = 0,
  kEpiStore = 1,
  kEpiDSwiglu = 2,
  kEpiWgrad = 3,
  kEpiSwigluSave = 4
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
// staged data. The compiler does not order these asynchronous LDS writes against LDS reads, so the
// pipeline waits explicitly: before stage j is read, s_waitcnt vmcnt(n) where n is the exact
// number of loads this wave issued after stage j's (counted at run time from the fixed issue
// order), then a barrier, so every wave's part of stage j is in LDS and no wave still reads the
// buffer the next DMA overwrites.
//
// Fragments are software-pipelined one k-step ahead: the LDS reads of k-step t+1 are in flight
// while the MFMAs of k-step t run, and the wait/barrier for the next stage sits inside the last
// k-step of the current one, so the first fragments of a stage are read before its MFMAs start.
//
// LDS rows are RB bytes, split into 16-byte slots; slot p of row r holds logical chunk p ^ f(r)
// (f(r) = ((r >> 1) ^ (r >> 2)) & 3 for RB = 64, (r ^ (r >> 3)) & 7 for RB = 128), which spreads
// the lanes that read one logical chunk of consecutive rows over distinct bank groups for both
// 8-lane and 16-lane LDS phases. The swizzle is applied on the global side: the DMA writes a
// wave's 64 lanes to 1 KB of consecutive LDS, and each lane fetches the chunk for its slot.
//
// Work order: the M tiles are cut into bands of about 256 / Nt tiles; all XCDs work on the same
// band at the same time (so the band's rows and its experts' weights stay in the MALL), and
// inside a band XCD x takes the x-th eighth of the band's tiles in N-major order, i.e. a block of
// about Nt/8 weight panels by band-height row panels, about the 32 tiles its CUs run at once and
// share through its L2. Workgroup L runs on XCD L % 8.
// ------------------------------------------------------------------------------------------------
constexpr int kBigBN = 256;
// band height in M tiles: about 256 tiles per band, i.e. about the 32 concurrent workgroups of
// each XCD per band share
__host__ __device__ inline int band_rows_for(int Nt) {
  const int b = (256 + Nt / 2) / Nt;
  return b < 4 ? 4 : (b > 16 ? 16 : b);
}

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

// vmcnt(n) for a wave-uniform run-time n in [LO, HI], by binary dispatch on the immediate
template <int LO, int HI>
__device__ __forceinline__ void wait_vmcnt_range(int n) {
  if constexpr (LO == HI) {
    wait_vmcnt<LO>();
  } else {
    constexpr int MID = (LO + HI + 1) / 2;
    if (n >= MID) wait_vmcnt_range<MID, HI>(n);
    else wait_vmcnt_range<LO, MID - 1>(n);
  }
}

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

// A 64-bit vector load the compiler does not track: it puts no wait of its own before the value's
// first use (it would wait for every LDS DMA load issued before, as it cannot count those), so the
// caller must have waited for it with the vmcnt of a later load. Host pass: never called.
__device__ __forceinline__ uint64_t load_dwordx2_untracked(const uint8_t* base, uint32_t off) {
  uint64_t v = 0;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("global_load_dwordx2 %0, %1, %2" : "=v"(v) : "v"(off), "s"(base));
#endif
  return v;
}

// every LDS read of this wave has returned, then all waves meet; no memory access moves across
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// K bytes per stage (whole 128-byte lines). The ring depths per tile height (big_ns, big_nsr) and
// the DMA issue order and wait counts are in moe_gemm_plan.h. LDS per workgroup:
// (NS * 256 + NSR * BM) * 128 bytes, at most 160 KB.
constexpr int kBigRB = 128;

template <int MODE, bool MX, int BM, int RB, int NS, int NSR>
__global__ __launch_bounds__(256, 1) void grouped_gemm_big_kernel(GemmArgs p) {
  constexpr int BN = kBigBN;
  constexpr int WSTAGE = BN * RB;                // one stage of the weight operand
  constexpr int RSTAGE = BM * RB;                // one stage of the routed rows
  constexpr int NI = 4;                          // weight fragments per wave
  constexpr int NJ = BM / 64;                    // row fragments per wave
  // the DMA plan (moe_gemm_plan.h): LOADS 16-byte units per thread per barrier point, QW of the
  // weight group and QR of the row group (the shallower ring's group first), issued in SPS parts
  // (one per k-step of the next stage, the last part, units [U0, LOADS), after the following
  // barrier), and the number of loads each barrier point's wait may leave in flight
  using PO = BigPlanOf<MX, BM, RB, NS, NSR>;
  constexpr BigPlan PL = PO::get();
  constexpr int LOADS = PL.LOADS;
  constexpr int SLOTS = PL.SLOTS;
  constexpr int SPS = PL.SPS;                    // MFMA k-steps per stage
  constexpr int PC = PL.PC;                      // stages per 256-element MX chunk
  constexpr int NSC = PL.NSC;                    // scale loads per chunk
  constexpr int NSTEADY = plan_steady_count(PO::get()); // in flight at a steady-state wait
  constexpr int NDEEP = NS > NSR ? NS : NSR;
  constexpr int NMAX = LOADS * NDEEP;            // bound of any wait count
  static_assert(PL.BN == BN && NSC == (MX ? NI + NJ : 0), "plan matches the tile");
  static_assert(SPS >= 2 && NSTEADY >= 0, "DMA parts per k-step");
  static_assert(NS >= 2 && NSR >= 2 && NSR >= NS - 1 && NSR <= NS + 1, "ring depths");
  static_assert(NMAX + NSC < 64, "vmcnt range");
  static_assert(!MX || PC == 2, "an MX chunk of 256 elements is two stages");
  static_assert(MX || SPS % 2 == 0, "fragment double buffer alternates within a stage");
  static_assert(NS * WSTAGE + NSR * RSTAGE <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint8_t lds[NS * WSTAGE + NSR * RSTAGE];
  // stage s: weight rows in ring slot s % NS, routed rows in ring slot s % NSR
  auto wbuf = [&](int s) { return lds + (s % NS) * WSTAGE; };
  auto rbuf = [&](int s) { return lds + NS * WSTAGE + (s % NSR) * RSTAGE; };

  // ---- which tile: band b of band_m M tiles, XCD x takes the x-th eighth of it (N-major)
  const int mt_total = MODE == kEpiWgrad ? p.tiles_total : *p.tile_count;
  const int Nt = p.N / BN;
  const int band_m = band_rows_for(Nt);
  const int x = blockIdx.x & 7;
  int jx = blockIdx.x >> 3;  // this workgroup's index among the XCD's workgroups
  const int nb_full = mt_total / band_m;
  const int tb_full = band_m * Nt;
  const int share_full = ((x + 1) * tb_full >> 3) - (x * tb_full >> 3);
  int band, band_rows, tb;
  if (jx < nb_full * share_full) {
    band = jx / share_full;
    jx -= band * share_full;
    band_rows = band_m;
    tb = tb_full;
  } else {
    jx -= nb_full * share_full;
    band = nb_full;
    band_rows = mt_total - nb_full * band_m;
    tb = band_rows * Nt;
    const int share_last = ((x + 1) * tb >> 3) - (x * tb >> 3);
    if (jx >= share_last) return;  // surplus workgroup: leaves before any barrier
  }
  const int pos = (x * tb >> 3) + jx;
  const int nt = pos / band_rows;
  const int ti = band * band_m + pos % band_rows;
  int e, row0, row_end;
  if constexpr (MODE == kEpiWgrad) {
    const int mtiles = p.M / BM;
    e = ti / mtiles;
    row0 = (ti % mtiles) * BM;
    row_end = p.M;
  } else {
    const int2 te = p.tiles[ti];
    e = te.x;
    row0 = te.y;
    row_end = p.offsets[e + 1];
  }
  const int n0 = nt * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases stay scalar
  const int wn = wave >> 1;
  const int wm = wave & 1;
  const int li = lane & 31;
  const int g = lane >> 5;

  // operand bases and K of this tile: per expert for the weight operand, or the expert's segment
  // of both operands (weight gradients)
  constexpr size_t EL = MX ? 1 : 2;
  int Kt = p.K;
  const uint8_t* wexp;
  const uint8_t* rows_b = p.rows;
  const uint8_t* wsb = nullptr;
  const uint8_t* rsb = p.row_scales;
  if constexpr (MODE == kEpiWgrad) {
    const int k0 = p.koff[e];
    Kt = p.koff[e + 1] - k0;
    wexp = p.w + (size_t)k0 * p.N * EL;
    rows_b = p.rows + (size_t)k0 * p.M * EL;
    if constexpr (MX) {
      wsb = p.w_scales + (size_t)(k0 / kMxBlock) * p.N;
      rsb = p.row_scales + (size_t)(k0 / kMxBlock) * p.M;
    }
  } else {
    wexp = p.w + (size_t)e * p.w_stride;
    if constexpr (MX) wsb = p.w_scales + (size_t)e * p.ws_stride;
  }
  const size_t ldk = (size_t)Kt * EL;

  // ---- DMA sources: unit id = q * 256 + tid is LDS row id / SLOTS (rows BN.. are the routed
  //      rows, at row id / SLOTS - BN of their ring slot), physical slot id % SLOTS, and must carry
  //      logical chunk slot ^ f(row) (f(BN + r) = f(r) for BN = 256). Unit q of a point is unit
  //      plan_group_index(q) of the weight group (plan_is_w) or of the row group; 32-bit offsets
  //      from the two (uniform) bases.
  uint32_t src[LOADS];
#pragma unroll
  for (int q = 0; q < LOADS; ++q) {
    const int u = plan_group_index(PO::get(), q);
    const int id = u * 256 + tid;
    const int row = id / SLOTS;  // row of the weight panel, or of the routed-row tile
    if (plan_is_w(PO::get(), q)) {
      const uint32_t cb = 16 * ((id % SLOTS) ^ big_swz<RB>(row));
      src[q] = p.w_tiled ? (uint32_t)((size_t)(n0 / BN) * ldk * BN) + row * RB + cb
                         : (uint32_t)((n0 + row) * ldk) + cb;
    } else {
      const uint32_t cb = 16 * ((id % SLOTS) ^ big_swz<RB>(BN + row));
      int r = row0 + row;
      r = r < row_end ? r : row_end - 1;  // rows past the expert's end are never stored
      if (p.row_src) r = p.row_src[r] / p.row_div;
      src[q] = (uint32_t)(r * ldk) + cb;
    }
  }
  // stage j holds K bytes [RB j, RB j + RB) of every row (whole cache lines for RB = 128)
  auto stage_off = [&](int j) -> size_t { return (size_t)RB * j; };
  const uint32_t wstage_bytes = p.w_tiled ? (uint32_t)WSTAGE : (uint32_t)RB;  // per weight stage
  const int nk = (int)(ldk / RB);
  const int nchunks = MX ? nk / PC : 0;
  // first unit of part t (t = SPS: the end)
  auto part_start = [](int t) { return plan_part_start(PO::get(), t); };
  // part `part` of barrier point b's groups W(b+NS-1), R(b+NSR-1), skipping stages that do not
  // exist; they go to the ring slots of stage b-1
  auto issue_part = [&](int b, int part) {
    const int sw = b + NS - 1, sr = b + NSR - 1;
    const bool hw = sw >= 0 && sw < nk, hr = sr >= 0 && sr < nk;
    const uint32_t offw = wstage_bytes * (uint32_t)(sw < 0 ? 0 : sw), offr = (uint32_t)stage_off(sr);
    uint8_t* bw = wbuf(sw < 0 ? 0 : sw) + wave * 1024;
    uint8_t* br = rbuf(sr < 0 ? 0 : sr) + wave * 1024;
    const int q0 = part_start(part), q1 = part_start(part + 1);
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
      if (q < q0 || q >= q1) continue;
      if (plan_is_w(PO::get(), q)) {
        if (hw) dma16(wexp + (src[q] + offw), bw + plan_group_index(PO::get(), q) * 4096);
      } else {
        if (hr) dma16(rows_b + (src[q] + offr), br + plan_group_index(PO::get(), q) * 4096);
      }
    }
  };

  // ---- MX scale words. In K order, MFMA step s of a 256-element chunk multiplies blocks 2s (its
  //      first block, scale from lane group 0) and 2s+1 (second block, lane group 1), so lane group
  //      g needs the scale bytes of blocks g, 2+g, 4+g, 6+g of the chunk: the row's 8 chunk scale
  //      bytes are loaded a chunk ahead and byte-permuted into that word once the chunk's first
  //      barrier point has waited for them; the MFMA's byte select picks step s. 32-bit offsets
  //      from the expert's and the rows' scale bases.
  uint32_t sw_off[NI], sr_off[NJ];
  int scw[NI], scr[NJ];
  uint64_t nscw[NI], nscr[NJ];
  const uint32_t perm_sel = g ? 0x07050301u : 0x06040200u;  // bytes g, 2+g of lo, g, 2+g of hi
  // byte offsets: row (or weight row) x, chunk cc at x * *_rs + cc * *_cs
  uint32_t w_cs = 8, r_cs = 8;
  if constexpr (MX) {
    const uint32_t nsb = (uint32_t)(Kt / kMxBlock);
    const uint32_t w_rs = p.w_sc_cm ? 8u : nsb, r_rs = p.r_sc_cm ? 8u : nsb;
    if (p.w_sc_cm) w_cs = 8u * (uint32_t)p.N;
    if (p.r_sc_cm) r_cs = 8u * (uint32_t)p.sc_rows;
#pragma unroll
    for (int i = 0; i < NI; ++i) sw_off[i] = (uint32_t)(n0 + 128 * wn + 32 * i + li) * w_rs;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      int r = row0 + (BM / 2) * wm + 32 * j + li;
      r = r < row_end ? r : row_end - 1;
      if (p.row_src) r = p.row_src[r] / p.row_div;
      sr_off[j] = (uint32_t)r * r_rs;
    }
  }
  // (issued ahead of a DMA load that the chunk's first barrier point waits for, so that wait
  // covers them)
  auto scale_raw = [&](const uint8_t* base, uint32_t off, uint32_t cs, int cc) -> uint64_t {
    return load_dwordx2_untracked(base, off + cs * (uint32_t)cc);
  };
  auto scale_word = [&](uint64_t v) -> int {
    return (int)__builtin_amdgcn_perm((uint32_t)(v >> 32), (uint32_t)v, perm_sel);
  };
  auto sload = [&](int cc, uint64_t (&w)[NI], uint64_t (&r)[NJ]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) w[i] = scale_raw(wsb, sw_off[i], w_cs, cc);
#pragma unroll
    for (int j = 0; j < NJ; ++j) r[j] = scale_raw(rsb, sr_off[j], r_cs, cc);
  };
  auto take_scales = [&]() {  // after the wait of the chunk's first barrier point
#pragma unroll
    for (int i = 0; i < NI; ++i) scw[i] = scale_word(nscw[i]);
#pragma unroll
    for (int q = 0; q < NJ; ++q) scr[q] = scale_word(nscr[q]);
  };

  // ---- issue order of this wave's vector-memory loads (fixed, so the counts are exact): the
  //   prologue issues S(0) and every point b < 0 whole; stage j then issues part t of point j's
  //   groups in its k-step t and the last part right after barrier point j+1; a chunk's first
  //   stage cc * PC starts with S(cc+1), the next chunk's scale words, ahead of its DMA parts
  //   (so the wait of chunk cc+1's first point covers them). Loads complete in issue order, so
  //   point j waits until at most plan_wait_count(j) loads are in flight: the DMA units issued
  //   after the later of W(j), R(j).
  auto wait_stage = [&](int j) {
    const int n = plan_wait_count(PO::get(), j, nk);
    asm volatile("" ::: "memory");
    wait_vmcnt_range<0, NMAX>(n);
  };
  // barrier point j: stage j is in LDS for every wave and stage j-1 read by every wave; then the
  // last part of point j-1's loads and the scale words of the next chunk
  auto barrier_point = [&](int j) {
    wait_stage(j);
    lds_barrier();
    if (j >= 1) issue_part(j - 1, SPS - 1);
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
    const int row = (BM / 2) * wm + 32 * j + li;  // within the routed-row ring slot
    fbr[j] = row * RB + 16 * big_swz<RB>(BN + row);
  }

  using FragT = typename std::conditional<MX, i32x8_t, bf16x8_t>::type;
  struct Frags {
    FragT w[NI];
    FragT r[NJ];
  };
  constexpr int NR = (MX ? 2 : 1) * (NI + NJ);  // 16-byte LDS reads per k-step
  // 16-byte piece `idx` (0 .. NR-1) of the fragments of k-step t from the stage's weight ring
  // slot bw and routed-row ring slot br; weight fragments first, each MX fragment being two
  // pieces (its two half blocks)
  auto load_piece = [&](Frags& F, const uint8_t* bw, const uint8_t* br, int t, int idx) {
    if constexpr (!MX) {
      const int c = 16 * (2 * t + g);
      if (idx < NI) F.w[idx] = *reinterpret_cast<const bf16x8_t*>(bw + (fbw[idx] ^ c));
      else F.r[idx - NI] = *reinterpret_cast<const bf16x8_t*>(br + (fbr[idx - NI] ^ c));
    } else {
      // MFMA step t of the stage: bytes 0-15 of lane (i, g) are K [64t + 16g, +16) (first block),
      // bytes 16-31 are K [64t + 32 + 16g, +16) (second block)
      const int f = idx >> 1, half = idx & 1;
      const int c = 16 * (4 * t + 2 * half + g);
      const uint8_t* b = f < NI ? bw : br;
      const int fb = f < NI ? fbw[f] : fbr[f - NI];
      const i32x4_t v = *reinterpret_cast<const i32x4_t*>(b + (fb ^ c));
      FragT& dst = f < NI ? F.w[f] : F.r[f - NI];
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[4 * half + q] = v[q];
    }
  };
  auto load_frags = [&](Frags& F, int j, int t) {  // k-step t of stage j
#pragma unroll
    for (int idx = 0; idx < NR; ++idx) load_piece(F, wbuf(j), rbuf(j), t, idx);
  };

  f32x16_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  constexpr int NM = NI * NJ;  // MFMAs per k-step
  auto mfma_k = [&](const Frags& F, int k, int sel) {
    const int i = k / NJ, j = k % NJ;
    if constexpr (MX) acc[i][j] = mfma_mx_sel(sel, F.w[i], F.r[j], acc[i][j], scw[i], scr[j]);
    else acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.w[i], F.r[j], acc[i][j], 0, 0, 0);
  };
  auto mfmas = [&](const Frags& F, int sel) {
#pragma unroll
    for (int k = 0; k < NM; ++k) mfma_k(F, k, sel);
  };

  // ---- prologue (an expert segment with no rows, weight gradients only, skips the K loop and
  //      stores zeros; the condition is uniform over the workgroup)
  Frags FA, FB;
  if (MODE != kEpiWgrad || nk > 0) {
  if constexpr (MX) {
    sload(0, nscw, nscr);
  }
#pragma unroll
  for (int b = -(NDEEP - 1); b < 0; ++b)
#pragma unroll
    for (int part = 0; part < SPS; ++part) issue_part(b, part);
  barrier_point(0);
  if constexpr (MX) take_scales();
  load_frags(FA, 0, 0);

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  // ---- steady-state k-step (stage j with j + max(NS, NSR) < nk, so every wait and load is
  // unconditional):
  // its MFMAs interleaved one by one with the other work, in a fixed order the compiler may not
  // change (sched_barrier): part t of barrier point j's DMA (into stage j-1's ring slots), the
  // next k-step's LDS reads, and in a stage's last k-step, right after the first MFMA, the wait
  // and barrier of point j+1 followed by the last DMA part and the reads of stage j+1's first
  // fragments. A chunk's first k-step starts with the next chunk's MX scale words.
  auto kstep_fast = [&](int j, auto t_tag, auto p_tag, Frags& cur, Frags& nxt) {
    constexpr int t = decltype(t_tag)::value;
    constexpr int P = decltype(p_tag)::value;
    constexpr bool LAST = t + 1 == SPS;
    constexpr bool SCALES = MX && t == 0 && P == 0;  // the first k-step of chunk cc
    constexpr int Q0 = plan_part_start(PO::get(), t);  // this k-step's DMA part: units [Q0, Q0 + NDMA)
    constexpr int NDMA = plan_part_start(PO::get(), t + 1) - Q0;
    constexpr int NSCL = SCALES ? NSC : 0;
    // the scale words of chunk cc + 1 went out at the start of stage cc * PC = j - P, as the
    // first loads of that stage; they may still be in flight at the wait of point j + 1 when both
    // of stage j + 1's groups went out before them (plan_scales_in_flight)
    constexpr int SCL_AFTER = plan_scales_in_flight(PO::get(), P);
    constexpr int NOPS = NDMA + NSCL + NR;
    constexpr int SLOTS_M = NM - 2;  // leave the last two MFMAs to cover the last reads
    constexpr int K = (NOPS + SLOTS_M - 1) / SLOTS_M;
    const uint8_t* rbw = LAST ? wbuf(j + 1) : wbuf(j);
    const uint8_t* rbr = LAST ? rbuf(j + 1) : rbuf(j);
    const int rt = LAST ? 0 : t + 1;
    const uint32_t doffw = wstage_bytes * (uint32_t)(j + NS - 1);  // point j's groups
    const uint32_t doffr = (uint32_t)stage_off(j + NSR - 1);
    uint8_t* dbw = wbuf(j + NS - 1) + wave * 1024;  // stage j-1's ring slots
    uint8_t* dbr = rbuf(j + NSR - 1) + wave * 1024;
    const int cc_next = min(j / PC + 1, nchunks - 1);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      mfma_k(cur, m, P * SPS + t);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (LAST) {
        if (m == 0) {
          wait_vmcnt_fenced<NSTEADY + SCL_AFTER>();
          lds_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int o = 0; o < K; ++o) {
        const int op = (m - 1) * K + o;
        if (m >= 1 && op < NOPS) {
          if (op < NSCL) {
            if constexpr (MX) {
              if (op < NI) nscw[op] = scale_raw(wsb, sw_off[op], w_cs, cc_next);
              else nscr[op - NI] = scale_raw(rsb, sr_off[op - NI], r_cs, cc_next);
            }
          } else if (op < NSCL + NDMA) {
            const int q = Q0 + op - NSCL;
            const int u = plan_group_index(PO::get(), q);
            if (plan_is_w(PO::get(), q)) dma16(wexp + (src[q] + doffw), dbw + u * 4096);
            else dma16(rows_b + (src[q] + doffr), dbr + u * 4096);
          } else {
            load_piece(nxt, rbw, rbr, rt, op - NDMA - NSCL);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- generic k-step for the last stages (conditional waits and loads)
  auto kstep = [&](int j, auto t_tag, auto p_tag, Frags& cur, Frags& nxt) {
    constexpr int t = decltype(t_tag)::value;
    constexpr int P = decltype(p_tag)::value;
    if constexpr (t + 1 < SPS) {
      if constexpr (MX && t == 0 && P == 0) {  // a chunk's first k-step: the next chunk's scales
        if (j / PC + 1 < nchunks) sload(j / PC + 1, nscw, nscr);
      }
      issue_part(j, t);
      load_frags(nxt, j, t + 1);
    } else {
      if (j + 1 < nk) {  // (the last stage's point has no groups left to issue)
        barrier_point(j + 1);
        load_frags(nxt, j + 1, 0);
      }
    }
    mfmas(cur, P * SPS + t);
  };

  // one stage; with an even number of k-steps it starts and ends on F0
  auto stage = [&](int j, auto p_tag, auto fast_tag, Frags& F0, Frags& F1) {
    constexpr int P = decltype(p_tag)::value;
    constexpr bool FAST = decltype(fast_tag)::value;
    auto ks = [&](auto t_tag, Frags& c, Frags& n) {
      if constexpr (FAST) kstep_fast(j, t_tag, p_tag, c, n);
      else kstep(j, t_tag, p_tag, c, n);
    };
    ks(I0{}, F0, F1);
    if constexpr (SPS >= 2) ks(I1{}, F1, F0);
    if constexpr (SPS >= 4) {
      ks(I2{}, F0, F1);
      ks(I3{}, F1, F0);
    }
    if constexpr (MX) {
      if constexpr (P == PC - 1) take_scales();  // the next stage starts a new chunk
    }
  };
  // stages [j0, j1) in blocks of PC (MX) or one by one (BF16)
  auto run = [&](int j0, int j1, auto fast_tag) {
    if constexpr (MX) {
      for (int j = j0; j < j1; j += PC) {
        if constexpr (SPS == 1) {  // one k-step per stage: the fragment set alternates per stage
          stage(j + 0, I0{}, fast_tag, FA, FB);
          stage(j + 1, I1{}, fast_tag, FB, FA);
          if constexpr (PC == 4) {
            stage(j + 2, I2{}, fast_tag, FA, FB);
            stage(j + 3, I3{}, fast_tag, FB, FA);
          }
        } else {
          stage(j + 0, I0{}, fast_tag, FA, FB);
          stage(j + 1, I1{}, fast_tag, FA, FB);
          if constexpr (PC == 4) {
            stage(j + 2, I2{}, fast_tag, FA, FB);
            stage(j + 3, I3{}, fast_tag, FA, FB);
          }
        }
      }
    } else {
      for (int j = j0; j < j1; ++j) stage(j, I0{}, fast_tag, FA, FB);
    }
  };
  // steady state: stages j with j + max(NS, NSR) < nk (rounded down to whole MX chunks), then
  // the rest
  const int jsteady = plan_steady_end(PO::get(), nk);
  run(0, jsteady, std::true_type{});
  run(jsteady, nk, std::false_type{});
  }  // nk > 0

  // ---- epilogue. acc[i][j][q]: weight row n0 + 128 wn + 32 i + 8 (q / 4) + 4 g + q % 4,
  //      routed row row0 + (BM/2) wm + 32 j + li
  if constexpr (MODE == kEpiSwiglu || MODE == kEpiSwigluSave) {
    if constexpr (MODE == kEpiSwigluSave) {  // G, U for a backward pass, weight-row order
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int r = row0 + (BM / 2) * wm + 32 * j + li;
        if (r >= row_end) continue;
        float* out = p.gu_out + (size_t)r * p.N + n0 + 128 * wn;
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4)
            *reinterpret_cast<f32x4_t*>(out + 32 * i + b4 * 8 + g * 4) =
                (f32x4_t){acc[i][j][4 * b4], acc[i][j][4 * b4 + 1], acc[i][j][4 * b4 + 2],
                          acc[i][j][4 * b4 + 3]};
      }
    }
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
            if (g == 0) {
              const int kb = col0 >> 5;  // MX block along m
              const size_t so = p.out_sc_cm
                                    ? ((size_t)(kb >> 3) * p.out_sc_rows + r) * 8 + (kb & 7)
                                    : (size_t)r * (Hn / kMxBlock) + kb;
              p.out_scales[so] = (uint8_t)(sx + 127);
            }
          }
        }
      }
    }
  } else if constexpr (MODE == kEpiStore) {
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
  } else if constexpr (MODE == kEpiDSwiglu) {
    // N = m dH columns. The 32-column tile i starting at column nb is one block of dG and one of
    // dU; they live at interleaved columns 2 nb + [0, 32) and 2 nb + 32 + [0, 32) of the [R][2m]
    // outputs, the same places the forward's G and U have in gu_in.
    const int N2 = 2 * p.N;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int cg = 2 * (n0 + 128 * wn + 32 * i);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int r = row0 + (BM / 2) * wm + 32 * j + li;
        const int rr = r < row_end ? r : row_end - 1;  // rows past the expert's end: loads only
        const float* gu = p.gu_in + (size_t)rr * N2 + cg + 4 * g;
        float dg[16], du[16];
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          const f32x4_t G = *reinterpret_cast<const f32x4_t*>(gu + 8 * b4);
          const f32x4_t U = *reinterpret_cast<const f32x4_t*>(gu + 32 + 8 * b4);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float dh = acc[i][j][4 * b4 + q];
            const float sg = 1.0f / (1.0f + expf(-G[q]));
            const float silu = G[q] * sg;
            const float dsilu = sg * (1.0f + G[q] * (1.0f - sg));
            dg[4 * b4 + q] = dh * U[q] * dsilu;
            du[4 * b4 + q] = dh * silu;
          }
        }
        if constexpr (MX) {
          float ag = 0.0f, au = 0.0f;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            ag = fmaxf(ag, fabsf(dg[q]));
            au = fmaxf(au, fabsf(du[q]));
          }
          ag = fmaxf(ag, __shfl_xor(ag, 32));  // the other 16 columns of each block
          au = fmaxf(au, __shfl_xor(au, 32));
          const int sg_ = mx_block_exponent(ag), su_ = mx_block_exponent(au);
          const float ig = mx_inv_scale(sg_), iu = mx_inv_scale(su_);
          if (r < row_end) {
            uint8_t* out = reinterpret_cast<uint8_t*>(p.out) + (size_t)r * N2 + cg + 4 * g;
#pragma unroll
            for (int b4 = 0; b4 < 4; ++b4) {
              const float* a4 = dg + 4 * b4;
              const float* c4 = du + 4 * b4;
              *reinterpret_cast<uint32_t*>(out + 8 * b4) =
                  e4m3_encode(a4[0] * ig) | (e4m3_encode(a4[1] * ig) << 8) |
                  (e4m3_encode(a4[2] * ig) << 16) | (e4m3_encode(a4[3] * ig) << 24);
              *reinterpret_cast<uint32_t*>(out + 32 + 8 * b4) =
                  e4m3_encode(c4[0] * iu) | (e4m3_encode(c4[1] * iu) << 8) |
                  (e4m3_encode(c4[2] * iu) << 16) | (e4m3_encode(c4[3] * iu) << 24);
            }
            // scale bytes of the dG block (lane group 0) and the dU block (lane group 1)
            const int kb = (cg >> 5) + g;  // MX block along 2m
            const size_t so = p.out_sc_cm
                                  ? ((size_t)(kb >> 3) * p.out_sc_rows + r) * 8 + (kb & 7)
                                  : (size_t)r * (N2 / kMxBlock) + kb;
            p.out_scales[so] = (uint8_t)((g ? su_ : sg_) + 127);
          }
        } else {
          if (r < row_end) {
            uint16_t* ob = reinterpret_cast<uint16_t*>(p.out) + (size_t)r * N2 + cg + 4 * g;
#pragma unroll
            for (int b4 = 0; b4 < 4; ++b4) {
              *reinterpret_cast<uint2*>(ob + 8 * b4) =
                  make_uint2(pack_bf16x2(dg[4 * b4], dg[4 * b4 + 1]),
                             pack_bf16x2(dg[4 * b4 + 2], dg[4 * b4 + 3]));
              *reinterpret_cast<uint2*>(ob + 32 + 8 * b4) =
                  make_uint2(pack_bf16x2(du[4 * b4], du[4 * b4 + 1]),
                             pack_bf16x2(du[4 * b4 + 2], du[4 * b4 + 3]));
            }
          }
        }
        if (p.d_f32 && r < row_end) {
          float* of = p.d_f32 + (size_t)r * N2 + cg + 4 * g;
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4) {
            *reinterpret_cast<f32x4_t*>(of + 8 * b4) =
                (f32x4_t){dg[4 * b4], dg[4 * b4 + 1], dg[4 * b4 + 2], dg[4 * b4 + 3]};
            *reinterpret_cast<f32x4_t*>(of + 32 + 8 * b4) =
                (f32x4_t){du[4 * b4], du[4 * b4 + 1], du[4 * b4 + 2], du[4 * b4 + 3]};
          }
        }
      }
    }
  } else {  // kEpiWgrad: out[e][r][n] of an M x N matrix per expert (or split gate / up halves)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int nb = n0 + 128 * wn + 32 * i;
      void* o = p.out;
      int col = nb, ld = p.N;
      if (p.split_gate_up) {  // N index: blocks of 32 alternate gate and up columns
        o = ((nb >> 5) & 1) ? p.out2 : p.out;
        col = (nb >> 6) * 32;
        ld = p.N >> 1;
      }
      const size_t ebase = (size_t)e * p.M * ld;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int r = row0 + (BM / 2) * wm + 32 * j + li;
        const size_t at = ebase + (size_t)r * ld + col + 4 * g;
        if (p.out_f32) {
          float* of = reinterpret_cast<float*>(o) + at;
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4)
            *reinterpret_cast<f32x4_t*>(of + 8 * b4) =
                (f32x4_t){acc[i][j][4 * b4], acc[i][j][4 * b4 + 1], acc[i][j][4 * b4 + 2],
                          acc[i][j][4 * b4 + 3]};
        } else {
          uint16_t* ob = reinterpret_cast<uint16_t*>(o) + at;
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4)
            *reinterpret_cast<uint2*>(ob + 8 * b4) =
                make_uint2(pack_bf16x2(acc[i][j][4 * b4], acc[i][j][4 * b4 + 1]),
                           pack_bf16x2(acc[i][j][4 * b4 + 2], acc[i][j][4 * b4 + 3]));
        }
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

// grid of the large-tile kernel for at most max_mt M tiles and nt N tiles: per XCD at most
// ceil(tiles / 8) plus one per band, and a multiple of 8 for the XCD remap
static dim3 big_grid(int max_mt, int nt) {
  return dim3(8 * ((max_mt * nt + 7) / 8 + max_mt / band_rows_for(nt) + 2));
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
  const PreparedLayout P = prepared_layout(E_loc, h, m, mx);
  const FfnLayout F = ffn_layout(R, h, m, E_loc, mx);
  const bool big = ffn_big(h, m);
  const uint8_t* pw = reinterpret_cast<const uint8_t*>(prepared);
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  int2* tiles = reinterpret_cast<int2*>(w + F.tiles);
  int* tile_count = reinterpret_cast<int*>(w + F.count);
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, st, offsets, E_loc, bm,
                     max_tiles, tiles, tile_count);
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
  a1.gu_out = gu_out;

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
    const dim3 g1 = big_grid(max_tiles, (2 * m) / kBigBN);
    const dim3 g2 = big_grid(max_tiles, h / kBigBN);
    a1.w_tiled = a2.w_tiled = 1;  // prepared K-tiled
    a1.row_src = row_src;  // GEMM-1 may read its rows through an index (GEMM-2 reads H)
    a1.row_div = row_div;
    const int n_src = row_src ? src_rows : R;  // rows of `rows` and of its scales
    if (mx) {  // chunk-major scales throughout: weights (prepared so), rows, and H
      if (!scales_cm) {
        const long long units = (long long)n_src * (h / 256);
        hipLaunchKernelGGL(scales_chunk_major_kernel, dim3((unsigned)((units + 255) / 256)),
                           dim3(256), 0, st, row_scales, n_src, h, w + F.Rs);
        a1.row_scales = w + F.Rs;
      }
      a1.w_sc_cm = a1.r_sc_cm = a1.out_sc_cm = 1;
      a1.sc_rows = n_src;
      a1.out_sc_rows = R;
      a2.w_sc_cm = a2.r_sc_cm = 1;
      a2.sc_rows = R;
    }
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

// the backward's routed-row GEMMs take 128-row tiles in both precisions (their epilogues do not
// fit the register file next to 256-row accumulators)
constexpr int kBwdBM = 128;

size_t gemm_tiles_bytes(int R, int E_loc) {
  return align_up(sizeof(int)) + (size_t)((R + kBwdBM - 1) / kBwdBM + E_loc) * sizeof(int2);
}

hipError_t launch_gemm_tiles(const int32_t* offsets, void* tiles_ws, int R, int E_loc,
                             hipStream_t st) {
  const int bm = kBwdBM;
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
  const int max_tiles = (R + kBwdBM - 1) / kBwdBM + E_loc;
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

  const dim3 ga = big_grid(max_tiles, m / kBigBN), gb = big_grid(max_tiles, h / kBigBN);
  if (mx) MOE_BIG(kEpiDSwiglu, true, kBwdBM, ga, a);
  else MOE_BIG(kEpiDSwiglu, false, kBwdBM, ga, a);
  if (ev_mid) (void)hipEventRecord(ev_mid, st);
  if (mx) MOE_BIG(kEpiStore, true, kBwdBM, gb, b);
  else MOE_BIG(kEpiStore, false, kBwdBM, gb, b);
  return hipGetLastError();
}

hipError_t launch_bwd_wgrad(const uint8_t* At, const uint8_t* At_s, const uint8_t* dGUt,
                            const uint8_t* dGUt_s, const uint8_t* Ht, const uint8_t* Ht_s,
                            const uint8_t* dOt, const uint8_t* dOt_s, const int32_t* koff,
                            void* dw_gate, void* dw_up, void* dw_down, bool out_f32, int h, int m,
                            int E_loc, bool mx, hipStream_t st, hipEvent_t ev_mid) {
  if (h % kBigBN || m % kBigBN) return hipErrorInvalidValue;
  const int bm = mx ? 128 : 256;
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
  if (mx) MOE_BIG(kEpiWgrad, true, 128, ga, a);
  else MOE_BIG(kEpiWgrad, false, 256, ga, a);
  if (ev_mid) (void)hipEventRecord(ev_mid, st);
  if (mx) MOE_BIG(kEpiWgrad, true, 128, gb, b);
  else MOE_BIG(kEpiWgrad, false, 256, gb, b);
  return hipGetLastError();
}

#undef MOE_BIG

}  // namespace moe
