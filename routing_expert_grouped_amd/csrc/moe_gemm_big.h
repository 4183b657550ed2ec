// The large-tile grouped GEMM as a device function (one output tile per call), shared by the
// grouped-GEMM kernels (one tile per workgroup) and the persistent forward (a workgroup runs the
// tiles it takes from a work queue), plus the argument block of every grouped GEMM.
#pragma once

#include <type_traits>

#include "moe_gemm_plan.h"
#include "moe_tile_order.h"
#include "moe_internal.h"

namespace moe {

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
  // large-tile kernel: M groups per band of the work order (big_tile_coords; 0 is taken as 1)
  int band_gm;
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

namespace {

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
// Work order: big_tile_coords (moe_tile_order.h), blocks of a band of about 256 tiles per XCD.
// ------------------------------------------------------------------------------------------------
constexpr int kBigBN = 256;

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

// a wave-uniform pointer, in scalar registers
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
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

// LDS bytes of a large tile's two rings
__host__ __device__ constexpr int big_lds_bytes(int bm, int rb, int ns, int nsr) {
  return (ns * kBigBN + nsr * bm) * rb;
}

// One output tile of the large-tile grouped GEMM, M tile ti (an entry of the tile table, or an
// (expert, M tile) pair for weight gradients) by N tile nt, computed by the calling workgroup's 256
// threads through the LDS rings at `lds` (big_lds_bytes). Returns with every DMA load of the tile
// complete; the caller separates two tiles on the same LDS by a barrier.
//
// PIPE = false: the fragments of a k-step are read from LDS right before its MFMAs instead of
// during the previous k-step's (one set of fragment registers instead of two), for a kernel that
// runs two workgroups per CU, where the other workgroup's MFMAs cover the LDS latency. The DMA
// issue order, and so every wait count, is the one of the pipelined loop.
template <int MODE, bool MX, int BM, int RB, int NS, int NSR, bool PIPE = true>
__device__ __forceinline__ void big_tile_at(const GemmArgs& p, int ti, int nt, uint8_t* lds) {
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
  static_assert(big_lds_bytes(BM, RB, NS, NSR) == NS * WSTAGE + NSR * RSTAGE, "LDS size");
  // stage s: weight rows in ring slot s % NS, routed rows in ring slot s % NSR
  auto wbuf = [&](int s) { return lds + (s % NS) * WSTAGE; };
  auto rbuf = [&](int s) { return lds + NS * WSTAGE + (s % NSR) * RSTAGE; };

  int e, row0, row_end;
  if constexpr (MODE == kEpiWgrad) {
    const int mtiles = p.M / BM;
    e = ti / mtiles;
    row0 = (ti % mtiles) * BM;
    row_end = p.M;
  } else {
    // uniform over the workgroup (the operand bases derived from them live in scalar registers)
    const int2 te = p.tiles[ti];
    e = __builtin_amdgcn_readfirstlane(te.x);
    row0 = __builtin_amdgcn_readfirstlane(te.y);
    row_end = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]);
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
  // the operand bases are uniform: keep them in scalar registers (the scale loads address
  // through a scalar base)
  wexp = uniform_ptr(wexp);
  rows_b = uniform_ptr(rows_b);
  if constexpr (MX) {
    wsb = uniform_ptr(wsb);
    rsb = uniform_ptr(rsb);
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
  if constexpr (MX && PIPE) {
    sload(0, nscw, nscr);
  }
#pragma unroll
  for (int b = -(NDEEP - 1); b < 0; ++b)
#pragma unroll
    for (int part = 0; part < SPS; ++part) issue_part(b, part);
  if constexpr (!PIPE) {
    // stage j: its wait and barrier (point j); at a chunk's first stage the chunk's scale words,
    // read here with ordinary loads the compiler waits for itself (in a loop, untracked loads
    // whose registers the compiler may copy or reuse while they are in flight are not safe; they
    // sit where the pipelined loop issues the next chunk's words, so the counted waits only get
    // stricter); then point j's DMA groups, and per k-step the fragments and MFMAs
    for (int j = 0; j < nk; ++j) {
      barrier_point(j);
      if constexpr (MX) {
        if (j % PC == 0) {
          const uint32_t cc = (uint32_t)(j / PC);
#pragma unroll
          for (int i = 0; i < NI; ++i)
            scw[i] = scale_word(*reinterpret_cast<const uint64_t*>(wsb + sw_off[i] + w_cs * cc));
#pragma unroll
          for (int q = 0; q < NJ; ++q)
            scr[q] = scale_word(*reinterpret_cast<const uint64_t*>(rsb + sr_off[q] + r_cs * cc));
        }
      }
#pragma unroll
      for (int part = 0; part < SPS; ++part) issue_part(j, part);
#pragma unroll
      for (int t = 0; t < SPS; ++t) {
        Frags F;
        load_frags(F, j, t);
#pragma unroll
        for (int k = 0; k < NM; ++k) mfma_k(F, k, (j % PC) * SPS + t);
      }
    }
  } else {
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
  }  // PIPE
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
              const uint32_t w4 = e4m3_pack4(hv[4 * b4 + 0] * inv, hv[4 * b4 + 1] * inv,
                                             hv[4 * b4 + 2] * inv, hv[4 * b4 + 3] * inv);
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
    // The bf16 tile goes out through LDS, so that each store instruction writes whole 128-byte
    // lines (16 bytes per lane, two rows of 512 bytes per wave) instead of 16 bytes of 32 rows.
    // Every DMA load and every fragment read of the main loop is complete before LDS is reused.
    constexpr int RS = BN * 2 + 16;  // LDS row stride in bytes (256 bf16 + 16 bytes of padding)
    static_assert(BM * RS <= NS * WSTAGE + NSR * RSTAGE, "the output tile fits the rings' LDS");
    wait_vmcnt<0>();
    lds_barrier();
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      uint8_t* lrow = lds + ((BM / 2) * wm + 32 * j + li) * RS + 2 * (128 * wn + 4 * g);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          uint2 v;
          v.x = pack_bf16x2(acc[i][j][4 * b4 + 0], acc[i][j][4 * b4 + 1]);
          v.y = pack_bf16x2(acc[i][j][4 * b4 + 2], acc[i][j][4 * b4 + 3]);
          *reinterpret_cast<uint2*>(lrow + 2 * (32 * i + 8 * b4)) = v;
        }
    }
    lds_barrier();
    const int c16 = tid & 31;  // 16-byte chunk of the row: output columns n0 + 8 c16 .. + 8
    // rows rr0 + tid / 32, eight rows per pass; a group's LDS reads all go out before its stores
    // (left alone, the compiler moves each read into its row's store condition and waits for it
    // there, one LDS latency per row)
    constexpr int NPASS = BM / 8, GRP = 8;
    static_assert(NPASS % GRP == 0, "whole groups of passes");
#pragma unroll
    for (int q0 = 0; q0 < NPASS; q0 += GRP) {
      uint4 v[GRP];
#pragma unroll
      for (int q = 0; q < GRP; ++q)
        v[q] = *reinterpret_cast<const uint4*>(lds + (8 * (q0 + q) + (tid >> 5)) * RS + 16 * c16);
#pragma unroll
      for (int q = 0; q < GRP; ++q)  // (after all of the group's reads: one wait for them)
        asm volatile("" : "+v"(v[q].x), "+v"(v[q].y), "+v"(v[q].z), "+v"(v[q].w));
#pragma unroll
      for (int q = 0; q < GRP; ++q) {
        const int r = row0 + 8 * (q0 + q) + (tid >> 5);
        if (r < row_end)
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.out) + (size_t)r * p.N + n0 +
                                    8 * c16) = v[q];
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
            const float sg = sigmoid_f(G[q]);
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
                  e4m3_pack4(a4[0] * ig, a4[1] * ig, a4[2] * ig, a4[3] * ig);
              *reinterpret_cast<uint32_t*>(out + 32 + 8 * b4) =
                  e4m3_pack4(c4[0] * iu, c4[1] * iu, c4[2] * iu, c4[3] * iu);
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
    // Staged through LDS as float32, half of the tile's rows at a time (the waves of row half wm
    // write theirs, then all 256 threads store them), so that the stores write whole lines: a row
    // of the tile is 256 outputs, 64 chunks of 4; with split_gate_up, chunk c of a row is output
    // column 4 (c % 32) of the gate half (c < 32) or the up half, i.e. tile column
    // 64 ((c % 32) / 8) + 32 (c / 32) + 4 (c % 8), since the N index alternates 32 gate and 32 up
    // columns.
    constexpr int RSW = BN * 4 + 16;  // LDS row stride in bytes (256 floats + 16 bytes of padding)
    static_assert((BM / 2) * RSW <= NS * WSTAGE + NSR * RSTAGE, "half a tile fits the rings' LDS");
    const int ld = p.split_gate_up ? (p.N >> 1) : p.N;
    const size_t ebase = (size_t)e * p.M * ld;
    wait_vmcnt<0>();
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      lds_barrier();  // the main loop's (or the previous half's) LDS reads are done
      if (wm == half) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          uint8_t* lrow = lds + (32 * j + li) * RSW + 4 * (128 * wn + 4 * g);
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int b4 = 0; b4 < 4; ++b4)
              *reinterpret_cast<f32x4_t*>(lrow + 4 * (32 * i + 8 * b4)) =
                  (f32x4_t){acc[i][j][4 * b4], acc[i][j][4 * b4 + 1], acc[i][j][4 * b4 + 2],
                            acc[i][j][4 * b4 + 3]};
        }
      }
      lds_barrier();
      const int c = tid & 63;  // chunk of 4 outputs
      int lcol = 4 * c;
      void* o = p.out;
      int col = n0 + 4 * c;
      if (p.split_gate_up) {
        const int hc = c >> 5, j4 = c & 31;
        lcol = 64 * (j4 >> 3) + 32 * hc + 4 * (j4 & 7);
        o = hc ? p.out2 : p.out;
        col = (n0 >> 1) + 4 * j4;
      }
      // rows rr0 + tid / 64, four per pass: every pass's LDS read goes out before the stores (one
      // LDS latency per half instead of one per row), and the output type is chosen once
      constexpr int NPASS = BM / 8;
      f32x4_t v[NPASS];
#pragma unroll
      for (int q = 0; q < NPASS; ++q)
        v[q] = *reinterpret_cast<const f32x4_t*>(lds + (4 * q + (tid >> 6)) * RSW + 4 * lcol);
#pragma unroll
      for (int q = 0; q < NPASS; ++q)  // (after all the reads: one wait for them)
        asm volatile("" : "+v"(v[q][0]), "+v"(v[q][1]), "+v"(v[q][2]), "+v"(v[q][3]));
      const size_t at0 = ebase + (size_t)(row0 + (BM / 2) * half + (tid >> 6)) * ld + col;
      if (p.out_f32) {
#pragma unroll
        for (int q = 0; q < NPASS; ++q)
          *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(o) + at0 + (size_t)(4 * q) * ld) =
              v[q];
      } else {
#pragma unroll
        for (int q = 0; q < NPASS; ++q)
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(o) + at0 + (size_t)(4 * q) * ld) =
              make_uint2(pack_bf16x2(v[q][0], v[q][1]), pack_bf16x2(v[q][2], v[q][3]));
      }
    }
  }
}


// the tile of workgroup jx of XCD x (big_tile_coords); none for a surplus workgroup
template <int MODE, bool MX, int BM, int RB, int NS, int NSR, bool PIPE = true>
__device__ __forceinline__ void big_tile(const GemmArgs& p, int x, int jx, uint8_t* lds) {
  const int mt_total = MODE == kEpiWgrad ? p.tiles_total : *p.tile_count;
  int ti, nt;
  // (before any barrier)
  if (!big_tile_coords(mt_total, p.N / kBigBN, p.band_gm, x, jx, ti, nt)) return;
  big_tile_at<MODE, MX, BM, RB, NS, NSR, PIPE>(p, ti, nt, lds);
}

}  // namespace

// Host: the forward FFN's two large-tile GEMMs (GEMM-1 with the SwiGLU epilogue into H, GEMM-2
// into out_rows) over a tile table of bm-row tiles in the FFN workspace `ws`, as the grouped-GEMM
// launcher sets them up; MXFP8 scales chunk-major throughout (the routed-row input's with
// row_scales_rows rows). Returns the table's capacity in tiles; G and U are not kept.
int ffn_big_gemm_args(const void* rows, const uint8_t* row_scales, int row_scales_rows,
                      const int32_t* offsets, const void* prepared, uint16_t* out_rows, void* ws,
                      int R, int h, int m, int E_loc, bool mx, const int32_t* row_src,
                      int row_div, int bm, GemmArgs& a1, GemmArgs& a2);

}  // namespace moe
