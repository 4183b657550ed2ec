// Internal declarations of the MI355X MoE library: device helpers shared by the kernels and the
// host-side launchers each kernel file exports to the C-ABI front end (moe_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ------------------------------------------------------------------------------------------------
// Vector types for 16-byte memory operations and MFMA operands (gfx950, wave64)
// ------------------------------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;

constexpr int kWave = 64;
constexpr int kMxBlock = 32;

// ------------------------------------------------------------------------------------------------
// bfloat16 <-> float32
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round a finite float32 to bfloat16, to nearest with ties to even.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ------------------------------------------------------------------------------------------------
// MX (OCP Microscaling) E4M3 elements with an E8M0 block scale
// ------------------------------------------------------------------------------------------------
// Block exponent of a block whose largest magnitude is amax: floor(log2 amax) - 8 (8 = exponent
// of E4M3's largest normal, 448), clamped to [-127, 127]; -127 for an all-zero block. Read off the
// float32 exponent field; float32 subnormal amax (< 2^-126) gives -127 after clamping too.
__device__ __forceinline__ int mx_block_exponent(float amax) {
  uint32_t ex = (__float_as_uint(amax) >> 23) & 0xffu;  // amax >= 0
  int s = (ex == 0u) ? -127 : (int)ex - 127 - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// 2^-s as a float (s in [-127, 127]): exact power of two. 2^127 is a normal float32.
__device__ __forceinline__ float mx_inv_scale(int s) {
  int e = 127 - s;  // biased exponent of 2^-s, in [0, 254]
  return e == 0 ? __uint_as_float(0x00400000u) /* 2^-127, subnormal */
                : __uint_as_float((uint32_t)e << 23);
}

// The logistic function 1 / (1 + e^-z) with the hardware base-2 exponential and reciprocal
// (v_exp_f32, v_rcp_f32: about one ulp each): e^-z = 2^(-z log2 e). For z far below zero the
// exponential overflows to +inf and the result is 0; far above, 2^-big is 0 and the result 1.
__device__ __forceinline__ float sigmoid_f(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// silu(z) = z * sigmoid(z)
__device__ __forceinline__ float silu_f(float z) { return z * sigmoid_f(z); }

// E4M3 code of y (already divided by the block scale): round to nearest, ties to even mantissa,
// |y| >= 448 saturates to 448, the sign of zero is kept, NaN is never produced.
// Normal range |y| >= 2^-6: with |y| = f * 2^e (1 <= f < 2) the mantissa is rint(|y| * 2^(3-e)) - 8,
// a carry to 16 moves to the next binade. Below 2^-6: n = rint(|y| * 2^9), n = 8 is code 0x08.
__device__ __forceinline__ uint32_t e4m3_encode_rule(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = __uint_as_float(u & 0x7fffffffu);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7eu;
  } else if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);  // exact scaling, then round half to even
  } else {
    int e = (int)((u >> 23) & 0xffu) - 127;          // -6 .. 8
    float scaled = a * __uint_as_float((uint32_t)(127 + 3 - e) << 23);  // exact: a * 2^(3-e)
    uint32_t n = (uint32_t)__builtin_rintf(scaled);  // 8 .. 16
    if (n == 16u) { n = 8u; ++e; }
    code = ((uint32_t)(e + 7) << 3) | (n - 8u);
  }
  return code | sign;
}

// The same code from the hardware conversion: v_cvt_pk_fp8_f32 rounds to nearest even into OCP
// E4M3 and keeps the sign of zero; the clamp to +-448 first gives the saturation. Equal to
// e4m3_encode_rule for every float32 (a GPU test compares the two over all of them up to 2^17).
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const float c = fminf(fmaxf(y, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xffu;
}

// Four codes in one word, a in the low byte: two packed conversions.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  c = fminf(fmaxf(c, -448.0f), 448.0f);
  d = fminf(fmaxf(d, -448.0f), 448.0f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// ------------------------------------------------------------------------------------------------
// Alignment helpers for workspace carving
// ------------------------------------------------------------------------------------------------
constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool aligned(const void* p) { return ((uintptr_t)p % kAlign) == 0; }

// ------------------------------------------------------------------------------------------------
// Host-side launchers (each returns hipGetLastError() after enqueueing)
// ------------------------------------------------------------------------------------------------
// Router (moe_route_kernels.hip): the logits on the matrix cores from x and the router matrix
// interleaved by 8 columns (bf16), in router_xf_bytes(T, h, E) bytes of scratch (the size of the
// float32 interleaved copy the persistent forward's vector-ALU router reads)
size_t router_xf_bytes(int T, int h, int E);
hipError_t launch_router_logits_xf(const uint16_t* x, const uint16_t* w_router, const float* bias,
                                   float* logits, int T, int h, int E, float* scratch,
                                   hipStream_t st);
hipError_t launch_topk_softmax(const float* logits, int32_t* idx, float* w, int T, int E, int k,
                               hipStream_t st);

// Schedule + gather (moe_permute_kernels.hip)
constexpr int kSchedChunk = 256;  // assignments per schedule block
size_t sched_workspace_bytes(int R, int E_loc);
hipError_t launch_schedule(const int32_t* assign, int R, int E_loc, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                           hipStream_t st);
hipError_t launch_gather_bf16(const uint16_t* x, const int32_t* inv, uint16_t* rows, int T, int h,
                              int k, hipStream_t st);
hipError_t launch_gather_mxfp8(const uint16_t* x, const int32_t* inv, uint8_t* rows,
                               uint8_t* scales, int T, int h, int k, hipStream_t st);
// x quantised once per token: codes [T][h] E4M3, scales chunk-major [h/256][T][8] E8M0 (h % 256
// == 0), for a grouped GEMM that gathers the routed rows through perm itself
hipError_t launch_quantize_tokens_mxfp8(const uint16_t* x, uint8_t* codes, uint8_t* scales_cm,
                                        int T, int h, hipStream_t st);

// Grouped GEMMs + weight preparation (moe_gemm_kernels.hip)
size_t ffn_workspace_bytes(int R, int h, int m, int E_loc, bool mx);
size_t prepared_bytes(int E_loc, int h, int m, bool mx);
hipError_t launch_prepare_weights(const uint16_t* w_gate, const uint16_t* w_up,
                                  const uint16_t* w_down, void* prepared, int E_loc, int h, int m,
                                  bool mx, hipStream_t st);
// ev (optional): three events recorded after the tile table, GEMM-1 and GEMM-2.
// gu_out (optional, large-tile shapes only): GEMM-1's G and U as float32 [R][2m], gate/up
// interleaved per 32 like the prepared W1 rows, kept for a backward pass.
// row_src (optional, large-tile shapes only): GEMM-1 reads routed row r from row
// row_src[r] / row_div of `rows` ([src_rows][h], e.g. the tokens x with row_src = perm,
// row_div = k: the gather done by the GEMM's own loads). scales_cm: row_scales are already
// chunk-major [h/256][rows][8] (else natural [rows][h/32]).
hipError_t launch_expert_ffn(const void* rows, const uint8_t* row_scales, const int32_t* offsets,
                             const void* prepared, uint16_t* out_rows, void* ws, int R, int h,
                             int m, int E_loc, bool mx, hipStream_t st,
                             const hipEvent_t* ev = nullptr, float* gu_out = nullptr,
                             const int32_t* row_src = nullptr, int row_div = 1, int src_rows = 0,
                             bool scales_cm = false);
bool ffn_big(int h, int m);

// Backward GEMMs (moe_gemm_kernels.hip). Both need h % 256 == 0 and m % 256 == 0.
// K segments of the weight gradients: each expert's routed rows padded to a multiple of this
inline int wgrad_k_align(bool mx) { return mx ? 256 : 64; }
// the M-tile table of the backward's routed-row GEMMs (count + tiles) and its size
size_t gemm_tiles_bytes(int R, int E_loc);
hipError_t launch_gemm_tiles(const int32_t* offsets, void* tiles_ws, int R, int E_loc, bool mx,
                             hipStream_t st);
// dG|dU (with the SwiGLU backward) from dO and the prepared W_down rows [e][m][h], then dA from
// dG|dU and the prepared [W_gate | W_up] rows [e][h][2m]; ev_mid (or null) between the two.
// gu: the forward's G | U (float32); dgu: bf16 or E4M3 (+ dgu_s); dgu_f32: the same in float32
hipError_t launch_bwd_dgrad(const void* dO, const uint8_t* dO_s, const int32_t* offsets,
                            const uint8_t* w2b, const uint8_t* w2b_s, const uint8_t* w1b,
                            const uint8_t* w1b_s, const float* gu, void* dgu, uint8_t* dgu_s,
                            float* dgu_f32, uint16_t* dA, const void* tiles_ws, int R, int h,
                            int m, int E_loc, bool mx, hipStream_t st, hipEvent_t ev_mid);
// weight gradients from the per-expert transposed operands ([C][kpad_e] at koff[e] * C)
hipError_t launch_bwd_wgrad(const uint8_t* At, const uint8_t* At_s, const uint8_t* dGUt,
                            const uint8_t* dGUt_s, const uint8_t* Ht, const uint8_t* Ht_s,
                            const uint8_t* dOt, const uint8_t* dOt_s, const int32_t* koff,
                            void* dw_gate, void* dw_up, void* dw_down, bool out_f32, int h, int m,
                            int E_loc, bool mx, hipStream_t st, hipEvent_t ev_mid);

// Backward data movement (moe_backward_kernels.hip)
size_t prepared_bwd_bytes(int E_loc, int h, int m, bool mx);
struct PreparedBwd {
  const uint8_t *w1b, *w1b_s, *w2b, *w2b_s;
};
PreparedBwd prepared_bwd_views(const void* prepared_bwd, int E_loc, int h, int m, bool mx);
hipError_t launch_prepare_bwd_weights(const uint16_t* w_gate, const uint16_t* w_up,
                                      const uint16_t* w_down, void* prepared_bwd, int E_loc,
                                      int h, int m, bool mx, hipStream_t st);
// koff[0..E_loc]: exclusive scan of the expert row counts rounded up to `align`
hipError_t launch_kpad_table(const int32_t* offsets, int E_loc, int align, int32_t* koff,
                             hipStream_t st);
// dO[r] = w[perm[r]] * dY[perm[r] / k] for the routed rows, bf16 or MX per 32 along h
hipError_t launch_uncombine(const uint16_t* dy, const int32_t* perm, const float* w,
                            const int32_t* offsets, int E_loc, void* dO, uint8_t* dO_s, int R,
                            int h, int k, bool mx, hipStream_t st);
// Sources of the per-expert transposes ([C][kpad_e] per expert, MX per 32 along the rows)
enum TransposeSrc : int {
  kTrX = 0,      // x[perm[r] / k], bf16                        (C = h)
  kTrDO = 1,     // w[perm[r]] * dY[perm[r] / k], dY bf16       (C = h)
  kTrH = 2,      // silu(G) * U from the saved float32 G | U    (C = m)
  kTrRows = 3,   // row r of a float32 [R][C] matrix            (C = 2m: dG | dU)
};
// rows_max: an upper bound of koff[E_loc] (R + E_loc * (align - 1))
hipError_t launch_bwd_transpose(int src_kind, const void* src, const int32_t* perm,
                                const float* w, const int32_t* offsets, const int32_t* koff,
                                int E_loc, int C, int k, int rows_max, uint8_t* dst,
                                uint8_t* dst_s, bool mx, hipStream_t st);

// Combine (moe_combine_kernels.hip); w == nullptr: every weight is 1 (the backward's un-permute).
// w_router != nullptr (the un-permute of a router layer): the router's part of the input gradient,
// sum_j dl[t k + j] W_r[assign[t k + j]], is added before the rounding.
hipError_t launch_combine(const uint16_t* out_rows, const int32_t* inv, const float* w,
                          const uint16_t* shared_out, uint16_t* y, int T, int h, int k,
                          hipStream_t st, const uint16_t* w_router = nullptr,
                          const int32_t* assign = nullptr, const float* dl = nullptr, int E = 0);

// Backward through the gate weights and the router (moe_router_backward_kernels.hip).
// dgate[a] = <dY[a / k], O[inv[a]]>; with dl != nullptr also the selected-logit gradients
// dl[a] = w[a] (dgate[a] - sum over the token's slots of w dgate)
hipError_t launch_gate_grads(const uint16_t* dy, const uint16_t* O, const int32_t* inv,
                             const float* w, float* dgate, float* dl, int T, int h, int k,
                             hipStream_t st);
// rows per chunk of the router-matrix gradient, and the chunk count bound for R rows, E experts
constexpr int kRouterChunk = 64;
size_t router_wgrad_tiles(int R, int E);
// dW_r [E][h] and db [E] (or null) from dl and the rows of each expert (chunk tile table built
// with launch_tile_table(bm = kRouterChunk)); partial: [max_tiles][h] float, partial_db [max_tiles]
hipError_t launch_router_wgrad(const int2* tiles, const int* tile_count, int max_tiles,
                               const int32_t* offsets, const int32_t* perm, const float* dl,
                               const uint16_t* x, int h, int k, int E, float* partial,
                               float* partial_db, float* dw_router, float* dbias,
                               hipStream_t st);
// (expert, first row) of every bm-row chunk of every expert's rows, entries past the count (-1, 0)
hipError_t launch_tile_table(const int32_t* offsets, int E_loc, int bm, int max_tiles,
                             int2* tiles, int* tile_count, hipStream_t st);

// the hardware E4M3 encoder against e4m3_encode_rule on every float32 below 2^17 (both signs),
// and the byte order of e4m3_pack4: *mismatches (device) = the number of differing inputs
hipError_t launch_check_e4m3(int64_t* mismatches, hipStream_t st);

// rows per M tile of the persistent forward's GEMMs: the 128-row large tile (its accumulators
// leave the registers the work loop around it needs; the 192- and 256-row tiles would spill)
constexpr int kPersistentRows = 128;

// The persistent forward's buffers (device pointers; the forward workspace's, plus the float32
// router matrix, the first tile of each expert and the synchronisation words).
struct PersistentBuffers {
  const uint16_t* x;
  const uint16_t* w_router;  // null: the assignment is given
  const float* bias;
  const int32_t* assign;
  const float* assign_w;
  const void* prepared;
  uint16_t* y;
  int32_t* status;
  float* wi;
  float* logits;
  int32_t* idx;
  float* tw;
  int32_t* cc;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
  uint8_t* qrows;
  uint8_t* qscales;
  void* ffn_ws;
  uint16_t* out_rows;
  int32_t* etile;
  int* sync;
  void* args;  // persistent_args_bytes(): the kernel's argument block, in device memory
};
// synchronisation words of the persistent forward over R rows in bm-row tiles
size_t persistent_sync_ints(int R, int E_loc, int bm);
size_t persistent_args_bytes();
// one launch of the persistent forward (after a small kernel that clears the synchronisation
// words); num_cu workgroups, each wait bounded by `timeout` wall-clock ticks
hipError_t launch_forward_persistent(const PersistentBuffers& b, int T, int h, int m, int E,
                                     int E_loc, int k, bool mx, int num_cu, long long timeout,
                                     hipStream_t st);

}  // namespace moe
