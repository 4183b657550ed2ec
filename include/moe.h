/*
 * moe.h - C ABI of the MI355X (gfx950) single-GPU mixture-of-experts layer.
 *
 * The library computes one GPU's share of an MoE layer forward pass: router logits, top-k gating
 * with softmax renormalisation, a device-side schedule that groups the routed rows by expert,
 * a gather of the rows (fused with MXFP8 quantisation), SwiGLU expert FFNs as grouped GEMMs in
 * BF16 or MXFP8, and a fixed-order weighted combine back to token order.
 *
 * The method is the Mixture-of-Kittens MoE layer ("Mixture-of-Kittens: Cursor's Open-Source MoE
 * Training Megakernel for NVL72": TL;DR, flowchart, Key claims), restricted to what one GPU
 * computes; the cross-GPU dispatch and combine are not part of this library.
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers unless marked "host". All tensors are dense and row-major.
 *     bfloat16 is passed as uint16_t bit patterns, E4M3 codes and E8M0 scales as uint8_t,
 *     indices as int32_t.
 *   - Notation: T source tokens, hidden h, expert width m, E router experts, top-k k, E_loc
 *     experts held by this GPU, R = T*k routed rows, assignment a = t*k + j (token t, slot j).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every call only enqueues
 *     work on it: no host synchronisation, no allocation, no state kept between calls (the one
 *     exception, moe_permute_static, keeps a static scratch array per GPU). Shapes alone size
 *     every launch; the device-side expert counts are never read by the host.
 *   - Ownership: the caller owns every buffer, including workspaces (sized by the *_bytes
 *     queries) and prepared weights. Buffers must not overlap unless stated.
 *   - Alignment: every pointer must be 16-byte aligned (torch allocations are 256-byte aligned).
 *   - Errors: arguments are checked on the host before anything is enqueued. MOE_EINVAL means a
 *     null required pointer, a misaligned pointer or an inconsistent shape, and nothing was
 *     enqueued. MOE_EUNSUPPORTED means a valid shape the kernels do not cover (see each call).
 *     MOE_EHIP means a launch failed (hipGetLastError). No C++ exception crosses the ABI.
 *   - Determinism: there are no floating-point atomics and no split reductions; every sum has a
 *     fixed order, so identical inputs give bitwise identical outputs (the page's "bitwise
 *     deterministic" property, TL;DR and Key claims).
 *   - Thread safety: calls on different streams with different buffers may run concurrently,
 *     except moe_permute_static calls on one GPU, which share that GPU's scratch array.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,
  MOE_EUNSUPPORTED = 2,
  MOE_EHIP = 3,
  MOE_ENOSCRATCH = 4, /* moe_permute_static: the shape needs more than the static scratch */
  MOE_ETIMEOUT = 5    /* moe_forward_persistent (device status word): a wait ran out of time */
} moe_status;

/* Expert GEMM precision. MOE_MXFP8: E4M3 elements with one E8M0 scale per 32 consecutive elements
 * along each GEMM's reduction axis (OCP Microscaling v1.0); the page's Key claims make MXFP8 the
 * default with activation quantisation fused into dispatch, the grouped GEMMs and the SwiGLU. */
typedef enum { MOE_BF16 = 0, MOE_MXFP8 = 1 } moe_dtype;

typedef struct {
  int32_t T;        /* source tokens, >= 1 */
  int32_t h;        /* hidden size, multiple of 64 (MXFP8: of 256) */
  int32_t m;        /* expert intermediate width, multiple of 32 (MXFP8: of 256) */
  int32_t E;        /* router experts, >= k (only the router uses it) */
  int32_t k;        /* top-k, 1 <= k <= min(E, 16) */
  int32_t E_loc;    /* experts held by this GPU, 1 .. 1024 (router use: E_loc == E) */
  int32_t m_shared; /* width of a BF16 shared SwiGLU expert over the T tokens, 0 = none */
} moe_shape;

/* The name and meaning of a status code; any int (a status held in an int, or an unknown code,
 * which gives "unknown moe_status"). */
const char* moe_status_string(int code);
int moe_abi_version(void);

/* Diagnostic: the E4M3 encoder the kernels use (the hardware conversion after a clamp to +-448)
 * against the rounding rule of the MX definition (round to nearest even, saturate to 448, keep the
 * sign of zero), on the current device, for every float32 of magnitude below 2^17 and both signs,
 * plus the byte order of the four-code packing. mismatches: device int64, set to the number of
 * inputs on which they differ (0 expected) once the stream has run. MOE_EINVAL for a null or
 * misaligned pointer. */
moe_status moe_check_e4m3(int64_t* mismatches, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Weight preparation (offline, not part of a forward pass).
 *
 * w_gate, w_up: [E_loc][h][m] bf16 (y = x W convention); w_down: [E_loc][m][h] bf16.
 * `prepared` receives moe_prepared_weight_bytes() bytes in the layout the grouped GEMMs read:
 *   MOE_BF16 : W1[e][2m][h] bf16 (row n = output column n of GEMM-1; gate and up columns
 *              interleaved in blocks of 32: rows 64c..64c+31 are gate columns 32c..32c+31,
 *              rows 64c+32..64c+63 the up columns of the same range), then W2[e][h][m] bf16
 *              (W_down transposed). When h % 256 == 0 and 2m % 256 == 0 (the large-tile
 *              kernels) each matrix is stored K-tiled: [e][rows/256][K bytes/128][256][128
 *              bytes], i.e. every 128-byte K slice of a 256-row panel is one contiguous 32 KB
 *              block (one pipeline stage of the GEMM, read with whole DRAM pages).
 *   MOE_MXFP8: the same two matrices as E4M3 codes (K-tiled as above; always so, since MXFP8
 *              needs h % 256 == 0 and m % 256 == 0), each followed by its E8M0 scales; blocks
 *              of 32 run along h for W1 and along m for W2, i.e. along each GEMM's reduction
 *              axis, and the scales are stored chunk-major: [e][h/256][2m][8] and
 *              [e][m/256][h][8], the 8 block scales of one 256-element chunk of a row side by
 *              side (so a tile's scale words for one chunk are a few cache lines).
 * The shared expert is prepared with the same call, shape.E_loc = 1, shape.m = m_shared, MOE_BF16.
 * ------------------------------------------------------------------------------------------- */
size_t moe_prepared_weight_bytes(const moe_shape* s, moe_dtype dt);
moe_status moe_prepare_weights(const moe_shape* s, moe_dtype dt, const uint16_t* w_gate,
                               const uint16_t* w_up, const uint16_t* w_down, void* prepared,
                               void* stream);

/* ---------------------------------------------------------------------------------------------
 * moe_route: router logits, top-k, renormalised softmax weights ("token routing" of the page's
 * companion news digest, Merged summary; the workloads define softmax over logits, top-k,
 * renormalise).
 *
 * x [T][h] bf16; w_router [E][h] bf16 (row e = expert e); bias [E] float or NULL.
 * logits [T][E] float (output): l[t,e] = sum_i x[t,i] w_router[e,i] + bias[e], summed in float32
 *   in the fixed order i = 0 .. h-1 starting from +0.0 (one rounding per step), then + bias.
 * topk_idx [T][k] int32 (output): the k largest logits per token, logit descending, lower expert
 *   index first on ties, -0.0 equal to +0.0; slot j holds the j-th ranked expert.
 * topk_w [T][k] float (output): exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected.
 * Requires E_loc == E. Unsupported: E > 1024 or k > 16.
 * ws: moe_route_workspace_bytes() bytes of scratch (w_router staged as float32, interleaved by 8
 *   columns, so a wave's row loads are contiguous; x is staged through LDS; the sum order above is
 *   unchanged).
 * ------------------------------------------------------------------------------------------- */
size_t moe_route_workspace_bytes(const moe_shape* s);
moe_status moe_route(const moe_shape* s, const uint16_t* x, const uint16_t* w_router,
                     const float* bias, float* logits, int32_t* topk_idx, float* topk_w,
                     void* ws, void* stream);

/* ---------------------------------------------------------------------------------------------
 * moe_permute: the device-side schedule and the gather (the page's flowchart: a device-side
 * schedule kernel with no CPU synchronisation; Key claims: dynamic per-expert counts absorbed by
 * a fixed-size buffer, no host synchronisation; quantisation fused into dispatch).
 *
 * assign [T*k] int32: local expert of assignment a (0 <= assign[a] < E_loc; e.g. topk_idx).
 * x [T][h] bf16.
 * Outputs: counts [E_loc], offsets [E_loc+1] (exclusive scan), perm [R] (routed row r holds
 *   assignment perm[r]; rows of expert e are offsets[e] .. offsets[e+1]-1 with assignments
 *   ascending), inv [R] (inv[perm[r]] == r), and the routed rows (capacity R, nothing dropped):
 *   MOE_BF16 : rows [R][h] bf16, rows[r] = x[perm[r] / k]; row_scales unused (may be NULL).
 *   MOE_MXFP8: rows [R][h] E4M3 codes and row_scales [R][h/32] E8M0 of x[perm[r] / k], quantised
 *              per 32 along h: s = floor(log2 amax) - 8 clamped to [-127, 127] (s = -127 for an
 *              all-zero block), code = E4M3(v / 2^s) with round-to-nearest-even, saturation at
 *              448, sign of zero kept; scale byte s + 127. Each token is quantised once.
 * ws: moe_permute_workspace_bytes() bytes of scratch.
 * ------------------------------------------------------------------------------------------- */
size_t moe_permute_workspace_bytes(const moe_shape* s);
moe_status moe_permute(const moe_shape* s, moe_dtype dt, const int32_t* assign,
                       const uint16_t* x, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* inv, void* rows, uint8_t* row_scales, void* ws, void* stream);

/* ---------------------------------------------------------------------------------------------
 * moe_permute_static: moe_permute for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc). The same arguments and
 * results as moe_permute, minus `ws`: the schedule's scratch (moe_permute_workspace_bytes() bytes:
 * the per-chunk expert histograms, every byte written before it is read, so nothing needs
 * clearing) is a static device array of MOE_PERMUTE_STATIC_SCRATCH_BYTES bytes that the library
 * holds on each GPU it runs on until the process ends. Its address on the current device is
 * looked up once per device on the first call there. The call allocates nothing.
 * Errors: as moe_permute; MOE_ENOSCRATCH (nothing enqueued) when moe_permute_workspace_bytes()
 * exceeds MOE_PERMUTE_STATIC_SCRATCH_BYTES (e.g. R * E_loc > 2^31 at 256 assignments per chunk);
 * MOE_EHIP when the array's address cannot be obtained.
 * Concurrency: every call on one GPU uses that GPU's one array, so calls that overlap in time on
 * one GPU (different streams, or threads) race and must be serialised by the caller; calls on
 * one stream never overlap.
 * ------------------------------------------------------------------------------------------- */
#define MOE_PERMUTE_STATIC_SCRATCH_BYTES ((size_t)8 << 20)
moe_status moe_permute_static(const moe_shape* s, moe_dtype dt, const int32_t* assign,
                              const uint16_t* x, int32_t* counts, int32_t* offsets,
                              int32_t* perm, int32_t* inv, void* rows, uint8_t* row_scales,
                              void* stream);

/* ---------------------------------------------------------------------------------------------
 * moe_expert_ffn: the SwiGLU experts as grouped GEMMs (Key claims: expert grouped GEMMs, MXFP8,
 * fused SwiGLU, fused quantisation).
 *
 * For each local expert e and each routed row r in offsets[e] .. offsets[e+1]-1:
 *   G = rows[r] W_gate[e], U = rows[r] W_up[e] (float32 accumulation), H = silu(G) * U,
 *   out_rows[r] = H W_down[e] rounded to bf16.
 *   MOE_BF16 : H is rounded to bf16 before the second GEMM.
 *   MOE_MXFP8: rows/row_scales as written by moe_permute; H is MX-quantised per 32 along m from
 *              its float32 value inside the first GEMM's epilogue.
 * rows: R = T*k rows (for the shared expert: T rows with shape.k = 1, E_loc = 1, offsets {0, T}).
 * offsets [E_loc+1] device int32 (from moe_permute); prepared from moe_prepare_weights.
 * ws: moe_expert_ffn_workspace_bytes() bytes (holds the tile table and H).
 * ------------------------------------------------------------------------------------------- */
size_t moe_expert_ffn_workspace_bytes(const moe_shape* s, moe_dtype dt);
moe_status moe_expert_ffn(const moe_shape* s, moe_dtype dt, const void* rows,
                          const uint8_t* row_scales, const int32_t* offsets, const void* prepared,
                          uint16_t* out_rows, void* ws, void* stream);

/* ---------------------------------------------------------------------------------------------
 * moe_combine: y[t] = S[t] + sum_{j = 0 .. k-1, ascending} w[t*k+j] * out_rows[inv[t*k+j]],
 * accumulated in float32 starting from S[t] (or +0.0) and rounded to bf16 once (the page's fixed
 * floating-point order, TL;DR and Key claims). Gather form, no atomics.
 * out_rows [R][h] bf16; inv [R]; topk_w [R] float; shared_out [T][h] bf16 or NULL; y [T][h] bf16.
 * ------------------------------------------------------------------------------------------- */
moe_status moe_combine(const moe_shape* s, const uint16_t* out_rows, const int32_t* inv,
                       const float* topk_w, const uint16_t* shared_out, uint16_t* y,
                       void* stream);

/* ---------------------------------------------------------------------------------------------
 * moe_forward: the whole layer on one stream, no host synchronisation:
 *   route (if w_router != NULL) -> permute -> expert FFN -> [shared expert] -> combine.
 * x [T][h] bf16.
 * Router use: w_router [E][h], bias [E] or NULL; assign/assign_w must be NULL; E_loc == E.
 * Expert-share use: w_router == NULL; assign [T*k] local expert ids and assign_w [T*k] gate
 *   weights given by the caller (one expert-parallel rank's share).
 * prepared: E_loc experts from moe_prepare_weights(dt); shared_prepared: BF16 shared expert
 *   (shape.m_shared > 0) or NULL. y [T][h] bf16 output.
 * saved: NULL, or moe_saved_bytes() bytes that receive what the backward needs (training): the
 *   schedule (offsets, perm, inv), the gate weight and local expert of every assignment, GEMM-1's
 *   G and U in float32 and the expert outputs [R][h] bf16 (GEMM-2 writes them there instead of
 *   into ws, so the out_rows view is then not written). Needs h % 256 == 0 and m % 256 == 0 (else
 *   MOE_EUNSUPPORTED).
 * ws: moe_forward_workspace_bytes() bytes. The intermediates stay in it; moe_forward_views()
 *   gives their addresses.
 * Gather: when h % 256 == 0 and 2m % 256 == 0 the first grouped GEMM reads routed row r straight
 *   from token perm[r] / k (of x, or of x quantised once per token for MXFP8) with its own loads,
 *   so the forward writes no routed-row copy; the result is the one moe_permute + moe_expert_ffn
 *   give (the same values enter the same MFMAs).
 * ------------------------------------------------------------------------------------------- */
size_t moe_forward_workspace_bytes(const moe_shape* s, moe_dtype dt);
size_t moe_saved_bytes(const moe_shape* s, moe_dtype dt);
moe_status moe_forward(const moe_shape* s, moe_dtype dt, const uint16_t* x,
                       const uint16_t* w_router, const float* bias, const int32_t* assign,
                       const float* assign_w, const void* prepared, const void* shared_prepared,
                       uint16_t* y, void* saved, void* ws, void* stream);

/* ---------------------------------------------------------------------------------------------
 * moe_forward_ring: the forward of any number of tokens through a fixed-size buffer (the pages'
 * macrobatch ring: "Mixture-of-Kittens" flowchart, a ring buffer of a few hundred MB; the news
 * digest's Merged summary and the 1.41x article: a fixed-size ring token buffer cycled at
 * minibatch granularity). The T tokens go through `ring` in consecutive minibatches of
 * moe_forward_ring_tokens(s, dt, ring_bytes) tokens (the last one shorter); each minibatch runs
 * moe_forward on its tokens with `ring` as its workspace, one after another on `stream`, with no
 * host synchronisation. Every output row depends only on its own token (routing, per-token MX
 * quantisation, per-row expert GEMMs with a fixed K order, per-token combine), so y is bitwise the
 * y of one moe_forward over all T tokens; memory stays at ring_bytes whatever T is. Expert weights
 * are read once per minibatch, so a ring too small for a few GEMM waves of rows per expert costs
 * throughput, not correctness. Arguments as moe_forward (no saved state). minibatch_tokens (host,
 * optional) receives the minibatch size. MOE_EINVAL (nothing enqueued) when even one token's
 * minibatch does not fit.
 * moe_forward_ring_tokens: the largest token count whose forward workspace fits ring_bytes, T if
 * that is all of them, else rounded down to a multiple of 4 / gcd(k, 4) so that every minibatch's
 * slice of assign and assign_w stays 16-byte aligned; 0 when no such count fits.
 * ------------------------------------------------------------------------------------------- */
int32_t moe_forward_ring_tokens(const moe_shape* s, moe_dtype dt, size_t ring_bytes);
moe_status moe_forward_ring(const moe_shape* s, moe_dtype dt, const uint16_t* x,
                            const uint16_t* w_router, const float* bias, const int32_t* assign,
                            const float* assign_w, const void* prepared,
                            const void* shared_prepared, uint16_t* y, void* ring,
                            size_t ring_bytes, int32_t* minibatch_tokens /* host */,
                            void* stream);

/* -------------------------------------------------------------------------------------------
 * moe_forward_persistent: the same forward as moe_forward, in one persistent kernel (the pages'
 * megakernel: Mixture-of-Kittens page, TL;DR and flowchart, where the SMs hand work to each other
 * through local counters rather than global barriers; news digest, Merged summary, on a schedule
 * that never waits for the CPU). One workgroup per CU takes work items (token blocks, assignment
 * chunks, GEMM tiles) from per-XCD queues in step order; GEMM-2 on an M tile starts as soon as
 * that tile's GEMM-1 N tiles are done, and a token's combine as soon as its rows' GEMM-2 tiles
 * are. Preceded by one small kernel that clears the queues and counters in ws.
 *
 * Arguments as moe_forward, without saved state or a shared expert. y is bitwise moe_forward's y.
 * status: device int32, set to MOE_OK by the launch and to MOE_ETIMEOUT if an internal wait
 * exceeded its bound (timeout_ms, wall clock; then y is undefined): read it after the stream
 * has finished. ws: moe_forward_persistent_workspace_bytes(). Shapes: h % 256 == 0,
 * m % 128 == 0 (2m % 256 == 0), k <= 16, else MOE_EUNSUPPORTED; m_shared > 0: MOE_EUNSUPPORTED.
 * The kernel needs every queue served: the launch has one workgroup per CU of the device.
 * ------------------------------------------------------------------------------------------- */
size_t moe_forward_persistent_workspace_bytes(const moe_shape* s, moe_dtype dt);
moe_status moe_forward_persistent(const moe_shape* s, moe_dtype dt, const uint16_t* x,
                                  const uint16_t* w_router, const float* bias,
                                  const int32_t* assign, const float* assign_w,
                                  const void* prepared, uint16_t* y, void* ws, int32_t* status,
                                  int32_t timeout_ms, void* stream);

/* Profiling variant of moe_forward: the same work on the same stream, plus hipEventRecord of the
 * caller's events at the stage boundaries, so a caller can time each kernel live:
 *   ev[0] router logits ev[1] top-k ev[2] schedule ev[3] gather ev[4] tile table ev[5] GEMM-1
 *   ev[6] GEMM-2 ev[7] shared expert ev[8] combine ev[9]
 * `events` is a host array of MOE_PROFILE_EVENTS hipEvent_t handles created by the caller
 * (hipEventCreate); stages that do not run for a shape have back-to-back events. */
#define MOE_PROFILE_EVENTS 10
moe_status moe_forward_profiled(const moe_shape* s, moe_dtype dt, const uint16_t* x,
                                const uint16_t* w_router, const float* bias,
                                const int32_t* assign, const float* assign_w,
                                const void* prepared, const void* shared_prepared, uint16_t* y,
                                void* saved, void* ws, void* const* events /* host */,
                                void* stream);

/* Addresses of the intermediates moe_forward leaves in `ws` (device pointers into ws; NULL when a
 * buffer does not exist for this shape). Host-only arithmetic, nothing is enqueued. */
typedef struct {
  float* logits;       /* [T][E]      router use only */
  int32_t* topk_idx;   /* [T][k]      router use only */
  float* topk_w;       /* [T][k]      router use only */
  int32_t* counts;     /* [E_loc] */
  int32_t* offsets;    /* [E_loc+1] */
  int32_t* perm;       /* [R] */
  int32_t* inv;        /* [R] */
  void* rows;          /* [R][h] bf16 or E4M3: the routed rows, when the forward materialises
                          them (h % 256 != 0 or 2m % 256 != 0); on the large-tile shapes GEMM-1
                          gathers them itself and this buffer holds, for MXFP8, the tokens
                          quantised once ([T][h] codes), for BF16 scratch */
  uint8_t* row_scales; /* [R][h/32], MXFP8 only (large-tile shapes: the tokens' scales,
                          [h/256][T][8]) */
  uint16_t* out_rows;  /* [R][h] bf16 */
  uint16_t* shared_out;/* [T][h] bf16 shared expert output, if any */
} moe_forward_views_t;
moe_status moe_forward_views(const moe_shape* s, moe_dtype dt, void* ws,
                             moe_forward_views_t* views /* host */);

/* ---------------------------------------------------------------------------------------------
 * Backward of the expert path (the page's Key claims measure the MXFP8 backward with the same
 * fused quantisation as the forward; its flowchart mirrors dispatch and combine backwards).
 * The gate weights are held fixed (the router's own gradient is not computed). With a = perm[r],
 * t = a / k and the forward's G, U, H = silu(G) * U of routed row r:
 *   dO[r] = w[a] dY[t];  dH = dO W_down^T;  dG = dH * U * silu'(G);  dU = dH * silu(G)
 *   dA = dG W_gate^T + dU W_up^T;   dX[t] = sum over j = 0 .. k-1 ascending of dA[inv[t*k+j]]
 *   dW_gate[e] = A_e^T dG_e;  dW_up[e] = A_e^T dU_e;  dW_down[e] = H_e^T dO_e
 * where A_e, dG_e, ... are expert e's routed rows. MOE_MXFP8 quantises every operand of these
 * GEMMs per 32 along that GEMM's reduction axis: dO, W_down along h; dG, dU, W_gate, W_up along
 * m; A, dG, dU, H, dO along the expert's rows (blocks from its first row, zero-padded). dO, dG,
 * dU and H are quantised from their float32 values (G and U are kept in float32 by the forward),
 * the A rows from the bf16 input. MOE_BF16 rounds dO, dG, dU and H to bf16 instead. Accumulation
 * is float32 everywhere, with no atomics and a fixed order.
 *
 * moe_prepare_bwd_weights: the backward's weight layout (offline), from the same bf16 weights as
 *   moe_prepare_weights: W_down rows [e][m][h] (K = h) and [W_gate | W_up] rows [e][h][2m]
 *   interleaved per 32 (K = 2m), MX-quantised along K for MOE_MXFP8 (codes first, then the
 *   scales chunk-major as in moe_prepare_weights: [e][K/256][rows][8]).
 * moe_backward: x [T][h] bf16 (the forward's input), dy [T][h] bf16, saved from moe_forward with
 *   the same shape and dtype, prepared_bwd from moe_prepare_bwd_weights. Outputs dx [T][h] bf16,
 *   dw_gate and dw_up [E_loc][h][m], dw_down [E_loc][m][h], float32 when dw_fp32 = 1, bf16 when 0
 *   (every element is written; an expert with no rows gets zeros).
 * Shapes: h % 256 == 0 and m % 256 == 0, else MOE_EUNSUPPORTED. ws: moe_backward_workspace_bytes().
 * ------------------------------------------------------------------------------------------- */
size_t moe_prepared_bwd_weight_bytes(const moe_shape* s, moe_dtype dt);
moe_status moe_prepare_bwd_weights(const moe_shape* s, moe_dtype dt, const uint16_t* w_gate,
                                   const uint16_t* w_up, const uint16_t* w_down,
                                   void* prepared_bwd, void* stream);
size_t moe_backward_workspace_bytes(const moe_shape* s, moe_dtype dt);
moe_status moe_backward(const moe_shape* s, moe_dtype dt, const uint16_t* x, const uint16_t* dy,
                        const void* saved, const void* prepared_bwd, uint16_t* dx, void* dw_gate,
                        void* dw_up, void* dw_down, int dw_fp32, void* ws, void* stream);

/* ---------------------------------------------------------------------------------------------
 * moe_backward_layer: the whole layer's backward (the page's Key claims measure the backward of
 * the whole isolated layer): the expert path as moe_backward, plus the gradients through the gate
 * weights, which moe_backward holds fixed. From the forward's expert outputs O (kept in `saved`):
 *   dgate[a] = <dY[t], O[inv[a]]>, t = a / k (0 for a dropped assignment)       [T*k] float out
 * Router use (w_router != NULL, the [E][h] bf16 matrix of the forward; E_loc == E): the gate
 * weights are the softmax of the k selected logits and the selection carries no gradient, so
 *   dl[t, j] = w[t, j] (dgate[t, j] - sum_i w[t, i] dgate[t, i]),
 *   dw_router[e] = sum over expert e's assignments of dl * x[t]   [E][h] float out (required),
 *   dbias[e] = sum over expert e's assignments of dl               [E] float out or NULL,
 * and dx also receives sum_j dl[t, j] w_router[e_j] (added before its one rounding, after the
 * expert path's rows, j ascending). Expert-share use (w_router == NULL): dw_router and dbias must
 * be NULL; dgate is what the owner of the router needs. Every sum has a fixed order (the router
 * matrix gradient over each expert's rows in schedule order, in chunks of 64 rows added in order).
 * ws: moe_backward_workspace_bytes() (for E == E_loc it holds the router's scratch too).
 * ------------------------------------------------------------------------------------------- */
moe_status moe_backward_layer(const moe_shape* s, moe_dtype dt, const uint16_t* x,
                              const uint16_t* w_router, const uint16_t* dy, const void* saved,
                              const void* prepared_bwd, uint16_t* dx, void* dw_gate, void* dw_up,
                              void* dw_down, int dw_fp32, float* dgate, float* dw_router,
                              float* dbias, void* ws, void* stream);

/* Profiling variant of moe_backward, events recorded at its stage boundaries:
 *   ev[0] tables ev[1] un-combine ev[2] dH + SwiGLU backward ev[3] dA ev[4] un-permute ev[5]
 *   transposes ev[6] dW_gate | dW_up ev[7] dW_down ev[8] */
#define MOE_BWD_PROFILE_EVENTS 9
moe_status moe_backward_profiled(const moe_shape* s, moe_dtype dt, const uint16_t* x,
                                 const uint16_t* dy, const void* saved, const void* prepared_bwd,
                                 uint16_t* dx, void* dw_gate, void* dw_up, void* dw_down,
                                 int dw_fp32, void* ws, void* const* events /* host */,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
