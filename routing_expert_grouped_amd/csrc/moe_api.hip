// C-ABI front end: argument checks, workspace layout and the launch sequence of each entry point.
// Nothing here allocates or synchronises; every call only enqueues kernels on the caller's stream.
#include <algorithm>
#include <mutex>

#include "moe_internal.h"

using namespace moe;

namespace {

constexpr int kMaxK = 16;
constexpr int kMaxExperts = 1024;
constexpr uintptr_t kPtrAlign = 16;

bool ok_ptr(const void* p) { return p != nullptr && ((uintptr_t)p % kPtrAlign) == 0; }
bool ok_opt(const void* p) { return p == nullptr || ((uintptr_t)p % kPtrAlign) == 0; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// Shape rules of the expert path. EINVAL: inconsistent; EUNSUPPORTED: valid but not tiled.
moe_status check_expert_shape(const moe_shape* s, moe_dtype dt) {
  if (!s) return MOE_EINVAL;
  if (s->T < 1 || s->h < 1 || s->m < 1 || s->k < 1 || s->E_loc < 1 || s->m_shared < 0)
    return MOE_EINVAL;
  if (dt != MOE_BF16 && dt != MOE_MXFP8) return MOE_EINVAL;
  if (dt == MOE_MXFP8 && (s->h % kMxBlock || s->m % kMxBlock)) return MOE_EINVAL;
  if (s->k > kMaxK || s->E_loc > kMaxExperts) return MOE_EUNSUPPORTED;
  if ((long long)s->T * s->k > (1ll << 30)) return MOE_EUNSUPPORTED;
  if (s->h % 128) return MOE_EUNSUPPORTED;
  if (s->m % 64) return MOE_EUNSUPPORTED;
  if (dt == MOE_MXFP8 && (s->h % 256 || s->m % 256)) return MOE_EUNSUPPORTED;
  if (s->m_shared && s->m_shared % 64) return MOE_EUNSUPPORTED;
  // the grouped GEMMs address rows with 32-bit byte offsets
  const size_t el = dt == MOE_MXFP8 ? 1 : 2;
  if ((size_t)s->T * s->k * std::max((size_t)s->h, 2 * (size_t)s->m) * el >= (1ull << 32))
    return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// Shapes the backward (and a forward that saves for it) covers.
moe_status check_backward_shape(const moe_shape* s, moe_dtype dt) {
  const moe_status st = check_expert_shape(s, dt);
  if (st != MOE_OK) return st;
  if (s->h % 256 || s->m % 256) return MOE_EUNSUPPORTED;
  const size_t el = dt == MOE_MXFP8 ? 1 : 2;
  const size_t kg = (size_t)wgrad_k_align(dt == MOE_MXFP8);
  const size_t kmax = ((size_t)s->T * s->k + (size_t)s->E_loc * (kg - 1)) / kg * kg;
  if (kmax >= (1ull << 31)) return MOE_EUNSUPPORTED;
  if (std::max((size_t)s->h, 2 * (size_t)s->m) * kmax * el >= (1ull << 32)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// Saved activations of a training forward (moe_saved_bytes).
struct SavedLayout {
  size_t offsets, perm, inv, w, assign, gu, o, total;
};

SavedLayout saved_layout(const moe_shape* s) {
  SavedLayout L{};
  const size_t R = (size_t)s->T * s->k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.offsets = take((size_t)(s->E_loc + 1) * 4);
  L.perm = take(R * 4);
  L.inv = take(R * 4);
  L.w = take(R * 4);
  L.assign = take(R * 4);              // each assignment's local expert
  L.gu = take(R * 2 * s->m * 4);       // float32
  L.o = take(R * (size_t)s->h * 2);    // the expert outputs (GEMM-2 writes them here), bf16
  L.total = off;
  return L;
}

// Workspace of the backward (moe_backward_workspace_bytes).
struct BackwardLayout {
  size_t tiles, koff, dO, dO_s, dgu, dgu_s, dgu_f32, dA, At, At_s, dOt, dOt_s, Ht, Ht_s, dGUt,
      dGUt_s, total;
  int kmax;
  // the router's gradients (shapes with E == E_loc): selected-logit gradients, the chunk tile
  // table and the partial sums of the router-matrix gradient
  size_t dl, rtiles, rpartial, rpartial_db;
  int rmax_tiles;
};

BackwardLayout backward_layout(const moe_shape* s, moe_dtype dt) {
  BackwardLayout L{};
  const bool mx = dt == MOE_MXFP8;
  const size_t el = mx ? 1 : 2;
  const int R = s->T * s->k, h = s->h, m = s->m;
  const int kg = wgrad_k_align(mx);
  L.kmax = (int)(((size_t)R + (size_t)s->E_loc * (kg - 1)) / kg * kg);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.tiles = take(gemm_tiles_bytes(R, s->E_loc));
  L.koff = take((size_t)(s->E_loc + 1) * 4);
  L.dO = take((size_t)R * h * el);
  L.dO_s = mx ? take((size_t)R * (h / kMxBlock)) : 0;
  L.dgu = take((size_t)R * 2 * m * el);
  L.dgu_s = mx ? take((size_t)R * (2 * m / kMxBlock)) : 0;
  L.dgu_f32 = take((size_t)R * 2 * m * 4);
  L.dA = take((size_t)R * h * 2);
  const size_t km = (size_t)L.kmax;
  L.At = take(h * km * el);
  L.At_s = mx ? take(h * km / kMxBlock) : 0;
  L.dOt = take(h * km * el);
  L.dOt_s = mx ? take(h * km / kMxBlock) : 0;
  L.Ht = take(m * km * el);
  L.Ht_s = mx ? take(m * km / kMxBlock) : 0;
  L.dGUt = take(2 * m * km * el);
  L.dGUt_s = mx ? take(2 * m * km / kMxBlock) : 0;
  if (s->E == s->E_loc) {
    L.rmax_tiles = (int)router_wgrad_tiles(R, s->E_loc);
    L.dl = take((size_t)R * 4);
    L.rtiles = take(align_up(sizeof(int)) + (size_t)L.rmax_tiles * sizeof(int2));
    L.rpartial = take((size_t)L.rmax_tiles * h * 4);
    L.rpartial_db = take((size_t)L.rmax_tiles * 4);
  }
  L.total = off;
  return L;
}

moe_status check_router_shape(const moe_shape* s) {
  if (!s) return MOE_EINVAL;
  if (s->T < 1 || s->h < 1 || s->k < 1 || s->E < s->k || s->E_loc != s->E) return MOE_EINVAL;
  if (s->h % 8) return MOE_EUNSUPPORTED;
  if (s->E > kMaxExperts || s->k > kMaxK) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

struct ForwardLayout {
  size_t logits, idx, w, counts, offsets, perm, inv, sched, rows, row_scales, ffn, out_rows;
  size_t xf;  // the router's float32 copies of x and W_r: inside `rows` (free until the gather)
              // if they fit
  size_t shared_off, shared_ffn, shared_out, total;
  bool router;
};

ForwardLayout forward_layout(const moe_shape* s, moe_dtype dt, bool router) {
  ForwardLayout L{};
  const bool mx = dt == MOE_MXFP8;
  const size_t R = (size_t)s->T * s->k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.router = router;
  L.logits = router ? take((size_t)s->T * s->E * 4) : 0;
  L.idx = router ? take(R * 4) : 0;
  L.w = router ? take(R * 4) : 0;
  L.counts = take((size_t)s->E_loc * 4);
  L.offsets = take((size_t)(s->E_loc + 1) * 4);
  L.perm = take(R * 4);
  L.inv = take(R * 4);
  L.sched = take(sched_workspace_bytes((int)R, s->E_loc));
  L.rows = take(R * s->h * (mx ? 1 : 2));
  L.row_scales = mx ? take(R * (s->h / kMxBlock)) : 0;
  L.ffn = take(ffn_workspace_bytes((int)R, s->h, s->m, s->E_loc, mx));
  L.out_rows = take(R * s->h * 2);
  if (router) {
    const size_t need = router_xf_bytes(s->T, s->h, s->E);
    L.xf = need <= R * s->h * (mx ? 1 : 2) ? L.rows : take(need);
  }
  if (s->m_shared > 0) {
    L.shared_off = take(2 * 4);
    L.shared_ffn = take(ffn_workspace_bytes(s->T, s->h, s->m_shared, 1, false));
    L.shared_out = take((size_t)s->T * s->h * 2);
  }
  L.total = off;
  return L;
}

__global__ void shared_offsets_kernel(int32_t* off, int T) {
  if (threadIdx.x == 0) {
    off[0] = 0;
    off[1] = T;
  }
}

}  // namespace

extern "C" {

const char* moe_status_string(int code) {
  switch (code) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: shape not covered by the kernels";
    case MOE_EHIP: return "MOE_EHIP: HIP launch error";
    case MOE_ENOSCRATCH:
      return "MOE_ENOSCRATCH: the shape needs more scratch than the static buffer holds";
    case MOE_ETIMEOUT: return "MOE_ETIMEOUT: a device-side wait ran out of time";
  }
  return "unknown moe_status";
}

int moe_abi_version(void) { return MOE_ABI_VERSION; }

moe_status moe_check_e4m3(int64_t* mismatches, void* stream) {
  if (!ok_ptr(mismatches)) return MOE_EINVAL;
  return hip_status(launch_check_e4m3(mismatches, as_stream(stream)));
}

size_t moe_prepared_weight_bytes(const moe_shape* s, moe_dtype dt) {
  if (check_expert_shape(s, dt) != MOE_OK) return 0;
  return prepared_bytes(s->E_loc, s->h, s->m, dt == MOE_MXFP8);
}

moe_status moe_prepare_weights(const moe_shape* s, moe_dtype dt, const uint16_t* w_gate,
                               const uint16_t* w_up, const uint16_t* w_down, void* prepared,
                               void* stream) {
  const moe_status st = check_expert_shape(s, dt);
  if (st != MOE_OK) return st;
  if (!ok_ptr(w_gate) || !ok_ptr(w_up) || !ok_ptr(w_down) || !ok_ptr(prepared)) return MOE_EINVAL;
  return hip_status(launch_prepare_weights(w_gate, w_up, w_down, prepared, s->E_loc, s->h, s->m,
                                           dt == MOE_MXFP8, as_stream(stream)));
}

size_t moe_route_workspace_bytes(const moe_shape* s) {
  if (check_router_shape(s) != MOE_OK) return 0;
  return router_xf_bytes(s->T, s->h, s->E);
}

moe_status moe_route(const moe_shape* s, const uint16_t* x, const uint16_t* w_router,
                     const float* bias, float* logits, int32_t* topk_idx, float* topk_w, void* ws,
                     void* stream) {
  const moe_status st = check_router_shape(s);
  if (st != MOE_OK) return st;
  if (!ok_ptr(x) || !ok_ptr(w_router) || !ok_opt(bias) || !ok_ptr(logits) || !ok_ptr(topk_idx) ||
      !ok_ptr(topk_w) || !ok_ptr(ws))
    return MOE_EINVAL;
  const hipStream_t hs = as_stream(stream);
  hipError_t e = launch_router_logits_xf(x, w_router, bias, logits, s->T, s->h, s->E,
                                         reinterpret_cast<float*>(ws), hs);
  if (e == hipSuccess) e = launch_topk_softmax(logits, topk_idx, topk_w, s->T, s->E, s->k, hs);
  return hip_status(e);
}

size_t moe_permute_workspace_bytes(const moe_shape* s) {
  if (!s || s->T < 1 || s->k < 1 || s->E_loc < 1 || s->k > kMaxK || s->E_loc > kMaxExperts ||
      (long long)s->T * s->k > (1ll << 30))
    return 0;
  return sched_workspace_bytes(s->T * s->k, s->E_loc);
}

moe_status moe_permute(const moe_shape* s, moe_dtype dt, const int32_t* assign,
                       const uint16_t* x, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* inv, void* rows, uint8_t* row_scales, void* ws, void* stream) {
  const moe_status st = check_expert_shape(s, dt);
  if (st != MOE_OK) return st;
  if (!ok_ptr(assign) || !ok_ptr(x) || !ok_ptr(counts) || !ok_ptr(offsets) || !ok_ptr(perm) ||
      !ok_ptr(inv) || !ok_ptr(rows) || !ok_ptr(ws))
    return MOE_EINVAL;
  if (dt == MOE_MXFP8 && !ok_ptr(row_scales)) return MOE_EINVAL;
  const hipStream_t hs = as_stream(stream);
  const int R = s->T * s->k;
  hipError_t e = launch_schedule(assign, R, s->E_loc, counts, offsets, perm, inv, ws, hs);
  if (e != hipSuccess) return MOE_EHIP;
  if (dt == MOE_MXFP8)
    e = launch_gather_mxfp8(x, inv, reinterpret_cast<uint8_t*>(rows), row_scales, s->T, s->h,
                            s->k, hs);
  else
    e = launch_gather_bf16(x, inv, reinterpret_cast<uint16_t*>(rows), s->T, s->h, s->k, hs);
  return hip_status(e);
}

}  // extern "C"

namespace {

// The schedule's scratch for moe_permute_static: one static array per GPU (each device holds its
// own copy of a __device__ variable). Host code never passes the array's name to a kernel (on the
// host it only stands in for the symbol): its device address is obtained with hipGetSymbolAddress
// once per device, with that device current, and kept here.
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[MOE_PERMUTE_STATIC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's array, or nullptr on a HIP error.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

moe_status moe_permute_static(const moe_shape* s, moe_dtype dt, const int32_t* assign,
                              const uint16_t* x, int32_t* counts, int32_t* offsets,
                              int32_t* perm, int32_t* inv, void* rows, uint8_t* row_scales,
                              void* stream) {
  const moe_status st = check_expert_shape(s, dt);
  if (st != MOE_OK) return st;
  if (!ok_ptr(assign) || !ok_ptr(x) || !ok_ptr(counts) || !ok_ptr(offsets) || !ok_ptr(perm) ||
      !ok_ptr(inv) || !ok_ptr(rows))
    return MOE_EINVAL;
  if (dt == MOE_MXFP8 && !ok_ptr(row_scales)) return MOE_EINVAL;
  if (sched_workspace_bytes(s->T * s->k, s->E_loc) > MOE_PERMUTE_STATIC_SCRATCH_BYTES)
    return MOE_ENOSCRATCH;
  void* ws = scratch_on_current_device();
  if (!ws) return MOE_EHIP;
  return moe_permute(s, dt, assign, x, counts, offsets, perm, inv, rows, row_scales, ws, stream);
}

size_t moe_expert_ffn_workspace_bytes(const moe_shape* s, moe_dtype dt) {
  if (check_expert_shape(s, dt) != MOE_OK) return 0;
  return ffn_workspace_bytes(s->T * s->k, s->h, s->m, s->E_loc, dt == MOE_MXFP8);
}

moe_status moe_expert_ffn(const moe_shape* s, moe_dtype dt, const void* rows,
                          const uint8_t* row_scales, const int32_t* offsets, const void* prepared,
                          uint16_t* out_rows, void* ws, void* stream) {
  const moe_status st = check_expert_shape(s, dt);
  if (st != MOE_OK) return st;
  if (!ok_ptr(rows) || !ok_ptr(offsets) || !ok_ptr(prepared) || !ok_ptr(out_rows) || !ok_ptr(ws))
    return MOE_EINVAL;
  if (dt == MOE_MXFP8 && !ok_ptr(row_scales)) return MOE_EINVAL;
  return hip_status(launch_expert_ffn(rows, row_scales, offsets, prepared, out_rows, ws,
                                      s->T * s->k, s->h, s->m, s->E_loc, dt == MOE_MXFP8,
                                      as_stream(stream)));
}

moe_status moe_combine(const moe_shape* s, const uint16_t* out_rows, const int32_t* inv,
                       const float* topk_w, const uint16_t* shared_out, uint16_t* y,
                       void* stream) {
  if (!s || s->T < 1 || s->h < 1 || s->k < 1) return MOE_EINVAL;
  if (s->k > kMaxK) return MOE_EUNSUPPORTED;
  if (s->h % 8) return MOE_EUNSUPPORTED;
  if (!ok_ptr(out_rows) || !ok_ptr(inv) || !ok_ptr(topk_w) || !ok_opt(shared_out) || !ok_ptr(y))
    return MOE_EINVAL;
  return hip_status(launch_combine(out_rows, inv, topk_w, shared_out, y, s->T, s->h, s->k,
                                   as_stream(stream)));
}

size_t moe_forward_workspace_bytes(const moe_shape* s, moe_dtype dt) {
  if (check_expert_shape(s, dt) != MOE_OK) return 0;
  // sized for the router use (a superset of the expert-share use) when E == E_loc
  const bool router = s->E == s->E_loc && s->E >= s->k;
  return forward_layout(s, dt, router).total;
}

moe_status moe_forward_views(const moe_shape* s, moe_dtype dt, void* ws,
                             moe_forward_views_t* v) {
  const moe_status st = check_expert_shape(s, dt);
  if (st != MOE_OK) return st;
  if (!ws || !v) return MOE_EINVAL;
  const bool router = s->E == s->E_loc && s->E >= s->k;
  const ForwardLayout L = forward_layout(s, dt, router);
  uint8_t* b = reinterpret_cast<uint8_t*>(ws);
  v->logits = router ? reinterpret_cast<float*>(b + L.logits) : nullptr;
  v->topk_idx = router ? reinterpret_cast<int32_t*>(b + L.idx) : nullptr;
  v->topk_w = router ? reinterpret_cast<float*>(b + L.w) : nullptr;
  v->counts = reinterpret_cast<int32_t*>(b + L.counts);
  v->offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  v->perm = reinterpret_cast<int32_t*>(b + L.perm);
  v->inv = reinterpret_cast<int32_t*>(b + L.inv);
  v->rows = b + L.rows;
  v->row_scales = dt == MOE_MXFP8 ? b + L.row_scales : nullptr;
  v->out_rows = reinterpret_cast<uint16_t*>(b + L.out_rows);
  v->shared_out = s->m_shared > 0 ? reinterpret_cast<uint16_t*>(b + L.shared_out) : nullptr;
  return MOE_OK;
}

}  // extern "C"

namespace {

moe_status forward_impl(const moe_shape* s, moe_dtype dt, const uint16_t* x,
                        const uint16_t* w_router, const float* bias, const int32_t* assign,
                        const float* assign_w, const void* prepared, const void* shared_prepared,
                        uint16_t* y, void* saved, void* ws, const hipEvent_t* ev, void* stream) {
  moe_status st = check_expert_shape(s, dt);
  if (st != MOE_OK) return st;
  if (saved) {
    if (!ok_ptr(saved)) return MOE_EINVAL;
    st = check_backward_shape(s, dt);
    if (st != MOE_OK) return st;
  }
  const bool router = w_router != nullptr;
  if (router) {
    st = check_router_shape(s);
    if (st != MOE_OK) return st;
    if (assign || assign_w || !ok_opt(bias)) return MOE_EINVAL;
  } else {
    if (!ok_ptr(assign) || !ok_ptr(assign_w) || bias) return MOE_EINVAL;
  }
  if (!ok_ptr(x) || !ok_ptr(prepared) || !ok_ptr(y) || !ok_ptr(ws)) return MOE_EINVAL;
  if ((s->m_shared > 0) != (shared_prepared != nullptr)) return MOE_EINVAL;
  if (shared_prepared && !ok_ptr(shared_prepared)) return MOE_EINVAL;

  const bool mx = dt == MOE_MXFP8;
  const bool router_layout = s->E == s->E_loc && s->E >= s->k;
  const ForwardLayout L = forward_layout(s, dt, router_layout);
  uint8_t* b = reinterpret_cast<uint8_t*>(ws);
  const hipStream_t hs = as_stream(stream);
  const int T = s->T, h = s->h, k = s->k, R = T * k;

  const int32_t* a_idx = assign;
  const float* a_w = assign_w;
  hipError_t e = hipSuccess;
  auto mark = [&](int i) {
    if (ev && e == hipSuccess) e = hipEventRecord(ev[i], hs);
  };
  mark(0);
  if (router) {
    float* logits = reinterpret_cast<float*>(b + L.logits);
    int32_t* idx = reinterpret_cast<int32_t*>(b + L.idx);
    float* w = reinterpret_cast<float*>(b + L.w);
    e = launch_router_logits_xf(x, w_router, bias, logits, T, h, s->E,
                                reinterpret_cast<float*>(b + L.xf), hs);
    mark(1);
    if (e == hipSuccess) e = launch_topk_softmax(logits, idx, w, T, s->E, k, hs);
    a_idx = idx;
    a_w = w;
  } else {
    mark(1);
  }
  mark(2);
  int32_t* counts = reinterpret_cast<int32_t*>(b + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(b + L.perm);
  int32_t* inv = reinterpret_cast<int32_t*>(b + L.inv);
  if (e == hipSuccess)
    e = launch_schedule(a_idx, R, s->E_loc, counts, offsets, perm, inv, b + L.sched, hs);
  mark(3);
  // On the large-tile GEMMs the gather is done by GEMM-1's own loads (routed row r reads token
  // perm[r] / k): BF16 reads x itself; MXFP8 quantises each token once into the row buffer
  // (codes [T][h], chunk-major scales) and GEMM-1 reads those. Otherwise the routed rows are
  // materialised by the gather kernels, as moe_permute does.
  const bool fused_gather = ffn_big(h, s->m);
  if (e == hipSuccess) {
    if (fused_gather) {
      if (mx) e = launch_quantize_tokens_mxfp8(x, b + L.rows, b + L.row_scales, T, h, hs);
    } else if (mx) {
      e = launch_gather_mxfp8(x, inv, b + L.rows, b + L.row_scales, T, h, k, hs);
    } else {
      e = launch_gather_bf16(x, inv, reinterpret_cast<uint16_t*>(b + L.rows), T, h, k, hs);
    }
  }
  mark(4);
  uint8_t* sv = reinterpret_cast<uint8_t*>(saved);
  const SavedLayout SL = saved_layout(s);
  // a training forward keeps the expert outputs for the gate-weight gradients: GEMM-2 writes them
  // straight into the saved buffer
  uint16_t* out_rows = reinterpret_cast<uint16_t*>(sv ? sv + SL.o : b + L.out_rows);
  float* gu_save = sv ? reinterpret_cast<float*>(sv + SL.gu) : nullptr;
  if (e == hipSuccess) {
    if (fused_gather)
      e = launch_expert_ffn(mx ? static_cast<const void*>(b + L.rows) : x,
                            mx ? b + L.row_scales : nullptr, offsets, prepared, out_rows, b + L.ffn,
                            R, h, s->m, s->E_loc, mx, hs, ev ? ev + 5 : nullptr, gu_save, perm, k,
                            T, /*scales_cm=*/true);
    else
      e = launch_expert_ffn(b + L.rows, mx ? b + L.row_scales : nullptr, offsets, prepared,
                            out_rows, b + L.ffn, R, h, s->m, s->E_loc, mx, hs,
                            ev ? ev + 5 : nullptr, gu_save);
  }
  uint16_t* shared_out = nullptr;
  if (e == hipSuccess && s->m_shared > 0) {
    int32_t* soff = reinterpret_cast<int32_t*>(b + L.shared_off);
    shared_out = reinterpret_cast<uint16_t*>(b + L.shared_out);
    hipLaunchKernelGGL(shared_offsets_kernel, dim3(1), dim3(64), 0, hs, soff, T);
    e = hipGetLastError();
    if (e == hipSuccess)
      e = launch_expert_ffn(x, nullptr, soff, shared_prepared, shared_out, b + L.shared_ffn, T, h,
                            s->m_shared, 1, false, hs);
  }
  mark(8);
  if (e == hipSuccess) e = launch_combine(out_rows, inv, a_w, shared_out, y, T, h, k, hs);
  mark(9);
  if (sv && e == hipSuccess) {  // what the backward needs besides G and U (a few bytes per row)
    e = hipMemcpyAsync(sv + SL.offsets, offsets, (size_t)(s->E_loc + 1) * 4,
                       hipMemcpyDeviceToDevice, hs);
    if (e == hipSuccess)
      e = hipMemcpyAsync(sv + SL.perm, perm, (size_t)R * 4, hipMemcpyDeviceToDevice, hs);
    if (e == hipSuccess)
      e = hipMemcpyAsync(sv + SL.inv, inv, (size_t)R * 4, hipMemcpyDeviceToDevice, hs);
    if (e == hipSuccess)
      e = hipMemcpyAsync(sv + SL.w, a_w, (size_t)R * 4, hipMemcpyDeviceToDevice, hs);
    if (e == hipSuccess)
      e = hipMemcpyAsync(sv + SL.assign, a_idx, (size_t)R * 4, hipMemcpyDeviceToDevice, hs);
  }
  return hip_status(e);
}

// dgate == nullptr: the expert path only (gate weights held fixed). Otherwise also dgate and, with
// w_router, the router's gradients (dw_router, dbias) and its part of dx.
moe_status backward_impl(const moe_shape* s, moe_dtype dt, const uint16_t* x, const uint16_t* dy,
                         const void* saved, const void* prepared_bwd, uint16_t* dx, void* dw_gate,
                         void* dw_up, void* dw_down, int dw_fp32, void* ws, const hipEvent_t* ev,
                         void* stream, const uint16_t* w_router = nullptr, float* dgate = nullptr,
                         float* dw_router = nullptr, float* dbias = nullptr) {
  const moe_status st = check_backward_shape(s, dt);
  if (st != MOE_OK) return st;
  if (!ok_ptr(x) || !ok_ptr(dy) || !ok_ptr(saved) || !ok_ptr(prepared_bwd) || !ok_ptr(dx) ||
      !ok_ptr(dw_gate) || !ok_ptr(dw_up) || !ok_ptr(dw_down) || !ok_ptr(ws))
    return MOE_EINVAL;
  if (dw_fp32 != 0 && dw_fp32 != 1) return MOE_EINVAL;
  if (w_router) {
    const moe_status rs = check_router_shape(s);
    if (rs != MOE_OK) return rs;
    if (!ok_ptr(w_router) || !ok_ptr(dgate) || !ok_ptr(dw_router) || !ok_opt(dbias))
      return MOE_EINVAL;
  } else if (dw_router || dbias) {
    return MOE_EINVAL;
  }
  const bool mx = dt == MOE_MXFP8;
  const int T = s->T, h = s->h, m = s->m, k = s->k, E_loc = s->E_loc, R = T * k;
  const hipStream_t hs = as_stream(stream);
  const SavedLayout SL = saved_layout(s);
  const BackwardLayout L = backward_layout(s, dt);
  const uint8_t* sv = reinterpret_cast<const uint8_t*>(saved);
  const int32_t* offsets = reinterpret_cast<const int32_t*>(sv + SL.offsets);
  const int32_t* perm = reinterpret_cast<const int32_t*>(sv + SL.perm);
  const int32_t* inv = reinterpret_cast<const int32_t*>(sv + SL.inv);
  const float* w = reinterpret_cast<const float*>(sv + SL.w);
  const float* gu = reinterpret_cast<const float*>(sv + SL.gu);
  const int32_t* assign = reinterpret_cast<const int32_t*>(sv + SL.assign);
  const uint16_t* O = reinterpret_cast<const uint16_t*>(sv + SL.o);
  const PreparedBwd P = prepared_bwd_views(prepared_bwd, E_loc, h, m, mx);
  uint8_t* b = reinterpret_cast<uint8_t*>(ws);
  int32_t* koff = reinterpret_cast<int32_t*>(b + L.koff);
  uint16_t* dA = reinterpret_cast<uint16_t*>(b + L.dA);
  float* dgu_f32 = reinterpret_cast<float*>(b + L.dgu_f32);  // dG | dU for the transposes

  hipError_t e = hipSuccess;
  auto mark = [&](int i) {
    if (ev && e == hipSuccess) e = hipEventRecord(ev[i], hs);
  };
  float* dl = w_router ? reinterpret_cast<float*>(b + L.dl) : nullptr;
  mark(0);
  // the gate weights' gradients (and the selected logits' for a router layer) first: the
  // un-permute below adds the router's part of dx from them
  if (dgate && e == hipSuccess) e = launch_gate_grads(dy, O, inv, w, dgate, dl, T, h, k, hs);
  if (e == hipSuccess) e = launch_kpad_table(offsets, E_loc, wgrad_k_align(mx), koff, hs);
  if (e == hipSuccess) e = launch_gemm_tiles(offsets, b + L.tiles, R, E_loc, mx, hs);
  mark(1);
  if (e == hipSuccess)
    e = launch_uncombine(dy, perm, w, offsets, E_loc, b + L.dO, mx ? b + L.dO_s : nullptr, R, h,
                         k, mx, hs);
  mark(2);
  if (e == hipSuccess)
    e = launch_bwd_dgrad(b + L.dO, mx ? b + L.dO_s : nullptr, offsets, P.w2b, P.w2b_s, P.w1b,
                         P.w1b_s, gu, b + L.dgu, mx ? b + L.dgu_s : nullptr,
                         dgu_f32, dA,
                         b + L.tiles, R, h, m, E_loc, mx, hs, ev ? ev[3] : nullptr);
  mark(4);
  if (e == hipSuccess)
    e = launch_combine(dA, inv, nullptr, nullptr, dx, T, h, k, hs, w_router, assign, dl, s->E);
  mark(5);
  const int km = L.kmax;
  if (e == hipSuccess)
    e = launch_bwd_transpose(kTrX, x, perm, w, offsets, koff, E_loc, h, k, km, b + L.At,
                             mx ? b + L.At_s : nullptr, mx, hs);
  if (e == hipSuccess)
    e = launch_bwd_transpose(kTrDO, dy, perm, w, offsets, koff, E_loc, h, k, km, b + L.dOt,
                             mx ? b + L.dOt_s : nullptr, mx, hs);
  if (e == hipSuccess)
    e = launch_bwd_transpose(kTrH, gu, perm, w, offsets, koff, E_loc, m, k, km, b + L.Ht,
                             mx ? b + L.Ht_s : nullptr, mx, hs);
  if (e == hipSuccess)
    e = launch_bwd_transpose(kTrRows, dgu_f32, perm, w, offsets, koff, E_loc, 2 * m, k, km,
                             b + L.dGUt, mx ? b + L.dGUt_s : nullptr, mx, hs);
  mark(6);
  if (e == hipSuccess)
    e = launch_bwd_wgrad(b + L.At, mx ? b + L.At_s : nullptr, b + L.dGUt,
                         mx ? b + L.dGUt_s : nullptr, b + L.Ht, mx ? b + L.Ht_s : nullptr,
                         b + L.dOt, mx ? b + L.dOt_s : nullptr, koff, dw_gate, dw_up, dw_down,
                         dw_fp32 == 1, h, m, E_loc, mx, hs, ev ? ev[7] : nullptr);
  if (w_router && e == hipSuccess) {  // the router matrix's (and bias's) gradient
    uint8_t* rt = b + L.rtiles;
    int* rcount = reinterpret_cast<int*>(rt);
    int2* rtiles = reinterpret_cast<int2*>(rt + align_up(sizeof(int)));
    e = launch_tile_table(offsets, E_loc, kRouterChunk, L.rmax_tiles, rtiles, rcount, hs);
    if (e == hipSuccess)
      e = launch_router_wgrad(rtiles, rcount, L.rmax_tiles, offsets, perm, dl, x, h, k, s->E,
                              reinterpret_cast<float*>(b + L.rpartial),
                              reinterpret_cast<float*>(b + L.rpartial_db), dw_router, dbias, hs);
  }
  mark(8);
  return hip_status(e);
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_shape* s, moe_dtype dt, const uint16_t* x,
                       const uint16_t* w_router, const float* bias, const int32_t* assign,
                       const float* assign_w, const void* prepared, const void* shared_prepared,
                       uint16_t* y, void* saved, void* ws, void* stream) {
  return forward_impl(s, dt, x, w_router, bias, assign, assign_w, prepared, shared_prepared, y,
                      saved, ws, nullptr, stream);
}

moe_status moe_forward_profiled(const moe_shape* s, moe_dtype dt, const uint16_t* x,
                                const uint16_t* w_router, const float* bias,
                                const int32_t* assign, const float* assign_w,
                                const void* prepared, const void* shared_prepared, uint16_t* y,
                                void* saved, void* ws, void* const* events, void* stream) {
  if (!events) return MOE_EINVAL;
  for (int i = 0; i < MOE_PROFILE_EVENTS; ++i)
    if (!events[i]) return MOE_EINVAL;
  return forward_impl(s, dt, x, w_router, bias, assign, assign_w, prepared, shared_prepared, y,
                      saved, ws, reinterpret_cast<const hipEvent_t*>(events), stream);
}

int32_t moe_forward_ring_tokens(const moe_shape* s, moe_dtype dt, size_t ring_bytes) {
  if (check_expert_shape(s, dt) != MOE_OK) return 0;
  // forward workspace bytes grow with the token count: the largest count that fits
  auto need = [&](int t) {
    moe_shape sub = *s;
    sub.T = t;
    return moe_forward_workspace_bytes(&sub, dt);
  };
  if (need(1) > ring_bytes) return 0;
  int lo = 1, hi = s->T;
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    if (need(mid) <= ring_bytes) lo = mid;
    else hi = mid - 1;
  }
  if (lo >= s->T) return s->T;  // one minibatch
  // every minibatch starts 16-byte aligned in assign / assign_w (k 4-byte entries per token):
  // a multiple of 4 / gcd(k, 4) tokens
  const int a = s->k % 4 == 0 ? 1 : (s->k % 2 == 0 ? 2 : 4);
  return lo / a * a;
}

moe_status moe_forward_ring(const moe_shape* s, moe_dtype dt, const uint16_t* x,
                            const uint16_t* w_router, const float* bias, const int32_t* assign,
                            const float* assign_w, const void* prepared,
                            const void* shared_prepared, uint16_t* y, void* ring,
                            size_t ring_bytes, int32_t* minibatch_tokens, void* stream) {
  const moe_status st = check_expert_shape(s, dt);
  if (st != MOE_OK) return st;
  if (!ok_ptr(ring) || !ok_ptr(x) || !ok_ptr(y)) return MOE_EINVAL;
  if (w_router ? (assign || assign_w) : (!ok_ptr(assign) || !ok_ptr(assign_w))) return MOE_EINVAL;
  const int tmb = moe_forward_ring_tokens(s, dt, ring_bytes);
  if (tmb < 1) return MOE_EINVAL;  // the ring cannot hold even one token's minibatch
  if (minibatch_tokens) *minibatch_tokens = tmb;
  const size_t h = (size_t)s->h, k = (size_t)s->k;
  for (int t0 = 0; t0 < s->T; t0 += tmb) {
    moe_shape sub = *s;
    sub.T = std::min(tmb, s->T - t0);
    const moe_status r = forward_impl(&sub, dt, x + t0 * h, w_router, bias,
                                      assign ? assign + t0 * k : nullptr,
                                      assign_w ? assign_w + t0 * k : nullptr, prepared,
                                      shared_prepared, y + t0 * h, nullptr, ring, nullptr, stream);
    if (r != MOE_OK) return r;
  }
  return MOE_OK;
}

}  // extern "C"

namespace {

struct PersistentLayout {
  ForwardLayout f;
  size_t xf, etile, sync, args, total;
  int bm;
};

// the forward workspace, plus its own float32 router matrix (the forward's may share the routed-row
// buffer, which the persistent kernel fills while the router still runs), the first tile of each
// expert and the synchronisation words
PersistentLayout persistent_layout(const moe_shape* s, moe_dtype dt, bool router) {
  PersistentLayout P{};
  P.f = forward_layout(s, dt, router);
  const int R = s->T * s->k;
  size_t off = P.f.total;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  P.xf = router ? take(router_xf_bytes(s->T, s->h, s->E)) : 0;
  P.bm = kPersistentRows;
  P.etile = take((size_t)(s->E_loc + 1) * 4);
  P.sync = take(persistent_sync_ints(R, s->E_loc, P.bm) * 4);
  P.args = take(persistent_args_bytes());
  P.total = off;
  return P;
}

moe_status check_persistent_shape(const moe_shape* s, moe_dtype dt) {
  const moe_status st = check_expert_shape(s, dt);
  if (st != MOE_OK) return st;
  if (s->m_shared > 0 || !ffn_big(s->h, s->m)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

struct DeviceFacts {
  int num_cu = 0;
  int clock_khz = 0;  // wall clock
};
std::mutex g_facts_mu;
DeviceFacts g_facts[kMaxDevices];

bool device_facts(DeviceFacts& out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lock(g_facts_mu);
  DeviceFacts& f = g_facts[dev];
  if (!f.num_cu) {
    int cu = 0, clk = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&clk, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
        cu < 1 || clk < 1)
      return false;
    f.num_cu = cu;
    f.clock_khz = clk;
  }
  out = f;
  return true;
}

}  // namespace

extern "C" {

size_t moe_forward_persistent_workspace_bytes(const moe_shape* s, moe_dtype dt) {
  if (check_persistent_shape(s, dt) != MOE_OK) return 0;
  const bool router = s->E == s->E_loc && s->E >= s->k;
  return persistent_layout(s, dt, router).total;
}

moe_status moe_forward_persistent(const moe_shape* s, moe_dtype dt, const uint16_t* x,
                                  const uint16_t* w_router, const float* bias,
                                  const int32_t* assign, const float* assign_w,
                                  const void* prepared, uint16_t* y, void* ws, int32_t* status,
                                  int32_t timeout_ms, void* stream) {
  moe_status st = check_persistent_shape(s, dt);
  if (st != MOE_OK) return st;
  const bool router = w_router != nullptr;
  if (router) {
    st = check_router_shape(s);
    if (st != MOE_OK) return st;
    if (assign || assign_w || !ok_opt(bias)) return MOE_EINVAL;
  } else {
    if (!ok_ptr(assign) || !ok_ptr(assign_w) || bias) return MOE_EINVAL;
  }
  if (!ok_ptr(x) || !ok_ptr(prepared) || !ok_ptr(y) || !ok_ptr(ws) || !ok_ptr(status) ||
      timeout_ms < 1)
    return MOE_EINVAL;
  DeviceFacts f;
  if (!device_facts(f)) return MOE_EHIP;
  const bool mx = dt == MOE_MXFP8;
  const bool router_layout = s->E == s->E_loc && s->E >= s->k;
  const PersistentLayout P = persistent_layout(s, dt, router_layout);
  const ForwardLayout& L = P.f;
  uint8_t* b = reinterpret_cast<uint8_t*>(ws);
  PersistentBuffers pb{};
  pb.x = x;
  pb.w_router = w_router;
  pb.bias = bias;
  pb.assign = assign;
  pb.assign_w = assign_w;
  pb.prepared = prepared;
  pb.y = y;
  pb.status = status;
  pb.wi = router ? reinterpret_cast<float*>(b + P.xf) : nullptr;
  pb.logits = router ? reinterpret_cast<float*>(b + L.logits) : nullptr;
  pb.idx = router ? reinterpret_cast<int32_t*>(b + L.idx) : nullptr;
  pb.tw = router ? reinterpret_cast<float*>(b + L.w) : nullptr;
  pb.cc = reinterpret_cast<int32_t*>(b + L.sched);
  pb.counts = reinterpret_cast<int32_t*>(b + L.counts);
  pb.offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  pb.perm = reinterpret_cast<int32_t*>(b + L.perm);
  pb.inv = reinterpret_cast<int32_t*>(b + L.inv);
  pb.qrows = mx ? b + L.rows : nullptr;
  pb.qscales = mx ? b + L.row_scales : nullptr;
  pb.ffn_ws = b + L.ffn;
  pb.out_rows = reinterpret_cast<uint16_t*>(b + L.out_rows);
  pb.etile = reinterpret_cast<int32_t*>(b + P.etile);
  pb.sync = reinterpret_cast<int*>(b + P.sync);
  pb.args = b + P.args;
  const long long timeout = (long long)f.clock_khz * timeout_ms;
  return hip_status(launch_forward_persistent(pb, s->T, s->h, s->m, s->E, s->E_loc, s->k, mx,
                                              f.num_cu, timeout, as_stream(stream)));
}

size_t moe_saved_bytes(const moe_shape* s, moe_dtype dt) {
  if (check_backward_shape(s, dt) != MOE_OK) return 0;
  return saved_layout(s).total;
}

size_t moe_prepared_bwd_weight_bytes(const moe_shape* s, moe_dtype dt) {
  if (check_backward_shape(s, dt) != MOE_OK) return 0;
  return prepared_bwd_bytes(s->E_loc, s->h, s->m, dt == MOE_MXFP8);
}

moe_status moe_prepare_bwd_weights(const moe_shape* s, moe_dtype dt, const uint16_t* w_gate,
                                   const uint16_t* w_up, const uint16_t* w_down,
                                   void* prepared_bwd, void* stream) {
  const moe_status st = check_backward_shape(s, dt);
  if (st != MOE_OK) return st;
  if (!ok_ptr(w_gate) || !ok_ptr(w_up) || !ok_ptr(w_down) || !ok_ptr(prepared_bwd))
    return MOE_EINVAL;
  return hip_status(launch_prepare_bwd_weights(w_gate, w_up, w_down, prepared_bwd, s->E_loc, s->h,
                                               s->m, dt == MOE_MXFP8, as_stream(stream)));
}

size_t moe_backward_workspace_bytes(const moe_shape* s, moe_dtype dt) {
  if (check_backward_shape(s, dt) != MOE_OK) return 0;
  return backward_layout(s, dt).total;
}

moe_status moe_backward(const moe_shape* s, moe_dtype dt, const uint16_t* x, const uint16_t* dy,
                        const void* saved, const void* prepared_bwd, uint16_t* dx, void* dw_gate,
                        void* dw_up, void* dw_down, int dw_fp32, void* ws, void* stream) {
  return backward_impl(s, dt, x, dy, saved, prepared_bwd, dx, dw_gate, dw_up, dw_down, dw_fp32, ws,
                       nullptr, stream);
}

moe_status moe_backward_layer(const moe_shape* s, moe_dtype dt, const uint16_t* x,
                              const uint16_t* w_router, const uint16_t* dy, const void* saved,
                              const void* prepared_bwd, uint16_t* dx, void* dw_gate, void* dw_up,
                              void* dw_down, int dw_fp32, float* dgate, float* dw_router,
                              float* dbias, void* ws, void* stream) {
  if (!ok_ptr(dgate)) return MOE_EINVAL;
  return backward_impl(s, dt, x, dy, saved, prepared_bwd, dx, dw_gate, dw_up, dw_down, dw_fp32, ws,
                       nullptr, stream, w_router, dgate, dw_router, dbias);
}

moe_status moe_backward_profiled(const moe_shape* s, moe_dtype dt, const uint16_t* x,
                                 const uint16_t* dy, const void* saved, const void* prepared_bwd,
                                 uint16_t* dx, void* dw_gate, void* dw_up, void* dw_down,
                                 int dw_fp32, void* ws, void* const* events, void* stream) {
  if (!events) return MOE_EINVAL;
  for (int i = 0; i < MOE_BWD_PROFILE_EVENTS; ++i)
    if (!events[i]) return MOE_EINVAL;
  return backward_impl(s, dt, x, dy, saved, prepared_bwd, dx, dw_gate, dw_up, dw_down, dw_fp32, ws,
                       reinterpret_cast<const hipEvent_t*>(events), stream);
}

}  // extern "C"
