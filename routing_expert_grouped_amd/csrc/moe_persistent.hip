// Persistent forward: the whole layer forward (router, top-k, schedule, token quantisation, tile
// table, both grouped GEMMs, combine) in one launch of one workgroup per CU, the one-GPU form of the
// Mixture-of-Kittens megakernel (TL;DR and flowchart: one persistent kernel whose groups of SMs
// hand work to each other through local counters instead of global barriers or kernel
// boundaries; the companion news digest, Merged summary, on the CPU-free schedule).
//
// Work. Every step is cut into items (a block of tokens, a chunk of assignments, a GEMM output
// tile, ...). Each XCD has its own work queue, an ordered list of items in step order: a
// workgroup on XCD x takes the next ticket of queue x with one atomic add and runs that item.
// The items of the round-robin steps are spread over the queues in turn; the GEMM tiles keep the
// grouped-GEMM kernels' band order, so XCD x runs the same tiles at the same time as there and
// they share its L2 the same way.
//
// Hand-off. An item that needs earlier work waits for a counter (thread 0 spins on a relaxed
// agent-scope load, then one agent-scope acquire), and a finished item publishes its stores with
// an agent-scope release and one atomic add on its counter. A step that needs all of the step
// before it (the histogram before the expert scan, ...) counts that step's finished items; GEMM-2
// tile (ti, n) waits only for the N tiles of GEMM-1 on its M tile ti, and a token's combine only
// for the GEMM-2 tiles holding its rows, so GEMM-2 starts on the first M tiles while GEMM-1 still
// runs on the last ones, and so does the combine.
//
// Progress. An item only ever waits for items of earlier steps. Take the earliest waiting item:
// what it waits for is finished or in a queue, ahead of it in step order; the workgroups of that
// queue run items of steps no later than it, none of which wait (it is the earliest), so they
// finish and the item is taken. Every wait is also bounded in time (the caller's bound on the
// 100 MHz wall clock): on expiry the kernel raises an error flag, every later wait gives up at
// once, the remaining items are skipped, the kernel drains and the status word says so.
//
// Arithmetic. Every item runs the same device code as the corresponding kernel of the multi-kernel
// forward, over the same data in the same order, so the outputs are bitwise equal to
// moe_forward's.
#include "moe_combine_body.h"
#include "moe_gemm_big.h"
#include "moe_route_body.h"
#include "moe_sched_body.h"

namespace moe {
namespace {

enum Phase : int {
  kPhWi = 0,   // router matrix as bf16, interleaved by 8 columns (router layers)
  kPhQuant,    // MXFP8: each token quantised once (GEMM-1 gathers its rows from these)
  kPhLogits,   // router logits
  kPhTopk,     // top-k and gate weights
  kPhCount,    // per-chunk expert histogram
  kPhEScan,    // per-expert chunk scan and counts
  kPhTiles,    // offsets, tile table, first tile of each expert (one item)
  kPhRank,     // rows of every assignment (perm, inv)
  kPhGemm1,    // GEMM-1 tiles + SwiGLU (+ MX quantisation of H)
  kPhGemm2,    // GEMM-2 tiles
  kPhCombine,  // fixed-order combine
  kPhases
};

// Item sizes. With one workgroup (four waves) per CU the bandwidth-bound steps get their memory
// parallelism inside each thread: the quantisation requests several blocks' loads at once, the
// combine three vectors' rows at once.
constexpr int kWiSteps = 16;        // 8-column steps of the router matrix per item
constexpr int kQuantJ = 4;          // quantisation blocks per thread per item
constexpr int kLogitTokens = kRouterTileTokens;  // tokens per router item (one router tile)
constexpr int kTopkTokens = 16;     // tokens per top-k item (4 per wave)
constexpr int kCombineTokens = 4;   // tokens per combine item

// the synchronisation words (ints): queue tickets, per-step finished items, the error flag, then
// per M tile the finished GEMM-1 and GEMM-2 N tiles
constexpr int kSyncQueue = 0;
constexpr int kSyncDone = 8;
constexpr int kSyncErr = kSyncDone + kPhases;
constexpr int kSyncTiles = 32;
static_assert(kSyncErr < kSyncTiles, "sync layout");

struct PersistArgs {
  GemmArgs g1, g2;
  const uint16_t* x;
  const uint16_t* w_router;
  const float* bias;
  const int32_t* assign;  // the assignments the schedule reads: given, or the top-k output
  const float* gate_w;    // their gate weights
  uint16_t* y;
  float* wi;  // the interleaved router matrix (bf16 in a float32-sized scratch)
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
  int2* tiles;
  int* tile_count;
  int32_t* etile;  // [E_loc + 1] first tile of each expert
  uint16_t* out_rows;
  int* sync;
  int32_t* status;
  long long timeout;  // wall-clock ticks one wait may take
  int T, h, E, E_loc, k, R, nchunks, bm, Nt1, Nt2;
  int per_xcd[2];     // GEMM-1 / GEMM-2 items per queue
  int n[kPhases];     // items per step
};

__device__ __forceinline__ int ld_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// thread 0: wait until *ctr >= target; false if the error flag is up or the wait ran out of time
// (which raises the flag). The caller acquires once after its last wait.
__device__ bool wait_count(const PersistArgs& a, const int* ctr, int target) {
  if (ld_relaxed(ctr) >= target) return !ld_relaxed(a.sync + kSyncErr);
  const long long start = wall_clock64();
  while (true) {
    if (ld_relaxed(a.sync + kSyncErr)) return false;
    if (ld_relaxed(ctr) >= target) return true;
    if (wall_clock64() - start > a.timeout) {
      __hip_atomic_store(a.sync + kSyncErr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

__device__ __forceinline__ void acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ int* done_of(const PersistArgs& a, int ph) {
  return a.sync + kSyncDone + ph;
}
__device__ __forceinline__ bool step_done(const PersistArgs& a, int ph) {
  return wait_count(a, done_of(a, ph), a.n[ph]);
}

// items of step ph in queue x
__device__ __forceinline__ int queue_items(const PersistArgs& a, int ph, int x) {
  if (ph == kPhGemm1) return a.per_xcd[0];
  if (ph == kPhGemm2) return a.per_xcd[1];
  return (a.n[ph] + 7 - x) / 8;
}

// offsets, tile table and first tile per expert from the expert counts, 256 threads (E_loc <=
// 1024, four experts per thread); integer sums, so the same values as the schedule's scan and
// the tile-table kernel
__device__ void tiles_item(const PersistArgs& a, int* sh) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int E = a.E_loc, bm = a.bm;
  int c[4], t[4], sc = 0, st = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * tid + q;
    c[q] = e < E ? a.counts[e] : 0;
    t[q] = (c[q] + bm - 1) / bm;
    sc += c[q];
    st += t[q];
  }
  int vc = sc, vt = st;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int oc = __shfl_up(vc, off), ot = __shfl_up(vt, off);
    if (lane >= off) {
      vc += oc;
      vt += ot;
    }
  }
  if (lane == 63) {
    sh[wid] = vc;
    sh[4 + wid] = vt;
  }
  __syncthreads();
  int rc = vc - sc, rt = vt - st, tot_t = 0;
  for (int w = 0; w < 4; ++w) {
    if (w < wid) {
      rc += sh[w];
      rt += sh[4 + w];
    }
    tot_t += sh[4 + w];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * tid + q;
    if (e < E) {
      a.offsets[e] = rc;
      a.etile[e] = rt;
      for (int j = 0; j < t[q]; ++j) a.tiles[rt + j] = make_int2(e, rc + j * bm);
    }
    rc += c[q];
    rt += t[q];
  }
  if (tid == 255) {
    a.offsets[E] = rc;
    a.etile[E] = rt;
    *a.tile_count = rt;
  }
  const int max_tiles = (a.R + bm - 1) / bm + E;
  for (int i = tot_t + tid; i < max_tiles; i += 256) a.tiles[i] = make_int2(-1, 0);
}

// The argument block lives in device memory (the set-up kernel copies it there) and is read
// through a pointer the compiler cannot see is loop-invariant: every item loads the fields it uses
// afresh (hits in the caches), instead of all of them being hoisted into scalar registers that stay
// live across the GEMM tiles (which need the whole register file).
__device__ __forceinline__ const PersistArgs* opaque(const PersistArgs* p) {
  asm volatile("" : "+s"(p));
  return p;
}

constexpr int kPend = 4;  // GEMM tiles whose counters one release publishes together

template <bool MX>
__global__ __launch_bounds__(256, 1) void forward_persistent_kernel(
    const PersistArgs* __restrict__ args) {
  constexpr int BM = kPersistentRows;
  constexpr int NS = big_ns(MX, BM), NSR = big_nsr(MX, BM);
  constexpr int LDS = big_lds_bytes(BM, kBigRB, NS, NSR);
  static_assert(LDS >= 4 * 1024 * 4, "LDS of the other steps");
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS];
  // four control words (ticket, ok, M tile, N tile) at the end of the LDS: written by thread 0
  // between items, read by every thread before the barrier that starts the item
  int* ctl = reinterpret_cast<int*>(lds + LDS - 16);
  const int tid = threadIdx.x, wid = tid >> 6;
  const int x = blockIdx.x & 7;  // this workgroup's queue (workgroup L runs on XCD L % 8)
  // this queue's step boundaries: tickets [qend[p-1], qend[p]) are the items of step p
  int qend[kPhases];
  int total = 0;
#pragma unroll
  for (int ph = 0; ph < kPhases; ++ph) {
    total += queue_items(*args, ph, x);
    qend[ph] = total;
  }

  // thread 0: the steps this workgroup has acquired complete, and the next ticket, taken one item
  // ahead (its latency hides behind the current item)
  unsigned acq = 0;
  int next = 0;
  if (tid == 0)
    next = __hip_atomic_fetch_add(args->sync + kSyncQueue + x, 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  // Finished items not yet published (every thread knows how many; thread 0 which tile counters
  // they add to): one release then covers up to kPend items of one step. Published before any
  // item of another step and before the workgroup leaves; within a step only the first item
  // waits, except GEMM-2 tiles waiting for GEMM-1 tiles (whose workgroups never wait for GEMM-2),
  // so no wait depends on items its own workgroup holds back. The combine publishes nothing:
  // nothing waits for it.
  int pend_n = 0, pend_ph = 0;
  int pend[kPend];
  auto flush = [&](const PersistArgs& a) {
    wait_vmcnt<0>();   // this wave's stores of the tiles have completed,
    __syncthreads();   // and every other wave's
    if (tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
#pragma unroll
      for (int q = 0; q < kPend; ++q)
        if (q < pend_n && pend[q] >= 0)
          __hip_atomic_fetch_add(a.sync + pend[q], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(done_of(a, pend_ph), pend_n, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
    pend_n = 0;
  };
  while (true) {
    const PersistArgs& a = *opaque(args);
    if (tid == 0) {
      ctl[0] = next;
      if (next < total)
        next = __hip_atomic_fetch_add(a.sync + kSyncQueue + x, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const int ticket = __builtin_amdgcn_readfirstlane(ctl[0]);
    if (ticket >= total) break;  // uniform
    int ph = 0, first = 0;
#pragma unroll
    for (int p = 0; p + 1 < kPhases; ++p)
      if (ticket >= qend[p]) ph = p + 1, first = qend[p];
    const int i = ticket - first;
    const bool gemm = ph == kPhGemm1 || ph == kPhGemm2;
    const int j = gemm ? i : i * 8 + x;  // item of its step
    if (pend_n > 0 && (ph != pend_ph || pend_n == kPend)) flush(a);

    // ---- wait for what the item reads. Thread 0 acquires once per step it has seen complete
    // (bit p of acq): an item whose inputs all come from such steps needs no wait and no
    // acquire. During the overlap of GEMM-1 with GEMM-2, and of GEMM-2 with the combine, an item
    // waits for its own tiles' counters instead and acquires after them.
    if (tid == 0) {
      bool ok = true;
      int ti = 0, nt = 0;
      auto need = [&](int p) {
        if (!ok || (acq >> p) & 1u) return;
        ok = step_done(a, p);
        if (ok) {
          acquire();
          acq |= 1u << p;
        }
      };
      // a GEMM step complete (all tiles of the table, every N tile): acquired once, as a step
      auto gemm_step_done = [&](int p, int nt_all) {
        if ((acq >> p) & 1u) return true;
        const int mt = ld_relaxed(a.tile_count);
        if (ld_relaxed(done_of(a, p)) < mt * nt_all) return false;
        acquire();
        acq |= 1u << p;
        return true;
      };
      switch (ph) {
        case kPhLogits: need(kPhWi); break;
        case kPhTopk: need(kPhLogits); break;
        case kPhCount: need(kPhTopk); break;
        case kPhEScan: need(kPhCount); break;
        case kPhTiles: need(kPhEScan); break;
        case kPhRank: need(kPhTiles); break;
        case kPhGemm1: need(kPhRank); need(kPhQuant); break;
        case kPhGemm2:
          need(kPhRank);
          if (ok) {
            if (!big_tile_coords(ld_relaxed(a.tile_count), a.Nt2, 1, x, j, ti, nt)) ti = -1;
            else if (!gemm_step_done(kPhGemm1, a.Nt1)) {
              ok = wait_count(a, a.sync + kSyncTiles + ti, a.Nt1);
              if (ok) acquire();
            }
          }
          break;
        case kPhCombine:
          need(kPhRank);
          if (ok && !gemm_step_done(kPhGemm2, a.Nt2)) {
            const int* g2 = a.sync + kSyncTiles + (a.R + a.bm - 1) / a.bm + a.E_loc;
            for (int u = 0; u < kCombineTokens && ok; ++u) {
              const int t = j * kCombineTokens + u;
              if (t >= a.T) break;
              for (int s = 0; s < a.k && ok; ++s) {
                const int r = a.inv[(size_t)t * a.k + s];
                if (r < 0) continue;
                const int e = a.assign[(size_t)t * a.k + s];
                ok = wait_count(a, g2 + a.etile[e] + (r - a.offsets[e]) / a.bm, a.Nt2);
              }
            }
            if (ok) acquire();
          }
          break;
        default: break;
      }
      ctl[1] = ok;
      ctl[2] = ti;
      ctl[3] = nt;
    }
    __syncthreads();
    const bool ok = __builtin_amdgcn_readfirstlane(ctl[1]) != 0;
    const int s_ti = __builtin_amdgcn_readfirstlane(ctl[2]);
    const int s_nt = __builtin_amdgcn_readfirstlane(ctl[3]);
    __syncthreads();  // every thread has its control words: the item may use all of the LDS
    if (!ok) continue;  // an error: skip the item

    // ---- the item; ctr: the GEMM tile counter it adds to (null: none); counted: it adds to its
    // step's counter
    int* ctr = nullptr;
    bool counted = ph != kPhCombine;
    switch (ph) {
      case kPhWi: {
        const int nvb = (a.h / 8 + kWiSteps - 1) / kWiSteps;
        const int eb = j / nvb, v0 = (j % nvb) * kWiSteps;
        for (int v = v0; v < v0 + kWiSteps && v < a.h / 8; ++v)
          w_interleave_bf16_one(a.w_router, a.E, a.h, reinterpret_cast<uint16_t*>(a.wi),
                                eb * 256 + tid, v);
        break;
      }
      case kPhQuant:
        quantize_token_blocks<kQuantJ>(a.x, a.qrows, a.qscales, a.h, a.T,
                                       (long long)j * 256 * kQuantJ);
        break;
      case kPhLogits: {
        const int nbx = (a.T + kLogitTokens - 1) / kLogitTokens;
        router_logits_mfma_tile(a.x, reinterpret_cast<const uint16_t*>(a.wi), a.bias, a.logits,
                                a.T, a.h, a.E, j % nbx, j / nbx);
        break;
      }
      case kPhTopk:
        for (int u = 0; u < kTopkTokens / 4; ++u) {
          const int t = j * kTopkTokens + wid * (kTopkTokens / 4) + u;
          if (t < a.T) topk_softmax_token(a.logits, a.idx, a.tw, a.E, a.k, t);
        }
        break;
      case kPhCount:
        sched_count_chunk(a.assign, a.R, a.E_loc, a.nchunks, a.cc, j, reinterpret_cast<int*>(lds));
        break;
      case kPhEScan:
        if (j * 4 + wid < a.E_loc) sched_expert_scan_wave(a.cc, a.nchunks, a.counts, j * 4 + wid);
        break;
      case kPhTiles:
        tiles_item(a, reinterpret_cast<int*>(lds));
        break;
      case kPhRank:
        sched_rank_chunk(a.assign, a.R, a.E_loc, a.nchunks, a.cc, a.offsets, a.perm, a.inv, j,
                         reinterpret_cast<int*>(lds));
        break;
      case kPhGemm1: {
        int ti, nt;
        const int mt = __builtin_amdgcn_readfirstlane(ld_relaxed(a.tile_count));
        if (!big_tile_coords(mt, a.Nt1, 1, x, j, ti, nt)) {
          counted = false;  // a surplus item
          break;
        }
        big_tile_at<kEpiSwiglu, MX, BM, kBigRB, NS, NSR>(a.g1, ti, nt, lds);
        ctr = a.sync + kSyncTiles + ti;
        break;
      }
      case kPhGemm2: {
        const int ti = s_ti;
        if (ti < 0) {
          counted = false;
          break;
        }
        big_tile_at<kEpiStore, MX, BM, kBigRB, NS, NSR>(a.g2, ti, s_nt, lds);
        ctr = a.sync + kSyncTiles + (a.R + a.bm - 1) / a.bm + a.E_loc + ti;
        break;
      }
      case kPhCombine:
        for (int u = 0; u < kCombineTokens; ++u) {
          const int t = j * kCombineTokens + u;
          if (t >= a.T) break;
          if (a.k <= 8)
            combine_token<8, 3, false>(a.out_rows, a.inv, a.gate_w, nullptr, a.y, a.h, a.k,
                                       nullptr, nullptr, nullptr, 0, t);
          else
            combine_token<16, 1, false>(a.out_rows, a.inv, a.gate_w, nullptr, a.y, a.h, a.k,
                                        nullptr, nullptr, nullptr, 0, t);
        }
        break;
      default: break;
    }
    __syncthreads();  // the LDS is free for the next item
    if (counted) {    // published with the next flush
      if (tid == 0) pend[pend_n] = ctr ? (int)(ctr - a.sync) : -1;
      pend_ph = ph;
      ++pend_n;
    }
  }
  const PersistArgs& a = *opaque(args);
  if (pend_n > 0) flush(a);
  if (tid == 0 && ld_relaxed(a.sync + kSyncErr)) *a.status = MOE_ETIMEOUT;
}

// clears the synchronisation words and the status, and puts the argument block in device memory
__global__ void persistent_init_kernel(PersistArgs a, PersistArgs* dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) a.sync[i] = 0;
  if (i == 0) {
    *a.status = MOE_OK;
    *dst = a;
  }
}

}  // namespace

size_t persistent_args_bytes() { return sizeof(PersistArgs); }

size_t persistent_sync_ints(int R, int E_loc, int bm) {
  return kSyncTiles + 2 * (size_t)((R + bm - 1) / bm + E_loc);
}

hipError_t launch_forward_persistent(const PersistentBuffers& b, int T, int h, int m, int E,
                                     int E_loc, int k, bool mx, int num_cu, long long timeout,
                                     hipStream_t st) {
  const int R = T * k;
  PersistArgs a{};
  const int max_tiles = ffn_big_gemm_args(
      mx ? static_cast<const void*>(b.qrows) : b.x, b.qscales, T, b.offsets, b.prepared,
      b.out_rows, b.ffn_ws, R, h, m, E_loc, mx, b.perm, k, kPersistentRows, a.g1, a.g2);
  const bool router = b.w_router != nullptr;
  const int bm = kPersistentRows;
  a.x = b.x;
  a.w_router = b.w_router;
  a.bias = b.bias;
  a.assign = router ? b.idx : b.assign;
  a.gate_w = router ? b.tw : b.assign_w;
  a.y = b.y;
  a.wi = b.wi;
  a.logits = b.logits;
  a.idx = b.idx;
  a.tw = b.tw;
  a.cc = b.cc;
  a.counts = b.counts;
  a.offsets = b.offsets;
  a.perm = b.perm;
  a.inv = b.inv;
  a.qrows = b.qrows;
  a.qscales = b.qscales;
  a.tiles = const_cast<int2*>(a.g1.tiles);
  a.tile_count = const_cast<int*>(a.g1.tile_count);
  a.etile = b.etile;
  a.out_rows = b.out_rows;
  a.sync = b.sync;
  a.status = b.status;
  a.timeout = timeout;
  a.T = T;
  a.h = h;
  a.E = E;
  a.E_loc = E_loc;
  a.k = k;
  a.R = R;
  a.nchunks = (R + kSchedChunk - 1) / kSchedChunk;
  a.bm = bm;
  a.Nt1 = 2 * m / kBigBN;
  a.Nt2 = h / kBigBN;
  auto per_xcd = [&](int nt) {  // the grouped-GEMM kernels' grid over 8 XCDs
    return big_grid_per_xcd(max_tiles, nt);
  };
  a.per_xcd[0] = per_xcd(a.Nt1);
  a.per_xcd[1] = per_xcd(a.Nt2);
  const int eb = (E + 255) / 256;
  a.n[kPhWi] = router ? eb * ((h / 8 + kWiSteps - 1) / kWiSteps) : 0;
  const long long qblocks = (long long)T * (h / kMxBlock);
  a.n[kPhQuant] = mx ? (int)((qblocks + 256 * kQuantJ - 1) / (256 * kQuantJ)) : 0;
  a.n[kPhLogits] = router ? eb * ((T + kLogitTokens - 1) / kLogitTokens) : 0;
  a.n[kPhTopk] = router ? (T + kTopkTokens - 1) / kTopkTokens : 0;
  a.n[kPhCount] = a.nchunks;
  a.n[kPhEScan] = (E_loc + 3) / 4;
  a.n[kPhTiles] = 1;
  a.n[kPhRank] = a.nchunks;
  a.n[kPhGemm1] = 8 * a.per_xcd[0];
  a.n[kPhGemm2] = 8 * a.per_xcd[1];
  a.n[kPhCombine] = (T + kCombineTokens - 1) / kCombineTokens;
  if (k > 16 || E_loc > 1024) return hipErrorInvalidValue;

  const int nsync = (int)persistent_sync_ints(R, E_loc, bm);
  PersistArgs* dev_args = reinterpret_cast<PersistArgs*>(b.args);
  hipLaunchKernelGGL(persistent_init_kernel, dim3((nsync + 255) / 256), dim3(256), 0, st, a,
                     dev_args, nsync);
  const dim3 grid(num_cu < 8 ? 8 : num_cu / 8 * 8);
  if (mx)
    hipLaunchKernelGGL((forward_persistent_kernel<true>), grid, dim3(256), 0, st, dev_args);
  else
    hipLaunchKernelGGL((forward_persistent_kernel<false>), grid, dim3(256), 0, st, dev_args);
  return hipGetLastError();
}

}  // namespace moe
