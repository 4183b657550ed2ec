// The DMA pipeline of the large-tile grouped GEMM (grouped_gemm_big_kernel): which 16-byte loads a
// wave issues in which order, and how many may still be in flight at each barrier point. Plain
// constexpr arithmetic, shared by the kernel and by a host-side check that replays the issue order
// (so the counts the kernel waits with are the ones that are checked).
//
// Vocabulary. A stage is RB K-bytes of every row of the tile: a weight group W(s) (BN weight rows)
// and a routed-row group R(s) (BM rows). The weight ring is NS stages deep and the row ring NSR:
// at barrier point b (before stage b's fragments are read) the groups W(b + NS - 1) and
// R(b + NSR - 1) are issued into the ring slots stage b - 1 has just freed. Each thread issues
// LOADS units per point, QW of the weight group and QR of the row group; the group of the
// shallower ring goes first (it is needed sooner). A point's units go out in SPS parts: parts
// 0 .. SPS-2 (units [0, U0)) spread over the k-steps of stage b, the last part (units [U0, LOADS),
// empty with the U0 chosen below) right after the barrier of point b + 1. The prologue issues
// every point b < 0 whole.
//
// Loads complete in issue order, so the wait of point j is "at most n loads outstanding", with n
// the number of units issued after the last unit of W(j) and R(j) and before the wait.
#pragma once

#if defined(__HIPCC__) || defined(__HIP__)
#define MOE_HD __host__ __device__
#else
#define MOE_HD
#endif

namespace moe {

struct BigPlan {
  int BN, BM, RB, NS, NSR;
  bool MX;
  int LOADS;   // 16-byte units per thread per point
  int SLOTS;   // 16-byte slots per LDS row
  int QW, QR;  // units of the weight and of the row group
  int SPS;     // MFMA k-steps per stage
  int PC;      // stages per 256-element MX chunk (1 for BF16)
  int NSC;     // untracked scale loads per MX chunk
  bool RFIRST; // the row group goes first (its ring is the shallower one)
  int U0;      // first unit of the last part
};

MOE_HD constexpr int plan_min(int a, int b) { return a < b ? a : b; }
MOE_HD constexpr int plan_max(int a, int b) { return a > b ? a : b; }
MOE_HD constexpr int plan_clamp(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

MOE_HD constexpr BigPlan make_big_plan(bool mx, int bm, int rb, int ns, int nsr) {
  BigPlan p{};
  p.BN = 256;
  p.BM = bm;
  p.RB = rb;
  p.NS = ns;
  p.NSR = nsr;
  p.MX = mx;
  p.LOADS = (p.BN + bm) * rb / 16 / 256;
  p.SLOTS = rb / 16;
  p.QW = p.BN * p.SLOTS / 256;
  p.QR = p.LOADS - p.QW;
  p.SPS = mx ? rb / 64 : rb / 32;
  p.PC = mx ? 4 / p.SPS : 1;
  p.NSC = mx ? 4 + bm / 64 : 0;
  p.RFIRST = nsr < ns;
  // Every unit of a point goes out in the k-steps of its own stage (U0 = LOADS, the last part is
  // empty): loads complete in issue order, so a unit deferred to after the next barrier would
  // shorten the lead of the group issued after it; this way the deeper ring's group keeps its
  // full depth of lead (measured a few percent faster than deferring half of the units).
  p.U0 = p.LOADS;
  return p;
}

// The plan of one kernel instantiation as a type (usable inside the kernel's lambdas, which
// capture no constexpr objects).
template <bool MX, int BM, int RB, int NS, int NSR>
struct BigPlanOf {
  MOE_HD static constexpr BigPlan get() { return make_big_plan(MX, BM, RB, NS, NSR); }
};

// units [lo, hi) of a point that belong to the weight group / the row group
MOE_HD constexpr int plan_w_units(const BigPlan& p, int lo, int hi) {
  const int a = p.RFIRST ? p.QR : 0, b = p.RFIRST ? p.LOADS : p.QW;
  return plan_max(0, plan_min(hi, b) - plan_max(lo, a));
}
MOE_HD constexpr int plan_r_units(const BigPlan& p, int lo, int hi) {
  return plan_max(0, hi - lo) - plan_w_units(p, lo, hi);
}
MOE_HD constexpr bool plan_is_w(const BigPlan& p, int q) {
  return p.RFIRST ? q >= p.QR : q < p.QW;
}
// index of unit q inside its group
MOE_HD constexpr int plan_group_index(const BigPlan& p, int q) {
  return p.RFIRST ? (q >= p.QR ? q - p.QR : q) : (q < p.QW ? q : q - p.QW);
}
MOE_HD constexpr int plan_part_start(const BigPlan& p, int t) {
  return t >= p.SPS ? p.LOADS : t * p.U0 / (p.SPS - 1);
}

MOE_HD constexpr bool plan_exists(int s, int nk) { return s >= 0 && s < nk; }

// existing units of point b in [lo, hi)
MOE_HD constexpr int plan_point_units(const BigPlan& p, int b, int lo, int hi, int nk) {
  return plan_w_units(p, lo, hi) * (plan_exists(b + p.NS - 1, nk) ? 1 : 0) +
         plan_r_units(p, lo, hi) * (plan_exists(b + p.NSR - 1, nk) ? 1 : 0);
}
// existing units of every point before b (all of them are issued before any unit of point b)
MOE_HD constexpr int plan_units_before(const BigPlan& p, int b, int nk) {
  return p.QW * plan_clamp(b + p.NS - 1, 0, nk) + p.QR * plan_clamp(b + p.NSR - 1, 0, nk);
}

// Loads a wave may still have in flight at the wait of barrier point j (0 <= j < nk): the DMA
// units issued after the last unit of W(j) and R(j). Untracked scale loads are not counted (any
// issued after that unit only make the wait stricter).
MOE_HD constexpr int plan_wait_count(const BigPlan& p, int j, int nk) {
  const int issued = j == 0 ? plan_units_before(p, 0, nk)
                            : plan_units_before(p, j - 1, nk) +
                                  plan_point_units(p, j - 1, 0, p.U0, nk);
  const int pw = j - p.NS + 1, pr = j - p.NSR + 1;
  const int lw = p.RFIRST ? p.LOADS : p.QW;  // one past the weight group's last unit
  const int lr = p.RFIRST ? p.QR : p.LOADS;
  const int upto_w = plan_units_before(p, pw, nk) + plan_point_units(p, pw, 0, lw, nk);
  const int upto_r = plan_units_before(p, pr, nk) + plan_point_units(p, pr, 0, lr, nk);
  return issued - plan_max(upto_w, upto_r);
}

// The same in the steady state (every stage the count looks at exists): independent of j.
MOE_HD constexpr int plan_steady_count(const BigPlan& p) {
  return plan_wait_count(p, 2 * (p.NS + p.NSR), 8 * (p.NS + p.NSR));
}

// Stages from which the branch-free k-step runs: stage j with j + max(NS, NSR) < nk issues every
// group of its points unconditionally; rounded down to whole MX chunks.
MOE_HD constexpr int plan_steady_end(const BigPlan& p, int nk) {
  const int e = nk - plan_max(p.NS, p.NSR);
  return e <= 0 ? 0 : e / p.PC * p.PC;
}

// Scale loads of the next chunk that the steady-state wait at point j + 1 may leave in flight
// (stage j being stage P of its chunk): the scale words go out at the start of the chunk's first
// stage, ahead of that stage's DMA parts; at the wait of the chunk's second stage they may still be
// in flight if both of that stage's groups were issued before them (both rings at least three
// deep). They are read only after the next chunk's first wait, which covers them.
MOE_HD constexpr int plan_scales_in_flight(const BigPlan& p, int P) {
  return p.MX && P == 0 && p.PC == 2 && plan_min(p.NS, p.NSR) >= 3 ? p.NSC : 0;
}

// Ring depths of each tile height: an MXFP8 192-row tile and a BF16 256-row tile take a three-deep
// weight ring and a two-deep row ring (144 KB and 160 KB of LDS); 128-row tiles three and four
// (160 KB). The instantiations the launchers use are listed in MOE_BIG_TILE_CONFIGS.
MOE_HD constexpr int big_ns(bool mx, int bm) { return (void)mx, (void)bm, 3; }
MOE_HD constexpr int big_nsr(bool mx, int bm) { return (void)mx, bm >= 192 ? 2 : 4; }
#define MOE_BIG_TILE_CONFIGS(X) X(true, 192) X(true, 128) X(false, 256) X(false, 128)

// The weight gradients' tile: 64 rows with two-deep rings (80 KB of LDS), two workgroups per CU,
// fragments read per k-step (no software pipelining; the DMA issue order is the generic loop's)
constexpr int kWgradRows = 64;
constexpr int kWgradNS = 2;
constexpr int kWgradNSR = 2;

}  // namespace moe
