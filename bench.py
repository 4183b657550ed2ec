#!/usr/bin/env python3
"""MoE layer forward throughput on one MI355X, with the dominant kernel's roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one moe_forward of the whole hot path over one batch of seeded synthetic inputs
(router, top-k, schedule, per-token MX quantisation, grouped SwiGLU GEMMs, combine; expert shares
skip the router). The default workload is the largest one that fits one GPU: the GLM-5.2-shaped
full layer (8,192 tokens, 256 experts, top-8, h = 6144, m = 2048, MXFP8, the pages' default
precision). The other four workloads are measured too, with fewer steps, as extra keys.

Inputs live in HBM before the timed region starts. The K timed steps run back to back between two
device synchronisations; each step records HIP events at its stage boundaries on the library's
stream, which gives every kernel's duration live. After the timed region, a few more steps each
preceded by a 1 GiB write give the bandwidth stages' GB/s with the 256 MB last-level cache flushed.
One JSON line is printed.

The CPU baseline times the oracle (oracle/, float64 NumPy) on a bounded sample of the same
workload's tokens on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

import moe_inputs as I_

METRIC = "MoE layer fwd tokens/s on 1 GPU + grouped-GEMM % MFMA peak (BF16/MXFP8)"
PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0}  # MI355X dense matrix peaks
PEAK_FP32_MFMA_TFLOPS = 157.3  # the router's float32 matrix-core peak
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="glm52")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-tokens", type=int, default=-1,
                    help="tokens of the oracle's timed sample (0 disables the CPU baseline; "
                         "default: every token of an expert share, 32 of a router layer)")
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0,
                    help="repeat the oracle's sample until this much wall time has run")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward timing of workloads that define one")
    ap.add_argument("--no-ring", action="store_true",
                    help="skip the macrobatch-ring timing (its minibatch forwards run the same GEMM "
                         "kernels on fewer rows, which would mix into per-kernel profiles)")
    ap.add_argument("--others", default="tiny,dsv4pro,qwen397,kimi",
                    help="further workloads measured as extra keys ('' for none)")
    ap.add_argument("--other-steps", type=int, default=10)
    ap.add_argument("--flush-steps", type=int, default=3,
                    help="steps after a 1 GiB cache flush for the bandwidth stages' GB/s")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reference for HBM counters)")
    return ap.parse_args()


def copy_calibration(mib: int) -> int:
    """A plain device-to-device copy of a known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch

    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n}), flush=True)
    return 0


def layer_flops(wl) -> dict:
    R = wl.T * wl.k
    f = {
        "gemm1": 4.0 * R * wl.h * wl.m,  # gate and up: 2 * R * h * (2m)
        "gemm2": 2.0 * R * wl.m * wl.h,
        "router": 2.0 * wl.T * wl.h * wl.E if wl.mode == "router" else 0.0,
        "shared": 6.0 * wl.T * wl.h * wl.m_shared,
    }
    f["total"] = sum(f.values())
    return f


def stage_bytes(wl) -> dict:
    """Algorithmic HBM bytes of the bandwidth-bound stages (each byte moved once).

    On the large-tile shapes (h % 256 == 0, 2m % 256 == 0: every benchmark workload) moe_forward
    gathers the routed rows inside GEMM-1's loads: the gather stage is then only the MXFP8
    per-token quantisation (read x, write T rows of codes and scales), or nothing for BF16."""
    R, T, h, k = wl.T * wl.k, wl.T, wl.h, wl.k
    mx = wl.dtype == "mxfp8"
    row_b = h * (1 + 1 / 32) if mx else 2 * h
    fused = h % 256 == 0 and (2 * wl.m) % 256 == 0
    gather = (T * h * 2 + T * row_b if mx else 0) if fused else T * h * 2 + R * row_b + R * 4
    return {
        "gather": gather,
        "combine": R * h * 2 + R * 8 + T * h * 2 + (T * h * 2 if wl.m_shared else 0),
        "topk": T * wl.E * 4 + R * 8 if wl.mode == "router" else 0,
    }


ROOT = os.path.dirname(os.path.abspath(__file__))
GEMM_SOURCES = [os.path.join(ROOT, "routing_expert_grouped_amd", "csrc", f)
                for f in ("moe_gemm_big.h", "moe_gemm_plan.h", "moe_tile_order.h",
                          "moe_gemm_kernels.hip")]


def gemm_source_sha256() -> str:
    """sha256 of the grouped-GEMM sources (the large-tile device code, its DMA plan, its work order
    and the kernels), concatenated in that order: the key under which GEMM counters are kept."""
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """L2-to-fabric bytes per GEMM-1 launch from the committed rocprofv3 counter summary of this
    workload (FETCH_SIZE + WRITE_SIZE, scaled by the copy calibration), or None when there is no
    summary or the GEMM source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"gemm1_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != gemm_source_sha256():
        return None
    return int(kv["gemm1_bytes_per_launch"])


def host_info() -> dict:
    """The host the CPU baseline ran on: usable cores, CPU model, NumPy's BLAS build."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:  # noqa: BLE001
        pass
    return {"cores": cores, "cpu_model": model, "blas": blas, "numpy": np.__version__}


def cpu_baseline(wl, inp, weights_of, shared_host, n_tokens: int, min_seconds: float) -> dict:
    """Times the oracle as it stands (oracle.moe.token_outputs: float64 NumPy, one expert at a
    time) on a bounded sample of the workload's tokens, repeating the pass until at least
    min_seconds of wall time have run, and reports tokens per second over all passes.

    An expert share (6 experts) is run on every token with BLAS on all usable cores. A router layer
    is run on n_tokens sampled tokens with the oracle's per-expert thread pool on all usable cores
    (one BLAS thread each): its sample touches most experts, and each expert's weights are
    MX-quantised once per pass, work that a whole-layer pass would spread over all of that
    expert's rows."""
    from threadpoolctl import threadpool_limits

    from oracle import moe as M  # the oracle is the baseline leg only
    info = host_info()
    cores = info["cores"]
    rng = np.random.default_rng(0)
    if wl.mode == "share":
        tokens = np.arange(min(n_tokens, wl.T))
    else:
        tokens = np.sort(rng.choice(wl.T, min(n_tokens, wl.T), replace=False))
    workers = 1 if wl.mode == "share" else cores
    n_exp = len({int(e) for e in (M.route(inp["x"][tokens], inp["w_router"], inp["bias"],
                                          wl.k)[1] if wl.mode == "router"
                                  else inp["assign"].reshape(-1, wl.k)[tokens]).reshape(-1)
                 if 0 <= e < wl.E_loc})
    passes = 0
    t0 = time.perf_counter()
    with threadpool_limits(1 if workers > 1 else cores):
        while True:
            M.token_outputs(wl, inp, tokens, weights_of, shared_host, workers=workers)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    what = ("every token" if len(tokens) == wl.T else
            f"{len(tokens)} of {wl.T} tokens (seeded sample)")
    return {"value": round(passes * len(tokens) / dt, 3), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{what} of the same workload through oracle.moe.token_outputs (float64 "
                      f"NumPy: routing, every selected expert's SwiGLU FFN with its MX steps, "
                      f"combine), touching {n_exp} of {wl.E_loc} experts, {passes} pass(es), "
                      f"{dt:.1f} s wall, "
                      + ("BLAS on all cores" if workers == 1 else
                         f"{workers} expert workers with one BLAS thread each"),
            "host": info}


def time_backward(G, wl, sh, x, wg, wu, wd, prepared, kw, inp, args) -> dict:
    """The expert-path backward of the same layer, timed on its own: one forward that keeps its
    saved state (timed too, as the training forward), then K backward steps from that state, each
    with HIP events at its stage boundaries, weight gradients in float32 (and, as context, the
    same steps with bf16 weight gradients). Then K steps of the whole layer's backward
    (moe_backward_layer: also the gate-weight, router-matrix and bias gradients and the router's
    part of dX), timed as a whole."""
    import torch

    dev = x.device
    saved = torch.empty(G.moe_saved_bytes(sh, wl.dtype), dtype=torch.uint8, device=dev)
    pbwd = G.moe_prepare_bwd_weights(sh, wl.dtype, wg, wu, wd)
    dy = torch.from_numpy(inp["dy"].view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty(wl.T, wl.h, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(G.moe_forward_workspace_bytes(sh, wl.dtype), dtype=torch.uint8, device=dev)
    fev = G.HipEvents()
    for _ in range(2):
        G.moe_forward_profiled(sh, wl.dtype, x, prepared, fev, y=y, ws=ws, saved=saved, **kw)
    torch.cuda.synchronize()
    fwd_saved_ms = fev.elapsed_ms(0, G.MOE_PROFILE_EVENTS - 1)
    fev.close()
    dx = torch.empty(wl.T, wl.h, dtype=torch.bfloat16, device=dev)
    dw = (torch.empty(wl.E_loc, wl.h, wl.m, dtype=torch.float32, device=dev),
          torch.empty(wl.E_loc, wl.h, wl.m, dtype=torch.float32, device=dev),
          torch.empty(wl.E_loc, wl.m, wl.h, dtype=torch.float32, device=dev))
    bws = torch.empty(G.moe_backward_workspace_bytes(sh, wl.dtype), dtype=torch.uint8, device=dev)
    evs = [G.HipEvents(G.MOE_BWD_PROFILE_EVENTS, G.BWD_STAGES) for _ in range(args.steps)]
    wev = G.HipEvents(G.MOE_BWD_PROFILE_EVENTS, G.BWD_STAGES)
    for _ in range(args.warmup):
        G.moe_backward_profiled(sh, wl.dtype, x, dy, saved, pbwd, wev, dx=dx, dw=dw, ws=bws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev in evs:
        G.moe_backward_profiled(sh, wl.dtype, x, dy, saved, pbwd, ev, dx=dx, dw=dw, ws=bws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    stages = {k: 0.0 for k in G.BWD_STAGES}
    for ev in evs:
        for k, v in ev.stage_ms().items():
            stages[k] += v / args.steps
    for ev in evs + [wev]:
        ev.close()
    # context for the store-bound weight gradients: the same steps with dW in bf16 (half the
    # bytes stored); the reported backward keeps float32
    dw16 = tuple(torch.empty(t.shape, dtype=torch.bfloat16, device=dev) for t in dw)
    evs16 = [G.HipEvents(G.MOE_BWD_PROFILE_EVENTS, G.BWD_STAGES) for _ in range(args.steps)]
    for ev in evs16[:1] * args.warmup:
        G.moe_backward_profiled(sh, wl.dtype, x, dy, saved, pbwd, ev, dx=dx, dw=dw16,
                                dw_fp32=False, ws=bws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev in evs16:
        G.moe_backward_profiled(sh, wl.dtype, x, dy, saved, pbwd, ev, dx=dx, dw=dw16,
                                dw_fp32=False, ws=bws)
    torch.cuda.synchronize()
    ms16 = (time.perf_counter() - t0) * 1e3 / args.steps
    st16 = {k: 0.0 for k in G.BWD_STAGES}
    for ev in evs16:
        for k, v in ev.stage_ms().items():
            st16[k] += v / args.steps
        ev.close()
    del dw16
    # the whole layer's backward: the expert path plus the gate-weight and router gradients
    wr = kw.get("w_router")
    lay = lambda: G.moe_backward_layer(sh, wl.dtype, x, dy, saved, pbwd, w_router=wr, dx=dx,
                                       dw=dw, ws=bws)
    for _ in range(args.warmup):
        lay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        lay()
    torch.cuda.synchronize()
    layer_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    R = wl.T * wl.k
    flops = 12.0 * R * wl.h * wl.m  # dH, dA (dgrad) and the three weight gradients
    peak = PEAK_TFLOPS[wl.dtype]
    gemm_ms = sum(stages[k] for k in ("dgrad_dh_dswiglu", "dgrad_da", "wgrad_gate_up",
                                       "wgrad_down"))
    return {"ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "gemm_mfma_frac": round(flops / (gemm_ms * 1e-3) / 1e12 / peak, 4),
            "flop": flops, "dw_dtype": "f32", "training_forward_ms": round(fwd_saved_ms, 4),
            "layer_backward_ms": round(layer_ms, 4),
            "stages_ms": {k: round(v, 4) for k, v in stages.items()},
            "bf16_dw": {"ms_per_step": round(ms16, 4),
                        "wgrad_gate_up": round(st16["wgrad_gate_up"], 4),
                        "wgrad_down": round(st16["wgrad_down"], 4)}}


def expert_roofline(wl, counts, g1_ms: float, g2_ms: float) -> dict:
    """The grouped GEMMs against the per-expert roofline: each expert e with n_e routed rows takes
    at least max(FLOP_e / MFMA peak, bytes_e / HBM peak), summed over experts. GEMM-1: FLOP_e =
    4 h m n_e, bytes_e = W1 (2 h m elements) + n_e input rows (h) + H written (n_e m); GEMM-2:
    FLOP_e = 2 h m n_e, bytes_e = W2 (h m) + H read (n_e m) + O written (n_e h, bf16). Element
    sizes: E4M3 1 byte + one scale byte per 32 (MXFP8), bf16 2 bytes."""
    mx = wl.dtype == "mxfp8"
    be = (1 + 1 / 32) if mx else 2.0
    pf = PEAK_TFLOPS[wl.dtype] * 1e12
    bw = PEAK_HBM_GBS * 1e9
    h, m = wl.h, wl.m
    n = np.asarray(counts, np.float64)
    n = n[n > 0]
    t1 = np.maximum(4 * h * m * n / pf, (2 * h * m * be + n * h * be + n * m * be) / bw).sum()
    t2 = np.maximum(2 * h * m * n / pf, (h * m * be + n * m * be + n * h * 2) / bw).sum()
    return {"gemm1_bound_ms": round(t1 * 1e3, 4), "gemm2_bound_ms": round(t2 * 1e3, 4),
            "gemm1_frac": round(t1 * 1e3 / g1_ms, 4), "gemm2_frac": round(t2 * 1e3 / g2_ms, 4),
            "gemms_frac": round((t1 + t2) * 1e3 / (g1_ms + g2_ms), 4)}


class Setup:
    """A workload's inputs, weights and prepared weights on the device."""

    def __init__(self, G, wl, dev, seed):
        import torch

        self.wl, self.dev = wl, dev
        self.inp = I_.make_inputs(wl, seed=seed)
        self.x = self.bf16(self.inp["x"])
        self.w = I_.torch_expert_weights(wl, dev, seed=seed)
        self.sh = G.make_shape(wl.T, wl.h, wl.m, wl.E, wl.k, wl.E_loc, wl.m_shared)
        self.prepared = G.moe_prepare_weights(self.sh, wl.dtype, *self.w)
        self.shared_w = self.shared_prep = None
        if wl.m_shared:
            self.shared_w = I_.torch_shared_weights(wl, dev, seed=seed)
            ssh = G.make_shape(wl.T, wl.h, wl.m_shared, 1, 1, 1)
            self.shared_prep = G.moe_prepare_weights(ssh, "bf16", *self.shared_w)
        self.kw = {}
        if wl.mode == "router":
            self.kw["w_router"] = self.bf16(self.inp["w_router"])
            self.kw["bias"] = (None if self.inp["bias"] is None
                               else torch.from_numpy(self.inp["bias"]).to(dev))
        else:
            self.kw["assign"] = torch.from_numpy(self.inp["assign"]).to(dev)
            self.kw["assign_w"] = torch.from_numpy(self.inp["assign_w"]).to(dev)
        self.y = torch.empty(wl.T, wl.h, dtype=torch.bfloat16, device=dev)
        self.ws = torch.empty(G.moe_forward_workspace_bytes(self.sh, wl.dtype), dtype=torch.uint8,
                              device=dev)

    def bf16(self, a):
        import torch
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.dev).view(
            torch.bfloat16)


def measure_forward(G, S: Setup, steps: int, warmup: int, flush_steps: int) -> dict:
    """Times `steps` back-to-back forwards (moe_forward, after `warmup`): ms_per_step. Then the
    same number of profiled forwards (moe_forward_profiled, the same launches with a HIP event at
    every stage boundary, which cost a few µs each) for the stage times; then `flush_steps`
    forwards each preceded by a 1 GiB write (outside the stage events) for the bandwidth stages'
    GB/s with the last-level cache flushed."""
    import torch

    wl = S.wl

    def step(ev):
        G.moe_forward_profiled(S.sh, wl.dtype, S.x, S.prepared, ev, shared_prepared=S.shared_prep,
                               y=S.y, ws=S.ws, **S.kw)

    def plain():
        G.moe_forward(S.sh, wl.dtype, S.x, S.prepared, shared_prepared=S.shared_prep, y=S.y,
                      ws=S.ws, **S.kw)

    events = [G.HipEvents() for _ in range(steps)]
    warm_ev = G.HipEvents()
    for _ in range(warmup):
        step(warm_ev)
        plain()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        plain()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    # the same forwards one by one between events on the launch stream: median, min and p90
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record()
    for i in range(steps):
        plain()
        marks[i + 1].record()
    torch.cuda.synchronize()
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    step_stats = {"median": round(per_step[steps // 2], 4), "min": round(per_step[0], 4),
                  "p90": round(per_step[min(steps - 1, (9 * steps) // 10)], 4)}
    t0 = time.perf_counter()
    for ev in events:
        step(ev)
    torch.cuda.synchronize()
    profiled_ms = (time.perf_counter() - t0) * 1e3 / steps
    stages = {k: 0.0 for k in G.STAGES}
    for ev in events:
        for k, v in ev.stage_ms().items():
            stages[k] += v / steps
    flushed = {k: 0.0 for k in G.STAGES}
    if flush_steps > 0:
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=S.dev)
        fev = [G.HipEvents() for _ in range(flush_steps)]
        for ev in fev:
            scratch.fill_(1)
            step(ev)
        torch.cuda.synchronize()
        for ev in fev:
            for k, v in ev.stage_ms().items():
                flushed[k] += v / flush_steps
            ev.close()
        # the practical HBM ceiling of this GPU for the bandwidth stages: a plain 1 GiB device
        # copy (read + write bytes over its event time)
        dst = torch.empty_like(scratch)
        dst.copy_(scratch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(scratch)
        e1.record()
        torch.cuda.synchronize()
        copy_gbs = round(2 * 5 * scratch.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        del scratch, dst
    else:
        copy_gbs = None
    for ev in events + [warm_ev]:
        ev.close()
    counts = G.moe_forward_views(S.sh, wl.dtype, S.ws)["counts"].cpu().numpy()
    fl = layer_flops(wl)
    by = stage_bytes(wl)
    peak = PEAK_TFLOPS[wl.dtype]
    g1_ms, g2_ms = stages["gemm1_gate_up_swiglu"], stages["gemm2_down"]

    def gbs(name, st):
        ms = st[name]
        return round(by[name] / (ms * 1e-3) / 1e9, 1) if ms > 0 and by[name] else None

    r = {
        "tokens_per_s": round(wl.T / (ms_per_step * 1e-3), 1),
        "ms_per_step": round(ms_per_step, 4),
        "step_ms": step_stats,
        "profiled_ms_per_step": round(profiled_ms, 4),
        "gemm1_tflops": round(fl["gemm1"] / (g1_ms * 1e-3) / 1e12, 1),
        "gemm1_mfma_frac": round(fl["gemm1"] / (g1_ms * 1e-3) / 1e12 / peak, 4),
        "grouped_gemm_mfma_frac": round((fl["gemm1"] + fl["gemm2"]) / ((g1_ms + g2_ms) * 1e-3)
                                        / 1e12 / peak, 4),
        "expert_roofline": expert_roofline(wl, counts, g1_ms, g2_ms),
        "layer_tflops": round(fl["total"] / (ms_per_step * 1e-3) / 1e12, 1),
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "stages_gbs": {k: gbs(k, stages) for k in ("gather", "combine", "topk")},
        "stages_gbs_flushed": ({k: gbs(k, flushed) for k in ("gather", "combine", "topk")}
                               if flush_steps > 0 else None),
        "hbm_copy_gbs": copy_gbs,
        "router_tflops": (round(fl["router"] / (stages["router_logits"] * 1e-3) / 1e12, 1)
                          if fl["router"] and stages["router_logits"] > 0 else None),
    }
    r["router_fp32_mfma_frac"] = (round(r["router_tflops"] / PEAK_FP32_MFMA_TFLOPS, 4)
                                  if r["router_tflops"] else None)
    return r


def measure_persistent(G, S: Setup, steps: int, warmup: int):
    """The same forward as one persistent kernel (moe_forward_persistent) against the plain
    multi-kernel moe_forward (no stage events), both timed over `steps` back-to-back calls; None
    for a shape the persistent kernel does not cover (a shared expert)."""
    import torch

    wl = S.wl
    if wl.m_shared or G.moe_forward_persistent_workspace_bytes(S.sh, wl.dtype) == 0:
        return None
    yp = torch.empty_like(S.y)
    wsp = torch.empty(G.moe_forward_persistent_workspace_bytes(S.sh, wl.dtype), dtype=torch.uint8,
                      device=S.dev)
    status = torch.zeros(1, dtype=torch.int32, device=S.dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    ms_p = timed(lambda: G.moe_forward_persistent(S.sh, wl.dtype, S.x, S.prepared, y=yp, ws=wsp,
                                                  status=status, **S.kw))
    ms_f = timed(lambda: G.moe_forward(S.sh, wl.dtype, S.x, S.prepared, y=S.y, ws=S.ws, **S.kw))
    same = bool(torch.equal(yp.view(torch.int16), S.y.view(torch.int16)))
    return {"ms_per_step": round(ms_p, 4), "multi_kernel_ms_per_step": round(ms_f, 4),
            "status": int(status.item()), "bitwise_equal_to_multi_kernel": same}


def library_dense_gemms(wl, dev) -> dict:
    """Context, not part of the path: the vendor library's dense GEMM (torch -> hipBLASLt) at the
    grouped GEMMs' shapes taken as one product over all routed rows, [R x K] by one [K x N] weight
    (GEMM-1: K = h, N = 2m; GEMM-2: K = m, N = h), in BF16, or for MXFP8 in FP8 E4M3 with one
    scale per tensor (torch._scaled_mm; the library has no block-scaled path here). One weight
    matrix stays in the caches, the grouped GEMMs stream every expert's weights."""
    import torch

    R = wl.T * wl.k
    out = {"dtype": ("fp8 e4m3, per-tensor scale" if wl.dtype == "mxfp8" else "bf16"),
           "shapes": {"gemm1": [R, 2 * wl.m, wl.h], "gemm2": [R, wl.h, wl.m]}}
    for name, (M, N, K) in (("gemm1", (R, 2 * wl.m, wl.h)), ("gemm2", (R, wl.h, wl.m))):
        try:
            if wl.dtype == "mxfp8":
                A = (torch.randn(M, K, device=dev) * 0.5).to(torch.float8_e4m3fn)
                B = (torch.randn(N, K, device=dev) * 0.5).to(torch.float8_e4m3fn)
                one = torch.ones((), device=dev)

                def f():
                    return torch._scaled_mm(A, B.t(), scale_a=one, scale_b=one,
                                            out_dtype=torch.bfloat16)
            else:
                A = torch.randn(M, K, device=dev).to(torch.bfloat16)
                B = torch.randn(N, K, device=dev).to(torch.bfloat16)

                def f():
                    return A @ B.t()
            for _ in range(3):
                f()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                f()
            e1.record()
            torch.cuda.synchronize()
            out[name + "_ms"] = round(e0.elapsed_time(e1) / 10, 4)
            del A, B
        except Exception as exc:  # a library without this path: report, do not fail the bench
            out[name + "_ms"] = None
            out[name + "_error"] = repr(exc)[:200]
    torch.cuda.empty_cache()
    return out


def measure_graph(G, S: Setup, steps: int, warmup: int) -> dict:
    """The same forward captured once into a HIP graph (torch.cuda.CUDAGraph) and replayed: the
    launch sequence is recorded, so each step is one graph launch (what a serving loop over small
    batches would run). Its output is compared bitwise with the eager forward's."""
    import torch

    wl = S.wl
    Y = torch.empty_like(S.y)

    def fwd():
        G.moe_forward(S.sh, wl.dtype, S.x, S.prepared, shared_prepared=S.shared_prep, y=Y,
                      ws=S.ws, **S.kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = Y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    same = bool(torch.equal(Y.view(torch.int16), ref.view(torch.int16)))
    del g
    return {"ms_per_step": round(ms, 4), "bitwise_equal_to_eager": same}


def measure_ring(G, S: Setup, steps: int, warmup: int) -> list:
    """moe_forward_ring: all T tokens streamed through a fixed buffer of a fraction of the one-shot
    workspace (the pages' macrobatch ring), in minibatches of the largest token count that fits;
    step time and whether y equals the one-shot forward bitwise."""
    import torch

    wl = S.wl
    full = G.moe_forward_workspace_bytes(S.sh, wl.dtype)
    ref = S.y.clone()
    out = []
    for frac in (0.5, 0.25, 0.125):
        nbytes = int(full * frac) // 256 * 256
        ring = torch.empty(nbytes, dtype=torch.uint8, device=S.dev)
        y = torch.empty_like(S.y)

        def run():
            return G.moe_forward_ring(S.sh, wl.dtype, S.x, S.prepared, ring,
                                      shared_prepared=S.shared_prep, y=y, **S.kw)[1]

        for _ in range(warmup):
            tmb = run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            run()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        out.append({"ring_bytes": nbytes, "fraction_of_workspace": frac,
                    "minibatch_tokens": tmb, "ms_per_step": round(ms, 4),
                    "bitwise_equal_to_one_forward": bool(torch.equal(y.view(torch.int16),
                                                                     ref.view(torch.int16)))})
        del ring, y
    torch.cuda.empty_cache()
    return out


def progress(msg: str) -> None:
    """One line on stderr per finished part of the run (the JSON line goes to stdout)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def main() -> int:
    args = parse()
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the library runs one GPU's share of the layer and has no multi-GPU path.",
              file=sys.stderr)
        return 2

    import torch

    import routing_expert_grouped_amd as G

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    wl = I_.get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S = Setup(G, wl, dev, args.seed)
    progress(f"{wl.name}: inputs and prepared weights ready")
    r = measure_forward(G, S, args.steps, args.warmup, args.flush_steps)
    progress(f"forward timed: {r['ms_per_step']} ms per step")
    persistent = measure_persistent(G, S, args.steps, args.warmup)
    progress(f"persistent forward timed: {persistent}")
    graph = measure_graph(G, S, args.steps, args.warmup)
    progress(f"graph-replayed forward timed: {graph}")
    ring = None if args.no_ring else measure_ring(G, S, max(3, args.steps // 4), 1)
    progress(f"macrobatch ring timed: {ring}")
    library = library_dense_gemms(wl, dev)
    progress(f"library dense GEMMs: {library}")

    backward = None
    if wl.backward and not args.no_backward:
        backward = time_backward(G, wl, S.sh, S.x, *S.w, S.prepared, S.kw, S.inp, args)
        progress(f"backward timed: {backward.get('ms_per_step')} ms per step")

    baseline = None
    n_cpu = args.cpu_sample_tokens
    if n_cpu < 0:
        n_cpu = wl.T if wl.mode == "share" else 32
    if n_cpu > 0:
        def host_bits(t):
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

        cache = {}

        def weights_of(e):
            """Expert weights copied to the host (kept for the few experts of a share)."""
            if e in cache:
                return cache[e]
            v = tuple(host_bits(t[e]) for t in S.w)
            if wl.mode == "share":
                cache[e] = v
            return v

        if wl.mode == "share":
            for e in range(wl.E_loc):
                weights_of(e)
        sh_host = tuple(host_bits(t) for t in S.shared_w) if S.shared_w is not None else None
        baseline = cpu_baseline(wl, S.inp, weights_of, sh_host, n_cpu, args.cpu_min_seconds)
        progress(f"cpu baseline: {baseline.get('value')} {baseline.get('unit')}")

    others = {}
    for name in [n for n in args.others.split(",") if n]:
        w2 = I_.get(name)
        if w2.name == wl.name:
            continue
        S2 = Setup(G, w2, dev, args.seed)
        o = measure_forward(G, S2, args.other_steps, 2, 0)
        others[w2.name] = {k: o[k] for k in ("tokens_per_s", "ms_per_step",
                                             "profiled_ms_per_step", "gemm1_mfma_frac",
                                             "grouped_gemm_mfma_frac", "expert_roofline",
                                             "stages_ms")}
        others[w2.name]["dtype"] = w2.dtype
        others[w2.name]["persistent"] = measure_persistent(G, S2, args.other_steps, 2)
        others[w2.name]["graph"] = measure_graph(G, S2, args.other_steps, 2)
        progress(f"{w2.name}: {o['ms_per_step']} ms per step")
        del S2
        torch.cuda.empty_cache()

    peak = PEAK_TFLOPS[wl.dtype]
    out = {
        "metric": METRIC,
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; random-init expert weights of the stated shapes)",
        "config": {"workload": wl.name, "T": wl.T, "h": wl.h, "m": wl.m, "E": wl.E,
                   "E_loc": wl.E_loc, "k": wl.k, "routed_rows": wl.T * wl.k,
                   "mode": wl.mode, "m_shared": wl.m_shared},
        "roofline": {"bound": "mfma", "kernel": "grouped GEMM-1 (gate/up + SwiGLU epilogue)",
                     "achieved": r["gemm1_tflops"], "peak": peak, "unit": "TFLOP/s",
                     "frac": r["gemm1_mfma_frac"], "traffic": measured_traffic(wl.name)},
        "expert_roofline": r["expert_roofline"],
        "grouped_gemm_mfma_frac": r["grouped_gemm_mfma_frac"],
        "layer_tflops": r["layer_tflops"],
        "router_tflops": r["router_tflops"],
        "router_fp32_mfma_frac": r["router_fp32_mfma_frac"],
        "step_ms": r["step_ms"],
        "profiled_ms_per_step": r["profiled_ms_per_step"],
        "stages_ms": r["stages_ms"],
        "stages_gbs": r["stages_gbs"],
        "stages_gbs_flushed": r["stages_gbs_flushed"],
        "hbm_copy_gbs": r["hbm_copy_gbs"],
        "library_dense_gemm": library,
        "persistent": persistent,
        "graph": graph,
        "ring": ring,
        "cpu_baseline": baseline,
        "other_workloads": others,
    }
    if backward is not None:
        out["backward"] = backward
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
