#!/usr/bin/env python3
"""MoE layer forward throughput on one MI355X, with the dominant kernel's roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one moe_forward of the whole hot path over one batch of seeded synthetic inputs
(expert shares: schedule, gather, grouped SwiGLU GEMMs, combine; full layers: router and top-k
first). The default workload is the DeepSeek-V4-Pro-shaped expert share of one GPU at expert
parallelism 64 (2,048 source tokens, 6 local experts, top-6, h = 7168, m = 3072, BF16).

Inputs live in HBM before the timed region starts. The K timed steps run back to back between two
device synchronisations; each step records HIP events at its stage boundaries on the library's
stream, which gives every kernel's duration live. One JSON line is printed.

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

METRIC = "MoE layer fwd tokens/s on 1 GPU + grouped-GEMM % MFMA peak (BF16/MXFP8)"
PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0}  # MI355X dense matrix peaks
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv4pro")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-tokens", type=int, default=2048,
                    help="tokens of the oracle's timed sample (0 disables the CPU baseline)")
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0,
                    help="repeat the oracle's sample until this much wall time has run")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward timing of workloads that define one")
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
GEMM_SOURCE = os.path.join(ROOT, "routing_expert_grouped_amd", "csrc", "moe_gemm_kernels.hip")


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
    src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    if kv.get("kernel_source_sha256") != src:
        return None
    return int(kv["gemm1_bytes_per_launch"])


def cpu_baseline(wl, inp, weights_host, shared_host, n_tokens: int, min_seconds: float) -> dict:
    """Times the oracle on the first n_tokens tokens, repeating the pass until at least
    min_seconds of wall time have run (a sample that is the whole workload takes only a few
    seconds on a many-core host), and reports tokens per second over all passes."""
    from oracle import moe as M  # the oracle is the baseline leg only
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    tokens = np.arange(min(n_tokens, wl.T))
    passes = 0
    t0 = time.perf_counter()
    while True:
        M.token_outputs(wl, inp, tokens, weights_host.__getitem__, shared_host)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": round(passes * len(tokens) / dt, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {len(tokens)} of {wl.T} tokens of the same workload through "
                      f"oracle.moe.token_outputs (float64 NumPy, routing + every selected "
                      f"expert's SwiGLU FFN + combine), {passes} pass(es), {dt:.1f} s wall"}


def time_backward(G, wl, sh, x, wg, wu, wd, prepared, kw, inp, args) -> dict:
    """The expert-path backward of the same layer, timed on its own: one forward that keeps its
    saved state (timed too, as the training forward), then K backward steps from that state, each
    with HIP events at its stage boundaries. Weight gradients in float32."""
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
    R = wl.T * wl.k
    flops = 12.0 * R * wl.h * wl.m  # dH, dA (dgrad) and the three weight gradients
    peak = PEAK_TFLOPS[wl.dtype]
    gemm_ms = sum(stages[k] for k in ("dgrad_dh_dswiglu", "dgrad_da", "wgrad_gate_up",
                                       "wgrad_down"))
    return {"ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "gemm_mfma_frac": round(flops / (gemm_ms * 1e-3) / 1e12 / peak, 4),
            "flop": flops, "dw_dtype": "f32", "training_forward_ms": round(fwd_saved_ms, 4),
            "stages_ms": {k: round(v, 4) for k, v in stages.items()}}


def main() -> int:
    args = parse()
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "this build has no multi-GPU path; see DESIGN.md for how it would shard.",
              file=sys.stderr)
        return 2

    import torch

    import moe_inputs as I
    import routing_expert_grouped_amd as G

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    wl = I.get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = I.make_inputs(wl, seed=args.seed)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    x = bf16(inp["x"])
    wg, wu, wd = I.torch_expert_weights(wl, dev, seed=args.seed)
    sh = G.make_shape(wl.T, wl.h, wl.m, wl.E, wl.k, wl.E_loc, wl.m_shared)
    prepared = G.moe_prepare_weights(sh, wl.dtype, wg, wu, wd)
    shared_prep = None
    shared_w = None
    if wl.m_shared:
        shared_w = I.torch_shared_weights(wl, dev, seed=args.seed)
        ssh = G.make_shape(wl.T, wl.h, wl.m_shared, 1, 1, 1)
        shared_prep = G.moe_prepare_weights(ssh, "bf16", *shared_w)
    kw = {}
    if wl.mode == "router":
        kw["w_router"] = bf16(inp["w_router"])
        kw["bias"] = None if inp["bias"] is None else torch.from_numpy(inp["bias"]).to(dev)
    else:
        kw["assign"] = torch.from_numpy(inp["assign"]).to(dev)
        kw["assign_w"] = torch.from_numpy(inp["assign_w"]).to(dev)
    y = torch.empty(wl.T, wl.h, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(G.moe_forward_workspace_bytes(sh, wl.dtype), dtype=torch.uint8, device=dev)
    events = [G.HipEvents() for _ in range(args.steps)]
    warm_ev = G.HipEvents()

    def step(ev):
        G.moe_forward_profiled(sh, wl.dtype, x, prepared, ev, shared_prepared=shared_prep, y=y,
                               ws=ws, **kw)

    for _ in range(args.warmup):
        step(warm_ev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    stages = {k: 0.0 for k in G.STAGES}
    for ev in events:
        for k, v in ev.stage_ms().items():
            stages[k] += v / args.steps
    for ev in events + [warm_ev]:
        ev.close()

    fl = layer_flops(wl)
    by = stage_bytes(wl)
    peak = PEAK_TFLOPS[wl.dtype]
    g1_ms = stages["gemm1_gate_up_swiglu"]
    g2_ms = stages["gemm2_down"]
    g1_tf = fl["gemm1"] / (g1_ms * 1e-3) / 1e12
    gemm_tf = (fl["gemm1"] + fl["gemm2"]) / ((g1_ms + g2_ms) * 1e-3) / 1e12
    tokens_per_s = wl.T / (ms_per_step * 1e-3)

    def gbs(name):
        ms = stages[name]
        return round(by[name] / (ms * 1e-3) / 1e9, 1) if ms > 0 and by[name] else None

    backward = None
    if wl.backward and not args.no_backward:
        backward = time_backward(G, wl, sh, x, wg, wu, wd, prepared, kw, inp, args)

    baseline = None
    if args.cpu_sample_tokens > 0:
        def host_bits(t):
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

        class HostWeights(dict):
            """Expert weights copied to the host on first use (all of them up front for an
            expert share, which holds only a few experts)."""

            def __missing__(self, e):
                self[e] = tuple(host_bits(t[e]) for t in (wg, wu, wd))
                return self[e]

        host = HostWeights()
        if wl.mode == "share":
            for e in range(wl.E_loc):
                host[e]
        sh_host = tuple(host_bits(t) for t in shared_w) if shared_w is not None else None
        baseline = cpu_baseline(wl, inp, host, sh_host, args.cpu_sample_tokens,
                                    args.cpu_min_seconds)

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; random-init expert weights of the stated shapes)",
        "config": {"workload": wl.name, "T": wl.T, "h": wl.h, "m": wl.m, "E": wl.E,
                   "E_loc": wl.E_loc, "k": wl.k, "routed_rows": wl.T * wl.k,
                   "mode": wl.mode, "m_shared": wl.m_shared},
        "roofline": {"bound": "mfma", "kernel": "grouped GEMM-1 (gate/up + SwiGLU epilogue)",
                     "achieved": round(g1_tf, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(g1_tf / peak, 4), "traffic": measured_traffic(wl.name)},
        "grouped_gemm_mfma_frac": round(gemm_tf / peak, 4),
        "layer_tflops": round(fl["total"] / (ms_per_step * 1e-3) / 1e12, 1),
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "stages_gbs": {k: gbs(k) for k in ("gather", "combine", "topk")},
        "cpu_baseline": baseline,
    }
    if backward is not None:
        out["backward"] = backward
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
