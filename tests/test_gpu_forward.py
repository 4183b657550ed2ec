"""GPU parity of moe_forward (the whole layer) on scaled-down versions of the five workloads:
routing and schedule bit-exact, output within tolerance, two runs bitwise identical, and the same
bits as the separate entry points composed (route, permute, expert FFN, combine)."""
import math
import numpy as np
import pytest

import moe_inputs as I
from oracle import moe as M
from tests._gpu_helpers import (BF16_TOL, MX_TOL, dev, dev_bf16, host_bf16_bits,
                                host_f64_from_bf16, normwise_err, note, poisoned, require_gpu,
                                torch)

pytestmark = pytest.mark.gpu

SCALED = {
    "tiny": dict(),
    "dsv4pro": dict(T=256, h=512, m=384),
    "qwen397": dict(T=320, h=512, m=128, E=64, E_loc=64),
    "kimi": dict(T=192, h=512, m=256, m_shared=256),
    "glm52": dict(T=300, h=768, m=512, E=64, E_loc=64),
}


def run_forward(G, wl, inp, weights, shared=None, y=None, ws=None):
    sh = G.make_shape(wl.T, wl.h, wl.m, wl.E, wl.k, wl.E_loc, wl.m_shared)
    prepared = G.moe_prepare_weights(sh, wl.dtype, *weights)
    shared_prep = None
    if shared is not None:
        ssh = G.make_shape(wl.T, wl.h, wl.m_shared, 1, 1, 1)
        shared_prep = G.moe_prepare_weights(ssh, "bf16", *shared)
    kw = {}
    if wl.mode == "router":
        kw["w_router"] = dev_bf16(inp["w_router"])
        kw["bias"] = None if inp["bias"] is None else dev(inp["bias"])
    else:
        kw["assign"] = dev(inp["assign"])
        kw["assign_w"] = dev(inp["assign_w"])
    y, ws = G.moe_forward(sh, wl.dtype, dev_bf16(inp["x"]), prepared,
                          shared_prepared=shared_prep, y=y, ws=ws, **kw)
    return sh, y, ws


@pytest.mark.parametrize("name", list(SCALED))
def test_forward_scaled_workloads(name):
    G = require_gpu()
    base = I.get(name)
    wl = I.scaled(base, **SCALED[name]) if SCALED[name] else base
    note(f"forward {wl.describe()}")
    inp = I.make_inputs(wl, seed=0)
    wts = [I.expert_weights(wl, e) for e in range(wl.E_loc)]
    weights = tuple(dev_bf16(np.stack([w[i] for w in wts])) for i in range(3))
    shared = None
    if wl.m_shared:
        sw = I.shared_weights(wl)
        shared = tuple(dev_bf16(v) for v in sw)
    y0 = poisoned((wl.T, wl.h), torch.bfloat16)
    sh, y, ws = run_forward(G, wl, inp, weights, shared, y=y0)
    torch.cuda.synchronize()
    ref = M.layer_forward(wl, inp, lambda e: wts[e],
                          shared_weights=I.shared_weights(wl) if wl.m_shared else None)
    v = G.moe_forward_views(sh, wl.dtype, ws)
    if wl.mode == "router":
        assert np.array_equal(v["logits"].cpu().numpy().view(np.uint32),
                              ref["logits"].view(np.uint32))
        assert np.array_equal(v["topk_idx"].cpu().numpy(), ref["idx"])
        assert np.allclose(v["topk_w"].cpu().numpy(), ref["w"], rtol=1e-6, atol=0)
    for key in ("counts", "offsets", "perm", "inv"):
        assert np.array_equal(v[key].cpu().numpy(), ref[key]), key
    got = host_f64_from_bf16(y)
    assert np.isfinite(got).all()
    err = normwise_err(got, ref["y"])
    note(f"  normwise error {err:.3e}")
    assert err <= (MX_TOL if wl.dtype == "mxfp8" else BF16_TOL)
    # run again into a fresh poisoned buffer and a fresh workspace: bitwise identical
    y1 = poisoned((wl.T, wl.h), torch.bfloat16)
    _, y1, _ = run_forward(G, wl, inp, weights, shared, y=y1)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(y), host_bf16_bits(y1))


@pytest.mark.parametrize("name", ["tiny", "dsv4pro", "qwen397", "kimi", "glm52"])
def test_forward_equals_composed_entry_points(name):
    """moe_forward (router on float32-staged operands, the gather done inside GEMM-1's loads, MXFP8
    tokens quantised once) gives bitwise the y, logits and schedule of the separate entry points
    moe_route -> moe_permute -> moe_expert_ffn (+ shared expert) -> moe_combine."""
    G = require_gpu()
    base = I.get(name)
    wl = I.scaled(base, **SCALED[name]) if SCALED[name] else base
    note(f"forward vs composed {wl.describe()}")
    inp = I.make_inputs(wl, seed=3)
    wts = [I.expert_weights(wl, e, seed=3) for e in range(wl.E_loc)]
    weights = tuple(dev_bf16(np.stack([w[i] for w in wts])) for i in range(3))
    shared = None
    if wl.m_shared:
        shared = tuple(dev_bf16(v) for v in I.shared_weights(wl, seed=3))
    sh, y, ws = run_forward(G, wl, inp, weights, shared)
    v = G.moe_forward_views(sh, wl.dtype, ws)

    x = dev_bf16(inp["x"])
    prepared = G.moe_prepare_weights(sh, wl.dtype, *weights)
    if wl.mode == "router":
        logits, idx, gw = G.moe_route(sh, x, dev_bf16(inp["w_router"]),
                                      None if inp["bias"] is None else dev(inp["bias"]))
        assign, gate_w = idx.reshape(-1).contiguous(), gw.reshape(-1).contiguous()
    else:
        assign, gate_w = dev(inp["assign"]), dev(inp["assign_w"])
    o = G.moe_permute(sh, wl.dtype, assign, x)
    out_rows = G.moe_expert_ffn(sh, wl.dtype, o["rows"], o["row_scales"], o["offsets"], prepared)
    shared_out = None
    if shared is not None:
        ssh = G.make_shape(wl.T, wl.h, wl.m_shared, 1, 1, 1)
        sprep = G.moe_prepare_weights(ssh, "bf16", *shared)
        soff = torch.tensor([0, wl.T], dtype=torch.int32, device=x.device)
        shared_out = G.moe_expert_ffn(ssh, "bf16", x, None, soff, sprep)
    y2 = G.moe_combine(sh, out_rows, o["inv"], gate_w, shared_out)
    torch.cuda.synchronize()
    if wl.mode == "router":
        assert np.array_equal(v["logits"].cpu().numpy().view(np.uint32),
                              logits.cpu().numpy().view(np.uint32))
    for key in ("counts", "offsets", "perm", "inv"):
        assert np.array_equal(v[key].cpu().numpy(), o[key].cpu().numpy()), key
    assert np.array_equal(host_bf16_bits(y), host_bf16_bits(y2))


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_dropped_assignments_forward_and_backward(dtype):
    """Assignments whose expert id is outside [0, E_loc) are dropped (the library's documented
    reading): inv = -1, no row, offsets[E_loc] = the number of valid ids, and y, dX and dW equal
    the oracle's layer with those slots ignored. Exercises the schedule, the gather inside GEMM-1,
    the combine, the un-combine, the transposes and the un-permute on a partly filled row buffer."""
    G = require_gpu()
    wl = I.Workload(name="drop", T=160, h=512, m=256, E=384, k=4, E_loc=5, dtype=dtype,
                    mode="share", zipf_s=1.0, backward=True)
    inp = I.make_inputs(wl, seed=9)
    bad = np.zeros(wl.R, bool)
    bad[3::7] = True
    ids = np.array([wl.E_loc, -1, 0x7FFFFFFF, wl.E_loc + 100], np.int32)
    inp["assign"] = np.where(bad, ids[np.arange(wl.R) % 4], inp["assign"]).astype(np.int32)
    note(f"dropped assignments {wl.describe()}: {int(bad.sum())} of {wl.R} dropped")
    wts = [I.expert_weights(wl, e, seed=9) for e in range(wl.E_loc)]
    weights = tuple(dev_bf16(np.stack([w[i] for w in wts])) for i in range(3))
    sh = G.make_shape(wl.T, wl.h, wl.m, wl.E, wl.k, wl.E_loc)
    x = dev_bf16(inp["x"])
    o = G.moe_permute(sh, dtype, dev(inp["assign"]), x)
    counts, offsets, perm, inv = M.schedule(inp["assign"], wl.E_loc, drop=True)
    assert offsets[-1] == wl.R - bad.sum()
    assert np.array_equal(o["counts"].cpu().numpy(), counts)
    assert np.array_equal(o["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(o["perm"].cpu().numpy()[:offsets[-1]], perm)
    assert np.array_equal(o["inv"].cpu().numpy(), inv)
    prepared = G.moe_prepare_weights(sh, dtype, *weights)
    saved = torch.empty(G.moe_saved_bytes(sh, dtype), dtype=torch.uint8, device="cuda")
    y = poisoned((wl.T, wl.h), torch.bfloat16)
    y, _ = G.moe_forward(sh, dtype, x, prepared, assign=dev(inp["assign"]),
                         assign_w=dev(inp["assign_w"]), y=y, saved=saved)
    pbwd = G.moe_prepare_bwd_weights(sh, dtype, *weights)
    dx = poisoned((wl.T, wl.h), torch.bfloat16)
    dx, dw, _ = G.moe_backward(sh, dtype, x, dev_bf16(inp["dy"]), saved, pbwd, dx=dx)
    torch.cuda.synchronize()
    fwd = M.layer_forward(wl, inp, lambda e: wts[e], keep=True)
    tol = MX_TOL if dtype == "mxfp8" else BF16_TOL
    err = normwise_err(host_f64_from_bf16(y), fwd["y"])
    note(f"  y normwise error {err:.3e}")
    assert err <= tol
    dX, dW = M.layer_backward(wl, inp, fwd, lambda e: wts[e])
    err = normwise_err(host_f64_from_bf16(dx), dX)
    note(f"  dX normwise error {err:.3e}")
    assert err <= tol
    for i, nm in enumerate(("dW_gate", "dW_up", "dW_down")):
        ref = np.stack([dW[e][i] for e in range(wl.E_loc)])
        err = normwise_err(dw[i].cpu().numpy().astype(np.float64), ref)
        note(f"  {nm} normwise error {err:.3e}")
        assert err <= tol, nm


def test_undersized_buffers_are_rejected_before_any_launch():
    """The binding refuses a workspace, saved state or prepared-weight buffer smaller than the
    size query for the shape (it would be written past its end), and a router matrix or bias of
    the wrong size, with ValueError and nothing enqueued."""
    G = require_gpu()
    wl = I.scaled(I.get("glm52"), T=64, h=512, m=256, E=16, E_loc=16)
    inp = I.make_inputs(wl, seed=0)
    wts = [I.expert_weights(wl, e) for e in range(wl.E_loc)]
    weights = tuple(dev_bf16(np.stack([w[i] for w in wts])) for i in range(3))
    sh = G.make_shape(wl.T, wl.h, wl.m, wl.E, wl.k, wl.E_loc)
    prepared = G.moe_prepare_weights(sh, wl.dtype, *weights)
    x, wr, b = dev_bf16(inp["x"]), dev_bf16(inp["w_router"]), dev(inp["bias"])
    nws = G.moe_forward_workspace_bytes(sh, wl.dtype)
    small = torch.empty(nws - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="ws"):
        G.moe_forward(sh, wl.dtype, x, prepared, w_router=wr, bias=b, ws=small)
    with pytest.raises(ValueError, match="saved"):
        G.moe_forward(sh, wl.dtype, x, prepared, w_router=wr, bias=b,
                      saved=torch.empty(1024, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError, match="prepared"):
        G.moe_forward(sh, wl.dtype, x, prepared[:-1], w_router=wr, bias=b)
    with pytest.raises(ValueError, match="w_router"):
        G.moe_forward(sh, wl.dtype, x, prepared, w_router=wr[:-1], bias=b)
    with pytest.raises(ValueError, match="bias"):
        G.moe_forward(sh, wl.dtype, x, prepared, w_router=wr, bias=b[:-1])
    with pytest.raises(ValueError, match="ws"):
        G.moe_route(sh, x, wr, b, ws=torch.empty(64, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    y, _ = G.moe_forward(sh, wl.dtype, x, prepared, w_router=wr, bias=b)  # the right sizes run
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()


@pytest.mark.parametrize("name,frac", [("tiny", 0.0), ("qwen397", 0.3), ("kimi", 0.45),
                                       ("glm52", 0.2), ("dsv4pro", 0.3)])
def test_forward_ring_equals_one_forward(name, frac):
    """moe_forward_ring (the tokens streamed through a fixed buffer in minibatches, here a fraction
    of the one-shot workspace: several minibatches and a short last one; frac 0 = a ring that holds
    the smallest minibatch) gives bitwise the y of one moe_forward over all tokens. The DeepSeek-V4-Pro-shaped
    share (k = 6) takes minibatches of an even token count, where its assignment slices stay
    16-byte aligned."""
    G = require_gpu()
    base = I.get(name)
    wl = I.scaled(base, **SCALED[name]) if SCALED[name] else base
    inp = I.make_inputs(wl, seed=2)
    wts = [I.expert_weights(wl, e, seed=2) for e in range(wl.E_loc)]
    weights = tuple(dev_bf16(np.stack([w[i] for w in wts])) for i in range(3))
    shared = tuple(dev_bf16(v) for v in I.shared_weights(wl, seed=2)) if wl.m_shared else None
    sh, y, _ = run_forward(G, wl, inp, weights, shared)
    prepared = G.moe_prepare_weights(sh, wl.dtype, *weights)
    sprep = None
    if shared is not None:
        sprep = G.moe_prepare_weights(G.make_shape(wl.T, wl.h, wl.m_shared, 1, 1, 1), "bf16",
                                      *shared)
    full = G.moe_forward_workspace_bytes(sh, wl.dtype)
    a = 4 // math.gcd(wl.k, 4)  # the smallest minibatch: 16-byte aligned assignment slices
    one = G.moe_forward_workspace_bytes(
        G.make_shape(a, wl.h, wl.m, wl.E, wl.k, wl.E_loc, wl.m_shared), wl.dtype)
    nbytes = max(one, int(full * frac)) // 256 * 256 + 256
    ring = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    kw = {}
    if wl.mode == "router":
        kw["w_router"] = dev_bf16(inp["w_router"])
        kw["bias"] = None if inp["bias"] is None else dev(inp["bias"])
    else:
        kw["assign"] = dev(inp["assign"])
        kw["assign_w"] = dev(inp["assign_w"])
    y2 = poisoned((wl.T, wl.h), torch.bfloat16)
    y2, tmb = G.moe_forward_ring(sh, wl.dtype, dev_bf16(inp["x"]), prepared, ring,
                                 shared_prepared=sprep, y=y2, **kw)
    torch.cuda.synchronize()
    note(f"ring forward {wl.describe()}: {nbytes} bytes, minibatches of {tmb} tokens")
    assert 1 <= tmb < wl.T
    assert np.array_equal(host_bf16_bits(y), host_bf16_bits(y2))


def test_forward_bitwise_under_a_concurrent_busy_kernel():
    """Bitwise determinism regardless of hardware scheduling: the forward of the GLM-5.2-shaped
    layer (scaled) run while a long float32 kernel keeps a second stream of the same priority busy
    (so the workgroups of both share the CUs in whatever order the hardware picks) gives bitwise
    the y, logits and schedule of a run on an idle GPU."""
    G = require_gpu()
    wl = I.scaled(I.get("glm52"), T=1024, h=1024, m=512, E=64, E_loc=64)
    inp = I.make_inputs(wl, seed=11)
    wts = [I.expert_weights(wl, e, seed=11) for e in range(wl.E_loc)]
    weights = tuple(dev_bf16(np.stack([w[i] for w in wts])) for i in range(3))
    sh, y_idle, ws_idle = run_forward(G, wl, inp, weights)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in G.moe_forward_views(sh, wl.dtype, ws_idle).items()
           if v is not None and k in ("logits", "topk_idx", "perm", "inv", "offsets")}
    busy = torch.cuda.Stream()  # default priority, like the current stream
    a = torch.randn(4096, 4096, device="cuda", dtype=torch.float32)
    b = torch.randn(4096, 4096, device="cuda", dtype=torch.float32)
    torch.cuda.synchronize()
    for rep in range(3):
        with torch.cuda.stream(busy):
            c = a
            for _ in range(6):
                c = torch.matmul(c, b) * 1e-3
        y = poisoned((wl.T, wl.h), torch.bfloat16)
        _, y, ws = run_forward(G, wl, inp, weights, y=y)
        torch.cuda.synchronize()
        assert np.array_equal(host_bf16_bits(y), host_bf16_bits(y_idle)), rep
        v = G.moe_forward_views(sh, wl.dtype, ws)
        for k, r in ref.items():
            assert torch.equal(v[k].view(torch.uint8), r.view(torch.uint8)), (rep, k)
        del c
