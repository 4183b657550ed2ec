"""GPU parity at the full sizes of the four benchmark workloads, through the entry points and launch
shapes bench.py times (moe_forward_profiled without saved state; moe_backward_profiled).

The oracle cannot run a whole router layer of this size in seconds, so it checks what it can
compute one by one, plus properties that hold at any size:
  - routing (router layers): logits bit-exact and top-k indices equal for every token;
  - schedule: counts, offsets, perm and inv equal to the oracle's schedule of the assignments;
  - outputs y against oracle.token_outputs, normwise over the checked tokens, written into a
    NaN-poisoned buffer: every token of the two expert shares; for the two router layers at least
    256 tokens chosen so that every M tile of every expert has a checked row at every tile height
    the grouped GEMMs use (128, 192 and 256 rows), plus each expert's first and last row;
  - the whole y, bitwise, against the separate entry points composed (moe_route, moe_permute,
    moe_expert_ffn, moe_combine), which reach the same MFMAs through a materialised row buffer
    instead of GEMM-1's own gather: this covers every tile of every expert at full size;
  - backward of the GLM-5.2-shaped layer: the training forward (128-row tiles, G and U kept) gives
    bitwise the y of the benchmarked forward (192-row tiles); dX of sampled tokens
    (oracle.token_input_grads) and the weight gradients of a hot and a cold expert
    (oracle.expert_weight_grads)."""
import numpy as np
import pytest

import moe_inputs as I
from oracle import moe as M
from tests._sampling import cover_tokens
from tests._gpu_helpers import (BF16_TOL, MX_TOL, dev, dev_bf16, host_bf16_bits,
                                host_f64_from_bf16, normwise_err, note, poisoned, require_gpu,
                                torch)

pytestmark = pytest.mark.gpu

ORACLE_WORKERS = 8


class DeviceExperts:
    """weights_of(e) for the oracle: expert e's bf16 weights copied from the device on demand."""

    def __init__(self, wg, wu, wd):
        self.t = (wg, wu, wd)

    def __call__(self, e):
        return tuple(host_bf16_bits(t[e]) for t in self.t)


def _setup(G, wl, seed=0):
    dvc = torch.device("cuda:0")
    inp = I.make_inputs(wl, seed=seed)
    wg, wu, wd = I.torch_expert_weights(wl, dvc, seed=seed)
    sh = G.make_shape(wl.T, wl.h, wl.m, wl.E, wl.k, wl.E_loc, wl.m_shared)
    prepared = G.moe_prepare_weights(sh, wl.dtype, wg, wu, wd)
    shared_w = shared_prep = shared_host = None
    if wl.m_shared:
        shared_w = I.torch_shared_weights(wl, dvc, seed=seed)
        ssh = G.make_shape(wl.T, wl.h, wl.m_shared, 1, 1, 1)
        shared_prep = G.moe_prepare_weights(ssh, "bf16", *shared_w)
        shared_host = tuple(host_bf16_bits(t) for t in shared_w)
    kw = {}
    if wl.mode == "router":
        kw["w_router"] = dev_bf16(inp["w_router"])
        kw["bias"] = None if inp["bias"] is None else dev(inp["bias"])
    else:
        kw["assign"] = dev(inp["assign"])
        kw["assign_w"] = dev(inp["assign_w"])
    return dict(inp=inp, w=(wg, wu, wd), sh=sh, prepared=prepared, shared_w=shared_w,
                shared_prep=shared_prep, shared_host=shared_host, kw=kw, x=dev_bf16(inp["x"]))


def _forward(G, wl, s, saved=None):
    ev = G.HipEvents()
    y = poisoned((wl.T, wl.h), torch.bfloat16)
    y, ws = G.moe_forward_profiled(s["sh"], wl.dtype, s["x"], s["prepared"], ev, y=y,
                                   shared_prepared=s["shared_prep"], saved=saved, **s["kw"])
    torch.cuda.synchronize()
    ev.close()
    return y, G.moe_forward_views(s["sh"], wl.dtype, ws)


def _composed(G, wl, s):
    """y of moe_route -> moe_permute -> moe_expert_ffn (+ shared expert) -> moe_combine."""
    sh, x = s["sh"], s["x"]
    if wl.mode == "router":
        _, idx, gw = G.moe_route(sh, x, s["kw"]["w_router"], s["kw"]["bias"])
        assign, gate_w = idx.reshape(-1).contiguous(), gw.reshape(-1).contiguous()
    else:
        assign, gate_w = s["kw"]["assign"], s["kw"]["assign_w"]
    o = G.moe_permute(sh, wl.dtype, assign, x)
    out_rows = G.moe_expert_ffn(sh, wl.dtype, o["rows"], o["row_scales"], o["offsets"],
                                s["prepared"])
    shared_out = None
    if wl.m_shared:
        ssh = G.make_shape(wl.T, wl.h, wl.m_shared, 1, 1, 1)
        soff = torch.tensor([0, wl.T], dtype=torch.int32, device=x.device)
        shared_out = G.moe_expert_ffn(ssh, "bf16", x, None, soff, s["shared_prep"])
    y = G.moe_combine(sh, out_rows, o["inv"], gate_w, shared_out)
    torch.cuda.synchronize()
    return y


def _check_schedule(v, ref_sched):
    counts, offsets, perm, inv = ref_sched
    for key, ref in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        assert np.array_equal(v[key].cpu().numpy(), ref), key


def _check_outputs(wl, s, y, tokens, weights_of, workers):
    from threadpoolctl import threadpool_limits
    note(f"  oracle y of {len(tokens)} tokens ...")
    if workers > 1:
        with threadpool_limits(1):  # one BLAS thread per expert worker
            ref = M.token_outputs(wl, s["inp"], tokens, weights_of, s["shared_host"],
                                  workers=workers)
    else:
        ref = M.token_outputs(wl, s["inp"], tokens, weights_of, s["shared_host"])
    got = host_f64_from_bf16(y)[tokens]
    assert np.isfinite(got).all()
    err = normwise_err(got, ref["y"])
    worst = max(normwise_err(got[i], ref["y"][i]) for i in range(len(tokens)))
    note(f"  y of {len(tokens)} tokens: normwise error {err:.3e} (worst token {worst:.3e})")
    assert err <= (MX_TOL if wl.dtype == "mxfp8" else BF16_TOL)
    return ref


@pytest.mark.parametrize("name", ["dsv4pro", "kimi"])
def test_fullsize_expert_share_every_token(name):
    G = require_gpu()
    wl = I.get(name)
    note(f"full size {wl.describe()}")
    s = _setup(G, wl)
    y, v = _forward(G, wl, s)
    _check_schedule(v, M.schedule(s["inp"]["assign"], wl.E_loc))
    note("  schedule equal to the oracle's")
    _check_outputs(wl, s, y, np.arange(wl.T), DeviceExperts(*s["w"]), workers=1)
    y2 = _composed(G, wl, s)
    assert np.array_equal(host_bf16_bits(y), host_bf16_bits(y2))
    note("  y bitwise equal to the composed entry points")


def test_fullsize_qwen_layer():
    G = require_gpu()
    wl = I.get("qwen397")
    note(f"full size {wl.describe()}")
    s = _setup(G, wl)
    y, v = _forward(G, wl, s)
    note("  oracle routing of all tokens ...")
    lg, idx, w = M.route(s["inp"]["x"], s["inp"]["w_router"], s["inp"]["bias"], wl.k)
    assert np.array_equal(v["logits"].cpu().numpy().view(np.uint32), lg.view(np.uint32))
    assert np.array_equal(v["topk_idx"].cpu().numpy(), idx)
    assert np.allclose(v["topk_w"].cpu().numpy(), w, rtol=1e-6, atol=0)
    note("  routing of every token bit-exact")
    sched = M.schedule(idx.reshape(-1), wl.E_loc)
    _check_schedule(v, sched)
    tokens = cover_tokens(sched[1], sched[2], sched[3], wl.k, 256, seed=11)
    _check_outputs(wl, s, y, tokens, DeviceExperts(*s["w"]), workers=ORACLE_WORKERS)
    y2 = _composed(G, wl, s)
    assert np.array_equal(host_bf16_bits(y), host_bf16_bits(y2))
    note("  y bitwise equal to the composed entry points")


def test_fullsize_glm_layer_forward():
    """The benchmarked GLM-5.2-shaped forward: 192-row MXFP8 tiles, no saved state."""
    G = require_gpu()
    wl = I.get("glm52")
    note(f"full size {wl.describe()} (forward as benchmarked)")
    s = _setup(G, wl)
    y, v = _forward(G, wl, s)
    note("  oracle routing of all tokens ...")
    lg, idx, w = M.route(s["inp"]["x"], s["inp"]["w_router"], s["inp"]["bias"], wl.k)
    assert np.array_equal(v["logits"].cpu().numpy().view(np.uint32), lg.view(np.uint32))
    assert np.array_equal(v["topk_idx"].cpu().numpy(), idx)
    assert np.allclose(v["topk_w"].cpu().numpy(), w, rtol=1e-6, atol=0)
    note("  routing of every token bit-exact")
    sched = M.schedule(idx.reshape(-1), wl.E_loc)
    _check_schedule(v, sched)
    tokens = cover_tokens(sched[1], sched[2], sched[3], wl.k, 256, seed=12)
    _check_outputs(wl, s, y, tokens, DeviceExperts(*s["w"]), workers=ORACLE_WORKERS)
    y2 = _composed(G, wl, s)
    assert np.array_equal(host_bf16_bits(y), host_bf16_bits(y2))
    note("  y bitwise equal to the composed entry points")


def test_fullsize_glm_layer_backward():
    G = require_gpu()
    wl = I.get("glm52")
    note(f"full size {wl.describe()} (training forward with saved state, then backward)")
    s = _setup(G, wl)
    y_bench, _ = _forward(G, wl, s)
    saved = torch.empty(G.moe_saved_bytes(s["sh"], wl.dtype), dtype=torch.uint8, device="cuda")
    y, v = _forward(G, wl, s, saved=saved)
    assert np.array_equal(host_bf16_bits(y), host_bf16_bits(y_bench))
    note("  training forward y bitwise equal to the benchmarked forward's")
    pbwd = G.moe_prepare_bwd_weights(s["sh"], wl.dtype, *s["w"])
    ev = G.HipEvents(G.MOE_BWD_PROFILE_EVENTS, G.BWD_STAGES)
    dx = poisoned((wl.T, wl.h), torch.bfloat16)
    dx, dw, _ = G.moe_backward_profiled(s["sh"], wl.dtype, s["x"], dev_bf16(s["inp"]["dy"]), saved,
                                        pbwd, ev, dx=dx)
    torch.cuda.synchronize()
    ev.close()
    assert torch.isfinite(dx).all()
    idx = v["topk_idx"].cpu().numpy()
    w = v["topk_w"].cpu().numpy().astype(np.float64)
    counts = v["counts"].cpu().numpy()
    experts = DeviceExperts(*s["w"])
    tok = [4099, 17]
    note(f"  dX of tokens {tok} ...")
    ref_dx = M.token_input_grads(wl, s["inp"], tok, experts)
    err = normwise_err(host_f64_from_bf16(dx)[tok], ref_dx)
    note(f"  dX normwise error {err:.3e}")
    assert err <= MX_TOL
    hot = int(np.argmax(counts))
    cold = int(np.argmin(np.where(counts > 0, counts, counts.max() + 1)))
    for e in (hot, cold):
        note(f"  weight gradients of expert {e} ({counts[e]} rows) ...")
        ref = M.expert_weight_grads(wl, s["inp"], idx.reshape(-1), w.reshape(-1), e, experts)
        for i, nm in enumerate(("dW_gate", "dW_up", "dW_down")):
            g = dw[i][e].float().cpu().numpy().astype(np.float64)
            err = normwise_err(g, ref[i])
            note(f"    {nm}[{e}] normwise error {err:.3e}")
            assert np.isfinite(g).all() and err <= MX_TOL, nm
