"""GPU parity at the full sizes of the four benchmark workloads, through the entry points and launch
shapes bench.py times (moe_forward_profiled, moe_backward_profiled).

The oracle cannot run a whole layer of this size in seconds, so it checks what it can compute one
by one, plus properties that hold at any size:
  - routing (router layers): logits bit-exact and top-k indices equal on sampled tokens (every
    token for the GLM-5.2-shaped layer, whose weight gradients need every token's experts);
  - schedule: counts, offsets, perm and inv exactly those of a stable counting sort of the
    assignments (the oracle's schedule of the given assignments for expert shares; for router
    layers the properties that make the stable sort unique: counts equal the histogram, rows of
    each expert hold its assignments in ascending order, inv inverts perm);
  - outputs y of sampled tokens (oracle.token_outputs), normwise over those rows;
  - backward of the GLM-5.2-shaped layer: dX of a sampled token (oracle.token_input_grads) and the
    weight gradients of a hot and a cold expert (oracle.expert_weight_grads).
Each test takes up to a minute or two, mostly oracle time on the host."""
import numpy as np
import pytest

import moe_inputs as I
from oracle import moe as M
from tests._gpu_helpers import (BF16_TOL, MX_TOL, dev, dev_bf16, host_bf16_bits,
                                host_f64_from_bf16, normwise_err, note, require_gpu, torch)

pytestmark = pytest.mark.gpu


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
    shared_prep = shared_host = None
    if wl.m_shared:
        sw = I.torch_shared_weights(wl, dvc, seed=seed)
        ssh = G.make_shape(wl.T, wl.h, wl.m_shared, 1, 1, 1)
        shared_prep = G.moe_prepare_weights(ssh, "bf16", *sw)
        shared_host = tuple(host_bf16_bits(t) for t in sw)
    kw = {}
    if wl.mode == "router":
        kw["w_router"] = dev_bf16(inp["w_router"])
        kw["bias"] = None if inp["bias"] is None else dev(inp["bias"])
    else:
        kw["assign"] = dev(inp["assign"])
        kw["assign_w"] = dev(inp["assign_w"])
    return dict(inp=inp, w=(wg, wu, wd), sh=sh, prepared=prepared, shared_prep=shared_prep,
                shared_host=shared_host, kw=kw, x=dev_bf16(inp["x"]))


def _forward(G, wl, s, saved=None):
    ev = G.HipEvents()
    y, ws = G.moe_forward_profiled(s["sh"], wl.dtype, s["x"], s["prepared"], ev,
                                   shared_prepared=s["shared_prep"], saved=saved, **s["kw"])
    torch.cuda.synchronize()
    ev.close()
    return y, G.moe_forward_views(s["sh"], wl.dtype, ws)


def _check_schedule(wl, v, assign):
    counts = v["counts"].cpu().numpy()
    offsets = v["offsets"].cpu().numpy()
    perm = v["perm"].cpu().numpy()
    inv = v["inv"].cpu().numpy()
    R = wl.T * wl.k
    assert np.array_equal(counts, np.bincount(assign, minlength=wl.E_loc))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts) and offsets[-1] == R
    assert np.array_equal(np.sort(perm), np.arange(R))
    assert np.array_equal(inv[perm], np.arange(R))
    for e in range(wl.E_loc):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(assign[seg] == e) and np.all(np.diff(seg) > 0), e


def _check_outputs(wl, s, y, tokens, weights_of):
    ref = M.token_outputs(wl, s["inp"], tokens, weights_of, s["shared_host"])
    got = host_f64_from_bf16(y)[tokens]
    err = normwise_err(got, ref["y"])
    note(f"  y on tokens {list(tokens)}: normwise error {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= (MX_TOL if wl.dtype == "mxfp8" else BF16_TOL)
    return ref


@pytest.mark.parametrize("name", ["dsv4pro", "kimi"])
def test_fullsize_expert_share(name):
    G = require_gpu()
    wl = I.get(name)
    note(f"full size {wl.describe()}")
    s = _setup(G, wl)
    y, v = _forward(G, wl, s)
    # the schedule is the oracle's for the given assignments, element for element
    counts, offsets, perm, inv = M.schedule(s["inp"]["assign"], wl.E_loc)
    for key, ref in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        assert np.array_equal(v[key].cpu().numpy(), ref), key
    note("  schedule equal to the oracle's")
    _check_outputs(wl, s, y, [0, 1027, wl.T - 1], DeviceExperts(*s["w"]))


def test_fullsize_qwen_layer():
    G = require_gpu()
    wl = I.get("qwen397")
    note(f"full size {wl.describe()}")
    s = _setup(G, wl)
    y, v = _forward(G, wl, s)
    rng = np.random.default_rng(11)
    sample = np.sort(rng.choice(wl.T, 64, replace=False))
    lg, idx, w = M.route(s["inp"]["x"][sample], s["inp"]["w_router"], s["inp"]["bias"], wl.k)
    assert np.array_equal(v["logits"].cpu().numpy()[sample].view(np.uint32), lg.view(np.uint32))
    assert np.array_equal(v["topk_idx"].cpu().numpy()[sample], idx)
    assert np.allclose(v["topk_w"].cpu().numpy()[sample], w, rtol=1e-6, atol=0)
    note("  routing of 64 sampled tokens bit-exact")
    _check_schedule(wl, v, v["topk_idx"].cpu().numpy().reshape(-1))
    note("  schedule is the stable counting sort of the routing")
    _check_outputs(wl, s, y, [0, 2222, wl.T - 1], DeviceExperts(*s["w"]))


def test_fullsize_glm_layer_forward_and_backward():
    G = require_gpu()
    wl = I.get("glm52")
    note(f"full size {wl.describe()} (forward with saved state, then backward)")
    s = _setup(G, wl)
    saved = torch.empty(G.moe_saved_bytes(s["sh"], wl.dtype), dtype=torch.uint8, device="cuda")
    y, v = _forward(G, wl, s, saved=saved)
    pbwd = G.moe_prepare_bwd_weights(s["sh"], wl.dtype, *s["w"])
    ev = G.HipEvents(G.MOE_BWD_PROFILE_EVENTS, G.BWD_STAGES)
    dx, dw, _ = G.moe_backward_profiled(s["sh"], wl.dtype, s["x"], dev_bf16(s["inp"]["dy"]), saved,
                                        pbwd, ev)
    torch.cuda.synchronize()
    ev.close()
    note("  oracle routing of all tokens ...")
    lg, idx, w = M.route(s["inp"]["x"], s["inp"]["w_router"], s["inp"]["bias"], wl.k)
    assert np.array_equal(v["logits"].cpu().numpy().view(np.uint32), lg.view(np.uint32))
    assert np.array_equal(v["topk_idx"].cpu().numpy(), idx)
    note("  routing of every token bit-exact")
    counts, offsets, perm, inv = M.schedule(idx.reshape(-1), wl.E_loc)
    for key, ref in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        assert np.array_equal(v[key].cpu().numpy(), ref), key
    experts = DeviceExperts(*s["w"])
    tok = [4099]
    _check_outputs(wl, s, y, tok, experts)
    note("  dX of the sampled token ...")
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
