"""GPU parity of the expert-path backward (moe_forward with `saved`, then moe_backward) against the
oracle's layer_backward: dX and every expert's dW_gate, dW_up, dW_down within 1e-2 (BF16) or
3e-2 (MXFP8) normwise, on router layers and expert shares with ragged, empty and multi-tile
experts; two backward runs bitwise identical; float32 and bf16 weight-gradient outputs."""
import numpy as np
import pytest

import moe_inputs as I
from oracle import moe as M
from tests._gpu_helpers import (BF16_TOL, MX_TOL, dev, dev_bf16, host_f64_from_bf16,
                                normwise_err, note, poisoned, require_gpu, torch)

pytestmark = pytest.mark.gpu

PER_EXPERT_BOUND = 3e-2  # the MXFP8 bar, per expert as well as over the whole tensor

CASES = {
    # router layers
    "bf16_router": dict(name="b1", T=64, h=256, m=256, E=4, k=2, dtype="bf16", mode="router"),
    "mx_router": dict(name="b2", T=128, h=512, m=256, E=8, k=2, dtype="mxfp8", mode="router"),
    # a GLM-5.2-shaped layer scaled down: hot-set bias, several experts of 300+ rows
    "mx_hotset": dict(name="b3", T=320, h=512, m=256, E=16, k=4, dtype="mxfp8", mode="router",
                      bias="hotset", hot_frac=0.1),
    # expert shares (Zipf assignments, a token may hold one expert twice)
    "bf16_share": dict(name="b4", T=96, h=256, m=256, E=384, k=6, E_loc=6, dtype="bf16",
                       mode="share", zipf_s=1.0),
    "mx_share_big": dict(name="b5", T=256, h=512, m=512, E=384, k=8, E_loc=3, dtype="mxfp8",
                         mode="share", zipf_s=1.2),
    # experts of 600+ rows: several 256-row tiles and K stages on every GEMM
    "bf16_big_rows": dict(name="b6", T=512, h=512, m=256, E=3, k=3, dtype="bf16", mode="router"),
}


def _workload(spec):
    spec = dict(spec)
    spec.setdefault("E_loc", spec["E"])
    return I.Workload(backward=True, **spec)


def _run(G, wl, inp, wts, dw_fp32=True, repeat=False):
    sh = G.make_shape(wl.T, wl.h, wl.m, wl.E, wl.k, wl.E_loc)
    weights = tuple(dev_bf16(np.stack([w[i] for w in wts])) for i in range(3))
    prepared = G.moe_prepare_weights(sh, wl.dtype, *weights)
    pbwd = G.moe_prepare_bwd_weights(sh, wl.dtype, *weights)
    saved = torch.empty(G.moe_saved_bytes(sh, wl.dtype), dtype=torch.uint8, device="cuda")
    kw = {}
    if wl.mode == "router":
        kw["w_router"] = dev_bf16(inp["w_router"])
        kw["bias"] = None if inp["bias"] is None else dev(inp["bias"])
    else:
        kw["assign"] = dev(inp["assign"])
        kw["assign_w"] = dev(inp["assign_w"])
    x = dev_bf16(inp["x"])
    dy = dev_bf16(inp["dy"])
    G.moe_forward(sh, wl.dtype, x, prepared, saved=saved, **kw)
    wdt = torch.float32 if dw_fp32 else torch.bfloat16
    dw = (poisoned((wl.E_loc, wl.h, wl.m), wdt), poisoned((wl.E_loc, wl.h, wl.m), wdt),
          poisoned((wl.E_loc, wl.m, wl.h), wdt))
    dx = poisoned((wl.T, wl.h), torch.bfloat16)
    dx, dw, ws = G.moe_backward(sh, wl.dtype, x, dy, saved, pbwd, dx=dx, dw=dw, dw_fp32=dw_fp32)
    out = [dx.clone()] + [t.clone() for t in dw]
    if repeat:
        dx2, dw2, _ = G.moe_backward(sh, wl.dtype, x, dy, saved, pbwd, dw_fp32=dw_fp32, ws=ws)
        out2 = [dx2] + list(dw2)
        torch.cuda.synchronize()
        for a, b in zip(out, out2):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "two runs differ"
    torch.cuda.synchronize()
    return out


def _check(wl, inp, wts, got):
    fwd = M.layer_forward(wl, inp, lambda e: wts[e], keep=True)
    dX, dW = M.layer_backward(wl, inp, fwd, lambda e: wts[e])
    tol = MX_TOL if wl.dtype == "mxfp8" else BF16_TOL
    gx = host_f64_from_bf16(got[0])
    assert np.isfinite(gx).all()
    err = normwise_err(gx, dX)
    note(f"  dX normwise error {err:.3e}")
    assert err <= tol
    counts = np.diff(fwd["offsets"])
    for i, name in enumerate(("dW_gate", "dW_up", "dW_down")):
        g = got[1 + i].float().cpu().numpy().astype(np.float64)
        assert np.isfinite(g).all(), name
        ref = np.stack([dW[e][i] for e in range(wl.E_loc)])
        err = normwise_err(g, ref)
        worst = 0.0
        for e in range(wl.E_loc):
            if counts[e] == 0:
                assert not g[e].any(), f"{name}[{e}] of an empty expert is not zero"
            else:
                worst = max(worst, normwise_err(g[e], ref[e]))
        note(f"  {name} normwise error {err:.3e} (worst expert {worst:.3e})")
        # every expert on its own within the MXFP8 bar too (a wrong segment or layout gives ~1)
        assert err <= tol and worst <= PER_EXPERT_BOUND, name


@pytest.mark.parametrize("case", list(CASES))
def test_backward_parity(case):
    G = require_gpu()
    wl = _workload(CASES[case])
    note(f"backward {case}: {wl.describe()}")
    inp = I.make_inputs(wl, seed=5)
    wts = [I.expert_weights(wl, e, seed=5) for e in range(wl.E_loc)]
    got = _run(G, wl, inp, wts, repeat=True)
    _check(wl, inp, wts, got)


def test_backward_bf16_weight_gradients_and_empty_expert():
    """bf16 weight-gradient outputs, and an expert that receives no rows (all zeros)."""
    G = require_gpu()
    wl = _workload(dict(name="b7", T=64, h=256, m=256, E=384, k=2, E_loc=4, dtype="mxfp8",
                        mode="share", zipf_s=1.0))
    inp = I.make_inputs(wl, seed=6)
    inp["assign"] = np.where(inp["assign"] == 2, 1, inp["assign"]).astype(np.int32)  # empty expert 2
    note(f"backward bf16 dW, empty expert: {wl.describe()}")
    wts = [I.expert_weights(wl, e, seed=6) for e in range(wl.E_loc)]
    got = _run(G, wl, inp, wts, dw_fp32=False)
    _check(wl, inp, wts, got)
