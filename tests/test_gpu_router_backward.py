"""GPU parity of moe_backward_layer (the expert path plus the gradients through the gate weights
and the router) against the oracle's layer_backward_full: dX (router and expert parts), every
expert's dW, the gate-weight gradients and, for router layers, the router-matrix and bias
gradients, each within 1e-2 (BF16) or 3e-2 (MXFP8) normwise; two runs bitwise identical; an
expert share with a dropped assignment (its gate gradient is exactly 0)."""
import numpy as np
import pytest

import moe_inputs as I
from oracle import moe as M
from tests._gpu_helpers import (BF16_TOL, MX_TOL, dev, dev_bf16, host_f64_from_bf16,
                                normwise_err, note, poisoned, require_gpu, torch)

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_router_bias": dict(name="rb1", T=96, h=256, m=256, E=8, k=2, dtype="bf16",
                             mode="router", bias="normal", bias_var=0.5),
    "mx_router_hotset": dict(name="rb2", T=320, h=512, m=256, E=16, k=4, dtype="mxfp8",
                             mode="router", bias="hotset", hot_frac=0.1),
    "bf16_router_k10": dict(name="rb3", T=80, h=256, m=256, E=64, k=10, dtype="bf16",
                            mode="router", bias="normal", bias_var=0.5),
    "mx_share_drop": dict(name="rb4", T=128, h=512, m=256, E=384, k=6, E_loc=4, dtype="mxfp8",
                          mode="share", zipf_s=1.0),
}


def _run(G, wl, inp, wts):
    sh = G.make_shape(wl.T, wl.h, wl.m, wl.E, wl.k, wl.E_loc)
    weights = tuple(dev_bf16(np.stack([w[i] for w in wts])) for i in range(3))
    prepared = G.moe_prepare_weights(sh, wl.dtype, *weights)
    pbwd = G.moe_prepare_bwd_weights(sh, wl.dtype, *weights)
    saved = torch.empty(G.moe_saved_bytes(sh, wl.dtype), dtype=torch.uint8, device="cuda")
    kw, wr = {}, None
    if wl.mode == "router":
        wr = dev_bf16(inp["w_router"])
        kw["w_router"] = wr
        kw["bias"] = None if inp["bias"] is None else dev(inp["bias"])
    else:
        kw["assign"] = dev(inp["assign"])
        kw["assign_w"] = dev(inp["assign_w"])
    x, dy = dev_bf16(inp["x"]), dev_bf16(inp["dy"])
    G.moe_forward(sh, wl.dtype, x, prepared, saved=saved, **kw)
    outs = []
    for _ in range(2):
        dx = poisoned((wl.T, wl.h), torch.bfloat16)
        dgate = poisoned((wl.R,), torch.float32)
        dwr = poisoned((wl.E, wl.h), torch.float32) if wr is not None else None
        db = poisoned((wl.E,), torch.float32) if wr is not None else None
        dx, dw, dgate, dwr, db, _ = G.moe_backward_layer(sh, wl.dtype, x, dy, saved, pbwd,
                                                         w_router=wr, dx=dx, dgate=dgate,
                                                         dw_router=dwr, dbias=db)
        outs.append([dx, *dw, dgate] + ([dwr, db] if wr is not None else []))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "two runs differ"
    return outs[0]


@pytest.mark.parametrize("case", list(CASES))
def test_backward_layer_parity(case):
    G = require_gpu()
    spec = dict(CASES[case])
    spec.setdefault("E_loc", spec["E"])
    wl = I.Workload(backward=True, **spec)
    inp = I.make_inputs(wl, seed=8)
    if wl.mode == "share":
        inp["assign"][7] = wl.E_loc + 1  # dropped: no row, zero gate gradient
    note(f"layer backward {case}: {wl.describe()}")
    wts = [I.expert_weights(wl, e, seed=8) for e in range(wl.E_loc)]
    got = _run(G, wl, inp, wts)
    fwd = M.layer_forward(wl, inp, lambda e: wts[e], keep=True)
    ref = M.layer_backward_full(wl, inp, fwd, lambda e: wts[e])
    tol = MX_TOL if wl.dtype == "mxfp8" else BF16_TOL
    checks = [("dX", host_f64_from_bf16(got[0]), ref["dX"]),
              ("dgate", got[4].cpu().numpy().astype(np.float64), ref["dgate"].reshape(-1))]
    for i, nm in enumerate(("dW_gate", "dW_up", "dW_down")):
        checks.append((nm, got[1 + i].cpu().numpy().astype(np.float64),
                       np.stack([ref["dW"][e][i] for e in range(wl.E_loc)])))
    if wl.mode == "router":
        checks += [("dW_r", got[5].cpu().numpy().astype(np.float64), ref["dW_r"]),
                   ("db", got[6].cpu().numpy().astype(np.float64), ref["db"])]
    else:
        assert got[4][7].item() == 0.0
    for nm, g, r in checks:
        assert np.isfinite(g).all(), nm
        err = normwise_err(g, r)
        note(f"  {nm} normwise error {err:.3e}")
        assert err <= tol, nm
