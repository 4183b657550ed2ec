"""Pins of the oracle's experts, combine and whole layer, plus its backward.

Textbook special cases: E = k = 1 is a dense SwiGLU FFN; W_gate = 0 gives exactly 0; k = E is
the dense softmax-weighted mixture with no permutation at all; identity experts make the combine
the gate-weighted sum of the token (spec identity-expert check); MX operands that are
already representable leave the first GEMM unchanged. The backward is pinned by central finite
differences.
"""
import numpy as np
import pytest
import scipy.special

import moe_inputs as I
from oracle import formats as F
from oracle import moe as M


def _dense_swiglu(x, wg, wu, wd):
    g = x @ wg
    return (g * scipy.special.expit(g) * (x @ wu)) @ wd


def _wl(**kw):
    base = dict(name="t", T=24, h=64, m=32, E=4, k=2, E_loc=4, dtype="bf16", mode="router")
    base.update(kw)
    return I.Workload(**base)


def test_single_expert_is_dense_swiglu():
    wl = _wl(E=1, E_loc=1, k=1)
    inp = I.make_inputs(wl, seed=3)
    wts = I.expert_weights(wl, 0, seed=3)
    out = M.layer_forward(wl, inp, lambda e: wts)
    x = F.bf16_to_f64(inp["x"])
    ref = _dense_swiglu(x, *(F.bf16_to_f64(w) for w in wts))
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12)
    assert np.all(out["w"] == 1.0)


def test_zero_gate_weights_give_zero():
    wl = _wl()
    inp = I.make_inputs(wl, seed=1)

    def wts(e):
        wg, wu, wd = I.expert_weights(wl, e, seed=1)
        return np.zeros_like(wg), wu, wd

    assert np.all(M.layer_forward(wl, inp, wts)["y"] == 0.0)


@pytest.mark.parametrize("mx", [False, True])
def test_k_equals_E_is_dense_mixture(mx):
    wl = _wl(E=5, E_loc=5, k=5, dtype="mxfp8" if mx else "bf16", h=64, m=64)
    inp = I.make_inputs(wl, seed=2)
    cache = {e: I.expert_weights(wl, e, seed=2) for e in range(5)}
    out = M.layer_forward(wl, inp, cache.__getitem__)
    x = F.bf16_to_f64(inp["x"])
    p = scipy.special.softmax(out["logits"].astype(np.float64), axis=1)
    ref = np.zeros_like(x)
    for e in range(5):
        wg, wu, wd = (F.bf16_to_f64(w) for w in cache[e])
        if mx:
            o = M.swiglu_ffn(x, wg, wu, wd, mx=True)  # per-row quantisation: row order is free
        else:
            o = _dense_swiglu(x, wg, wu, wd)
        ref += p[:, e:e + 1] * o
    assert np.allclose(out["y"], ref, rtol=1e-11, atol=1e-12)


def test_identity_experts_combine_is_weighted_token_sum(rng):
    wl = _wl(T=30, E=6, E_loc=6, k=3)
    inp = I.make_inputs(wl, seed=4)
    logits, idx, w = M.route(inp["x"], inp["w_router"], None, wl.k)
    counts, offsets, perm, inv = M.schedule(idx.reshape(-1), wl.E)
    x = F.bf16_to_f64(inp["x"])
    A = M.gather_rows(x, perm, wl.k)  # identity experts: O = A
    y = M.combine(A, inv, w.reshape(-1), wl.k)
    assert np.allclose(y, x * w.sum(axis=1, keepdims=True), rtol=1e-14, atol=0)
    assert np.allclose(y, x, rtol=1e-14, atol=1e-15)
    # k = 1: the output is the row itself
    counts, offsets, perm, inv = M.schedule(idx[:, 0], wl.E)
    A1 = M.gather_rows(x, perm, 1)
    assert np.array_equal(M.combine(A1, inv, np.ones(wl.T), 1), x)


def test_share_workload_assignments_and_shared_expert():
    wl = I.scaled(I.get("kimi"), T=32, h=64, m=32, m_shared=32)
    inp = I.make_inputs(wl, seed=0)
    cache = {e: I.expert_weights(wl, e) for e in range(wl.E_loc)}
    sh = I.shared_weights(wl)
    out = M.layer_forward(wl, inp, cache.__getitem__, shared_weights=sh)
    x = F.bf16_to_f64(inp["x"])
    ref = M.swiglu_ffn(x, *(F.bf16_to_f64(v) for v in sh))
    a = inp["assign"].reshape(wl.T, wl.k)
    wts = inp["assign_w"].reshape(wl.T, wl.k).astype(np.float64)
    for t in range(wl.T):
        for j in range(wl.k):
            wg, wu, wd = (F.bf16_to_f64(v) for v in cache[int(a[t, j])])
            ref[t] += wts[t, j] * M.swiglu_ffn(x[t:t + 1], wg, wu, wd, mx=True)[0]
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12)
    tok = M.token_outputs(wl, inp, [0, 5, 31], cache.__getitem__, sh)
    assert np.allclose(tok["y"], out["y"][[0, 5, 31]], rtol=1e-12, atol=1e-12)


def test_token_outputs_match_layer_router():
    wl = _wl(T=20, E=8, E_loc=8, k=3, h=64, m=64, dtype="mxfp8", bias="normal", bias_var=0.5)
    inp = I.make_inputs(wl, seed=5)
    cache = {e: I.expert_weights(wl, e, seed=5) for e in range(8)}
    out = M.layer_forward(wl, inp, cache.__getitem__)
    tok = M.token_outputs(wl, inp, [1, 19], cache.__getitem__)
    assert np.array_equal(tok["idx"], out["idx"][[1, 19]])
    assert np.allclose(tok["y"], out["y"][[1, 19]], rtol=1e-12, atol=1e-12)


def test_mx_ffn_quantises_along_each_reduction_axis(rng):
    # operands built exactly representable along the reduction axis: a along h (axis 1), W_gate
    # and W_up along h (axis 0), W_down along m (axis 0). The first GEMM is then unchanged by
    # quantisation, and the only effect left is the requantisation of H along m.
    n, h, m = 8, 64, 64
    grid = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))

    def rep(shape, axis):
        c = rng.choice(grid, size=shape) * rng.choice([-1.0, 1.0], size=shape)
        c = np.moveaxis(c, axis, -1)
        c[..., ::32] = 320.0  # an E4M3 value in the top binade; pins each block's scale to 2**0 before the 2**-8 shift
        return np.moveaxis(c, -1, axis) * 2.0 ** -8

    a, wg, wu, wd = rep((n, h), 1), rep((h, m), 0), rep((h, m), 0), rep((m, h), 0)
    o, kept = M.swiglu_ffn(a, wg, wu, wd, mx=True, keep=True)
    assert np.array_equal(kept["G"], a @ wg) and np.array_equal(kept["U"], a @ wu)
    hq = kept["Hq"]
    assert not np.array_equal(hq, kept["H"])
    # each 32-wide block of a row of H shares one power-of-two scale (blocks run along m)
    for r in range(n):
        for b in range(m // 32):
            blk = kept["H"][r, 32 * b:32 * b + 32]
            s = np.floor(np.log2(np.abs(blk).max())) - 8
            assert np.allclose(hq[r, 32 * b:32 * b + 32], F.mx_roundtrip(blk)), (r, b)
            assert np.all(np.abs(hq[r, 32 * b:32 * b + 32] / 2.0 ** s) <= 448)
    assert np.array_equal(o, hq @ wd)


def test_backward_vs_finite_differences():
    wl = _wl(T=6, E=3, E_loc=3, k=2, h=32, m=16, backward=True)
    inp = I.make_inputs(wl, seed=7)
    cache = {e: I.expert_weights(wl, e, seed=7) for e in range(3)}
    fwd = M.layer_forward(wl, inp, cache.__getitem__, keep=True)
    dy = np.random.default_rng(1).standard_normal((wl.T, wl.h))
    dX, dW = M.layer_backward(wl, inp, fwd, cache.__getitem__, dy_f64=dy)
    x0 = F.bf16_to_f64(inp["x"])
    w_fixed = fwd["w"].reshape(-1)
    wts = {e: [F.bf16_to_f64(v) for v in cache[e]] for e in range(3)}

    def loss(x, wmod=None):
        A = M.gather_rows(x, fwd["perm"], wl.k)
        O = np.zeros_like(A)
        for e in range(3):
            r0, r1 = fwd["offsets"][e], fwd["offsets"][e + 1]
            ws = wmod(e) if wmod else wts[e]
            O[r0:r1] = M.swiglu_ffn(A[r0:r1], *ws)
        return float(np.sum(M.combine(O, fwd["inv"], w_fixed, wl.k) * dy))

    eps = 1e-6
    for (t, i) in [(0, 0), (3, 17), (5, 31)]:
        xp, xm = x0.copy(), x0.copy()
        xp[t, i] += eps
        xm[t, i] -= eps
        fd = (loss(xp) - loss(xm)) / (2 * eps)
        assert abs(fd - dX[t, i]) <= 1e-6 * max(1.0, abs(fd))
    for e, which, (p, q) in [(0, 0, (3, 5)), (1, 1, (10, 2)), (2, 2, (7, 30))]:
        def wmod_factory(delta):
            def wmod(ee):
                ws = [w.copy() for w in wts[ee]]
                if ee == e:
                    ws[which][p, q] += delta
                return ws
            return wmod
        fd = (loss(x0, wmod_factory(eps)) - loss(x0, wmod_factory(-eps))) / (2 * eps)
        assert abs(fd - dW[e][which][p, q]) <= 1e-6 * max(1.0, abs(fd)), (e, which)


def test_dropped_assignments_contribute_nothing():
    """Reading: assignments with an expert id outside [0, E_loc) are dropped. The layer then equals
    the same layer with those slots sent to a valid expert at gate weight 0 (0 * O = 0), and the
    sampled-token path agrees with the whole layer (also with a thread pool over experts)."""
    wl = I.scaled(I.get("dsv4pro"), T=40, h=64, m=64, name="drop")
    inp = I.make_inputs(wl, seed=4)
    wts = [I.expert_weights(wl, e, seed=4) for e in range(wl.E_loc)]
    bad = np.zeros(wl.R, bool)
    bad[::5] = True
    dropped = dict(inp)
    dropped["assign"] = np.where(bad, np.int32(wl.E_loc + 2), inp["assign"]).astype(np.int32)
    zeroed = dict(inp)
    zeroed["assign_w"] = np.where(bad, np.float32(0.0), inp["assign_w"]).astype(np.float32)
    a = M.layer_forward(wl, dropped, lambda e: wts[e])
    b = M.layer_forward(wl, zeroed, lambda e: wts[e])
    assert np.array_equal(a["y"], b["y"])
    assert a["offsets"][-1] == wl.R - bad.sum() and np.all(a["inv"][bad] == -1)
    toks = np.arange(wl.T)
    t1 = M.token_outputs(wl, dropped, toks, lambda e: wts[e])
    t4 = M.token_outputs(wl, dropped, toks, lambda e: wts[e], workers=4)
    assert np.array_equal(t1["y"], t4["y"])
    assert np.allclose(t1["y"], a["y"], rtol=1e-12, atol=1e-12)
