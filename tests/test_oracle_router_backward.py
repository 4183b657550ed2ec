"""Pins of the oracle's backward through the gate weights and the router (gate_grads,
selected_logit_grads, router_backward, layer_backward_full): central finite differences of the
scalar L = <dY, y> of a float64 layer (router logits in float64, no quantisation), with respect to
the router matrix, the bias, the input x (router and expert paths together) and, for an expert
share, the gate weights; plus the closed forms that selection carries no gradient and that the
logit gradients of a token sum to zero (softmax shift invariance)."""
import numpy as np

import moe_inputs as I
from oracle import formats as F
from oracle import moe as M


def _wl(**kw):
    base = dict(name="rb", T=7, h=32, m=16, E=6, k=2, E_loc=6, dtype="bf16", mode="router",
                bias="normal", bias_var=0.5, backward=True)
    base.update(kw)
    return I.Workload(**base)


def _forward_f64(wl, x, wr, b, wts, assign=None, assign_w=None):
    """The layer in float64 throughout (logits included): y and its pieces."""
    if wl.mode == "router":
        l = x @ wr.T + (0.0 if b is None else b)[None, :]
        idx = M.topk(l, wl.k)
        w = M.topk_weights(l, idx)
        a = idx.reshape(-1)
    else:
        l, idx, w = None, assign.reshape(-1, wl.k), assign_w.reshape(-1, wl.k)
        a = assign
    counts, offsets, perm, inv = M.schedule(a, wl.E_loc)
    A = M.gather_rows(x, perm, wl.k)
    O = np.zeros_like(A)
    for e in range(wl.E_loc):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            O[r0:r1] = M.swiglu_ffn(A[r0:r1], *wts[e])
    y = M.combine(O, inv, w.reshape(-1), wl.k)
    return dict(l=l, idx=idx, w=w, perm=perm, inv=inv, offsets=offsets, O=O, y=y, A=A)


def test_router_gradients_vs_finite_differences():
    wl = _wl()
    inp = I.make_inputs(wl, seed=3)
    cache = {e: I.expert_weights(wl, e, seed=3) for e in range(wl.E)}
    wts = {e: [F.bf16_to_f64(v) for v in cache[e]] for e in range(wl.E)}
    x0, wr0 = F.bf16_to_f64(inp["x"]), F.bf16_to_f64(inp["w_router"])
    b0 = inp["bias"].astype(np.float64)
    dy = np.random.default_rng(2).standard_normal((wl.T, wl.h))
    f = _forward_f64(wl, x0, wr0, b0, wts)
    srt = -np.sort(-f["l"], axis=1)
    assert (srt[:, wl.k - 1] - srt[:, wl.k]).min() > 1e-4  # no selection change under +-eps

    # gradients at the base point (the oracle's functions, logits from the same float64 values)
    dgate = M.gate_grads(dy, f["O"], f["inv"], wl.k)
    dl = M.selected_logit_grads(f["w"], dgate)
    dWr, db, dXr, dlogits = M.router_backward(inp["x"], inp["w_router"], f["idx"], dl)
    fwd = dict(perm=f["perm"], inv=f["inv"], offsets=f["offsets"], w=f["w"], A=f["A"])
    dXe, _ = M.layer_backward(wl, inp, fwd, cache.__getitem__, dy_f64=dy, mx=False)

    def loss(x=x0, wr=wr0, b=b0):
        g = _forward_f64(wl, x, wr, b, wts)
        assert np.array_equal(g["idx"], f["idx"])
        return float(np.sum(g["y"] * dy))

    eps = 1e-6

    def fd(**kw):
        name, (arr, pos) = next(iter(kw.items()))
        p, m = arr.copy(), arr.copy()
        p[pos] += eps
        m[pos] -= eps
        return (loss(**{name: p}) - loss(**{name: m})) / (2 * eps)

    sel = set(f["idx"].reshape(-1).tolist())
    unused = [e for e in range(wl.E) if e not in sel]
    for e, i in [(int(f["idx"][0, 0]), 3), (int(f["idx"][4, 1]), 30)] + [(e, 5) for e in unused]:
        g = fd(wr=(wr0, (e, i)))
        assert abs(g - dWr[e, i]) <= 1e-6 * max(1.0, abs(g)), (e, i)
    for e in range(wl.E):
        g = fd(b=(b0, (e,)))
        assert abs(g - db[e]) <= 1e-6 * max(1.0, abs(g)), e
    for t, i in [(0, 0), (3, 17), (6, 31)]:
        g = fd(x=(x0, (t, i)))
        tot = dXe[t, i] + dXr[t, i]
        assert abs(g - tot) <= 1e-6 * max(1.0, abs(g)), (t, i)
    for e in unused:  # an expert no token selected gets no router gradient at all
        assert not dWr[e].any() and db[e] == 0.0
    # softmax over the selected logits is shift invariant: each token's logit gradients sum to 0
    assert np.allclose(dl.sum(axis=1), 0.0, atol=1e-12 * np.abs(dl).max())
    assert np.allclose(dlogits.sum(axis=1), 0.0, atol=1e-12 * np.abs(dl).max())

    # the assembled function gives the same pieces
    full = M.layer_backward_full(wl, inp, dict(fwd, O=f["O"], idx=f["idx"]), cache.__getitem__,
                                 dy_f64=dy, mx=False)
    assert np.allclose(full["dW_r"], dWr, rtol=0, atol=0)
    assert np.allclose(full["dX"], dXe + dXr, rtol=0, atol=0)


def test_gate_weight_gradients_of_a_share_vs_finite_differences():
    wl = _wl(mode="share", E=384, E_loc=3, k=3, zipf_s=1.0, bias="none", bias_var=0.0)
    inp = I.make_inputs(wl, seed=4)
    inp["assign"][5] = 7  # a dropped assignment: no row, gradient 0
    cache = {e: I.expert_weights(wl, e, seed=4) for e in range(wl.E_loc)}
    wts = {e: [F.bf16_to_f64(v) for v in cache[e]] for e in range(wl.E_loc)}
    x0 = F.bf16_to_f64(inp["x"])
    dy = np.random.default_rng(5).standard_normal((wl.T, wl.h))
    w0 = inp["assign_w"].astype(np.float64)

    def fwd(w):
        a = inp["assign"]
        counts, offsets, perm, inv = M.schedule(a, wl.E_loc, drop=True)
        A = M.gather_rows(x0, perm, wl.k)
        O = np.zeros_like(A)
        for e in range(wl.E_loc):
            O[offsets[e]:offsets[e + 1]] = M.swiglu_ffn(A[offsets[e]:offsets[e + 1]], *wts[e])
        return O, inv, M.combine(O, inv, w, wl.k)

    O, inv, _ = fwd(w0)
    dgate = M.gate_grads(dy, O, inv, wl.k).reshape(-1)
    assert dgate[5] == 0.0
    eps = 1e-6
    for a in [0, 4, 5, 11, wl.R - 1]:
        p, m = w0.copy(), w0.copy()
        p[a] += eps
        m[a] -= eps
        g = (np.sum(fwd(p)[2] * dy) - np.sum(fwd(m)[2] * dy)) / (2 * eps)
        assert abs(g - dgate[a]) <= 1e-6 * max(1.0, abs(g)), a
