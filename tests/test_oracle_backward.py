"""Pins of the oracle's MXFP8 backward (expert_backward / layer_backward with mx=True).

The unquantised backward is pinned by central finite differences in test_oracle_layer.py. For the
MX variant the plausible mistakes are a wrong quantisation axis for one of the GEMM operands, or MX
blocks along an expert's rows that do not start at its first row. Each test below scales every
other slice of one operand along one axis by 2^-20. MX blocks that run along the *other* axis keep
each slice's own scale, so every slice of the affected result stays within MX precision of the
unquantised float64 result. Blocks that mix the two magnitudes flush the small slices (a ratio of
2^-20 is below E4M3's 2^-17.8 range under one block scale), and those result slices come out
(nearly) zero, i.e. with relative error about 1.
"""
import numpy as np
import pytest

import moe_inputs as I
from oracle import formats as F
from oracle import moe as M

SKEW = 2.0 ** -20
TOL = 0.25  # per-slice relative error: MX precision is a few percent; a flushed slice is ~1


def _operands(rng, n=64, h=64, m=64):
    a = rng.standard_normal((n, h))
    dO = rng.standard_normal((n, h))
    wg = rng.standard_normal((h, m)) / np.sqrt(h)
    wu = rng.standard_normal((h, m)) / np.sqrt(h)
    wd = rng.standard_normal((m, h)) / np.sqrt(m)
    return a, dO, wg, wu, wd


def _slice_err(got, ref, axis):
    """Relative error of every slice along `axis` (axis=0: each row, axis=1: each column)."""
    num = np.linalg.norm(got - ref, axis=1 - axis)
    den = np.linalg.norm(ref, axis=1 - axis)
    return num / den


def _both(a, dO, wg, wu, wd):
    return (M.expert_backward(a, dO, wg, wu, wd, mx=True),
            M.expert_backward(a, dO, wg, wu, wd, mx=False))


def test_mx_backward_unskewed_is_close_to_exact(rng):
    (dA, dWg, dWu, dWd), (rA, rWg, rWu, rWd) = _both(*_operands(rng))
    for got, ref in [(dA, rA), (dWg, rWg), (dWu, rWu), (dWd, rWd)]:
        err = np.abs(got - ref).max() / np.abs(ref).max()
        assert 1e-4 < err < 0.2  # quantised (not exact), within a few E4M3 steps


def test_dgrad_quantises_dO_and_dG_dU_along_the_hidden_and_expert_axes(rng):
    # rows of dO skewed: the dgrad GEMMs must quantise dO (and dG, dU, whose rows inherit the
    # skew) within rows, along h and m
    a, dO, wg, wu, wd = _operands(rng)
    dO[1::2] *= SKEW
    (dA, *_), (rA, *_) = _both(a, dO, wg, wu, wd)
    assert _slice_err(dA, rA, axis=0).max() < TOL


def test_wgrad_quantises_dO_along_rows(rng):
    a, dO, wg, wu, wd = _operands(rng)
    dO[:, 1::2] *= SKEW  # columns of dO skewed: dW_down's columns inherit it
    (_, _, _, dWd), (_, _, _, rWd) = _both(a, dO, wg, wu, wd)
    assert _slice_err(dWd, rWd, axis=1).max() < TOL


def test_wgrad_quantises_the_input_rows_along_rows(rng):
    a, dO, wg, wu, wd = _operands(rng)
    a[:, 1::2] *= SKEW  # columns of a skewed: rows of dW_gate and dW_up inherit it
    (_, dWg, dWu, _), (_, rWg, rWu, _) = _both(a, dO, wg, wu, wd)
    assert _slice_err(dWg, rWg, axis=0).max() < TOL
    assert _slice_err(dWu, rWu, axis=0).max() < TOL


def test_dgrad_quantises_W_down_along_h_and_wgrad_quantises_dG_dU_along_rows(rng):
    a, dO, wg, wu, wd = _operands(rng)
    wd[1::2] *= SKEW  # rows of W_down skewed: columns of dH, dG, dU, dW_gate, dW_up inherit it
    (_, dWg, dWu, _), (_, rWg, rWu, _) = _both(a, dO, wg, wu, wd)
    assert _slice_err(dWg, rWg, axis=1).max() < TOL
    assert _slice_err(dWu, rWu, axis=1).max() < TOL


def test_forward_quantises_W_up_along_h_and_wgrad_quantises_H_along_rows(rng):
    a, dO, wg, wu, wd = _operands(rng)
    wu[:, 1::2] *= SKEW  # columns of W_up skewed: columns of U and H, rows of dW_down inherit it
    (_, _, _, dWd), (_, _, _, rWd) = _both(a, dO, wg, wu, wd)
    assert _slice_err(dWd, rWd, axis=0).max() < TOL


def test_dgrad_quantises_W_gate_and_W_up_along_m(rng):
    a, dO, wg, wu, wd = _operands(rng)
    wg[1::2] *= SKEW  # rows of W_gate and W_up skewed: columns of dA inherit it
    wu[1::2] *= SKEW
    (dA, *_), (rA, *_) = _both(a, dO, wg, wu, wd)
    assert _slice_err(dA, rA, axis=1).max() < TOL


def test_row_blocks_start_at_the_experts_first_row(rng):
    # 40 rows: rows 32..39 form the second block on their own (zero-padded), so scaling them
    # down must not flush them. Blocks counted from the end would put rows 8..39 together.
    a, dO, wg, wu, wd = _operands(rng, n=40)
    dO[32:] *= SKEW
    a[32:] *= SKEW
    dA, dWg, dWu, dWd = M.expert_backward(a, dO, wg, wu, wd, mx=True)
    # the contribution of rows 32..39 alone, with and without quantisation
    part = M.expert_backward(a[32:], dO[32:], wg, wu, wd, mx=True)
    full_first = M.expert_backward(a[:32], dO[:32], wg, wu, wd, mx=True)
    # weight gradients are sums over rows; quantisation blocks never straddle row 32, so the
    # 40-row result is exactly the sum of the two segments' results
    for i in (1, 2, 3):
        got = (dA, dWg, dWu, dWd)[i]
        assert np.allclose(got, full_first[i] + part[i], rtol=1e-12, atol=0.0)
    # and the small segment's own contribution is not flushed
    rpart = M.expert_backward(a[32:], dO[32:], wg, wu, wd, mx=False)
    assert np.abs(part[3] - rpart[3]).max() < TOL * np.abs(rpart[3]).max()


def test_empty_expert_has_zero_gradients(rng):
    a, dO, wg, wu, wd = _operands(rng, n=0)
    for mx in (False, True):
        dA, dWg, dWu, dWd = M.expert_backward(a, dO, wg, wu, wd, mx=mx)
        assert dA.shape == (0, 64)
        assert not dWg.any() and not dWu.any() and not dWd.any()


@pytest.mark.parametrize("mx", [False, True])
def test_layer_backward_assembles_experts_and_unpermutes(mx):
    wl = I.Workload(name="t", T=20, h=64, m=32, E=4, k=2, E_loc=4,
                    dtype="mxfp8" if mx else "bf16", mode="router", backward=True)
    inp = I.make_inputs(wl, seed=4)
    cache = {e: I.expert_weights(wl, e, seed=4) for e in range(4)}
    fwd = M.layer_forward(wl, inp, cache.__getitem__, keep=True)
    dX, dW = M.layer_backward(wl, inp, fwd, cache.__getitem__)
    dy = F.bf16_to_f64(inp["dy"])
    # dX[t] collects, over the token's slots, the per-expert input gradient of its routed row
    # computed on the expert's own rows only
    x = F.bf16_to_f64(inp["x"])
    for t in (0, 7, 19):
        acc = np.zeros(wl.h)
        for j in range(wl.k):
            e = fwd["idx"][t, j]
            r0, r1 = fwd["offsets"][e], fwd["offsets"][e + 1]
            rows = fwd["perm"][r0:r1]
            a = x[rows // wl.k]
            dO = fwd["w"].reshape(-1)[rows][:, None] * dy[rows // wl.k]
            dA = M.expert_backward(a, dO, *(F.bf16_to_f64(v) for v in cache[e]), mx=mx)[0]
            acc += dA[list(rows).index(t * wl.k + j)]
        assert np.allclose(dX[t], acc, rtol=1e-12, atol=1e-12)
    assert len(dW) == 4 and dW[0][0].shape == (64, 32) and dW[0][2].shape == (32, 64)


@pytest.mark.parametrize("mode,mx", [("router", False), ("router", True), ("share", True)])
def test_sampled_gradients_match_whole_layer(mode, mx):
    kw = dict(name="t", T=40, h=64, m=64, E=4, k=2, E_loc=4, dtype="mxfp8" if mx else "bf16",
              mode=mode, backward=True)
    if mode == "share":
        kw.update(E=384, E_loc=3, k=3, zipf_s=1.0)
    wl = I.Workload(**kw)
    inp = I.make_inputs(wl, seed=8)
    cache = {e: I.expert_weights(wl, e, seed=8) for e in range(wl.E_loc)}
    fwd = M.layer_forward(wl, inp, cache.__getitem__, keep=True)
    dX, dW = M.layer_backward(wl, inp, fwd, cache.__getitem__)
    toks = [0, 17, 39]
    got = M.token_input_grads(wl, inp, toks, cache.__getitem__)
    assert np.allclose(got, dX[toks], rtol=1e-12, atol=1e-12)
    if mode == "router":
        assign, aw = fwd["idx"].reshape(-1), fwd["w"].reshape(-1)
    else:
        assign, aw = inp["assign"], inp["assign_w"]
    for e in range(wl.E_loc):
        g = M.expert_weight_grads(wl, inp, assign, aw, e, cache.__getitem__)
        for i in range(3):
            assert np.allclose(g[i], dW[e][i], rtol=1e-12, atol=1e-12), (e, i)
