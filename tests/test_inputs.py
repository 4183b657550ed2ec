"""The seeded input generator: determinism, stream independence, and the workload recipes."""
import numpy as np
import pytest

import moe_inputs as I
from oracle import moe as M
from oracle.formats import bf16_to_f64


def test_deterministic_and_seed_dependent():
    wl = I.scaled(I.get("qwen397"), T=300, h=64, E=16, E_loc=16, k=4)
    a, b, c = I.make_inputs(wl, 0), I.make_inputs(wl, 0), I.make_inputs(wl, 1)
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["bias"], b["bias"])
    assert not np.array_equal(a["x"], c["x"])
    # chunked generation: the first rows do not depend on how many rows exist
    wl2 = I.scaled(wl, T=40)
    assert np.array_equal(I.make_inputs(wl2, 0)["x"], a["x"][:40])


def test_expert_streams_independent():
    wl = I.scaled(I.get("dsv4pro"), h=64, m=32)
    w3 = I.expert_weights(wl, 3)
    wl_more = I.scaled(wl, E_loc=6)
    assert all(np.array_equal(p, q) for p, q in zip(w3, I.expert_weights(wl_more, 3)))
    assert not np.array_equal(w3[0], I.expert_weights(wl, 2)[0])


def test_distributions():
    wl = I.scaled(I.get("qwen397"), T=512, h=256, m=128, E=64, E_loc=64, k=4)
    d = I.make_inputs(wl, 0)
    x = bf16_to_f64(d["x"])
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    wr = bf16_to_f64(d["w_router"])
    assert abs(wr.std() * np.sqrt(wl.h) - 1) < 0.05  # N(0, 1/h): variance 1/h
    assert abs(d["bias"].std() - np.sqrt(0.5)) < 0.15  # N(0, 0.5): variance 0.5
    wg, wu, wd = (bf16_to_f64(v) for v in I.expert_weights(wl, 0))
    assert abs(wg.std() * np.sqrt(wl.h) - 1) < 0.05 and abs(wd.std() * np.sqrt(wl.m) - 1) < 0.05


@pytest.mark.parametrize("name,s", [("dsv4pro", 1.0), ("kimi", 1.2)])
def test_share_zipf_and_gate_weights(name, s):
    wl = I.get(name)
    d = I.make_inputs(I.scaled(wl, h=32), 0)
    a = d["assign"]
    assert a.shape == (wl.T * wl.k,) and a.min() >= 0 and a.max() < wl.E_loc
    counts = np.bincount(a, minlength=wl.E_loc)
    assert counts.sum() == wl.T * wl.k
    p = np.arange(1, wl.E_loc + 1) ** -s
    p /= p.sum()
    expect = p * wl.T * wl.k
    assert np.all(np.abs(counts - expect) < 5 * np.sqrt(expect))  # multinomial spread
    assert np.all(np.diff(counts) < 0)  # expert 0 heaviest
    w = d["assign_w"].reshape(wl.T, wl.k).astype(np.float64)
    assert np.all(w > 0) and np.allclose(w.sum(axis=1), 1.0, atol=1e-6)


@pytest.mark.slow
def test_glm52_hot_set_receives_half_of_routed_rows():
    wl = I.get("glm52")
    d = I.make_inputs(wl, 0)
    hot = I.hot_experts(wl, 0)
    assert len(hot) == 26
    logits = M.router_logits_f64(d["x"], d["w_router"], d["bias"])
    idx = M.topk(logits, wl.k)
    share = np.isin(idx, hot).mean()
    assert 0.495 <= share <= 0.505, share


def test_cover_tokens_hits_every_tile():
    """The full-size tests' token choice: every M tile of every expert at every tile height, and
    every expert's first and last row, has a routed row of a chosen token (checked by brute
    force on a router-shaped schedule with a hot set and empty experts)."""
    from oracle import moe as M
    from tests._sampling import TILE_HEIGHTS, cover_tokens
    rng = np.random.default_rng(2)
    T, E, k = 3000, 40, 4
    l = rng.standard_normal((T, E))
    l[:, :4] += 2.5  # a few hot experts with many tiles
    l[:, 30:] -= 50.0  # some experts that receive nothing
    idx = M.topk(l, k)
    counts, offsets, perm, inv = M.schedule(idx.reshape(-1), E)
    toks = cover_tokens(offsets, perm, inv, k, 100, seed=0)
    assert len(toks) >= 100 and len(set(toks.tolist())) == len(toks)
    rows = set(inv.reshape(-1, k)[toks].reshape(-1).tolist())
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            assert a in rows and b - 1 in rows
        for bm in TILE_HEIGHTS:
            for r0 in range(a, b, bm):
                assert any(r in rows for r in range(r0, min(b, r0 + bm))), (e, bm, r0)
