"""GPU parity of moe_route: router logits bit-exact against the oracle's fixed float32 order,
top-k indices bit-exact, gate weights within 1e-6 relative."""
import numpy as np
import pytest

import moe_inputs as I
from oracle import moe as M
from tests._gpu_helpers import dev, dev_bf16, note, require_gpu, torch

pytestmark = pytest.mark.gpu


def _run_route(G, wl, x, wr, bias):
    sh = G.make_shape(wl.T, wl.h, wl.m, wl.E, wl.k)
    logits, idx, w = G.moe_route(sh, dev_bf16(x), dev_bf16(wr),
                                 None if bias is None else dev(bias))
    torch.cuda.synchronize()
    return logits.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


CASES = [
    dict(T=64, h=256, E=8, k=2, bias="none"),                   # the tiny layer
    dict(T=67, h=512, E=512, k=10, bias="normal", bias_var=0.5),  # ragged T, wide E
    dict(T=33, h=768, E=256, k=8, bias="hotset", hot_frac=0.1),
    dict(T=9, h=128, E=1, k=1, bias="none"),                     # single expert
    dict(T=20, h=64, E=1000, k=16, bias="normal", bias_var=2.0),  # E near the 1024 limit
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"T{c['T']}_h{c['h']}_E{c['E']}_k{c['k']}")
def test_route_bit_exact(case):
    G = require_gpu()
    wl = I.Workload(name="route", m=64, E_loc=case["E"], dtype="bf16", mode="router", **case)
    inp = I.make_inputs(wl, seed=11)
    note(f"route parity {wl.describe()}")
    logits, idx, w = _run_route(G, wl, inp["x"], inp["w_router"], inp["bias"])
    ref_l = M.router_logits_fixed_order(inp["x"], inp["w_router"], inp["bias"])
    assert np.array_equal(logits.view(np.uint32), ref_l.view(np.uint32))
    ref_idx = M.topk(ref_l, wl.k)
    assert np.array_equal(idx, ref_idx)
    ref_w = M.topk_weights(ref_l, ref_idx)
    assert np.allclose(w, ref_w, rtol=1e-6, atol=0)


def test_route_exact_ties_and_signed_zero():
    G = require_gpu()
    T, h, E, k = 16, 64, 70, 5
    x = np.zeros((T, h), np.uint16)
    x[:, 0] = 0x3F80  # 1.0
    x[1::2, 1] = 0x8000  # -0.0 in some tokens
    wr = np.zeros((E, h), np.uint16)
    wr[::3, 0] = 0x3F80  # a third of the experts tie at logit 1.0, the rest at +-0
    wr[1::7, 0] = 0x8000  # -0.0 * 1.0 = -0.0 logits
    wl = I.Workload(name="ties", T=T, h=h, m=64, E=E, k=k, E_loc=E, dtype="bf16", mode="router")
    logits, idx, w = _run_route(G, wl, x, wr, None)
    ref_l = M.router_logits_fixed_order(x, wr)
    assert np.array_equal(logits.view(np.uint32), ref_l.view(np.uint32))
    assert np.array_equal(idx, M.topk(ref_l, k))
    assert idx[0].tolist() == [0, 3, 6, 9, 12]  # equal logits: lowest indices first
    assert np.allclose(w, 1.0 / k, rtol=1e-6)
