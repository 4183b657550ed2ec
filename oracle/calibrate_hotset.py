"""Calibrate the common logit bias of the hot experts of the GLM-5.2-shaped layer.

TEST INFRASTRUCTURE ONLY. The workload asks for a router bias under which the top 10% of experts
receive about half of the routed rows. This script routes the seed-0 inputs with the oracle
(fixed-order float32 logits, top-k) and bisects on the bias given to the hot experts, then rounds
it to a multiple of 2**-7. Its printed value is the constant ``moe_inputs.HOTSET_BIAS``.

    python -m oracle.calibrate_hotset
"""
from __future__ import annotations

import time

import numpy as np

import moe_inputs as I
from oracle import moe as M


def hot_share(acc: np.ndarray, hot: np.ndarray, beta: float, k: int) -> float:
    bias = np.zeros(acc.shape[1], np.float32)
    bias[hot] = np.float32(beta)
    idx = M.topk(acc + bias[None, :], k)
    return float(np.isin(idx, hot).mean())


def main() -> None:
    wl = I.get("glm52")
    t0 = time.time()
    inp = I.make_inputs(wl, seed=0, hot_bias=0.0)
    acc = M.router_logits_fixed_order(inp["x"], inp["w_router"], None)
    print(f"logits in {time.time() - t0:.1f} s")
    hot = I.hot_experts(wl, 0)
    lo, hi = 0.0, 4.0
    for _ in range(24):
        mid = 0.5 * (lo + hi)
        if hot_share(acc, hot, mid, wl.k) < 0.5:
            lo = mid
        else:
            hi = mid
    beta = round(0.5 * (lo + hi) * 128) / 128
    print(f"bias {beta!r}  hot share {hot_share(acc, hot, beta, wl.k):.4f}")


if __name__ == "__main__":
    main()
