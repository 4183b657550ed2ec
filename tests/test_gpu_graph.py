"""moe_forward and moe_forward_persistent captured into a HIP graph (torch.cuda.CUDAGraph), for
callers that replay the layer, e.g. small decode batches where launch overhead dominates. The
library allocates nothing and issues no memset on the forward path, so the whole launch sequence
is captured. Every replay, with eager forwards and synchronisations of the same program between
the replays and the captured input buffer refilled with alternating inputs, is bitwise equal to
the eager forward of that input."""
import numpy as np
import pytest

import moe_inputs as I
from tests._gpu_helpers import dev, dev_bf16, host_bf16_bits, note, poisoned, require_gpu, torch

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": ("tiny", dict()),
    "glm52": ("glm52", dict(T=300, h=768, m=512, E=64, E_loc=64)),
    "kimi": ("kimi", dict(T=256, h=512, m=256)),
    "dsv4pro": ("dsv4pro", dict(T=256, h=512, m=384)),
}


def _setup(G, wl, seed):
    inp = I.make_inputs(wl, seed=seed)
    weights = I.torch_expert_weights(wl, torch.device("cuda"), seed=seed)
    sh = G.make_shape(wl.T, wl.h, wl.m, wl.E, wl.k, wl.E_loc, wl.m_shared)
    prepared = G.moe_prepare_weights(sh, wl.dtype, *weights)
    shared = None
    if wl.m_shared:
        sw = I.torch_shared_weights(wl, torch.device("cuda"), seed=seed)
        shared = G.moe_prepare_weights(G.make_shape(wl.T, wl.h, wl.m_shared, 1, 1, 1), "bf16", *sw)
    kw = {}
    if wl.mode == "router":
        kw["w_router"] = dev_bf16(inp["w_router"])
        kw["bias"] = None if inp["bias"] is None else dev(inp["bias"])
    else:
        kw["assign"] = dev(inp["assign"])
        kw["assign_w"] = dev(inp["assign_w"])
    return inp, sh, prepared, shared, kw


@pytest.mark.parametrize("name", list(CASES))
def test_forward_graph_replays_equal_eager(name):
    G = require_gpu()
    base, over = CASES[name]
    wl = I.scaled(I.get(base), **over) if over else I.get(base)
    note(f"graph-captured forward {wl.describe()}")
    inp, sh, prepared, shared, kw = _setup(G, wl, seed=11)
    x0 = dev_bf16(inp["x"])
    x1 = dev_bf16(I.make_inputs(wl, seed=12)["x"])

    def eager(x):
        y, _ = G.moe_forward(sh, wl.dtype, x, prepared, shared_prepared=shared,
                             y=poisoned((wl.T, wl.h), torch.bfloat16), **kw)
        torch.cuda.synchronize()
        return host_bf16_bits(y)

    ref = [eager(x0), eager(x1)]
    # the captured buffers: input, output, workspace
    X = x0.clone()
    Y = poisoned((wl.T, wl.h), torch.bfloat16)
    WS = torch.empty(G.moe_forward_workspace_bytes(sh, wl.dtype), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture, as torch asks
        G.moe_forward(sh, wl.dtype, X, prepared, shared_prepared=shared, y=Y, ws=WS, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        G.moe_forward(sh, wl.dtype, X, prepared, shared_prepared=shared, y=Y, ws=WS, **kw)
    torch.cuda.synchronize()
    for rep in range(4):
        X.copy_(x0 if rep % 2 == 0 else x1)
        Y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        note(f"  replay {rep}")
        assert np.array_equal(host_bf16_bits(Y), ref[rep % 2]), f"replay {rep}"
        # the program's own eager work between replays
        assert np.array_equal(eager(x1 if rep % 2 == 0 else x0), ref[(rep + 1) % 2])
    del g


def test_persistent_forward_graph_replays_equal_eager():
    """The persistent forward's set-up kernel clears its counters inside the graph (a kernel, not
    a memset), so every replay starts from zero."""
    G = require_gpu()
    wl = I.scaled(I.get("glm52"), T=300, h=768, m=512, E=64, E_loc=64)
    note(f"graph-captured persistent forward {wl.describe()}")
    inp, sh, prepared, _, kw = _setup(G, wl, seed=13)
    x0 = dev_bf16(inp["x"])
    x1 = dev_bf16(I.make_inputs(wl, seed=14)["x"])

    def eager(x):
        y, _ = G.moe_forward(sh, wl.dtype, x, prepared, y=poisoned((wl.T, wl.h), torch.bfloat16),
                             **kw)
        torch.cuda.synchronize()
        return host_bf16_bits(y)

    ref = [eager(x0), eager(x1)]
    X = x0.clone()
    Y = poisoned((wl.T, wl.h), torch.bfloat16)
    WS = torch.empty(G.moe_forward_persistent_workspace_bytes(sh, wl.dtype), dtype=torch.uint8,
                     device="cuda")
    ST = torch.empty(1, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        G.moe_forward_persistent(sh, wl.dtype, X, prepared, y=Y, ws=WS, status=ST, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        G.moe_forward_persistent(sh, wl.dtype, X, prepared, y=Y, ws=WS, status=ST, **kw)
    torch.cuda.synchronize()
    for rep in range(4):
        X.copy_(x0 if rep % 2 == 0 else x1)
        Y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        note(f"  replay {rep}")
        assert int(ST.item()) == 0
        assert np.array_equal(host_bf16_bits(Y), ref[rep % 2]), f"replay {rep}"
        assert np.array_equal(eager(x1 if rep % 2 == 0 else x0), ref[(rep + 1) % 2])
    del g
