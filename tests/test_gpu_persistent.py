"""GPU parity of moe_forward_persistent (the whole forward in one persistent kernel): on scaled and
full-size workloads its y, logits, top-k and schedule are bitwise those of moe_forward (which the
forward tests check against the oracle), its status word says MOE_OK, a second run is bitwise the
same, so is a run beside a busy kernel on another stream, and dropped assignments behave as in the
forward. A small case is also checked against the oracle directly."""
import numpy as np
import pytest

import moe_inputs as I
from oracle import moe as M
from tests._gpu_helpers import (BF16_TOL, MX_TOL, dev, dev_bf16, host_bf16_bits,
                                host_f64_from_bf16, normwise_err, note, poisoned, require_gpu,
                                torch)

pytestmark = pytest.mark.gpu

SCALED = {
    "tiny": dict(),
    "dsv4pro": dict(T=256, h=512, m=384),
    "qwen397": dict(T=320, h=512, m=128, E=64, E_loc=64),
    "glm52": dict(T=300, h=768, m=512, E=64, E_loc=64),
}


def _setup(G, wl, seed, device_weights=False):
    inp = I.make_inputs(wl, seed=seed)
    if device_weights:  # full-size expert weights, drawn on the GPU
        wts = None
        weights = I.torch_expert_weights(wl, torch.device("cuda"), seed=seed)
    else:
        wts = [I.expert_weights(wl, e, seed=seed) for e in range(wl.E_loc)]
        weights = tuple(dev_bf16(np.stack([w[i] for w in wts])) for i in range(3))
    sh = G.make_shape(wl.T, wl.h, wl.m, wl.E, wl.k, wl.E_loc, wl.m_shared)
    prepared = G.moe_prepare_weights(sh, wl.dtype, *weights)
    kw = {}
    if wl.mode == "router":
        kw["w_router"] = dev_bf16(inp["w_router"])
        kw["bias"] = None if inp["bias"] is None else dev(inp["bias"])
    else:
        kw["assign"] = dev(inp["assign"])
        kw["assign_w"] = dev(inp["assign_w"])
    return inp, wts, sh, prepared, kw


def _persistent(G, wl, sh, x, prepared, kw, stream=None):
    y = poisoned((wl.T, wl.h), torch.bfloat16)
    y, ws, status = G.moe_forward_persistent(sh, wl.dtype, x, prepared, y=y, stream=stream, **kw)
    return y, ws, status


def _compare_to_forward(G, wl, sh, x, prepared, kw):
    y0, ws0 = G.moe_forward(sh, wl.dtype, x, prepared, y=poisoned((wl.T, wl.h), torch.bfloat16),
                            **kw)
    y1, ws1, status = _persistent(G, wl, sh, x, prepared, kw)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "persistent forward reported a timeout"
    assert np.array_equal(host_bf16_bits(y0), host_bf16_bits(y1))
    # the persistent workspace starts with the forward's layout
    v0 = G.moe_forward_views(sh, wl.dtype, ws0)
    v1 = G.moe_forward_views(sh, wl.dtype, ws1)
    keys = ["counts", "offsets", "perm", "inv"]
    if wl.mode == "router":
        keys += ["logits", "topk_idx", "topk_w"]
    nrows = int(v0["offsets"][-1].item())  # rows past the valid ones are never written
    for key in keys:
        a, b = v0[key].cpu().numpy(), v1[key].cpu().numpy()
        if key == "perm":
            a, b = a[:nrows], b[:nrows]
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b), key
    return y1


@pytest.mark.parametrize("name", list(SCALED))
def test_persistent_equals_forward_scaled(name):
    G = require_gpu()
    base = I.get(name)
    wl = I.scaled(base, **SCALED[name]) if SCALED[name] else base
    note(f"persistent forward {wl.describe()}")
    inp, wts, sh, prepared, kw = _setup(G, wl, seed=5)
    x = dev_bf16(inp["x"])
    y = _compare_to_forward(G, wl, sh, x, prepared, kw)
    if name in ("tiny", "glm52"):  # also straight against the oracle
        ref = M.layer_forward(wl, inp, lambda e: wts[e])
        err = normwise_err(host_f64_from_bf16(y), ref["y"])
        note(f"  normwise error vs oracle {err:.3e}")
        assert err <= (MX_TOL if wl.dtype == "mxfp8" else BF16_TOL)
    # a second run: bitwise the same
    y2, _, st2 = _persistent(G, wl, sh, x, prepared, kw)
    torch.cuda.synchronize()
    assert int(st2.item()) == 0
    assert np.array_equal(host_bf16_bits(y), host_bf16_bits(y2))


@pytest.mark.parametrize("name", ["tiny", "dsv4pro", "qwen397", "glm52"])
def test_persistent_equals_forward_full_size(name):
    """The benchmark shapes themselves (GLM: 8192 tokens, 256 experts, MXFP8)."""
    G = require_gpu()
    wl = I.get(name)
    note(f"persistent forward full size {wl.describe()}")
    inp, _, sh, prepared, kw = _setup(G, wl, seed=0, device_weights=True)
    _compare_to_forward(G, wl, sh, dev_bf16(inp["x"]), prepared, kw)


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_persistent_dropped_assignments(dtype):
    """Assignments to experts outside [0, E_loc) get no row and no contribution, as in
    moe_forward."""
    G = require_gpu()
    wl = I.scaled(I.get("dsv4pro"), T=200, h=512, m=256, dtype=dtype)
    inp, _, sh, prepared, kw = _setup(G, wl, seed=9)
    a = inp["assign"].copy()
    a[::7] = wl.E_loc + 3
    a[5] = -1
    kw["assign"] = dev(a)
    note(f"persistent forward with dropped ids {wl.describe()}")
    _compare_to_forward(G, wl, sh, dev_bf16(inp["x"]), prepared, kw)


def test_persistent_under_a_concurrent_busy_kernel():
    """With float32 matrix products running on a second stream of the same (default) priority the
    persistent kernel's workgroups share the CUs; its hand-offs still finish and the bits are the
    same."""
    G = require_gpu()
    wl = I.scaled(I.get("glm52"), T=1024, h=1024, m=512, E=64, E_loc=64)
    inp, _, sh, prepared, kw = _setup(G, wl, seed=4)
    x = dev_bf16(inp["x"])
    y0, _, st0 = _persistent(G, wl, sh, x, prepared, kw)
    torch.cuda.synchronize()
    assert int(st0.item()) == 0
    busy = torch.cuda.Stream()
    a = torch.randn(4096, 4096, device="cuda")
    main = torch.cuda.current_stream()
    for rep in range(3):
        note(f"  persistent beside a busy stream, rep {rep}")
        with torch.cuda.stream(busy):
            for _ in range(4):
                b = a @ a
        y1, _, st1 = _persistent(G, wl, sh, x, prepared, kw, stream=main)
        torch.cuda.synchronize()
        assert int(st1.item()) == 0
        assert np.array_equal(host_bf16_bits(y0), host_bf16_bits(y1))
    del b
