"""GPU parity of moe_permute: counts, offsets, perm and inv bit-exact against the oracle's stable
schedule; gathered BF16 rows bit-exact; MXFP8 codes and scales bit-exact against the oracle's MX
quantisation of each token."""
import numpy as np
import pytest

import moe_inputs as I
from oracle import formats as F
from oracle import moe as M
from tests._gpu_helpers import dev, dev_bf16, host_bf16_bits, note, require_gpu, torch

pytestmark = pytest.mark.gpu


def _assign(kind, T, k, E_loc, rng):
    R = T * k
    if kind == "uniform":
        return rng.integers(0, E_loc, size=R).astype(np.int32)
    if kind == "one_expert":
        return np.full(R, E_loc - 1, np.int32)
    if kind == "sparse":  # most experts empty
        return rng.choice([0, 3, E_loc - 1], size=R).astype(np.int32)
    if kind == "zipf":
        p = np.arange(1, E_loc + 1) ** -1.2
        return rng.choice(E_loc, size=R, p=p / p.sum()).astype(np.int32)
    raise ValueError(kind)


CASES = [
    ("uniform", 64, 256, 2, 8, "bf16"),
    ("zipf", 333, 256, 6, 6, "bf16"),        # R = 1998: ragged last chunk
    ("one_expert", 50, 256, 3, 16, "bf16"),
    ("sparse", 129, 512, 8, 256, "mxfp8"),
    ("uniform", 700, 256, 10, 512, "mxfp8"),
    ("uniform", 1, 256, 1, 1, "mxfp8"),      # a single row
    ("zipf", 40, 256, 16, 1024, "bf16"),     # k and E_loc at their limits
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "_".join(map(str, c)))
def test_permute_bit_exact(case):
    G = require_gpu()
    kind, T, h, k, E_loc, dt = case
    rng = np.random.default_rng(T * 7 + E_loc)
    wl = I.Workload(name="perm", T=T, h=h, m=256, E=E_loc, k=k, E_loc=E_loc, dtype=dt,
                    mode="router")
    x = I.make_inputs(wl, seed=5)["x"]
    if dt == "mxfp8":  # exercise signed zeros, all-zero blocks and saturating magnitudes too
        x = x.copy()
        x[0, :32] = 0x8000
        x[-1, 32:64] = 0
        x[min(1, T - 1), 64:96] = 0x7F00 if T > 1 else x[0, 64:96]
    assign = _assign(kind, T, k, E_loc, rng)
    note(f"permute {case}")
    sh = G.make_shape(T, h, 256, E_loc, k)
    o = G.moe_permute(sh, dt, dev(assign), dev_bf16(x))
    torch.cuda.synchronize()
    counts, offsets, perm, inv = M.schedule(assign, E_loc)
    assert np.array_equal(o["counts"].cpu().numpy(), counts)
    assert np.array_equal(o["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(o["perm"].cpu().numpy(), perm)
    assert np.array_equal(o["inv"].cpu().numpy(), inv)
    if dt == "bf16":
        rows = host_bf16_bits(o["rows"])
        assert np.array_equal(rows, M.gather_rows(x, perm, k))
    else:
        q, s = F.mx_quantize(F.bf16_to_f64(x), axis=1)
        rows = o["rows"].cpu().numpy()
        scales = o["row_scales"].cpu().numpy()
        assert np.array_equal(scales, M.gather_rows(s, perm, k))
        assert np.array_equal(rows, M.gather_rows(q, perm, k))


def test_permute_is_deterministic():
    G = require_gpu()
    T, h, k, E_loc = 2048, 256, 8, 64
    rng = np.random.default_rng(3)
    assign = dev(rng.integers(0, E_loc, size=T * k).astype(np.int32))
    x = dev_bf16(I.f32_to_bf16(rng.standard_normal((T, h)).astype(np.float32)))
    sh = G.make_shape(T, h, 256, E_loc, k)
    a = G.moe_permute(sh, "mxfp8", assign, x)
    b = G.moe_permute(sh, "mxfp8", assign, x)
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "perm", "inv", "rows", "row_scales"):
        assert torch.equal(a[key], b[key]), key
