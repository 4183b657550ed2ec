"""GPU parity of moe_prepare_weights + moe_expert_ffn (the grouped SwiGLU GEMMs) against the
oracle's per-expert SwiGLU FFN: BF16 within 1e-2 and MXFP8 within 3e-2 normwise, on ragged
per-expert row counts (empty experts, counts that are not tile multiples, several tiles)."""
import numpy as np
import pytest

import moe_inputs as I
from oracle import formats as F
from oracle import moe as M
from tests._gpu_helpers import (BF16_TOL, MX_TOL, dev, dev_bf16, host_f64_from_bf16, normwise_err,
                                note, poisoned, require_gpu, torch)

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, rows per expert, h, m (tile heights: BF16 256 rows from 224 rows per expert when the
    # 256-row tiles number 256 or more; MXFP8 192 rows from 128 rows per expert; else 128;
    # h % 256 != 0 takes the small-tile kernel)
    ("bf16", [16, 0, 40, 200], 256, 128),
    ("bf16", [1, 129, 0, 300, 127, 2], 384, 192),  # small-tile kernel
    ("bf16", [517], 512, 256),
    ("bf16", [300, 0, 700, 31], 256, 256),         # 128-row tiles (too few 256-row ones)
    ("bf16", [2000, 513], 1024, 512),              # many K stages, several N tiles
    ("bf16", [1100, 0, 900, 61], 256, 4096),       # 256-row tiles (288 of them)
    ("mxfp8", [16, 0, 40, 200], 256, 256),
    ("mxfp8", [1, 129, 0, 300, 127, 2], 512, 256),
    ("mxfp8", [0, 0, 259], 768, 512),
    ("mxfp8", [600, 0, 301], 512, 256),            # 192-row tiles
    ("mxfp8", [1500, 700], 1024, 512),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_{'-'.join(map(str, c[1]))}_h{c[2]}_m{c[3]}")
def test_expert_ffn_parity(case):
    G = require_gpu()
    dt, counts, h, m = case
    E_loc = len(counts)
    R = int(sum(counts))
    wl = I.Workload(name="ffn", T=R, h=h, m=m, E=E_loc, k=1, E_loc=E_loc, dtype=dt, mode="router")
    rng = np.random.default_rng(R + h)
    x = I.f32_to_bf16(rng.standard_normal((R, h)).astype(np.float32))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    wts = [I.expert_weights(wl, e, seed=2) for e in range(E_loc)]
    note(f"ffn {case}")
    sh = G.make_shape(R, h, m, E_loc, 1)
    wg = dev_bf16(np.stack([w[0] for w in wts]))
    wu = dev_bf16(np.stack([w[1] for w in wts]))
    wd = dev_bf16(np.stack([w[2] for w in wts]))
    prepared = G.moe_prepare_weights(sh, dt, wg, wu, wd)
    x64 = F.bf16_to_f64(x)
    if dt == "mxfp8":
        q, s = F.mx_quantize(x64, axis=1)
        rows, scales = dev(q), dev(s)
    else:
        rows, scales = dev_bf16(x), None
    out = poisoned((R, h), torch.bfloat16)
    G.moe_expert_ffn(sh, dt, rows, scales, dev(offsets), prepared, out_rows=out)
    torch.cuda.synchronize()
    got = host_f64_from_bf16(out)
    ref = M.expert_outputs(x64, offsets, lambda e: wts[e], mx=(dt == "mxfp8"))
    assert np.isfinite(got).all()
    err = normwise_err(got, ref)
    note(f"  normwise error {err:.3e}")
    assert err <= (MX_TOL if dt == "mxfp8" else BF16_TOL)
    # every expert on its own is within tolerance too
    for e in range(E_loc):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            assert normwise_err(got[r0:r1], ref[r0:r1]) <= (MX_TOL if dt == "mxfp8" else BF16_TOL)


def test_prepared_mx_weights_bit_exact():
    """The MXFP8 prepared layout (K-tiled codes, chunk-major scales) holds exactly the oracle's MX
    codes and scales of each weight column."""
    G = require_gpu()
    h, m, E_loc = 256, 256, 2
    wl = I.Workload(name="prep", T=1, h=h, m=m, E=E_loc, k=1, E_loc=E_loc, dtype="mxfp8",
                    mode="router")
    wts = [I.expert_weights(wl, e, seed=9) for e in range(E_loc)]
    sh = G.make_shape(1, h, m, E_loc, 1)
    prepared = G.moe_prepare_weights(sh, "mxfp8", *(dev_bf16(np.stack([w[i] for w in wts]))
                                                    for i in range(3)))
    torch.cuda.synchronize()
    p = prepared.cpu().numpy()
    n1 = E_loc * 2 * m * h
    # codes K-tiled: [E][2m/256][h/128][256][128], one contiguous 32 KB block per 128-byte stage of
    # a 256-row panel
    w1 = (p[:n1].reshape(E_loc, 2 * m // 256, h // 128, 256, 128).transpose(0, 1, 3, 2, 4)
          .reshape(E_loc, 2 * m, h))
    off = (n1 + 255) // 256 * 256
    # scales chunk-major: [E][h/256][2m][8], the 8 block scales of one 256-element chunk of
    # every weight row side by side
    w1s = (p[off:off + E_loc * 2 * m * h // 32].reshape(E_loc, h // 256, 2 * m, 8)
           .transpose(0, 2, 1, 3).reshape(E_loc, 2 * m, h // 32))
    for e in range(E_loc):
        qg, sg = F.mx_quantize(F.bf16_to_f64(wts[e][0]), axis=0)  # [h, m] along h
        rowsel = np.array([64 * (n // 32) + n % 32 for n in range(m)])
        assert np.array_equal(w1[e][rowsel], qg.T)
        assert np.array_equal(w1s[e][rowsel], sg.T)
