"""The allocation-free moe_permute_static (schedule scratch in the library's static per-GPU array)
against moe_permute with a caller workspace, through the C ABI: counts, offsets, perm, inv and the
routed rows (codes and scales for MXFP8) bit for bit, on two calls in a row on the same GPU, the
second with a smaller input (the array keeps the first call's contents)."""
import numpy as np
import pytest

import moe_inputs as I
from tests._gpu_helpers import dev, dev_bf16, note, require_gpu, torch

pytestmark = pytest.mark.gpu


def _outputs(G, sh, dtype):
    R, h = sh.T * sh.k, sh.h
    mx = dtype == "mxfp8"
    o = {"counts": torch.full((sh.E_loc,), -7, dtype=torch.int32, device="cuda"),
         "offsets": torch.full((sh.E_loc + 1,), -7, dtype=torch.int32, device="cuda"),
         "perm": torch.full((R,), -7, dtype=torch.int32, device="cuda"),
         "inv": torch.full((R,), -7, dtype=torch.int32, device="cuda")}
    if mx:
        o["rows"] = torch.full((R, h), 0x7F, dtype=torch.uint8, device="cuda")
        o["row_scales"] = torch.full((R, h // 32), 0x7F, dtype=torch.uint8, device="cuda")
    else:
        o["rows"] = torch.full((R, h), float("nan"), dtype=torch.bfloat16, device="cuda")
        o["row_scales"] = None
    return o


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_permute_static_equals_permute_twice(dtype):
    G = require_gpu()
    for T, h, E_loc, k, seed in ((3000, 512, 200, 8, 1), (300, 256, 33, 4, 2)):
        wl = I.Workload(name="noalloc", T=T, h=h, m=256, E=E_loc, k=k, E_loc=E_loc, dtype=dtype,
                        mode="share", zipf_s=1.1)
        note(f"moe_permute_static vs moe_permute: {wl.describe()}")
        inp = I.make_inputs(wl, seed=seed)
        sh = G.make_shape(T, h, 256, E_loc, k, E_loc)
        x, assign = dev_bf16(inp["x"]), dev(inp["assign"])
        ref = G.moe_permute(sh, dtype, assign, x)
        got = G.moe_permute_static(sh, dtype, assign, x, _outputs(G, sh, dtype))
        torch.cuda.synchronize()
        for key in ("counts", "offsets", "perm", "inv", "rows", "row_scales"):
            if ref[key] is None:
                continue
            a = ref[key].contiguous().view(torch.uint8).cpu().numpy()
            b = got[key].contiguous().view(torch.uint8).cpu().numpy()
            assert np.array_equal(a, b), key
