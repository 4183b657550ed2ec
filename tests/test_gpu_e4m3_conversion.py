"""The library's E4M3 encoder uses the hardware conversion (v_cvt_pk_fp8_f32 after a clamp to
+-448). Its contract is the rounding rule of the MX definition written out in e4m3_encode_rule
(round to nearest even, saturation to 448, sign of zero kept), which the oracle's codec follows
(pinned on the CPU against an exhaustive nearest-code search). moe_check_e4m3 compares the two on
the GPU for every float32 of magnitude below 2^17, both signs (zero, the float32 subnormals and
every normal), together with the byte order of the four-code packing."""
import pytest

from tests._gpu_helpers import note, require_gpu

pytestmark = pytest.mark.gpu


def test_hardware_e4m3_conversion_follows_the_rule():
    G = require_gpu()
    bad = G.moe_check_e4m3()
    note(f"E4M3 encoder vs rule: {bad} mismatching inputs of 2 x 2^30")
    assert bad == 0
