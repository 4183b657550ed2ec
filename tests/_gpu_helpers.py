"""Helpers of the GPU parity tests: moving seeded inputs to the device, reading results back, and
the error measure. Nothing here computes any part of the MoE layer."""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import moe_inputs as I  # noqa: E402

BF16_TOL = 1e-2  # normwise, GPU BF16 path vs float64 oracle
MX_TOL = 3e-2    # normwise, GPU MXFP8 path vs float64 oracle (with MX steps)


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import routing_expert_grouped_amd as G  # noqa: F401  (raises if the library is missing)
    return G


def note(msg: str) -> None:
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def dev_bf16(a: np.ndarray) -> "torch.Tensor":
    """uint16 bf16 bit patterns -> CUDA bfloat16 tensor (bits unchanged)."""
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.cuda().view(torch.bfloat16)


def dev(a: np.ndarray) -> "torch.Tensor":
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bf16_bits(t) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64_from_bf16(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def normwise_err(y: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(y - ref))) / (den if den > 0 else 1.0)


def poisoned(shape, dtype) -> "torch.Tensor":
    """Output buffer pre-filled with NaN (or 0x7f bytes) so unwritten elements are caught."""
    t = torch.empty(shape, dtype=dtype, device="cuda")
    if dtype.is_floating_point:
        t.fill_(float("nan"))
    else:
        t.view(torch.uint8).fill_(0x7F)
    return t
