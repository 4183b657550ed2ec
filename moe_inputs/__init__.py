"""Seeded synthetic inputs for the single-GPU MoE layer forward (and the backward of one workload).

This module is shared by the CPU oracle and the GPU harness. It holds the workload table and the
random draws, and nothing of the MoE method itself: no routing, no top-k, no permutation, no
quantisation, no expert arithmetic. The only arithmetic here is input preparation: scaling
standard normals, rounding them to bfloat16 (round to nearest even) and renormalising uniform gate
weights per token.

Random streams. Every tensor comes from NumPy's PCG64 seeded with ``SeedSequence((seed, tag,
chunk))``, where ``tag`` is the CRC-32 of the tensor's name and ``chunk`` the index of a fixed-size
row block (or the expert id for expert weights). A tensor therefore does not depend on how many
threads generate it, and one expert's weights can be regenerated without the others.

Distribution conventions: ``N(mu, v)`` means mean mu and *variance* v, so the router matrix
``N(0, 1/h)`` gives unit-variance logits.

The model shapes are the ones the Mixture-of-Kittens page lists under "Key claims" (Kimi K2.7 Code,
GLM-5.2, Qwen3.5-397B-A17B, DeepSeek-V4-Pro), and the 2,048 tokens per GPU at expert-parallel
degree 64 that the same list and the 1.41x article quote for the isolated-layer benchmark.
"""
from __future__ import annotations

import dataclasses
import zlib
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "get",
    "scaled",
    "f32_to_bf16",
    "make_inputs",
    "expert_weights",
    "shared_weights",
    "HOTSET_BIAS",
]

# Rows per random chunk for activations; expert weights use one chunk per expert.
_ROW_CHUNK = 256
_THREADS = 8


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic MoE layer workload.

    mode "router": the layer routes its own tokens (router GEMM, top-k, softmax renormalisation),
    all E experts are local (E_loc == E).
    mode "share": one expert-parallel rank's share. The T source tokens each have k assignments
    a = t*k + j; each assignment's local expert is drawn i.i.d. from a Zipf(s) law over the E_loc
    local experts (expert 0 heaviest) and its gate weight from U(0,1), renormalised per token.
    """

    name: str
    T: int
    h: int
    m: int
    E: int
    k: int
    E_loc: int
    dtype: str  # "bf16" or "mxfp8"
    mode: str  # "router" or "share"
    bias: str = "none"  # "none" | "normal" | "hotset"
    bias_var: float = 0.0
    zipf_s: float = 0.0
    m_shared: int = 0  # >0: a BF16 shared SwiGLU expert of this width over the T source tokens
    backward: bool = False
    hot_frac: float = 0.0  # hotset: fraction of experts made hot

    @property
    def R(self) -> int:
        return self.T * self.k

    def describe(self) -> str:
        return (f"{self.name}: T={self.T} h={self.h} m={self.m} E={self.E} (local {self.E_loc}) "
                f"k={self.k} {self.dtype} {self.mode}")


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_T64_h256_m128_E8_k2_bf16", T=64, h=256, m=128, E=8, k=2, E_loc=8,
                 dtype="bf16", mode="router"),
        Workload("dsv4pro_share_T2048_h7168_m3072_E384_k6_bf16", T=2048, h=7168, m=3072, E=384,
                 k=6, E_loc=6, dtype="bf16", mode="share", zipf_s=1.0),
        Workload("qwen397_layer_T4096_h4096_m1024_E512_k10_bf16", T=4096, h=4096, m=1024, E=512,
                 k=10, E_loc=512, dtype="bf16", mode="router", bias="normal", bias_var=0.5),
        Workload("kimi_share_T2048_h7168_m2048_E384_k8_mxfp8", T=2048, h=7168, m=2048, E=384, k=8,
                 E_loc=6, dtype="mxfp8", mode="share", zipf_s=1.2, m_shared=2048),
        Workload("glm52_layer_T8192_h6144_m2048_E256_k8_mxfp8", T=8192, h=6144, m=2048, E=256,
                 k=8, E_loc=256, dtype="mxfp8", mode="router", bias="hotset", backward=True,
                 hot_frac=0.1),
    ]
}

# Short aliases used by tests and the bench command line.
ALIASES = {
    "tiny": "tiny_T64_h256_m128_E8_k2_bf16",
    "dsv4pro": "dsv4pro_share_T2048_h7168_m3072_E384_k6_bf16",
    "qwen397": "qwen397_layer_T4096_h4096_m1024_E512_k10_bf16",
    "kimi": "kimi_share_T2048_h7168_m2048_E384_k8_mxfp8",
    "glm52": "glm52_layer_T8192_h6144_m2048_E256_k8_mxfp8",
}

# Common logit bias added to the hot experts of the GLM-5.2-shaped layer so that the hot 10% of
# experts receive half of the routed rows on the seed-0 inputs. Calibrated by
# oracle/calibrate_hotset.py (bisection on the oracle's routing of the seed-0 inputs); the CPU test
# suite re-checks the resulting share.
HOTSET_BIAS = 1.09375


def get(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]


def scaled(base: Workload, **overrides) -> Workload:
    """A smaller (or edge-case) variant of a workload with the same distributions."""
    fields = dataclasses.asdict(base)
    fields.update(overrides)
    if "name" not in overrides:
        fields["name"] = base.name + "_scaled_" + "_".join(
            f"{k}{v}" for k, v in sorted(overrides.items()))
    wl = Workload(**fields)
    if wl.mode == "router" and wl.E_loc != wl.E:
        raise ValueError("router workloads keep every expert local")
    return wl


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Inputs here are finite normals, so no NaN handling is needed.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _tag(name: str) -> int:
    return zlib.crc32(name.encode("ascii"))


def _rng(seed: int, name: str, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence((seed, _tag(name), chunk))))


def _normal_bf16(seed: int, name: str, rows: int, cols: int, var: float) -> np.ndarray:
    """[rows, cols] bf16 bit patterns of N(0, var), generated in row chunks (thread-count free)."""
    out = np.empty((rows, cols), dtype=np.uint16)
    std = np.float32(np.sqrt(var))
    nchunks = (rows + _ROW_CHUNK - 1) // _ROW_CHUNK

    def job(c: int) -> None:
        r0, r1 = c * _ROW_CHUNK, min(rows, (c + 1) * _ROW_CHUNK)
        g = _rng(seed, name, c)
        v = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        v *= std
        out[r0:r1] = f32_to_bf16(v)

    if nchunks == 1:
        job(0)
    else:
        with ThreadPoolExecutor(min(_THREADS, nchunks)) as ex:
            list(ex.map(job, range(nchunks)))
    return out


def _zipf_probs(n: int, s: float) -> np.ndarray:
    p = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    return p / p.sum()


def hot_experts(wl: Workload, seed: int = 0) -> np.ndarray:
    """Indices of the hot experts of a hotset workload: the first round(hot_frac*E) entries of a
    seeded permutation of the experts."""
    n_hot = int(round(wl.hot_frac * wl.E))
    perm = _rng(seed, "hot_experts", 0).permutation(wl.E)
    return np.sort(perm[:n_hot]).astype(np.int32)


def make_inputs(wl: Workload, seed: int = 0, hot_bias: Optional[float] = None) -> dict:
    """Activations and routing inputs of a workload (expert weights come from expert_weights).

    Returns a dict with
      x        uint16 [T, h]    bf16 bits, N(0, 1)
      router workloads:
        w_router uint16 [E, h]  bf16 bits, N(0, 1/h); row e is expert e's router vector
        bias     float32 [E] or None
      share workloads:
        assign   int32  [T*k]   local expert of assignment a = t*k + j
        assign_w float32 [T*k]  gate weight of assignment a (rows of k sum to 1 per token)
      backward workloads:
        dy       uint16 [T, h]  bf16 bits, N(0, 1)
    """
    d: dict = {"x": _normal_bf16(seed, "x", wl.T, wl.h, 1.0)}
    if wl.mode == "router":
        d["w_router"] = _normal_bf16(seed, "w_router", wl.E, wl.h, 1.0 / wl.h)
        if wl.bias == "none":
            d["bias"] = None
        elif wl.bias == "normal":
            g = _rng(seed, "bias", 0)
            d["bias"] = (g.standard_normal(wl.E) * np.sqrt(wl.bias_var)).astype(np.float32)
        elif wl.bias == "hotset":
            b = np.zeros(wl.E, dtype=np.float32)
            b[hot_experts(wl, seed)] = np.float32(HOTSET_BIAS if hot_bias is None else hot_bias)
            d["bias"] = b
        else:
            raise ValueError(wl.bias)
    elif wl.mode == "share":
        g = _rng(seed, "assign", 0)
        p = _zipf_probs(wl.E_loc, wl.zipf_s)
        d["assign"] = g.choice(wl.E_loc, size=wl.R, p=p).astype(np.int32)
        gu = _rng(seed, "assign_w", 0)
        u = gu.random((wl.T, wl.k))
        d["assign_w"] = (u / u.sum(axis=1, keepdims=True)).astype(np.float32).reshape(-1)
    else:
        raise ValueError(wl.mode)
    if wl.backward:
        d["dy"] = _normal_bf16(seed, "dy", wl.T, wl.h, 1.0)
    return d


def expert_weights(wl: Workload, e: int, seed: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """SwiGLU weights of local expert e as bf16 bits: W_gate, W_up [h, m] ~ N(0, 1/h) and
    W_down [m, h] ~ N(0, 1/m) (variance 1/fan_in). Independent of how many experts are built."""
    return (
        _normal_bf16(seed, f"w_gate/{e}", wl.h, wl.m, 1.0 / wl.h),
        _normal_bf16(seed, f"w_up/{e}", wl.h, wl.m, 1.0 / wl.h),
        _normal_bf16(seed, f"w_down/{e}", wl.m, wl.h, 1.0 / wl.m),
    )


def all_expert_weights(wl: Workload, seed: int = 0):
    """Stacked [E_loc, h, m], [E_loc, h, m], [E_loc, m, h] bf16 bits (GPU harness helper)."""
    wg = np.empty((wl.E_loc, wl.h, wl.m), np.uint16)
    wu = np.empty((wl.E_loc, wl.h, wl.m), np.uint16)
    wd = np.empty((wl.E_loc, wl.m, wl.h), np.uint16)
    for e in range(wl.E_loc):
        wg[e], wu[e], wd[e] = expert_weights(wl, e, seed)
    return wg, wu, wd


def shared_weights(wl: Workload, seed: int = 0):
    """The BF16 shared expert of width m_shared: W_gate, W_up [h, m_s], W_down [m_s, h]."""
    if wl.m_shared <= 0:
        raise ValueError("workload has no shared expert")
    ms = wl.m_shared
    return (
        _normal_bf16(seed, "shared/w_gate", wl.h, ms, 1.0 / wl.h),
        _normal_bf16(seed, "shared/w_up", wl.h, ms, 1.0 / wl.h),
        _normal_bf16(seed, "shared/w_down", ms, wl.h, 1.0 / ms),
    )


# ------------------------------------------------------------------------------------------------
# Device-side generation of expert weights for full-size runs (GPU harness and bench). Each expert
# has its own torch CUDA generator seeded from (seed, name, expert); values are N(0, 1/fan_in)
# drawn in float32 and rounded to bfloat16 by torch. The oracle reads the same tensors back.
# ------------------------------------------------------------------------------------------------


def _torch_seed(seed: int, name: str, e: int) -> int:
    ss = np.random.SeedSequence((seed, _tag(name), e, 0x7E57))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64((1 << 63) - 1))


def torch_expert_weights(wl: Workload, device, seed: int = 0):
    """Stacked W_gate, W_up [E_loc, h, m] and W_down [E_loc, m, h] as torch bfloat16 on `device`."""
    import torch

    out = []
    for name, (a, b), var in (("tw_gate", (wl.h, wl.m), 1.0 / wl.h),
                              ("tw_up", (wl.h, wl.m), 1.0 / wl.h),
                              ("tw_down", (wl.m, wl.h), 1.0 / wl.m)):
        t = torch.empty((wl.E_loc, a, b), dtype=torch.bfloat16, device=device)
        g = torch.Generator(device=device)
        for e in range(wl.E_loc):
            g.manual_seed(_torch_seed(seed, name, e))
            t[e].copy_(torch.randn((a, b), generator=g, device=device, dtype=torch.float32)
                       .mul_(float(np.sqrt(var))))
        out.append(t)
    return tuple(out)


def torch_shared_weights(wl: Workload, device, seed: int = 0):
    """The shared expert's W_gate, W_up [h, m_s], W_down [m_s, h] as torch bfloat16."""
    import torch

    ms = wl.m_shared
    out = []
    for name, (a, b), var in (("tshared/w_gate", (wl.h, ms), 1.0 / wl.h),
                              ("tshared/w_up", (wl.h, ms), 1.0 / wl.h),
                              ("tshared/w_down", (ms, wl.h), 1.0 / ms)):
        g = torch.Generator(device=device)
        g.manual_seed(_torch_seed(seed, name, 0))
        out.append(torch.randn((a, b), generator=g, device=device, dtype=torch.float32)
                   .mul_(float(np.sqrt(var))).to(torch.bfloat16))
    return tuple(out)
