"""ctypes loader and signatures of libmoe_mi355x.so (the C ABI declared in include/moe.h).

The library is loaded from this package directory only; a missing library raises immediately,
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP, MOE_ENOSCRATCH, MOE_ETIMEOUT = 0, 1, 2, 3, 4, 5
MOE_PERMUTE_STATIC_SCRATCH_BYTES = 8 << 20
MOE_BF16, MOE_MXFP8 = 0, 1

# every function the header declares, for the symbol check
EXPORTS = [
    "moe_status_string", "moe_abi_version", "moe_check_e4m3",
    "moe_prepared_weight_bytes", "moe_prepare_weights",
    "moe_route_workspace_bytes", "moe_route",
    "moe_permute_workspace_bytes", "moe_permute", "moe_permute_static",
    "moe_expert_ffn_workspace_bytes", "moe_expert_ffn",
    "moe_combine",
    "moe_forward_workspace_bytes", "moe_forward", "moe_forward_profiled", "moe_forward_views",
    "moe_forward_ring_tokens", "moe_forward_ring",
    "moe_forward_persistent_workspace_bytes", "moe_forward_persistent",
    "moe_saved_bytes", "moe_prepared_bwd_weight_bytes", "moe_prepare_bwd_weights",
    "moe_backward_workspace_bytes", "moe_backward", "moe_backward_layer",
    "moe_backward_profiled",
]

MOE_PROFILE_EVENTS = 10
STAGES = ["router_logits", "topk", "schedule", "gather", "tile_table", "gemm1_gate_up_swiglu",
          "gemm2_down", "shared_expert", "combine"]
MOE_BWD_PROFILE_EVENTS = 9
BWD_STAGES = ["tables", "uncombine", "dgrad_dh_dswiglu", "dgrad_da", "unpermute", "transposes",
              "wgrad_gate_up", "wgrad_down"]


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("h", ctypes.c_int32), ("m", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("E_loc", ctypes.c_int32),
                ("m_shared", ctypes.c_int32)]


class MoeForwardViews(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("logits", "topk_idx", "topk_w", "counts", "offsets", "perm", "inv", "rows",
                 "row_scales", "out_rows", "shared_out")]


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} returned {code}: {msg}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree library (raise if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m routing_expert_grouped_amd.build` "
            "(the MoE path has no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, S, I, Z = ctypes.c_void_p, ctypes.POINTER(MoeShape), ctypes.c_int, ctypes.c_size_t
    sig = {
        "moe_status_string": (ctypes.c_char_p, [I]),
        "moe_abi_version": (I, []),
        "moe_check_e4m3": (I, [P, P]),
        "moe_prepared_weight_bytes": (Z, [S, I]),
        "moe_prepare_weights": (I, [S, I, P, P, P, P, P]),
        "moe_route_workspace_bytes": (Z, [S]),
        "moe_route": (I, [S, P, P, P, P, P, P, P, P]),
        "moe_permute_workspace_bytes": (Z, [S]),
        "moe_permute": (I, [S, I, P, P, P, P, P, P, P, P, P, P]),
        "moe_permute_static": (I, [S, I, P, P, P, P, P, P, P, P, P]),
        "moe_expert_ffn_workspace_bytes": (Z, [S, I]),
        "moe_expert_ffn": (I, [S, I, P, P, P, P, P, P, P]),
        "moe_combine": (I, [S, P, P, P, P, P, P]),
        "moe_forward_workspace_bytes": (Z, [S, I]),
        "moe_forward": (I, [S, I, P, P, P, P, P, P, P, P, P, P, P]),
        "moe_forward_profiled": (I, [S, I, P, P, P, P, P, P, P, P, P, P, P, P]),
        "moe_forward_views": (I, [S, I, P, ctypes.POINTER(MoeForwardViews)]),
        "moe_forward_ring_tokens": (ctypes.c_int32, [S, I, Z]),
        "moe_forward_ring": (I, [S, I, P, P, P, P, P, P, P, P, P, Z, ctypes.POINTER(ctypes.c_int32),
                                 P]),
        "moe_forward_persistent_workspace_bytes": (Z, [S, I]),
        "moe_forward_persistent": (I, [S, I, P, P, P, P, P, P, P, P, P, ctypes.c_int32, P]),
        "moe_saved_bytes": (Z, [S, I]),
        "moe_prepared_bwd_weight_bytes": (Z, [S, I]),
        "moe_prepare_bwd_weights": (I, [S, I, P, P, P, P, P]),
        "moe_backward_workspace_bytes": (Z, [S, I]),
        "moe_backward": (I, [S, I, P, P, P, P, P, P, P, P, I, P, P]),
        "moe_backward_layer": (I, [S, I, P, P, P, P, P, P, P, P, P, I, P, P, P, P, P]),
        "moe_backward_profiled": (I, [S, I, P, P, P, P, P, P, P, P, I, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn: str, code: int) -> None:
    if code != MOE_OK:
        msg = load().moe_status_string(code).decode()
        raise MoeError(fn, code, msg)
