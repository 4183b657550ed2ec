"""MI355X (gfx950) single-GPU mixture-of-experts layer: Python binding of libmoe_mi355x.so.

Every function here marshals torch tensors (device memory) and the current torch stream into the
C ABI of include/moe.h and allocates outputs the caller did not pass; all computation happens in
the library's HIP kernels. The names follow the C entry points.

Tensors: bfloat16 tensors for bf16 data, torch.uint8 for E4M3 codes / E8M0 scales / prepared
weights / workspaces, int32 for indices, float32 for logits and gate weights. All must be
contiguous CUDA tensors.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from ._lib import (BWD_STAGES, MOE_BF16, MOE_BWD_PROFILE_EVENTS, MOE_MXFP8,
                   MOE_PERMUTE_STATIC_SCRATCH_BYTES, MOE_PROFILE_EVENTS, STAGES, MoeError,
                   MoeForwardViews, MoeShape, check, load)

__all__ = [
    "MOE_BF16", "MOE_MXFP8", "MoeError", "make_shape", "dtype_code",
    "moe_prepared_weight_bytes", "moe_prepare_weights", "moe_route", "moe_permute_workspace_bytes",
    "moe_permute", "moe_permute_static", "moe_expert_ffn_workspace_bytes", "moe_expert_ffn", "moe_combine",
    "moe_forward_workspace_bytes", "moe_forward", "moe_forward_profiled", "moe_forward_views",
    "moe_forward_ring_tokens", "moe_forward_ring",
    "moe_forward_persistent_workspace_bytes", "moe_forward_persistent", "moe_check_e4m3",
    "HipEvents", "STAGES", "BWD_STAGES", "MOE_BWD_PROFILE_EVENTS",
    "moe_saved_bytes", "moe_prepared_bwd_weight_bytes", "moe_prepare_bwd_weights",
    "moe_backward_workspace_bytes", "moe_backward", "moe_backward_layer",
    "moe_backward_profiled",
]


def make_shape(T: int, h: int, m: int, E: int, k: int, E_loc: Optional[int] = None,
               m_shared: int = 0) -> MoeShape:
    return MoeShape(T, h, m, E, k, E if E_loc is None else E_loc, m_shared)


def dtype_code(dtype) -> int:
    if dtype in (MOE_BF16, "bf16"):
        return MOE_BF16
    if dtype in (MOE_MXFP8, "mxfp8"):
        return MOE_MXFP8
    raise ValueError(f"unknown expert dtype {dtype!r}")


def _stream_obj(stream):
    """The torch stream the call enqueues on (None: the current stream; a raw hipStream_t handle
    is wrapped). Buffers the binding allocates are allocated on it, so the caching allocator does
    not hand them out again while that stream's kernels still use them."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _stream(stream) -> int:
    return _stream_obj(stream).cuda_stream


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, numel: Optional[int] = None):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: need a contiguous CUDA tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _buf(t: Optional[torch.Tensor], name: str, nbytes: int):
    """Pointer of a caller-owned byte buffer (workspace, saved state, prepared weights) that must
    hold at least nbytes bytes: a smaller one would be written past its end by the kernels."""
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: need a contiguous CUDA tensor")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name}: {have} bytes, the shape needs {nbytes}")
    return t.data_ptr()


def _dev(ref: torch.Tensor):
    return ref.device


def moe_prepared_weight_bytes(shape: MoeShape, dtype) -> int:
    return load().moe_prepared_weight_bytes(ctypes.byref(shape), dtype_code(dtype))


def moe_prepare_weights(shape: MoeShape, dtype, w_gate, w_up, w_down, prepared=None, stream=None):
    dt = dtype_code(dtype)
    n = moe_prepared_weight_bytes(shape, dt)
    if n == 0:
        raise MoeError("moe_prepared_weight_bytes", 1, "shape rejected")
    st = _stream_obj(stream)
    if prepared is None:
        with torch.cuda.stream(st):
            prepared = torch.empty(n, dtype=torch.uint8, device=_dev(w_gate))
    e, h, m = shape.E_loc, shape.h, shape.m
    check("moe_prepare_weights", load().moe_prepare_weights(
        ctypes.byref(shape), dt,
        _ptr(w_gate, "w_gate", torch.bfloat16, e * h * m),
        _ptr(w_up, "w_up", torch.bfloat16, e * h * m),
        _ptr(w_down, "w_down", torch.bfloat16, e * m * h),
        _ptr(prepared, "prepared", torch.uint8, n), st.cuda_stream))
    return prepared


def moe_route_workspace_bytes(shape: MoeShape) -> int:
    return load().moe_route_workspace_bytes(ctypes.byref(shape))


def moe_route(shape: MoeShape, x, w_router, bias=None, logits=None, topk_idx=None, topk_w=None,
              ws=None, stream=None):
    T, E, k = shape.T, shape.E, shape.k
    dev = _dev(x)
    n = moe_route_workspace_bytes(shape)
    if n == 0:
        raise MoeError("moe_route_workspace_bytes", 1, "shape rejected")
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        ws = torch.empty(n, dtype=torch.uint8, device=dev) if ws is None else ws
        logits = torch.empty(T, E, dtype=torch.float32, device=dev) if logits is None else logits
        topk_idx = torch.empty(T, k, dtype=torch.int32, device=dev) if topk_idx is None \
            else topk_idx
        topk_w = torch.empty(T, k, dtype=torch.float32, device=dev) if topk_w is None else topk_w
    check("moe_route", load().moe_route(
        ctypes.byref(shape), _ptr(x, "x", torch.bfloat16, T * shape.h),
        _ptr(w_router, "w_router", torch.bfloat16, E * shape.h),
        _ptr(bias, "bias", torch.float32, E),
        _ptr(logits, "logits", torch.float32, T * E),
        _ptr(topk_idx, "topk_idx", torch.int32, T * k),
        _ptr(topk_w, "topk_w", torch.float32, T * k), _buf(ws, "ws", n), st.cuda_stream))
    return logits, topk_idx, topk_w


def moe_permute_workspace_bytes(shape: MoeShape) -> int:
    return load().moe_permute_workspace_bytes(ctypes.byref(shape))


def moe_permute(shape: MoeShape, dtype, assign, x, out: Optional[dict] = None, ws=None,
                stream=None) -> dict:
    dt = dtype_code(dtype)
    T, h, k, E_loc = shape.T, shape.h, shape.k, shape.E_loc
    R = T * k
    dev = _dev(x)
    mx = dt == MOE_MXFP8
    nws = moe_permute_workspace_bytes(shape)
    if nws == 0:
        raise MoeError("moe_permute_workspace_bytes", 1, "shape rejected")
    st = _stream_obj(stream)
    o = dict(out or {})
    with torch.cuda.stream(st):
        o.setdefault("counts", torch.empty(E_loc, dtype=torch.int32, device=dev))
        o.setdefault("offsets", torch.empty(E_loc + 1, dtype=torch.int32, device=dev))
        o.setdefault("perm", torch.empty(R, dtype=torch.int32, device=dev))
        o.setdefault("inv", torch.empty(R, dtype=torch.int32, device=dev))
        if mx:
            o.setdefault("rows", torch.empty(R, h, dtype=torch.uint8, device=dev))
            o.setdefault("row_scales", torch.empty(R, h // 32, dtype=torch.uint8, device=dev))
        else:
            o.setdefault("rows", torch.empty(R, h, dtype=torch.bfloat16, device=dev))
            o.setdefault("row_scales", None)
        ws = torch.empty(nws, dtype=torch.uint8, device=dev) if ws is None else ws
    check("moe_permute", load().moe_permute(
        ctypes.byref(shape), dt, _ptr(assign, "assign", torch.int32, R),
        _ptr(x, "x", torch.bfloat16, T * h), _ptr(o["counts"], "counts", torch.int32, E_loc),
        _ptr(o["offsets"], "offsets", torch.int32, E_loc + 1),
        _ptr(o["perm"], "perm", torch.int32, R), _ptr(o["inv"], "inv", torch.int32, R),
        _ptr(o["rows"], "rows", torch.uint8 if mx else torch.bfloat16, R * h),
        _ptr(o["row_scales"], "row_scales", torch.uint8, R * (h // 32)) if mx else None,
        _buf(ws, "ws", nws), st.cuda_stream))
    return o


def moe_permute_static(shape: MoeShape, dtype, assign, x, out: dict, stream=None) -> dict:
    """moe_permute with the schedule's scratch in the library's static per-GPU array (the C call
    allocates nothing). Every output buffer is the caller's: out holds counts, offsets, perm, inv,
    rows (and row_scales for MXFP8), as moe_permute returns them. Calls that overlap in time on
    one GPU share that array and race."""
    dt = dtype_code(dtype)
    T, h, k, E_loc = shape.T, shape.h, shape.k, shape.E_loc
    R = T * k
    mx = dt == MOE_MXFP8
    check("moe_permute_static", load().moe_permute_static(
        ctypes.byref(shape), dt, _ptr(assign, "assign", torch.int32, R),
        _ptr(x, "x", torch.bfloat16, T * h), _ptr(out["counts"], "counts", torch.int32, E_loc),
        _ptr(out["offsets"], "offsets", torch.int32, E_loc + 1),
        _ptr(out["perm"], "perm", torch.int32, R), _ptr(out["inv"], "inv", torch.int32, R),
        _ptr(out["rows"], "rows", torch.uint8 if mx else torch.bfloat16, R * h),
        _ptr(out["row_scales"], "row_scales", torch.uint8, R * (h // 32)) if mx else None,
        _stream(stream)))
    return out


def moe_expert_ffn_workspace_bytes(shape: MoeShape, dtype) -> int:
    return load().moe_expert_ffn_workspace_bytes(ctypes.byref(shape), dtype_code(dtype))


def moe_expert_ffn(shape: MoeShape, dtype, rows, row_scales, offsets, prepared, out_rows=None,
                   ws=None, stream=None):
    dt = dtype_code(dtype)
    R, h = shape.T * shape.k, shape.h
    mx = dt == MOE_MXFP8
    dev = _dev(rows)
    n = moe_expert_ffn_workspace_bytes(shape, dt)
    if n == 0:
        raise MoeError("moe_expert_ffn_workspace_bytes", 1, "shape rejected")
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        out_rows = torch.empty(R, h, dtype=torch.bfloat16, device=dev) if out_rows is None \
            else out_rows
        ws = torch.empty(n, dtype=torch.uint8, device=dev) if ws is None else ws
    check("moe_expert_ffn", load().moe_expert_ffn(
        ctypes.byref(shape), dt, _ptr(rows, "rows", torch.uint8 if mx else torch.bfloat16, R * h),
        _ptr(row_scales, "row_scales", torch.uint8, R * (h // 32)) if mx else None,
        _ptr(offsets, "offsets", torch.int32, shape.E_loc + 1),
        _buf(prepared, "prepared", moe_prepared_weight_bytes(shape, dt)),
        _ptr(out_rows, "out_rows", torch.bfloat16, R * h), _buf(ws, "ws", n), st.cuda_stream))
    return out_rows


def moe_combine(shape: MoeShape, out_rows, inv, topk_w, shared_out=None, y=None, stream=None):
    T, h, k = shape.T, shape.h, shape.k
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        y = torch.empty(T, h, dtype=torch.bfloat16, device=_dev(out_rows)) if y is None else y
    check("moe_combine", load().moe_combine(
        ctypes.byref(shape), _ptr(out_rows, "out_rows", torch.bfloat16, T * k * h),
        _ptr(inv, "inv", torch.int32, T * k), _ptr(topk_w, "topk_w", torch.float32, T * k),
        _ptr(shared_out, "shared_out", torch.bfloat16, T * h),
        _ptr(y, "y", torch.bfloat16, T * h), st.cuda_stream))
    return y


def moe_forward_workspace_bytes(shape: MoeShape, dtype) -> int:
    return load().moe_forward_workspace_bytes(ctypes.byref(shape), dtype_code(dtype))


def _forward_args(shape, dtype, x, prepared, w_router, bias, assign, assign_w, shared_prepared,
                  y, ws, saved, stream):
    """Checked argument list of moe_forward / moe_forward_profiled (without events and stream),
    and the buffers the call writes."""
    dt = dtype_code(dtype)
    T, h, k, E = shape.T, shape.h, shape.k, shape.E
    dev = _dev(x)
    n = moe_forward_workspace_bytes(shape, dt)
    if n == 0:
        raise MoeError("moe_forward_workspace_bytes", 1, "shape rejected")
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        y = torch.empty(T, h, dtype=torch.bfloat16, device=dev) if y is None else y
        ws = torch.empty(n, dtype=torch.uint8, device=dev) if ws is None else ws
    nsaved = moe_saved_bytes(shape, dt) if saved is not None else 0
    if saved is not None and nsaved == 0:
        raise MoeError("moe_saved_bytes", 2, "shape has no backward")
    nshared = 0
    if shared_prepared is not None:
        nshared = moe_prepared_weight_bytes(make_shape(T, h, shape.m_shared, 1, 1, 1), MOE_BF16)
    args = [ctypes.byref(shape), dt, _ptr(x, "x", torch.bfloat16, T * h),
            _ptr(w_router, "w_router", torch.bfloat16, E * h),
            _ptr(bias, "bias", torch.float32, E),
            _ptr(assign, "assign", torch.int32, T * k),
            _ptr(assign_w, "assign_w", torch.float32, T * k),
            _buf(prepared, "prepared", moe_prepared_weight_bytes(shape, dt)),
            _buf(shared_prepared, "shared_prepared", nshared),
            _ptr(y, "y", torch.bfloat16, T * h), _buf(saved, "saved", nsaved),
            _buf(ws, "ws", n)]
    return args, y, ws, st


def moe_forward(shape: MoeShape, dtype, x, prepared, w_router=None, bias=None, assign=None,
                assign_w=None, shared_prepared=None, y=None, ws=None, saved=None, stream=None):
    """The whole layer. Returns (y, ws); moe_forward_views(shape, dtype, ws) exposes the
    intermediates left in ws. saved: a moe_saved_bytes() uint8 tensor that receives what
    moe_backward needs, or None."""
    args, y, ws, st = _forward_args(shape, dtype, x, prepared, w_router, bias, assign, assign_w,
                                    shared_prepared, y, ws, saved, stream)
    check("moe_forward", load().moe_forward(*args, st.cuda_stream))
    return y, ws


def moe_forward_ring_tokens(shape: MoeShape, dtype, ring_bytes: int) -> int:
    """Tokens per minibatch of moe_forward_ring with a ring of ring_bytes bytes (0: too small)."""
    return load().moe_forward_ring_tokens(ctypes.byref(shape), dtype_code(dtype), ring_bytes)


def moe_forward_ring(shape: MoeShape, dtype, x, prepared, ring, w_router=None, bias=None,
                     assign=None, assign_w=None, shared_prepared=None, y=None, stream=None):
    """The forward of all T tokens through the fixed buffer `ring` (a uint8 CUDA tensor), in
    minibatches of moe_forward_ring_tokens(shape, dtype, ring.numel()) tokens. Returns
    (y, minibatch_tokens)."""
    dt = dtype_code(dtype)
    T, h, k, E = shape.T, shape.h, shape.k, shape.E
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        y = torch.empty(T, h, dtype=torch.bfloat16, device=_dev(x)) if y is None else y
    nshared = 0
    if shared_prepared is not None:
        nshared = moe_prepared_weight_bytes(make_shape(T, h, shape.m_shared, 1, 1, 1), MOE_BF16)
    if not ring.is_cuda or not ring.is_contiguous():
        raise ValueError("ring: need a contiguous CUDA tensor")
    nb = ring.numel() * ring.element_size()
    tmb = ctypes.c_int32(0)
    check("moe_forward_ring", load().moe_forward_ring(
        ctypes.byref(shape), dt, _ptr(x, "x", torch.bfloat16, T * h),
        _ptr(w_router, "w_router", torch.bfloat16, E * h), _ptr(bias, "bias", torch.float32, E),
        _ptr(assign, "assign", torch.int32, T * k),
        _ptr(assign_w, "assign_w", torch.float32, T * k),
        _buf(prepared, "prepared", moe_prepared_weight_bytes(shape, dt)),
        _buf(shared_prepared, "shared_prepared", nshared), _ptr(y, "y", torch.bfloat16, T * h),
        ring.data_ptr(), nb, ctypes.byref(tmb), st.cuda_stream))
    return y, tmb.value


def moe_check_e4m3(stream=None) -> int:
    """Runs the library's E4M3 encoder against the rounding rule on every float32 below 2^17 on the
    current device; returns the number of mismatching inputs (synchronises the stream)."""
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        out = torch.zeros(1, dtype=torch.int64, device="cuda")
    check("moe_check_e4m3", load().moe_check_e4m3(out.data_ptr(), st.cuda_stream))
    st.synchronize()
    return int(out.item())


def moe_forward_persistent_workspace_bytes(shape: MoeShape, dtype) -> int:
    return load().moe_forward_persistent_workspace_bytes(ctypes.byref(shape), dtype_code(dtype))


def moe_forward_persistent(shape: MoeShape, dtype, x, prepared, w_router=None, bias=None,
                           assign=None, assign_w=None, y=None, ws=None, status=None,
                           timeout_ms: int = 2000, stream=None):
    """The forward in one persistent kernel (no saved state, no shared expert). Returns
    (y, ws, status): status is a 1-element int32 CUDA tensor, MOE_OK or MOE_ETIMEOUT once the
    stream has run."""
    dt = dtype_code(dtype)
    T, h, k, E = shape.T, shape.h, shape.k, shape.E
    dev = _dev(x)
    n = moe_forward_persistent_workspace_bytes(shape, dt)
    if n == 0:
        raise MoeError("moe_forward_persistent_workspace_bytes", 2, "shape not covered")
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        y = torch.empty(T, h, dtype=torch.bfloat16, device=dev) if y is None else y
        ws = torch.empty(n, dtype=torch.uint8, device=dev) if ws is None else ws
        status = torch.empty(1, dtype=torch.int32, device=dev) if status is None else status
    check("moe_forward_persistent", load().moe_forward_persistent(
        ctypes.byref(shape), dt, _ptr(x, "x", torch.bfloat16, T * h),
        _ptr(w_router, "w_router", torch.bfloat16, E * h), _ptr(bias, "bias", torch.float32, E),
        _ptr(assign, "assign", torch.int32, T * k),
        _ptr(assign_w, "assign_w", torch.float32, T * k),
        _buf(prepared, "prepared", moe_prepared_weight_bytes(shape, dt)),
        _ptr(y, "y", torch.bfloat16, T * h), _buf(ws, "ws", n),
        _ptr(status, "status", torch.int32, 1), int(timeout_ms), st.cuda_stream))
    return y, ws, status


class HipEvents:
    """Timing events from the HIP runtime (hipEventCreate / ElapsedTime), one per stage boundary
    of a profiled forward (default) or backward (names=BWD_STAGES)."""

    def __init__(self, n: int = MOE_PROFILE_EVENTS, names=None):
        self.names = list(STAGES if names is None else names)
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.handles = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles[i] = h
        self.n = n

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.handles[i], self.handles[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def synchronize(self) -> None:
        self._hip.hipEventSynchronize(self.handles[self.n - 1])

    def stage_ms(self) -> dict:
        """Milliseconds of each stage of the last profiled forward."""
        return {name: self.elapsed_ms(i, i + 1) for i, name in enumerate(self.names)}

    def close(self) -> None:
        for i in range(self.n):
            if self.handles[i]:
                self._hip.hipEventDestroy(self.handles[i])
                self.handles[i] = None


def moe_forward_profiled(shape: MoeShape, dtype, x, prepared, events: HipEvents, w_router=None,
                         bias=None, assign=None, assign_w=None, shared_prepared=None, y=None,
                         ws=None, saved=None, stream=None):
    """moe_forward plus HIP events at the stage boundaries (events.stage_ms() afterwards)."""
    if events.n != MOE_PROFILE_EVENTS:
        raise ValueError(f"events: {events.n} handles, moe_forward_profiled records "
                         f"{MOE_PROFILE_EVENTS}")
    args, y, ws, st = _forward_args(shape, dtype, x, prepared, w_router, bias, assign, assign_w,
                                    shared_prepared, y, ws, saved, stream)
    check("moe_forward_profiled", load().moe_forward_profiled(
        *args, ctypes.cast(events.handles, ctypes.c_void_p), st.cuda_stream))
    return y, ws


def moe_forward_views(shape: MoeShape, dtype, ws) -> dict:
    """Tensors viewing the intermediates moe_forward leaves in ws (None where absent)."""
    dt = dtype_code(dtype)
    v = MoeForwardViews()
    check("moe_forward_views", load().moe_forward_views(
        ctypes.byref(shape), dt, ctypes.c_void_p(_buf(ws, "ws", moe_forward_workspace_bytes(
            shape, dt))), ctypes.byref(v)))
    T, h, k, E, E_loc = shape.T, shape.h, shape.k, shape.E, shape.E_loc
    R = T * k
    base = ws.data_ptr()

    def view(ptr, nbytes, dtype_, shp):
        if not ptr:
            return None
        off = ptr - base
        return ws[off:off + nbytes].view(dtype_).view(*shp)

    mx = dt == MOE_MXFP8
    return {
        "logits": view(v.logits, T * E * 4, torch.float32, (T, E)),
        "topk_idx": view(v.topk_idx, R * 4, torch.int32, (T, k)),
        "topk_w": view(v.topk_w, R * 4, torch.float32, (T, k)),
        "counts": view(v.counts, E_loc * 4, torch.int32, (E_loc,)),
        "offsets": view(v.offsets, (E_loc + 1) * 4, torch.int32, (E_loc + 1,)),
        "perm": view(v.perm, R * 4, torch.int32, (R,)),
        "inv": view(v.inv, R * 4, torch.int32, (R,)),
        "rows": view(v.rows, R * h * (1 if mx else 2), torch.uint8 if mx else torch.bfloat16,
                     (R, h)),
        "row_scales": view(v.row_scales, R * (h // 32), torch.uint8, (R, h // 32)),
        "out_rows": view(v.out_rows, R * h * 2, torch.bfloat16, (R, h)),
        "shared_out": view(v.shared_out, T * h * 2, torch.bfloat16, (T, h)),
    }


def moe_saved_bytes(shape: MoeShape, dtype) -> int:
    return load().moe_saved_bytes(ctypes.byref(shape), dtype_code(dtype))


def moe_prepared_bwd_weight_bytes(shape: MoeShape, dtype) -> int:
    return load().moe_prepared_bwd_weight_bytes(ctypes.byref(shape), dtype_code(dtype))


def moe_prepare_bwd_weights(shape: MoeShape, dtype, w_gate, w_up, w_down, prepared_bwd=None,
                            stream=None):
    dt = dtype_code(dtype)
    n = moe_prepared_bwd_weight_bytes(shape, dt)
    if n == 0:
        raise MoeError("moe_prepared_bwd_weight_bytes", 2, "shape rejected")
    st = _stream_obj(stream)
    if prepared_bwd is None:
        with torch.cuda.stream(st):
            prepared_bwd = torch.empty(n, dtype=torch.uint8, device=_dev(w_gate))
    e, h, m = shape.E_loc, shape.h, shape.m
    check("moe_prepare_bwd_weights", load().moe_prepare_bwd_weights(
        ctypes.byref(shape), dt,
        _ptr(w_gate, "w_gate", torch.bfloat16, e * h * m),
        _ptr(w_up, "w_up", torch.bfloat16, e * h * m),
        _ptr(w_down, "w_down", torch.bfloat16, e * m * h),
        _ptr(prepared_bwd, "prepared_bwd", torch.uint8, n), st.cuda_stream))
    return prepared_bwd


def moe_backward_workspace_bytes(shape: MoeShape, dtype) -> int:
    return load().moe_backward_workspace_bytes(ctypes.byref(shape), dtype_code(dtype))


def _backward_args(shape, dtype, x, dy, saved, prepared_bwd, dx, dw, dw_fp32, ws, stream):
    dt = dtype_code(dtype)
    T, h, m, E_loc = shape.T, shape.h, shape.m, shape.E_loc
    dev = _dev(x)
    wdt = torch.float32 if dw_fp32 else torch.bfloat16
    n = moe_backward_workspace_bytes(shape, dt)
    if n == 0:
        raise MoeError("moe_backward_workspace_bytes", 2, "shape rejected")
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        dx = torch.empty(T, h, dtype=torch.bfloat16, device=dev) if dx is None else dx
        if dw is None:
            dw = (torch.empty(E_loc, h, m, dtype=wdt, device=dev),
                  torch.empty(E_loc, h, m, dtype=wdt, device=dev),
                  torch.empty(E_loc, m, h, dtype=wdt, device=dev))
        ws = torch.empty(n, dtype=torch.uint8, device=dev) if ws is None else ws
    args = [ctypes.byref(shape), dt, _ptr(x, "x", torch.bfloat16, T * h),
            _ptr(dy, "dy", torch.bfloat16, T * h),
            _buf(saved, "saved", moe_saved_bytes(shape, dt)),
            _buf(prepared_bwd, "prepared_bwd", moe_prepared_bwd_weight_bytes(shape, dt)),
            _ptr(dx, "dx", torch.bfloat16, T * h),
            _ptr(dw[0], "dw_gate", wdt, E_loc * h * m), _ptr(dw[1], "dw_up", wdt, E_loc * h * m),
            _ptr(dw[2], "dw_down", wdt, E_loc * m * h), 1 if dw_fp32 else 0, _buf(ws, "ws", n)]
    return args, dx, dw, ws, st


def moe_backward(shape: MoeShape, dtype, x, dy, saved, prepared_bwd, dx=None, dw=None,
                 dw_fp32: bool = True, ws=None, stream=None):
    """Backward of the expert path. Returns (dx, (dw_gate, dw_up, dw_down), ws)."""
    args, dx, dw, ws, st = _backward_args(shape, dtype, x, dy, saved, prepared_bwd, dx, dw,
                                          dw_fp32, ws, stream)
    check("moe_backward", load().moe_backward(*args, st.cuda_stream))
    return dx, dw, ws


def moe_backward_layer(shape: MoeShape, dtype, x, dy, saved, prepared_bwd, w_router=None,
                       dx=None, dw=None, dw_fp32: bool = True, dgate=None, dw_router=None,
                       dbias=None, ws=None, stream=None):
    """The whole layer's backward: the expert path plus the gate-weight gradients dgate [T*k]
    and, with w_router (router use), the router matrix and bias gradients (its part of dx is
    included). Returns (dx, (dw_gate, dw_up, dw_down), dgate, dw_router, dbias, ws); dw_router
    and dbias are None for an expert share."""
    args, dx, dw, ws, st = _backward_args(shape, dtype, x, dy, saved, prepared_bwd, dx, dw,
                                          dw_fp32, ws, stream)
    T, k, E, h = shape.T, shape.k, shape.E, shape.h
    dev = _dev(x)
    with torch.cuda.stream(st):
        dgate = torch.empty(T * k, dtype=torch.float32, device=dev) if dgate is None else dgate
        if w_router is not None:
            dw_router = torch.empty(E, h, dtype=torch.float32, device=dev) if dw_router is None \
                else dw_router
            dbias = torch.empty(E, dtype=torch.float32, device=dev) if dbias is None else dbias
    # insert w_router after x, then the gate outputs before ws
    largs = args[:3] + [_ptr(w_router, "w_router", torch.bfloat16, E * h)] + args[3:11] + [
        _ptr(dgate, "dgate", torch.float32, T * k),
        _ptr(dw_router, "dw_router", torch.float32, E * h),
        _ptr(dbias, "dbias", torch.float32, E)] + args[11:]
    check("moe_backward_layer", load().moe_backward_layer(*largs, st.cuda_stream))
    return dx, dw, dgate, dw_router, dbias, ws


def moe_backward_profiled(shape: MoeShape, dtype, x, dy, saved, prepared_bwd, events: HipEvents,
                          dx=None, dw=None, dw_fp32: bool = True, ws=None, stream=None):
    """moe_backward plus HIP events at its stage boundaries (events.stage_ms() afterwards; create
    the events with HipEvents(MOE_BWD_PROFILE_EVENTS, BWD_STAGES))."""
    if events.n != MOE_BWD_PROFILE_EVENTS:
        raise ValueError(f"events: {events.n} handles, moe_backward_profiled records "
                         f"{MOE_BWD_PROFILE_EVENTS}")
    args, dx, dw, ws, st = _backward_args(shape, dtype, x, dy, saved, prepared_bwd, dx, dw,
                                          dw_fp32, ws, stream)
    check("moe_backward_profiled", load().moe_backward_profiled(
        *args, ctypes.cast(events.handles, ctypes.c_void_p), st.cuda_stream))
    return dx, dw, ws
