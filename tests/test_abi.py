"""The C-ABI library without a GPU: it loads, exports every function include/moe.h declares, its
size queries are consistent, and invalid arguments are rejected on the host before anything is
enqueued (every call below fails validation, so no HIP work is ever launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    from routing_expert_grouped_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from routing_expert_grouped_amd import build
        build.build(verbose=False)
    return _lib


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    L = lib.load()
    declared = _declared_functions()
    assert sorted(lib.EXPORTS) == declared
    for name in declared:
        assert hasattr(L, name), name


def test_version_and_status_strings(lib):
    L = lib.load()
    assert L.moe_abi_version() == 5
    for code in range(6):
        assert L.moe_status_string(code).decode().startswith("MOE_")


def _shape(lib, **kw):
    base = dict(T=64, h=256, m=128, E=8, k=2, E_loc=8, m_shared=0)
    base.update(kw)
    return lib.MoeShape(**base)


def test_size_queries(lib):
    L = lib.load()
    s = _shape(lib)
    R, h, m, E = 128, 256, 128, 8
    assert L.moe_prepared_weight_bytes(ctypes.byref(s), 0) == 3 * E * h * m * 2
    mx = _shape(lib, m=256)
    n = L.moe_prepared_weight_bytes(ctypes.byref(mx), 1)
    assert n >= 3 * E * h * 256 * (1 + 1 / 32)
    assert L.moe_forward_workspace_bytes(ctypes.byref(s), 0) > R * h * 4
    assert L.moe_expert_ffn_workspace_bytes(ctypes.byref(s), 0) >= R * m * 2
    assert L.moe_permute_workspace_bytes(ctypes.byref(s)) > 0
    # rejected shapes size to 0
    assert L.moe_prepared_weight_bytes(ctypes.byref(_shape(lib, h=200)), 0) == 0
    assert L.moe_forward_workspace_bytes(ctypes.byref(_shape(lib, k=0)), 0) == 0


FAKE = 1 << 20  # aligned, never dereferenced: each call below fails validation first


def test_route_validation(lib):
    L = lib.load()
    P = FAKE
    ok = _shape(lib)
    assert L.moe_route(None, P, P, None, P, P, P, P, None) == lib.MOE_EINVAL
    assert L.moe_route(ctypes.byref(_shape(lib, k=9)), P, P, None, P, P, P, P, None) == lib.MOE_EINVAL
    assert L.moe_route(ctypes.byref(_shape(lib, E=8, E_loc=4)), P, P, None, P, P, P, P, None) == \
        lib.MOE_EINVAL
    assert L.moe_route(ctypes.byref(ok), None, P, None, P, P, P, P, None) == lib.MOE_EINVAL
    assert L.moe_route(ctypes.byref(ok), P + 2, P, None, P, P, P, P, None) == lib.MOE_EINVAL
    assert L.moe_route(ctypes.byref(ok), P, P, P + 4, P, P, P, P, None) == lib.MOE_EINVAL
    assert L.moe_route(ctypes.byref(ok), P, P, None, P, P, P, None, None) == lib.MOE_EINVAL  # ws
    assert L.moe_route_workspace_bytes(ctypes.byref(ok)) > 0
    assert L.moe_route_workspace_bytes(ctypes.byref(_shape(lib, k=9))) == 0
    assert L.moe_route(ctypes.byref(_shape(lib, E=2000, E_loc=2000)), P, P, None, P, P, P, P,
                       None) == lib.MOE_EUNSUPPORTED
    assert L.moe_route(ctypes.byref(_shape(lib, E=40, E_loc=40, k=17)), P, P, None, P, P, P, P,
                       None) == lib.MOE_EUNSUPPORTED


def test_expert_path_validation(lib):
    L = lib.load()
    P = FAKE
    ok = _shape(lib)
    # permute
    assert L.moe_permute(ctypes.byref(ok), 0, None, P, P, P, P, P, P, None, P, None) == \
        lib.MOE_EINVAL
    assert L.moe_permute(ctypes.byref(_shape(lib, m=256)), 1, P, P, P, P, P, P, P, None, P,
                         None) == lib.MOE_EINVAL  # MXFP8 needs row_scales
    assert L.moe_permute(ctypes.byref(ok), 7, P, P, P, P, P, P, P, None, P, None) == \
        lib.MOE_EINVAL  # unknown dtype
    # expert ffn: shapes the kernels do not tile
    assert L.moe_expert_ffn(ctypes.byref(_shape(lib, h=192)), 0, P, None, P, P, P, P, None) == \
        lib.MOE_EUNSUPPORTED
    assert L.moe_expert_ffn(ctypes.byref(_shape(lib, m=96)), 0, P, None, P, P, P, P, None) == \
        lib.MOE_EUNSUPPORTED
    assert L.moe_expert_ffn(ctypes.byref(_shape(lib, h=240)), 1, P, P, P, P, P, P, None) == \
        lib.MOE_EINVAL  # MXFP8 needs h % 32 == 0
    assert L.moe_expert_ffn(ctypes.byref(_shape(lib, m=128)), 1, P, P, P, P, P, P, None) == \
        lib.MOE_EUNSUPPORTED  # MXFP8 K chunks are 256 wide
    assert L.moe_expert_ffn(ctypes.byref(ok), 0, P, None, P, None, P, P, None) == lib.MOE_EINVAL
    # combine
    assert L.moe_combine(ctypes.byref(_shape(lib, k=17)), P, P, P, None, P, None) == \
        lib.MOE_EUNSUPPORTED
    assert L.moe_combine(ctypes.byref(ok), P, P, None, None, P, None) == lib.MOE_EINVAL
    # forward: router and share arguments are exclusive; shared expert consistency
    assert L.moe_forward(ctypes.byref(ok), 0, P, P, None, P, P, P, None, P, None, P, None) == \
        lib.MOE_EINVAL
    assert L.moe_forward(ctypes.byref(ok), 0, P, None, None, None, None, P, None, P, None, P,
                         None) == lib.MOE_EINVAL
    assert L.moe_forward(ctypes.byref(_shape(lib, m_shared=128)), 0, P, P, None, None, None, P,
                         None, P, None, P, None) == lib.MOE_EINVAL
    assert L.moe_forward(ctypes.byref(ok), 0, P, P, None, None, None, P, None, P, None, None,
                         None) == lib.MOE_EINVAL
    # a training forward (saved != NULL) needs m % 256 == 0 and an aligned buffer
    assert L.moe_forward(ctypes.byref(ok), 0, P, P, None, None, None, P, None, P, P, P, None) == \
        lib.MOE_EUNSUPPORTED
    assert L.moe_forward(ctypes.byref(_shape(lib, m=256)), 0, P, P, None, None, None, P, None, P,
                         P + 8, P, None) == lib.MOE_EINVAL
    # prepare weights
    assert L.moe_prepare_weights(ctypes.byref(ok), 0, P, P, None, P, None) == lib.MOE_EINVAL


def test_views_are_host_arithmetic(lib):
    L = lib.load()
    s = _shape(lib)
    v = lib.MoeForwardViews()
    base = 1 << 30
    assert L.moe_forward_views(ctypes.byref(s), 0, base, ctypes.byref(v)) == lib.MOE_OK
    ptrs = [getattr(v, n) for n, _ in lib.MoeForwardViews._fields_ if getattr(v, n)]
    assert all(p % 256 == 0 and base <= p < base + L.moe_forward_workspace_bytes(
        ctypes.byref(s), 0) for p in ptrs)
    assert v.row_scales is None and v.shared_out is None and v.logits is not None


def test_backward_sizes_and_validation(lib):
    L = lib.load()
    P = FAKE
    ok = _shape(lib, m=256)
    R, h, m, E = 128, 256, 256, 8
    for dt in (0, 1):
        el = 2 if dt == 0 else 1
        assert L.moe_saved_bytes(ctypes.byref(ok), dt) >= R * (12 + 2 * m * 2)
        assert L.moe_prepared_bwd_weight_bytes(ctypes.byref(ok), dt) >= 3 * E * h * m * el
        assert L.moe_backward_workspace_bytes(ctypes.byref(ok), dt) > R * h * 2
        # m % 256 != 0: not covered by the backward
        assert L.moe_saved_bytes(ctypes.byref(_shape(lib, m=128)), dt) == 0
        assert L.moe_backward_workspace_bytes(ctypes.byref(_shape(lib, m=128)), dt) == 0
    args = [P, P, P, P, P, P, P, P]  # x dy saved prepared_bwd dx dw_gate dw_up dw_down
    assert L.moe_backward(ctypes.byref(ok), 0, *args, 2, P, None) == lib.MOE_EINVAL
    assert L.moe_backward(ctypes.byref(ok), 0, P, P, None, P, P, P, P, P, 1, P, None) == \
        lib.MOE_EINVAL
    assert L.moe_backward(ctypes.byref(ok), 1, P, P, P, P, P, P, P, P + 4, 1, P, None) == \
        lib.MOE_EINVAL
    assert L.moe_backward(ctypes.byref(_shape(lib, m=128)), 0, *args, 1, P, None) == \
        lib.MOE_EUNSUPPORTED
    assert L.moe_backward_profiled(ctypes.byref(ok), 0, *args, 1, P, None, None) == \
        lib.MOE_EINVAL  # no events
    assert L.moe_prepare_bwd_weights(ctypes.byref(_shape(lib, h=384)), 0, P, P, P, P, None) == \
        lib.MOE_EUNSUPPORTED


def test_binding_buffer_checks_without_gpu():
    """The binding's pointer checks, on stand-in tensors (no GPU needed): a byte buffer smaller
    than the shape's size query is refused, as are wrong dtypes and element counts."""
    import pytest as _pt
    torch = _pt.importorskip("torch")
    import routing_expert_grouped_amd as G

    class Fake:
        is_cuda = True

        def __init__(self, n, dtype=torch.uint8, contiguous=True):
            self.n, self.dtype, self.c = n, dtype, contiguous

        def is_contiguous(self):
            return self.c

        def numel(self):
            return self.n

        def element_size(self):
            return torch.empty(0, dtype=self.dtype).element_size()

        def data_ptr(self):
            return 4096

    assert G._buf(Fake(1000), "ws", 1000) == 4096
    assert G._buf(Fake(250, torch.float32), "ws", 1000) == 4096
    assert G._buf(None, "ws", 1000) is None
    with _pt.raises(ValueError, match="ws: 999 bytes"):
        G._buf(Fake(999), "ws", 1000)
    with _pt.raises(ValueError, match="contiguous"):
        G._buf(Fake(1000, contiguous=False), "ws", 10)
    with _pt.raises(ValueError, match="dtype"):
        G._ptr(Fake(8, torch.float32), "bias", torch.bfloat16, 8)
    with _pt.raises(ValueError, match="elements"):
        G._ptr(Fake(7, torch.float32), "bias", torch.float32, 8)


def test_permute_static_rejects_shapes_beyond_its_scratch(lib):
    """moe_permute_static checks the schedule's scratch size against the static array on the host
    and returns MOE_ENOSCRATCH before touching the GPU (and EINVAL for null pointers first)."""
    L = lib.load()
    big = _shape(lib, T=70000, k=8, h=256, m=128, E=1024, E_loc=1024)
    need = L.moe_permute_workspace_bytes(ctypes.byref(big))
    assert need > lib.MOE_PERMUTE_STATIC_SCRATCH_BYTES
    args = [FAKE] * 8
    assert L.moe_permute_static(ctypes.byref(big), 0, *args, None, None) == lib.MOE_ENOSCRATCH
    small = _shape(lib)
    assert L.moe_permute_workspace_bytes(ctypes.byref(small)) <= \
        lib.MOE_PERMUTE_STATIC_SCRATCH_BYTES
    assert L.moe_permute_static(ctypes.byref(small), 0, None, *args[1:], None, None) == \
        lib.MOE_EINVAL
    assert "static buffer" in L.moe_status_string(lib.MOE_ENOSCRATCH).decode()


def test_forward_ring_minibatch_sizes(lib):
    """moe_forward_ring_tokens is host arithmetic: the largest token count whose forward workspace
    fits the ring (0 when one token does not), non-decreasing in the ring size, T for a ring that
    holds the whole batch; moe_forward_ring refuses a ring that holds no minibatch before any
    launch."""
    L = lib.load()
    # k = 4: any count keeps assign 16-byte aligned; k = 6 (even): pairs; k = 5 (odd): fours
    for k, a in ((4, 1), (6, 2), (5, 4)):
        s = _shape(lib, T=1000, h=512, m=256, E=64, k=k, E_loc=64)
        full = L.moe_forward_workspace_bytes(ctypes.byref(s), 1)
        assert L.moe_forward_ring_tokens(ctypes.byref(s), 1, full) == 1000
        assert L.moe_forward_ring_tokens(ctypes.byref(s), 1, 1 << 40) == 1000
        prev = 0
        for frac in (0.05, 0.1, 0.3, 0.5, 0.9):
            t = L.moe_forward_ring_tokens(ctypes.byref(s), 1, int(full * frac))
            assert prev <= t < 1000 and t % a == 0 and (t * k * 4) % 16 == 0
            one = _shape(lib, T=t, h=512, m=256, E=64, k=k, E_loc=64)
            two = _shape(lib, T=t + a, h=512, m=256, E=64, k=k, E_loc=64)
            assert L.moe_forward_workspace_bytes(ctypes.byref(one), 1) <= int(full * frac) < \
                L.moe_forward_workspace_bytes(ctypes.byref(two), 1)
            prev = t
    s = _shape(lib, T=1000, h=512, m=256, E=64, k=4, E_loc=64)
    assert L.moe_forward_ring_tokens(ctypes.byref(s), 1, 1000) == 0
    tmb = ctypes.c_int32(-1)
    st = L.moe_forward_ring(ctypes.byref(s), 1, FAKE, FAKE, None, None, None, FAKE, None, FAKE,
                            FAKE, 1000, ctypes.byref(tmb), None)
    assert st == lib.MOE_EINVAL and tmb.value == -1


def test_persistent_forward_host_checks(lib):
    """moe_forward_persistent: its workspace holds the forward's plus its own buffers; shapes it
    does not cover (a shared expert, a small-tile shape) and bad arguments are refused on the host
    before any HIP call."""
    L = lib.load()
    s = _shape(lib, T=300, h=768, m=512, E=64, k=8, E_loc=64)
    for dt in (0, 1):
        nf = L.moe_forward_workspace_bytes(ctypes.byref(s), dt)
        npst = L.moe_forward_persistent_workspace_bytes(ctypes.byref(s), dt)
        assert npst > nf > 0
    shared = _shape(lib, T=64, h=512, m=256, E=8, k=2, E_loc=8, m_shared=256)
    assert L.moe_forward_persistent_workspace_bytes(ctypes.byref(shared), 0) == 0
    small = _shape(lib, T=64, h=384, m=128, E=8, k=2, E_loc=8)  # h % 256 != 0: small tiles
    assert L.moe_forward_persistent_workspace_bytes(ctypes.byref(small), 0) == 0
    args = [FAKE, FAKE, None, None, None, FAKE, FAKE, FAKE, FAKE]  # router layer
    assert L.moe_forward_persistent(ctypes.byref(shared), 0, *args, 1000, None) == \
        lib.MOE_EUNSUPPORTED
    assert L.moe_forward_persistent(ctypes.byref(small), 0, *args, 1000, None) == \
        lib.MOE_EUNSUPPORTED
    assert L.moe_forward_persistent(ctypes.byref(s), 0, *args[:-1], None, 1000, None) == \
        lib.MOE_EINVAL  # no status word
    assert L.moe_forward_persistent(ctypes.byref(s), 0, *args, 0, None) == lib.MOE_EINVAL
    both = [FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]  # router and an assignment
    assert L.moe_forward_persistent(ctypes.byref(s), 0, *both, 1000, None) == lib.MOE_EINVAL
    assert "time" in L.moe_status_string(lib.MOE_ETIMEOUT).decode()
