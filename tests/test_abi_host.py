"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, sizes its buffers as documented, and rejects bad arguments
before enqueuing anything (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

import free_ffn_activation_prox_amd as P
from free_ffn_activation_prox_amd import _Proxy, _Weights, _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "prox.h")

INVALID, UNSUPPORTED, MISMATCH, WORKSPACE = -1, -2, -3, -4


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|prox_status|size_t|int32_t)\s+(prox_\w+)\s*\(",
                                 src, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 8
    lib = ctypes.CDLL(P.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version():
    assert P.abi_version() == 4


def _align(v, a):
    return (v + a - 1) // a * a


@pytest.mark.parametrize("d,F", [(4096, 11008), (512, 1376), (8192, 28672), (3584, 18944)])
def test_proxy_bytes_layout(d, F):
    fp8, fp4 = _align(F, 64), _align(F, 128)
    assert P.proxy_bytes(d, F, "int8") == _align((fp8 // 64) * d * 128, 256) + 2 * 1 * fp8 * 4
    assert P.proxy_bytes(d, F, "int4") == _align((fp4 // 128) * d * 128, 256) + 2 * (d // 128) * fp4 * 4


def test_size_queries_reject_bad_shapes():
    assert P.proxy_bytes(100, 64, "int8") == 0           # d % 8 != 0
    assert P.proxy_bytes(520, 64, "int4") == 0           # int4 needs d % 128 == 0
    assert P.proxy_bytes(32768, 64, "int8") == 0         # above the d_model limit
    assert _lib.prox_proxy_bytes(512, 64, 7) == 0        # unknown kind
    assert P.workspace_bytes(512, 64, 0, "int8") == 0
    assert P.workspace_bytes(512, 64, 4097, "int8") == 0
    # prefill batches share one sub-batch workspace
    assert P.workspace_bytes(512, 64, 4096, "int8") == P.workspace_bytes(512, 64, 64, "int8")
    assert P.workspace_bytes(4096, 11008, 1, "int8") > 0


FAKE = 0x10000000  # never dereferenced: every call below fails validation first


def _weights(d=512, F=1376, null_down=False):
    return _Weights(d, F, FAKE, FAKE, 0 if null_down else FAKE)


def _proxy(d=512, F=1376, kind=1, **over):
    tc = 64 if kind == 1 else 128
    fp = _align(F, tc)
    groups = 1 if kind == 1 else d // 128
    so = _align((fp // tc) * d * 128, 256)
    p = _Proxy(kind, d, F, fp, groups, tc, 128, so, so + 2 * groups * fp * 4, FAKE)
    for k, v in over.items():
        setattr(p, k, v)
    return p


def _fwd(x=FAKE, B=1, w=None, p=None, k_in=256, k_ff=688, y=FAKE, ws=FAKE, ws_bytes=1 << 40):
    w = w or _weights()
    p = p or _proxy()
    return _lib.prox_ffn_forward(x, B, ctypes.byref(w), ctypes.byref(p), k_in, k_ff, y, None, None,
                                 ws, ws_bytes, None)


def test_forward_validation():
    assert _fwd(x=0) == INVALID
    assert _fwd(y=0) == INVALID
    assert _fwd(ws=0) == INVALID
    assert _fwd(w=_weights(null_down=True)) == INVALID
    assert _fwd(B=0) == INVALID
    assert _fwd(B=4097) == UNSUPPORTED
    assert _fwd(k_in=-1) == INVALID
    assert _fwd(k_in=513) == INVALID
    assert _fwd(k_ff=1377) == INVALID
    assert _fwd(k_ff=-2) == INVALID
    assert _fwd(p=_proxy(F=1000)) == MISMATCH
    assert _fwd(p=_proxy(row_stride=1)) == MISMATCH
    assert _fwd(p=_proxy(tile_ch=128)) == MISMATCH
    assert _fwd(p=_proxy(kind=3)) == INVALID
    assert _fwd(x=FAKE + 2) == INVALID                   # misaligned x
    assert _fwd(ws=FAKE + 16) == INVALID                 # workspace needs 256-byte alignment
    assert _fwd(ws_bytes=1024) == WORKSPACE
    big = _Weights(32768, 64, FAKE, FAKE, FAKE)
    assert _fwd(w=big, p=_proxy(d=32768, F=64)) == UNSUPPORTED


def test_last_error_text():
    assert _fwd(ws_bytes=1024) == WORKSPACE
    assert "workspace" in _lib.prox_last_error().decode()
    assert _lib.prox_status_str(WORKSPACE).decode() == "PROX_E_WORKSPACE"


def test_build_proxy_validation():
    w = _weights()
    out = _Proxy()
    assert _lib.prox_build_proxy(ctypes.byref(w), 1, FAKE, 10, ctypes.byref(out), None) == INVALID
    assert _lib.prox_build_proxy(ctypes.byref(w), 1, FAKE + 64, 1 << 30, ctypes.byref(out), None) == INVALID
    assert _lib.prox_build_proxy(ctypes.byref(w), 9, FAKE, 1 << 30, ctypes.byref(out), None) == INVALID
    assert _lib.prox_build_proxy(None, 1, FAKE, 1 << 30, ctypes.byref(out), None) == INVALID
    w4 = _Weights(520, 64, FAKE, FAKE, FAKE)
    assert _lib.prox_build_proxy(ctypes.byref(w4), 2, FAKE, 1 << 30, ctypes.byref(out), None) == INVALID


def test_noalloc_rejects_oversized_shape_before_any_launch():
    # d_model 16384, d_ff 32768, 64 tokens need far more than the 32 MiB
    # scratch: rejected on the host (no device pointer is touched)
    assert P.noalloc_scratch_bytes() == 32 << 20
    assert P.workspace_bytes(16384, 32768, 64, "int8") > P.noalloc_scratch_bytes()
    w = _Weights(16384, 32768, FAKE, FAKE, FAKE)
    p = _Proxy()
    p.kind, p.d_model, p.d_ff = 1, 16384, 32768
    st = _lib.prox_ffn_forward_noalloc(FAKE, 64, ctypes.byref(w), ctypes.byref(p), 100, 100,
                                       FAKE, FAKE, FAKE, None)
    assert st == UNSUPPORTED
    assert b"scratch" in _lib.prox_last_error()


def test_exact_kind_host_side():
    # exact-mask mode needs no proxy buffer; a forward with k_in != d_model is
    # rejected on the host
    assert P.proxy_bytes(4096, 11008, "exact") == 0
    assert P.workspace_bytes(4096, 11008, 1, "exact") > P.workspace_bytes(4096, 11008, 1, "int8") - 1
    w = _Weights(512, 1000, FAKE, FAKE, FAKE)
    desc = _Proxy()
    assert _lib.prox_build_proxy(ctypes.byref(w), 3, None, 0, ctypes.byref(desc), None) == 0
    assert desc.kind == 3 and desc.bytes == 0 and desc.f_pad == 1024
    st = _lib.prox_ffn_forward(FAKE, 1, ctypes.byref(w), ctypes.byref(desc), 100, 10, FAKE, FAKE, FAKE,
                               FAKE, 1 << 30, None)
    assert st == INVALID and b"k_in" in _lib.prox_last_error()


def test_quality_rejects_partial_arguments():
    assert _lib.prox_quality(FAKE, None, 1, 10, None, None, 8, FAKE, None, None) == INVALID
    assert _lib.prox_quality(None, None, 1, 10, FAKE, FAKE, 8, None, None, None) == INVALID
    assert _lib.prox_quality(None, None, 1, 10, None, None, 8, None, None, None) == INVALID
    assert _lib.prox_quality(None, None, 0, 10, FAKE, FAKE, 8, None, FAKE, None) == INVALID
