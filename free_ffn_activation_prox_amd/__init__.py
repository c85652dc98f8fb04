"""Prox sparse SwiGLU FFN decode path on MI355X — thin Python binding.

Argument marshalling over the C ABI in ``include/prox.h`` (ctypes).  Every
step of the path runs in the HIP library ``libprox_hip.so``; torch only
provides device memory and the stream.  Importing fails loudly when the
library has not been built (``python -m free_ffn_activation_prox_amd.build``).

Method: "Prox: Training-Free FFN Activation Sparsity via Approximate
Intermediate-Channel Salience in LLMs", Abstract (two stages: input-sparse
quantized proxy -> shared channel mask -> exact sparse SwiGLU).
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, Optional, Tuple

# torch first: the library then binds to the HIP runtime torch has loaded, so
# the process holds one runtime (one device context) whichever module a
# program imports first.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libprox_hip.so")

PROX_OK = 0
KINDS = {"int8": 1, "int4": 2, "exact": 3}


class ProxError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {_status_str(status)}: {detail}")


class _Weights(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("w_gate_t", ctypes.c_void_p), ("w_up_t", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p)]


class _Proxy(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("f_pad", ctypes.c_int32), ("groups", ctypes.c_int32), ("tile_ch", ctypes.c_int32),
                ("row_stride", ctypes.c_size_t), ("scale_offset", ctypes.c_size_t),
                ("bytes", ctypes.c_size_t), ("buf", ctypes.c_void_p)]


class _QWeights(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("scale_offset", ctypes.c_size_t),
                ("bytes", ctypes.c_size_t), ("buf", ctypes.c_void_p)]


class _Taps(ctypes.Structure):
    _fields_ = [("in_idx", ctypes.c_void_p), ("key", ctypes.c_void_p), ("h_hat", ctypes.c_void_p),
                ("events", ctypes.POINTER(ctypes.c_void_p)), ("n_events", ctypes.c_int32),
                ("event_mode", ctypes.c_int32), ("stream_idx", ctypes.c_void_p), ("timeline", ctypes.c_void_p)]


N_PHASES = 3
PHASES = ("stage1", "stage2", "reduce_y")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"Prox HIP library missing: {LIB_PATH}; build it with "
                          "`python -m free_ffn_activation_prox_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "prox_abi_version": (I32, []),
        "prox_proxy_bytes": (SZ, [I32, I32, I32]),
        "prox_build_proxy": (I32, [ctypes.POINTER(_Weights), I32, P, SZ, ctypes.POINTER(_Proxy), P]),
        "prox_workspace_bytes": (SZ, [I32, I32, I32, I32]),
        "prox_ffn_forward": (I32, [P, I32, ctypes.POINTER(_Weights), ctypes.POINTER(_Proxy), I32, I32,
                                   P, P, P, P, SZ, P]),
        "prox_ffn_forward_taps": (I32, [P, I32, ctypes.POINTER(_Weights), ctypes.POINTER(_Proxy), I32,
                                        I32, P, P, P, P, SZ, ctypes.POINTER(_Taps), P]),
        "prox_noalloc_scratch_bytes": (SZ, []),
        "prox_ffn_forward_noalloc": (I32, [P, I32, ctypes.POINTER(_Weights), ctypes.POINTER(_Proxy), I32, I32,
                                           P, P, P, P]),
        "prox_read_probe": (I32, [P, SZ, P, I32, P]),
        "prox_quality": (I32, [P, P, I32, I32, P, P, I32, P, P, P]),
        "prox_qweights_bytes": (SZ, [I32, I32]),
        "prox_build_qweights": (I32, [ctypes.POINTER(_Weights), P, SZ, ctypes.POINTER(_QWeights), P]),
        "prox_ffn_forward_q8": (I32, [P, I32, ctypes.POINTER(_QWeights), ctypes.POINTER(_Proxy), I32, I32, P, P, P,
                                      P, SZ, ctypes.POINTER(_Taps), P]),
        "prox_status_str": (ctypes.c_char_p, [I32]),
        "prox_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = _load()


def _status_str(st: int) -> str:
    return _lib.prox_status_str(st).decode()


def _check(st: int, where: str) -> None:
    if st != PROX_OK:
        raise ProxError(st, where, _lib.prox_last_error().decode())


def abi_version() -> int:
    return _lib.prox_abi_version()


def library_sha256() -> str:
    """sha256 (first 16 hex digits) of the loaded library file."""
    import hashlib
    with open(LIB_PATH, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def proxy_bytes(d_model: int, d_ff: int, kind: str) -> int:
    return _lib.prox_proxy_bytes(d_model, d_ff, KINDS[kind])


def workspace_bytes(d_model: int, d_ff: int, batch: int, kind: str) -> int:
    return _lib.prox_workspace_bytes(d_model, d_ff, batch, KINDS[kind])


def _stream_ptr(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


@dataclass
class Weights:
    """bf16 device tensors: w_gate_t, w_up_t [d_ff][d_model]; w_down [d_ff][d_model]."""

    w_gate_t: "object"
    w_up_t: "object"
    w_down: "object"

    def __post_init__(self):
        import torch
        for n in ("w_gate_t", "w_up_t", "w_down"):
            t = getattr(self, n)
            if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 2:
                raise ValueError(f"{n} must be a contiguous 2-D bf16 CUDA tensor")
        F, d = self.w_gate_t.shape
        if tuple(self.w_up_t.shape) != (F, d) or tuple(self.w_down.shape) != (F, d):
            raise ValueError("w_gate_t, w_up_t and w_down must all be [d_ff][d_model]")
        self.d_ff, self.d_model = int(F), int(d)
        self._c = _Weights(self.d_model, self.d_ff, self.w_gate_t.data_ptr(),
                           self.w_up_t.data_ptr(), self.w_down.data_ptr())


@dataclass
class Proxy:
    kind: str
    buf: "object"          # uint8 device tensor owning the proxy bytes
    desc: _Proxy

    @property
    def f_pad(self) -> int:
        return self.desc.f_pad

    def codes_and_scales(self):
        """Device views: codes [tiles][d][128] uint8, scales [2][groups][f_pad] fp32."""
        import torch
        d, fp, tc = self.desc.d_model, self.desc.f_pad, self.desc.tile_ch
        codes = self.buf[: (fp // tc) * d * 128].view(fp // tc, d, 128)
        n = 2 * self.desc.groups * fp
        so = self.desc.scale_offset
        scales = self.buf[so: so + 4 * n].view(torch.float32).view(2, self.desc.groups, fp)
        return codes, scales


def build_proxy(weights: Weights, kind: str, stream=None) -> Proxy:
    """Quantized proxy of W_gate / W_up (one-time, training-free).  kind
    "exact" (exact-mask mode) builds nothing: the weights rank themselves."""
    import torch
    if kind == "exact":
        desc = _Proxy()
        _check(_lib.prox_build_proxy(ctypes.byref(weights._c), KINDS[kind], None, 0, ctypes.byref(desc),
                                     _stream_ptr(stream)), "prox_build_proxy")
        return Proxy(kind, None, desc)
    nbytes = proxy_bytes(weights.d_model, weights.d_ff, kind)
    if nbytes == 0:
        raise ValueError("invalid shape/kind for a proxy")
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=weights.w_gate_t.device)
    off = (-buf.data_ptr()) % 256
    buf = buf[off: off + nbytes]
    desc = _Proxy()
    _check(_lib.prox_build_proxy(ctypes.byref(weights._c), KINDS[kind], buf.data_ptr(), nbytes,
                                 ctypes.byref(desc), _stream_ptr(stream)), "prox_build_proxy")
    return Proxy(kind, buf, desc)


@dataclass
class QWeights:
    """Quantized Stage-2 weights: int8 rows of W_gate^T, W_up^T, W_down and
    their fp32 scales in one device buffer (prox_build_qweights)."""

    buf: "object"
    desc: _QWeights

    @property
    def d_model(self) -> int:
        return self.desc.d_model

    @property
    def d_ff(self) -> int:
        return self.desc.d_ff

    def codes_and_scales(self):
        """Device views: codes [3][F][d] int8, scales [3][F] fp32."""
        import torch
        d, F = self.desc.d_model, self.desc.d_ff
        codes = self.buf[: 3 * F * d].view(torch.int8).view(3, F, d)
        so = self.desc.scale_offset
        scales = self.buf[so: so + 12 * F].view(torch.float32).view(3, F)
        return codes, scales


def qweights_bytes(d_model: int, d_ff: int) -> int:
    return _lib.prox_qweights_bytes(d_model, d_ff)


def build_qweights(weights: Weights, stream=None) -> QWeights:
    import torch
    n = qweights_bytes(weights.d_model, weights.d_ff)
    if n == 0:
        raise ValueError("invalid shape for quantized weights")
    raw = torch.empty(n + 256, dtype=torch.uint8, device=weights.w_gate_t.device)
    off = (-raw.data_ptr()) % 256
    buf = raw[off: off + n]
    desc = _QWeights()
    _check(_lib.prox_build_qweights(ctypes.byref(weights._c), buf.data_ptr(), n, ctypes.byref(desc),
                                    _stream_ptr(stream)), "prox_build_qweights")
    return QWeights(buf, desc)


def alloc_workspace(d_model: int, d_ff: int, batch: int, kind: str, device="cuda"):
    import torch
    n = workspace_bytes(d_model, d_ff, batch, kind)
    if n == 0:
        raise ValueError("invalid shape/batch for a workspace")
    # scratch: its contents on entry do not matter
    raw = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % 256
    return raw[off: off + n]


def ffn_forward(x, weights, proxy: Proxy, k_in: int, k_ff: int, *, y=None, mask=None,
                idx=None, workspace=None, taps: bool = False, events=None, kernel_events: bool = False,
                stream=None):
    """Sparse SwiGLU forward for x [B][d] bf16.  Returns (y fp32 [B][d], mask u8 [B][F],
    idx int32 [B][k_ff]) and, with ``taps``, a dict of in_idx / key / h_hat.
    ``events`` (measurement hook): torch.cuda.Event(enable_timing=True) objects
    already recorded once, or raw hipEvent_t handles (int).  By default
    N_PHASES + 1 events recorded at the phase boundaries on the launch stream;
    with ``kernel_events``, 2 * N_PHASES events carried by the kernels
    themselves: events[2p] .. events[2p + 1] spans phase p's kernels alone."""
    import torch
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous() or x.dim() != 2:
        raise ValueError("x must be a contiguous 2-D bf16 CUDA tensor")
    B, d = x.shape
    F = weights.d_ff
    dev = x.device
    q8 = isinstance(weights, QWeights)
    if y is None:
        y = torch.empty(B, d, dtype=torch.float32, device=dev)
    if mask is None:
        mask = torch.empty(B, F, dtype=torch.uint8, device=dev)
    if idx is None:
        idx = torch.empty(B, max(k_ff, 1), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(d, F, B, proxy.kind, dev)
    sp = _stream_ptr(stream)
    if events is not None:
        arr = (ctypes.c_void_p * len(events))(*[getattr(e, "cuda_event", e) for e in events])
        ct = _Taps(None, None, None, arr, len(events), 1 if kernel_events else 0, None, None)
        _call_forward(q8, x, B, weights, proxy, k_in, k_ff, y, mask, idx, workspace, ct, sp)
        return y, mask, idx[:, :k_ff]
    if taps:
        t = {"in_idx": torch.empty(B, max(k_in, 1), dtype=torch.int32, device=dev),
             "key": torch.empty(B, F, dtype=torch.float32, device=dev),
             "h_hat": torch.empty(B, F, dtype=torch.float64, device=dev),
             "stream_idx": torch.full((B, max(k_ff, 1)), -1, dtype=torch.int32, device=dev)}
        ct = _Taps(t["in_idx"].data_ptr(), t["key"].data_ptr(), t["h_hat"].data_ptr(), None, 0, 0,
                   t["stream_idx"].data_ptr(), None)
        _call_forward(q8, x, B, weights, proxy, k_in, k_ff, y, mask, idx, workspace, ct, sp)
        t["in_idx"] = t["in_idx"][:, :k_in]
        t["stream_idx"] = t["stream_idx"][:, :k_ff]
        return y, mask, idx[:, :k_ff], t
    if q8:
        _call_forward(True, x, B, weights, proxy, k_in, k_ff, y, mask, idx, workspace, None, sp)
    else:
        _check(_lib.prox_ffn_forward(x.data_ptr(), B, ctypes.byref(weights._c), ctypes.byref(proxy.desc),
                                     k_in, k_ff, y.data_ptr(), mask.data_ptr(), idx.data_ptr(),
                                     workspace.data_ptr(), workspace.numel(), sp),
               "prox_ffn_forward")
    return y, mask, idx[:, :k_ff]


def _call_forward(q8, x, B, weights, proxy, k_in, k_ff, y, mask, idx, workspace, ct, sp):
    tp = ctypes.byref(ct) if ct is not None else None
    if q8:
        _check(_lib.prox_ffn_forward_q8(x.data_ptr(), B, ctypes.byref(weights.desc), ctypes.byref(proxy.desc), k_in,
                                        k_ff, y.data_ptr(), mask.data_ptr(), idx.data_ptr(), workspace.data_ptr(),
                                        workspace.numel(), tp, sp),
               "prox_ffn_forward_q8")
    else:
        _check(_lib.prox_ffn_forward_taps(x.data_ptr(), B, ctypes.byref(weights._c), ctypes.byref(proxy.desc),
                                          k_in, k_ff, y.data_ptr(), mask.data_ptr(), idx.data_ptr(),
                                          workspace.data_ptr(), workspace.numel(), tp, sp),
               "prox_ffn_forward_taps")


def read_probe(buf, sink, blocks: int, stream=None) -> None:
    """Measurement helper: one plain streaming read of the device tensor `buf`
    (prox_read_probe); `sink` is an int32/uint32 device tensor of blocks * 512."""
    if sink.numel() < blocks * 512:
        raise ValueError("sink needs blocks * 512 words")
    _check(_lib.prox_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), blocks,
                                _stream_ptr(stream)), "prox_read_probe")


def timeline_forward(x, weights: Weights, proxy: Proxy, k_in: int, k_ff: int, *, y, mask, idx, workspace,
                     stream=None):
    """Measurement hook: the forward with the per-block timeline tap; returns
    the uint64 device tensor [2][1024][8] of 100 MHz counter stamps."""
    import torch
    tl = torch.zeros(2 * 1024 * 8, dtype=torch.int64, device=x.device)
    ct = _Taps(None, None, None, None, 0, 0, None, tl.data_ptr())
    B = x.shape[0]
    _check(_lib.prox_ffn_forward_taps(x.data_ptr(), B, ctypes.byref(weights._c), ctypes.byref(proxy.desc), k_in,
                                      k_ff, y.data_ptr(), mask.data_ptr(), idx.data_ptr(), workspace.data_ptr(),
                                      workspace.numel(), ctypes.byref(ct), _stream_ptr(stream)),
           "prox_ffn_forward_taps")
    return tl.view(2, 1024, 8)


def quality(mask_a, mask_b, y, y_ref, stream=None):
    """Quality diagnostics (prox_quality) on device tensors: per token, the kept
    channels two masks share (uint8 [B][F] each) and ||y - y_ref|| / ||y_ref||
    (fp32 [B][d] each).  Returns (overlap int32 [B], err float64 [B])."""
    import torch
    B, F = mask_a.shape
    d = y.shape[1]
    for t, dt in ((mask_a, torch.uint8), (mask_b, torch.uint8), (y, torch.float32), (y_ref, torch.float32)):
        if t.dtype != dt or not t.is_contiguous() or t.shape[0] != B:
            raise ValueError("quality: wrong dtype, layout or batch")
    overlap = torch.empty(B, dtype=torch.int32, device=y.device)
    err = torch.empty(B, dtype=torch.float64, device=y.device)
    _check(_lib.prox_quality(mask_a.data_ptr(), mask_b.data_ptr(), B, F, y.data_ptr(), y_ref.data_ptr(), d,
                             overlap.data_ptr(), err.data_ptr(), _stream_ptr(stream)), "prox_quality")
    return overlap, err


def noalloc_scratch_bytes() -> int:
    return _lib.prox_noalloc_scratch_bytes()


def ffn_forward_noalloc(x, weights: Weights, proxy: Proxy, k_in: int, k_ff: int, *, y, mask, idx,
                        stream=None):
    """prox_ffn_forward_noalloc: the forward with the library's fixed device
    scratch as workspace (no allocation in the call).  y, mask and idx are the
    caller's ([B][d] fp32, [B][F] uint8, [B][>= max(k_ff, 1)] int32)."""
    import torch
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous() or x.dim() != 2:
        raise ValueError("x must be a contiguous 2-D bf16 CUDA tensor")
    B, d = x.shape
    for t, dt, shape in ((y, torch.float32, (B, d)), (mask, torch.uint8, (B, weights.d_ff))):
        if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError("y / mask: wrong dtype, shape or layout")
    if idx.dtype != torch.int32 or idx.dim() != 2 or idx.shape[0] != B or idx.shape[1] < max(k_ff, 1) \
            or not idx.is_contiguous():
        raise ValueError("idx must be int32 [B][>= max(k_ff, 1)]")
    _check(_lib.prox_ffn_forward_noalloc(x.data_ptr(), B, ctypes.byref(weights._c), ctypes.byref(proxy.desc),
                                         k_in, k_ff, y.data_ptr(), mask.data_ptr(), idx.data_ptr(),
                                         _stream_ptr(stream)),
           "prox_ffn_forward_noalloc")
    return y, mask, idx[:, :k_ff]


__all__ = ["QWeights", "build_qweights", "qweights_bytes", "quality", "timeline_forward", "read_probe", "noalloc_scratch_bytes", "ffn_forward_noalloc", "Weights", "Proxy", "ProxError", "abi_version", "library_sha256", "proxy_bytes", "workspace_bytes",
           "build_proxy", "alloc_workspace", "ffn_forward", "LIB_PATH", "KINDS", "N_PHASES", "PHASES"]
