"""Thin ctypes binding over libmosaicq.so (declared in include/mosaicq.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Torch tensors provide device memory and the current HIP stream.
There is no fallback: if the library is missing or a call fails, an
exception is raised.

Function names follow the C ABI without the ``mq_`` prefix; the prefixed
names are aliases.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import inspect
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmosaicq.so")

GROUP = 128
FLAG_DUMP_ACC = 1
FLAG_INT8_TILE = 2
FLAG_FP6_TILE = 4

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_vp = ctypes.c_void_p

_SIGS = {
    "mq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "mq_last_error": (ctypes.c_char_p, []),
    "mq_version": (ctypes.c_int, []),
    "mq_quantize_act": (ctypes.c_int, [_vp, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp]),
    "mq_select_blocks": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32,
                                        _vp, _vp, _vp, _vp]),
    "mq_pack_weights": (ctypes.c_int, [_vp, _c_i64, _c_i64, _c_i32, _vp, _c_i32, _vp, _vp,
                                       _vp, _vp, _vp, _vp, _vp]),
    "mq_fused_gemm_workspace": (ctypes.c_int, [_c_i64, _c_i64, _c_i64,
                                               ctypes.POINTER(ctypes.c_size_t)]),
    "mq_fused_gemm": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i64, _c_i64, _vp, _vp, _c_i32,
                                     _c_i32, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp,
                                     ctypes.c_size_t, ctypes.c_uint32, _vp, _vp]),
    "mq_fused_layer_workspace": (ctypes.c_int, [_c_i64, _c_i64, _c_i64,
                                                ctypes.POINTER(ctypes.c_size_t)]),
    "mq_fused_layer": (ctypes.c_int, [_vp, _c_i64, _c_i64, _c_i64, _c_i64, _vp, _vp, _c_i32,
                                      _c_i32, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp,
                                      ctypes.c_size_t, _vp]),
    "mq_validate_csr": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i64, _c_i32, _c_i32, _vp]),
    "mq_residual_merge": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _vp,
                                         _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "mq_smooth_weights": (ctypes.c_int, [_vp, _c_i64, _vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp]),
    "mq_smooth_acts": (ctypes.c_int, [_vp, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp]),
    "mq_measure_mfma": (ctypes.c_int, [_c_i32, _c_i32, _vp, _vp, _vp]),
    "mq_distortion_workspace": (ctypes.c_int, [_c_i64, _c_i64, _c_i64, _c_i32,
                                               ctypes.POINTER(ctypes.c_size_t)]),
    "mq_distortion": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i64, _c_i64, _c_i32, _vp, _c_i32, _vp,
                                     _vp, ctypes.c_size_t, _vp]),
    "mq_select_exact_workspace": (ctypes.c_int, [_c_i64, _c_i64, _c_i64, _c_i32,
                                                 ctypes.POINTER(ctypes.c_size_t)]),
    "mq_select_exact_greedy": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32,
                                              _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "mq_fused_layer_noalloc": (ctypes.c_int, [_vp, _c_i64, _c_i64, _c_i64, _c_i64, _vp, _vp, _c_i32,
                                              _c_i32, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "mq_fp6_sizes": (ctypes.c_int, [_c_i64, _c_i64, _c_i64, _c_i32, _c_i32] +
                     [ctypes.POINTER(ctypes.c_size_t)] * 3),
    "mq_fp6_prepare_acts": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _vp]),
    "mq_fp6_prepare_weights": (ctypes.c_int, [_vp, _c_i64, _c_i64, _c_i32, _c_i32, _vp, _vp, _vp]),
    "mq_fused_gemm_fp6": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i64, _c_i64, _vp, _vp, _c_i32, _c_i32,
                                         _vp, _vp, _vp, _vp, _c_i64, _vp, ctypes.c_size_t,
                                         ctypes.c_uint32, _vp, _vp]),
}

NOALLOC_SCRATCH_BYTES = 128 << 20

_lib = None


class MosaicQError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed: {status_str(status)} ({status}): {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libmosaicq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m dense_sparse_w4a4_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_str(s: int) -> str:
    return lib().mq_status_str(int(s)).decode()


def last_error() -> str:
    return lib().mq_last_error().decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MosaicQError(fn, status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(fn):
    """Run the wrapped entry point with its `stream` argument (when one is
    given) as the current stream, so the outputs and workspaces it allocates
    belong to that stream: the caching allocator then never hands their
    memory to other work while the call's kernels may still use it."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        stream = sig.bind(*args, **kwargs).arguments.get("stream")
        with torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext():
            return fn(*args, **kwargs)
    return wrapper


def _dev(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


# ----------------------------------------------------------------------------
# Entry points
# ----------------------------------------------------------------------------

@_on_stream
def quantize_act(x: torch.Tensor, qa: Optional[torch.Tensor] = None,
                 sa: Optional[torch.Tensor] = None, stream=None):
    """x fp16 [M, K] (row stride % 8 == 0) -> (qa uint8 [M, K/2], sa fp32 [M, K/128])."""
    _dev(x, torch.float16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    M, K = x.shape
    if qa is None:
        qa = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if sa is None:
        sa = torch.empty((M, max(K // GROUP, 0)), dtype=torch.float32, device=x.device)
    _check("mq_quantize_act", lib().mq_quantize_act(
        _ptr(x), M, K, x.stride(0), _ptr(qa), _ptr(sa), _stream(stream)))
    return qa, sa


@_on_stream
def select_blocks(w: torch.Tensor, x_calib: torch.Tensor, block: int, n_select: int,
                  stream=None):
    """Delta-score top-K.  Returns (selected int32 [n_select] ascending,
    delta fp64 [B], hdiag fp64 [K])."""
    _dev(w, torch.float16, "w")
    _dev(x_calib, torch.float16, "x_calib")
    w = w.contiguous()
    x_calib = x_calib.contiguous()
    N, K = w.shape
    T = x_calib.shape[0]
    if x_calib.shape[1] != K:
        raise ValueError("x_calib must have K columns")
    B = (N // block) * (K // block) if block else 0
    sel = torch.empty(max(n_select, 0), dtype=torch.int32, device=w.device)
    delta = torch.empty(max(B, 1), dtype=torch.float64, device=w.device)
    H = torch.empty(K, dtype=torch.float64, device=w.device)
    _check("mq_select_blocks", lib().mq_select_blocks(
        _ptr(w), _ptr(x_calib) if T else None, N, K, T, block, n_select,
        _ptr(sel) if n_select else None, _ptr(delta), _ptr(H), _stream(stream)))
    return sel, delta[:B], H


def _exact_ws(fn: str, N: int, K: int, T: int, block: int) -> int:
    n = ctypes.c_size_t(0)
    _check(fn, getattr(lib(), fn)(N, K, T, block, ctypes.byref(n)))
    return int(n.value)


@_on_stream
def distortion(w: torch.Tensor, x: torch.Tensor, block: int, selected: torch.Tensor,
               stream=None) -> torch.Tensor:
    """Exact output distortion ||X (W - deq Q - R_S)^T||_F^2 (fp64 [1] device)."""
    _dev(w, torch.float16, "w")
    _dev(x, torch.float16, "x")
    _dev(selected, torch.int32, "selected")
    w, x, selected = w.contiguous(), x.contiguous(), selected.contiguous()
    N, K = w.shape
    T = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x must have K columns")
    ws = torch.empty(max(_exact_ws("mq_distortion_workspace", N, K, T, block), 1),
                     dtype=torch.uint8, device=w.device)
    out = torch.empty(1, dtype=torch.float64, device=w.device)
    n = int(selected.numel())
    _check("mq_distortion", lib().mq_distortion(
        _ptr(w), _ptr(x) if T else None, N, K, T, block, _ptr(selected) if n else None, n,
        _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


@_on_stream
def select_exact_greedy(w: torch.Tensor, x_calib: torch.Tensor, block: int, n_select: int,
                        stream=None):
    """Greedy selection by exact output distortion.  Returns (selected int32
    [n_select] ascending, order int32 [n_select] as picked, gains fp64
    [n_select], dist fp64 [2] = D({}), D(selected) on x_calib)."""
    _dev(w, torch.float16, "w")
    _dev(x_calib, torch.float16, "x_calib")
    w, x_calib = w.contiguous(), x_calib.contiguous()
    N, K = w.shape
    T = x_calib.shape[0]
    if x_calib.shape[1] != K:
        raise ValueError("x_calib must have K columns")
    ws = torch.empty(max(_exact_ws("mq_select_exact_workspace", N, K, T, block), 1),
                     dtype=torch.uint8, device=w.device)
    k = max(n_select, 0)
    sel = torch.empty(k, dtype=torch.int32, device=w.device)
    order = torch.empty(k, dtype=torch.int32, device=w.device)
    gains = torch.empty(k, dtype=torch.float64, device=w.device)
    dist = torch.empty(2, dtype=torch.float64, device=w.device)
    _check("mq_select_exact_greedy", lib().mq_select_exact_greedy(
        _ptr(w), _ptr(x_calib) if T else None, N, K, T, block, n_select,
        _ptr(sel) if k else None, _ptr(order) if k else None, _ptr(gains) if k else None,
        _ptr(dist), _ptr(ws), ws.numel(), _stream(stream)))
    return sel, order, gains, dist


@dataclass
class PackedLayer:
    """Packed dense base + CSR residual (device tensors), as mq_pack_weights writes it."""
    N: int
    K: int
    block: int
    qw: torch.Tensor       # uint8 [N/16, K/128, 64, 16] (slab layout)
    sw: torch.Tensor       # fp16  [N, K/128]
    row_ptr: torch.Tensor  # int32 [N/b + 1]
    col_idx: torch.Tensor  # int32 [n_select]
    qr: torch.Tensor       # uint8 [n_select, b, b/2]
    sr: torch.Tensor       # fp16  [n_select, b]

    @property
    def n_select(self) -> int:
        return int(self.col_idx.numel())

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.qw, self.sw, self.row_ptr, self.col_idx, self.qr, self.sr))

    def clone(self) -> "PackedLayer":
        return PackedLayer(self.N, self.K, self.block, self.qw.clone(), self.sw.clone(),
                           self.row_ptr.clone(), self.col_idx.clone(), self.qr.clone(),
                           self.sr.clone())


@_on_stream
def pack_weights(w: torch.Tensor, block: int, selected: torch.Tensor, stream=None) -> PackedLayer:
    """w fp16 [N, K] + ascending selected block ids -> PackedLayer."""
    _dev(w, torch.float16, "w")
    _dev(selected, torch.int32, "selected")
    w = w.contiguous()
    selected = selected.contiguous()
    N, K = w.shape
    ns = int(selected.numel())
    dev = w.device
    b = int(block)
    qw = torch.empty((N // 16, K // GROUP, 64, 16), dtype=torch.uint8, device=dev)
    sw = torch.empty((N, K // GROUP), dtype=torch.float16, device=dev)
    row_ptr = torch.empty(N // b + 1 if b else 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(ns, dtype=torch.int32, device=dev)
    qr = torch.empty((ns, b, b // 2), dtype=torch.uint8, device=dev)
    sr = torch.empty((ns, b), dtype=torch.float16, device=dev)
    _check("mq_pack_weights", lib().mq_pack_weights(
        _ptr(w), N, K, b, _ptr(selected) if ns else None, ns, _ptr(qw), _ptr(sw),
        _ptr(row_ptr), _ptr(col_idx) if ns else None, _ptr(qr) if ns else None,
        _ptr(sr) if ns else None, _stream(stream)))
    return PackedLayer(N, K, b, qw, sw, row_ptr, col_idx, qr, sr)


def fused_gemm_workspace(M: int, N: int, K: int) -> int:
    n = ctypes.c_size_t(0)
    _check("mq_fused_gemm_workspace", lib().mq_fused_gemm_workspace(M, N, K, ctypes.byref(n)))
    return int(n.value)


@_on_stream
def fused_gemm(qa: torch.Tensor, sa: torch.Tensor, layer: PackedLayer,
               out: Optional[torch.Tensor] = None, dump: bool = False,
               workspace: Optional[torch.Tensor] = None, stream=None, route: Optional[str] = None):
    """Y fp16 [M, N] = deq(Qa(X) Q(W)^T) + deq(Qa(X) R^T).

    With dump=True also returns the exact accumulators
    (acc_base int32 [M, N, K/128], acc_res int32 [n_select, M, b]).
    route="int8" or "fp6" picks the prefill kernel's route for M > 32
    (default: fp6 from M = 1024 on, when block is 64 or 128); same y."""
    if route not in (None, "int8", "fp6"):
        raise ValueError("route must be None, 'int8' or 'fp6'")
    _dev(qa, torch.uint8, "qa")
    _dev(sa, torch.float32, "sa")
    M = qa.shape[0]
    N, K, b, ns = layer.N, layer.K, layer.block, layer.n_select
    if qa.shape[1] * 2 != K or not qa.is_contiguous() or not sa.is_contiguous():
        raise ValueError("qa/sa must be contiguous and match the layer's K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=qa.device)
    _dev(out, torch.float16, "out")
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != M or out.shape[1] != N:
        raise ValueError("out must be [M, N] with unit column stride")
    wsb = fused_gemm_workspace(M, N, K)
    if wsb and (workspace is None or workspace.numel() * workspace.element_size() < wsb):
        workspace = torch.empty(wsb, dtype=torch.uint8, device=qa.device)
    G = K // GROUP
    acc = None
    if dump:
        acc = torch.empty(M * N * G + ns * M * b, dtype=torch.int32, device=qa.device)
    _check("mq_fused_gemm", lib().mq_fused_gemm(
        _ptr(qa), _ptr(sa), M, N, K, _ptr(layer.qw), _ptr(layer.sw), b, ns,
        _ptr(layer.row_ptr) if ns else None, _ptr(layer.col_idx) if ns else None,
        _ptr(layer.qr) if ns else None, _ptr(layer.sr) if ns else None,
        _ptr(out), out.stride(0), _ptr(workspace) if wsb else None, wsb,
        (FLAG_DUMP_ACC if dump else 0) | {None: 0, "int8": FLAG_INT8_TILE, "fp6": FLAG_FP6_TILE}[route],
        _ptr(acc), _stream(stream)))
    if dump:
        base = acc[: M * N * G].view(M, N, G)
        res = acc[M * N * G:].view(ns, M, b)
        return out, base, res
    return out


def fused_layer_workspace(M: int, N: int, K: int) -> int:
    n = ctypes.c_size_t(0)
    _check("mq_fused_layer_workspace", lib().mq_fused_layer_workspace(M, N, K, ctypes.byref(n)))
    return int(n.value)


@_on_stream
def fused_layer(x: torch.Tensor, layer: PackedLayer, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Y fp16 [M, N] from fp16 activations: Qa(X) and the fused GEMM, as one
    kernel for decode-sized M (the GEMM quantises the token tile itself), or
    the two kernels through the workspace otherwise.  Same result as
    fused_gemm(*quantize_act(x), layer)."""
    _dev(x, torch.float16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [M, K] with unit column stride")
    M, K = x.shape
    N, b, ns = layer.N, layer.block, layer.n_select
    if K != layer.K:
        raise ValueError("x must match the layer's K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _dev(out, torch.float16, "out")
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != M or out.shape[1] != N:
        raise ValueError("out must be [M, N] with unit column stride")
    wsb = fused_layer_workspace(M, N, K)
    if wsb and (workspace is None or workspace.numel() * workspace.element_size() < wsb):
        workspace = torch.empty(wsb, dtype=torch.uint8, device=x.device)
    _check("mq_fused_layer", lib().mq_fused_layer(
        _ptr(x), M, K, x.stride(0), N, _ptr(layer.qw), _ptr(layer.sw), b, ns,
        _ptr(layer.row_ptr) if ns else None, _ptr(layer.col_idx) if ns else None,
        _ptr(layer.qr) if ns else None, _ptr(layer.sr) if ns else None,
        _ptr(out), out.stride(0), _ptr(workspace) if wsb else None, wsb, _stream(stream)))
    return out


def fused_layer_noalloc(x: torch.Tensor, layer: PackedLayer, out: torch.Tensor,
                        stream=None) -> torch.Tensor:
    """fused_layer without a workspace: the library's per-device scratch
    serves instead (same y bits).  Allocates nothing; `out` is required.
    Calls that overlap on one device race on the scratch."""
    _dev(x, torch.float16, "x")
    _dev(out, torch.float16, "out")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [M, K] with unit column stride")
    M, K = x.shape
    N, b, ns = layer.N, layer.block, layer.n_select
    if K != layer.K:
        raise ValueError("x must match the layer's K")
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != M or out.shape[1] != N:
        raise ValueError("out must be [M, N] with unit column stride")
    _check("mq_fused_layer_noalloc", lib().mq_fused_layer_noalloc(
        _ptr(x), M, K, x.stride(0), N, _ptr(layer.qw), _ptr(layer.sw), b, ns,
        _ptr(layer.row_ptr) if ns else None, _ptr(layer.col_idx) if ns else None,
        _ptr(layer.qr) if ns else None, _ptr(layer.sr) if ns else None,
        _ptr(out), out.stride(0), _stream(stream)))
    return out


def fp6_sizes(M: int, N: int, K: int, block: int, n_select: int):
    """(activation image, weight image, split-K partials) bytes of the fp6 route."""
    a, w, p = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("mq_fp6_sizes", lib().mq_fp6_sizes(M, N, K, block, n_select, ctypes.byref(a),
                                               ctypes.byref(w), ctypes.byref(p)))
    return int(a.value), int(w.value), int(p.value)


@_on_stream
def fp6_prepare_acts(qa: torch.Tensor, K: int, out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """Packed activation codes [M, K/2] -> the fp6 route's activation image."""
    _dev(qa, torch.uint8, "qa")
    M = qa.shape[0]
    if qa.dim() != 2 or qa.shape[1] * 2 != K or not qa.is_contiguous():
        raise ValueError("qa must be contiguous [M, K/2]")
    nbytes = -(-M // 32) * (K // GROUP) * 3072
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=qa.device)
    _dev(out, torch.uint8, "out")
    if out.numel() < nbytes:
        raise ValueError("out is smaller than the activation image")
    _check("mq_fp6_prepare_acts", lib().mq_fp6_prepare_acts(_ptr(qa), M, K, _ptr(out), _stream(stream)))
    return out


@_on_stream
def fp6_prepare_weights(layer: PackedLayer, out: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """The packed layer's base and residual codes -> the fp6 weight image."""
    N, K, b, ns = layer.N, layer.K, layer.block, layer.n_select
    _, wb, _ = fp6_sizes(0, N, K, b, ns)
    if out is None:
        out = torch.empty(wb, dtype=torch.uint8, device=layer.qw.device)
    _dev(out, torch.uint8, "out")
    if out.numel() < wb:
        raise ValueError("out is smaller than the weight image")
    _check("mq_fp6_prepare_weights", lib().mq_fp6_prepare_weights(
        _ptr(layer.qw), N, K, b, ns, _ptr(layer.qr) if ns else None, _ptr(out), _stream(stream)))
    return out


@_on_stream
def fused_gemm_fp6(act_img: torch.Tensor, sa: torch.Tensor, M: int, layer: PackedLayer,
                   weight_img: torch.Tensor, out: Optional[torch.Tensor] = None, dump: bool = False,
                   split_ws: Optional[torch.Tensor] = None, stream=None):
    """fused_gemm on prepared fp6 images (same accumulators, same y bits)."""
    _dev(act_img, torch.uint8, "act_img")
    _dev(sa, torch.float32, "sa")
    _dev(weight_img, torch.uint8, "weight_img")
    N, K, b, ns = layer.N, layer.K, layer.block, layer.n_select
    ab, wb, pb = fp6_sizes(M, N, K, b, ns)
    if act_img.numel() < ab or weight_img.numel() < wb or sa.numel() < M * (K // GROUP):
        raise ValueError("act_img, weight_img or sa is too small for the shape")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=sa.device)
    _dev(out, torch.float16, "out")
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != M or out.shape[1] != N:
        raise ValueError("out must be [M, N] with unit column stride")
    if pb and (split_ws is None or split_ws.numel() * split_ws.element_size() < pb):
        split_ws = torch.empty(pb, dtype=torch.uint8, device=sa.device)
    G = K // GROUP
    acc = torch.empty(M * N * G + ns * M * b, dtype=torch.int32, device=sa.device) if dump else None
    _check("mq_fused_gemm_fp6", lib().mq_fused_gemm_fp6(
        _ptr(act_img), _ptr(sa), M, N, K, _ptr(weight_img), _ptr(layer.sw), b, ns,
        _ptr(layer.row_ptr) if ns else None, _ptr(layer.col_idx) if ns else None,
        _ptr(layer.sr) if ns else None, _ptr(out), out.stride(0), _ptr(split_ws) if pb else None, pb,
        FLAG_DUMP_ACC if dump else 0, _ptr(acc), _stream(stream)))
    if dump:
        return out, acc[: M * N * G].view(M, N, G), acc[M * N * G:].view(ns, M, b)
    return out


@_on_stream
def residual_merge(qa: torch.Tensor, sa: torch.Tensor, layer: PackedLayer, out: torch.Tensor,
                   stream=None) -> torch.Tensor:
    """Unfused ablation: out += deq(Qa(X) R^T) by a standalone residual kernel."""
    _dev(qa, torch.uint8, "qa")
    _dev(sa, torch.float32, "sa")
    _dev(out, torch.float16, "out")
    M = qa.shape[0]
    N, K, b, ns = layer.N, layer.K, layer.block, layer.n_select
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != M or out.shape[1] != N:
        raise ValueError("out must be [M, N] with unit column stride")
    _check("mq_residual_merge", lib().mq_residual_merge(
        _ptr(qa), _ptr(sa), M, N, K, b, ns, _ptr(layer.row_ptr) if ns else None,
        _ptr(layer.col_idx) if ns else None, _ptr(layer.qr) if ns else None,
        _ptr(layer.sr) if ns else None, _ptr(out), out.stride(0), _stream(stream)))
    return out


@_on_stream
def smooth_weights(x_calib: torch.Tensor, w: torch.Tensor, stream=None):
    """Outlier migration: -> (scales fp32 [K], migrated w fp16 [N, K], x_absmax, w_absmax)."""
    _dev(x_calib, torch.float16, "x_calib")
    _dev(w, torch.float16, "w")
    x_calib, w = x_calib.contiguous(), w.contiguous()
    T, K = x_calib.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("x_calib and w must have the same K")
    f = dict(dtype=torch.float32, device=w.device)
    ax, aw, s = torch.empty(K, **f), torch.empty(K, **f), torch.empty(K, **f)
    w_out = torch.empty_like(w)
    _check("mq_smooth_weights", lib().mq_smooth_weights(
        _ptr(x_calib), T, _ptr(w), N, K, _ptr(ax), _ptr(aw), _ptr(s), _ptr(w_out), _stream(stream)))
    return s, w_out, ax, aw


@_on_stream
def smooth_acts(x: torch.Tensor, scales: torch.Tensor, stream=None) -> torch.Tensor:
    """Migrated activations x / scales (fp16 [M, K])."""
    _dev(x, torch.float16, "x")
    _dev(scales, torch.float32, "scales")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [M, K] with unit column stride")
    M, K = x.shape
    out = torch.empty((M, K), dtype=torch.float16, device=x.device)
    _check("mq_smooth_acts", lib().mq_smooth_acts(
        _ptr(x), M, K, x.stride(0), _ptr(scales), _ptr(out), _stream(stream)))
    return out


def validate_csr(layer: PackedLayer, stream=None) -> None:
    ns = layer.n_select
    _check("mq_validate_csr", lib().mq_validate_csr(
        _ptr(layer.row_ptr), _ptr(layer.col_idx) if ns else None, layer.N, layer.K,
        layer.block, ns, _stream(stream)))


@_on_stream
def measure_mfma(blocks: int, iters: int, stream=None):
    """Launch the matrix-core rate probe (measurement only).  Returns the
    device tensors (cycles int64 [4*blocks], sink int32 [256*blocks]); the
    caller times the launch."""
    dev = torch.device("cuda", torch.cuda.current_device())
    cycles = torch.empty(4 * blocks, dtype=torch.int64, device=dev)
    sink = torch.empty(256 * blocks, dtype=torch.int32, device=dev)
    _check("mq_measure_mfma", lib().mq_measure_mfma(blocks, iters, _ptr(cycles), _ptr(sink),
                                                    _stream(stream)))
    return cycles, sink


def layer_forward(x: torch.Tensor, layer: PackedLayer, out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """The online hot path: Qa(X) then the fused GEMM (two launches)."""
    qa, sa = quantize_act(x, stream=stream)
    return fused_gemm(qa, sa, layer, out=out, stream=stream)


mq_quantize_act = quantize_act
mq_select_blocks = select_blocks
mq_pack_weights = pack_weights
mq_fused_gemm = fused_gemm
mq_fused_gemm_workspace = fused_gemm_workspace
mq_fused_layer = fused_layer
mq_fused_layer_workspace = fused_layer_workspace
mq_fused_layer_noalloc = fused_layer_noalloc
mq_validate_csr = validate_csr
mq_residual_merge = residual_merge
mq_smooth_weights = smooth_weights
mq_smooth_acts = smooth_acts
mq_measure_mfma = measure_mfma
mq_fp6_sizes = fp6_sizes
mq_fp6_prepare_acts = fp6_prepare_acts
mq_fp6_prepare_weights = fp6_prepare_weights
mq_fused_gemm_fp6 = fused_gemm_fp6
