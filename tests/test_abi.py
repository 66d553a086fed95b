"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/mosaicq.h declares, and rejects invalid arguments with the documented
status codes before touching the device (fake, never-dereferenced pointer
values are used where a pointer must be non-NULL)."""
import ctypes
import os
import re

import pytest

from dense_sparse_w4a4_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mosaicq.h")

OK, NULLP, SHAPE, ALIGN, BLOCK, BUDGET, CSR, WS, HIP, ARG = range(10)

P = ctypes.c_void_p(0x1000)      # aligned fake device address (never reached)
PMIS = ctypes.c_void_p(0x1008)   # misaligned by 8


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ops.LIB_PATH):
        from dense_sparse_w4a4_amd import build
        build.build(verbose=False)
    return ops.lib()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mq_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    syms = declared_symbols()
    assert {"mq_quantize_act", "mq_select_blocks", "mq_pack_weights", "mq_fused_gemm"} <= set(syms)
    for s in syms:
        assert hasattr(L, s), f"{s} not exported"


def test_status_strings_and_version(L):
    assert ops.status_str(0) == "MQ_OK"
    assert ops.status_str(SHAPE) == "MQ_ERR_SHAPE"
    assert ops.status_str(99) == "MQ_ERR_UNKNOWN"
    assert L.mq_version() >> 16 == 1


def test_quantize_act_validation(L):
    f = L.mq_quantize_act
    assert f(P, 4, 100, 128, P, P, None) == SHAPE            # K % 128
    assert f(P, -1, 128, 128, P, P, None) == SHAPE           # M < 0
    assert f(P, 4, 128, 64, P, P, None) == SHAPE             # ldx < K
    assert f(None, 4, 128, 128, P, P, None) == NULLP
    assert f(P, 4, 128, 132, P, P, None) == ALIGN            # ldx % 8
    assert f(PMIS, 4, 128, 128, P, P, None) == ALIGN
    assert "128" in ops.last_error() or "align" in ops.last_error()
    assert f(None, 0, 128, 128, None, None, None) == OK      # M == 0: nothing to do


def test_select_validation(L):
    f = L.mq_select_blocks
    assert f(P, P, 512, 512, 64, 48, 6, P, P, P, None) == BLOCK
    assert f(P, P, 500, 512, 64, 64, 6, P, P, P, None) == SHAPE
    assert f(P, P, 512, 500, 64, 64, 6, P, P, P, None) == SHAPE
    assert f(P, P, 512, 512, 64, 64, 65, P, P, P, None) == BUDGET
    assert f(P, P, 512, 512, 64, 64, -1, P, P, P, None) == BUDGET
    assert f(P, P, 512, 512, 64, 64, 6, None, P, P, None) == NULLP
    assert f(P, None, 512, 512, 64, 64, 6, P, P, P, None) == NULLP
    assert f(P, P, 512, 512, 64, 64, 6, P, None, P, None) == NULLP
    assert f(P, P, 512, 512, 64, 64, 6, P, P, PMIS, None) == ALIGN


def test_pack_validation(L):
    f = L.mq_pack_weights
    args = dict(w=P, N=512, K=512, b=64, sel=P, ns=6, qw=P, sw=P, rp=P, ci=P, qr=P, sr=P)

    def call(**kw):
        a = {**args, **kw}
        return f(a["w"], a["N"], a["K"], a["b"], a["sel"], a["ns"], a["qw"], a["sw"], a["rp"],
                 a["ci"], a["qr"], a["sr"], None)
    assert call(b=16) == BLOCK
    assert call(N=96) == SHAPE
    assert call(K=192) == SHAPE
    assert call(ns=65) == BUDGET
    assert call(qr=None) == NULLP
    assert call(rp=None) == NULLP
    assert call(sw=PMIS) == ALIGN


def _gemm(L, **kw):
    a = dict(qa=P, sa=P, M=16, N=512, K=512, qw=P, sw=P, b=64, ns=6, rp=P, ci=P, qr=P, sr=P,
             y=P, ldy=512, ws=None, wsb=0, flags=0, dump=None)
    a.update(kw)
    return L.mq_fused_gemm(a["qa"], a["sa"], a["M"], a["N"], a["K"], a["qw"], a["sw"], a["b"],
                           a["ns"], a["rp"], a["ci"], a["qr"], a["sr"], a["y"], a["ldy"], a["ws"],
                           a["wsb"], a["flags"], a["dump"], None)


def test_fused_gemm_validation(L):
    assert _gemm(L, flags=8) == ARG
    assert _gemm(L, flags=2 | 4) == ARG  # the int8 and fp6 routes exclude each other
    assert _gemm(L, b=100) == BLOCK
    assert _gemm(L, M=-3) == SHAPE
    assert _gemm(L, N=100) == SHAPE
    assert _gemm(L, K=640 - 64) == SHAPE
    assert _gemm(L, ldy=256) == SHAPE
    assert _gemm(L, ns=65) == BUDGET
    assert _gemm(L, qa=None) == NULLP
    assert _gemm(L, ci=None) == NULLP
    assert _gemm(L, flags=1) == NULLP                 # dump without a buffer
    assert _gemm(L, ldy=516) == ALIGN
    assert _gemm(L, qw=PMIS) == ALIGN
    assert _gemm(L, M=0, qa=None, y=None) == OK      # empty batch
    # 32-bit kernel offsets: packed weights or activations of 4 GiB or more are refused
    assert _gemm(L, N=65536, K=131072, ldy=65536, b=128) == SHAPE
    assert "4 GiB" in ops.last_error()
    assert _gemm(L, M=1 << 16, N=512, K=131072, b=128) == SHAPE


def test_workspace_query(L):
    n = ctypes.c_size_t(123)
    assert L.mq_fused_gemm_workspace(16, 4096, 4096, ctypes.byref(n)) == OK
    assert n.value == 0
    assert L.mq_fused_gemm_workspace(16, 4096, 4096, None) == NULLP


def test_validate_csr_argument_errors(L):
    f = L.mq_validate_csr
    assert f(P, P, 512, 512, 48, 6, None) == BLOCK
    assert f(None, P, 512, 512, 64, 6, None) == NULLP
    assert f(P, None, 512, 512, 64, 6, None) == NULLP


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(ops, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(ops, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        ops.lib()


def _layer_call(L, **kw):
    a = dict(x=P, M=4, K=512, ldx=512, N=512, qw=P, sw=P, b=64, ns=6, rp=P, ci=P, qr=P, sr=P,
             y=P, ldy=512, ws=None, wsb=0)
    a.update(kw)
    return L.mq_fused_layer(a["x"], a["M"], a["K"], a["ldx"], a["N"], a["qw"], a["sw"], a["b"],
                            a["ns"], a["rp"], a["ci"], a["qr"], a["sr"], a["y"], a["ldy"], a["ws"],
                            a["wsb"], None)


def test_fused_layer_workspace_and_validation(L):
    n = ctypes.c_size_t(123)
    # decode-sized token tiles are quantised inside the GEMM: no workspace
    for M in (1, 4):
        assert L.mq_fused_layer_workspace(M, 4096, 4096, ctypes.byref(n)) == OK
        assert n.value == 0
    # otherwise codes in 16-token tiles (M padded to a multiple of 16, K/2
    # bytes per token) and scales [M][K/128] fp32, each rounded up to 256 bytes
    assert L.mq_fused_layer_workspace(16, 4096, 4096, ctypes.byref(n)) == OK
    assert n.value == 16 * 2048 + 16 * 32 * 4
    assert L.mq_fused_layer_workspace(5, 512, 640, ctypes.byref(n)) == OK
    assert n.value == 16 * 320 + 256
    assert L.mq_fused_layer_workspace(4, 4096, 4096, None) == NULLP
    assert _layer_call(L, b=100) == BLOCK
    assert _layer_call(L, ldx=256) == SHAPE
    assert _layer_call(L, ldy=256) == SHAPE
    assert _layer_call(L, K=500) == SHAPE
    assert _layer_call(L, ns=65) == BUDGET
    assert _layer_call(L, x=None) == NULLP
    assert _layer_call(L, ldx=516) == ALIGN
    assert _layer_call(L, x=PMIS) == ALIGN
    assert _layer_call(L, M=16) == WS                     # two-kernel route needs the workspace
    assert _layer_call(L, M=16, ws=P, wsb=16 * 256 + 16 * 4 * 4 - 1) == WS
    assert _layer_call(L, M=0, x=None, y=None) == OK      # empty batch


def test_smooth_size_limits(L):
    # sizes whose launches would exceed 32-bit work-item counts are refused
    # before anything is enqueued (fake pointers are never dereferenced)
    big = 1 << 31
    fw = L.mq_smooth_weights
    assert fw(P, 4, P, 4, 0, P, P, P, ctypes.c_void_p(0x2000), None) == SHAPE       # K < 1
    assert fw(P, big, P, 4, 1, P, P, P, ctypes.c_void_p(0x2000), None) == SHAPE     # T >= 2^31
    assert fw(P, 4, P, big, 1, P, P, P, ctypes.c_void_p(0x2000), None) == SHAPE     # N >= 2^31
    assert fw(P, 4, P, 1 << 21, 1 << 19, P, P, P, ctypes.c_void_p(0x2000), None) == SHAPE  # N*K = 2^40
    assert fw(P, 4, P, 4, 8, P, P, P, P, None) == ARG                               # w_out aliases w
    fa = L.mq_smooth_acts
    assert fa(P, big, 8, 8, P, P, None) == SHAPE                                    # M >= 2^31
    assert fa(P, 4, big, big, P, P, None) == SHAPE                                  # K >= 2^31
    assert fa(P, 1 << 21, 1 << 19, 1 << 19, P, P, None) == SHAPE                    # M*K = 2^40
    assert fa(None, 0, 8, 8, None, None, None) == OK                                # empty batch


def test_measure_mfma_validation(L):
    f = L.mq_measure_mfma
    assert f(0, 10, P, P, None) == SHAPE
    assert f(4, 0, P, P, None) == SHAPE
    assert f(4, 10, None, P, None) == NULLP
    assert f(4, 10, P, PMIS, None) == ALIGN


def test_fused_layer_noalloc_validation(L):
    f = L.mq_fused_layer_noalloc

    def call(**kw):
        a = dict(x=P, M=4, K=512, ldx=512, N=512, qw=P, sw=P, b=64, ns=6, rp=P, ci=P, qr=P, sr=P,
                 y=P, ldy=512)
        a.update(kw)
        return f(a["x"], a["M"], a["K"], a["ldx"], a["N"], a["qw"], a["sw"], a["b"], a["ns"], a["rp"],
                 a["ci"], a["qr"], a["sr"], a["y"], a["ldy"], None)
    assert call(b=100) == BLOCK
    assert call(K=500) == SHAPE
    assert call(ns=65) == BUDGET
    assert call(x=None) == NULLP
    assert call(x=PMIS) == ALIGN
    assert call(M=0, x=None, y=None) == OK
    # a shape whose workspace passes the 128 MiB scratch is refused before any
    # device call
    assert call(M=8192, K=25600, ldx=25600, N=128, ldy=128, ns=0) == WS
    assert "scratch" in ops.last_error()


def test_exact_selection_validation(L):
    n = ctypes.c_size_t(0)
    fw = L.mq_select_exact_workspace
    assert fw(512, 512, 128, 64, ctypes.byref(n)) == OK
    # rem fp64 + R_hat fp32 per weight, outputs fp64 per (token, output), and
    # per-block gains, tile partials, flags, order and pick gains
    assert n.value >= 12 * 512 * 512 + 8 * 128 * 512 + 64 * (8 + 2 * 2 * 8 + 1 + 4 + 8)
    assert fw(512, 512, 128, 48, ctypes.byref(n)) == BLOCK
    assert fw(500, 512, 128, 64, ctypes.byref(n)) == SHAPE
    assert fw(512, 512, 1 << 22, 64, ctypes.byref(n)) == SHAPE
    assert fw(1 << 17, 1 << 17, 8, 32, ctypes.byref(n)) == SHAPE   # 2^24 blocks
    assert fw(512, 512, 128, 64, None) == NULLP

    g = L.mq_select_exact_greedy

    def call(**kw):
        a = dict(w=P, x=P, N=512, K=512, T=128, b=64, ns=6, sel=P, order=None, gains=None,
                 dist=None, ws=P, wsb=1 << 30)
        a.update(kw)
        return g(a["w"], a["x"], a["N"], a["K"], a["T"], a["b"], a["ns"], a["sel"], a["order"],
                 a["gains"], a["dist"], a["ws"], a["wsb"], None)
    assert call(b=100) == BLOCK
    assert call(K=500) == SHAPE
    assert call(ns=65) == BUDGET
    assert call(ns=-1) == BUDGET
    assert call(w=None) == NULLP
    assert call(x=None) == NULLP
    assert call(sel=None) == NULLP
    assert call(ws=None) == NULLP
    assert call(order=PMIS) == ALIGN
    assert call(wsb=1024) == WS

    d = L.mq_distortion
    fd = L.mq_distortion_workspace
    assert fd(512, 512, 128, 64, ctypes.byref(n)) == OK and n.value >= 8 * 512 * 512

    def dcall(**kw):
        a = dict(w=P, x=P, N=512, K=512, T=128, b=64, sel=P, ns=6, dist=P, ws=P, wsb=1 << 30)
        a.update(kw)
        return d(a["w"], a["x"], a["N"], a["K"], a["T"], a["b"], a["sel"], a["ns"], a["dist"],
                 a["ws"], a["wsb"], None)
    assert dcall(b=16) == BLOCK
    assert dcall(N=96) == SHAPE
    assert dcall(ns=-2) == BUDGET
    assert dcall(sel=None) == NULLP
    assert dcall(dist=None) == NULLP
    assert dcall(x=PMIS) == ALIGN
    assert dcall(wsb=4096) == WS


def test_fp6_route_validation(L):
    a, w, p = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    sz = lambda *args: L.mq_fp6_sizes(*args, ctypes.byref(a), ctypes.byref(w), ctypes.byref(p))  # noqa: E731
    assert sz(4096, 25600, 5120, 64, 3200) == OK
    assert a.value == 4096 // 32 * 40 * 3072
    assert w.value == 5120 * 25600 * 3 // 4 + 3200 * 64 * 64 * 3 // 4  # (base a multiple of 256)
    assert p.value == 0  # 3200 tiles: 12.5 rounds, no split
    assert sz(4096, 5120, 25600, 64, 3200) == OK
    assert p.value == 2 * 4096 * 5120 * 4  # 640 tiles, 2.5 rounds: two splits, 5 rounds
    assert sz(300, 256, 2048, 64, 10) == OK and p.value == 300 * 256 * 4 * 2  # two K splits
    assert sz(4096, 5120, 25600, 32, 0) == BLOCK
    assert sz(4096, 5120, 25600, 64, 10 ** 6) == BUDGET
    assert sz(4096, 5000, 25600, 64, 0) == SHAPE
    assert L.mq_fp6_sizes(64, 64, 128, 64, 0, None, None, None) == NULLP
    prep = L.mq_fp6_prepare_weights
    assert prep(P, 64, 128, 32, 0, None, P, None) == BLOCK
    assert prep(None, 64, 128, 64, 0, None, P, None) == NULLP
    assert prep(P, 64, 128, 64, 1, None, P, None) == NULLP
    assert prep(PMIS, 64, 128, 64, 0, None, P, None) == ALIGN
    assert L.mq_fp6_prepare_acts(P, 64, 100, P, None) == SHAPE
    assert L.mq_fp6_prepare_acts(None, 64, 128, P, None) == NULLP
    g = lambda **kw: L.mq_fused_gemm_fp6(  # noqa: E731
        kw.get("ai", P), P, kw.get("M", 64), kw.get("N", 128), kw.get("K", 256), P, P, kw.get("b", 64), 0,
        None, None, None, P, kw.get("ldy", 128), kw.get("ws", None), kw.get("wsb", 0),
        kw.get("flags", 0), None, None)
    assert g(M=16) == SHAPE
    assert g(b=32) == BLOCK
    assert g(flags=2) == ARG
    assert g(flags=1) == NULLP  # dump without acc_dump
    assert g(ai=None) == NULLP
    assert g(ldy=100) == SHAPE
    assert g(M=300, N=256, K=2048, ldy=256) == WS  # split-K partials needed, none given
    assert g(M=0) == OK
