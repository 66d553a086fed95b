"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: activation codes and scales, H, Delta, selected ids, packed base
and residual bytes and scales, the int32 accumulators (debug dump).
Within tolerance (parity_util.YTOL): the fp16 output y.
Full-size layer shapes check every integer/byte output in full and y on
sampled block-row tiles the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
from dense_sparse_w4a4_amd import ops
from dense_sparse_w4a4_amd import synthetic as syn
from parity_util import (assert_packed_equal, assert_y_close, dev, f16_bits, host,
                         tile_rows_reference)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()
    yield
    torch.cuda.synchronize()


def _check_act(x16: np.ndarray, ldx_pad: int = 0):
    M, K = x16.shape
    if ldx_pad:
        big = np.zeros((M, K + ldx_pad), np.float16)
        big[:, :K] = x16
        xt = dev(big)[:, :K]
    else:
        xt = dev(x16)
    qa, sa = ops.quantize_act(xt)
    rq, rs = oracle.quantize_act(x16)
    torch.cuda.synchronize()
    assert np.array_equal(host(qa), oracle.pack_nibbles(rq))
    assert np.array_equal(host(sa).view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("M,K,pad", [(1, 128, 0), (5, 512, 8), (16, 4096, 0), (17, 14336, 0),
                                     (300, 1024, 64),
                                     # prefill sizes, a padded row stride
                                     (1025, 4096, 0), (2048, 4096, 8)])
def test_act_quant_bit_exact(M, K, pad):
    spec = syn.LayerSpec("t", K=K, N=128)
    _check_act(syn.make_acts(spec, M, seed=M), pad)


def test_act_quant_special_values():
    rng = np.random.default_rng(0)
    x = np.zeros((8, 256), np.float16)
    x[0, :] = 0                                                    # all-zero groups
    x[1, :] = (rng.standard_normal(256) * 1e-6).astype(np.float16)  # subnormals
    x[2, :] = np.float16(65504.0) * np.sign(rng.standard_normal(256)).astype(np.float16)
    x[3, :128] = np.arange(128) * 0.5 - 32                         # ties at amax 32 -> s = 32/7
    x[4, :128] = 7.0 * (np.arange(128) % 3 - 1)
    x[4, 128:] = np.linspace(-3.5, 3.5, 128)
    x[5, :] = np.float16(6e-8)
    x[6, :] = rng.standard_normal(256).astype(np.float16)          # an infinite value per group:
    x[6, 17], x[6, 200] = np.inf, -np.inf                          # scale +inf, every code 0
    x[7, :128] = np.inf
    x[7, 128:] = rng.standard_normal(128).astype(np.float16)
    _check_act(x)


def _layer(spec, seed=0):
    return syn.make_weight(spec, seed), syn.make_calib(spec, seed)


@pytest.mark.parametrize("b", [32, 64, 128])
def test_select_bit_exact_tiny(b):
    spec = syn.TINY.with_block(b)
    w, xc = _layer(spec)
    sel, delta, H = ops.select_blocks(dev(w), dev(xc), b, spec.n_select)
    rsel, rdelta, rH = oracle.select_blocks(w, xc, b, spec.n_select)
    torch.cuda.synchronize()
    assert np.array_equal(host(H).view(np.uint64), rH.view(np.uint64))
    assert np.array_equal(host(delta).view(np.uint64), rdelta.view(np.uint64))
    assert np.array_equal(host(sel), rsel)


def test_select_ties_and_extremes():
    # integer weights with a 7 in every group: E = 0, every score is 0, ties
    # must resolve to the lowest ids; also n_select = 0 and n_select = B
    rng = np.random.default_rng(1)
    w = rng.integers(-7, 8, size=(128, 256)).astype(np.float16)
    w[:, ::128] = 7
    xc = rng.standard_normal((16, 256)).astype(np.float16)
    for ns in (0, 3, 8):
        sel, delta, _ = ops.select_blocks(dev(w), dev(xc), 64, ns)
        torch.cuda.synchronize()
        assert host(sel).tolist() == list(range(ns))
        assert not np.any(host(delta))
    spec = syn.TINY
    w, xc = _layer(spec, seed=3)
    sel, _, _ = ops.select_blocks(dev(w), dev(xc), 64, spec.n_blocks)
    torch.cuda.synchronize()
    assert host(sel).tolist() == list(range(spec.n_blocks))


def test_pack_golden_residual_row():
    # the hand-derived residual row (tests/golden/hand_quant.json): the GPU's
    # packed bytes and scale bits against the stored values directly
    import json
    import os
    f = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_quant.json")))["residual_row_b32"]
    b = f["block"]
    w = np.zeros((b, 128), np.float16)
    w[0, :len(f["values"])] = f["values"]
    layer = ops.pack_weights(dev(w), b, torch.zeros(1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    qr, sr = host(layer.qr), host(layer.sr).view(np.uint16)
    assert qr[0, 0, :3].tolist() == f["qr_bytes"]
    assert not np.any(qr[0, 0, 3:]) and not np.any(qr[0, 1:])
    assert int(sr[0, 0]) == f["sr_f16_bits"] and not np.any(sr[0, 1:])
    assert host(layer.row_ptr).tolist() == [0, 1] and host(layer.col_idx).tolist() == [0]


@pytest.mark.parametrize("b,rho", [(32, 0.1), (64, 0.0), (64, 0.1), (64, 1.0), (128, 0.2)])
def test_pack_bit_exact(b, rho):
    spec = syn.TINY.with_block(b, rho)
    w, xc = _layer(spec, seed=b)
    rsel, _, _ = oracle.select_blocks(w, xc, b, spec.n_select)
    layer = ops.pack_weights(dev(w), b, dev(rsel.astype(np.int32)))
    ref = oracle.pack_weights(w, b, rsel)
    torch.cuda.synchronize()
    assert_packed_equal(layer, ref)
    ops.validate_csr(layer)


GEMM_CASES = [
    # M, N, K, b, rho
    (16, 512, 512, 64, 0.10),
    (1, 512, 512, 64, 0.10),
    (17, 256, 384, 32, 0.25),
    (40, 384, 256, 128, 0.50),
    (3, 128, 128, 64, 1.00),
    (16, 512, 512, 64, 0.0),
    (70, 256, 1024, 64, 0.10),
    (2, 64, 2048, 32, 0.05),
    # large-M tile kernel: 32-wide blocks, partial channel tiles, ragged M
    (100, 256, 512, 32, 0.30),
    (130, 96, 384, 32, 0.20),
    (257, 192, 256, 64, 0.15),
    (64, 128, 1024, 128, 0.25),
    (33, 64, 128, 64, 1.00),
    # split-K tile schedule (few tiles, long K): fp32 partials + ordered reduce
    (300, 256, 2048, 64, 0.10),
    (40, 128, 4096, 128, 0.25),
    (129, 384, 3072, 32, 0.15),
    # uneven split-K: 25 groups over 3 splits of 8, 8 and 9 groups (an odd
    # count in the last split)
    (40, 128, 3200, 64, 0.10),
    # streaming kernel with four 16-channel slabs per workgroup (M > 4 and
    # 128 workgroups of 64 channels x two token tiles, the second ragged)
    (20, 8192, 4096, 64, 0.10),
]


@pytest.mark.parametrize("M,N,K,b,rho", GEMM_CASES)
def test_fused_gemm_accumulators_exact_and_y(M, N, K, b, rho):
    spec = syn.LayerSpec("g", K=K, N=N, w_outlier_frac=0.01, x_outlier_count=3,
                         T=32, block=b, rho=rho)
    w, xc = _layer(spec, seed=M + N)
    x = syn.make_acts(spec, M, seed=K)
    rsel, _, _ = oracle.select_blocks(w, xc, b, spec.n_select)
    ref = oracle.pack_weights(w, b, rsel)
    rqa, rsa = oracle.quantize_act(x)
    y_ref, acc_ref, res_ref = oracle.fused_gemm(rqa, rsa, ref)
    # the GPU GEMM consumes the oracle's packed data (inputs, not expected values)
    layer = ops.PackedLayer(N, K, b, dev(ref["qw"]), dev(ref["sw"]), dev(ref["row_ptr"]),
                            dev(ref["col_idx"]), dev(ref["qr"]), dev(ref["sr"]))
    qa, sa = dev(oracle.pack_nibbles(rqa)), dev(rsa)
    y, acc, res = ops.fused_gemm(qa, sa, layer, dump=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc).astype(np.int64), acc_ref)
    if len(res_ref):
        assert np.array_equal(host(res).astype(np.int64), np.stack(res_ref))
    assert_y_close(y, y_ref)
    # the production launch (no dump) gives the same bits
    y2 = ops.fused_gemm(qa, sa, layer)
    torch.cuda.synchronize()
    assert np.array_equal(host(y2).view(np.uint16), host(y).view(np.uint16))


@pytest.mark.parametrize("M,N,K,b,rho", [(257, 192, 256, 64, 0.15), (300, 256, 2048, 64, 0.10),
                                         (64, 128, 1024, 128, 0.25), (40, 128, 3200, 64, 0.10),
                                         (513, 640, 1536, 64, 0.20), (1000, 384, 640, 128, 0.10),
                                         (1030, 256, 1024, 64, 0.10)])
def test_fp6_route_matches_int8_route(M, N, K, b, rho):
    # the prefill kernel's two routes on the same codes: identical exact
    # accumulators (the oracle's) and identical y bits, with and without the
    # dump; below 1024 tokens the fp6 route re-encodes the packed base codes
    # in the kernel, from 1024 it converts them into an image first
    print(f"fp6 vs int8 M={M} N={N} K={K} b={b} rho={rho}", flush=True)
    spec = syn.LayerSpec("r", K=K, N=N, w_outlier_frac=0.01, x_outlier_count=3,
                         T=32, block=b, rho=rho)
    w, xc = _layer(spec, seed=M + 7)
    x = syn.make_acts(spec, M, seed=N)
    rsel, _, _ = oracle.select_blocks(w, xc, b, spec.n_select)
    ref = oracle.pack_weights(w, b, rsel)
    rqa, rsa = oracle.quantize_act(x)
    layer = ops.PackedLayer(N, K, b, dev(ref["qw"]), dev(ref["sw"]), dev(ref["row_ptr"]),
                            dev(ref["col_idx"]), dev(ref["qr"]), dev(ref["sr"]))
    qa, sa = dev(oracle.pack_nibbles(rqa)), dev(rsa)
    y6, a6, r6 = ops.fused_gemm(qa, sa, layer, dump=True, route="fp6")
    y8, a8, r8 = ops.fused_gemm(qa, sa, layer, dump=True, route="int8")
    z6 = ops.fused_gemm(qa, sa, layer, route="fp6")
    z8 = ops.fused_gemm(qa, sa, layer, route="int8")
    torch.cuda.synchronize()
    assert torch.equal(a6, a8) and torch.equal(r6, r8)
    y_ref, acc_ref, res_ref = oracle.fused_gemm(rqa, rsa, ref)
    assert np.array_equal(host(a6).astype(np.int64), acc_ref)
    if len(res_ref):
        assert np.array_equal(host(r6).astype(np.int64), np.stack(res_ref))
    assert_y_close(y6, y_ref)
    assert np.array_equal(host(y6).view(np.uint16), host(y8).view(np.uint16))
    assert np.array_equal(host(z6).view(np.uint16), host(z8).view(np.uint16))
    assert np.array_equal(host(z6).view(np.uint16), host(y6).view(np.uint16))


def test_end_to_end_tiny_and_determinism():
    spec = syn.TINY
    x = syn.make_acts(spec, syn.TINY_M)
    w, xc = _layer(spec)
    ref = oracle.layer_reference(x, w, xc, spec.block, spec.n_select)
    sel, _, _ = ops.select_blocks(dev(w), dev(xc), spec.block, spec.n_select)
    layer = ops.pack_weights(dev(w), spec.block, sel)
    xt = dev(x)
    y = ops.layer_forward(xt, layer)
    y_again = ops.layer_forward(xt, layer)
    torch.cuda.synchronize()
    assert np.array_equal(host(sel), ref["selected"])
    assert_packed_equal(layer, ref["packed"])
    assert_y_close(y, ref["y"])
    assert np.array_equal(host(y).view(np.uint16), host(y_again).view(np.uint16))


def test_empty_batch_is_a_no_op():
    spec = syn.TINY
    w, xc = _layer(spec)
    layer = ops.pack_weights(dev(w), 64, torch.zeros(0, dtype=torch.int32, device="cuda"))
    x = torch.zeros((0, 512), dtype=torch.float16, device="cuda")
    y = ops.layer_forward(x, layer)
    torch.cuda.synchronize()
    assert y.shape == (0, 512)


FULL = [(K, N, M) for (K, N) in syn.LLAMA3_8B_SHAPES for M in (1, 16, 2048)]


@pytest.mark.parametrize("K,N,M", FULL)
def test_full_size_llama3_8b(K, N, M):
    spec = syn.llama3_8b(K, N)
    w, xc = _layer(spec)
    x = syn.make_acts(spec, M)
    wt = dev(w)
    sel, delta, H = ops.select_blocks(wt, dev(xc), spec.block, spec.n_select)
    layer = ops.pack_weights(wt, spec.block, sel)
    qa, sa = ops.quantize_act(dev(x))
    y = ops.fused_gemm(qa, sa, layer)
    torch.cuda.synchronize()
    # integer/byte outputs in full
    rqa, rsa = oracle.quantize_act(x)
    assert np.array_equal(host(qa), oracle.pack_nibbles(rqa))
    assert np.array_equal(host(sa).view(np.uint32), rsa.view(np.uint32))
    rsel, rdelta, rH = oracle.select_blocks(w, xc, spec.block, spec.n_select)
    assert np.array_equal(host(H).view(np.uint64), rH.view(np.uint64))
    assert np.array_equal(host(delta).view(np.uint64), rdelta.view(np.uint64))
    assert np.array_equal(host(sel), rsel)
    ref = oracle.pack_weights(w, spec.block, rsel)
    assert_packed_equal(layer, ref)
    # y on sampled block-row tiles (includes the tiles with the most residual blocks)
    counts = np.diff(ref["row_ptr"])
    NT = N // spec.block
    tiles = sorted({0, NT - 1, int(np.argmax(counts)), NT // 2})
    yt = host(y)
    for nt, yref in tile_rows_reference(rqa, rsa, ref, tiles).items():
        b = spec.block
        assert_y_close(torch.from_numpy(yt[:, nt * b:(nt + 1) * b]), yref)


def test_graph_replay_matches_eager():
    # capture act-quant + fused GEMM in a HIP graph; replay it several times
    # with eager work and synchronisations in between; every replay must
    # reproduce the eager output bit for bit
    spec = syn.llama3_8b(4096, 4096)
    w, xc = _layer(spec)
    x = dev(syn.make_acts(spec, 4))
    wt = dev(w)
    sel, _, _ = ops.select_blocks(wt, dev(xc), spec.block, spec.n_select)
    layer = ops.pack_weights(wt, spec.block, sel)
    qa = torch.empty((4, 2048), dtype=torch.uint8, device="cuda")
    sa = torch.empty((4, 32), dtype=torch.float32, device="cuda")
    y = torch.empty((4, 4096), dtype=torch.float16, device="cuda")
    ops.quantize_act(x, qa, sa)
    ops.fused_gemm(qa, sa, layer, out=y)
    torch.cuda.synchronize()
    ref = host(y).view(np.uint16).copy()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        ops.quantize_act(x, qa, sa)
        ops.fused_gemm(qa, sa, layer, out=y)
    for i in range(4):
        y.zero_()
        qa.fill_(0x77)
        junk = ops.fused_gemm(qa, sa, layer)  # eager work on the same stream between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y).view(np.uint16), ref), f"replay {i} differs"
        del junk


def test_split_k_without_workspace_matches():
    # the same call with the workspace withheld runs one pass over K: the
    # accumulators are identical and y agrees within the tolerance
    M, N, K, b = 300, 256, 2048, 64
    assert ops.fused_gemm_workspace(M, N, K) > 0
    spec = syn.LayerSpec("s", K=K, N=N, T=32, block=b, rho=0.1)
    w, xc = _layer(spec, seed=5)
    x = syn.make_acts(spec, M, seed=6)
    rsel, _, _ = oracle.select_blocks(w, xc, b, spec.n_select)
    ref = oracle.pack_weights(w, b, rsel)
    rqa, rsa = oracle.quantize_act(x)
    y_ref, _, _ = oracle.fused_gemm(rqa, rsa, ref)
    layer = ops.PackedLayer(N, K, b, dev(ref["qw"]), dev(ref["sw"]), dev(ref["row_ptr"]),
                            dev(ref["col_idx"]), dev(ref["qr"]), dev(ref["sr"]))
    qa, sa = dev(oracle.pack_nibbles(rqa)), dev(rsa)
    y_split = ops.fused_gemm(qa, sa, layer)
    y_one = torch.empty_like(y_split)
    st = ops._check("mq_fused_gemm", ops.lib().mq_fused_gemm(
        ops._ptr(qa), ops._ptr(sa), M, N, K, ops._ptr(layer.qw), ops._ptr(layer.sw), b,
        layer.n_select, ops._ptr(layer.row_ptr), ops._ptr(layer.col_idx), ops._ptr(layer.qr),
        ops._ptr(layer.sr), ops._ptr(y_one), N, None, 0, 0, None, ops._stream(None)))
    torch.cuda.synchronize()
    assert st is None
    assert_y_close(y_split, y_ref)
    assert_y_close(y_one, y_ref)


def _gemm_without_workspace(qa, sa, layer, M, dump=False):
    """mq_fused_gemm with no workspace (the tile kernel then makes one pass over K)."""
    N, K, b, ns = layer.N, layer.K, layer.block, layer.n_select
    y = torch.empty((M, N), dtype=torch.float16, device=qa.device)
    acc = None
    if dump:
        acc = torch.empty(M * N * (K // 128) + ns * M * b, dtype=torch.int32, device=qa.device)
    st = ops._check("mq_fused_gemm", ops.lib().mq_fused_gemm(
        ops._ptr(qa), ops._ptr(sa), M, N, K, ops._ptr(layer.qw), ops._ptr(layer.sw), b, ns,
        ops._ptr(layer.row_ptr) if ns else None, ops._ptr(layer.col_idx) if ns else None,
        ops._ptr(layer.qr) if ns else None, ops._ptr(layer.sr) if ns else None,
        ops._ptr(y), N, None, 0, ops.FLAG_DUMP_ACC if dump else 0, ops._ptr(acc),
        ops._stream(None)))
    assert st is None
    return y, acc


@pytest.mark.parametrize("M,b", [(290, 32), (290, 64), (290, 128), (16, 64), (3, 32)])
def test_full_nibble_range(M, b):
    # codes over the whole nibble range [-8, 7] on every operand (the
    # quantisers stop at +-7), extreme rows and channels at -8: exact
    # accumulators through the tile kernel with split-K (workspace) and in one
    # pass (none), and through the streaming kernel for small M
    N, K = 256, 2048
    rng = np.random.default_rng(b + M)
    qa_codes = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    qa_codes[:2] = -8
    qw_codes = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    qw_codes[:16] = -8
    KT = K // b
    nsel = (N // b) * KT // 3
    sel = np.sort(rng.choice((N // b) * KT, size=nsel, replace=False)).astype(np.int32)
    row_ptr, col_idx = oracle.build_csr(sel, N, K, b)
    qr = rng.integers(0, 256, size=(nsel, b, b // 2)).astype(np.uint8)
    ref = dict(qw=oracle.slab_layout(oracle.pack_nibbles(qw_codes)),
               sw=(rng.random((N, K // 128)) * 0.02 + 1e-3).astype(np.float16),
               row_ptr=row_ptr, col_idx=col_idx, qr=qr,
               sr=(rng.random((nsel, b)) * 0.01 + 1e-4).astype(np.float16), block=b, N=N, K=K)
    sa_h = (rng.random((M, K // 128)) * 0.5 + 0.01).astype(np.float32)
    y_ref, acc_ref, res_ref = oracle.fused_gemm(qa_codes, sa_h, ref)
    layer = ops.PackedLayer(N, K, b, dev(ref["qw"]), dev(ref["sw"]), dev(row_ptr), dev(col_idx),
                            dev(qr), dev(ref["sr"]))
    qa, sa = dev(oracle.pack_nibbles(qa_codes)), dev(sa_h)
    if M > 32:
        assert ops.fused_gemm_workspace(M, N, K) > 0  # split-K with the workspace
    y, base, res = ops.fused_gemm(qa, sa, layer, dump=True)
    y1, acc1 = _gemm_without_workspace(qa, sa, layer, M, dump=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(base).astype(np.int64), acc_ref)
    assert np.array_equal(host(res).astype(np.int64), np.stack(res_ref))
    assert torch.equal(torch.cat([base.reshape(-1), res.reshape(-1)]), acc1)
    assert_y_close(y, y_ref)
    assert_y_close(y1, y_ref)
    if M > 32 and b != 32:
        # the fp6 route: -8 is the one code whose field leaves the subnormal
        # range (|q| = 8, exponent field 1)
        y6, base6, res6 = ops.fused_gemm(qa, sa, layer, dump=True, route="fp6")
        torch.cuda.synchronize()
        assert torch.equal(base6, base) and torch.equal(res6, res)
        assert np.array_equal(host(y6).view(np.uint16), host(y).view(np.uint16))


@pytest.mark.parametrize("M,b", [(16, 64), (300, 32), (70, 128)])
def test_unfused_ablation_matches(M, b):
    # dense-only fused GEMM followed by the standalone residual kernel gives
    # the layer output within the tolerance (the merge rounds y to fp16 once
    # more, which the tolerance covers)
    N, K = 512, 1024
    spec = syn.LayerSpec("abl", K=K, N=N, w_outlier_frac=0.01, x_outlier_count=3, T=32,
                         block=b, rho=0.2)
    w, xc = _layer(spec, seed=11)
    x = syn.make_acts(spec, M, seed=12)
    rsel, _, _ = oracle.select_blocks(w, xc, b, spec.n_select)
    ref = oracle.pack_weights(w, b, rsel)
    rqa, rsa = oracle.quantize_act(x)
    y_ref, _, _ = oracle.fused_gemm(rqa, rsa, ref)
    layer = ops.PackedLayer(N, K, b, dev(ref["qw"]), dev(ref["sw"]), dev(ref["row_ptr"]),
                            dev(ref["col_idx"]), dev(ref["qr"]), dev(ref["sr"]))
    dense = ops.PackedLayer(N, K, b, layer.qw, layer.sw, torch.zeros_like(layer.row_ptr),
                            layer.col_idx[:0], layer.qr[:0], layer.sr[:0])
    qa, sa = dev(oracle.pack_nibbles(rqa)), dev(rsa)
    y = ops.fused_gemm(qa, sa, dense)
    ops.residual_merge(qa, sa, layer, y)
    torch.cuda.synchronize()
    # the unfused design rounds the dense partial to fp16 before the merge:
    # one more rounding of at most 2^-12 |y_dense| on top of the layer's bound
    dref = oracle.pack_weights(w, b, rsel[:0])
    y_dense_ref, _, _ = oracle.fused_gemm(rqa, rsa, dref)
    yg = host(y).astype(np.float64)
    rms = float(np.sqrt(np.mean(y_ref * y_ref)))
    bound = 1e-3 * np.maximum(np.abs(y_ref), rms) + 2.0 ** -12 * np.abs(y_dense_ref)
    assert np.all(np.abs(yg - y_ref) <= bound)


def test_smooth_bit_exact():
    rng = np.random.default_rng(21)
    K, N, T, M = 1024, 384, 64, 20
    spec = syn.LayerSpec("sm", K=K, N=N, w_outlier_frac=0.01, T=T, block=64, rho=0.1)
    w = syn.make_weight(spec)
    xc = syn.make_calib(spec)
    x = syn.make_acts(spec, M)
    xc[:, 7] = 0           # zero calibration column -> s = 1
    w[:, 9] = 0            # zero weight column -> s = 1
    w[3, 11] = np.float16(-65504.0)
    s, w2, ax, aw = ops.smooth_weights(dev(xc), dev(w))
    x2 = ops.smooth_acts(dev(x), s)
    rs = oracle.smooth_scales(xc, w)
    torch.cuda.synchronize()
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(w2).view(np.uint16), oracle.smooth_weights(w, rs).view(np.uint16))
    assert np.array_equal(host(x2).view(np.uint16), oracle.smooth_acts(x, rs).view(np.uint16))
    assert np.array_equal(host(ax), np.abs(xc.astype(np.float32)).max(0))
    assert np.array_equal(host(aw), np.abs(w.astype(np.float32)).max(0))


def _sanitized(ref, row_ptr, col_idx):
    """The residual the kernels use for an arbitrary CSR: per block row, the
    entries [clip(rp[nt]), clip(rp[nt+1])) with rp clipped to [0, n_select]
    and non-decreasing, minus entries whose block column is out of range."""
    ns = len(ref["qr"])
    KT = ref["K"] // ref["block"]
    keep, rows = [], [0]
    for nt in range(len(row_ptr) - 1):
        e0 = min(max(int(row_ptr[nt]), 0), ns)
        e1 = min(max(int(row_ptr[nt + 1]), e0), ns)
        kept = [e for e in range(e0, e1) if 0 <= int(col_idx[e]) < KT]
        keep += kept
        rows.append(rows[-1] + len(kept))
    keep = np.array(keep, dtype=np.int64)
    return dict(ref, row_ptr=np.array(rows, np.int32), col_idx=col_idx[keep].astype(np.int32),
                qr=ref["qr"][keep], sr=ref["sr"][keep])


@pytest.mark.parametrize("M,merge", [(5, False), (70, False), (5, True), (70, True)])
def test_corrupt_csr_is_clipped_not_read_out_of_bounds(M, merge):
    # a CSR the validator rejects: row pointers past n_select or negative,
    # block columns outside [0, K/b), and (merge) a negative then an
    # oversized pointer that make one block row span every entry.  The
    # kernels clip the row ranges and skip out-of-range columns, so every
    # access stays in bounds.  The streaming kernel (M = 5) adds every entry
    # of a row, which is the sanitised reference below; the tile kernel
    # (M = 70) keeps one entry per (row, column), so where clipping merges
    # rows that hold the same column its output is only required to be
    # finite.
    N, K, b = 256, 1024, 64
    spec = syn.LayerSpec("c", K=K, N=N, T=32, block=b, rho=0.25)
    w, xc = _layer(spec, seed=11)
    rsel, _, _ = oracle.select_blocks(w, xc, b, spec.n_select)
    ref = oracle.pack_weights(w, b, rsel)
    ns = len(rsel)
    rp = ref["row_ptr"].copy()
    ci = ref["col_idx"].copy()
    rp[0] = -3
    rp[-1] = ns + 7
    ci[0] = -5
    ci[min(3, ns - 1)] = K // b + 3
    if merge:
        rp[1] = -3
        rp[2] = ns + 7
    layer = ops.PackedLayer(N, K, b, dev(ref["qw"]), dev(ref["sw"]), dev(rp), dev(ci),
                            dev(ref["qr"]), dev(ref["sr"]))
    with pytest.raises(ops.MosaicQError):
        ops.validate_csr(layer)
    x = syn.make_acts(spec, M, seed=3)
    rqa, rsa = oracle.quantize_act(x)
    qa, sa = dev(oracle.pack_nibbles(rqa)), dev(rsa)
    print(f"corrupt CSR M={M} merge={merge}", flush=True)
    y = ops.fused_gemm(qa, sa, layer)
    # the unfused ablation on the same CSR: dense-only GEMM, then the merge
    dense = ops.PackedLayer(N, K, b, layer.qw, layer.sw, torch.zeros_like(layer.row_ptr),
                            layer.col_idx[:0], layer.qr[:0], layer.sr[:0])
    yu = ops.fused_gemm(qa, sa, dense)
    ops.residual_merge(qa, sa, layer, yu)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(host(y).astype(np.float64)))
    assert np.all(np.isfinite(host(yu).astype(np.float64)))
    y_ref, _, _ = oracle.fused_gemm(rqa, rsa, _sanitized(ref, rp, ci))
    yd_ref, _, _ = oracle.fused_gemm(rqa, rsa, dict(ref, row_ptr=np.zeros_like(rp), col_idx=ci[:0],
                                                    qr=ref["qr"][:0], sr=ref["sr"][:0]))
    bound = 1e-3 * np.maximum(np.abs(y_ref), np.sqrt(np.mean(y_ref ** 2))) + 2.0 ** -12 * np.abs(yd_ref)
    # the standalone residual kernel adds every entry, like the streaming kernel
    assert np.all(np.abs(host(yu).astype(np.float64) - y_ref) <= bound)
    if M <= 32 or not merge:
        assert_y_close(y, y_ref)
