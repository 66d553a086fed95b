"""GPU parity at the largest configured shapes (Qwen3-32B MLP, Llama-3-70B
FFN), in the launch configuration the benchmark times (mq_fused_layer), on
outputs the oracle computes one block row at a time.

Everything the method computes per block row is local to that row (base
codes and scales, base error, residual candidates, Delta given H), so the
oracle recomputes sampled block rows of the full layer on its own and they
must match the GPU bit for bit; H is checked in full.  The top-K selection
is global: the GPU's selected set must be exactly what the oracle's
selection rule (largest Delta, lower id on ties) gives on the GPU's Delta
array, whose sampled rows were just pinned.  y is checked on the sampled
block rows against the oracle's fused GEMM of those rows.
"""
import numpy as np
import pytest
import torch

import oracle
from dense_sparse_w4a4_amd import ops
from dense_sparse_w4a4_amd import synthetic as syn
from parity_util import assert_y_close, dev, f16_bits, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()
    yield
    torch.cuda.synchronize()


def _check(spec, Ms):
    b = spec.block
    K, N = spec.K, spec.N
    w = syn.make_weight(spec)
    xc = syn.make_calib(spec)
    wt = dev(w)
    sel, delta, H = ops.select_blocks(wt, dev(xc), b, spec.n_select)
    layer = ops.pack_weights(wt, b, sel)
    torch.cuda.synchronize()
    gH, gd, gsel = host(H), host(delta), host(sel)
    assert np.array_equal(gH.view(np.uint64), oracle.hdiag(xc).view(np.uint64))
    assert np.array_equal(gsel, oracle.select_top(gd, spec.n_select))
    rp = host(layer.row_ptr)
    NT, KT = N // b, K // b
    rows = sorted({0, NT - 1, NT // 2, int(np.argmax(np.diff(rp)))})
    ys, refs = {}, {}
    for M in Ms:
        print(f"{spec.name} M={M}", flush=True)
        x = syn.make_acts(spec, M)
        ys[M] = host(ops.fused_layer(dev(x), layer))
        refs[M] = oracle.quantize_act(x)
    qws, sws, ci, qr, sr = host(layer.qw), host(layer.sw), host(layer.col_idx), host(layer.qr), host(layer.sr)
    for nt in rows:
        wr = w[nt * b:(nt + 1) * b]
        qw_r, sw_r = oracle.quantize_base(wr)
        E = oracle.base_error(wr, qw_r, sw_r)
        _, _, rhat = oracle.residual_all_blocks(E, b)
        d_r = oracle.delta_scores(E, rhat, gH, b)
        assert np.array_equal(gd[nt * KT:(nt + 1) * KT].view(np.uint64), d_r.view(np.uint64)), f"Delta row {nt}"
        e0, e1 = int(rp[nt]), int(rp[nt + 1])
        sub_sel = gsel[e0:e1] - nt * KT
        ref = oracle.pack_weights(wr, b, sub_sel)
        assert np.array_equal(qws[nt * b // 16:(nt + 1) * b // 16], ref["qw"]), f"qw row {nt}"
        assert np.array_equal(f16_bits(sws[nt * b:(nt + 1) * b]), f16_bits(ref["sw"]))
        assert np.array_equal(ci[e0:e1], ref["col_idx"])
        assert np.array_equal(qr[e0:e1], ref["qr"])
        assert np.array_equal(f16_bits(sr[e0:e1]), f16_bits(ref["sr"]))
        for M in Ms:
            y_ref, _, _ = oracle.fused_gemm(*refs[M], ref)
            assert_y_close(torch.from_numpy(ys[M][:, nt * b:(nt + 1) * b]), y_ref)


@pytest.mark.parametrize("K,N", syn.QWEN3_32B_SHAPES)
def test_full_size_qwen3_32b(K, N):
    # every M of the Qwen3-32B sweep; at M = 256, K = 25600 the tile kernel
    # splits the 200 groups over 6 workgroups (33 or 34 groups each)
    _check(syn.qwen3_32b(K, N), syn.QWEN3_32B_M)


@pytest.mark.parametrize("K,N", syn.LLAMA3_8B_SHAPES)
def test_full_size_llama3_8b_decode(K, N):
    # the decode launches the benchmark's secondary workload times (M = 1
    # and 4 as one kernel quantising in its prologue where the shape allows,
    # M = 16 through act-quant + fused GEMM)
    _check(syn.llama3_8b(K, N), syn.LLAMA3_8B_DECODE_M)


@pytest.mark.parametrize("b,rho", [(32, 0.20), (64, 0.10), (128, 0.05)])
def test_full_size_llama3_70b_ffn(b, rho):
    # every block size of the Llama-3-70B grid, at a budget from its range
    _check(syn.llama3_70b(b, rho), [syn.LLAMA3_70B_M])
