"""GPU test of mq_fused_layer_noalloc, the entry point for callers that
cannot allocate: through the C ABI it must give the same y bits as
mq_fused_layer with a caller workspace, on consecutive calls that reuse the
device scratch (the second call smaller than the first), on every route the
layer takes (act-quant + split-K tile kernel, act-quant + streaming kernel,
one kernel with no scratch at all)."""
import numpy as np
import pytest
import torch

import oracle
from dense_sparse_w4a4_amd import ops
from dense_sparse_w4a4_amd import synthetic as syn
from parity_util import assert_y_close, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()
    yield
    torch.cuda.synchronize()


def _layer(M, N, K, b, rho, seed):
    spec = syn.LayerSpec("n", K=K, N=N, w_outlier_frac=0.01, x_outlier_count=3, T=32, block=b, rho=rho)
    w, xc = syn.make_weight(spec, seed), syn.make_calib(spec, seed)
    sel, _, _ = ops.select_blocks(dev(w), dev(xc), b, spec.n_select)
    return spec, w, xc, ops.pack_weights(dev(w), b, sel), syn.make_acts(spec, M, seed=seed + 1)


def _bits(t):
    return host(t).view(np.uint16)


# (M, N, K, b, rho): consecutive calls, each smaller than the one before
SEQUENCES = [
    # act-quant + split-K tile kernel (codes, scales and partials in the
    # scratch), then a smaller uneven split-K call
    [(300, 256, 2048, 64, 0.10), (40, 128, 3200, 64, 0.10)],
    # act-quant + streaming kernel, then one kernel with no scratch, then
    # act-quant + streaming kernel again on fewer tokens
    [(16, 512, 4096, 32, 0.10), (2, 512, 1024, 64, 0.10), (5, 256, 512, 128, 0.20)],
]


@pytest.mark.parametrize("seq", SEQUENCES)
def test_noalloc_matches_fused_layer(seq):
    for i, (M, N, K, b, rho) in enumerate(seq):
        print(f"call {i}: M={M} N={N} K={K} b={b} rho={rho}", flush=True)
        spec, w, xc, layer, x = _layer(M, N, K, b, rho, seed=M + N)
        xt = dev(x)
        y_ref = ops.fused_layer(xt, layer)
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        ops.fused_layer_noalloc(xt, layer, y)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y), _bits(y_ref)), f"call {i} differs from mq_fused_layer"
        ref = oracle.layer_reference(x, w, xc, b, spec.n_select)
        assert_y_close(y, ref["y"])


def test_noalloc_refuses_shapes_beyond_the_scratch():
    # M x K whose codes alone pass 128 MiB: refused before anything is enqueued
    K, N, M = 25600, 128, 8192
    assert ops.fused_layer_workspace(M, N, K) > ops.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    layer = ops.PackedLayer(N, K, 64, torch.zeros((N // 16, K // 128, 64, 16), dtype=torch.uint8, device="cuda"),
                            torch.zeros((N, K // 128), dtype=torch.float16, device="cuda"),
                            torch.zeros(N // 64 + 1, dtype=torch.int32, device="cuda"),
                            torch.zeros(0, dtype=torch.int32, device="cuda"),
                            torch.zeros((0, 64, 32), dtype=torch.uint8, device="cuda"),
                            torch.zeros((0, 64), dtype=torch.float16, device="cuda"))
    y = torch.zeros((M, N), dtype=torch.float16, device="cuda")
    with pytest.raises(ops.MosaicQError, match="MQ_ERR_WORKSPACE"):
        ops.fused_layer_noalloc(x, layer, y)
    torch.cuda.synchronize()
    assert not torch.any(y)
