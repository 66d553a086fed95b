"""GPU parity of the one-call layer mq_fused_layer (fp16 activations in,
y out).  For decode-sized M it is one kernel that quantises the token tile in
its prologue; it must give the same y bits as mq_quantize_act followed by
mq_fused_gemm (which the other parity tests pin to the oracle), and y within
the tolerance of the oracle's layer.  Larger M and shapes whose token tile
does not fit the prologue take the two-kernel route through the workspace,
with the same bits."""
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


def _gpu_layer(spec, seed):
    w = syn.make_weight(spec, seed)
    xc = syn.make_calib(spec, seed)
    sel, _, _ = ops.select_blocks(dev(w), dev(xc), spec.block, spec.n_select)
    return w, xc, ops.pack_weights(dev(w), spec.block, sel)


def _bits(t):
    return host(t).view(np.uint16)


CASES = [
    # M, N, K, b, rho, fused-in-one-kernel expected
    (1, 512, 512, 64, 0.10, True),
    (2, 256, 1024, 32, 0.25, True),
    (3, 384, 256, 128, 0.50, True),
    (4, 512, 2048, 64, 0.10, True),
    (4, 128, 128, 64, 1.00, True),
    (1, 64, 4096, 32, 0.05, True),
    (2, 256, 14336, 64, 0.10, True),
    (4, 256, 14336, 64, 0.10, False),
    (1, 512, 512, 64, 0.0, True),
    (5, 512, 512, 64, 0.10, False),
    (16, 256, 1024, 32, 0.10, False),
    (40, 384, 256, 128, 0.20, False),
    # the two-kernel decode route reads its codes in 16-token tiles: a second,
    # mostly padding tile, and a ragged one with 32-wide blocks
    (17, 256, 1024, 64, 0.10, False),
    (31, 128, 640, 32, 0.20, False),
]


@pytest.mark.parametrize("M,N,K,b,rho,one_kernel", CASES)
def test_fused_layer_matches_two_kernels_and_oracle(M, N, K, b, rho, one_kernel):
    print(f"case M={M} N={N} K={K} b={b} rho={rho}", flush=True)
    spec = syn.LayerSpec("f", K=K, N=N, w_outlier_frac=0.01, x_outlier_count=3, T=32, block=b, rho=rho)
    w, xc, layer = _gpu_layer(spec, seed=M + K)
    x = syn.make_acts(spec, M, seed=N)
    assert (ops.fused_layer_workspace(M, N, K) == 0) == one_kernel
    xt = dev(x)
    y = ops.fused_layer(xt, layer)
    qa, sa = ops.quantize_act(xt)
    y2 = ops.fused_gemm(qa, sa, layer)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), _bits(y2))
    # every case against the oracle's layer (the largest, N = 256 x K = 14336,
    # takes the oracle about a second)
    ref = oracle.layer_reference(x, w, xc, b, spec.n_select)
    assert_y_close(y, ref["y"])


FP6_CASES = [
    # M, N, K, b, rho: the prefill kernel (the layer takes the fp6 route from
    # M = 1024 when b is 64 or 128): ragged token and channel tiles, split-K,
    # a second token band
    (300, 256, 2048, 64, 0.10),
    (1100, 640, 768, 64, 0.15),
    (1024, 128, 4096, 128, 0.20),
    (1300, 256, 1536, 64, 0.10),
]


@pytest.mark.parametrize("M,N,K,b,rho", FP6_CASES)
def test_fused_layer_fp6_route_matches_int8_route_and_oracle(M, N, K, b, rho):
    # The fp6 route (act-quant into FP6 images, weight and residual
    # conversion, fp6 tile kernel) gives the int8 route's y bit for bit: the
    # two form the same products sa*sw*dot, scaled by powers of two.
    print(f"case M={M} N={N} K={K} b={b} rho={rho}", flush=True)
    spec = syn.LayerSpec("f6", K=K, N=N, w_outlier_frac=0.01, x_outlier_count=3, T=32, block=b, rho=rho)
    w, xc, layer = _gpu_layer(spec, seed=M + N)
    x = syn.make_acts(spec, M, seed=K)
    xt = dev(x)
    y = ops.fused_layer(xt, layer)
    qa, sa = ops.quantize_act(xt)
    y6 = ops.fused_gemm(qa, sa, layer, route="fp6")
    y8 = ops.fused_gemm(qa, sa, layer, route="int8")
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), _bits(y8))
    assert np.array_equal(_bits(y6), _bits(y8))
    ref = oracle.layer_reference(x, w, xc, b, spec.n_select)
    assert_y_close(y, ref["y"])


def test_fused_layer_special_values_and_padded_rows():
    # all-zero groups, an infinite value (its group's codes are 0 and y is NaN
    # on that row on both routes), subnormals, fp16 extremes, exact .5 ties
    # of v/s, and a leading dimension larger than K
    K, N, b = 512, 256, 64
    spec = syn.LayerSpec("s", K=K, N=N, T=32, block=b, rho=0.2)
    w, xc, layer = _gpu_layer(spec, seed=3)
    rng = np.random.default_rng(5)
    x = np.zeros((4, K), np.float16)
    x[0, 300] = np.inf                                   # group 2 of row 0: scale +inf, codes 0
    x[1, :] = (rng.standard_normal(K) * 1e-6).astype(np.float16)
    x[2, :] = np.float16(65504.0) * np.sign(rng.standard_normal(K)).astype(np.float16)
    x[3, :128] = np.arange(128) * 0.5 - 32
    x[3, 128:256] = 7.0 * (np.arange(128) % 3 - 1)
    x[3, 256:] = np.linspace(-3.5, 3.5, 256)
    big = np.zeros((4, K + 24), np.float16)
    big[:, :K] = x
    for M in (1, 2, 4):
        xt = dev(big)[:M, :K]
        assert xt.stride(0) == K + 24
        y = ops.fused_layer(xt, layer)
        qa, sa = ops.quantize_act(xt)
        y2 = ops.fused_gemm(qa, sa, layer)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y), _bits(y2)), f"M={M}"
        rqa, rsa = oracle.quantize_act(x[:M])
        assert np.array_equal(host(qa), oracle.pack_nibbles(rqa))
        assert np.array_equal(host(sa).view(np.uint32), rsa.view(np.uint32))


@pytest.mark.parametrize("K,N,Ms", [(k, n, syn.LLAMA3_8B_DECODE_M) for k, n in syn.LLAMA3_8B_SHAPES] +
                         [(k, n, [1, 16, 24]) for k, n in syn.QWEN3_32B_SHAPES])
def test_fused_layer_full_size_decode(K, N, Ms):
    # the launch configurations the benchmark times (M = 1 and 4 in one
    # kernel, M = 16 through the workspace with the codes in 16-token tiles;
    # M = 24 adds a ragged second tile)
    spec = syn.llama3_8b(K, N) if (K, N) in syn.LLAMA3_8B_SHAPES else syn.qwen3_32b(K, N)
    w, xc, layer = _gpu_layer(spec, seed=0)
    for M in Ms:
        print(f"K={K} N={N} M={M}", flush=True)
        xt = dev(syn.make_acts(spec, M))
        y = ops.fused_layer(xt, layer)
        qa, sa = ops.quantize_act(xt)
        y2 = ops.fused_gemm(qa, sa, layer)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y), _bits(y2))


def test_fused_layer_graph_replay():
    spec = syn.llama3_8b(4096, 4096)
    w, xc, layer = _gpu_layer(spec, seed=0)
    x = dev(syn.make_acts(spec, 4))
    y = torch.empty((4, 4096), dtype=torch.float16, device="cuda")
    ops.fused_layer(x, layer, out=y)
    torch.cuda.synchronize()
    ref = _bits(y).copy()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        ops.fused_layer(x, layer, out=y)
    for i in range(3):
        y.zero_()
        junk = ops.fused_layer(x[:1], layer)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y), ref), f"replay {i} differs"
        del junk


def test_explicit_stream_allocations():
    # outputs and workspaces the binding allocates for a call on a stream that
    # is not the current one belong to that stream; the result equals the
    # same call on the current stream
    spec = syn.llama3_8b(4096, 4096)
    w, xc, layer = _gpu_layer(spec, seed=0)
    x = dev(syn.make_acts(spec, 16))
    ref = ops.fused_layer(x, layer)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    y = ops.fused_layer(x, layer, stream=s)
    qa, sa = ops.quantize_act(x, stream=s)
    y2 = ops.fused_gemm(qa, sa, layer, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), _bits(ref))
    assert np.array_equal(_bits(y2), _bits(ref))
