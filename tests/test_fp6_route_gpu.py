"""The prefill kernel's fp6 route with prepared operands (mq_fp6_sizes,
mq_fp6_prepare_acts, mq_fp6_prepare_weights, mq_fused_gemm_fp6).

The images are checked byte for byte against a numpy construction written
here from the layout the header states (six-bit sign-magnitude fields, value
q/8, at bit 6i of a lane's six dwords), and the GEMM on prepared images
against the oracle's exact accumulators and y, and bit for bit against
mq_fused_gemm's int8 route on the same codes."""
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


def lane_dwords(codes32: np.ndarray) -> np.ndarray:
    """32 codes (int, [-8, 7]) -> the six dwords of one lane: field i =
    |q| | (q < 0) << 5 at bits 6i .. 6i+5 of the 192-bit value."""
    v = 0
    for i, q in enumerate(codes32):
        q = int(q)
        v |= ((abs(q) & 0x1F) | (0x20 if q < 0 else 0)) << (6 * i)
    return np.array([(v >> (32 * d)) & 0xFFFFFFFF for d in range(6)], dtype=np.uint32)


def image_of_rows(q: np.ndarray) -> np.ndarray:
    """int codes [R, K] -> the image bytes [ceil(R/32)][K/128][3072]."""
    R, K = q.shape
    nb, G = -(-R // 32), K // 128
    img = np.zeros((nb, G, 3072), dtype=np.uint8)
    qp = np.zeros((nb * 32, K), dtype=np.int64)
    qp[:R] = q
    for rb in range(nb):
        for j in range(G):
            frag = img[rb, j].view(np.uint32)
            for u in range(2):
                for l in range(64):
                    r, h = l % 32, l // 32
                    k0 = j * 128 + 64 * u + 32 * h
                    d = lane_dwords(qp[rb * 32 + r, k0:k0 + 32])
                    frag[(u * 1024 + 16 * l) // 4:(u * 1024 + 16 * l) // 4 + 4] = d[:4]
                    frag[(2048 + u * 512 + 8 * l) // 4:(2048 + u * 512 + 8 * l) // 4 + 2] = d[4:]
    return img.reshape(-1)


def residual_image(qr_codes: np.ndarray, b: int) -> np.ndarray:
    """int codes [n_sel, b, b] -> the residual image (per block, per 32 rows
    c and slice u a 1536-byte piece at (c*(b/64) + u)*1536)."""
    out = np.zeros((len(qr_codes), b * b * 3 // 4), dtype=np.uint8)
    for e, blk in enumerate(qr_codes):
        for c in range(b // 32):
            for u in range(b // 64):
                piece = out[e, (c * (b // 64) + u) * 1536:(c * (b // 64) + u + 1) * 1536].view(np.uint32)
                for l in range(64):
                    r, h = l % 32, l // 32
                    d = lane_dwords(blk[32 * c + r, 64 * u + 32 * h:64 * u + 32 * h + 32])
                    piece[4 * l:4 * l + 4] = d[:4]
                    piece[256 + 2 * l:256 + 2 * l + 2] = d[4:]
    return out.reshape(-1)


def _codes_layer(rng, M, N, K, b, frac):
    qa = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    KT = K // b
    nsel = int((N // b) * KT * frac)
    sel = np.sort(rng.choice((N // b) * KT, size=nsel, replace=False)).astype(np.int32)
    row_ptr, col_idx = oracle.build_csr(sel, N, K, b)
    qr_codes = rng.integers(-8, 8, size=(nsel, b, b)).astype(np.int8)
    ref = dict(qw=oracle.slab_layout(oracle.pack_nibbles(qw)),
               sw=(rng.random((N, K // 128)) * 0.02 + 1e-3).astype(np.float16),
               row_ptr=row_ptr, col_idx=col_idx,
               qr=oracle.pack_nibbles(qr_codes) if nsel else np.zeros((0, b, b // 2), np.uint8),
               sr=(rng.random((nsel, b)) * 0.01 + 1e-4).astype(np.float16), block=b, N=N, K=K)
    sa = (rng.random((M, K // 128)) * 0.5 + 0.01).astype(np.float32)
    return qa, qw, qr_codes, ref, sa


@pytest.mark.parametrize("M,N,K,b", [(33, 64, 256, 64), (70, 128, 384, 128)])
def test_images_match_the_stated_layout(M, N, K, b):
    print(f"fp6 images M={M} N={N} K={K} b={b}", flush=True)
    rng = np.random.default_rng(M + b)
    qa, qw, qr_codes, ref, _ = _codes_layer(rng, M, N, K, b, 0.3)
    layer = ops.PackedLayer(N, K, b, dev(ref["qw"]), dev(ref["sw"]), dev(ref["row_ptr"]),
                            dev(ref["col_idx"]), dev(ref["qr"]), dev(ref["sr"]))
    ab, wb, _ = ops.fp6_sizes(M, N, K, b, len(qr_codes))
    aimg = ops.fp6_prepare_acts(dev(oracle.pack_nibbles(qa)), K)
    wimg = ops.fp6_prepare_weights(layer)
    torch.cuda.synchronize()
    assert ab == -(-M // 32) * (K // 128) * 3072
    assert np.array_equal(host(aimg)[:ab], image_of_rows(qa))
    base_b = N * K * 3 // 4
    rbase = -(-base_b // 256) * 256
    assert wb == rbase + len(qr_codes) * b * b * 3 // 4
    w = host(wimg)
    assert np.array_equal(w[:base_b], image_of_rows(qw))
    assert np.array_equal(w[rbase:wb], residual_image(qr_codes, b))


@pytest.mark.parametrize("M,N,K,b,frac", [(290, 256, 2048, 64, 0.3), (100, 384, 640, 128, 0.25),
                                          (1030, 256, 1024, 64, 0.1), (40, 128, 3200, 64, 0.1),
                                          (257, 192, 256, 64, 0.0)])
def test_gemm_on_prepared_images(M, N, K, b, frac):
    # full nibble range on every operand; split-K where the shape has it
    print(f"fp6 prepared gemm M={M} N={N} K={K} b={b}", flush=True)
    rng = np.random.default_rng(M * 3 + N)
    qa, _, _, ref, sa_h = _codes_layer(rng, M, N, K, b, frac)
    y_ref, acc_ref, res_ref = oracle.fused_gemm(qa, sa_h, ref)
    ns = len(ref["qr"])
    layer = ops.PackedLayer(N, K, b, dev(ref["qw"]), dev(ref["sw"]), dev(ref["row_ptr"]),
                            dev(ref["col_idx"]), dev(ref["qr"]), dev(ref["sr"]))
    qa_d, sa = dev(oracle.pack_nibbles(qa)), dev(sa_h)
    aimg = ops.fp6_prepare_acts(qa_d, K)
    wimg = ops.fp6_prepare_weights(layer)
    y6, base, res = ops.fused_gemm_fp6(aimg, sa, M, layer, wimg, dump=True)
    z6 = ops.fused_gemm_fp6(aimg, sa, M, layer, wimg)
    y8 = ops.fused_gemm(qa_d, sa, layer, route="int8")
    torch.cuda.synchronize()
    assert np.array_equal(host(base).astype(np.int64), acc_ref)
    if ns:
        assert np.array_equal(host(res).astype(np.int64), np.stack(res_ref))
    assert_y_close(y6, y_ref)
    assert np.array_equal(host(y6).view(np.uint16), host(y8).view(np.uint16))
    assert np.array_equal(host(z6).view(np.uint16), host(y8).view(np.uint16))


def test_split_tail_tiles():
    # 260 tiles of 256 x 128 (M = 1024, N = 8320, 16 groups): 256 tiles take
    # all of K in one round and the last four (channels 8192-8319 in the
    # banded order) are split two ways, their partials summed by the reduce
    M, N, K, b = 1024, 8320, 2048, 64
    print(f"fp6 split tail M={M} N={N} K={K} b={b}", flush=True)
    rng = np.random.default_rng(11)
    qa, _, _, ref, sa_h = _codes_layer(rng, M, N, K, b, 0.05)
    layer = ops.PackedLayer(N, K, b, dev(ref["qw"]), dev(ref["sw"]), dev(ref["row_ptr"]),
                            dev(ref["col_idx"]), dev(ref["qr"]), dev(ref["sr"]))
    _, _, pb = ops.fp6_sizes(M, N, K, b, len(ref["qr"]))
    assert pb == 2 * M * N * 4  # two K splits
    qa_d, sa = dev(oracle.pack_nibbles(qa)), dev(sa_h)
    y6 = ops.fused_gemm_fp6(ops.fp6_prepare_acts(qa_d, K), sa, M, layer, ops.fp6_prepare_weights(layer))
    yr = ops.fused_gemm(qa_d, sa, layer, route="fp6")
    y8 = ops.fused_gemm(qa_d, sa, layer, route="int8")  # one K split at 260 tiles
    torch.cuda.synchronize()
    h6, h8 = host(y6), host(y8)
    assert np.array_equal(host(yr).view(np.uint16), h6.view(np.uint16))
    # the tiles over all of K: one fp32 chain on both routes
    assert np.array_equal(h6[:, :8192].view(np.uint16), h8[:, :8192].view(np.uint16))
    # the split tiles: two chains summed, within one fp16 rounding of the int8 route
    assert_y_close(y6[:, 8192:], h8[:, 8192:].astype(np.float64), tol=2.0 ** -10)
    # rows of every token tile (and the last) against the oracle
    rows = np.r_[0:6, 250:262, 509:515, 700:704, 1018:1024]
    y_ref, _, _ = oracle.fused_gemm(qa[rows], sa_h[rows], ref)
    assert_y_close(y6[torch.from_numpy(rows).to(y6.device)], y_ref)


def test_full_size_qwen3_32b_prefill_prepared():
    # the configured Qwen3-32B MLP shapes at M = 4096 (the kernel the default
    # benchmark times): prepared route against the one-call layer and the
    # int8 route
    for K, N in syn.QWEN3_32B_SHAPES:
        M = 4096
        print(f"fp6 full size K={K} N={N} M={M}", flush=True)
        spec = syn.qwen3_32b(K, N)
        w = syn.make_weight(spec, 1)
        xc = syn.make_calib(spec, 1)
        sel, _, _ = ops.select_blocks(dev(w), dev(xc), spec.block, spec.n_select)
        layer = ops.pack_weights(dev(w), spec.block, sel)
        x = dev(syn.make_acts(spec, M, seed=2))
        qa, sa = ops.quantize_act(x)
        wimg = ops.fp6_prepare_weights(layer)
        aimg = ops.fp6_prepare_acts(qa, K)
        y6 = ops.fused_gemm_fp6(aimg, sa, M, layer, wimg)
        y8 = ops.fused_gemm(qa, sa, layer, route="int8")
        yl = ops.fused_layer(x, layer)
        torch.cuda.synchronize()
        # the layer and the prepared GEMM: the same route and K split
        assert np.array_equal(host(yl).view(np.uint16), host(y6).view(np.uint16))
        # the int8 route: bit for bit where both run one K split; 25600 x 5120
        # is split in two on the fp6 route only (a partial last round
        # otherwise), which changes the fp32 summation order, so y may move
        # by one fp16 rounding there (plus the fp32 order's own rounding,
        # ~1e-6 of the output's rms, where y nearly cancels)
        a6, a8 = host(y6).astype(np.float64), host(y8).astype(np.float64)
        if K == 25600:
            assert_y_close(y6, a8, tol=2.0 ** -10)
            assert np.mean(a6 == a8) > 0.9
        else:
            assert np.array_equal(host(y6).view(np.uint16), host(y8).view(np.uint16))
        del wimg, aimg, y6, y8, yl, layer
        torch.cuda.empty_cache()
