"""Shared helpers for the GPU parity tests (HIP path vs the CPU oracle)."""
import numpy as np
import torch

import oracle

# y tolerance: |y_gpu - y_ref| <= YTOL * max(|y_ref|, rms(y_ref)) per element.
# fp16 output rounding alone contributes up to 2^-11 ~ 4.9e-4 of |y|; the fp32
# scale products and the fp32 sum over groups add a few 2^-24 relative terms
# per group, far below that.
YTOL = 1e-3


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def f16_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def assert_y_close(y_gpu: torch.Tensor, y_ref: np.ndarray, tol: float = YTOL):
    yg = host(y_gpu).astype(np.float64)
    yr = np.asarray(y_ref, np.float64)
    assert yg.shape == yr.shape
    assert np.all(np.isfinite(yg))
    rms = float(np.sqrt(np.mean(yr * yr))) if yr.size else 0.0
    bound = tol * np.maximum(np.abs(yr), rms)
    err = np.abs(yg - yr)
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if yr.size else 0.0
    assert np.all(err <= bound), f"y mismatch: worst err/bound = {worst:.3f}"
    return worst


def oracle_packed_from_gpu_layout(layer) -> dict:
    """Convert a PackedLayer's device tensors into the oracle's dict layout
    (host copies only; used to compare, never to produce expected values)."""
    return dict(qw=host(layer.qw), sw=host(layer.sw), row_ptr=host(layer.row_ptr),
                col_idx=host(layer.col_idx), qr=host(layer.qr), sr=host(layer.sr),
                block=layer.block, N=layer.N, K=layer.K)


def assert_packed_equal(layer, ref: dict):
    g = oracle_packed_from_gpu_layout(layer)
    assert np.array_equal(g["qw"], ref["qw"]), "qw bytes differ"
    assert np.array_equal(f16_bits(g["sw"]), f16_bits(ref["sw"])), "sw differs"
    assert np.array_equal(g["row_ptr"], ref["row_ptr"]), "row_ptr differs"
    assert np.array_equal(g["col_idx"], ref["col_idx"]), "col_idx differs"
    assert np.array_equal(g["qr"], ref["qr"]), "qr bytes differ"
    assert np.array_equal(f16_bits(g["sr"]), f16_bits(ref["sr"])), "sr differs"


def tile_rows_reference(qa_codes, sa, ref_packed: dict, tiles):
    """Oracle output for whole block-row tiles `tiles` (sub-layer of the packed
    dict; the oracle's own functions do all arithmetic)."""
    b = ref_packed["block"]
    K = ref_packed["K"]
    outs = {}
    for nt in tiles:
        r0, r1 = int(ref_packed["row_ptr"][nt]), int(ref_packed["row_ptr"][nt + 1])
        sub = dict(qw=ref_packed["qw"][nt * b // 16:(nt + 1) * b // 16], sw=ref_packed["sw"][nt * b:(nt + 1) * b],
                   row_ptr=np.array([0, r1 - r0], np.int32), col_idx=ref_packed["col_idx"][r0:r1],
                   qr=ref_packed["qr"][r0:r1], sr=ref_packed["sr"][r0:r1], block=b, N=b, K=K)
        y, _, _ = oracle.fused_gemm(qa_codes, sa, sub)
        outs[nt] = y
    return outs
