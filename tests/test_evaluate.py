"""The measurement helper's distortion equals the oracle's on tiny layers.

Both read the same packed layer (the oracle's), so this pins the helper's
unpacking and CSR placement; the oracle itself is pinned in test_oracle_*.
"""
import numpy as np
import pytest
import torch

import oracle
from dense_sparse_w4a4_amd import evaluate
from dense_sparse_w4a4_amd import synthetic as syn
from dense_sparse_w4a4_amd.ops import PackedLayer


def _layer(packed, N, K, b):
    t = torch.from_numpy
    return PackedLayer(N, K, b, t(packed["qw"]), t(packed["sw"].view(np.float16)),
                       t(packed["row_ptr"]), t(packed["col_idx"]), t(packed["qr"]),
                       t(packed["sr"].view(np.float16)))


@pytest.mark.parametrize("b,rho", [(32, 0.1), (64, 0.0), (64, 0.2), (128, 1.0)])
def test_distortion_matches_oracle(b, rho):
    spec = syn.TINY.with_block(b, rho)
    w = syn.make_weight(spec)
    xc = syn.make_calib(spec)
    sel, _, _ = oracle.select_blocks(w, xc, b, spec.n_select)
    packed = oracle.pack_weights(w, b, sel)
    qw, sw = oracle.quantize_base(w)
    E = oracle.base_error(w, qw, sw)
    _, _, rhat = oracle.residual_all_blocks(E, b)
    ref = oracle.distortion(xc, w, qw, sw, rhat, sel, b)
    got = evaluate.distortion(torch.from_numpy(xc), torch.from_numpy(w), _layer(packed, *w.shape, b))
    assert got == pytest.approx(ref, rel=1e-12)
    base_only = evaluate.distortion(torch.from_numpy(xc), torch.from_numpy(w),
                                    _layer(packed, *w.shape, b), with_residual=False)
    assert base_only == pytest.approx(oracle.distortion(xc, w, qw, sw, rhat, [], b), rel=1e-12)
    assert got <= base_only * (1 + 1e-12)
