"""Pins for the oracle's Hessian diagonal, Delta-score and top-K selection (CPU only).

The strongest pin is a special case with a closed form: when the calibration
tokens have exactly orthogonal columns (a Sylvester-Hadamard matrix with one
scale per column), X^T X is diagonal, the diagonal Hessian is exact, and the
Delta-score of a block must equal the exact reduction of output distortion
that block's residual buys.  Brute force over every subset then shows the
top-K set is the best K-subset.
"""
import itertools

import numpy as np
import pytest

import oracle
from dense_sparse_w4a4_amd import synthetic as syn


def hadamard(n):
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def orthogonal_calib(T, K, seed):
    rng = np.random.default_rng(seed)
    d = rng.choice([0.5, 1.0, 1.5, 2.0, 3.0, 4.0], size=K)
    xc = (hadamard(T)[:, :K] * d[None, :]).astype(np.float16)
    assert np.array_equal(xc.astype(np.float64), hadamard(T)[:, :K] * d[None, :])
    return xc, d


def outlier_weight(N, K, seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K)) * 0.02
    w[:, rng.choice(K, 3, replace=False)] *= 20
    return w.astype(np.float16)


def test_hdiag_closed_form_on_hadamard_calibration():
    xc, d = orthogonal_calib(256, 256, 0)
    H = oracle.hdiag(xc)
    assert np.array_equal(H, 256.0 * d * d)


def test_hdiag_sums_in_token_order():
    # 1 + 2^-53 + 2^-53 ... : left-to-right accumulation in fp64 loses each
    # tiny term, a pairwise or reordered sum would not
    xc = np.zeros((5, 128), np.float16)
    xc[0, 0] = 1.0
    xc[1:, 0] = np.float16(2.0 ** -12)   # square 2^-24 per token
    H = oracle.hdiag(xc)
    assert H[0] == 1.0 + 4 * 2.0 ** -24
    xc[:, 1] = np.float16(3.0)
    assert oracle.hdiag(xc)[1] == 45.0


@pytest.mark.parametrize("b", [32, 64, 128])
def test_delta_equals_exact_distortion_reduction_with_orthogonal_calibration(b):
    N, K, T = 256, 256, 256
    w = outlier_weight(N, K, 10 + b)
    xc, _ = orthogonal_calib(T, K, 20 + b)
    qw, sw = oracle.quantize_base(w)
    E = oracle.base_error(w, qw, sw)
    _, _, rhat = oracle.residual_all_blocks(E, b)
    H = oracle.hdiag(xc)
    delta = oracle.delta_scores(E, rhat, H, b)
    B = (N // b) * (K // b)
    assert delta.shape == (B,) and np.all(delta >= 0)
    d0 = oracle.distortion(xc, w, qw, sw, rhat, [], b)
    rng = np.random.default_rng(b)
    for bid in rng.choice(B, size=min(B, 12), replace=False):
        red = d0 - oracle.distortion(xc, w, qw, sw, rhat, [bid], b)
        assert red == pytest.approx(delta[bid], rel=1e-6, abs=1e-9 * d0)


def test_proxy_is_additive_in_delta():
    spec = syn.TINY
    w = syn.make_weight(spec)
    xc = syn.make_calib(spec)
    b = spec.block
    qw, sw = oracle.quantize_base(w)
    E = oracle.base_error(w, qw, sw)
    _, _, rhat = oracle.residual_all_blocks(E, b)
    H = oracle.hdiag(xc)
    delta = oracle.delta_scores(E, rhat, H, b)
    p0 = oracle.proxy_distortion(H, E, rhat, [], b)
    for S in ([0], [5, 17, 40], list(range(0, 64, 3))):
        pS = oracle.proxy_distortion(H, E, rhat, S, b)
        assert pS == pytest.approx(p0 - delta[S].sum(), rel=1e-10)


def test_top_k_is_best_subset_by_brute_force():
    # 4 x 4 blocks of 32 (K = N = 128): every 4-subset of the 16 blocks
    b, N, K, k = 32, 128, 128, 4
    w = outlier_weight(N, K, 5)
    xc, _ = orthogonal_calib(128, K, 6)
    sel, delta, H = oracle.select_blocks(w, xc, b, k)
    qw, sw = oracle.quantize_base(w)
    E = oracle.base_error(w, qw, sw)
    _, _, rhat = oracle.residual_all_blocks(E, b)
    best = min(oracle.distortion(xc, w, qw, sw, rhat, list(S), b)
               for S in itertools.combinations(range(16), k))
    got = oracle.distortion(xc, w, qw, sw, rhat, list(sel), b)
    assert got == pytest.approx(best, rel=1e-9)
    assert list(sel) == sorted(sel)


def test_ties_break_to_lower_id_and_selection_is_nested():
    d = np.array([3.0, 1.0, 3.0, 2.0, 3.0, 0.0, 2.0, 0.0])
    assert oracle.select_top(d, 2).tolist() == [0, 2]
    assert oracle.select_top(d, 4).tolist() == [0, 2, 3, 4]
    assert oracle.select_top(d, 5).tolist() == [0, 2, 3, 4, 6]
    assert oracle.select_top(d, 7).tolist() == [0, 1, 2, 3, 4, 5, 6]
    assert oracle.select_top(d, 0).tolist() == []
    assert oracle.select_top(d, 8).tolist() == list(range(8))
    rng = np.random.default_rng(0)
    d = rng.integers(0, 5, size=300).astype(np.float64)
    prev = set()
    for n in range(0, 301, 7):
        cur = set(oracle.select_top(d, n).tolist())
        assert prev <= cur and len(cur) == n
        prev = cur


def test_zero_error_layer_gives_zero_scores_and_lowest_ids():
    # integer weights in [-7, 7] with a 7 in every group are represented
    # exactly by the base: E = 0, every Delta is 0 and ties pick ids 0..n-1
    rng = np.random.default_rng(1)
    w = rng.integers(-7, 8, size=(128, 256)).astype(np.float16)
    w[:, ::128] = 7
    xc = rng.standard_normal((16, 256)).astype(np.float16)
    sel, delta, _ = oracle.select_blocks(w, xc, 64, 3)
    assert not np.any(delta)
    assert sel.tolist() == [0, 1, 2]


def test_distortion_falls_with_budget_on_tiny_layer():
    spec = syn.TINY
    w = syn.make_weight(spec)
    xc = syn.make_calib(spec)
    xe = syn.make_acts(spec, 256, seed=7)
    b = spec.block
    qw, sw = oracle.quantize_base(w)
    E = oracle.base_error(w, qw, sw)
    _, _, rhat = oracle.residual_all_blocks(E, b)
    H = oracle.hdiag(xc)
    delta = oracle.delta_scores(E, rhat, H, b)
    B = delta.size
    prev_d, prev_p = np.inf, np.inf
    rec = {}
    for rho in (0.0, 0.05, 0.10, 0.20, 0.50, 1.0):
        S = oracle.select_top(delta, int(np.floor(rho * B + 1e-9)))
        dS = oracle.distortion(xc, w, qw, sw, rhat, S, b)
        pS = oracle.proxy_distortion(H, E, rhat, S, b)
        assert pS <= prev_p          # provable: nested sets, Delta >= 0
        assert dS <= prev_d          # exact distortion: empirical on this layer
        prev_d, prev_p = dS, pS
        rec[rho] = dS
    # held-out tokens as well
    S10 = oracle.select_top(delta, int(0.1 * B))
    assert (oracle.distortion(xe, w, qw, sw, rhat, S10, b)
            < oracle.distortion(xe, w, qw, sw, rhat, [], b))
    frac = 1 - rec[0.10] / rec[0.0]
    print(f"tiny layer: distortion recovered at 10% of blocks = {frac:.3f}")
    assert frac > 0
