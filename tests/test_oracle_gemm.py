"""Pins for the oracle's fused layer output (CPU only).

  * scale-1 integer layer: every scale is exactly 1 and Y = X W^T exactly;
  * residual budget 0 equals plain W4A4 (a dequantised matmul, another route);
  * residual on every block equals deq(Qa X) (deq Q + R_hat)^T;
  * integer accumulators against a brute-force int64 triple loop;
  * packing round trip and CSR structure.
"""
import numpy as np
import pytest

import oracle
from dense_sparse_w4a4_amd import synthetic as syn


def _deq_act(qa, sa):
    return np.repeat(sa.astype(np.float64), 128, axis=1) * qa.astype(np.float64)


def _layer(spec, M, seed=0):
    return syn.make_acts(spec, M, seed), syn.make_weight(spec, seed), syn.make_calib(spec, seed)


def test_scale_one_integer_layer_is_exact():
    rng = np.random.default_rng(0)
    M, N, K, b = 9, 128, 384, 64
    x = rng.integers(-7, 8, size=(M, K))
    w = rng.integers(-7, 8, size=(N, K))
    for j in range(K // 128):
        x[:, j * 128 + rng.integers(128)] = 7 * rng.choice([-1, 1], size=M)
        w[:, j * 128 + rng.integers(128)] = 7 * rng.choice([-1, 1], size=N)
    xc = rng.standard_normal((32, K)).astype(np.float16)
    ref = oracle.layer_reference(x.astype(np.float16), w.astype(np.float16), xc, b, 5)
    assert np.all(ref["sa"] == 1.0) and np.all(ref["packed"]["sw"] == 1.0)
    assert np.array_equal(ref["qa"], x)
    assert np.array_equal(ref["y"], (x @ w.T).astype(np.float64))
    assert not np.any(ref["packed"]["qr"]) and not np.any(ref["packed"]["sr"])


def test_budget_zero_is_plain_w4a4():
    spec = syn.TINY
    x, w, _ = _layer(spec, 16)
    qa, sa = oracle.quantize_act(x)
    qw, sw = oracle.quantize_base(w)
    packed = oracle.pack_weights(w, spec.block, np.zeros(0, np.int64))
    y, _, res = oracle.fused_gemm(qa, sa, packed)
    assert res == []
    ref = _deq_act(qa, sa) @ oracle.dequant_weight(qw, sw).astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("b", [32, 64, 128])
def test_full_budget_equals_dense_base_plus_residual(b):
    spec = syn.TINY.with_block(b, 1.0)
    x, w, _ = _layer(spec, 16, seed=b)
    qa, sa = oracle.quantize_act(x)
    qw, sw = oracle.quantize_base(w)
    E = oracle.base_error(w, qw, sw)
    _, _, rhat = oracle.residual_all_blocks(E, b)
    B = spec.n_blocks
    packed = oracle.pack_weights(w, b, np.arange(B))
    y, _, res = oracle.fused_gemm(qa, sa, packed)
    assert len(res) == B
    wq = oracle.dequant_weight(qw, sw).astype(np.float64) + rhat.astype(np.float64)
    ref = _deq_act(qa, sa) @ wq.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # and the residual moves the output towards the unquantised weight
    exact = _deq_act(qa, sa) @ w.astype(np.float64).T
    base = _deq_act(qa, sa) @ oracle.dequant_weight(qw, sw).astype(np.float64).T
    assert np.linalg.norm(y - exact) < np.linalg.norm(base - exact)


def test_accumulators_against_brute_force_triple_loop():
    rng = np.random.default_rng(3)
    M, N, K, b = 3, 64, 256, 32
    x = (rng.standard_normal((M, K)) * 2).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    xc = rng.standard_normal((8, K)).astype(np.float16)
    ref = oracle.layer_reference(x, w, xc, b, 6)
    qa = [[int(v) for v in row] for row in ref["qa"]]
    slabs = ref["packed"]["qw"]

    def code(n, k):
        # the slab layout by its definition: channel n is row n%16 of slab
        # n//16; byte (k%128)//2 of its group segment sits in lane
        # 16*(byte//16) + n%16 at position byte%16; even k in the low nibble
        byte = (k % 128) // 2
        v = int(slabs[n // 16, k // 128, 16 * (byte // 16) + n % 16, byte % 16])
        v = (v >> 4) if k % 2 else (v & 15)
        return v - 16 if v >= 8 else v

    for m in range(M):
        for n in range(N):
            for j in range(K // 128):
                s = 0
                for k in range(j * 128, (j + 1) * 128):
                    s += qa[m][k] * code(n, k)
                assert ref["acc_base"][m, n, j] == s
    rp, ci = ref["packed"]["row_ptr"], ref["packed"]["col_idx"]
    i = 0
    for nt in range(N // b):
        for e in range(rp[nt], rp[nt + 1]):
            kt = int(ci[e])
            qr = oracle.unpack_nibbles(ref["packed"]["qr"][e]).tolist()
            for m in range(M):
                for r in range(b):
                    s = sum(qa[m][kt * b + c] * qr[r][c] for c in range(b))
                    assert ref["acc_res"][i][m, r] == s
            i += 1
    assert i == 6
    # and the fp64 output from the accumulators by a scalar loop
    sa, sw = ref["sa"], ref["packed"]["sw"]
    for (m, n) in [(0, 0), (2, 63), (1, 17)]:
        t = 0.0
        for j in range(K // 128):
            t += float(sa[m, j]) * float(sw[n, j]) * int(ref["acc_base"][m, n, j])
        i = 0
        for nt in range(N // b):
            for e in range(rp[nt], rp[nt + 1]):
                if nt == n // b:
                    kt = int(ci[e])
                    t += float(sa[m, kt * b // 128]) * float(ref["packed"]["sr"][e][n - nt * b]) * int(ref["acc_res"][i][m, n - nt * b])
                i += 1
        assert ref["y"][m, n] == pytest.approx(t, rel=1e-13, abs=1e-15)


def test_pack_round_trip_and_csr():
    spec = syn.TINY
    w = syn.make_weight(spec)
    sel = np.array([0, 3, 9, 10, 11, 40, 63])
    p = oracle.pack_weights(w, 64, sel)
    assert p["qw"].shape == (32, 4, 64, 16) and p["qw"].dtype == np.uint8
    assert p["sw"].shape == (512, 4) and p["sw"].dtype == np.float16
    assert p["row_ptr"].tolist() == [0, 2, 5, 5, 5, 5, 6, 6, 7]
    assert p["col_idx"].tolist() == [0, 3, 1, 2, 3, 0, 7]
    assert p["qr"].shape == (7, 64, 32) and p["sr"].shape == (7, 64)
    qw, blocks = oracle.unpack_packed(p)
    q0, _ = oracle.quantize_base(w)
    assert np.array_equal(qw, q0)
    E = oracle.base_error(w, *oracle.quantize_base(w))
    qr_all, sr_all, _ = oracle.residual_all_blocks(E, 64)
    for (nt, kt, qr, sr), bid in zip(blocks, sel):
        assert bid == nt * 8 + kt
        assert np.array_equal(qr, qr_all[nt * 64:(nt + 1) * 64, kt * 64:(kt + 1) * 64])
        assert np.array_equal(sr, sr_all[nt, kt])


def test_tiny_reference_selects_ten_percent():
    spec = syn.TINY
    x, w, xc = _layer(spec, 16)
    ref = oracle.layer_reference(x, w, xc, spec.block, spec.n_select)
    assert spec.n_select == 6
    assert len(ref["selected"]) == 6 and ref["y"].shape == (16, 512)
    assert np.all(np.isfinite(ref["y"]))


def test_slab_layout_by_definition_and_round_trip():
    N, Kh = 48, 192                      # 3 slabs, 3 groups
    rows = ((np.arange(N)[:, None] * 37 + np.arange(Kh)[None, :] * 11) % 251).astype(np.uint8)
    slabs = oracle.slab_layout(rows)
    assert slabs.shape == (3, 3, 64, 16)
    for s_ in range(3):
        for j in range(3):
            for lane in range(64):
                for t in range(16):
                    n = 16 * s_ + lane % 16
                    assert slabs[s_, j, lane, t] == rows[n, j * 64 + 16 * (lane // 16) + t]
    assert np.array_equal(oracle.row_layout(slabs), rows)
