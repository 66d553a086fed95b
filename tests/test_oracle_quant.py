"""Pins for the oracle's quantisers and packing (CPU only).

Each check comes from outside the oracle: an exhaustive comparison with an
independent rounding route, hand-derived fixtures, invariants that any
correct symmetric round-to-nearest quantiser satisfies, and round trips.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_quant.json")


def _all_finite_f16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    return v[np.isfinite(v)]


def _independent_code(v16, s32):
    """clamp(round-half-even(fl32(v/s))) by another route: the quotient in
    fp64 rounded once to fp32 (double rounding is innocuous for division from
    24 to 53 bits), then floor(x + 1/2) with an explicit tie correction."""
    x = (v16.astype(np.float64) / np.float64(s32)).astype(np.float32).astype(np.float64)
    f = np.floor(x + 0.5)
    tie = (f - x) == 0.5
    odd = np.mod(f, 2) != 0
    f = np.where(tie & odd, f - 1, f)
    return np.clip(f, -7, 7)


SCALES = [1.0, 0.5, 0.25, 2.0, 1.0 / 7.0, 0.1234567, 3.3, 1000.0, 0.0123,
          float(np.float16(2.0 ** -20)), 6.0e-8, 1.7e-5, 65504.0 / 7.0]


def test_quant4_exhaustive_fp16_against_independent_rounding():
    v = _all_finite_f16()
    assert v.size == 63488
    for s in SCALES:
        s32 = np.float32(s)
        q = oracle.quant4(v.astype(np.float32), s32)
        ref = _independent_code(v, s32)
        assert q.dtype == np.int8
        assert np.array_equal(q.astype(np.float64), ref), f"scale {s}"


def test_quant4_zero_scale_gives_zero():
    v = _all_finite_f16().astype(np.float32)
    assert not np.any(oracle.quant4(v, np.float32(0.0)))


def test_quant4_invariants():
    v = _all_finite_f16().astype(np.float32)
    for s in SCALES:
        s32 = np.float32(s)
        q = oracle.quant4(v, s32).astype(np.float64)
        assert np.all(np.abs(q) <= 7)
        # monotone non-decreasing in v
        order = np.argsort(v, kind="stable")
        assert np.all(np.diff(q[order]) >= 0)
        # unclipped values are within half a step
        inside = np.abs(v.astype(np.float64)) <= 7.0 * float(s32)
        err = np.abs(v.astype(np.float64) - float(s32) * q)
        assert np.all(err[inside] <= 0.5 * float(s32) * (1 + 2.0 ** -20))
        # odd symmetry
        assert np.array_equal(oracle.quant4(-v, s32).astype(np.float64), -q)


def test_ties_round_to_even():
    s = np.float32(0.5)
    v = np.array([0.25, 0.75, 1.25, 1.75, -0.25, -0.75, 3.25, 3.75], np.float32)
    assert oracle.quant4(v, s).tolist() == [0, 2, 2, 4, 0, -2, 6, 7]


def test_golden_hand_fixtures():
    g = json.load(open(GOLD))
    pk = g["nibble_packing"]
    assert oracle.pack_nibbles(np.array(pk["codes"], np.int8)).tolist() == pk["bytes"]
    assert oracle.unpack_nibbles(np.array(pk["bytes"], np.uint8)).tolist() == pk["codes"]
    for key in ("act_group_amax7", "act_group_amax14"):
        f = g[key]
        x = np.zeros((1, 128), np.float16)
        x[0, :len(f["values"])] = f["values"]
        qa, sa = oracle.quantize_act(x)
        assert float(sa[0, 0]) == f["scale"]
        assert qa[0, :len(f["codes"])].tolist() == f["codes"]
        assert not np.any(qa[0, len(f["codes"]):])
    f = g["weight_group_amax1"]
    w = np.zeros((1, 128), np.float16)
    w[0, :len(f["values"])] = f["values"]
    qw, sw = oracle.quantize_base(w)
    assert int(sw.view(np.uint16)[0, 0]) == f["scale_f16_bits"]
    assert float(sw[0, 0]) == f["scale"]
    assert qw[0, :4].tolist() == f["codes"]
    E = oracle.base_error(w, qw, sw)
    assert E[0, :4].tolist() == f["errors"]


def test_act_quant_scale_rule_and_max_maps_to_seven():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((37, 512)) * 3).astype(np.float16)
    qa, sa = oracle.quantize_act(x)
    assert qa.shape == (37, 512) and sa.shape == (37, 4) and sa.dtype == np.float32
    xg = x.astype(np.float32).reshape(37, 4, 128)
    amax = np.abs(xg).max(axis=2)
    # sa*7 reproduces amax to within one fp32 rounding of the division
    assert np.allclose(sa.astype(np.float64) * 7.0, amax, rtol=2 ** -23, atol=0)
    # the element of largest magnitude gets code +-7
    arg = np.abs(xg).argmax(axis=2)
    qg = qa.reshape(37, 4, 128)
    picked = np.take_along_axis(qg, arg[:, :, None], axis=2)[:, :, 0]
    assert np.all(np.abs(picked) == 7)


def test_act_quant_all_zero_group():
    x = np.zeros((3, 256), np.float16)
    x[1, 200] = 1.0
    qa, sa = oracle.quantize_act(x)
    assert sa[0, 0] == 0 and sa[0, 1] == 0 and sa[1, 0] == 0
    assert not np.any(qa[0]) and qa[1, 200] == 7 and np.count_nonzero(qa) == 1


def test_base_quant_invariants_and_subnormal_scales():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((64, 384)) * 0.02).astype(np.float16)
    w[3, :128] = (rng.standard_normal(128) * 1e-6).astype(np.float16)   # fp16 subnormals
    w[5, 128:256] = 0
    qw, sw = oracle.quantize_base(w)
    assert sw.dtype == np.float16 and sw.shape == (64, 3)
    assert np.all(np.abs(qw) <= 7)
    assert sw[5, 1] == 0 and not np.any(qw[5, 128:256])
    E = oracle.base_error(w, qw, sw)
    s = np.repeat(sw.astype(np.float64), 128, axis=1)
    normal = s >= 2.0 ** -14
    # normal-range scales: error within half a step
    assert np.all(np.abs(E.astype(np.float64))[normal] <= 0.5 * s[normal] * (1 + 1e-6) + 1e-12)
    # any scale: quantising never increases magnitude error beyond |w|
    assert np.all(np.abs(E.astype(np.float64)) <= np.abs(w.astype(np.float64)) + 1e-12)
    # the E arithmetic is exact up to the final fp32 rounding
    exact = w.astype(np.float64) - s * qw.astype(np.float64)
    assert np.all(np.abs(E.astype(np.float64) - exact) <= np.abs(exact) * 2.0 ** -24)


def test_residual_invariants():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((128, 256)) * 0.02).astype(np.float16)
    w[:, 7] *= 20
    qw, sw = oracle.quantize_base(w)
    E = oracle.base_error(w, qw, sw)
    for b in (32, 64, 128):
        qr, sr, rhat = oracle.residual_all_blocks(E, b)
        assert sr.shape == (128 // b, 256 // b, b)
        assert np.all(np.abs(qr) <= 7)
        e = E.astype(np.float64)
        d = e - rhat.astype(np.float64)
        assert np.all(d * d <= e * e)
        s = sr.transpose(0, 2, 1).astype(np.float64)          # [nt, r, kt]
        s = np.repeat(s.reshape(128, 256 // b), b, axis=1)     # [n, k]
        normal = s >= 2.0 ** -14
        assert np.all(np.abs(d)[normal] <= 0.5 * s[normal] * (1 + 1e-6))


@pytest.mark.parametrize("shape", [(1, 2), (3, 64), (5, 7, 16)])
def test_pack_roundtrip(shape):
    rng = np.random.default_rng(4)
    q = rng.integers(-7, 8, size=shape).astype(np.int8)
    p = oracle.pack_nibbles(q)
    assert p.shape == shape[:-1] + (shape[-1] // 2,)
    assert np.array_equal(oracle.unpack_nibbles(p), q)


def test_golden_residual_row():
    # one block row of the residual, derived by hand (see the fixture): the
    # base error, the fp16 row scale bits, the residual codes and bytes
    f = json.load(open(GOLD))["residual_row_b32"]
    b = f["block"]
    w = np.zeros((b, 128), np.float16)
    w[0, :len(f["values"])] = f["values"]
    qw, sw = oracle.quantize_base(w)
    n = len(f["values"])
    assert qw[0, :n].tolist() == f["base_codes"] and float(sw[0, 0]) == 1.0
    E = oracle.base_error(w, qw, sw)
    assert E[0, :n].tolist() == f["errors"]
    qr, sr, rhat = oracle.residual_all_blocks(E, b)
    assert int(sr.view(np.uint16)[0, 0, 0]) == f["sr_f16_bits"]
    assert float(sr[0, 0, 0]) == f["sr"]
    assert qr[0, :n].tolist() == f["codes"] and not np.any(qr[0, n:b])
    assert rhat[0, :n].tolist() == f["rhat"]
    packed = oracle.pack_weights(w, b, np.array([0]))
    assert packed["qr"][0, 0, :3].tolist() == f["qr_bytes"]
    assert not np.any(packed["qr"][0, 0, 3:]) and not np.any(packed["qr"][0, 1:])
    assert int(packed["sr"].view(np.uint16)[0, 0]) == f["sr_f16_bits"]


def test_infinite_group_rule():
    # a group whose largest magnitude is infinite: scale +inf and every code 0
    # (v/inf = 0 for finite v; inf/inf is not a number and gives 0 too)
    x = np.ones((2, 256), np.float16)
    x[0, 5] = np.inf
    x[1, 130] = -np.inf
    x[1, 131] = np.inf
    qa, sa = oracle.quantize_act(x)
    assert np.isposinf(sa[0, 0]) and np.isposinf(sa[1, 1])
    assert not np.any(qa[0, :128]) and not np.any(qa[1, 128:])
    assert np.all(qa[0, 128:] == 7) and np.all(qa[1, :128] == 7)
    assert oracle.quant4(np.array([np.inf, -np.inf, 3.0], np.float32), np.float32(np.inf)).tolist() == [0, 0, 0]
