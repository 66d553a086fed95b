"""Step-by-step CPU reference of the MosaicQuant layer (test infrastructure only).

Notation: W is the (already outlier-migrated) weight, fp16 [N, K], rows are
output channels n, columns input channels k.  X is fp16 [M, K].  Xc is fp16
[T, K] calibration tokens.  G = K/128 groups.  b is the residual block edge,
blocks are b x b and tile-aligned; block id = nt*(K/b) + kt.

Conventions (readings of the pages, see the package docstring):
  f16(.)  round-to-nearest-even to binary16, subnormals kept
  rint    round half to even
  "/"     IEEE division in the stated precision (fp32 for scales and codes)
"""
from __future__ import annotations

import numpy as np

GROUP = 128
QMAX = 7

__all__ = [
    "GROUP", "QMAX", "quant4", "quantize_act", "quantize_base", "base_error",
    "residual_all_blocks", "hdiag", "delta_scores", "select_top", "select_blocks",
    "pack_nibbles", "unpack_nibbles", "slab_layout", "row_layout", "build_csr",
    "pack_weights", "unpack_packed",
    "gemm_accumulators", "gemm_output", "fused_gemm", "dequant_weight",
    "residual_dense", "distortion", "proxy_distortion", "layer_reference",
    "select_exact_greedy", "smooth_scales", "smooth_weights", "smooth_acts",
]


# ----------------------------------------------------------------------------
# 4-bit symmetric codes
# ----------------------------------------------------------------------------

def quant4(v: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Symmetric 4-bit code of v under scale s: clamp(rint(v/s), -7, 7); 0 if s == 0.

    [summary-pt] Metodologia 1: both the base and the residual are 4-bit.
    Reading: symmetric range [-7, 7], the quotient formed by an IEEE fp32
    division and rounded half-to-even.  A quotient that is not a number
    (inf/inf in a group whose largest magnitude is infinite) gives code 0,
    as the finite values of such a group do (v/inf = 0).
    """
    v32 = np.asarray(v, dtype=np.float32)
    s32 = np.asarray(s, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        r = np.rint(v32 / s32)
    q = np.clip(r, -QMAX, QMAX)
    q = np.where((s32 == 0) | np.isnan(q), np.float32(0), q)
    return q.astype(np.int8)


def _group_view(a: np.ndarray) -> np.ndarray:
    rows, K = a.shape
    assert K % GROUP == 0, "K must be a multiple of 128"
    return a.reshape(rows, K // GROUP, GROUP)


def quantize_act(x: np.ndarray):
    """Per-token, per-group-128 activation codes and fp32 scales.

    [summary-pt] Metodologia 3 lists quantisation as one of the four
    operations of the online pipeline; Resultados: W4A4.
    Reading: amax over the 128 values of token m in group j; sa = amax/7 in
    fp32 (kept fp32); qa = quant4(x, sa).
    Returns (qa int8 [M, K], sa float32 [M, G]).
    """
    x16 = np.asarray(x, dtype=np.float16)
    M, K = x16.shape
    xg = _group_view(x16.astype(np.float32))
    amax = np.abs(xg).max(axis=2) if M else np.zeros((0, K // GROUP), np.float32)
    sa = (amax / np.float32(QMAX)).astype(np.float32)
    qa = quant4(xg, sa[:, :, None]).reshape(M, K)
    return qa, sa


def quantize_base(w: np.ndarray):
    """Dense 4-bit base Q(W): symmetric INT4, one fp16 scale per (row, group of 128).

    [summary-pt] Metodologia 1 (dense 4-bit base capturing the inliers) and
    [abstract] (the full weight matrix is quantised into the dense base).
    Reading: sw = f16(amax/7) with the division in fp32; codes use the
    rounded scale.  Returns (qw int8 [N, K], sw float16 [N, G]).
    """
    w16 = np.asarray(w, dtype=np.float16)
    wg = _group_view(w16.astype(np.float32))
    amax = np.abs(wg).max(axis=2)
    sw = (amax / np.float32(QMAX)).astype(np.float32).astype(np.float16)
    qw = quant4(wg, sw.astype(np.float32)[:, :, None]).reshape(w16.shape)
    return qw, sw


def dequant_weight(qw: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """fp32 deq(Q(W)): every element sw[n, k//128] * qw[n, k] (exact in fp32)."""
    N, K = qw.shape
    s = np.repeat(sw.astype(np.float32), GROUP, axis=1)
    return s * qw.astype(np.float32)


def base_error(w: np.ndarray, qw: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """E = W - deq(Q(W)) in fp32 (the product is exact, one rounding in the difference).

    [summary-pt] Metodologia 1: the residual compensates the quantisation
    error of the base.
    """
    return (np.asarray(w, np.float16).astype(np.float32) - dequant_weight(qw, sw)).astype(np.float32)


def _block_view(a: np.ndarray, b: int) -> np.ndarray:
    """[N, K] -> [N/b, b, K/b, b] indexed [nt, r, kt, c]."""
    N, K = a.shape
    return a.reshape(N // b, b, K // b, b)


def residual_all_blocks(E: np.ndarray, b: int):
    """Candidate 4-bit residual for every b x b block.

    [summary-pt] Metodologia 1 (sparse 4-bit residual R) and 2 (allocated per
    block).  Reading: one fp16 scale per (block, row), sr = f16(max_c |E|/7);
    codes qr = quant4(E, sr); R_hat = sr * qr (exact in fp32).
    Returns (qr int8 [N, K], sr float16 [N/b, K/b, b] indexed [nt, kt, r],
    R_hat float32 [N, K]).
    """
    Eb = _block_view(np.asarray(E, np.float32), b)            # [nt, r, kt, c]
    a = np.abs(Eb).max(axis=3)                                 # [nt, r, kt]
    sr = (a / np.float32(QMAX)).astype(np.float32).astype(np.float16)
    s32 = sr.astype(np.float32)[:, :, :, None]
    qr = quant4(Eb, s32)
    rhat = (s32 * qr.astype(np.float32)).astype(np.float32)
    N, K = E.shape
    return (qr.reshape(N, K), np.ascontiguousarray(sr.transpose(0, 2, 1)),
            rhat.reshape(N, K))


# ----------------------------------------------------------------------------
# Hessian-guided block selection
# ----------------------------------------------------------------------------

def hdiag(xc: np.ndarray) -> np.ndarray:
    """Diagonal Hessian estimate of the input channels, H[k] = sum_t Xc[t,k]^2.

    [summary-pt] Metodologia 2: the score weights the residual error by the
    activation sensitivity (diagonal Hessian estimate) of the input channels.
    Reading: diag(Xc^T Xc) without the 2/T factor (a positive scale does not
    change a top-K ranking), fp64, summed over t = 0, 1, ... in order.
    """
    x = np.asarray(xc, dtype=np.float16)
    T, K = x.shape
    H = np.zeros(K, dtype=np.float64)
    for t in range(T):
        r = x[t].astype(np.float64)
        H = H + r * r
    return H


def delta_scores(E: np.ndarray, rhat: np.ndarray, H: np.ndarray, b: int) -> np.ndarray:
    """Delta-score of every block: sum over the block of H[k]*(E^2 - (E - R_hat)^2).

    [summary-pt] Metodologia 2: Delta approximates the marginal reduction of
    output distortion that a block's residual buys, weighting the residual
    error by the input-channel sensitivity H.
    Reading: fp64, one rounding per operation, no contraction.  Per block
    row r the b terms are summed left to right over c from +0, then the b row
    sums are summed left to right over r from +0.
    Returns float64 [N/b * K/b] in block-id order (id = nt*(K/b) + kt).
    """
    Eb = _block_view(np.asarray(E, np.float32), b).astype(np.float64)     # [nt, r, kt, c]
    Rb = _block_view(np.asarray(rhat, np.float32), b).astype(np.float64)
    NT, _, KT, _ = Eb.shape
    Hb = np.asarray(H, np.float64).reshape(KT, b)                          # [kt, c]
    total = np.zeros((NT, KT), dtype=np.float64)
    for r in range(b):
        row = np.zeros((NT, KT), dtype=np.float64)
        for c in range(b):
            e = Eb[:, r, :, c]
            d = e - Rb[:, r, :, c]
            gain = e * e - d * d
            row = row + Hb[None, :, c] * gain
        total = total + row
    return total.reshape(-1)


def select_top(delta: np.ndarray, n_select: int) -> np.ndarray:
    """Ids of the n_select largest scores, ties to the lower id, returned ascending.

    [summary-pt] Metodologia 2: the top-K blocks by Delta receive the residual.
    Reading: rank by (Delta descending, id ascending).
    """
    d = np.asarray(delta, np.float64)
    B = d.size
    if not (0 <= n_select <= B):
        raise ValueError("n_select out of range")
    order = np.lexsort((np.arange(B), -d))
    return np.sort(order[:n_select]).astype(np.int32)


def select_blocks(w: np.ndarray, xc: np.ndarray, b: int, n_select: int):
    """Full offline selection: base quant -> E -> candidate residuals -> H -> Delta -> top-K.

    Returns (selected int32 ascending, delta float64 [B], H float64 [K]).
    """
    qw, sw = quantize_base(w)
    E = base_error(w, qw, sw)
    _, _, rhat = residual_all_blocks(E, b)
    H = hdiag(xc)
    d = delta_scores(E, rhat, H, b)
    return select_top(d, n_select), d, H


# ----------------------------------------------------------------------------
# Packed storage
# ----------------------------------------------------------------------------

def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """Two's-complement 4-bit codes, two per byte along the last axis:
    byte i = (q[2i] & 0xF) | ((q[2i+1] & 0xF) << 4)."""
    q = np.asarray(q, dtype=np.int8)
    lo = q[..., 0::2].astype(np.uint8) & np.uint8(0x0F)
    hi = q[..., 1::2].astype(np.uint8) & np.uint8(0x0F)
    return (lo | (hi << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(p: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles: uint8 [..., n] -> int8 [..., 2n]."""
    p = np.asarray(p, dtype=np.uint8)
    lo = (p & 0x0F).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def slab_layout(rows: np.ndarray) -> np.ndarray:
    """Packed base codes, row-major uint8 [N, K/2] -> the slab layout uint8
    [N/16, K/128, 64, 16] the library stores.

    The pages fix no byte layout; this one is the library's contract.  For
    slab s (channels 16s .. 16s+15), group j and lane l = 16c + r (c < 4,
    r < 16), entry [s, j, l, :] holds the 16 packed bytes j*64 + 16c ..
    j*64 + 16c + 15 of channel 16s + r: bytes 16c .. 16c+15 of that
    channel's 64-byte group.  It is a permutation of the row-major bytes
    inside each 16-channel slab and group.
    """
    rows = np.asarray(rows, dtype=np.uint8)
    N, Kh = rows.shape
    G = Kh // (GROUP // 2)
    # [s, r, j, c, t] -> [s, j, c, r, t]
    return np.ascontiguousarray(rows.reshape(N // 16, 16, G, 4, 16).transpose(0, 2, 3, 1, 4)
                                .reshape(N // 16, G, 64, 16))


def row_layout(slabs: np.ndarray) -> np.ndarray:
    """Inverse of slab_layout: uint8 [N/16, K/128, 64, 16] -> [N, K/2]."""
    slabs = np.asarray(slabs, dtype=np.uint8)
    S, G = slabs.shape[:2]
    # [s, j, c, r, t] -> [s, r, j, c, t]
    return np.ascontiguousarray(slabs.reshape(S, G, 4, 16, 16).transpose(0, 3, 1, 2, 4)
                                .reshape(S * 16, G * (GROUP // 2)))


def build_csr(selected: np.ndarray, N: int, K: int, b: int):
    """CSR of selected blocks by output tile row: row_ptr[N/b+1], col_idx[n_sel] = kt."""
    sel = np.asarray(selected, dtype=np.int64)
    KT = K // b
    nt = sel // KT
    row_ptr = np.zeros(N // b + 1, dtype=np.int32)
    for t in range(N // b):
        row_ptr[t + 1] = row_ptr[t] + int(np.count_nonzero(nt == t))
    return row_ptr, (sel % KT).astype(np.int32)


def pack_weights(w: np.ndarray, b: int, selected: np.ndarray) -> dict:
    """Packed base + residual for the given (ascending) selected block ids.

    qw uint8 [N/16, G, 64, 16] (slab_layout of the row-major packed codes),
    sw fp16 [N, G], row_ptr int32 [N/b+1], col_idx int32 [n_sel], qr uint8
    [n_sel, b, b/2] (block row r = output nt*b+r, column c = input kt*b+c),
    sr fp16 [n_sel, b].
    """
    w16 = np.asarray(w, np.float16)
    N, K = w16.shape
    qw, sw = quantize_base(w16)
    E = base_error(w16, qw, sw)
    qr_all, sr_all, _ = residual_all_blocks(E, b)
    sel = np.asarray(selected, dtype=np.int64)
    KT = K // b
    row_ptr, col_idx = build_csr(sel, N, K, b)
    qrb = _block_view(qr_all, b)                       # [nt, r, kt, c]
    qr = np.zeros((sel.size, b, b // 2), dtype=np.uint8)
    sr = np.zeros((sel.size, b), dtype=np.float16)
    for i, bid in enumerate(sel):
        nt, kt = divmod(int(bid), KT)
        qr[i] = pack_nibbles(qrb[nt, :, kt, :])
        sr[i] = sr_all[nt, kt]
    return dict(qw=slab_layout(pack_nibbles(qw)), sw=sw, row_ptr=row_ptr, col_idx=col_idx,
                qr=qr, sr=sr, block=b, N=N, K=K)


def unpack_packed(packed: dict):
    """Codes back from a packed dict: (qw int8 [N,K], list of (nt, kt, qr int8 [b,b], sr fp16 [b]))."""
    b = packed["block"]
    qw = unpack_nibbles(row_layout(packed["qw"]))
    blocks = []
    rp, ci = packed["row_ptr"], packed["col_idx"]
    for nt in range(len(rp) - 1):
        for i in range(int(rp[nt]), int(rp[nt + 1])):
            blocks.append((nt, int(ci[i]), unpack_nibbles(packed["qr"][i]), packed["sr"][i]))
    return qw, blocks


# ----------------------------------------------------------------------------
# The layer output
# ----------------------------------------------------------------------------

def gemm_accumulators(qa: np.ndarray, qw: np.ndarray, blocks, b: int):
    """Exact integer accumulators.

    acc_base[m, n, j] = sum_{k in group j} qa[m,k]*qw[n,k];
    acc_res[i][m, r]  = sum_{c<b} qa[m, kt_i*b + c]*qr_i[r, c].
    Products of codes are integers and every partial sum is below 2^24, so
    the fp64 matrix product per group is exact.
    """
    M, K = qa.shape
    N = qw.shape[0]
    G = K // GROUP
    A = qa.astype(np.float64)
    Wq = qw.astype(np.float64)
    acc = np.empty((M, N, G), dtype=np.int64)
    for j in range(G):
        sl = slice(j * GROUP, (j + 1) * GROUP)
        acc[:, :, j] = np.rint(A[:, sl] @ Wq[:, sl].T).astype(np.int64)
    res = []
    for (nt, kt, qr, sr) in blocks:
        sl = slice(kt * b, (kt + 1) * b)
        res.append(np.rint(A[:, sl] @ qr.astype(np.float64).T).astype(np.int64))
    return acc, res


def gemm_output(acc_base, acc_res, sa, sw, blocks, b: int) -> np.ndarray:
    """fp64 Y = sum_j sa[m,j]*sw[n,j]*acc_base[m,n,j] + sum_i sa[m,j_i]*sr_i[r]*acc_res_i[m,r].

    [summary-pt] Metodologia 3: the dense product and the sparse compensation
    are combined by a reduce-sum; [abstract]: sparse block computation fused
    into the dense 4-bit GEMM.  Reading: scales applied in fp64.
    """
    M, N, G = acc_base.shape
    sa64 = np.asarray(sa, np.float64)
    sw64 = np.asarray(sw, np.float64)
    y = np.zeros((M, N), dtype=np.float64)
    for j in range(G):
        y = y + (sa64[:, j, None] * sw64[None, :, j]) * acc_base[:, :, j].astype(np.float64)
    for (nt, kt, qr, sr), ar in zip(blocks, acc_res):
        j = (kt * b) // GROUP
        rows = slice(nt * b, (nt + 1) * b)
        y[:, rows] = y[:, rows] + (sa64[:, j, None] * np.asarray(sr, np.float64)[None, :]) * ar.astype(np.float64)
    return y


def fused_gemm(qa: np.ndarray, sa: np.ndarray, packed: dict):
    """Y for activation codes (int8 [M,K]) and a packed layer; returns (y fp64, acc_base, acc_res)."""
    b = packed["block"]
    qw, blocks = unpack_packed(packed)
    acc, res = gemm_accumulators(qa, qw, blocks, b)
    y = gemm_output(acc, res, sa, packed["sw"], blocks, b)
    return y, acc, res


def layer_reference(x: np.ndarray, w: np.ndarray, xc: np.ndarray, b: int, n_select: int) -> dict:
    """End to end: select, pack, quantise X, fused GEMM."""
    sel, d, H = select_blocks(w, xc, b, n_select)
    packed = pack_weights(w, b, sel)
    qa, sa = quantize_act(x)
    y, acc, res = fused_gemm(qa, sa, packed)
    return dict(selected=sel, delta=d, hdiag=H, packed=packed, qa=qa, sa=sa,
                y=y, acc_base=acc, acc_res=res)


# ----------------------------------------------------------------------------
# Output distortion
# ----------------------------------------------------------------------------

def residual_dense(rhat: np.ndarray, selected, b: int) -> np.ndarray:
    """Dense fp32 matrix holding R_hat on the selected blocks and 0 elsewhere."""
    N, K = rhat.shape
    out = np.zeros_like(rhat, dtype=np.float32)
    KT = K // b
    for bid in np.asarray(selected, dtype=np.int64):
        nt, kt = divmod(int(bid), KT)
        sl = (slice(nt * b, (nt + 1) * b), slice(kt * b, (kt + 1) * b))
        out[sl] = rhat[sl]
    return out


def distortion(xe: np.ndarray, w: np.ndarray, qw: np.ndarray, sw: np.ndarray,
               rhat: np.ndarray, selected, b: int) -> float:
    """Exact output distortion ||Xe (W - deq Q - sum_{i in S} R_hat_i)^T||_F^2 in fp64.

    [summary-pt] Metodologia 2 and Contribuições 2: the costly exact
    output-distortion evaluation that the Delta-score stands in for.
    """
    rem = (np.asarray(w, np.float16).astype(np.float64)
           - dequant_weight(qw, sw).astype(np.float64)
           - residual_dense(rhat, selected, b).astype(np.float64))
    out = np.asarray(xe, np.float16).astype(np.float64) @ rem.T
    return float(np.sum(out * out))


def proxy_distortion(H: np.ndarray, E: np.ndarray, rhat: np.ndarray, selected, b: int) -> float:
    """Diagonal-Hessian proxy sum_{n,k} H[k]*(E - R_hat_S)^2 in fp64."""
    rem = np.asarray(E, np.float64) - residual_dense(rhat, selected, b).astype(np.float64)
    return float(np.sum(np.asarray(H, np.float64)[None, :] * rem * rem))


# ----------------------------------------------------------------------------
# Exact-distortion selection (the costly evaluation the Delta-score replaces)
# ----------------------------------------------------------------------------

def select_exact_greedy(w: np.ndarray, xe: np.ndarray, b: int, n_select: int) -> np.ndarray:
    """Greedy top-K by exact output distortion, for comparison with Delta.

    [summary-pt] Metodologia 2 and Contribuições 2: the Hessian-guided
    Delta-score stands in for a costly exact evaluation of output
    distortion.  This is that evaluation, made selection by selection: at
    each step, add the block whose candidate residual lowers
    ||Xe (W - deq Q - R_S)^T||_F^2 the most given the blocks already chosen
    (ties to the lower id).  Adding block (nt, kt) changes only the outputs
    of its b channels: out[:, rows] -= Xe[:, cols] @ R_hat_block^T, so the
    gain of every block is re-evaluated from the current outputs each step.
    Returns the chosen ids ascending.  fp64 throughout.
    """
    w16 = np.asarray(w, np.float16)
    N, K = w16.shape
    qw, sw = quantize_base(w16)
    E = base_error(w16, qw, sw).astype(np.float64)
    _, _, rhat = residual_all_blocks(E.astype(np.float32), b)
    X = np.asarray(xe, np.float16).astype(np.float64)
    out = X @ E.T                                   # [T, N] outputs of the remainder
    NT, KT = N // b, K // b
    R = _block_view(np.asarray(rhat, np.float64), b)  # [nt, r, kt, c]
    chosen = np.zeros(NT * KT, dtype=bool)
    picks = []
    for _ in range(n_select):
        best, best_gain = -1, -np.inf
        for nt in range(NT):
            o = out[:, nt * b:(nt + 1) * b]          # [T, b]
            base = float(np.sum(o * o))
            for kt in range(KT):
                bid = nt * KT + kt
                if chosen[bid]:
                    continue
                d = X[:, kt * b:(kt + 1) * b] @ R[nt, :, kt, :].T   # [T, b]
                o2 = o - d
                gain = base - float(np.sum(o2 * o2))
                if gain > best_gain:
                    best, best_gain = bid, gain
        nt, kt = divmod(best, KT)
        out[:, nt * b:(nt + 1) * b] -= X[:, kt * b:(kt + 1) * b] @ R[nt, :, kt, :].T
        chosen[best] = True
        picks.append(best)
    return np.sort(np.asarray(picks, dtype=np.int32))


# ----------------------------------------------------------------------------
# Outlier migration before the decomposition (SmoothQuant-style)
# ----------------------------------------------------------------------------

def smooth_scales(xc: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Per-input-channel migration scales s[k] = sqrt(max_t |Xc[t,k]| / max_n |W[n,k]|).

    [summary-pt] Metodologia 1: outliers are first migrated between
    activations and weights, then the migrated weight is decomposed into the
    dense 4-bit base and the sparse residual.  The pages name the step, not
    the rule; reading: SmoothQuant's balance with exponent 1/2, computed in
    fp32 (max of |fp16| is exact; IEEE division and square root, each
    correctly rounded), and s = 1 where either maximum is 0.
    Returns float32 [K].
    """
    ax = np.max(np.abs(np.asarray(xc, np.float16).astype(np.float32)), axis=0)
    aw = np.max(np.abs(np.asarray(w, np.float16).astype(np.float32)), axis=0)
    s = np.ones(ax.shape, dtype=np.float32)
    ok = (ax > 0) & (aw > 0)
    s[ok] = np.sqrt(ax[ok] / aw[ok], dtype=np.float32)
    return s


def smooth_weights(w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Migrated weight W'[n,k] = f16(f32(W[n,k]) * s[k])."""
    return (np.asarray(w, np.float16).astype(np.float32) * np.asarray(s, np.float32)[None, :]).astype(np.float16)


def smooth_acts(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Migrated activations X'[t,k] = f16(f32(X[t,k]) / s[k]), so X' W'^T ~ X W^T."""
    return (np.asarray(x, np.float16).astype(np.float32) / np.asarray(s, np.float32)[None, :]).astype(np.float16)
