"""Layer-quality metrics for measurement runs (not part of the layer's path).

The output distortion of a decomposition, ||Xe (W - deq Q - R_S)^T||_F^2, is
what the Delta-score stands in for (MosaicQuant technical summary,
gist.science/pt/paper/2606.15652, Metodologia 2: the Hessian-guided score
approximates each block's marginal reduction of output distortion).  The
benchmark reports it as "distortion recovered" = 1 - D(S_rho) / D(empty).

These functions read a packed layer as the library wrote it (4-bit codes,
fp16 scales, CSR residual) and rebuild the dequantised weight with torch, on
whatever device the tensors live on, in float64.
"""
from __future__ import annotations

import torch

GROUP = 128


def unpack_codes(p: torch.Tensor) -> torch.Tensor:
    """uint8 [..., K/2] two's-complement nibbles (low first) -> int8 [..., K]."""
    lo = (p & 0xF).to(torch.int16)
    hi = (p >> 4).to(torch.int16)
    q = torch.stack((lo, hi), dim=-1).reshape(*p.shape[:-1], p.shape[-1] * 2)
    return torch.where(q >= 8, q - 16, q).to(torch.int8)


def row_bytes(qw: torch.Tensor) -> torch.Tensor:
    """Packed base codes from the slab layout [N/16, K/128, 64, 16] (lane
    l = 16c + r of slab s, group j holds bytes 16c..16c+15 of channel
    16s + r's 64-byte group) back to row-major uint8 [N, K/2]."""
    S, G = qw.shape[:2]
    return qw.reshape(S, G, 4, 16, 16).permute(0, 3, 1, 2, 4).reshape(S * 16, G * 64)


def dequant_base(layer) -> torch.Tensor:
    """deq Q(W) as float64 [N, K]."""
    q = unpack_codes(row_bytes(layer.qw)).to(torch.float64)
    s = layer.sw.to(torch.float64).repeat_interleave(GROUP, dim=1)
    return q * s


def dequant_residual(layer) -> torch.Tensor:
    """Dense float64 [N, K] holding deq R on the selected blocks, 0 elsewhere."""
    b = layer.block
    out = torch.zeros((layer.N, layer.K), dtype=torch.float64, device=layer.qw.device)
    ns = layer.n_select
    if ns == 0:
        return out
    rows = torch.repeat_interleave(torch.arange(layer.N // b, device=layer.row_ptr.device),
                                   torch.diff(layer.row_ptr.long()))
    cols = layer.col_idx.long()
    r = unpack_codes(layer.qr).to(torch.float64) * layer.sr.to(torch.float64)[:, :, None]
    blocks = out.view(layer.N // b, b, layer.K // b, b)
    blocks[rows, :, cols, :] = r
    return out


def distortion(xe: torch.Tensor, w: torch.Tensor, layer, with_residual: bool = True) -> float:
    """||Xe (W - deq Q - deq R)^T||_F^2 in float64."""
    rem = w.to(torch.float64) - dequant_base(layer)
    if with_residual:
        rem = rem - dequant_residual(layer)
    out = xe.to(torch.float64) @ rem.T
    return float((out * out).sum())
