"""Caller-side token permutation for the two layouts (done once, outside the
hot path).

The library takes q (one device's share) and the N K/V blocks already stored
in the layout's token order. This module produces them from global-order
tensors:
  contiguous: block i holds global tokens [i*B, (i+1)*B)
  striped:    block i holds global tokens i, i+N, i+2N, ... (token t goes to
              block t mod N), the striped assignment the Ultralytics "Ring
              Attention" page describes in section "How ring attention works".
"""

from __future__ import annotations

import torch


def share_tokens(layout: str, n_ring: int, block: int, block_len: int, device="cpu") -> torch.Tensor:
    """Global token indices held by `block`, in local order."""
    a = torch.arange(block_len, dtype=torch.int64, device=device)
    if layout == "contiguous":
        return block * block_len + a
    if layout == "striped":
        return a * n_ring + block
    raise ValueError(f"unknown layout {layout!r}")


def blocks_from_global(x: torch.Tensor, layout: str, n_ring: int) -> torch.Tensor:
    """[B, S, H, d] in global order -> [N, B, S/N, H, d] blocks (contiguous copy)."""
    bsz, seq, h, d = x.shape
    if seq % n_ring:
        raise ValueError("sequence length must be a multiple of n_ring")
    blen = seq // n_ring
    if layout == "contiguous":
        return x.reshape(bsz, n_ring, blen, h, d).transpose(0, 1).contiguous()
    if layout == "striped":
        return x.reshape(bsz, blen, n_ring, h, d).permute(2, 0, 1, 3, 4).contiguous()
    raise ValueError(f"unknown layout {layout!r}")
