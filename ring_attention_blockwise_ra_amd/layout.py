"""Caller-side token permutation for the layouts (done once, outside the hot
path).

The library takes q (one device's share) and the N K/V blocks already stored
in the layout's token order. This module produces them from global-order
tensors:
  contiguous: block i holds global tokens [i*B, (i+1)*B)
  striped:    block i holds global tokens i, i+N, i+2N, ... (token t goes to
              block t mod N), the striped assignment the Ultralytics "Ring
              Attention" page describes in section "How ring attention works".
  zigzag:     the sequence is cut into 2N chunks of B/2 tokens and block i
              holds chunk i followed by chunk 2N-1-i (the AI Understanding
              page names zigzag as a variant that rebalances causal work).
Packed sequences (several sequences of different lengths concatenated, the
variable-length case the troisinh page lists among the trade-offs): each
sequence is split by the layout on its own and block i holds, sequence after
sequence, the tokens the layout gives it.
"""

from __future__ import annotations

import torch

LAYOUTS = ("contiguous", "striped", "zigzag")


def share_tokens(layout: str, n_ring: int, block: int, block_len: int, device="cpu") -> torch.Tensor:
    """Global token indices held by `block`, in local order."""
    a = torch.arange(block_len, dtype=torch.int64, device=device)
    if layout == "contiguous":
        return block * block_len + a
    if layout == "striped":
        return a * n_ring + block
    if layout == "zigzag":
        if block_len % 2:
            raise ValueError("zigzag needs an even block length")
        h = block_len // 2
        chunk = torch.where(a < h, torch.full_like(a, block), torch.full_like(a, 2 * n_ring - 1 - block))
        return chunk * h + a % h
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
    if layout == "zigzag":
        out = torch.empty((n_ring, bsz, blen, h, d), dtype=x.dtype, device=x.device)
        for j in range(n_ring):
            out[j] = x.index_select(1, share_tokens(layout, n_ring, j, blen, device=x.device))
        return out
    raise ValueError(f"unknown layout {layout!r}")


def packed_share_tokens(layout: str, n_ring: int, block: int, cu_seqlens, device="cpu") -> torch.Tensor:
    """Global packed token indices held by `block` when the sequences
    [cu_seqlens[s], cu_seqlens[s+1]) are split over the ring one by one."""
    cu = [int(c) for c in cu_seqlens]
    parts = []
    for s in range(len(cu) - 1):
        L = cu[s + 1] - cu[s]
        if L % n_ring:
            raise ValueError(f"sequence {s}: length {L} is not a multiple of n_ring")
        if L:
            parts.append(cu[s] + share_tokens(layout, n_ring, block, L // n_ring, device=device))
    if not parts:
        return torch.zeros(0, dtype=torch.int64, device=device)
    return torch.cat(parts)


def packed_blocks_from_global(x: torch.Tensor, layout: str, n_ring: int, cu_seqlens) -> torch.Tensor:
    """[1, T, H, d] packed global order -> [N, 1, T/N, H, d] blocks."""
    bsz, seq, h, d = x.shape
    blen = seq // n_ring
    out = torch.empty((n_ring, bsz, blen, h, d), dtype=x.dtype, device=x.device)
    for j in range(n_ring):
        out[j] = x.index_select(1, packed_share_tokens(layout, n_ring, j, cu_seqlens, device=x.device))
    return out
