"""The named workloads as device tensors, ready for the library.

Builds one device's share (q) and the N K/V blocks of a workload in the
layout's token order from the seeded global-order generators, and computes the
work a share represents (visible query/key pairs, counted FLOPs) for
throughput reporting. Holds no attention arithmetic.
"""

from __future__ import annotations

import torch

from . import synth
from .layout import blocks_from_global, packed_blocks_from_global, packed_share_tokens, share_tokens


def visible_pairs(layout: str, causal: bool, n_ring: int, rank: int, block_len: int,
                  seqlens=None) -> int:
    """Unmasked (query, key) pairs of one share over all N blocks, per head and
    batch row: non-causal N*B^2; contiguous causal r*B^2 + B(B+1)/2 (blocks
    before the share fully visible, its own block a triangle); striped causal
    N*B(B-1)/2 + (r+1)*B (every block a triangle, blocks after the share
    without their diagonal); zigzag causal (N-1)*B^2/2 + B(B+1)/2 for every
    rank (half of each other block, a triangle of its own). Packed
    sequences: the sum over sequences with B = L_s / N."""
    if seqlens is not None:
        return sum(visible_pairs(layout, causal, n_ring, rank, int(L) // n_ring) for L in seqlens)
    n, b, r = n_ring, block_len, rank
    if not causal:
        return n * b * b
    if layout == "contiguous":
        return r * b * b + b * (b + 1) // 2
    if layout == "zigzag":
        return (n - 1) * b * b // 2 + b * (b + 1) // 2
    return n * b * (b - 1) // 2 + (r + 1) * b


def counted_flops(layout, causal, n_ring, rank, block_len, hq, head_dim, batch=1,
                  seqlens=None) -> int:
    """4*d FLOPs (2d for q.k, 2d for p*v) per visible pair per query head."""
    return 4 * head_dim * hq * batch * visible_pairs(layout, causal, n_ring, rank, block_len,
                                                     seqlens)


def prepare(cfg_name: str, layout: str, rank: int, device="cuda", keep_global: bool = False):
    """Device tensors of one share of a named workload.

    Returns a dict with q [1, B, hq, d], k/v [N, 1, B, hkv, d] (layout order),
    q_tokens (global token index of each local query row), the config dict,
    seqlens / cu_seqlens of packed workloads (else None), and, when
    keep_global, the global-order k and v.
    """
    c = synth.CONFIGS[cfg_name]
    n, blen = c["n_ring"], c["block"]
    lens = synth.config_seqlens(cfg_name, layout)
    cu = None
    if lens is None:
        q_tok = share_tokens(layout, n, rank, blen, device="cpu")
    else:
        cu = [0]
        for L in lens:
            cu.append(cu[-1] + L)
        q_tok = packed_share_tokens(layout, n, rank, cu, device="cpu")
    q, k_glob, v_glob = synth.config_global(cfg_name, device=device, q_rows=q_tok.to(device))
    if cu is None:
        kb = blocks_from_global(k_glob, layout, n)
        vb = blocks_from_global(v_glob, layout, n)
    else:
        kb = packed_blocks_from_global(k_glob, layout, n, cu)
        vb = packed_blocks_from_global(v_glob, layout, n, cu)
    out = dict(cfg=c, q=q.contiguous(), k=kb, v=vb, q_tokens=q_tok, layout=layout, rank=rank,
               seqlens=lens, cu_seqlens=cu)
    if keep_global:
        out["k_global"], out["v_global"] = k_glob, v_glob
    else:
        del k_glob, v_glob
    return out


def sample_rows(block_len: int, n: int, seed: int = 0, tile_edges=(128, 256),
                n_random: int | None = None) -> torch.Tensor:
    """Local query rows to check at full size, at most n: the first 8 and the
    last 8 rows, rows on both sides of tile edges (and of the block's
    middle), then seeded random rows. At least n_random (default n // 2)
    of the n are random rows, so every sample mixes edges with the interior;
    when n is small the edge rows are kept in that order of priority."""
    n = max(0, min(n, block_len))
    n_random = n // 2 if n_random is None else min(n_random, n)
    edges = []
    for r in list(range(min(8, block_len))) + list(range(max(0, block_len - 8), block_len)):
        if r not in edges:
            edges.append(r)
    for t in tile_edges:
        for e in (t - 1, t, 2 * t - 1, 2 * t, block_len // 2 - 1, block_len // 2):
            if 0 <= e < block_len and e not in edges:
                edges.append(e)
    chosen = set(edges[:n - n_random])
    g = torch.Generator().manual_seed(seed)
    while len(chosen) < n:
        chosen.add(int(torch.randint(0, block_len, (1,), generator=g)))
    return torch.tensor(sorted(chosen), dtype=torch.int64)
