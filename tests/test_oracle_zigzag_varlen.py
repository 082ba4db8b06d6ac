"""Pins of the oracle's zigzag layout and packed variable-length sequences.

Zigzag ([AU] "Framtiden for sekvensparallellism och ringuppmarksamhet" names
it as a variant that rebalances causal work; the chunk pairing is the plain
reading): 2N chunks of B/2 tokens, block i = chunk i then chunk 2N-1-i.
Packed sequences ([TS] "Trade-off thuc te"): each sequence is split over the
blocks by the layout on its own; attention never crosses sequences.

Every expected value here comes from torch's float64 SDPA (with an explicit
block-diagonal mask for packed sequences), scalar loops, or token placement
written out per layout in the tests, never from the oracle itself.
"""

import itertools
import math

import numpy as np
import pytest
import torch

from oracle import ring_oracle as orc
from tests.test_oracle_pins import _blocks_from_global, _rand, _sdpa64, _share_rows

LAYOUTS3 = ("contiguous", "striped", "zigzag")


def _masked_sdpa64(q, k, v, mask):
    """float64 SDPA on [1, T, H, d] arrays with a [T, T] boolean mask (True =
    visible); KV heads repeated for grouped queries. Rows with no visible
    key are not produced by the callers."""
    hq, hkv = q.shape[2], k.shape[2]
    tq = torch.from_numpy(np.ascontiguousarray(q)).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.ascontiguousarray(k)).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, 1)
    tv = torch.from_numpy(np.ascontiguousarray(v)).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, 1)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask))
    return o.permute(0, 2, 1, 3).numpy()


def _packed_mask(cu, causal):
    t = cu[-1]
    seq = np.zeros(t, dtype=np.int64)
    for s in range(len(cu) - 1):
        seq[cu[s]:cu[s + 1]] = s
    mask = seq[:, None] == seq[None, :]
    if causal:
        mask &= np.tril(np.ones((t, t), dtype=bool))
    return mask


def _packed_rows(layout, n, block, cu):
    """Global packed token index of every local token of `block`."""
    rows = []
    for s in range(len(cu) - 1):
        L = cu[s + 1] - cu[s]
        if L:
            rows.extend((cu[s] + _share_rows(layout, n, block, L // n)).tolist())
    return np.array(rows, dtype=np.int64)


# ------------------------------------------------------------------ zigzag --
def test_zigzag_positions_partition_and_order():
    for n, blen in [(1, 2), (2, 4), (3, 6), (4, 8), (8, 16)]:
        allpos = np.concatenate([orc.global_positions("zigzag", n, j, blen) for j in range(n)])
        assert sorted(allpos.tolist()) == list(range(n * blen))
        for j in range(n):
            p = orc.global_positions("zigzag", n, j, blen)
            np.testing.assert_array_equal(p, _share_rows("zigzag", n, j, blen))
            assert np.all(np.diff(p) > 0)  # local order follows position order
    with pytest.raises(ValueError):
        orc.global_positions("zigzag", 2, 0, 3)


def test_zigzag_hand_example():
    # N=2, B=4: chunks of 2 tokens; block 0 = chunks 0 and 3, block 1 = 1 and 2
    np.testing.assert_array_equal(orc.global_positions("zigzag", 2, 0, 4), [0, 1, 6, 7])
    np.testing.assert_array_equal(orc.global_positions("zigzag", 2, 1, 4), [2, 3, 4, 5])


@pytest.mark.parametrize("n,blen,heads,causal",
                         list(itertools.product([1, 2, 3, 4], [2, 4, 6], [(1, 1), (4, 2)], [False, True])))
def test_zigzag_brute_force_tiny_vs_sdpa(n, blen, heads, causal):
    hq, hkv = heads
    q, k, v = _rand(n * 10 + blen, 1, n * blen, hq, hkv, 16)
    ref = _sdpa64(q, k, v, causal)
    kb, vb = _blocks_from_global(k, "zigzag", n), _blocks_from_global(v, "zigzag", n)
    for r in range(n):
        rows = _share_rows("zigzag", n, r, blen)
        o2, _ = orc.ring_share(q[:, rows], kb, vb, r, n, "zigzag", causal)
        np.testing.assert_allclose(o2, ref[:, rows], atol=1e-12, rtol=0)


def test_zigzag_row0_and_arrival_order():
    n, blen = 4, 6
    q, k, v = _rand(12, 1, n * blen, 4, 2, 8)
    q = 3.0 * q
    kb, vb = _blocks_from_global(k, "zigzag", n), _blocks_from_global(v, "zigzag", n)
    rng = np.random.default_rng(2)
    for r in range(n):
        rows = _share_rows("zigzag", n, r, blen)
        base, lse0 = orc.ring_share(q[:, rows], kb, vb, r, n, "zigzag", True)
        if r == 0:  # token 0 is local row 0 of rank 0 and sees only itself
            for h in range(4):
                np.testing.assert_allclose(base[:, 0, h], v[:, 0, h // 2], atol=1e-15, rtol=0)
        for _ in range(3):
            o, lse = orc.ring_share(q[:, rows], kb, vb, r, n, "zigzag", True,
                                    order=list(rng.permutation(n)))
            np.testing.assert_allclose(o, base, atol=1e-13, rtol=0)
            np.testing.assert_allclose(lse, lse0, atol=1e-13, rtol=0)


def test_zigzag_pure_python():
    n, blen, d = 2, 4, 3
    q, k, v = _rand(19, 1, n * blen, 1, 1, d)
    kb, vb = _blocks_from_global(k, "zigzag", n), _blocks_from_global(v, "zigzag", n)
    for r in range(n):
        rows = _share_rows("zigzag", n, r, blen)
        o2, _ = orc.ring_share(q[:, rows], kb, vb, r, n, "zigzag", True)
        for a, t in enumerate(rows):
            w = [(u, math.exp(sum(q[0, t, 0, i] * k[0, u, 0, i] for i in range(d)) / math.sqrt(d)))
                 for u in range(t + 1)]
            z = sum(e for _, e in w)
            for i in range(d):
                assert abs(o2[0, a, 0, i] - sum(e * v[0, u, 0, i] for u, e in w) / z) < 1e-13


def test_zigzag_balances_causal_work():
    for n, blen in [(2, 4), (4, 8), (8, 16), (3, 10)]:
        counts = set()
        for r in range(n):
            want = sum(1 for t in _share_rows("zigzag", n, r, blen) for u in range(n * blen) if u <= t)
            assert orc.visible_pairs_bruteforce("zigzag", True, n, r, blen) == want
            assert orc.visible_pairs_closed_form("zigzag", True, n, r, blen) == want
            counts.add(want)
        assert len(counts) == 1  # every rank does the same causal work
    # at the 1M-token share: 7 B^2/2 + B(B+1)/2 for every rank
    b = 131072
    assert orc.visible_pairs_closed_form("zigzag", True, 8, 3, b) == 7 * b * b // 2 + b * (b + 1) // 2


def test_zigzag_tile_classes():
    n, blen = 3, 8
    for r, j in itertools.product(range(n), range(n)):
        rows, keys = _share_rows("zigzag", n, r, blen), _share_rows("zigzag", n, j, blen)
        for tq, tk in [(1, 1), (2, 4), (4, 2), (3, 3), (8, 8)]:
            c = orc.tile_classes_bruteforce("zigzag", True, n, r, j, blen, blen, tq, tk)
            for qt in range(-(-blen // tq)):
                for kt in range(-(-blen // tk)):
                    vis = [u <= t for t in rows[qt * tq:(qt + 1) * tq] for u in keys[kt * tk:(kt + 1) * tk]]
                    want = orc.FULL if all(vis) else (orc.SKIP if not any(vis) else orc.PARTIAL)
                    assert c[qt, kt] == want
            cnt = orc.tile_class_counts("zigzag", True, n, r, j, blen, blen, tq, tk)
            assert cnt == (int((c == orc.FULL).sum()), int((c == orc.PARTIAL).sum()),
                           int((c == orc.SKIP).sum()))


# ----------------------------------------------------------------- varlen --
SEQLENS = {
    "contiguous": [3, 9, 0, 6],
    "striped": [6, 3, 12],
    "zigzag": [6, 12, 0, 18],
}


def test_varlen_positions_partition_each_sequence():
    for layout in LAYOUTS3:
        n = 3
        lens = SEQLENS[layout]
        seen = {s: [] for s in range(len(lens))}
        for j in range(n):
            ids, pos = orc.varlen_positions(layout, n, j, lens)
            assert ids.size == pos.size == sum(lens) // n
            assert np.all(np.diff(ids) >= 0)
            for s in range(len(lens)):
                seen[s].extend(pos[ids == s].tolist())
        for s, L in enumerate(lens):
            assert sorted(seen[s]) == list(range(L))
    with pytest.raises(ValueError):
        orc.varlen_positions("zigzag", 3, 0, [3])


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_naive_vs_masked_sdpa(causal):
    cu = [0, 5, 5, 12, 20]
    q, k, v = _rand(77, 1, 20, 4, 2, 8)
    out, lse = orc.naive_attention_varlen(q, k, v, cu, causal)
    ref = _masked_sdpa64(q, k, v, _packed_mask(cu, causal))
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)
    # lse of the last sequence's rows against the library log-sum-exp
    s = torch.from_numpy(q[0, 12:, 1] @ k[0, 12:, 0].T / math.sqrt(8))
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(8, 8, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse[0, 12:, 1], torch.logsumexp(s, -1).numpy(), atol=1e-13, rtol=0)


@pytest.mark.parametrize("layout", LAYOUTS3)
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_ring_vs_masked_sdpa(layout, causal):
    n = 3
    lens = SEQLENS[layout]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(int).tolist()
    q, k, v = _rand(5, 1, cu[-1], 4, 2, 8)
    q = 2.0 * q
    ref = _masked_sdpa64(q, k, v, _packed_mask(cu, causal))
    kb = np.stack([k[:, _packed_rows(layout, n, j, cu)] for j in range(n)])
    vb = np.stack([v[:, _packed_rows(layout, n, j, cu)] for j in range(n)])
    for r in range(n):
        rows = _packed_rows(layout, n, r, cu)
        o2, lse2 = orc.ring_share(q[:, rows], kb, vb, r, n, layout, causal, seqlens=lens)
        np.testing.assert_allclose(o2, ref[:, rows], atol=1e-12, rtol=0)
        assert np.all(np.isfinite(lse2))


def test_varlen_pair_counts_and_tile_classes():
    n = 3
    for layout in LAYOUTS3:
        lens = SEQLENS[layout]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(int).tolist()
        seq = np.repeat(np.arange(len(lens)), lens)
        blen = cu[-1] // n
        for causal in (False, True):
            for r in range(n):
                rows = _packed_rows(layout, n, r, cu)
                want = sum(1 for t in rows for u in range(cu[-1])
                           if seq[u] == seq[t] and (u <= t or not causal))
                assert orc.visible_pairs_bruteforce(layout, causal, n, r, blen, seqlens=lens) == want
                assert orc.visible_pairs_closed_form(layout, causal, n, r, blen, seqlens=lens) == want
                for j in range(n):
                    keys = _packed_rows(layout, n, j, cu)
                    c = orc.tile_classes_bruteforce(layout, causal, n, r, j, blen, blen, 2, 3, seqlens=lens)
                    for qt in range(-(-blen // 2)):
                        for kt in range(-(-blen // 3)):
                            vis = [seq[u] == seq[t] and (u <= t or not causal)
                                   for t in rows[2 * qt:2 * qt + 2] for u in keys[3 * kt:3 * kt + 3]]
                            want_c = orc.FULL if all(vis) else (orc.SKIP if not any(vis) else orc.PARTIAL)
                            assert c[qt, kt] == want_c
