"""Pins of the oracle's row-subset path (naive_attention_rows).

Sampled-row parity at full size (the 131072-, 1,048,576- and 921,600-token
shares), the packed and rotary 1M-token tests and bench.py's CPU baseline all
call naive_attention_rows with an arbitrary subset of query rows: positions
that are not 0..R-1, not sorted, and keys truncated at the largest position
seen. naive_attention only ever calls it with every row in order, so the
pins here check the subset path itself, against torch's float64 SDPA over the
whole sequence (a library routine written independently of the oracle) and
against the same rows of naive_attention:

- the row sets of contiguous, striped and zigzag shares (token placement
  written out per layout in the tests), a shuffled subset with repeats, a
  single late row and row 0 alone;
- causal and non-causal, grouped-query heads (4/2, 4/1) and plain heads;
- packed sequences: each sequence's rows against its own keys (positions
  counted from the sequence start), as the packed full-size tests slice them,
  against SDPA with an explicit block-diagonal mask.

Planted mistakes in the subset path (the causal mask built from the row
index instead of the position, keys truncated at the row count or one short
of the largest position, lse from the unshifted sum) must fail these pins
while naive_attention on all rows stays correct.
"""

import numpy as np
import pytest

from oracle import ring_oracle as orc
from tests.test_oracle_pins import _rand, _sdpa64, _share_rows
from tests.test_oracle_zigzag_varlen import _masked_sdpa64, _packed_mask, _packed_rows


def _lse64(q, k, causal):
    """log-sum-exp of the scaled scores per (batch, row, head), float64,
    computed here from the definition with torch (GQA by repeating heads)."""
    import torch
    tq = torch.from_numpy(np.ascontiguousarray(q))
    tk = torch.from_numpy(np.ascontiguousarray(k))
    hq, hkv = tq.shape[2], tk.shape[2]
    tk = tk.repeat_interleave(hq // hkv, dim=2)
    s = torch.einsum("bthd,buhd->bhtu", tq, tk) / np.sqrt(q.shape[-1])
    if causal:
        t = s.shape[-1]
        s = s.masked_fill(torch.triu(torch.ones(t, t, dtype=torch.bool), 1), float("-inf"))
    return torch.logsumexp(s, dim=-1).permute(0, 2, 1).numpy()


def _row_sets(n, blen, seed):
    """Named subsets of global query positions of an n*blen-token sequence."""
    rng = np.random.default_rng(seed)
    seq = n * blen
    sets = {}
    for layout in ("contiguous", "striped", "zigzag"):
        for r in (0, n - 1):
            sets[f"{layout}_r{r}"] = _share_rows(layout, n, r, blen)
    shuffled = rng.choice(seq, size=seq // 2, replace=True)
    sets["shuffled_with_repeats"] = shuffled
    sets["single_late_row"] = np.array([seq - 3])
    sets["row0"] = np.array([0])
    return sets


def _rows_pins_hold(tol=1e-12) -> bool:
    """Every subset of rows, every head grouping, causal and not, equals the
    same rows of float64 SDPA over the whole sequence (and of the oracle's
    all-rows call); lse equals the definition's log-sum-exp."""
    try:
        n, blen = 4, 6
        for hq, hkv, seed in ((1, 1, 1), (4, 2, 2), (4, 1, 3)):
            q, k, v = _rand(seed, 2, n * blen, hq, hkv, 16)
            q = 1.5 * q
            for causal in (False, True):
                ref = _sdpa64(q, k, v, causal)
                ref_lse = _lse64(q, k, causal)
                full, full_lse = orc.naive_attention(q, k, v, causal)
                for name, pos in _row_sets(n, blen, seed).items():
                    out, lse = orc.naive_attention_rows(q[:, pos], pos, k, v, causal)
                    if out.shape != (2, len(pos), hq, 16):
                        return False
                    if not np.allclose(out, ref[:, pos], atol=tol, rtol=0):
                        return False
                    if not np.allclose(lse, ref_lse[:, pos], atol=tol, rtol=0):
                        return False
                    if not np.allclose(out, full[:, pos], atol=1e-13, rtol=0):
                        return False
                    if not np.allclose(lse, full_lse[:, pos], atol=1e-13, rtol=0):
                        return False
        # packed sequences, rows sliced per sequence as the full-size tests do
        n, cu = 3, [0, 6, 18, 18, 24]
        q, k, v = _rand(5, 1, 24, 4, 2, 8)
        q = 2.0 * q
        for causal in (False, True):
            ref = _masked_sdpa64(q, k, v, _packed_mask(cu, causal))
            for layout in ("contiguous", "striped", "zigzag"):
                for r in range(n):
                    tok = _packed_rows(layout, n, r, cu)
                    seqid = np.searchsorted(np.asarray(cu), tok, side="right") - 1
                    for s in np.unique(seqid):
                        sel = tok[seqid == s]
                        start, end = cu[s], cu[s + 1]
                        rel = sel - start
                        kmax = int(rel.max()) + 1 if causal else end - start
                        o, _ = orc.naive_attention_rows(q[:, sel], rel, k[:, start:start + kmax],
                                                        v[:, start:start + kmax], causal)
                        if not np.allclose(o, ref[:, sel], atol=tol, rtol=0):
                            return False
        return True
    except (ValueError, IndexError, FloatingPointError):
        return False


def test_row_subsets_match_sdpa_and_all_rows():
    assert _rows_pins_hold()


def test_row_subset_causal_row_zero_is_v0_and_late_row_sees_prefix():
    """Closed forms on a subset: position 0 alone returns V[0] exactly; a row
    at position p with constant keys returns the mean of V[0..p]."""
    q, k, v = _rand(9, 1, 40, 2, 1, 16)
    out, _ = orc.naive_attention_rows(q[:, [0]], [0], k, v, True)
    assert np.array_equal(out[0, 0, 0], v[0, 0, 0]) and np.array_equal(out[0, 0, 1], v[0, 0, 0])
    kc = np.repeat(k[:, :1], 40, axis=1)
    pos = np.array([31, 7, 19])
    out, _ = orc.naive_attention_rows(q[:, pos], pos, kc, v, True)
    for i, p in enumerate(pos):
        np.testing.assert_allclose(out[0, i, 0], v[0, :p + 1, 0].mean(axis=0), atol=1e-13, rtol=0)


# ----------------------------------------------------------------- mutants --
def _rows_variant(mask_rows=False, kmax_rows=False, kmax_short=False, lse_unshifted=False):
    """A copy of the oracle's subset path with one planted mistake."""
    def fn(q_rows, q_pos, k, v, causal, scale=None):
        q_rows, k, v = orc._f64(q_rows), orc._f64(k), orc._f64(v)
        q_pos = np.asarray(q_pos, dtype=np.int64)
        bsz, nrows, hq, d = q_rows.shape
        hkv = k.shape[2]
        if scale is None:
            scale = orc.default_scale(d)
        k_pos = np.arange(k.shape[1], dtype=np.int64)
        out = np.zeros((bsz, nrows, hq, d))
        lse = np.full((bsz, nrows, hq), -np.inf)
        for b in range(bsz):
            for h in range(hq):
                g = orc.kv_head_of(h, hq, hkv)
                kk, vv = k[b, :, g, :], v[b, :, g, :]
                if causal:
                    kmax = int(q_pos.max()) + 1
                    if kmax_rows:
                        kmax = nrows
                    if kmax_short:
                        kmax -= 1
                    kk, vv, kp = kk[:kmax], vv[:kmax], k_pos[:kmax]
                else:
                    kp = k_pos
                s = (q_rows[b, :, h, :] @ kk.T) * scale
                qp = np.arange(nrows, dtype=np.int64) if mask_rows else q_pos
                vis = orc._visibility(qp, kp, causal)
                s = np.where(vis, s, -np.inf)
                mx = s.max(axis=1, keepdims=True)
                has = np.isfinite(mx)
                base = np.where(has, mx, 0.0)
                e = np.where(vis, np.exp(s - base), 0.0)
                den = e.sum(axis=1, keepdims=True)
                safe = np.where(den > 0, den, 1.0)
                out[b, :, h, :] = np.where(den > 0, (e / safe) @ vv, 0.0)
                lse_b = np.log(safe[:, 0]) if lse_unshifted else base[:, 0] + np.log(safe[:, 0])
                lse[b, :, h] = np.where(has[:, 0], lse_b, -np.inf)
        return out, lse
    return fn


ROW_MUTANTS = {
    "mask_from_row_index": _rows_variant(mask_rows=True),
    "keys_truncated_at_row_count": _rows_variant(kmax_rows=True),
    "keys_one_short": _rows_variant(kmax_short=True),
    "lse_without_max": _rows_variant(lse_unshifted=True),
}


def test_unmutated_copy_passes():
    """The mutants' template without a planted mistake passes the pins (so
    each failure below comes from its one change)."""
    import unittest.mock as um
    with um.patch.object(orc, "naive_attention_rows", _rows_variant()):
        assert _rows_pins_hold()


@pytest.mark.parametrize("name", sorted(ROW_MUTANTS))
def test_row_pins_catch_mutant(name, monkeypatch):
    monkeypatch.setattr(orc, "naive_attention_rows", ROW_MUTANTS[name])
    # the all-rows call is unaffected by the mask and truncation mutants ...
    if name in ("mask_from_row_index", "keys_truncated_at_row_count"):
        q, k, v = _rand(4, 1, 24, 4, 2, 16)
        ref = _sdpa64(q, k, v, True)
        out, _ = orc.naive_attention(q, k, v, True)
        np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)
    # ... but the subset pins catch every one
    assert not _rows_pins_hold()
