"""Planted mistakes in the oracle must be caught by its pins.

Each mutant replaces one oracle function with a plausible wrong version (a
dropped term, a wrong sign or index, a transposed operand). The pin battery
below -- comparisons against torch's float64 SDPA, the Ultralytics worked
example and closed forms, all computed without the oracle -- must fail for
every mutant and pass for the unmutated oracle. Mistakes are planted only in
the oracle, on the CPU.
"""

import math

import numpy as np
import pytest
import torch

from oracle import ring_oracle as orc
from tests.test_oracle_pins import _blocks_from_global, _rand, _sdpa64, _share_rows
from tests.test_oracle_zigzag_varlen import _masked_sdpa64, _packed_mask, _packed_rows


def _pins_hold() -> bool:
    try:
        # GQA, causal and non-causal, both layouts, vs float64 SDPA
        for layout in ("contiguous", "striped", "zigzag"):
            for causal in (False, True):
                n, blen = 3, 4
                q, k, v = _rand(7, 1, n * blen, 4, 2, 8)
                q = 2.0 * q
                ref = _sdpa64(q, k, v, causal)
                out, lse = orc.naive_attention(q, k, v, causal)
                if not np.allclose(out, ref, atol=1e-10, rtol=0):
                    return False
                kb, vb = _blocks_from_global(k, layout, n), _blocks_from_global(v, layout, n)
                for r in range(n):
                    rows = _share_rows(layout, n, r, blen)
                    o2, lse2 = orc.ring_share(q[:, rows], kb, vb, r, n, layout, causal)
                    if not np.allclose(o2, ref[:, rows], atol=1e-10, rtol=0):
                        return False
                    if not np.allclose(lse2, lse[:, rows], atol=1e-10, rtol=0):
                        return False
                # counted work: closed form against an independent count
                for r in range(n):
                    rows = _share_rows(layout, n, r, blen)
                    want = sum(1 for t in rows for u in range(n * blen) if (u <= t or not causal))
                    if orc.visible_pairs_closed_form(layout, causal, n, r, blen) != want:
                        return False
                    for j in range(n):
                        keys = _share_rows(layout, n, j, blen)
                        c = orc.tile_classes_bruteforce(layout, causal, n, r, j, blen, blen, 2, 2)
                        for qt in range(2):
                            for kt in range(2):
                                vis = [(u <= t or not causal) for t in rows[2 * qt:2 * qt + 2]
                                       for u in keys[2 * kt:2 * kt + 2]]
                                want_c = orc.FULL if all(vis) else (orc.SKIP if not any(vis) else orc.PARTIAL)
                                if c[qt, kt] != want_c:
                                    return False
        # positions of all blocks partition the sequence, block by block as placed by hand
        for layout in ("contiguous", "striped", "zigzag"):
            for n, blen in ((3, 4), (4, 6)):
                for j in range(n):
                    if not np.array_equal(orc.global_positions(layout, n, j, blen),
                                          _share_rows(layout, n, j, blen)):
                        return False
        # packed sequences, every layout, vs SDPA with an explicit block-diagonal mask
        n, lens = 3, [6, 12, 0, 6]
        cu = [0, 6, 18, 18, 24]
        q, k, v = _rand(3, 1, 24, 2, 1, 8)
        q = 2.0 * q
        for layout in ("contiguous", "striped", "zigzag"):
            for causal in (False, True):
                ref = _masked_sdpa64(q, k, v, _packed_mask(cu, causal))
                kb = np.stack([k[:, _packed_rows(layout, n, j, cu)] for j in range(n)])
                vb = np.stack([v[:, _packed_rows(layout, n, j, cu)] for j in range(n)])
                for r in range(n):
                    rows = _packed_rows(layout, n, r, cu)
                    o2, _ = orc.ring_share(q[:, rows], kb, vb, r, n, layout, causal, seqlens=lens)
                    if not np.allclose(o2, ref[:, rows], atol=1e-10, rtol=0):
                        return False
                    seq = np.repeat(np.arange(4), lens)
                    want = sum(1 for t in rows for u in range(24)
                               if seq[u] == seq[t] and (u <= t or not causal))
                    if orc.visible_pairs_closed_form(layout, causal, n, r, 8, seqlens=lens) != want:
                        return False
        # the page's literal (no max subtraction) form on its worked example size
        q, k, v = _rand(0, 1, 32, 1, 1, 16)
        kb, vb = _blocks_from_global(k, "contiguous", 4), _blocks_from_global(v, "contiguous", 4)
        lit = np.concatenate([orc.ring_share_literal(q[:, 8 * i:8 * i + 8], kb, vb, i, 4)
                              for i in range(4)], axis=1)
        if not np.allclose(lit, _sdpa64(q, k, v, False), atol=1e-10, rtol=0):
            return False
        # merge: empty partial is the identity, and a scaled copy merges exactly
        rng = np.random.default_rng(0)
        m = rng.standard_normal((1, 3, 2))
        l = rng.uniform(1, 2, (1, 3, 2))
        acc = rng.standard_normal((1, 3, 2, 4))
        x = (m, l, acc)
        y = (m - 1.0, l, acc)
        mm, ll, aa = orc.merge_partials(x, y)
        if not (np.allclose(mm, m) and np.allclose(ll, l * (1 + math.exp(-1.0)))
                and np.allclose(aa, acc * (1 + math.exp(-1.0)))):
            return False
        e = orc.empty_partial(1, 3, 2, 4)
        mm, ll, aa = orc.merge_partials(e, x)
        if not (np.array_equal(mm, m) and np.array_equal(ll, l) and np.array_equal(aa, acc)):
            return False
        return True
    except (ValueError, IndexError, FloatingPointError):
        return False


def test_unmutated_oracle_passes_battery():
    assert _pins_hold()


def _mut_kv_head(h, hq, hkv):
    return h % hkv


def _mut_scale(d):
    return 1.0 / d


def _mut_positions_striped(layout, n_ring, block, block_len):
    a = np.arange(block_len, dtype=np.int64)
    if layout == "contiguous":
        return block * block_len + a
    return block * block_len + a  # striped treated as contiguous


def _mut_positions_contiguous_off_by_one(layout, n_ring, block, block_len):
    a = np.arange(block_len, dtype=np.int64)
    if layout == "contiguous":
        return block * (block_len - 1) + a  # blocks overlap by one position
    return a * n_ring + block


def _mut_zigzag_late_chunk(layout, n_ring, block, block_len):
    if layout != "zigzag":
        return _orig_positions(layout, n_ring, block, block_len)
    a = np.arange(block_len, dtype=np.int64)
    h = block_len // 2
    chunk = np.where(a < h, block, 2 * n_ring - block)  # should be 2N-1-block
    return chunk * h + (a % h)


def _mut_zigzag_halves_swapped(layout, n_ring, block, block_len):
    if layout != "zigzag":
        return _orig_positions(layout, n_ring, block, block_len)
    a = np.arange(block_len, dtype=np.int64)
    h = block_len // 2
    chunk = np.where(a < h, 2 * n_ring - 1 - block, block)
    return chunk * h + (a % h)


def _mut_varlen_packed_positions(layout, n_ring, block, seqlens):
    # positions taken over the packed block as if it were one sequence
    ids, _ = _orig_varlen(layout, n_ring, block, seqlens)
    total = sum(int(L) for L in seqlens) // n_ring
    return ids, orc.global_positions(layout, n_ring, block, total)


_orig_positions = orc.global_positions
_orig_varlen = orc.varlen_positions
_orig_merge = orc.merge_partials
_orig_block_partial = orc.block_partial
_orig_visibility = orc._visibility
_orig_finalize = orc.finalize
_orig_literal = orc.ring_share_literal
_orig_closed = orc.visible_pairs_closed_form


def _mut_merge_no_rescale(p1, p2):
    m1, l1, a1 = p1
    m2, l2, a2 = p2
    return np.maximum(m1, m2), l1 + l2, a1 + a2


def _mut_merge_wrong_sign(p1, p2):
    m1, l1, a1 = p1
    m2, l2, a2 = p2
    m = np.maximum(m1, m2)
    f1 = np.where(np.isfinite(m1), np.exp(np.where(np.isfinite(m1), m - m1, 0.0)), 0.0)
    f2 = np.where(np.isfinite(m2), np.exp(np.where(np.isfinite(m2), m - m2, 0.0)), 0.0)
    return m, f1 * l1 + f2 * l2, f1[..., None] * a1 + f2[..., None] * a2


def _mut_merge_acc_unscaled(p1, p2):
    m, l, _ = _orig_merge(p1, p2)
    return m, l, p1[2] + p2[2]


def _mut_visibility_strict(q_pos, k_pos, causal, q_seq=None, k_seq=None):
    vis = _orig_visibility(q_pos, k_pos, causal, q_seq, k_seq)
    if causal:
        vis = vis & (k_pos[None, :] != q_pos[:, None])
    return vis


def _mut_visibility_transposed(q_pos, k_pos, causal, q_seq=None, k_seq=None):
    if not causal:
        return _orig_visibility(q_pos, k_pos, causal, q_seq, k_seq)
    return _orig_visibility(k_pos, q_pos, causal).T & _orig_visibility(q_pos, k_pos, False, q_seq, k_seq)


def _mut_visibility_ignores_sequences(q_pos, k_pos, causal, q_seq=None, k_seq=None):
    return _orig_visibility(q_pos, k_pos, causal)


def _mut_block_partial_transposed_v(q, q_pos, k, v, k_pos, causal, scale=None, q_seq=None, k_seq=None):
    m, l, acc = _orig_block_partial(q, q_pos, k, v, k_pos, causal, scale, q_seq, k_seq)
    return m, l, acc[:, ::-1]


def _mut_finalize_no_divide(state):
    m, l, acc = state
    return acc, m + np.log(np.where(l > 0, l, 1.0))


def _mut_literal_no_scale(q_share, k_blocks, v_blocks, rank, n_ring, scale=None):
    return _orig_literal(q_share, k_blocks, v_blocks, rank, n_ring, scale=1.0)


def _mut_closed_form(layout, causal, n_ring, rank, block_len, seqlens=None):
    if causal and layout == "striped" and seqlens is None:
        return n_ring * block_len * (block_len - 1) // 2 + rank * block_len
    return _orig_closed(layout, causal, n_ring, rank, block_len, seqlens)


def _mut_zigzag_closed_form(layout, causal, n_ring, rank, block_len, seqlens=None):
    if causal and layout == "zigzag" and seqlens is None:
        return (n_ring - 1) * block_len * block_len // 2 + block_len * (block_len - 1) // 2
    return _orig_closed(layout, causal, n_ring, rank, block_len, seqlens)


def _mut_ring_order(rank, n_ring):
    return [(rank + s) % n_ring for s in range(n_ring - 1)]  # drops the last block


MUTANTS = {
    "gqa_head_map": ("kv_head_of", _mut_kv_head),
    "scale_1_over_d": ("default_scale", _mut_scale),
    "striped_positions": ("global_positions", _mut_positions_striped),
    "contiguous_off_by_one": ("global_positions", _mut_positions_contiguous_off_by_one),
    "merge_no_rescale": ("merge_partials", _mut_merge_no_rescale),
    "merge_wrong_sign": ("merge_partials", _mut_merge_wrong_sign),
    "merge_acc_unscaled": ("merge_partials", _mut_merge_acc_unscaled),
    "causal_excludes_self": ("_visibility", _mut_visibility_strict),
    "causal_mask_transposed": ("_visibility", _mut_visibility_transposed),
    "acc_rows_permuted": ("block_partial", _mut_block_partial_transposed_v),
    "finalize_no_divide": ("finalize", _mut_finalize_no_divide),
    "literal_no_scale": ("ring_share_literal", _mut_literal_no_scale),
    "striped_pair_count": ("visible_pairs_closed_form", _mut_closed_form),
    "ring_order_drops_block": ("ring_order", _mut_ring_order),
    "zigzag_late_chunk_index": ("global_positions", _mut_zigzag_late_chunk),
    "zigzag_halves_swapped": ("global_positions", _mut_zigzag_halves_swapped),
    "zigzag_pair_count": ("visible_pairs_closed_form", _mut_zigzag_closed_form),
    "varlen_crosses_sequences": ("_visibility", _mut_visibility_ignores_sequences),
    "varlen_packed_positions": ("varlen_positions", _mut_varlen_packed_positions),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    with np.errstate(all="ignore"):
        assert not _pins_hold(), f"mutant {name} survived the pins"


# ---------------------------------------------------------------- backward --
from tests.test_oracle_backward import _torch_grads  # noqa: E402

_orig_block_grad = orc.block_grad
_orig_naive_grad = orc.naive_attention_grad


def _bwd_pins_hold() -> bool:
    try:
        n, blen = 3, 4
        q, k, v = _rand(21, 1, n * blen, 4, 2, 8)
        q = 2.0 * q
        dout = np.random.default_rng(4).standard_normal(q.shape)
        for layout in ("contiguous", "striped", "zigzag"):
            for causal in (False, True):
                out, lse = orc.naive_attention(q, k, v, causal)
                tq, tk, tv, _ = _torch_grads(q, k, v, dout, causal)
                dq0, dk0, dv0 = orc.naive_attention_grad(q, k, v, dout, causal)
                if not (np.allclose(dq0, tq, atol=1e-10) and np.allclose(dk0, tk, atol=1e-10)
                        and np.allclose(dv0, tv, atol=1e-10)):
                    return False
                kb, vb = _blocks_from_global(k, layout, n), _blocks_from_global(v, layout, n)
                dk_glob, dv_glob = np.zeros(k.shape), np.zeros(v.shape)
                for r in range(n):
                    rows = _share_rows(layout, n, r, blen)
                    dq, dk, dv = orc.ring_share_grad(q[:, rows], kb, vb, out[:, rows],
                                                     dout[:, rows], lse[:, rows], r, n, layout,
                                                     causal)
                    if not np.allclose(dq, tq[:, rows], atol=1e-10):
                        return False
                    for j in range(n):
                        keys = _share_rows(layout, n, j, blen)
                        dk_glob[:, keys] += dk[j]
                        dv_glob[:, keys] += dv[j]
                if not (np.allclose(dk_glob, tk, atol=1e-10) and np.allclose(dv_glob, tv, atol=1e-10)):
                    return False
        return True
    except (ValueError, IndexError, FloatingPointError):
        return False


def test_unmutated_backward_passes_battery():
    assert _bwd_pins_hold()


def _mut_bg_no_delta(q, q_pos, k, v, k_pos, dout, lse, delta, causal, scale=None, q_seq=None, k_seq=None):
    return _orig_block_grad(q, q_pos, k, v, k_pos, dout, lse, np.zeros_like(delta), causal, scale,
                            q_seq, k_seq)


def _mut_bg_dk_unscaled(q, q_pos, k, v, k_pos, dout, lse, delta, causal, scale=None, q_seq=None, k_seq=None):
    dq, dk, dv = _orig_block_grad(q, q_pos, k, v, k_pos, dout, lse, delta, causal, scale, q_seq, k_seq)
    s = orc.default_scale(q.shape[-1]) if scale is None else scale
    return dq, dk / s, dv


def _mut_bg_local_softmax(q, q_pos, k, v, k_pos, dout, lse, delta, causal, scale=None, q_seq=None, k_seq=None):
    # renormalises P over the visiting block instead of using the saved lse
    m, l, _ = orc.block_partial(q, q_pos, k, v, k_pos, causal, scale, q_seq, k_seq)
    local = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return _orig_block_grad(q, q_pos, k, v, k_pos, dout, local, delta, causal, scale, q_seq, k_seq)


def _mut_delta_wrong_operand(out, dout):
    return (np.asarray(dout, np.float64) ** 2).sum(axis=-1)


def _mut_naive_grad_dq_unscaled(q, k, v, dout, causal, scale=None, cu_seqlens=None):
    dq, dk, dv = _orig_naive_grad(q, k, v, dout, causal, scale, cu_seqlens)
    s = orc.default_scale(np.asarray(q).shape[-1]) if scale is None else scale
    return dq / s, dk, dv


def _mut_ring_grad_wrong_block(q_share, k_blocks, v_blocks, out, dout, lse, rank, n_ring, layout,
                               causal, scale=None, order=None, seqlens=None):
    dq, dk, dv = _orig_ring_grad(q_share, k_blocks, v_blocks, out, dout, lse, rank, n_ring, layout,
                                 causal, scale, order, seqlens)
    return dq, np.roll(dk, 1, axis=0), dv


_orig_ring_grad = orc.ring_share_grad

BWD_MUTANTS = {
    "grad_without_delta": ("block_grad", _mut_bg_no_delta),
    "grad_dk_unscaled": ("block_grad", _mut_bg_dk_unscaled),
    "grad_block_local_softmax": ("block_grad", _mut_bg_local_softmax),
    "grad_delta_wrong_operand": ("grad_delta", _mut_delta_wrong_operand),
    "naive_grad_dq_unscaled": ("naive_attention_grad", _mut_naive_grad_dq_unscaled),
    "ring_grad_wrong_block": ("ring_share_grad", _mut_ring_grad_wrong_block),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_pins_catch_mutant(name, monkeypatch):
    attr, fn = BWD_MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    with np.errstate(all="ignore"):
        assert not _bwd_pins_hold(), f"mutant {name} survived the pins"


# ---------------------------------------------------------------- rope ------
from tests.test_oracle_rope import _rope_complex  # noqa: E402

_orig_rope = orc.rope_rotate
_orig_angles = orc.rope_angles
_orig_ring_rope = orc.ring_share_rope


def _rope_pins_hold() -> bool:
    try:
        x = np.array([1.0, 0.0, 0.0, 1.0]).reshape(1, 1, 1, 4)
        want = [math.cos(3), math.sin(3), -math.sin(0.3), math.cos(0.3)]
        if not np.allclose(orc.rope_rotate(x, [3], base=100.0).reshape(-1), want, atol=1e-12):
            return False
        xr, _, _ = _rand(1, 1, 5, 2, 1, 16)
        pos = np.array([0, 3, 77, 4096, 99999])
        if not np.allclose(orc.rope_rotate(xr, pos), _rope_complex(xr, pos, 10000.0), atol=1e-10):
            return False
        n, blen = 3, 4
        q, k, v = _rand(6, 1, n * blen, 2, 1, 16)
        gp = np.arange(n * blen)
        ref = _sdpa64(_rope_complex(q, gp, 10000.0), _rope_complex(k, gp, 10000.0), v, True)
        for layout in ("contiguous", "striped", "zigzag"):
            kb, vb = _blocks_from_global(k, layout, n), _blocks_from_global(v, layout, n)
            for r in range(n):
                rows = _share_rows(layout, n, r, blen)
                out, _ = orc.ring_share_rope(q[:, rows], kb, vb, r, n, layout, True)
                if not np.allclose(out, ref[:, rows], atol=1e-10):
                    return False
        return True
    except (ValueError, IndexError, FloatingPointError):
        return False


def test_unmutated_rope_passes_battery():
    assert _rope_pins_hold()


def _mut_rope_half_split(x, pos, base=10000.0, inverse=False):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    inv = np.argsort(perm)
    return _orig_rope(x[..., inv], pos, base, inverse)[..., perm]


def _mut_rope_clockwise(x, pos, base=10000.0, inverse=False):
    return _orig_rope(x, pos, base, not inverse)


def _mut_rope_angles_exponent(pos, head_dim, base=10000.0):
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.asarray(pos, dtype=np.float64)[:, None] * (base ** (-i / head_dim))[None, :]


def _mut_ring_rope_local_positions(q_share, k_blocks, v_blocks, rank, n_ring, layout, causal,
                                   base=10000.0, scale=None, seqlens=None):
    lq = q_share.shape[1]
    qr = _orig_rope(q_share, np.arange(lq), base)
    kr = np.stack([_orig_rope(k_blocks[j], np.arange(k_blocks.shape[2]), base)
                   for j in range(n_ring)])
    return orc.ring_share(qr, kr, v_blocks, rank, n_ring, layout, causal, scale, seqlens=seqlens)


ROPE_MUTANTS = {
    "rope_half_split_pairs": ("rope_rotate", _mut_rope_half_split),
    "rope_clockwise": ("rope_rotate", _mut_rope_clockwise),
    "rope_frequency_exponent": ("rope_angles", _mut_rope_angles_exponent),
    "rope_local_positions": ("ring_share_rope", _mut_ring_rope_local_positions),
}


@pytest.mark.parametrize("name", sorted(ROPE_MUTANTS))
def test_rope_pins_catch_mutant(name, monkeypatch):
    attr, fn = ROPE_MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    with np.errstate(all="ignore"):
        assert not _rope_pins_hold(), f"mutant {name} survived the pins"
