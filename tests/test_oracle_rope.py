"""Pins of the oracle's rotary position embedding ([TS] "RoPE va Position
Embedding": an arriving key block is rotated by m*theta for each token's own
position m). Expected values come from complex-number multiplication, a
hand-worked case, orthogonality, the relative-position property and plain
attention on globally rotated inputs (torch SDPA), never from the oracle's
own rotation."""

import math

import numpy as np
import pytest
import torch

from oracle import ring_oracle as orc
from tests.test_oracle_pins import _blocks_from_global, _rand, _sdpa64, _share_rows
from tests.test_oracle_zigzag_varlen import _masked_sdpa64, _packed_mask, _packed_rows


def _rope_complex(x, pos, base):
    """The same rotation as complex multiplication z * exp(i m theta_i)."""
    d = x.shape[-1]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    th = base ** (-np.arange(d // 2) * 2.0 / d)
    z = z * np.exp(1j * np.asarray(pos, float)[None, :, None, None] * th)
    y = np.empty(x.shape)
    y[..., 0::2], y[..., 1::2] = z.real, z.imag
    return y


def test_hand_worked_case():
    # d = 4, base 100: pair 0 turns by m, pair 1 by m / 10
    x = np.array([1.0, 0.0, 0.0, 1.0]).reshape(1, 1, 1, 4)
    y = orc.rope_rotate(x, [3], base=100.0)
    want = [math.cos(3), math.sin(3), -math.sin(0.3), math.cos(0.3)]
    np.testing.assert_allclose(y.reshape(-1), want, atol=1e-15)
    assert np.array_equal(orc.rope_rotate(x, [0], base=100.0), x)  # position 0: identity


def test_complex_form_orthogonality_inverse():
    x, _, _ = _rand(1, 2, 9, 3, 1, 16)
    pos = np.array([0, 1, 5, 100, 4095, 65537, 131071, 524288, 1048575])
    y = orc.rope_rotate(x, pos, 500000.0)
    np.testing.assert_allclose(y, _rope_complex(x, pos, 500000.0), atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(orc.rope_rotate(y, pos, 500000.0, inverse=True), x, atol=1e-12)


def test_relative_position_property():
    """<R(m) q, R(n) k> depends on m - n only."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 1, 32))
    k = rng.standard_normal((1, 1, 1, 32))
    for m, n in [(5, 2), (1000, 997), (777777, 777774)]:
        a = float((orc.rope_rotate(q, [m]) * orc.rope_rotate(k, [n])).sum())
        b = float((orc.rope_rotate(q, [3]) * orc.rope_rotate(k, [0])).sum())
        assert abs(a - b) < 1e-9


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("causal", [False, True])
def test_ring_rope_equals_rotated_plain_attention(layout, causal):
    n, blen = 3, 4
    q, k, v = _rand(6, 1, n * blen, 4, 2, 16)
    pos = np.arange(n * blen)
    ref = _sdpa64(_rope_complex(q, pos, 10000.0), _rope_complex(k, pos, 10000.0), v, causal)
    kb, vb = _blocks_from_global(k, layout, n), _blocks_from_global(v, layout, n)
    for r in range(n):
        rows = _share_rows(layout, n, r, blen)
        out, _ = orc.ring_share_rope(q[:, rows], kb, vb, r, n, layout, causal)
        np.testing.assert_allclose(out, ref[:, rows], atol=1e-12, rtol=0)


def test_ring_rope_packed_positions_restart_per_sequence():
    n, lens = 3, [6, 12, 6]
    cu = [0, 6, 18, 24]
    q, k, v = _rand(7, 1, 24, 2, 1, 8)
    pos = np.concatenate([np.arange(L) for L in lens])
    ref = _masked_sdpa64(_rope_complex(q, pos, 10000.0), _rope_complex(k, pos, 10000.0), v,
                         _packed_mask(cu, True))
    for layout in ("contiguous", "zigzag"):
        kb = np.stack([k[:, _packed_rows(layout, n, j, cu)] for j in range(n)])
        vb = np.stack([v[:, _packed_rows(layout, n, j, cu)] for j in range(n)])
        for r in range(n):
            rows = _packed_rows(layout, n, r, cu)
            out, _ = orc.ring_share_rope(q[:, rows], kb, vb, r, n, layout, True, seqlens=lens)
            np.testing.assert_allclose(out, ref[:, rows], atol=1e-12, rtol=0)
