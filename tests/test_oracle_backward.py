"""Pins of the oracle's backward pass ([TS] "Blockwise Backward").

Expected values come from torch autograd in float64 (through SDPA, or an
explicit masked softmax for packed sequences), central finite differences of
the pinned forward oracle, and closed forms (the columns of dV add up to the
summed upstream gradient; the rows of dS, hence the columns of dK, add up to
zero). None comes from the oracle's backward itself.
"""

import itertools

import numpy as np
import pytest
import torch

from oracle import ring_oracle as orc
from tests.test_oracle_pins import _blocks_from_global, _rand, _share_rows
from tests.test_oracle_zigzag_varlen import _packed_mask, _packed_rows

LAYOUTS3 = ("contiguous", "striped", "zigzag")


def _torch_grads(q, k, v, dout, causal=False, mask=None, scale=None):
    """float64 autograd of SDPA on [B, S, H, d] arrays (KV heads repeated for
    grouped queries; the repeat's backward sums the group)."""
    hq, hkv = q.shape[2], k.shape[2]
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kk = tk.permute(0, 2, 1, 3).repeat_interleave(hq // hkv, 1)
    vv = tv.permute(0, 2, 1, 3).repeat_interleave(hq // hkv, 1)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(0, 2, 1, 3), kk, vv, is_causal=causal and mask is None,
        attn_mask=None if mask is None else torch.from_numpy(mask), scale=scale)
    o.permute(0, 2, 1, 3).backward(torch.tensor(dout))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(), o.permute(0, 2, 1, 3).detach().numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(1, 1), (4, 2), (6, 3)])
def test_naive_grad_vs_autograd(causal, heads):
    hq, hkv = heads
    q, k, v = _rand(3 + hq, 2, 11, hq, hkv, 8)
    dout = np.random.default_rng(9).standard_normal(q.shape)
    q = 2.0 * q
    dq, dk, dv = orc.naive_attention_grad(q, k, v, dout, causal)
    tq, tk, tv, _ = _torch_grads(q, k, v, dout, causal)
    np.testing.assert_allclose(dq, tq, atol=1e-12, rtol=0)
    np.testing.assert_allclose(dk, tk, atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, tv, atol=1e-12, rtol=0)


def test_naive_grad_custom_scale_and_packed():
    cu = [0, 4, 4, 9, 16]
    q, k, v = _rand(4, 1, 16, 4, 2, 8)
    dout = np.random.default_rng(1).standard_normal(q.shape)
    for causal in (False, True):
        dq, dk, dv = orc.naive_attention_grad(q, k, v, dout, causal, scale=0.3, cu_seqlens=cu)
        tq, tk, tv, _ = _torch_grads(q, k, v, dout, mask=_packed_mask(cu, causal), scale=0.3)
        np.testing.assert_allclose(dq, tq, atol=1e-12, rtol=0)
        np.testing.assert_allclose(dk, tk, atol=1e-12, rtol=0)
        np.testing.assert_allclose(dv, tv, atol=1e-12, rtol=0)


def test_naive_grad_finite_differences():
    """Central differences of L = sum(dO * O1(q, k, v)) with the forward oracle."""
    q, k, v = _rand(12, 1, 5, 2, 1, 3)
    dout = np.random.default_rng(2).standard_normal(q.shape)
    dq, dk, dv = orc.naive_attention_grad(q, k, v, dout, True)
    eps = 1e-6

    def loss(qq, kk, vv):
        return float((orc.naive_attention(qq, kk, vv, True)[0] * dout).sum())

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in itertools.islice(np.ndindex(x.shape), 0, None, 3):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-7, (name, idx, fd, g[idx])


def test_grad_closed_forms():
    """Per KV head: the keys' dV add up to the upstream gradients of the
    group's queries (rows of P add to 1); the keys' dK add up to 0 (rows of dS
    add to 0)."""
    q, k, v = _rand(5, 1, 9, 4, 2, 8)
    dout = np.random.default_rng(3).standard_normal(q.shape)
    for causal in (False, True):
        dq, dk, dv = orc.naive_attention_grad(q, k, v, dout, causal)
        for g in range(2):
            np.testing.assert_allclose(dv[0, :, g].sum(axis=0), dout[0, :, 2 * g:2 * g + 2].sum(axis=(0, 1)),
                                       atol=1e-12)
            np.testing.assert_allclose(dk[0, :, g].sum(axis=0), 0.0, atol=1e-12)
    # constant keys: every row's scores are equal, so dS = 0 and dQ = 0
    kc = np.broadcast_to(np.linspace(-1, 1, 8), k.shape).copy()
    dq, _, _ = orc.naive_attention_grad(q, kc, v, dout, True)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)


@pytest.mark.parametrize("layout", LAYOUTS3)
@pytest.mark.parametrize("causal", [False, True])
def test_ring_grad_sums_to_naive(layout, causal):
    n, blen = 3, 4
    q, k, v = _rand(21, 2, n * blen, 4, 2, 8)
    q = 2.0 * q
    dout = np.random.default_rng(4).standard_normal(q.shape)
    out, lse = orc.naive_attention(q, k, v, causal)
    tq, tk, tv, _ = _torch_grads(q, k, v, dout, causal)
    kb, vb = _blocks_from_global(k, layout, n), _blocks_from_global(v, layout, n)
    dk_glob, dv_glob = np.zeros(k.shape), np.zeros(v.shape)
    for r in range(n):
        rows = _share_rows(layout, n, r, blen)
        dq, dk, dv = orc.ring_share_grad(q[:, rows], kb, vb, out[:, rows], dout[:, rows],
                                         lse[:, rows], r, n, layout, causal)
        np.testing.assert_allclose(dq, tq[:, rows], atol=1e-12, rtol=0)
        for j in range(n):
            keys = _share_rows(layout, n, j, blen)
            dk_glob[:, keys] += dk[j]
            dv_glob[:, keys] += dv[j]
        # arrival order does not matter
        perm = list(np.random.default_rng(r).permutation(n))
        dq2, dk2, _ = orc.ring_share_grad(q[:, rows], kb, vb, out[:, rows], dout[:, rows],
                                          lse[:, rows], r, n, layout, causal, order=perm)
        np.testing.assert_allclose(dq2, dq, atol=1e-13, rtol=0)
        np.testing.assert_allclose(dk2, dk, atol=1e-13, rtol=0)
    np.testing.assert_allclose(dk_glob, tk, atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv_glob, tv, atol=1e-12, rtol=0)


def test_ring_grad_packed():
    n, lens = 3, [6, 0, 12, 18]
    cu = [0, 6, 6, 18, 36]
    q, k, v = _rand(8, 1, 36, 2, 1, 8)
    dout = np.random.default_rng(6).standard_normal(q.shape)
    for layout in LAYOUTS3:
        out, lse = orc.naive_attention_varlen(q, k, v, cu, True)
        tq, tk, tv, _ = _torch_grads(q, k, v, dout, mask=_packed_mask(cu, True))
        kb = np.stack([k[:, _packed_rows(layout, n, j, cu)] for j in range(n)])
        vb = np.stack([v[:, _packed_rows(layout, n, j, cu)] for j in range(n)])
        dk_glob, dv_glob = np.zeros(k.shape), np.zeros(v.shape)
        for r in range(n):
            rows = _packed_rows(layout, n, r, cu)
            dq, dk, dv = orc.ring_share_grad(q[:, rows], kb, vb, out[:, rows], dout[:, rows],
                                             lse[:, rows], r, n, layout, True, seqlens=lens)
            np.testing.assert_allclose(dq, tq[:, rows], atol=1e-12, rtol=0)
            for j in range(n):
                keys = _packed_rows(layout, n, j, cu)
                dk_glob[:, keys] += dk[j]
                dv_glob[:, keys] += dv[j]
        np.testing.assert_allclose(dk_glob, tk, atol=1e-12, rtol=0)
        np.testing.assert_allclose(dv_glob, tv, atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_grad_rows_match_whole_gradient(causal):
    q, k, v = _rand(31, 2, 13, 4, 2, 8)
    dout = np.random.default_rng(5).standard_normal(q.shape)
    tq, _, _, _ = _torch_grads(q, k, v, dout, causal)
    rows = np.array([0, 3, 7, 12])
    got = orc.naive_grad_rows(q[:, rows], rows, k, v, dout[:, rows], causal)
    np.testing.assert_allclose(got, tq[:, rows], atol=1e-12, rtol=0)
    np.testing.assert_allclose(got, orc.naive_attention_grad(q, k, v, dout, causal)[0][:, rows],
                               atol=1e-13, rtol=0)
