"""Score dynamics that stress the online softmax: scores that rise along the
key axis (the running maximum moves by more than the lazy-rescale threshold
many times per row, so every rescale path runs), scores that fall (the
maximum is met at once and everything after it decays towards underflow),
and large-magnitude random inputs (nearly one-hot rows). The HIP path,
through the C ABI, against the fp64 oracle: 1e-2 for bfloat16 inputs as in
the other parity tests; for float32 inputs 1e-5 plus the error that float32
scores of this magnitude carry by themselves (see _f32_bounds)."""

import sys

import numpy as np
import pytest
import torch

from oracle import ring_oracle as orc
from ring_attention_blockwise_ra_amd import binding as B
from ring_attention_blockwise_ra_amd import synth
from ring_attention_blockwise_ra_amd.layout import blocks_from_global, share_tokens

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("side_stream_always", "both_forward_shapes")]
DEV = "cuda"
TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2}
# lse = m + ln l: with bfloat16 inputs l sums weights rounded to bfloat16 (at
# most 2^-9 relative each), so ln l can be off by ~2e-3; float32 keeps the
# weights exact
LSE_TOL = {"f32": 1e-5, "bf16": 5e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def _np64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def _ramp(seed, seq, hq, hkv, d, slope, rising, dtype):
    """Global q, k, v: key t carries slope * t/seq (rising) or slope * (1 - t/seq)
    in dimension 0, every query 6 there, plus N(0, 0.1) noise elsewhere; the
    scaled score of key t then moves by about 6 * slope / sqrt(d) over the
    sequence (slope 120, d 128: ~64 nats, ~92 in log2 units)."""
    g = torch.Generator().manual_seed(seed)
    q = 0.1 * torch.randn(1, seq, hq, d, generator=g)
    k = 0.1 * torch.randn(1, seq, hkv, d, generator=g)
    v = torch.randn(1, seq, hkv, d, generator=g)
    pos = torch.arange(seq, dtype=torch.float32) / seq
    q[..., 0] = 6.0
    k[..., 0] = (slope * (pos if rising else 1.0 - pos))[None, :, None]
    dt = synth.torch_dtype(dtype)
    return tuple(t.to(dt).to(DEV) for t in (q, k, v))


def _f32_bounds(q, k, v):
    """(output bound, lse bound) for float32 inputs: 1e-5 plus the part of the
    error these inputs force. A score s carries a rounding of about 2^-24 |s|;
    every weight exp(s - m) inherits it as a relative error, so the output
    moves by up to that times |v| and lse = m + ln l by up to that; taken as
    4 * 2^-24 * max|s| (* max|v| for the output), scores in fp64 on the host."""
    qd, kd = q.double().cpu(), k.double().cpu()
    g = qd.shape[2] // kd.shape[2]
    kd = kd.repeat_interleave(g, dim=2)
    s_max = float((torch.einsum("bqhd,bkhd->bhqk", qd, kd) / np.sqrt(q.shape[-1])).abs().max())
    e = 4 * 2.0 ** -24 * s_max
    return TOL[torch.float32] + e * float(v.double().abs().max()), LSE_TOL["f32"] + e


def _ring_err(q, k, v, n, layout, causal, dtype):
    seq = q.shape[1]
    blen = seq // n
    ref, ref_lse = orc.naive_attention(_np64(q), _np64(k), _np64(v), causal)
    kb, vb = blocks_from_global(k, layout, n), blocks_from_global(v, layout, n)
    worst = worst_lse = 0.0
    for r in range(n):
        rows = share_tokens(layout, n, r, blen)
        out, lse = B.ra_ring_fwd(q[:, rows.to(DEV)].contiguous(), kb, vb, n_ring=n, causal=causal,
                                 layout=layout, rank=r)
        torch.cuda.synchronize()
        o = _np64(out)
        assert np.isfinite(o).all()
        worst = max(worst, np.abs(o - ref[:, rows.numpy()]).max())
        worst_lse = max(worst_lse, np.abs(_np64(lse) - ref_lse[:, rows.numpy()]).max())
    return worst, worst_lse


@pytest.mark.parametrize("dtype,layout,causal,rising", [
    ("bf16", "contiguous", True, True),
    ("bf16", "striped", True, True),
    ("bf16", "zigzag", True, True),
    ("bf16", "contiguous", False, True),
    ("bf16", "contiguous", True, False),
    ("bf16", "striped", False, False),
    ("f32", "contiguous", True, True),
    ("f32", "striped", False, False),
])
def test_ring_with_moving_maximum(dtype, layout, causal, rising):
    n, blen, hq, hkv, d = 4, 256, 4, 2, 128
    say(f"ramp: {dtype} {layout} causal={causal} rising={rising}")
    q, k, v = _ramp(5, n * blen, hq, hkv, d, 120.0, rising, dtype)
    err, err_lse = _ring_err(q, k, v, n, layout, causal, dtype)
    tol, tol_lse = _f32_bounds(q, k, v) if dtype == "f32" else (TOL[torch.bfloat16], LSE_TOL["bf16"])
    assert err <= tol, (err, tol)
    assert err_lse <= tol_lse, (err_lse, tol_lse)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_partial_max_is_exact_under_a_rising_ramp(dtype):
    """m of a partial is the row's exact maximum scaled score even when the
    kernel's reference moved many times on the way there; l and acc follow."""
    n, blen, hq, hkv, d = 2, 512, 4, 1, 128
    say(f"ramp partial: {dtype}")
    q, k, v = _ramp(9, n * blen, hq, hkv, d, 160.0, True, dtype)
    kb, vb = blocks_from_global(k, "contiguous", n), blocks_from_global(v, "contiguous", n)
    # scores reach ~85 nats: float32 bound from _f32_bounds, bfloat16 1e-2
    bound = _f32_bounds(q, k, v)[0] if dtype == "f32" else TOL[torch.bfloat16]
    for r in range(n):
        rows = share_tokens("contiguous", n, r, blen)
        qs = q[:, rows.to(DEV)].contiguous()
        for j in range(n):
            m, l, acc = B.ra_block_attn_partial(qs, kb[j], vb[j], j, n_ring=n, rank=r, causal=False)
            torch.cuda.synchronize()
            rm, rl, racc = orc.block_partial(_np64(qs), rows.numpy(), _np64(kb[j]), _np64(vb[j]),
                                             orc.global_positions("contiguous", n, j, blen), False)
            gm, gl, gacc = _np64(m), _np64(l), _np64(acc)
            assert np.abs(gm - rm).max() <= 1e-5 * max(1.0, np.abs(rm).max())
            assert np.abs(gl / rl - 1).max() <= (1e-4 if dtype == "f32" else 4e-3)
            ref_o = racc / rl[..., None]
            assert np.abs(gacc / gl[..., None] - ref_o).max() <= bound


@pytest.mark.parametrize("dtype,layout", [("bf16", "striped"), ("bf16", "contiguous"), ("f32", "contiguous")])
def test_ring_large_magnitude_scores(dtype, layout):
    """q, k ~ N(0, 4^2): scaled scores with a standard deviation of ~16 nats,
    rows nearly one-hot."""
    n, blen, hq, hkv, d = 4, 192, 8, 2, 128
    say(f"large scores: {dtype} {layout}")
    q, k, v = synth.random_global(21, 1, n * blen, hq, hkv, d, dtype=dtype, device=DEV)
    q = (q.float() * 4).to(q.dtype)
    k = (k.float() * 4).to(k.dtype)
    err, err_lse = _ring_err(q, k, v, n, layout, True, dtype)
    tol, tol_lse = _f32_bounds(q, k, v) if dtype == "f32" else (TOL[torch.bfloat16], LSE_TOL["bf16"])
    assert err <= tol, (err, tol)
    assert err_lse <= tol_lse, (err_lse, tol_lse)


def _term_scales(q, k, v, dout, causal):
    """Magnitude of the summed terms of each gradient, |dS| |k| scale for dq,
    |dS|^T |q| scale for dk, P^T |dout| for dv (fp64, plain softmax): under a
    score ramp dS sums to zero against keys that share a large component, so
    the gradients are small differences of large terms, and rounding P and dS
    to bfloat16 (2^-9 each) errs relative to the terms, not to the result."""
    q, k, v, dout = (_np64(t)[0] for t in (q, k, v, dout))
    seq, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d)
    vis = np.tril(np.ones((seq, seq), dtype=bool)) if causal else np.ones((seq, seq), dtype=bool)
    tq, tk, tv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for h in range(hq):
        g = h * hkv // hq
        s_ = np.where(vis, q[:, h] @ k[:, g].T * scale, -np.inf)
        p = np.exp(s_ - s_.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o = p @ v[:, g]
        ds = p * (dout[:, h] @ v[:, g].T - (dout[:, h] * o).sum(axis=1, keepdims=True))
        tq[:, h] = scale * np.abs(ds) @ np.abs(k[:, g])
        tk[:, g] += scale * np.abs(ds).T @ np.abs(q[:, h])
        tv[:, g] += p.T @ np.abs(dout[:, h])
    return tq[None], tk[None], tv[None]


def _excess(got, ref, terms, tol, rel):
    """Largest error beyond the elementwise bound tol * max(1, max|ref|) +
    rel * terms (<= 0 when every element is inside it)."""
    bound = tol * max(1.0, float(np.abs(ref).max(initial=0.0))) + rel * terms
    return float((np.abs(got - ref) - bound).max(initial=-1.0))


@pytest.mark.parametrize("dtype,layout,rising", [
    ("bf16", "contiguous", True),
    ("bf16", "striped", True),
    ("bf16", "zigzag", False),
    ("f32", "contiguous", True),
])
def test_ring_backward_with_moving_maximum(dtype, layout, rising):
    """Forward and backward of every rank under a score ramp (causal): dq per
    rank, dk and dv summed over the ranks, against the plain gradient, element
    by element within tol * max(1, max|ref|) + rel * (that element's summed
    terms, _term_scales): tol 1e-2 and rel 2^-8 for bfloat16 (P and dS are
    rounded to bfloat16, 2^-9 each); tol 1e-5 and rel 4 * 2^-24 * max|s| for
    float32 (the scores' own rounding, carried by every weight)."""
    n, blen, hq, hkv, d = 4, 128, 4, 2, 128
    say(f"ramp backward: {dtype} {layout} rising={rising}")
    q, k, v = _ramp(13, n * blen, hq, hkv, d, 120.0, rising, dtype)
    g = torch.Generator().manual_seed(3)
    dout_g = torch.randn(q.shape, generator=g).to(q.dtype).to(DEV)
    rq, rk, rv = orc.naive_attention_grad(_np64(q), _np64(k), _np64(v), _np64(dout_g), True)
    sq, sk, sv = _term_scales(q, k, v, dout_g, True)
    if dtype == "f32":
        tol, rel = TOL[torch.float32], _f32_bounds(q, k, v)[1] - LSE_TOL["f32"]
    else:
        tol, rel = TOL[torch.bfloat16], 2.0 ** -8
    kb, vb = blocks_from_global(k, layout, n), blocks_from_global(v, layout, n)
    dk = torch.zeros(kb.shape, dtype=torch.float32, device=DEV)
    dv = torch.zeros(vb.shape, dtype=torch.float32, device=DEV)
    for r in range(n):
        rows = share_tokens(layout, n, r, blen).to(DEV)
        qs, dout = q[:, rows].contiguous(), dout_g[:, rows].contiguous()
        out, lse = B.ra_ring_fwd(qs, kb, vb, n_ring=n, causal=True, layout=layout, rank=r)
        dq, _, _ = B.ra_ring_bwd(qs, kb, vb, out, dout, lse, n_ring=n, causal=True, layout=layout,
                                 rank=r, dk=dk, dv=dv)
        torch.cuda.synchronize()
        idx = rows.cpu().numpy()
        x = _excess(_np64(dq), rq[:, idx], sq[:, idx], tol, rel)
        assert x <= 0, ("dq", r, x)
    for j in range(n):
        keys = share_tokens(layout, n, j, blen).numpy()
        x_k = _excess(_np64(dk[j]), rk[:, keys], sk[:, keys], tol, rel)
        x_v = _excess(_np64(dv[j]), rv[:, keys], sv[:, keys], tol, rel)
        assert x_k <= 0, ("dk", j, x_k)
        assert x_v <= 0, ("dv", j, x_v)
