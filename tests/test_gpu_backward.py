"""GPU parity of the blockwise backward pass (troisinh "Blockwise Backward")
through the C ABI, against the CPU oracle.

Tolerance: the gradients are compared by max-abs error relative to the
reference's largest magnitude (floored at 1): 1e-2 for bfloat16 inputs (the
kernels round P and dS to bfloat16 before the value- and key-side products,
each a relative 2^-9, accumulated in float32) and 1e-5 for float32 inputs.
At the 1M-token share, dq is compared on sampled rows, each computed by the
oracle from that row's visible keys alone, and dk, dv through properties that
hold at any size (the keys' dV add up to the group's upstream gradients; the
keys' dK add up to zero up to the rounding of dS).
"""

import math
import sys

import numpy as np
import pytest
import torch

from oracle import ring_oracle as orc
from ring_attention_blockwise_ra_amd import binding as B
from ring_attention_blockwise_ra_amd import synth, workloads
from ring_attention_blockwise_ra_amd.layout import (blocks_from_global, packed_blocks_from_global,
                                                    packed_share_tokens, share_tokens)

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("side_stream_always")]
TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2}
DEV = "cuda"


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
    torch.cuda.empty_cache()


def _np64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def _dt(dtype):
    return "bf16" if dtype == torch.bfloat16 else "f32"


def _rel_err(got, ref):
    return float(np.abs(got - ref).max(initial=0.0)) / max(1.0, float(np.abs(ref).max(initial=0.0)))


def _dout(seed, shape, dtype):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype).to(DEV)


def test_delta_kernel():
    say("backward: delta = rowsum(dO * O)")
    for dtype in (torch.bfloat16, torch.float32):
        for d in (16, 32, 64, 128):
            g = torch.Generator().manual_seed(d)
            out = torch.randn(2, 37, 3, d, generator=g).to(DEV)
            dout = torch.randn(2, 37, 3, d, generator=g).to(dtype).to(DEV)
            delta = B.ra_attn_bwd_delta(out, dout)
            torch.cuda.synchronize()
            ref = orc.grad_delta(_np64(out), _np64(dout))
            assert np.abs(_np64(delta) - ref).max() <= 1e-4 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("dtype,d,hq,hkv,blen,n,layout,causal", [
    (torch.bfloat16, 128, 4, 2, 200, 3, "contiguous", True),
    (torch.bfloat16, 128, 8, 2, 256, 2, "striped", True),
    (torch.bfloat16, 128, 4, 1, 130, 3, "zigzag", True),
    (torch.bfloat16, 64, 2, 2, 97, 2, "contiguous", False),
    (torch.bfloat16, 32, 3, 1, 70, 4, "striped", True),
    (torch.bfloat16, 16, 2, 2, 66, 3, "zigzag", True),
    (torch.bfloat16, 128, 6, 1, 150, 2, "contiguous", False),
    (torch.bfloat16, 64, 8, 1, 120, 2, "striped", True),
    (torch.float32, 128, 4, 2, 90, 3, "contiguous", True),
    (torch.float32, 64, 2, 1, 64, 2, "zigzag", True),
    (torch.float32, 16, 1, 1, 33, 3, "striped", False),
])
def test_block_bwd_matches_oracle(dtype, d, hq, hkv, blen, n, layout, causal):
    say(f"block bwd: {dtype} d={d} hq={hq} hkv={hkv} B={blen} N={n} {layout} causal={causal}")
    qg, kg, vg = synth.random_global(31 + blen, 1, n * blen, hq, hkv, d, dtype=_dt(dtype), device=DEV)
    kb, vb = blocks_from_global(kg, layout, n), blocks_from_global(vg, layout, n)
    ref_out, ref_lse = orc.naive_attention(_np64(qg), _np64(kg), _np64(vg), causal)
    for r in range(n):
        rows = share_tokens(layout, n, r, blen)
        q = qg[:, rows.to(DEV)].contiguous()
        dout = _dout(100 + r, q.shape, dtype)
        # the oracle's forward statistics of this share, as float32 inputs
        lse = torch.from_numpy(ref_lse[:, rows.numpy()]).float().to(DEV)
        delta = torch.from_numpy(orc.grad_delta(ref_out[:, rows.numpy()], _np64(dout))).float().to(DEV)
        for j in range(n):
            dq, dk, dv = B.ra_block_attn_bwd(q, kb[j], vb[j], dout, lse, delta, j, n_ring=n, rank=r,
                                             causal=causal, layout=layout)
            torch.cuda.synchronize()
            rq, rk, rv = orc.block_grad(_np64(q), rows.numpy(), _np64(kb[j]), _np64(vb[j]),
                                        orc.global_positions(layout, n, j, blen), _np64(dout),
                                        _np64(lse), _np64(delta), causal)
            for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
                e = _rel_err(_np64(got), ref)
                assert e <= TOL[dtype], (name, r, j, e)


@pytest.mark.parametrize("dtype,layout,causal,heads,d", [
    (torch.bfloat16, "contiguous", True, (8, 2), 128),
    (torch.bfloat16, "striped", True, (4, 4), 64),
    (torch.bfloat16, "zigzag", True, (8, 2), 128),
    (torch.bfloat16, "contiguous", False, (4, 2), 128),
    (torch.float32, "zigzag", True, (4, 2), 32),
])
def test_ring_bwd_all_ranks_matches_plain_gradient(dtype, layout, causal, heads, d):
    say(f"ring bwd: {dtype} {layout} causal={causal} heads={heads} d={d}")
    hq, hkv = heads
    n, blen = 4, 96
    qg, kg, vg = synth.random_global(41, 2, n * blen, hq, hkv, d, dtype=_dt(dtype), device=DEV)
    dout_g = _dout(7, qg.shape, dtype)
    rq, rk, rv = orc.naive_attention_grad(_np64(qg), _np64(kg), _np64(vg), _np64(dout_g), causal)
    kb, vb = blocks_from_global(kg, layout, n), blocks_from_global(vg, layout, n)
    dk = torch.zeros(kb.shape, dtype=torch.float32, device=DEV)
    dv = torch.zeros(vb.shape, dtype=torch.float32, device=DEV)
    for r in range(n):
        rows = share_tokens(layout, n, r, blen).to(DEV)
        q = qg[:, rows].contiguous()
        dout = dout_g[:, rows].contiguous()
        out, lse = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=causal, layout=layout, rank=r)
        dq, _, _ = B.ra_ring_bwd(q, kb, vb, out, dout, lse, n_ring=n, causal=causal, layout=layout,
                                 rank=r, dk=dk, dv=dv)
        torch.cuda.synchronize()
        e = _rel_err(_np64(dq), rq[:, rows.cpu().numpy()])
        assert e <= TOL[dtype], ("dq", r, e)
    for j in range(n):
        keys = share_tokens(layout, n, j, blen).numpy()
        assert _rel_err(_np64(dk[j]), rk[:, keys]) <= TOL[dtype], ("dk", j)
        assert _rel_err(_np64(dv[j]), rv[:, keys]) <= TOL[dtype], ("dv", j)


@pytest.mark.parametrize("layout", ["zigzag", "contiguous"])
def test_ring_bwd_packed(layout):
    say(f"ring bwd: packed sequences, {layout}")
    n, lens = 3, [240, 0, 18, 420, 6]
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    qg, kg, vg = synth.random_global(43, 1, cu[-1], 4, 2, 128, dtype="bf16", device=DEV)
    dout_g = _dout(8, qg.shape, torch.bfloat16)
    rq, rk, rv = orc.naive_attention_grad(_np64(qg), _np64(kg), _np64(vg), _np64(dout_g), True,
                                          cu_seqlens=cu)
    kb = packed_blocks_from_global(kg, layout, n, cu)
    vb = packed_blocks_from_global(vg, layout, n, cu)
    dk = torch.zeros(kb.shape, dtype=torch.float32, device=DEV)
    dv = torch.zeros(vb.shape, dtype=torch.float32, device=DEV)
    for r in range(n):
        rows = packed_share_tokens(layout, n, r, cu).to(DEV)
        q = qg[:, rows].contiguous()
        dout = dout_g[:, rows].contiguous()
        out, lse = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=True, layout=layout, rank=r, cu_seqlens=cu)
        dq, _, _ = B.ra_ring_bwd(q, kb, vb, out, dout, lse, n_ring=n, causal=True, layout=layout,
                                 rank=r, dk=dk, dv=dv, cu_seqlens=cu)
        torch.cuda.synchronize()
        assert _rel_err(_np64(dq), rq[:, rows.cpu().numpy()]) <= 1e-2, r
    for j in range(n):
        keys = packed_share_tokens(layout, n, j, cu).numpy()
        assert _rel_err(_np64(dk[j]), rk[:, keys]) <= 1e-2, ("dk", j)
        assert _rel_err(_np64(dv[j]), rv[:, keys]) <= 1e-2, ("dv", j)


def test_ring_bwd_order_and_split_invariance():
    """The ring's dq equals block addends summed in any order (block entry
    point, fresh zero accumulators), within tolerance."""
    say("ring bwd: arrival order")
    n, blen, hq, hkv, d = 4, 128, 4, 2, 128
    qg, kg, vg = synth.random_global(47, 1, n * blen, hq, hkv, d, dtype="bf16", device=DEV)
    kb, vb = blocks_from_global(kg, "striped", n), blocks_from_global(vg, "striped", n)
    r = 2
    q = qg[:, share_tokens("striped", n, r, blen).to(DEV)].contiguous()
    dout = _dout(9, q.shape, torch.bfloat16)
    out, lse = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=True, layout="striped", rank=r)
    dq, dk, dv = B.ra_ring_bwd(q, kb, vb, out, dout, lse, n_ring=n, causal=True, layout="striped", rank=r)
    delta = B.ra_attn_bwd_delta(out, dout)
    for order in ([3, 1, 0, 2], [0, 1, 2, 3]):
        dq2 = torch.zeros_like(dq)
        for j in order:
            _, dkj, dvj = B.ra_block_attn_bwd(q, kb[j], vb[j], dout, lse, delta, j, n_ring=n, rank=r,
                                              causal=True, layout="striped", dq=dq2)
            torch.cuda.synchronize()
            assert (dkj - dk[j]).abs().max().item() <= 1e-6 * max(1.0, dk[j].abs().max().item())
            assert (dvj - dv[j]).abs().max().item() <= 1e-6 * max(1.0, dv[j].abs().max().item())
        assert (dq2 - dq).abs().max().item() <= 1e-5 * max(1.0, dq.abs().max().item())


def test_bwd_fully_masked_and_empty():
    say("ring bwd: fully masked blocks and empty shares")
    n, blen, hq, d = 4, 64, 2, 64
    qg, kg, vg = synth.random_global(5, 1, n * blen, hq, hq, d, dtype="bf16", device=DEV)
    kb, vb = blocks_from_global(kg, "contiguous", n), blocks_from_global(vg, "contiguous", n)
    q = qg[:, :blen].contiguous()
    dout = _dout(3, q.shape, torch.bfloat16)
    out, lse = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=True, rank=0)
    dq, dk, dv = B.ra_ring_bwd(q, kb, vb, out, dout, lse, n_ring=n, causal=True, rank=0)
    torch.cuda.synchronize()
    # rank 0 sees only its own block: blocks 1..3 get no addend
    assert torch.all(dk[1:] == 0) and torch.all(dv[1:] == 0)
    assert torch.isfinite(dq).all() and dk[0].abs().sum() > 0
    qe = torch.zeros(1, 0, 2, 64, dtype=torch.bfloat16, device=DEV)
    ke = torch.zeros(2, 1, 0, 2, 64, dtype=torch.bfloat16, device=DEV)
    oe = torch.zeros(1, 0, 2, 64, dtype=torch.float32, device=DEV)
    le = torch.zeros(1, 0, 2, dtype=torch.float32, device=DEV)
    B.ra_ring_bwd(qe, ke, ke, oe, qe, le, n_ring=2, causal=True, rank=1)
    torch.cuda.synchronize()


# --------------------------------------------------------------- full size --
@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
def test_c4_backward_rank7(layout):
    say(f"c4 backward: causal {layout}, 1,048,576 tokens, GQA 32/8, rank 7")
    w = workloads.prepare("c4", layout, 7, device=DEV, keep_global=True)
    q, k, v = w["q"], w["k"], w["v"]
    dout = _dout(77, q.shape, torch.bfloat16)
    out, lse = B.ra_ring_fwd(q, k, v, n_ring=8, causal=True, layout=layout, rank=7)
    dq, dk, dv = B.ra_ring_bwd(q, k, v, out, dout, lse, n_ring=8, causal=True, layout=layout, rank=7)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    # dq on sampled rows, each from the oracle with that row's visible keys
    rows = workloads.sample_rows(w["cfg"]["block"], 12, seed=81)
    tok = w["q_tokens"][rows].numpy()
    kmax = int(tok.max()) + 1
    say("c4", layout, "oracle dq for", len(rows), "rows over", kmax, "keys")
    ref = orc.naive_grad_rows(_np64(q[:, rows.to(DEV)]), tok, _np64(w["k_global"][:, :kmax]),
                              _np64(w["v_global"][:, :kmax]), _np64(dout[:, rows.to(DEV)]), True)
    worst = _rel_err(_np64(dq[:, rows.to(DEV)]), ref)
    say("c4", layout, "dq sampled rel err", worst)
    assert worst <= 1e-2
    hq, hkv = 32, 8
    # dv: for every KV head and dim, the keys' addends add up to the group's
    # upstream gradient over the share's rows (rows of P sum to 1; bf16 P
    # moves each row's sum by at most 2^-9)
    sv = dv.double().sum(dim=(0, 1, 2))                      # [hkv, d]
    do64 = dout.double().reshape(1, -1, hkv, hq // hkv, 128)
    want = do64.sum(dim=(0, 1, 3))                           # [hkv, d]
    bound = do64.abs().sum(dim=(0, 1, 3)) * 2.0 ** -9 + 1e-3
    assert torch.all((sv - want).abs() <= bound), (sv - want).abs().max().item()
    # dk: rows of dS sum to zero, so the keys' dK add up to zero up to the
    # bf16 rounding of dS: |sum_k dK| <= scale 2^-9 sum_rows |q| sum_k |dS|,
    # with sum_k |dS| <= 2 max_k |dP| <= 2 |dO| max |v|
    sk = dk.double().sum(dim=(0, 1, 2))
    vmax = v.abs().max().double()
    qn = q.double().abs().reshape(1, -1, hkv, hq // hkv, 128)
    don = dout.double().norm(dim=-1).reshape(1, -1, hkv, hq // hkv, 1)
    vn = v.double().norm(dim=-1).max()
    bound_k = (qn * don).sum(dim=(0, 1, 3)) * 2 * vn / math.sqrt(128) * 2.0 ** -9 + 1e-3
    assert torch.all(sk.abs() <= bound_k), (sk.abs() / bound_k).max().item()
    say("c4", layout, "dv / dk sums within", (sv - want).abs().max().item(), sk.abs().max().item())
    del vmax
