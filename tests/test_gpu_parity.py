"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Tolerances (max-abs on the float32 output): 1e-5 for float32 inputs and 1e-2
for bfloat16 inputs with float32 accumulation. Index and tile-class results
must match bit for bit. Inputs are seeded; the oracle receives the exact
input values the GPU read.
"""

import math
import sys

import numpy as np
import pytest
import torch

from oracle import ring_oracle as orc
from ring_attention_blockwise_ra_amd import binding as B
from ring_attention_blockwise_ra_amd import synth, workloads
from ring_attention_blockwise_ra_amd.layout import blocks_from_global, share_tokens

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("side_stream_always", "both_forward_shapes")]

TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2}
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()  # fail loudly if the library is missing
    yield
    torch.cuda.synchronize()


def _np64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def _rand_global(seed, bsz, seq, hq, hkv, d, dtype, scale=1.0):
    return synth.random_global(seed, bsz, seq, hq, hkv, d, dtype=dtype, device=DEV, scale=scale)


def _ring_vs_oracle(q_glob, k_glob, v_glob, n, layout, causal, ranks, dtype, scale=None, **kw):
    bsz, seq, hq, d = q_glob.shape
    blen = seq // n
    ref, _ = orc.naive_attention(_np64(q_glob), _np64(k_glob), _np64(v_glob), causal, scale)
    kb, vb = blocks_from_global(k_glob, layout, n), blocks_from_global(v_glob, layout, n)
    worst = 0.0
    for r in ranks:
        rows = share_tokens(layout, n, r, blen)
        q = q_glob[:, rows.to(DEV)].contiguous()
        out, lse = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=causal, layout=layout, rank=r,
                                 scale=scale, **kw)
        torch.cuda.synchronize()
        err = np.abs(_np64(out) - ref[:, rows.numpy()]).max() if out.numel() else 0.0
        worst = max(worst, err)
        assert np.isfinite(_np64(out)).all()
        assert err <= TOL[dtype], (layout, causal, r, err)
    return worst


# ---------------------------------------------------------------- c1 ---------
def test_c1_worked_example_fp32():
    """The Ultralytics four-device simulation through ra_ring_fwd, fp32."""
    say("c1: fp32 N=4 B=8 d=16 non-causal, ra_ring_fwd all ranks")
    q, k, v = (t.to(DEV) for t in synth.c1_qkv())
    err = _ring_vs_oracle(q, k, v, 4, "contiguous", False, range(4), torch.float32)
    full = torch.softmax(q[0, :, 0] @ k[0, :, 0].T / 4.0, dim=-1) @ v[0, :, 0]
    kb, vb = blocks_from_global(k, "contiguous", 4), blocks_from_global(v, "contiguous", 4)
    outs = [B.ra_ring_fwd(q[:, 8 * i:8 * i + 8].contiguous(), kb, vb, n_ring=4, causal=False,
                          rank=i)[0] for i in range(4)]
    ring = torch.cat(outs, dim=1)[0, :, 0]
    assert torch.allclose(ring, full, atol=1e-5)
    say("c1 max-abs vs oracle", err)


# ---------------------------------------------------------------- block partial
_PARTIAL_CASES = [
    # dtype, d, hq, hkv, blen, n, layout, causal
    (torch.bfloat16, 128, 4, 2, 200, 3, "contiguous", True),
    (torch.bfloat16, 128, 8, 2, 256, 2, "striped", True),
    (torch.bfloat16, 64, 2, 2, 130, 2, "contiguous", False),
    (torch.bfloat16, 32, 3, 1, 97, 4, "striped", True),
    (torch.bfloat16, 16, 1, 1, 70, 3, "contiguous", True),
    (torch.bfloat16, 128, 16, 2, 64, 2, "striped", False),
    (torch.float32, 128, 4, 2, 150, 3, "contiguous", True),
    (torch.float32, 64, 2, 1, 100, 2, "striped", True),
    (torch.float32, 32, 4, 4, 33, 3, "contiguous", False),
    (torch.float32, 16, 1, 1, 8, 4, "contiguous", False),
]


@pytest.mark.parametrize("dtype,d,hq,hkv,blen,n,layout,causal", _PARTIAL_CASES)
def test_block_partial_matches_oracle(dtype, d, hq, hkv, blen, n, layout, causal):
    say(f"partial: {dtype} d={d} hq={hq} hkv={hkv} B={blen} N={n} {layout} causal={causal}")
    qg, kg, vg = _rand_global(7 + d + blen, 2, n * blen, hq, hkv, d, "bf16" if dtype == torch.bfloat16 else "f32")
    kb, vb = blocks_from_global(kg, layout, n), blocks_from_global(vg, layout, n)
    tol = TOL[dtype]
    for r in range(n):
        rows = share_tokens(layout, n, r, blen)
        q = qg[:, rows.to(DEV)].contiguous()
        for j in range(n):
            m, l, acc = B.ra_block_attn_partial(q, kb[j], vb[j], j, n_ring=n, rank=r,
                                                causal=causal, layout=layout)
            torch.cuda.synchronize()
            rm, rl, racc = orc.block_partial(_np64(q), rows.numpy(), _np64(kb[j]), _np64(vb[j]),
                                             orc.global_positions(layout, n, j, blen), causal)
            gm, gl, gacc = _np64(m), _np64(l), _np64(acc)
            empty = ~np.isfinite(rm)
            assert np.array_equal(~np.isfinite(gm), empty), "empty rows differ"
            assert np.all(gm[empty] == -np.inf) and np.all(gl[empty] == 0)
            assert np.all(gacc[empty] == 0)
            ok = ~empty
            assert np.abs(gm[ok] - rm[ok]).max(initial=0) <= 1e-5 * np.maximum(1, np.abs(rm[ok])).max(initial=1)
            # bf16: l sums the bf16-rounded weights that also form acc (each weight
            # carries at most 2^-9 relative rounding), so l matches to ~4e-3 while
            # acc / l stays a convex combination of V with those same weights.
            l_tol = 1e-4 if dtype == torch.float32 else 4e-3
            assert np.abs(gl[ok] / rl[ok] - 1).max(initial=0) <= l_tol
            o_g = gacc[ok] / gl[ok][:, None]
            o_r = racc[ok] / rl[ok][:, None]
            assert np.abs(o_g - o_r).max(initial=0) <= tol


# ---------------------------------------------------------------- merge/finalize
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_merge_and_finalize_match_oracle(d):
    say(f"merge/finalize d={d}")
    g = torch.Generator().manual_seed(d)
    shape = (3, 37, 5)
    def part(empty_frac):
        m = torch.randn(shape, generator=g, dtype=torch.float64) * 4
        l = torch.rand(shape, generator=g, dtype=torch.float64) * 9 + 1
        acc = torch.randn(shape + (d,), generator=g, dtype=torch.float64)
        e = torch.rand(shape, generator=g) < empty_frac
        m[e], l[e], acc[e] = -math.inf, 0.0, 0.0
        return m, l, acc
    p1, p2 = part(0.2), part(0.3)
    t1 = [x.to(torch.float32).to(DEV) for x in p1]
    t2 = [x.to(torch.float32).to(DEV) for x in p2]
    m, l, acc = B.ra_merge_partials(*t1, *t2)
    ref = orc.merge_partials(tuple(_np64(x) for x in t1), tuple(_np64(x) for x in t2))
    np.testing.assert_array_equal(_np64(m), ref[0])
    np.testing.assert_allclose(_np64(l), ref[1], rtol=2e-6, atol=0)
    np.testing.assert_allclose(_np64(acc), ref[2], rtol=2e-6, atol=1e-6)
    # in place into input 1
    B.ra_merge_partials(*t1, *t2, out=tuple(t1))
    np.testing.assert_array_equal(_np64(t1[0]), ref[0])
    np.testing.assert_allclose(_np64(t1[2]), ref[2], rtol=2e-6, atol=1e-6)
    out, lse = B.ra_finalize(m, l, acc)
    ro, rlse = orc.finalize(ref)
    np.testing.assert_allclose(_np64(out), ro, rtol=2e-6, atol=1e-6)
    np.testing.assert_allclose(_np64(lse), rlse, rtol=2e-6, atol=1e-6)


# ---------------------------------------------------------------- ring, small
_RING_CASES = [
    ("bf16", 1, 4, 256, 32, 8, 128, "contiguous", True),
    ("bf16", 1, 4, 256, 32, 8, 128, "striped", True),
    ("bf16", 2, 3, 130, 4, 4, 64, "striped", True),
    ("bf16", 1, 2, 333, 6, 3, 32, "contiguous", True),
    ("bf16", 1, 1, 300, 2, 1, 128, "contiguous", True),
    ("bf16", 1, 5, 64, 2, 2, 16, "contiguous", False),
    ("f32", 1, 4, 96, 4, 2, 128, "striped", True),
    ("f32", 2, 3, 50, 2, 2, 64, "contiguous", True),
    ("f32", 1, 2, 40, 2, 1, 32, "contiguous", False),
]


@pytest.mark.parametrize("dt,bsz,n,blen,hq,hkv,d,layout,causal", _RING_CASES)
def test_ring_small_all_ranks(dt, bsz, n, blen, hq, hkv, d, layout, causal):
    say(f"ring: {dt} b={bsz} N={n} B={blen} hq={hq} hkv={hkv} d={d} {layout} causal={causal}")
    qg, kg, vg = _rand_global(100 + n * blen, bsz, n * blen, hq, hkv, d, dt)
    dtype = synth.torch_dtype(dt)
    _ring_vs_oracle(qg, kg, vg, n, layout, causal, range(n), dtype)
    # serial copies on the compute stream give the same answer
    _ring_vs_oracle(qg, kg, vg, n, layout, causal, [n - 1], dtype, copy_stream=None)


def test_ring_poisoned_workspace_and_delayed_copy_stream():
    """NaN-filled staging buffers and a copy stream held back by a spin: a
    missing copy->compute wait would read NaN."""
    say("ring: stream ordering with poisoned workspace")
    n, blen, hq, hkv, d = 4, 512, 8, 2, 128
    qg, kg, vg = _rand_global(5, 1, n * blen, hq, hkv, d, "bf16")
    kb, vb = blocks_from_global(kg, "striped", n), blocks_from_global(vg, "striped", n)
    r = 2
    q = qg[:, share_tokens("striped", n, r, blen).to(DEV)].contiguous()
    prob = B.make_problem(dtype=torch.bfloat16, batch=1, hq=hq, hkv=hkv, head_dim=d, q_len=blen,
                          kv_len=blen, n_ring=n, rank=r, causal=True, layout="striped")
    ws = torch.full((B.ra_ring_workspace_bytes(prob),), 0xFF, dtype=torch.uint8, device=DEV)
    side = B.side_stream(torch.device(DEV))
    ref, _ = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=True, layout="striped", rank=r,
                           copy_stream=None)
    torch.cuda.synchronize()
    for _ in range(3):
        ws.fill_(0xFF)
        if hasattr(torch.cuda, "_sleep"):
            with torch.cuda.stream(side):
                torch.cuda._sleep(2_000_000)
        out, _ = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=True, layout="striped", rank=r,
                               workspace=ws, copy_stream=side)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        assert torch.equal(out, ref)


def test_ring_on_a_side_compute_stream_keeps_its_own_workspace():
    """The ring runs on a compute stream that is not the current one, held
    back by a spin, with the workspace allocated inside the call. Buffers of
    the same size allocated and NaN-filled on the current stream right after
    the call must not land on that workspace while the ring still uses it."""
    say("ring: internal workspace on a non-current compute stream")
    n, blen, hq, hkv, d = 4, 512, 8, 2, 128
    qg, kg, vg = _rand_global(6, 1, n * blen, hq, hkv, d, "bf16")
    kb, vb = blocks_from_global(kg, "striped", n), blocks_from_global(vg, "striped", n)
    r = 3
    q = qg[:, share_tokens("striped", n, r, blen).to(DEV)].contiguous()
    prob = B.make_problem(dtype=torch.bfloat16, batch=1, hq=hq, hkv=hkv, head_dim=d, q_len=blen,
                          kv_len=blen, n_ring=n, rank=r, causal=True, layout="striped")
    need = B.ra_ring_workspace_bytes(prob)
    ref, _ = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=True, layout="striped", rank=r)
    torch.cuda.synchronize()
    cs = torch.cuda.Stream()
    for _ in range(3):
        cs.wait_stream(torch.cuda.current_stream())
        if hasattr(torch.cuda, "_sleep"):
            with torch.cuda.stream(cs):
                torch.cuda._sleep(2_000_000)
        out, _ = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=True, layout="striped", rank=r,
                               compute_stream=cs)
        junk = [torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device=DEV) for _ in range(2)]
        torch.cuda.synchronize()
        del junk
        assert torch.isfinite(out).all()
        assert torch.equal(out, ref)


def test_ring_bwd_on_a_side_compute_stream_after_held_back_zero_fills():
    """ra_ring_bwd on a compute stream that is not the current one, with dk
    and dv allocated and zero-filled by the binding on the current stream,
    which a spin holds back: the ring adds into dk, dv, so it must run after
    those fills. Every gradient must equal the current-stream result."""
    say("ring backward: zero fills on the held-back current stream, ring on a side stream")
    n, blen, hq, hkv, d = 4, 256, 8, 2, 128
    qg, kg, vg = _rand_global(8, 1, n * blen, hq, hkv, d, "bf16")
    kb, vb = blocks_from_global(kg, "striped", n), blocks_from_global(vg, "striped", n)
    r = 1
    q = qg[:, share_tokens("striped", n, r, blen).to(DEV)].contiguous()
    out, lse = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=True, layout="striped", rank=r)
    g = torch.Generator(device=DEV).manual_seed(3)
    dout = torch.randn(q.shape, generator=g, device=DEV).to(torch.bfloat16)
    ref = B.ra_ring_bwd(q, kb, vb, out, dout, lse, n_ring=n, causal=True, layout="striped", rank=r)
    torch.cuda.synchronize()
    assert float(ref[1].abs().max()) > 0 and float(ref[2].abs().max()) > 0
    cs = torch.cuda.Stream()
    for _ in range(3):
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(2_000_000)   # on the current stream, before the fills
        got = B.ra_ring_bwd(q, kb, vb, out, dout, lse, n_ring=n, causal=True, layout="striped",
                            rank=r, compute_stream=cs)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), name


# ---------------------------------------------------------------- invariants
def test_causal_row0_and_constant_keys_on_gpu():
    say("invariants: row 0 = V[0]; constant keys = mean of visible V")
    n, blen, hq, hkv, d = 4, 128, 4, 2, 64
    qg, kg, vg = _rand_global(9, 1, n * blen, hq, hkv, d, "bf16")
    for layout in ("contiguous", "striped"):
        kb, vb = blocks_from_global(kg, layout, n), blocks_from_global(vg, layout, n)
        q = qg[:, share_tokens(layout, n, 0, blen).to(DEV)].contiguous()
        out, _ = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=True, layout=layout, rank=0)
        torch.cuda.synchronize()
        for h in range(hq):
            assert torch.equal(out[0, 0, h], vg[0, 0, h // (hq // hkv)].float())
    kc = torch.zeros_like(kg)
    kc[..., 0] = 1.0
    kb, vb = blocks_from_global(kc, "contiguous", n), blocks_from_global(vg, "contiguous", n)
    for r in range(n):
        q = qg[:, r * blen:(r + 1) * blen].contiguous()
        out, _ = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=True, layout="contiguous", rank=r)
        torch.cuda.synchronize()
        cums = torch.cumsum(vg.double(), dim=1) / torch.arange(1, n * blen + 1, device=DEV).double()[None, :, None, None]
        want = cums[:, r * blen:(r + 1) * blen].repeat_interleave(hq // hkv, dim=2)
        assert (out.double() - want).abs().max().item() <= 1e-2


def test_arrival_order_and_split_ring_on_gpu():
    """Partials merged in any order (and a ring split in two) give the same
    output within tolerance."""
    say("invariants: arrival order / split ring via partial + merge")
    n, blen, hq, hkv, d = 5, 96, 4, 1, 128
    layout, r = "striped", 3
    qg, kg, vg = _rand_global(13, 1, n * blen, hq, hkv, d, "bf16")
    kb, vb = blocks_from_global(kg, layout, n), blocks_from_global(vg, layout, n)
    q = qg[:, share_tokens(layout, n, r, blen).to(DEV)].contiguous()
    ref, _ = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=True, layout=layout, rank=r)
    g = torch.Generator().manual_seed(0)
    for _ in range(3):
        order = torch.randperm(n, generator=g).tolist()
        state = None
        for j in order:
            p = B.ra_block_attn_partial(q, kb[j], vb[j], j, n_ring=n, rank=r, causal=True,
                                        layout=layout)
            state = p if state is None else B.ra_merge_partials(*state, *p)
        out, _ = B.ra_finalize(*state)
        torch.cuda.synchronize()
        assert (out - ref).abs().max().item() <= 1e-5


def test_fully_masked_block_partial_is_empty():
    say("edge: fully masked block partial")
    n, blen, hq, d = 4, 64, 2, 128
    qg, kg, vg = _rand_global(3, 1, n * blen, hq, hq, d, "bf16")
    kb, vb = blocks_from_global(kg, "contiguous", n), blocks_from_global(vg, "contiguous", n)
    q = qg[:, :blen].contiguous()
    m, l, acc = B.ra_block_attn_partial(q, kb[2], vb[2], 2, n_ring=n, rank=0, causal=True)
    torch.cuda.synchronize()
    assert torch.all(m == -math.inf) and torch.all(l == 0) and torch.all(acc == 0)
    # striped j > r: local row 0 sees nothing, other rows see keys < a
    kb, vb = blocks_from_global(kg, "striped", n), blocks_from_global(vg, "striped", n)
    q = qg[:, share_tokens("striped", n, 1, blen).to(DEV)].contiguous()
    m, l, acc = B.ra_block_attn_partial(q, kb[3], vb[3], 3, n_ring=n, rank=1, causal=True,
                                        layout="striped")
    torch.cuda.synchronize()
    assert torch.all(m[0, 0] == -math.inf) and torch.all(l[0, 0] == 0)
    assert torch.all(torch.isfinite(m[0, 1:]))


def test_empty_share_is_noop():
    say("edge: empty share")
    q = torch.zeros(1, 0, 2, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(2, 1, 0, 2, 64, dtype=torch.bfloat16, device=DEV)
    out, lse = B.ra_ring_fwd(q, k, k, n_ring=2, causal=True, rank=1)
    torch.cuda.synchronize()
    assert out.shape == (1, 0, 2, 64)


def test_noncausal_rows_without_keys():
    say("edge: kv_len = 0, non-causal")
    q = torch.randn(1, 5, 2, 32, device=DEV).to(torch.bfloat16)
    k = torch.zeros(3, 1, 0, 2, 32, dtype=torch.bfloat16, device=DEV)
    out, lse = B.ra_ring_fwd(q, k, k, n_ring=3, causal=False, rank=1)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(lse == -math.inf)


def test_tile_classes_device_match_host():
    say("scheduler: device vs host classes")
    for layout in ("contiguous", "striped"):
        for (n, blen, tq, tk) in [(8, 1000, 128, 64), (4, 77, 16, 8), (8, 131072, 128, 128),
                                  (3, 5, 1, 2)]:
            for r in (0, n // 2, n - 1):
                for j in range(n):
                    prob = B.make_problem(dtype=torch.bfloat16, batch=1, hq=1, hkv=1, head_dim=64,
                                          q_len=blen, kv_len=blen, n_ring=n, rank=r, causal=True,
                                          layout=layout)
                    dev = B.ra_tile_classes_device(prob, j, tq, tk).cpu().numpy()
                    host = B.ra_tile_classes_host(prob, j, tq, tk)
                    np.testing.assert_array_equal(dev, host)
                    if blen <= 1000:
                        want = orc.tile_classes_bruteforce(layout, True, n, r, j, blen, blen, tq, tk)
                        np.testing.assert_array_equal(host, want)  # same integer codes
                    else:  # the device form's class counts against the oracle's own counts
                        cnt = np.bincount(dev.ravel().astype(np.int64), minlength=3)
                        assert (int(cnt[B.RA_TILE_FULL]), int(cnt[B.RA_TILE_PARTIAL]),
                                int(cnt[B.RA_TILE_SKIP])) == \
                            orc.tile_class_counts(layout, True, n, r, j, blen, blen, tq, tk)


def test_invalid_head_dim_raises():
    q = torch.zeros(1, 8, 1, 48, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(2, 1, 8, 1, 48, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(B.RaError) as ei:
        B.ra_ring_fwd(q, k, k, n_ring=2, causal=True, rank=0)
    assert ei.value.status == B.RA_ERR_UNSUPPORTED
