"""GPU parity of the rotary position embedding applied on arrival (troisinh
"RoPE va Position Embedding") through the C ABI, against the CPU oracle.

The rotation kernel is compared with the oracle's float64 rotation at
positions up to 2^20 (its angle is reduced in float64): max-abs 2e-6 of the
input's scale for float32 output, and one bfloat16 rounding (2^-8 of the
scale) for bfloat16 output. Ring outputs use the usual 1e-2 / 1e-5 bars;
gradients the relative bar of the backward tests.
"""

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
THETA = 10000.0


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


def _rel_err(got, ref):
    return float(np.abs(got - ref).max(initial=0.0)) / max(1.0, float(np.abs(ref).max(initial=0.0)))


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_rope_kernel_large_positions(layout):
    say(f"rope kernel: {layout}, block 7 of 8 x 131072 tokens")
    n, blen, d = 8, 131072, 128
    prob = B.make_problem(dtype=torch.bfloat16, batch=1, hq=2, hkv=1, head_dim=d, q_len=blen,
                          kv_len=blen, n_ring=n, rank=7, causal=True, layout=layout,
                          rope_theta=500000.0)
    g = torch.Generator().manual_seed(3)
    x32 = torch.randn(1, blen, 1, d, generator=g).to(DEV)
    pos = orc.global_positions(layout, n, 6, blen)
    ref = orc.rope_rotate(_np64(x32), pos, 500000.0)
    y32 = B.ra_rope_apply(x32, prob, target="keys", block_j=6)
    torch.cuda.synchronize()
    assert np.abs(_np64(y32) - ref).max() <= 2e-6 * np.abs(ref).max()
    xb = x32.to(torch.bfloat16)
    refb = orc.rope_rotate(_np64(xb), pos, 500000.0)
    yb = B.ra_rope_apply(xb, prob, target="keys", block_j=6)
    torch.cuda.synchronize()
    assert np.abs(_np64(yb) - refb).max() <= 2.0 ** -8 * np.abs(refb).max()
    # inverse undoes, accumulate adds
    back = B.ra_rope_apply(y32, prob, target="keys", block_j=6, inverse=True)
    acc = torch.ones_like(x32)
    B.ra_rope_apply(x32, prob, target="keys", block_j=6, out=acc, accumulate=True)
    torch.cuda.synchronize()
    assert (back - x32).abs().max().item() <= 2e-6 * x32.abs().max().item()
    assert np.abs(_np64(acc) - (ref + 1.0)).max() <= 4e-6 * np.abs(ref).max()
    # queries use the share's own positions (rank 7)
    yq = B.ra_rope_apply(xb.repeat(1, 1, 2, 1).contiguous(), prob, target="queries")
    torch.cuda.synchronize()
    refq = orc.rope_rotate(_np64(xb.repeat(1, 1, 2, 1)), orc.global_positions(layout, n, 7, blen), 500000.0)
    assert np.abs(_np64(yq) - refq).max() <= 2.0 ** -8 * np.abs(refq).max()


@pytest.mark.parametrize("dtype,layout,causal", [
    (torch.bfloat16, "contiguous", True), (torch.bfloat16, "striped", True),
    (torch.bfloat16, "zigzag", True), (torch.bfloat16, "contiguous", False),
    (torch.float32, "zigzag", True),
])
def test_ring_fwd_rope(dtype, layout, causal):
    say(f"ring fwd rope: {dtype} {layout} causal={causal}")
    n, blen, hq, hkv, d = 4, 96, 8, 2, 128
    qg, kg, vg = synth.random_global(61, 2, n * blen, hq, hkv, d,
                                     dtype="bf16" if dtype == torch.bfloat16 else "f32", device=DEV)
    kb, vb = blocks_from_global(kg, layout, n), blocks_from_global(vg, layout, n)
    for r in range(n):
        rows = share_tokens(layout, n, r, blen)
        q = qg[:, rows.to(DEV)].contiguous()
        out, lse = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=causal, layout=layout, rank=r,
                                 rope_theta=THETA)
        torch.cuda.synchronize()
        ref, ref_lse = orc.ring_share_rope(_np64(q), _np64(kb), _np64(vb), r, n, layout, causal, THETA)
        assert np.abs(_np64(out) - ref).max() <= TOL[dtype], r


def test_ring_fwd_rope_packed():
    say("ring fwd rope: packed zigzag")
    n, lens = 3, [240, 0, 18, 420, 6]
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    qg, kg, vg = synth.random_global(62, 1, cu[-1], 4, 2, 128, dtype="bf16", device=DEV)
    kb = packed_blocks_from_global(kg, "zigzag", n, cu)
    vb = packed_blocks_from_global(vg, "zigzag", n, cu)
    for r in range(n):
        q = qg[:, packed_share_tokens("zigzag", n, r, cu).to(DEV)].contiguous()
        out, _ = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=True, layout="zigzag", rank=r,
                               cu_seqlens=cu, rope_theta=THETA)
        torch.cuda.synchronize()
        ref, _ = orc.ring_share_rope(_np64(q), _np64(kb), _np64(vb), r, n, "zigzag", True, THETA,
                                     seqlens=lens)
        assert np.abs(_np64(out) - ref).max() <= 1e-2, r


@pytest.mark.parametrize("dtype,layout", [(torch.bfloat16, "zigzag"), (torch.bfloat16, "contiguous"),
                                          (torch.float32, "striped")])
def test_ring_bwd_rope(dtype, layout):
    say(f"ring bwd rope: {dtype} {layout}")
    n, blen, hq, hkv, d = 4, 64, 4, 2, 64
    qg, kg, vg = synth.random_global(63, 1, n * blen, hq, hkv, d,
                                     dtype="bf16" if dtype == torch.bfloat16 else "f32", device=DEV)
    g = torch.Generator().manual_seed(5)
    dout_g = torch.randn(qg.shape, generator=g).to(dtype).to(DEV)
    pos = np.arange(n * blen)
    qr, kr = orc.rope_rotate(_np64(qg), pos, THETA), orc.rope_rotate(_np64(kg), pos, THETA)
    dqr, dkr, dv_ref = orc.naive_attention_grad(qr, kr, _np64(vg), _np64(dout_g), True)
    dq_ref = orc.rope_rotate(dqr, pos, THETA, inverse=True)
    dk_ref = orc.rope_rotate(dkr, pos, THETA, inverse=True)
    kb, vb = blocks_from_global(kg, layout, n), blocks_from_global(vg, layout, n)
    dk = torch.zeros(kb.shape, dtype=torch.float32, device=DEV)
    dv = torch.zeros(vb.shape, dtype=torch.float32, device=DEV)
    tol = TOL[dtype]
    for r in range(n):
        rows = share_tokens(layout, n, r, blen).to(DEV)
        q, dout = qg[:, rows].contiguous(), dout_g[:, rows].contiguous()
        out, lse = B.ra_ring_fwd(q, kb, vb, n_ring=n, causal=True, layout=layout, rank=r,
                                 rope_theta=THETA)
        dq, _, _ = B.ra_ring_bwd(q, kb, vb, out, dout, lse, n_ring=n, causal=True, layout=layout,
                                 rank=r, dk=dk, dv=dv, rope_theta=THETA)
        torch.cuda.synchronize()
        assert _rel_err(_np64(dq), dq_ref[:, rows.cpu().numpy()]) <= tol, ("dq", r)
    for j in range(n):
        keys = share_tokens(layout, n, j, blen).numpy()
        assert _rel_err(_np64(dk[j]), dk_ref[:, keys]) <= tol, ("dk", j)
        assert _rel_err(_np64(dv[j]), dv_ref[:, keys]) <= tol, ("dv", j)


def test_c4_rope_rank7_sampled():
    say("c4 rope: causal zigzag, 1,048,576 tokens, rank 7; 16 sampled rows")
    w = workloads.prepare("c4", "zigzag", 7, device=DEV, keep_global=True)
    out, _ = B.ra_ring_fwd(w["q"], w["k"], w["v"], n_ring=8, causal=True, layout="zigzag", rank=7,
                           rope_theta=500000.0)
    torch.cuda.synchronize()
    rows = workloads.sample_rows(w["cfg"]["block"], 16, seed=91, tile_edges=(128, 65536))
    tok = w["q_tokens"][rows].numpy()
    kmax = int(tok.max()) + 1
    qr = orc.rope_rotate(_np64(w["q"][:, rows.to(DEV)]), tok, 500000.0)
    kr = orc.rope_rotate(_np64(w["k_global"][:, :kmax]), np.arange(kmax), 500000.0)
    ref, _ = orc.naive_attention_rows(qr, tok, kr, _np64(w["v_global"][:, :kmax]), True)
    err = float(np.abs(_np64(out[:, rows.to(DEV)]) - ref).max())
    say("c4 rope max-abs", err)
    assert err <= 1e-2
