"""ra_block_attn_accumulate: one ring step's running update in one kernel.

Block j's partial merged into a running state in place must equal the
state merged with ra_block_attn_partial's partial by ra_merge_partials (the
same merge arithmetic; float32 rounding of the fused multiply-adds may
differ), and the oracle's merge of its own partials; a block with no visible
pair leaves the state bit for bit unchanged. bf16 (8- and 4-wave
workgroups) and fp32 kernels, packed sequences, ragged tails.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import ring_oracle as orc
from ring_attention_blockwise_ra_amd import binding as B
from ring_attention_blockwise_ra_amd import synth
from ring_attention_blockwise_ra_amd.layout import blocks_from_global, share_tokens

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("both_forward_shapes")]
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


def _np64(t):
    return t.detach().double().cpu().numpy()


@pytest.mark.parametrize("dtype,d,blen,hq,hkv,layout,r", [
    ("bf16", 128, 300, 8, 2, "striped", 3),
    ("bf16", 64, 257, 4, 4, "contiguous", 2),
    ("bf16", 32, 96, 8, 1, "zigzag", 1),
    ("f32", 128, 100, 4, 2, "contiguous", 3),
])
def test_accumulate_equals_partial_then_merge(dtype, d, blen, hq, hkv, layout, r):
    n = 4
    say(f"accumulate: {dtype} d={d} blen={blen} {layout} r={r}")
    qg, kg, vg = synth.random_global(41, 1, n * blen, hq, hkv, d, dtype=dtype, device=DEV)
    rows = share_tokens(layout, n, r, blen)
    q = qg[:, rows.to(DEV)].contiguous()
    kb, vb = blocks_from_global(kg, layout, n), blocks_from_global(vg, layout, n)
    kw = dict(n_ring=n, rank=r, causal=True, layout=layout)
    # running state: the share's own block, then block j merged in
    for j in [x for x in range(n) if x != r]:
        m0, l0, a0 = B.ra_block_attn_partial(q, kb[r], vb[r], r, **kw)
        p = B.ra_block_attn_partial(q, kb[j], vb[j], j, **kw)
        ref = B.ra_merge_partials(m0, l0, a0, *p)
        m, l, a = m0.clone(), l0.clone(), a0.clone()
        B.ra_block_attn_accumulate(q, kb[j], vb[j], j, m=m, l=l, acc=a, **kw)
        torch.cuda.synchronize()
        assert torch.equal(torch.isinf(m), torch.isinf(ref[0]))
        fin = torch.isfinite(ref[0])
        assert torch.equal(m[fin], ref[0][fin]), j          # max: no rounding
        np.testing.assert_allclose(_np64(l), _np64(ref[1]), rtol=2e-7, atol=0)
        np.testing.assert_allclose(_np64(a), _np64(ref[2]), rtol=0, atol=2e-6 * float(ref[2].abs().max()))
        # against the oracle's merge of its own partials of the same rows
        q64 = _np64(q)
        o0 = orc.block_partial(q64, rows.numpy(), _np64(kb[r]), _np64(vb[r]),
                               orc.global_positions(layout, n, r, blen), True)
        o1 = orc.block_partial(q64, rows.numpy(), _np64(kb[j]), _np64(vb[j]),
                               orc.global_positions(layout, n, j, blen), True)
        om, ol, oa = orc.merge_partials(o0, o1)
        tol = 2e-2 if dtype == "bf16" else 1e-5
        fo = np.isfinite(om)
        assert np.array_equal(np.isfinite(_np64(m)), fo)
        np.testing.assert_allclose(_np64(m)[fo], om[fo], atol=1e-4)
        ok = ol > 0
        np.testing.assert_allclose((_np64(a)[ok] / _np64(l)[ok][:, None]),
                                   oa[ok] / ol[ok][:, None], atol=tol)


def test_invisible_block_leaves_the_state_unchanged():
    n, blen, hq, hkv, d, r = 4, 128, 4, 2, 64, 1
    say("accumulate: invisible block")
    qg, kg, vg = synth.random_global(42, 1, n * blen, hq, hkv, d, dtype="bf16", device=DEV)
    q = qg[:, share_tokens("contiguous", n, r, blen).to(DEV)].contiguous()
    kb, vb = blocks_from_global(kg, "contiguous", n), blocks_from_global(vg, "contiguous", n)
    kw = dict(n_ring=n, rank=r, causal=True, layout="contiguous")
    m, l, a = B.ra_block_attn_partial(q, kb[r], vb[r], r, **kw)
    m1, l1, a1 = m.clone(), l.clone(), a.clone()
    B.ra_block_attn_accumulate(q, kb[3], vb[3], 3, m=m, l=l, acc=a, **kw)  # future block
    torch.cuda.synchronize()
    assert torch.equal(m, m1) and torch.equal(l, l1) and torch.equal(a, a1)


@pytest.mark.parametrize("layout,r", [("contiguous", 0), ("contiguous", 3), ("striped", 2)])
def test_ring_final_divide_without_lse_and_against_finalize(layout, r):
    """The ring's last computed launch divides in its epilogue: with lse not
    requested the output is the same bits; and it equals the per-block
    entry points followed by ra_finalize (the separate divide kernel), the
    same arithmetic. Contiguous rank 0 computes only its own block, so there
    the first launch is also the last."""
    n, blen, hq, hkv, d = 4, 160, 8, 2, 64
    say(f"final divide: {layout} r={r}")
    qg, kg, vg = synth.random_global(43, 1, n * blen, hq, hkv, d, dtype="bf16", device=DEV)
    q = qg[:, share_tokens(layout, n, r, blen).to(DEV)].contiguous()
    kb, vb = blocks_from_global(kg, layout, n), blocks_from_global(vg, layout, n)
    kw = dict(n_ring=n, rank=r, causal=True, layout=layout)
    out, lse = B.ra_ring_fwd(q, kb, vb, **kw)
    out2, lse2 = B.ra_ring_fwd(q, kb, vb, want_lse=False, **kw)
    m, l, a = B.ra_block_attn_partial(q, kb[r], vb[r], r, **kw)
    for s in range(1, n):
        j = (r - s) % n
        B.ra_block_attn_accumulate(q, kb[j], vb[j], j, m=m, l=l, acc=a, **kw)
    o3, lse3 = B.ra_finalize(m, l, a)
    torch.cuda.synchronize()
    assert lse2 is None
    assert torch.equal(out, out2)
    assert torch.equal(out, o3) and torch.equal(lse, lse3)
