"""The running partial as a checkpoint of the ring.

The running state (m, l, acc) after ring steps 0..k-1 is a complete
checkpoint: merged with the state of steps k..N-1 it gives the full ring's
result, because the online-softmax merge is associative ([TS] "Tai sao no
hoat dong"). Built here from the library's own block partials and merges
(two merge trees that differ from the ring's left fold, so equality holds to
float32 rounding), for several split points k, and compared with
ra_ring_fwd of the same share.
"""

import sys

import pytest
import torch

from ring_attention_blockwise_ra_amd import binding as B
from ring_attention_blockwise_ra_amd import synth
from ring_attention_blockwise_ra_amd.layout import blocks_from_global, share_tokens

pytestmark = pytest.mark.gpu
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


@pytest.mark.parametrize("layout,r", [("striped", 6), ("contiguous", 5), ("zigzag", 2)])
def test_state_after_k_steps_merged_with_the_rest_equals_the_ring(layout, r):
    n, blen, hq, hkv, d = 8, 256, 8, 2, 128
    say(f"checkpoint: {layout} rank {r}")
    qg, kg, vg = synth.random_global(31, 1, n * blen, hq, hkv, d, dtype="bf16", device=DEV)
    q = qg[:, share_tokens(layout, n, r, blen).to(DEV)].contiguous()
    kb, vb = blocks_from_global(kg, layout, n), blocks_from_global(vg, layout, n)
    kw = dict(n_ring=n, rank=r, causal=True, layout=layout)
    ref, ref_lse = B.ra_ring_fwd(q, kb, vb, **kw)

    def state(steps):
        st = None
        for s in steps:
            j = (r - s) % n
            part = B.ra_block_attn_partial(q, kb[j], vb[j], j, **kw)
            st = part if st is None else B.ra_merge_partials(*st, *part)
        return st

    for k in (1, 3, 7):
        m, l, acc = B.ra_merge_partials(*state(range(k)), *state(range(k, n)))
        out, lse = B.ra_finalize(m, l, acc)
        torch.cuda.synchronize()
        err = float((out - ref).abs().max())
        lerr = float((lse - ref_lse).abs().max())
        say(f"  k={k}: out {err:.2e} lse {lerr:.2e}")
        assert torch.isfinite(out).all()
        assert err <= 1e-5 and lerr <= 1e-5, (k, err, lerr)
