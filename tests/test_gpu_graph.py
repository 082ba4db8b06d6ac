"""The ring entry points under HIP graph capture.

ra_ring_fwd and ra_ring_bwd enqueue only kernels, device-to-device copies and
cross-stream event waits (no memsets, no synchronous calls), and the staging
stream joins the caller's stream through an event recorded on it, so a
caller can capture a whole ring step in a graph and replay it; the launch
count of a small share then stops mattering. Each test captures once,
replays three times on fresh inputs with eager ring calls and
synchronisations in between, and requires every replay to equal the eager
result bit for bit (the same kernels run in the same order).
"""

import sys

import pytest
import torch

from ring_attention_blockwise_ra_amd import binding as B
from ring_attention_blockwise_ra_amd import synth
from ring_attention_blockwise_ra_amd.layout import blocks_from_global, share_tokens

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("side_stream_always")]
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


def _share(seed, n, blen, hq, hkv, d, layout):
    qg, kg, vg = synth.random_global(seed, 1, n * blen, hq, hkv, d, dtype="bf16", device=DEV)
    q = qg[:, share_tokens(layout, n, n - 1, blen).to(DEV)].contiguous()
    return q, blocks_from_global(kg, layout, n), blocks_from_global(vg, layout, n)


def _warm(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()


@pytest.mark.parametrize("layout,theta", [("striped", 0.0), ("zigzag", 10000.0)])
def test_ring_fwd_graph_replays_equal_eager(layout, theta):
    n, blen, hq, hkv, d = 8, 256, 8, 2, 128
    say(f"graph fwd: {layout} theta={theta}")
    qs, ks, vs = _share(1, n, blen, hq, hkv, d, layout)
    kw = dict(n_ring=n, causal=True, layout=layout, rank=n - 1, rope_theta=theta)
    _warm(lambda: B.ra_ring_fwd(qs, ks, vs, **kw))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out_g, lse_g = B.ra_ring_fwd(qs, ks, vs, **kw)
    for rep in range(3):
        q, k, v = _share(10 + rep, n, blen, hq, hkv, d, layout)
        qs.copy_(q)
        ks.copy_(k)
        vs.copy_(v)
        g.replay()
        torch.cuda.synchronize()
        out_e, lse_e = B.ra_ring_fwd(q, k, v, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), rep
        assert torch.equal(lse_g, lse_e), rep
    say("graph fwd ok")


def test_ring_bwd_graph_replays_equal_eager():
    n, blen, hq, hkv, d = 4, 192, 8, 2, 128
    layout = "zigzag"
    say("graph bwd")
    kw = dict(n_ring=n, causal=True, layout=layout, rank=n - 1)
    qs, ks, vs = _share(2, n, blen, hq, hkv, d, layout)
    dos = torch.randn(qs.shape, device=DEV).to(torch.bfloat16)
    outs, lses = B.ra_ring_fwd(qs, ks, vs, **kw)
    dks = torch.zeros(ks.shape, dtype=torch.float32, device=DEV)
    dvs = torch.zeros_like(dks)
    _warm(lambda: B.ra_ring_bwd(qs, ks, vs, outs, dos, lses, dk=dks, dv=dvs, **kw))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dq_g, _, _ = B.ra_ring_bwd(qs, ks, vs, outs, dos, lses, dk=dks, dv=dvs, **kw)
    for rep in range(3):
        q, k, v = _share(20 + rep, n, blen, hq, hkv, d, layout)
        do = torch.randn(q.shape, device=DEV).to(torch.bfloat16)
        out, lse = B.ra_ring_fwd(q, k, v, **kw)
        for dst, src in ((qs, q), (ks, k), (vs, v), (dos, do), (outs, out), (lses, lse)):
            dst.copy_(src)
        dks.zero_()
        dvs.zero_()
        g.replay()
        torch.cuda.synchronize()
        dq_e, dk_e, dv_e = B.ra_ring_bwd(q, k, v, out, do, lse, **kw)
        torch.cuda.synchronize()
        assert torch.equal(dq_g, dq_e), rep
        assert torch.equal(dks, dk_e), rep
        assert torch.equal(dvs, dv_e), rep
    say("graph bwd ok")
