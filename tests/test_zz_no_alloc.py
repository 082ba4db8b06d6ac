"""The allocation-free ring entry point (ra_ring_fwd_noalloc) against
ra_ring_fwd: the same kernels on the library's static per-GPU workspace, so
outputs and lse must be bit-identical. Two calls in a row, the second with a
smaller problem (the array keeps the first call's contents), a third with
rotary embedding, and a problem too large for the static workspace, which
must be refused with nothing written."""

import ctypes
import sys

import pytest
import torch

from ring_attention_blockwise_ra_amd import binding as B
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


def _share(seed, n, blen, hq, hkv, d, layout, r):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn(1, n * blen, hq, d, generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn(1, n * blen, hkv, d, generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn(1, n * blen, hkv, d, generator=g, device=DEV).to(torch.bfloat16)
    kb, vb = blocks_from_global(k, layout, n), blocks_from_global(v, layout, n)
    qs = q[:, share_tokens(layout, n, r, blen).to(DEV)].contiguous()
    return qs, kb, vb


def _compare(qs, kb, vb, n, layout, r, causal, rope_theta=0.0):
    prob = B.make_problem(dtype=torch.bfloat16, batch=1, hq=qs.shape[2], hkv=kb.shape[3],
                          head_dim=qs.shape[3], q_len=qs.shape[1], kv_len=kb.shape[2],
                          n_ring=n, rank=r, causal=causal, layout=layout, rope_theta=rope_theta)
    need = B.ra_ring_workspace_bytes(prob)
    assert 0 < need <= B.RA_NOALLOC_WORKSPACE_BYTES, need
    ref, ref_lse = B.ra_ring_fwd(qs, kb, vb, n_ring=n, causal=causal, layout=layout, rank=r,
                                 rope_theta=rope_theta)
    out = torch.full(ref.shape, float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full(ref_lse.shape, float("nan"), dtype=torch.float32, device=DEV)
    B.ra_ring_fwd_noalloc(qs, kb, vb, n_ring=n, causal=causal, layout=layout, rank=r, out=out,
                          lse=lse, rope_theta=rope_theta)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(lse, ref_lse)
    return need


def test_noalloc_matches_ring_fwd_twice_then_smaller():
    # 1024 tokens x 32 heads x d 128 per block, N = 8, causal contiguous, rank 7:
    # the workspace (~48.5 MiB) nearly fills the static array
    say("noalloc: call 1, 8 blocks of 1024 tokens, 32 heads, causal contiguous, rank 7")
    qs, kb, vb = _share(1, 8, 1024, 32, 32, 128, "contiguous", 7)
    need1 = _compare(qs, kb, vb, 8, "contiguous", 7, True)
    # a smaller problem right after: the array still holds call 1's data
    say("noalloc: call 2, 4 blocks of 384 tokens, GQA 8/2, causal striped, rank 2")
    qs, kb, vb = _share(2, 4, 384, 8, 2, 128, "striped", 2)
    need2 = _compare(qs, kb, vb, 4, "striped", 2, True)
    assert need2 < need1
    say("noalloc: call 3, 4 blocks of 256 tokens, GQA 8/2, causal zigzag with rotary embedding")
    qs, kb, vb = _share(3, 4, 256, 8, 2, 64, "zigzag", 1)
    _compare(qs, kb, vb, 4, "zigzag", 1, True, rope_theta=10000.0)
    say("noalloc: call 4, non-causal, 2 blocks of 200 tokens (ragged tiles), d 32")
    qs, kb, vb = _share(4, 2, 200, 4, 4, 32, "contiguous", 0)
    _compare(qs, kb, vb, 2, "contiguous", 0, False)


def test_noalloc_refuses_a_problem_beyond_its_workspace():
    say("noalloc: a share whose workspace exceeds the static array is refused")
    qs, kb, vb = _share(5, 8, 2048, 32, 32, 128, "contiguous", 7)
    out = torch.full((1, 2048, 32, 128), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(B.RaError) as ei:
        B.ra_ring_fwd_noalloc(qs, kb, vb, n_ring=8, causal=True, out=out)
    assert ei.value.status == B.RA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
