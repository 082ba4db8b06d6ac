"""The C ABI without Python on the device path: the plain-C client
(tests/capi_ring.c, built beside libra_amd.so) runs ra_ring_fwd on the GPU
with its own device buffers and streams (HIP's C API only). Its output must
match the fp64 oracle to the bf16 tolerance and equal, bit for bit, what the
Python binding computes for the same inputs."""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from oracle import ring_oracle as orc
from ring_attention_blockwise_ra_amd import binding as B
from ring_attention_blockwise_ra_amd import build as BUILD
from ring_attention_blockwise_ra_amd import synth
from ring_attention_blockwise_ra_amd.layout import blocks_from_global, share_tokens

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("side_stream_always")]
LAYOUT_ID = {"contiguous": 0, "striped": 1, "zigzag": 2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("layout,rank", [("striped", 3), ("zigzag", 0), ("contiguous", 2)])
def test_ring_forward_from_plain_c(tmp_path, layout, rank):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = BUILD.C_CLIENT
    assert os.path.exists(exe), f"{exe} missing: run python -m ring_attention_blockwise_ra_amd.build"
    n, blen, hq, hkv, d = 4, 256, 8, 2, 128
    say(f"capi ring: {layout} rank {rank}")
    q, k, v = synth.random_global(11, 1, n * blen, hq, hkv, d, dtype="bf16", device="cpu")
    rows = share_tokens(layout, n, rank, blen)
    qs = q[:, rows].contiguous()
    kb, vb = blocks_from_global(k, layout, n), blocks_from_global(v, layout, n)
    src, dst = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    with open(src, "wb") as f:
        for t in (qs, kb, vb):
            f.write(t.contiguous().view(torch.int16).numpy().tobytes())
    r = subprocess.run([exe, src, dst, str(n), str(rank), str(blen), str(hq), str(hkv), str(d),
                        str(LAYOUT_ID[layout]), "1"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    res = np.fromfile(dst, dtype=np.float32)
    assert res.size == blen * hq * d + blen * hq
    out_c = res[:blen * hq * d].reshape(1, blen, hq, d)
    lse_c = res[blen * hq * d:].reshape(1, blen, hq)

    ref, ref_lse = orc.naive_attention(*(t.double().numpy() for t in (q, k, v)), causal=True)
    idx = rows.numpy()
    assert np.abs(out_c - ref[:, idx]).max() <= 1e-2
    assert np.abs(lse_c - ref_lse[:, idx]).max() <= 1e-2

    dev = torch.device("cuda", 0)
    out_p, lse_p = B.ra_ring_fwd(qs.to(dev), kb.to(dev), vb.to(dev), n_ring=n, causal=True, layout=layout,
                                 rank=rank)
    torch.cuda.synchronize()
    assert np.array_equal(out_p.cpu().numpy(), out_c)
    assert np.array_equal(lse_p.cpu().numpy(), lse_c)
    say("capi ring ok")
