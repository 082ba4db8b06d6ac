"""Seeded synthetic inputs for tests, smoke and bench.

This module holds no attention arithmetic: it only draws numbers. It is the
one module that both the HIP-side harness and the CPU oracle's tests use, so
that both see bit-identical inputs.

Every tensor is generated in global token order, [batch, seq, heads, dim],
as float32 and then rounded to the target dtype (bfloat16: round to nearest
even, torch's conversion). Large tensors are generated in row chunks, each
chunk from its own seeded generator, so that any subset of rows can be
produced without holding the whole float32 tensor.

Workload shapes (sizes and value distributions of the pages' workloads):
  c1  fp32, 1 head, d=16, 32 tokens, N=4 blocks of 8, non-causal: the
      four-device single-process simulation on the Ultralytics "Ring
      Attention" page (section "How ring attention works"): one seeded
      draw of shape (3, 32, 16) split into q, k, v.
  c2  bf16, 32 heads, d=128, 8192 tokens, N=8, causal contiguous, N(0,1).
  c3  bf16, 32 q heads / 8 kv heads, d=128, 131072 tokens, N=8, causal
      striped, N(0,1).
  c4  bf16, 32 q / 8 kv heads, d=128, 1,048,576 tokens, N=8, causal,
      contiguous and striped; N(0,1) with k scaled by 0.5 (in fp32, then
      rounded).
  c5  bf16, 32 heads, d=128, 921,600 tokens = 3600 frames x 256 tokens
      (the Ultralytics page's video geometry: 256 tokens per frame, one hour
      at one frame per second), N=8, non-causal; each of q, k, v is
      N(0,1) plus a per-(frame, head, dim) offset ~ N(0, 0.5^2) shared by
      the frame's 256 tokens.
"""

from __future__ import annotations

import torch

CHUNK_ROWS = 65536

CONFIGS = {
    "c1": dict(dtype="f32", n_ring=4, block=8, hq=1, hkv=1, d=16, causal=False,
               layouts=("contiguous",), ranks=(0, 1, 2, 3), seed=0),
    "c2": dict(dtype="bf16", n_ring=8, block=1024, hq=32, hkv=32, d=128, causal=True,
               layouts=("contiguous",), ranks=tuple(range(8)), seed=2),
    "c3": dict(dtype="bf16", n_ring=8, block=16384, hq=32, hkv=8, d=128, causal=True,
               layouts=("striped",), ranks=(7,), seed=3),
    "c4": dict(dtype="bf16", n_ring=8, block=131072, hq=32, hkv=8, d=128, causal=True,
               layouts=("contiguous", "striped"), ranks=(7,), seed=4, k_scale=0.5),
    "c5": dict(dtype="bf16", n_ring=8, block=115200, hq=32, hkv=32, d=128, causal=False,
               layouts=("contiguous",), ranks=(0,), seed=5, frame_tokens=256,
               frame_sigma=0.5),
    # the 1M-token share of c4 with the sequence packed from documents of
    # mixed lengths (varlen); same token values as c4
    "c4p": dict(dtype="bf16", n_ring=8, block=131072, hq=32, hkv=8, d=128, causal=True,
                layouts=("zigzag", "contiguous", "striped"), ranks=(7,), seed=4, k_scale=0.5,
                values_from="c4", packed=dict(seed=44, min_len=16384, max_len=262144)),
}

_TENSOR_ID = {"q": 1, "k": 2, "v": 3}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def c1_qkv():
    """The Ultralytics simulation's inputs: generator seeded with 0, one
    standard-normal draw of shape (3, 32, 16) split into q, k, v. Returned as
    float32 [1, 32, 1, 16] each (batch 1, one head)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(0)
    x = torch.randn(3, 32, 16, generator=g)
    q, k, v = x[0], x[1], x[2]
    return tuple(t.reshape(1, 32, 1, 16).contiguous() for t in (q, k, v))


def _chunk_generator(seed: int, tensor_id: int, chunk: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + tensor_id * 7919 + chunk)
    return g


def normal_rows(name: str, seed: int, batch: int, seq: int, heads: int, dim: int,
                device="cpu", rows=None, out_dtype=torch.bfloat16, scale: float = 1.0,
                frame_tokens: int = 0, frame_sigma: float = 0.0) -> torch.Tensor:
    """Rows of a global [batch, seq, heads, dim] tensor of N(0,1) draws.

    rows: None for all rows, else a 1-D LongTensor of global token indices
    (any order); the result is [batch, len(rows), heads, dim].
    scale multiplies the float32 draw before rounding (c4's k x 0.5).
    frame_tokens/frame_sigma add a per-(frame, head, dim) offset drawn from
    N(0, frame_sigma^2), frame = token // frame_tokens (c5).
    """
    tid = _TENSOR_ID[name]
    n_chunks = -(-seq // CHUNK_ROWS)
    if rows is not None:
        rows = torch.as_tensor(rows, dtype=torch.int64, device=device)
        out = torch.empty(batch, rows.numel(), heads, dim, dtype=out_dtype, device=device)
    else:
        out = torch.empty(batch, seq, heads, dim, dtype=out_dtype, device=device)
    offsets = None
    if frame_tokens:
        n_frames = -(-seq // frame_tokens)
        go = _chunk_generator(seed, tid + 100, 0, device)
        offsets = torch.randn(batch, n_frames, heads, dim, generator=go, device=device) * frame_sigma
    for c in range(n_chunks):
        r0, r1 = c * CHUNK_ROWS, min(seq, (c + 1) * CHUNK_ROWS)
        if rows is not None:
            sel = ((rows >= r0) & (rows < r1)).nonzero().flatten()
            if sel.numel() == 0:
                continue
        g = _chunk_generator(seed, tid, c, device)
        x = torch.randn(batch, r1 - r0, heads, dim, generator=g, device=device)
        if scale != 1.0:
            x = x * scale
        if offsets is not None:
            fidx = torch.arange(r0, r1, device=device) // frame_tokens
            x = x + offsets[:, fidx]
        if rows is not None:
            out[:, sel] = x[:, rows[sel] - r0].to(out_dtype)
        else:
            out[:, r0:r1] = x.to(out_dtype)
    return out


def config_global(cfg_name: str, device="cpu", q_rows=None):
    """Global-order (q, k, v) of a named workload.

    q_rows: None for every query row, else the global token indices of the
    query rows wanted (a device's share). k and v are always whole.
    """
    if cfg_name == "c1":
        q, k, v = c1_qkv()
        if q_rows is not None:
            q = q[:, torch.as_tensor(q_rows, dtype=torch.int64)]
        return q.to(device), k.to(device), v.to(device)
    c = CONFIGS[CONFIGS[cfg_name].get("values_from", cfg_name)]
    seq = c["n_ring"] * c["block"]
    dt = torch_dtype(c["dtype"])
    extra = {}
    if "frame_tokens" in c:
        extra = dict(frame_tokens=c["frame_tokens"], frame_sigma=c["frame_sigma"])
    q = normal_rows("q", c["seed"], 1, seq, c["hq"], c["d"], device, rows=q_rows, out_dtype=dt, **extra)
    k = normal_rows("k", c["seed"], 1, seq, c["hkv"], c["d"], device, out_dtype=dt,
                    scale=c.get("k_scale", 1.0), **extra)
    v = normal_rows("v", c["seed"], 1, seq, c["hkv"], c["d"], device, out_dtype=dt, **extra)
    return q, k, v


def random_global(seed: int, batch: int, seq: int, hq: int, hkv: int, d: int,
                  dtype: str = "bf16", device="cpu", scale: float = 1.0):
    """Global-order (q, k, v) ~ N(0,1) (k, v times `scale`) for ad-hoc shapes."""
    dt = torch_dtype(dtype)
    q = normal_rows("q", seed, batch, seq, hq, d, device, out_dtype=dt)
    k = normal_rows("k", seed, batch, seq, hkv, d, device, out_dtype=dt, scale=scale)
    v = normal_rows("v", seed, batch, seq, hkv, d, device, out_dtype=dt, scale=scale)
    return q, k, v


def packed_seqlens(total: int, multiple: int, seed: int, min_len: int, max_len: int) -> list[int]:
    """Lengths of packed sequences filling `total` tokens: log-uniform draws in
    [min_len, max_len] rounded down to a multiple of `multiple` (at least
    one multiple), in draw order; the last sequence takes what is left."""
    g = torch.Generator().manual_seed(seed)
    lens, used = [], 0
    lo, hi = torch.log(torch.tensor(float(min_len))), torch.log(torch.tensor(float(max_len)))
    while True:
        u = float(torch.rand((), generator=g))
        L = int(torch.exp(lo + u * (hi - lo))) // multiple * multiple
        L = max(L, multiple)
        if used + L >= total:
            lens.append(total - used)
            return lens
        lens.append(L)
        used += L


def config_seqlens(cfg_name: str, layout: str):
    """Packed sequence lengths of a named workload (None if not packed); each
    a multiple of 2N so that every layout, zigzag included, can split it."""
    c = CONFIGS[cfg_name]
    if "packed" not in c:
        return None
    pk = c["packed"]
    return packed_seqlens(c["n_ring"] * c["block"], 2 * c["n_ring"], pk["seed"], pk["min_len"],
                          pk["max_len"])
