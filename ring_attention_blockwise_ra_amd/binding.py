"""Thin ctypes binding of the C ABI in include/ra.h (argument marshalling only).

Every function here checks tensor shapes, dtypes and devices, allocates
outputs with torch when the caller did not pass them, and calls the HIP
library with raw device pointers and the current HIP stream. No step of the
attention path runs in Python. If the built library is missing, every call
raises: there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libra_amd.so")

RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_WORKSPACE, RA_ERR_HIP = range(5)
RA_F32, RA_BF16 = 0, 1
RA_LAYOUT_CONTIGUOUS, RA_LAYOUT_STRIPED, RA_LAYOUT_ZIGZAG = 0, 1, 2
RA_TILE_SKIP, RA_TILE_PARTIAL, RA_TILE_FULL = 0, 1, 2
RA_MAX_SEQS = 256
RA_ROPE_QUERIES, RA_ROPE_KEYS = 0, 1

_LAYOUT = {"contiguous": RA_LAYOUT_CONTIGUOUS, "striped": RA_LAYOUT_STRIPED,
           "zigzag": RA_LAYOUT_ZIGZAG, RA_LAYOUT_CONTIGUOUS: RA_LAYOUT_CONTIGUOUS,
           RA_LAYOUT_STRIPED: RA_LAYOUT_STRIPED, RA_LAYOUT_ZIGZAG: RA_LAYOUT_ZIGZAG}
_DTYPE = {torch.float32: RA_F32, torch.bfloat16: RA_BF16}

EXPORTED = (
    "ra_block_attn_partial", "ra_merge_partials", "ra_finalize", "ra_ring_workspace_bytes",
    "ra_ring_fwd", "ra_tile_class_host", "ra_tile_classes_host", "ra_tile_classes_device",
    "ra_attn_bwd_delta", "ra_block_attn_bwd", "ra_ring_bwd_workspace_bytes", "ra_ring_bwd",
    "ra_rope_apply", "ra_last_error", "ra_ring_fwd_noalloc", "ra_block_attn_accumulate",
)
RA_NOALLOC_WORKSPACE_BYTES = 64 << 20


class RaProblem(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("batch", ctypes.c_int32), ("hq", ctypes.c_int32),
        ("hkv", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("q_len", ctypes.c_int64),
        ("kv_len", ctypes.c_int64), ("n_ring", ctypes.c_int32), ("rank", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("layout", ctypes.c_int32), ("scale", ctypes.c_float),
        ("n_seqs", ctypes.c_int32), ("cu_seqlens", ctypes.c_void_p),
        ("rope_theta", ctypes.c_float),
    ]
    # keeps the host cu_seqlens array alive as long as the problem
    _keep = None


class RaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"ra status {status}: {message}")
        self.status = status
        self.message = message


_lib = None
_lib_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """Load libra_amd.so (built by ring_attention_blockwise_ra_amd.build)."""
    global _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"HIP library not built: {LIB_PATH} is missing "
                    "(run python -m ring_attention_blockwise_ra_amd.build)")
            L = ctypes.CDLL(LIB_PATH)
            P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
            PP = ctypes.POINTER(RaProblem)
            L.ra_block_attn_partial.argtypes = [PP, I32, P, P, P, P, P, P, P]
            L.ra_block_attn_partial.restype = I32
            L.ra_block_attn_accumulate.argtypes = [PP, I32, P, P, P, P, P, P, P]
            L.ra_block_attn_accumulate.restype = I32
            L.ra_merge_partials.argtypes = [I64, I32, P, P, P, P, P, P, P, P, P, P]
            L.ra_merge_partials.restype = I32
            L.ra_finalize.argtypes = [I64, I32, P, P, P, P, P]
            L.ra_finalize.restype = I32
            L.ra_ring_workspace_bytes.argtypes = [PP]
            L.ra_ring_workspace_bytes.restype = ctypes.c_size_t
            L.ra_ring_fwd.argtypes = [PP, P, P, P, P, P, P, ctypes.c_size_t, P, P]
            L.ra_ring_fwd.restype = I32
            L.ra_tile_class_host.argtypes = [PP, I32, I64, I64, I64, I64]
            L.ra_tile_class_host.restype = I32
            L.ra_tile_classes_host.argtypes = [PP, I32, I32, I32, P]
            L.ra_tile_classes_host.restype = I32
            L.ra_tile_classes_device.argtypes = [PP, I32, I32, I32, P, P]
            L.ra_tile_classes_device.restype = I32
            L.ra_attn_bwd_delta.argtypes = [I64, I32, I32, P, P, P, P]
            L.ra_attn_bwd_delta.restype = I32
            L.ra_block_attn_bwd.argtypes = [PP, I32, P, P, P, P, P, P, P, P, P, P]
            L.ra_block_attn_bwd.restype = I32
            L.ra_ring_bwd_workspace_bytes.argtypes = [PP]
            L.ra_ring_bwd_workspace_bytes.restype = ctypes.c_size_t
            L.ra_ring_bwd.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P, P]
            L.ra_ring_bwd.restype = I32
            L.ra_rope_apply.argtypes = [PP, I32, I32, I32, I32, P, I32, P, I32, I32, P]
            L.ra_rope_apply.restype = I32
            L.ra_ring_fwd_noalloc.argtypes = [PP, P, P, P, P, P, P, P]
            L.ra_ring_fwd_noalloc.restype = I32
            L.ra_last_error.argtypes = []
            L.ra_last_error.restype = ctypes.c_char_p
            _lib = L
    return _lib


def _check(status: int):
    if status != RA_OK:
        raise RaError(status, lib().ra_last_error().decode(errors="replace"))


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(None if t is None else t.data_ptr())


class _OnStream:
    """Orders a library call on stream `s` (None: the current stream) after
    the current stream, and keeps the tensors this binding allocated for the
    call reserved for `s` and `extra` streams.

    The binding allocates outputs (and zero-fills accumulated ones) on the
    current stream. When the call runs elsewhere, `s` first waits for the
    current stream, so those fills land before the library writes or adds
    into the tensors; and each allocated tensor is recorded on `s` (and on a
    side copy stream), so the caching allocator does not hand its memory to
    later work on the current stream while `s` may still use it."""

    def __init__(self, s, device, extra=()):
        cur = torch.cuda.current_stream(device)
        self.stream = cur if s is None else s
        self.other = self.stream != cur
        if self.other:
            self.stream.wait_stream(cur)
        self.extra = [x for x in extra if isinstance(x, torch.cuda.Stream) and x != cur]
        self.owned = []

    def own(self, t):
        if t is not None:
            self.owned.append(t)
        return t

    def handle(self) -> ctypes.c_void_p:
        return ctypes.c_void_p(self.stream.cuda_stream)

    def done(self):
        targets = ([self.stream] if self.other else []) + [x for x in self.extra
                                                            if x != self.stream]
        for t in self.owned:
            for st in targets:
                t.record_stream(st)


def make_problem(*, dtype, batch, hq, hkv, head_dim, q_len, kv_len, n_ring, rank, causal,
                 layout, scale=None, cu_seqlens=None, rope_theta=0.0) -> RaProblem:
    """cu_seqlens: offsets [n_seqs + 1] of packed sequences in the global
    packed sequence (host list/array/tensor), or None. rope_theta: base of
    the rotary embedding the ring applies on arrival (0: none)."""
    p = RaProblem(
        dtype=_DTYPE[dtype] if isinstance(dtype, torch.dtype) else int(dtype),
        batch=int(batch), hq=int(hq), hkv=int(hkv), head_dim=int(head_dim),
        q_len=int(q_len), kv_len=int(kv_len), n_ring=int(n_ring), rank=int(rank),
        causal=int(bool(causal)), layout=_LAYOUT[layout],
        scale=float(scale) if scale is not None else 0.0, rope_theta=float(rope_theta))
    if cu_seqlens is not None:
        if isinstance(cu_seqlens, torch.Tensor):
            cu_seqlens = cu_seqlens.detach().cpu().numpy()
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        p._keep = cu
        p.n_seqs = max(int(cu.size) - 1, 0)
        p.cu_seqlens = cu.ctypes.data if cu.size else None
    return p


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _qkv_problem(q, k, n_ring, rank, causal, layout, scale, cu_seqlens=None, rope_theta=0.0):
    if q.dim() != 4 or k.dim() < 4:
        raise ValueError("q must be [batch, q_len, hq, d]; k, v [.., batch, kv_len, hkv, d]")
    if q.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    b, lq, hq, d = q.shape
    lk, hkv = k.shape[-3], k.shape[-2]
    return make_problem(dtype=q.dtype, batch=b, hq=hq, hkv=hkv, head_dim=d, q_len=lq, kv_len=lk,
                        n_ring=n_ring, rank=rank, causal=causal, layout=layout, scale=scale,
                        cu_seqlens=cu_seqlens, rope_theta=rope_theta)


def ra_block_attn_partial(q, k, v, kv_block_j: int, *, n_ring: int, rank: int, causal: bool,
                          layout="contiguous", scale=None, m=None, l=None, acc=None, stream=None,
                          cu_seqlens=None):
    """Partial (m, l, acc) of q against KV block kv_block_j (see include/ra.h)."""
    _need(q, "q")
    prob = _qkv_problem(q, k, n_ring, rank, causal, layout, scale, cu_seqlens)
    b, lq, hq, d = q.shape
    _need(k, "k", q.dtype, (b, prob.kv_len, prob.hkv, d), q.device)
    _need(v, "v", q.dtype, (b, prob.kv_len, prob.hkv, d), q.device)
    with torch.cuda.device(q.device):
        on = _OnStream(stream, q.device)
        m = on.own(torch.empty(b, lq, hq, dtype=torch.float32, device=q.device)) if m is None else m
        l = on.own(torch.empty(b, lq, hq, dtype=torch.float32, device=q.device)) if l is None else l
        acc = on.own(torch.empty(b, lq, hq, d, dtype=torch.float32, device=q.device)) \
            if acc is None else acc
        _need(m, "m", torch.float32, (b, lq, hq), q.device)
        _need(l, "l", torch.float32, (b, lq, hq), q.device)
        _need(acc, "acc", torch.float32, (b, lq, hq, d), q.device)
        _check(lib().ra_block_attn_partial(ctypes.byref(prob), int(kv_block_j), _ptr(q), _ptr(k),
                                           _ptr(v), _ptr(m), _ptr(l), _ptr(acc), on.handle()))
        on.done()
    return m, l, acc


def ra_block_attn_accumulate(q, k, v, kv_block_j: int, *, n_ring: int, rank: int, causal: bool,
                             m, l, acc, layout="contiguous", scale=None, stream=None,
                             cu_seqlens=None):
    """Block kv_block_j's partial merged into the running (m, l, acc) in place
    (see include/ra.h); returns (m, l, acc)."""
    _need(q, "q")
    prob = _qkv_problem(q, k, n_ring, rank, causal, layout, scale, cu_seqlens)
    b, lq, hq, d = q.shape
    _need(k, "k", q.dtype, (b, prob.kv_len, prob.hkv, d), q.device)
    _need(v, "v", q.dtype, (b, prob.kv_len, prob.hkv, d), q.device)
    _need(m, "m", torch.float32, (b, lq, hq), q.device)
    _need(l, "l", torch.float32, (b, lq, hq), q.device)
    _need(acc, "acc", torch.float32, (b, lq, hq, d), q.device)
    with torch.cuda.device(q.device):
        on = _OnStream(stream, q.device)
        _check(lib().ra_block_attn_accumulate(ctypes.byref(prob), int(kv_block_j), _ptr(q),
                                              _ptr(k), _ptr(v), _ptr(m), _ptr(l), _ptr(acc),
                                              on.handle()))
        on.done()
    return m, l, acc


def ra_merge_partials(m1, l1, acc1, m2, l2, acc2, *, out=None, stream=None):
    """(m1, l1, acc1) merged with (m2, l2, acc2); out=(m, l, acc) may be input 1."""
    _need(acc1, "acc1", torch.float32)
    d = acc1.shape[-1]
    rows = acc1.numel() // d if d else 0
    dev = acc1.device
    for name, t in (("m1", m1), ("l1", l1), ("m2", m2), ("l2", l2)):
        _need(t, name, torch.float32, device=dev)
        if t.numel() != rows:
            raise ValueError(f"{name} has {t.numel()} elements, expected {rows}")
    _need(acc2, "acc2", torch.float32, acc1.shape, dev)
    with torch.cuda.device(dev):
        on = _OnStream(stream, dev)
        if out is None:
            out = (on.own(torch.empty_like(m1)), on.own(torch.empty_like(l1)),
                   on.own(torch.empty_like(acc1)))
        mo, lo, ao = out
        _need(mo, "m_out", torch.float32, m1.shape, dev)
        _need(lo, "l_out", torch.float32, l1.shape, dev)
        _need(ao, "acc_out", torch.float32, acc1.shape, dev)
        _check(lib().ra_merge_partials(rows, d, _ptr(m1), _ptr(l1), _ptr(acc1), _ptr(m2),
                                       _ptr(l2), _ptr(acc2), _ptr(mo), _ptr(lo), _ptr(ao),
                                       on.handle()))
        on.done()
    return mo, lo, ao


def ra_finalize(m, l, acc, *, lse=None, want_lse=True, stream=None):
    """acc <- acc / l in place; returns (acc, lse)."""
    _need(acc, "acc", torch.float32)
    d = acc.shape[-1]
    rows = acc.numel() // d if d else 0
    dev = acc.device
    _need(m, "m", torch.float32, device=dev)
    _need(l, "l", torch.float32, device=dev)
    with torch.cuda.device(dev):
        on = _OnStream(stream, dev)
        if lse is None and want_lse:
            lse = on.own(torch.empty_like(m))
        _check(lib().ra_finalize(rows, d, _ptr(m), _ptr(l), _ptr(acc), _ptr(lse), on.handle()))
        on.done()
    return acc, lse


def ra_ring_workspace_bytes(prob: RaProblem) -> int:
    return int(lib().ra_ring_workspace_bytes(ctypes.byref(prob)))


def ra_ring_fwd(q, k, v, *, n_ring: int, causal: bool, layout="contiguous", rank: int = None,
                scale=None, out=None, lse=None, want_lse=True, workspace=None,
                compute_stream=None, copy_stream="auto", cu_seqlens=None, rope_theta=0.0):
    """One device's share: q [b, lq, hq, d]; k, v [n_ring, b, lk, hkv, d].
    cu_seqlens: packed sequences (batch 1), global offsets [n_seqs + 1].
    rope_theta > 0: rotary embedding applied on arrival (q and k unrotated).

    Returns (out fp32 [b, lq, hq, d], lse fp32 [b, lq, hq] or None).
    copy_stream: "auto" (a dedicated side stream per device), None (copies
    in order on the compute stream) or a torch.cuda.Stream.
    """
    if rank is None:
        rank = n_ring - 1
    _need(q, "q")
    prob = _qkv_problem(q, k, n_ring, rank, causal, layout, scale, cu_seqlens, rope_theta)
    b, lq, hq, d = q.shape
    dev = q.device
    _need(k, "k", q.dtype, (n_ring, b, prob.kv_len, prob.hkv, d), dev)
    _need(v, "v", q.dtype, (n_ring, b, prob.kv_len, prob.hkv, d), dev)
    need = ra_ring_workspace_bytes(prob)
    if need == 0 and b * lq * hq > 0:
        _check(lib().ra_ring_fwd(ctypes.byref(prob), None, None, None, None, None, None, 0,
                                 None, None))
    with torch.cuda.device(dev):
        if copy_stream == "auto":
            copy_stream = side_stream(dev)
        on = _OnStream(compute_stream, dev, extra=(copy_stream,))
        out = on.own(torch.empty(b, lq, hq, d, dtype=torch.float32, device=dev)) \
            if out is None else out
        _need(out, "out", torch.float32, (b, lq, hq, d), dev)
        if lse is None and want_lse:
            lse = on.own(torch.empty(b, lq, hq, dtype=torch.float32, device=dev))
        if lse is not None:
            _need(lse, "lse", torch.float32, (b, lq, hq), dev)
        if workspace is None:
            workspace = on.own(torch.empty(max(need, 1), dtype=torch.uint8, device=dev))
        _need(workspace, "workspace", torch.uint8, device=dev)
        xs = ctypes.c_void_p(None) if copy_stream is None else ctypes.c_void_p(copy_stream.cuda_stream)
        _check(lib().ra_ring_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                 _ptr(lse), _ptr(workspace), workspace.numel(), on.handle(), xs))
        on.done()
    return out, lse


def ra_ring_fwd_noalloc(q, k, v, *, n_ring: int, causal: bool, out, lse=None,
                        layout="contiguous", rank: int = None, scale=None, compute_stream=None,
                        copy_stream="auto", cu_seqlens=None, rope_theta=0.0):
    """ra_ring_fwd on the library's static per-GPU workspace (no device
    allocation by the library, none by this binding): the caller passes out
    [b, lq, hq, d] float32 and optionally lse [b, lq, hq] float32. Problems
    whose workspace exceeds RA_NOALLOC_WORKSPACE_BYTES raise RaError
    (RA_ERR_WORKSPACE). Calls that overlap on one GPU race on that workspace."""
    if rank is None:
        rank = n_ring - 1
    _need(q, "q")
    prob = _qkv_problem(q, k, n_ring, rank, causal, layout, scale, cu_seqlens, rope_theta)
    b, lq, hq, d = q.shape
    dev = q.device
    _need(k, "k", q.dtype, (n_ring, b, prob.kv_len, prob.hkv, d), dev)
    _need(v, "v", q.dtype, (n_ring, b, prob.kv_len, prob.hkv, d), dev)
    _need(out, "out", torch.float32, (b, lq, hq, d), dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (b, lq, hq), dev)
    with torch.cuda.device(dev):
        if copy_stream == "auto":
            copy_stream = side_stream(dev)
        on = _OnStream(compute_stream, dev)
        xs = ctypes.c_void_p(None) if copy_stream is None else ctypes.c_void_p(copy_stream.cuda_stream)
        _check(lib().ra_ring_fwd_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(out), _ptr(lse), on.handle(), xs))
    return out, lse


def ra_attn_bwd_delta(out, dout, *, delta=None, stream=None):
    """delta = rowsum(dout * out) over the last dimension (float32)."""
    _need(out, "out", torch.float32)
    _need(dout, "dout", shape=out.shape, device=out.device)
    if dout.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {dout.dtype}")
    d = out.shape[-1]
    rows = out.numel() // d if d else 0
    with torch.cuda.device(out.device):
        on = _OnStream(stream, out.device)
        if delta is None:
            delta = on.own(torch.empty(out.shape[:-1], dtype=torch.float32, device=out.device))
        _need(delta, "delta", torch.float32, out.shape[:-1], out.device)
        _check(lib().ra_attn_bwd_delta(rows, d, _DTYPE[dout.dtype], _ptr(out), _ptr(dout),
                                       _ptr(delta), on.handle()))
        on.done()
    return delta


def ra_block_attn_bwd(q, k, v, dout, lse, delta, kv_block_j: int, *, n_ring: int, rank: int,
                      causal: bool, layout="contiguous", scale=None, dq=None, dk=None, dv=None,
                      stream=None, cu_seqlens=None):
    """Block j's backward addends, ACCUMULATED into dq, dk, dv (new zeroed
    tensors when not given); see include/ra.h."""
    _need(q, "q")
    prob = _qkv_problem(q, k, n_ring, rank, causal, layout, scale, cu_seqlens)
    b, lq, hq, d = q.shape
    dev = q.device
    kshape = (b, prob.kv_len, prob.hkv, d)
    _need(k, "k", q.dtype, kshape, dev)
    _need(v, "v", q.dtype, kshape, dev)
    _need(dout, "dout", q.dtype, q.shape, dev)
    _need(lse, "lse", torch.float32, (b, lq, hq), dev)
    _need(delta, "delta", torch.float32, (b, lq, hq), dev)
    with torch.cuda.device(dev):
        new = [t is None for t in (dq, dk, dv)]
        dq = torch.zeros(b, lq, hq, d, dtype=torch.float32, device=dev) if dq is None else dq
        dk = torch.zeros(kshape, dtype=torch.float32, device=dev) if dk is None else dk
        dv = torch.zeros(kshape, dtype=torch.float32, device=dev) if dv is None else dv
        on = _OnStream(stream, dev)   # ordered after the zero fills just queued
        for t, n in zip((dq, dk, dv), new):
            if n:
                on.own(t)
        _need(dq, "dq", torch.float32, (b, lq, hq, d), dev)
        _need(dk, "dk", torch.float32, kshape, dev)
        _need(dv, "dv", torch.float32, kshape, dev)
        _check(lib().ra_block_attn_bwd(ctypes.byref(prob), int(kv_block_j), _ptr(q), _ptr(k),
                                       _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq),
                                       _ptr(dk), _ptr(dv), on.handle()))
        on.done()
    return dq, dk, dv


def ra_ring_bwd_workspace_bytes(prob: RaProblem) -> int:
    return int(lib().ra_ring_bwd_workspace_bytes(ctypes.byref(prob)))


def ra_ring_bwd(q, k, v, out, dout, lse, *, n_ring: int, causal: bool, layout="contiguous",
                rank: int = None, scale=None, dq=None, dk=None, dv=None, workspace=None,
                compute_stream=None, copy_stream="auto", cu_seqlens=None, rope_theta=0.0):
    """Backward of one device's share: returns (dq, dk, dv). dq is written;
    this share's addends are ADDED to dk, dv [n_ring, b, lk, hkv, d] (new
    zeroed tensors when not given)."""
    if rank is None:
        rank = n_ring - 1
    _need(q, "q")
    prob = _qkv_problem(q, k, n_ring, rank, causal, layout, scale, cu_seqlens, rope_theta)
    b, lq, hq, d = q.shape
    dev = q.device
    kshape = (n_ring, b, prob.kv_len, prob.hkv, d)
    _need(k, "k", q.dtype, kshape, dev)
    _need(v, "v", q.dtype, kshape, dev)
    _need(out, "out", torch.float32, (b, lq, hq, d), dev)
    _need(dout, "dout", q.dtype, q.shape, dev)
    _need(lse, "lse", torch.float32, (b, lq, hq), dev)
    need = ra_ring_bwd_workspace_bytes(prob)
    if need == 0 and b * lq * hq > 0:
        _check(lib().ra_ring_bwd(ctypes.byref(prob), None, None, None, None, None, None, None,
                                 None, None, None, 0, None, None))
    with torch.cuda.device(dev):
        if copy_stream == "auto":
            copy_stream = side_stream(dev)
        new = [t is None for t in (dq, dk, dv, workspace)]
        dq = torch.empty(b, lq, hq, d, dtype=torch.float32, device=dev) if dq is None else dq
        dk = torch.zeros(kshape, dtype=torch.float32, device=dev) if dk is None else dk
        dv = torch.zeros(kshape, dtype=torch.float32, device=dev) if dv is None else dv
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        # the ring adds into dk, dv on the compute stream: it waits for their
        # zero fills on the current stream first
        on = _OnStream(compute_stream, dev, extra=(copy_stream,))
        for t, n in zip((dq, dk, dv, workspace), new):
            if n:
                on.own(t)
        _need(dq, "dq", torch.float32, (b, lq, hq, d), dev)
        _need(dk, "dk", torch.float32, kshape, dev)
        _need(dv, "dv", torch.float32, kshape, dev)
        _need(workspace, "workspace", torch.uint8, device=dev)
        xs = ctypes.c_void_p(None) if copy_stream is None else ctypes.c_void_p(copy_stream.cuda_stream)
        _check(lib().ra_ring_bwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                 _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                 _ptr(workspace), workspace.numel(), on.handle(), xs))
        on.done()
    return dq, dk, dv


def ra_rope_apply(x, prob: RaProblem, *, target="keys", block_j: int = 0, out=None,
                  out_dtype=None, inverse=False, accumulate=False, stream=None):
    """Rotary embedding of x [b, len, heads, d] with the positions of block
    block_j's keys (target="keys") or of the local queries ("queries")."""
    _need(x, "x")
    if x.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {x.dtype}")
    out_dtype = out_dtype or x.dtype
    tgt = RA_ROPE_QUERIES if target == "queries" else RA_ROPE_KEYS
    with torch.cuda.device(x.device):
        fresh = out is None
        if fresh:
            out = torch.zeros(x.shape, dtype=out_dtype, device=x.device) if accumulate else \
                torch.empty(x.shape, dtype=out_dtype, device=x.device)
        on = _OnStream(stream, x.device)
        if fresh:
            on.own(out)
        _need(out, "out", out_dtype, x.shape, x.device)
        _check(lib().ra_rope_apply(ctypes.byref(prob), tgt, int(block_j), int(x.shape[2]),
                                   _DTYPE[x.dtype], _ptr(x), _DTYPE[out_dtype], _ptr(out),
                                   int(bool(inverse)), int(bool(accumulate)), on.handle()))
        on.done()
    return out


_side = {}


def side_stream(device) -> torch.cuda.Stream:
    """A default-priority side stream per device for K/V staging copies."""
    idx = torch.device(device).index
    if idx is None:
        idx = torch.cuda.current_device()
    if idx not in _side:
        _side[idx] = torch.cuda.Stream(device=idx)
    return _side[idx]


def ra_tile_class_host(prob: RaProblem, kv_block_j: int, a_lo, a_hi, b_lo, b_hi) -> int:
    c = lib().ra_tile_class_host(ctypes.byref(prob), int(kv_block_j), int(a_lo), int(a_hi),
                                 int(b_lo), int(b_hi))
    if c < 0:
        raise RaError(RA_ERR_INVALID_ARG, lib().ra_last_error().decode())
    return c


def ra_tile_classes_host(prob: RaProblem, kv_block_j: int, tq: int, tk: int) -> np.ndarray:
    nqt, nkt = -(-prob.q_len // tq), -(-prob.kv_len // tk)
    out = np.zeros((nqt, nkt), dtype=np.int8)
    _check(lib().ra_tile_classes_host(ctypes.byref(prob), int(kv_block_j), int(tq), int(tk),
                                      out.ctypes.data_as(ctypes.c_void_p)))
    return out


def ra_tile_classes_device(prob: RaProblem, kv_block_j: int, tq: int, tk: int, device="cuda",
                           stream=None) -> torch.Tensor:
    nqt, nkt = -(-prob.q_len // tq), -(-prob.kv_len // tk)
    out = torch.full((nqt, nkt), -1, dtype=torch.int8, device=device)
    with torch.cuda.device(out.device):
        on = _OnStream(stream, out.device)   # after the fill just queued
        on.own(out)
        _check(lib().ra_tile_classes_device(ctypes.byref(prob), int(kv_block_j), int(tq), int(tk),
                                            _ptr(out), on.handle()))
        on.done()
    return out


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
