"""CPU-only tests of the HIP library's host side: it loads, exports every
symbol include/ra.h declares, validates arguments before any HIP call, and its
causal tile scheduler (host mirror) matches the oracle's element brute force
bit for bit. No compute call is made (there may be no GPU)."""

import ctypes
import itertools
import os
import re

import numpy as np
import pytest

from oracle import ring_oracle as orc
from ring_attention_blockwise_ra_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ra.h")

_ORACLE_CLASS = {B.RA_TILE_SKIP: orc.SKIP, B.RA_TILE_PARTIAL: orc.PARTIAL, B.RA_TILE_FULL: orc.FULL}


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from ring_attention_blockwise_ra_amd import build
        build.build()
    return B.lib()


def test_library_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert len(names) >= 9
    assert set(names) == set(B.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def _prob(**kw):
    base = dict(dtype=B.RA_BF16, batch=1, hq=4, hkv=2, head_dim=64, q_len=256, kv_len=256,
                n_ring=4, rank=1, causal=1, layout="contiguous")
    base.update(kw)
    return B.make_problem(**base)


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation fails first


def _partial(L, prob, j=0, ptr=FAKE):
    return L.ra_block_attn_partial(ctypes.byref(prob), j, ptr, ptr, ptr, ptr, ptr, ptr, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), B.RA_ERR_INVALID_ARG),
    (dict(batch=-1), B.RA_ERR_INVALID_ARG),
    (dict(hq=0), B.RA_ERR_INVALID_ARG),
    (dict(hq=6, hkv=4), B.RA_ERR_INVALID_ARG),
    (dict(head_dim=96), B.RA_ERR_UNSUPPORTED),
    (dict(head_dim=256), B.RA_ERR_UNSUPPORTED),
    (dict(head_dim=0), B.RA_ERR_INVALID_ARG),
    (dict(n_ring=0, rank=0), B.RA_ERR_INVALID_ARG),
    (dict(rank=4), B.RA_ERR_INVALID_ARG),
    (dict(rank=-1), B.RA_ERR_INVALID_ARG),
    (dict(q_len=128), B.RA_ERR_INVALID_ARG),          # causal needs q_len == kv_len
    (dict(q_len=-5, causal=0), B.RA_ERR_INVALID_ARG),
    (dict(q_len=(1 << 30) + 1, kv_len=(1 << 30) + 1), B.RA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), B.RA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), B.RA_ERR_INVALID_ARG),
])
def test_problem_validation_before_any_hip_call(L, kw, status):
    prob = _prob(**kw)
    assert _partial(L, prob) == status
    assert L.ra_last_error()  # message set
    assert L.ra_ring_workspace_bytes(ctypes.byref(prob)) == 0


def _grid_prob(**kw):
    base = dict(dtype=B.RA_BF16, batch=1, hq=1, hkv=1, head_dim=128, q_len=1 << 20,
                kv_len=1 << 20, n_ring=1, rank=0, causal=0, layout="contiguous")
    base.update(kw)
    return B.make_problem(**base)


def _fwd_status(L, prob):
    """Status of a forward call whose q pointer is NULL: a problem that passes
    every launch check is rejected for the pointer ("q is NULL"), one that does
    not for its grid; nothing is enqueued either way."""
    st = L.ra_block_attn_partial(ctypes.byref(prob), 0, None, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    return st, L.ra_last_error().decode()


def _bwd_status(L, prob):
    st = L.ra_block_attn_bwd(ctypes.byref(prob), 0, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, FAKE, None)
    return st, L.ra_last_error().decode()


@pytest.mark.parametrize("dtype,head_dim,batch,ok", [
    # fp32 at d = 128: 64 rows and 256 work items per workgroup; 2^20 rows per
    # head -> 16384 workgroups: 1024 heads fill 2^32 work items exactly (one too
    # many), 1023 fit
    (B.RA_F32, 128, 1024, False),
    (B.RA_F32, 128, 1023, True),
    (B.RA_F32, 128, 2048, False),   # was accepted when tiles were assumed to hold 128 rows
    # fp32 at d = 16: 256 rows per workgroup of 256 work items
    (B.RA_F32, 16, 4096, False),
    (B.RA_F32, 16, 4095, True),
    # bf16: 256 rows and 512 work items per workgroup
    (B.RA_BF16, 128, 2048, False),
    (B.RA_BF16, 128, 2047, True),
])
def test_forward_grid_checked_against_the_kernels_real_tiles(L, dtype, head_dim, batch, ok):
    st, msg = _fwd_status(L, _grid_prob(dtype=dtype, head_dim=head_dim, batch=batch))
    assert st == B.RA_ERR_INVALID_ARG
    if ok:
        assert "q is NULL" in msg, msg
    else:
        assert "too large for one launch of the attention kernel" in msg, msg
    prob = _grid_prob(dtype=dtype, head_dim=head_dim, batch=batch)
    st = L.ra_ring_fwd(ctypes.byref(prob), None, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None, None)
    assert st == B.RA_ERR_INVALID_ARG
    assert ("q is NULL" in L.ra_last_error().decode()) == ok


def test_backward_grid_checks_both_kernels(L):
    # one query row against 2^26 keys per head: the dq launch is tiny, the dk/dv
    # launch (128 keys and 256 work items per workgroup) needs 2^27 work items
    # per head, so 32 heads are one too many for a dispatch
    big = _grid_prob(head_dim=16, q_len=1, kv_len=1 << 26, batch=32)
    st, msg = _bwd_status(L, big)
    assert st == B.RA_ERR_INVALID_ARG and "dk/dv kernel" in msg, msg
    st, msg = _fwd_status(L, big)   # the forward launch is small
    assert st == B.RA_ERR_INVALID_ARG and "q is NULL" in msg, msg
    st, msg = _bwd_status(L, _grid_prob(head_dim=16, q_len=1, kv_len=1 << 26, batch=31))
    assert st == B.RA_ERR_INVALID_ARG and "q is NULL" in msg, msg
    # the dq launch (256 rows, 512 work items) binds on a long query share
    st, msg = _bwd_status(L, _grid_prob(batch=2048))
    assert st == B.RA_ERR_INVALID_ARG and "dq kernel" in msg, msg
    prob = _grid_prob(batch=2048)
    st = L.ra_ring_bwd(ctypes.byref(prob), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                       FAKE, 1 << 40, None, None)
    assert st == B.RA_ERR_INVALID_ARG and b"dq kernel" in L.ra_last_error()


def test_noalloc_validation_before_any_hip_call(L):
    """The allocation-free ring refuses, with no HIP call, an invalid problem,
    missing tensors, and a share whose workspace exceeds its static array."""
    big = _prob(n_ring=8, rank=7, q_len=2048, kv_len=2048, hq=32, hkv=32, head_dim=128)
    assert L.ra_ring_workspace_bytes(ctypes.byref(big)) > B.RA_NOALLOC_WORKSPACE_BYTES
    assert L.ra_ring_fwd_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, None, None, None) \
        == B.RA_ERR_WORKSPACE
    assert b"static workspace" in L.ra_last_error()
    assert L.ra_ring_fwd_noalloc(ctypes.byref(big), None, FAKE, FAKE, FAKE, None, None, None) \
        == B.RA_ERR_INVALID_ARG
    assert b"q is NULL" in L.ra_last_error()
    bad = _prob(hq=6, hkv=4)
    assert L.ra_ring_fwd_noalloc(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, None, None, None) \
        == B.RA_ERR_INVALID_ARG
    assert L.ra_ring_fwd_noalloc(None, FAKE, FAKE, FAKE, FAKE, None, None, None) \
        == B.RA_ERR_INVALID_ARG


def test_bad_layout_and_causal_flags(L):
    prob = _prob()
    prob.layout = 5
    assert _partial(L, prob) == B.RA_ERR_INVALID_ARG
    prob = _prob()
    prob.causal = 2
    assert _partial(L, prob) == B.RA_ERR_INVALID_ARG


def test_pointer_checks(L):
    prob = _prob()
    assert L.ra_block_attn_partial(ctypes.byref(prob), 0, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None) == B.RA_ERR_INVALID_ARG
    assert b"q is NULL" in L.ra_last_error()
    odd = ctypes.c_void_p(0x10008)
    assert L.ra_block_attn_partial(ctypes.byref(prob), 0, FAKE, odd, FAKE, FAKE, FAKE, FAKE,
                                   None) == B.RA_ERR_INVALID_ARG
    assert b"aligned" in L.ra_last_error()
    # j out of range
    assert _partial(L, prob, j=4) == B.RA_ERR_INVALID_ARG
    assert L.ra_block_attn_partial(ctypes.byref(prob), 0, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None) == B.RA_ERR_INVALID_ARG
    assert L.ra_block_attn_partial(None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) \
        == B.RA_ERR_INVALID_ARG


def test_output_aliasing_rejected(L):
    prob = _prob()
    base = 0x100000
    q = ctypes.c_void_p(base)
    acc = ctypes.c_void_p(base + 64)  # inside q
    other = ctypes.c_void_p(0x40000000)
    st = L.ra_block_attn_partial(ctypes.byref(prob), 0, q, other, other, ctypes.c_void_p(0x50000000),
                                 ctypes.c_void_p(0x60000000), acc, None)
    assert st == B.RA_ERR_INVALID_ARG
    assert b"overlap" in L.ra_last_error()


def test_merge_validation(L):
    p = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(9)]
    assert L.ra_merge_partials(-1, 64, *p, None) == B.RA_ERR_INVALID_ARG
    assert L.ra_merge_partials(10, 48, *p, None) == B.RA_ERR_UNSUPPORTED
    # acc_out partially overlapping acc1 is rejected, exact aliasing is allowed (and then
    # the call would run, so only the rejection is checked here)
    q = list(p)
    q[8] = ctypes.c_void_p(p[2].value + 16)
    assert L.ra_merge_partials(10, 64, *q, None) == B.RA_ERR_INVALID_ARG
    # rows == 0: nothing to do, no HIP call
    assert L.ra_merge_partials(0, 64, *p, None) == B.RA_OK
    assert L.ra_finalize(-2, 64, p[0], p[1], p[2], None, None) == B.RA_ERR_INVALID_ARG
    assert L.ra_finalize(0, 64, p[0], p[1], p[2], None, None) == B.RA_OK


def test_ring_workspace_size_and_checks(L):
    prob = _prob(batch=2, hq=8, hkv=2, head_dim=128, q_len=1000, kv_len=1000, n_ring=8, rank=7)
    got = L.ra_ring_workspace_bytes(ctypes.byref(prob))
    blk = 2 * 1000 * 2 * 128 * 2
    rows = 2 * 1000 * 8
    def a(x):
        return (x + 255) // 256 * 256
    want = 4 * a(blk) + 2 * a(rows * 4)
    assert got == want
    ws_small = ctypes.c_size_t(got - 1)
    buf = [ctypes.c_void_p(0x1000000 * (i + 1)) for i in range(5)]
    st = L.ra_ring_fwd(ctypes.byref(prob), buf[0], buf[1], buf[2], buf[3], None, buf[4],
                       ws_small, None, None)
    assert st == B.RA_ERR_WORKSPACE
    st = L.ra_ring_fwd(ctypes.byref(prob), buf[0], buf[1], buf[2], buf[3], None, None,
                       ctypes.c_size_t(got), None, None)
    assert st == B.RA_ERR_WORKSPACE
    # empty share: nothing to do
    empty = _prob(q_len=0, kv_len=0)
    assert L.ra_ring_fwd(ctypes.byref(empty), None, None, None, None, None, None, 0, None, None) \
        == B.RA_OK


# ---- causal tile scheduler: host mirror vs oracle brute force --------------
@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_tile_classes_host_match_bruteforce(L, layout):
    sizes = [1, 2, 4, 8, 16]
    for n, blen in [(2, 8), (3, 13), (4, 16), (8, 9), (1, 5)]:
        for tq, tk in itertools.product(sizes, sizes):
            for r, j in itertools.product(range(n), range(n)):
                for causal in (True, False):
                    prob = _prob(n_ring=n, rank=r, q_len=blen, kv_len=blen, causal=causal,
                                 layout=layout)
                    got = B.ra_tile_classes_host(prob, j, tq, tk)
                    want = orc.tile_classes_bruteforce(layout, causal, n, r, j, blen, blen, tq, tk)
                    mapped = np.vectorize(_ORACLE_CLASS.get)(got)
                    np.testing.assert_array_equal(mapped, want)


def _counts(got):
    c = np.bincount(got.ravel().astype(np.int64), minlength=3)
    return int(c[B.RA_TILE_FULL]), int(c[B.RA_TILE_PARTIAL]), int(c[B.RA_TILE_SKIP])


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("tq,tk", [(128, 128), (64, 32)])
def test_tile_classes_host_real_size_counts(L, layout, tq, tk):
    """1M-token share, 8 blocks of 131072: the host mirror's class counts
    equal the oracle's O(#tiles) counts for every rank and block, with
    128 x 128 tiles and with the attention kernel's own unit (a workgroup's
    256 rows are 64 positions x 4 heads at GQA 32/8; keys go in units of
    32)."""
    blen = 131072
    for r, j in itertools.product(range(8), range(8)):
        prob = _prob(n_ring=8, rank=r, q_len=blen, kv_len=blen, layout=layout)
        got = B.ra_tile_classes_host(prob, j, tq, tk)
        assert _counts(got) == orc.tile_class_counts(layout, True, 8, r, j, blen, blen, tq, tk), \
            (layout, r, j)


def test_tile_class_single(L):
    prob = _prob(n_ring=8, rank=3, q_len=16, kv_len=16, layout="striped")
    assert B.ra_tile_class_host(prob, 5, 4, 7, 4, 7) == B.RA_TILE_PARTIAL  # delta 1 diagonal
    assert B.ra_tile_class_host(prob, 5, 4, 7, 0, 3) == B.RA_TILE_FULL
    assert B.ra_tile_class_host(prob, 5, 0, 3, 4, 7) == B.RA_TILE_SKIP
    with pytest.raises(B.RaError):
        B.ra_tile_class_host(prob, 5, 0, 16, 0, 3)


# ---- zigzag layout and packed sequences -------------------------------------
def test_tile_classes_host_zigzag_match_bruteforce(L):
    sizes = [1, 2, 3, 4, 8, 16]
    for n, blen in [(2, 8), (3, 12), (4, 16), (1, 6), (8, 2)]:
        for tq, tk in itertools.product(sizes, sizes):
            for r, j in itertools.product(range(n), range(n)):
                for causal in (True, False):
                    prob = _prob(n_ring=n, rank=r, q_len=blen, kv_len=blen, causal=causal,
                                 layout="zigzag")
                    got = B.ra_tile_classes_host(prob, j, tq, tk)
                    want = orc.tile_classes_bruteforce("zigzag", causal, n, r, j, blen, blen, tq, tk)
                    np.testing.assert_array_equal(np.vectorize(_ORACLE_CLASS.get)(got), want)


PACKED = {
    "contiguous": [3, 9, 0, 6, 3],
    "striped": [6, 3, 12, 0],
    "zigzag": [6, 12, 0, 18, 6],
}


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_tile_classes_host_packed_match_bruteforce(L, layout):
    n, lens = 3, PACKED[layout]
    cu = np.concatenate([[0], np.cumsum(lens)])
    blen = int(cu[-1]) // n
    for tq, tk in itertools.product([1, 2, 3, 5, 16], [1, 2, 4, 7]):
        for r, j in itertools.product(range(n), range(n)):
            for causal in (True, False):
                prob = _prob(n_ring=n, rank=r, q_len=blen, kv_len=blen, causal=causal,
                             layout=layout, cu_seqlens=cu)
                got = B.ra_tile_classes_host(prob, j, tq, tk)
                want = orc.tile_classes_bruteforce(layout, causal, n, r, j, blen, blen, tq, tk,
                                                   seqlens=lens)
                np.testing.assert_array_equal(np.vectorize(_ORACLE_CLASS.get)(got), want)


@pytest.mark.parametrize("kw,msg", [
    (dict(layout="zigzag", q_len=255, kv_len=255), b"even"),
    (dict(cu_seqlens=[0, 512, 1024], batch=2), b"batch == 1"),
    (dict(cu_seqlens=[0, 512, 1022]), b"multiple"),
    (dict(cu_seqlens=[0, 600, 512, 1024]), b"decreases"),
    (dict(cu_seqlens=[4, 512, 1024]), b"cu_seqlens[0]"),
    (dict(cu_seqlens=[0, 512, 1020]), b"expected q_len * n_ring"),
    (dict(cu_seqlens=[0, 510, 1024]), b"multiple"),
    (dict(cu_seqlens=[0, 512, 1032]), b"expected q_len * n_ring"),
    (dict(cu_seqlens=[0, 4, 1024], layout="zigzag"), b"multiple of 8"),
    (dict(cu_seqlens=[0, 512, 1024], q_len=256, kv_len=512, causal=0), b"q_len == kv_len"),
    (dict(cu_seqlens=[0] + [4] * 256 + [1024]), b"n_seqs"),
])
def test_packed_and_zigzag_validation(L, kw, msg):
    prob = _prob(**kw)
    assert _partial(L, prob) == B.RA_ERR_INVALID_ARG
    assert msg in L.ra_last_error(), L.ra_last_error()
    assert L.ra_ring_workspace_bytes(ctypes.byref(prob)) == 0


def test_packed_problem_accepted(L):
    prob = _prob(cu_seqlens=[0, 0, 512, 516, 1024])
    assert L.ra_ring_workspace_bytes(ctypes.byref(prob)) > 0
    prob = _prob(cu_seqlens=[0] + [4] * 255 + [1024])  # 256 sequences, all but one empty
    assert L.ra_ring_workspace_bytes(ctypes.byref(prob)) > 0
    prob = _prob(layout="zigzag", cu_seqlens=[0, 8, 1024])
    assert L.ra_ring_workspace_bytes(ctypes.byref(prob)) > 0


# ---- backward entry points ---------------------------------------------------
def test_backward_validation_before_any_hip_call(L):
    bad = _prob(head_dim=96)
    args = [FAKE] * 9
    assert L.ra_block_attn_bwd(ctypes.byref(bad), 0, *args, None) == B.RA_ERR_UNSUPPORTED
    assert L.ra_ring_bwd_workspace_bytes(ctypes.byref(bad)) == 0
    prob = _prob()
    assert L.ra_block_attn_bwd(ctypes.byref(prob), 9, *args, None) == B.RA_ERR_INVALID_ARG
    assert b"kv_block_j" in L.ra_last_error()
    a = [FAKE] * 9
    a[3] = None  # dout
    assert L.ra_block_attn_bwd(ctypes.byref(prob), 0, *a, None) == B.RA_ERR_INVALID_ARG
    assert b"dout is NULL" in L.ra_last_error()
    # dq aliasing q is refused
    assert L.ra_block_attn_bwd(ctypes.byref(prob), 0, *args, None) == B.RA_ERR_INVALID_ARG
    assert b"overlap" in L.ra_last_error()
    assert L.ra_attn_bwd_delta(10, 64, 5, FAKE, FAKE, FAKE, None) == B.RA_ERR_INVALID_ARG
    assert L.ra_attn_bwd_delta(10, 48, B.RA_BF16, FAKE, FAKE, FAKE, None) == B.RA_ERR_UNSUPPORTED
    assert L.ra_attn_bwd_delta(0, 64, B.RA_BF16, None, None, None, None) == B.RA_OK


def test_ring_bwd_workspace_and_checks(L):
    prob = _prob(n_ring=4, q_len=256, kv_len=256)
    need = L.ra_ring_bwd_workspace_bytes(ctypes.byref(prob))
    blk = 1 * 256 * 2 * 64 * 2
    rows = 1 * 256 * 4
    assert need >= 4 * blk + rows * 4
    base = 0x100000
    ptr = lambda off: ctypes.c_void_p(base + off)  # noqa: E731
    big = 1 << 24
    args = [ptr(i * big) for i in range(9)]  # q k v out dout lse dq dk dv
    assert L.ra_ring_bwd(ctypes.byref(prob), *args, None, 0, None, None) == B.RA_ERR_WORKSPACE
    assert L.ra_ring_bwd(ctypes.byref(prob), *args, ptr(11 * big), need - 1, None, None) \
        == B.RA_ERR_WORKSPACE
    assert b"workspace of" in L.ra_last_error()
    # workspace overlapping dq
    assert L.ra_ring_bwd(ctypes.byref(prob), *args, ptr(6 * big), need, None, None) \
        == B.RA_ERR_INVALID_ARG
    one = _prob(n_ring=1, rank=0)
    assert L.ra_ring_bwd_workspace_bytes(ctypes.byref(one)) < need  # no staging buffers


def test_rope_validation(L):
    prob = _prob(rope_theta=float("nan"))
    assert _partial(L, prob) == B.RA_ERR_INVALID_ARG
    prob = _prob(rope_theta=-1.0)
    assert _partial(L, prob) == B.RA_ERR_INVALID_ARG
    p0 = _prob()  # rope_theta 0: ra_rope_apply refuses
    assert L.ra_rope_apply(ctypes.byref(p0), 1, 0, 2, B.RA_BF16, FAKE, B.RA_BF16, FAKE, 0, 0, None) \
        == B.RA_ERR_INVALID_ARG
    p = _prob(rope_theta=10000.0)
    assert L.ra_rope_apply(ctypes.byref(p), 5, 0, 2, B.RA_BF16, FAKE, B.RA_BF16, FAKE, 0, 0, None) \
        == B.RA_ERR_INVALID_ARG
    assert L.ra_rope_apply(ctypes.byref(p), 1, 4, 2, B.RA_BF16, FAKE, B.RA_BF16, FAKE, 0, 0, None) \
        == B.RA_ERR_INVALID_ARG  # block out of range
    assert L.ra_rope_apply(ctypes.byref(p), 1, 0, 2, B.RA_BF16, FAKE, B.RA_BF16, FAKE, 0, 1, None) \
        == B.RA_ERR_INVALID_ARG  # accumulate into bf16
    assert L.ra_rope_apply(ctypes.byref(p), 1, 0, 2, B.RA_F32, FAKE, B.RA_BF16, FAKE, 0, 0, None) \
        == B.RA_ERR_INVALID_ARG  # in place with different dtypes
    assert L.ra_ring_workspace_bytes(ctypes.byref(p)) > L.ra_ring_workspace_bytes(ctypes.byref(_prob()))


def test_debug_switches_leave_validation_before_any_hip_call(L, monkeypatch):
    """RA_DEBUG_SYNC / RA_DEBUG_POISON only act after a call's launches: an
    invalid call still returns its status with no HIP call (no GPU here)."""
    monkeypatch.setenv("RA_DEBUG_SYNC", "1")
    monkeypatch.setenv("RA_DEBUG_POISON", "1")
    prob = _prob()
    prob.layout = 5
    assert _partial(L, prob) == B.RA_ERR_INVALID_ARG
    big = _prob(n_ring=8, rank=7, q_len=2048, kv_len=2048, hq=32, hkv=32, head_dim=128)
    assert L.ra_ring_fwd_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, None, None, None) \
        == B.RA_ERR_WORKSPACE
    assert L.ra_merge_partials(-1, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               None) == B.RA_ERR_INVALID_ARG
