"""Plain, slow, obviously-correct CPU oracle for one device's share of Ring
Attention, in float64 NumPy.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no
code with the HIP library (no kernels, headers, helpers or tables); the only
thing both sides use is the seeded input generator module, which holds no
attention arithmetic.

Pages cited (by title and section; the pages are web text on Ring Attention):

  [UL] Ultralytics glossary, "Ring Attention" (Arabic edition), section
       "How ring attention works": the N-step schedule, the four-device
       single-process simulation, the remark that production kernels subtract
       a running maximum, and the remark on striped token assignment.
  [TS] troisinh.com, "Ring Attention -- K/V truyen vong giua GPU, context
       trieu token": sections "Y tuong cot loi" (core idea: fixed Q, K/V
       rotating, associative merge), "Tai sao no hoat dong" (why it works: the
       online-softmax update of the running max and normaliser, output
       rescaled the same way) and "Y nghia thuc te" (practical implications:
       causal masking wastes about half of the FLOPs).
  [JS] jisaku.com glossary, "Ring Attention (ring attention)": sections on the
       processing flow (step t uses the block received at step t-1) and on
       communication/compute overlap.
  [AU] AI Understanding, "Sekvensparallellism och ringuppmarksamhet": sections
       "Djupdykning" (each device owns a contiguous chunk of tokens),
       "Teknisk insikt" (online softmax makes blockwise equal to full
       attention) and "Framtiden for sekvensparallellism och
       ringuppmarksamhet" (striped and zigzag variants rebalance the work
       that causal masking leaves uneven).
  [TS] also, section "Trade-off thuc te" (practical trade-offs): balancing
       sequences of different lengths is named as a difficulty; and section
       "Blockwise Backward": the backward pass does not keep the attention
       matrix but recomputes the attention statistics, each device only on
       the K/V block visiting it; and section "RoPE va Position Embedding":
       a key block arriving from another device must be rotated by the angle
       m*theta of each token's own position m, carried as position metadata
       with the block.

Conventions
  * Tensors are [batch, seq, heads, head_dim] (the shape convention of the
    package call shown on the [JS] page).
  * Query head h reads KV head floor(h * Hkv / Hq) (grouped-query attention;
    the pages are silent, this is the plain reading).
  * scale defaults to 1/sqrt(head_dim), applied to the scores before the
    softmax ([UL] simulation divides the scores by the square root of dim).
  * Causal: a key is visible to a query iff its global position is <= the
    query's global position ([TS] "Y nghia thuc te": autoregressive masking).
  * Layouts: "contiguous" -- block i holds tokens [i*B, (i+1)*B) ([AU]
    "Djupdykning"); "striped" -- token t belongs to block t mod N at local
    index floor(t / N) ([UL] closing remark: each device receives tokens
    spread evenly over the sequence); "zigzag" -- the sequence is cut into
    2N chunks of B/2 tokens and block i holds chunk i followed by chunk
    2N-1-i ([AU] names zigzag as a rebalancing variant without defining it;
    this pairing of an early with a late chunk is the plain reading, and it
    gives every device the same causal work).
  * Packed variable-length sequences ([TS] "Trade-off thuc te"): several
    sequences of lengths L_s (each a multiple of N, of 2N for zigzag) are
    concatenated; every sequence is split over the N blocks by the layout on
    its own, and a block is the concatenation of its slices, sequence by
    sequence. A key is visible to a query only inside the same sequence
    (and, if causal, at a position within that sequence <= the query's).
  * A partial is (m, l, acc): m = max visible scaled score, l = sum of
    exp(s - m), acc = sum of exp(s - m) * v. A row with no visible key has
    the empty partial (-inf, 0, 0), which is the identity of the merge.

Every function is pinned by tests under tests/ against values the pages fix,
closed forms, invariants, brute force and library routines (see the
docstrings). No function here is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

# Tile classes. The integer values are this module's own; tests compare the
# HIP library's classes through an explicit mapping, not through shared code.
SKIP = 0
PARTIAL = 1
FULL = 2

_LAYOUTS = ("contiguous", "striped", "zigzag")


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def default_scale(head_dim: int) -> float:
    """1/sqrt(d): the [UL] simulation divides q.k by dim ** 0.5."""
    return 1.0 / math.sqrt(head_dim)


def kv_head_of(h: int, hq: int, hkv: int) -> int:
    """KV head read by query head h: floor(h*Hkv/Hq) (groups of Hq/Hkv)."""
    return (h * hkv) // hq


def global_positions(layout: str, n_ring: int, block: int, block_len: int) -> np.ndarray:
    """Global token positions of the block_len tokens of ring block `block`.

    contiguous: [AU] "Djupdykning" -- each device owns one contiguous chunk,
                so position = block*block_len + a.
    striped:    [UL] "How ring attention works", closing remark on striping --
                tokens are spread evenly: token t -> block t mod N, local index
                t // N, so position = a*N + block.
    zigzag:     [AU] "Framtiden ..." -- chunks of h = block_len/2 tokens;
                local a < h is chunk `block`, a >= h is chunk 2N-1-block:
                position = c*h + (a mod h) for that chunk c.
    Pinned by tests: positions of all blocks partition range(N*B) exactly;
    local order is increasing in position; zigzag gives every rank the same
    number of causal pairs.
    """
    if layout not in _LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}")
    a = np.arange(block_len, dtype=np.int64)
    if layout == "contiguous":
        return block * block_len + a
    if layout == "striped":
        return a * n_ring + block
    if block_len % 2:
        raise ValueError("zigzag needs an even block length")
    h = block_len // 2
    chunk = np.where(a < h, block, 2 * n_ring - 1 - block)
    return chunk * h + (a % h)


def varlen_positions(layout: str, n_ring: int, block: int, seqlens):
    """(sequence id, position within the sequence) of every token of ring
    block `block` when sequences of lengths `seqlens` are packed: the block
    holds, sequence after sequence, the L_s / N tokens the layout gives it
    from each sequence ([TS] "Trade-off thuc te"; layouts as above).
    Pinned by tests: over all blocks, the (id, position) pairs of each
    sequence partition range(L_s)."""
    ids, pos = [], []
    for s, L in enumerate(seqlens):
        L = int(L)
        mult = 2 * n_ring if layout == "zigzag" else n_ring
        if L % mult:
            raise ValueError(f"sequence {s}: length {L} is not a multiple of {mult}")
        b = L // n_ring
        ids.append(np.full(b, s, dtype=np.int64))
        pos.append(global_positions(layout, n_ring, block, b))
    if not ids:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    return np.concatenate(ids), np.concatenate(pos)


def ring_order(rank: int, n_ring: int) -> list[int]:
    """Block visited at each step: j = (rank - step) mod N ([UL] simulation:
    at each step the device uses the block that arrived from the previous
    device; [JS] processing flow: step 0 is the device's own block)."""
    return [(rank - s) % n_ring for s in range(n_ring)]


def _visibility(q_pos: np.ndarray, k_pos: np.ndarray, causal: bool,
                q_seq: np.ndarray | None = None, k_seq: np.ndarray | None = None) -> np.ndarray:
    """[Lq, Lk] boolean: key visible to query (causal: key pos <= query pos;
    packed sequences: also the same sequence id)."""
    if not causal:
        vis = np.ones((q_pos.size, k_pos.size), dtype=bool)
    else:
        vis = k_pos[None, :] <= q_pos[:, None]
    if q_seq is not None:
        vis = vis & (k_seq[None, :] == q_seq[:, None])
    return vis


# --------------------------------------------------------------------------
# O1 -- the plain definition, global token order.
# --------------------------------------------------------------------------

def naive_attention(q, k, v, causal: bool, scale: float | None = None):
    """O = softmax(scale * Q K^T [+ causal mask]) V over the whole sequence.

    q: [B, S, Hq, d]; k, v: [B, S, Hkv, d], all in global token order.
    Returns (out [B, S, Hq, d] float64, lse [B, S, Hq] float64).
    This is exact attention, the result ring attention must reproduce
    ([UL] opening paragraph: no approximation of attention; [TS] "Tai sao no
    hoat dong": the softmax with the row max subtracted).
    Pinned by: torch CPU scaled_dot_product_attention in float64 (tiny
    shapes), closed forms (constant keys -> mean of V; causal row 0 -> V[0]),
    the affine-V invariant.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    pos = np.arange(q.shape[1], dtype=np.int64)
    return naive_attention_rows(q, pos, k, v, causal, scale)


def naive_attention_rows(q_rows, q_pos, k, v, causal: bool, scale: float | None = None):
    """O1 for a subset of query rows.

    q_rows: [B, R, Hq, d] with global positions q_pos [R]; k, v: [B, S, Hkv, d]
    in global order (key u has position u). Used for sampled-row parity at
    sizes where the full product is too large for a CPU.
    """
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    bsz, nrows, hq, d = q_rows.shape
    hkv = k.shape[2]
    if scale is None:
        scale = default_scale(d)
    k_pos = np.arange(k.shape[1], dtype=np.int64)
    out = np.zeros((bsz, nrows, hq, d))
    lse = np.full((bsz, nrows, hq), -np.inf)
    for b in range(bsz):
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            kk, vv = k[b, :, g, :], v[b, :, g, :]
            if causal:
                # only keys up to the largest query position can be visible
                kmax = int(q_pos.max()) + 1
                kk, vv, kp = kk[:kmax], vv[:kmax], k_pos[:kmax]
            else:
                kp = k_pos
            s = (q_rows[b, :, h, :] @ kk.T) * scale
            vis = _visibility(q_pos, kp, causal)
            s = np.where(vis, s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            has = np.isfinite(mx)
            base = np.where(has, mx, 0.0)
            e = np.where(vis, np.exp(s - base), 0.0)
            den = e.sum(axis=1, keepdims=True)
            safe = np.where(den > 0, den, 1.0)
            out[b, :, h, :] = np.where(den > 0, (e / safe) @ vv, 0.0)
            lse[b, :, h] = np.where(has[:, 0], base[:, 0] + np.log(safe[:, 0]), -np.inf)
    return out, lse


def naive_attention_varlen(q, k, v, cu_seqlens, causal: bool, scale: float | None = None):
    """O1 for packed sequences: plain attention of each sequence on its own.

    q: [1, T, Hq, d]; k, v: [1, T, Hkv, d] in global packed order, sequence s
    occupying tokens [cu_seqlens[s], cu_seqlens[s+1]). Returns (out, lse) of
    shape [1, T, Hq, d] and [1, T, Hq].
    Pinned by: torch CPU scaled_dot_product_attention with a block-diagonal
    mask in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    out = np.zeros(q.shape)
    lse = np.full(q.shape[:3], -np.inf)
    cu = [int(x) for x in cu_seqlens]
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b > a:
            o, l_ = naive_attention(q[:, a:b], k[:, a:b], v[:, a:b], causal, scale)
            out[:, a:b], lse[:, a:b] = o, l_
    return out, lse


# --------------------------------------------------------------------------
# O2 -- blockwise ring with online-softmax merge (separate code from O1).
# --------------------------------------------------------------------------

def empty_partial(bsz: int, lq: int, hq: int, d: int):
    """(-inf, 0, 0): the state before any block arrives. The [UL] simulation
    starts numerator and denominator at zero; the running max starts at -inf
    so that the first merge takes the block's own max."""
    return (np.full((bsz, lq, hq), -np.inf), np.zeros((bsz, lq, hq)), np.zeros((bsz, lq, hq, d)))


def block_partial(q, q_pos, k, v, k_pos, causal: bool, scale: float | None = None,
                  q_seq=None, k_seq=None):
    """Partial (m, l, acc) of the local queries against one arriving K/V block.

    [UL] "How ring attention works": each device keeps a running sum of the
    exponentiated scores and a running sum of the weighted values; production
    kernels subtract a running maximum before exponentiating. So for each query
    row: m = max of visible scaled scores, l = sum exp(s - m),
    acc = sum exp(s - m) v. A row with no visible key gets (-inf, 0, 0).

    q: [B, Lq, Hq, d] with positions q_pos [Lq]; k, v: [B, Lk, Hkv, d] with
    positions k_pos [Lk]. q_seq, k_seq: sequence ids of packed sequences
    (None: one sequence).
    Pinned by: m equals the exact max of visible scores and 1 <= l <= #visible
    (invariant); merged over all blocks equals O1 (brute force, SDPA).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    bsz, lq, hq, d = q.shape
    hkv = k.shape[2]
    if scale is None:
        scale = default_scale(d)
    vis = _visibility(np.asarray(q_pos, np.int64), np.asarray(k_pos, np.int64), causal,
                      None if q_seq is None else np.asarray(q_seq, np.int64),
                      None if k_seq is None else np.asarray(k_seq, np.int64))
    has = vis.any(axis=1)
    m, l, acc = empty_partial(bsz, lq, hq, d)
    for b in range(bsz):
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            s = (q[b, :, h, :] @ k[b, :, g, :].T) * scale
            s_vis = np.where(vis, s, -np.inf)
            mrow = s_vis.max(axis=1)
            base = np.where(has, mrow, 0.0)
            p = np.where(vis, np.exp(s - base[:, None]), 0.0)
            m[b, :, h] = np.where(has, mrow, -np.inf)
            l[b, :, h] = p.sum(axis=1)
            acc[b, :, h, :] = p @ v[b, :, g, :]
    return m, l, acc


def merge_partials(p1, p2):
    """Online-softmax merge of two partials ([TS] "Tai sao no hoat dong"):
        m = max(m1, m2)
        l = exp(m1 - m) l1 + exp(m2 - m) l2
        acc = exp(m1 - m) acc1 + exp(m2 - m) acc2   (output rescaled the same way)
    A side whose m is -inf contributes a factor of exactly 0; if both are -inf
    the result stays the empty partial (no NaN).
    Pinned by: merge algebra (identity, merge(x, x), commutativity,
    associativity) and ring == O1.
    """
    m1, l1, a1 = p1
    m2, l2, a2 = p2
    m = np.maximum(m1, m2)
    fin = np.isfinite(m)
    base = np.where(fin, m, 0.0)
    f1 = np.where(np.isfinite(m1), np.exp(np.where(np.isfinite(m1), m1, 0.0) - base), 0.0)
    f2 = np.where(np.isfinite(m2), np.exp(np.where(np.isfinite(m2), m2, 0.0) - base), 0.0)
    l = f1 * l1 + f2 * l2
    acc = f1[..., None] * a1 + f2[..., None] * a2
    return np.where(fin, m, -np.inf), l, acc


def finalize(state):
    """Divide the accumulated numerator by the denominator at the end ([UL]
    "How ring attention works"). Also returns lse = m + ln l (the statistic a
    backward pass recomputes from, [TS] "Tai sao no hoat dong", blockwise
    backward). Rows with l == 0 give out = 0 and lse = -inf."""
    m, l, acc = state
    pos = l > 0
    safe = np.where(pos, l, 1.0)
    out = np.where(pos[..., None], acc / safe[..., None], 0.0)
    lse = np.where(pos, m + np.log(safe), -np.inf)
    return out, lse


def ring_state(q_share, k_blocks, v_blocks, rank: int, n_ring: int, layout: str,
               causal: bool, scale: float | None = None, blocks=None, state=None,
               seqlens=None):
    """Running (m, l, acc) after visiting `blocks` (default: the ring order of
    `rank`), starting from `state` (default: empty).

    q_share: [B, Lq, Hq, d] -- the local query block, fixed for the whole ring
    ([TS] "Y tuong cot loi"; [JS] ring structure). k_blocks, v_blocks:
    [N, B, Lk, Hkv, d] -- block j holds the tokens the layout gives to block j.
    seqlens: lengths of packed sequences (batch 1), or None for one sequence
    per batch row.
    Pinned by: the split-ring invariant (state after k steps merged with the
    rest equals the whole ring).
    """
    q_share = _f64(q_share)
    bsz, lq, hq, d = q_share.shape
    lk = k_blocks.shape[2]
    if seqlens is None:
        q_pos, q_seq = global_positions(layout, n_ring, rank, lq), None
    else:
        q_seq, q_pos = varlen_positions(layout, n_ring, rank, seqlens)
    if blocks is None:
        blocks = ring_order(rank, n_ring)
    if state is None:
        state = empty_partial(bsz, lq, hq, d)
    for j in blocks:
        if seqlens is None:
            k_pos, k_seq = global_positions(layout, n_ring, j, lk), None
        else:
            k_seq, k_pos = varlen_positions(layout, n_ring, j, seqlens)
        part = block_partial(q_share, q_pos, k_blocks[j], v_blocks[j], k_pos, causal, scale,
                             q_seq, k_seq)
        state = merge_partials(state, part)
    return state


def ring_share(q_share, k_blocks, v_blocks, rank: int, n_ring: int, layout: str,
               causal: bool, scale: float | None = None, order=None, seqlens=None):
    """O2: one device's output after all N ring steps, (out, lse).

    Steps follow ring_order(rank) unless `order` (any permutation of the N
    blocks) is given; the result does not depend on it (merge is associative
    and commutative, [TS] "Y tuong cot loi").
    Pinned by: equality with O1 on the [UL] worked example and on brute-force
    tiny cases, arrival-order invariance, torch SDPA.
    """
    return finalize(ring_state(q_share, k_blocks, v_blocks, rank, n_ring, layout,
                               causal, scale, blocks=order, seqlens=seqlens))


def ring_share_literal(q_share, k_blocks, v_blocks, rank: int, n_ring: int,
                       scale: float | None = None):
    """O2': the [UL] simulation's own formulation, non-causal, without max
    subtraction: numerator += exp(s) v, denominator += sum exp(s), one divide at
    the end. Exact in real arithmetic; used on small-score inputs only.
    Pinned by: the [UL] printed result (matches full attention within 1e-5)."""
    q_share = _f64(q_share)
    bsz, lq, hq, d = q_share.shape
    hkv = k_blocks.shape[3]
    if scale is None:
        scale = default_scale(d)
    num = np.zeros((bsz, lq, hq, d))
    den = np.zeros((bsz, lq, hq))
    for j in ring_order(rank, n_ring):
        kb, vb = _f64(k_blocks[j]), _f64(v_blocks[j])
        for b in range(bsz):
            for h in range(hq):
                g = kv_head_of(h, hq, hkv)
                e = np.exp((q_share[b, :, h, :] @ kb[b, :, g, :].T) * scale)
                num[b, :, h, :] += e @ vb[b, :, g, :]
                den[b, :, h] += e.sum(axis=1)
    return num / den[..., None]


# --------------------------------------------------------------------------
# Rotary position embedding ([TS] "RoPE va Position Embedding").
#
# The page fixes only that a token at position m is rotated by the angle
# m*theta. The plain reading, the rotary embedding's usual form: head
# dimensions pair up as (2i, 2i+1), pair i turns by m * theta_i with
# theta_i = base^(-2i/d) (base 10000 by default), counter-clockwise:
#   (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a),  a = m theta_i.
# q and k are rotated (v is not); the scores then depend on positions only
# through m - n. Positions are global positions (packed sequences: positions
# within the sequence).
# --------------------------------------------------------------------------

def rope_angles(pos, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """[len(pos), head_dim/2] angles m * base^(-2i/d) in float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]


def rope_rotate(x, pos, base: float = 10000.0, inverse: bool = False) -> np.ndarray:
    """Rotate x [B, L, H, d] (token t at position pos[t]) pairwise as above;
    inverse=True turns by -a (the transpose, used on gradients).
    Pinned by: complex-number multiplication, a hand-worked d=4 case,
    orthogonality, the relative-position property."""
    x = _f64(x)
    a = rope_angles(pos, x.shape[-1], base)
    if inverse:
        a = -a
    c, s_ = np.cos(a)[None, :, None, :], np.sin(a)[None, :, None, :]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s_
    y[..., 1::2] = x0 * s_ + x1 * c
    return y


def ring_share_rope(q_share, k_blocks, v_blocks, rank: int, n_ring: int, layout: str,
                    causal: bool, base: float = 10000.0, scale: float | None = None, seqlens=None):
    """O2 with rotary embedding applied on arrival: the local queries are
    rotated by their own positions once, and every arriving key block by the
    positions of its tokens (the block's position metadata) before its
    partial is formed. Returns (out, lse) as ring_share.
    Pinned by: equality with plain attention on globally rotated q, k."""
    lq, lk = q_share.shape[1], k_blocks.shape[2]
    if seqlens is None:
        qp = global_positions(layout, n_ring, rank, lq)
        kps = [global_positions(layout, n_ring, j, lk) for j in range(n_ring)]
    else:
        qp = varlen_positions(layout, n_ring, rank, seqlens)[1]
        kps = [varlen_positions(layout, n_ring, j, seqlens)[1] for j in range(n_ring)]
    qr = rope_rotate(q_share, qp, base)
    kr = np.stack([rope_rotate(k_blocks[j], kps[j], base) for j in range(n_ring)])
    return ring_share(qr, kr, v_blocks, rank, n_ring, layout, causal, scale, seqlens=seqlens)


# --------------------------------------------------------------------------
# Backward pass ([TS] "Blockwise Backward").
#
# With P = softmax(scale Q K^T) (masked), O = P V and an upstream gradient dO:
#   dV = P^T dO
#   dP = dO V^T
#   dS = P * (dP - D),  D = rowsum(dP * P) = rowsum(dO * O)
#   dQ = scale dS K,    dK = scale dS^T Q
# (the derivative of a row softmax: dS_i = P_i (dP_i - P_i . dP_i)). Grouped
# query heads add their dK, dV into the KV head they read.
# --------------------------------------------------------------------------

def naive_attention_grad(q, k, v, dout, causal: bool, scale: float | None = None, cu_seqlens=None):
    """(dq, dk, dv) of O1, the plain definition above, global token order.

    q, dout: [B, S, Hq, d]; k, v: [B, S, Hkv, d]. cu_seqlens: packed
    sequences (batch 1), attention inside each sequence only.
    Pinned by: torch autograd through float64 SDPA / an explicit masked
    softmax, and central finite differences on tiny inputs.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    bsz, seq, hq, d = q.shape
    hkv = k.shape[2]
    if scale is None:
        scale = default_scale(d)
    pos = np.arange(seq, dtype=np.int64)
    sid = None
    if cu_seqlens is not None:
        sid = np.zeros(seq, dtype=np.int64)
        cu = [int(c) for c in cu_seqlens]
        for s in range(len(cu) - 1):
            sid[cu[s]:cu[s + 1]] = s
    vis = _visibility(pos, pos, causal, sid, sid)
    has = vis.any(axis=1)
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(bsz):
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            s_ = np.where(vis, (q[b, :, h] @ k[b, :, g].T) * scale, -np.inf)
            mx = np.where(has, s_.max(axis=1), 0.0)
            e = np.where(vis, np.exp(s_ - mx[:, None]), 0.0)
            den = e.sum(axis=1)
            p = e / np.where(den > 0, den, 1.0)[:, None]
            o = p @ v[b, :, g]
            dp = dout[b, :, h] @ v[b, :, g].T
            delta = (dout[b, :, h] * o).sum(axis=1)
            ds = p * (dp - delta[:, None])
            dq[b, :, h] = scale * ds @ k[b, :, g]
            dk[b, :, g] += scale * ds.T @ q[b, :, h]
            dv[b, :, g] += p.T @ dout[b, :, h]
    return dq, dk, dv


def naive_grad_rows(q_rows, q_pos, k, v, dout_rows, causal: bool, scale: float | None = None):
    """dq of selected query rows only (those rows of naive_attention_grad's
    dq), each from its own visible keys: softmax row P, O = P v,
    D = dO . O, dS = P (dO v^T - D), dq = scale dS k. For sampled-row checks
    at sizes where the whole gradient is too large for a CPU.

    q_rows, dout_rows: [B, R, Hq, d] with global positions q_pos [R]; k, v:
    [B, S, Hkv, d] in global order.
    Pinned by: equality with naive_attention_grad's dq rows (and autograd)."""
    q_rows, k, v, dout_rows = _f64(q_rows), _f64(k), _f64(v), _f64(dout_rows)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    bsz, nrows, hq, d = q_rows.shape
    hkv = k.shape[2]
    if scale is None:
        scale = default_scale(d)
    kmax = int(q_pos.max()) + 1 if causal else k.shape[1]
    kp = np.arange(kmax, dtype=np.int64)
    vis = _visibility(q_pos, kp, causal)
    has = vis.any(axis=1)
    dq = np.zeros(q_rows.shape)
    for b in range(bsz):
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            kk, vv = k[b, :kmax, g], v[b, :kmax, g]
            s_ = np.where(vis, (q_rows[b, :, h] @ kk.T) * scale, -np.inf)
            mx = np.where(has, s_.max(axis=1), 0.0)
            e = np.where(vis, np.exp(s_ - mx[:, None]), 0.0)
            den = e.sum(axis=1)
            p = e / np.where(den > 0, den, 1.0)[:, None]
            o = p @ vv
            dp = dout_rows[b, :, h] @ vv.T
            ds = p * (dp - (dout_rows[b, :, h] * o).sum(axis=1)[:, None])
            dq[b, :, h] = scale * ds @ kk
    return dq


def grad_delta(out, dout):
    """D = rowsum(dO * O) per (batch, row, head): the softmax-derivative term
    that lets each block's dS be formed without the whole row of P."""
    return (_f64(out) * _f64(dout)).sum(axis=-1)


def block_grad(q, q_pos, k, v, k_pos, dout, lse, delta, causal: bool, scale: float | None = None,
               q_seq=None, k_seq=None):
    """One arriving block's share of the backward pass ([TS] "Blockwise
    Backward": statistics recomputed on the visiting block only):
        P = exp(scale q k^T - lse) on visible pairs (the saved lse makes it the
            true softmax restricted to this block's keys, no second pass),
        dV_j = P^T dO,  dS = P * (dO v^T - D),
        dQ_j = scale dS k_j,  dK_j = scale dS^T q.
    Returns (dq_j [B,Lq,Hq,d], dk_j [B,Lk,Hkv,d], dv_j [B,Lk,Hkv,d]).
    Pinned by: summed over the ring it equals naive_attention_grad."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    lse, delta = _f64(lse), _f64(delta)
    bsz, lq, hq, d = q.shape
    hkv = k.shape[2]
    if scale is None:
        scale = default_scale(d)
    vis = _visibility(np.asarray(q_pos, np.int64), np.asarray(k_pos, np.int64), causal,
                      None if q_seq is None else np.asarray(q_seq, np.int64),
                      None if k_seq is None else np.asarray(k_seq, np.int64))
    dq = np.zeros(q.shape)
    dk, dv = np.zeros(k.shape), np.zeros(v.shape)
    for b in range(bsz):
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            s_ = (q[b, :, h] @ k[b, :, g].T) * scale
            fin = np.isfinite(lse[b, :, h])
            base = np.where(fin, lse[b, :, h], 0.0)
            p = np.where(vis & fin[:, None], np.exp(s_ - base[:, None]), 0.0)
            dp = dout[b, :, h] @ v[b, :, g].T
            ds = p * (dp - delta[b, :, h][:, None])
            dq[b, :, h] = scale * ds @ k[b, :, g]
            dk[b, :, g] += scale * ds.T @ q[b, :, h]
            dv[b, :, g] += p.T @ dout[b, :, h]
    return dq, dk, dv


def ring_share_grad(q_share, k_blocks, v_blocks, out, dout, lse, rank: int, n_ring: int,
                    layout: str, causal: bool, scale: float | None = None, order=None,
                    seqlens=None):
    """Backward pass of one device's share over the ring.

    q_share, out, dout: [B, Lq, Hq, d] (out and lse from the forward pass);
    k_blocks, v_blocks: [N, B, Lk, Hkv, d]. Returns (dq [B,Lq,Hq,d],
    dk [N,B,Lk,Hkv,d], dv [N,B,Lk,Hkv,d]): dq is complete (queries stay on
    their device); dk[j], dv[j] are this share's addends to block j's
    gradients, which in the ring travel with block j and collect every
    device's addend.
    Pinned by: the sum over ranks, placed in global order, equals
    naive_attention_grad; any arrival order gives the same result.
    """
    q_share = _f64(q_share)
    bsz, lq, hq, d = q_share.shape
    lk = k_blocks.shape[2]
    if seqlens is None:
        q_pos, q_seq = global_positions(layout, n_ring, rank, lq), None
    else:
        q_seq, q_pos = varlen_positions(layout, n_ring, rank, seqlens)
    delta = grad_delta(out, dout)
    dq = np.zeros(q_share.shape)
    dk = np.zeros(k_blocks.shape)
    dv = np.zeros(v_blocks.shape)
    for j in (ring_order(rank, n_ring) if order is None else order):
        if seqlens is None:
            k_pos, k_seq = global_positions(layout, n_ring, j, lk), None
        else:
            k_seq, k_pos = varlen_positions(layout, n_ring, j, seqlens)
        gq, gk, gv = block_grad(q_share, q_pos, k_blocks[j], v_blocks[j], k_pos, dout, lse, delta,
                                causal, scale, q_seq, k_seq)
        dq += gq
        dk[j] += gk
        dv[j] += gv
    return dq, dk, dv


# --------------------------------------------------------------------------
# O3 -- integer references: tile classes and counted work.
# --------------------------------------------------------------------------

def tile_classes_bruteforce(layout: str, causal: bool, n_ring: int, rank: int, j: int,
                            q_len: int, kv_len: int, tq: int, tk: int, seqlens=None) -> np.ndarray:
    """[ceil(q_len/tq), ceil(kv_len/tk)] classes by counting visible elements.

    A (q-tile, k-tile) pair is FULL when every in-bounds (query, key) pair of
    it is visible, SKIP when none is, PARTIAL otherwise. Visibility uses global
    positions of the local query share (block `rank`) and of block j.
    Motivation: without skipping, causal ring attention spends about half its
    FLOPs on masked pairs ([TS] "Y nghia thuc te"); devices holding early
    queries skip most key blocks ([UL] closing remark). With packed
    sequences (`seqlens`), q_len == kv_len == sum(seqlens) / N.
    """
    if seqlens is None:
        q_pos = global_positions(layout, n_ring, rank, q_len)
        k_pos = global_positions(layout, n_ring, j, kv_len)
        vis = _visibility(q_pos, k_pos, causal)
    else:
        q_seq, q_pos = varlen_positions(layout, n_ring, rank, seqlens)
        k_seq, k_pos = varlen_positions(layout, n_ring, j, seqlens)
        vis = _visibility(q_pos, k_pos, causal, q_seq, k_seq)
    nqt = -(-q_len // tq)
    nkt = -(-kv_len // tk)
    out = np.empty((nqt, nkt), dtype=np.int8)
    for qt in range(nqt):
        for kt in range(nkt):
            t = vis[qt * tq:(qt + 1) * tq, kt * tk:(kt + 1) * tk]
            cnt = int(t.sum())
            out[qt, kt] = FULL if cnt == t.size else (SKIP if cnt == 0 else PARTIAL)
    return out


def tile_class_counts(layout: str, causal: bool, n_ring: int, rank: int, j: int,
                      q_len: int, kv_len: int, tq: int, tk: int):
    """(#FULL, #PARTIAL, #SKIP) without materialising elements, for real sizes.

    For a fixed query, visible keys of a block form a prefix b <= lim(a)
    (key positions increase with b), and lim is nondecreasing in a. A q-tile
    [a0, a1] therefore sees k-tiles with b_hi <= lim(a0) fully, k-tiles with
    b_lo > lim(a1) not at all, and the rest partially.
    Pinned by: equality with tile_classes_bruteforce on small shapes.
    """
    q_pos = global_positions(layout, n_ring, rank, q_len)
    k_pos = global_positions(layout, n_ring, j, kv_len)
    nkt = -(-kv_len // tk)
    full = part = skip = 0
    for a0 in range(0, q_len, tq):
        a1 = min(a0 + tq, q_len) - 1
        if causal:
            lim0 = int(np.searchsorted(k_pos, q_pos[a0], side="right")) - 1
            lim1 = int(np.searchsorted(k_pos, q_pos[a1], side="right")) - 1
        else:
            lim0 = lim1 = kv_len - 1
        # k-tiles fully visible: b_hi <= lim0 with b_hi = min((kt+1)tk, kv_len) - 1
        n_full = 0 if lim0 < 0 else (lim0 + 1) // tk
        if lim0 == kv_len - 1:
            n_full = nkt
        # k-tiles with any visible element: b_lo <= lim1
        n_any = 0 if lim1 < 0 else lim1 // tk + 1
        full += n_full
        part += n_any - n_full
        skip += nkt - n_any
    return full, part, skip


def visible_pairs_bruteforce(layout: str, causal: bool, n_ring: int, rank: int, block_len: int,
                             seqlens=None) -> int:
    """Number of visible (query, key) pairs of one device's share over all
    blocks, counted element by element (packed sequences if `seqlens`)."""
    if seqlens is not None:
        q_seq, q_pos = varlen_positions(layout, n_ring, rank, seqlens)
        total = 0
        for j in range(n_ring):
            k_seq, k_pos = varlen_positions(layout, n_ring, j, seqlens)
            total += int(_visibility(q_pos, k_pos, causal, q_seq, k_seq).sum())
        return total
    q_pos = global_positions(layout, n_ring, rank, block_len)
    total = 0
    for j in range(n_ring):
        total += int(_visibility(q_pos, global_positions(layout, n_ring, j, block_len), causal).sum())
    return total


def visible_pairs_closed_form(layout: str, causal: bool, n_ring: int, rank: int, block_len: int,
                              seqlens=None) -> int:
    """Closed forms (per query head, per batch row):
      non-causal: N B^2
      contiguous causal: r B^2 + B(B+1)/2 (blocks j<r full, j=r triangle, j>r none)
      striped causal: N B(B-1)/2 + (r+1) B (blocks j<=r keep the diagonal,
                      blocks j>r lose it)
      zigzag causal: (N-1) B^2/2 + B(B+1)/2 for every rank (a block j != r
                      pairs one chunk before and one after the query chunks:
                      half of its pairs are visible; j = r is a triangle)
    Packed sequences: the sum over sequences with B = L_s / N.
    Pinned by: visible_pairs_bruteforce for many (N, B, r)."""
    if seqlens is not None:
        return sum(visible_pairs_closed_form(layout, causal, n_ring, rank, int(L) // n_ring)
                   for L in seqlens)
    n, b, r = n_ring, block_len, rank
    if not causal:
        return n * b * b
    if layout == "contiguous":
        return r * b * b + b * (b + 1) // 2
    if layout == "zigzag":
        return (n - 1) * b * b // 2 + b * (b + 1) // 2
    return n * b * (b - 1) // 2 + (r + 1) * b


def counted_flops(pairs: int, head_dim: int, hq: int, batch: int = 1) -> int:
    """Algorithmic FLOPs: 2d for the score dot product plus 2d for the
    weighted sum of V, per visible pair per query head. Exponentials, masked
    elements and skipped tiles are not counted."""
    return 4 * head_dim * hq * batch * pairs
