#!/usr/bin/env python3
"""Benchmark of one device's share of Ring Attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4]

A step is one full pass of the hot path over the workload: ra_ring_fwd for
the share (8 ring steps: the attention kernel per block, the first block's
partial starting the running state and every later one merged into it in
the kernel's epilogue, staging copies on a side stream, finalize). For the 1M-token causal workload (c4, the
default) a step runs the rank-7 share in both token layouts, contiguous then
striped. Inputs are resident in HBM before timing starts.

Printed (one JSON line): TFLOP/s over causal-counted FLOPs (4*d per visible
(query, key) pair per query head), the roofline of the attention kernel
(its FLOPs per launch over its average launch time, measured with HIP events
on its own stream), the cost of the staging copies (staged ring against the
same kernels reading every block in place, interleaved pairs), the HBM
bandwidth of the standalone merge entry point, the backward ring, the other
workloads' ring TFLOP/s (the 8192-token sequence, the 131072-token striped share at every rank, the
921,600-token video share), and the fp64 CPU oracle timed on a bounded sample
of the same workload (a reported baseline, not a target) together with the
max-abs error of the GPU output on those sampled rows (`parity`).

Separate runs: --backward-only (the backward leg), --overlap-only (the
overlap leg, for kernel traces), --cu-scaling n1,n2,... (the attention
kernel's throughput per busy CU against the number of busy CUs).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from ring_attention_blockwise_ra_amd import binding as B  # noqa: E402
from ring_attention_blockwise_ra_amd import synth, workloads  # noqa: E402
from ring_attention_blockwise_ra_amd.profiling import kernel_source_hash  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_bf16_mfma_c4_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def timed(fn, stream=None):
    """Run fn once between two HIP events on `stream`; returns ms."""
    s = stream or torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1)


class ClockSampler:
    """Samples the GPU's graphics clock and socket power (amdsmi GPU metrics)
    on a background thread while a timed region runs. The firmware refreshes
    these metrics about once a second. Every failure (no amdsmi, no access to
    the metrics) leaves the result None; timing never depends on it."""

    MAX_GFXCLK_MHZ = 2400.0   # MI355X peak engine clock, the clock of the published peaks

    def __init__(self, period_s=0.05):
        self.period_s = period_s
        self.samples = []
        self._stop = None
        self._thread = None
        self._smi = None
        self._h = None
        self.power_cap_w = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            hs = amdsmi.amdsmi_get_processor_handles()
            if len(hs) == 1:   # the one GPU this process uses
                self._smi, self._h = amdsmi, hs[0]
                cap = amdsmi.amdsmi_get_power_cap_info(self._h).get("power_cap")
                self.power_cap_w = cap / 1e6 if isinstance(cap, (int, float)) and cap > 0 else None
        except Exception:
            self._smi = None

    def _run(self):
        while not self._stop.is_set():
            try:
                m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
                clk, pw = m.get("current_gfxclk"), m.get("current_socket_power")
                if isinstance(clk, (int, float)) and isinstance(pw, (int, float)):
                    self.samples.append((float(clk), float(pw)))
            except Exception:
                pass
            self._stop.wait(self.period_s)

    # the firmware refreshes the metrics about once a second: a shorter
    # region reads a stale value, so it reports none
    MIN_SECONDS = 2.0

    def __enter__(self):
        self._t0 = time.perf_counter()
        self._t1 = None
        if self._smi is not None:
            import threading
            self._stop = threading.Event()
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._t1 = time.perf_counter()
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        if not self.samples:
            return None
        if self._t1 is not None and self._t1 - self._t0 < self.MIN_SECONDS:
            return None
        clks = sorted(c for c, _ in self.samples)
        pws = sorted(p for _, p in self.samples)
        med = lambda xs: xs[len(xs) // 2]
        return {"gfxclk_mhz_median": med(clks), "gfxclk_mhz_min": clks[0], "gfxclk_mhz_max": clks[-1],
                "gfxclk_mhz_peak_spec": self.MAX_GFXCLK_MHZ,
                "socket_power_w_median": med(pws), "power_cap_w": self.power_cap_w,
                "samples": len(self.samples),
                "source": "amdsmi GPU metrics sampled during the timed steps (firmware refresh ~1 s)"}


def ring_call(w, out, lse, ws, copy_stream="auto"):
    c = w["cfg"]
    return B.ra_ring_fwd(w["q"], w["k"], w["v"], n_ring=c["n_ring"], causal=c["causal"],
                         layout=w["layout"], rank=w["rank"], out=out, lse=lse, workspace=ws,
                         copy_stream=copy_stream, cu_seqlens=w.get("cu_seqlens"),
                         rope_theta=w.get("rope_theta", 0.0))


def kernel_leg(w):
    """Attention kernel alone, as the ring launches it: one launch per
    computed block (the first writing the running state, the others merging
    into it), HIP events on the launch stream. Returns (total counted FLOPs,
    total ms, launches)."""
    c = w["cfg"]
    n, r, blen = c["n_ring"], w["rank"], c["block"]
    q = w["q"]
    b, lq, hq, d = q.shape
    m = torch.empty(b, lq, hq, dtype=torch.float32, device=q.device)
    l = torch.empty_like(m)
    acc = torch.empty(b, lq, hq, d, dtype=torch.float32, device=q.device)
    flops = ms = 0.0
    launches = 0
    for s in range(n):
        j = (r - s) % n
        pairs = block_pairs(w["layout"], c["causal"], n, r, j, blen, w.get("seqlens"))
        if pairs == 0:
            continue
        # as the ring runs it: the first block's partial starts the running
        # state, every later block is merged into it by the same kernel
        fn = B.ra_block_attn_partial if launches == 0 else B.ra_block_attn_accumulate
        ms += timed(lambda: fn(q, w["k"][j], w["v"][j], j, n_ring=n, rank=r, causal=c["causal"],
                               layout=w["layout"], m=m, l=l, acc=acc,
                               cu_seqlens=w.get("cu_seqlens")))
        flops += 4.0 * d * hq * b * pairs
        launches += 1
    return flops, ms, launches


def block_pairs(layout, causal, n, r, j, blen, seqlens=None):
    """Visible pairs of one (share, block) per head: full, none, half (zigzag
    blocks other than the share's own), or a triangle with or without its
    diagonal. Packed sequences: the sum over sequences."""
    if seqlens is not None:
        return sum(block_pairs(layout, causal, n, r, j, L // n) for L in seqlens)
    if not causal:
        return blen * blen
    if layout == "contiguous":
        if j < r:
            return blen * blen
        if j > r:
            return 0
        return blen * (blen + 1) // 2
    if layout == "zigzag":
        return blen * (blen + 1) // 2 if j == r else blen * blen // 2
    return blen * (blen + 1) // 2 if j <= r else blen * (blen - 1) // 2


def captured(fn):
    """fn captured once in a HIP graph (after a warm-up on a side stream);
    returns the graph's replay."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    return g.replay


def overlap_leg(w, out, lse, ws, reps=11, graph=False, copy_stream="auto"):
    """Cost of the staging copies: T_ring (the ring as the library runs it:
    copies on a side stream, or in order for small blocks), T_nocopy (the
    same kernels through the public entry points, every block read in place
    from the sources), T_copy (the N-1 staging copies alone).

    The ring and the no-copy sequence are timed in `reps` interleaved pairs,
    so clock drift hits both alike; the cost is the median of the paired
    differences T_ring - T_nocopy, reported with its quartiles and range.
    efficiency = 1 - max(0, median difference) / T_copy: 1 when the copies
    cost nothing, 0 when they cost as much as running them alone.
    graph: the ring and the no-copy sequence are each captured in a HIP graph
    and replayed (no per-launch host cost)."""
    c = w["cfg"]
    n, r = c["n_ring"], w["rank"]
    q = w["q"]
    b, lq, hq, d = q.shape
    rm = torch.empty(b, lq, hq, dtype=torch.float32, device=q.device)
    rl = torch.empty_like(rm)

    def nocopy():
        B.ra_block_attn_partial(q, w["k"][r], w["v"][r], r, n_ring=n, rank=r, causal=c["causal"],
                                layout=w["layout"], m=rm, l=rl, acc=out,
                                cu_seqlens=w.get("cu_seqlens"))
        for s in range(1, n):
            j = (r - s) % n
            if block_pairs(w["layout"], c["causal"], n, r, j, c["block"], w.get("seqlens")) == 0:
                continue
            B.ra_block_attn_accumulate(q, w["k"][j], w["v"][j], j, n_ring=n, rank=r,
                                       causal=c["causal"], layout=w["layout"], m=rm, l=rl,
                                       acc=out, cu_seqlens=w.get("cu_seqlens"))
        B.ra_finalize(rm, rl, out, lse=lse)

    stage_k = torch.empty_like(w["k"][0])
    stage_v = torch.empty_like(w["v"][0])

    def copies():
        for s in range(1, n):
            j = (r - s) % n
            stage_k.copy_(w["k"][j])
            stage_v.copy_(w["v"][j])

    ring_fn = lambda: ring_call(w, out, lse, ws, copy_stream=copy_stream)  # noqa: E731
    nocopy_fn = nocopy
    if graph:
        ring_fn, nocopy_fn = captured(ring_fn), captured(nocopy_fn)
    tr, tn = [], []
    for _ in range(reps):
        tr.append(timed(ring_fn))
        tn.append(timed(nocopy_fn))
    diffs = sorted(a - b for a, b in zip(tr, tn))
    q_ = lambda xs, f: xs[min(len(xs) - 1, int(round(f * (len(xs) - 1))))]  # noqa: E731
    med = q_(diffs, 0.5)
    t_copy = sorted(timed(copies) for _ in range(5))[2]
    eff = 1.0 - max(0.0, med) / t_copy if t_copy > 0 else 1.0
    return dict(efficiency=round(eff, 4), cost_ms_median=round(med, 4),
                cost_ms_q1=round(q_(diffs, 0.25), 4), cost_ms_q3=round(q_(diffs, 0.75), 4),
                cost_ms_min=round(diffs[0], 4), cost_ms_max=round(diffs[-1], 4),
                cost_frac_of_ring=round(med / q_(sorted(tr), 0.5), 6),
                t_ring_ms=round(q_(sorted(tr), 0.5), 4), t_nocopy_ms=round(q_(sorted(tn), 0.5), 4),
                t_copy_ms=round(t_copy, 4), reps=reps,
                copy_bytes=int(2 * (n - 1) * w["k"][0].numel() * w["k"].element_size()))


def merge_leg(w, reps=5):
    q = w["q"]
    b, lq, hq, d = q.shape
    rows = b * lq * hq
    g = torch.Generator(device=q.device).manual_seed(1)
    parts = []
    for _ in range(2):
        m = torch.randn(b, lq, hq, device=q.device, generator=g)
        l = torch.rand(b, lq, hq, device=q.device, generator=g) + 1
        a = torch.randn(b, lq, hq, d, device=q.device, generator=g)
        parts.append((m, l, a))
    out = (torch.empty_like(parts[0][0]), torch.empty_like(parts[0][1]),
           torch.empty_like(parts[0][2]))
    B.ra_merge_partials(*parts[0], *parts[1], out=out)
    ms = min(timed(lambda: B.ra_merge_partials(*parts[0], *parts[1], out=out)) for _ in range(reps))
    nbytes = 3 * rows * (4 * d + 8)
    return dict(gbs=round(nbytes / ms / 1e6, 1), ms=round(ms, 4), bytes=nbytes,
                frac_of_peak=round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4))


def cpu_baseline_leg(w, n_rows, k_global, v_global, gpu_out=None):
    """The fp64 oracle (untuned) on n_rows sampled query rows x all heads of
    the share; rate in counted TFLOP/s of those rows. With gpu_out (the
    ring's output of the same share), also the max-abs error of those rows
    against the oracle."""
    from oracle import ring_oracle as orc
    c = w["cfg"]
    rows = workloads.sample_rows(c["block"], n_rows, seed=3)
    tok = w["q_tokens"][rows]
    q_rows = w["q"][:, rows.to(w["q"].device)].to(torch.float64).cpu().numpy()
    kmax = int(tok.max()) + 1 if c["causal"] else k_global.shape[1]
    k64 = k_global[:, :kmax].to(torch.float64).cpu().numpy()
    v64 = v_global[:, :kmax].to(torch.float64).cpu().numpy()
    t0 = time.perf_counter()
    ref, ref_lse = orc.naive_attention_rows(q_rows, tok.numpy(), k64, v64, c["causal"])
    dt = time.perf_counter() - t0
    parity = None
    if gpu_out is not None:
        got_o, got_l = gpu_out
        d_o = (got_o[:, rows.to(got_o.device)].to(torch.float64).cpu().numpy() - ref)
        d_l = (got_l[:, rows.to(got_l.device)].to(torch.float64).cpu().numpy() - ref_lse)
        parity = dict(max_abs=float(abs(d_o).max()), lse_max_abs=float(abs(d_l).max()),
                      tol=1e-2, rows=len(tok), heads=c["hq"],
                      reference="oracle O1 (fp64 softmax(QK^T/sqrt(d))V), every visible key",
                      rows_sample="first/last 8, tile edges, seeded random rows",
                      layout=w["layout"], rank=w["rank"])
    pairs = int((tok + 1).sum()) if c["causal"] else len(tok) * k_global.shape[1]
    flops = 4.0 * c["d"] * c["hq"] * pairs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=int(threads),
                kind="oracle",
                sample=(f"{len(tok)} query rows x {c['hq']} heads of the {w['layout']} rank-{w['rank']}"
                        f" share, all visible keys, fp64 NumPy; {dt:.1f} s"),
                seconds=round(dt, 2), host_cpus=len(os.sched_getaffinity(0))), parity


def setup_ring(w, dev):
    """Outputs, workspace and counted FLOPs of a prepared share."""
    c = w["cfg"]
    b, lq, hq, d = w["q"].shape
    prob = B.make_problem(dtype=w["q"].dtype, batch=b, hq=hq, hkv=w["k"].shape[3], head_dim=d,
                          q_len=lq, kv_len=w["k"].shape[2], n_ring=c["n_ring"], rank=w["rank"],
                          causal=c["causal"], layout=w["layout"], cu_seqlens=w.get("cu_seqlens"))
    w["out"] = torch.empty(b, lq, hq, d, dtype=torch.float32, device=dev)
    w["lse"] = torch.empty(b, lq, hq, dtype=torch.float32, device=dev)
    w["ws"] = torch.empty(B.ra_ring_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    w["flops"] = workloads.counted_flops(w["layout"], c["causal"], c["n_ring"], w["rank"],
                                         c["block"], hq, d, b, seqlens=w.get("seqlens"))


def widened_leg(dev, cases, reps=2):
    """Ring TF/s of the same 1M-token share in the layouts, packings and
    with the rotary embedding beyond the headline pair (one warm-up, median
    of `reps`). A case is (workload, layout, rope_theta)."""
    res = {}
    for name, layout, theta in cases:
        w = workloads.prepare(name, layout, 7, device=dev)
        setup_ring(w, dev)
        if theta:
            c = w["cfg"]
            b, lq, hq, d = w["q"].shape
            prob = B.make_problem(dtype=w["q"].dtype, batch=b, hq=hq, hkv=w["k"].shape[3],
                                  head_dim=d, q_len=lq, kv_len=w["k"].shape[2],
                                  n_ring=c["n_ring"], rank=7, causal=c["causal"],
                                  layout=layout, rope_theta=theta)
            w["ws"] = torch.empty(B.ra_ring_workspace_bytes(prob), dtype=torch.uint8, device=dev)
        w["rope_theta"] = theta
        ring_call(w, w["out"], w["lse"], w["ws"])
        torch.cuda.synchronize()
        ts = sorted(timed(lambda: ring_call(w, w["out"], w["lse"], w["ws"])) for _ in range(reps))
        ms = ts[len(ts) // 2]
        key = f"{name}_{layout}" + ("_rope" if theta else "")
        res[key] = dict(ms=round(ms, 3), tflops=round(w["flops"] / (ms / 1e3) / 1e12, 2),
                        counted_flops=w["flops"],
                        sequences=None if w.get("seqlens") is None else len(w["seqlens"]))
        del w
        torch.cuda.empty_cache()
        log(f"[bench] widened {key} done")
    return res


def configs_leg(dev, reps=3):
    """Ring TF/s of the other bf16 workloads, each ring as the library runs it
    by default (one warm-up, median of `reps`): the 8192-token causal
    sequence (every rank's share, times summed), the 131072-token striped GQA
    share at every rank r = 0..7 (r = 7 is the headline rank; the sweep shows
    the load of the early-query devices), and the non-causal 921,600-token
    video share (rank 0; all ranks do equal work)."""
    res = {}

    def ring_ms(w):
        ring_call(w, w["out"], w["lse"], w["ws"])
        torch.cuda.synchronize()
        ts = sorted(timed(lambda: ring_call(w, w["out"], w["lse"], w["ws"])) for _ in range(reps))
        return ts[len(ts) // 2]

    def entry(ms, flops):
        tf = flops / (ms / 1e3) / 1e12
        return dict(ms=round(ms, 4), tflops=round(tf, 2),
                    pct_bf16_peak=round(100 * tf / PEAK_BF16_TFLOPS, 2), counted_flops=flops)

    tot_ms = tot_f = 0.0
    for r in range(8):
        w = workloads.prepare("c2", "contiguous", r, device=dev)
        setup_ring(w, dev)
        tot_ms += ring_ms(w)
        tot_f += w["flops"]
        del w
    res["c2"] = dict(workload="8192 tokens, N=8 blocks of 1024, 32 heads, causal contiguous, "
                              "every rank (ring times summed)", **entry(tot_ms, tot_f))
    log("[bench] configs c2 done")
    sweep = {}
    for r in range(8):
        w = workloads.prepare("c3", "striped", r, device=dev)
        setup_ring(w, dev)
        sweep[str(r)] = entry(ring_ms(w), w["flops"])
        del w
    torch.cuda.empty_cache()
    res["c3"] = dict(workload="131072 tokens, N=8 blocks of 16384, GQA 32/8, causal striped",
                     rank7=sweep["7"], rank_sweep=sweep)
    log("[bench] configs c3 done")
    w = workloads.prepare("c5", "contiguous", 0, device=dev)
    setup_ring(w, dev)
    res["c5"] = dict(workload="921,600 tokens (3600 frames x 256), N=8 blocks of 115200, 32 heads, "
                              "non-causal, rank 0", **entry(ring_ms(w), w["flops"]))
    del w
    torch.cuda.empty_cache()
    log("[bench] configs c5 done")
    return res


def backward_leg(dev, layouts, reps=1):
    """Backward ring (ra_ring_bwd) of the 1M-token share, rank 7: one
    warm-up, then `reps` timed runs. Counted work: 10*d FLOPs per visible
    pair per query head (S = q k^T recomputed, dP = dO v^T, dV = P^T dO,
    dK = dS^T q, dQ = dS k)."""
    res = {}
    tot_f = tot_ms = 0.0
    for layout in layouts:
        w = workloads.prepare("c4", layout, 7, device=dev)
        setup_ring(w, dev)
        ring_call(w, w["out"], w["lse"], w["ws"])
        g = torch.Generator(device=dev).manual_seed(11)
        dout = torch.randn(w["q"].shape, generator=g, device=dev).to(w["q"].dtype)
        c = w["cfg"]
        b, lq, hq, d = w["q"].shape
        dq = torch.empty(b, lq, hq, d, dtype=torch.float32, device=dev)
        dk = torch.zeros(w["k"].shape, dtype=torch.float32, device=dev)
        dv = torch.zeros_like(dk)
        prob = B.make_problem(dtype=w["q"].dtype, batch=b, hq=hq, hkv=w["k"].shape[3], head_dim=d,
                              q_len=lq, kv_len=w["k"].shape[2], n_ring=c["n_ring"], rank=7,
                              causal=c["causal"], layout=layout)
        ws = torch.empty(B.ra_ring_bwd_workspace_bytes(prob), dtype=torch.uint8, device=dev)

        def run():
            B.ra_ring_bwd(w["q"], w["k"], w["v"], w["out"], dout, w["lse"], n_ring=c["n_ring"],
                          causal=c["causal"], layout=layout, rank=7, dq=dq, dk=dk, dv=dv,
                          workspace=ws)

        run()
        torch.cuda.synchronize()
        ms = min(timed(run) for _ in range(reps))
        flops = 10.0 * d * hq * b * workloads.visible_pairs(layout, c["causal"], c["n_ring"], 7,
                                                            c["block"])
        res[layout] = dict(ms=round(ms, 3), tflops=round(flops / (ms / 1e3) / 1e12, 2),
                           counted_flops=flops)
        tot_f += flops
        tot_ms += ms
        del w, dout, dq, dk, dv, ws
        torch.cuda.empty_cache()
        log(f"[bench] backward {layout} done")
    res["tflops"] = round(tot_f / (tot_ms / 1e3) / 1e12, 2)
    res["pct_bf16_peak"] = round(100 * res["tflops"] / PEAK_BF16_TFLOPS, 2)
    res["note"] = ("ra_ring_bwd of the same share (dq written, dk/dv addends of all 8 blocks); "
                   "10*d FLOPs per visible pair; not part of value")
    return res


def cu_scaling_leg(dev, n_wgs, kv=131072, d=128, seconds=4.0):
    """Throughput per busy CU of the attention kernel against the number of
    busy CUs: one non-causal 131072-key block of one KV head, 8-wave
    workgroups of 256 query rows, q_len = 256 * n_wg rows, so a launch is
    n_wg workgroups, one per CU (the LDS ring allows one per CU). Each count
    runs back-to-back launches for `seconds` with the engine clock and
    socket power sampled. Separates the kernel's efficiency per clock from
    the clock the power limit leaves it."""
    prev = os.environ.get("RA_WAVES")
    os.environ["RA_WAVES"] = "8"   # the headline kernel's shape at every count
    try:
        g = torch.Generator(device=dev).manual_seed(3)
        k = (0.5 * torch.randn(1, kv, 1, d, generator=g, device=dev)).to(torch.bfloat16)
        v = torch.randn(1, kv, 1, d, generator=g, device=dev).to(torch.bfloat16)
        res = []
        for n_wg in n_wgs:
            rows = 256 * n_wg
            q = torch.randn(1, rows, 1, d, generator=g, device=dev).to(torch.bfloat16)
            m = torch.empty(1, rows, 1, dtype=torch.float32, device=dev)
            l = torch.empty_like(m)
            acc = torch.empty(1, rows, 1, d, dtype=torch.float32, device=dev)

            def f():
                B.ra_block_attn_partial(q, k, v, 0, n_ring=1, rank=0, causal=False,
                                        m=m, l=l, acc=acc)
            f()
            one = timed(f)
            reps = max(3, int(seconds * 1e3 / one))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            sampler = ClockSampler()
            with sampler:
                e0.record()
                for _ in range(reps):
                    f()
                e1.record()
                e1.synchronize()
            ms = e0.elapsed_time(e1) / reps
            c = sampler.summary() or {}
            tf = 4.0 * d * rows * kv / ms / 1e9
            mhz = c.get("gfxclk_mhz_median")
            per_cu_peak = PEAK_BF16_TFLOPS / 256 * ((mhz or ClockSampler.MAX_GFXCLK_MHZ) /
                                                    ClockSampler.MAX_GFXCLK_MHZ)
            res.append(dict(busy_cus=n_wg, ms=round(ms, 4), tflops=round(tf, 1),
                            tflops_per_cu=round(tf / n_wg, 3), gfxclk_mhz=mhz,
                            socket_power_w=c.get("socket_power_w_median"), reps=reps,
                            frac_of_cu_peak_at_clock=round(tf / n_wg / per_cu_peak, 4)))
            log(f"[bench] cu scaling {n_wg}: {res[-1]}")
            del q, m, l, acc
        return res
    finally:
        if prev is None:
            os.environ.pop("RA_WAVES", None)
        else:
            os.environ["RA_WAVES"] = prev


def load_counters(src_hash, kernel="attention"):
    """HBM traffic per launch of the attention kernel (or, kernel="merge", of
    the merge kernel) from committed rocprofv3 counter runs, only if they
    were taken on the current kernel source."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != src_hash:
        return None
    if kernel == "merge":
        return (c.get("merge") or {}).get("hbm_bytes_per_launch")
    return c.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="c4", choices=sorted(synth.CONFIGS))
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--layouts", default=None, help="comma list; default: the workload's")
    ap.add_argument("--cpu-rows", type=int, default=64)
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before timing, one device copy of this size (counter calibration)")
    ap.add_argument("--skip-extras", action="store_true",
                    help="only the timed steps (for profiler runs)")
    ap.add_argument("--skip-backward", action="store_true", help="no backward leg")
    ap.add_argument("--backward-only", action="store_true",
                    help="only the backward leg (kernel-trace runs of the backward kernels)")
    ap.add_argument("--overlap-reps", type=int, default=11,
                    help="interleaved (ring, no-copy) pairs per layout in the overlap leg")
    ap.add_argument("--overlap-only", action="store_true",
                    help="only the overlap leg of the workload's layouts (kernel-trace runs of "
                         "the staged ring against the no-copy sequence)")
    ap.add_argument("--cu-scaling", default=None,
                    help="comma list of busy-CU counts: only the attention kernel's throughput per "
                         "busy CU against the number of busy CUs, with clock and power")
    ap.add_argument("--skip-aux", action="store_true",
                    help="no 8192-token overlap and no widened leg, so that every attention "
                         "launch has the headline workload's shape (kernel-trace runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the ring; multi-GPU runs are not "
              "supported (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    B.lib()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.backward_only:
        print(json.dumps({"backward": backward_leg(dev, ["contiguous", "striped"])}), flush=True)
        return
    if args.cu_scaling:
        counts = [int(x) for x in args.cu_scaling.split(",")]
        print(json.dumps({"cu_scaling": cu_scaling_leg(dev, counts)}), flush=True)
        return

    c = synth.CONFIGS[args.workload]
    layouts = args.layouts.split(",") if args.layouts else list(c["layouts"])
    rank = args.rank if args.rank is not None else c["ranks"][-1]
    log(f"[bench] workload {args.workload} layouts {layouts} rank {rank}")

    ws_list = []
    for layout in layouts:
        t0 = time.time()
        w = workloads.prepare(args.workload, layout, rank, device=dev,
                              keep_global=(not args.skip_cpu and layout == layouts[0]))
        setup_ring(w, dev)
        ws_list.append(w)
        torch.cuda.synchronize()
        log(f"[bench] prepared {layout} in {time.time() - t0:.1f}s")

    if args.overlap_only:
        ov = {}
        for w in ws_list:
            ring_call(w, w["out"], w["lse"], w["ws"])
            torch.cuda.synchronize()
            ov[w["layout"]] = overlap_leg(w, w["out"], w["lse"], w["ws"], reps=args.overlap_reps)
            log(f"[bench] overlap {w['layout']} done")
        print(json.dumps({"overlap": ov}), flush=True)
        return

    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done")
        # the standalone merge at this share, so that the same counter runs
        # measure its bytes too (the ring itself launches none)
        merge_leg(ws_list[0], reps=1)
        torch.cuda.synchronize()
        log("[bench] merge for the counters done")

    def step():
        for w in ws_list:
            ring_call(w, w["out"], w["lse"], w["ws"])

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")

    torch.cuda.synchronize()
    per_layout_ms = {w["layout"]: 0.0 for w in ws_list}
    sampler = ClockSampler()
    t_start = time.perf_counter()
    with sampler:
        for i in range(args.steps):
            for w in ws_list:
                per_layout_ms[w["layout"]] += timed(lambda: ring_call(w, w["out"], w["lse"], w["ws"]))
            log(f"[bench] step {i + 1}/{args.steps} done")
        torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    clock = sampler.summary()
    total_ms = sum(per_layout_ms.values())
    ms_per_step = total_ms / args.steps
    total_flops = sum(w["flops"] for w in ws_list) * args.steps
    value = total_flops / (total_ms / 1e3) / 1e12

    result = {
        "metric": "ring-attn fwd TFLOP/s (causal-counted) + % bf16 MFMA peak, 1 GPU, "
                  "causal 1M-token share",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if c["dtype"] == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1), bf16-rounded)",
        "config": {
            "workload": (f"{args.workload}: one device's share, N={c['n_ring']} blocks of "
                         f"{c['block']} tokens, {'causal' if c['causal'] else 'non-causal'}, "
                         f"rank {rank}, layouts {'+'.join(layouts)}"),
            "seq_len": c["n_ring"] * c["block"], "block": c["block"], "n_ring": c["n_ring"],
            "rank": rank, "hq": c["hq"], "hkv": c["hkv"], "head_dim": c["d"], "batch": 1,
            "layouts": layouts,
        },
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "wall_s_timed": round(wall, 2),
        "clock": clock,
        "layouts": {
            w["layout"]: {"ms": round(per_layout_ms[w["layout"]] / args.steps, 3),
                          "tflops": round(w["flops"] / (per_layout_ms[w["layout"]] / args.steps / 1e3) / 1e12, 2),
                          "counted_flops": w["flops"]}
            for w in ws_list},
    }

    if not args.skip_extras:
        # dominant kernel: the attention partial, launched once per computed block
        kf = km = 0.0
        nl = 0
        for w in ws_list:
            f, ms, n = kernel_leg(w)
            kf += f
            km += ms
            nl += n
        achieved = kf / (km / 1e3) / 1e12
        src_hash = kernel_source_hash()
        traffic = load_counters(src_hash)
        result["roofline"] = {
            "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "attn_bf16_mfma<128,8>" if c["dtype"] == "bf16" else "attn_f32_fma",
            "launches": nl, "avg_launch_ms": round(km / max(nl, 1), 3),
            "flops_per_launch_avg": kf / max(nl, 1),
            "kernel_source_hash": src_hash,
        }
        if clock:
            # the same peak scaled to the engine clock observed in the timed steps
            peak_obs = PEAK_BF16_TFLOPS * clock["gfxclk_mhz_median"] / ClockSampler.MAX_GFXCLK_MHZ
            result["roofline"]["peak_at_observed_clock"] = round(peak_obs, 1)
            result["roofline"]["frac_at_observed_clock"] = round(achieved / peak_obs, 4)
        log("[bench] kernel leg done")
        # every layout, so that the attention launches of the whole run have the
        # same mix as the kernel leg (its average is compared with rocprofv3's)
        ov = {}
        for w in ws_list:
            ov[w["layout"]] = overlap_leg(w, w["out"], w["lse"], w["ws"], reps=args.overlap_reps)
            log(f"[bench] overlap {w['layout']} done")
        tot = {k: sum(o[k] for o in ov.values())
               for k in ("t_ring_ms", "t_nocopy_ms", "t_copy_ms", "cost_ms_median")}
        eff = 1.0 - max(0.0, tot["cost_ms_median"]) / tot["t_copy_ms"]
        result["overlap"] = dict(
            efficiency=round(eff, 4), **{k: round(v, 4) for k, v in tot.items()},
            per_layout=ov,
            note=("cost = median over interleaved (ring, no-copy) pairs of T_ring - T_nocopy; "
                  "efficiency = 1 - max(0, cost) / T_copy; quartiles and range per layout"))
        if args.workload != "c2" and not args.skip_aux:
            w2 = workloads.prepare("c2", "contiguous", 7, device=dev)
            setup_ring(w2, dev)
            out2, lse2, ws2 = w2["out"], w2["lse"], w2["ws"]
            ring_call(w2, out2, lse2, ws2)
            small = dict(workload="c2: 8192 tokens, N=8 blocks of 1024, causal contiguous, rank 7",
                         default=overlap_leg(w2, out2, lse2, ws2, reps=41),
                         graph=overlap_leg(w2, out2, lse2, ws2, reps=41, graph=True))
            # the two-stream scheme forced at this size (the library would run
            # copies this small in order on the compute stream)
            prev = os.environ.get("RA_SIDE_STREAM_MIN_BYTES")
            os.environ["RA_SIDE_STREAM_MIN_BYTES"] = "0"
            try:
                small["side_stream_forced"] = overlap_leg(w2, out2, lse2, ws2, reps=41)
            finally:
                if prev is None:
                    os.environ.pop("RA_SIDE_STREAM_MIN_BYTES", None)
                else:
                    os.environ["RA_SIDE_STREAM_MIN_BYTES"] = prev
            result["overlap"]["small_workload"] = small
            del w2, out2, lse2, ws2
        log("[bench] overlap leg done")
        result["merge"] = merge_leg(ws_list[0])
        # measured HBM bytes per merge at this share (counters), if current
        result["merge"]["traffic"] = load_counters(src_hash, "merge") if args.workload == "c4" else None
        log("[bench] merge leg done")
        if args.workload == "c4" and not args.skip_aux and not args.skip_backward:
            result["backward"] = backward_leg(dev, layouts)
        if args.workload == "c4" and not args.skip_aux:
            result["widened"] = dict(
                note=("same 1M-token causal share, rank 7: zigzag layout, the sequence packed "
                      "from mixed-length documents (c4p) in zigzag and contiguous layouts, and "
                      "zigzag with the rotary embedding applied on arrival (base 500000); not "
                      "part of value"),
                **widened_leg(dev, [("c4", "zigzag", 0.0), ("c4p", "zigzag", 0.0),
                                    ("c4p", "contiguous", 0.0), ("c4", "zigzag", 500000.0)]))
            result["configs"] = configs_leg(dev)

    if not args.skip_cpu and ws_list[0].get("cu_seqlens") is None:
        w = ws_list[0]
        ring_call(w, w["out"], w["lse"], w["ws"])   # the ring's own output of this share
        torch.cuda.synchronize()
        log(f"[bench] cpu baseline: oracle on {args.cpu_rows} rows ...")
        result["cpu_baseline"], result["parity"] = cpu_baseline_leg(
            w, args.cpu_rows, w["k_global"], w["v_global"], gpu_out=(w["out"], w["lse"]))
        log("[bench] cpu baseline done")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
