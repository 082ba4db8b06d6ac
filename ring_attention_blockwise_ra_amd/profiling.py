"""Summaries of rocprofv3 output for the attention path.

    python -m ring_attention_blockwise_ra_amd.profiling trace  <kernel_trace.csv> <kernel_stats.csv> [ms_per_step launches_per_step]
    python -m ring_attention_blockwise_ra_amd.profiling traffic <fetch_dir> <write_dir> <out.json>
    python -m ring_attention_blockwise_ra_amd.profiling sq <pmc_dir> [kernel name part]
    python -m ring_attention_blockwise_ra_amd.profiling overlap <kernel_trace.csv> <launches per ring>

trace:   per-kernel statistics of the attention, merge and finalize kernels,
         and how much of the side-queue staging copy time ran while an
         attention kernel was executing (the overlap of the staged ring).
traffic: HBM bytes per attention launch from two counter runs (FETCH_SIZE,
         then WRITE_SIZE; KiB per dispatch), each scaled by what the same
         counter reads for the calibration copy of known size that bench.py
         performs with --calib-copy-mib. Writes a JSON that bench.py reports
         as roofline.traffic while the kernel source hash still matches.
overlap: attention-kernel time of each staged ring against each no-copy
         sequence in a trace of bench.py --overlap-only (what concurrent
         staging copies cost the kernels).
sq:      shader-sequencer counters of the attention launches (one --pmc run
         with SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA, SQ_INSTS_VALU,
         SQ_INSTS_VALU_TRANS_F32, SQ_INSTS_LDS, GRBM_GUI_ACTIVE and others):
         matrix-core busy fraction per SIMD cycle, the engine clock implied by
         GRBM_GUI_ACTIVE over the dispatch times, executed MFMA FLOPs and
         instruction mix per MFMA.
"""

from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

ATTN = "attn_bf16_mfma"
COPY = "copyBuffer"          # the runtime's device copy (calibration copies, rotary-path V)
STAGE_COPY = "copy2_kernel"  # the ring's staging copy of K and V


def _is_copy(name: str) -> bool:
    return COPY in name or STAGE_COPY in name
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = ["ring_attention_blockwise_ra_amd/csrc/ra_kernels.hip",
                  "ring_attention_blockwise_ra_amd/csrc/ra_device.h",
                  "ring_attention_blockwise_ra_amd/csrc/ra_sched.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def trace_summary(trace_csv: str, stats_csv: str, ms_per_step: float | None = None,
                  launches_per_step: int | None = None) -> dict:
    """With ms_per_step (bench's figure of the same run) and the attention
    launches one step makes, also checks that the traced average launch time
    fits the timed step: launches_per_step x average <= ms_per_step (a trace
    taken on a slower box, or of other source, cannot stand for the run)."""
    rows = _rows(trace_csv)
    attn = [r for r in rows if ATTN in r["Kernel_Name"]]
    attn_q = {r["Queue_Id"] for r in attn}
    spans = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in attn)
    # staging copies: blit-copy kernels on a queue the attention kernel does not use
    copies = [r for r in rows if _is_copy(r["Kernel_Name"]) and r["Queue_Id"] not in attn_q]
    tot = hidden = 0
    for r in copies:
        s, e = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        tot += e - s
        o = sum(max(0, min(e, b) - max(s, a)) for a, b in spans)
        hidden += min(o, e - s)
    stats = {}
    for r in _rows(stats_csv):
        name = r["Name"]
        for key in ("attn_bf16_mfma", "attn_f32_fma", "merge_partials", "finalize_kernel",
                    "fill_empty", COPY, STAGE_COPY):
            if key in name:
                stats[name[:80]] = dict(calls=int(r["Calls"]), avg_ms=float(r["AverageNs"]) / 1e6,
                                        total_ms=float(r["TotalDurationNs"]) / 1e6,
                                        pct=float(r["Percentage"]))
    out = dict(kernels=stats, staging_copies=len(copies), staging_copy_ms=tot / 1e6,
               staging_copy_hidden_ms=hidden / 1e6,
               staging_copy_hidden_frac=(hidden / tot) if tot else None)
    if ms_per_step is not None and launches_per_step:
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6 for r in attn]
        avg = sum(durs) / len(durs)
        out["attention_avg_ms"] = avg
        out["attention_ms_per_step"] = launches_per_step * avg
        out["ms_per_step"] = ms_per_step
        if launches_per_step * avg > ms_per_step:
            raise ValueError(f"{launches_per_step} launches x {avg:.3f} ms = "
                             f"{launches_per_step * avg:.1f} ms exceed the step's {ms_per_step:.1f} ms")
    return out


def overlap_summary(trace_csv: str, launches: int) -> dict:
    """Attention-kernel time of the staged ring against the no-copy sequence,
    from a kernel trace of bench.py --overlap-only: attention dispatches in
    start order, taken `launches` at a time (one ring, or one no-copy
    sequence); a run is "staged" when staging copies ran on another queue
    within its span. Returns the summed attention duration of each run, the
    mean per kind, and the staged-minus-no-copy difference: what concurrent
    copies cost the kernels themselves. Also the compute queue's idle time
    inside each run (its span minus the union of the kernels on that queue):
    what the cross-stream waits add to the ring's critical path."""
    rows = _rows(trace_csv)
    attn = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Queue_Id"])
                  for r in rows if ATTN in r["Kernel_Name"])
    attn_q = {q for _, _, q in attn}
    copies = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
              if _is_copy(r["Kernel_Name"]) and r["Queue_Id"] not in attn_q]
    # every kernel on the attention's queue(s): the ring's critical path
    lane = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
                  if r["Queue_Id"] in attn_q)
    runs = {"staged": [], "nocopy": []}
    gaps = {"staged": [], "nocopy": []}
    seq = []   # (kind, attention ms, idle ms, copy ms) in trace order
    for i in range(0, len(attn) - launches + 1, launches):
        grp = attn[i:i + launches]
        a, b = grp[0][0], grp[-1][1]
        staged = any(s < b and e > a for s, e in copies)
        kind = "staged" if staged else "nocopy"
        runs[kind].append(sum(e - s for s, e, _ in grp) / 1e6)
        # idle time of the compute queue between the run's first and last
        # attention launch: span minus the union of its kernels' busy time
        busy, cur = 0, None
        for s, e in lane:
            if e <= a or s >= b:
                continue
            s, e = max(s, a), min(e, b)
            if cur is None or s > cur[1]:
                if cur is not None:
                    busy += cur[1] - cur[0]
                cur = [s, e]
            else:
                cur[1] = max(cur[1], e)
        if cur is not None:
            busy += cur[1] - cur[0]
        gaps[kind].append((b - a - busy) / 1e6)
        cms = sum(min(e, b) - max(s, a) for s, e in copies if s < b and e > a) / 1e6
        seq.append((kind, runs[kind][-1], gaps[kind][-1], cms))
    # paired: each no-copy run against the staged run just before it (bench
    # times them as interleaved pairs, so the two see the same clock)
    pairs = [(p[1] - q[1], p[2] - q[2], p[3]) for p, q in zip(seq, seq[1:])
             if p[0] == "staged" and q[0] == "nocopy"]
    mean = {k: (sum(v) / len(v) if v else None) for k, v in runs.items()}
    gmean = {k: (sum(v) / len(v) if v else None) for k, v in gaps.items()}
    diff = (mean["staged"] - mean["nocopy"]) if None not in mean.values() else None
    gdiff = (gmean["staged"] - gmean["nocopy"]) if None not in gmean.values() else None
    return dict(launches_per_run=launches, runs={k: len(v) for k, v in runs.items()},
                attention_ms_per_run=runs, mean_attention_ms=mean,
                staged_minus_nocopy_ms=diff,
                staged_minus_nocopy_frac=(diff / mean["nocopy"]) if diff is not None else None,
                queue_idle_ms_per_run=gaps, mean_queue_idle_ms=gmean,
                queue_idle_staged_minus_nocopy_ms=gdiff,
                paired=_paired(pairs),
                staging_copies=len(copies),
                staging_copy_ms=sum(e - s for s, e in copies) / 1e6)


def _paired(pairs):
    """Median and range of the paired differences (attention time, queue idle
    time) of staged minus no-copy runs, and the copy time of a staged run."""
    if not pairs:
        return None
    med = lambda xs: sorted(xs)[len(xs) // 2] if len(xs) % 2 else \
        (sorted(xs)[len(xs) // 2 - 1] + sorted(xs)[len(xs) // 2]) / 2  # noqa: E731
    da, di, dc = zip(*pairs)
    cost = med(da) + med(di)
    return dict(pairs=len(pairs), attention_diff_ms=list(da), queue_idle_diff_ms=list(di),
                attention_diff_ms_median=med(da), attention_diff_ms_range=[min(da), max(da)],
                queue_idle_diff_ms_median=med(di), copy_ms_per_staged_run=med(dc),
                cost_ms=cost,
                efficiency=1.0 - max(0.0, cost) / med(dc) if med(dc) > 0 else None)


def _counter_values(run_dir: str, counter: str):
    """{dispatch_id: (kernel_name, value)} from a --pmc csv directory."""
    out = {}
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {run_dir}")
    for path in files:
        for r in _rows(path):
            if r.get("Counter_Name") != counter:
                continue
            did = r.get("Dispatch_Id") or r.get("Correlation_Id")
            val = float(r["Counter_Value"])
            name = r.get("Kernel_Name", "")
            if did in out:  # several rows per dispatch (per XCD / instance): sum
                out[did] = (name, out[did][1] + val)
            else:
                out[did] = (name, val)
    return out


MERGE = "merge_partials_kernel"


def traffic(fetch_dir: str, write_dir: str, calib_bytes: int) -> dict:
    res = {}
    merge = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = _counter_values(d, counter)
        copies = [v for n, v in vals.values() if COPY in n]
        if not copies:
            raise RuntimeError(f"{counter}: no calibration copy dispatch found")
        calib_kib = max(copies)  # the calibration copy is the largest copy dispatch
        factor = calib_bytes / (calib_kib * 1024.0)
        attn = [v for n, v in vals.values() if ATTN in n]
        per_launch = sum(attn) / len(attn) * 1024.0 * factor
        res[counter] = dict(calib_kib=calib_kib, factor=factor, launches=len(attn),
                            bytes_per_launch=per_launch)
        mg = [v for n, v in vals.values() if MERGE in n]
        if mg:
            merge[counter] = dict(launches=len(mg), bytes_per_launch=sum(mg) / len(mg) * 1024.0 * factor)
    res["hbm_bytes_per_launch"] = res["FETCH_SIZE"]["bytes_per_launch"] + \
        res["WRITE_SIZE"]["bytes_per_launch"]
    if len(merge) == 2:  # the merge kernel's measured HBM bytes, same scaling
        merge["hbm_bytes_per_launch"] = merge["FETCH_SIZE"]["bytes_per_launch"] + \
            merge["WRITE_SIZE"]["bytes_per_launch"]
        res["merge"] = merge
    return res


MFMA_FLOPS = 32 * 32 * 16 * 2   # one v_mfma_f32_32x32x16_bf16


def sq_summary(run_dir: str, kernel: str = ATTN) -> dict:
    """Counters summed over the dispatches of `kernel`. GRBM_GUI_ACTIVE sums
    the busy cycles of every XCD, so per-XCD cycles are that over Num_Xcc;
    SQ_VALU_MFMA_BUSY_CYCLES sums matrix-core busy cycles over all SIMDs."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {run_dir}")
    sums = defaultdict(float)
    spans = {}
    for path in files:
        for r in _rows(path):
            if kernel not in r.get("Kernel_Name", ""):
                continue
            sums[r["Counter_Name"]] += float(r["Counter_Value"])
            did = r.get("Dispatch_Id") or r.get("Correlation_Id")
            spans[did] = (int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
    agents = glob.glob(os.path.join(run_dir, "**", "*agent_info.csv"), recursive=True)
    simds = n_xcc = None
    for path in agents:
        for r in _rows(path):
            if r.get("Name", "").startswith("gfx"):
                simds, n_xcc = int(r["Simd_Count"]), int(r["Num_Xcc"])
    dur_ns = sum(e - s for s, e in spans.values())
    out = dict(kernel=kernel, dispatches=len(spans), duration_ms=dur_ns / 1e6,
               counters={k: v for k, v in sorted(sums.items())}, simd_count=simds, num_xcc=n_xcc)
    grbm = sums.get("GRBM_GUI_ACTIVE")
    if grbm and n_xcc and dur_ns:
        cyc = grbm / n_xcc
        out["engine_clock_ghz"] = cyc / dur_ns
        if "SQ_VALU_MFMA_BUSY_CYCLES" in sums and simds:
            out["mfma_busy_frac"] = sums["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * simds)
    n_mfma = sums.get("SQ_INSTS_MFMA")
    if n_mfma:
        out["mfma_executed_flops"] = n_mfma * MFMA_FLOPS
        if dur_ns:
            out["mfma_executed_tflops"] = n_mfma * MFMA_FLOPS / dur_ns / 1e3
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS"):
            if k in sums:
                out[k.lower() + "_per_mfma"] = sums[k] / n_mfma
    return out


def main(argv):
    if len(argv) >= 3 and argv[0] == "trace":
        extra = (float(argv[3]), int(argv[4])) if len(argv) >= 5 else (None, None)
        print(json.dumps(trace_summary(argv[1], argv[2], *extra), indent=1))
    elif len(argv) >= 4 and argv[0] == "traffic":
        calib = int(argv[4]) if len(argv) > 4 else 1 << 30
        t = traffic(argv[1], argv[2], calib)
        t["kernel_source_hash"] = kernel_source_hash()
        with open(argv[3], "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t, indent=1))
    elif len(argv) >= 3 and argv[0] == "overlap":
        print(json.dumps(overlap_summary(argv[1], int(argv[2])), indent=1))
    elif len(argv) >= 2 and argv[0] == "sq":
        print(json.dumps(sq_summary(argv[1], *argv[2:3]), indent=1))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
