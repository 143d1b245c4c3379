"""Benchmark of the Mamba-2 SSD hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one ssd_chunk_scan over the Mamba-2-2.7B-shaped layer (batch 4,
8192 tokens, 80 heads x 64, dstate 128, 1 group, chunk 256; bf16 x/B/C/y,
fp32 dt/A/D/state), seeded synthetic inputs resident in HBM.  ``value`` is
prefill tokens/s (batch x seqlen per step time).  The decode half of the
metric (1000 in-place ssd_decode_step calls on a [256, 80, 64, 128] fp32 state,
fresh tokens each step) is reported under ``decode``; batches 1, 16, 64 are
reported as effective bandwidth (their state fits in the 256 MB MALL or the
step is launch-bound).  ``decode_steps`` runs the same 1000 steps as one
ssd_decode_steps launch (state held on-chip across the steps), whose bound is
fp32 VALU arithmetic.  ``prefill_configs`` holds the 130M-shaped layer and the
131072-token long-context prefill (8 B/C groups).

Order: the decode legs and the other prefill configurations run first, then the
headline's W warm-up steps and its K timed steps.  The GPU's clock ramps up over
the first ~20 ms of back-to-back work and a prefill step is 0.3 ms, so with a
short warm-up on an idle GPU the timed steps would measure the ramp rather than
the sustained rate.

Prints ONE JSON line.  ``roofline`` is the dominant prefill kernel
(chunk_scan_kernel): algorithmic bytes of the layer per launch / its average
launch time measured with HIP events on the launch stream; ``roofline_step``
the same bytes over the event-timed whole step;
``decode.roofline`` likewise for decode_rows_kernel.  ``traffic`` comes from
committed rocprofv3 FETCH_SIZE / WRITE_SIZE counters (profiles/counters.json)
when they were taken on the current kernel sources, else null; so does the
counted MFMA FLOP behind ``mfma.counted``.  ``cpu_baseline`` times the fp64
oracle (as it stands) on a bounded sample of the same workload, on all the
CPUs the process may use (at most 16) and on one thread.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, TFLOP/s (256 CU x 2.4 GHz x 256 FLOP/clk)
# The same without packed fp32 (one FMA per lane and instruction: 4 SIMDs x 16
# lanes x 2 FLOP per clock and CU), the ceiling of kernels built without
# packed fp32 instructions, as libssd is
FP32_UNPACKED_PEAK_TFLOPS = 78.6
UNPACKED_NOTE = ("frac_unpacked: against 78.6 TFLOP/s, the fp32 vector rate without packed fp32 "
                 "instructions (libssd is built without them)")
METRIC = "SSD prefill tokens/s (MFMA %) + decode steps/s (HBM GB/s %) at 2.7B-layer shape"
CSRC = "state_space_model_mamba_amd/csrc/"
# the source of each measured kernel; its counters in profiles/counters.json are
# used while that file and the shared header are unchanged
KERNEL_SOURCE = {"seg_state_kernel": "ssd_scan_bf16.hip", "chunk_scan_kernel": "ssd_scan_bf16.hip",
                 "decode_rows_kernel": "ssd_decode.hip", "decode_kernel": "ssd_decode.hip",
                 "decode_steps_kernel": "ssd_decode_steps.hip",
                 "gdn_decode_kernel": "ssd_gdn.hip", "gdn_steps_kernel": "ssd_gdn.hip",
                 "scan_f32_kernel": "ssd_scan_f32.hip"}


def prefill_bytes(w) -> int:
    """Minimum HBM bytes of one prefill: read x, B, C, dt, write y and the final state."""
    esz = 2
    x = w.batch * w.seqlen * w.nheads * w.headdim * esz
    bc = 2 * w.batch * w.seqlen * w.ngroups * w.dstate * esz
    dt = w.batch * w.seqlen * w.nheads * 4
    state = w.batch * w.nheads * w.headdim * w.dstate * 4
    return 2 * x + bc + dt + state + 2 * w.nheads * 4


def prefill_useful_flops(w) -> int:
    """Useful FLOPs of the chunked algorithm (causal triangle only): C B^T per
    group, intra-chunk product, chunk state and state->output per head."""
    Q, P, N = w.chunk, w.headdim, w.dstate
    nc = w.seqlen // Q
    tri = Q * (Q + 1) // 2
    cb = tri * N * 2 * w.batch * nc * w.ngroups
    per_head = (tri * P * 2 + 2 * Q * P * N * 2) * w.batch * nc * w.nheads
    return cb + per_head


def decode_bytes(b, w) -> int:
    """HBM bytes of one decode step: state read + write, x, y, B, C, dt."""
    state = b * w.nheads * w.headdim * w.dstate * 4
    return 2 * state + 2 * b * w.nheads * w.headdim * 2 + 2 * b * w.ngroups * w.dstate * 2 + b * w.nheads * 4


def decode_steps_flops(b, w) -> int:
    """Arithmetic of one decode step: per state element alpha*H, u*B, their sum,
    H*C and its accumulation (5 FLOP); per state row dt*x, D*x and its add (3)."""
    rows = b * w.nheads * w.headdim
    return rows * (5 * w.dstate + 3)


def source_digest(kernel: str) -> str:
    """sha256 of the kernel's source file and the shared kernel header."""
    h = hashlib.sha256()
    for f in (KERNEL_SOURCE[kernel], "ssd_kernels.h"):
        with open(os.path.join(ROOT, CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


COUNTERS = os.path.join(ROOT, "profiles", "counters.json")


def _counter_record(kernel: str, wname: str | None):
    """The committed counter record of a kernel (for workload `wname`, or the
    first workload that has one), if it was taken on the current sources."""
    if not os.path.exists(COUNTERS):
        return None, None
    rec = json.load(open(COUNTERS))
    for wl, kernels in rec.get("workloads", {}).items():
        if wname is not None and wl != wname:
            continue
        k = kernels.get(kernel)
        if k and k.get("source_sha256") == source_digest(kernel):
            return k, (rec.get("copy_scale") or {}).get(wl)
    return None, None


def committed_traffic(kernel: str, wname: str | None = None):
    k, scale = _counter_record(kernel, wname)
    if not k or "fetch_bytes" not in k or "write_bytes" not in k:
        return None
    return {"fetch_bytes": k["fetch_bytes"], "write_bytes": k["write_bytes"],
            "total_bytes": k["fetch_bytes"] + k["write_bytes"], "scale": scale,
            "source": "profiles/counters.json"}


def step_traffic(kernels, wname):
    """Counted HBM bytes of a whole step (every kernel's), if all are current."""
    parts = [committed_traffic(k, wname) for k in kernels]
    if any(p is None for p in parts):
        return None
    return {"fetch_bytes": sum(p["fetch_bytes"] for p in parts),
            "write_bytes": sum(p["write_bytes"] for p in parts),
            "total_bytes": sum(p["total_bytes"] for p in parts),
            "source": "profiles/counters.json"}


def committed_mfma(kernel: str, wname: str):
    k, _ = _counter_record(kernel, wname)
    return None if not k or "mfma_flop" not in k else k["mfma_flop"]


COPY_KERNEL = "__amd_rocclr_copyBuffer"     # the device copy made by --copy-calibration
COPY_BYTES = 1 << 30
KERNELS = ("seg_state_kernel", "chunk_scan_kernel", "decode_rows_kernel", "decode_steps_kernel",
           "gdn_decode_kernel", "gdn_steps_kernel", "decode_kernel", "scan_f32_kernel")


def _counter_means(path, counter):
    """Per-kernel mean of one rocprofv3 counter (per dispatch) over every
    dispatch of the kernel in the run, and the copy kernel's total."""
    import csv
    per, copy = {}, 0.0
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        v = float(r["Counter_Value"])
        if name.startswith(COPY_KERNEL):
            copy += v
        short = name.split("(")[0].split("::")[-1]
        for k in KERNELS:
            if (k in short or k in name) and "multi" not in name:
                per.setdefault(k, []).append(v)
                break
    return {k: sum(v) / len(v) for k, v in per.items()}, copy


def write_counters(wname, fetch_csv, write_csv, mops_csv):
    """Merge one workload's counters into profiles/counters.json: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) from two runs of `bench.py --copy-calibration`,
    each scaled so that the 1 GiB copy reads and writes 1 GiB, and
    SQ_INSTS_VALU_MFMA_MOPS_BF16 (512 FLOP per unit) from a third run."""
    fetch, fcopy = _counter_means(fetch_csv, "FETCH_SIZE")
    write, wcopy = _counter_means(write_csv, "WRITE_SIZE")
    mops = _counter_means(mops_csv, "SQ_INSTS_VALU_MFMA_MOPS_BF16")[0] if mops_csv else {}
    if fcopy <= 0 or wcopy <= 0:
        raise SystemExit("no copy-calibration dispatches in the counter files")
    fs, ws = COPY_BYTES / (fcopy * 1024), COPY_BYTES / (wcopy * 1024)
    rec = json.load(open(COUNTERS)) if os.path.exists(COUNTERS) else {}
    rec.setdefault("copy_bytes", COPY_BYTES)
    rec.setdefault("copy_scale", {})[wname] = {"fetch": fs, "write": ws}
    kernels = {}
    for k in fetch:
        kernels[k] = {"source_sha256": source_digest(k),
                      "fetch_bytes": fetch[k] * 1024 * fs,
                      "write_bytes": write.get(k, 0.0) * 1024 * ws,
                      "fetch_kib_raw": fetch[k], "write_kib_raw": write.get(k, 0.0)}
        if k in mops:
            kernels[k]["mfma_flop"] = mops[k] * 512
    rec.setdefault("workloads", {})[wname] = kernels
    os.makedirs(os.path.dirname(COUNTERS), exist_ok=True)
    with open(COUNTERS, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({wname: kernels}, indent=1))


def trace_runs(trace_csv):
    """Per-dispatch rows of a rocprofv3 kernel trace, grouped into blocks of
    consecutive dispatches in dispatch order: one kernel with one grid, or the
    two prefill kernels (state and scan kernel, each with one grid) of the
    same steps.  Returns [(kernel, grid, count, mean_us, later_half_mean_us,
    min_us, max_us)] for every kernel of every block."""
    import csv
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Dispatch_Id"]))
    pair = ("seg_state_kernel", "chunk_scan_kernel")
    blocks = []          # [{(kernel, grid): [us, ...]}]
    for r in rows:
        name = r["Kernel_Name"]
        short = next((k for k in KERNELS + ("seg_state_multi_kernel", "chunk_scan_multi_kernel")
                      if k in name), name.split("(")[0][:40])
        if "<true>" in name or "ILb1E" in name:
            short += "<softplus>"
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        key = (short, grid)
        cur = blocks[-1] if blocks else None
        joins = False
        if cur is not None:
            if key in cur:
                joins = True
            elif len(cur) == 1 and short.split("<")[0] in pair:
                (k0, _), = cur.keys()
                joins = k0.split("<")[0] in pair and k0.split("<")[0] != short.split("<")[0]
        if joins:
            cur.setdefault(key, []).append(us)
        else:
            blocks.append({key: [us]})
    out = []
    for b in blocks:
        for (k, g), v in b.items():
            half = v[len(v) // 2:]
            out.append((k, g, len(v), sum(v) / len(v), sum(half) / len(half), min(v), max(v)))
    return out


def to_dev(a, bf16=False):
    import torch
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


PREFILL_WORKLOADS = {
    "m2_2p7b": "Mamba-2-2.7B-shaped SSD layer prefill (ssd_chunk_scan)",
    "m2_130m": "Mamba-2-130M-shaped SSD layer prefill (ssd_chunk_scan)",
    "longctx_2p7b": "long-context prefill at the 2.7B head shape, 8 B/C groups (ssd_chunk_scan)",
}


def prefill_config(w):
    return {"batch": w.batch, "seq_len": w.seqlen, "nheads": w.nheads, "headdim": w.headdim,
            "dstate": w.dstate, "ngroups": w.ngroups, "chunk": w.chunk, "state": "fp32",
            "io": "bf16"}


def prefill_setup(wname):
    """A prefill workload's seeded inputs, outputs and workspace, resident in HBM."""
    import torch

    import ssd_inputs as si
    import state_space_model_mamba_amd as ssd

    w = si.WORKLOADS[wname]
    A, D = si.head_params(w)
    inp = si.prefill_inputs(w)
    t = {"w": w, "x": to_dev(inp["x"], True), "dt": to_dev(inp["dt"]),
         "B": to_dev(inp["B"], True), "C": to_dev(inp["C"], True), "A": to_dev(A), "D": to_dev(D)}
    del inp
    t["y"] = torch.empty_like(t["x"])
    t["fs"] = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32,
                          device="cuda")
    nws = ssd.ssd_chunk_scan_workspace_size(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate,
                                            w.ngroups, w.chunk)
    t["ws"] = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    return t


def bench_prefill(args, wname, t, steps=None, warmup=None, extras=False):
    """K timed ssd_chunk_scan calls on one workload (inputs `t` already in HBM)
    after W untimed ones, then per-kernel HIP-event times (ssd_chunk_scan_timed);
    with `extras`, the same step with the fused step-size prep.  Only GPU work
    and its host launches run here, so the clock does not drop between legs."""
    import torch

    import state_space_model_mamba_amd as ssd

    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    w = t["w"]
    x, dt, B, C, dA, dD = t["x"], t["dt"], t["B"], t["C"], t["A"], t["D"]
    y, fs, ws = t["y"], t["fs"], t["ws"]

    def step():
        ssd.ssd_chunk_scan(x, dt, dA, B, C, dD, w.chunk, y=y, final_state=fs, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = e0.elapsed_time(e1) / steps
    ms = wall * 1e3 / steps

    # per-kernel device times: HIP events recorded around each launch on the
    # stream the kernels run on.  An untimed step is queued ahead of each timed
    # one, so that the first kernel's start event is not taken on an idle GPU
    # (the timed entry point synchronises at its end).
    per = {}
    for _ in range(max(3, min(steps, 10))):
        step()
        _, _, times = ssd.ssd_chunk_scan_timed(x, dt, dA, B, C, dD, w.chunk, y=y, final_state=fs,
                                               workspace=ws)
        for name, t in times:
            per.setdefault(name, []).append(t)
    kern = {k: float(np.mean(v)) for k, v in per.items()}

    sp = None
    if extras:
        # the same step with the fused step-size prep (dt read as u, softplus(u +
        # bias) formed in the kernels; u and the bias are arbitrary here, only
        # time matters), timed in alternating blocks with the plain step, all
        # queued back to back, so that both see the same clock
        bias = torch.zeros(w.nheads, dtype=torch.float32, device="cuda")

        def fused():
            ssd.ssd_chunk_scan(x, dt, dA, B, C, dD, w.chunk, y=y, final_state=fs, workspace=ws,
                               dt_softplus=True, dt_bias=bias)

        blk, rounds = max(5, min(steps, 20)), 5
        for _ in range(10):      # the fused code loaded, the clock back up after the syncs above
            fused()
            step()
        marks = []
        for _ in range(rounds):
            for fn in (step, fused):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(blk):
                    fn()
                b.record()
                marks.append((a, b))
        torch.cuda.synchronize()
        per_blk = [a.elapsed_time(b) / blk for a, b in marks]
        blk_plain, blk_sp = float(np.median(per_blk[0::2])), float(np.median(per_blk[1::2]))
        # sustained: each form runs warm, 10 untimed calls ahead of a block of
        # `long` timed ones, the two forms still alternating; short blocks
        # above charge every switch between the two kernel instantiations to
        # the block after it
        long, lp, lf = max(20, min(steps, 100)), [], []
        for _ in range(rounds):
            for fn, acc in ((step, lp), (fused, lf)):
                for _ in range(10):
                    fn()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(long):
                    fn()
                b.record()
                torch.cuda.synchronize()
                acc.append(a.elapsed_time(b) / long)
        plain_ms, sp_ms = float(np.median(lp)), float(np.median(lf))
        sp = {"event_ms_per_step": sp_ms, "plain_event_ms_per_step": plain_ms,
              "overhead_pct": 100.0 * (sp_ms / plain_ms - 1.0),
              "timing": f"{rounds} alternating pairs of {long}-step blocks (plain, fused), each "
                        "after 10 untimed calls of its own form; medians of the blocks",
              "short_blocks": {"overhead_pct": 100.0 * (blk_sp / blk_plain - 1.0),
                               "event_ms_per_step": blk_sp, "plain_event_ms_per_step": blk_plain,
                               "timing": f"{rounds} alternating pairs of {blk}-step blocks, "
                                         "queued back to back (each block pays the switch from "
                                         "the other form); medians of the blocks"}}
    nbytes = prefill_bytes(w)
    flops = prefill_useful_flops(w)
    k3 = kern["chunk_scan_kernel"]
    step_k = sum(kern.values())
    tokens = w.batch * w.seqlen
    counted = {k: committed_mfma(k, wname) for k in kern}
    mfma_counted = None
    if all(v is not None for v in counted.values()):
        cf = sum(counted.values())
        mfma_counted = {"flop_per_step": cf, "achieved_tflops": cf / (ev_ms * 1e-3) / 1e12,
                        "frac": cf / (ev_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                        "per_kernel": {k: {"flop": v,
                                           "frac": v / (kern[k] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
                                       for k, v in counted.items()},
                        "source": "profiles/counters.json (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 "
                                  "per launch)"}
    res = {
        "w": w, "ms": ms, "ev_ms": ev_ms, "tokens_per_s": tokens / (ms * 1e-3),
        "kernels_ms": kern, "bytes": nbytes, "flops": flops,
        "roofline": {
            "bound": "hbm", "kernel": "chunk_scan_kernel",
            "achieved": nbytes / (k3 * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": nbytes / (k3 * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": committed_traffic("chunk_scan_kernel", wname),
            "bytes_per_launch": nbytes, "avg_launch_ms": k3,
        },
        "roofline_step": {
            "bound": "hbm", "kernels": sorted(kern),
            "achieved": nbytes / (ev_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": nbytes / (ev_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bytes_per_step": nbytes, "event_ms_per_step": ev_ms,
            "kernel_ms_per_step": step_k,
            "traffic": step_traffic(sorted(kern), wname),
            "note": "the layer's algorithmic bytes over the HIP-event time of a whole step "
                    "(the timed steps back to back); kernel_ms_per_step sums the per-kernel "
                    "events",
        },
        "mfma": {
            "useful_gflop_per_step": flops / 1e9,
            "achieved_tflops": flops / (ev_ms * 1e-3) / 1e12, "peak_tflops": BF16_PEAK_TFLOPS,
            "frac": flops / (ev_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "counted": mfma_counted,
            "note": "useful (causal-triangle) FLOPs of the whole scan over the event-timed "
                    "step; `counted`: the MFMA FLOPs rocprofv3 counts per launch (committed) "
                    "over the same live step time, and per kernel over its own event time",
        },
        "path_gbs": nbytes / (ms * 1e-3) / 1e9,
        "dt_softplus": sp,
    }
    return res


def prefill_line(pre, wname):
    """The JSON object of one prefill workload (secondary configs)."""
    w = pre["w"]
    return {"workload": PREFILL_WORKLOADS[wname], "config": prefill_config(w),
            "tokens_per_s": pre["tokens_per_s"], "ms_per_step": pre["ms"],
            "event_ms_per_step": pre["ev_ms"], "kernels_ms": pre["kernels_ms"],
            "roofline": pre["roofline"], "roofline_step": pre["roofline_step"],
            "mfma": pre["mfma"]}


def bench_decode(args):
    import torch

    import ssd_inputs as si
    import state_space_model_mamba_amd as ssd

    w = si.WORKLOADS["decode_2p7b"]
    A, D = si.head_params(w)
    dA, dD = to_dev(A), to_dev(D)
    out = {}
    for b in args.decode_batches:
        steps = args.decode_steps
        tok = si.decode_tokens(w, b, 0, steps)
        x, dt = to_dev(tok["x"], True), to_dev(tok["dt"])
        B, C = to_dev(tok["B"], True), to_dev(tok["C"], True)
        del tok
        state = to_dev(si.random_state(w, b))
        y = torch.empty((steps, b, w.nheads, w.headdim), dtype=torch.bfloat16, device="cuda")
        for k in range(min(5, steps)):             # warm-up (advances the state)
            ssd.ssd_decode_step(x[k], dt[k], dA, B[k], C[k], dD, state, y=y[k])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for k in range(steps):
            ssd.ssd_decode_step(x[k], dt[k], dA, B[k], C[k], dD, state, y=y[k])
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ev_ms = e0.elapsed_time(e1) / steps
        nb = decode_bytes(b, w)
        out[b] = {"steps": steps, "ms_per_step": wall * 1e3 / steps, "event_ms_per_step": ev_ms,
                  "steps_per_s": steps / wall, "bytes_per_step": nb,
                  "gbs": nb / (ev_ms * 1e-3) / 1e9, "frac": nb / (ev_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        # the same steps captured into one HIP graph and replayed (no per-step
        # host launch); the state keeps advancing, which costs the same
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for k in range(steps):
                    ssd.ssd_decode_step(x[k], dt[k], dA, B[k], C[k], dD, state, y=y[k])
        torch.cuda.current_stream().wait_stream(side)
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        gwall = time.perf_counter() - t0
        g_ms = e0.elapsed_time(e1) / steps
        out[b].update({"graph_ms_per_step": gwall * 1e3 / steps, "graph_steps_per_s": steps / gwall,
                       "graph_gbs": nb / (g_ms * 1e-3) / 1e9})
        del graph
        # the same steps as one ssd_decode_steps launch (state read and written once)
        ssd.ssd_decode_steps(x, dt, dA, B, C, dD, state, y=y)
        torch.cuda.synchronize()
        reps = 3
        t0 = time.perf_counter()
        e0.record()
        for _ in range(reps):
            ssd.ssd_decode_steps(x, dt, dA, B, C, dD, state, y=y)
        e1.record()
        torch.cuda.synchronize()
        mwall = time.perf_counter() - t0
        m_ms = e0.elapsed_time(e1) / (reps * steps)
        fl = decode_steps_flops(b, w)
        out[b].update({"steps_launch_ms_per_step": mwall * 1e3 / (reps * steps),
                       "steps_launch_steps_per_s": reps * steps / mwall,
                       "steps_launch_event_ms_per_step": m_ms,
                       "steps_launch_tflops": fl / (m_ms * 1e-3) / 1e12})
        del x, dt, B, C, y, state
        torch.cuda.empty_cache()
    return w, out


def gdn_bytes(b, sh, esz=2) -> int:
    """HBM bytes of one GDN decode step: the state read and written once, q, k, v, o, g, beta."""
    state = b * sh["v_heads"] * sh["dk"] * sh["dv"] * 4
    return (2 * state + 2 * b * sh["qk_heads"] * sh["dk"] * esz + 2 * b * sh["v_heads"] * sh["dv"] * esz
            + 2 * b * sh["v_heads"] * 4)


def gdn_flops(b, sh) -> int:
    """Arithmetic of one GDN step per state element: the retrieval and readout
    products and sums (4 FLOP) and the update g S + k dv (3 FLOP)."""
    return 7 * b * sh["v_heads"] * sh["dk"] * sh["dv"]


def bench_gdn(args):
    """Gated DeltaNet decode (ssd_gdn_decode_step) at the FPGA page's shape: 32 value
    heads over 16 query/key heads, 128 x 128 fp32 state per value head, bf16 q/k/v/o;
    consecutive in-place steps with fresh tokens, eager and graph-replayed."""
    import torch

    import ssd_inputs as si
    import state_space_model_mamba_amd as ssd

    sh = si.GDN_SHAPE
    out = {}
    nsteps = 200   # also in the counter runs, whose decode steps are fewer
    for b in [b for b in (256, 1) if b in args.decode_batches]:
        steps = nsteps
        tok = si.gdn_tokens(400 + b, steps, b, sh["qk_heads"], sh["v_heads"], sh["dk"], sh["dv"])
        q, k, v = to_dev(tok["q"], True), to_dev(tok["k"], True), to_dev(tok["v"], True)
        g, beta = to_dev(tok["g"]), to_dev(tok["beta"])
        state = to_dev(tok["state0"])
        del tok
        o = torch.empty_like(v)

        def run():
            for t in range(steps):
                ssd.ssd_gdn_decode_step(q[t], k[t], v[t], g[t], beta[t], state, o=o[t])

        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                run()
        torch.cuda.current_stream().wait_stream(side)
        graph.replay()
        torch.cuda.synchronize()
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        gms = e0.elapsed_time(e1) / steps
        nb = gdn_bytes(b, sh)
        # the same steps as one ssd_gdn_decode_steps launch (state kept on-chip)
        ssd.ssd_gdn_decode_steps(q, k, v, g, beta, state, o=o)
        torch.cuda.synchronize()
        e0.record()
        ssd.ssd_gdn_decode_steps(q, k, v, g, beta, state, o=o)
        e1.record()
        torch.cuda.synchronize()
        sms = e0.elapsed_time(e1) / steps
        fl = gdn_flops(b, sh)
        out[b] = {"event_ms_per_step": ms, "graph_ms_per_step": gms, "bytes_per_step": nb,
                  "gbs": nb / (ms * 1e-3) / 1e9, "graph_gbs": nb / (gms * 1e-3) / 1e9,
                  "steps_launch_ms_per_step": sms,
                  "steps_launch_tflops": fl / (sms * 1e-3) / 1e12}
        del q, k, v, g, beta, state, o, graph
        torch.cuda.empty_cache()
    r = out[256]
    return {"workload": "ssd_gdn_decode_step, 32 value heads over 16 query/key heads, "
                        "128 x 128 fp32 state per value head (2 MB per sequence), bf16 q/k/v/o, "
                        f"{nsteps} consecutive in-place steps",
            "roofline": {"bound": "hbm", "kernel": "gdn_decode_kernel", "batch": 256,
                         "achieved": r["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": r["gbs"] / HBM_PEAK_GBS,
                         "traffic": committed_traffic("gdn_decode_kernel"),
                         "bytes_per_launch": r["bytes_per_step"],
                         "avg_launch_ms": r["event_ms_per_step"]},
            "batches": {str(b): v for b, v in sorted(out.items())},
            "steps_launch": {"roofline": {
                "bound": "alu", "kernel": "gdn_steps_kernel", "batch": 256,
                "achieved": r["steps_launch_tflops"], "peak": FP32_VALU_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": r["steps_launch_tflops"] / FP32_VALU_PEAK_TFLOPS,
                "frac_unpacked": r["steps_launch_tflops"] / FP32_UNPACKED_PEAK_TFLOPS,
                "note": UNPACKED_NOTE,
                "flops_per_step": gdn_flops(256, sh),
                "avg_launch_ms": r["steps_launch_ms_per_step"] * nsteps},
                "note": f"the same {nsteps} steps as one ssd_gdn_decode_steps launch, the state read and "
                        "written once and held in registers across the steps"},
            "note": "batch 1 moves 2 MB per step (MALL-resident, launch-bound eager)"}


VARLEN_LENGTHS = (8192, 6144, 4096, 4096, 2048, 1024, 512, 512)


def bench_varlen(args):
    """A continuous-batching prefill: prompts of mixed lengths packed into one
    ssd_chunk_scan_varlen call at the 2.7B head shape (80 x 64, dstate 128,
    chunk 256, bf16)."""
    import torch

    import ssd_inputs as si
    import state_space_model_mamba_amd as ssd

    T = sum(VARLEN_LENGTHS)
    w = si.small_workload(batch=1, seqlen=T, nheads=80, headdim=64, dstate=128, ngroups=1,
                          chunk=256, seed=211)
    A, D = si.head_params(w)
    inp = si.prefill_inputs(w)
    x, dt = to_dev(inp["x"][0], True), to_dev(inp["dt"][0])
    B, C = to_dev(inp["B"][0], True), to_dev(inp["C"][0], True)
    dA, dD = to_dev(A), to_dev(D)
    del inp
    cu = np.concatenate([[0], np.cumsum(VARLEN_LENGTHS)]).astype(np.int64)
    y = torch.empty_like(x)
    fs = torch.empty((len(VARLEN_LENGTHS), 80, 64, 128), dtype=torch.float32, device="cuda")
    nws = ssd.ssd_chunk_scan_varlen_workspace_size(cu, 80, 64, 128, 1, 256)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")

    def step():
        ssd.ssd_chunk_scan_varlen(x, dt, dA, B, C, dD, cu, 256, y=y, final_states=fs, workspace=ws)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    runs = sum(1 for i in range(len(VARLEN_LENGTHS))
               if i == 0 or VARLEN_LENGTHS[i] != VARLEN_LENGTHS[i - 1])
    return {"workload": f"ssd_chunk_scan_varlen, {len(VARLEN_LENGTHS)} packed sequences of "
                        f"lengths {list(VARLEN_LENGTHS)} ({T} tokens), 80 heads x 64, dstate 128, "
                        f"chunk 256, bf16",
            "event_ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
            "runs_of_equal_length": runs, "kernel_launches": 2 * ((runs + 7) // 8)}


NONCACHED_CONTEXTS = (256, 1024, 4096, 16384, 32768)
NONCACHED_NEW = 64


def bench_noncached(args):
    """Cached against non-cached generation on one 2.7B-shaped layer (80 heads x
    64, dstate 128, 1 group, chunk 256), batch 1, bf16 tokens: the comparison of
    the Compiler-First page's evaluation (section 4) on one layer.  Non-cached:
    each new token re-runs ssd_chunk_scan over the prefix and the token from a
    zero state (the token's output is the last row); cached: ssd_chunk_scan over
    the prefix once, then one ssd_decode_step per token on the carried state.
    For each context length: the time per token of both, the decode step timed on
    the state that the prefill of that context produced (eager and replayed from
    a captured graph), and the time to generate NONCACHED_NEW tokens after the
    prompt both ways."""
    import torch

    import ssd_inputs as si
    import state_space_model_mamba_amd as ssd

    top = max(NONCACHED_CONTEXTS) + NONCACHED_NEW
    w = si.small_workload("noncached_2p7b", batch=1, seqlen=top, nheads=80, headdim=64,
                          dstate=128, ngroups=1, chunk=256, seed=410)
    A, D = si.head_params(w)
    inp = si.prefill_inputs(w)
    x, dt = to_dev(inp["x"], True), to_dev(inp["dt"])
    B, C = to_dev(inp["B"], True), to_dev(inp["C"], True)
    del inp
    dA, dD = to_dev(A), to_dev(D)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def scan(n):                      # batch 1: the first n tokens are a contiguous prefix
        return ssd.ssd_chunk_scan(x[:, :n], dt[:, :n], dA, B[:, :n], C[:, :n], dD, w.chunk)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def decode(state, t):
        return ssd.ssd_decode_step(x[:, t], dt[:, t], dA, B[:, t], C[:, t], dD, state)

    rows = []
    for ctx in NONCACHED_CONTEXTS:
        nc_ms = timed(lambda: scan(ctx + 1), 10)
        pre_ms = timed(lambda: scan(ctx), 10)
        _, state = scan(ctx)
        decode(state.clone(), ctx)           # warm-up on a copy
        st = state.clone()
        torch.cuda.synchronize()
        e0.record()
        for i in range(NONCACHED_NEW):
            decode(st, ctx + i)
        e1.record()
        torch.cuda.synchronize()
        dec_ms = e0.elapsed_time(e1) / NONCACHED_NEW
        st = state.clone()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for i in range(NONCACHED_NEW):
                    decode(st, ctx + i)
        torch.cuda.current_stream().wait_stream(side)
        graph.replay()
        torch.cuda.synchronize()
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        gdec_ms = e0.elapsed_time(e1) / NONCACHED_NEW
        del graph
        # NONCACHED_NEW tokens after the prompt, both ways
        e0.record()
        for i in range(NONCACHED_NEW):
            scan(ctx + i + 1)
        e1.record()
        torch.cuda.synchronize()
        gen_nc = e0.elapsed_time(e1)
        e0.record()
        _, st = scan(ctx)
        for i in range(NONCACHED_NEW):
            decode(st, ctx + i)
        e1.record()
        torch.cuda.synchronize()
        gen_c = e0.elapsed_time(e1)
        rows.append({"context": ctx, "noncached_ms_per_token": nc_ms, "prefill_ms": pre_ms,
                     "cached_ms_per_token": dec_ms, "cached_graph_ms_per_token": gdec_ms,
                     f"generate_{NONCACHED_NEW}_noncached_ms": gen_nc,
                     f"generate_{NONCACHED_NEW}_cached_ms": gen_c,
                     "cached_tokens_per_s": 1e3 / dec_ms, "noncached_tokens_per_s": 1e3 / nc_ms})
    del x, dt, B, C
    torch.cuda.empty_cache()
    return {"workload": "one Mamba-2-2.7B-shaped layer (80 heads x 64, dstate 128, 1 group, "
                        "chunk 256), batch 1, bf16 tokens; non-cached = ssd_chunk_scan over "
                        "the prefix and the token for every token, cached = one "
                        "ssd_chunk_scan over the prompt, then ssd_decode_step per token",
            "rows": rows}


def host_info():
    """The host the oracle runs on: logical CPUs of the machine, those this
    process may run on, and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"host_nproc": os.cpu_count(), "cpus_available": avail, "cpu_model": model}


def oracle_threads():
    """Threads for the all-core oracle run: the CPUs this process may use, at
    most 16 (the CPU share of a one-GPU machine)."""
    return max(1, min(16, host_info()["cpus_available"] or 1))


def cpu_baseline_prefill(w, npairs=None, single_pairs=16):
    """The fp64 oracle on `npairs` of the layer's (batch, head) sequences, full
    length each, threaded over pairs, and on `single_pairs` of them with one
    thread (the plain sequential baseline); tokens/s scaled to the whole layer."""
    import oracle
    import ssd_inputs as si

    threads = oracle_threads()
    A, D = si.head_params(w)
    inp = si.prefill_inputs(w)
    H = w.nheads
    npairs = npairs or w.batch * H
    pairs = [(k // H, k % H) for k in range(npairs)]
    xs = np.stack([si.widen(inp["x"][b, :, h], "bf16") for b, h in pairs])[:, :, None]
    dts = np.stack([inp["dt"][b, :, h] for b, h in pairs]).astype(np.float64)[:, :, None]
    Bs = np.stack([si.widen(inp["B"][b, :, h // (H // w.ngroups)], "bf16") for b, h in pairs])[:, :, None]
    Cs = np.stack([si.widen(inp["C"][b, :, h // (H // w.ngroups)], "bf16") for b, h in pairs])[:, :, None]
    del inp
    from concurrent.futures import ThreadPoolExecutor

    def one(i):
        b, h = pairs[i]
        oracle.ssd_scan(xs[i:i + 1], dts[i:i + 1], A[h:h + 1], Bs[i:i + 1], Cs[i:i + 1], D[h:h + 1])

    oracle.load()
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(npairs)))
    T = time.perf_counter() - t0
    t0 = time.perf_counter()
    for i in range(single_pairs):
        one(i)
    T1 = time.perf_counter() - t0
    full_pairs = w.batch * H
    tok_s = (w.batch * w.seqlen) / (T * full_pairs / npairs)
    tok_s1 = (w.batch * w.seqlen) / (T1 * full_pairs / single_pairs)
    return {"value": tok_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle on {npairs} of the {full_pairs} (batch, head) sequences of "
                      f"the {w.batch}x{w.seqlen}x{H} layer, all {w.seqlen} tokens each, "
                      f"{threads} threads over sequences; {T:.2f} s wall, tokens/s scaled by "
                      f"{npairs}/{full_pairs}",
            "single_thread": {"value": tok_s1, "unit": "tokens/s", "cores": 1,
                              "sample": f"{single_pairs} of the {full_pairs} sequences, one "
                                        f"thread; {T1:.2f} s wall, scaled by "
                                        f"{single_pairs}/{full_pairs}"},
            **host_info()}


def cpu_baseline_decode(w, batch=256, nseq=64, steps=200, single_seq=8):
    """The oracle's decode step on `nseq` sequences for `steps` steps (threaded
    over (sequence, head)), and on `single_seq` with one thread; steps/s scaled
    to the full batch."""
    import oracle
    import ssd_inputs as si

    threads = oracle_threads()
    A, D = si.head_params(w)
    tok = si.decode_tokens(w, nseq, 0, steps)
    st0 = si.random_state(w, nseq).astype(np.float64)
    xs = si.widen(tok["x"], "bf16")
    Bs, Cs = si.widen(tok["B"], "bf16"), si.widen(tok["C"], "bf16")
    dts = tok["dt"].astype(np.float64)
    st = st0
    t0 = time.perf_counter()
    for k in range(steps):
        _, st = oracle.ssd_decode_step(st, xs[k], dts[k], A, Bs[k], Cs[k], D, nthreads=threads)
    T = time.perf_counter() - t0
    st = st0[:single_seq]
    t0 = time.perf_counter()
    for k in range(steps):
        _, st = oracle.ssd_decode_step(st, xs[k, :single_seq], dts[k, :single_seq], A,
                                       Bs[k, :single_seq], Cs[k, :single_seq], D, nthreads=1)
    T1 = time.perf_counter() - t0
    return {"value": steps / (T * batch / nseq), "unit": "steps/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{nseq} of {batch} sequences x {steps} steps, {threads} threads; "
                      f"{T:.2f} s, scaled by {nseq}/{batch}",
            "single_thread": {"value": steps / (T1 * batch / single_seq), "unit": "steps/s",
                              "cores": 1,
                              "sample": f"{single_seq} of {batch} sequences x {steps} steps, one "
                                        f"thread; {T1:.2f} s, scaled by {single_seq}/{batch}"},
            **host_info()}


def cpu_baseline_gdn(nseq=32, steps=40, batch=256):
    """The fp64 GDN oracle (three passes, numpy, BLAS held to one thread) on `nseq`
    sequences of the page's shape for `steps` steps; steps/s scaled to the full batch."""
    from threadpoolctl import threadpool_limits

    from oracle import gdn
    import ssd_inputs as si

    sh = si.GDN_SHAPE
    tok = si.gdn_tokens(401, steps, nseq, sh["qk_heads"], sh["v_heads"], sh["dk"], sh["dv"], "f32")
    S = tok["state0"].astype(np.float64)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        for t in range(steps):
            _, S = gdn.gdn_decode_step(S, tok["q"][t], tok["k"][t], tok["v"][t], tok["g"][t],
                                       tok["beta"][t])
        T = time.perf_counter() - t0
    return {"value": steps / (T * batch / nseq), "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{nseq} of {batch} sequences x {steps} steps, one thread; "
                      f"{T:.1f} s, scaled by {nseq}/{batch}", **host_info()}


def decode_line(wd, dec):
    main_b = max(dec)
    d = dec[main_b]
    out = {}
    out["decode"] = {
        "workload": f"decode_step at the 2.7B shape, state [{main_b},80,64,128] fp32, "
                    f"{d['steps']} consecutive in-place steps, fresh bf16 tokens",
        "steps_per_s": d["steps_per_s"], "ms_per_step": d["ms_per_step"],
        "roofline": {"bound": "hbm", "kernel": "decode_rows_kernel", "achieved": d["gbs"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": d["frac"],
                     "traffic": committed_traffic("decode_rows_kernel"),
                     "bytes_per_launch": d["bytes_per_step"],
                     "avg_launch_ms": d["event_ms_per_step"]},
        "batches": {str(b): {k: v for k, v in r.items()} for b, r in sorted(dec.items())},
        "note": "batch <= 64 keeps the state (<= 168 MB) in the 256 MB MALL or is "
                "launch-bound: effective bandwidth, not HBM; graph_*: the same steps "
                "replayed from one captured HIP graph",
    }
    fl = decode_steps_flops(main_b, wd)
    m_ms = d["steps_launch_event_ms_per_step"]
    out["decode_steps"] = {
        "workload": f"ssd_decode_steps at the 2.7B shape: the same {d['steps']} steps on a "
                    f"[{main_b},80,64,128] fp32 state as one launch (state read and written "
                    f"once, held in registers across the steps)",
        "steps_per_s": d["steps_launch_steps_per_s"],
        "ms_per_step": d["steps_launch_ms_per_step"],
        "roofline": {"bound": "alu", "kernel": "decode_steps_kernel",
                     "achieved": fl / (m_ms * 1e-3) / 1e12, "peak": FP32_VALU_PEAK_TFLOPS,
                     "unit": "TFLOP/s",
                     "frac": fl / (m_ms * 1e-3) / 1e12 / FP32_VALU_PEAK_TFLOPS,
                     "frac_unpacked": fl / (m_ms * 1e-3) / 1e12 / FP32_UNPACKED_PEAK_TFLOPS,
                     "note": UNPACKED_NOTE,
                     "traffic": committed_traffic("decode_steps_kernel"),
                     "flops_per_step": fl, "avg_launch_ms": m_ms * d["steps"]},
        "batches": {str(b): {"steps_per_s": r["steps_launch_steps_per_s"],
                             "ms_per_step": r["steps_launch_ms_per_step"],
                             "event_ms_per_step": r["steps_launch_event_ms_per_step"],
                             "tflops": r["steps_launch_tflops"]}
                    for b, r in sorted(dec.items())},
    }
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--headline", default="m2_2p7b", choices=sorted(PREFILL_WORKLOADS),
                    help="the prefill workload of `value` (other choices: counter runs)")
    ap.add_argument("--secondary", default="m2_130m,longctx_2p7b",
                    help="further prefill workloads reported under `prefill_configs` ('' = none)")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--decode-batches", type=str, default="256,64,16,1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the fused-softplus, mixed-length and non-cached timings (counter "
                         "and trace runs: every dispatch of a kernel is then the main workload's)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (scales the HBM byte counters)")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="host only: print the runs of consecutive dispatches of one kernel and "
                         "grid in a rocprofv3 kernel trace (count, mean, later-half mean) and exit")
    ap.add_argument("--write-counters", nargs=4, metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV", "MOPS_CSV"),
                    help="host only: merge three rocprofv3 counter_collection.csv files "
                         "(FETCH_SIZE, WRITE_SIZE, SQ_INSTS_VALU_MFMA_MOPS_BF16; MOPS_CSV may "
                         "be '-') into profiles/counters.json under WORKLOAD and exit")
    args = ap.parse_args()
    if args.trace_summary:
        print("| # | kernel | grid (work-items) | dispatches | mean us | later-half mean us | min us | max us |")
        print("|---|---|---|---|---|---|---|---|")
        for i, (k, g, n, m, h, lo, hi) in enumerate(trace_runs(args.trace_summary)):
            if n >= 3 and not k.startswith("__amd") and not k.startswith("void at::"):
                print(f"| {i} | {k} | {g} | {n} | {m:.2f} | {h:.2f} | {lo:.2f} | {hi:.2f} |")
        return
    if args.write_counters:
        wl, f, wr, m = args.write_counters
        write_counters(wl, f, wr, None if m == "-" else m)
        return
    args.decode_batches = [int(v) for v in args.decode_batches.split(",") if v]
    secondary = [v for v in args.secondary.split(",") if v and v != args.headline]
    for v in secondary:
        if v not in PREFILL_WORKLOADS:
            raise SystemExit(f"unknown prefill workload {v}")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the SSD hot path here is a single-GPU build "
              "(no sharding or collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)                 # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
    extra = {}
    # Every prefill input is generated and moved to HBM first.  The decode half
    # of the metric and the other prefill configurations run next, then the
    # headline prefill's warm-up and timed steps, with no host-side gap (input
    # generation) between the GPU legs.
    def progress(what):
        print(f"[bench] {what} done", file=sys.stderr, flush=True)

    resident = {v: prefill_setup(v) for v in [args.headline] + secondary}
    progress("inputs")
    if not args.no_decode:
        wd, dec = bench_decode(args)
        extra.update(decode_line(wd, dec))
        progress("decode")
        if 256 in args.decode_batches:
            extra["gdn_decode"] = bench_gdn(args)
            progress("gdn decode")
    others = {}
    for v in secondary:
        others[v] = prefill_line(bench_prefill(args, v, resident[v], steps=max(args.steps // 2, 5),
                                                warmup=max(args.warmup, 5)), v)
        del resident[v]
        progress(f"prefill {v}")
    pre = bench_prefill(args, args.headline, resident[args.headline],
                        extras=not args.no_extras)
    progress(f"prefill {args.headline}")
    del resident
    torch.cuda.empty_cache()
    w = pre["w"]
    line = {
        "metric": METRIC,
        "value": pre["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": PREFILL_WORKLOADS[args.headline], **prefill_config(w)},
        "event_ms_per_step": pre["ev_ms"],
        "kernels_ms": pre["kernels_ms"],
        "path_gbs": pre["path_gbs"],
        "roofline": pre["roofline"],
        "roofline_step": pre["roofline_step"],
        "mfma": pre["mfma"],
    }
    if others:
        line["prefill_configs"] = others
    if not args.no_extras:
        line["prefill_fused_dt_softplus"] = dict(
            pre["dt_softplus"],
            note="the same prefill with dt passed as u and softplus(u + dt_bias) formed "
                 "inside the scan kernels (ssd_dims.flags = SSD_DT_SOFTPLUS)")
        line["prefill_varlen"] = bench_varlen(args)
        progress("varlen prefill")
        line["noncached_vs_cached"] = bench_noncached(args)
        progress("non-cached sweep")
    line.update(extra)
    if not args.no_cpu_baseline:
        if "gdn_decode" in line:
            line["gdn_decode"]["cpu_baseline"] = cpu_baseline_gdn()
        if "decode" in line:
            line["decode"]["cpu_baseline"] = cpu_baseline_decode(wd)
            line["decode_steps"]["cpu_baseline"] = dict(
                line["decode"]["cpu_baseline"],
                sample=line["decode"]["cpu_baseline"]["sample"] + " (the oracle has one decode "
                       "form: the same run serves both)")
        line["cpu_baseline"] = cpu_baseline_prefill(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
