#!/usr/bin/env python3
"""Throughput of the Sparse Delta Memory step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--config mid]
                    [--no-cpu-baseline] [--train [--train-dense]]
                    [--front [--d-model 4096]]

One step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: the learned-state copy M[b,h] = M0[h] (sdm_state_init),
the write and read product-key selections (sdm_select x2) and the T-step
gated-delta write + sparse read (sdm_scan).  The state copy (HBM-bound) and the
two selections (ALU-bound, independent of it) run concurrently on two HIP
streams; the scan follows both (--no-overlap runs them back to back).  The
default workload is the
N = 2^20, d_v = 128 configuration "mid" (B8 H8 n1024 T4096 W=R=64, fp32
state); the others are parity-test cases.

Printed: one JSON line with tokens/s of the whole step (B*T tokens per step),
the roofline of the dominant kernel (the scan, HBM-bound; achieved =
algorithmic slot bytes (2W+R)*d_v*4 per head-token times B*H*T, divided by the
scan's mean duration from HIP events on its stream), and the CPU oracle timed
on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SDM scan tokens/sec + slot-traffic HBM GB/s (% of peak), N=2^20, d_v=128"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_mid_traffic.json")
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_bwd_mid_traffic.json")
LONG_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_long_traffic.json")
PROJ_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "project_front_traffic.json")
BF16_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_mid_bf16_traffic.json")
FP8_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_mid_fp8_traffic.json")
LONG_PLANNED_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_long_planned_traffic.json")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
_CSRC = os.path.join(ROOT, "sparse_memory_linear_sdm_amd", "csrc")
SCAN_SOURCES = [os.path.join(_CSRC, f)
                for f in ("scan.hip", "scan_rows.h", "ranges.h", "device_common.h")]
BWD_SOURCES = [os.path.join(_CSRC, f) for f in ("backward.hip", "ranges.h", "device_common.h")]
PROJ_SOURCES = [os.path.join(_CSRC, f) for f in ("project.hip", "device_common.h", "internal.h")]
PLANNED_SOURCES = [os.path.join(_CSRC, f) for f in
                   ("scan_planned.hip", "planned.h", "scan_rows.h", "ranges.h", "device_common.h")]
DECODE_SOURCES = [os.path.join(_CSRC, f) for f in
                  ("decode.hip", "select_wave.h", "device_common.h", "internal.h")]


def _code_only(text: str) -> str:
    """Source text without comments and whitespace, so that counter records
    stay tied to the code itself and not to its commentary."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return re.sub(r"\s+", "", text)


def scan_source_sha(sources=None) -> str:
    h = hashlib.sha256()
    for f in sources or SCAN_SOURCES:
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(n_launch_bytes: float, path=TRAFFIC_FILE, sources=None):
    """HBM bytes per launch from a committed counter summary, or None when
    there is none or the kernel's sources have changed since it was taken."""
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != scan_source_sha(sources):
        return None
    return rec.get("bytes_per_launch")


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(cfg, n_heads: int = 4):
    """The oracle, as it stands, on memories (b, h) for h < n_heads and all b,
    all T steps; one memory per thread.  Returns the record."""
    import numpy as np

    import oracle
    import sdm_inputs as S

    names = ("s1", "s2", "q1", "q2", "v", "alpha", "beta")
    host = {k: S.host_block(cfg, k, 0, cfg.B, 0, n_heads) for k in names}
    M0 = S.host_block(cfg, "M0", h0=0, nh=n_heads)
    jobs = [(b, h) for h in range(n_heads) for b in range(cfg.B)]
    P = min(workers(), len(jobs))

    def run(job):
        b, h = job
        M = M0[h].copy()
        oracle.run_memory(M, oracle.F32, *(host[k][b, h] for k in names), cfg.W, cfg.R)
        return cfg.T

    t0 = time.perf_counter()
    with ThreadPoolExecutor(P) as ex:
        head_steps = sum(ex.map(run, jobs))
    dt = time.perf_counter() - t0
    tokens = head_steps / cfg.H  # one token = H head-steps
    return {"value": tokens / dt, "unit": "tokens/s", "cores": P, "kind": "oracle",
            "sample": f"{len(jobs)} of {cfg.B * cfg.H} memories (heads 0..{n_heads - 1}, all "
                      f"{cfg.B} sequences), all {cfg.T} steps: selections + scan; "
                      f"{dt:.1f} s wall on {P} threads",
            "seconds": dt}


def _common_record(cfg, args, value, unit, ms_step, dtype, workload, roofline, extra):
    rec = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded Philox4x32-10 inputs generated on the GPU)",
        "config": {"workload": workload, "B": cfg.B, "H": cfg.H, "n": cfg.n, "N": cfg.N,
                   "d_v": cfg.d_v, "T": cfg.T, "W": cfg.W, "R": cfg.R, "state": args.state},
        "roofline": roofline,
    }
    rec.update(extra)
    return rec


def calibration_copy(args, torch, dev):
    """One plain device copy of --calib-copy-mib MiB: a kernel of known
    traffic for scaling the HBM byte counters of the same run."""
    if args.calib_copy_mib > 0:
        nelem = args.calib_copy_mib * (1 << 20) // 4
        csrc = torch.ones(nelem, dtype=torch.float32, device=dev)
        cdst = torch.empty_like(csrc)
        torch.cuda.synchronize()
        cdst.copy_(csrc)
        torch.cuda.synchronize()
        del csrc, cdst


def run_prefill(cfg, args, torch, S, sdm):
    """One step = state init + two selections + the T-step scan over the whole
    [B, H, T] batch (the headline workload)."""
    dev = torch.device("cuda:0")
    B, H, T, n, d_v, W, R, N = cfg.B, cfg.H, cfg.T, cfg.n, cfg.d_v, cfg.W, cfg.R, cfg.N
    sdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[args.state]
    es = {"f32": 4, "bf16": 2, "fp8": 1}[args.state]
    print(f"[bench] {cfg.name}: B{B} H{H} n{n} N={N} d_v{d_v} T{T} W{W} R{R} {args.state} "
          f"state; generating inputs on the GPU", file=sys.stderr, flush=True)
    f32 = torch.float32
    inp = {}
    for k in ("s1", "s2", "q1", "q2"):
        inp[k] = torch.empty((B, H, T, n), dtype=f32, device=dev)
    inp["v"] = torch.empty((B, H, T, d_v), dtype=f32, device=dev)
    inp["alpha"] = torch.empty((B, H, T), dtype=f32, device=dev)
    inp["beta"] = torch.empty((B, H, T), dtype=f32, device=dev)
    for k, t in inp.items():
        S.device_block(cfg, k, t)
    M0 = torch.empty((H, N, d_v), dtype=f32, device=dev)
    S.device_block(cfg, "M0", M0)
    M = torch.empty((B, H, N, d_v), dtype=sdt, device=dev)
    widx = torch.empty((B, H, T, W), dtype=torch.int32, device=dev)
    wk = torch.empty((B, H, T, W), dtype=f32, device=dev)
    ridx = torch.empty((B, H, T, R), dtype=torch.int32, device=dev)
    rw = torch.empty((B, H, T, R), dtype=f32, device=dev)
    out = torch.empty((B, H, T, d_v), dtype=f32, device=dev)
    torch.cuda.synchronize()

    calibration_copy(args, torch, dev)

    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()  # default priority
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # --pipeline: the selections of the next batch run on the side stream
    # beside this batch's scan (ALU-bound beside HBM-bound), into the other
    # of two selection buffers; each step still runs one batch's state init,
    # selections and scan.
    sel = [(widx, wk, ridx, rw)]
    if args.pipeline:
        sel.append(tuple(torch.empty_like(x) for x in (widx, wk, ridx, rw)))
    pipe = {"i": 0, "scan_done": [None, None]}

    def select_into(buf, s):
        wi, wkk, ri, rww = sel[buf]
        sdm.select(inp["s1"], inp["s2"], W, out=(wi, None, wkk), stream=s)
        sdm.select(inp["q1"], inp["q2"], R, out=(ri, None, rww), stream=s)

    if args.pipeline:  # batch 0's selections, before the first step
        select_into(0, stream)
        pipe["ready"] = torch.cuda.Event()
        pipe["ready"].record(stream)

    def step_pipelined(record=None):
        i = pipe["i"]
        cur, nxt = i % 2, (i + 1) % 2
        e = [ev() for _ in range(6)]
        e[0].record(stream)
        sdm.state_init(M0, B, out=M, stream=stream)
        e[1].record(stream)
        # next batch's selections: after this init (so they sit beside the
        # scan), and after the scan that last read buffer nxt
        side.wait_event(e[1])
        if pipe["scan_done"][nxt] is not None:
            side.wait_event(pipe["scan_done"][nxt])
        e[2].record(side)
        select_into(nxt, side)
        e[3].record(side)
        stream.wait_event(pipe["ready"])
        e[4].record(stream)
        wi, wkk, ri, rww = sel[cur]
        sdm.scan(M, wi, wkk, ri, rww, inp["v"], inp["alpha"], inp["beta"], out=out,
                 stream=stream)
        e[5].record(stream)
        pipe["scan_done"][cur] = e[5]
        pipe["ready"] = e[3]
        pipe["i"] = i + 1
        if record is not None:
            record.append(e)

    def step(record=None):
        """init on the main stream; the two selections on the side stream (they
        are independent of the init, and ALU-bound while the init is
        HBM-bound); the scan on the main stream after both."""
        if args.pipeline:
            return step_pipelined(record)
        e = [ev() for _ in range(6)]
        e[0].record(stream)
        if args.no_overlap:
            sdm.state_init(M0, B, out=M, stream=stream)
            e[1].record(stream)
            e[2].record(stream)
            sdm.select(inp["s1"], inp["s2"], W, out=(widx, None, wk), stream=stream)
            sdm.select(inp["q1"], inp["q2"], R, out=(ridx, None, rw), stream=stream)
            e[3].record(stream)
        else:
            side.wait_event(e[0])  # the previous scan has consumed the selections
            sdm.state_init(M0, B, out=M, stream=stream)
            e[1].record(stream)
            e[2].record(side)
            sdm.select(inp["s1"], inp["s2"], W, out=(widx, None, wk), stream=side)
            sdm.select(inp["q1"], inp["q2"], R, out=(ridx, None, rw), stream=side)
            e[3].record(side)
            stream.wait_event(e[3])
        e[4].record(stream)
        sdm.scan(M, widx, wk, ridx, rw, inp["v"], inp["alpha"], inp["beta"], out=out,
                 stream=stream)
        e[5].record(stream)
        if record is not None:
            record.append(e)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    g0, g1 = ev(), ev()
    g0.record(stream)
    for _ in range(args.steps):
        step(recs)
    if args.pipeline:
        stream.wait_event(pipe["ready"])  # the last step's selections are inside the span
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = g0.elapsed_time(g1) / args.steps
    init_ms = sum(r[0].elapsed_time(r[1]) for r in recs) / args.steps
    sel_ms = sum(r[2].elapsed_time(r[3]) for r in recs) / args.steps
    scan_ms = sum(r[4].elapsed_time(r[5]) for r in recs) / args.steps

    tokens_per_step = B * T
    slot_bytes = B * H * T * (2 * W + R) * d_v * es  # algorithmic, one scan launch
    scan_gbps = slot_bytes / (scan_ms * 1e-3) / 1e9
    kname = {4: "scan_kernel<float,32,1,false>", 2: "scan_kernel<uint16_t(bf16),32,1,false>",
             1: "scan_kernel<fp8e4m3,32,1,false>"}[es]
    traffic_file = {4: TRAFFIC_FILE, 2: BF16_TRAFFIC_FILE, 1: FP8_TRAFFIC_FILE}[es]
    traffic = measured_traffic(slot_bytes, traffic_file) if cfg.name == "mid" else None
    workload = (f"{cfg.name}: B{B} H{H} n{n} (N={N}) d_v{d_v} T{T} W={W} R={R} "
                f"{args.state} state")
    roofline = {"bound": "hbm", "achieved": scan_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": scan_gbps / HBM_PEAK_GBPS, "traffic": traffic, "kernel": kname,
                "algorithmic_bytes_per_launch": slot_bytes}
    extra = {"breakdown_ms": {"state_init": init_ms, "select_write_read": sel_ms,
                              "scan": scan_ms,
                              "overlap": ("select(k+1) || scan(k)" if args.pipeline else
                                          "select || state_init" if not args.no_overlap
                                          else "none")},
             "scan_tokens_per_s": tokens_per_step / (scan_ms * 1e-3),
             "schedule": ("pipelined: selections of batch k+1 beside the scan of batch k"
                          if args.pipeline else ("serial" if args.no_overlap else
                                                 "selections beside the state init")),
             "wall_s": wall}
    rec = _common_record(cfg, args, tokens_per_step / (ms_step * 1e-3), "tokens/s", ms_step,
                         {4: "f32", 2: "f32 math, bf16 state", 1: "f32 math, fp8 e4m3 state"}[es],
                         workload, roofline, extra)
    if not args.no_cpu_baseline and es == 4:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(cfg, n_heads=cfg.H)  # the whole batch
    else:
        rec["cpu_baseline"] = None
    return rec


def cpu_baseline_train(cfg, n_mem: int = 8):
    """The oracle's training pass (selections, then the backward, which
    replays the forward) on memories (b, 0) for b < n_mem; one per thread."""
    import numpy as np

    import oracle
    import sdm_inputs as S

    names = ("s1", "s2", "q1", "q2", "v", "alpha", "beta")
    nb = min(n_mem, cfg.B)
    host = {k: S.host_block(cfg, k, 0, nb, 0, 1) for k in names}
    dout = S.host_block(cfg, "dout", 0, nb, 0, 1)
    M0 = S.host_block(cfg, "M0", h0=0, nh=1)
    P = min(workers(), nb)

    def run(b):
        wi, _, wk = oracle.select(host["s1"][b, 0], host["s2"][b, 0], cfg.W)
        ri, _, rw = oracle.select(host["q1"][b, 0], host["q2"][b, 0], cfg.R)
        g = oracle.scan_backward(M0[0], wi, wk, ri, rw, host["v"][b, 0], host["alpha"][b, 0],
                                 host["beta"][b, 0], dout[b, 0])
        oracle.select_backward(wi, wk, g["dwk"], cfg.n)
        oracle.select_backward(ri, rw, g["drw"], cfg.n)
        return cfg.T

    t0 = time.perf_counter()
    with ThreadPoolExecutor(P) as ex:
        head_steps = sum(ex.map(run, range(nb)))
    dt = time.perf_counter() - t0
    return {"value": head_steps / cfg.H / dt, "unit": "tokens/s", "cores": P, "kind": "oracle",
            "sample": f"{nb} of {cfg.B * cfg.H} memories (head 0, sequences 0..{nb - 1}), all "
                      f"{cfg.T} steps: selections, forward replay, reverse pass and the "
                      f"selection-weight gradients; {dt:.1f} s wall on {P} threads",
            "seconds": dt}


def run_train(cfg, args, torch, S, sdm):
    """One training step over one batch: the forward (state init, two
    selections beside it, the scan keeping its tape) and the reverse pass
    (the reverse scan, both selection-weight gradients to the halves, and the
    M0 gradient).  The loss reads the outputs only, so the final-state
    gradient is zero: in the sparse mode (default) the rows' last selections
    are recorded beside the forward scan and the gradient table is never
    cleared; --train-dense zeroes it instead and sums all of it."""
    dev = torch.device("cuda:0")
    B, H, T, n, d_v, W, R, N = cfg.B, cfg.H, cfg.T, cfg.n, cfg.d_v, cfg.W, cfg.R, cfg.N
    if args.state != "f32":
        raise SystemExit("--train runs on fp32 state only")
    print(f"[bench] {cfg.name} training step: B{B} H{H} n{n} N={N} d_v{d_v} T{T} W{W} R{R}; "
          f"generating inputs on the GPU", file=sys.stderr, flush=True)
    f32 = torch.float32
    inp = {k: torch.empty((B, H, T, n), dtype=f32, device=dev) for k in ("s1", "s2", "q1", "q2")}
    inp["v"] = torch.empty((B, H, T, d_v), dtype=f32, device=dev)
    inp["dout"] = torch.empty((B, H, T, d_v), dtype=f32, device=dev)
    inp["alpha"] = torch.empty((B, H, T), dtype=f32, device=dev)
    inp["beta"] = torch.empty((B, H, T), dtype=f32, device=dev)
    for k, t in inp.items():
        S.device_block(cfg, k, t)
    M0 = torch.empty((H, N, d_v), dtype=f32, device=dev)
    S.device_block(cfg, "M0", M0)
    M = torch.empty((B, H, N, d_v), dtype=f32, device=dev)
    G = torch.empty((B, H, N, d_v), dtype=f32, device=dev)
    dM0 = torch.empty((H, N, d_v), dtype=f32, device=dev)
    tape = torch.empty((B, H, T, W + R, d_v), dtype=f32, device=dev)
    widx = torch.empty((B, H, T, W), dtype=torch.int32, device=dev)
    wk = torch.empty((B, H, T, W), dtype=f32, device=dev)
    ridx = torch.empty((B, H, T, R), dtype=torch.int32, device=dev)
    rw = torch.empty((B, H, T, R), dtype=f32, device=dev)
    out = torch.empty((B, H, T, d_v), dtype=f32, device=dev)
    wsb = int(sdm.lib().sdm_scan_backward_workspace_size(B, H, d_v, T, W, R))
    ws = torch.empty((wsb + 3) // 4, dtype=f32, device=dev)
    sparse = not args.train_dense
    seen = torch.empty((B, H, (N + 31) // 32), dtype=torch.int32, device=dev) if sparse else None
    first = torch.empty((B, H, T, 2), dtype=torch.int64, device=dev) if sparse else None
    if sparse:
        G.fill_(float("nan"))  # contents never read in this mode
    torch.cuda.synchronize()
    calibration_copy(args, torch, dev)
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()  # default priority
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    x = {"v": inp["v"], "alpha": inp["alpha"], "beta": inp["beta"]}

    def step(record=None):
        e = [ev() for _ in range(12)]
        e[0].record(stream)
        side.wait_event(e[0])
        sdm.state_init(M0, B, out=M, stream=stream)
        e[1].record(stream)
        e[2].record(side)
        sdm.select(inp["s1"], inp["s2"], W, out=(widx, None, wk), stream=side)
        sdm.select(inp["q1"], inp["q2"], R, out=(ridx, None, rw), stream=side)
        e[3].record(side)
        stream.wait_event(e[3])
        e[4].record(stream)
        if sparse:  # after the selections, beside the init or the forward scan
            e[11].record(side)
            sdm.touch_prepare(widx, ridx, N, seen=seen, first=first, stream=side)
            e[10].record(side)
        sdm.scan_train(M, widx, wk, ridx, rw, x["v"], x["alpha"], x["beta"], out=out,
                       tape=tape, stream=stream)
        e[5].record(stream)
        if sparse:
            stream.wait_event(e[10])
        else:
            G.zero_()
        e[6].record(stream)
        g = sdm.scan_backward(widx, wk, ridx, rw, x["v"], x["alpha"], x["beta"], tape,
                              inp["dout"], G, workspace=ws, first=first, stream=stream)
        e[7].record(stream)
        sdm.select_backward(widx, wk, g["dwk"], n, stream=stream)
        sdm.select_backward(ridx, rw, g["drw"], n, stream=stream)
        e[8].record(stream)
        sdm.state_init_backward(G, out=dM0, seen=seen, stream=stream)
        e[9].record(stream)
        if record is not None:
            record.append(e)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    g0, g1 = ev(), ev()
    g0.record(stream)
    for _ in range(args.steps):
        step(recs)
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = g0.elapsed_time(g1) / args.steps
    avg = lambda a, b: sum(r[a].elapsed_time(r[b]) for r in recs) / args.steps  # noqa: E731
    bd = {"state_init": avg(0, 1), "select_write_read": avg(2, 3), "scan_train": avg(4, 5),
          "scan_backward": avg(6, 7), "select_backward": avg(7, 8),
          "state_init_backward": avg(8, 9), "overlap": "select || state_init"}
    if sparse:
        bd["touch_prepare"] = avg(11, 10)
        bd["overlap"] += "; touch_prepare after the selections, beside state_init or scan_train"
        bd["mode"] = "sparse (gradient table never cleared)"
    else:
        bd["zero_G"] = avg(5, 6)
        bd["mode"] = "dense (gradient table zeroed)"
    # reverse: G's W + R rows read and written, the tape's W + R rows read;
    # forward with tape: M's W rows read and written and R rows read, W + R
    # tape rows written.  In the sparse mode a row's first touch in reverse
    # reads no G: those gathers (counted from the masks) are not algorithmic.
    bwd_bytes = B * H * T * (3 * W + 3 * R) * d_v * 4
    if sparse:
        import numpy as np

        fm = first.cpu().numpy().view(np.uint8)
        skipped = int(np.unpackbits(fm).sum())
        bwd_bytes -= skipped * d_v * 4
        bd["first_touch_slots"] = skipped
    fwd_bytes = B * H * T * (3 * W + 2 * R) * d_v * 4
    gbps = bwd_bytes / (bd["scan_backward"] * 1e-3) / 1e9
    workload = (f"{cfg.name} training step: B{B} H{H} n{n} (N={N}) d_v{d_v} T{T} W={W} R={R} "
                f"f32 state, {'sparse' if sparse else 'dense'} gradient table")
    traffic = (measured_traffic(bwd_bytes, BWD_TRAFFIC_FILE, BWD_SOURCES)
               if cfg.name == "mid" and sparse else None)
    roofline = {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": gbps / HBM_PEAK_GBPS, "traffic": traffic,
                "kernel": ("scan_bwd_kernel<16>" if sparse else "scan_bwd_kernel<32>") + " + scan_bwd_finish",
                "algorithmic_bytes_per_launch": bwd_bytes}
    extra = {"breakdown_ms": bd, "wall_s": wall,
             "scan_train_GBps": fwd_bytes / (bd["scan_train"] * 1e-3) / 1e9,
             "backward_tokens_per_s": B * T / (bd["scan_backward"] * 1e-3)}
    rec = _common_record(cfg, args, B * T / (ms_step * 1e-3), "tokens/s", ms_step, "f32",
                         workload, roofline, extra)
    rec["metric"] = METRIC + " (training step: forward + reverse pass)"
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle's training pass on a bounded sample",
              file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline_train(cfg)
    else:
        rec["cpu_baseline"] = None
    return rec


def run_decode(cfg, args, torch, S, sdm):
    """One step = the T single-token calls of one batch of sequences
    (sdm_step_decode on every (b,h)); the state is initialised once before the
    timed steps and persists, as in generation."""
    dev = torch.device("cuda:0")
    B, H, T, n, d_v, W, R, N = cfg.B, cfg.H, cfg.T, cfg.n, cfg.d_v, cfg.W, cfg.R, cfg.N
    sdt = torch.bfloat16 if args.state == "bf16" else torch.float32
    es = 2 if args.state == "bf16" else 4
    print(f"[bench] {cfg.name}: B{B} H{H} n{n} N={N} d_v{d_v} {T} calls W{W} R{R} {args.state} "
          f"state", file=sys.stderr, flush=True)
    f32 = torch.float32
    # per-call inputs laid out [T, B, H, ...] so each call's slice is contiguous
    inp = {}
    for k in ("s1", "s2", "q1", "q2", "v", "alpha", "beta"):
        last = (n,) if k in ("s1", "s2", "q1", "q2") else ((d_v,) if k == "v" else ())
        tmp = torch.empty((B, H, T) + last, dtype=f32, device=dev)
        S.device_block(cfg, k, tmp)
        inp[k] = tmp.movedim(2, 0).contiguous()
        del tmp
    M0 = torch.empty((H, N, d_v), dtype=f32, device=dev)
    S.device_block(cfg, "M0", M0)
    M = sdm.state_init(M0, B, sdt)
    del M0
    torch.cuda.empty_cache()
    calibration_copy(args, torch, dev)
    out = torch.empty((B, H, d_v), dtype=f32, device=dev)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    names = ("s1", "s2", "q1", "q2", "v", "alpha", "beta")

    def calls():
        for t in range(T):
            sdm.step_decode(M, *(inp[k][t] for k in names), W, R, out=out, want_idx=False)

    # The T calls are captured once into a HIP graph and replayed, so the host
    # launch cost of T small kernels is not what gets measured.
    calls()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0, g1 = ev(), ev()
    g0.record(stream)
    for _ in range(args.steps):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = g0.elapsed_time(g1) / args.steps
    per_call_us = ms_step * 1e3 / T
    call_bytes = B * H * ((2 * W + R) * d_v * es + 4 * n * 4 + d_v * 4 * 2)
    gbps = call_bytes / (per_call_us * 1e-6) / 1e9
    workload = (f"{cfg.name}: B{B} H{H} n{n} (N={N}) d_v{d_v} {T} single-token calls "
                f"W={W} R={R} {args.state} state")
    # counted bytes per call, from the committed counter summary of the bf16 decode workload
    traffic = (measured_traffic(call_bytes, DECODE_TRAFFIC_FILE, DECODE_SOURCES)
               if es == 2 else None)
    roofline = {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": gbps / HBM_PEAK_GBPS, "traffic": traffic,
                "kernel": "decode_kernel<16,bf16>" if es == 2 else "decode_kernel<16,f32>",
                "algorithmic_bytes_per_launch": call_bytes}
    extra = {"us_per_call": per_call_us, "wall_s": wall, "cpu_baseline": None}
    return _common_record(cfg, args, B * T / (ms_step * 1e-3), "tokens/s", ms_step,
                          "f32 math, bf16 state" if es == 2 else "f32", workload, roofline,
                          extra)


def cpu_baseline_front(cfg, d_model: int, n_tokens: int = 512):
    """The oracle's projections and selections for the first n_tokens tokens
    of sequence 0, all heads; the tokens split over the threads."""
    import numpy as np

    import oracle
    import sdm_inputs as S

    H, n, d_v = cfg.H, cfg.n, cfg.d_v
    P = 4 * n + d_v + 2
    Xb, Wb = S.projection_inputs(1, n_tokens, d_model, H, P, seed=11)
    Pw = min(workers(), n_tokens)
    t0 = time.perf_counter()
    y, _ = oracle.project(Xb[0], Wb, H, threads=Pw)
    halves = y[:, :, :4 * n].astype(np.float32)  # the binary32 values the selection takes
    oracle.select(halves[..., :n], halves[..., n:2 * n], cfg.W, threads=Pw)
    oracle.select(halves[..., 2 * n:3 * n], halves[..., 3 * n:], cfg.R, threads=Pw)
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": Pw, "kind": "oracle",
            "sample": f"{n_tokens} tokens x {H} heads, d_model {d_model}: projections "
                      f"(float64 dot products) + write and read selections; {dt:.1f} s wall "
                      f"on {Pw} threads", "seconds": dt}


def run_front(cfg, args, torch, S, sdm):
    """One step = the front end over the whole [B, T] batch: the token
    projections (sdm_project, one MFMA GEMM of B*T x d_model by d_model x
    H*(4n + d_v + 2)) and the write and read selections on its halves."""
    dev = torch.device("cuda:0")
    B, H, T, n, d_v, W, R, N = cfg.B, cfg.H, cfg.T, cfg.n, cfg.d_v, cfg.W, cfg.R, cfg.N
    d_model = args.d_model or 2 * n * H
    P = 4 * n + d_v + 2
    print(f"[bench] front end {cfg.name}: B{B} T{T} d_model{d_model} -> H{H} x P{P} "
          f"(n{n} d_v{d_v}), selections W{W} R{R}; generating inputs on the host",
          file=sys.stderr, flush=True)
    Xb, Wb = S.projection_inputs(B, T, d_model, H, P, seed=2024)
    X = torch.from_numpy(Xb.view("int16")).to(dev).view(torch.bfloat16)
    Wt = torch.from_numpy(Wb.view("int16")).to(dev).view(torch.bfloat16)
    del Xb, Wb
    f32 = torch.float32
    outs = tuple(torch.empty(sh, dtype=f32, device=dev) for sh in
                 [(B, H, T, n)] * 4 + [(B, H, T, d_v), (B, H, T), (B, H, T)])
    widx = torch.empty((B, H, T, W), dtype=torch.int32, device=dev)
    wk = torch.empty((B, H, T, W), dtype=f32, device=dev)
    ridx = torch.empty((B, H, T, R), dtype=torch.int32, device=dev)
    rw = torch.empty((B, H, T, R), dtype=f32, device=dev)
    torch.cuda.synchronize()
    calibration_copy(args, torch, dev)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(record=None):
        e = [ev() for _ in range(3)]
        e[0].record(stream)
        sdm.project(X, Wt, n, out=outs, stream=stream)
        e[1].record(stream)
        sdm.select(outs[0], outs[1], W, out=(widx, None, wk), stream=stream)
        sdm.select(outs[2], outs[3], R, out=(ridx, None, rw), stream=stream)
        e[2].record(stream)
        if record is not None:
            record.append(e)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    g0, g1 = ev(), ev()
    g0.record(stream)
    for _ in range(args.steps):
        step(recs)
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = g0.elapsed_time(g1) / args.steps
    proj_ms = sum(r[0].elapsed_time(r[1]) for r in recs) / args.steps
    sel_ms = sum(r[1].elapsed_time(r[2]) for r in recs) / args.steps
    flops = 2.0 * B * T * d_model * H * P  # algorithmic, one projection launch
    tflops = flops / (proj_ms * 1e-3) / 1e12
    workload = (f"front end of {cfg.name}: B{B} T{T} d_model{d_model} -> H{H} (n{n}, N={N}, "
                f"d_v{d_v}), bf16 projections + selections W={W} R={R}")
    # traffic: HBM bytes per launch from the committed counter summary (null
    # once the kernel's sources differ from the ones it was taken on)
    traffic = measured_traffic(flops, path=PROJ_TRAFFIC_FILE, sources=PROJ_SOURCES) \
        if (B, T, H, n, d_v, d_model) == (8, 4096, 8, 1024, 128, 16384) else None
    roofline = {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic,
                "kernel": "project_kernel", "algorithmic_flops_per_launch": flops}
    extra = {"breakdown_ms": {"project": proj_ms, "select_write_read": sel_ms},
             "d_model": d_model, "wall_s": wall}
    rec = _common_record(cfg, args, B * T / (ms_step * 1e-3), "tokens/s", ms_step,
                         "bf16 in, f32 accumulate", workload, roofline, extra)
    rec["config"]["d_model"] = d_model
    rec["data"] = ("synthetic (seeded PCG64 bf16 tokens and random projection weights, "
                   "generated on the host)")
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline_front(cfg, d_model)
    else:
        rec["cpu_baseline"] = None
    return rec


def run_long(cfg, args, torch, S, sdm):
    """One step = the whole T = 2^20 stream in chunks of 16384 steps.  The
    inputs of each chunk are generated on the GPU outside the timed spans.
    Timed: the selections (and plan) of chunk 0, then per chunk c one span
    holding the scan of chunk c on the main stream and, beside it on a
    second stream, the selections and plan of chunk c + 1 (the planned
    scan's workgroups, two per CU, leave LDS and wave slots free).  The scan
    is the planned scan (sdm_scan_plan + sdm_scan_planned); --sdm-scan runs
    sdm_scan on the selections instead.  --no-overlap times selections and
    scan of each chunk in turn."""
    dev = torch.device("cuda:0")
    B, H, T, n, d_v, W, R, N = cfg.B, cfg.H, cfg.T, cfg.n, cfg.d_v, cfg.W, cfg.R, cfg.N
    C = 16384
    nch = T // C
    f32 = torch.float32
    print(f"[bench] {cfg.name}: B{B} H{H} n{n} N={N} d_v{d_v} T{T} in chunks of {C}",
          file=sys.stderr, flush=True)
    M0 = torch.empty((H, N, d_v), dtype=f32, device=dev)
    S.device_block(cfg, "M0", M0)
    M = sdm.state_init(M0, B)
    del M0
    nbuf = 1 if args.no_overlap else 2
    inp, sel = [], []
    for _ in range(nbuf):
        d = {k: torch.empty((B, H, C, n), dtype=f32, device=dev) for k in ("s1", "s2", "q1", "q2")}
        d["v"] = torch.empty((B, H, C, d_v), dtype=f32, device=dev)
        d["alpha"] = torch.empty((B, H, C), dtype=f32, device=dev)
        d["beta"] = torch.empty((B, H, C), dtype=f32, device=dev)
        inp.append(d)
        sel.append((torch.empty((B, H, C, W), dtype=torch.int32, device=dev),
                    torch.empty((B, H, C, W), dtype=f32, device=dev),
                    torch.empty((B, H, C, R), dtype=torch.int32, device=dev),
                    torch.empty((B, H, C, R), dtype=f32, device=dev)))
    out = torch.empty((B, H, C, d_v), dtype=f32, device=dev)
    planned = not args.sdm_scan
    if planned:  # one plan workspace per chunk buffer
        wsb = sdm.scan_plan_workspace_size(B, H, d_v, C)
        plans = [torch.empty((wsb,), dtype=torch.uint8, device=dev) for _ in range(nbuf)]
    torch.cuda.synchronize()
    calibration_copy(args, torch, dev)
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()  # default priority
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def generate(c):
        for k, t in inp[c % nbuf].items():
            S.device_block(cfg, k, t, 0, 0, c * C)

    def select(c, s):
        x, (wi, wkk, ri, rww) = inp[c % nbuf], sel[c % nbuf]
        sdm.select(x["s1"], x["s2"], W, out=(wi, None, wkk), stream=s)
        sdm.select(x["q1"], x["q2"], R, out=(ri, None, rww), stream=s)
        if planned:  # the planned scan's lists for this chunk, beside the previous scan too
            sdm.scan_plan(wi, wkk, ri, rww, N, d_v, workspace=plans[c % nbuf], stream=s)

    def scan(c):
        x, (wi, wkk, ri, rww) = inp[c % nbuf], sel[c % nbuf]
        if planned:
            sdm.scan_planned(M, x["v"], x["alpha"], x["beta"], plans[c % nbuf], out=out,
                             stream=stream)
        else:
            sdm.scan(M, wi, wkk, ri, rww, x["v"], x["alpha"], x["beta"], out=out, stream=stream)

    def timed(fn):
        e0, e1 = ev(), ev()
        e0.record(stream)
        fn(e0)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    sel_ms = scan_ms = span_ms = 0.0
    steps = max(1, args.steps)
    t0w = time.perf_counter()
    for rep in range(steps):
        if args.no_overlap:
            for c in range(nch):
                generate(c)
                torch.cuda.synchronize()
                sel_ms += timed(lambda e0, c=c: select(c, stream))
                scan_ms += timed(lambda e0, c=c: scan(c))
        else:
            generate(0)
            torch.cuda.synchronize()
            sel_ms += timed(lambda e0: select(0, stream))
            for c in range(nch):
                if c + 1 < nch:
                    generate(c + 1)  # the buffers of chunk c - 1, whose scan has finished
                    torch.cuda.synchronize()

                es = [ev(), ev()]

                def body(e0, c=c, es=es):
                    if c + 1 < nch:
                        side.wait_event(e0)
                        select(c + 1, side)
                        e_side = torch.cuda.Event()
                        e_side.record(side)
                    es[0].record(stream)
                    scan(c)
                    es[1].record(stream)
                    if c + 1 < nch:
                        stream.wait_event(e_side)
                span_ms += timed(body)
                scan_ms += es[0].elapsed_time(es[1])  # the scan kernel alone, on its stream
    wall = time.perf_counter() - t0w
    sel_ms /= steps
    scan_ms /= steps
    span_ms /= steps
    ms_step = sel_ms + scan_ms if args.no_overlap else sel_ms + span_ms
    slot_bytes = B * H * T * (2 * W + R) * d_v * 4
    gbps = slot_bytes / (scan_ms * 1e-3) / 1e9
    workload = f"{cfg.name}: B{B} H{H} n{n} (N={N}) d_v{d_v} T{T} W={W} R={R} fp32 state"
    if planned:
        workload += ", planned scan"
        kernel = ("planned_kernel<7,2,16>, eight row shards of 32-column tiles (duration includes "
                  "the shards' combine kernel of the same call)")
        traffic = measured_traffic(slot_bytes // nch, LONG_PLANNED_TRAFFIC_FILE, PLANNED_SOURCES)
    else:
        kernel = ("scan_kernel<float,16,3,false>, two row shards (duration includes the output "
                  "zero fill of the same call)")
        traffic = measured_traffic(slot_bytes // nch, LONG_TRAFFIC_FILE)
    roofline = {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": gbps / HBM_PEAK_GBPS, "traffic": traffic, "kernel": kernel,
                "algorithmic_bytes_per_launch": slot_bytes // nch}
    side_work = "selections and plan" if planned else "selections"
    bd = ({"select_write_read": sel_ms, "scan": scan_ms} if args.no_overlap else
          {"select_chunk0": sel_ms, "spans": span_ms, "scan": scan_ms,
           "overlap": f"{side_work} of chunk c+1 || scan of chunk c"})
    extra = {"breakdown_ms": bd, "wall_s": wall, "cpu_baseline": None}
    return _common_record(cfg, args, B * T / (ms_step * 1e-3), "tokens/s", ms_step, "f32",
                          workload, roofline, extra)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="mid",
                    help="mid (default, the headline), small, decode or long")
    ap.add_argument("--state", default=None,
                    help="f32, bf16 or fp8 (E4M3) (default: the config's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--train", action="store_true",
                    help="time a training step (forward with tape + reverse pass) instead")
    ap.add_argument("--train-dense", action="store_true",
                    help="with --train: zero the gradient table and sum all of it (dense mode)"
                         " instead of the sparse-mode bookkeeping")
    ap.add_argument("--sdm-scan", action="store_true",
                    help="with --config long: run the chunks with sdm_scan on the selections "
                         "instead of the planned scan (sdm_scan_plan beside the previous "
                         "chunk, then sdm_scan_planned)")
    ap.add_argument("--front", action="store_true",
                    help="time the front end instead: token projections (bf16 MFMA GEMM) + "
                         "the two selections")
    ap.add_argument("--d-model", type=int, default=0,
                    help="with --front: model width feeding the projections (default 2*n*H: "
                         "the key projection as wide as the model, as in the baseline)")
    ap.add_argument("--no-overlap", action="store_true",
                    help="run the step's kernels back to back on one stream")
    ap.add_argument("--pipeline", action="store_true",
                    help="prefill: run the next batch's selections beside this batch's scan")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before the steps, run one plain device copy of this many MiB "
                         "(a known-size kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs the SDM step on one GPU only: each (b,h) memory is independent, "
              "so several GPUs would each run their own share with no exchange; "
              "use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import sdm_inputs as S
    import sparse_memory_linear_sdm_amd as sdm

    if not os.path.exists(sdm.LIB_PATH) or not os.path.exists(S.DEV_LIB):
        import __graft_entry__

        __graft_entry__.build()

    cfg = S.CONFIGS[args.config]
    if args.state is None:
        args.state = cfg.state
    if args.front:
        rec = run_front(cfg, args, torch, S, sdm)
    elif args.train:
        rec = run_train(cfg, args, torch, S, sdm)
    elif cfg.decode:
        rec = run_decode(cfg, args, torch, S, sdm)
    elif cfg.name == "long":
        rec = run_long(cfg, args, torch, S, sdm)
    else:
        rec = run_prefill(cfg, args, torch, S, sdm)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
