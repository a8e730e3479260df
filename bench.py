#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one forward (fa_fwd) and one backward (fa_bwd: D preprocess,
dK/dV kernel, dQ kernel) over one batch of synthetic inputs that are already
resident in HBM. The default workload is GPT-2-medium-shaped attention:
batch 64, 16 heads, N = 1024, d = 64, bf16, non-causal (the FlashAttention
paper's forward+backward micro-benchmark shape).

Prints one JSON line with whole-job throughput (algorithmic fwd+bwd TFLOP/s),
per-kernel HIP-event timings, the dominant kernel's roofline position, and
the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd & fwd+bwd TFLOP/s + % of bf16 MFMA peak, B64 H16 N1024 d64"
DECODE_METRIC = ("decode attention KV-cache read GB/s (one query row per head), "
                 "B16 Hq32 Hkv8 cache 32K d128")
KERNEL_SOURCES = {
    "decode": ["fa_decode.hip", "fa_stage.h", "fa_device.h"],
    "decode_combine": ["fa_decode.hip"],
    "fwd": ["fa_fwd.hip", "fa_stage.h", "fa_device.h", "fa_philox.h"],
    "fwd_fp8": ["fa_fwd_fp8.hip", "fa_stage.h", "fa_device.h"],
    "bwd_dkdv": ["fa_bwd.hip", "fa_stage.h", "fa_device.h", "fa_philox.h"],
    "bwd_dq": ["fa_bwd.hip", "fa_stage.h", "fa_device.h", "fa_philox.h"],
}


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="write this many MiB of scratch between timed steps (outside the "
                         "kernel events) so that no K/V tile survives in L2 or MALL from one "
                         "step to the next; value then comes from the summed kernel times")
    ap.add_argument("--workload", type=int, default=2,
                    help="workload id (2 = the headline B64 H16 N1024 d64 shape; 7 = decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (for profiler runs)")
    ap.add_argument("--no-w3-record", action="store_true",
                    help="with the default workload, skip the w3_record field (the causal "
                         "key-padded B8 H16 N4096 d128 workload measured in the same run)")
    ap.add_argument("--w3-steps", type=int, default=20,
                    help="timed steps of the w3_record measurement")
    ap.add_argument("--w3-warmup", type=int, default=5,
                    help="untimed warmup steps of the w3_record measurement")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--io-sweep", action="store_true",
                    help="instead of the benchmark: forward + backward at N = 1K .. 16K, d = 128, "
                         "B * H * N fixed, one JSON line per N with the three byte models")
    ap.add_argument("--fill", choices=("random", "zeros", "half"), default="random",
                    help="power analysis only: overwrite Q, K, V and dO with zeros or 0.5 "
                         "(same shapes, masks and kernels; the data field says so). The clock "
                         "follows board power, so timing depends on the data")
    ap.add_argument("--timeline", action="store_true",
                    help="instead of the benchmark line: time the workload with the release "
                         "library, then with libfa_timeline.so (per-workgroup stamps in the "
                         "16x16x32 kernels), and print one JSON line per stamped kernel: slot "
                         "occupancy, time outside the tile loops, per-XCD speed and end times")
    ap.add_argument("--mix-ceiling", action="store_true",
                    help="instead of the benchmark: time the instruction-mix grid of "
                         "libfa_mixbench.so (64 matrix products per wave-tile with E "
                         "exponentials and F other VALU operations, two waves per SIMD); one "
                         "JSON line per mix")
    return ap.parse_args()


MIX_ITERS = 1024     # wave-tiles per wave in one timed launch
MIX_REPS = 3         # timed launches per mix (the best one counts)
MIX_WAVES = 512 * 4  # 512 workgroups of four waves: two per SIMD on 256 CUs


def mix_ceiling():
    """Time every mix of the measurement library's grid and print one JSON
    line each: nanoseconds per wave-tile per SIMD (two waves share a SIMD)
    and the matrix-product rate that mix allows."""
    import ctypes

    path = os.path.join(ROOT, "exact_io_aware_29_amd", "libfa_mixbench.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_io_aware_29_amd.build`")
    lib = ctypes.CDLL(path)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.fa_mixbench_grid.restype = ctypes.c_int
    lib.fa_mixbench_grid.argtypes = [ip, ip, ip, ip, ip]
    lib.fa_mixbench.restype = ctypes.c_int
    lib.fa_mixbench.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(ctypes.c_float)]
    ne, nf, nl = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    rows, trs = (ctypes.c_int * 8)(), (ctypes.c_int * 8)()
    lib.fa_mixbench_grid(ctypes.byref(ne), ctypes.byref(nf), ctypes.byref(nl), rows, trs)
    # About a second of the heaviest mix first, so that every timed mix runs
    # at the board's settled clock and power (the first launches of a fresh
    # process otherwise run while the clock is still moving).
    ms = ctypes.c_float()
    rc = lib.fa_mixbench(ne.value - 1, nf.value - 1, nl.value - 1, 4 * MIX_ITERS, 200,
                         ctypes.byref(ms))
    if rc != 0:
        raise RuntimeError(f"fa_mixbench warm-up failed with code {rc}")
    flops = MIX_WAVES * MIX_ITERS * 64 * 2 * 16 * 16 * 32
    for li in range(nl.value):
        for ei in range(ne.value):
            for fi in range(nf.value):
                rc = lib.fa_mixbench(ei, fi, li, MIX_ITERS, MIX_REPS, ctypes.byref(ms))
                if rc != 0:
                    raise RuntimeError(f"fa_mixbench({ei}, {fi}, {li}) failed with code {rc}")
                print(json.dumps({
                    "mix_ceiling": True, "mfma_per_tile": 64, "exp_per_tile": 8 * ei,
                    "valu_per_tile": 32 * fi, "lds_row_reads": rows[li], "lds_tr_reads": trs[li],
                    "ms": round(ms.value, 4),
                    "ns_per_wave_tile_per_simd": round(ms.value * 1e6 / (2 * MIX_ITERS), 1),
                    "tflops": round(flops / (ms.value * 1e-3) / 1e12, 1)}), flush=True)


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "exact_io_aware_29_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str, workload: int):
    """HBM bytes per launch measured by rocprofv3 counters, if the summary in
    profiles/ was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_w{workload}.md")
    if not os.path.exists(path):
        return None
    pat = re.compile(r"^traffic\s+(\S+)\s+bytes_per_launch=(\d+)\s+src=(\w+)", re.M)
    with open(path) as fh:
        for name, nbytes, src in pat.findall(fh.read()):
            if name == kernel and src == source_hash(kernel):
                return int(nbytes)
    return None


def cpu_baseline(inp, pairs_per_head, budget_s):
    """Time the fp64 oracle's forward + backward head by head until the time
    budget is spent; report algorithmic TFLOP/s over the heads done."""
    import numpy as np
    import oracle
    from oracle.attention import mask_for

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    w = inp.workload
    G = w.heads_q // w.heads_kv
    dr = None if w.dropout is None else oracle.Dropout(float(np.float32(w.dropout[0])),
                                                       w.dropout[1], w.dropout[2])
    done, flop = 0, 0
    t0 = time.perf_counter()
    if w.seqlen > 8192:
        # One whole head would take minutes: time row chunks of head (0, 0)
        # instead -- the forward and the dQ part of the backward (S, dP, dQ
        # rebuilt for those rows), counted as (4 + 6) d per allowed pair.
        from exact_io_aware_29_amd import accounting as acc
        m = mask_for(0, causal=w.causal, seqlens=inp.seqlens, block_mask=inp.block_mask,
                     window=w.window)
        per_row = acc.allowed_pairs_per_row(
            w.seqlen, causal=w.causal, seqlen_k=None if inp.seqlens is None else int(inp.seqlens[0]),
            block_mask=inp.block_mask, window=w.window)
        q, k, v = inp.as_f64("q", (0, 0)), inp.as_f64("k", (0, 0)), inp.as_f64("v", (0, 0))
        do = inp.as_f64("do", (0, 0)) if w.backward else None
        drop = None if dr is None else dr.head(0)
        rows_done = 0
        for r0 in range(0, w.seqlen, 256):
            rows = np.arange(r0, min(r0 + 256, w.seqlen))
            oracle.head_forward(q, k, v, inp.scale, m, rows=rows, drop=drop)
            if w.backward:
                oracle.head_backward(q, k, v, do, inp.scale, m, q_rows=rows, drop=drop)
            rows_done += len(rows)
            flop += ((4 + 6) if w.backward else 4) * w.head_dim * int(per_row[rows].sum())
            if time.perf_counter() - t0 >= budget_s:
                break
        el = time.perf_counter() - t0
        return {"value": round(flop / el / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
                "kind": "oracle", "cpu": cpu_model(), "blas": blas_info(),
                "sample": f"fp64 oracle forward{' and the dQ part of the backward' if w.backward else ''}"
                          f" over the first {rows_done} rows of (batch 0, head 0), {el:.1f} s; "
                          f"{'(4 + 6)' if w.backward else '4'} d flops per allowed pair"}
    for b in range(w.batch):
        m = mask_for(b, causal=w.causal, seqlens=inp.seqlens, block_mask=inp.block_mask,
                     window=w.window)
        for h in range(w.heads_q):
            q = inp.as_f64("q", (b, h))
            k = inp.as_f64("k", (b, h // G))
            v = inp.as_f64("v", (b, h // G))
            drop = None if dr is None else dr.head(b * w.heads_q + h)
            oracle.head_forward(q, k, v, inp.scale, m, drop=drop)
            if w.backward:
                oracle.head_backward(q, k, v, inp.as_f64("do", (b, h)), inp.scale, m, drop=drop)
            done += 1
            flop += (14 if w.backward else 4) * w.head_dim * pairs_per_head[b]
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {
        "value": round(flop / el / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "cpu": cpu_model(),
        "blas": blas_info(),
        "sample": f"fp64 oracle {'fwd+bwd' if w.backward else 'fwd'} of the first {done} (batch, head) pairs of "
                  f"{w.batch * w.heads_q}, {el:.1f} s; same algorithmic flop count",
    }


def decode_cpu_baseline(inp, budget_s):
    """Time the fp64 oracle's decode batch entry by batch entry until the
    budget is spent; report GB/s of the same algorithmic bytes."""
    import oracle
    from exact_io_aware_29_amd import accounting as acc

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    w = inp.workload
    done, nbytes = 0, 0
    t0 = time.perf_counter()
    for b in range(w.batch):
        sl = slice(b, b + 1)
        oracle.attention_decode(inp.as_f64("q", (sl,))[:, :, 0, :], inp.as_f64("k", (sl,)),
                                inp.as_f64("v", (sl,)), inp.scale, seqlens=inp.seqlens[sl])
        done += 1
        nbytes += acc.decode_bytes(1, w.heads_q, w.heads_kv, w.head_dim, inp.seqlens[sl])
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle", "cpu": cpu_model(), "blas": blas_info(),
            "sample": f"fp64 oracle decode of the first {done} of {w.batch} sequences, "
                      f"{el:.1f} s; same algorithmic bytes"}


def decode_main(args, w, inp, dev):
    """One step = one fa_decode call (split kernel + combine) over the batch."""
    import numpy as np
    import torch

    import exact_io_aware_29_amd as fa
    from exact_io_aware_29_amd import accounting as acc

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = t(inp.q), t(inp.k), t(inp.v)
    sl = None if inp.seqlens is None else torch.from_numpy(inp.seqlens).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    p = fa.make_params(batch=w.batch, heads_q=w.heads_q, heads_kv=w.heads_kv, seqlen=w.seqlen,
                       head_dim=w.head_dim)
    ws = torch.empty(fa.fa_decode_workspace_size(p) // 4 + 4, dtype=torch.float32, device=dev)

    def step():
        fa.fa_decode(q, k, v, scale=inp.scale, seqlens_k=sl, out=o, lse=lse, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for ev in events:
        for e in ev:
            e.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        events[i][0].record()
        step()
        events[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(np.mean([events[i][0].elapsed_time(events[i][1]) for i in range(args.steps)]))
    copy_calibration(args, dev)
    lens = inp.seqlens if inp.seqlens is not None else [w.seqlen] * w.batch
    nbytes = acc.decode_bytes(w.batch, w.heads_q, w.heads_kv, w.head_dim, lens)
    ms_step = wall / args.steps * 1e3
    value = nbytes / (ms_step * 1e-3) / 1e9
    ach = nbytes / (ms * 1e-3) / 1e9
    kernels = {"decode": {"ms": round(ms, 4), "bound": "hbm", "achieved": round(ach, 1),
                          "peak": acc.HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(ach / acc.HBM_PEAK_GBS, 4)}}
    rec = {
        "metric": DECODE_METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs, rounded to bf16)",
        "config": {"workload": w.describe(), "batch": w.batch, "heads_q": w.heads_q,
                   "heads_kv": w.heads_kv, "cache_len": w.seqlen, "head_dim": w.head_dim,
                   "pass": "decode"},
        "algorithmic_bytes": nbytes,
        "device": device_info(),
        "kernels": kernels,
        "roofline": dict(kernel="decode", **{k_: kernels["decode"][k_] for k_ in
                                             ("bound", "achieved", "peak", "unit", "frac")},
                         traffic=decode_traffic(args.workload)),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = decode_cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def decode_traffic(workload: int):
    """Counter bytes of one decode pass: the split kernel plus the combine
    kernel, both inside the timed region (None if either record is stale)."""
    a = recorded_traffic("decode", workload)
    b = recorded_traffic("decode_combine", workload)
    return None if a is None or b is None else a + b


def device_info():
    """Name, compute units and architecture of the GPU the numbers come from."""
    import torch
    pr = torch.cuda.get_device_properties(0)
    rec = {"name": pr.name, "compute_units": pr.multi_processor_count,
           "arch": getattr(pr, "gcnArchName", ""),
           "peak_clock_assumed_mhz": 2400}
    clk = getattr(pr, "clock_rate", None)  # kHz, where torch exposes it
    if clk:
        rec["max_clock_mhz"] = round(clk / 1000)
    return rec


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_info():
    """The BLAS numpy's oracle runs on, as threadpoolctl reports it."""
    try:
        import numpy  # noqa: F401  (loads the BLAS, so that it is listed)
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                arch = f" ({i['architecture']})" if i.get("architecture") else ""
                return f"{i.get('internal_api', '?')} {i.get('version', '?')}{arch}"
    except Exception:  # pragma: no cover
        pass
    return "unknown"


def copy_calibration(args, dev):
    """A plain device copy of known size, run (outside every timed region)
    so that one counter pass also reads FETCH_SIZE / WRITE_SIZE for it."""
    if not args.copy_calib_mib:
        return
    import torch
    n = args.copy_calib_mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


IO_SWEEP_N = (1024, 2048, 4096, 8192, 16384)


def io_sweep(args):
    """Non-causal bf16 attention at d = 128 with B * H * N fixed at 2^19 rows
    (H = 16): compulsory bytes stay constant over the sweep while the tile
    model and Algorithm 0 grow in proportion to N. Prints per N the timings
    and the byte models; the HBM bytes come from counter passes over this
    same command (one kernel dispatch group per N, in this order)."""
    import numpy as np
    import torch

    import exact_io_aware_29_amd as fa
    from exact_io_aware_29_amd import accounting as acc

    dev = torch.device("cuda:0")
    d, H = 128, 16
    for N in IO_SWEEP_N:
        B = (1 << 19) // (H * N)
        g = torch.Generator(device="cpu").manual_seed(N)
        q, k, v, do = (torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
                       .to(torch.bfloat16).to(dev) for _ in range(4))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        p = fa.make_params(batch=B, heads_q=H, heads_kv=H, seqlen=N, head_dim=d)
        ws = torch.empty(fa.fa_bwd_workspace_size(p) // 4 + 4, dtype=torch.float32, device=dev)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        tf, tb = [], []
        for it in range(args.warmup + args.steps):
            ev[0].record()
            fa.fa_fwd(q, k, v, out=o, lse=lse)
            ev[1].record()
            fa.fa_bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws)
            ev[2].record()
            torch.cuda.synchronize()
            if it >= args.warmup:
                tf.append(ev[0].elapsed_time(ev[1]))
                tb.append(ev[1].elapsed_time(ev[2]))
        tiles = B * H * (N // 128) ** 2
        m = acc.bytes_models(B, H, H, N, d, 2, tiles=tiles)
        fl = acc.flops(B * H * N * N, d)
        print(json.dumps({"io_sweep": True, "N": N, "batch": B, "heads": H, "head_dim": d,
                          "fwd_ms": round(float(np.median(tf)), 4),
                          "bwd_ms": round(float(np.median(tb)), 4),
                          "fwd_tflops": round(fl["fwd"] / (np.median(tf) * 1e-3) / 1e12, 1),
                          "bwd_tflops": round(fl["bwd"] / (np.median(tb) * 1e-3) / 1e12, 1),
                          "bytes_models": m}), flush=True)
        del q, k, v, do, o, dq, dk, dv, ws
    copy_calibration(args, dev)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path shards over "
              "(batch, head) with no communication, so one GPU's figure is the per-GPU rate.",
              file=sys.stderr)
        sys.exit(2)

    if args.mix_ceiling:
        mix_ceiling()
        return

    import numpy as np
    import torch

    if args.io_sweep:
        io_sweep(args)
        return

    from synth import WORKLOADS, draw

    w = WORKLOADS[args.workload]
    inp = draw(w, args.workload)
    dev = torch.device("cuda:0")
    if w.decode:
        decode_main(args, w, inp, dev)
        return
    if args.timeline:
        timeline(args, w, inp, dev)
        return
    rec = measure(args, args.workload, w, inp, dev, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        per_b = rec.pop("_per_b")
        rec["cpu_baseline"] = cpu_baseline(inp, per_b, args.cpu_seconds)
    rec.pop("_per_b", None)
    del inp
    if args.workload == 2 and not args.no_w3_record:
        rec["w3_record"] = w3_record(args, dev)
    print(json.dumps(rec), flush=True)


TIMELINE_WORDS = 65536 * 16  # FA_TIMELINE_WORKGROUPS x FA_TIMELINE_SLOTS (include/fa_timeline.h)


def timeline_stats(rows):
    """Summary of one kernel launch's stamps (rows of workgroups that ran;
    layout in include/fa_timeline.h). Times in microseconds."""
    import numpy as np

    us = 0.01  # the real-time counter runs at 100 MHz
    t0 = rows[:, 0].min()
    start, end = (rows[:, 0] - t0) * us, (rows[:, 10] - t0) * us
    span = float(end.max())
    xcc = (rows[:, 1] >> 32) & 0xF
    loop = np.zeros(len(rows))
    tiles = np.zeros(len(rows))
    for r in range(2):
        ran = rows[:, 2 + 4 * r] > 0
        loop += np.where(ran, (rows[:, 4 + 4 * r] - rows[:, 3 + 4 * r]) * us, 0.0)
        tiles += np.where(ran, rows[:, 5 + 4 * r] & 0xFFFF, 0)
    grid = np.linspace(0.0, span, 401)
    conc = np.array([((start <= t) & (end > t)).sum() for t in grid])
    slots = int(conc.max())
    busy = float((end - start).sum())
    per_xcc_end = [float(end[xcc == x].max()) for x in range(8) if (xcc == x).any()]
    per_xcc_rate = [float(loop[xcc == x].sum() / tiles[xcc == x].sum())
                    for x in range(8) if tiles[xcc == x].sum() > 0]
    return {
        "workgroups": int(len(rows)),
        "span_us": round(span, 1),
        "resident_slots": slots,
        "slot_occupancy": round(busy / (slots * span), 3),
        "share_outside_tile_loop": round(1.0 - float(loop.sum()) / busy, 3),
        "us_per_workgroup_tile": round(float(loop.sum() / tiles.sum()), 3),
        "xcd_us_per_tile_min_max": [round(min(per_xcc_rate), 3), round(max(per_xcc_rate), 3)],
        "xcd_end_us_min_max": [round(min(per_xcc_end), 1), round(max(per_xcc_end), 1)],
        "last_start_us": round(float(start.max()), 1),
    }


def timeline(args, w, inp, dev):
    """Time the workload with the release library, then with
    libfa_timeline.so, and print one JSON line per stamped kernel with the
    last launch's timeline summary and both libraries' kernel times (the
    stamps perturb the kernels slightly; the release time is the reference)."""
    import ctypes

    import numpy as np

    from exact_io_aware_29_amd import _abi

    path = os.path.join(ROOT, "exact_io_aware_29_amd", "libfa_timeline.so")
    release = measure(args, args.workload, w, inp, dev, args.steps, args.warmup)
    raw = ctypes.CDLL(path)
    raw.fa_timeline_fwd_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    raw.fa_timeline_bwd_read.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t]
    saved = _abi.load()
    _abi._lib = _abi.load_variant(path)
    try:
        for fn in (raw.fa_timeline_fwd_clear, raw.fa_timeline_bwd_clear):
            if fn() != 0:
                raise RuntimeError("clearing the timeline arrays failed")
        stamped = measure(args, args.workload, w, inp, dev, args.steps, args.warmup)
    finally:
        _abi._lib = saved
    for name, read in (("fwd", lambda b: raw.fa_timeline_fwd_read(b.ctypes.data, b.size)),
                       ("bwd_dq", lambda b: raw.fa_timeline_bwd_read(0, b.ctypes.data, b.size)),
                       ("bwd_dkdv", lambda b: raw.fa_timeline_bwd_read(1, b.ctypes.data, b.size))):
        buf = np.zeros(TIMELINE_WORDS, dtype=np.uint64)
        if read(buf) != 0:
            raise RuntimeError(f"reading the {name} timeline failed")
        rows = buf.reshape(-1, 16).astype(np.int64)
        rows = rows[(rows[:, 0] > 0) & (rows[:, 10] > 0)]
        if len(rows) == 0:
            continue  # not a 16x16x32 kernel at this shape
        rec = {"timeline": name, "workload": release["config"]["workload"],
               "ms_release": release["kernels"][name]["ms"],
               "ms_stamped": stamped["kernels"][name]["ms"]}
        rec.update(timeline_stats(rows))
        print(json.dumps(rec), flush=True)


# Targets of the causal key-padded B8 H16 N4096 d128 configuration: the
# forward at >= 50 % and forward + backward at >= 35 % of the bf16 dense
# matrix-core peak.
W3_TARGET_PCT = {"fwd": 50.0, "fwd_bwd": 35.0}


def w3_record(args, dev):
    """The causal, key-padded B8 H16 N4096 d128 bf16 workload (workload 3),
    measured in the same run as the headline line: forward and
    forward + backward time, TFLOP/s and % of the bf16 peak, each kernel's
    time and roofline fraction, and whether the targets are met."""
    from synth import WORKLOADS, draw

    w = WORKLOADS[3]
    inp = draw(w, 3)
    r = measure(args, 3, w, inp, dev, args.w3_steps, args.w3_warmup)
    del inp
    k = r["kernels"]
    fwd_ms = k["fwd"]["ms"]
    fb_ms = sum(v["ms"] for v in k.values())
    fwd_pct = 100 * r["fwd_tflops"] / k["fwd"]["peak"]
    fb_tf = r["algorithmic_flop"]["fwd_bwd"] / (fb_ms * 1e-3) / 1e12
    fb_pct = 100 * fb_tf / k["fwd"]["peak"]
    return {
        "workload": r["config"]["workload"],
        "steps": args.w3_steps, "warmup": args.w3_warmup,
        "fwd_ms": round(fwd_ms, 4),
        "fwd_tflops": r["fwd_tflops"],
        "pct_of_peak_fwd": round(fwd_pct, 2),
        "fwd_bwd_ms": round(fb_ms, 4),
        "fwd_bwd_tflops": round(fb_tf, 1),
        "pct_of_peak_fwd_bwd": round(fb_pct, 2),
        "ms_per_step_wall": r["ms_per_step"],
        "kernels": {n: {"ms": v["ms"], "achieved": v["achieved"], "frac": v["frac"]}
                    for n, v in k.items()},
        "dominant_kernel": r["roofline"]["kernel"],
        "dominant_frac": r["roofline"]["frac"],
        "target_pct": W3_TARGET_PCT,
        "target_met": {"fwd": fwd_pct >= W3_TARGET_PCT["fwd"],
                       "fwd_bwd": fb_pct >= W3_TARGET_PCT["fwd_bwd"]},
    }


def measure(args, workload_id, w, inp, dev, steps, warmup):
    """Time `steps` steps of one workload (after `warmup` untimed ones) and
    return the bench record without the CPU baseline."""
    import numpy as np
    import torch

    import exact_io_aware_29_amd as fa
    from exact_io_aware_29_amd import accounting as acc

    def t(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(dev)
        if w.dtype == "fp8":
            return torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).to(dev)
        return torch.from_numpy(a).to(dev)

    q, k, v = t(inp.q), t(inp.k), t(inp.v)
    do = t(inp.do) if w.backward else None
    if args.fill != "random" and w.dtype != "fp8":
        for x in (q, k, v) + ((do,) if do is not None else ()):
            x.fill_(0.0 if args.fill == "zeros" else 0.5)
    sl = None if inp.seqlens is None else torch.from_numpy(inp.seqlens).to(dev)
    bm = None if inp.block_mask is None else torch.from_numpy(inp.block_mask).to(dev)
    kw = dict(scale=inp.scale, causal=w.causal, seqlens_k=sl, block_mask=bm, window=w.window)
    if w.dropout is not None:
        kw.update(dropout_p=w.dropout[0], dropout_seed=w.dropout[1], dropout_offset=w.dropout[2])
    if w.dtype == "fp8":
        kw.update(descale=inp.descale)
    o = torch.empty(q.shape, dtype=torch.bfloat16 if w.dtype == "fp8" else q.dtype, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    if w.backward:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        p = fa.make_params(batch=w.batch, heads_q=w.heads_q, heads_kv=w.heads_kv,
                           seqlen=w.seqlen, head_dim=w.head_dim)
        ws = torch.empty(fa.fa_bwd_workspace_size(p) // 4 + 4, dtype=torch.float32, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_fwd(q, k, v, out=o, lse=lse, **kw)
        if ev is not None:
            ev[1].record()
        if w.backward:
            fa.fa_bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws,
                      stage_events=None if ev is None else ev[2:5], **kw)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for ev in events:
        for e in ev:
            e.record()  # create the events outside the timed region
    torch.cuda.synchronize()

    scratch = (torch.empty(args.flush_mib << 18, dtype=torch.float32, device=dev)
               if args.flush_mib else None)
    t0 = time.perf_counter()
    for i in range(steps):
        if scratch is not None:
            scratch.fill_(float(i))  # evicts L2 and MALL between steps
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    copy_calibration(args, dev)

    def times(a, b):
        return np.array([events[i][a].elapsed_time(events[i][b]) for i in range(steps)])

    spans = {"fwd": (0, 1)}
    if w.backward:
        spans.update(bwd_dq=(2, 3), bwd_dkdv=(3, 4))
    kern_t = {k: times(*v) for k, v in spans.items()}
    kern_ms = {k: float(t.mean()) for k, t in kern_t.items()}

    per_b = [int(acc.allowed_pairs_per_row(
        w.seqlen, causal=w.causal, seqlen_k=None if inp.seqlens is None else int(inp.seqlens[b]),
        block_mask=inp.block_mask, window=w.window).sum()) for b in range(w.batch)]
    pairs = sum(per_b) * w.heads_q
    fl = acc.flops(pairs, w.head_dim)
    ms_step = wall / steps * 1e3
    if scratch is not None:  # the scratch writes are not part of a step
        ms_step = sum(kern_ms.values())
    step_flop = fl["fwd_bwd"] if w.backward else fl["fwd"]
    value = step_flop / (ms_step * 1e-3) / 1e12
    peak = {"bf16": acc.MFMA_BF16_PEAK_TFLOPS, "fp8": acc.MFMA_FP8_PEAK_TFLOPS}.get(
        w.dtype, acc.MFMA_FP32_PEAK_TFLOPS)

    kernels = {}
    for name, ms in kern_ms.items():
        ach = fl[name] / (ms * 1e-3) / 1e12
        kernels[name] = {"ms": round(ms, 4), "ms_median": round(float(np.median(kern_t[name])), 4),
                         "ms_min": round(float(kern_t[name].min()), 4),
                         "bound": "mfma", "achieved": round(ach, 1),
                         "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4)}
    # Work the tile structure executes: every visited 128 x 128 tile counted
    # in full (the algorithmic count above takes only the allowed pairs).
    tiles = acc.visited_tiles(w.batch, w.heads_q, w.seqlen, causal=w.causal,
                              seqlens=inp.seqlens, block_mask=inp.block_mask, window=w.window)
    tile_fl = acc.flops(tiles * 128 * 128, w.head_dim)
    dom = max(kern_ms, key=kern_ms.get)
    dk_ = kernels[dom]
    roofline = {"kernel": dom, "bound": dk_["bound"], "achieved": dk_["achieved"],
                "peak": dk_["peak"], "unit": dk_["unit"], "frac": dk_["frac"],
                "traffic": recorded_traffic("fwd_fp8" if w.dtype == "fp8" and dom == "fwd"
                                            else dom, workload_id)}

    fwd_tf = fl["fwd"] / (kern_ms["fwd"] * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": ("synthetic (seeded N(0,1) inputs, encoded as e4m3 of x / descale)"
                 if w.dtype == "fp8" else
                 "synthetic (seeded N(0,1) inputs, rounded to bf16)" if args.fill == "random" else
                 f"synthetic, every input element {'0' if args.fill == 'zeros' else '0.5'} "
                 "(power analysis, not a benchmark value)"),
        "config": {"workload": w.describe(), "batch": w.batch, "heads_q": w.heads_q,
                   "heads_kv": w.heads_kv, "seqlen": w.seqlen, "head_dim": w.head_dim,
                   "causal": w.causal, "pass": "fwd+bwd" if w.backward else "fwd",
                   "dropout_p": 0.0 if w.dropout is None else w.dropout[0]},
        "pct_of_peak_fwd_bwd": round(100 * value / peak, 2),
        "fwd_tflops": round(fwd_tf, 2),
        "pct_of_peak_fwd": round(100 * fwd_tf / peak, 2),
        "algorithmic_flop": {"fwd": fl["fwd"], "fwd_bwd": fl["fwd_bwd"], "pairs": pairs},
        "tile_flop": {"fwd": tile_fl["fwd"], "fwd_bwd": tile_fl["fwd_bwd"], "tiles_128": tiles},
        "device": device_info(),
        "kernels": kernels,
        "roofline": roofline,
    }
    if scratch is not None:
        rec["flush_mib"] = args.flush_mib
        rec["timing"] = "sum of kernel event times; scratch written between steps"
    rec["_per_b"] = per_b
    del q, k, v, do, o, lse
    if w.backward:
        del dq, dk, dv, ws
    return rec


if __name__ == "__main__":
    main()
