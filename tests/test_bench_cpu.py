"""Host-side checks of bench.py that need no GPU: the one-GPU contract, the
CPU-baseline legs (fields, bounded time, the long-sequence row sample), the
kernel source hashes and the recorded-traffic parser."""
import os
import subprocess
import sys
import time

import numpy as np

import bench
from synth import Workload, draw, draw_case

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _check_baseline(rec, unit):
    assert rec["kind"] == "oracle" and rec["unit"] == unit
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert isinstance(rec["cpu"], str) and rec["sample"]
    assert isinstance(rec["blas"], str) and rec["blas"]


def test_cpu_baseline_fields_and_budget():
    inp = draw_case(2, 2, 1, 192, 64, "bf16", causal=True, seqlens=[150, 192], seed=3)
    per_b = [int(x) for x in (150 * 151 // 2 + 42 * 150, 192 * 193 // 2)]
    t0 = time.perf_counter()
    rec = bench.cpu_baseline(inp, per_b, 0.2)
    assert time.perf_counter() - t0 < 30
    _check_baseline(rec, "TFLOP/s")


def test_cpu_baseline_long_sequence_samples_rows():
    w = Workload("t", 1, 1, 1, 16384, 64, "bf16", butterfly=True)
    inp = draw(w, 5)
    t0 = time.perf_counter()
    rec = bench.cpu_baseline(inp, [1], 0.5)
    assert time.perf_counter() - t0 < 60
    _check_baseline(rec, "TFLOP/s")
    assert "rows of (batch 0, head 0)" in rec["sample"]


def test_decode_cpu_baseline_fields():
    w = Workload("t", 2, 4, 2, 512, 64, "bf16", pad_range=(100, 512), backward=False, decode=True)
    inp = draw(w, 7)
    rec = bench.decode_cpu_baseline(inp, 0.2)
    _check_baseline(rec, "GB/s")


def test_every_kernel_source_hashes():
    for k in bench.KERNEL_SOURCES:
        h = bench.source_hash(k)
        assert len(h) == 16 and int(h, 16) >= 0


def test_recorded_traffic_lines_parse():
    """Every committed traffic line names a known kernel and a byte count;
    recorded_traffic returns it only while the source hash still matches."""
    import re
    pat = re.compile(r"^traffic\s+(\S+)\s+bytes_per_launch=(\d+)\s+src=(\w+)", re.M)
    found = 0
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        m = re.match(r"hbm_traffic_w(\d+)\.md$", name)
        if not m:
            continue
        text = open(os.path.join(ROOT, "profiles", name)).read()
        for kernel, nbytes, src in pat.findall(text):
            assert kernel in bench.KERNEL_SOURCES, kernel
            got = bench.recorded_traffic(kernel, int(m.group(1)))
            assert got == (int(nbytes) if src == bench.source_hash(kernel) else None)
            found += 1
    assert found > 0


def test_mixbench_library_exports_its_entry_points():
    """The instruction-mix measurement library is built beside libfa.so and
    exports the grid query and the timing call (no GPU call made here)."""
    import ctypes

    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "exact_io_aware_29_amd", "libfa_mixbench.so")
    assert os.path.exists(path), "build first: python -m exact_io_aware_29_amd.build"
    lib = ctypes.CDLL(path)
    ne, nf, nl = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    rows, trs = (ctypes.c_int * 3)(), (ctypes.c_int * 3)()
    assert lib.fa_mixbench_grid(ctypes.byref(ne), ctypes.byref(nf), ctypes.byref(nl), rows, trs) == 0
    assert (ne.value, nf.value, nl.value) == (5, 6, 3)
    assert list(rows) == [0, 16, 24] and list(trs) == [0, 32, 32]
    ms = ctypes.c_float()
    # an index outside the grid or a bad count is refused before any HIP call
    assert lib.fa_mixbench(5, 0, 0, 1, 1, ctypes.byref(ms)) == -1
    assert lib.fa_mixbench(0, -1, 0, 1, 1, ctypes.byref(ms)) == -1
    assert lib.fa_mixbench(0, 0, 3, 1, 1, ctypes.byref(ms)) == -1
    assert lib.fa_mixbench(0, 0, 0, 0, 1, ctypes.byref(ms)) == -1


def test_timeline_library_exports_its_entry_points_and_release_does_not():
    """libfa_timeline.so (the stamped debug build) exports the four
    fa_timeline_* calls of include/fa_timeline.h; libfa.so exports none.
    Only symbol lookups here, no GPU call."""
    import ctypes

    pkg = os.path.join(ROOT, "exact_io_aware_29_amd")
    names = ("fa_timeline_fwd_read", "fa_timeline_fwd_clear", "fa_timeline_bwd_read",
             "fa_timeline_bwd_clear")
    tl = ctypes.CDLL(os.path.join(pkg, "libfa_timeline.so"))
    for n in names:
        assert hasattr(tl, n), n
    rel = ctypes.CDLL(os.path.join(pkg, "libfa.so"))
    for n in names:
        assert not hasattr(rel, n), n
    assert bench.TIMELINE_WORDS == 65536 * 16


def _timeline_rows():
    """Four workgroups on two XCDs, two per XCD, in one slot each, stamped in
    100 MHz ticks: entry, first tile ready, loop end and exit of one block
    (word 5 = tiles), XCC id in word 1's high half."""
    rows = np.zeros((4, 16), dtype=np.int64)
    # (xcc, entry, block start, first tile, loop end, tiles, exit) in ticks
    spec = [(0, 100, 110, 200, 1200, 10, 1300),
            (0, 1300, 1310, 1400, 2400, 10, 2500),
            (1, 100, 110, 200, 1700, 10, 1800),
            (1, 1800, 1810, 1900, 3400, 10, 3500)]
    for i, (x, e, s, f, l, t, q) in enumerate(spec):
        rows[i, [0, 2, 3, 4, 5, 10]] = [e, s, f, l, t, q]
        rows[i, 1] = (x << 32) | 7
    return rows


def test_timeline_stats_on_a_hand_made_launch():
    st = bench.timeline_stats(_timeline_rows())
    # span: first entry at 100 ticks, last exit at 3500 ticks -> 34 us
    assert st["span_us"] == 34.0
    assert st["workgroups"] == 4 and st["resident_slots"] == 2
    # busy: 12 + 12 + 17 + 17 = 58 us of 2 x 34 us
    assert st["slot_occupancy"] == round(58 / 68, 3)
    # loop time: 10 + 10 + 15 + 15 = 50 us of 58 busy
    assert st["share_outside_tile_loop"] == round(1 - 50 / 58, 3)
    assert st["us_per_workgroup_tile"] == round(50 / 40, 3)
    # XCD 0 runs 1.0 us per tile and ends at 24 us; XCD 1 1.5 us, 34 us
    assert st["xcd_us_per_tile_min_max"] == [1.0, 1.5]
    assert st["xcd_end_us_min_max"] == [24.0, 34.0]
    assert st["last_start_us"] == 17.0
