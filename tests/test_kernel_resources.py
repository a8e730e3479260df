"""Compile-time resource check of every gfx950 kernel (no GPU needed).

Each HIP source is compiled to device assembly with the library's own
flags; the code-object metadata then gives every kernel instance's VGPR
count, spill count and static LDS. The design depends on these numbers, so
they are pinned here:

* no kernel spills VGPRs, except the dK/dV instance with dropout at d=128,
  whose few spilled values are stored once before the key-block loop and
  reloaded once per key block (never inside the step loop);
* every bf16, FP8 and decode kernel fits two waves per SIMD (at most 256
  VGPRs), and the bf16 forward at d=64 fits four (at most 128), which is
  what makes it fast; the fp32 reference-precision forward (a parity path)
  may take the whole 512;
* static LDS of the resident workgroups that give two waves per SIMD fits
  the CU's 160 KiB: two workgroups of 256 threads, or one of 512 (the
  eight-wave dQ and dK/dV kernels);
* scratch memory appears only in the documented VGPR-spilling instances;
* scalar-register spills (to vector-register lanes, not memory) of the
  instances the timed workloads run stay within the counts measured when
  their speed was last checked. Re-reading the kernel arguments per block
  cut the causal-pair dK/dV instance's 47 to 24 but made it 3-5% slower, so
  these counts are a regression guard, not a target.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from exact_io_aware_29_amd import build as B

HIP_SOURCES = [s for s in B.SOURCES
               if s.endswith(".hip") and "__global__" in open(os.path.join(B.CSRC, s)).read()]
needs_hipcc = pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC),
                                 reason="hipcc not available")

# (kernel-name pattern, maximum VGPR spills) for the documented exceptions:
# the d=128 dK/dV kernel with dropout, and one combination no timed workload
# uses, at the 256-register limit: causal pairing with a block mask at d=128.
SPILL_ALLOWED = [(re.compile(r"bwd_dkdv_kernelILi128ELb1E"), 12),
                 (re.compile(r"bwd_dkdv_kernelILi128ELb0ELi2ELb1E"), 4)]


def _kernels(src: str):
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "k.s")
        cmd = [B.HIPCC, *B.FLAGS, *B.EXTRA.get(src, []), "-x", "hip", *B.KERNEL_FLAGS,
               "--offload-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        text = open(out).read()
    ks = []
    for block in re.split(r"\n\s+- \.agpr_count:", text)[1:]:
        def field(name):
            m = re.search(rf"\.{name}:\s+(\S+)", block)
            return m.group(1) if m else None
        ks.append({"name": field("name"), "vgpr": int(field("vgpr_count")),
                   "spill": int(field("vgpr_spill_count")),
                   "sspill": int(field("sgpr_spill_count")),
                   "scratch": int(field("private_segment_fixed_size")),
                   "lds": int(field("group_segment_fixed_size")),
                   "threads": int(field("max_flat_workgroup_size"))})
    assert ks, f"no kernel metadata found for {src}"
    return ks


@pytest.fixture(scope="module")
def kernels():
    import concurrent.futures
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(HIP_SOURCES)) as ex:
        return {s: k for s, k in zip(HIP_SOURCES, ex.map(_kernels, HIP_SOURCES))}


@needs_hipcc
def test_every_source_has_kernels(kernels):
    names = [k["name"] for ks in kernels.values() for k in ks]
    for stem in ("fwd_kernel_bf16", "fwd_kernel_m16", "fwd_kernel_fp8", "bwd_dkdv_kernel",
                 "bwd_dkdv_kernel_m16", "bwd_dq_kernel", "bwd_dq_kernel_m16",
                 "decode_split_kernel", "decode_combine_kernel"):
        assert any(stem in n for n in names), stem


@needs_hipcc
def test_no_unexpected_spills(kernels):
    for src, ks in kernels.items():
        for k in ks:
            limit = next((lim for pat, lim in SPILL_ALLOWED if pat.search(k["name"])), 0)
            assert k["spill"] <= limit, f"{src}: {k['name']} spills {k['spill']} VGPRs"


# Scalar spills allowed in the instances the timed workloads run (W2-W6:
# the lean forward, dQ and dK/dV kernels), by mangled-name pattern.
SCALAR_SPILL_MAX = [
    (re.compile(r"fwd_kernel_m16ILi128ELi2E"), 0),                # W3 (causal pairs)
    (re.compile(r"fwd_kernel_m16ILi128ELi1E"), 6),                # W4, W6
    (re.compile(r"fwd_kernel_bf16ILi64ELb0ELi1ELb0E"), 0),        # W2
    (re.compile(r"bwd_dq_kernel_m16ILi64ELi1ELi4E"), 0),          # W2
    (re.compile(r"bwd_dq_kernel_m16ILi128ELi2ELi4E"), 4),         # W3
    (re.compile(r"bwd_dq_kernel_m16ILi128ELi2ELi8E"), 11),        # W4
    (re.compile(r"bwd_dq_kernel_m16ILi128ELi1ELi4E"), 0),         # W6
    (re.compile(r"bwd_dkdv_kernel_m16ILi128ELi2ELi8E"), 47),      # W3, W4
    (re.compile(r"bwd_dkdv_kernel_m16ILi128ELi1ELi8E"), 9),       # W6
    (re.compile(r"bwd_dkdv_kernelILi64ELb0ELi1ELb0E"), 0),        # W2
]


@needs_hipcc
def test_scratch_only_where_documented(kernels):
    for src, ks in kernels.items():
        for k in ks:
            if any(pat.search(k["name"]) for pat, _ in SPILL_ALLOWED):
                continue
            assert k["scratch"] == 0, f"{src}: {k['name']} uses {k['scratch']} bytes of scratch"


@needs_hipcc
def test_scalar_spills_of_timed_instances(kernels):
    names = [k["name"] for ks in kernels.values() for k in ks]
    for pat, limit in SCALAR_SPILL_MAX:
        hits = [k for ks in kernels.values() for k in ks if pat.search(k["name"])]
        assert hits, f"no kernel matches {pat.pattern} among {len(names)}"
        for k in hits:
            assert k["sspill"] <= limit, f"{k['name']} spills {k['sspill']} SGPRs (limit {limit})"


@needs_hipcc
def test_occupancy_budgets(kernels):
    for src, ks in kernels.items():
        for k in ks:
            budget = 512 if "fwd_kernelIf" in k["name"] else 256
            assert k["vgpr"] <= budget, f"{k['name']}: {k['vgpr']} VGPRs"
            assert k["threads"] in (64, 256, 512), f"{k['name']}: {k['threads']} threads"
            # Two waves per SIMD: two workgroups of 256 threads or one of 512
            # (the 64-thread decode combine uses no LDS).
            resident = 1 if k["threads"] == 512 else 2
            assert resident * k["lds"] <= 160 * 1024, f"{k['name']}: {k['lds']} bytes of LDS"
            if "fwd_kernel_bf16ILi64ELb0ELi1E" in k["name"]:
                assert k["vgpr"] <= 128, f"{k['name']}: {k['vgpr']} VGPRs (four waves need 128)"
