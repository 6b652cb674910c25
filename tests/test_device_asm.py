"""Checks on the gfx950 assembly of every kernel source (CPU only: hipcc cross-compiles).

* `m0` is written only by the direct global->LDS loads of fa_common.hpp, each
  followed by exactly one `s_nop 0` and then its load: an SALU write of m0
  needs one wait state before an LDS-DMA load consumes it, and the hazard
  recognizer does not look inside asm blocks (the inline assembly lists `m0`
  as clobbered, and no compiler-generated code may hold a value in it across
  those statements);
* no packed FP32 VALU instruction appears (the build turns the feature off);
* no kernel spills registers or uses scratch memory;
* the forward's workgroup shape matches the rows per workgroup that bench.py's
  I/O model assumes.
"""
import os
import re
import subprocess
import tempfile

import pytest

from exact_io_aware_61_amd import build as fab

SOURCES = [s for s in fab.SOURCES if s not in ("fa_api.hip", "fa_noalloc.hip")]   # kernels only


@pytest.fixture(scope="module")
def asm():
    try:
        hipcc = fab.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = {}
    with tempfile.TemporaryDirectory() as d:
        procs = []
        for src in SOURCES:
            path = os.path.join(d, src + ".s")
            cmd = [hipcc, *fab.DEVICE_FLAGS, "-I", fab.INCLUDE, "-I", fab.CSRC, "--cuda-device-only",
                   "-S", os.path.join(fab.CSRC, src), "-o", path]
            procs.append((src, path, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                      stderr=subprocess.PIPE, text=True)))
        for src, path, p in procs:
            _, err = p.communicate()
            assert p.returncode == 0, f"{src}: {err[-2000:]}"
            with open(path) as f:
                out[src] = f.read()
    return out


def _code_lines(text):
    for line in text.split("\n"):
        s = line.strip()
        if not s or s.startswith(";") or s.startswith(".") or s.endswith(":"):
            continue
        yield s


@pytest.mark.parametrize("src", SOURCES)
def test_m0_written_only_for_direct_loads(asm, src):
    lines = list(_code_lines(asm[src]))
    for i, s in enumerate(lines):
        if re.search(r"\bm0\b", s):
            assert s.startswith("s_mov_b32 m0,"), f"{src}: unexpected use of m0: {s}"
            assert i + 2 < len(lines) and lines[i + 1] == "s_nop 0", \
                f"{src}: m0 write not followed by a wait state: {s} / {lines[i + 1]}"
            assert lines[i + 2].startswith("global_load_lds_"), \
                f"{src}: m0 set without a direct load after it: {s} / {lines[i + 2]}"


@pytest.mark.parametrize("src", SOURCES)
def test_no_packed_fp32(asm, src):
    bad = [s for s in _code_lines(asm[src]) if re.match(r"v_pk_(add|mul|fma)_f32\b", s)]
    assert not bad, f"{src}: {bad[:3]}"


@pytest.mark.parametrize("src", SOURCES)
def test_no_spills_or_scratch(asm, src):
    text = asm[src]
    names = re.findall(r"^\s+\.name:\s+(\S+)", text, re.M)
    for key in ("vgpr_spill_count", "sgpr_spill_count", "private_segment_fixed_size"):
        vals = [int(v) for v in re.findall(rf"^\s+\.{key}:\s+(\d+)", text, re.M)]
        assert vals, f"{src}: no {key} in the kernel metadata"
        if key == "sgpr_spill_count":
            continue   # SGPR spills go to VGPR lanes, not memory
        assert all(v == 0 for v in vals), f"{src}: {key} {list(zip(names, vals))}"


def _kernel_entries(text):
    """(name, max_flat_workgroup_size) of every kernel in the code-object metadata."""
    out = []
    for chunk in re.split(r"\n\s+- \.agpr_count:", text)[1:]:
        name = re.search(r"^\s+\.name:\s+(\S+)", chunk, re.M)
        size = re.search(r"^\s+\.max_flat_workgroup_size:\s+(\d+)", chunk, re.M)
        if name and size:
            out.append((name.group(1), int(size.group(1))))
    return out


def test_forward_rows_per_workgroup_match_bench_model(asm):
    import bench
    seen = 0
    for name, threads in _kernel_entries(asm["fa_fwd.hip"]):
        m = re.search(r"fa_fwd_kernelILi(\d+)ELb([01])ELb([01])E", name)
        if not m:
            continue
        d, block = int(m.group(1)), m.group(3) == "1"
        rows = threads // 64 * 32   # every wave owns 32 query rows
        assert rows == bench.fwd_rows_per_workgroup(d, block), (name, threads)
        seen += 1
    assert seen == 8, seen   # d in {64, 128} x causal x block mask


def test_no_bit_cast_of_a_vector_element():
    """`__builtin_bit_cast(T, v[i])` on an element of an ext_vector_type vector compiles, with
    this hipcc, to a read of element 0 whatever i is (a kernel that summed four packed pairs
    this way read the first pair four times). The kernels copy such an element into a scalar
    before casting it; this keeps the construct out of the sources."""
    import re
    pat = re.compile(r"__builtin_bit_cast\(\s*[\w:]+\s*,\s*[\w.]+(\s*\[[^\]]+\])+\s*\)")
    csrc = fab.CSRC
    bad = []
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")):
            for n, line in enumerate(open(os.path.join(csrc, name)), 1):
                if pat.search(line):
                    bad.append(f"{name}:{n}: {line.strip()}")
    assert not bad, bad
    assert pat.search("x = __builtin_bit_cast(bf16x2, pku[k][h]);")      # the pattern works
    assert not pat.search("x = __builtin_bit_cast(bf16x8, v);")
