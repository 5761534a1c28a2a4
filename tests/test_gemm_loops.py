"""The expert GEMMs' main loops as the compiler emits them for gfx950 (no GPU
needed).

Each GEMM keeps two slabs of operand loads in flight through a 4-stage LDS
ring, ordered by its own vmcnt waits.  Three things the compiler can put in
the loop silently undo that, at no cost to correctness, so only the code
shows them:

* `s_waitcnt vmcnt(0)`: a wait for every load in flight.  The compiler
  inserts one before an LDS read it cannot tell apart from the LDS-DMA
  loads' destinations (the transposing reads, unless they go through a
  restrict pointer), and wherever its register tracking gives up;
* scalar loads: they complete out of order with LDS reads, so every wait
  for a fragment read becomes `lgkmcnt(0)`, which also waits for them;
* scratch accesses: a spill reload in the loop is a vector-memory load that
  its wait must see through all the slab loads issued before it.

The test compiles the GEMM sources to assembly and checks the innermost
loop of every GEMM kernel (the one that issues the MFMAs) for all three."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_free_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# the GEMM kernels are instantiated in these two sources
SOURCES = ["ffn.hip", "backward.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S"]

LABEL = re.compile(r"^(\.LBB\d+_\d+):")
BRANCH = re.compile(r"\bs_cbranch_\w+\s+(\.LBB\d+_\d+)")
KERNEL = re.compile(r"^(_ZN8moe_gemm11gemm_kernel\w+):")


def innermost_mfma_loops(body):
    """(start, end) line ranges of the loops (backward branches) that issue
    MFMAs and hold no other such loop."""
    labels = {}
    for i, line in enumerate(body):
        m = LABEL.match(line)
        if m:
            labels[m.group(1)] = i
    loops = []
    for i, line in enumerate(body):
        m = BRANCH.search(line)
        if m and m.group(1) in labels and labels[m.group(1)] < i:
            a = labels[m.group(1)]
            if any("v_mfma" in x for x in body[a:i]):
                loops.append((a, i))
    return [(a, b) for a, b in loops
            if not any((a2, b2) != (a, b) and a <= a2 and b2 <= b for a2, b2 in loops)]


def kernels(asm):
    lines = asm.splitlines()
    for i, line in enumerate(lines):
        m = KERNEL.match(line)
        if m:
            end = next(j for j in range(i, len(lines)) if "s_endpgm" in lines[j])
            yield m.group(1), lines[i:end]


def loop_findings(body, a, b):
    bad = []
    for line in body[a:b + 1]:
        ins = line.split(";")[0].strip()
        if "vmcnt(0)" in ins:
            bad.append(ins)
        elif ins.startswith(("s_load", "s_buffer_load", "scratch_")):
            bad.append(ins)
    return bad


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="ROCm toolchain not found")
def test_gemm_inner_loops_keep_their_loads_in_flight(tmp_path):
    def compile_one(src):
        out = str(tmp_path / (src + ".s"))
        r = subprocess.run([HIPCC, *FLAGS, os.path.join(CSRC, src), "-o", out], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        asms = list(ex.map(compile_one, SOURCES))
    checked, problems = 0, []
    for src, asm in zip(SOURCES, asms):
        for name, body in kernels(asm):
            loops = innermost_mfma_loops(body)
            assert loops, f"{src} {name}: no MFMA loop found"
            for a, b in loops:
                checked += 1
                bad = loop_findings(body, a, b)
                if bad:
                    problems.append(f"{src} {name} lines {a}-{b}: {sorted(set(bad))}")
    # every GEMM instantiation: 4 in the forward source, 10 in the backward one
    assert checked >= 14, checked
    assert not problems, "\n".join(problems)
    shutil.rmtree(tmp_path, ignore_errors=True)


def test_loop_finder_on_a_listing():
    """The parser on a hand-written listing: an outer loop around an inner
    MFMA loop, and a findings list that flags each kind of drain."""
    body = """k:
.LBB0_1:
\tv_add_u32 v1, v1, v2
.LBB0_2:
\ts_waitcnt vmcnt(8)
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]
\ts_cbranch_scc0 .LBB0_2
\ts_waitcnt vmcnt(0)
\ts_cbranch_scc0 .LBB0_1
\ts_endpgm""".splitlines()
    loops = innermost_mfma_loops(body)
    assert loops == [(3, 6)]
    assert loop_findings(body, *loops[0]) == []
    drained = body[:4] + ["\ts_waitcnt vmcnt(0)", "\ts_load_dwordx8 s[8:15], s[0:1], 0x0",
                          "\tscratch_load_dword v0, off, off"] + body[4:]
    (a, b), = innermost_mfma_loops(drained)
    assert loop_findings(drained, a, b) == ["s_waitcnt vmcnt(0)", "s_load_dwordx8 s[8:15], s[0:1], 0x0",
                                            "scratch_load_dword v0, off, off"]
