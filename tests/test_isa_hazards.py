"""Wait-state hazards around the hand-issued global->LDS direct loads (CPU only).

The GEMM kernels issue `global_load_lds_dwordx*` as inline asm so that the
compiler's `lgkmcnt` waits on fragment reads stay exact.  The compiler's
hazard recognizer does not look inside an asm statement, so the wait states
the gfx9-family ISA requires before such a load are the asm's own business:

* a VALU instruction that writes an SGPR needs 5 wait states before a
  vector-memory instruction reads that SGPR (the load's `m0`, or its `saddr`
  base pair);
* a scalar write of `m0` needs 1 wait state before an LDS-DMA load reads it.

A stale `m0` or base sends the load to the wrong LDS row or the wrong global
address.  This test compiles the kernel sources to gfx950 assembly and walks
back from every direct load through straight-line code to the last writer of
each SGPR it reads, counting wait states (`s_nop N` counts N + 1, every other
instruction 1).  A load whose writer is not found before a label or branch
fails the test too: the rule has to be visible in the block itself.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import combine_top_softmax_amd.build as B

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["ffn.hip", "bwd.hip", "mx.hip", "route.hip", "rows.hip"]
# sources whose kernels issue the hand-written direct loads
DMA_SOURCES = ["ffn.hip", "bwd.hip", "mx.hip"]

_SREG = re.compile(r"^s\[(\d+):(\d+)\]$|^s(\d+)$|^(m0|vcc|vcc_lo|vcc_hi|exec)$")


def sgprs(op: str) -> set[str]:
    """SGPR names an assembly operand names (`s[4:5]` -> {s4, s5})."""
    m = _SREG.match(op.strip())
    if not m:
        return set()
    if m.group(1):
        return {f"s{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    return {f"s{m.group(3)}"} if m.group(3) else {m.group(4)}


def operands(line: str) -> list[str]:
    parts = line.split(None, 1)
    if len(parts) < 2:
        return []
    # drop modifiers such as "offset:16" that follow the last comma-free operand
    return [p.strip().split()[0] for p in parts[1].split(",") if p.strip()]


def direct_load_hazards(asm: str) -> tuple[int, list[str]]:
    """(number of direct loads, list of violations) for one assembly listing."""
    lines = [ln.split(";")[0].strip() for ln in asm.splitlines()]
    n, bad = 0, []
    for i, ln in enumerate(lines):
        if not ln.startswith(("global_load_lds", "buffer_load_lds")) and not (
                ln.startswith("buffer_load") and " lds" in ln):
            continue
        n += 1
        ops = operands(ln)
        need = {"m0"}
        if ln.startswith("global_load_lds") and len(ops) > 1 and ops[1] != "off":
            need |= sgprs(ops[1])
        ws, j, issues = 0, i - 1, []
        while need:
            if j < 0:
                issues.append(f"no writer of {sorted(need)} found")
                break
            t = lines[j]
            j -= 1
            if t.endswith(":") or t.startswith(("s_branch", "s_cbranch", "s_setpc", "s_swappc")):
                issues.append(f"writer of {sorted(need)} not in the block")
                break
            if not t or t.startswith("."):   # directives
                continue
            mnem = t.split()[0]
            if mnem == "s_nop":
                ws += int(t.split()[1], 0) + 1
                continue
            tops = operands(t)
            if mnem.startswith("v_"):
                # conservative: a VALU naming the register anywhere may write it
                # (carry-outs and readfirstlane results are SGPR operands)
                hit = set().union(*(sgprs(o) for o in tops)) & need if tops else set()
                if hit and ws < 5:
                    issues.append(f"{mnem} writes {sorted(hit)} {ws} wait states before "
                                  f"(5 needed)")
                need -= hit
            elif mnem.startswith("s_") and tops:
                hit = sgprs(tops[0]) & need
                if hit and "m0" in hit and ws < 1:
                    issues.append(f"{mnem} writes m0 right before")
                need -= hit
            ws += 1
        if issues:
            bad.append(f"line {i + 1}: {ln}: " + "; ".join(issues))
    return n, bad


def _compile(src: str, out_dir: str) -> str:
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    out = os.path.join(out_dir, src + ".s")
    cmd = [HIPCC, *flags, "-S", "--cuda-device-only",
           "-I", os.path.join(B.ROOT, "include"), "-I", os.path.join(B.PKG, "csrc"),
           os.path.join(B.PKG, "csrc", src), "-o", out]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc -S {src} failed:\n{proc.stderr[-2000:]}")
    return open(out).read()


@pytest.fixture(scope="module")
def listings():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(len(SOURCES)) as ex:
            return dict(zip(SOURCES, ex.map(lambda s: _compile(s, d), SOURCES)))


@pytest.mark.parametrize("src", DMA_SOURCES)
def test_direct_loads_respect_wait_states(listings, src):
    n, bad = direct_load_hazards(listings[src])
    assert n > 0, f"{src}: no direct loads found (listing format changed?)"
    assert not bad, f"{src}: {len(bad)} of {n} direct loads violate wait states:\n" + \
        "\n".join(bad[:10])


def test_checker_flags_a_valu_written_base():
    # a base pair written by readfirstlane one wait state before the load
    asm = "\n".join([
        "s_mov_b32 m0, s31",
        "v_readfirstlane_b32 s5, v71",
        "v_readfirstlane_b32 s4, v70",
        "s_nop 0",
        "global_load_lds_dwordx4 v72, s[4:5]",
    ])
    n, bad = direct_load_hazards(asm)
    assert n == 1 and len(bad) == 1 and "v_readfirstlane_b32" in bad[0]
    # the same with the 5 wait states the ISA asks for, and the VGPR-address form
    ok = asm.replace("s_nop 0", "s_nop 4")
    assert direct_load_hazards(ok) == (1, [])
    vform = "s_mov_b32 m0, s2\ns_nop 0\nglobal_load_lds_dwordx4 v[2:3], off"
    assert direct_load_hazards(vform) == (1, [])
    # m0 written by the instruction right before the load
    assert len(direct_load_hazards("s_mov_b32 m0, s2\nglobal_load_lds_dwordx4 v[2:3], off")[1]) == 1
    # writer hidden behind a label
    assert len(direct_load_hazards("s_mov_b32 m0, s2\n.LBB0_1:\ns_nop 0\n"
                                   "global_load_lds_dwordx4 v[2:3], off")[1]) == 1


def kernel_resources(asm: str) -> dict:
    """Per kernel of a listing's metadata: (private segment bytes, VGPR spills)."""
    names = re.findall(r"^\s+\.name:\s+(\S+)", asm, flags=re.M)
    priv = re.findall(r"^\s+\.private_segment_fixed_size:\s+(\d+)", asm, flags=re.M)
    spill = re.findall(r"^\s+\.vgpr_spill_count:\s+(\d+)", asm, flags=re.M)
    assert len(names) == len(priv) == len(spill) and names, "kernel metadata not found"
    return {n: (int(p), int(v)) for n, p, v in zip(names, priv, spill)}


@pytest.mark.parametrize("src", SOURCES)
def test_no_kernel_spills_to_scratch(listings, src):
    """No kernel keeps registers in scratch memory. The GEMMs' hand-written
    waits count only their own direct loads; compiler-made scratch loads and
    stores would be vector-memory traffic outside that bookkeeping (and a
    spilled main loop is slow): a kernel that needs more registers than a
    wave has must be restructured, not left to spill."""
    res = kernel_resources(listings[src])
    bad = {k: v for k, v in res.items() if v != (0, 0)}
    assert not bad, f"{src}: kernels with scratch use (bytes, VGPR spills): {bad}"
