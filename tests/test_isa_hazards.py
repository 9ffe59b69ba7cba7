"""Static check of the attention kernel's gfx950 ISA for MFMA data hazards.

The attention kernel issues its MFMA instructions from inline assembly (so
that the accumulators stay resident in AGPRs), which hides them from the
compiler's hazard recognizer. Each asm statement therefore carries its own
wait states. This test compiles the kernel to assembly (CPU only, hipcc
cross-compiles for gfx950) and scans it in program order:

  * a VALU instruction that writes a VGPR which a following MFMA reads must
    be at least MIN_VALU_TO_MFMA wait states before that MFMA, unless a
    memory load overwrites the register in between (the MFMA then reads the
    load's data, which the memory counter waits cover);
  * an MFMA result in VGPRs must not be read by a VALU instruction within
    MIN_MFMA_TO_VALU wait states; an MFMA result in AGPRs must not be read by
    v_accvgpr_read within the same distance.

Wait states are counted as one per instruction plus N for s_nop N-1. The scan
follows the instruction order of the file (branches are not modelled); the
kernel's hazard-prone sequences are straight-line.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "kv_cache_compression_mla_amd", "csrc", "attn_mfma.hip")
MIN_VALU_TO_MFMA = 5
MIN_MFMA_TO_VALU = 18


def _regs(tok):
    """Register numbers named by an operand like v5, v[4:7], a[0:15]."""
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return m.group(1), set(range(int(m.group(2)), int(m.group(3)) + 1))
    m = re.fullmatch(r"([va])(\d+)", tok)
    if m:
        return m.group(1), {int(m.group(2))}
    return None, set()


def _instructions(asm_text, kernel_prefix):
    lines = asm_text.splitlines()
    out, inside = [], False
    for ln in lines:
        s = ln.split(";")[0].strip()
        if s.startswith(kernel_prefix) and s.endswith(":"):
            inside = True
            continue
        if not inside:
            continue
        if s.startswith("s_endpgm"):
            break
        if not s or s.endswith(":") or s.startswith("."):
            continue
        out.append(s)
    return out


@pytest.fixture(scope="module")
def kernels():
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-S", "--cuda-device-only",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.dirname(SRC),
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    names = sorted(set(re.findall(r"^(_ZN\S*attn_mfma_kernel\S*):", r.stdout, re.M)))
    assert names, "no attention kernel found in the assembly"
    return {n: _instructions(r.stdout, n) for n in names}


def _wait_states(ins):
    m = re.match(r"s_nop\s+(\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def test_valu_writes_before_mfma_reads(kernels):
    for name, insts in kernels.items():
        for i, ins in enumerate(insts):
            if not ins.startswith("v_mfma"):
                continue
            ops = [o.strip() for o in ins.split(None, 1)[1].split(",")]
            srcs = set()
            for o in ops[1:3]:
                f, regs = _regs(o)
                if f == "v":
                    srcs |= regs
            dist = 0
            for j in range(i - 1, max(-1, i - 40), -1):
                prev = insts[j]
                dst = prev.split(None, 1)[1].split(",")[0].strip() if " " in prev else ""
                f, regs = _regs(dst)
                if prev.startswith(("ds_read", "global_load", "buffer_load")) and f == "v":
                    # a later load overwrites these registers: their last
                    # writer is the load, covered by the memory counters
                    srcs -= regs
                elif prev.startswith("v_") and not prev.startswith("v_mfma") and \
                        not prev.startswith("v_accvgpr_write"):
                    if f == "v" and regs & srcs:
                        assert dist >= MIN_VALU_TO_MFMA, (name, i, prev, ins, dist)
                        break
                dist += _wait_states(prev)
                if dist >= MIN_VALU_TO_MFMA or not srcs:
                    break


def test_mfma_results_not_read_early(kernels):
    for name, insts in kernels.items():
        for i, ins in enumerate(insts):
            if not ins.startswith("v_mfma"):
                continue
            dst = ins.split(None, 1)[1].split(",")[0].strip()
            f, regs = _regs(dst)
            dist = 0
            for j in range(i + 1, min(len(insts), i + 60)):
                nxt = insts[j]
                if nxt.startswith("v_mfma"):
                    # a following MFMA that reads or rewrites the block is the
                    # accumulation chain; the hardware orders those
                    dist += 1
                    continue
                if nxt.startswith("v_") and " " in nxt:
                    srcs = [o.strip() for o in nxt.split(None, 1)[1].split(",")[1:]]
                    for o in srcs:
                        g, rr = _regs(o)
                        if g == f and rr & regs:
                            assert dist >= MIN_MFMA_TO_VALU, (name, i, ins, nxt, dist)
                dist += _wait_states(nxt)
                if dist >= MIN_MFMA_TO_VALU:
                    break
