"""CPU check of the GEMM kernels' generated gfx950 code.

The MFMA GEMM (`k_gemm`) issues v_mfma_f32_16x16x32_bf16 from inline asm with
its accumulators pinned to AGPRs, so the compiler's hazard recogniser does not
see the MFMA's write-back latency. The kernel waits it out itself (three
`s_nop 15`, 48 wait states) before anything reads an accumulator. A compiler
transformation that copies or reads accumulators in between (e.g. a peeled
loop iteration whose accumulators live in other AGPRs) gives wrong results
without any fault, so every instantiation is checked: after each MFMA, no
v_accvgpr_read / v_accvgpr_mov of its result registers may come before the
drain.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "weight_quantization_aware_amd")


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


def _device_asm(src: str) -> str:
    from weight_quantization_aware_amd import build
    out = os.path.join(tempfile.mkdtemp(), "k.s")
    cmd = [_hipcc(), *build.FLAGS, "--cuda-device-only", "-S", os.path.join(PKG, "csrc", src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def _agprs(op: str):
    """The AGPR numbers an operand names (a5, a[4:7])."""
    m = re.fullmatch(r"a(\d+)", op) or re.fullmatch(r"a\[(\d+):(\d+)\]", op)
    if not m:
        return set()
    lo = int(m.group(1))
    hi = int(m.group(2)) if m.lastindex == 2 else lo
    return set(range(lo, hi + 1))


def accumulator_hazards(asm: str):
    """{kernel: count} of reads or moves of an MFMA's result AGPRs between the MFMA and the drain.

    The kernel text is walked in order; the result registers of every MFMA
    since the last drain (three `s_nop 15`) are pending, and a v_accvgpr_read
    or v_accvgpr_mov whose source is pending counts. (Moves of other AGPRs,
    e.g. zeros copied into accumulators before their first MFMA, do not.)
    """
    found = {}
    for m in re.finditer(r"^(_Z[^:\s]+):", asm, re.M):
        name = m.group(1)
        end = asm.index(".Lfunc_end", m.end())
        pending, nops, cnt = set(), 0, 0
        for line in asm[m.end():end].split("\n"):
            t = line.split(";")[0].strip()
            ops = [o.strip() for o in t.split(None, 1)[1].split(",")] if " " in t else []
            if t.startswith("v_mfma"):
                pending |= _agprs(ops[0])
                nops = 0
            elif pending and t.startswith("s_nop 15"):
                nops += 1
                if nops == 3:
                    pending, nops = set(), 0
            elif pending and (t.startswith("v_accvgpr_read") or t.startswith("v_accvgpr_mov")):
                if _agprs(ops[1]) & pending:
                    cnt += 1
        if cnt:
            found[name] = cnt
    return found


def test_scanner_flags_a_copy_before_the_drain():
    asm = """_Zk:
\tv_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]
\tv_accvgpr_mov_b32 a4, a0
\ts_nop 15
\ts_nop 15
\ts_nop 15
\tv_accvgpr_read_b32 v8, a0
.Lfunc_end0:
_Zok:
\tv_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]
\ts_nop 15
\ts_nop 15
\ts_nop 15
\tv_accvgpr_read_b32 v8, a0
.Lfunc_end1:
_Zzero:
\tv_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]
\tv_accvgpr_mov_b32 a5, a24
\tv_accvgpr_read_b32 v9, a2 ; the MFMA's result
\ts_nop 15
.Lfunc_end2:
"""
    assert accumulator_hazards(asm) == {"_Zk": 1, "_Zzero": 1}


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_asm_mfma_gemms_wait_before_reading_accumulators():
    asm = _device_asm("qat_gemm.hip")
    kernels = re.findall(r"^(_ZN3qat6k_gemmI[^:\s]+):", asm, re.M)
    assert len(kernels) >= 20
    bad = {k: n for k, n in accumulator_hazards(asm).items() if k.startswith("_ZN3qat6k_gemmI")}
    assert not bad, bad
