"""The wait states after tied-accumulator MFMAs, checked in the gfx950
assembly the compiler emits for the kernels (CPU only: hipcc cross-compiles).

Tiles whose accumulators fill the accumulation-register file issue their
MFMAs as inline assembly with the accumulator as one read-write operand, so
the compiler does not know they are MFMAs and pads no hazard after them. The
engine pads by hand: each pair of K steps ends with s_nop 7; s_nop 7; s_nop 3
(20 wait states, at least the 19 an 8-pass XDL op needs before another
instruction may read or overwrite its result). This test is the tripwire for
edits or compiler changes that put an access too close: in every kernel with
inline-asm MFMAs, every non-MFMA instruction that touches an accumulation
register written by one of them must come at least 19 wait states after it,
counted along the code in program order (s_nop n counts n + 1, any other
instruction 1; code after an unconditional branch, up to the next label,
is not on that path). In the current code the loop exit also runs a dozen
scalar instructions, a wait and a barrier before the first accumulator
read, so the pad is a margin there rather than the only guard; the check is
that the distance holds, whatever provides it."""
import importlib.util
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

WAIT_STATES = 19
AREG = re.compile(r"\ba(\d+)\b|\ba\[(\d+):(\d+)\]")


def _aregs(text):
    regs = set()
    for m in AREG.finditer(text):
        if m.group(1) is not None:
            regs.add(int(m.group(1)))
        else:
            regs.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return regs


def check_tied_hazards(asm: str):
    """Returns {function: [tied MFMAs, accesses inside the window]} and the
    violations [(function, instruction, wait states)]."""
    stats, bad = {}, []
    fn, inasm, elapsed, dead = None, False, {}, False
    for ln in asm.split("\n"):
        m = re.match(r"^(_Z\S+):", ln)
        if m:
            fn, inasm, elapsed = m.group(1), False, {}
            continue
        if fn is None:
            continue
        if ln.startswith(".Lfunc_end"):
            fn = None
            continue
        if ";;#ASMSTART" in ln:
            inasm = True
            continue
        if ";;#ASMEND" in ln:
            inasm = False
            continue
        code = ln.split(";")[0].strip()
        if code.endswith(":"):
            dead = False      # a branch target: reached again
            continue
        if not code or code.startswith(".") or dead:
            continue
        op = code.split()[0]
        if op == "s_branch":
            dead = True       # nothing after it falls through from here
            continue
        if op == "s_nop":
            n = int(code.split()[1], 0) + 1
            elapsed = {r: w + n for r, w in elapsed.items() if w + n < WAIT_STATES}
            continue
        if op.startswith("v_mfma"):
            if inasm:
                st = stats.setdefault(fn, [0, 0])
                st[0] += 1
                dst = code[len(op):].split(",")[0]
                for r in _aregs(dst):
                    elapsed[r] = -1   # the increment below makes it 0
        else:
            touched = _aregs(code[len(op):]) & set(elapsed)
            if touched:
                stats.setdefault(fn, [0, 0])[1] += 1
                bad.append((fn, code, min(elapsed[r] for r in touched)))
        elapsed = {r: w + 1 for r, w in elapsed.items() if w + 1 < WAIT_STATES}
    return stats, bad


def _compile_asm(tmp):
    # the package's build script, loaded by path (no module-name lookup)
    spec = importlib.util.spec_from_file_location(
        "ocg_build", os.path.join(ROOT, "communication_overlapped_gemm_amd", "build.py"))
    B = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(B)
    out = os.path.join(tmp, "kernels.s")
    cmd = [B.hipcc(), *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, "kernels.hip"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        pytest.fail("hipcc -S failed:\n" + res.stderr[-2000:])
    with open(out) as f:
        return f.read()


def test_checker_flags_a_missing_pad():
    """The checker itself: an access 3 wait states after a tied MFMA is
    flagged; after the engine's 20-state pad it is not."""
    body = ("_Zk:\n\t;;#ASMSTART\n\tv_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]\n\t;;#ASMEND\n"
            "\ts_nop 2\n\tv_accvgpr_read_b32 v8, a2\n.Lfunc_end0:\n")
    _, bad = check_tied_hazards(body)
    assert len(bad) == 1 and bad[0][2] == 3
    padded = body.replace("\ts_nop 2\n", "\ts_nop 7\n\ts_nop 7\n\ts_nop 3\n")
    _, bad = check_tied_hazards(padded)
    assert bad == []


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc (ROCm)")
def test_tied_mfma_results_are_padded():
    with tempfile.TemporaryDirectory() as tmp:
        asm = _compile_asm(tmp)
    stats, bad = check_tied_hazards(asm)
    # the kernels that use tied accumulators: 256x256 AG-GEMM (whole tiles
    # and K halves), 256x256 GEMM-RS, 288x224 grouped GEMM
    tied = {f for f, (n, _) in stats.items() if n > 0}
    assert len(tied) >= 4, sorted(tied)
    assert not bad, "accumulators touched too soon after a tied MFMA:\n" + "\n".join(
        f"{f[:60]}: '{c}' after {w} wait states" for f, c, w in bad[:10])
