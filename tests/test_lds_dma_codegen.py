"""Code-generation guard for the direct global/buffer -> LDS loads of the
grouped GEMM, the attention kernel and the memory read.

Such a load writes lane i's bytes at M0 + 16 i, with M0 (the LDS address)
taken from a scalar register.  Issued under a lane mask, the compiler may
merge it with a neighbouring load across the branch and then compute M0 with
a v_readfirstlane of a value that differs between the lane groups (it did
so for the GEMM's leftover-block loads: NaN at 96-row tiles).  The kernels
therefore issue every such load with the full wave active, choosing between
loads with wave-uniform (scalar) branches only.  This test compiles the
sources to gfx950 assembly with the build's flags and checks that no LDS
load sits inside a lane-masked region and that M0 is never set from a
readfirstlane result.  (The memory read's runtime-width variant wraps its
buffer loads in the compiler's own descriptor loops; it is excluded.)
CPU only; needs hipcc."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_recurrent_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")

_EXEC_OPEN = re.compile(r"s_(and|or|xor|andn2)_saveexec_b64|s_(and|xor|andn2)_b64 exec,")
_EXEC_CLOSE = re.compile(r"s_or_b64 exec, exec|s_mov_b64 exec,")


def _assembly(src, tmp_path):
    from long_context_recurrent_amd import build as B
    out = os.path.join(str(tmp_path), os.path.basename(src) + ".s")
    cmd = [B.hipcc(), *B.COMMON, *B.DEVICE_FLAGS, *B.EXTRA.get(os.path.basename(src), []),
           "--cuda-device-only", "-S", src, "-o", out]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-2000:]
    with open(out) as f:
        return f.read()


def _kernels(asm):
    for m in re.finditer(r"^(_Z\w+):", asm, re.M):
        end = asm.find(".Lfunc_end", m.start())
        if end > 0:
            yield m.group(1), asm[m.start():end].splitlines()


def _violations(lines):
    masked, bad, loads = False, [], 0
    for n, line in enumerate(lines):
        t = line.strip()
        if _EXEC_CLOSE.match(t):
            masked = False
        elif _EXEC_OPEN.match(t):
            masked = True
        if "global_load_lds" in t or ("buffer_load" in t and " lds" in t):
            loads += 1
            if masked:
                bad.append((n, "LDS load under a lane mask"))
        m = re.match(r"s_mov_b32 m0, (s\d+)", t)
        if m and any(f"v_readfirstlane_b32 {m.group(1)}," in lines[k] for k in range(max(0, n - 6), n)):
            bad.append((n, "M0 from readfirstlane"))
    return loads, bad


def test_lds_loads_issue_with_the_full_wave(tmp_path):
    import concurrent.futures as cf
    sources = ["gemm_bf16.hip", "attention.hip", "memory_mfma.hip"]
    with cf.ThreadPoolExecutor(len(sources)) as ex:
        asms = dict(zip(sources, ex.map(lambda s: _assembly(os.path.join(CSRC, s), tmp_path), sources)))
    for source, asm in asms.items():
        checked = 0
        for name, lines in _kernels(asm):
            if "memread_norm" in name and "ELb0E" in name:
                continue   # runtime-width variant: descriptor loops of the compiler's own
            loads, bad = _violations(lines)
            if loads:
                checked += 1
            assert not bad, f"{source} {name}: {bad[:5]}"
        assert checked > 0, f"{source}: no kernel with LDS loads found"
