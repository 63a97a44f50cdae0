"""The waits that cover the kernels' LDS copies, checked in the gfx950
assembly (CPU, no device).

The batch-1 and MFMA kernels copy h into LDS with global_load_lds_dwordx4,
issue their first weight loads, and then wait with an explicit
s_waitcnt vmcnt(N) before reading the copy: vector memory loads retire in
issue order, so the copies have landed once at most N loads are
outstanding, provided at least N vector loads were issued after the last
copy.  The compiler does not know that the copy writes LDS, so nothing else
checks that count: a load that the compiler turns into a scalar load, or
merges, leaves the wait one short and the kernel reading h before it lands.
This test compiles every kernel source with the library's flags and checks,
for every kernel that copies into LDS, that the last vmcnt wait before its
first LDS read is covered by vector loads issued, in straight-line code,
after its last copy (the first such wait, which the kernels place before
any LDS read).

The same listings give each MFMA kernel's static LDS (the finish's tables),
which the launch planner keeps out of the h slice's budget
(MFMA_STATIC_LDS): a kernel that outgrew it could be planned a slice whose
launch fails for want of LDS.
"""
import concurrent.futures
import glob
import os
import re
import subprocess

import pytest

from reduced_vocab_nvfp4_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "reduced_vocab_nvfp4_amd", "csrc")
VMEM = re.compile(r"^\s+(global|buffer|flat|scratch)_(load|store|atomic)\w*")
CF = re.compile(r"^(\.L\w+:|\s+s_(cbranch\w*|branch|setpc\w*|swappc\w*))")


def _asm(src, out):
    flags = [f for f in _build.HIP_FLAGS if f not in ("-shared",)]
    cmd = [_build.HIPCC, *flags, "-I", os.path.join(ROOT, "include"), "-I",
           CSRC, "-S", "--offload-device-only", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    with open(out) as f:
        return f.read().splitlines()


def _kernels(lines):
    """(name, body lines) of every kernel in an assembly listing."""
    out, name, body = [], None, []
    for ln in lines:
        m = re.match(r"^(_Z\w+):", ln)
        if m:
            name, body = m.group(1), []
            continue
        if name is not None:
            body.append(ln)
            if "s_endpgm" in ln:
                out.append((name, body))
                name = None
    return out


def _check(name, body):
    copies = [i for i, l in enumerate(body) if "global_load_lds" in l]
    if not copies:
        return None
    last = copies[-1]
    read = next((i for i in range(last + 1, len(body))
                 if re.match(r"^\s+ds_(read|load)", body[i])), None)
    assert read is not None, f"{name}: no LDS read after the copies"
    waits = [i for i in range(last + 1, read) if "vmcnt(" in body[i]
             and "s_waitcnt" in body[i]]
    assert waits, f"{name}: no vmcnt wait between the copies and the read"
    w = waits[0]  # the first wait after the copies
    n = int(re.search(r"vmcnt\((\d+)\)", body[w]).group(1))
    vm = [i for i in range(last + 1, w) if VMEM.match(body[i])]
    assert len(vm) >= n, (f"{name}: vmcnt({n}) after only {len(vm)} vector "
                          f"loads: the copies may still be in flight")
    if n == 0:
        return n, len(vm)
    # The loads form one straight-line block, and the wait can only be
    # reached through it: every label between the block and the wait is
    # the target of branches from that stretch only.
    first, lastv = vm[0], vm[-1]
    assert not any(CF.match(body[i]) for i in range(first, lastv + 1)), (
        f"{name}: the loads before the wait are not straight-line code")
    labels = {body[i].split(":")[0] for i in range(lastv + 1, w + 1)
              if re.match(r"^\.L\w+:", body[i])}
    for i, l in enumerate(body):
        m = re.match(r"^\s+s_c?branch\w*\s+(\.L\w+)", l)
        if m and m.group(1) in labels:
            assert lastv < i < w, (
                f"{name}: the wait after the copies is reached by a branch "
                f"from outside the loads before it (line {i})")
    return n, len(vm)


@pytest.mark.skipif(not os.path.exists(_build.HIPCC), reason="needs hipcc")
def test_lds_copy_waits_cover_the_copies(tmp_path):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(min(len(srcs), 8)) as ex:
        listings = list(ex.map(
            lambda s: (s, _asm(s, str(tmp_path / (os.path.basename(s) + ".s")))),
            srcs))
    checked = 0
    for src, lines in listings:
        for name, body in _kernels(lines):
            if _check(name, body) is not None:
                checked += 1
    # the batch-1 kernels and the MFMA kernels of every format and mode
    assert checked >= 40, checked


@pytest.mark.skipif(not os.path.exists(_build.HIPCC), reason="needs hipcc")
def test_mfma_static_lds_within_the_reserve(tmp_path):
    src = os.path.join(CSRC, "gemv_mfma.hip")
    text = "\n".join(_asm(src, str(tmp_path / "mfma.s")))
    with open(os.path.join(CSRC, "gemv_common.h")) as f:
        reserve = int(re.search(r"MFMA_STATIC_LDS = (\d+);", f.read()).group(1))
    sizes = [int(m.group(1)) for m in re.finditer(
        r"\.amdhsa_group_segment_fixed_size (\d+)", text)]
    assert len(sizes) >= 20, len(sizes)
    assert max(sizes) <= reserve, (max(sizes), reserve)
