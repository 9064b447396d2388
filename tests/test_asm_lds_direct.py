"""The prefill kernel that loads activations straight into LDS waits for them
itself: the loads are issued from inline assembly, which the compiler's
wait-count pass does not see, and before each group's barrier the wave waits
vmcnt(N), N being the number of vector-memory instructions it issues after
them.  That holds only if the compiler keeps at least N of them after the
loads.  This test compiles prefill.hip for gfx950 (device code only, to
assembly) and checks, for that kernel, that before every barrier the last
vmcnt wait is no larger than the vector-memory instructions issued since the
last LDS-direct load.  CPU only: hipcc cross-compiles."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "gemm_int8_act_amd"))
import build  # noqa: E402

KERNEL = "_ZN3pq214prefill_kernelILi128ELi128ELb0ELb1ELi128ELi4EEEvPKaPKfPKhPKtPfiiii"
VMEM = re.compile(r"^\s*(buffer|global|scratch)_(load|store)")


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "prefill.s"
    cmd = [hipcc, *build.COMMON_FLAGS, *build.EXTRA_FLAGS["prefill.hip"], "--cuda-device-only", "-S",
           os.path.join(build.CSRC, "prefill.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    text = out.read_text()
    start = text.index(KERNEL + ":")
    end = text.index("s_endpgm", start)
    return text[start:end].splitlines()


def test_lds_direct_waits_cover_the_loads(kernel_asm):
    lds_loads = 0
    after = None
    last_wait = None
    barriers = 0
    for line in kernel_asm:
        t = line.strip()
        if "offen lds" in t:
            lds_loads += 1
            after, last_wait = 0, None
            continue
        m = re.search(r"s_waitcnt.*vmcnt\((\d+)\)", t)
        if m:
            last_wait = int(m.group(1))
        if after is None:
            continue
        if VMEM.match(t):
            after += 1
        if t.startswith("s_barrier"):
            barriers += 1
            assert last_wait is not None and last_wait <= after, \
                f"barrier with vmcnt({last_wait}) but only {after} vector-memory instructions after the LDS loads"
    assert lds_loads >= 8 and barriers >= 8, (lds_loads, barriers)
