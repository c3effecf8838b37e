"""The persistent attention's work queues, checked on the host: the table
builder and the item decode of csrc/work_queues.h (the functions the kernels
run) are compiled for the host with hipcc and driven over 4000 random
launches (tests/work_queue_driver.hip states what is checked)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_chunked_context_amd", "csrc")


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_every_item_exactly_once(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "work_queue_driver")
    cmd = [hipcc, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "work_queue_driver.hip"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout[-3000:]
