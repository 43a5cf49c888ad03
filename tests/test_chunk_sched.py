"""Host check of the persistent chunk solver's task order (no GPU).

The two-sided solver's leaves run as one persistent launch per chunk of
tile-diagonals: workgroups draw tickets, and each task polls the values it
reads (the outputs of the chunk's tiles before it in its row and column) until
they are written (`csrc/kq_chunk_sched.hpp`).  `chunk_sched_check.cpp` builds
that header's ticket decoding on the host and checks, for every chunk the
recursion makes on the configured shapes and on small, ragged and degenerate
tile grids, that every value a task reads is written by a task with a smaller
ticket of the same chunk (so a launch always drains, whatever number of its
workgroups is resident; FastKron page, section 2.3: an entry depends on every
entry above and to the left of it); then it runs chunks on host threads with
random delays.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, os.pardir, "two_sided_gptq_damped_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not found")
def test_chunk_task_order(tmp_path):
    exe = str(tmp_path / "chunk_sched_check")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-I", CSRC,
                    os.path.join(HERE, "chunk_sched_check.cpp"), "-o", exe, "-lpthread"],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
