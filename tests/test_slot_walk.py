"""The 64-row decode's slot walk (mla_slot_walk.h, included by the kernel)
built for the host and checked on random batches, tables and partitions:
block-table entries are read only for pages that hold tokens and inside the
row, copies are sized to the live tokens, and the walk covers exactly its
partition.  CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_slot_walk_host_check(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "slot_walk_check")
    subprocess.run([cxx, "-std=c++17", "-O1", "-Wall", "-Werror", "-I",
                    os.path.join(ROOT, "mla_paged_kv_06_amd", "csrc"),
                    os.path.join(ROOT, "tests", "slot_walk_check.cpp"), "-o", exe], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout + res.stderr
