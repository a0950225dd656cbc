"""The decode launches' work-unit numbering (``pa::unit_of`` in
``paged_kv_cache_365_amd/csrc/pa_units.h``, the function the kernel calls) is
a permutation of the workgroup ids onto (sibling, partition, KV head,
sequence) units for every grid shape swept, and it places the sibling
workgroups of a unit on one XCD, back to back, outside the tail
(tests/unit_of_check.cpp, compiled for the host with g++)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_unit_numbering_is_a_permutation(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    exe = str(tmp_path / "unit_of_check")
    r = subprocess.run([gxx, "-std=c++17", "-O1", "-Wall", os.path.join(HERE, "unit_of_check.cpp"),
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok "), r.stdout + r.stderr
    shapes, ids = map(int, r.stdout.split()[1:3])
    assert shapes == 9 * 9 * 8 * 11 and ids > 10 ** 6
