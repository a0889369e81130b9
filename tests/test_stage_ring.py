"""The staging ring of plan uploads (kv.plan PinnedIndexRing; attn.dense
force_double_buffer), checked on the CPU: the ring's own code (csrc/stage.h)
built with g++ against a simulated GPU reader."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "stage_ring_check.cpp")
CSRC = os.path.join(ROOT, "paged_kv_attention_plan_amd", "csrc")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("stage") / "stage_ring_check")
    subprocess.run([gxx, "-std=c++17", "-O2", "-pthread", "-I", CSRC, SRC, "-o", out], check=True)
    return out


def _run(exe, mode):
    res = subprocess.run([exe, mode], capture_output=True, text=True, timeout=60)
    print(res.stdout)
    return res


def test_every_upload_reads_its_own_plan(exe):
    res = _run(exe, "ring")
    assert res.returncode == 0, res.stdout


def test_the_check_sees_an_unguarded_overwrite(exe):
    # Without acquire() the host rewrites a buffer the reader has not copied:
    # the same check must catch it, or it proves nothing about the guard.
    res = _run(exe, "unguarded")
    assert res.returncode == 3, res.stdout


def test_unfinished_reader_times_out(exe):
    res = _run(exe, "timeout")
    assert res.returncode == 0, res.stdout


def test_flags_of_an_earlier_upload_do_not_free_the_buffer(exe):
    res = _run(exe, "stale")
    assert res.returncode == 0, res.stdout
