"""Host-side check of the streaming kernels' work split (stream_schedule.hpp): the kernels and this
checker include the same header. Over a sweep of CU counts, blocks per CU, units per row tile and
row-tile counts, every unit must fall in exactly one block's range, and no range may touch more row
tiles than the kernels stage in LDS (see stream_schedule_check.cpp)."""
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_stream_schedule_covers_every_unit_once(tmp_path):
    exe = tmp_path / "stream_schedule_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Wextra", "-Werror",
                    f"-I{ROOT / 'gemm_nvfp4_amd' / 'csrc'}", str(ROOT / "tests" / "stream_schedule_check.cpp"),
                    "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0 and res.stdout.startswith("ok "), res.stdout + res.stderr
