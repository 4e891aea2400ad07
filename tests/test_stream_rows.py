"""Host check of the in-place chunked-prefill row mapping (stream_rows.cuh):
compiled with g++ against the HIP headers' host definitions and run on the
CPU over every key tile of ~53,000 (n_sink, window, chunk, n_seen) cases."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_stream_rows_mapping(tmp_path):
    exe = tmp_path / "stream_rows_check"
    cmd = ["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "streamingllm_sink_attn_amd", "csrc"),
           "-o", str(exe), os.path.join(HERE, "native", "stream_rows_check.cpp")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("bad 0"), r.stdout
