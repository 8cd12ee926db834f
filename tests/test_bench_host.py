"""bench.py's host-side contract, without a GPU: more than one GPU is refused
with a message and exit status 2, and the HBM traffic recorded from the
counter passes is reported only for the workload it was measured on and
while the kernel sources hash as they did then.
"""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_traffic_follows_the_sources(monkeypatch, tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel\n__global__ void k(int* p) { p[0] = 1; }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    entry = {"sources": ["kernel.hip"], "sources_sha256_16": bench.sources_hash(["kernel.hip"]),
             "workload": "w", "M": 4, "seed": 0, "unique_experts": 3,
             "fetch_kib": 1000.0, "write_kib": 10.0, "copy_fetch_kib": 131072.0, "copy_write_kib": 262144.0}
    monkeypatch.setattr(bench, "GEMM1_TRAFFIC", [entry])
    # the copy read 256 MiB as half that: FETCH_SIZE is scaled by 2, WRITE_SIZE by 1
    assert bench.gemm1_traffic("w", 4, 0, 3) == (2000 + 10) * 1024
    assert bench.gemm1_traffic("w", 8, 0, 3) is None      # another token count
    assert bench.gemm1_traffic("w", 4, 0, 4) is None      # other experts touched
    # comments and layout do not count: the compiled kernel is the same
    src.write_text("/* the kernel */\n__global__ void k(int* p)\n{\n  p[0] = 1;  // store\n}\n")
    assert bench.gemm1_traffic("w", 4, 0, 3) == (2000 + 10) * 1024
    src.write_text("// kernel\n__global__ void k(int* p) { p[0] = 2; }\n")
    assert bench.gemm1_traffic("w", 4, 0, 3) is None      # code changed since the counters
