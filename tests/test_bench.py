"""bench.py's host-side contract, CPU only: the single-GPU refusal, the counter record's hash
gate, the algorithmic byte counts and the CPU-baseline record."""
import json
import os
import subprocess
import sys

import numpy as np

import kvgen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_traffic_needs_the_current_kernel_sources(tmp_path):
    rec = {"kernel_source_sha256": bench.kernel_source_hash(),
           "workloads": {"c4": {"hbm_bytes_per_launch": 1234}}}
    good = tmp_path / "t.json"
    good.write_text(json.dumps(rec))
    assert bench.measured_traffic(str(good), "c4") == 1234
    assert bench.measured_traffic(str(good), "m-t4") is None          # not measured
    rec["kernel_source_sha256"] = "0" * 64                             # another kernel
    stale = tmp_path / "s.json"
    stale.write_text(json.dumps(rec))
    assert bench.measured_traffic(str(stale), "c4") is None
    assert bench.measured_traffic(str(tmp_path / "missing.json"), "c4") is None


def test_algorithmic_bytes_closed_forms():
    # 16 sequences x 32768 tokens x 8 KV heads x 256 B (FP8) = 2^30
    s = kvgen.SPECS["c4"]
    assert s.num_seqs * s.context * s.num_kv_heads * kvgen.kv_bytes_per_token_head("fp8", 128) == 1 << 30
    # a chunk of n_q queries under a window W reads min(L, W + n_q - 1) keys per sequence
    inp = kvgen.make_inputs(kvgen.spec("c1", pool_total=None, queries_per_seq=5, num_seqs=3),
                            lengths=[300, 40, 9], windows=[100, 0, 7])
    assert inp.spans().tolist() == [104, 40, 9]
    assert inp.kv_bytes() == (104 + 40 + 9) * 1 * 256


def test_cpu_baseline_record():
    inp = kvgen.make_inputs(kvgen.spec("c1", fmt="turbo4", head_dim=128, context=200))
    rec = bench.cpu_baseline(inp, 0.5)
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s"
    assert rec["value"] > 0 and rec["cores"] >= 1 and "pairs" in rec["sample"]
    assert np.isfinite(rec["value"])
