"""CPU tests of bench.py's host side: the workload's operation count, the
refusal of more than one GPU, and that the committed counter summaries the
bench quotes were taken on the matmul source as it stands."""
import hashlib
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_chain_operation_count():
    """The value's numerator: 2 * tokens * od * id summed over the seven
    matmuls of a layer, times 28 layers at 3314 tokens (43.25 TOP)."""
    per_layer = (2 * 3584 * 3584 + 512 * 3584 + 3584 * 512 + 2 * 18944 * 3584 + 3584 * 18944)
    assert bench.chain_ops() == 2 * 3314 * 28 * per_layer
    assert abs(bench.chain_ops() / 1e12 - 43.25) < 0.01
    assert {wt for _, wt, _, _, _ in bench.LAYER_GEMMS} == {"q4_K", "q6_K"}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _gemm_sha():
    with open(os.path.join(ROOT, "quantized_matmul_rmsnorm_amd", "csrc", "gemm.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _json_line(name, key):
    with open(os.path.join(ROOT, "profiles", name)) as f:
        for line in f:
            if line.startswith(key + ":"):
                return json.loads(line.split(":", 1)[1])
    raise AssertionError(f"{name} has no {key} line")


def test_traffic_summary_matches_the_matmul_source():
    """bench.py reports the HBM traffic only while the summary's source hash
    matches gemm.hip; a kernel change must come with re-taken counters."""
    rec = _json_line("k_gemm_da_q4k_traffic_7b_chain.txt", "traffic_json")
    assert rec["gemm_sha256"] == _gemm_sha()
    assert bench.measured_traffic() == rec
    # the f16 tiles' per-call traffic lies between the compulsory bytes of
    # their layout (about 206 MB per call) and the counted re-reads
    assert 206e6 < rec["bytes_per_launch"] < 2e9
    assert rec["packed_bytes_per_launch"] < rec["bytes_per_launch"]


def test_counter_summary_matches_the_matmul_source():
    rec = _json_line("k_gemm_da_counters_7b_gate_qo_down.txt", "counters_json")
    assert rec["gemm_sha256"] == _gemm_sha()
    for shape, v in rec.items():
        if shape == "gemm_sha256":
            continue
        assert 0 < v["mfma_util"] < 1 and 0 < v["valu_busy"] < 1, shape
