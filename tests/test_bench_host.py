"""Host-side checks of bench.py: the one-GPU refusal, the rule that counter
traffic is reported only for the kernel source it was taken on, and the
arithmetic of the committed counter summaries."""
import glob
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    msg = json.loads(res.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def _fake_tree(tmp_path, src_text, rec):
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "sparse_attention_decode_row_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "kernels.hip").write_text(src_text)
    with open(tmp_path / "profiles" / "dsa_decode_kernel_long_hbm_counters.json", "w") as f:
        json.dump(rec, f)
    return csrc / "kernels.hip"


def test_traffic_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    src_text = "// kernel source\n"
    sha = hashlib.sha256(src_text.encode()).hexdigest()
    rec = {"kernel": "dsa_decode_kernel", "workload": "long", "kernel_source_sha256": sha,
           "rows_per_sequence": 1, "traffic_bytes_per_launch": 12345}
    src = _fake_tree(tmp_path, src_text, rec)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("long") == 12345.0
    assert bench.measured_traffic("long", rows_per_sequence=1) == 12345.0
    assert bench.measured_traffic("long", rows_per_sequence=4) is None
    assert bench.measured_traffic("glm") is None          # no summary for it
    src.write_text(src_text + "// changed\n")
    assert bench.measured_traffic("long") is None         # the kernel changed since


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_counters.json"))),
                         ids=lambda p: os.path.basename(p))
def test_committed_counter_summaries_add_up(path):
    """traffic = FETCH_SIZE * fetch factor + WRITE_SIZE * write factor, in
    bytes (the counters read KiB per dispatch), for the workload the file
    is named for."""
    with open(path) as f:
        rec = json.load(f)
    name = os.path.basename(path)
    assert name == f"{rec['kernel']}_{rec['workload']}_hbm_counters.json"
    want = (rec["fetch_kib_per_dispatch"] * rec["fetch_factor"]
            + rec["write_kib_per_dispatch"] * rec["write_factor"]) * 1024
    assert abs(rec["traffic_bytes_per_launch"] - want) <= 1024
    assert len(rec["kernel_source_sha256"]) == 64
