"""bench.py host logic without a GPU: the algorithmic byte counts of the
workloads, the dominant-kernel choice per path, the one-GPU contract and the
source hash that keys the stored counter records, and the counter record of
the calibration workload."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_algorithmic_bytes_of_the_workloads():
    # label stream and selected K/V rows per step at S = S0 + 1
    ab = bench.algorithmic_bytes(synth.CONFIGS["llama2_7b_4k"], 4097)
    assert ab["labels"] == 32 * 32 * 4097 * 6          # int4 r = 8: 4 B codes + 2 B scale
    assert ab["rows"] == 32 * 32 * 256 * 256 * 2       # k rows of K and V, 256 B each
    ab = bench.algorithmic_bytes(synth.CONFIGS["qwen25_7b_gqa_8k"], 8193)
    assert ab["labels"] == 64 * 4 * 8193 * 32          # fp16 r = 16
    assert ab["q"] == 64 * 28 * 128 * 2 and ab["out"] == 64 * 28 * 128 * 2
    ab = bench.algorithmic_bytes(synth.CONFIGS["leank_dense"], 32769)
    assert ab["labels"] == 0 and ab["rows"] == 32 * 4 * 32769 * (32 + 128) * 2


def test_dominant_kernel_per_path():
    ab = {"labels": 10, "append": 1, "rows": 100, "q": 2, "out": 3}
    assert bench.dominant_kernel({"path": "fused", "n_split": 1}, ab, 1) == ("k_decode_fused", 116)
    assert bench.dominant_kernel({"path": "fused", "n_split": 1}, ab, 7)[0] == "k_decode_fused_g"
    assert bench.dominant_kernel({"path": "local", "n_split": 8}, ab, 1) == ("k_attn", 102)
    assert bench.dominant_kernel({"path": "dense", "n_split": 1}, ab, 7) == ("k_attn", 105)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    d = tmp_path / "sparse_attention_decode_ds_amd" / "csrc"
    d.mkdir(parents=True)
    (d / "k.hip").write_text("int f() { return 1; }  // one\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h1 = bench.source_hash()
    (d / "k.hip").write_text("/* two */\nint f() {\n  return 1;\n}\n")
    assert bench.source_hash() == h1
    (d / "k.hip").write_text("int f() { return 2; }\n")
    assert bench.source_hash() != h1


def test_traffic_record_for_the_calibration_workload(tmp_path):
    # two synthetic counter files: the reference copy (neg_kernel) and the
    # calibration column kernel, two dispatches each, values split over XCDs
    def csv(path, counter, copy_kib, kern_kib):
        rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
        for d in (1, 2):
            for half in (0.25, 0.75):
                rows.append("%d,neg_kernel,%s,%.1f" % (d, counter, copy_kib * half))
        for d in (3, 4):
            rows.append("%d,ds::k_calib_cols(ds::CalibArgs),%s,%.1f" % (d, counter, kern_kib))
        path.write_text("\n".join(rows) + "\n")
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    csv(f, "FETCH_SIZE", 131072.0, 66000.0)   # FETCH_SIZE reads half of a 256 MiB copy
    csv(w, "WRITE_SIZE", 262144.0, 1000.0)
    out = tmp_path / "rec.json"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload",
                        "calib_llama2_7b_4k", "--calib-copy-mb", "256", "--traffic-from", str(f),
                        str(w), "--traffic-kernel", "k_calib_cols", "--traffic-out", str(out)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    import json
    rec = json.loads(out.read_text())
    assert rec["workload"] == "calib_llama2_7b_4k" and rec["kernel"] == "k_calib_cols"
    assert rec["calibration"]["fetch_factor"] == 2.0 and rec["calibration"]["write_factor"] == 1.0
    assert rec["bytes_per_launch"] == int(round((66000.0 * 2 + 1000.0) * 1024))
    assert rec["dispatches"] == [2, 2]
