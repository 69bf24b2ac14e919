"""bench.py host logic without a GPU: the algorithmic byte counts of the
workloads, the kernels of each path and their bytes, the one-GPU contract and the
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


def test_kernels_of_each_path_and_their_bytes():
    """Every kernel a step launches, per path, with its algorithmic bytes: the
    one-kernel step owns all of them; the label stream belongs to the score
    kernel, the selected rows, query and (with one split) the output to the
    attention kernel, the output to the merge of splits, none to the select."""
    ab = {"labels": 10, "append": 1, "rows": 100, "q": 2, "out": 3}
    mha, gqa = synth.CONFIGS["llama2_7b_4k"], synth.CONFIGS["qwen25_7b_gqa_8k"]
    assert bench.stage_kernels({"path": "fused", "n_split": 1}, mha, True) == {"attn": "k_decode_fused"}
    assert bench.stage_kernels({"path": "fused", "n_split": 1}, gqa, True) == {"attn": "k_decode_fused_g"}
    loc = bench.stage_kernels({"path": "local", "n_split": 8}, mha, True)
    assert loc == {"score": "k_score_local", "select": "k_select_merge", "attn": "k_attn",
                   "combine": "k_combine"}
    st = bench.stage_kernels({"path": "stream", "n_split": 1}, gqa, True)
    assert st == {"append": "k_label", "score": "k_score_chunk", "select": "k_select_stream",
                  "attn": "k_attn_gqa"}
    dense = bench.stage_kernels({"path": "dense", "n_split": 4}, synth.CONFIGS["leank_dense"], False)
    assert dense == {"attn": "k_attn_gqa", "combine": "k_combine"}
    kb = bench.kernel_bytes
    assert kb("attn", "k_decode_fused", ab, True) == 116
    assert kb("score", "k_score_local", ab, False) == 11
    assert kb("score", "k_score_chunk", ab, False) == 10
    assert kb("append", "k_label", ab, False) == 1
    assert kb("select", "k_select_merge", ab, False) == 0
    assert kb("attn", "k_attn", ab, False) == 102 and kb("attn", "k_attn", ab, True) == 105
    assert kb("combine", "k_combine", ab, False) == 3
    # the kernels of a local step together own every algorithmic byte once
    assert sum(kb(s, k, ab, False) for s, k in loc.items()) == sum(ab.values())


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


def test_kernel_stats_record(tmp_path):
    # a synthetic rocprofv3 kernel_stats.csv: two instantiations of one
    # library kernel (averaged by calls), another library kernel, and a
    # framework kernel that the record leaves out
    p = tmp_path / "run_kernel_stats.csv"
    p.write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void ds::(anonymous namespace)::k_attn<1, false, false>(ds::AttnArgs)",30,0,10000.0,1,1,1,1\n'
        '"void ds::(anonymous namespace)::k_attn<1, true, false>(ds::AttnArgs)",10,0,20000.0,1,1,1,1\n'
        '"void ds::(anonymous namespace)::k_combine(ds::AttnArgs, int)",40,0,4000.0,1,1,1,1\n'
        '"void at::native::vectorized_elementwise_kernel<4>(int)",5,0,999.0,1,1,1,1\n')
    out = tmp_path / "kstats.json"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "long_128k",
                        "--stats-from", str(p), "--traffic-out", str(out)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    import json
    rec = json.loads(out.read_text())
    assert rec["workload"] == "long_128k" and rec["source_hash"] == bench.source_hash()
    assert rec["kernels"] == {"k_attn": {"calls": 40, "avg_us": 12.5},
                              "k_combine": {"calls": 40, "avg_us": 4.0}}


def test_further_workload_measured_in_a_child_process(monkeypatch, capsys):
    """A further workload runs in a child process of its own: the command
    names it (with a bounded oracle sample, or none when the headline has
    none), the child's progress lines pass through, its JSON line is returned,
    and a failing child yields None."""
    import io
    import types

    calls = []

    class Child:
        def __init__(self, cmd, stdout=None, text=None):
            calls.append(cmd)
            self.rc = 0 if "long_128k" in cmd else 3
            self.stdout = io.StringIO('bench: progress\n{"value": 1.5, "ms_per_step": 0.1}\n')
            self.returncode = None

        def wait(self):
            self.returncode = self.rc
            return self.rc

    monkeypatch.setattr(subprocess, "Popen", Child)
    args = types.SimpleNamespace(steps=16, warmup=4, stage_events="kernel", unfused=False,
                                 page_size=0, no_cpu_baseline=False, cpu_seconds=10.0)
    r = bench.measure_in_child("long_128k", args)
    assert r == {"value": 1.5, "ms_per_step": 0.1}
    cmd = calls[-1]
    assert cmd[cmd.index("--workload") + 1] == "long_128k" and "--also" in cmd
    assert cmd[cmd.index("--cpu-seconds") + 1] == "5.0" and "--no-cpu-baseline" not in cmd
    assert "bench: progress" in capsys.readouterr().out
    args.no_cpu_baseline = True
    bench.measure_in_child("long_128k", args)
    assert "--no-cpu-baseline" in calls[-1] and "--cpu-seconds" not in calls[-1]
    assert bench.measure_in_child("leank_ds", args) is None
