"""CPU checks of the measurement plumbing in bench.py: the one-GPU refusal,
the comment-free source hash that keys stored counter results, and the
conversion of two counter runs into HBM bytes per call."""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_source_hash_ignores_comments_only():
    code = "int f(int a) {\n  return a + 1;  // add one\n}\n/* block\n comment */\n"
    assert bench._code_only(code) == bench._code_only(code.replace("add one", "plus 1"))
    assert bench._code_only(code) == bench._code_only("int f(int a) {\n  return a + 1;\n}\n")
    assert bench._code_only(code) != bench._code_only(code.replace("a + 1", "a + 2"))
    assert len(bench.kernel_source_hash()) == 16


def _write(path, counter, rows):
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, (name, value) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                         "Counter_Value": value})


def test_ingest_counters_scales_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    dec = "void pa::(anonymous namespace)::decode_flat_kernel<128, 16, 0, 4, true>(...)"
    mer = "void pa::(anonymous namespace)::flat_merge_heads_kernel<128>(...)"
    copy = "__amd_rocclr_copyBuffer"
    # two calls of decode + merge; the 1 GiB copy reads half its bytes in
    # FETCH_SIZE and all of them in WRITE_SIZE
    _write(tmp_path / "f.csv", "FETCH_SIZE", [(dec, 1000.0), (mer, 10.0), (dec, 1002.0),
                                              (mer, 12.0)] + [(copy, 524288.0)] * 3)
    _write(tmp_path / "w.csv", "WRITE_SIZE", [(dec, 50.0), (mer, 2.0), (dec, 50.0),
                                              (mer, 2.0)] + [(copy, 1048576.0)] * 3)
    e = bench.ingest_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 1.0,
                              "llama3_8b_b64", ["cmd1", "cmd2"])
    assert e["fetch"]["factor"] == 2.0 and e["write"]["factor"] == 1.0
    assert e["fetch"]["bytes_per_call"] == int(1012.0 * 1024 * 2.0)
    assert e["write"]["bytes_per_call"] == int(52.0 * 1024)
    assert e["bytes_per_launch"] == e["fetch"]["bytes_per_call"] + e["write"]["bytes_per_call"]
    assert e["fetch"]["kib_raw_by_kernel"] == {"decode_flat_kernel": 1001.0,
                                               "flat_merge_heads_kernel": 11.0}
    stored = json.load(open(tmp_path / "traffic.json"))
    assert stored["llama3_8b_b64"]["kernel_source_hash"] == bench.kernel_source_hash()
    assert stored["llama3_8b_b64"]["commands"] == ["cmd1", "cmd2"]


def test_ingest_counters_takes_the_grouped_path_only(tmp_path, monkeypatch):
    """A grouped workload's run also times the plain pa_decode on the same
    step: its decode_kernel dispatches are not part of the grouped call."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    grp = "void pa::(anonymous namespace)::decode_group_kernel<128, 16, 0, 4, true>(...)"
    plain = "void pa::(anonymous namespace)::decode_kernel<128, 16, 0, 4, false, false>(...)"
    copy = "__amd_rocclr_copyBuffer"
    _write(tmp_path / "f.csv", "FETCH_SIZE", [(grp, 300.0), (plain, 900.0), (grp, 302.0),
                                              (plain, 900.0)] + [(copy, 524288.0)] * 3)
    _write(tmp_path / "w.csv", "WRITE_SIZE", [(grp, 8.0), (plain, 8.0), (grp, 8.0),
                                              (plain, 8.0)] + [(copy, 1048576.0)] * 3)
    e = bench.ingest_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 1.0,
                              "prefix_share_bs16", [])
    assert e["fetch"]["kib_raw_by_kernel"] == {"decode_group_kernel": 301.0}
    assert e["fetch"]["bytes_per_call"] == int(301.0 * 1024 * 2.0)
    assert e["write"]["bytes_per_call"] == int(8.0 * 1024)


def test_warm_up_runs_exactly_the_requested_steps():
    seen = []
    assert bench.warm_up(seen.append, 3) == 3
    assert seen == [0, 1, 2]


def test_default_warm_up_runs_at_least_twenty_steps_and_a_quarter_second(monkeypatch):
    import torch
    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)
    clock = iter(range(0, 10_000))                   # each reading 10 ms later
    monkeypatch.setattr(bench.time, "perf_counter", lambda: next(clock) * 0.01)
    seen = []
    n = bench.warm_up(seen.append, None)
    assert n == len(seen) and seen == list(range(n))
    assert n >= 25                                   # 20 steps are not yet 250 ms
