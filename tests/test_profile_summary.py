"""Kernel-name matching of the rocprofv3 summariser: exact names, never substrings
(a substring match once merged score_prefill_kernel into prefill_kernel's counters)."""
import csv
import os
import subprocess
import sys

from profile_summary import kernel_key, matches

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kernel_key_and_exact_matching():
    assert kernel_key("void spa::(anonymous namespace)::decode_bf16_kernel<2>(spa::DecodeArgs, int, int)") == \
        "decode_bf16_kernel<2>"
    assert kernel_key("spa::(anonymous namespace)::score_prefill_kernel(signed char const*, int)") == \
        "score_prefill_kernel"
    assert matches(kernel_key("void spa::(anonymous namespace)::prefill_kernel(spa::PrefillArgs)"), "prefill_kernel")
    assert not matches("score_prefill_kernel", "prefill_kernel")
    assert matches("select_kernel<11, false>", "select_kernel")
    assert matches("select_kernel<11, false>", "select_kernel<11, false>")
    assert not matches("select_kernel<11, false>", "select_kernel<11, true>")


def _write_counters(d, rows):
    os.makedirs(os.path.join(d, "host"), exist_ok=True)
    with open(os.path.join(d, "host", "1_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)


def test_counter_summary_keeps_kernels_apart(tmp_path):
    # one copy of 1 MiB counted as 512 KiB read / 1024 KiB written; two kernels whose names nest
    fetch = str(tmp_path / "fetch")
    write = str(tmp_path / "write")
    _write_counters(fetch, [(1, "void spa::permute_kernel(int)", "FETCH_SIZE", 512.0),
                            (2, "void spa::prefill_kernel(int)", "FETCH_SIZE", 1000.0),
                            (3, "void spa::score_prefill_kernel(int)", "FETCH_SIZE", 1.0),
                            (4, "void spa::prefill_kernel(int)", "FETCH_SIZE", 1000.0)])
    _write_counters(write, [(1, "void spa::permute_kernel(int)", "WRITE_SIZE", 1024.0),
                            (2, "void spa::prefill_kernel(int)", "WRITE_SIZE", 10.0),
                            (3, "void spa::score_prefill_kernel(int)", "WRITE_SIZE", 3.0)])
    js = str(tmp_path / "t.json")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "profile_summary.py"), "counters", "--pass", fetch,
                        "--pass", write, "--kernel", "prefill_kernel=4096000", "--kernel", "score_prefill_kernel",
                        "--calib-mib", "1", "--title", "t", "--json", js], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    import json
    s = json.load(open(js))
    k = s["kernels"]["prefill_kernel"]
    assert k["dispatches"] == 2 and k["FETCH_SIZE"] == 1000.0
    assert s["fetch_factor"] == 2048.0 and s["write_factor"] == 1024.0
    assert k["traffic_bytes"] == 1000.0 * 2048 + 10.0 * 1024
    assert s["kernels"]["score_prefill_kernel"]["FETCH_SIZE"] == 1.0
