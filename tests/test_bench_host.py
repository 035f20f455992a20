"""Host-side parts of bench.py (no GPU): the traffic record written from rocprofv3
counter files, the hash guard that drops it when kernel sources change, and the
one-GPU guard."""

import csv
import json
import subprocess
import sys
from pathlib import Path

import bench

ROOT = Path(__file__).resolve().parent.parent


def _pmc(dirpath: Path, counter: str, rows):
    dirpath.mkdir(parents=True)
    with open(dirpath / "pmc_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, name, val in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": val})


def test_record_then_read_traffic(tmp_path):
    split = "void pgqa::(anonymous namespace)::decode_split_kernel<2, 128, 4, 1, 2>(pgqa::(anonymous namespace)::DecodeArgs)"
    merge = "void pgqa::(anonymous namespace)::decode_merge_kernel<2, 128, 4>(pgqa::(anonymous namespace)::DecodeArgs)"
    pre = "void pgqa::(anonymous namespace)::prefill_kernel<128, 4, false, false, false, false>(pgqa::(anonymous namespace)::PrefillArgs)"
    # two counter instances per dispatch are summed; dispatches are averaged
    _pmc(tmp_path / "fetch_decode", "FETCH_SIZE", [(1, split, 100), (1, split, 50), (2, split, 170), (3, merge, 10)])
    _pmc(tmp_path / "write_decode", "WRITE_SIZE", [(1, split, 3), (2, split, 5), (3, merge, 1)])
    _pmc(tmp_path / "fetch_prefill", "FETCH_SIZE", [(4, pre, 1000)])
    _pmc(tmp_path / "write_prefill", "WRITE_SIZE", [(4, pre, 20)])
    rec_path = tmp_path / "traffic.json"
    base = json.loads((ROOT / "profiles" / "traffic_counters.json").read_text())
    rec_path.write_text(json.dumps({"copy_calibration": base["copy_calibration"]}))
    rec = bench.record_traffic(str(tmp_path), str(rec_path))
    k = rec["decode"]["kernels"]
    assert k["decode_split_kernel<2,128,4,1,2>"] == {"fetch_kib": 160.0, "write_kib": 4.0}
    assert k["decode_merge_kernel<2,128,4>"] == {"fetch_kib": 10.0, "write_kib": 1.0}
    assert "long_ctx" not in rec              # no counter runs for it: left out
    got = bench.recorded_traffic(str(rec_path))
    cal = rec["copy_calibration"]
    want = int((160 + 10) * 1024 * cal["fetch_factor"] + (4 + 1) * 1024 * cal["write_factor"])
    assert got["decode"] == want and got["prefill"] == int(1000 * 1024 * cal["fetch_factor"] + 20 * 1024 * cal["write_factor"])
    assert got["long_ctx"] is None
    # a changed source hash drops the figure
    rec["decode"]["sha256_16"] = "0" * 16
    rec_path.write_text(json.dumps(rec))
    assert bench.recorded_traffic(str(rec_path))["decode"] is None


def test_item_selection():
    assert bench.selected_legs(bench._args([])) == bench.LEGS
    assert bench.selected_legs(bench._args(["--only", "window,mqa"])) == ["window", "mqa"]
    legs = bench.selected_legs(bench._args(["--no-extend", "--no-long-ctx"]))
    assert "chunked_prefill" not in legs and "spec_verify" not in legs and "long_ctx" not in legs and "window" in legs


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
