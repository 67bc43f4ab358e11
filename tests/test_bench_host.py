"""Host logic of bench.py (no GPU): the counter-to-traffic arithmetic and the single-GPU guard."""
import csv
import os
import subprocess
import sys

import bench


def _write_pass(d, name, rows):
    os.makedirs(os.path.join(d, name))
    with open(os.path.join(d, name, f"{name}_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (kernel, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": name.split("_", 1)[1],
                        "Counter_Value": value})


def test_write_traffic_scales_by_the_copy(tmp_path):
    d = str(tmp_path)
    dec = "void kda::(anonymous namespace)::kda_decode_kernel<kda::BF16>(StepArgs, int)"
    cp = "void at::native::vectorized_elementwise_kernel<4, MulFunctor>"
    fill = "void at::native::vectorized_elementwise_kernel<4, FillFunctor>"
    # the copy of 256 MiB reads half its bytes on FETCH_SIZE and all of them on WRITE_SIZE
    _write_pass(d, "dec_FETCH_SIZE", [(dec, 25000.0), (dec, 25002.0)])
    _write_pass(d, "dec_WRITE_SIZE", [(dec, 49000.0), (dec, 49000.0)])
    _write_pass(d, "copy_FETCH_SIZE", [(fill, 16.0)] + [(cp, 131072.0)] * 20)
    _write_pass(d, "copy_WRITE_SIZE", [(fill, 262144.0)] + [(cp, 262144.0)] * 20)
    t = bench.write_traffic(d, out=os.path.join(d, "t.json"))
    assert t["copy_calibration"]["fetch_factor"] == 2.0 and t["copy_calibration"]["write_factor"] == 1.0
    assert t["fetch_bytes_per_launch"] == 25001 * 1024 * 2
    assert t["write_bytes_per_launch"] == 49000 * 1024
    assert t["algorithmic_bytes_per_launch"] == 768 * 132612
    assert t["source_hash"] == bench.src_hash("kda_step.hip", "kda_common.hpp")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in (r.stdout + r.stderr)
