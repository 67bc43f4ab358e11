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


def test_contract_decode_bytes_enumerate_the_positions():
    """The contract decode's per-(request, head) bytes, averaged over the 16 positions of the open chunk,
    equal an explicit walk: a call at position r reads S_e and r open rows, writes row r unless r = 15,
    writes S_e when r = 15, and moves the token's inputs, output and position."""
    D, row = 128, 3 * 128 * 4
    total = 0
    for r in range(16):
        moved = D * D * 4 + r * row            # S_e and the open rows
        moved += D * D * 4 if r == 15 else row  # the close rewrites S_e; otherwise the new row
        moved += 3 * 2 * D + 4 * D + 4          # q, k, v bf16; g fp32; beta
        moved += 2 * D + 8                      # o bf16; position read and written
        total += moved
    assert total / 16 == bench.CONTRACT_DECODE_BYTES_PER_HEAD


def test_contract_flops_enumerate_one_chunk():
    """Per token-head flops of the contract prefill, from one 16-token chunk counted operation by operation."""
    D = 128
    flops = 0
    for r in range(16):
        flops += 2 * (2 * D * D)                # S_e^T k_hat and S_e^T q_hat (fused multiply-add = 2)
        flops += (r + 1) * D * 7                # Gram entries: difference, exponential, product, 2 fmas
        flops += (2 * r + 1) * 2 * D            # u (r terms) and o (r + 1 terms)
    flops += 16 * D * 3 + D * D * (1 + 2 * 16)  # the close: key factors, then S_e update
    assert flops / 16 == bench.FLOP_PER_TOKEN_HEAD_CONTRACT
