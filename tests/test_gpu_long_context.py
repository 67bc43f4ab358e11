"""GPU parity of the segmented long-context prefill (pass 1 -> compose -> pass 2).

The oracle never segments: every check compares against the unsplit
token-by-token recurrence.  The full-size case (one 1,048,576-token sequence in
16 segments plus 8 ragged 1K-32K sequences with nonzero initial states, 12
heads, bf16) is checked on samples the oracle can afford: every head of every
ragged sequence, and two heads of the long sequence end to end, each slice
regenerated from its seed and replayed block by block by a worker process.
"""
import os
import time

import numpy as np
import pytest
import torch

from gated_delta_rule_15_amd import inputs as gen
from oracle import kda_oracle as orc

from kda_testutil import packed_to_dev, rel_l2, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_segmented_prefill_small(dtype):
    from gated_delta_rule_15_amd.long_context import kda_prefill_segmented, plan_segments
    lens = [2000, 300, 64, 1, 777]
    p = gen.packed_batch(seed=51, seqlens=lens, H=2, dtype=dtype, init_state=[False, True, True, True, True])
    d = packed_to_dev(p)
    plan = plan_segments(p.cu_seqlens, 256)
    assert plan.n_rows == 8 + 2 + 1 + 1 + 4 and plan.multi == [0, 1, 4]
    o, S = kda_prefill_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], p.cu_seqlens, seg_len=256,
                                 initial_state=d["initial_state"])
    torch.cuda.synchronize()
    o_ref, S_ref = orc.prefill(p.f64("q"), p.f64("k"), p.f64("v"), p.f64("g"), p.f64("beta"), p.cu_seqlens,
                               p.initial_state)
    tol = 2e-3 if dtype == "bf16" else 1e-5
    eo, es = rel_l2(to_f64(o), o_ref), rel_l2(to_f64(S), S_ref)
    print(f"segmented {dtype}: o={eo:.3e} S={es:.3e}")
    assert eo <= tol and es <= tol


def _oracle_slice(args):
    """Worker: regenerate one (sequence, head) slice block by block, replay it in fp64,
    and accumulate the squared error of the GPU outputs held in shared memory."""
    from multiprocessing import shared_memory
    seed, s, h, a, b, H, dtype, shm_name, T, S0 = args
    shm = shared_memory.SharedMemory(name=shm_name)
    try:
        o_gpu = np.ndarray((T, H, 128), dtype=np.uint16, buffer=shm.buf)
        S = None if S0 is None else S0.astype(np.float64)
        err = ref = 0.0
        for blk, b0 in enumerate(range(0, b - a, gen.BLOCK)):
            n = min(gen.BLOCK, b - a - b0)
            q, k, v, beta, g = gen._draw_block(seed, s, h, blk, n, 128, 128)
            q64, k64, v64 = (gen.as_f64(gen._cast(x, dtype), dtype) for x in (q, k, v))
            o_ref, S = orc.recurrence(q64, k64, v64, g.astype(np.float64), beta.astype(np.float64), S)
            o_b = gen.bf16_bits_to_f32(np.array(o_gpu[a + b0:a + b0 + n, h])).astype(np.float64)
            err += float(np.sum((o_b - o_ref) ** 2))
            ref += float(np.sum(o_ref ** 2))
        del o_gpu
    finally:
        shm.close()
    return s, h, err, ref, S


def test_long_context_full_size_sampled():
    """1,048,576 tokens in 16 segments + 8 ragged sequences, 12 heads, bf16, as bench.py --long runs it
    (each 65,536-token segment as eight 8,192-token fragments)."""
    import multiprocessing as mp
    from multiprocessing import shared_memory

    from gated_delta_rule_15_amd.long_context import kda_prefill_segmented, plan_segments
    workers = max(2, min(16, len(os.sched_getaffinity(0))))
    t = time.time()
    p = gen.long_context_batch(seed=5, workers=workers)
    print(f"inputs: T={p.T} drawn in {time.time() - t:.1f}s", flush=True)
    try:
        d = packed_to_dev(p)
    finally:
        p.release()
    H, T = 12, p.T
    o, S = kda_prefill_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], p.cu_seqlens,
                                 plan=plan_segments(p.cu_seqlens, 8192, cut_longer_than=65536),
                                 initial_state=d["initial_state"])
    torch.cuda.synchronize()
    del d
    shm = shared_memory.SharedMemory(create=True, size=T * H * 128 * 2)
    try:
        host = np.ndarray((T, H, 128), dtype=np.uint16, buffer=shm.buf)
        host[:] = o.view(torch.int16).cpu().numpy().view(np.uint16)
        S_gpu = to_f64(S)
        assert np.all(np.isfinite(S_gpu))
        cu = p.cu_seqlens
        tasks = [(5, 0, h, int(cu[0]), int(cu[1]), H, "bf16", shm.name, T, None) for h in (0, 7)]
        tasks += [(5, s, h, int(cu[s]), int(cu[s + 1]), H, "bf16", shm.name, T, p.initial_state[s, h])
                  for s in range(1, len(cu) - 1) for h in range(H)]
        t = time.time()
        with mp.get_context("spawn").Pool(workers) as pool:
            res = pool.map(_oracle_slice, tasks, chunksize=1)
        print(f"oracle: {len(tasks)} slices on {workers} workers in {time.time() - t:.1f}s", flush=True)
        del host
    finally:
        shm.close()
        shm.unlink()
    long_err = sum(r[2] for r in res if r[0] == 0) / sum(r[3] for r in res if r[0] == 0)
    extra_err = sum(r[2] for r in res if r[0] > 0) / sum(r[3] for r in res if r[0] > 0)
    S_ref = {(r[0], r[1]): r[4] for r in res}
    es_long = rel_l2(np.stack([S_gpu[0, h] for h in (0, 7)]), np.stack([S_ref[(0, h)] for h in (0, 7)]))
    keys = [(s, h) for s in range(1, len(cu) - 1) for h in range(H)]
    es_extra = rel_l2(np.stack([S_gpu[s, h] for s, h in keys]), np.stack([S_ref[k] for k in keys]))
    print(f"long sequence (heads 0, 7): o={np.sqrt(long_err):.3e} S={es_long:.3e}; "
          f"8 extras x 12 heads: o={np.sqrt(extra_err):.3e} S={es_extra:.3e}")
    assert np.sqrt(long_err) <= 2e-3 and np.sqrt(extra_err) <= 2e-3
    assert es_long <= 2e-3 and es_extra <= 2e-3


def test_segmented_auto_4096x12_bf16():
    """The 4096-token x 12-head prefill through the segmented driver with the automatic segment length."""
    from gated_delta_rule_15_amd.long_context import auto_seg_len, kda_prefill_segmented
    p = gen.packed_batch(seed=3, seqlens=[4096], H=12, dtype="bf16")
    assert auto_seg_len(p.cu_seqlens, 12) == 704
    d = packed_to_dev(p)
    o, S = kda_prefill_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], p.cu_seqlens, seg_len=None)
    torch.cuda.synchronize()
    o_ref, S_ref = orc.prefill(p.f64("q"), p.f64("k"), p.f64("v"), p.f64("g"), p.f64("beta"), p.cu_seqlens, None)
    eo, es = rel_l2(to_f64(o), o_ref), rel_l2(to_f64(S), S_ref)
    print(f"segmented (704) 4096x12: o={eo:.3e} S={es:.3e}")
    assert eo <= 2e-3 and es <= 2e-3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_segmented_weak_decay(dtype):
    """Decay 100x weaker than the workloads' (log alpha in (-0.001, 0]), so every segment's entry state
    still carries most of the earlier tokens: a wrong transition or composition shows in the outputs."""
    from gated_delta_rule_15_amd.long_context import kda_prefill_segmented, plan_segments
    lens = [1500, 700]
    p = gen.packed_batch(seed=52, seqlens=lens, H=2, dtype=dtype, init_state=True)
    p.g *= np.float32(0.01)
    d = packed_to_dev(p)
    o, S = kda_prefill_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], p.cu_seqlens, seg_len=256,
                                 initial_state=d["initial_state"])
    torch.cuda.synchronize()
    o_ref, S_ref = orc.prefill(p.f64("q"), p.f64("k"), p.f64("v"), p.f64("g"), p.f64("beta"), p.cu_seqlens,
                               p.initial_state)
    # the same tokens with every segment started from zero: far from the reference
    cuts = plan_segments(p.cu_seqlens, 256).rows
    o_cut, _ = orc.prefill(p.f64("q"), p.f64("k"), p.f64("v"), p.f64("g"), p.f64("beta"), cuts, None)
    assert rel_l2(o_cut, o_ref) > 0.1
    tol = 2e-3 if dtype == "bf16" else 1e-5
    eo, es = rel_l2(to_f64(o), o_ref), rel_l2(to_f64(S), S_ref)
    print(f"segmented weak decay {dtype}: o={eo:.3e} S={es:.3e} (cut-at-segments o={rel_l2(o_cut, o_ref):.2f})")
    assert eo <= tol and es <= tol
