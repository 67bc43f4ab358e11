"""GPU parity of the segmented long-context prefill (pass 1 -> compose -> pass 2).

The oracle never segments: every check compares against the unsplit
token-by-token recurrence.  The full-size case (one 1,048,576-token sequence in
16 segments plus 8 ragged 1K-32K sequences with nonzero initial states, 12
heads, bf16) is checked on every (sequence, head) slice, each regenerated from
its seed and replayed block by block by a worker process.
"""
import os
import time

import numpy as np
import pytest
import torch

from gated_delta_rule_15_amd import inputs as gen
from oracle import kda_oracle as orc

from kda_testutil import check_parity, packed_slices, packed_to_dev, rel_l2, to_f64, unit_slices

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
    check_parity(o, o_ref, tol, packed_slices(p.cu_seqlens, 2), bf16_out=dtype == "bf16", tag=f"segmented {dtype} o")
    check_parity(S, S_ref, tol, unit_slices(len(lens), 2), tag=f"segmented {dtype} S")


SEG_CHECK = 65536  # the long sequence is also checked segment by segment (a multiple of the input block)


def _oracle_slice(args):
    """Worker: regenerate one (sequence, head) slice block by block, replay it in fp64, and compare the
    GPU outputs held in shared memory.  Returns, per 65,536-token piece of the slice, the squared error
    and squared reference, and per piece the largest excess of an element over one bf16 ulp,
    max(|o - o_ref| - 2^-7 |o_ref|), for the per-element bound; and the final state."""
    from multiprocessing import shared_memory
    seed, s, h, a, b, H, dtype, shm_name, T, S0 = args
    shm = shared_memory.SharedMemory(name=shm_name)
    try:
        o_gpu = np.ndarray((T, H, 128), dtype=np.uint16, buffer=shm.buf)
        S = None if S0 is None else S0.astype(np.float64)
        n_piece = max(1, -(-(b - a) // SEG_CHECK))
        err, ref, excess = np.zeros(n_piece), np.zeros(n_piece), np.zeros(n_piece)
        for blk, b0 in enumerate(range(0, b - a, gen.BLOCK)):
            n = min(gen.BLOCK, b - a - b0)
            q, k, v, beta, g = gen._draw_block(seed, s, h, blk, n, 128, 128)
            q64, k64, v64 = (gen.as_f64(gen._cast(x, dtype), dtype) for x in (q, k, v))
            o_ref, S = orc.recurrence(q64, k64, v64, g.astype(np.float64), beta.astype(np.float64), S)
            o_b = gen.bf16_bits_to_f32(np.array(o_gpu[a + b0:a + b0 + n, h])).astype(np.float64)
            piece = b0 // SEG_CHECK
            d = np.abs(o_b - o_ref)
            err[piece] += float(np.sum(d ** 2))
            ref[piece] += float(np.sum(o_ref ** 2))
            excess[piece] = max(excess[piece], float(np.max(d - 2.0 ** -7 * np.abs(o_ref))))
            assert np.all(np.isfinite(o_b))
        del o_gpu
    finally:
        shm.close()
    return s, h, err, ref, excess, S


def test_long_context_full_size():
    """1,048,576 tokens in 16 segments + 8 ragged sequences, 12 heads, bf16, as bench.py runs it (each
    65,536-token segment as eight 8,192-token fragments).  Every (sequence, head) slice is replayed by
    the oracle: all 12 heads of the long sequence end to end and every head of the 8 extras.  Checked
    per slice and, for the long sequence, per 65,536-token segment: rel-L2 of the outputs and of each
    final state <= 2e-3, and every output within one bf16 ulp plus 1e-3 of its segment's RMS."""
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
        # the twelve long slices first: they set the pace
        tasks = [(5, 0, h, int(cu[0]), int(cu[1]), H, "bf16", shm.name, T, None) for h in range(H)]
        tasks += [(5, s, h, int(cu[s]), int(cu[s + 1]), H, "bf16", shm.name, T, p.initial_state[s, h])
                  for s in range(1, len(cu) - 1) for h in range(H)]
        t = time.time()
        res = gen.pool_map(_oracle_slice, tasks, workers)
        print(f"oracle: {len(tasks)} slices on {workers} workers in {time.time() - t:.1f}s", flush=True)
        del host
    finally:
        shm.close()
        shm.unlink()
    worst_slice = worst_piece = worst_elem = worst_state = 0.0
    for s, h, err, ref, excess, S_ref in res:
        e_slice = np.sqrt(err.sum() / ref.sum())
        e_piece = np.sqrt(err / ref)
        e_elem = excess / (1e-3 * np.sqrt(ref / np.maximum(1, np.minimum(SEG_CHECK, int(cu[s + 1] - cu[s]))
                                                        * 128)))
        es = rel_l2(S_gpu[s, h], S_ref)
        assert e_slice <= 2e-3, f"sequence {s} head {h}: outputs rel-L2 {e_slice:.3e}"
        assert np.all(e_piece <= 2e-3), f"sequence {s} head {h}: segment rel-L2 {e_piece.max():.3e}"
        assert es <= 2e-3, f"sequence {s} head {h}: final state rel-L2 {es:.3e}"
        worst_slice, worst_piece = max(worst_slice, e_slice), max(worst_piece, float(e_piece.max()))
        worst_state = max(worst_state, es)
        # pieces hold SEG_CHECK tokens (the long sequence) or the whole sequence (an extra)
        assert np.all(e_elem <= 1.0), f"sequence {s} head {h}: element {e_elem.max():.2f} of its bound"
        worst_elem = max(worst_elem, float(e_elem.max()))
    long_err = np.sqrt(sum(r[2].sum() for r in res if r[0] == 0) / sum(r[3].sum() for r in res if r[0] == 0))
    extra_err = np.sqrt(sum(r[2].sum() for r in res if r[0] > 0) / sum(r[3].sum() for r in res if r[0] > 0))
    print(f"long sequence, 12 heads: o={long_err:.3e}; 8 extras x 12 heads: o={extra_err:.3e}; worst slice "
          f"{worst_slice:.3e}, worst 65,536-token segment {worst_piece:.3e}, worst final state {worst_state:.3e}, "
          f"worst element {worst_elem:.2f} of its bound")
    assert long_err <= 2e-3 and extra_err <= 2e-3


def test_segmented_auto_4096x12_bf16():
    """The 4096-token x 12-head prefill through the segmented driver with the automatic segment length."""
    from gated_delta_rule_15_amd.long_context import auto_seg_len, kda_prefill_segmented
    p = gen.packed_batch(seed=3, seqlens=[4096], H=12, dtype="bf16")
    assert auto_seg_len(p.cu_seqlens, 12) == 704
    d = packed_to_dev(p)
    o, S = kda_prefill_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], p.cu_seqlens, seg_len=None)
    torch.cuda.synchronize()
    o_ref, S_ref = orc.prefill(p.f64("q"), p.f64("k"), p.f64("v"), p.f64("g"), p.f64("beta"), p.cu_seqlens, None)
    check_parity(o, o_ref, 2e-3, packed_slices(p.cu_seqlens, 12), bf16_out=True, tag="segmented (704) 4096x12 o")
    check_parity(S, S_ref, 2e-3, unit_slices(1, 12), tag="segmented (704) 4096x12 S")


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
    print(f"segmented weak decay {dtype}: cut-at-segments o={rel_l2(o_cut, o_ref):.2f}")
    check_parity(o, o_ref, tol, packed_slices(p.cu_seqlens, 2), bf16_out=dtype == "bf16",
                 tag=f"segmented weak decay {dtype} o")
    check_parity(S, S_ref, tol, unit_slices(len(lens), 2), tag=f"segmented weak decay {dtype} S")


@pytest.mark.parametrize("lens", [[1500, 300, 64, 1, 777], [1500, 777, 257]], ids=["mixed", "all_cut"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_segmented_split_passes_bitwise_equal(dtype, lens):
    """The segmented driver on the split path (pass 1 over every row with the output operands kept,
    pass 2 reusing that one preparation through KDA_WS_PREPARED) equals the driver on the single
    kernel bit for bit, and the oracle.  When every sequence is cut, the split path takes final
    states from the scan through the last segment instead of pass 2's walk: outputs stay bitwise
    equal (same entry states), final states are checked against the oracle."""
    from gated_delta_rule_15_amd.long_context import alloc_work, kda_prefill_segmented, plan_segments
    all_cut = min(lens) > 256
    p = gen.packed_batch(seed=53, seqlens=lens, H=2, dtype=dtype, init_state=[False] + [True] * (len(lens) - 1))
    d = packed_to_dev(p)
    plan = plan_segments(p.cu_seqlens, 256)
    assert (len(plan.multi) == len(lens)) == all_cut
    outs = []
    for split in (False, True):
        work = alloc_work(plan, 2, d["q"].device, d["q"].dtype, split=split)
        assert (work["ws"] is not None) == split
        o, S = kda_prefill_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], p.cu_seqlens, plan=plan, work=work,
                                     initial_state=d["initial_state"])
        torch.cuda.synchronize()
        outs.append((o, S))
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(outs[0][0].view(bits), outs[1][0].view(bits))
    if not all_cut:
        assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))
    o_ref, S_ref = orc.prefill(p.f64("q"), p.f64("k"), p.f64("v"), p.f64("g"), p.f64("beta"), p.cu_seqlens,
                               p.initial_state)
    tol = 2e-3 if dtype == "bf16" else 1e-5
    check_parity(outs[1][0], o_ref, tol, packed_slices(p.cu_seqlens, 2), bf16_out=dtype == "bf16",
                 tag=f"segmented split passes {dtype} o")
    check_parity(outs[1][1], S_ref, tol, unit_slices(len(lens), 2), tag=f"segmented split passes {dtype} S")
