#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

Headline (the JSON line's ``value``): decode state-update HBM GB/s for one
single-token decode step of 64 requests x 12 heads (d_k = d_v = 128, fp32
state updated in place, bf16 q/k/v/o).  A timed step is one decode launch over
one batch; K steps run back to back from a HIP graph, rotating 8 independent
state sets (8 x 48 MiB, beyond the 256 MB Infinity Cache) so that the state
bytes come from HBM.  ``ms_per_step`` is the mean step time.

The other rows of the hot path are timed in the same run and reported under
``rows``: chunked prefill of 4096 tokens x 12 heads (bf16), draft-block verify
plus replay commit for 32 requests x 12 heads x 8 tokens, and (unless
--no-long) the 1,048,576-token + 8 ragged-sequence long-context prefill
through segment composition.  Decode and verify also report the median over
11 replays of a graph of >= 100 launches, and a plain copy of the decode's
footprint gives the measured memory roof beside the 8 TB/s one.

``roofline`` is for the decode kernel (algorithmic bytes per launch / mean
launch time vs 8 TB/s).  ``cpu_baseline`` is the CPU oracle (fp64, token by
token) timed on this host's cores on a bounded sample of the same decode
workload; ``rows.cpu_oracle_prefill`` times it on the three prefill workloads.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-long] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
D = 128
FLOP_PER_TOKEN_HEAD_PREFILL = 6 * D * D + 10 * 64 * D  # 180,224 algorithmic flop (chunk 64)
BYTES_PER_TOKEN_HEAD_PREFILL_BF16 = 3 * 2 * D + 4 * D + 4 + 2 * D  # q,k,v bf16 + g fp32 + beta + o bf16 = 1540
STATE_BYTES = D * D * 4
FP32_VALU_PEAK_TFLOPS = 157.3

# Row contract (16-token chunks), per token-head, averaged over the 16 positions r of a chunk:
#   S_e^T k_hat and S_e^T q_hat: 2 * 2 * D * D flop; Gram entries for s <= r: (r + 1) * D * 7
#   (difference, exponential, product, two fused multiply-adds); u and o: (2r + 1) * 2 * D;
#   the close once per 16 tokens: 16 * D * 3 (key factors) + D * D * (1 + 2 * 16) (the S_e update).
CONTRACT_CHUNK = 16
FLOP_PER_TOKEN_HEAD_CONTRACT = (4 * D * D + sum((r + 1) * D * 7 + (2 * r + 1) * 2 * D for r in range(16)) / 16
                                + (16 * D * 3 + D * D * 33) / 16)
# Decode through the contract, per (request, head) and step, averaged over the 16 positions: read
# S_e; read the r open rows (k, b, u fp32); write the new row unless it closes the chunk; write S_e
# when it does; q/k/v bf16, g fp32, beta in; o bf16 out; position read and written.
ROW_BYTES = 3 * D * 4
CONTRACT_DECODE_BYTES_PER_HEAD = (STATE_BYTES + sum(r * ROW_BYTES for r in range(16)) / 16
                                  + ROW_BYTES * 15 / 16 + STATE_BYTES / 16 + 3 * 2 * D + 4 * D + 4 + 2 * D + 8)


def decode_bytes_per_head(in_bytes=2):
    # state read + write, q/k/v/g/beta in, o out
    return 2 * STATE_BYTES + 3 * in_bytes * D + 4 * D + 4 + in_bytes * D


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_delta_rule_15_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
def to_dev(x, dtype="f32"):
    import numpy as np
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


EAGER = False  # --eager: plain launches (for counter collection), no graph


def eager_time_ms(fns, warmup):
    import torch
    for _ in range(warmup):
        for f in fns[: min(len(fns), 8)]:
            f()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for f in fns:
        f()
    end.record()
    end.synchronize()
    return start.elapsed_time(end) / len(fns)


def graph_time_ms(fns, warmup):
    """Capture fns (called in order) into one HIP graph; return mean ms per fn over one replay."""
    import torch
    if EAGER:
        return eager_time_ms(fns, warmup)
    for _ in range(warmup):
        for f in fns[: min(len(fns), 8)]:
            f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns[: min(len(fns), 8)]:  # warm the capture stream
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    g.replay()  # untimed replay
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    g.replay()
    end.record()
    end.synchronize()
    return start.elapsed_time(end) / len(fns)


def graph_replay_stats_ms(fns, warmup, replays=11):
    """Capture fns (>= 100 launches) into one HIP graph and time `replays` replays of it with events
    on the graph's stream: returns (median, min, max) of the per-launch mean of each replay."""
    import statistics
    import torch
    for _ in range(warmup):
        for f in fns[: min(len(fns), 8)]:
            f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns[: min(len(fns), 8)]:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(replays):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        g.replay()
        end.record()
        end.synchronize()
        per.append(start.elapsed_time(end) / len(fns))
    return statistics.median(per), min(per), max(per)


def bench_decode(steps, warmup, n_sets=8, prologue=False):
    """The decode step (64 x 12, bf16); ``prologue``: raw inputs through kda_decode_step_prologue
    (same algorithmic bytes: q, k, g are read and o written once either way)."""
    import torch
    from gated_delta_rule_15_amd import inputs as gen
    from gated_delta_rule_15_amd import kda
    N, H = 64, 12
    b = gen.step_batch(seed=2, N=N, G=1, H=H, dtype="bf16", raw=prologue)
    pro = kda.Prologue() if prologue else None
    sets = []
    for i in range(n_sets):
        sets.append(dict(q=to_dev(b.q[:, 0], "bf16"), k=to_dev(b.k[:, 0], "bf16"), v=to_dev(b.v[:, 0], "bf16"),
                         g=to_dev(b.g[:, 0]), beta=to_dev(b.beta[:, 0]), state=to_dev(b.state),
                         o=torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda:0")))
    fns = []
    for i in range(steps):
        s = sets[i % n_sets]
        fns.append(lambda s=s: kda.kda_decode_step(s["q"], s["k"], s["v"], s["g"], s["beta"], s["state"], o=s["o"],
                                                   prologue=pro))
    ms = graph_time_ms(fns, warmup)
    nbytes = N * H * decode_bytes_per_head(2)
    out = dict(ms=ms, bytes=nbytes, gbps=nbytes / (ms * 1e-3) / 1e9, N=N, H=H, n_sets=n_sets)
    if not prologue and not EAGER:
        fns100 = [(lambda s=sets[i % n_sets]: kda.kda_decode_step(s["q"], s["k"], s["v"], s["g"], s["beta"],
                                                                  s["state"], o=s["o"]))
                  for i in range(max(100, len(fns)))]
        med, lo, hi = graph_replay_stats_ms(fns100, warmup)
        out.update(median_ms=med, median_gbps=nbytes / (med * 1e-3) / 1e9,
                   median_protocol=f"median over 11 replays of a graph of {len(fns100)} launches "
                                   f"(per-replay means {lo * 1e3:.2f}-{hi * 1e3:.2f} us)")
    return out


def bench_copy_probe(steps, warmup, n_sets=8):
    """The decode's memory roof measured: a plain device copy of the same footprint (48 MiB read and
    48 MiB written per launch, the size of the 64 x 12 state), rotating the same number of buffer
    pairs, timed the same way: the library's probe (kda_copy_probe, nontemporal float4, eight per
    thread) and, for context, torch's copy_."""
    import torch
    from gated_delta_rule_15_amd import kda
    n = 64 * 12 * D * D
    pairs = [(torch.ones(n, device="cuda:0"), torch.empty(n, device="cuda:0")) for _ in range(n_sets)]
    fns = [lambda p=pairs[i % n_sets]: kda.copy_probe(p[0], p[1]) for i in range(max(100, steps))]
    med, lo, hi = graph_replay_stats_ms(fns, warmup)
    fns_t = [lambda p=pairs[i % n_sets]: p[1].copy_(p[0]) for i in range(max(100, steps))]
    med_t, _, _ = graph_replay_stats_ms(fns_t, warmup)
    del pairs, fns, fns_t
    # the decode's own pattern: its 64 x 12 states rewritten in place in its tiling, 8 rotated sets
    states = [torch.ones((64 * 12, D, D), device="cuda:0") for _ in range(n_sets)]
    fns_s = [lambda t=states[i % n_sets]: kda.copy_probe_state(t, t) for i in range(max(100, steps))]
    med_s, lo_s, hi_s = graph_replay_stats_ms(fns_s, warmup)
    # ... and with the decode's ordering: a workgroup's stores only after all of its loads
    fns_d = [lambda t=states[i % n_sets]: kda.copy_probe_state(t, t, True) for i in range(max(100, steps))]
    med_d, _, _ = graph_replay_stats_ms(fns_d, warmup)
    nbytes = 2 * n * 4
    return dict(ms=med, bytes=nbytes, gbps=nbytes / (med * 1e-3) / 1e9, n_sets=n_sets,
                kernel="kda_copy_probe (nontemporal float4 copy, 8 per thread)",
                torch_copy_ms=med_t, torch_copy_gbps=nbytes / (med_t * 1e-3) / 1e9,
                pattern_ms=med_s, pattern_gbps=nbytes / (med_s * 1e-3) / 1e9,
                pattern_kernel="kda_copy_probe_state (the decode's tiling and lane order, in place, no arithmetic)",
                pattern_spread_us=[round(lo_s * 1e3, 3), round(hi_s * 1e3, 3)],
                dependent_ms=med_d, dependent_gbps=nbytes / (med_d * 1e-3) / 1e9,
                dependent_kernel="kda_copy_probe_state, dependent: the same copy with every store of a workgroup "
                                 "after all of its loads (the decode's ordering)")


def bench_mfma_probe(iters=8000, waves_per_simd=2):
    """The prefill's matrix roof measured: kda_mfma_probe (a loop of bf16 16x16x32 MFMAs over eight
    independent accumulators per wave, waves_per_simd waves on every SIMD), timed with events; the
    median of 5 launches."""
    import statistics
    import torch
    from gated_delta_rule_15_amd import kda
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = cus * waves_per_simd  # 4 waves per workgroup: waves_per_simd waves on each of the 4 SIMDs
    out = torch.empty(blocks * 1024, device="cuda:0")
    kda.mfma_probe(out, blocks, 10)
    times = []
    for _ in range(5):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        flops = kda.mfma_probe(out, blocks, iters)
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    ms = statistics.median(times)
    return dict(ms=ms, flops=flops, tflops=flops / (ms * 1e-3) / 1e12,
                frac_of_peak=flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                kernel="kda_mfma_probe (v_mfma_f32_16x16x32_bf16 loop)", blocks=blocks, iters=iters)


def bench_verify(reps, warmup, n_sets=8, prologue=False):
    import numpy as np
    import torch
    from gated_delta_rule_15_amd import inputs as gen
    from gated_delta_rule_15_amd import kda
    N, G, H = 32, 8, 12
    b = gen.step_batch(seed=4, N=N, G=G, H=H, dtype="bf16", accepted=True, raw=prologue)
    pro = kda.Prologue() if prologue else None
    sets = []
    for i in range(n_sets):
        sets.append(dict(q=to_dev(b.q, "bf16"), k=to_dev(b.k, "bf16"), v=to_dev(b.v, "bf16"), g=to_dev(b.g),
                         beta=to_dev(b.beta), state=to_dev(b.state), acc=to_dev(b.accepted_len),
                         o=torch.empty((N, G, H, D), dtype=torch.bfloat16, device="cuda:0")))
    fns = []
    for i in range(reps):
        s = sets[i % n_sets]
        fns.append(lambda s=s: kda.kda_verify_block(s["q"], s["k"], s["v"], s["g"], s["beta"], s["state"], o=s["o"],
                                                    accepted_len=s["acc"], prologue=pro))
    ms = graph_time_ms(fns, warmup)
    per_head_verify = STATE_BYTES + G * (3 * 2 * D + 4 * D + 4) + G * 2 * D
    per_token_commit = 2 * D + 2 * D + 4 * D + 4
    acc = b.accepted_len.astype(np.int64)
    nbytes = H * (N * per_head_verify + N * 2 * STATE_BYTES + int(acc.sum()) * per_token_commit)
    out = dict(ms=ms, bytes=nbytes, gbps=nbytes / (ms * 1e-3) / 1e9, frac_hbm_peak=nbytes / (ms * 1e-3) / 1e9 /
               HBM_PEAK_GBPS, N=N, G=G, H=H, mean_accepted=float(acc.mean()))
    if not prologue and not EAGER:
        fns100 = [(lambda s=sets[i % n_sets]: kda.kda_verify_block(s["q"], s["k"], s["v"], s["g"], s["beta"],
                                                                   s["state"], o=s["o"], accepted_len=s["acc"]))
                  for i in range(max(100, reps))]
        med, lo, hi = graph_replay_stats_ms(fns100, warmup)
        out.update(median_ms=med, median_gbps=nbytes / (med * 1e-3) / 1e9,
                   median_protocol=f"median over 11 replays of a graph of {len(fns100)} launches "
                                   f"(per-replay means {lo * 1e3:.2f}-{hi * 1e3:.2f} us)")
    return out


def _event_time_ms(run, reps, warmup, groups=3):
    """Mean ms per call of ``reps`` back-to-back calls, timed with events on the current stream after
    ``warmup`` untimed calls; the median over ``groups`` such timed groups (the first calls over large,
    freshly written inputs run slower: 32 x 4096 x 12 prefill 1.41 ms in the first group, 1.27 ms after)."""
    import statistics
    import torch
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    per = []
    for _ in range(groups):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            run()
        end.record()
        end.synchronize()
        per.append(start.elapsed_time(end) / reps)
    return statistics.median(per)


def bench_prefill(reps, warmup):
    """4096 tokens x 12 heads, bf16.  Timed three ways: one kda_prefill call over the
    whole sequence on the single-kernel path, the same call on the split path (a
    workspace: every chunk prepared in one chunk-parallel launch, then the state walk),
    and the segmented driver (automatic segment length: the sequence is cut so that
    (segment, head) units fill the GPU, then composed; its passes take the split path);
    the row's ``ms`` is the fastest."""
    import numpy as np
    import torch
    from gated_delta_rule_15_amd import inputs as gen
    from gated_delta_rule_15_amd import kda
    from gated_delta_rule_15_amd.long_context import (alloc_work, auto_seg_len, auto_seg_len_split,
                                                      kda_prefill_segmented, plan_segments)
    p = gen.packed_batch(seed=3, seqlens=[4096], H=12, dtype="bf16")
    q, k, v = to_dev(p.q, "bf16"), to_dev(p.k, "bf16"), to_dev(p.v, "bf16")
    g, beta, cu = to_dev(p.g), to_dev(p.beta), to_dev(p.cu_seqlens)
    o = torch.empty_like(q)
    S = torch.empty((1, 12, D, D), device="cuda:0")
    cu_h = torch.from_numpy(p.cu_seqlens.copy())
    ms_kernel = _event_time_ms(lambda: kda.kda_prefill(q, k, v, g, beta, cu, cu_h, o=o, final_state=S,
                                                       workspace=None), reps, warmup)
    ws = kda.kda_prefill_workspace(1, 4096, 12, q.dtype, q.device)
    ms_split = _event_time_ms(lambda: kda.kda_prefill(q, k, v, g, beta, cu, cu_h, o=o, final_state=S,
                                                      workspace=ws), reps, warmup)
    seg = auto_seg_len(p.cu_seqlens, 12)
    plan = plan_segments(p.cu_seqlens, seg)
    work = alloc_work(plan, 12, q.device)
    o2 = torch.empty_like(q)
    S2 = torch.empty_like(S)
    ms_seg = _event_time_ms(lambda: kda_prefill_segmented(q, k, v, g, beta, p.cu_seqlens, o=o2, final_state=S2,
                                                          plan=plan, work=work), reps, warmup)
    seg_s = auto_seg_len_split(p.cu_seqlens, 12)
    plan_s = plan_segments(p.cu_seqlens, seg_s)
    work_s = alloc_work(plan_s, 12, q.device, split=True)
    seg_split_call = lambda: kda_prefill_segmented(q, k, v, g, beta, p.cu_seqlens, o=o2, final_state=S2, plan=plan_s,
                                                   work=work_s)
    ms_seg_split = _event_time_ms(seg_split_call, reps, warmup)
    # the same calls replayed from a HIP graph (the driver's launches prebuilt; 100 calls per replay)
    ms_seg_split_graph = None
    if not EAGER:
        ms_seg_split_graph, _, _ = graph_replay_stats_ms([seg_split_call] * 100, warmup)
    del work_s
    # checkpoints every 512 tokens (7 per sequence and head) in the single launch
    C = torch.empty((kda.kda_prefill_checkpoint_count(cu_h, 512), 12, D, D), device="cuda:0")
    ms_ckpt = _event_time_ms(lambda: kda.kda_prefill_checkpointed(q, k, v, g, beta, cu, cu_h, 512, o=o, final_state=S,
                                                                    checkpoints=C), reps, warmup)
    # raw inputs through the in-kernel prologue (q/k normalisation, gate logits), single launch
    pr = gen.packed_batch(seed=3, seqlens=[4096], H=12, dtype="bf16", raw=True)
    qr, kr, gr = to_dev(pr.q, "bf16"), to_dev(pr.k, "bf16"), to_dev(pr.g)
    pro = kda.Prologue()
    ms_pro = _event_time_ms(lambda: kda.kda_prefill(qr, kr, v, gr, beta, cu, cu_h, o=o, final_state=S, prologue=pro,
                                                    workspace=ws), reps, warmup)
    paths = {"single launch": ms_kernel, "split": ms_split, "segmented": ms_seg, "segmented, split passes": ms_seg_split}
    if ms_seg_split_graph is not None:
        paths["segmented, split passes, graph replay"] = ms_seg_split_graph
    path = min(paths, key=paths.get)
    ms = paths[path]
    th = 4096 * 12
    flops = th * FLOP_PER_TOKEN_HEAD_PREFILL
    nbytes = th * BYTES_PER_TOKEN_HEAD_PREFILL_BF16 + 12 * STATE_BYTES
    return dict(ms=ms, tokens_per_s=4096 / (ms * 1e-3), algorithmic_tflops=flops / (ms * 1e-3) / 1e12,
                frac_mfma_peak=flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                gbps=nbytes / (ms * 1e-3) / 1e9, frac_hbm_peak=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                path=path, single_launch_ms=ms_kernel, split_ms=ms_split, segmented_ms=ms_seg,
                segmented_split_passes_ms=ms_seg_split, segmented_split_passes_graph_ms=ms_seg_split_graph,
                segment_len_split_passes=seg_s, segment_len=seg,
                segments=plan.n_rows, single_launch_checkpoints_every_512_ms=ms_ckpt, split_prologue_ms=ms_pro)


def bench_prefill_batch(reps, warmup):
    """32 sequences x 4096 tokens x 12 heads, bf16: 384 (sequence, head) units, the 128-column
    workgroup shape, one launch (the throughput shape of many independent prompts)."""
    import torch
    from gated_delta_rule_15_amd import inputs as gen
    from gated_delta_rule_15_amd import kda
    n, T, H = 32, 4096, 12
    p = gen.packed_batch(seed=3, seqlens=[T] * n, H=H, dtype="bf16")
    q, k, v = to_dev(p.q, "bf16"), to_dev(p.k, "bf16"), to_dev(p.v, "bf16")
    g, beta, cu = to_dev(p.g), to_dev(p.beta), to_dev(p.cu_seqlens)
    o = torch.empty_like(q)
    S = torch.empty((n, H, D, D), device="cuda:0")
    ms = _event_time_ms(lambda: kda.kda_prefill(q, k, v, g, beta, cu, o=o, final_state=S), reps, warmup)
    th = n * T * H
    flops = th * FLOP_PER_TOKEN_HEAD_PREFILL
    nbytes = th * BYTES_PER_TOKEN_HEAD_PREFILL_BF16 + n * H * STATE_BYTES
    return dict(ms=ms, tokens_per_s=n * T / (ms * 1e-3), algorithmic_tflops=flops / (ms * 1e-3) / 1e12,
                frac_mfma_peak=flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                gbps=nbytes / (ms * 1e-3) / 1e9, frac_hbm_peak=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS)


def bench_contract(steps, warmup, n_sets=8):
    """The batch-invariant row contract: decode 64 x 12 (each request at its own position in the
    open 16-token chunk, uniform over 0..15; 8 rotated pool sets; every set takes a multiple of 16
    calls per replay, so each request passes every position equally often), verify + commit of 8
    drafts for 32 x 12 (the plain verify workload; positions drift as commits land; the commit
    copies the rows the verify stashed, and the recomputing commit is timed beside it), and the
    contract prefill of 4096 x 12 and 32 x 4096 x 12 (bf16)."""
    import numpy as np
    import torch
    from gated_delta_rule_15_amd import inputs as gen
    from gated_delta_rule_15_amd import kda
    N, H = 64, 12
    rng = np.random.default_rng(37)
    pos = rng.integers(0, CONTRACT_CHUNK, N)
    lens = [CONTRACT_CHUNK + int(x) + 1 for x in pos]
    p = gen.packed_batch(seed=37, seqlens=lens, H=H, dtype="bf16", init_state=True)
    pre = np.concatenate([np.arange(p.cu_seqlens[n], p.cu_seqlens[n + 1] - 1) for n in range(N)])
    last = p.cu_seqlens[1:] - 1
    cu_pre = np.concatenate([[0], np.cumsum([L - 1 for L in lens])]).astype(np.int32)
    base = kda.kda_contract_pools(N, H, "cuda:0", to_dev(p.initial_state))
    kda.kda_contract_prefill(to_dev(p.q[pre], "bf16"), to_dev(p.k[pre], "bf16"), to_dev(p.v[pre], "bf16"),
                             to_dev(p.g[pre]), to_dev(p.beta[pre]), to_dev(cu_pre), *base, with_output=False)
    tok = dict(q=to_dev(p.q[last], "bf16"), k=to_dev(p.k[last], "bf16"), v=to_dev(p.v[last], "bf16"),
               g=to_dev(p.g[last]), beta=to_dev(p.beta[last]))
    sets = [tuple(x.clone() for x in base) for _ in range(n_sets)]
    outs = [torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda:0") for _ in range(n_sets)]
    calls = max(CONTRACT_CHUNK * n_sets, (steps // (CONTRACT_CHUNK * n_sets)) * CONTRACT_CHUNK * n_sets)
    fns = [lambda i=i: kda.kda_contract_decode(tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"],
                                               *sets[i % n_sets], o=outs[i % n_sets]) for i in range(calls)]
    ms = graph_time_ms(fns, warmup)
    nbytes = N * H * CONTRACT_DECODE_BYTES_PER_HEAD
    dec = dict(ms=ms, bytes=nbytes, gbps=nbytes / (ms * 1e-3) / 1e9,
               frac_hbm_peak=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, N=N, H=H, n_sets=n_sets, calls=calls)
    del sets, outs
    res = {"contract_decode_64x12_bf16": dec}
    for n_seq in (1, 32):
        T = 4096
        pf = gen.packed_batch(seed=3, seqlens=[T] * n_seq, H=H, dtype="bf16")
        q, k, v = to_dev(pf.q, "bf16"), to_dev(pf.k, "bf16"), to_dev(pf.v, "bf16")
        g, beta, cu = to_dev(pf.g), to_dev(pf.beta), to_dev(pf.cu_seqlens)
        o = torch.empty_like(q)
        pools = kda.kda_contract_pools(n_seq, H, "cuda:0")
        # the 12-unit prefill takes the split build, which reads the full chunks' prepared sets from a
        # workspace (kda_contract_prefill_ex); the 384-unit batch takes the unsplit build, which reads none
        cu_h = torch.from_numpy(pf.cu_seqlens.copy())
        ws = kda.kda_contract_prefill_workspace(n_seq * T, H, "cuda:0") if n_seq == 1 else None
        ms = _event_time_ms(lambda: kda.kda_contract_prefill(q, k, v, g, beta, cu, *pools, cu_seqlens_host=cu_h,
                                                             o=o, workspace=ws), 3, 1)
        flops = n_seq * T * H * FLOP_PER_TOKEN_HEAD_CONTRACT
        res[f"contract_prefill_{'' if n_seq == 1 else '32x'}4096x12_bf16"] = dict(
            ms=ms, tokens_per_s=n_seq * T / (ms * 1e-3), fp32_tflops=flops / (ms * 1e-3) / 1e12,
            frac_fp32_valu_peak=flops / (ms * 1e-3) / 1e12 / FP32_VALU_PEAK_TFLOPS, workspace=ws is not None)
        del q, k, v, g, beta, o, pools, ws
    # verify (read-only) + commit of 8 drafts for 32 requests x 12 heads, each request at its own position
    Nv, G = 32, 8
    posv = rng.integers(0, CONTRACT_CHUNK, Nv)
    lensv = [CONTRACT_CHUNK + int(x) for x in posv]
    pv = gen.packed_batch(seed=38, seqlens=[L + G for L in lensv], H=H, dtype="bf16", init_state=True)
    prev = np.concatenate([np.arange(pv.cu_seqlens[n], pv.cu_seqlens[n] + lensv[n]) for n in range(Nv)])
    blk = np.stack([pv.cu_seqlens[n] + lensv[n] + np.arange(G) for n in range(Nv)])
    cu_prev = np.concatenate([[0], np.cumsum(lensv)]).astype(np.int32)
    basev = kda.kda_contract_pools(Nv, H, "cuda:0", to_dev(pv.initial_state))
    kda.kda_contract_prefill(to_dev(pv.q[prev], "bf16"), to_dev(pv.k[prev], "bf16"), to_dev(pv.v[prev], "bf16"),
                             to_dev(pv.g[prev]), to_dev(pv.beta[prev]), to_dev(cu_prev), *basev, with_output=False)
    bq, bk, bv = to_dev(pv.q[blk], "bf16"), to_dev(pv.k[blk], "bf16"), to_dev(pv.v[blk], "bf16")
    bg, bb = to_dev(pv.g[blk]), to_dev(pv.beta[blk])
    acc = to_dev(gen.accepted_lengths(seed=4, N=Nv, G=G))
    vsets = [tuple(x.clone() for x in basev) for _ in range(n_sets)]
    vo = torch.empty((Nv, G, H, D), dtype=torch.bfloat16, device="cuda:0")
    reps = max(16, steps // 4)

    stash = kda.kda_contract_stash(Nv, G, H, "cuda:0")

    def vc(i):  # verify keeping its rows, commit from them
        st = vsets[i % n_sets]
        kda.kda_contract_verify(bq, bk, bv, bg, bb, *st, o=vo, stash=stash)
        kda.kda_contract_commit_stash(stash, acc, *st, G=G)

    def vc_recompute(i):  # verify, then a commit that recomputes the accepted rows
        st = vsets[i % n_sets]
        kda.kda_contract_verify(bq, bk, bv, bg, bb, *st, o=vo)
        kda.kda_contract_commit(bk, bv, bg, bb, acc, *st, q=bq)
    ms_vc = graph_time_ms([lambda i=i: vc(i) for i in range(reps)], warmup)
    ms_rc = graph_time_ms([lambda i=i: vc_recompute(i) for i in range(reps)], warmup)
    res["contract_verify_commit_32x12x8_bf16"] = dict(ms=ms_vc, recomputing_commit_ms=ms_rc, N=Nv, G=G, H=H,
                                                      mean_accepted=float(acc.float().mean()))
    del vsets
    return res


LONG_SUB_SEGMENT = 8192  # each 65,536-token segment of the long sequence runs as 8 fragments


def bench_long(reps, warmup=2, gen_workers=None):
    """1,048,576-token sequence (16 segments of 65,536) + 8 ragged 1K-32K sequences, 12 heads, bf16.

    Each 65,536-token segment is computed as eight 8,192-token fragments, so pass 1
    has 127 x 12 units (each workgroup builds a fragment's state and transition from one
    preparation of its chunks) and pass 2 128 x 12 + 8 x 12 (the scan over the 128
    fragments equals composing each segment from its fragments and then scanning the
    16 segments: the composition is associative).  Measured with separate state and
    transition workgroups in pass 1: 31.4 ms with whole 65,536-token segments, 23.4 ms
    with 32,768-token fragments, 22.4 ms with 8,192 (pass 2 starts its longest rows
    first); with the combined pass-1 workgroups 18.7-19.7 ms at 8,192 (20.3 ms at 4,096,
    19.7 ms at 16,384).  Inputs are drawn by ``gen_workers`` spawned processes (default:
    the host's cores, at most 16); 1 draws them in this process (for runs under a
    profiler)."""
    import torch
    from gated_delta_rule_15_amd import inputs as gen
    from gated_delta_rule_15_amd.long_context import alloc_work, kda_prefill_segmented, plan_segments
    workers = gen_workers or max(1, min(16, len(os.sched_getaffinity(0))))
    t = time.time()
    p = gen.long_context_batch(seed=5, workers=workers)
    log(f"long context: inputs drawn in {time.time() - t:.1f}s (T={p.T})")
    try:
        q, k, v = to_dev(p.q, "bf16"), to_dev(p.k, "bf16"), to_dev(p.v, "bf16")
        g, beta = to_dev(p.g), to_dev(p.beta)
    finally:
        if hasattr(p, "release"):
            p.release()
    init = to_dev(p.initial_state)
    H, T = 12, p.T
    plan = plan_segments(p.cu_seqlens, LONG_SUB_SEGMENT, cut_longer_than=65536)  # the 8 extras stay whole
    work = alloc_work(plan, H, q.device)
    o = torch.empty_like(q)
    fs = torch.empty((len(p.cu_seqlens) - 1, H, D, D), device="cuda:0")
    run = lambda: kda_prefill_segmented(q, k, v, g, beta, p.cu_seqlens, initial_state=init, o=o, final_state=fs,
                                        plan=plan, work=work)
    ms = _event_time_ms(run, reps, warmup)
    th = T * H
    flops = th * FLOP_PER_TOKEN_HEAD_PREFILL
    nbytes = th * BYTES_PER_TOKEN_HEAD_PREFILL_BF16
    return dict(ms=ms, tokens=T, segments_long=16, fragments_long=len(plan.row_of_seq[0]),
                fragment_len=LONG_SUB_SEGMENT, tokens_per_s=T / (ms * 1e-3),
                algorithmic_tflops=flops / (ms * 1e-3) / 1e12,
                frac_mfma_peak=flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                gbps=nbytes / (ms * 1e-3) / 1e9, frac_hbm_peak=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS)


# ---------------------------------------------------------------------------
def _oracle_decode_worker(args):
    seed, lo, hi, rounds = args
    import numpy as np
    from gated_delta_rule_15_amd import inputs as gen
    from oracle import kda_oracle as orc
    b = gen.step_batch(seed=seed, N=64, G=1, H=12, dtype="bf16")
    q, k, v, g, beta, S = b.f64("q")[:, 0], b.f64("k")[:, 0], b.f64("v")[:, 0], b.f64("g")[:, 0], \
        b.f64("beta")[:, 0], b.f64("state")
    t0 = time.perf_counter()
    for _ in range(rounds):
        orc.decode_step(q[lo:hi], k[lo:hi], v[lo:hi], g[lo:hi], beta[lo:hi], S[lo:hi])
    return time.perf_counter() - t0


def _oracle_slice_worker(args):
    """Replay tokens [lo, hi) of one (sequence, head) slice of a seeded workload through the oracle's
    token recurrence (from the slice's initial state when it has one); returns the oracle's compute
    time (input generation excluded) and the token count."""
    import numpy as np
    from gated_delta_rule_15_amd import inputs as gen
    from oracle import kda_oracle as orc
    seed, s, h, lo, hi, seq_len, dtype, with_state = args
    S = gen.draw_state(seed, s, h, D, D).astype(np.float64) if with_state else None
    spent = 0.0
    for b0 in range(lo - lo % gen.BLOCK, hi, gen.BLOCK):
        n = min(gen.BLOCK, seq_len - b0)  # the block's own length: its stream depends on it
        q, k, v, beta, g = gen._draw_block(seed, s, h, b0 // gen.BLOCK, n, D, D)
        a, b = max(lo, b0) - b0, min(hi, b0 + gen.BLOCK) - b0
        q64, k64, v64 = (gen.as_f64(gen._cast(x[a:b], dtype), dtype) for x in (q, k, v))
        g64, beta64 = g[a:b].astype(np.float64), beta[a:b].astype(np.float64)
        t0 = time.perf_counter()
        _, S = orc.recurrence(q64, k64, v64, g64, beta64, S)
        spent += time.perf_counter() - t0
    return spent, hi - lo


def cpu_oracle_prefill_rows(cores):
    """The oracle's prefill on host cores for the three prefill workloads: the tiny fp32 prefill (whole,
    one core), the 4096 x 12 prefill (whole, one worker per head; and its 1-core figure, extrapolated
    from one head), and the long-context workload (a sample of 16 blocks of 4096 tokens spread over the
    long sequence and the extras, extrapolated to all 1,134,121 tokens x 12 heads)."""
    from gated_delta_rule_15_amd import inputs as gen
    rows = {}
    t, n = _oracle_slice_worker((1, 0, 0, 0, 256, 256, "f32", False))
    rows["tiny_prefill_f32"] = dict(tokens_per_s=n / t, cores=1, kind="oracle", sample="whole workload, 256 tokens x 1 head")
    res = gen.pool_map(_oracle_slice_worker, [(3, 0, h, 0, 4096, 4096, "bf16", False) for h in range(12)], min(cores, 12))
    one = sum(r[0] for r in res)   # the same work on one core
    # heads run in parallel: the slowest head's compute time when every head has a core of its own
    wall = max(r[0] for r in res) if cores >= 12 else one / cores
    rows["prefill_4096x12_bf16"] = dict(tokens_per_s=4096 / wall, cores=min(cores, 12), kind="oracle",
                                        tokens_per_s_1core=4096 / one,
                                        sample="whole workload, one worker per head; 1-core figure = sum of the "
                                               "12 heads' compute times")
    lens = gen.long_context_layout(5)
    T = sum(lens)
    tasks = []
    for i in range(16):  # 12 blocks over the long sequence, 4 over the extras, heads round-robin
        s = 0 if i < 12 else 1 + 2 * (i - 12)
        start = (i * 87_381) // gen.BLOCK * gen.BLOCK if s == 0 else 0
        tasks.append((5, s, i % 12, start, min(start + gen.BLOCK, lens[s]), lens[s], "bf16", s > 0))
    res = gen.pool_map(_oracle_slice_worker, tasks, min(cores, 16))
    th_per_s_core = sum(r[1] for r in res) / sum(r[0] for r in res)  # token-heads per second per core
    rows["long_context_1m_plus_8"] = dict(
        tokens_per_s=th_per_s_core * cores / 12, cores=cores, kind="oracle",
        tokens_per_s_1core=th_per_s_core / 12, projected_total_s=T * 12 / (th_per_s_core * cores),
        sample=f"extrapolated: 16 blocks of <= 4096 tokens (12 over the 1,048,576-token sequence, 4 over the "
               f"extras) at {th_per_s_core:.0f} token-heads/s per core, scaled to {cores} cores (108 independent "
               f"(sequence, head) units) and {T} tokens x 12 heads")
    return rows


def cpu_baseline(target_s=12.0):
    """The oracle's decode step on host cores: all 64 requests x 12 heads, split over workers."""
    from gated_delta_rule_15_amd import inputs as gen
    cores = len(os.sched_getaffinity(0))
    cores = max(1, min(cores, 16))
    # one round of all 64 requests on one core takes t1; a worker holds 64 / cores requests,
    # so `rounds` rounds keep each worker busy for about target_s seconds
    t1 = _oracle_decode_worker((2, 0, 64, 1))
    rounds = max(1, int(round(target_s * cores / max(t1, 1e-3))))
    chunks = [(2, 64 * i // cores, 64 * (i + 1) // cores, rounds) for i in range(cores)]
    times = gen.pool_map(_oracle_decode_worker, chunks, cores)
    wall = max(times)  # the slowest worker's compute time (pool start-up excluded)
    nbytes = rounds * 64 * 12 * decode_bytes_per_head(2)
    return dict(value=nbytes / wall / 1e9, unit="GB/s", cores=cores, kind="oracle",
                sample=f"{rounds} decode steps of 64 requests x 12 heads (fp64 numpy, token by token), "
                       f"requests split over {cores} worker processes; slowest worker {wall:.1f} s")


def traffic_from_profile(kernel_hash):
    path = os.path.join(ROOT, "profiles", "decode_64x12_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_hash:
        return None
    return t.get("bytes_per_launch")


def calibrate_copy(nbytes=256 << 20, reps=20):
    import torch
    src = torch.ones(nbytes // 4, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes_read": nbytes, "bytes_written": nbytes, "launches": reps}))


def write_traffic(prof_dir, out=None):
    """Write profiles/decode_64x12_traffic.json from two rocprofv3 counter passes over the decode
    launches (``dec_FETCH_SIZE``, ``dec_WRITE_SIZE``) and the same passes over the copy calibration
    (``copy_FETCH_SIZE``, ``copy_WRITE_SIZE``), all under ``prof_dir`` (CSV output)."""
    import csv
    import glob
    import statistics

    def counter(pass_name, kernel_key):
        files = glob.glob(os.path.join(prof_dir, pass_name, "*counter_collection.csv"))
        if not files:
            raise SystemExit(f"no counter CSV under {os.path.join(prof_dir, pass_name)}")
        with open(files[0]) as f:
            return [float(r["Counter_Value"]) for r in csv.DictReader(f) if kernel_key in r["Kernel_Name"]]

    dec_f = counter("dec_FETCH_SIZE", "kda_decode_kernel")
    dec_w = counter("dec_WRITE_SIZE", "kda_decode_kernel")
    # the copy run's dispatches: 20 copies and the fill of the source; the median is a copy
    cp_f = statistics.median(counter("copy_FETCH_SIZE", "elementwise"))
    cp_w = statistics.median(counter("copy_WRITE_SIZE", "elementwise"))
    nbytes = 256 << 20
    ff, fw = nbytes / (cp_f * 1024), nbytes / (cp_w * 1024)
    fetch = statistics.mean(dec_f) * 1024 * ff
    write = statistics.mean(dec_w) * 1024 * fw
    alg = 64 * 12 * decode_bytes_per_head(2)
    t = {
        "kernel": "kda_decode_kernel<BF16, false>",
        "workload": "decode step, 64 requests x 12 heads, d_k=d_v=128, fp32 state in place, bf16 q/k/v/o",
        "source_hash": src_hash("kda_step.hip", "kda_common.hpp"),
        "fetch_size_kib_per_dispatch": round(statistics.mean(dec_f), 1),
        "write_size_kib_per_dispatch": round(statistics.mean(dec_w), 1),
        "dispatches": len(dec_f),
        "copy_calibration": {
            "kernel": "torch.mul(src, 1.0, out=dst) over 256 MiB fp32",
            "bytes_read": nbytes, "bytes_written": nbytes,
            "fetch_size_kib": cp_f, "write_size_kib": cp_w,
            "fetch_factor": round(ff, 5), "write_factor": round(fw, 5),
        },
        "fetch_bytes_per_launch": int(round(fetch)),
        "write_bytes_per_launch": int(round(write)),
        "bytes_per_launch": int(round(fetch + write)),
        "algorithmic_bytes_per_launch": alg,
        "ratio_to_algorithmic": round((fetch + write) / alg, 4),
    }
    out = out or os.path.join(ROOT, "profiles", "decode_64x12_traffic.json")
    with open(out, "w") as f:
        json.dump(t, f, indent=2)
        f.write("\n")
    print(json.dumps(t))
    return t


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--long", action="store_true", help="(default) time the 1M-token long-context prefill")
    ap.add_argument("--no-long", action="store_true", help="skip the 1M-token long-context prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-decode", action="store_true", help="time only the decode rows (for profiling)")
    ap.add_argument("--only-prefill", action="store_true",
                    help="time only the prefill rows, 4096 x 12 and 32 x 4096 x 12 (for profiling)")
    ap.add_argument("--only-contract", action="store_true",
                    help="time only the row-contract rows, decode 64 x 12 and prefill (for profiling)")
    ap.add_argument("--only-verify", action="store_true",
                    help="time only verify + commit 32 x 12 x 8 (for profiling)")
    ap.add_argument("--only-long", action="store_true",
                    help="time only the 1M-token long-context prefill (for profiling)")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--write-traffic", metavar="DIR",
                    help="write profiles/decode_64x12_traffic.json from rocprofv3 counter CSVs under DIR")
    ap.add_argument("--eager", action="store_true", help="launch without a HIP graph (counter collection)")
    ap.add_argument("--gen-workers", type=int, default=None,
                    help="processes drawing the long-context inputs (1: in this process, e.g. under a profiler)")
    args = ap.parse_args()
    global EAGER
    EAGER = args.eager
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only (the KDA hot path here is single-GPU; "
              "multi-GPU sharding is design-only). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.write_traffic:
        write_traffic(args.write_traffic)
        return
    from gated_delta_rule_15_amd import _lib
    _lib.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    log("decode: 64 requests x 12 heads ...")
    if args.only_prefill:
        pf = bench_prefill(reps=5, warmup=2)
        pb = bench_prefill_batch(reps=10, warmup=3)
        print(json.dumps({"prefill_4096x12_bf16": pf, "prefill_32x4096x12_bf16": pb}), flush=True)
        return
    if args.only_contract:
        print(json.dumps(bench_contract(args.steps, args.warmup)), flush=True)
        return
    if args.only_verify:
        print(json.dumps({"verify_commit_32x12x8_bf16": bench_verify(reps=max(16, args.steps // 2),
                                                                      warmup=args.warmup)}), flush=True)
        return
    if args.only_long:
        print(json.dumps({"long_context_1m_plus_8": bench_long(reps=2, gen_workers=args.gen_workers)}), flush=True)
        return
    dec = bench_decode(args.steps, args.warmup)
    log(f"decode: {dec['ms'] * 1e3:.2f} us/step, {dec['gbps']:.0f} GB/s")
    rows = {}
    if not args.only_decode:
        log("prefill: 4096 tokens x 12 heads ...")
        pf = bench_prefill(reps=max(5, args.steps // 20), warmup=3)
        log(f"prefill: {pf['ms']:.3f} ms, {pf['tokens_per_s'] / 1e6:.2f} M tokens/s ({pf['path']}; single launch "
            f"{pf['single_launch_ms']:.3f} ms, split {pf['split_ms']:.3f} ms, segmented x{pf['segments']} "
            f"{pf['segmented_ms']:.3f} ms)")
        rows["prefill_4096x12_bf16"] = pf
        log("prefill: 32 sequences x 4096 tokens x 12 heads ...")
        pb = bench_prefill_batch(reps=max(10, args.steps // 40), warmup=3)
        log(f"prefill batch: {pb['ms']:.3f} ms, {pb['tokens_per_s'] / 1e6:.1f} M tokens/s")
        rows["prefill_32x4096x12_bf16"] = pb
        log("verify+commit: 32 requests x 12 heads x 8 drafts ...")
        vf = bench_verify(reps=max(16, args.steps // 2), warmup=args.warmup)
        log(f"verify+commit: {vf['ms'] * 1e3:.2f} us, {vf['gbps']:.0f} GB/s")
        rows["verify_commit_32x12x8_bf16"] = vf
        log("prologue (raw q/k, gate logits): decode 64 x 12, verify+commit 32 x 12 x 8 ...")
        dp = bench_decode(max(40, args.steps // 4), args.warmup, prologue=True)
        vp = bench_verify(reps=max(16, args.steps // 2), warmup=args.warmup, prologue=True)
        log(f"prologue: decode {dp['ms'] * 1e3:.2f} us ({dp['gbps']:.0f} GB/s), verify+commit {vp['ms'] * 1e3:.2f} us")
        rows["prologue_decode_64x12_bf16"] = dict(ms=dp["ms"], gbps=dp["gbps"])
        rows["prologue_verify_commit_32x12x8_bf16"] = dict(ms=vp["ms"], gbps=vp["gbps"])
        log("row contract: decode 64 x 12, prefill 4096 x 12 and 32 x 4096 x 12 ...")
        ct = bench_contract(max(128, args.steps), args.warmup)
        cd = ct["contract_decode_64x12_bf16"]
        log(f"row contract: decode {cd['ms'] * 1e3:.2f} us ({cd['gbps']:.0f} GB/s), verify+commit "
            f"{ct['contract_verify_commit_32x12x8_bf16']['ms'] * 1e3:.2f} us, prefill "
            f"{ct['contract_prefill_4096x12_bf16']['ms']:.3f} ms, 32 x 4096 x 12 "
            f"{ct['contract_prefill_32x4096x12_bf16']['ms']:.3f} ms")
        rows.update(ct)
        if not args.no_long:
            log("long context: 1,048,576 + 8 ragged sequences x 12 heads ...")
            lc = bench_long(reps=2, gen_workers=args.gen_workers)
            log(f"long context: {lc['ms']:.2f} ms, {lc['tokens_per_s'] / 1e6:.1f} M tokens/s")
            rows["long_context_1m_plus_8"] = lc

    if not args.only_decode and not EAGER:
        mf = bench_mfma_probe()
        log(f"mfma probe (bf16 16x16x32 loop): {mf['tflops']:.0f} TFLOP/s ({100 * mf['frac_of_peak']:.1f} % of "
            f"{BF16_MFMA_PEAK_TFLOPS:.0f})")
        rows["mfma_probe"] = mf
        for key in ("prefill_4096x12_bf16", "prefill_32x4096x12_bf16", "long_context_1m_plus_8"):
            if key in rows and "algorithmic_tflops" in rows[key]:
                rows[key]["frac_of_measured_mfma"] = rows[key]["algorithmic_tflops"] / mf["tflops"]
    khash = src_hash("kda_step.hip", "kda_common.hpp")
    traffic = traffic_from_profile(khash)
    copy = None
    if not EAGER:
        copy = bench_copy_probe(args.steps, args.warmup)
        log(f"copy probe (same footprint): {copy['ms'] * 1e3:.2f} us, {copy['gbps']:.0f} GB/s "
            f"(torch copy_ {copy['torch_copy_ms'] * 1e3:.2f} us); in the decode's pattern "
            f"{copy['pattern_ms'] * 1e3:.2f} us, {copy['pattern_gbps']:.0f} GB/s; with its ordering "
            f"{copy['dependent_ms'] * 1e3:.2f} us, {copy['dependent_gbps']:.0f} GB/s")
    roof = dict(bound="hbm", achieved=round(dec["gbps"], 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                frac=round(dec["gbps"] / HBM_PEAK_GBPS, 4), traffic=traffic,
                kernel="kda_decode_kernel<BF16, false>", algorithmic_bytes_per_launch=dec["bytes"],
                mean_launch_us=round(dec["ms"] * 1e3, 3),
                median_launch_us=round(dec["median_ms"] * 1e3, 3) if "median_ms" in dec else None,
                measured_copy_gbps=round(copy["gbps"], 1) if copy else None,
                measured_copy_kernel=copy["kernel"] if copy else None,
                frac_of_measured_copy=round(dec["gbps"] / copy["gbps"], 4) if copy else None,
                measured_pattern_copy_gbps=round(copy["pattern_gbps"], 1) if copy else None,
                measured_pattern_copy_kernel=copy["pattern_kernel"] if copy else None,
                # medians over the same replay protocol on both sides
                median_frac_of_pattern_copy=(round(dec["median_gbps"] / copy["pattern_gbps"], 4)
                                             if copy and "median_gbps" in dec else None),
                measured_ordered_copy_gbps=round(copy["dependent_gbps"], 1) if copy else None,
                measured_ordered_copy_kernel=copy["dependent_kernel"] if copy else None,
                median_frac_of_ordered_copy=(round(dec["median_gbps"] / copy["dependent_gbps"], 4)
                                             if copy and "median_gbps" in dec else None))
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline()
        log(f"cpu baseline: {cpu['value']:.4f} GB/s on {cpu['cores']} cores")
        if not args.only_decode:
            rows["cpu_oracle_prefill"] = cpu_oracle_prefill_rows(cpu["cores"])
            log("cpu oracle prefill: " + ", ".join(f"{k} {v['tokens_per_s']:.0f} tokens/s"
                                                   for k, v in rows["cpu_oracle_prefill"].items()))

    line = {
        "metric": "KDA prefill tokens/s and decode state-update HBM GB/s (12 heads, 1 GPU)",
        "value": round(dec["gbps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode step, 64 requests x 12 heads, d_k=d_v=128, fp32 state in place, "
                               "bf16 q/k/v/o, 8 rotated state sets",
                   "requests": 64, "heads": 12, "d": 128, "state_sets": dec["n_sets"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
