"""HIP graph capture and replay of the library's entry points (GPU).

The library allocates nothing and issues no memset or copy: each entry point
is kernel launches on the caller's stream, so a caller may capture it in a
HIP graph.  Each test captures a sequence of calls, then replays the graph
several times; before each replay the states are restored and unrelated eager
work runs with a synchronisation, and every replay must reproduce the eager
run of the same calls bit for bit.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_15_amd import inputs as gen

from kda_testutil import DEV, packed_to_dev, steps_to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    from gated_delta_rule_15_amd import kda  # noqa: F401
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _kda():
    from gated_delta_rule_15_amd import kda
    return kda


def _eager_noise():
    """Unrelated work on the default stream between replays."""
    x = torch.randn(512, 512, device=DEV)
    y = (x @ x).sum()
    torch.cuda.synchronize()
    return float(y)


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(g, reset, outputs, expected, n_out):
    """outputs[:n_out] are pure outputs (poisoned before each replay); the rest
    are states that reset() restores."""
    for _ in range(REPLAYS):
        reset()
        for t in outputs[:n_out]:
            t.fill_(float("nan"))
        _eager_noise()
        g.replay()
        torch.cuda.synchronize()
        for got, ref in zip(outputs, expected):
            assert torch.equal(got, ref)


def test_decode_steps_in_a_graph():
    kda = _kda()
    N, H, T = 8, 4, 3
    b = gen.step_batch(91, N, T, H, dtype="bf16")
    d = steps_to_dev(b)
    toks = [{k: d[k][:, t].contiguous() for k in ("q", "k", "v", "g", "beta")} for t in range(T)]
    state0 = d["state"].clone()
    slots = torch.tensor([5, 0, 7, 2, 1, 6, 3, 4], dtype=torch.int32, device=DEV)
    pool = torch.empty((N, H, 128, 128), dtype=torch.float32, device=DEV)
    outs = [torch.empty((N, H, 128), dtype=torch.bfloat16, device=DEV) for _ in range(T)]

    def run():
        for t in range(T):
            x = toks[t]
            kda.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], pool, o=outs[t], slots=slots, scale=0.8)

    def reset():
        pool.copy_(state0)

    reset()
    run()
    torch.cuda.synchronize()
    expected = [o.clone() for o in outs] + [pool.clone()]
    reset()
    g = _capture(run)
    _replay_and_check(g, reset, outs + [pool], expected, T)


def test_verify_commit_in_a_graph():
    kda = _kda()
    N, G, H = 6, 8, 4
    b = gen.step_batch(92, N, G, H, dtype="bf16", accepted=True)
    d = steps_to_dev(b)
    state0 = d["state"].clone()
    pool = torch.empty_like(state0)
    o = torch.empty((N, G, H, 128), dtype=torch.bfloat16, device=DEV)

    def run():
        kda.kda_verify_block(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, o=o, accepted_len=d["accepted_len"])

    def reset():
        pool.copy_(state0)

    reset()
    run()
    torch.cuda.synchronize()
    expected = [o.clone(), pool.clone()]
    reset()
    g = _capture(run)
    _replay_and_check(g, reset, [o, pool], expected, 1)


def test_prefill_in_a_graph():
    kda = _kda()
    p = gen.packed_batch(93, [70, 1, 130, 0, 64], 4, dtype="bf16", init_state=[True, False, True, False, True])
    d = packed_to_dev(p)
    final = torch.empty_like(d["initial_state"])
    o = torch.empty((p.T, 4, 128), dtype=torch.bfloat16, device=DEV)

    def run():
        kda.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                        cu_seqlens_host=d["cu_seqlens_host"], initial_state=d["initial_state"], final_state=final,
                        o=o, scale=1.1)

    run()
    torch.cuda.synchronize()
    expected = [o.clone(), final.clone()]
    g = _capture(run)
    _replay_and_check(g, lambda: None, [o, final], expected, 2)


def test_segmented_prefill_split_passes_in_a_graph():
    """The segmented driver on split passes (prep build, pass 1, composition, pass 2, with a preallocated
    plan, workspace and outputs) is kernel launches only: replays reproduce the eager call bit for bit."""
    from gated_delta_rule_15_amd.long_context import alloc_work, auto_seg_len_split, kda_prefill_segmented, plan_segments
    H = 4
    p = gen.packed_batch(94, [1024], H, dtype="bf16")
    d = packed_to_dev(p)
    seg = auto_seg_len_split(p.cu_seqlens, H)
    plan = plan_segments(p.cu_seqlens, seg)
    assert plan.n_rows > 1
    work = alloc_work(plan, H, torch.device(DEV), torch.bfloat16, split=True)
    assert work["ws"] is not None
    o = torch.empty((p.T, H, 128), dtype=torch.bfloat16, device=DEV)
    final = torch.empty((1, H, 128, 128), device=DEV)

    def run():
        kda_prefill_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], p.cu_seqlens, o=o, final_state=final,
                              plan=plan, work=work)

    run()
    torch.cuda.synchronize()
    expected = [o.clone(), final.clone()]
    g = _capture(run)
    _replay_and_check(g, lambda: None, [o, final], expected, 2)


def test_contract_prefill_and_decode_in_a_graph():
    kda = _kda()
    N, H = 4, 4
    lens = [21, 16, 3, 40]
    p = gen.packed_batch(94, lens, H, dtype="bf16", init_state=True)
    d = packed_to_dev(p)
    b = gen.step_batch(95, N, 2, H, dtype="bf16")
    db = steps_to_dev(b)
    toks = [{k: db[k][:, t].contiguous() for k in ("q", "k", "v", "g", "beta")} for t in range(2)]
    S, R, P = kda.kda_contract_pools(N, H, DEV)
    S0 = d["initial_state"].clone()
    o = torch.empty((p.T, H, 128), dtype=torch.bfloat16, device=DEV)
    od = [torch.empty((N, H, 128), dtype=torch.bfloat16, device=DEV) for _ in range(2)]

    def run():
        kda.kda_contract_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], S, R, P,
                                 cu_seqlens_host=d["cu_seqlens_host"], o=o)
        for t in range(2):
            x = toks[t]
            kda.kda_contract_decode(x["q"], x["k"], x["v"], x["g"], x["beta"], S, R, P, o=od[t])

    def reset():
        S.copy_(S0)
        R.fill_(0.0)
        P.fill_(0)

    reset()
    run()
    torch.cuda.synchronize()
    expected = [o.clone(), od[0].clone(), od[1].clone(), S.clone(), R.clone(), P.clone()]
    assert np.array_equal(P.cpu().numpy(), np.repeat(np.array([(n + 2) % 16 for n in lens])[:, None], H, 1))
    reset()
    g = _capture(run)
    _replay_and_check(g, reset, [o, od[0], od[1], S, R, P], expected, 3)
