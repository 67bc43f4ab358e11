"""GPU parity: chunked prefill, transitions and segment composition against the CPU oracle."""
import numpy as np
import pytest
import torch

from gated_delta_rule_15_amd import inputs as gen
from oracle import kda_oracle as orc

from kda_testutil import check_parity, packed_slices, packed_to_dev, rel_l2, to_dev, to_f64, unit_slices

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(p: gen.Packed, **kw):
    from gated_delta_rule_15_amd.kda import kda_prefill
    d = packed_to_dev(p)
    o, S = kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["cu_seqlens_host"],
                       initial_state=d["initial_state"], **kw)
    torch.cuda.synchronize()
    return o, S, d


def _oracle(p: gen.Packed, scale=1.0):
    return orc.prefill(p.f64("q"), p.f64("k"), p.f64("v"), p.f64("g"), p.f64("beta"), p.cu_seqlens,
                       p.initial_state, scale)


def _check(p, o, S, tag, scale=1.0):
    """Outputs per (sequence, head) slice and per element, final states per (sequence, head)."""
    o_ref, S_ref = _oracle(p, scale)
    eo = check_parity(o, o_ref, TOL[p.dtype], packed_slices(p.cu_seqlens, p.H), bf16_out=p.dtype == "bf16",
                      tag=f"{tag} o") if o_ref.size else 0.0
    es = check_parity(S, S_ref, TOL[p.dtype], unit_slices(p.num_seqs, p.H), tag=f"{tag} S")
    return eo, es


def _check_transitions(p, M, tag):
    M_ref = np.empty((p.num_seqs, p.H, 128, 128))
    for n in range(p.num_seqs):
        a, b = p.cu_seqlens[n], p.cu_seqlens[n + 1]
        for h in range(p.H):
            M_ref[n, h] = orc.transition(p.f64("k")[a:b, h], p.f64("g")[a:b, h], p.f64("beta")[a:b, h])
    return check_parity(M, M_ref, TOL[p.dtype], unit_slices(p.num_seqs, p.H), tag=f"{tag} M")


def test_tiny_prefill_fp32():
    """1 head, T = 256, fp32 throughout, zero initial state (tolerance 1e-5)."""
    p = gen.packed_batch(seed=1, seqlens=[256], H=1, dtype="f32")
    o, S, _ = _run(p)
    _check(p, o, S, "tiny fp32 T=256")


def test_prefill_4096x12_bf16():
    """One sequence of 4096 tokens, 12 heads, bf16 q/k/v, zero initial state."""
    p = gen.packed_batch(seed=3, seqlens=[4096], H=12, dtype="bf16")
    o, S, _ = _run(p)
    _check(p, o, S, "prefill 4096x12 bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 130])
def test_prefill_ragged_lengths_nonzero_state(T, dtype):
    p = gen.packed_batch(seed=100 + T, seqlens=[T], H=2, dtype=dtype, init_state=True)
    o, S, _ = _run(p)
    _check(p, o, S, f"T={T} {dtype} S0!=0")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_packed_batch_with_empty_sequence(dtype):
    p = gen.packed_batch(seed=7, seqlens=[5, 0, 64, 100, 1, 200], H=3, dtype=dtype,
                         init_state=[True, True, False, True, True, False])
    o, S, _ = _run(p)
    _check(p, o, S, f"packed batch {dtype}")


def test_prefill_wide_slices_many_sequences():
    """More (sequence, head) pairs than half the CUs select 128-column workgroups."""
    lens = [1 + (37 * i) % 150 for i in range(32)]
    p = gen.packed_batch(seed=8, seqlens=lens, H=8, dtype="bf16", init_state=True)
    o, S, _ = _run(p)
    _check(p, o, S, "32 seqs x 8 heads (wide)")


def test_prefill_scale_and_in_place_state():
    from gated_delta_rule_15_amd.kda import kda_prefill
    p = gen.packed_batch(seed=9, seqlens=[77, 150], H=2, dtype="f32", init_state=True)
    d = packed_to_dev(p)
    st = d["initial_state"]
    o, S = kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], initial_state=st,
                       final_state=st, scale=0.5)
    torch.cuda.synchronize()
    assert S.data_ptr() == st.data_ptr()
    _check(p, o, S, "in-place state, scale 0.5", scale=0.5)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_transition_output(dtype):
    """M = M_T ... M_1 per sequence, so that final = M S0 + S~."""
    p = gen.packed_batch(seed=10, seqlens=[100, 64, 3], H=2, dtype=dtype, init_state=True)
    M = torch.empty((3, 2, 128, 128), device="cuda:0")
    o, S, _ = _run(p, transition_out=M)
    _check(p, o, S, f"with transition {dtype}")
    _check_transitions(p, M, f"transition {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gate", ["uniform", "bound"])
def test_prefill_strong_decay(dtype, gate):
    """Gates down to the lower bound on log-decay (-5): log alpha ~ U(-5, 0), or -5 everywhere.
    A 32-token chunk then decays by up to e^-160, beyond fp32 range for a chunk-start reference."""
    p = gen.packed_batch(seed=13, seqlens=[300, 77, 32, 5], H=2, dtype=dtype, init_state=True)
    if gate == "uniform":
        p.g *= np.float32(50.0)
    else:
        p.g[:] = np.float32(-5.0)
    M = torch.empty((4, 2, 128, 128), device="cuda:0")
    o, S, _ = _run(p, transition_out=M)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all() and torch.isfinite(M).all()
    _check(p, o, S, f"strong decay ({gate}) {dtype}")
    _check_transitions(p, M, f"strong decay ({gate}) {dtype}")


@pytest.mark.parametrize("dtype,lens,H,interval,init", [
    ("bf16", [300, 64, 65, 0, 1, 200], 3, 64, True),
    ("f32", [300, 64, 65, 0, 1, 200], 3, 64, False),
    ("bf16", [1000, 129, 128], 2, 128, True),
    ("bf16", [1 + (37 * i) % 300 for i in range(32)], 8, 64, True),   # 256 units: 128-column workgroups
])
def test_prefill_checkpoints(dtype, lens, H, interval, init):
    """States after every `interval` tokens of each sequence, against the oracle's chained recurrence."""
    from gated_delta_rule_15_amd.kda import kda_prefill_checkpoint_count, kda_prefill_checkpointed
    p = gen.packed_batch(seed=14, seqlens=lens, H=H, dtype=dtype, init_state=init)
    d = packed_to_dev(p)
    n = kda_prefill_checkpoint_count(d["cu_seqlens_host"], interval)
    assert n == sum((L - 1) // interval if L else 0 for L in lens)
    o, S, C = kda_prefill_checkpointed(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                       d["cu_seqlens_host"], interval, initial_state=d["initial_state"])
    torch.cuda.synchronize()
    _check(p, o, S, f"checkpointed prefill {dtype}")
    C_ref = orc.prefill_checkpoints(p.f64("k"), p.f64("v"), p.f64("g"), p.f64("beta"), p.cu_seqlens, interval,
                                    p.initial_state)
    assert C.shape[0] == C_ref.shape[0] == n
    check_parity(C, C_ref, TOL[dtype], unit_slices(n, H), tag=f"checkpoints {dtype} x{n}")


def test_compose_matches_oracle():
    from gated_delta_rule_15_amd.kda import kda_compose_segments
    rng = np.random.default_rng(5)
    n, H = 5, 3
    M = (rng.standard_normal((n, H, 128, 128)) / np.sqrt(128)).astype(np.float32)
    St = rng.standard_normal((n, H, 128, 128)).astype(np.float32)
    S0 = rng.standard_normal((H, 128, 128)).astype(np.float32)
    S_in, S_fin = kda_compose_segments(to_dev(M), to_dev(St), to_dev(S0))
    torch.cuda.synchronize()
    for h in range(H):
        ref_in, ref_fin = orc.compose(M[:, h], St[:, h], S0[h])
        check_parity(S_in[:, h], ref_in, 1e-5, [(f"segment {i}", np.s_[i]) for i in range(n)],
                     tag=f"compose head {h} entry states")
        check_parity(S_fin[h], ref_fin, 1e-5, tag=f"compose head {h} final state")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_split_prefill_composes_to_unsplit(dtype):
    """Fragments (M, S~) of 3 segments -> compose -> per-segment outputs equal the unsplit sequence."""
    from gated_delta_rule_15_amd.kda import kda_compose_segments, kda_prefill
    T, H = 3 * 128 + 50, 2
    p = gen.packed_batch(seed=11, seqlens=[T], H=H, dtype=dtype, init_state=True)
    d = packed_to_dev(p)
    seg = torch.tensor([0, 128, 256, T], dtype=torch.int32)
    cu = seg.to("cuda:0")
    M = torch.empty((3, H, 128, 128), device="cuda:0")
    _, St = kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, seg, transition_out=M, with_output=False)
    S_in, S_fin = kda_compose_segments(M, St, d["initial_state"][0])
    o, S_seg = kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, seg, initial_state=S_in)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(p)
    check_parity(o, o_ref, TOL[dtype], packed_slices([0, T], H), bf16_out=dtype == "bf16",
                 tag=f"split+compose {dtype} o")
    check_parity(S_fin, S_ref[0], TOL[dtype], [(f"head {h}", np.s_[h]) for h in range(H)],
                 tag=f"split+compose {dtype} S(compose)")
    check_parity(S_seg[2], S_ref[0], TOL[dtype], [(f"head {h}", np.s_[h]) for h in range(H)],
                 tag=f"split+compose {dtype} S(pass 2)")


def test_prefill_deterministic():
    p = gen.packed_batch(seed=12, seqlens=[300, 20], H=4, dtype="bf16", init_state=True)
    o1, S1, _ = _run(p)
    o2, S2, _ = _run(p)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(S1.view(torch.int32), S2.view(torch.int32))


@pytest.mark.parametrize("H,transitions", [(2, True), (8, False)])
def test_prefill_ordered_equals_natural_order(H, transitions):
    """Starting the sequences in another order changes nothing, bit for bit (narrow and wide grids)."""
    from gated_delta_rule_15_amd.kda import kda_prefill, kda_prefill_ordered
    from gated_delta_rule_15_amd.long_context import longest_first
    lens = [1 + (53 * i) % 200 for i in range(40)]
    p = gen.packed_batch(seed=13, seqlens=lens, H=H, dtype="bf16", init_state=True)
    d = packed_to_dev(p)
    N = len(lens)
    M1 = torch.empty((N, H, 128, 128), device="cuda:0") if transitions else None
    M2 = torch.empty((N, H, 128, 128), device="cuda:0") if transitions else None
    o1, S1 = kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["cu_seqlens_host"],
                         initial_state=d["initial_state"], transition_out=M1)
    for order in (longest_first(p.cu_seqlens), np.random.default_rng(0).permutation(N).astype(np.int32)):
        o2, S2 = kda_prefill_ordered(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                     torch.from_numpy(order).to("cuda:0"), d["cu_seqlens_host"],
                                     initial_state=d["initial_state"], transition_out=M2)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(S1.view(torch.int32), S2.view(torch.int32))
        if transitions:
            assert torch.equal(M1.view(torch.int32), M2.view(torch.int32))
    _check(p, o1, S1, f"{N} seqs x {H} heads")


def test_prefill_all_sequences_empty():
    """No tokens at all: every final state is the initial state, and no output row is written."""
    from gated_delta_rule_15_amd.kda import kda_prefill
    p = gen.packed_batch(seed=14, seqlens=[0, 0, 0], H=2, dtype="bf16", init_state=True)
    d = packed_to_dev(p)
    q = torch.zeros((1, 2, 128), dtype=torch.bfloat16, device="cuda:0")
    g = torch.zeros((1, 2, 128), device="cuda:0")
    beta = torch.zeros((1, 2), device="cuda:0")
    o = torch.full((1, 2, 128), 7.0, dtype=torch.bfloat16, device="cuda:0")
    _, S = kda_prefill(q, q, q, g, beta, d["cu_seqlens"], d["cu_seqlens_host"], initial_state=d["initial_state"],
                       o=o)
    torch.cuda.synchronize()
    assert torch.equal(S, d["initial_state"])
    assert torch.all(o.float() == 7.0)


def test_prefill_long_single_head_bf16():
    """One head, 3,001 tokens (94 chunks, a ragged tail), bf16: the longest chunk walk of the suite."""
    p = gen.packed_batch(seed=15, seqlens=[3001], H=1, dtype="bf16", init_state=True)
    o, S, _ = _run(p)
    _check(p, o, S, "3001 tokens x 1 head")


@pytest.mark.parametrize("prologue", [False, True])
def test_prefill_batch_invariant_across_launch_shapes(prologue):
    """A sequence's outputs, final state and transition are bit-identical whether it runs in a small
    batch (64-column workgroups) or a large one (128-column workgroups): the shapes share one
    association of every reduction (decay prefix, and the prologue's norms)."""
    from gated_delta_rule_15_amd.kda import Prologue, kda_prefill
    lens = [1 + (67 * i) % 180 for i in range(40)]
    H = 8
    pro = Prologue() if prologue else None
    p = gen.packed_batch(seed=16, seqlens=lens, H=H, dtype="bf16", init_state=True, raw=prologue)
    d = packed_to_dev(p)
    o_all, S_all = kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["cu_seqlens_host"],
                               initial_state=d["initial_state"], prologue=pro)      # 320 units: 128-column shape
    n = 10
    cu_sub = d["cu_seqlens"][:n + 1].contiguous()
    o_sub, S_sub = kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_sub, d["cu_seqlens_host"][:n + 1],
                               initial_state=d["initial_state"][:n].contiguous(), prologue=pro)  # 80 units: 64
    M_all = torch.empty((len(lens), H, 128, 128), device="cuda:0")
    M_sub = torch.empty((n, H, 128, 128), device="cuda:0")
    kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["cu_seqlens_host"],
                initial_state=d["initial_state"], transition_out=M_all, prologue=pro)
    kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_sub, d["cu_seqlens_host"][:n + 1],
                initial_state=d["initial_state"][:n].contiguous(), transition_out=M_sub, prologue=pro)
    torch.cuda.synchronize()
    t = int(p.cu_seqlens[n])
    assert torch.equal(o_all[:t].view(torch.int16), o_sub[:t].view(torch.int16))
    assert torch.equal(S_all[:n].view(torch.int32), S_sub.view(torch.int32))
    assert torch.equal(M_all[:n].view(torch.int32), M_sub.view(torch.int32))


@pytest.mark.parametrize("case", range(6))
def test_prefill_random_batches(case):
    """Seeded random batches: head count, ragged lengths with empty sequences, initial states on some
    sequences, input type and scale all vary; outputs and final states against the oracle."""
    rng = np.random.default_rng(900 + case)
    H = int(rng.choice([1, 3, 5, 12]))
    n_seq = int(rng.integers(1, 7))
    lens = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 300, n_seq)]
    if sum(lens) == 0:
        lens[0] = 37
    dtype = "bf16" if case % 2 == 0 else "f32"
    init = [bool(x) for x in rng.random(n_seq) < 0.6]
    scale = float(rng.uniform(0.2, 1.5))
    p = gen.packed_batch(seed=900 + case, seqlens=lens, H=H, dtype=dtype, init_state=init)
    o, S, _ = _run(p, scale=scale)
    _check(p, o, S, f"random batch {case}: H={H} lens={lens} {dtype}", scale=scale)


def _edge_batch(case, dtype, lens=(300, 77, 5, 64), H=2, seed=17):
    """The special cases the KDA math box prints: beta = 1 replaces the value along the key, beta = 0
    keeps the state and only decays it, g = 0 (alpha = 1) is the plain delta rule."""
    p = gen.packed_batch(seed=seed, seqlens=list(lens), H=H, dtype=dtype,
                         init_state=case != "beta0_zero_state")
    if case == "beta1":
        p.beta[:] = np.float32(1.0)
        p.q[:] = p.k  # then o_t = S_t^T k_t = v_t for unit keys
    elif case in ("beta0", "beta0_zero_state"):
        p.beta[:] = np.float32(0.0)
    elif case == "g0":
        p.g[:] = np.float32(0.0)
    return p


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", ["beta1", "beta0", "beta0_zero_state", "g0"])
def test_prefill_edge_gates(case, dtype):
    """beta = 1, beta = 0 (with and without an initial state) and g = 0 on the GPU: against the oracle
    per slice and per element, and against the closed forms these cases have."""
    p = _edge_batch(case, dtype)
    M = torch.empty((p.num_seqs, p.H, 128, 128), device="cuda:0")
    o, S, _ = _run(p, transition_out=M)
    _check(p, o, S, f"edge {case} {dtype}")
    _check_transitions(p, M, f"edge {case} {dtype}")
    o64, S64 = to_f64(o), to_f64(S)
    cu = p.cu_seqlens
    if case == "beta1":
        # S_t^T k_t = (1 - |k|^2) (Diag(alpha) S)^T k_t + |k|^2 v_t: v_t up to the keys' norm error
        v = p.f64("v")
        nk = np.sum(p.f64("k") ** 2, axis=-1, keepdims=True)
        tol = 2e-2 if dtype == "bf16" else 1e-5
        assert np.max(np.abs(nk - 1.0)) < (1e-2 if dtype == "bf16" else 1e-6)
        assert rel_l2(o64, v) <= tol, rel_l2(o64, v)
    elif case.startswith("beta0"):
        # pure channel decay: S_t = Diag(e^{b_t}) S0 and o_t = S_t^T q_t, in closed form
        S0 = np.zeros((p.num_seqs, p.H, 128, 128)) if p.initial_state is None else p.initial_state.astype(np.float64)
        q, g = p.f64("q"), p.f64("g")
        o_cf = np.zeros_like(o64)
        S_cf = np.empty_like(S64)
        for n in range(p.num_seqs):
            a, b = int(cu[n]), int(cu[n + 1])
            for h in range(p.H):
                bcum = np.cumsum(g[a:b, h], axis=0)                         # [t, d_k]
                o_cf[a:b, h] = np.einsum("tk,kv->tv", q[a:b, h] * np.exp(bcum), S0[n, h])
                S_cf[n, h] = np.exp(bcum[-1] if b > a else 0.0)[:, None] * S0[n, h]
        if case == "beta0_zero_state":
            assert torch.count_nonzero(o) == 0 and torch.count_nonzero(S) == 0
        else:
            check_parity(o, o_cf, TOL[dtype], packed_slices(cu, p.H), bf16_out=dtype == "bf16",
                         tag=f"edge {case} {dtype} o vs closed form")
            check_parity(S, S_cf, TOL[dtype], unit_slices(p.num_seqs, p.H), tag=f"edge {case} {dtype} S vs closed form")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("variant", ["plain", "transitions", "prologue", "ordered", "offset"])
def test_split_path_bitwise_equals_fused(dtype, variant):
    """With a workspace, a grid smaller than the device prepares every chunk in one chunk-parallel launch
    and walks the chunks with the state waves alone; outputs, final states and transitions equal the
    single-kernel path's bit for bit (ragged lengths, empty sequences, a batch that starts past token 0,
    the input prologue, a start order).  Against the oracle too."""
    from gated_delta_rule_15_amd.kda import Prologue, kda_prefill, kda_prefill_ordered, kda_prefill_workspace_size
    lens = [300, 0, 33, 64, 1, 129, 31]
    H = 3
    pro = Prologue() if variant == "prologue" else None
    p = gen.packed_batch(seed=18, seqlens=lens, H=H, dtype=dtype, init_state=[True, False] * 3 + [True],
                         raw=variant == "prologue")
    d = packed_to_dev(p)
    cu_d, cu_h = d["cu_seqlens"], d["cu_seqlens_host"]
    if variant == "offset":  # the last five sequences alone: the row set starts at token 300
        cu_d, cu_h = cu_d[2:].contiguous(), cu_h[2:].contiguous()
        init = d["initial_state"][2:].contiguous()
    else:
        init = d["initial_state"]
    N = cu_h.shape[0] - 1
    assert kda_prefill_workspace_size(N, p.T, H, d["q"].dtype, variant == "transitions") > 0
    outs = []
    for ws in (None, "auto"):
        M = torch.full((N, H, 128, 128), 7.0, device="cuda:0") if variant == "transitions" else None
        kw = dict(initial_state=init, transition_out=M, prologue=pro, workspace=ws)
        if variant == "ordered":
            order = torch.tensor(np.random.default_rng(1).permutation(N).astype(np.int32), device="cuda:0")
            kw.pop("prologue")
            o, S = kda_prefill_ordered(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_d, order, cu_h, **kw)
        else:
            o, S = kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_d, cu_h, **kw)
        torch.cuda.synchronize()
        outs.append((o, S, M))
    (o1, S1, M1), (o2, S2, M2) = outs
    t0 = int(cu_h[0])
    assert torch.equal(o1[t0:].view(torch.int32 if dtype == "f32" else torch.int16),
                       o2[t0:].view(torch.int32 if dtype == "f32" else torch.int16))
    assert torch.equal(S1.view(torch.int32), S2.view(torch.int32))
    if M1 is not None:
        assert torch.equal(M1.view(torch.int32), M2.view(torch.int32))
    if variant in ("plain", "transitions"):
        _check(p, o2, S2, f"split path {variant} {dtype}")
        if M2 is not None:
            _check_transitions(p, M2, f"split path {dtype}")


def test_split_path_workspace_errors():
    """A workspace needs the host copy of cu_seqlens and at least the size the library asks for."""
    from gated_delta_rule_15_amd import _lib
    from gated_delta_rule_15_amd.kda import kda_prefill, kda_prefill_workspace_size
    p = gen.packed_batch(seed=19, seqlens=[100, 50], H=2, dtype="bf16")
    d = packed_to_dev(p)
    need = kda_prefill_workspace_size(2, p.T, 2, torch.bfloat16)
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(_lib.KdaError, match="workspace"):
        kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["cu_seqlens_host"], workspace=small)
    with pytest.raises(ValueError, match="cu_seqlens_host"):
        kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], None,
                    workspace=torch.empty(need, dtype=torch.uint8, device="cuda:0"))
    # a grid that fills the device needs none
    assert kda_prefill_workspace_size(256, 4096, 1, torch.bfloat16) == 0
    assert kda_prefill_workspace_size(128, 4096, 1, torch.bfloat16, transitions=True) == 0
    # transitions without outputs walk one workgroup per (sequence, head)
    assert kda_prefill_workspace_size(128, 4096, 1, torch.bfloat16, transitions=True, outputs=False) > 0
    # unknown request flags are invalid arguments
    assert _lib.load().kda_prefill_workspace_size(2, 4096, 1, 128, 128, _lib.KDA_BF16, 4) == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_state_and_transition_build_bitwise(dtype):
    """A call for final states and transitions without outputs on a grid that fills the device (a
    segmented prefill's pass 1) runs one workgroup per (sequence, head) holding both; it equals, bit
    for bit, the same call with outputs (separate state and transition workgroups), and the oracle."""
    from gated_delta_rule_15_amd.kda import kda_prefill
    H = 12
    lens = [int(x) for x in np.random.default_rng(61).integers(1, 200, size=24)]
    lens[3] = 0
    p = gen.packed_batch(seed=61, seqlens=lens, H=H, dtype=dtype, init_state=[i % 3 != 0 for i in range(24)])
    d = packed_to_dev(p)
    N = len(lens)
    M1 = torch.empty((N, H, 128, 128), device="cuda:0")
    M2 = torch.empty_like(M1)
    _, S1 = kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["cu_seqlens_host"],
                        initial_state=d["initial_state"], transition_out=M1, with_output=False, workspace=None)
    o2, S2 = kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["cu_seqlens_host"],
                         initial_state=d["initial_state"], transition_out=M2, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(S1.view(torch.int32), S2.view(torch.int32))
    assert torch.equal(M1.view(torch.int32), M2.view(torch.int32))
    _check(p, o2, S1, f"state+transition build {dtype}")
    _check_transitions(p, M1, f"state+transition build {dtype}")


@pytest.mark.parametrize("n_seg", [1, 2, 5, 17])
def test_compose_split_operands(n_seg):
    """The scan on bf16 MFMA with hi/lo split operands (KDA_COMPOSE_SPLIT_BF16): each product keeps
    about 16 significant bits per operand (hi*hi + hi*lo + lo*hi, the dropped lo*lo and the two
    roundings below 2^-16 relative), so the entry states stay within 5e-5 of the fp64 scan over 17
    steps; results are deterministic and the same for a head whatever the grid (3 heads: one round
    of workgroups; 40 heads: 320 workgroups, more than the CUs)."""
    from gated_delta_rule_15_amd.kda import kda_compose_segments
    rng = np.random.default_rng(70 + n_seg)
    H = 40
    M = (rng.standard_normal((n_seg, H, 128, 128)) / np.sqrt(128)).astype(np.float32)
    St = rng.standard_normal((n_seg, H, 128, 128)).astype(np.float32)
    S0 = rng.standard_normal((H, 128, 128)).astype(np.float32)
    big = kda_compose_segments(to_dev(M), to_dev(St), to_dev(S0), split_bf16=True)
    again = kda_compose_segments(to_dev(M), to_dev(St), to_dev(S0), split_bf16=True)
    few = kda_compose_segments(to_dev(np.ascontiguousarray(M[:, :3])), to_dev(np.ascontiguousarray(St[:, :3])),
                               to_dev(np.ascontiguousarray(S0[:3])), split_bf16=True)
    # zero entry state, no final state requested
    zero_in, no_fin = kda_compose_segments(to_dev(np.ascontiguousarray(M[:, :2])),
                                           to_dev(np.ascontiguousarray(St[:, :2])), None, with_final=False,
                                           split_bf16=True)
    torch.cuda.synchronize()
    assert no_fin is None
    for a, b in zip(big, again):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(big[0][:, :3].contiguous().view(torch.int32), few[0].view(torch.int32))
    assert torch.equal(big[1][:3].contiguous().view(torch.int32), few[1].view(torch.int32))
    for h in (0, 2, 39):
        ref_in, ref_fin = orc.compose(M[:, h], St[:, h], S0[h])
        check_parity(big[0][:, h], ref_in, 5e-5, [(f"segment {i}", np.s_[i]) for i in range(n_seg)],
                     tag=f"split compose, head {h}")
        check_parity(big[1][h], ref_fin, 5e-5, tag=f"split compose, head {h} final")
    for h in range(2):
        ref_in, _ = orc.compose(M[:, h], St[:, h], np.zeros((128, 128), np.float32))
        check_parity(zero_in[:, h], ref_in, 5e-5, [(f"segment {i}", np.s_[i]) for i in range(n_seg)],
                     tag=f"split compose from zeros, head {h}")


@pytest.mark.parametrize("n_seg", [1, 2, 5])
def test_compose_kernels_agree_bitwise(n_seg):
    """A scan over few heads takes the staged kernel (M through LDS), one over many heads the register
    kernel; they use the same contraction order, so the heads both compute come out bit for bit alike,
    and the oracle agrees with both (40 heads: 320 workgroups, more than the CUs of the part)."""
    from gated_delta_rule_15_amd.kda import kda_compose_segments
    rng = np.random.default_rng(50 + n_seg)
    H = 40
    M = (rng.standard_normal((n_seg, H, 128, 128)) / np.sqrt(128)).astype(np.float32)
    St = rng.standard_normal((n_seg, H, 128, 128)).astype(np.float32)
    S0 = rng.standard_normal((H, 128, 128)).astype(np.float32)
    big = kda_compose_segments(to_dev(M), to_dev(St), to_dev(S0))
    few = kda_compose_segments(to_dev(np.ascontiguousarray(M[:, :3])), to_dev(np.ascontiguousarray(St[:, :3])),
                               to_dev(np.ascontiguousarray(S0[:3])))
    torch.cuda.synchronize()
    assert torch.equal(big[0][:, :3].contiguous().view(torch.int32), few[0].view(torch.int32))
    assert torch.equal(big[1][:3].contiguous().view(torch.int32), few[1].view(torch.int32))
    for h in (0, 2, 39):
        ref_in, ref_fin = orc.compose(M[:, h], St[:, h], S0[h])
        check_parity(big[0][:, h], ref_in, 1e-5, [(f"segment {i}", np.s_[i]) for i in range(n_seg)],
                     tag=f"compose 40 heads, head {h}")
        check_parity(big[1][h], ref_fin, 1e-5, tag=f"compose 40 heads, head {h} final")
