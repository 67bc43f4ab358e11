"""GPU parity of the in-kernel input prologue (unnormalised q, k; gate logits) against the CPU
oracle's prologue followed by the recurrence, and its bitwise replay invariants."""
import numpy as np
import pytest
import torch

from gated_delta_rule_15_amd import inputs as gen
from oracle import kda_oracle as orc
from oracle import kda_prologue as pro

from kda_testutil import check_parity, packed_slices, packed_to_dev, rel_l2, steps_to_dev, to_f64, unit_slices

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}
VARIANTS = [(True, True), (True, False), (False, True)]  # (l2norm_qk, gate_logits)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _prologue(l2, gate):
    from gated_delta_rule_15_amd.kda import Prologue
    return Prologue(l2norm_qk=l2, l2norm_eps=1e-6, gate_logits=gate, g_min=-5.0)


def _ref_inputs(q, k, g, l2, gate):
    return pro.apply_prologue(q, k, g, l2norm=l2, eps=1e-6, gate_logits=gate, g_min=-5.0)


def _valid_inputs(batch, l2, gate):
    """What the prologue does not do, the caller does: without the gate map the g input must already
    be a log-decay (<= 0), so the raw logits are mapped on the host in fp32; without the normalisation
    q and k must already be unit vectors (raw keys of norm ~11 make the recurrence blow up), so they
    are normalised on the host in fp32 and cast back, as the standard workloads are."""
    if not gate:
        x = batch.g.astype(np.float32)
        batch.g = (np.float32(-5.0) / (np.float32(1.0) + np.exp(-x))).astype(np.float32)
    if not l2:
        for name in ("q", "k"):
            x = getattr(batch, name)
            f = gen.bf16_bits_to_f32(x) if batch.dtype == "bf16" else x.astype(np.float32)
            f = f / np.sqrt(np.sum(f * f, axis=-1, keepdims=True, dtype=np.float32))
            setattr(batch, name, gen.f32_to_bf16_bits(f) if batch.dtype == "bf16" else f.astype(np.float32))
    return batch


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("l2,gate", VARIANTS)
def test_decode_prologue_matches_oracle(dtype, l2, gate):
    from gated_delta_rule_15_amd.kda import kda_decode_step
    b = _valid_inputs(gen.step_batch(seed=61, N=24, G=1, H=6, dtype=dtype, raw=True), l2, gate)
    d = steps_to_dev(b, squeeze_g=True)
    o = kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], scale=0.8,
                        prologue=_prologue(l2, gate))
    torch.cuda.synchronize()
    q, k, g = _ref_inputs(b.f64("q")[:, 0], b.f64("k")[:, 0], b.f64("g")[:, 0], l2, gate)
    o_ref, S_ref = orc.decode_step(q, k, b.f64("v")[:, 0], g, b.f64("beta")[:, 0], b.f64("state"), 0.8)
    tag = f"decode prologue {dtype} l2={l2} gate={gate}"
    check_parity(o, o_ref, TOL[dtype], unit_slices(24, 6), bf16_out=dtype == "bf16", tag=f"{tag} o")
    check_parity(d["state"], S_ref, TOL[dtype], unit_slices(24, 6), tag=f"{tag} S")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("l2,gate", VARIANTS)
def test_verify_commit_prologue_matches_oracle(dtype, l2, gate):
    from gated_delta_rule_15_amd.kda import kda_verify_block
    b = _valid_inputs(gen.step_batch(seed=62, N=12, G=8, H=5, dtype=dtype, accepted=True, raw=True), l2, gate)
    d = steps_to_dev(b)
    o = kda_verify_block(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], accepted_len=d["accepted_len"],
                         scale=0.8, prologue=_prologue(l2, gate))
    torch.cuda.synchronize()
    q, k, g = _ref_inputs(b.f64("q"), b.f64("k"), b.f64("g"), l2, gate)
    o_ref, S_ref = orc.verify_block(q, k, b.f64("v"), g, b.f64("beta"), b.f64("state"), b.accepted_len, 0.8)
    tag = f"verify+commit prologue {dtype} l2={l2} gate={gate}"
    check_parity(o, o_ref, TOL[dtype], unit_slices(12, 5, steps=True), bf16_out=dtype == "bf16", tag=f"{tag} o")
    check_parity(d["state"], S_ref, TOL[dtype], unit_slices(12, 5), tag=f"{tag} S")


@pytest.mark.parametrize("N,H", [(6, 3), (32, 12)])
def test_prologue_verify_and_commit_bitwise_equal_decode_steps(N, H):
    """With the prologue, verify's o_t equals the t-th decode step's o and commit(L) equals L decode
    steps, bit for bit (the norms and gates are formed by the same arithmetic on every path)."""
    from gated_delta_rule_15_amd.kda import kda_decode_step, kda_verify_block, kda_verify_commit
    G = 8
    p = _prologue(True, True)
    b = gen.step_batch(seed=63, N=N, G=G, H=H, dtype="bf16", accepted=True, raw=True)
    d = steps_to_dev(b)
    o_ver = kda_verify_block(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], scale=0.8, prologue=p)
    committed = d["state"].clone()
    kda_verify_commit(d["k"], d["v"], d["g"], d["beta"], committed, d["accepted_len"], prologue=p)
    S = d["state"].clone()
    S_at_L = torch.empty_like(S)
    for t in range(G):
        o_t = kda_decode_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(), d["v"][:, t].contiguous(),
                              d["g"][:, t].contiguous(), d["beta"][:, t].contiguous(), S, scale=0.8, prologue=p)
        assert torch.equal(o_t.view(torch.int16), o_ver[:, t].contiguous().view(torch.int16)), f"step {t}"
        for n in range(N):
            if b.accepted_len[n] == t + 1:
                S_at_L[n] = S[n]
    torch.cuda.synchronize()
    assert torch.equal(committed.view(torch.int32), S_at_L.view(torch.int32))


def test_prologue_on_prenormalised_inputs_is_close_to_plain():
    """Inputs that are already unit vectors (the standard workloads) pass the normalisation almost
    unchanged: the prologue decode agrees with the plain decode to fp32 rounding of the norm."""
    from gated_delta_rule_15_amd.kda import kda_decode_step
    b = gen.step_batch(seed=64, N=16, G=1, H=4, dtype="f32")
    d1 = steps_to_dev(b, squeeze_g=True)
    d2 = steps_to_dev(b, squeeze_g=True)
    o1 = kda_decode_step(d1["q"], d1["k"], d1["v"], d1["g"], d1["beta"], d1["state"])
    o2 = kda_decode_step(d2["q"], d2["k"], d2["v"], d2["g"], d2["beta"], d2["state"],
                         prologue=_prologue(True, False))
    torch.cuda.synchronize()
    assert rel_l2(to_f64(o2), to_f64(o1)) <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("l2,gate", VARIANTS)
def test_prefill_prologue_matches_oracle(dtype, l2, gate):
    """Ragged packed batch with initial states (64-column workgroups), raw inputs."""
    from gated_delta_rule_15_amd.kda import kda_prefill
    p = _valid_inputs(gen.packed_batch(seed=65, seqlens=[70, 130, 1, 64, 0, 200], H=3, dtype=dtype,
                                       init_state=True, raw=True), l2, gate)
    d = packed_to_dev(p)
    o, S = kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["cu_seqlens_host"],
                       initial_state=d["initial_state"], scale=0.8, prologue=_prologue(l2, gate))
    torch.cuda.synchronize()
    q, k, g = _ref_inputs(p.f64("q"), p.f64("k"), p.f64("g"), l2, gate)
    o_ref, S_ref = orc.prefill(q, k, p.f64("v"), g, p.f64("beta"), p.cu_seqlens, p.initial_state, 0.8)
    tag = f"prefill prologue {dtype} l2={l2} gate={gate}"
    check_parity(o, o_ref, TOL[dtype], packed_slices(p.cu_seqlens, 3), bf16_out=dtype == "bf16", tag=f"{tag} o")
    check_parity(S, S_ref, TOL[dtype], unit_slices(p.num_seqs, 3), tag=f"{tag} S")


def test_prefill_prologue_wide_and_transitions():
    """More units than half the CUs (128-column workgroups) with transitions: M of the normalised
    keys and mapped gates, so that final = M S0 + S~."""
    from gated_delta_rule_15_amd.kda import kda_prefill
    lens = [1 + (41 * i) % 120 for i in range(34)]
    p = gen.packed_batch(seed=66, seqlens=lens, H=8, dtype="bf16", init_state=True, raw=True)
    d = packed_to_dev(p)
    N, H = len(lens), 8
    M = torch.empty((N, H, 128, 128), device="cuda:0")
    o, S = kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["cu_seqlens_host"],
                       initial_state=d["initial_state"], transition_out=M, prologue=_prologue(True, True))
    torch.cuda.synchronize()
    q, k, g = _ref_inputs(p.f64("q"), p.f64("k"), p.f64("g"), True, True)
    o_ref, S_ref = orc.prefill(q, k, p.f64("v"), g, p.f64("beta"), p.cu_seqlens, p.initial_state)
    cu = p.cu_seqlens
    check_parity(o, o_ref, 2e-3, packed_slices(cu, H), bf16_out=True, tag="prefill prologue wide o")
    check_parity(S, S_ref, 2e-3, unit_slices(N, H), tag="prefill prologue wide S")
    M_ref = np.stack([np.stack([orc.transition(k[cu[n]:cu[n + 1], h], g[cu[n]:cu[n + 1], h],
                                               p.f64("beta")[cu[n]:cu[n + 1], h]) for h in range(H)])
                      for n in range(0, N, 5)])
    check_parity(to_f64(M)[::5], M_ref, 2e-3, unit_slices(M_ref.shape[0], H), tag="prefill prologue wide M")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("l2,gate", VARIANTS)
def test_record_verify_and_commit(dtype, l2, gate):
    """The raw-input record (ReplaySSM): the recording verify gives the prologue verify's outputs bit for
    bit; the record holds each step's key and log-decay as the prologue made them (against the oracle's
    prologue at fp32 rounding); the commit that folds the record writes the prologue commit's state bit
    for bit, and it matches the oracle."""
    from gated_delta_rule_15_amd.kda import (kda_verify_block, kda_verify_block_record, kda_verify_commit,
                                             kda_verify_commit_record)
    N, G, H = 10, 8, 3
    b = _valid_inputs(gen.step_batch(seed=65, N=N, G=G, H=H, dtype=dtype, accepted=True, raw=True), l2, gate)
    d = steps_to_dev(b)
    p = _prologue(l2, gate)
    o_ref_gpu = kda_verify_block(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], scale=0.8, prologue=p)
    o_rec, rec = kda_verify_block_record(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], prologue=p,
                                         scale=0.8)
    bits = torch.int16 if dtype == "bf16" else torch.int32
    torch.cuda.synchronize()
    assert torch.equal(o_rec.view(bits), o_ref_gpu.view(bits))
    q_ref, k_ref, g_ref = _ref_inputs(b.f64("q"), b.f64("k"), b.f64("g"), l2, gate)
    # the record's key and log-decay against the oracle's prologue (fp32 arithmetic on the device)
    check_parity(rec[:, :, :, 0], k_ref, 1e-6, unit_slices(N, H, steps=True), tag=f"record k {dtype}")
    check_parity(rec[:, :, :, 1], g_ref, 1e-6, unit_slices(N, H, steps=True), tag=f"record g {dtype}")
    # the commit from the record equals the recomputing prologue commit, bit for bit
    S_pro = d["state"].clone()
    kda_verify_commit(d["k"], d["v"], d["g"], d["beta"], S_pro, d["accepted_len"], prologue=p)
    S_rec = d["state"].clone()
    kda_verify_commit_record(rec, d["v"], d["beta"], S_rec, d["accepted_len"])
    torch.cuda.synchronize()
    assert torch.equal(S_rec.view(torch.int32), S_pro.view(torch.int32))
    _, S_ref = orc.verify_block(q_ref, k_ref, b.f64("v"), g_ref, b.f64("beta"), b.f64("state"), b.accepted_len, 0.8)
    check_parity(S_rec, S_ref, TOL[dtype], unit_slices(N, H), tag=f"record commit {dtype} l2={l2} gate={gate} S")


@pytest.mark.parametrize("lens", [[1500, 777, 64], [1500, 777]], ids=["mixed", "all_cut"])
@pytest.mark.parametrize("split", [False, True])
def test_segmented_prefill_with_prologue(split, lens):
    """The segmented driver on raw inputs: both passes apply the prologue (single-kernel passes, or split
    passes sharing one preparation), and the result matches the oracle's prologue then recurrence."""
    from gated_delta_rule_15_amd.long_context import alloc_work, kda_prefill_segmented, plan_segments
    p = gen.packed_batch(seed=67, seqlens=lens, H=2, dtype="bf16", init_state=[False] + [True] * (len(lens) - 1),
                         raw=True)
    d = packed_to_dev(p)
    plan = plan_segments(p.cu_seqlens, 256)
    work = alloc_work(plan, 2, d["q"].device, d["q"].dtype, split=split)
    assert (work["ws"] is not None) == split
    o, S = kda_prefill_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], p.cu_seqlens, plan=plan, work=work,
                                 initial_state=d["initial_state"], scale=0.8, prologue=_prologue(True, True))
    torch.cuda.synchronize()
    q, k, g = _ref_inputs(p.f64("q"), p.f64("k"), p.f64("g"), True, True)
    o_ref, S_ref = orc.prefill(q, k, p.f64("v"), g, p.f64("beta"), p.cu_seqlens, p.initial_state, 0.8)
    tag = f"segmented prologue split={split} {len(lens)} seqs"
    check_parity(o, o_ref, TOL["bf16"], packed_slices(p.cu_seqlens, 2), bf16_out=True, tag=f"{tag} o")
    check_parity(S, S_ref, TOL["bf16"], unit_slices(len(lens), 2), tag=f"{tag} S")
