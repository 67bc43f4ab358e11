"""GPU tests at pool sizes past 2^31 elements (the maximum-size edge case).

A state pool of 11,000 slots x 12 heads x 128 x 128 fp32 holds 2.16e9 elements
(8.65 GB), so every slot from 10,923 on starts beyond element 2^31 and every
slot from 5,462 on beyond byte 2^32.  Each kernel is run twice on the same
inputs, once on such a pool with the requests in high slots and once on a
compact pool, and the two must agree bit for bit (the kernels' arithmetic does
not depend on where a state lives); untouched slots must stay untouched.  The
compact results are checked against the oracle as well, so a wrong address
cannot hide behind two equal wrong answers.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_15_amd import inputs as gen
from oracle import kda_contract as cf
from oracle import kda_oracle as orc

from kda_testutil import DEV, check_parity, packed_slices, packed_to_dev, steps_to_dev, to_dev, to_f64, unit_slices

pytestmark = pytest.mark.gpu

P_BIG = 11_000
H = 12
D = 128
SLOTS = [10_999, 0, 10_923, 5_462, 8_191, 10_998]  # past 2^31 elements, first slot, past 2^32 bytes, ...
TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu_with_room():
    from gated_delta_rule_15_amd import kda  # noqa: F401
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    free, _ = torch.cuda.mem_get_info()
    if free < 48 * (1 << 30):
        pytest.skip(f"needs 48 GiB of free device memory, {free / 2**30:.1f} GiB free")
    yield
    torch.cuda.empty_cache()


def _kda():
    from gated_delta_rule_15_amd import kda
    return kda


def _zeros_except(pool: torch.Tensor, slots) -> bool:
    """True when every slot of pool other than `slots` is zero (pool is left zeroed there)."""
    idx = torch.tensor(slots, dtype=torch.long, device=pool.device)
    pool.index_fill_(0, idx, 0.0)
    return int(torch.count_nonzero(pool)) == 0


def test_decode_and_verify_commit_high_slots():
    kda = _kda()
    N = len(SLOTS)
    slots = torch.tensor(SLOTS, dtype=torch.int32, device=DEV)
    idx = slots.long()

    # decode, in place
    b = gen.step_batch(81, N, 1, H, dtype="bf16")
    d = steps_to_dev(b, squeeze_g=True)
    big = torch.zeros((P_BIG, H, D, D), dtype=torch.float32, device=DEV)
    big[idx] = d["state"]
    small = d["state"].clone()
    o_big = kda.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], big, slots=slots, scale=0.9)
    o_small = kda.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], small, scale=0.9)
    torch.cuda.synchronize()
    assert torch.equal(o_big, o_small)
    assert torch.equal(big[idx], small)
    o_ref, S_ref = orc.decode_step(b.f64("q")[:, 0], b.f64("k")[:, 0], b.f64("v")[:, 0], b.f64("g")[:, 0],
                                   b.f64("beta")[:, 0], b.f64("state"), scale=0.9)
    check_parity(o_small, o_ref, TOL, unit_slices(N, H), bf16_out=True, tag="high-slot decode o")
    check_parity(small, S_ref, TOL, unit_slices(N, H), tag="high-slot decode S")
    assert _zeros_except(big, SLOTS)

    # verify of 8 drafts with the commit of the accepted prefix, into the same pool
    G = 8
    bv = gen.step_batch(82, N, G, H, dtype="bf16", accepted=True)
    dv = steps_to_dev(bv)
    big[idx] = dv["state"]
    small = dv["state"].clone()
    ov_big = kda.kda_verify_block(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], big, slots=slots,
                                  accepted_len=dv["accepted_len"])
    ov_small = kda.kda_verify_block(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], small,
                                    accepted_len=dv["accepted_len"])
    torch.cuda.synchronize()
    assert torch.equal(ov_big, ov_small)
    assert torch.equal(big[idx], small)
    for n in range(N):
        L = int(bv.accepted_len[n])
        for h in (0, H - 1):
            _, S_L = orc.recurrence(bv.f64("q")[n, :L, h], bv.f64("k")[n, :L, h], bv.f64("v")[n, :L, h],
                                    bv.f64("g")[n, :L, h], bv.f64("beta")[n, :L, h], bv.f64("state")[n, h])
            check_parity(small[n, h], S_L, TOL, tag=f"high-slot commit request {n} head {h}")
    assert _zeros_except(big, SLOTS)
    del big
    torch.cuda.empty_cache()


def test_prefill_many_sequences_past_2_31():
    """11,000 sequences, all but the last four empty: the last four's initial and
    final states lie beyond element 2^31 of their arrays; the empty ones must
    come out as their initial states."""
    kda = _kda()
    lens = [70, 1, 130, 64]
    n_fill = P_BIG - len(lens)
    p = gen.packed_batch(83, lens, H, dtype="bf16", init_state=True)
    d = packed_to_dev(p)
    cu_big = np.concatenate([np.zeros(n_fill, dtype=np.int32), p.cu_seqlens]).astype(np.int32)
    cu_big_dev = to_dev(cu_big)
    cu_big_host = torch.from_numpy(cu_big.copy())

    init = torch.empty((P_BIG, H, D, D), dtype=torch.float32, device=DEV)
    gen_t = torch.Generator(device=DEV)
    gen_t.manual_seed(84)
    init[:n_fill].normal_(0.0, 0.02, generator=gen_t)
    init[n_fill:] = d["initial_state"]
    final = torch.empty_like(init)
    o_big, _ = kda.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_big_dev, cu_seqlens_host=cu_big_host,
                               initial_state=init, final_state=final)
    o_small, f_small = kda.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                       cu_seqlens_host=d["cu_seqlens_host"], initial_state=d["initial_state"])
    torch.cuda.synchronize()
    assert torch.equal(o_big, o_small)
    assert torch.equal(final[n_fill:], f_small)
    assert torch.equal(final[:n_fill], init[:n_fill])
    o_ref, S_ref = orc.prefill(p.f64("q"), p.f64("k"), p.f64("v"), p.f64("g"), p.f64("beta"), p.cu_seqlens,
                               p.initial_state.astype(np.float64))
    check_parity(o_small, o_ref, TOL, packed_slices(p.cu_seqlens, H), bf16_out=True, tag="high-row prefill o")
    check_parity(f_small, S_ref, TOL, unit_slices(len(lens), H), tag="high-row prefill S")
    del init, final
    torch.cuda.empty_cache()


def test_contract_pools_high_slots():
    """Row contract: a prefill then one decode step for four sequences held in high
    slots of 11,000-slot pools, bit-identical to compact pools, states per oracle."""
    kda = _kda()
    lens = [21, 16, 40, 3]
    slots_l = [10_999, 10_923, 5_462, 10_950]
    slots = torch.tensor(slots_l, dtype=torch.int32, device=DEV)
    idx = slots.long()
    p = gen.packed_batch(85, lens, H, dtype="bf16", init_state=True)
    d = packed_to_dev(p)
    S0 = d["initial_state"]

    S_big, R_big, P_big = kda.kda_contract_pools(P_BIG, H, DEV)
    S_big[idx] = S0
    S_sm, R_sm, P_sm = kda.kda_contract_pools(len(lens), H, DEV, initial_state=S0)
    o_big = kda.kda_contract_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], S_big, R_big,
                                     P_big, cu_seqlens_host=d["cu_seqlens_host"], slots=slots)
    o_sm = kda.kda_contract_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], S_sm, R_sm, P_sm,
                                    cu_seqlens_host=d["cu_seqlens_host"])
    b = gen.step_batch(86, len(lens), 1, H, dtype="bf16")
    db = steps_to_dev(b, squeeze_g=True)
    od_big = kda.kda_contract_decode(db["q"], db["k"], db["v"], db["g"], db["beta"], S_big, R_big, P_big,
                                     slots=slots)
    od_sm = kda.kda_contract_decode(db["q"], db["k"], db["v"], db["g"], db["beta"], S_sm, R_sm, P_sm)
    st_big = kda.kda_contract_state(S_big, R_big, P_big, slots=slots)
    st_sm = kda.kda_contract_state(S_sm, R_sm, P_sm)
    torch.cuda.synchronize()
    assert torch.equal(o_big, o_sm) and torch.equal(od_big, od_sm)
    assert torch.equal(S_big[idx], S_sm) and torch.equal(R_big[idx], R_sm) and torch.equal(P_big[idx], P_sm)
    assert torch.equal(st_big, st_sm)
    # the oracle: the token recurrence over the prefill tokens and the decode token
    for n in range(len(lens)):
        t0, t1 = int(p.cu_seqlens[n]), int(p.cu_seqlens[n + 1])
        for h in (0, H - 1):
            cat = lambda x, y: np.concatenate([x[t0:t1, h], y[n, :, h]])
            o_ref, S_ref = orc.recurrence(cat(p.f64("q"), b.f64("q")), cat(p.f64("k"), b.f64("k")),
                                          cat(p.f64("v"), b.f64("v")), cat(p.f64("g"), b.f64("g")),
                                          np.concatenate([p.f64("beta")[t0:t1, h], b.f64("beta")[n, :, h]]),
                                          p.initial_state[n, h].astype(np.float64))
            got = np.concatenate([to_f64(o_sm[t0:t1, h]), to_f64(od_sm[n:n + 1, h])])
            check_parity(got, o_ref, TOL, bf16_out=True, tag=f"high-slot contract seq {n} head {h} o")
            check_parity(st_sm[n, h], S_ref, TOL, tag=f"high-slot contract seq {n} head {h} S")
            assert int(P_sm[n, h]) == (lens[n] + 1) % cf.CHUNK
    assert _zeros_except(S_big, slots_l) and _zeros_except(R_big, slots_l)
    assert int(torch.count_nonzero(P_big.index_fill_(0, idx, 0))) == 0
    del S_big, R_big, P_big
    torch.cuda.empty_cache()
