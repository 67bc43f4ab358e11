"""GPU tests of the batch-invariant row contract (kda_contract_*).

Parity: outputs, the chunk-entry states, the open rows and the running state
(kda_contract_state) against the fp64 contract oracle and the token recurrence,
relative L2 within 2e-3 for bf16 inputs and 1e-5 for fp32 inputs.
Bit-identity, the contract's purpose: one sequence gives the same output and
state bits whether it runs as one prefill, as a prefill cut anywhere followed
by decode steps and more prefill, alone or inside a batch.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_15_amd import inputs as gen
from oracle import kda_contract as cf
from oracle import kda_oracle as orc

from kda_testutil import DEV, check_parity, packed_slices, rel_l2, to_dev, to_f64, unit_slices

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    from gated_delta_rule_15_amd import kda  # noqa: F401
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _kda():
    from gated_delta_rule_15_amd import kda
    return kda


def _slice(p: gen.Packed, ranges):
    """Device tensors of the token ranges [a_n, b_n) of each sequence of p, packed."""
    idx, cu = [], [0]
    for n, (a, b) in enumerate(ranges):
        s0 = int(p.cu_seqlens[n])
        idx.extend(range(s0 + a, s0 + b))
        cu.append(cu[-1] + (b - a))
    idx = np.asarray(idx, dtype=np.int64)
    pick = lambda x: np.ascontiguousarray(x[idx])
    return dict(q=to_dev(pick(p.q), p.dtype), k=to_dev(pick(p.k), p.dtype), v=to_dev(pick(p.v), p.dtype),
                g=to_dev(pick(p.g)), beta=to_dev(pick(p.beta)),
                cu_seqlens=to_dev(np.asarray(cu, dtype=np.int32)),
                cu_seqlens_host=torch.tensor(cu, dtype=torch.int32))


def _prefill(d, pools, **kw):
    S, R, P = pools
    o = _kda().kda_contract_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], S, R, P,
                                    cu_seqlens_host=d["cu_seqlens_host"], **kw)
    torch.cuda.synchronize()
    return o


def _decode_token(p: gen.Packed, t_of_seq, pools, **kw):
    """One decode step: token t_of_seq[n] of every sequence n."""
    idx = np.asarray([int(p.cu_seqlens[n]) + t for n, t in enumerate(t_of_seq)], dtype=np.int64)
    pick = lambda x: np.ascontiguousarray(x[idx])
    S, R, P = pools
    o = _kda().kda_contract_decode(to_dev(pick(p.q), p.dtype), to_dev(pick(p.k), p.dtype),
                                   to_dev(pick(p.v), p.dtype), to_dev(pick(p.g)), to_dev(pick(p.beta)),
                                   S, R, P, **kw)
    torch.cuda.synchronize()
    return o


def _pools(p: gen.Packed):
    S0 = None if p.initial_state is None else to_dev(p.initial_state)
    return _kda().kda_contract_pools(p.num_seqs, p.H, DEV, S0)


def _oracle_states(p: gen.Packed):
    dk, dv = p.k.shape[2], p.v.shape[2]
    S0 = p.initial_state if p.initial_state is not None else np.zeros((p.num_seqs, p.H, dk, dv))
    return [[cf.ContractState(S0[n, h]) for h in range(p.H)] for n in range(p.num_seqs)]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _assert_same_state(a, b, slots=None):
    """Same entry-state bits, positions and open rows (rows at or past the position are stale)."""
    sl = slice(None) if slots is None else slots
    assert torch.equal(a[2][sl], b[2][sl])
    assert torch.equal(_bits(a[0][sl]), _bits(b[0][sl]))
    pos = a[2][sl].cpu()
    ra, rb = a[1][sl].cpu(), b[1][sl].cpu()
    for i in range(pos.shape[0]):
        for h in range(pos.shape[1]):
            r = int(pos[i, h])
            assert torch.equal(_bits(ra[i, h, :r]), _bits(rb[i, h, :r]))


def _check_pools_against_oracle(pools, states, tol):
    S, R, P = (x.cpu() for x in pools)
    for n, row in enumerate(states):
        for h, st in enumerate(row):
            assert int(P[n, h]) == st.pos
            assert rel_l2(S[n, h].double().numpy(), st.S_e) <= tol
            for s, (k_s, b_s, u_s) in enumerate(st.rows):
                assert np.array_equal(R[n, h, s, 0].double().numpy(), k_s)  # keys are stored exactly
                np.testing.assert_allclose(R[n, h, s, 1].double().numpy(), b_s, rtol=1e-6, atol=1e-6)
                assert rel_l2(R[n, h, s, 2].double().numpy(), u_s) <= 10 * tol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_then_decode_match_oracle(dtype):
    lens = [1, 15, 16, 17, 50, 0, 77, 33]
    H = 3
    p = gen.packed_batch(seed=31, seqlens=[L + 20 for L in lens], H=H, dtype=dtype,
                         init_state=[True, False, True, True, False, True, False, True])
    pools = _pools(p)
    states = _oracle_states(p)
    # prefill the first lens[n] tokens of every sequence
    o = _prefill(_slice(p, [(0, L) for L in lens]), pools, scale=0.75)
    q, k, v, g, beta = (p.f64(x) for x in ("q", "k", "v", "g", "beta"))
    o_ref = np.full((sum(lens), H, 128), np.nan)
    t = 0
    for n, L in enumerate(lens):
        s0 = int(p.cu_seqlens[n])
        for h in range(H):
            o_ref[t:t + L, h] = cf.contract_tokens(states[n][h], q[s0:s0 + L, h], k[s0:s0 + L, h], v[s0:s0 + L, h],
                                                   g[s0:s0 + L, h], beta[s0:s0 + L, h], scale=0.75)
        t += L
    cu_pre = np.concatenate([[0], np.cumsum(lens)])
    check_parity(o, o_ref, TOL[dtype], packed_slices(cu_pre, H), bf16_out=dtype == "bf16",
                 tag=f"contract prefill {dtype} o")
    _check_pools_against_oracle(pools, states, TOL[dtype])
    # 20 decode steps on top (crossing chunk closes at different steps per sequence)
    errs = []
    for step in range(20):
        od = _decode_token(p, [L + step for L in lens], pools, scale=0.75)
        od_ref = np.empty((len(lens), H, 128))
        for n, L in enumerate(lens):
            tt = int(p.cu_seqlens[n]) + L + step
            for h in range(H):
                od_ref[n, h] = cf.contract_tokens(states[n][h], q[tt:tt + 1, h], k[tt:tt + 1, h], v[tt:tt + 1, h],
                                                  g[tt:tt + 1, h], beta[tt:tt + 1, h], scale=0.75)[0]
        errs.append(check_parity(od, od_ref, TOL[dtype], unit_slices(len(lens), H), bf16_out=dtype == "bf16",
                                 tag=f"contract decode step {step} {dtype} o"))
    print(f"contract decode {dtype}: max rel-L2 o over 20 steps {max(errs):.3e}")
    _check_pools_against_oracle(pools, states, TOL[dtype])
    # the running state equals the token recurrence over all tokens taken
    S_run = to_f64(_kda().kda_contract_state(*pools))
    _, S_ref = orc.prefill(q, k, v, g, beta, p.cu_seqlens, p.initial_state, scale=0.75)
    check_parity(S_run, S_ref, TOL[dtype], unit_slices(len(lens), H), tag=f"contract running state {dtype}")


def test_paths_are_bit_identical():
    """One prefill of everything == prefill of a prefix, decode steps, prefill of the rest."""
    lens = [40, 23, 64, 9, 18]
    p = gen.packed_batch(seed=32, seqlens=lens, H=2, dtype="bf16", init_state=True)
    whole = _pools(p)
    o_whole = _prefill(_slice(p, [(0, L) for L in lens]), whole)
    cut = [13, 0, 16, 2, 11]
    steps = 5
    split = _pools(p)
    o1 = _prefill(_slice(p, [(0, c) for c in cut]), split)
    od = [_decode_token(p, [c + s for c in cut], split) for s in range(steps)]
    o3 = _prefill(_slice(p, [(c + steps, L) for c, L in zip(cut, lens)]), split)
    # reassemble the split run's outputs in packed order
    parts, a1, a3 = [], 0, 0
    for n, (c, L) in enumerate(zip(cut, lens)):
        parts.append(o1[a1:a1 + c])
        parts.extend(od[s][n:n + 1] for s in range(steps))
        parts.append(o3[a3:a3 + L - c - steps])
        a1 += c
        a3 += L - c - steps
    o_split = torch.cat(parts)
    assert torch.equal(_bits(o_split), _bits(o_whole))
    _assert_same_state(whole, split)


def test_batch_invariance():
    """A sequence's bits do not depend on what else is in its batch (prefill and decode)."""
    lens = [37, 5, 64, 19, 1, 50]
    p = gen.packed_batch(seed=33, seqlens=[L + 1 for L in lens] + [3], H=4, dtype="bf16", init_state=True)
    full = _pools(p)
    o_full = _prefill(_slice(p, [(0, L) for L in lens] + [(0, 0)]), full)
    od_full = _decode_token(p, lens + [0], full)
    for n in (0, 2, 4):
        alone = _pools(p)
        slots = torch.tensor([n], dtype=torch.int32, device=DEV)
        d = _slice(p, [(0, lens[n]) if m == n else (0, 0) for m in range(len(lens) + 1)])
        keep = torch.arange(sum(lens[:n]), sum(lens[:n + 1]))
        d1 = dict(q=d["q"], k=d["k"], v=d["v"], g=d["g"], beta=d["beta"],
                  cu_seqlens=torch.tensor([0, lens[n]], dtype=torch.int32, device=DEV),
                  cu_seqlens_host=torch.tensor([0, lens[n]], dtype=torch.int32))
        o1 = _prefill(d1, alone, slots=slots)
        assert torch.equal(_bits(o1), _bits(o_full[keep.to(DEV)]))
        tt = int(p.cu_seqlens[n]) + lens[n]
        od1 = _kda().kda_contract_decode(to_dev(p.q[tt:tt + 1], "bf16"), to_dev(p.k[tt:tt + 1], "bf16"),
                                         to_dev(p.v[tt:tt + 1], "bf16"), to_dev(p.g[tt:tt + 1]),
                                         to_dev(p.beta[tt:tt + 1]), *alone, slots=slots)
        torch.cuda.synchronize()
        assert torch.equal(_bits(od1[0]), _bits(od_full[n]))
        _assert_same_state(alone, full, [n])


def test_empty_sequences_and_slots():
    """Empty sequences leave their slot untouched; slots route sequences to pool rows."""
    lens = [0, 21, 0, 16]
    p = gen.packed_batch(seed=34, seqlens=lens, H=2, dtype="bf16", init_state=True)
    P = 6
    S0 = torch.zeros((P, 2, 128, 128), dtype=torch.float32, device=DEV)
    S0[:4] = to_dev(p.initial_state)
    pools = _kda().kda_contract_pools(P, 2, DEV, S0)
    pools[1].normal_()  # stale rows in the pool must not matter at position 0
    slots = torch.tensor([5, 0, 2, 3], dtype=torch.int32, device=DEV)
    # sequence n of the batch uses slot slots[n]; give each slot its sequence's initial state
    for n in range(4):
        pools[0][int(slots[n])] = S0[n]
    before = [x.clone() for x in pools]
    o = _prefill(_slice(p, [(0, L) for L in lens]), pools, slots=slots)
    for n in (0, 2):  # empty: slot unchanged, bit for bit
        sl = int(slots[n])
        for x, y in zip(pools, before):
            assert torch.equal(x[sl], y[sl])
    for sl in (1, 4):  # untouched slots
        for x, y in zip(pools, before):
            assert torch.equal(x[sl], y[sl])
    states = _oracle_states(p)
    q, k, v, g, beta = (p.f64(x) for x in ("q", "k", "v", "g", "beta"))
    o_ref = np.empty((37, 2, 128))
    for n, (a, b) in ((1, (0, 21)), (3, (21, 37))):
        for h in range(2):
            o_ref[a:b, h] = cf.contract_tokens(states[n][h], q[a:b, h], k[a:b, h], v[a:b, h], g[a:b, h], beta[a:b, h])
    check_parity(o, o_ref, 2e-3, packed_slices([0, 21, 37], 2), bf16_out=True, tag="contract with slots o")
    assert int(pools[2][int(slots[1]), 0]) == 5 and int(pools[2][int(slots[3]), 1]) == 0
    # an all-empty batch is a no-op
    _prefill(_slice(p, [(0, 0)] * 4), pools, slots=slots)
    # no output buffer: same state as with one
    again = _kda().kda_contract_pools(P, 2, DEV, S0)
    for n in range(4):
        again[0][int(slots[n])] = S0[n]
    _prefill(_slice(p, [(0, L) for L in lens]), again, slots=slots, with_output=False)
    for x, y in zip(again[:1] + again[2:], pools[:1] + pools[2:]):
        assert torch.equal(x, y)


def test_decode_workload_sampled_parity():
    """Decode at 64 requests x 12 heads, each at its own position in the open chunk (prefix of
    16 + pos tokens prefilled), one step; sampled (request, head) units against the oracle."""
    N, H = 64, 12
    rng = np.random.default_rng(35)
    pos = rng.integers(0, 16, N)
    lens = [16 + int(x) + 1 for x in pos]
    p = gen.packed_batch(seed=35, seqlens=lens, H=H, dtype="bf16", init_state=True)
    pools = _pools(p)
    _prefill(_slice(p, [(0, L - 1) for L in lens]), pools, with_output=False)
    assert torch.equal(pools[2].cpu(), torch.tensor(np.repeat(pos[:, None], H, 1), dtype=torch.int32))
    od = _decode_token(p, [L - 1 for L in lens], pools)
    q, k, v, g, beta = (p.f64(x) for x in ("q", "k", "v", "g", "beta"))
    od_ref = np.empty((N, H, 128))
    for n in range(N):
        a, b = int(p.cu_seqlens[n]), int(p.cu_seqlens[n + 1])
        for h in range(H):
            o_ref, _ = orc.recurrence(q[a:b, h], k[a:b, h], v[a:b, h], g[a:b, h], beta[a:b, h], p.initial_state[n, h])
            od_ref[n, h] = o_ref[-1]
    check_parity(od, od_ref, 2e-3, unit_slices(N, H), bf16_out=True, tag="contract decode 64 x 12 o")


def test_prefill_workload_parity():
    """4096 tokens x 12 heads in one prefill; every head against the token recurrence."""
    p = gen.packed_batch(seed=36, seqlens=[4096], H=12, dtype="bf16")
    pools = _pools(p)
    o = _prefill(_slice(p, [(0, 4096)]), pools)
    S_run = to_f64(_kda().kda_contract_state(*pools))
    o_ref, S_ref = orc.prefill(*(p.f64(x) for x in ("q", "k", "v", "g", "beta")), p.cu_seqlens, None)
    check_parity(o, o_ref, 2e-3, packed_slices(p.cu_seqlens, 12), bf16_out=True, tag="contract prefill 4096 x 12 o")
    check_parity(S_run, S_ref, 2e-3, unit_slices(1, 12), tag="contract prefill 4096 x 12 S")
    assert int(pools[2][0, 0]) == 0  # 4096 = 256 closed chunks


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_state_handover_to_the_plain_decode(dtype):
    """kda_contract_state gives the running state at any position; the plain decode continues from it."""
    lens = [7, 16, 29]
    p = gen.packed_batch(seed=38, seqlens=[L + 3 for L in lens], H=2, dtype=dtype, init_state=True)
    pools = _pools(p)
    _prefill(_slice(p, [(0, L) for L in lens]), pools, with_output=False)
    S_run = _kda().kda_contract_state(*pools)
    q, k, v, g, beta = (p.f64(x) for x in ("q", "k", "v", "g", "beta"))
    for step in range(3):
        idx = [int(p.cu_seqlens[n]) + L + step for n, L in enumerate(lens)]
        pick = lambda x: np.ascontiguousarray(x[idx])
        o = _kda().kda_decode_step(to_dev(pick(p.q), dtype), to_dev(pick(p.k), dtype), to_dev(pick(p.v), dtype),
                                   to_dev(pick(p.g)), to_dev(pick(p.beta)), S_run)
        torch.cuda.synchronize()
        od_ref = np.empty((len(lens), 2, 128))
        for n, L in enumerate(lens):
            a = int(p.cu_seqlens[n])
            for h in range(2):
                o_ref, _ = orc.recurrence(q[a:a + L + step + 1, h], k[a:a + L + step + 1, h], v[a:a + L + step + 1, h],
                                          g[a:a + L + step + 1, h], beta[a:a + L + step + 1, h], p.initial_state[n, h])
                od_ref[n, h] = o_ref[-1]
        check_parity(o, od_ref, TOL[dtype], unit_slices(len(lens), 2), bf16_out=dtype == "bf16",
                     tag=f"handover step {step} {dtype}")


def test_strong_decay_beyond_the_fused_prefill_range():
    """log-decays down to -20 per step (the fused prefill supports >= -5): the contract's exponent
    differences stay finite and the results match the recurrence."""
    lens = [40, 17]
    p = gen.packed_batch(seed=39, seqlens=lens, H=2, dtype="f32", init_state=True)
    rng = np.random.default_rng(39)
    p.g[:] = rng.uniform(-20.0, 0.0, p.g.shape).astype(np.float32)
    pools = _pools(p)
    o = _prefill(_slice(p, [(0, L) for L in lens]), pools)
    q, k, v, g, beta = (p.f64(x) for x in ("q", "k", "v", "g", "beta"))
    o_ref, S_ref = orc.prefill(q, k, v, g, beta, p.cu_seqlens, p.initial_state)
    assert torch.isfinite(o).all()
    check_parity(o, o_ref, 1e-5, packed_slices(p.cu_seqlens, 2), tag="contract strong decay o")
    check_parity(_kda().kda_contract_state(*pools), S_ref, 1e-5, unit_slices(2, 2), tag="contract strong decay S")


def test_paths_are_bit_identical_f32():
    lens = [33, 20]
    p = gen.packed_batch(seed=40, seqlens=lens, H=3, dtype="f32", init_state=True)
    whole = _pools(p)
    o_whole = _prefill(_slice(p, [(0, L) for L in lens]), whole)
    split = _pools(p)
    o1 = _prefill(_slice(p, [(0, 15), (0, 4)]), split)
    od = _decode_token(p, [15, 4], split)
    o3 = _prefill(_slice(p, [(16, 33), (5, 20)]), split)
    o_split = torch.cat([o1[:15], od[0:1], o3[:17], o1[15:], od[1:2], o3[17:]])
    assert torch.equal(_bits(o_split), _bits(o_whole))
    _assert_same_state(whole, split)


def _block_inputs(p: gen.Packed, starts, G):
    """[N, G, H, 128] blocks: tokens starts[n] .. starts[n] + G - 1 of sequence n."""
    idx = np.stack([int(p.cu_seqlens[n]) + s + np.arange(G) for n, s in enumerate(starts)])
    pick = lambda x: np.ascontiguousarray(x[idx])
    return (to_dev(pick(p.q), p.dtype), to_dev(pick(p.k), p.dtype), to_dev(pick(p.v), p.dtype),
            to_dev(pick(p.g)), to_dev(pick(p.beta)))


def _positioned_pools(seed, N, H, G, dtype="bf16"):
    """Pools after a prefill of 16 + pos_n tokens (pos_n spread over the chunk), with G more tokens per sequence."""
    pos = np.arange(N) % 16
    lens = [16 + int(x) for x in pos]
    p = gen.packed_batch(seed=seed, seqlens=[L + G for L in lens], H=H, dtype=dtype, init_state=True)
    pools = _pools(p)
    _prefill(_slice(p, [(0, L) for L in lens]), pools, with_output=False)
    return p, pools, lens


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_verify_equals_decode_steps_and_reads_only(dtype):
    N, H, G = 20, 2, 8
    p, pools, lens = _positioned_pools(41, N, H, G, dtype)
    before = [x.clone() for x in pools]
    q, k, v, g, beta = _block_inputs(p, lens, G)
    o = _kda().kda_contract_verify(q, k, v, g, beta, *pools)
    torch.cuda.synchronize()
    for x, y in zip(pools, before):
        assert torch.equal(x, y)  # the state is only read
    steps = [x.clone() for x in pools]
    for t in range(G):
        od = _kda().kda_contract_decode(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
                                        g[:, t].contiguous(), beta[:, t].contiguous(), *steps)
        torch.cuda.synchronize()
        assert torch.equal(_bits(o[:, t]), _bits(od))
    # and against the oracle
    states = _oracle_states(p)
    qq, kk, vv, gg, bb = (p.f64(x) for x in ("q", "k", "v", "g", "beta"))
    o_ref = np.empty((N, G, H, 128))
    for n, L in enumerate(lens):
        a = int(p.cu_seqlens[n])
        for h in range(H):
            st = states[n][h]
            cf.contract_tokens(st, qq[a:a + L, h], kk[a:a + L, h], vv[a:a + L, h], gg[a:a + L, h], bb[a:a + L, h])
            o_ref[n, :, h] = cf.contract_tokens(st, qq[a + L:a + L + G, h], kk[a + L:a + L + G, h],
                                                vv[a + L:a + L + G, h], gg[a + L:a + L + G, h],
                                                bb[a + L:a + L + G, h])
    check_parity(o, o_ref, TOL[dtype], unit_slices(N, H, steps=True), bf16_out=dtype == "bf16",
                 tag=f"contract verify {dtype} o")


def test_commit_equals_decode_steps():
    N, H, G = 24, 2, 8
    p, pools, lens = _positioned_pools(42, N, H, G)
    q, k, v, g, beta = _block_inputs(p, lens, G)
    acc = np.array([(3 * n) % 9 for n in range(N)], dtype=np.int32)  # 0 .. 8, every value
    acc[5] = 12  # clamped to G
    steps = [x.clone() for x in pools]
    _kda().kda_contract_commit(k, v, g, beta, to_dev(acc), *pools)
    torch.cuda.synchronize()
    # reference: decode steps for each request's accepted prefix (requests stepped one slot at a time)
    for n in range(N):
        sl = torch.tensor([n], dtype=torch.int32, device=DEV)
        for t in range(min(int(acc[n]), G)):
            _kda().kda_contract_decode(q[n:n + 1, t].contiguous(), k[n:n + 1, t].contiguous(),
                                       v[n:n + 1, t].contiguous(), g[n:n + 1, t].contiguous(),
                                       beta[n:n + 1, t].contiguous(), *steps, slots=sl)
    torch.cuda.synchronize()
    _assert_same_state(pools, steps)


def test_verify_commit_workload_parity():
    """32 requests x 12 heads x 8 drafts (the verify workload), positions spread over the chunk; every
    (request, head) against the token recurrence."""
    N, H, G = 32, 12, 8
    p, pools, lens = _positioned_pools(43, N, H, G)
    q, k, v, g, beta = _block_inputs(p, lens, G)
    o = _kda().kda_contract_verify(q, k, v, g, beta, *pools)
    acc = to_dev(gen.accepted_lengths(43, N, G))
    _kda().kda_contract_commit(k, v, g, beta, acc, *pools, q=q)
    torch.cuda.synchronize()
    S_run = to_f64(_kda().kda_contract_state(*pools))
    qq, kk, vv, gg, bb = (p.f64(x) for x in ("q", "k", "v", "g", "beta"))
    accn = acc.cpu().numpy()
    o_all = np.empty((N, G, H, 128))
    S_all = np.empty((N, H, 128, 128))
    for n in range(N):
        a, L = int(p.cu_seqlens[n]), lens[n]
        m = L + int(accn[n])
        for h in range(H):
            o_ref, _ = orc.recurrence(qq[a:a + L + G, h], kk[a:a + L + G, h], vv[a:a + L + G, h],
                                      gg[a:a + L + G, h], bb[a:a + L + G, h], p.initial_state[n, h])
            o_all[n, :, h] = o_ref[L:]
            _, S_all[n, h] = orc.recurrence(qq[a:a + m, h], kk[a:a + m, h], vv[a:a + m, h], gg[a:a + m, h],
                                            bb[a:a + m, h], p.initial_state[n, h])
    check_parity(o, o_all, 2e-3, unit_slices(N, H, steps=True), bf16_out=True, tag="contract verify 32 x 12 x 8 o")
    check_parity(S_run, S_all, 2e-3, unit_slices(N, H), tag="contract commit 32 x 12 x 8 S")


@pytest.mark.parametrize("G", [8, 16])
def test_commit_from_the_verify_stash(G):
    """Verify with a stash, then commit from it: the pools equal those of the recomputing commit, bit for
    bit, for every accepted length (requests at every position, so drafts cross the chunk end or not);
    the verify's outputs do not change with the stash."""
    N, H = 24, 2
    p, pools, lens = _positioned_pools(44 + G, N, H, G)
    q, k, v, g, beta = _block_inputs(p, lens, G)
    acc = np.array([(5 * n) % (G + 1) for n in range(N)], dtype=np.int32)
    acc[3] = G + 4  # clamped
    ref = [x.clone() for x in pools]
    o_plain = _kda().kda_contract_verify(q, k, v, g, beta, *pools)
    stash = _kda().kda_contract_stash(N, G, H, DEV)
    o_st = _kda().kda_contract_verify(q, k, v, g, beta, *pools, stash=stash)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o_plain), _bits(o_st))
    _kda().kda_contract_commit_stash(stash, to_dev(acc), *pools, G=G)
    _kda().kda_contract_commit(k, v, g, beta, to_dev(acc), *ref, q=q)
    torch.cuda.synchronize()
    _assert_same_state(pools, ref)


@pytest.mark.parametrize("G", [1, 2, 3, 5, 7, 9, 12, 15])
def test_draft_blocks_of_every_length(G):
    """Draft blocks on both sides of the 8-row / 16-row builds, from every position in the chunk
    (short passes, passes that close the chunk and continue): verify outputs equal decode steps bit
    for bit with or without a stash, and the stash commit, the recomputing commit and decode steps of
    the accepted tokens leave the same pools."""
    N, H = 16, 2
    p, pools, lens = _positioned_pools(60 + G, N, H, G)
    q, k, v, g, beta = _block_inputs(p, lens, G)
    acc = np.array([(3 * n + 1) % (G + 1) for n in range(N)], dtype=np.int32)
    ref = [x.clone() for x in pools]
    steps = [x.clone() for x in pools]
    o = _kda().kda_contract_verify(q, k, v, g, beta, *pools)
    stash = _kda().kda_contract_stash(N, G, H, DEV)
    o_st = _kda().kda_contract_verify(q, k, v, g, beta, *pools, stash=stash)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o), _bits(o_st))
    full = [x.clone() for x in pools]  # every draft decoded: the verify's outputs
    before = [x.clone() for x in steps]
    for t in range(G):
        tok = (q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(), g[:, t].contiguous(),
               beta[:, t].contiguous())
        od = _kda().kda_contract_decode(*tok, *full)
        _kda().kda_contract_decode(*tok, *steps)
        torch.cuda.synchronize()
        assert torch.equal(_bits(o[:, t]), _bits(od))
        done = [n for n in range(N) if acc[n] <= t]  # accepted prefix already ended: undo this step
        if done:
            idx = torch.tensor(done, dtype=torch.long, device=DEV)
            for x, y in zip(steps, before):
                x[idx] = y[idx]
        before = [x.clone() for x in steps]
    _kda().kda_contract_commit_stash(stash, to_dev(acc), *pools, G=G)
    _kda().kda_contract_commit(k, v, g, beta, to_dev(acc), *ref, q=q)
    torch.cuda.synchronize()
    _assert_same_state(pools, ref)
    _assert_same_state(pools, steps)


@pytest.mark.parametrize("width", [2, 4])
def test_split_widths_equal_unsplit_bitwise(width):
    """The prefill with each unit's value columns split over `width` workgroups (and the shared rows
    written by the second launch) equals the unsplit prefill bit for bit, from position 0 and from a
    nonzero open-chunk position (a prefill cut, then a prefill of the rest), whatever the CU count."""
    rng = np.random.default_rng(80 + width)
    N, H = 9, 2
    cut = [int(x) for x in rng.integers(0, 20, N)]
    rest = [int(x) for x in rng.integers(0, 45, N)]
    rest[2], cut[3], rest[3] = 16 - cut[2] % 16, 16, 16  # ends on a chunk close; starts at a close
    p = gen.packed_batch(seed=80 + width, seqlens=[a + b for a, b in zip(cut, rest)], H=H, dtype="bf16",
                         init_state=True)
    pools = {w: _pools(p) for w in (1, width)}
    outs = {}
    for w, pl in pools.items():
        o1 = _prefill(_slice(p, [(0, c) for c in cut]), pl, split_width=w)
        o2 = _prefill(_slice(p, [(c, c + r) for c, r in zip(cut, rest)]), pl, split_width=w)
        outs[w] = (o1, o2)
    for a, b in zip(outs[1], outs[width]):
        assert torch.equal(_bits(a), _bits(b))
    _assert_same_state(pools[1], pools[width])


@pytest.mark.parametrize("width", [2, 4])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prepared_chunks_equal_walk_bitwise(width, dtype):
    """With a workspace the split prefill reads each full chunk's decays, rescaled keys and queries,
    Gram entries and close factors from a chunk-parallel first kernel (kda_contract_prefill_ex): the
    results equal the split walk without a workspace and the unsplit walk bit for bit, from position 0
    and from a nonzero open-chunk position, with sequences shorter than a chunk, ending on a close, and
    pool rows reached through permuted slots."""
    rng = np.random.default_rng(90 + width)
    N, H = 9, 2
    cut = [int(x) for x in rng.integers(0, 20, N)]
    rest = [int(x) for x in rng.integers(0, 70, N)]
    rest[2], cut[3], rest[3], cut[4], rest[4] = 16 - cut[2] % 16, 16, 48, 0, 5
    p = gen.packed_batch(seed=90 + width, seqlens=[a + b for a, b in zip(cut, rest)], H=H, dtype=dtype,
                         init_state=True)
    slots = torch.tensor(list(reversed(range(N))), dtype=torch.int32, device=DEV)
    runs = {"unsplit": dict(split_width=1), "split": dict(split_width=width),
            "prepared": dict(split_width=width, workspace="auto")}
    pools = {name: _pools(p) for name in runs}
    outs = {}
    for name, kw in runs.items():
        o1 = _prefill(_slice(p, [(0, c) for c in cut]), pools[name], slots=slots, **kw)
        o2 = _prefill(_slice(p, [(c, c + r) for c, r in zip(cut, rest)]), pools[name], slots=slots, **kw)
        outs[name] = (o1, o2)
    for name in ("split", "prepared"):
        for a, b in zip(outs["unsplit"], outs[name]):
            assert torch.equal(_bits(a), _bits(b)), name
        _assert_same_state(pools["unsplit"], pools[name])


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_prepared_chunks_random_batches_bitwise(seed):
    """Random batches (1-20 sequences of 0-100 tokens, 1-4 heads, resumed from random open-chunk
    positions, bf16 or fp32): the prefill with a workspace equals the one without, bit for bit."""
    rng = np.random.default_rng(300 + seed)
    N, H = int(rng.integers(1, 21)), int(rng.integers(1, 5))
    dtype = "bf16" if seed % 2 == 0 else "f32"
    cut = [int(x) for x in rng.integers(0, 40, N)]
    rest = [int(x) for x in rng.integers(0, 101, N)]
    p = gen.packed_batch(seed=300 + seed, seqlens=[a + b for a, b in zip(cut, rest)], H=H, dtype=dtype,
                         init_state=bool(seed % 3))
    runs = {"walk": {}, "prepared": dict(workspace="auto")}
    pools = {name: _pools(p) for name in runs}
    outs = {}
    for name, kw in runs.items():
        o1 = _prefill(_slice(p, [(0, c) for c in cut]), pools[name], **kw)
        o2 = _prefill(_slice(p, [(c, c + r) for c, r in zip(cut, rest)]), pools[name], **kw)
        outs[name] = (o1, o2)
    for a, b in zip(outs["walk"], outs["prepared"]):
        assert torch.equal(_bits(a), _bits(b))
    _assert_same_state(pools["walk"], pools["prepared"])


def test_prepared_chunks_4096x12_bitwise():
    """The 4,096-token x 12-head contract prefill (four-way split on a 256-CU part) with and without the
    workspace: bit-identical outputs, entry states, open rows and positions."""
    p = gen.packed_batch(seed=31, seqlens=[4096], H=12, dtype="bf16", init_state=True)
    d = _slice(p, [(0, 4096)])
    a, b = _pools(p), _pools(p)
    oa = _prefill(d, a)
    ob = _prefill(d, b, workspace="auto")
    assert torch.equal(_bits(oa), _bits(ob))
    _assert_same_state(a, b)


@pytest.mark.parametrize("total", [72, 144])
def test_split_and_unsplit_prefill_are_bit_identical(total):
    """The automatic split width: a grid of at most CUs / 4 (CUs / 2) (sequence, head) units splits
    four (two) ways, a larger one does not.  `total` sequences in one call and the same sequences in two
    calls of total / 2 give the same outputs, entry states, open rows and positions, bit for bit (on a
    256-CU part, 72: two-way vs four-way; 144: unsplit vs two-way; each width is compared with the
    unsplit path directly in test_split_widths_equal_unsplit_bitwise)."""
    rng = np.random.default_rng(70 + total)
    lens = [int(x) for x in rng.integers(0, 41, total)]
    lens[5], lens[40] = 16, 32  # ends exactly at a chunk close
    p = gen.packed_batch(seed=70 + total, seqlens=lens, H=1, dtype="bf16", init_state=True)
    whole = _pools(p)
    o_whole = _prefill(_slice(p, [(0, L) for L in lens]), whole)
    parted = _pools(p)
    outs = []
    half = total // 2
    for seqs in (range(0, half), range(half, total)):  # split calls; pool rows through slots
        idx = np.concatenate([np.arange(p.cu_seqlens[n], p.cu_seqlens[n + 1]) for n in seqs]).astype(np.int64)
        cu = np.concatenate([[0], np.cumsum([lens[n] for n in seqs])]).astype(np.int32)
        pick = lambda x: np.ascontiguousarray(x[idx])
        d = dict(q=to_dev(pick(p.q), p.dtype), k=to_dev(pick(p.k), p.dtype), v=to_dev(pick(p.v), p.dtype),
                 g=to_dev(pick(p.g)), beta=to_dev(pick(p.beta)), cu_seqlens=to_dev(cu),
                 cu_seqlens_host=torch.from_numpy(cu.copy()))
        slots = torch.tensor(list(seqs), dtype=torch.int32, device=DEV)
        outs.append(_prefill(d, parted, slots=slots))
    assert torch.equal(_bits(o_whole), _bits(torch.cat(outs)))
    _assert_same_state(whole, parted)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", ["beta1", "beta0", "g0"])
def test_edge_gates(case, dtype):
    """beta = 1 (the value along the key is replaced; with q = k the output is v), beta = 0 (pure channel
    decay) and g = 0 (the plain delta rule) through a contract prefill and three decode steps: against
    the token recurrence per slice and per element."""
    lens = [40, 17, 5]
    H = 2
    p = gen.packed_batch(seed=90, seqlens=[L + 3 for L in lens], H=H, dtype=dtype, init_state=True)
    if case == "beta1":
        p.beta[:] = np.float32(1.0)
        p.q[:] = p.k
    elif case == "beta0":
        p.beta[:] = np.float32(0.0)
    else:
        p.g[:] = np.float32(0.0)
    pools = _pools(p)
    o = _prefill(_slice(p, [(0, L) for L in lens]), pools)
    od = [_decode_token(p, [L + s for L in lens], pools) for s in range(3)]
    q, k, v, g, beta = (p.f64(x) for x in ("q", "k", "v", "g", "beta"))
    o_ref, S_ref = orc.prefill(q, k, v, g, beta, p.cu_seqlens, p.initial_state)
    pre = np.concatenate([np.arange(p.cu_seqlens[n], p.cu_seqlens[n] + L) for n, L in enumerate(lens)])
    cu_pre = np.concatenate([[0], np.cumsum(lens)])
    check_parity(o, o_ref[pre], TOL[dtype], packed_slices(cu_pre, H), bf16_out=dtype == "bf16",
                 tag=f"contract edge {case} {dtype} prefill o")
    for s in range(3):
        idx = [int(p.cu_seqlens[n]) + L + s for n, L in enumerate(lens)]
        check_parity(od[s], o_ref[idx], TOL[dtype], unit_slices(len(lens), H), bf16_out=dtype == "bf16",
                     tag=f"contract edge {case} {dtype} decode {s} o")
    check_parity(_kda().kda_contract_state(*pools), S_ref, TOL[dtype], unit_slices(len(lens), H),
                 tag=f"contract edge {case} {dtype} running state")
    if case == "beta1":
        assert rel_l2(to_f64(o), v[pre]) <= (2e-2 if dtype == "bf16" else 1e-5)
