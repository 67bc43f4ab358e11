"""Pins of the row-contract oracle (no GPU).

Each test compares the contract against something it does not share code
with: the token recurrence of ``kda_oracle`` (itself pinned by test_oracle),
the exact equality the contract promises between splits of one sequence, the
beta = 0 closed form, and a decay too strong for separately rescaled keys.
"""
import numpy as np
import pytest

from oracle import kda_contract as cf
from oracle import kda_oracle as orc


def _problem(rng, T, dk, dv, g_lo=-0.6):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, dv))
    g = rng.uniform(g_lo, 0.0, (T, dk))
    beta = rng.uniform(0.05, 0.95, T)
    S0 = rng.standard_normal((dk, dv))
    return q, k, v, g, beta, S0


@pytest.mark.parametrize("T", [1, 15, 16, 17, 33, 50])
@pytest.mark.parametrize("dk,dv", [(8, 5), (32, 24)])
def test_contract_equals_recurrence(T, dk, dv):
    rng = np.random.default_rng(100 + T + dk)
    q, k, v, g, beta, S0 = _problem(rng, T, dk, dv)
    o_ref, S_ref = orc.recurrence(q, k, v, g, beta, S0, scale=0.7)
    st = cf.ContractState(S0)
    o = cf.contract_tokens(st, q, k, v, g, beta, scale=0.7)
    assert st.pos == T % cf.CHUNK
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-11 * np.abs(o_ref).max())
    np.testing.assert_allclose(cf.materialize(st), S_ref, rtol=0, atol=1e-11 * np.abs(S_ref).max())


def test_chunk_entry_state_at_a_close_is_the_recurrence_state():
    """After 16 and 32 tokens the open chunk is empty and S_e is the state itself."""
    rng = np.random.default_rng(7)
    q, k, v, g, beta, S0 = _problem(rng, 32, 16, 16)
    st = cf.ContractState(S0)
    for n in (16, 32):
        cf.contract_tokens(st, *(x[n - 16:n] for x in (q, k, v, g, beta)))
        assert st.pos == 0
        _, S_ref = orc.recurrence(q[:n], k[:n], v[:n], g[:n], beta[:n], S0)
        np.testing.assert_allclose(st.S_e, S_ref, rtol=0, atol=1e-12 * np.abs(S_ref).max())


@pytest.mark.parametrize("cuts", [[1], [5, 6, 20], [16], [3, 19, 35], list(range(1, 40))])
def test_any_split_gives_identical_bits(cuts):
    """The contract's defining property: each token's arithmetic depends on the
    open chunk's state only, so running the sequence in pieces (a prefill, then
    decode steps, then more prefill) reproduces the unsplit run exactly."""
    rng = np.random.default_rng(9)
    q, k, v, g, beta, S0 = _problem(rng, 40, 16, 12)
    whole = cf.ContractState(S0)
    o_whole = cf.contract_tokens(whole, q, k, v, g, beta, scale=1.3)
    part = cf.ContractState(S0)
    bounds = [0] + cuts + [40]
    o_part = np.concatenate([cf.contract_tokens(part, *(x[a:b] for x in (q, k, v, g, beta)), scale=1.3)
                             for a, b in zip(bounds[:-1], bounds[1:])])
    assert np.array_equal(o_part, o_whole)
    assert np.array_equal(part.S_e, whole.S_e) and part.pos == whole.pos
    for (ka, ba, ua), (kb, bb, ub) in zip(part.rows, whole.rows):
        assert np.array_equal(ka, kb) and np.array_equal(ba, bb) and np.array_equal(ua, ub)


def test_beta_zero_is_pure_channel_decay():
    rng = np.random.default_rng(3)
    q, k, v, g, beta, S0 = _problem(rng, 21, 8, 6)
    beta[:] = 0.0
    st = cf.ContractState(S0)
    o = cf.contract_tokens(st, q, k, v, g, beta)
    cum = np.cumsum(g, axis=0)
    for t in range(21):
        S_t = np.exp(cum[t])[:, None] * S0
        np.testing.assert_allclose(o[t], S_t.T @ q[t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(cf.materialize(st), np.exp(cum[-1])[:, None] * S0, rtol=1e-12, atol=1e-13)


def test_strong_decay_stays_finite():
    """g = -60 per step: over 16 rows e^{-b} would reach e^{960}, beyond fp64;
    the exponent-difference form never forms it and still equals the recurrence."""
    rng = np.random.default_rng(4)
    q, k, v, g, beta, S0 = _problem(rng, 20, 8, 8)
    g[:, :3] = -60.0
    with np.errstate(over="ignore"):
        assert not np.isfinite(np.exp(-np.cumsum(g[:16], axis=0))).all()
    st = cf.ContractState(S0)
    o = cf.contract_tokens(st, q, k, v, g, beta)
    o_ref, S_ref = orc.recurrence(q, k, v, g, beta, S0)
    assert np.isfinite(o).all()
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-11 * np.abs(o_ref).max())
    np.testing.assert_allclose(cf.materialize(st), S_ref, rtol=0, atol=1e-11 * np.abs(S_ref).max())


def test_packed_helpers_match_per_sequence_runs():
    rng = np.random.default_rng(5)
    H, dk, dv = 2, 8, 4
    lens = [3, 17, 0, 20]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v = rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dv))
    g, beta = rng.uniform(-0.5, 0, (T, H, dk)), rng.uniform(0.1, 0.9, (T, H))
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    states = [[cf.ContractState(S0[n, h]) for h in range(H)] for n in range(len(lens))]
    o = cf.contract_prefill(q, k, v, g, beta, cu, states)
    o_ref, S_ref = orc.prefill(q, k, v, g, beta, cu, S0)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-11)
    for n in range(len(lens)):
        for h in range(H):
            np.testing.assert_allclose(cf.materialize(states[n][h]), S_ref[n, h], atol=1e-11)
    # one more token per sequence through the decode helper equals the recurrence continued
    qd, kd, vd = rng.standard_normal((4, H, dk)), rng.standard_normal((4, H, dk)), rng.standard_normal((4, H, dv))
    gd, bd = rng.uniform(-0.5, 0, (4, H, dk)), rng.uniform(0.1, 0.9, (4, H))
    od = cf.contract_decode(qd, kd, vd, gd, bd, states)
    od_ref, _ = orc.decode_step(qd, kd, vd, gd, bd, S_ref)
    np.testing.assert_allclose(od, od_ref, rtol=0, atol=1e-11)
