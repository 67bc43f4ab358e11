"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these checks re-types the oracle's own loop: each compares it with an
independent statement — an identity the pages give, a closed form, a value
printed in the pages' teaching example, or brute-force products of explicit
d x d matrices — chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign, decay on the wrong axis, readout before the write, a transposed
state, an off-by-one in a segment or accepted length) fails at least one.
"""
import json
import os

import numpy as np
import pytest

from oracle import kda_oracle as orc


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_problem(rng, T, dk, dv, unit_keys=True, g_lo=-0.5):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    if unit_keys:
        q, k = _unit(q), _unit(k)
    v = rng.standard_normal((T, dv))
    g = rng.uniform(g_lo, 0.0, (T, dk))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    S0 = rng.standard_normal((dk, dv))
    return q, k, v, g, beta, S0


# ----------------------------------------------------------------------------
# 1. per-step readout identity (gate-then-delta split, unit keys)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dk,dv", [(8, 5), (16, 16), (128, 128)])
def test_readout_identity_every_step(dk, dv):
    """For unit k: S_t^T k_t = (1 - beta) (Diag(alpha) S_{t-1})^T k_t + beta v_t."""
    rng = np.random.default_rng(11)
    q, k, v, g, beta, S = _rand_problem(rng, 24, dk, dv)
    for t in range(24):
        _, S_new = orc.recurrence(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], S)
        r_old = (np.exp(g[t])[:, None] * S).T @ k[t]
        expect = (1.0 - beta[t]) * r_old + beta[t] * v[t]
        np.testing.assert_allclose(S_new.T @ k[t], expect, rtol=0, atol=1e-12 * (1 + np.abs(expect).max()))
        S = S_new


def test_readout_identity_alpha_one_deltanet():
    """alpha = 1 reduces KDA to DeltaNet: r_new = (1 - beta) r_old + beta v with r_old = S_{t-1}^T k."""
    rng = np.random.default_rng(12)
    q, k, v, g, beta, S = _rand_problem(rng, 16, 32, 24)
    g[:] = 0.0
    for t in range(16):
        _, S_new = orc.recurrence(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], S)
        r_old = S.T @ k[t]
        np.testing.assert_allclose(S_new.T @ k[t], (1 - beta[t]) * r_old + beta[t] * v[t], atol=1e-12)
        # and the write is rank one along k_t: the part of S orthogonal to k_t is untouched
        P_perp = np.eye(32) - np.outer(k[t], k[t])
        np.testing.assert_allclose(P_perp @ S_new, P_perp @ S, atol=1e-12)
        S = S_new


# ----------------------------------------------------------------------------
# 2. beta = 0: pure channel decay (closed form)
# ----------------------------------------------------------------------------
def test_beta_zero_pure_channel_decay():
    rng = np.random.default_rng(13)
    dk, dv, T = 12, 7, 40
    q, k, v, g, beta, S0 = _rand_problem(rng, T, dk, dv, g_lo=-0.3)
    beta[:] = 0.0
    o, S_T = orc.recurrence(q, k, v, g, beta, S0, scale=0.75)
    b = np.cumsum(g, axis=0)   # cumulative log-decay per key channel
    np.testing.assert_allclose(S_T, np.exp(b[-1])[:, None] * S0, rtol=1e-13, atol=1e-15)
    for t in range(T):
        S_t = np.exp(b[t])[:, None] * S0          # rows (key channels) decay, columns do not
        np.testing.assert_allclose(o[t], S_t.T @ (0.75 * q[t]), rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------
# 3. beta = 1 with unit keys: replacement along k
# ----------------------------------------------------------------------------
def test_beta_one_replaces_along_key():
    rng = np.random.default_rng(14)
    q, k, v, g, beta, S = _rand_problem(rng, 20, 16, 9)
    beta[:] = 1.0
    for t in range(20):
        _, S = orc.recurrence(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], S)
        np.testing.assert_allclose(S.T @ k[t], v[t], atol=1e-12)


# ----------------------------------------------------------------------------
# 4. the pages' two-dimensional teaching slice
# ----------------------------------------------------------------------------
def test_two_dimensional_teaching_slice(golden_dir):
    with open(os.path.join(golden_dir, "kda_2d_slice.json"), encoding="utf-8") as f:
        gold = json.load(f)
    k_a = np.array(gold["k_a"])
    k_b = np.array(gold["k_b"])
    a1, a2 = gold["first_value"], gold["second_value"]
    assert abs(k_a @ k_b) < 1e-15 and abs(k_a @ k_a - 1) < 1e-15

    def write(S, key, val, beta, alpha=(1.0, 1.0)):
        _, S = orc.recurrence(np.zeros((1, 2)), key[None], np.array([[val]]),
                              np.log(np.array(alpha))[None], np.array([beta]), S)
        return S

    # naive linear attention (the contrast the pages draw): S = sum k v^T
    S_naive = np.outer(k_a, [a1]) + np.outer(k_a, [a2])
    assert (S_naive.T @ k_a)[0] == pytest.approx(gold["naive_sum_readout"], abs=1e-14)

    S1 = write(np.zeros((2, 1)), k_a, a1, beta=1.0)
    assert (S1.T @ k_a)[0] == pytest.approx(a1, abs=1e-14)
    for beta, key in ((1.0, "delta_readout_beta_1"), (0.0, "delta_readout_beta_0")):
        S2 = write(S1, k_a, a2, beta=beta)
        assert (S2.T @ k_a)[0] == pytest.approx(gold[key], abs=1e-14)
    for beta in (0.25, 0.5, 0.8):
        S2 = write(S1, k_a, a2, beta=beta)
        assert (S2.T @ k_a)[0] == pytest.approx((1 - beta) * a1 + beta * a2, abs=1e-14)
    # orthogonal key: writing B along k_b leaves A's readout exactly as it was
    S2 = write(S1, k_a, a2, beta=1.0)
    S3 = write(S2, k_b, -3.0, beta=1.0)
    assert (S3.T @ k_a)[0] - (S2.T @ k_a)[0] == pytest.approx(gold["orthogonal_crosstalk"], abs=1e-14)
    assert (S3.T @ k_b)[0] == pytest.approx(-3.0, abs=1e-14)
    # with a per-channel gate the old value decays row-wise before the write:
    # r_old = sum_j alpha_j k_a[j] S1[j] = (alpha_1 + alpha_2) / 2
    for alpha in ((0.5, 0.9), (0.2, 1.0)):
        S2 = write(S1, k_a, a2, beta=0.3, alpha=alpha)
        r_old = 0.5 * (alpha[0] + alpha[1]) * a1
        assert (S2.T @ k_a)[0] == pytest.approx(0.7 * r_old + 0.3 * a2, abs=1e-14)


# ----------------------------------------------------------------------------
# 5. brute force: unrolled products of explicit d x d matrices
# ----------------------------------------------------------------------------
def _explicit_state(k, v, g, beta, S0, t):
    """S_t = [prod_{u=1..t} M_u] S0 + sum_{s<=t} [prod_{u=s+1..t} M_u] beta_s k_s v_s^T."""
    dk = k.shape[1]
    Ms = [(np.eye(dk) - beta[u] * np.outer(k[u], k[u])) @ np.diag(np.exp(g[u])) for u in range(t)]

    def prod(lo, hi):  # M_hi ... M_{lo+1} for 0-based token indices lo..hi-1
        P = np.eye(dk)
        for u in range(lo, hi):
            P = Ms[u] @ P
        return P

    S = prod(0, t) @ S0
    for s in range(t):
        S = S + prod(s + 1, t) @ (beta[s] * np.outer(k[s], v[s]))
    return S


@pytest.mark.parametrize("dk,dv,T,unit", [(2, 1, 6, True), (2, 3, 9, False), (4, 4, 12, True),
                                          (8, 5, 16, False), (8, 8, 16, True)])
def test_bruteforce_unrolled_products(dk, dv, T, unit):
    rng = np.random.default_rng(100 + dk * 10 + T)
    q, k, v, g, beta, S0 = _rand_problem(rng, T, dk, dv, unit_keys=unit, g_lo=-1.0)
    scale = 0.6
    o, S_T = orc.recurrence(q, k, v, g, beta, S0, scale=scale)
    for t in range(1, T + 1):
        S_t = _explicit_state(k, v, g, beta, S0, t)
        np.testing.assert_allclose(o[t - 1], S_t.T @ (scale * q[t - 1]), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S_T, _explicit_state(k, v, g, beta, S0, T), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------
# 6. segment fragments and composition
# ----------------------------------------------------------------------------
def test_transition_matches_explicit_product_and_affinity():
    rng = np.random.default_rng(21)
    q, k, v, g, beta, S0 = _rand_problem(rng, 30, 16, 11)
    M, S_tilde = orc.segment_fragments(k, v, g, beta)
    # affinity: the final state from any S0 is M S0 + S~
    _, S_T = orc.recurrence(q, k, v, g, beta, S0)
    np.testing.assert_allclose(S_T, M @ S0 + S_tilde, rtol=1e-12, atol=1e-13)
    # M applied to S0 is the state with all writes removed (v = 0)
    _, S_nov = orc.recurrence(q, k, np.zeros_like(v), g, beta, S0)
    np.testing.assert_allclose(S_nov, M @ S0, rtol=1e-12, atol=1e-13)
    # M from the recurrence run on the identity with no writes
    _, M_run = orc.recurrence(np.zeros((30, 16)), k, np.zeros((30, 16)), g, beta, np.eye(16))
    np.testing.assert_allclose(M, M_run, rtol=1e-12, atol=1e-14)


def test_transition_nonexpansive():
    """||(I - beta k k^T) Diag(alpha)||_2 <= 1 for unit k, beta in [0,1], alpha <= 1, so ||M||_2 <= 1."""
    rng = np.random.default_rng(22)
    _, k, v, g, beta, _ = _rand_problem(rng, 50, 12, 3)
    M = orc.transition(k, g, beta)
    assert np.linalg.norm(M, 2) <= 1.0 + 1e-12


@pytest.mark.parametrize("cuts", [[17], [5, 23], [1, 2, 40, 63]])
def test_split_and_compose_equals_unsplit(cuts):
    rng = np.random.default_rng(23 + len(cuts))
    T, dk, dv = 64, 16, 10
    q, k, v, g, beta, S0 = _rand_problem(rng, T, dk, dv)
    o_ref, S_ref = orc.recurrence(q, k, v, g, beta, S0)
    bounds = [0] + cuts + [T]
    Ms, Sts = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        M, St = orc.segment_fragments(k[a:b], v[a:b], g[a:b], beta[a:b])
        Ms.append(M)
        Sts.append(St)
    S_in, S_fin = orc.compose(np.stack(Ms), np.stack(Sts), S0)
    np.testing.assert_allclose(S_fin, S_ref, rtol=1e-12, atol=1e-13)
    o_parts = []
    for i, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        _, S_a = orc.recurrence(q[:a], k[:a], v[:a], g[:a], beta[:a], S0)
        np.testing.assert_allclose(S_in[i], S_a, rtol=1e-12, atol=1e-13)   # true entry state
        o_i, _ = orc.recurrence(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], S_in[i])
        o_parts.append(o_i)
    np.testing.assert_allclose(np.concatenate(o_parts), o_ref, rtol=1e-11, atol=1e-12)


def test_value_columns_are_independent():
    rng = np.random.default_rng(24)
    q, k, v, g, beta, S0 = _rand_problem(rng, 20, 8, 12)
    o, S = orc.recurrence(q, k, v, g, beta, S0)
    cols = [1, 4, 5, 11]
    o_c, S_c = orc.recurrence(q, k, v[:, cols], g, beta, S0[:, cols])
    np.testing.assert_allclose(o_c, o[:, cols], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S_c, S[:, cols], rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------
# 7. packed batches, decode, verify/commit
# ----------------------------------------------------------------------------
def test_prefill_packed_sequences_are_independent():
    rng = np.random.default_rng(31)
    H, dk, dv = 2, 8, 6
    lens = [5, 0, 9, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = _unit(rng.standard_normal((T, H, dk)))
    k = _unit(rng.standard_normal((T, H, dk)))
    v = rng.standard_normal((T, H, dv))
    g = rng.uniform(-0.2, 0, (T, H, dk))
    beta = rng.uniform(0, 1, (T, H))
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    o, S_fin = orc.prefill(q, k, v, g, beta, cu, S0)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        for h in range(H):
            S = S0[n, h]
            for t in range(a, b):   # explicit one-token-at-a-time chaining
                o_t, S = orc.recurrence(q[t:t + 1, h], k[t:t + 1, h], v[t:t + 1, h], g[t:t + 1, h],
                                        beta[t:t + 1, h], S)
                np.testing.assert_allclose(o[t, h], o_t[0], atol=1e-14)
            np.testing.assert_allclose(S_fin[n, h], S, atol=1e-14)
    # the empty sequence passes its state through
    np.testing.assert_array_equal(S_fin[1], S0[1])


def test_verify_commit_replays_accepted_prefix():
    rng = np.random.default_rng(32)
    N, G, H, dk, dv = 3, 8, 2, 8, 8
    q = _unit(rng.standard_normal((N, G, H, dk)))
    k = _unit(rng.standard_normal((N, G, H, dk)))
    v = rng.standard_normal((N, G, H, dv))
    g = rng.uniform(-0.1, 0, (N, G, H, dk))
    beta = rng.uniform(0, 1, (N, G, H))
    S0 = rng.standard_normal((N, H, dk, dv))
    acc = np.array([1, 8, 3])
    S0_copy = S0.copy()
    o, S_c = orc.verify_block(q, k, v, g, beta, S0, acc)
    np.testing.assert_array_equal(S0, S0_copy)   # the committed state is read, never written
    for n in range(N):
        for h in range(H):
            S = S0[n, h]
            for t in range(G):
                o1, S = orc.decode_step(q[n, t, h][None, None], k[n, t, h][None, None], v[n, t, h][None, None],
                                        g[n, t, h][None, None], beta[n, t, h][None, None], S[None, None])
                S = S[0, 0]
                np.testing.assert_allclose(o[n, t, h], o1[0, 0], atol=1e-13)
                if t + 1 == acc[n]:
                    np.testing.assert_allclose(S_c[n, h], S, atol=1e-13)


def test_compose_single_segment_is_affine_map():
    rng = np.random.default_rng(33)
    M = rng.standard_normal((1, 6, 6))
    St = rng.standard_normal((1, 6, 4))
    S0 = rng.standard_normal((6, 4))
    S_in, S_fin = orc.compose(M, St, S0)
    np.testing.assert_array_equal(S_in[0], S0)
    np.testing.assert_allclose(S_fin, M[0] @ S0 + St[0], atol=1e-14)


def test_rel_l2():
    a = np.array([3.0, 4.0])
    assert orc.rel_l2(a, a) == 0.0
    assert orc.rel_l2(a + np.array([0.3, 0.4]), a) == pytest.approx(0.1)


def test_checkpoints_are_affine_prefixes():
    """A checkpoint at p maps to the final state through the explicit-product transition of
    tokens p..L plus the zero-start state of those tokens (affinity), for every checkpoint."""
    rng = np.random.default_rng(77)
    dk = dv = 4
    lens = [13, 8, 1, 0, 9]
    cu = np.cumsum([0] + lens)
    T, H = int(cu[-1]), 2
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -0.3 * rng.random((T, H, dk))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, H))))
    q = rng.standard_normal((T, H, dk))
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    interval = 4
    C = orc.prefill_checkpoints(k, v, g, beta, cu, interval, S0)
    assert C.shape == (sum((L - 1) // interval if L else 0 for L in lens), H, dk, dv)
    _, S_fin = orc.prefill(q, k, v, g, beta, cu, S0)
    row = 0
    for n, L in enumerate(lens):
        a = int(cu[n])
        for m in range(1, ((L - 1) // interval if L else 0) + 1):
            p = a + m * interval
            for h in range(H):
                M = orc.transition(k[p:a + L, h], g[p:a + L, h], beta[p:a + L, h])
                _, S_tail = orc.recurrence(q[p:a + L, h], k[p:a + L, h], v[p:a + L, h], g[p:a + L, h],
                                           beta[p:a + L, h], None)
                assert np.allclose(M @ C[row, h] + S_tail, S_fin[n, h], atol=1e-12)
            row += 1
    assert row == C.shape[0]
