"""The chunked form the HIP prefill computes, re-derived in fp64 and checked against the oracle.

Within a chunk with entry state S and cumulative log-decay b_r = sum_{s<=r} g_s
(per key channel), unrolling the update gives

    (I + A) U = diag(beta) (V - K^ S),   A = strict_lower(diag(beta) K^ Kv^T)
    O = Q^ S + lower(Q^ Kv^T) U,         S_end = Diag(e^{b_last}) S + K-^T U

with K^ = K e^{b}, Kv = K e^{-b}, Q^ = scale Q e^{b}, K- = K e^{b_last - b}.
This is the WY/UT representation of the chunk's product of
(I - beta k k^T) Diag(alpha) factors (the update is from "Kimi K3：架构与 SGLang
Day-0 Support", section "attention 机制详解：KDA"; the rescaling of keys by
the inverse cumulative decay is the chunkwise remark in the same box).
The kernel applies T' = (I + A)^{-1} diag(beta) to the residual V - K^ S
instead of forming W = T' K^ and U~ = T' V; both are checked here.
Padding a ragged tail with k = q = v = 0, beta = 0, g = 0 must not change it.
"""
import numpy as np
import pytest

from oracle import kda_oracle as orc


def _chunk_pass(q, k, v, g, beta, S0, C, scale=1.0, pad=True, form="residual"):
    T, dk = k.shape
    dv = v.shape[1]
    S = S0.copy()
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        sl = slice(c0, c0 + n)
        Q, K, V, Gm, B = q[sl], k[sl], v[sl], g[sl], beta[sl]
        if pad and n < C:   # the kernel zero-fills a ragged tail to a full chunk
            z = lambda x, w: np.concatenate([x, np.zeros((C - n, w))])
            Q, K, V, Gm = z(Q, dk), z(K, dk), z(V, dv), z(Gm, dk)
            B = np.concatenate([B, np.zeros(C - n)])
        m = K.shape[0]
        b = np.cumsum(Gm, axis=0)
        Kh, Kv, Qh = K * np.exp(b), K * np.exp(-b), scale * Q * np.exp(b)
        Kb = K * np.exp(b[-1] - b)
        A = np.tril(B[:, None] * (Kh @ Kv.T), -1)
        P = np.tril(Qh @ Kv.T)
        Tinv = np.linalg.solve(np.eye(m) + A, np.eye(m))
        Tp = Tinv * B[None, :]
        if form == "residual":
            U = Tp @ (V - Kh @ S)
        else:
            W, Ut = Tp @ Kh, Tp @ V
            U = Ut - W @ S
        O = Qh @ S + P @ U
        S = np.exp(b[-1])[:, None] * S + Kb.T @ U
        o[sl] = O[:n]
    return o, S


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 130, 256])
@pytest.mark.parametrize("form", ["residual", "wy"])
def test_chunk_form_equals_token_loop(C, T, form):
    rng = np.random.default_rng(1000 + T + C)
    dk, dv = 32, 24
    q = rng.standard_normal((T, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    g = rng.uniform(-0.5, 0, (T, dk))
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    S0 = 0.1 * rng.standard_normal((dk, dv))
    o_ref, S_ref = orc.recurrence(q, k, v, g, beta, S0, scale=0.9)
    o, S = _chunk_pass(q, k, v, g, beta, S0, C, scale=0.9, form=form)
    assert orc.rel_l2(o, o_ref) < 1e-12
    assert orc.rel_l2(S, S_ref) < 1e-12


def test_chunk_transition_is_identity_run():
    """The segment transition M is the same pass run on S0 = I with V = 0."""
    rng = np.random.default_rng(7)
    T, dk = 100, 16
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    g = rng.uniform(-0.1, 0, (T, dk))
    beta = rng.uniform(0, 1, T)
    _, M_chunk = _chunk_pass(np.zeros((T, dk)), k, np.zeros((T, dk)), g, beta, np.eye(dk), 64)
    assert orc.rel_l2(M_chunk, orc.transition(k, g, beta)) < 1e-12


def test_chunk_form_config_like_ranges():
    """At the workloads' decay (g in (-0.1, 0], C = 64) the rescaled keys stay within e^{6.4}."""
    rng = np.random.default_rng(8)
    T, dk, dv = 256, 128, 128
    q = rng.standard_normal((T, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    g = rng.uniform(-0.1, 0, (T, dk))
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    b = np.cumsum(g.reshape(4, 64, dk), axis=1)
    assert np.exp(-b).max() <= np.exp(6.4)
    o_ref, S_ref = orc.recurrence(q, k, v, g, beta, None)
    o, S = _chunk_pass(q, k, v, g, beta, np.zeros((dk, dv)), 64)
    assert orc.rel_l2(o, o_ref) < 1e-12 and orc.rel_l2(S, S_ref) < 1e-12
