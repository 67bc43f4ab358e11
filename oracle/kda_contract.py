"""CPU oracle for the batch-invariant row contract of KDA — TEST INFRASTRUCTURE.

Like ``kda_oracle``, this is the plain fp64 reference the HIP library is
checked against; only the test suite may import it, and it shares no code with
the kernels.

The contract ("Kimi K3.1 Pro" inference / zero-mismatch article, LLMNews
2026-11-05, section 6.1 on KDA) fixes one row-level computation that both the
chunked prefill and the token-by-token decode follow, so that a token's result
does not depend on which path, or which batch, computed it.  The chunk length
is 16 tokens (the page's current contract version).  The per-sequence, per-head
state is not the running S_t but

* S_e: the state at the entry of the current (open) chunk, and
* the open chunk's rows so far, one per token s already in it: the key k_s,
  the cumulative log-decay b_s = g_0 + ... + g_s since the chunk entry (per key
  channel), and the delta-write vector u_s; their count is the position.

A token r of the open chunk is computed from S_e and the earlier rows only, by
the chunk form of the recurrence restated per row (its derivation: the UT/WY
form of the product of the per-token factors; the update itself is the one in
"Kimi K3：架构与 SGLang Day-0 Support", section "attention 机制详解：KDA"):

    b_r  = b_{r-1} + g_r                          (b_{-1} = 0)
    u_r  = beta_r (v_r - S_e^T (k_r * e^{b_r}) - sum_{s<r} G_k[r,s] u_s)
    o_r  = S_e^T (q'_r * e^{b_r}) + sum_{s<=r} G_q[r,s] u_s        (q' = scale q)
    G_k[r,s] = sum_c k_rc k_sc e^{b_rc - b_sc},  G_q[r,s] = sum_c q'_rc k_sc e^{b_rc - b_sc}

and when the chunk holds 16 rows it closes:

    S_e <- Diag(e^{b_15}) S_e + sum_s (k_s * e^{b_15 - b_s}) u_s^T,  rows <- {}.

At any position the running state is S_t = Diag(e^{b_r}) S_e + sum_{s<=r}
(k_s * e^{b_r - b_s}) u_s^T (``materialize``).

Readings taken where the page is silent: the cached row holds (k_s, b_s, u_s)
and the Gram entries use the exponent difference b_r - b_s <= 0 rather than
separately rescaled keys k * e^{-b}, so no factor exceeds 1 whatever the decay
(the page's per-head row cache has 17 rows of 256 floats; its contents are not
printed); the decode and the prefill both close a chunk exactly when its 16th
row is written.

Pins (tests/test_oracle_contract.py): outputs and the materialised state equal
the token recurrence of ``kda_oracle`` at every length and start position;
running a sequence in any split into pieces gives the same fp64 bits (the
contract's defining property); beta = 0 gives pure channel decay; a decay too
strong for rescaled keys stays finite and still equals the recurrence.
"""
from __future__ import annotations

import numpy as np

__all__ = ["CHUNK", "ContractState", "contract_tokens", "materialize", "contract_prefill",
           "contract_decode"]

CHUNK = 16


class ContractState:
    """One (sequence, head): the chunk-entry state and the open chunk's rows."""

    def __init__(self, S_e, rows=None):
        self.S_e = np.array(S_e, dtype=np.float64)
        self.rows = [] if rows is None else [tuple(np.array(x, dtype=np.float64) for x in r) for r in rows]

    @property
    def pos(self):
        return len(self.rows)

    def copy(self):
        return ContractState(self.S_e, self.rows)


def contract_tokens(st: ContractState, q, k, v, g, beta, scale=1.0):
    """Run tokens through the contract, updating ``st`` in place.

    q, k, g: [T, d_k]; v: [T, d_v]; beta: [T].  Returns o [T, d_v] in fp64.
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    o = np.empty((k.shape[0], v.shape[1]))
    for t in range(k.shape[0]):
        b = g[t] + (st.rows[-1][1] if st.rows else 0.0)
        decay = np.exp(b)
        qs = scale * q[t]
        a = st.S_e.T @ (k[t] * decay)          # S_e^T k_hat
        w = st.S_e.T @ (qs * decay)            # S_e^T q_hat
        resid = v[t] - a
        out = w.copy()
        for k_s, b_s, u_s in st.rows:          # earlier rows of the open chunk
            rel = np.exp(b - b_s)              # e^{b_r - b_s} <= 1
            resid -= np.sum(k[t] * k_s * rel) * u_s
            out += np.sum(qs * k_s * rel) * u_s
        u = beta[t] * resid
        out += np.dot(qs, k[t]) * u            # s = r: relative decay e^0 = 1
        o[t] = out
        st.rows.append((k[t].copy(), b, u))
        if len(st.rows) == CHUNK:              # close the chunk
            b_last = st.rows[-1][1]
            S = np.exp(b_last)[:, None] * st.S_e
            for k_s, b_s, u_s in st.rows:
                S += np.outer(k_s * np.exp(b_last - b_s), u_s)
            st.S_e, st.rows = S, []
    return o


def materialize(st: ContractState):
    """The running state S_t of the recurrence after the last token taken."""
    if not st.rows:
        return st.S_e.copy()
    b_last = st.rows[-1][1]
    S = np.exp(b_last)[:, None] * st.S_e
    for k_s, b_s, u_s in st.rows:
        S += np.outer(k_s * np.exp(b_last - b_s), u_s)
    return S


def contract_prefill(q, k, v, g, beta, cu_seqlens, states, scale=1.0, heads=None):
    """Packed ragged batch through the contract: q,k,g [T, H, d_k]; v [T, H, d_v];
    beta [T, H]; states[n][h] are ContractState objects, updated in place.
    Returns o [T, H, d_v] (NaN where ``heads`` excludes a head)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, _ = np.shape(k)
    o = np.full((T, H, np.shape(v)[2]), np.nan)
    for n in range(cu.shape[0] - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        for h in (range(H) if heads is None else heads):
            o[a:b, h] = contract_tokens(states[n][h], q[a:b, h], k[a:b, h], v[a:b, h], g[a:b, h],
                                        beta[a:b, h], scale)
    return o


def contract_decode(q, k, v, g, beta, states, scale=1.0):
    """One token per request: q,k,g [N, H, d_k]; v [N, H, d_v]; beta [N, H]."""
    N, H, _ = np.shape(k)
    o = np.empty((N, H, np.shape(v)[2]))
    for n in range(N):
        for h in range(H):
            o[n, h] = contract_tokens(states[n][h], q[n:n + 1, h], k[n:n + 1, h], v[n:n + 1, h],
                                      g[n:n + 1, h], beta[n:n + 1, h], scale)[0]
    return o
