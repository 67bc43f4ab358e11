"""CPU oracle for the Kimi Delta Attention (KDA) recurrence — TEST INFRASTRUCTURE.

This module is the plain, slow, obviously correct reference that the HIP
library is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does, and
it shares no code with the HIP kernels or their binding.

Everything is fp64 numpy and runs token by token, in the order the pages give:

* The update, from "Kimi K3：架构与 SGLang Day-0 Support" (yichizhang.dev),
  section "attention 机制详解：KDA", math-details box:
      S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
  alpha_t in (0,1)^{d_k} scales row j of S (rows are key channels), beta_t is a
  scalar.  The same box splits one step into a gate and a delta write:
      S~ = Diag(alpha_t) S_{t-1};  r_old = S~^T k_t;  S_t = S~ + beta_t k_t (v_t - r_old)^T.
  ``recurrence`` computes exactly this split (it is the full update with the
  product multiplied out; no reordering beyond that).
* The readout o = S^T q, read after the write, from the same page's
  "attention 机制详解：linear attention" section.
* The gate enters as its log: g = log(alpha), one fp32 value per key channel,
  as the raw per-step inputs (v, k, gk, beta) are named in "SGLang 和 Miles 为
  Kimi K3 提供首日支持", section "ReplaySSM：针对 KDA 状态的原始输入重放".
* Segment fragments (M, S~) and their composition S_in2 = M1 S_in1 + S~1, with
  M_t = (I - beta_t k_t k_t^T) Diag(alpha_t), from "Kimi K3 的训练与 Serving
  Infra：KDA 换掉 attention 后，系统要重做什么", sections 4.1 and 4.2 (KCP).
* Verify then commit: the verify pass reads the committed state and never
  writes it; the commit replays only the accepted prefix from that state, per
  the ReplaySSM section above and section 7 of the training/serving-infra page.

Readings taken where the pages are silent: q is multiplied by ``scale``
(default 1; the pages print o = S^T q with no factor); sequences in a packed
batch are independent and each starts from its own initial state (zeros if
none); an accepted length L counts the accepted positions, so the committed
state is the state after tokens 1..L.

Pins (tests/test_oracle.py): the per-step readout identity for unit keys, the
beta = 0 closed form (pure channel decay), beta = 1 replacement, the pages'
two-dimensional teaching slice, brute-force products of explicit d x d
matrices on tiny shapes, split-and-compose against the unsplit run, affinity
and non-expansiveness of M.  No function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "recurrence",
    "prefill",
    "decode_step",
    "verify_block",
    "transition",
    "segment_fragments",
    "compose",
    "rel_l2",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def recurrence(q, k, v, g, beta, S0=None, scale=1.0):
    """One (sequence, head): o_t = S_t^T (scale q_t) after each token's update.

    q, k, g: [T, d_k]; v: [T, d_v]; beta: [T]; S0: [d_k, d_v] or None (zeros).
    Returns (o [T, d_v], S_T [d_k, d_v]) in fp64.
    """
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.empty((T, dv))
    for t in range(T):
        alpha = np.exp(g[t])                  # per-key-channel retention
        S_gated = alpha[:, None] * S          # Diag(alpha) S: scales row j by alpha[j]
        r_old = S_gated.T @ k[t]              # prediction along the current key
        u = beta[t] * (v[t] - r_old)          # delta write strength times residual
        S = S_gated + np.outer(k[t], u)       # write along k_t
        o[t] = S.T @ (scale * q[t])           # read after the write
    return o, S


def prefill(q, k, v, g, beta, cu_seqlens, S0=None, scale=1.0, heads=None):
    """Packed ragged batch: q,k,g [T_total, H, d_k]; v [T_total, H, d_v]; beta [T_total, H].

    cu_seqlens: [N + 1] offsets; S0: [N, H, d_k, d_v] or None.  Each sequence and
    head runs ``recurrence`` independently.  ``heads`` restricts the work to a
    subset of heads (the other entries of the result are left as NaN).
    Returns (o [T_total, H, d_v], S_final [N, H, d_k, d_v]).
    """
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    T, H, dk = k.shape
    dv = v.shape[2]
    o = np.full((T, H, dv), np.nan)
    S_final = np.full((N, H, dk, dv), np.nan)
    hs = range(H) if heads is None else heads
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        for h in hs:
            s0 = None if S0 is None else S0[n, h]
            o_nh, S_nh = recurrence(q[a:b, h], k[a:b, h], v[a:b, h], g[a:b, h], beta[a:b, h], s0, scale)
            o[a:b, h] = o_nh
            S_final[n, h] = S_nh
    return o, S_final


def prefill_checkpoints(k, v, g, beta, cu_seqlens, interval, S0=None):
    """States at chunk boundaries of a packed batch: for each sequence (length L)
    and m = 1, 2, ... with m * interval < L, the state after its first
    m * interval tokens, in sequence order (the rows a checkpointed prefill
    stores; a fixed-size state is what a prefix cache keeps, per the serving
    pages).  Each state is ``recurrence`` chained over the interval-long pieces.
    Returns [n_ckpt, H, d_k, d_v].
    """
    k, v, g, beta = _f64(k), _f64(v), _f64(g), _f64(beta)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, dk = k.shape
    dv = v.shape[2]
    out = []
    for n in range(cu.shape[0] - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        m_count = (b - a - 1) // interval if b > a else 0
        rows = np.empty((m_count, H, dk, dv))
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[n, h], dtype=np.float64)
            for m in range(m_count):
                lo, hi = a + m * interval, a + (m + 1) * interval
                zq = np.zeros((hi - lo, dk))
                _, S = recurrence(zq, k[lo:hi, h], v[lo:hi, h], g[lo:hi, h], beta[lo:hi, h], S)
                rows[m, h] = S
        out.append(rows)
    return np.concatenate(out, axis=0) if out else np.empty((0, H, dk, dv))


def decode_step(q, k, v, g, beta, S, scale=1.0):
    """One token per request: q,k,g [N, H, d_k]; v [N, H, d_v]; beta [N, H]; S [N, H, d_k, d_v].

    Returns (o [N, H, d_v], S_new [N, H, d_k, d_v]); the input S is not modified.
    """
    q, k, v, g, beta, S = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta), _f64(S)
    N, H, dk = k.shape
    dv = v.shape[2]
    o = np.empty((N, H, dv))
    S_new = np.empty_like(S)
    for n in range(N):
        for h in range(H):
            o_nh, S_nh = recurrence(q[n, h][None], k[n, h][None], v[n, h][None],
                                    g[n, h][None], beta[n, h][None], S[n, h], scale)
            o[n, h] = o_nh[0]
            S_new[n, h] = S_nh
    return o, S_new


def verify_block(q, k, v, g, beta, S0, accepted_len=None, scale=1.0):
    """Draft-block verify from a read-only committed state, then the commit.

    q,k,g [N, G, H, d_k]; v [N, G, H, d_v]; beta [N, G, H]; S0 [N, H, d_k, d_v];
    accepted_len [N] in 1..G or None.  Returns (o [N, G, H, d_v], S_commit) where
    S_commit [N, H, d_k, d_v] is S0 advanced by the first accepted_len[n] tokens,
    obtained by replaying those tokens from S0 (None if accepted_len is None).
    """
    q, k, v, g, beta, S0 = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta), _f64(S0)
    N, G, H, dk = k.shape
    dv = v.shape[3]
    o = np.empty((N, G, H, dv))
    S_commit = None if accepted_len is None else np.empty_like(S0)
    for n in range(N):
        for h in range(H):
            o_nh, _ = recurrence(q[n, :, h], k[n, :, h], v[n, :, h], g[n, :, h], beta[n, :, h],
                                 S0[n, h], scale)
            o[n, :, h] = o_nh
            if accepted_len is not None:
                L = int(accepted_len[n])
                _, S_L = recurrence(q[n, :L, h], k[n, :L, h], v[n, :L, h], g[n, :L, h],
                                    beta[n, :L, h], S0[n, h], scale)
                S_commit[n, h] = S_L
    return o, S_commit


def transition(k, g, beta):
    """M = M_T ... M_1 with M_t = (I - beta_t k_t k_t^T) Diag(alpha_t), as explicit d_k x d_k products."""
    k, g, beta = _f64(k), _f64(g), _f64(beta)
    T, dk = k.shape
    M = np.eye(dk)
    for t in range(T):
        M_t = (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(g[t]))
        M = M_t @ M
    return M


def segment_fragments(k, v, g, beta):
    """(M, S~) of one segment: its transition and the state it produces from zero."""
    M = transition(k, g, beta)
    T, dk = np.shape(k)
    dummy_q = np.zeros((T, dk))
    _, S_tilde = recurrence(dummy_q, k, v, g, beta, None)
    return M, S_tilde


def compose(M, S_tilde, S_in0=None):
    """Entry states of consecutive segments: S_in[0] = S_in0, S_in[i+1] = M[i] S_in[i] + S~[i].

    M: [n, d_k, d_k]; S_tilde: [n, d_k, d_v].  Returns (S_in [n, d_k, d_v], S_final).
    """
    M, S_tilde = _f64(M), _f64(S_tilde)
    n, dk, dv = S_tilde.shape
    S = np.zeros((dk, dv)) if S_in0 is None else _f64(S_in0).copy()
    S_in = np.empty((n, dk, dv))
    for i in range(n):
        S_in[i] = S
        S = M[i] @ S + S_tilde[i]
    return S_in, S


def rel_l2(x, ref):
    """||x - ref||_2 / ||ref||_2 over the whole tensor, in fp64."""
    x, ref = _f64(x), _f64(ref)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return float(num / den) if den > 0 else float(num)
