"""CPU oracle for the KDA input prologue — TEST INFRASTRUCTURE.

Like ``kda_oracle``, this is the plain fp64 reference the HIP library is
checked against; only the test suite may import it, and it shares no code
with the kernels.

The prologue turns the raw per-token inputs into the ones the recurrence
consumes ("Kimi K3：架构与 SGLang Day-0 Support", section "attention 机制详解：
KDA", math-details box):

* Unit keys and queries.  The box's readout identity S_t^T k_t =
  (1 - beta) r_old + beta v holds for unit k_t, so keys (and queries) are
  L2-normalised per token and head: x / sqrt(sum x^2 + eps).  Reading: eps
  sits inside the square root (it keeps the zero vector finite), 1e-6 by
  default; the page gives no eps.
* A lower-bounded log-decay.  The box bounds the log-decay of alpha below with
  a scaled sigmoid, g_min = -5, so that every step keeps more than e^-5 of the
  state.  Reading: g = g_min * sigmoid(x) for the gate logit x, one value per
  key channel.  The bound, its value and the sigmoid shape are the page's; the
  orientation (sigmoid(x) rather than sigmoid(-x)) is not printed, so that
  detail is parity unpinned: the tests pin everything the two orientations
  share (range, midpoint, symmetry, monotonicity, the printed retention bound)
  and one orientation is chosen.
"""
from __future__ import annotations

import numpy as np

__all__ = ["l2_normalize", "gate_log_decay", "apply_prologue"]


def l2_normalize(x, eps=1e-6):
    """x / sqrt(sum(x^2) + eps) over the last axis, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def gate_log_decay(x, g_min=-5.0):
    """g = g_min * sigmoid(x), in fp64: a log-decay in (g_min, 0)."""
    x = np.asarray(x, dtype=np.float64)
    return g_min / (1.0 + np.exp(-x))


def apply_prologue(q, k, g_raw, l2norm=True, eps=1e-6, gate_logits=True, g_min=-5.0):
    """The inputs the recurrence sees: (q, k, g) after the optional normalisation and gate map."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    g = np.asarray(g_raw, dtype=np.float64)
    if l2norm:
        q, k = l2_normalize(q, eps), l2_normalize(k, eps)
    if gate_logits:
        g = gate_log_decay(g, g_min)
    return q, k, g
