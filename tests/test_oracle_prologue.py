"""Pins of the prologue oracle (no GPU): what the math and the page fix about
the key/query normalisation and the lower-bounded log-decay."""
import numpy as np

from oracle import kda_oracle as orc
from oracle import kda_prologue as pro


def test_l2_normalize_gives_unit_vectors_along_the_input():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 3, 128)) * rng.uniform(0.1, 10.0, (50, 3, 1))
    y = pro.l2_normalize(x, eps=0.0)
    assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=0, atol=1e-14)
    cos = np.sum(x * y, axis=-1) / np.linalg.norm(x, axis=-1)
    assert np.allclose(cos, 1.0, rtol=0, atol=1e-14)
    # positive rescaling of the input changes nothing (eps = 0)
    assert np.allclose(pro.l2_normalize(7.5 * x, eps=0.0), y, rtol=0, atol=1e-14)


def test_l2_normalize_eps_inside_the_root():
    x = np.zeros(128)
    assert np.all(pro.l2_normalize(x, eps=1e-6) == 0.0)      # zero stays finite
    x[3] = 1e-3                                               # |x|^2 = 1e-6 = eps: norm 1/sqrt(2)
    assert abs(np.linalg.norm(pro.l2_normalize(x, eps=1e-6)) - 2 ** -0.5) < 1e-15


def test_gate_is_a_scaled_sigmoid_with_the_printed_bound():
    x = np.linspace(-30, 30, 3001)                              # (fp64 sigmoid saturates to 1 beyond ~37)
    g = pro.gate_log_decay(x, g_min=-5.0)
    assert np.all(g < 0) and np.all(g > -5.0)                 # inside (g_min, 0)
    assert np.all(np.diff(g) < 0)                              # one orientation: monotone in x
    assert pro.gate_log_decay(0.0) == -2.5                     # midpoint g_min / 2
    assert np.allclose(g + pro.gate_log_decay(-x), -5.0, rtol=0, atol=1e-12)  # sigmoid symmetry
    assert abs(pro.gate_log_decay(-40.0)) < 1e-16 and abs(pro.gate_log_decay(40.0) + 5.0) < 1e-16
    # the page: each step keeps more than e^-5 ~ 6.7e-3 of the state
    assert np.all(np.exp(g) > 6.7e-3) and abs(np.exp(-5.0) - 6.7e-3) < 1e-4


def test_unit_key_readout_identity_after_normalisation():
    """The box's identity S_t^T k_t = (1 - beta) (Diag(alpha) S)^T k_t + beta v_t needs unit keys:
    it holds for prologue-normalised raw keys (eps = 0) and fails for the raw ones."""
    rng = np.random.default_rng(1)
    d, T = 16, 6
    q, k, g, = rng.standard_normal((T, d)) * 3, rng.standard_normal((T, d)) * 3, rng.standard_normal((T, d))
    v, beta = rng.standard_normal((T, 4)), rng.uniform(0.1, 0.9, T)
    S0 = rng.standard_normal((d, 4))
    qn, kn, gn = pro.apply_prologue(q, k, g, eps=0.0, g_min=-5.0)
    S = S0.copy()
    for t in range(T):
        r_old = (np.exp(gn[t])[:, None] * S).T @ kn[t]
        _, S_next = orc.recurrence(qn[t:t + 1], kn[t:t + 1], v[t:t + 1], gn[t:t + 1], beta[t:t + 1], S)
        assert np.allclose(S_next.T @ kn[t], (1 - beta[t]) * r_old + beta[t] * v[t], atol=1e-12)
        S = S_next
    # raw keys of norm ~ 3 * 4: the identity does not hold
    _, S_raw = orc.recurrence(q[:1], k[:1], v[:1], g[:1], beta[:1], S0)
    r_raw = (np.exp(g[0])[:, None] * S0).T @ k[0]
    assert not np.allclose(S_raw.T @ k[0], (1 - beta[0]) * r_raw + beta[0] * v[0], atol=1e-3)
