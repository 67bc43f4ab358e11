"""Host-side checks of the seeded input generators (no GPU)."""
import numpy as np
import torch

from gated_delta_rule_15_amd import inputs as gen


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10 ** rng.uniform(-8, 8, 10000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, np.inf, -np.inf], dtype=np.float32)])
    bits = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    back = gen.bf16_bits_to_f32(bits)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_packed_batch_deterministic_and_shaped():
    a = gen.packed_batch(3, [70, 5], H=2, dk=16, dv=8, dtype="bf16", init_state=[False, True])
    b = gen.packed_batch(3, [70, 5], H=2, dk=16, dv=8, dtype="bf16", init_state=[False, True])
    for name in ("q", "k", "v", "g", "beta", "cu_seqlens", "initial_state"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    assert a.q.shape == (75, 2, 16) and a.v.shape == (75, 2, 8) and a.beta.shape == (75, 2)
    assert list(a.cu_seqlens) == [0, 70, 75]
    assert np.all(a.initial_state[0] == 0) and np.any(a.initial_state[1] != 0)
    # keys are unit length before the cast; after bf16 rounding within 2^-8
    kn = np.linalg.norm(a.f64("k"), axis=-1)
    assert np.all(np.abs(kn - 1) < 8e-3)
    assert np.all(a.g <= 0) and np.all(a.g > -0.1 - 1e-7)
    assert np.all((a.beta > 0) & (a.beta < 1))


def test_slices_are_independent_of_batch_composition():
    """A (sequence, head) slice depends only on (seed, seq, head): adding sequences after it changes nothing."""
    a = gen.packed_batch(9, [33], H=3, dk=8, dv=8, dtype="f32")
    b = gen.packed_batch(9, [33, 12], H=3, dk=8, dv=8, dtype="f32")
    np.testing.assert_array_equal(a.q, b.q[:33])
    np.testing.assert_array_equal(a.g, b.g[:33])


def test_accepted_lengths_distribution():
    acc = gen.accepted_lengths(4, 20000, 8)
    assert acc.min() >= 1 and acc.max() <= 8
    assert abs(acc.mean() - (1 - 0.64 ** 8) / 0.36) < 0.05


def test_loguniform_lengths_range():
    ls = gen.loguniform_lengths(5, 1000)
    assert min(ls) >= 1024 and max(ls) < 32768
