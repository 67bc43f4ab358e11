"""The roof probes: the memory-roof copies (kda_copy_probe, kda_copy_probe_state) copy exactly, including a
partial last workgroup and in place; the matrix-roof probe keeps its work and counts its flops."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [4, 8188, 8192, 8196, 64 * 12 * 128 * 128])
def test_copy_probe_copies_exactly(n):
    from gated_delta_rule_15_amd.kda import copy_probe
    g = torch.Generator(device="cuda:0").manual_seed(n)
    src = torch.randn(n, device="cuda:0", generator=g)
    dst = torch.full((n + 4,), 7.0, device="cuda:0")
    copy_probe(src, dst[:n])
    torch.cuda.synchronize()
    assert torch.equal(dst[:n].view(torch.int32), src.view(torch.int32))
    assert torch.equal(dst[n:], torch.full((4,), 7.0, device="cuda:0"))  # nothing past the end


@pytest.mark.parametrize("dependent", [False, True])
@pytest.mark.parametrize("n_states", [1, 3, 64 * 12])
def test_copy_probe_state_copies_exactly(n_states, dependent):
    """The decode-pattern copy (either ordering) moves every element of every state (out of place, nothing
    past the end) and rewrites a state unchanged in place."""
    from gated_delta_rule_15_amd.kda import copy_probe_state
    g = torch.Generator(device="cuda:0").manual_seed(n_states)
    src = torch.randn((n_states, 128, 128), device="cuda:0", generator=g)
    dst = torch.full((n_states + 1, 128, 128), 7.0, device="cuda:0")
    copy_probe_state(src, dst[:n_states], dependent)
    keep = src.clone()
    copy_probe_state(src, src, dependent)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n_states].view(torch.int32), keep.view(torch.int32))
    assert torch.equal(dst[n_states:], torch.full((1, 128, 128), 7.0, device="cuda:0"))
    assert torch.equal(src.view(torch.int32), keep.view(torch.int32))


def test_mfma_probe_is_deterministic_and_counts_its_flops():
    """The matrix-roof probe keeps its work (finite accumulators, stored), gives the same result on a second
    launch, and reports blocks x 4 waves x iters (rounded up to a multiple of 4) x 8 products of 16 x 16 x 32 x 2 flops."""
    from gated_delta_rule_15_amd.kda import mfma_probe
    blocks, iters = 64, 50  # rounded up to 52: the probe runs whole rounds of four
    a = torch.full((blocks * 1024,), float("nan"), device="cuda:0")
    b = torch.empty_like(a)
    fa = mfma_probe(a, blocks, iters)
    fb = mfma_probe(b, blocks, iters)
    torch.cuda.synchronize()
    assert fa == fb == blocks * 4 * 52 * 8 * 16 * 16 * 32 * 2
    assert torch.isfinite(a).all() and (a != 0).any()
    assert torch.equal(a, b)
