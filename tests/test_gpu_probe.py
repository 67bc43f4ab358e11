"""The memory-roof probe (kda_copy_probe) copies exactly, including a partial last workgroup."""
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
