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
