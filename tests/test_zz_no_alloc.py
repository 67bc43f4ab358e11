"""GPU test of the allocation-free prefill (kda_prefill_noalloc) through the C ABI.

Two calls in a row share the library's per-device scratch, the second with a
smaller input; each must equal kda_prefill_ex with a caller workspace bit for
bit (the same kernels), and the oracle within the bf16 bar.  A call that
would need more scratch than the library holds is rejected with
KDA_ERR_WORKSPACE.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_15_amd import inputs as gen
from oracle import kda_oracle as orc

from kda_testutil import check_parity, packed_slices, packed_to_dev, unit_slices

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(p):
    from gated_delta_rule_15_amd.kda import kda_prefill, kda_prefill_noalloc, kda_prefill_workspace
    d = packed_to_dev(p)
    N, H = p.num_seqs, p.H
    ws = kda_prefill_workspace(N, p.T, H, d["q"].dtype, "cuda:0")
    assert ws is not None  # a grid this small takes the split path, which uses the workspace / scratch
    o1, S1 = kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["cu_seqlens_host"],
                         initial_state=d["initial_state"], workspace=ws)
    o2 = torch.full_like(o1, 3.0)
    S2 = torch.full((N, H, 128, 128), 5.0, device="cuda:0")
    torch.cuda.synchronize()
    kda_prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["cu_seqlens_host"], o=o2,
                        final_state=S2, initial_state=d["initial_state"])
    torch.cuda.synchronize()
    return (o1, S1), (o2, S2)


def test_noalloc_equals_workspace_path_twice():
    """A 4096-token x 12-head prefill (104 MB of scratch), then a smaller ragged batch with initial
    states: each equals the workspace path bit for bit, and the oracle."""
    for p in (gen.packed_batch(seed=3, seqlens=[4096], H=12, dtype="bf16"),
              gen.packed_batch(seed=71, seqlens=[300, 0, 77, 5], H=3, dtype="bf16", init_state=True)):
        (o1, S1), (o2, S2) = _both(p)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(S1.view(torch.int32), S2.view(torch.int32))
        o_ref, S_ref = orc.prefill(p.f64("q"), p.f64("k"), p.f64("v"), p.f64("g"), p.f64("beta"), p.cu_seqlens,
                                   p.initial_state)
        check_parity(o2, o_ref, 2e-3, packed_slices(p.cu_seqlens, p.H), bf16_out=True, tag=f"noalloc T={p.T} o")
        check_parity(S2, S_ref, 2e-3, unit_slices(p.num_seqs, p.H), tag=f"noalloc T={p.T} S")


def test_noalloc_rejects_more_than_its_scratch():
    from gated_delta_rule_15_amd import _lib
    from gated_delta_rule_15_amd.kda import kda_prefill_noalloc, kda_prefill_workspace_size
    lib = _lib.load()
    cap = lib.kda_prefill_noalloc_max_scratch()
    T, H = 32 * 1024, 4  # 4 heads x 1,025 chunk slots x 66,560 bytes: 273 MB
    assert kda_prefill_workspace_size(1, T, H, torch.bfloat16) > cap
    q = torch.zeros((T, H, 128), dtype=torch.bfloat16, device="cuda:0")
    g = torch.zeros((T, H, 128), device="cuda:0")
    beta = torch.zeros((T, H), device="cuda:0")
    cu = torch.tensor([0, T], dtype=torch.int32)
    o = torch.empty_like(q)
    with pytest.raises(_lib.KdaError, match="workspace"):
        kda_prefill_noalloc(q, q, q, g, beta, cu.to("cuda:0"), cu, o=o)
