"""Helpers shared by the GPU tests: move seeded inputs to the device and back."""
import numpy as np
import torch

from gated_delta_rule_15_amd import inputs as gen

DEV = "cuda:0"


def to_dev(x: np.ndarray, dtype: str = "f32") -> torch.Tensor:
    """numpy array -> device tensor; bf16 inputs arrive as uint16 bit patterns."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def packed_to_dev(p: gen.Packed):
    d = dict(q=to_dev(p.q, p.dtype), k=to_dev(p.k, p.dtype), v=to_dev(p.v, p.dtype),
             g=to_dev(p.g), beta=to_dev(p.beta), cu_seqlens=to_dev(p.cu_seqlens),
             cu_seqlens_host=torch.from_numpy(p.cu_seqlens.copy()))
    d["initial_state"] = None if p.initial_state is None else to_dev(p.initial_state)
    return d


def steps_to_dev(b: gen.StepBatch, squeeze_g: bool = False):
    def sq(x):
        return x[:, 0] if squeeze_g else x
    d = dict(q=to_dev(sq(b.q), b.dtype), k=to_dev(sq(b.k), b.dtype), v=to_dev(sq(b.v), b.dtype),
             g=to_dev(sq(b.g)), beta=to_dev(sq(b.beta)), state=to_dev(b.state))
    if b.accepted_len is not None:
        d["accepted_len"] = to_dev(b.accepted_len)
    return d


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


def bf16_floor(ref) -> float:
    """rel-L2 of rounding the exact reference itself to bf16 (the output-format floor)."""
    r32 = np.asarray(ref, dtype=np.float32)
    rb = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(r32)).astype(np.float64)
    return rel_l2(rb, ref)
