"""Thin torch binding of the KDA C ABI (include/kda.h).

Argument marshalling only: shape/dtype/device checks, output allocation with
torch, raw pointers and the current HIP stream handed to libkda.so.  Every
step of the computation runs in the library's HIP kernels; there is no CPU
fallback, and a missing library raises ``KdaError``.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib

D = 128


@dataclass(frozen=True)
class Prologue:
    """Input prologue applied inside the kernels (kda_prologue_t): per-token L2 normalisation of q
    and k, x / sqrt(sum x^2 + eps), and gate logits x -> log-decay g_min * sigmoid(x)."""
    l2norm_qk: bool = True
    l2norm_eps: float = 1e-6
    gate_logits: bool = True
    g_min: float = -5.0

    def _c(self) -> "_lib.KdaPrologue":
        return _lib.KdaPrologue(int(bool(self.l2norm_qk)), float(self.l2norm_eps), int(bool(self.gate_logits)),
                                float(self.g_min))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.KDA_BF16
    if t.dtype == torch.float32:
        return _lib.KDA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _need(t: Optional[torch.Tensor], name: str, shape, dtype=None, device=None) -> None:
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def kda_decode_step(q, k, v, g, beta, state_pool, o=None, slots=None, scale: float = 1.0,
                    with_output: bool = True, prologue: Optional[Prologue] = None):
    """One token per request; ``state_pool`` [P, H, 128, 128] fp32 is updated in place.

    q, k, v, g: [N, H, 128]; beta: [N, H]; slots: int32 [N] pool rows (None = 0..N-1).
    Returns o [N, H, 128] (dtype of q) or None when ``with_output`` is False.
    With ``prologue`` the call goes to kda_decode_step_prologue (raw q, k; g may hold gate logits).
    """
    N, H, _ = q.shape
    dt = q.dtype
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (N, H, D), dt, dev)
    _need(g, "g", (N, H, D), torch.float32, dev)
    _need(beta, "beta", (N, H), torch.float32, dev)
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, D, D):
        raise ValueError("state_pool must be [P, H, 128, 128]")
    _need(state_pool, "state_pool", state_pool.shape, torch.float32, dev)
    if slots is None and state_pool.shape[0] < N:
        raise ValueError("state_pool has fewer rows than requests")
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    if with_output and o is None:
        o = torch.empty((N, H, D), dtype=dt, device=dev)
    _need(o, "o", (N, H, D), dt, dev)
    lib = _lib.load()
    if prologue is None:
        _lib.check(lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
                                       _ptr(slots), N, H, D, D, _dtype_code(q), float(scale), _ptr(o), _stream()),
                   "kda_decode_step")
    else:
        pc = prologue._c()
        _lib.check(lib.kda_decode_step_prologue(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
                                                _ptr(slots), N, H, D, D, _dtype_code(q), float(scale), _ptr(o),
                                                ctypes.addressof(pc), _stream()),
                   "kda_decode_step_prologue")
    return o


def kda_decode_step_prologue(q, k, v, g, beta, state_pool, prologue: Prologue, **kw):
    """kda_decode_step with the input prologue (required)."""
    if prologue is None:
        raise ValueError("prologue is required")
    return kda_decode_step(q, k, v, g, beta, state_pool, prologue=prologue, **kw)


def kda_verify_block(q, k, v, g, beta, state_pool, o=None, slots=None, accepted_len=None,
                     state_out_pool=None, scale: float = 1.0, prologue: Optional[Prologue] = None):
    """Verify gamma1 draft tokens per request from the committed (read-only) states.

    q, k, v, g: [N, G, H, 128]; beta: [N, G, H].  Returns o [N, G, H, 128].
    With ``accepted_len`` (int32 [N] on the device) the commit of the accepted
    prefix is also enqueued, into ``state_out_pool`` (defaults to ``state_pool``).
    """
    N, G, H, _ = q.shape
    dt = q.dtype
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (N, G, H, D), dt, dev)
    _need(g, "g", (N, G, H, D), torch.float32, dev)
    _need(beta, "beta", (N, G, H), torch.float32, dev)
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, D, D):
        raise ValueError("state_pool must be [P, H, 128, 128]")
    _need(state_pool, "state_pool", state_pool.shape, torch.float32, dev)
    if slots is None and state_pool.shape[0] < N:
        raise ValueError("state_pool has fewer rows than requests")
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    if o is None:
        o = torch.empty((N, G, H, D), dtype=dt, device=dev)
    _need(o, "o", (N, G, H, D), dt, dev)
    if accepted_len is not None:
        _need(accepted_len, "accepted_len", (N,), torch.int32, dev)
        if state_out_pool is None:
            state_out_pool = state_pool
        _need(state_out_pool, "state_out_pool", state_pool.shape, torch.float32, dev)
    lib = _lib.load()
    if prologue is None:
        _lib.check(lib.kda_verify_block(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
                                        _ptr(slots), N, G, H, D, D, _dtype_code(q), float(scale), _ptr(o),
                                        _ptr(accepted_len), _ptr(state_out_pool), _stream()),
                   "kda_verify_block")
    else:
        pc = prologue._c()
        _lib.check(lib.kda_verify_block_prologue(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
                                                 _ptr(slots), N, G, H, D, D, _dtype_code(q), float(scale), _ptr(o),
                                                 _ptr(accepted_len), _ptr(state_out_pool), ctypes.addressof(pc),
                                                 _stream()),
                   "kda_verify_block_prologue")
    return o


def kda_verify_block_prologue(q, k, v, g, beta, state_pool, prologue: Prologue, **kw):
    """kda_verify_block with the input prologue (required)."""
    if prologue is None:
        raise ValueError("prologue is required")
    return kda_verify_block(q, k, v, g, beta, state_pool, prologue=prologue, **kw)


def kda_verify_commit(k, v, g, beta, state_pool, accepted_len, slots=None, prologue: Optional[Prologue] = None):
    """Replay each request's accepted prefix from its committed state, in place (with ``prologue``:
    the one the verify used)."""
    N, G, H, _ = k.shape
    dt = k.dtype
    dev = k.device
    _need(k, "k", (N, G, H, D), dt, dev)
    _need(v, "v", (N, G, H, D), dt, dev)
    _need(g, "g", (N, G, H, D), torch.float32, dev)
    _need(beta, "beta", (N, G, H), torch.float32, dev)
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, D, D):
        raise ValueError("state_pool must be [P, H, 128, 128]")
    _need(state_pool, "state_pool", state_pool.shape, torch.float32, dev)
    _need(accepted_len, "accepted_len", (N,), torch.int32, dev)
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    elif state_pool.shape[0] < N:
        raise ValueError("state_pool has fewer rows than requests")
    lib = _lib.load()
    if prologue is None:
        _lib.check(lib.kda_verify_commit(_ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool), _ptr(slots),
                                         _ptr(accepted_len), N, G, H, D, D, _dtype_code(k), _stream()),
                   "kda_verify_commit")
    else:
        pc = prologue._c()
        _lib.check(lib.kda_verify_commit_prologue(_ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
                                                  _ptr(slots), _ptr(accepted_len), N, G, H, D, D, _dtype_code(k),
                                                  ctypes.addressof(pc), _stream()),
                   "kda_verify_commit_prologue")


def kda_verify_block_record(q, k, v, g, beta, state_pool, prologue: Prologue, record=None, o=None, slots=None,
                            scale: float = 1.0):
    """kda_verify_block_record: the prologue verify that also writes its raw-input record (the key and
    log-decay of every draft step as used, [N, G, H, 2, 128] fp32).  Returns (o, record)."""
    if prologue is None:
        raise ValueError("prologue is required")
    N, G, H, _ = q.shape
    dt, dev = q.dtype, q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (N, G, H, D), dt, dev)
    _need(g, "g", (N, G, H, D), torch.float32, dev)
    _need(beta, "beta", (N, G, H), torch.float32, dev)
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, D, D):
        raise ValueError("state_pool must be [P, H, 128, 128]")
    _need(state_pool, "state_pool", state_pool.shape, torch.float32, dev)
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    elif state_pool.shape[0] < N:
        raise ValueError("state_pool has fewer rows than requests")
    if o is None:
        o = torch.empty((N, G, H, D), dtype=dt, device=dev)
    _need(o, "o", (N, G, H, D), dt, dev)
    if record is None:
        record = torch.empty((N, G, H, 2, D), dtype=torch.float32, device=dev)
    _need(record, "record", (N, G, H, 2, D), torch.float32, dev)
    pc = prologue._c()
    _lib.check(_lib.load().kda_verify_block_record(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
                                                   _ptr(slots), N, G, H, D, D, _dtype_code(q), float(scale), _ptr(o),
                                                   _ptr(record), ctypes.addressof(pc), _stream()),
               "kda_verify_block_record")
    return o, record


def kda_verify_commit_record(record, v, beta, state_pool, accepted_len, slots=None):
    """kda_verify_commit_record: replay each request's accepted prefix, in place, from the verify's record
    (keys and log-decays as the verify used them) with v and beta as given."""
    N, G, H, _ = v.shape
    dev = v.device
    _need(record, "record", (N, G, H, 2, D), torch.float32, dev)
    _need(v, "v", (N, G, H, D), v.dtype, dev)
    _need(beta, "beta", (N, G, H), torch.float32, dev)
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, D, D):
        raise ValueError("state_pool must be [P, H, 128, 128]")
    _need(state_pool, "state_pool", state_pool.shape, torch.float32, dev)
    _need(accepted_len, "accepted_len", (N,), torch.int32, dev)
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    elif state_pool.shape[0] < N:
        raise ValueError("state_pool has fewer rows than requests")
    _lib.check(_lib.load().kda_verify_commit_record(_ptr(record), _ptr(v), _ptr(beta), _ptr(state_pool), _ptr(slots),
                                                    _ptr(accepted_len), N, G, H, D, D, _dtype_code(v), _stream()),
               "kda_verify_commit_record")


def kda_verify_commit_prologue(k, v, g, beta, state_pool, accepted_len, prologue: Prologue, **kw):
    """kda_verify_commit with the input prologue (required)."""
    if prologue is None:
        raise ValueError("prologue is required")
    return kda_verify_commit(k, v, g, beta, state_pool, accepted_len, prologue=prologue, **kw)


def kda_prefill(q, k, v, g, beta, cu_seqlens, cu_seqlens_host=None, initial_state=None, final_state=None,
                o=None, transition_out=None, scale: float = 1.0, with_output: bool = True,
                with_final_state: bool = True, prologue: Optional[Prologue] = None, workspace="auto",
                ws_flags: int = 0):
    """Chunked prefill of a packed ragged batch.

    q, k, v, g: [T, H, 128]; beta: [T, H]; cu_seqlens: int32 [N + 1] on the device
    (``cu_seqlens_host``: optional CPU int32 copy, validated by the library).
    Returns (o or None, final_state or None).  ``final_state`` may be the same
    tensor as ``initial_state`` (in-place continuation).  With ``prologue`` the call goes to
    kda_prefill_prologue (raw q, k; g may hold gate logits).

    ``workspace``: "auto" allocates what ``kda_prefill_workspace_size`` asks for (nothing for a
    grid that fills the device, without ``cu_seqlens_host``, or above AUTO_WORKSPACE_MAX), so small
    grids take the split path (kda_prefill_ex); a device uint8 tensor is used as given; None takes
    the single-kernel path.  ``ws_flags``: KDA_WS_PREPARED / KDA_WS_KEEP_OUTPUT_OPERANDS of kda_prefill_ex, for
    two calls over the same rows that share one workspace preparation.
    """
    return _prefill(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, initial_state, final_state, o, transition_out,
                    scale, with_output, with_final_state, None, prologue, workspace, ws_flags)


def copy_probe(src: torch.Tensor, dst: torch.Tensor) -> None:
    """kda_copy_probe: the memory-roof probe, a nontemporal float4 copy of src into dst (contiguous fp32
    device tensors of one size, a multiple of 4 elements)."""
    if src.dtype != torch.float32 or dst.dtype != torch.float32 or not src.is_cuda or dst.device != src.device:
        raise ValueError("copy_probe takes fp32 tensors on one device")
    if not src.is_contiguous() or not dst.is_contiguous() or src.numel() != dst.numel():
        raise ValueError("copy_probe takes contiguous tensors of one size")
    _lib.check(_lib.load().kda_copy_probe(_ptr(src), _ptr(dst), src.numel(), _stream()), "kda_copy_probe")


def copy_probe_state(src: torch.Tensor, dst: torch.Tensor, dependent: bool = False) -> None:
    """kda_copy_probe_state: the decode pattern's memory-roof probe, a copy of [..., 128, 128] fp32 states
    (contiguous device tensors of one shape) in the decode step's tiling; dst may be src (in place).
    ``dependent``: no store before all of the workgroup's loads are in (the decode step's ordering)."""
    if src.dtype != torch.float32 or dst.dtype != torch.float32 or not src.is_cuda or dst.device != src.device:
        raise ValueError("copy_probe_state takes fp32 tensors on one device")
    if not src.is_contiguous() or not dst.is_contiguous() or src.shape != dst.shape or src.dim() < 2 \
            or tuple(src.shape[-2:]) != (D, D):
        raise ValueError("copy_probe_state takes contiguous [..., 128, 128] tensors of one shape")
    _lib.check(_lib.load().kda_copy_probe_state(_ptr(src), _ptr(dst), src.numel() // (D * D), int(dependent),
                                                _stream()),
               "kda_copy_probe_state")


def mfma_probe(out: torch.Tensor, blocks: int, iters: int) -> int:
    """kda_mfma_probe: the matrix-roof probe (bf16 16x16x32 MFMA loop); out: fp32 device tensor of at least
    blocks x 1024 elements.  Returns the flops of the launch."""
    if out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous() or out.numel() < blocks * 1024:
        raise ValueError("mfma_probe needs a contiguous fp32 device tensor of blocks x 1024 elements")
    flops = ctypes.c_int64(0)
    _lib.check(_lib.load().kda_mfma_probe(_ptr(out), int(blocks), int(iters), ctypes.byref(flops), _stream()),
               "kda_mfma_probe")
    return int(flops.value)


# "auto" workspaces stop here: a few long sequences on few heads would need one operand set per
# 32-token chunk (about 2 KB per token and head); such calls run the single kernel, or go through
# long_context.kda_prefill_segmented, which cuts them first.
AUTO_WORKSPACE_MAX = 1 << 30


def kda_prefill_workspace_size(num_seqs: int, T_total: int, H: int, dtype: torch.dtype,
                               transitions: bool = False, outputs: bool = True) -> int:
    """Workspace bytes kda_prefill_ex can use for a call that requests transitions or not and
    outputs or not (0: the call takes the single-kernel path)."""
    code = _lib.KDA_BF16 if dtype == torch.bfloat16 else _lib.KDA_F32
    flags = (_lib.KDA_PREFILL_TRANSITIONS if transitions else 0) | (0 if outputs else _lib.KDA_PREFILL_NO_OUTPUT)
    return int(_lib.load().kda_prefill_workspace_size(int(num_seqs), int(T_total), int(H), D, D, code, flags))


def kda_prefill_workspace(num_seqs: int, T_total: int, H: int, dtype: torch.dtype, device,
                          transitions: bool = False, outputs: bool = True) -> Optional[torch.Tensor]:
    """A workspace for kda_prefill(..., workspace=...) (None when the call needs none)."""
    n = kda_prefill_workspace_size(num_seqs, T_total, H, dtype, transitions, outputs)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def kda_prefill_noalloc(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, o=None, final_state=None, initial_state=None,
                        transition_out=None, scale: float = 1.0, seq_order=None, prologue: Optional[Prologue] = None):
    """kda_prefill_noalloc: the prefill without any allocation, the split path's workspace being the
    library's per-device scratch (kda_prefill_noalloc_max_scratch() bytes).  Outputs are written only
    into the buffers passed (o [T, H, 128], final_state / transition_out [N, H, 128, 128]; None skips
    one); this wrapper allocates nothing either.  Calls that overlap on one device race on the scratch."""
    T, H, _ = q.shape
    dt, dev = q.dtype, q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (T, H, D), dt, dev)
    _need(g, "g", (T, H, D), torch.float32, dev)
    _need(beta, "beta", (T, H), torch.float32, dev)
    N = cu_seqlens.shape[0] - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if cu_seqlens_host is not None and (cu_seqlens_host.is_cuda or cu_seqlens_host.dtype != torch.int32
                                        or cu_seqlens_host.shape != cu_seqlens.shape
                                        or not cu_seqlens_host.is_contiguous()):
        raise ValueError("cu_seqlens_host must be a contiguous CPU int32 copy of cu_seqlens")
    for name, t in (("initial_state", initial_state), ("final_state", final_state),
                    ("transition_out", transition_out)):
        _need(t, name, (N, H, D, D), torch.float32, dev)
    _need(o, "o", (T, H, D), dt, dev)
    if seq_order is not None:
        _need(seq_order, "seq_order", (N,), torch.int32, dev)
    pc = prologue._c() if prologue is not None else None
    _lib.check(_lib.load().kda_prefill_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), _ptr(cu_seqlens_host), N, H, D, D,
        _dtype_code(q), float(scale), _ptr(initial_state), _ptr(final_state), _ptr(o), _ptr(transition_out),
        _ptr(seq_order), ctypes.addressof(pc) if pc is not None else None, _stream()), "kda_prefill_noalloc")
    return o, final_state


def kda_prefill_prologue(q, k, v, g, beta, cu_seqlens, prologue: Prologue, **kw):
    """kda_prefill with the input prologue (required)."""
    if prologue is None:
        raise ValueError("prologue is required")
    return kda_prefill(q, k, v, g, beta, cu_seqlens, prologue=prologue, **kw)


def kda_prefill_ordered(q, k, v, g, beta, cu_seqlens, seq_order, cu_seqlens_host=None, initial_state=None,
                        final_state=None, o=None, transition_out=None, scale: float = 1.0, with_output: bool = True,
                        with_final_state: bool = True, workspace="auto", ws_flags: int = 0,
                        prologue: Optional[Prologue] = None):
    """kda_prefill whose sequences are started in the order ``seq_order`` (device int32 [N], a
    permutation of 0..N-1; e.g. longest first).  Same results as kda_prefill, bit for bit."""
    if seq_order is None:
        raise ValueError("seq_order is required")
    return _prefill(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, initial_state, final_state, o, transition_out,
                    scale, with_output, with_final_state, seq_order, prologue, workspace, ws_flags)


def _prefill(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, initial_state, final_state, o, transition_out, scale,
             with_output, with_final_state, seq_order, prologue, workspace="auto", ws_flags: int = 0):
    T, H, _ = q.shape
    dt = q.dtype
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (T, H, D), dt, dev)
    _need(g, "g", (T, H, D), torch.float32, dev)
    _need(beta, "beta", (T, H), torch.float32, dev)
    if cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be 1-D")
    _need(cu_seqlens, "cu_seqlens", cu_seqlens.shape, torch.int32, dev)
    N = cu_seqlens.shape[0] - 1
    if cu_seqlens_host is not None:
        if cu_seqlens_host.is_cuda or cu_seqlens_host.dtype != torch.int32 or not cu_seqlens_host.is_contiguous():
            raise ValueError("cu_seqlens_host must be a contiguous CPU int32 tensor")
        if cu_seqlens_host.shape != cu_seqlens.shape:
            raise ValueError("cu_seqlens_host and cu_seqlens differ in shape")
        if int(cu_seqlens_host[-1]) > T or int(cu_seqlens_host[0]) < 0:
            raise ValueError("cu_seqlens_host must lie within the packed tokens")
    _need(initial_state, "initial_state", (N, H, D, D), torch.float32, dev)
    if with_final_state and final_state is None:
        final_state = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    _need(final_state, "final_state", (N, H, D, D), torch.float32, dev)
    if with_output and o is None:
        o = torch.empty((T, H, D), dtype=dt, device=dev)
    _need(o, "o", (T, H, D), dt, dev)
    _need(transition_out, "transition_out", (N, H, D, D), torch.float32, dev)
    lib = _lib.load()
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a device uint8 tensor')
        workspace = None
        if cu_seqlens_host is not None and N > 0:
            n = kda_prefill_workspace_size(N, int(cu_seqlens_host[-1]), H, dt, transition_out is not None,
                                               o is not None)
            if 0 < n <= AUTO_WORKSPACE_MAX:
                workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    if workspace is not None or (prologue is not None and seq_order is not None):
        # kda_prefill_ex: a workspace, or a start order with the prologue
        if workspace is not None:
            if cu_seqlens_host is None:
                raise ValueError("a workspace needs cu_seqlens_host")
            if not workspace.is_cuda or workspace.device != dev or workspace.dtype != torch.uint8 \
                    or not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
        pc = prologue._c() if prologue is not None else None
        if seq_order is not None:
            _need(seq_order, "seq_order", (N,), torch.int32, dev)
        _lib.check(lib.kda_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                      _ptr(cu_seqlens_host), N, H, D, D, _dtype_code(q), float(scale),
                                      _ptr(initial_state), _ptr(final_state), _ptr(o), _ptr(transition_out),
                                      _ptr(seq_order), ctypes.addressof(pc) if pc is not None else None,
                                      _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                      int(ws_flags), _stream()),
                   "kda_prefill_ex")
        return o, final_state
    if prologue is not None:
        pc = prologue._c()
        _lib.check(lib.kda_prefill_prologue(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                            _ptr(cu_seqlens_host), N, H, D, D, _dtype_code(q), float(scale),
                                            _ptr(initial_state), _ptr(final_state), _ptr(o), _ptr(transition_out),
                                            ctypes.addressof(pc), _stream()),
                   "kda_prefill_prologue")
    elif seq_order is None:
        _lib.check(lib.kda_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                   _ptr(cu_seqlens_host), N, H, D, D, _dtype_code(q), float(scale),
                                   _ptr(initial_state), _ptr(final_state), _ptr(o), _ptr(transition_out), _stream()),
                   "kda_prefill")
    else:
        _need(seq_order, "seq_order", (N,), torch.int32, dev)
        _lib.check(lib.kda_prefill_ordered(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                           _ptr(cu_seqlens_host), N, H, D, D, _dtype_code(q), float(scale),
                                           _ptr(initial_state), _ptr(final_state), _ptr(o), _ptr(transition_out),
                                           _ptr(seq_order), _stream()),
                   "kda_prefill_ordered")
    return o, final_state


def kda_prefill_checkpoint_count(cu_seqlens_host, ckpt_interval: int) -> int:
    """Rows kda_prefill_checkpointed writes: sum over sequences of floor((len - 1) / ckpt_interval)."""
    cu = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
    if cu.is_cuda or cu.dim() != 1:
        raise ValueError("cu_seqlens_host must be a 1-D CPU int32 array")
    n = _lib.load().kda_prefill_checkpoint_count(_ptr(cu), cu.shape[0] - 1, int(ckpt_interval))
    if n < 0:
        raise ValueError("ckpt_interval must be a positive multiple of 64 and cu_seqlens non-decreasing")
    return int(n)


def kda_prefill_checkpointed(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, ckpt_interval: int, initial_state=None,
                             final_state=None, o=None, checkpoints=None, scale: float = 1.0, with_output: bool = True,
                             with_final_state: bool = True):
    """kda_prefill that also returns the state after every ``ckpt_interval`` tokens of each sequence
    (strictly inside the sequence).  ``cu_seqlens_host`` (CPU int32) is required to size the
    checkpoint buffer.  Returns (o or None, final_state or None, checkpoints [n_ckpt, H, 128, 128])."""
    T, H, _ = q.shape
    dt = q.dtype
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (T, H, D), dt, dev)
    _need(g, "g", (T, H, D), torch.float32, dev)
    _need(beta, "beta", (T, H), torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", cu_seqlens.shape, torch.int32, dev)
    N = cu_seqlens.shape[0] - 1
    if cu_seqlens_host is None or cu_seqlens_host.is_cuda or cu_seqlens_host.dtype != torch.int32 \
            or cu_seqlens_host.shape != cu_seqlens.shape or not cu_seqlens_host.is_contiguous():
        raise ValueError("cu_seqlens_host must be a contiguous CPU int32 copy of cu_seqlens")
    if int(cu_seqlens_host[-1]) > T or int(cu_seqlens_host[0]) < 0:
        raise ValueError("cu_seqlens_host must lie within the packed tokens")
    n_ckpt = kda_prefill_checkpoint_count(cu_seqlens_host, ckpt_interval)
    _need(initial_state, "initial_state", (N, H, D, D), torch.float32, dev)
    if with_final_state and final_state is None:
        final_state = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    _need(final_state, "final_state", (N, H, D, D), torch.float32, dev)
    if with_output and o is None:
        o = torch.empty((T, H, D), dtype=dt, device=dev)
    _need(o, "o", (T, H, D), dt, dev)
    if checkpoints is None:
        checkpoints = torch.empty((max(n_ckpt, 1), H, D, D), dtype=torch.float32, device=dev)
    if checkpoints.shape[0] < n_ckpt:
        raise ValueError(f"checkpoints needs {n_ckpt} rows")
    _need(checkpoints, "checkpoints", tuple(checkpoints.shape), torch.float32, dev)
    lib = _lib.load()
    _lib.check(lib.kda_prefill_checkpointed(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                            _ptr(cu_seqlens_host), N, H, D, D, _dtype_code(q), float(scale),
                                            _ptr(initial_state), _ptr(final_state), _ptr(o), int(ckpt_interval),
                                            _ptr(checkpoints), _stream()),
               "kda_prefill_checkpointed")
    return o, final_state, checkpoints[:n_ckpt]


def kda_compose_segments(M, S_tilde, S_in0=None, S_in=None, S_final=None, with_final: bool = True,
                         split_bf16: bool = False):
    """Entry states of consecutive segments: S_in[0] = S_in0, S_in[i+1] = M[i] S_in[i] + S~[i].

    M, S_tilde: [n_seg, H, 128, 128] fp32.  Returns (S_in, S_final).  ``split_bf16``: products on
    bf16 MFMA with hi/lo split operands (kda_compose_segments_ex, KDA_COMPOSE_SPLIT_BF16).
    """
    n, H = S_tilde.shape[0], S_tilde.shape[1]
    dev = S_tilde.device
    _need(M, "M", (n, H, D, D), torch.float32, dev)
    _need(S_tilde, "S_tilde", (n, H, D, D), torch.float32, dev)
    _need(S_in0, "S_in0", (H, D, D), torch.float32, dev)
    if S_in is None:
        S_in = torch.empty((n, H, D, D), dtype=torch.float32, device=dev)
    _need(S_in, "S_in", (n, H, D, D), torch.float32, dev)
    if with_final and S_final is None:
        S_final = torch.empty((H, D, D), dtype=torch.float32, device=dev)
    _need(S_final, "S_final", (H, D, D), torch.float32, dev)
    lib = _lib.load()
    flags = _lib.KDA_COMPOSE_SPLIT_BF16 if split_bf16 else 0
    _lib.check(lib.kda_compose_segments_ex(_ptr(M), _ptr(S_tilde), _ptr(S_in0), _ptr(S_in), _ptr(S_final), n, H, D,
                                           D, flags, _stream()),
               "kda_compose_segments_ex")
    return S_in, S_final


# ---------------------------------------------------------------------------
# Batch-invariant row contract (kda_contract_* of include/kda.h)
# ---------------------------------------------------------------------------
CONTRACT_CHUNK = 16


def kda_contract_pools(P: int, H: int, device, initial_state=None):
    """Allocate contract pools for P slots: (S_pool [P, H, 128, 128] fp32 = initial_state or zeros,
    rows_pool [P, H, 16, 3, 128] fp32, pos_pool [P, H] int32 = 0)."""
    S = torch.zeros((P, H, D, D), dtype=torch.float32, device=device)
    if initial_state is not None:
        S.copy_(initial_state)
    rows = torch.zeros((P, H, CONTRACT_CHUNK, 3, D), dtype=torch.float32, device=device)
    pos = torch.zeros((P, H), dtype=torch.int32, device=device)
    return S, rows, pos


def _need_pools(S_pool, rows_pool, pos_pool, H, dev):
    if S_pool.dim() != 4 or tuple(S_pool.shape[1:]) != (H, D, D):
        raise ValueError("S_pool must be [P, H, 128, 128]")
    P = S_pool.shape[0]
    _need(S_pool, "S_pool", (P, H, D, D), torch.float32, dev)
    _need(rows_pool, "rows_pool", (P, H, CONTRACT_CHUNK, 3, D), torch.float32, dev)
    _need(pos_pool, "pos_pool", (P, H), torch.int32, dev)
    return P


def kda_contract_prefill(q, k, v, g, beta, cu_seqlens, S_pool, rows_pool, pos_pool, cu_seqlens_host=None,
                         slots=None, o=None, scale: float = 1.0, with_output: bool = True, split_width: int = 0,
                         workspace=None):
    """Packed ragged batch through the row contract, pools updated in place.

    q, k, v, g: [T, H, 128]; beta: [T, H]; cu_seqlens: device int32 [N + 1]; slots: int32 [N] pool rows
    (None = 0..N-1).  split_width: workgroups per (sequence, head), 1, 2 or 4 (kda_contract_prefill_split),
    0 picks by grid size.  workspace: None, "auto" (allocated from kda_contract_prefill_workspace_size; needs
    cu_seqlens_host) or a device uint8 tensor of at least that size, read by the split build only
    (kda_contract_prefill_ex).  Returns o [T, H, 128] (dtype of q) or None."""
    T, H, _ = q.shape
    dt = q.dtype
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (T, H, D), dt, dev)
    _need(g, "g", (T, H, D), torch.float32, dev)
    _need(beta, "beta", (T, H), torch.float32, dev)
    if cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be 1-D")
    _need(cu_seqlens, "cu_seqlens", cu_seqlens.shape, torch.int32, dev)
    N = cu_seqlens.shape[0] - 1
    if cu_seqlens_host is not None:
        if cu_seqlens_host.is_cuda or cu_seqlens_host.dtype != torch.int32 or not cu_seqlens_host.is_contiguous():
            raise ValueError("cu_seqlens_host must be a contiguous CPU int32 tensor")
        if cu_seqlens_host.shape != cu_seqlens.shape:
            raise ValueError("cu_seqlens_host and cu_seqlens differ in shape")
        if int(cu_seqlens_host[-1]) > T or int(cu_seqlens_host[0]) < 0:
            raise ValueError("cu_seqlens_host must lie within the packed tokens")
    P = _need_pools(S_pool, rows_pool, pos_pool, H, dev)
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    elif P < N:
        raise ValueError("the pools have fewer rows than sequences")
    if with_output and o is None:
        o = torch.empty((T, H, D), dtype=dt, device=dev)
    _need(o, "o", (T, H, D), dt, dev)
    lib = _lib.load()
    if split_width not in (0, 1, 2, 4):
        raise ValueError("split_width must be 0, 1, 2 or 4")
    ws_bytes = 0
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be None, "auto" or a tensor')
        if cu_seqlens_host is None:
            raise ValueError("a workspace needs cu_seqlens_host")
        workspace = kda_contract_prefill_workspace(int(cu_seqlens_host[-1]), H, dev)
    if workspace is not None:
        if cu_seqlens_host is None:
            raise ValueError("a workspace needs cu_seqlens_host")
        if not workspace.is_cuda or workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the device of q")
        ws_bytes = workspace.numel() * workspace.element_size()
    _lib.check(lib.kda_contract_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                           _ptr(cu_seqlens_host), N, H, D, D, _dtype_code(q), float(scale),
                                           _ptr(S_pool), _ptr(rows_pool), _ptr(pos_pool), _ptr(slots), _ptr(o),
                                           int(split_width), _ptr(workspace), ws_bytes, _stream()),
               "kda_contract_prefill")
    return o


def kda_contract_prefill_workspace(T_total: int, H: int, device) -> torch.Tensor:
    """Workspace of kda_contract_prefill_ex for T_total packed tokens and H heads (uint8)."""
    n = int(_lib.load().kda_contract_prefill_workspace_size(int(T_total), int(H)))
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def kda_contract_decode(q, k, v, g, beta, S_pool, rows_pool, pos_pool, slots=None, o=None, scale: float = 1.0,
                        with_output: bool = True):
    """One token per request through the row contract, pools updated in place.

    q, k, v, g: [N, H, 128]; beta: [N, H].  Returns o [N, H, 128] (dtype of q) or None."""
    N, H, _ = q.shape
    dt = q.dtype
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (N, H, D), dt, dev)
    _need(g, "g", (N, H, D), torch.float32, dev)
    _need(beta, "beta", (N, H), torch.float32, dev)
    P = _need_pools(S_pool, rows_pool, pos_pool, H, dev)
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    elif P < N:
        raise ValueError("the pools have fewer rows than requests")
    if with_output and o is None:
        o = torch.empty((N, H, D), dtype=dt, device=dev)
    _need(o, "o", (N, H, D), dt, dev)
    lib = _lib.load()
    _lib.check(lib.kda_contract_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), N, H, D, D, _dtype_code(q),
                                       float(scale), _ptr(S_pool), _ptr(rows_pool), _ptr(pos_pool), _ptr(slots),
                                       _ptr(o), _stream()),
               "kda_contract_decode")
    return o


def kda_contract_state(S_pool, rows_pool, pos_pool, slots=None, N: Optional[int] = None, state_out=None):
    """The running states S_t of N contract slots (slots: int32 [N] or None = 0..N-1) as
    [N, H, 128, 128] fp32; the pools are not changed."""
    H = S_pool.shape[1]
    dev = S_pool.device
    P = _need_pools(S_pool, rows_pool, pos_pool, H, dev)
    if N is None:
        N = slots.shape[0] if slots is not None else P
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    elif P < N:
        raise ValueError("the pools have fewer rows than requested")
    if state_out is None:
        state_out = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    _need(state_out, "state_out", (N, H, D, D), torch.float32, dev)
    lib = _lib.load()
    _lib.check(lib.kda_contract_state(_ptr(S_pool), _ptr(rows_pool), _ptr(pos_pool), _ptr(slots), N, H, D, D,
                                      _ptr(state_out), _stream()),
               "kda_contract_state")
    return state_out


def _need_block(q, k, v, g, beta):
    N, G, H, _ = k.shape
    dt = k.dtype
    dev = k.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (N, G, H, D), dt, dev)
    _need(g, "g", (N, G, H, D), torch.float32, dev)
    _need(beta, "beta", (N, G, H), torch.float32, dev)
    return N, G, H, dt, dev


def kda_contract_stash(N: int, G: int, H: int, device):
    """A verify stash for kda_contract_verify / kda_contract_commit_stash: fp32 [N, H, G * 3 * 128 + 128 * 128]."""
    return torch.empty((N, H, G * 3 * D + D * D), dtype=torch.float32, device=device)


def kda_contract_verify(q, k, v, g, beta, S_pool, rows_pool, pos_pool, slots=None, o=None, scale: float = 1.0,
                        stash=None):
    """Outputs of gamma1 draft tokens per request from the contract state, which is not changed.

    q, k, v, g: [N, G, H, 128]; beta: [N, G, H].  Returns o [N, G, H, 128]; o[:, t] equals, bit for bit,
    the output of the (t+1)-th of t+1 kda_contract_decode calls.  With ``stash`` (kda_contract_stash,
    G <= 16) the verify also keeps what kda_contract_commit_stash needs."""
    N, G, H, dt, dev = _need_block(q, k, v, g, beta)
    P = _need_pools(S_pool, rows_pool, pos_pool, H, dev)
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    elif P < N:
        raise ValueError("the pools have fewer rows than requests")
    if o is None:
        o = torch.empty((N, G, H, D), dtype=dt, device=dev)
    _need(o, "o", (N, G, H, D), dt, dev)
    if stash is not None:
        if G > 16:
            raise ValueError("a stash holds at most 16 drafts")
        _need(stash, "stash", (N, H, G * 3 * D + D * D), torch.float32, dev)
    lib = _lib.load()
    _lib.check(lib.kda_contract_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), N, G, H, D, D,
                                       _dtype_code(k), float(scale), _ptr(S_pool), _ptr(rows_pool), _ptr(pos_pool),
                                       _ptr(slots), _ptr(o), _ptr(stash), _stream()),
               "kda_contract_verify")
    return o


def kda_contract_commit_stash(stash, accepted_len, S_pool, rows_pool, pos_pool, G: int, slots=None):
    """Commit the accepted drafts from a verify's stash, in place: bit-identical to kda_contract_commit."""
    N, H = stash.shape[0], stash.shape[1]
    dev = stash.device
    if G < 1 or G > 16:
        raise ValueError("G must be in 1 .. 16")
    _need(stash, "stash", (N, H, G * 3 * D + D * D), torch.float32, dev)
    P = _need_pools(S_pool, rows_pool, pos_pool, H, dev)
    _need(accepted_len, "accepted_len", (N,), torch.int32, dev)
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    elif P < N:
        raise ValueError("the pools have fewer rows than requests")
    lib = _lib.load()
    _lib.check(lib.kda_contract_commit_stash(_ptr(stash), _ptr(accepted_len), N, G, H, D, D, _ptr(S_pool),
                                             _ptr(rows_pool), _ptr(pos_pool), _ptr(slots), _stream()),
               "kda_contract_commit_stash")


def kda_contract_commit(k, v, g, beta, accepted_len, S_pool, rows_pool, pos_pool, slots=None, q=None):
    """Apply the first accepted_len[n] (device int32 [N], clamped to 0..G) of each request's G tokens to
    its contract state, in place: bit-identical to that many kda_contract_decode calls."""
    N, G, H, _ = k.shape
    dev = k.device
    qq = q if q is not None else k
    _need_block(qq, k, v, g, beta)
    P = _need_pools(S_pool, rows_pool, pos_pool, H, dev)
    _need(accepted_len, "accepted_len", (N,), torch.int32, dev)
    if slots is not None:
        _need(slots, "slots", (N,), torch.int32, dev)
    elif P < N:
        raise ValueError("the pools have fewer rows than requests")
    lib = _lib.load()
    _lib.check(lib.kda_contract_commit(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(accepted_len), N, G, H,
                                       D, D, _dtype_code(k), _ptr(S_pool), _ptr(rows_pool), _ptr(pos_pool),
                                       _ptr(slots), _stream()),
               "kda_contract_commit")
