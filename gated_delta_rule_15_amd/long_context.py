"""Segmented (KCP-style) prefill of long sequences on one GPU.

A sequence longer than ``seg_len`` tokens is cut into segments that run in
parallel.  Every step runs in the library's kernels; this module only plans the
segment rows and sequences three library calls
("Kimi K3 的训练与 Serving Infra：KDA 换掉 attention 后，系统要重做什么",
sections 4.1-4.2: each segment computes its fixed-size fragments (M, S~), a
prefix scan over them recovers each segment's true entry state, then each
segment computes its outputs):

  pass 1   kda_prefill over the segments 0..n-2 of every multi-segment
           sequence: zero entry state, no outputs; final state = S~, and the
           transition M (transition_out).
  compose  kda_compose_segments_ex per multi-segment sequence: entry states
           S_in(i+1) = M(i) S_in(i) + S~(i), written straight into the rows of
           pass 2's initial-state buffer (bf16 inputs: products on split bf16
           operands, KDA_COMPOSE_SPLIT_BF16).
  pass 2   kda_prefill over every segment of every sequence from its true entry
           state, longest rows started first (kda_prefill_ordered): the
           outputs and the final states.

Segment boundaries are multiples of 64 tokens from each sequence start, so
the chunking inside every segment is the one the unsplit sequence would use.
Copies of the caller's initial states into pass 2's row buffer, and of final
states out of it, are plain device-to-device moves (buffer marshalling).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from . import _lib, kda

D = 128


@dataclass
class SegmentPlan:
    seg_len: int
    rows: np.ndarray            # [R + 1] int32 token offsets of all segment rows (pass 2)
    row_of_seq: List[range]     # pass-2 rows of each sequence
    multi: List[int]            # sequences with >= 2 segments

    @property
    def n_rows(self) -> int:
        return int(self.rows.shape[0] - 1)


def auto_seg_len(cu_seqlens_host, H: int, n_cu: int = 256, min_seg: int = 512) -> int:
    """Segment length for a batch whose (sequence, head) units are too few to fill the GPU.

    A prefill walks each sequence's chunks in order, so a batch of few long
    sequences leaves most compute units idle.  Cutting every sequence into
    ``n`` segments gives ``n`` times the units at the cost of the segment
    passes (transition columns in pass 1, composition, recomputed outputs).
    The rule aims at about ``n_cu / 4`` (segment, head) units with segments of
    at least ``min_seg`` tokens; with 4096 tokens x 12 heads it picks
    704-token segments.  Returns the longest sequence length rounded up to 64
    (no cut) when the batch already has enough units or is short.
    """
    cu = np.asarray(cu_seqlens_host, dtype=np.int64)
    lens = np.diff(cu)
    t_max = int(lens.max()) if lens.size else 0
    units = int((lens > 0).sum()) * H
    if units == 0:
        return 64
    n_seg = max(1, -(-n_cu // (4 * units)))
    seg = max(min_seg, -(-t_max // n_seg))
    return ((seg + 63) // 64) * 64


def auto_seg_len_split(cu_seqlens_host, H: int, n_cu: int = 256, min_seg: int = 256) -> int:
    """Segment length for the split path (``alloc_work(..., split=True)``): each of its passes runs
    one workgroup per (row, head) (pass 1 holds a row's state and transition together), so the
    rule cuts the longest sequence into as many segments as keep that within ``n_cu``
    workgroups, each at least ``min_seg`` tokens (4096 tokens x 12 heads: 256-token segments,
    16 rows, 192 workgroups)."""
    cu = np.asarray(cu_seqlens_host, dtype=np.int64)
    lens = np.diff(cu)
    t_max = int(lens.max()) if lens.size else 0
    units = int((lens > 0).sum()) * H
    if units == 0:
        return 64
    n_seg = max(1, n_cu // units)
    seg = max(min_seg, -(-t_max // n_seg))
    seg = ((seg + 63) // 64) * 64
    # rounding up to 64 can leave the last segment short: more rows than wanted is still within n_cu
    # as long as every sequence's row count stays at n_seg
    while seg < t_max and -(-t_max // seg) > n_seg:
        seg += 64
    return seg


def plan_segments(cu_seqlens_host, seg_len: int, cut_longer_than: int = 0) -> SegmentPlan:
    """Segment rows of a packed batch: every sequence longer than
    ``max(seg_len, cut_longer_than)`` tokens is cut every ``seg_len`` tokens
    from its start; the others stay whole."""
    if seg_len <= 0 or seg_len % 64:
        raise ValueError("seg_len must be a positive multiple of 64")
    cu = np.asarray(cu_seqlens_host, dtype=np.int64)
    rows = [int(cu[0])]
    row_of_seq, multi = [], []
    for n in range(cu.shape[0] - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        first = len(rows) - 1
        cuts = list(range(a + seg_len, b, seg_len)) if b - a > cut_longer_than else []
        rows.extend(cuts + [b])
        row_of_seq.append(range(first, len(rows) - 1))
        if cuts:
            multi.append(n)
    return SegmentPlan(seg_len, np.asarray(rows, dtype=np.int32), row_of_seq, multi)


def kda_prefill_segmented(q, k, v, g, beta, cu_seqlens_host, seg_len: Optional[int] = 65536, initial_state=None,
                          o=None, final_state=None, scale: float = 1.0, plan: Optional[SegmentPlan] = None,
                          work: Optional[dict] = None, prologue: Optional[kda.Prologue] = None,
                          compose_split_bf16: Optional[bool] = None):
    """Prefill of a packed ragged batch with long sequences split into segments.

    Same arguments and results as ``kda.kda_prefill`` (cu_seqlens_host: CPU
    int32 [N + 1]); returns (o, final_state).  ``seg_len=None`` picks it with
    ``auto_seg_len``.  With a ``plan``, preallocated buffers ``work`` from
    ``alloc_work`` and the outputs ``o`` and ``final_state`` passed in, a call
    allocates no device memory.  ``prologue``: raw q, k and gate logits, as
    ``kda.kda_prefill(..., prologue=...)``; both passes apply it.
    ``compose_split_bf16``: run the scan's products on bf16 MFMA with hi/lo split operands (the
    precision class of the passes' own products on bf16 inputs); default: for bf16 inputs only.
    """
    dev = q.device
    H = q.shape[1]
    cu_host = torch.as_tensor(np.asarray(cu_seqlens_host, dtype=np.int32))
    N = cu_host.shape[0] - 1
    if plan is None and seg_len is None:
        seg_len = auto_seg_len(cu_host.numpy(), H)
    plan = plan or plan_segments(cu_host.numpy(), seg_len)
    work = work or alloc_work(plan, H, dev, q.dtype)
    if o is None:
        o = torch.empty_like(q)
    if final_state is None:
        final_state = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    init2, fin2 = work["init2"], work["fin2"]
    ws = work["ws"]
    split_bf16 = q.dtype == torch.bfloat16 if compose_split_bf16 is None else compose_split_bf16
    # split path with every sequence cut: pass 1 gives every row's (M, S~), so the scan runs through
    # the last segment and yields each sequence's final state (and its first row's entry state);
    # pass 2 then only writes outputs
    all_cut = ws is not None and len(plan.multi) == N

    if not all_cut:
        # entry states of first segments: the caller's initial states (or zeros)
        first_rows = work["first_rows"]
        if initial_state is not None:
            init2.index_copy_(0, first_rows, initial_state)
        else:
            init2.index_fill_(0, first_rows, 0.0)

    if ws is not None:
        # split path: pass 1 runs over every row (the rows it does not need cost little on a grid
        # this small), so both passes walk the same chunks and share one preparation
        kda.kda_prefill(q, k, v, g, beta, work["rows_d"], work["rows_h"], final_state=work["St_all"],
                        transition_out=work["M_all"], with_output=False, scale=scale, workspace=ws,
                        ws_flags=_lib.KDA_WS_KEEP_OUTPUT_OPERANDS, prologue=prologue)
    for n in plan.multi:
        r = plan.row_of_seq[n]
        nf = len(r) - 1
        if all_cut:
            kda.kda_compose_segments(work["M_all"][r.start:r.stop], work["St_all"][r.start:r.stop],
                                     None if initial_state is None else initial_state[n],
                                     S_in=init2[r.start:r.stop], S_final=final_state[n], split_bf16=split_bf16)
            continue
        if ws is not None:
            M, St = work["M_all"][r.start:r.start + nf], work["St_all"][r.start:r.start + nf]
        else:
            # pass 1: fragments of segments 0 .. nf-1
            M, St = work["M"][n], work["St"][n]
            kda.kda_prefill(q, k, v, g, beta, work["frag_cu"][n], work["frag_cu_h"][n], final_state=St,
                            transition_out=M, with_output=False, scale=scale, workspace=None, prologue=prologue)
        # compose: entry states of segments 1 .. nf (segment 0's is the sequence's own),
        # written into pass 2's rows; S_in[0] lands on row r.start, which already holds S_in0
        kda.kda_compose_segments(M, St, init2[r.start], S_in=init2[r.start:r.start + nf],
                                 S_final=init2[r.start + nf], split_bf16=split_bf16)

    # pass 2: every segment from its entry state, longest rows started first
    kda.kda_prefill_ordered(q, k, v, g, beta, work["rows_d"], work["order2"], work["rows_h"], initial_state=init2,
                            final_state=None if all_cut else fin2, with_final_state=not all_cut, o=o, scale=scale,
                            workspace=ws, ws_flags=_lib.KDA_WS_PREPARED if ws is not None else 0,
                            prologue=prologue)
    if not all_cut:
        torch.index_select(fin2, 0, work["last_rows"], out=final_state)
    return o, final_state


def longest_first(rows) -> np.ndarray:
    """Order in which to start the rows of a packed batch (offsets ``rows``): longest first, ties
    in row order.  A prefill walks each row's chunks in sequence, so a long row started late
    sets the batch's finish time."""
    lens = np.diff(np.asarray(rows, dtype=np.int64))
    return np.argsort(-lens, kind="stable").astype(np.int32)


def alloc_work(plan: SegmentPlan, H: int, dev, dtype=torch.bfloat16, split: bool = False) -> dict:
    """Buffers of one segmented call: pass 2's entry and final states, and per cut sequence its
    fragments' transitions and states.  ``split``: when the passes' grids are small enough for
    the split path, its workspace instead (one preparation serves both passes) and every row's
    transition and state for a pass 1 over all rows."""
    R = plan.n_rows
    T_end = int(plan.rows[-1]) if len(plan.rows) else 0
    n_ws = kda.kda_prefill_workspace_size(R, T_end, H, dtype, transitions=True, outputs=False) if split else 0
    ws = torch.empty(n_ws, dtype=torch.uint8, device=dev) if n_ws > 0 else None
    work = {
        "order2": torch.from_numpy(longest_first(plan.rows)).to(dev),
        "init2": torch.empty((R, H, D, D), dtype=torch.float32, device=dev),
        "fin2": torch.empty((R, H, D, D), dtype=torch.float32, device=dev),
        "rows_d": torch.from_numpy(plan.rows.copy()).to(dev),
        "rows_h": torch.from_numpy(plan.rows.copy()),
        "first_rows": torch.tensor([r.start for r in plan.row_of_seq], dtype=torch.long, device=dev),
        "last_rows": torch.tensor([r.stop - 1 for r in plan.row_of_seq], dtype=torch.long, device=dev),
        "M": {}, "St": {}, "frag_cu": {}, "frag_cu_h": {}, "ws": ws,
    }
    if ws is not None:
        work["M_all"] = torch.empty((R, H, D, D), dtype=torch.float32, device=dev)
        work["St_all"] = torch.empty((R, H, D, D), dtype=torch.float32, device=dev)
        return work
    for n in plan.multi:
        r = plan.row_of_seq[n]
        nf = len(r) - 1
        work["M"][n] = torch.empty((nf, H, D, D), dtype=torch.float32, device=dev)
        work["St"][n] = torch.empty((nf, H, D, D), dtype=torch.float32, device=dev)
        work["frag_cu_h"][n] = torch.from_numpy(plan.rows[r.start:r.start + nf + 1].copy())
        work["frag_cu"][n] = work["frag_cu_h"][n].to(dev)
    return work
