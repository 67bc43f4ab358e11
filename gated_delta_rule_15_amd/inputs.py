"""Seeded synthetic inputs for the KDA workloads.

This module only draws random numbers and lays them out. It holds none of the
recurrence's arithmetic, so both the HIP path (through the binding) and the CPU
oracle (through the tests and the benchmark's CPU leg) take their inputs from
here and from nowhere else.

Recipe (per (sequence, head, 4096-token block) the generator is
``numpy.random.default_rng([seed, seq, head, block])`` (PCG64), and it draws, in
this order, for the block's n tokens):

1. q ~ N(0, 1) [n, d_k]; 2. k ~ N(0, 1) [n, d_k]; 3. v ~ N(0, 1) [n, d_v];
4. z ~ N(0, 1) [n], beta = sigmoid(z); 5. g ~ U(-0.1, 0) [n, d_k] (log-decay).

q and k are then L2-normalised per token in fp32 (the recurrence assumes unit
keys; the caller, not the kernel, normalises) and cast to the workload dtype
(bf16 by round-to-nearest-even, or kept fp32).  An initial state, where a
workload has one, is N(0, 0.02^2) fp32 from ``default_rng([seed, seq, head,
STATE_TAG])``.  Accepted verify lengths and ragged sequence lengths come from
their own streams (``ACC_TAG``, ``LEN_TAG``).

Raw inputs for the in-kernel prologue (``raw=True``): the same draws, but q and
k are left unnormalised (cast straight from N(0, 1)), and the g array holds gate
logits x ~ N(-4, 2) drawn after the five above (6.), so that the log-decay
g_min * sigmoid(x) spans mostly slow channels (x = -4: g = -0.09) with a tail
of fast ones (x > 0: g < -2.5).

Arrays are packed the way the library takes them: q, k, v, g as
[T_total, H, d]; beta as [T_total, H]; states as [N, H, d_k, d_v] (rows are key
channels); ``cu_seqlens`` int32 [N + 1].  bf16 tensors are returned as numpy
uint16 bit patterns; ``bf16_bits_to_f32`` widens them exactly.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

BLOCK = 4096
STATE_TAG = 0x5354415445  # "STATE"
ACC_TAG = 0x414343  # "ACC"
LEN_TAG = 0x4C454E  # "LEN"
STATE_STD = 0.02


# --------------------------------------------------------------------------
# dtype helpers (exact conversions; no arithmetic of the method)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs cannot carry past bit 31 (largest finite pattern 0xFF7FFFFF + 0x8000)
    out = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32, exact."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of an input array held as ``dtype`` ('bf16' or 'f32')."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# one (sequence, head, block) draw
# --------------------------------------------------------------------------
def _draw_block(seed: int, seq: int, head: int, block: int, n: int, dk: int, dv: int, raw: bool = False):
    rng = np.random.default_rng([seed, seq, head, block])
    q = rng.standard_normal((n, dk), dtype=np.float32)
    k = rng.standard_normal((n, dk), dtype=np.float32)
    v = rng.standard_normal((n, dv), dtype=np.float32)
    z = rng.standard_normal(n, dtype=np.float32)
    g = rng.random((n, dk), dtype=np.float32) * np.float32(-0.1)
    if raw:
        g = (rng.standard_normal((n, dk), dtype=np.float32) * np.float32(2.0) - np.float32(4.0)).astype(np.float32)
    else:
        q /= np.sqrt(np.sum(q * q, axis=1, keepdims=True, dtype=np.float32))
        k /= np.sqrt(np.sum(k * k, axis=1, keepdims=True, dtype=np.float32))
    beta = (np.float32(1.0) / (np.float32(1.0) + np.exp(-z))).astype(np.float32)
    return q, k, v, beta, g


def draw_state(seed: int, seq: int, head: int, dk: int, dv: int) -> np.ndarray:
    rng = np.random.default_rng([seed, seq, head, STATE_TAG])
    return (rng.standard_normal((dk, dv), dtype=np.float32) * np.float32(STATE_STD)).astype(np.float32)


@dataclass
class Packed:
    """A packed ragged batch, as the library takes it."""

    dtype: str                 # 'bf16' or 'f32' (q, k, v); g, beta, states are fp32
    q: np.ndarray              # [T, H, dk]  uint16 bits (bf16) or float32
    k: np.ndarray              # [T, H, dk]
    v: np.ndarray              # [T, H, dv]
    g: np.ndarray              # [T, H, dk]  float32 log-decay
    beta: np.ndarray           # [T, H]      float32
    cu_seqlens: np.ndarray     # [N + 1]     int32
    initial_state: Optional[np.ndarray]  # [N, H, dk, dv] float32 or None (zeros)

    @property
    def num_seqs(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def H(self) -> int:
        return int(self.q.shape[1])

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    def f64(self, name: str) -> np.ndarray:
        """Exact fp64 copy of one input tensor."""
        x = getattr(self, name)
        if name in ("q", "k", "v"):
            return as_f64(x, self.dtype)
        return np.asarray(x, dtype=np.float64)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)


def packed_batch(seed: int, seqlens: Sequence[int], H: int, dk: int = 128, dv: int = 128,
                 dtype: str = "bf16", init_state: Sequence[bool] | bool = False, raw: bool = False) -> Packed:
    """Ragged batch of ``len(seqlens)`` sequences, each slice drawn per (seq, head, block).

    ``init_state`` selects, per sequence (or for all), whether it gets an
    N(0, 0.02^2) initial state (others start from zeros).  ``raw``: prologue
    inputs (unnormalised q, k; gate logits in g).
    """
    seqlens = [int(s) for s in seqlens]
    N = len(seqlens)
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    T = int(cu[-1])
    qd = np.uint16 if dtype == "bf16" else np.float32
    q = np.empty((T, H, dk), dtype=qd)
    k = np.empty((T, H, dk), dtype=qd)
    v = np.empty((T, H, dv), dtype=qd)
    g = np.empty((T, H, dk), dtype=np.float32)
    beta = np.empty((T, H), dtype=np.float32)
    for s in range(N):
        for h in range(H):
            for b0 in range(0, seqlens[s], BLOCK):
                n = min(BLOCK, seqlens[s] - b0)
                qq, kk, vv, bb, gg = _draw_block(seed, s, h, b0 // BLOCK, n, dk, dv, raw)
                t0 = int(cu[s]) + b0
                q[t0:t0 + n, h] = _cast(qq, dtype)
                k[t0:t0 + n, h] = _cast(kk, dtype)
                v[t0:t0 + n, h] = _cast(vv, dtype)
                g[t0:t0 + n, h] = gg
                beta[t0:t0 + n, h] = bb
    if isinstance(init_state, bool):
        init_state = [init_state] * N
    S0 = None
    if any(init_state):
        S0 = np.zeros((N, H, dk, dv), dtype=np.float32)
        for s in range(N):
            if init_state[s]:
                for h in range(H):
                    S0[s, h] = draw_state(seed, s, h, dk, dv)
    return Packed(dtype, q, k, v, g, beta, cu, S0)


# --------------------------------------------------------------------------
# decode / verify batches: one "sequence" per request, gamma1 tokens each
# --------------------------------------------------------------------------
@dataclass
class StepBatch:
    dtype: str
    q: np.ndarray        # [N, G, H, dk] (G = gamma1; G == 1 for decode)
    k: np.ndarray
    v: np.ndarray        # [N, G, H, dv]
    g: np.ndarray        # [N, G, H, dk] float32
    beta: np.ndarray     # [N, G, H]     float32
    state: np.ndarray    # [N, H, dk, dv] float32
    accepted_len: Optional[np.ndarray] = None  # [N] int32 in 1..G

    def f64(self, name: str) -> np.ndarray:
        x = getattr(self, name)
        if name in ("q", "k", "v"):
            return as_f64(x, self.dtype)
        return np.asarray(x, dtype=np.float64)


def step_batch(seed: int, N: int, G: int, H: int, dk: int = 128, dv: int = 128,
               dtype: str = "bf16", accepted: bool = False, raw: bool = False) -> StepBatch:
    qd = np.uint16 if dtype == "bf16" else np.float32
    q = np.empty((N, G, H, dk), dtype=qd)
    k = np.empty((N, G, H, dk), dtype=qd)
    v = np.empty((N, G, H, dv), dtype=qd)
    g = np.empty((N, G, H, dk), dtype=np.float32)
    beta = np.empty((N, G, H), dtype=np.float32)
    state = np.empty((N, H, dk, dv), dtype=np.float32)
    for n in range(N):
        for h in range(H):
            qq, kk, vv, bb, gg = _draw_block(seed, n, h, 0, G, dk, dv, raw)
            q[n, :, h] = _cast(qq, dtype)
            k[n, :, h] = _cast(kk, dtype)
            v[n, :, h] = _cast(vv, dtype)
            g[n, :, h] = gg
            beta[n, :, h] = bb
            state[n, h] = draw_state(seed, n, h, dk, dv)
    acc = accepted_lengths(seed, N, G) if accepted else None
    return StepBatch(dtype, q, k, v, g, beta, state, acc)


def accepted_lengths(seed: int, N: int, G: int = 8, p: float = 0.64) -> np.ndarray:
    """Accepted prefix length per request: 1 + run of consecutive acceptances.

    Each of the G - 1 drafts is accepted with probability p until the first
    rejection; with p = 0.64 and G = 8 the mean is (1 - p^8) / (1 - p) = 2.70.
    """
    rng = np.random.default_rng([seed, ACC_TAG])
    u = rng.random((N, G - 1))
    acc = np.ones(N, dtype=np.int32)
    for n in range(N):
        for j in range(G - 1):
            if u[n, j] < p:
                acc[n] += 1
            else:
                break
    return acc


def loguniform_lengths(seed: int, count: int, lo: int = 1024, hi: int = 32768) -> list:
    """Ragged lengths floor(exp(U(ln lo, ln hi))), not rounded to any chunk size."""
    rng = np.random.default_rng([seed, LEN_TAG])
    u = rng.random(count)
    return [int(math.floor(math.exp(math.log(lo) + x * (math.log(hi) - math.log(lo))))) for x in u]


# --------------------------------------------------------------------------
# the five workloads (sizes as stated for the KDA hot path)
# --------------------------------------------------------------------------
WORKLOADS = {
    "tiny_prefill_f32": dict(seed=1, seqlens=[256], H=1, dtype="f32"),
    "decode_64x12": dict(seed=2, N=64, G=1, H=12, dtype="bf16"),
    "prefill_4096x12": dict(seed=3, seqlens=[4096], H=12, dtype="bf16"),
    "verify_32x12x8": dict(seed=4, N=32, G=8, H=12, dtype="bf16"),
    "long_1m_plus_8": dict(seed=5, long_len=1 << 20, n_segments=16, n_extra=8, H=12, dtype="bf16"),
}


def long_context_layout(seed: int = 5, long_len: int = 1 << 20, n_extra: int = 8):
    """Lengths of the long-context batch: one long sequence, then the extras."""
    return [long_len] + loguniform_lengths(seed, n_extra)


# --------------------------------------------------------------------------
# parallel generation (same streams, same arrays) for the 1M-token workload
# --------------------------------------------------------------------------
def _fill_units(args):
    """Worker: fill (seq, head, block) units into shared-memory arrays."""
    from multiprocessing import shared_memory
    names, shapes, dtypes, units, seed, dk, dv, dtype, cu = args
    shms = [shared_memory.SharedMemory(name=nm) for nm in names]
    try:
        arrs = [np.ndarray(sh, dtype=np.dtype(dt), buffer=m.buf) for m, sh, dt in zip(shms, shapes, dtypes)]
        q, k, v, g, beta = arrs
        for s, h, blk, n in units:
            qq, kk, vv, bb, gg = _draw_block(seed, s, h, blk, n, dk, dv)
            t0 = int(cu[s]) + blk * BLOCK
            q[t0:t0 + n, h] = _cast(qq, dtype)
            k[t0:t0 + n, h] = _cast(kk, dtype)
            v[t0:t0 + n, h] = _cast(vv, dtype)
            g[t0:t0 + n, h] = gg
            beta[t0:t0 + n, h] = bb
        del arrs, q, k, v, g, beta
    finally:
        for m in shms:
            m.close()
    return len(units)


class SharedPacked(Packed):
    """A Packed whose big arrays live in shared memory; call release() when done."""

    _shms: list = []

    def release(self):
        """Drop the shared arrays and free their memory (shapes stay readable via ``T``/``H``)."""
        import gc
        self._T, self._H = self.T, self.H
        self.q = self.k = self.v = self.g = self.beta = None
        gc.collect()
        for m in self._shms:
            try:
                m.close()
            except BufferError:  # a view is still alive somewhere; the name is still removed
                pass
            try:
                m.unlink()
            except FileNotFoundError:
                pass
        self._shms = []

    @property
    def T(self) -> int:
        return int(self.q.shape[0]) if self.q is not None else self._T

    @property
    def H(self) -> int:
        return int(self.q.shape[1]) if self.q is not None else self._H


def pool_map(fn, args, workers: int, chunksize: int = 1) -> list:
    """map() over a pool of spawned worker processes that are let exit on their own.

    The pool is closed and joined rather than terminated (a context-managed pool
    sends its idle workers SIGTERM, which a profiler's preloaded signal handler
    turns into aborts); it is terminated only when the map itself fails.
    """
    import multiprocessing as mp
    pool = mp.get_context("spawn").Pool(workers)
    try:
        out = pool.map(fn, args, chunksize=chunksize)
        pool.close()
    except BaseException:
        pool.terminate()
        raise
    finally:
        pool.join()
    return out


def packed_batch_parallel(seed: int, seqlens: Sequence[int], H: int, dk: int = 128, dv: int = 128,
                          dtype: str = "bf16", init_state: Sequence[bool] | bool = False,
                          workers: int = 8) -> SharedPacked:
    """Same arrays as ``packed_batch`` (identical per-block streams), drawn by a process pool."""
    from multiprocessing import shared_memory
    seqlens = [int(s) for s in seqlens]
    N = len(seqlens)
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    T = int(cu[-1])
    qd = np.uint16 if dtype == "bf16" else np.float32
    specs = [((T, H, dk), qd), ((T, H, dk), qd), ((T, H, dv), qd), ((T, H, dk), np.float32), ((T, H), np.float32)]
    shms, arrs = [], []
    for shape, dt in specs:
        nbytes = max(1, int(np.prod(shape)) * np.dtype(dt).itemsize)
        m = shared_memory.SharedMemory(create=True, size=nbytes)
        shms.append(m)
        arrs.append(np.ndarray(shape, dtype=dt, buffer=m.buf))
    units = [(s, h, b0 // BLOCK, min(BLOCK, seqlens[s] - b0))
             for s in range(N) for h in range(H) for b0 in range(0, seqlens[s], BLOCK)]
    workers = max(1, min(workers, len(units)))
    chunks = [units[i::workers] for i in range(workers)]
    args = [([m.name for m in shms], [sp[0] for sp in specs], [np.dtype(sp[1]).str for sp in specs], c, seed, dk, dv,
             dtype, cu) for c in chunks]
    pool_map(_fill_units, args, workers)
    if isinstance(init_state, bool):
        init_state = [init_state] * N
    S0 = None
    if any(init_state):
        S0 = np.zeros((N, H, dk, dv), dtype=np.float32)
        for s in range(N):
            if init_state[s]:
                for h in range(H):
                    S0[s, h] = draw_state(seed, s, h, dk, dv)
    out = SharedPacked(dtype, arrs[0], arrs[1], arrs[2], arrs[3], arrs[4], cu, S0)
    out._shms = shms
    return out


def long_context_batch(seed: int = 5, long_len: int = 1 << 20, n_extra: int = 8, H: int = 12,
                       dtype: str = "bf16", workers: int = 8):
    """The long-context workload: one long sequence (zero initial state) followed by
    ``n_extra`` log-uniform 1K-32K sequences with N(0, 0.02^2) initial states."""
    lens = long_context_layout(seed, long_len, n_extra)
    init = [False] + [True] * n_extra
    if workers > 1:
        return packed_batch_parallel(seed, lens, H, dtype=dtype, init_state=init, workers=workers)
    return packed_batch(seed, lens, H, dtype=dtype, init_state=init)
