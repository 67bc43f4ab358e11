"""ctypes loader for libkda.so (the HIP library).  Raises if it is not built."""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP, KDA_ERR_WORKSPACE = 0, 1, 2, 3, 4
KDA_F32, KDA_BF16 = 0, 1
KDA_WS_PREPARED, KDA_WS_KEEP_OUTPUT_OPERANDS = 1, 2
KDA_PREFILL_TRANSITIONS, KDA_PREFILL_NO_OUTPUT = 1, 2
KDA_COMPOSE_SPLIT_BF16 = 1

# (name, restype, argtypes) for every symbol include/kda.h declares
_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
SIGNATURES = {
    "kda_version": (ctypes.c_int, []),
    "kda_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kda_decode_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _F, _P, _P]),
    "kda_verify_block": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_int, _F, _P, _P, _P,
                                        _P]),
    "kda_verify_commit": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_int, _P]),
    "kda_decode_step_prologue": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _F, _P,
                                                _P, _P]),
    "kda_verify_block_prologue": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_int, _F,
                                                 _P, _P, _P, _P, _P]),
    "kda_verify_block_record": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_int, _F,
                                               _P, _P, _P, _P]),
    "kda_verify_commit_record": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_int, _P]),
    "kda_verify_commit_prologue": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_int, _P,
                                                  _P]),
    "kda_prefill": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _F, _P, _P, _P, _P, _P]),
    "kda_copy_probe": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P]),
    "kda_copy_probe_state": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int32, _P]),
    "kda_mfma_probe": (ctypes.c_int, [_P, _I, _I, _P, _P]),
    "kda_prefill_workspace_size": (ctypes.c_size_t, [_I, ctypes.c_int64, _I, _I, _I, ctypes.c_int, _I]),
    "kda_prefill_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _F, _P, _P, _P,
                                           _P, _P, _P, _P]),
    "kda_prefill_noalloc_max_scratch": (ctypes.c_size_t, []),
    "kda_prefill_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _F, _P, _P, _P, _P,
                                      _P, _P, _P, ctypes.c_size_t, _I, _P]),
    "kda_prefill_prologue": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _F, _P, _P,
                                            _P, _P, _P, _P]),
    "kda_prefill_ordered": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _F, _P, _P, _P,
                                           _P, _P, _P]),
    "kda_prefill_checkpointed": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _F, _P, _P,
                                                _P, _I, _P, _P]),
    "kda_prefill_checkpoint_count": (ctypes.c_int64, [_P, _I, _I]),
    "kda_compose_segments": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "kda_compose_segments_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "kda_contract_prefill": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _F, _P, _P,
                                            _P, _P, _P, _P]),
    "kda_contract_prefill_split": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _F, _P,
                                                  _P, _P, _P, _P, _I, _P]),
    "kda_contract_prefill_workspace_size": (ctypes.c_size_t, [ctypes.c_int64, _I]),
    "kda_contract_prefill_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _F, _P, _P,
                                               _P, _P, _P, _I, _P, ctypes.c_size_t, _P]),
    "kda_contract_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _F, _P, _P, _P, _P,
                                           _P, _P]),
    "kda_contract_state": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "kda_contract_verify": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_int, _F, _P, _P, _P, _P,
                                           _P, _P, _P]),
    "kda_contract_commit_stash": (ctypes.c_int, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P]),
    "kda_contract_commit": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_int, _P, _P, _P, _P,
                                           _P]),
}

class KdaPrologue(ctypes.Structure):
    """kda_prologue_t of include/kda.h."""
    _fields_ = [("l2norm_qk", ctypes.c_int32), ("l2norm_eps", ctypes.c_float),
                ("gate_logits", ctypes.c_int32), ("g_min", ctypes.c_float)]


_lock = threading.Lock()
_lib = None


class KdaError(RuntimeError):
    pass


def load() -> ctypes.CDLL:
    """Load libkda.so once.  torch is imported first so that the library binds to
    the HIP runtime torch already loaded (one runtime per process)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise KdaError(
                f"{LIB_PATH} is missing: build it with `python -m gated_delta_rule_15_amd.build` "
                "(there is no CPU fallback for the KDA kernels)")
        import torch  # noqa: F401  (binds the HIP runtime before the library loads)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def check(status: int, what: str) -> None:
    if status != KDA_OK:
        msg = load().kda_status_string(status).decode()
        raise KdaError(f"{what} failed: status {status} ({msg})")
