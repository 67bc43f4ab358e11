"""The C ABI library: loads, exports every declared symbol, rejects bad host arguments.

No test here launches a kernel: every call either returns before touching the
device (argument errors, empty work) or is a pure host query.
"""
import ctypes
import os
import re

import pytest

from gated_delta_rule_15_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libkda.so not built (run __graft_entry__.build())")
    return _lib.load()


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for name in ("kda_prefill", "kda_decode_step", "kda_verify_block", "kda_verify_commit",
                 "kda_compose_segments", "kda_compose_segments_ex", "kda_prefill_checkpointed", "kda_prefill_checkpoint_count",
                 "kda_prefill_ordered", "kda_decode_step_prologue", "kda_verify_block_prologue",
                 "kda_verify_commit_prologue", "kda_prefill_prologue", "kda_contract_prefill",
                 "kda_contract_decode", "kda_contract_state", "kda_contract_verify", "kda_contract_commit",
                 "kda_contract_commit_stash", "kda_contract_prefill_split", "kda_contract_prefill_ex",
                 "kda_contract_prefill_workspace_size",
                 "kda_verify_block_record", "kda_verify_commit_record",
                 "kda_copy_probe", "kda_copy_probe_state", "kda_mfma_probe", "kda_status_string", "kda_version"):
        assert name in syms
    assert set(syms) == set(_lib.SIGNATURES), "binding signatures and header disagree"


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.kda_version() >= 100
    for code in range(4):
        assert lib.kda_status_string(code)
    assert b"unknown" in lib.kda_status_string(99)


def test_decode_argument_errors(lib):
    p = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation first
    # unsupported head dims
    assert lib.kda_decode_step(p, p, p, p, p, p, None, 4, 2, 64, 128, 1, 1.0, p, None) == _lib.KDA_ERR_UNSUPPORTED
    assert lib.kda_decode_step(p, p, p, p, p, p, None, 4, 2, 128, 256, 1, 1.0, p, None) == _lib.KDA_ERR_UNSUPPORTED
    # unknown dtype
    assert lib.kda_decode_step(p, p, p, p, p, p, None, 4, 2, 128, 128, 7, 1.0, p, None) == _lib.KDA_ERR_UNSUPPORTED
    # negative sizes, null pointers
    assert lib.kda_decode_step(p, p, p, p, p, p, None, -1, 2, 128, 128, 1, 1.0, p, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_decode_step(p, p, p, p, p, None, None, 4, 2, 128, 128, 1, 1.0, p, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_decode_step(None, p, p, p, p, p, None, 4, 2, 128, 128, 1, 1.0, p, None) == _lib.KDA_ERR_INVALID_ARG
    # empty batch is a no-op
    assert lib.kda_decode_step(None, None, None, None, None, None, None, 0, 2, 128, 128, 1, 1.0, None, None) == 0


def test_verify_argument_errors(lib):
    p = ctypes.c_void_p(16)
    assert lib.kda_verify_block(p, p, p, p, p, p, None, 4, 0, 2, 128, 128, 1, 1.0, p, None, None, None) == \
        _lib.KDA_ERR_INVALID_ARG
    # accepted_len without an output pool
    assert lib.kda_verify_block(p, p, p, p, p, p, None, 4, 8, 2, 128, 128, 1, 1.0, p, p, None, None) == \
        _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_verify_commit(p, p, p, p, p, None, None, 4, 8, 2, 128, 128, 1, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_verify_commit(p, p, p, p, p, None, p, 4, 8, 2, 96, 128, 1, None) == _lib.KDA_ERR_UNSUPPORTED


def test_prefill_argument_errors(lib):
    p = ctypes.c_void_p(16)
    bad_start = (ctypes.c_int32 * 3)(-1, 5, 9)
    decreasing = (ctypes.c_int32 * 3)(0, 9, 5)
    for cu in (bad_start, decreasing):
        assert lib.kda_prefill(p, p, p, p, p, p, cu, 2, 2, 128, 128, 1, 1.0, None, p, p, None, None) == \
            _lib.KDA_ERR_INVALID_ARG
    good = (ctypes.c_int32 * 3)(0, 5, 9)
    assert lib.kda_prefill(p, p, p, p, p, None, good, 2, 2, 128, 128, 1, 1.0, None, p, p, None, None) == \
        _lib.KDA_ERR_INVALID_ARG  # no device cu_seqlens
    assert lib.kda_prefill(p, None, p, p, p, p, good, 2, 2, 128, 128, 1, 1.0, None, p, p, None, None) == \
        _lib.KDA_ERR_INVALID_ARG  # no k
    assert lib.kda_prefill(p, p, p, p, p, p, good, 2, 2, 128, 64, 1, 1.0, None, p, p, None, None) == \
        _lib.KDA_ERR_UNSUPPORTED
    # nothing requested / no sequences: no-op
    assert lib.kda_prefill(p, p, p, p, p, p, good, 2, 2, 128, 128, 1, 1.0, None, None, None, None, None) == 0
    assert lib.kda_prefill(None, None, None, None, None, None, None, 0, 2, 128, 128, 1, 1.0, None, None, None,
                           None, None) == 0


def test_checkpoint_argument_errors(lib):
    p = ctypes.c_void_p(16)
    good = (ctypes.c_int32 * 3)(0, 130, 200)
    for interval in (0, -64, 100):
        assert lib.kda_prefill_checkpointed(p, p, p, p, p, p, good, 2, 2, 128, 128, 1, 1.0, None, p, p, interval, p,
                                            None) == _lib.KDA_ERR_INVALID_ARG
        assert lib.kda_prefill_checkpoint_count(good, 2, interval) == -1
    # the checkpoint buffer is required
    assert lib.kda_prefill_checkpointed(p, p, p, p, p, p, good, 2, 2, 128, 128, 1, 1.0, None, p, p, 64, None,
                                        None) == _lib.KDA_ERR_INVALID_ARG
    # counts: floor((130 - 1) / 64) + floor((70 - 1) / 64) = 2 + 1
    assert lib.kda_prefill_checkpoint_count(good, 2, 64) == 3
    assert lib.kda_prefill_checkpoint_count(good, 2, 128) == 1
    decreasing = (ctypes.c_int32 * 3)(0, 9, 5)
    assert lib.kda_prefill_checkpoint_count(decreasing, 2, 64) == -1


def test_ordered_prefill_argument_errors(lib):
    p = ctypes.c_void_p(16)
    good = (ctypes.c_int32 * 3)(0, 130, 200)
    # the order array is required
    assert lib.kda_prefill_ordered(p, p, p, p, p, p, good, 2, 2, 128, 128, 1, 1.0, None, p, p, None, None,
                                   None) == _lib.KDA_ERR_INVALID_ARG
    # the other checks are kda_prefill's (no launch happens for these)
    bad = (ctypes.c_int32 * 3)(0, 130, 100)
    assert lib.kda_prefill_ordered(p, p, p, p, p, p, bad, 2, 2, 128, 128, 1, 1.0, None, p, p, None, p,
                                   None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_prefill_ordered(p, p, p, p, p, p, good, 2, 2, 64, 128, 1, 1.0, None, p, p, None, p,
                                   None) == _lib.KDA_ERR_UNSUPPORTED
    assert lib.kda_prefill_ordered(None, None, None, None, None, None, None, 0, 2, 128, 128, 1, 1.0, None, None,
                                   None, None, p, None) == 0


def test_prologue_argument_errors(lib):
    p = ctypes.c_void_p(16)
    Pro = _lib.KdaPrologue
    bad = [None, Pro(1, -1.0, 0, 0.0), Pro(1, float("nan"), 0, 0.0), Pro(1, float("inf"), 0, 0.0),
           Pro(0, 0.0, 1, 0.0), Pro(0, 0.0, 1, 1.0), Pro(0, 0.0, 1, float("nan")), Pro(0, 0.0, 1, float("-inf"))]
    for pro in bad:
        ref = None if pro is None else ctypes.addressof(pro)
        assert lib.kda_decode_step_prologue(p, p, p, p, p, p, None, 2, 2, 128, 128, 1, 1.0, p, ref,
                                            None) == _lib.KDA_ERR_INVALID_ARG
        assert lib.kda_verify_block_prologue(p, p, p, p, p, p, None, 2, 8, 2, 128, 128, 1, 1.0, p, None, None, ref,
                                             None) == _lib.KDA_ERR_INVALID_ARG
        assert lib.kda_verify_commit_prologue(p, p, p, p, p, None, p, 2, 8, 2, 128, 128, 1, ref,
                                              None) == _lib.KDA_ERR_INVALID_ARG
        good = (ctypes.c_int32 * 3)(0, 130, 200)
        assert lib.kda_prefill_prologue(p, p, p, p, p, p, good, 2, 2, 128, 128, 1, 1.0, None, p, p, None, ref,
                                        None) == _lib.KDA_ERR_INVALID_ARG
    # a valid prologue leaves the plain checks in place (no launch happens for these)
    ok = Pro(1, 1e-6, 1, -5.0)
    assert lib.kda_decode_step_prologue(p, p, p, p, p, p, None, 2, 2, 64, 128, 1, 1.0, p, ctypes.addressof(ok),
                                        None) == _lib.KDA_ERR_UNSUPPORTED
    assert lib.kda_decode_step_prologue(p, p, p, p, p, p, None, 0, 2, 128, 128, 1, 1.0, p, ctypes.addressof(ok),
                                        None) == 0
    assert lib.kda_verify_commit_prologue(p, p, p, p, p, None, None, 2, 8, 2, 128, 128, 1, ctypes.addressof(ok),
                                          None) == _lib.KDA_ERR_INVALID_ARG


def test_compose_argument_errors(lib):
    p = ctypes.c_void_p(16)
    assert lib.kda_compose_segments(p, p, None, p, None, -1, 2, 128, 128, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_compose_segments(None, p, None, p, None, 3, 2, 128, 128, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_compose_segments(p, p, None, p, None, 3, 2, 32, 128, None) == _lib.KDA_ERR_UNSUPPORTED
    assert lib.kda_compose_segments(None, None, None, None, None, 0, 2, 128, 128, None) == 0
    for flags in (2, -1, 1 << 30):
        assert lib.kda_compose_segments_ex(p, p, None, p, None, 3, 2, 128, 128, flags, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_compose_segments_ex(None, p, None, p, None, 3, 2, 128, 128, 1, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_compose_segments_ex(p, p, None, p, None, 3, 2, 128, 64, 1, None) == _lib.KDA_ERR_UNSUPPORTED
    assert lib.kda_compose_segments_ex(None, None, None, None, None, 0, 2, 128, 128, 1, None) == 0


def test_contract_argument_errors(lib):
    p = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation first
    E, U = _lib.KDA_ERR_INVALID_ARG, _lib.KDA_ERR_UNSUPPORTED
    # decode: sizes, dims, dtype, missing buffers (o and slots may be NULL)
    assert lib.kda_contract_decode(p, p, p, p, p, -1, 2, 128, 128, 1, 1.0, p, p, p, None, p, None) == E
    assert lib.kda_contract_decode(p, p, p, p, p, 4, 0, 128, 128, 1, 1.0, p, p, p, None, p, None) == E
    assert lib.kda_contract_decode(p, p, p, p, p, 4, 2, 64, 128, 1, 1.0, p, p, p, None, p, None) == U
    assert lib.kda_contract_decode(p, p, p, p, p, 4, 2, 128, 128, 5, 1.0, p, p, p, None, p, None) == U
    assert lib.kda_contract_decode(p, p, p, p, p, 4, 2, 128, 128, 1, 1.0, p, None, p, None, p, None) == E
    assert lib.kda_contract_decode(p, p, p, p, p, 4, 2, 128, 128, 1, 1.0, p, p, None, None, p, None) == E
    assert lib.kda_contract_decode(None, p, p, p, p, 4, 2, 128, 128, 1, 1.0, p, p, p, None, p, None) == E
    assert lib.kda_contract_decode(None, None, None, None, None, 0, 2, 128, 128, 1, 1.0, None, None, None, None,
                                   None, None) == 0
    # prefill: cu_seqlens checks on the host copy, missing pools
    good = (ctypes.c_int32 * 3)(0, 5, 9)
    bad = (ctypes.c_int32 * 3)(0, 5, 4)
    neg = (ctypes.c_int32 * 3)(-1, 5, 9)
    empty = (ctypes.c_int32 * 3)(3, 3, 3)
    args = lambda cu_h, S=p, R=p, P=p: (p, p, p, p, p, p, cu_h, 2, 2, 128, 128, 1, 1.0, S, R, P, None, p, None)
    assert lib.kda_contract_prefill(*args(bad)) == E
    assert lib.kda_contract_prefill(*args(neg)) == E
    assert lib.kda_contract_prefill(*args(good, R=None)) == E
    assert lib.kda_contract_prefill(*args(good, P=None)) == E
    assert lib.kda_contract_prefill(None, None, None, None, None, p, empty, 2, 2, 128, 128, 1, 1.0, p, p, p, None,
                                    None, None) == 0  # no tokens: nothing to do, inputs may be NULL
    assert lib.kda_contract_prefill(None, p, p, p, p, p, good, 2, 2, 128, 128, 1, 1.0, p, p, p, None, p, None) == E
    # prefill with a workspace: needs the host offsets and enough bytes (sized from cu_seqlens_host[-1])
    ex = lambda cu_h, nbytes, w=1: (p, p, p, p, p, p, cu_h, 2, 2, 128, 128, 1, 1.0, p, p, p, None, p, 0, p if w else None,
                                    nbytes, None)
    need = lib.kda_contract_prefill_workspace_size(9, 2)
    assert need == 1 * 2 * 35392  # one 16-token window of 9 tokens, 2 heads, 8,848 floats each
    assert lib.kda_contract_prefill_workspace_size(17, 3) == 2 * 3 * 35392
    assert lib.kda_contract_prefill_workspace_size(0, 3) == 0
    assert lib.kda_contract_prefill_ex(*ex(None, need)) == E
    assert lib.kda_contract_prefill_ex(*ex(good, need - 1)) == _lib.KDA_ERR_WORKSPACE
    assert lib.kda_contract_prefill_ex(*ex(bad, need)) == E
    assert lib.kda_contract_prefill_ex(p, p, p, p, p, p, good, 2, 2, 128, 128, 1, 1.0, p, p, p, None, p, 3, None, 0,
                                       None) == E  # split width
    assert lib.kda_contract_prefill(p, p, p, p, p, None, good, 2, 2, 128, 128, 1, 1.0, p, p, p, None, p, None) == E
    assert lib.kda_contract_prefill(p, p, p, p, p, p, good, 2, 2, 128, 128, 3, 1.0, p, p, p, None, p, None) == U
    for w in (3, -1, 8):  # split widths other than 0, 1, 2, 4
        assert lib.kda_contract_prefill_split(p, p, p, p, p, p, good, 2, 2, 128, 128, 1, 1.0, p, p, p, None, p, w,
                                              None) == E
    assert lib.kda_contract_prefill_split(*args(bad)[:-1], 2, None) == E
    # verify (read-only; o required) and commit (q may be NULL; accepted_len required)
    assert lib.kda_contract_verify(p, p, p, p, p, 4, 0, 2, 128, 128, 1, 1.0, p, p, p, None, p, None, None) == E
    assert lib.kda_contract_verify(p, p, p, p, p, 4, 8, 2, 128, 128, 1, 1.0, p, p, p, None, None, None, None) == E
    assert lib.kda_contract_verify(p, p, p, p, p, 4, 8, 2, 128, 64, 1, 1.0, p, p, p, None, p, None, None) == U
    assert lib.kda_contract_verify(p, p, p, p, p, 4, 17, 2, 128, 128, 1, 1.0, p, p, p, None, p, p, None) == E
    assert lib.kda_contract_verify(None, None, None, None, None, 0, 8, 2, 128, 128, 1, 1.0, None, None, None, None,
                                   None, None, None) == 0
    assert lib.kda_contract_commit_stash(p, p, 4, 0, 2, 128, 128, p, p, p, None, None) == E
    assert lib.kda_contract_commit_stash(p, p, 4, 17, 2, 128, 128, p, p, p, None, None) == E
    assert lib.kda_contract_commit_stash(None, p, 4, 8, 2, 128, 128, p, p, p, None, None) == E
    assert lib.kda_contract_commit_stash(p, p, 4, 8, 2, 64, 128, p, p, p, None, None) == U
    assert lib.kda_contract_commit_stash(None, None, 0, 8, 2, 128, 128, None, None, None, None, None) == 0
    assert lib.kda_contract_commit(None, p, p, p, p, None, 4, 8, 2, 128, 128, 1, p, p, p, None, None) == E
    assert lib.kda_contract_commit(None, p, p, p, p, p, 4, -1, 2, 128, 128, 1, p, p, p, None, None) == E
    assert lib.kda_contract_commit(None, p, p, p, p, p, 4, 8, 2, 128, 128, 9, p, p, p, None, None) == U
    # state
    assert lib.kda_contract_state(p, p, p, None, 2, 2, 128, 128, None, None) == E
    assert lib.kda_contract_state(p, None, p, None, 2, 2, 128, 128, p, None) == E
    assert lib.kda_contract_state(p, p, p, None, 2, 2, 128, 96, p, None) == U
    assert lib.kda_contract_state(None, None, None, None, 0, 2, 128, 128, None, None) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libkda.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(_lib.KdaError, match="no CPU fallback"):
        _lib.load()


def test_copy_probe_argument_errors(lib):
    """The memory-roof probe rejects counts that are not whole 16-byte pieces and misaligned buffers
    before touching the device; an empty copy does nothing."""
    p = ctypes.c_void_p(1 << 20)
    assert lib.kda_copy_probe(p, p, -4, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_copy_probe(p, p, 6, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_copy_probe(ctypes.c_void_p((1 << 20) + 4), p, 8, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_copy_probe(None, p, 8, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_copy_probe(None, None, 0, None) == _lib.KDA_OK


def test_copy_probe_state_argument_errors(lib):
    """The decode-pattern probe rejects negative counts, null or misaligned buffers and partially
    overlapping ranges before touching the device; in place (src == dst) and empty calls are accepted."""
    p = ctypes.c_void_p(1 << 20)
    state = 128 * 128 * 4
    assert lib.kda_copy_probe_state(p, p, -1, 0, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_copy_probe_state(p, p, 1, 2, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_copy_probe_state(p, p, (1 << 29) + 1, 0, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_copy_probe_state(None, p, 1, 0, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_copy_probe_state(ctypes.c_void_p((1 << 20) + 4), ctypes.c_void_p(1 << 24), 1, 0, None) \
        == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_copy_probe_state(p, ctypes.c_void_p((1 << 20) + state), 2, 1, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_copy_probe_state(None, None, 0, 1, None) == _lib.KDA_OK


def test_mfma_probe_argument_errors(lib):
    p = ctypes.c_void_p(1 << 20)
    assert lib.kda_mfma_probe(p, 0, 10, None, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_mfma_probe(p, 4, 0, None, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_mfma_probe(None, 4, 10, None, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_mfma_probe(ctypes.c_void_p((1 << 20) + 4), 4, 10, None, None) == _lib.KDA_ERR_INVALID_ARG


def test_record_entry_points_argument_errors(lib):
    """The record verify needs a prologue and a record buffer; the record commit needs the record."""
    p = ctypes.c_void_p(1 << 20)
    # no prologue
    assert lib.kda_verify_block_record(p, p, p, p, p, p, None, 2, 8, 2, 128, 128, _lib.KDA_BF16, 1.0, p, p, None,
                                       None) == _lib.KDA_ERR_INVALID_ARG
    # no record
    assert lib.kda_verify_commit_record(None, p, p, p, None, p, 2, 8, 2, 128, 128, _lib.KDA_BF16,
                                        None) == _lib.KDA_ERR_INVALID_ARG
    # misaligned record
    assert lib.kda_verify_commit_record(ctypes.c_void_p((1 << 20) + 4), p, p, p, None, p, 2, 8, 2, 128, 128,
                                        _lib.KDA_BF16, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_verify_commit_record(p, p, p, p, None, p, 2, 8, 2, 64, 128, _lib.KDA_BF16,
                                        None) == _lib.KDA_ERR_UNSUPPORTED
    assert lib.kda_verify_commit_record(None, None, None, None, None, None, 0, 8, 2, 128, 128, _lib.KDA_BF16,
                                        None) == _lib.KDA_OK
