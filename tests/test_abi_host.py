"""Host-side checks of the C ABI: the library loads, exports every call that
include/idx.h declares, and rejects bad arguments before touching the GPU."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "idx.h")
# IDX_LIBRARY: another build of the same library (the sanitizer build of test_host_sanitizers)
LIB = os.environ.get("IDX_LIBRARY") or os.path.join(ROOT, "two_level_top_amd", "libidx.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libidx.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(idx_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_seven_calls():
    names = declared_functions()
    for n in ("idx_score_dense", "idx_amax8_varlen", "idx_topk_blocks", "idx_expand_candidates",
              "idx_score_sparse_paged", "idx_topk_rows", "idx_prefill_tail"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_no_torch_types_in_the_abi():
    text = open(HEADER).read()
    assert "torch" not in text.lower().replace("pytorch", "")
    assert "at::" not in text and "c10" not in text


@pytest.fixture(scope="module")
def lib():
    import two_level_top_amd as t
    return t.load()


FAKE = ctypes.c_void_p(0x100000)      # never dereferenced: validation fails first
FAKE_ODD = ctypes.c_void_p(0x100004)
FAKE_ODD2 = ctypes.c_void_p(0x100002)  # not even 4-byte aligned


def _err(lib):
    return lib.idx_last_error().decode()


def test_amax8_validation(lib):
    assert lib.idx_amax8_varlen(FAKE, 12, FAKE, 4, FAKE, 4, 0, None) == -2     # ld % 8
    assert "multiple of 8" in _err(lib)
    assert lib.idx_amax8_varlen(FAKE_ODD, 16, FAKE, 4, FAKE, 4, 0, None) == -2  # 32-byte alignment
    assert lib.idx_amax8_varlen(None, 16, FAKE, 4, FAKE, 4, 0, None) == -1
    assert lib.idx_amax8_varlen(FAKE, 16, FAKE, -1, FAKE, 4, 0, None) == -1
    assert lib.idx_amax8_varlen(FAKE, 16, FAKE, 4, FAKE, 0, 0, None) == -1     # ldk < 1
    assert lib.idx_amax8_varlen(FAKE, 1 << 30, FAKE, 4, FAKE, 4, 0, None) == -1  # row above 2^29
    assert "above 2^29" in _err(lib)
    assert lib.idx_amax8_varlen(FAKE, 16, FAKE, 4, FAKE, 1 << 30, 0, None) == -1  # ldk above 2^29
    assert lib.idx_amax8_varlen(FAKE, 16, FAKE, 0, FAKE, 4, 0, None) == 0       # nothing to do
    assert _err(lib) == ""


def test_topk_validation(lib):
    assert lib.idx_topk_blocks(FAKE, 4, FAKE, 2, 0, FAKE, FAKE, None, 0, None) == -1   # kb < 1
    assert lib.idx_topk_rows(FAKE, 8, FAKE, 2, 0, 0, None, 0, None, FAKE, None, 0, None) == -1  # k < 1
    assert lib.idx_topk_rows(FAKE, 8, FAKE, 2, 4, 7, None, 0, None, FAKE, None, 0, None) == -1  # mode
    assert lib.idx_topk_rows(FAKE, 8, FAKE, 2, 4, 1, None, 4, None, FAKE, None, 0, None) == -1  # no blocks
    assert lib.idx_topk_rows(FAKE, 8, FAKE, 2, 4, 1, FAKE, 4, None, FAKE, None, 0, None) == -3  # ld < kb*8


def _structs():
    import two_level_top_amd as t
    q = t._Query(FAKE, FAKE, FAKE, 4, 64, 128)
    kp = t._KPool(FAKE, 16, 64, 128, FAKE, 1, 16)
    rows = t._Rows(FAKE, FAKE, None, 4)
    tbl = t._Table(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, 4, 16, None)
    return t, q, kp, rows, tbl


def test_score_validation(lib):
    t, q, kp, rows, tbl = _structs()
    P = ctypes.byref
    bad = t._Query(FAKE, FAKE, FAKE, 4, 64, 64)
    W = 1 << 20
    assert lib.idx_score_dense(P(bad), P(kp), P(rows), FAKE, 1024, FAKE, W, None) == -4   # dim
    bad = t._Query(FAKE, FAKE, FAKE, 4, 65, 128)
    assert lib.idx_score_dense(P(bad), P(kp), P(rows), FAKE, 1024, FAKE, W, None) == -4   # heads
    bad = t._Query(FAKE_ODD, FAKE, FAKE, 4, 64, 128)
    assert lib.idx_score_dense(P(bad), P(kp), P(rows), FAKE, 1024, FAKE, W, None) == -2   # alignment
    badkp = t._KPool(FAKE, 16, 32, 128, FAKE, 1, 16)
    assert lib.idx_score_dense(P(q), P(badkp), P(rows), FAKE, 1024, FAKE, W, None) == -4  # page size
    r3 = t._Rows(FAKE, FAKE, None, 3)
    assert lib.idx_score_dense(P(q), P(kp), P(r3), FAKE, 1024, FAKE, W, None) == -3       # rows
    assert lib.idx_score_dense(None, P(kp), P(rows), FAKE, 1024, FAKE, W, None) == -1
    assert lib.idx_score_dense(P(q), P(kp), P(rows), FAKE, 1024, FAKE, 100, None) == -6   # workspace
    assert lib.idx_score_dense(P(q), P(kp), P(rows), FAKE, 1024, FAKE_ODD, W, None) == -2
    small = t._Table(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 4, 16, None)
    assert lib.idx_score_sparse_paged(P(q), P(kp), P(small), FAKE, 128, FAKE, W, None) == -6  # schedule
    assert lib.idx_score_sparse_paged(P(q), P(kp), P(tbl), FAKE, 64, FAKE, W, None) == -3     # ld
    assert lib.idx_score_sparse_paged(P(q), P(kp), P(tbl), FAKE, 128, None, 0, None) == -6   # workspace
    assert lib.idx_expand_candidates(P(kp), P(r3), P(tbl), None) == -3


def test_score_dense_keys_validation(lib):
    t, q, kp, rows, tbl = _structs()
    P = ctypes.byref
    W = 1 << 20
    f = lib.idx_score_dense_keys
    assert f(P(q), P(kp), P(rows), FAKE, 1024, None, 128, 0, FAKE, W, None) == -1     # keys NULL
    assert "keys" in _err(lib)
    assert f(P(q), P(kp), P(rows), FAKE, 1020, FAKE, 128, 0, FAKE, W, None) == -2     # ld % 8
    assert f(P(q), P(kp), P(rows), FAKE, 1024, FAKE, 0, 0, FAKE, W, None) == -1       # ldk < 1
    assert f(P(q), P(kp), P(rows), FAKE, 1024, FAKE, 128, -1, FAKE, W, None) == -1    # skip < 0
    assert f(P(q), P(kp), P(rows), FAKE, 1024, FAKE_ODD2, 128, 0, FAKE, W, None) == -2  # keys align
    assert f(P(q), P(kp), P(rows), FAKE, 1024, FAKE, 128, 0, FAKE, 100, None) == -6   # workspace
    bad = t._Query(FAKE, FAKE, FAKE, 4, 64, 64)
    assert f(P(bad), P(kp), P(rows), FAKE, 1024, FAKE, 128, 0, FAKE, W, None) == -4   # dim
    r0 = t._Rows(FAKE, FAKE, None, 0)
    q0 = t._Query(FAKE, FAKE, FAKE, 0, 64, 128)
    assert f(P(q0), P(kp), P(r0), None, 1024, None, 128, 0, None, 0, None) == 0       # nothing to do


def test_q_rope_quant_validation(lib):
    f = lib.idx_q_rope_quant
    args = lambda **kw: [kw.get("q", FAKE), FAKE, kw.get("cs", FAKE), kw.get("maxpos", 16), FAKE,
                         kw.get("rows", 4), kw.get("heads", 8), kw.get("neox", 1),
                         ctypes.c_float(1.0), ctypes.c_float(1.0), kw.get("vals", FAKE), FAKE, FAKE, None]
    assert f(*args(rows=-1)) == -1
    assert f(*args(heads=65)) == -4
    assert f(*args(maxpos=0)) == -1
    assert f(*args(neox=2)) == -1
    assert f(*args(q=None)) == -1
    assert f(*args(q=FAKE_ODD)) == -2            # 16-byte alignment of q
    assert f(*args(cs=FAKE_ODD)) == -2
    assert f(*args(vals=FAKE_ODD2)) == -2
    assert f(*args(rows=0, q=None)) == 0            # nothing to do


def test_tail_validation(lib):
    t, q, kp, rows, tbl = _structs()
    P = ctypes.byref
    tail = t._Table(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, 4, 16, None)
    W = lib.idx_workspace_bytes(4, 2, 0, 0)
    assert lib.idx_prefill_tail(P(tbl), FAKE, FAKE, -1, P(tail), FAKE, W, None) == -1    # num_req
    assert lib.idx_prefill_tail(P(tbl), None, FAKE, 2, P(tail), FAKE, W, None) == -1     # no lengths
    bad_kb = t._Table(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, 4, 8, None)
    assert lib.idx_prefill_tail(P(tbl), FAKE, FAKE, 2, P(bad_kb), FAKE, W, None) == -3   # kb
    assert lib.idx_prefill_tail(P(tbl), FAKE, FAKE, 0, P(tail), FAKE, W, None) == -3     # no requests
    empty = t._Table(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, 0, 16, None)
    assert lib.idx_prefill_tail(P(empty), FAKE, FAKE, 2, P(tail), FAKE, W, None) == -3   # no source rows
    assert lib.idx_prefill_tail(P(tbl), FAKE, FAKE, 2, P(tail), FAKE, W - 4, None) == -6  # workspace
    assert lib.idx_prefill_tail(P(tbl), FAKE, FAKE, 2, P(tail), FAKE_ODD2, W, None) == -2  # alignment
    small = t._Table(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 4, 16, None)
    assert lib.idx_prefill_tail(P(tbl), FAKE, FAKE, 2, P(small), FAKE, W, None) == -6   # schedule


def test_library_never_synchronises():
    """Every call only enqueues work: no host-side wait on a stream, event or
    the device anywhere in the library's sources (so calls can be captured)."""
    csrc = os.path.join(ROOT, "two_level_top_amd", "csrc")
    for name in os.listdir(csrc):
        text = open(os.path.join(csrc, name)).read()
        for call in ("Synchronize", "hipMemcpy", "hipMalloc", "hipFree", "hipEventQuery",
                     "hipStreamQuery"):
            assert call not in text, f"{name} calls {call}"


def test_noalloc_rejects_rows_above_its_scratch(lib):
    t, q, kp, rows, tbl = _structs()
    P = ctypes.byref
    big = t._Query(FAKE, FAKE, FAKE, 4097, 64, 128)
    assert lib.idx_score_sparse_paged_noalloc(P(big), P(kp), P(tbl), FAKE, 1 << 14, None) == -4
    assert "4096" in _err(lib)
    assert lib.idx_score_sparse_paged_noalloc(None, P(kp), P(tbl), FAKE, 1 << 14, None) == -1


def test_workspace_sizes(lib):
    assert lib.idx_workspace_bytes(3, 16384, 2048, 0) == 16 + 16384 * 32 * 8
    assert lib.idx_workspace_bytes(4, 100, 0, 0) == (2 * 100 + 1) * 4 + 12   # 16-byte multiple
    assert lib.idx_workspace_bytes(1, 100, 32768, 2048) == 0
    assert lib.idx_workspace_bytes(5, 100, 0, 0) == 100 * 1088


def test_fold_queries_validation(lib):
    t, q, kp, rows, tbl = _structs()
    P = ctypes.byref
    f = lib.idx_fold_queries
    qs = (t._Query * 2)(q, q)
    ws = (ctypes.c_void_p * 2)(FAKE, FAKE)
    W = 1 << 20
    sizes = (ctypes.c_size_t * 2)(W, W)
    assert f(qs, 0, ws, sizes, None) == -1                      # n < 1
    assert f(qs, 17, ws, sizes, None) == -1                     # n > 16
    assert "1..16" in _err(lib)
    assert f(None, 2, ws, sizes, None) == -1
    assert f(qs, 2, None, sizes, None) == -1
    small = (ctypes.c_size_t * 2)(W, 100)
    assert f(qs, 2, ws, small, None) == -6                      # workspace of batch 1
    odd = (ctypes.c_void_p * 2)(FAKE, FAKE_ODD)
    assert f(qs, 2, odd, sizes, None) == -2                     # 16-byte alignment
    bad = (t._Query * 2)(q, t._Query(FAKE, FAKE, FAKE, 4, 64, 64))
    assert f(bad, 2, ws, sizes, None) == -4                     # dim of batch 1
    # a folded query replaces the workspace of the score calls, and must be aligned
    qf = t._Query(FAKE, FAKE, FAKE, 4, 64, 128, FAKE_ODD)
    assert lib.idx_score_dense(P(qf), P(kp), P(rows), FAKE, 1024, None, 0, None) == -2
    assert "folded" in _err(lib)
