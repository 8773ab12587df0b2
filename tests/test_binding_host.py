"""Host-side checks of the Python binding: every call rejects operands whose
leading dimension (or width) disagrees with the row count before it reaches
the C ABI, which cannot see device buffer sizes.  CPU tensors suffice: the
shape checks of a call run before its device checks."""

from __future__ import annotations

import pytest

torch = pytest.importorskip("torch")

import two_level_top_amd as t


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def fake_table(rows, kb):
    tbl = object.__new__(t.Table)
    tbl.rows, tbl.kb, tbl.ready = rows, kb, None
    return tbl


def raises(fn, *args, match, **kw):
    with pytest.raises(t.IdxError, match=match):
        fn(*args, **kw)


def test_query_shapes():
    raises(t.Query, u8(4, 8, 64), u8(4, 8, 4), f32(4, 7), match="query shapes")
    raises(t.Query, u8(4, 8, 64), u8(5, 8, 4), f32(4, 8), match="query shapes")
    raises(t.Query, u8(4, 8, 64), u8(4, 8, 4), f32(4, 8), match="must be on the GPU")


def test_rows_shapes():
    raises(t.Rows, i32(4), i32(5), match="len: leading dimension")
    raises(t.Rows, i32(4), i32(4), i32(3), match="pos_offset: leading dimension")
    raises(t.Rows, i32(4), i32(4), match="must be on the GPU")


def test_amax8_shapes():
    raises(t.idx_amax8_varlen, f32(3, 64), i32(4), f32(4, 8), match="S: leading dimension")
    raises(t.idx_amax8_varlen, f32(4, 64), i32(4), f32(5, 8), match="keys: leading dimension")


def test_topk_blocks_shapes():
    raises(t.idx_topk_blocks, f32(4, 64), i32(4), 16, i32(3, 16), i32(4), match="blocks: leading")
    raises(t.idx_topk_blocks, f32(4, 64), i32(4), 16, i32(4, 16), i32(2), match="n_kept: leading")
    raises(t.idx_topk_blocks, f32(2, 64), i32(4), 16, i32(4, 16), i32(4), match="keys: leading")
    raises(t.idx_topk_blocks, f32(4, 64), i32(4), 16, i32(4, 8), i32(4), match="blocks must be")


def test_topk_rows_shapes():
    raises(t.idx_topk_rows, f32(3, 128), i32(4), 8, i32(4, 8), match="X: leading")
    raises(t.idx_topk_rows, f32(4, 128), i32(4), 8, i32(5, 8), match="out: leading")
    raises(t.idx_topk_rows, f32(4, 128), i32(4), 8, i32(4, 7), match="out must be")
    raises(t.idx_topk_rows, f32(4, 128), i32(4), 8, i32(4, 8), mode=t.COLS_BLOCKMAP,
           blocks=i32(3, 16), match="blocks: leading")
    raises(t.idx_topk_rows, f32(4, 100), i32(4), 8, i32(4, 8), mode=t.COLS_BLOCKMAP,
           blocks=i32(4, 16), match="needs at least 128 columns")
    raises(t.idx_topk_rows, f32(4, 128), i32(4), 8, i32(4, 8), mode=t.COLS_GATHER,
           match="blocks are required")
    raises(t.idx_topk_rows, f32(4, 128), i32(4), 8, i32(4, 8), pos_offset=i32(2),
           match="pos_offset: leading")
    raises(t.idx_topk_rows_bf16, torch.zeros((3, 128), dtype=torch.bfloat16), i32(4), 8, i32(4, 8),
           match="X: leading")


def test_score_shapes():
    q = object.__new__(t.Query)
    q.rows, q.heads = 4, 8
    rows = object.__new__(t.Rows)
    rows.rows = 5
    raises(t.idx_score_dense, q, None, rows, f32(4, 64), match="query rows 4 != rows 5")
    rows.rows = 4
    raises(t.idx_score_dense, q, None, rows, f32(3, 64), match="S: leading")
    raises(t.idx_score_dense_keys, q, None, rows, f32(4, 64), f32(3, 8), match="keys: leading")
    raises(t.idx_score_sparse_paged, q, None, fake_table(4, 16), f32(3, 128), match="T: leading")
    raises(t.idx_score_sparse_paged, q, None, fake_table(4, 16), f32(4, 127), match="at least 128")
    raises(t.idx_score_sparse_paged, q, None, fake_table(5, 16), f32(4, 128), match="table rows 5")
    raises(t.idx_expand_candidates, None, rows, fake_table(3, 16), match="table rows 3 != rows 4")


def test_tail_shapes():
    tail = fake_table(2, 16)
    tail.blocks = i32(2, 16)
    raises(t.idx_prefill_tail, fake_table(4, 16), i32(3), i32(2), tail, match="tail_len: leading")
