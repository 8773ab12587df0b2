"""Python binding of libidx, the gfx950 two-level candidate indexer.

Argument marshalling only: torch tensors in, raw device pointers and the
current HIP stream out to the C ABI of include/idx.h.  Every step runs in the
library's HIP kernels; there is no fallback.  If libidx.so has not been built
(``python -c "import __graft_entry__ as g; g.build()"``), every call raises.

Names follow the C ABI: idx_score_dense, idx_score_dense_keys, idx_q_rope_quant,
idx_amax8_varlen, idx_topk_blocks,
idx_expand_candidates, idx_score_sparse_paged, idx_score_sparse_paged_bf16, idx_topk_rows,
idx_topk_rows_bf16, idx_prefill_tail.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "IdxError", "Query", "KPool", "Rows", "Table", "load",
    "idx_score_dense", "idx_score_dense_keys", "idx_q_rope_quant", "idx_amax8_varlen", "idx_topk_blocks",
    "idx_topk_blocks_nested", "idx_expand_candidates",
    "idx_score_sparse_paged", "idx_score_sparse_paged_bf16", "idx_score_sparse_paged_noalloc",
    "idx_topk_rows", "idx_topk_rows_bf16",
    "idx_prefill_tail", "idx_workspace_bytes",
    "COLS_IDENTITY", "COLS_BLOCKMAP", "COLS_GATHER", "stream_wait_table", "score_workspace",
    "tail_workspace",
]

HERE = os.path.dirname(os.path.abspath(__file__))
# IDX_LIBRARY selects another build of the same library (e.g. a sanitizer build
# of its host code); the default is the in-tree gfx950 build
LIB_PATH = os.environ.get("IDX_LIBRARY") or os.path.join(HERE, "libidx.so")

COLS_IDENTITY, COLS_BLOCKMAP, COLS_GATHER = 0, 1, 2
OP_TOPK_BLOCKS, OP_TOPK_ROWS, OP_SCHEDULE, OP_TAIL, OP_SCORE = 1, 2, 3, 4, 5
INT32_MAX = 2 ** 31 - 1


class IdxError(RuntimeError):
    pass


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


class _Query(ctypes.Structure):
    _fields_ = [("vals", _P), ("scales", _P), ("w", _P), ("rows", _I32), ("heads", _I32),
                ("dim", _I32), ("folded", _P)]


class _KPool(ctypes.Structure):
    _fields_ = [("pool", _P), ("num_pages", _I32), ("page_size", _I32), ("dim", _I32),
                ("page_table", _P), ("num_req", _I32), ("max_pages", _I32)]


class _Rows(ctypes.Structure):
    _fields_ = [("req", _P), ("len", _P), ("pos_offset", _P), ("rows", _I32)]


class _Table(ctypes.Structure):
    _fields_ = [("blocks", _P), ("n_kept", _P), ("phys", _P), ("valid_len", _P), ("len", _P),
                ("req", _P), ("schedule", _P), ("schedule_bytes", ctypes.c_size_t),
                ("rows", _I32), ("kb", _I32), ("ready", _P)]


_lib = None
_hip = None


def load():
    """Load libidx.so (and the HIP runtime for events); raise if it is not built."""
    global _lib, _hip
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise IdxError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    st = ctypes.c_int
    sig = {
        "idx_score_dense": [ctypes.POINTER(_Query), ctypes.POINTER(_KPool), ctypes.POINTER(_Rows), _P, _I64, _P, ctypes.c_size_t, _P],
        "idx_amax8_varlen": [_P, _I64, _P, _I32, _P, _I64, _I32, _P],
        "idx_q_rope_quant": [_P, _P, _P, _I32, _P, _I32, _I32, _I32, ctypes.c_float, ctypes.c_float, _P, _P, _P, _P],
        "idx_score_dense_keys": [ctypes.POINTER(_Query), ctypes.POINTER(_KPool), ctypes.POINTER(_Rows), _P, _I64, _P, _I64, _I32, _P, ctypes.c_size_t, _P],
        "idx_topk_blocks": [_P, _I64, _P, _I32, _I32, _P, _P, _P, ctypes.c_size_t, _P],
        "idx_topk_blocks_nested": [_P, _I64, _P, _I32, _I32, _P, _P, _I32, _P, _P, _P, ctypes.c_size_t, _P],
        "idx_expand_candidates": [ctypes.POINTER(_KPool), ctypes.POINTER(_Rows), ctypes.POINTER(_Table), _P],
        "idx_score_sparse_paged": [ctypes.POINTER(_Query), ctypes.POINTER(_KPool), ctypes.POINTER(_Table), _P, _I64, _P, ctypes.c_size_t, _P],
        "idx_topk_rows": [_P, _I64, _P, _I32, _I32, ctypes.c_int, _P, _I32, _P, _P, _P, ctypes.c_size_t, _P],
        "idx_topk_rows_bf16": [_P, _I64, _P, _I32, _I32, ctypes.c_int, _P, _I32, _P, _P, _P, ctypes.c_size_t, _P],
        "idx_score_sparse_paged_bf16": [ctypes.POINTER(_Query), ctypes.POINTER(_KPool), ctypes.POINTER(_Table), _P, _I64, _P, ctypes.c_size_t, _P],
        "idx_prefill_tail": [ctypes.POINTER(_Table), _P, _P, _I32, ctypes.POINTER(_Table), _P, ctypes.c_size_t, _P],
        "idx_score_sparse_paged_noalloc": [ctypes.POINTER(_Query), ctypes.POINTER(_KPool), ctypes.POINTER(_Table), _P, _I64, _P],
        "idx_fold_queries": [ctypes.POINTER(_Query), _I32, ctypes.POINTER(_P), ctypes.POINTER(ctypes.c_size_t), _P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = st
    lib.idx_last_error.restype = ctypes.c_char_p
    lib.idx_last_error.argtypes = []
    lib.idx_version.restype = ctypes.c_char_p
    lib.idx_version.argtypes = []
    lib.idx_workspace_bytes.restype = ctypes.c_size_t
    lib.idx_workspace_bytes.argtypes = [ctypes.c_int, _I32, _I64, _I32]
    _lib = lib
    return lib


def _hip_rt():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(_P), ctypes.c_uint]
        _hip.hipEventCreateWithFlags.restype = ctypes.c_int
        _hip.hipEventDestroy.argtypes = [_P]
        _hip.hipEventDestroy.restype = ctypes.c_int
        _hip.hipStreamWaitEvent.argtypes = [_P, _P, ctypes.c_uint]
        _hip.hipStreamWaitEvent.restype = ctypes.c_int
    return _hip


def stream_wait_table(tbl: "Table", stream=None):
    """Make `stream` (default: current) wait until tbl.ready has been reached."""
    if tbl.ready is None:
        return
    rc = _hip_rt().hipStreamWaitEvent(_stream(stream), tbl.ready, 0)
    if rc != 0:
        raise IdxError(f"hipStreamWaitEvent failed ({rc})")


def _check(status: int, name: str):
    if status != 0:
        msg = load().idx_last_error().decode(errors="replace")
        raise IdxError(f"{name} failed ({status}): {msg}")


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _req(t: torch.Tensor, dtype, name: str, rows: int | None = None, gpu: bool = True):
    """Type, dtype, contiguity and (when given) leading dimension of one operand;
    with gpu=False the device is left to a later _on_gpu call, so that every
    shape check of a call runs before any device check."""
    if not isinstance(t, torch.Tensor):
        raise IdxError(f"{name}: expected a tensor")
    if t.dtype != dtype:
        raise IdxError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise IdxError(f"{name}: must be contiguous")
    if rows is not None and (t.dim() == 0 or int(t.shape[0]) != rows):
        raise IdxError(f"{name}: leading dimension {tuple(t.shape)[:1]} != {rows} rows")
    if gpu:
        _on_gpu(t, names=(name,))
    return t


def _on_gpu(*ts, names=None):
    for i, t in enumerate(ts):
        if t is not None and not t.is_cuda:
            raise IdxError(f"{names[i] if names else 'operand'}: must be on the GPU")


def _width(t: torch.Tensor, need: int, name: str):
    if t.dim() != 2 or int(t.shape[1]) < need:
        raise IdxError(f"{name}: shape {tuple(t.shape)} needs at least {need} columns")


# ---------------------------------------------------------------------------
# operand bundles
# ---------------------------------------------------------------------------

class Query:
    """One index layer's query batch: vals u8 [R,H,64], scales u8 [R,H,4], w f32 [R,H].
    `folded`: None, or a workspace that idx_fold_queries filled with this batch's
    folded query; the score calls then read it instead of folding themselves."""

    def __init__(self, vals, scales, w):
        self.folded = None
        self.vals = _req(vals, torch.uint8, "vals", gpu=False)
        self.scales = _req(scales, torch.uint8, "scales", gpu=False)
        self.w = _req(w, torch.float32, "w", gpu=False)
        if vals.dim() != 3:
            raise IdxError("query shapes must be [R,H,64], [R,H,4], [R,H]")
        self.rows, self.heads = int(vals.shape[0]), int(vals.shape[1])
        if tuple(vals.shape) != (self.rows, self.heads, 64) or \
           tuple(scales.shape) != (self.rows, self.heads, 4) or tuple(w.shape) != (self.rows, self.heads):
            raise IdxError("query shapes must be [R,H,64], [R,H,4], [R,H]")
        _on_gpu(self.vals, self.scales, self.w, names=("vals", "scales", "w"))

    def c(self):
        folded = None
        if self.folded is not None:
            folded = _req(self.folded, torch.uint8, "folded")
            if folded.numel() < idx_workspace_bytes(OP_SCORE, self.rows, 0, 0):
                raise IdxError("folded: smaller than the query's fold workspace")
        return _Query(_ptr(self.vals), _ptr(self.scales), _ptr(self.w), self.rows, self.heads, 128,
                      _ptr(folded))


class KPool:
    """Paged MXFP4 index-K pool u8 [pages, 64*68] and page table i32 [num_req, max_pages]."""

    def __init__(self, pool, page_table, page_size: int = 64):
        self.pool = _req(pool, torch.uint8, "pool", gpu=False)
        self.page_table = _req(page_table, torch.int32, "page_table", gpu=False)
        self.page_size = page_size
        if pool.dim() != 2 or pool.shape[1] != page_size * 68:
            raise IdxError("pool must be [num_pages, page_size * 68]")
        if page_table.dim() != 2:
            raise IdxError("page_table must be [num_req, max_pages]")
        _on_gpu(self.pool, self.page_table, names=("pool", "page_table"))

    def c(self):
        return _KPool(_ptr(self.pool), int(self.pool.shape[0]), self.page_size, 128,
                      _ptr(self.page_table), int(self.page_table.shape[0]),
                      int(self.page_table.shape[1]))


class Rows:
    """Per-row request ids, compress_lens and optional output offsets (all i32 [R])."""

    def __init__(self, req, lens, pos_offset=None):
        if not isinstance(req, torch.Tensor) or req.dim() != 1:
            raise IdxError("req must be a 1-d tensor")
        self.rows = int(req.shape[0])
        self.req = _req(req, torch.int32, "req", gpu=False)
        self.len = _req(lens, torch.int32, "len", rows=self.rows, gpu=False)
        self.pos_offset = None if pos_offset is None else \
            _req(pos_offset, torch.int32, "pos_offset", rows=self.rows, gpu=False)
        _on_gpu(self.req, self.len, self.pos_offset, names=("req", "len", "pos_offset"))

    def c(self):
        return _Rows(_ptr(self.req), _ptr(self.len), _ptr(self.pos_offset), self.rows)


class Table:
    """A published candidate table; allocated on the current (consumer) stream."""

    def __init__(self, rows: int, kb: int, device="cuda", with_event: bool = True):
        lib = load()
        i32 = dict(dtype=torch.int32, device=device)
        self.rows, self.kb = rows, kb
        self.blocks = torch.empty((rows, kb), **i32)
        self.n_kept = torch.empty((rows,), **i32)
        self.phys = torch.empty((rows, kb), **i32)
        self.valid_len = torch.empty((rows,), **i32)
        self.len = torch.empty((rows,), **i32)
        self.req = torch.empty((rows,), **i32)
        nb = lib.idx_workspace_bytes(OP_SCHEDULE, rows, kb, 0)
        self.schedule = torch.empty((max(nb, 16),), dtype=torch.uint8, device=device)
        self.ready = None
        if with_event:
            ev = _P()
            rc = _hip_rt().hipEventCreateWithFlags(ctypes.byref(ev), 0x2)  # disable timing
            if rc != 0:
                raise IdxError(f"hipEventCreateWithFlags failed ({rc})")
            self.ready = ev

    def tensors(self):
        return [self.blocks, self.n_kept, self.phys, self.valid_len, self.len, self.req, self.schedule]

    def record_stream(self, stream):
        for t in self.tensors():
            t.record_stream(stream)

    def c(self):
        return _Table(_ptr(self.blocks), _ptr(self.n_kept), _ptr(self.phys), _ptr(self.valid_len),
                      _ptr(self.len), _ptr(self.req), _ptr(self.schedule),
                      int(self.schedule.numel()), self.rows, self.kb, self.ready)

    def __del__(self):
        if getattr(self, "ready", None) is not None and _hip is not None:
            try:
                _hip.hipEventDestroy(self.ready)
            except Exception:
                pass
            self.ready = None


# ---------------------------------------------------------------------------
# the seven calls
# ---------------------------------------------------------------------------

def idx_workspace_bytes(op: int, rows: int, width: int, k: int) -> int:
    return int(load().idx_workspace_bytes(op, rows, width, k))


def score_workspace(rows: int, device="cuda") -> torch.Tensor:
    """Workspace of idx_score_dense / idx_score_sparse_paged for `rows` query rows."""
    n = max(16, idx_workspace_bytes(OP_SCORE, rows, 0, 0))
    return torch.empty((n,), dtype=torch.uint8, device=device)


def idx_fold_queries(queries, workspaces, stream=None):
    """The folded queries of several query batches in one launch: workspaces[i]
    (score_workspace(queries[i].rows)) gets batch i's; set queries[i].folded to it
    for the score calls that follow."""
    n = len(queries)
    if n != len(workspaces) or not 1 <= n <= 16:
        raise IdxError("idx_fold_queries: 1..16 queries, one workspace each")
    qs = (_Query * n)(*[q.c() for q in queries])
    ws = [_req(w, torch.uint8, "ws") for w in workspaces]
    for q, w in zip(queries, ws):
        if w.numel() < idx_workspace_bytes(OP_SCORE, q.rows, 0, 0):
            raise IdxError("idx_fold_queries: workspace too small")
        _on_gpu(q.vals, w, names=("vals", "ws"))
    ptrs = (_P * n)(*[_ptr(w) for w in ws])
    sizes = (ctypes.c_size_t * n)(*[w.numel() for w in ws])
    _check(load().idx_fold_queries(qs, n, ptrs, sizes, _stream(stream)), "idx_fold_queries")


def _numel(t):
    return 0 if t is None else t.numel()


def _score_ws(ws, rows, device, stream, q=None):
    if q is not None and q.folded is not None:
        return None   # the folded query is read from q.folded
    if ws is None:
        ws = score_workspace(rows, device)
        if stream is not None:
            ws.record_stream(stream)
    return _req(ws, torch.uint8, "ws")


def idx_score_dense(q: Query, kp: KPool, rows: Rows, S: torch.Tensor, ws=None, stream=None):
    if q.rows != rows.rows:
        raise IdxError(f"query rows {q.rows} != rows {rows.rows}")
    _req(S, torch.float32, "S", rows=rows.rows)
    ws = _score_ws(ws, q.rows, S.device, stream, q)
    q_c, kp_c, rows_c = q.c(), kp.c(), rows.c()
    _check(load().idx_score_dense(ctypes.byref(q_c), ctypes.byref(kp_c), ctypes.byref(rows_c),
                                  _ptr(S), S.stride(0), _ptr(ws), _numel(ws), _stream(stream)),
           "idx_score_dense")


def idx_score_dense_keys(q: Query, kp: KPool, rows: Rows, S: torch.Tensor | None, keys: torch.Tensor,
                         skip_le_blocks: int = 0, ws=None, stream=None, ld: int | None = None):
    """S=None: keys only (the scores are never written); then `ld` (>= the longest
    row, a multiple of 8) must be given, as the stride the scores would have."""
    if q.rows != rows.rows:
        raise IdxError(f"query rows {q.rows} != rows {rows.rows}")
    if S is not None:
        _req(S, torch.float32, "S", rows=rows.rows, gpu=False)
        ld = S.stride(0)
    elif ld is None:
        raise IdxError("keys only (S=None) needs ld")
    _req(keys, torch.float32, "keys", rows=rows.rows, gpu=False)
    _on_gpu(S, keys, names=("S", "keys"))
    ws = _score_ws(ws, q.rows, keys.device, stream, q)
    q_c, kp_c, rows_c = q.c(), kp.c(), rows.c()
    _check(load().idx_score_dense_keys(ctypes.byref(q_c), ctypes.byref(kp_c), ctypes.byref(rows_c),
                                       _ptr(S), int(ld), _ptr(keys), keys.stride(0),
                                       int(skip_le_blocks), _ptr(ws), _numel(ws), _stream(stream)),
           "idx_score_dense_keys")


def idx_q_rope_quant(q_bits: torch.Tensor, positions: torch.Tensor, cos_sin: torch.Tensor,
                     w: torch.Tensor, is_neox: bool, softmax_scale: float, head_scale: float,
                     vals: torch.Tensor, scales: torch.Tensor, w_out: torch.Tensor, stream=None):
    """q_bits: bf16 bit patterns as int16 [rows, heads, 128]; outputs an idx_query's arrays."""
    args = {"q": (q_bits, torch.int16), "positions": (positions, torch.int32),
            "cos_sin": (cos_sin, torch.float32), "w": (w, torch.float32),
            "vals": (vals, torch.uint8), "scales": (scales, torch.uint8),
            "w_out": (w_out, torch.float32)}
    for name, (t, dt) in args.items():
        _req(t, dt, name, gpu=False)
    if q_bits.dim() != 3:
        raise IdxError("q must be [rows, heads, 128]")
    rows, heads = int(q_bits.shape[0]), int(q_bits.shape[1])
    shapes = {"q": (q_bits, (rows, heads, 128)), "positions": (positions, (rows,)),
              "w": (w, (rows, heads)), "vals": (vals, (rows, heads, 64)),
              "scales": (scales, (rows, heads, 4)), "w_out": (w_out, (rows, heads))}
    for name, (t, shape) in shapes.items():
        if tuple(t.shape) != shape:
            raise IdxError(f"{name}: shape {tuple(t.shape)}, expected {shape}")
    if cos_sin.dim() != 2 or cos_sin.shape[1] != 64:
        raise IdxError("cos_sin must be [max_pos, 64]")
    _on_gpu(*(t for t, _ in args.values()), names=tuple(args))
    _check(load().idx_q_rope_quant(_ptr(q_bits), _ptr(positions), _ptr(cos_sin), int(cos_sin.shape[0]),
                                   _ptr(w), rows, heads, 1 if is_neox else 0, float(softmax_scale),
                                   float(head_scale), _ptr(vals), _ptr(scales), _ptr(w_out),
                                   _stream(stream)), "idx_q_rope_quant")


def idx_amax8_varlen(S, lens, keys, skip_le_blocks: int = 0, stream=None):
    _req(lens, torch.int32, "len", gpu=False)
    n = int(lens.shape[0]) if lens.dim() == 1 else -1
    _req(S, torch.float32, "S", rows=n, gpu=False)
    _req(keys, torch.float32, "keys", rows=n, gpu=False)
    _on_gpu(S, lens, keys, names=("S", "len", "keys"))
    _check(load().idx_amax8_varlen(_ptr(S), S.stride(0), _ptr(lens), n, _ptr(keys),
                                   keys.stride(0), int(skip_le_blocks), _stream(stream)),
           "idx_amax8_varlen")


def idx_topk_blocks(keys, lens, kb: int, blocks, n_kept, stream=None):
    _req(lens, torch.int32, "len", gpu=False)
    n = int(lens.shape[0]) if lens.dim() == 1 else -1
    _req(keys, torch.float32, "keys", rows=n, gpu=False)
    _req(blocks, torch.int32, "blocks", rows=n, gpu=False)
    _req(n_kept, torch.int32, "n_kept", rows=n, gpu=False)
    if blocks.dim() != 2 or blocks.shape[-1] != kb:
        raise IdxError("blocks must be [rows, kb]")
    _on_gpu(keys, lens, blocks, n_kept, names=("keys", "len", "blocks", "n_kept"))
    _check(load().idx_topk_blocks(_ptr(keys), keys.stride(0), _ptr(lens), n, kb,
                                  _ptr(blocks), _ptr(n_kept), None, 0, _stream(stream)),
           "idx_topk_blocks")


def idx_topk_blocks_nested(keys, lens, kb: int, blocks, n_kept, k2: int, blocks2, n_kept2,
                           stream=None):
    _req(lens, torch.int32, "len", gpu=False)
    n = int(lens.shape[0]) if lens.dim() == 1 else -1
    _req(keys, torch.float32, "keys", rows=n, gpu=False)
    for name, t in (("blocks", blocks), ("n_kept", n_kept), ("blocks2", blocks2), ("n_kept2", n_kept2)):
        _req(t, torch.int32, name, rows=n, gpu=False)
    if blocks.dim() != 2 or blocks.shape[-1] != kb:
        raise IdxError("blocks must be [rows, kb]")
    if blocks2.dim() != 2 or blocks2.shape[-1] != k2:
        raise IdxError("blocks2 must be [rows, k2]")
    _on_gpu(keys, lens, blocks, n_kept, blocks2, n_kept2,
            names=("keys", "len", "blocks", "n_kept", "blocks2", "n_kept2"))
    _check(load().idx_topk_blocks_nested(_ptr(keys), keys.stride(0), _ptr(lens), n, kb, _ptr(blocks),
                                         _ptr(n_kept), k2, _ptr(blocks2), _ptr(n_kept2), None, 0,
                                         _stream(stream)), "idx_topk_blocks_nested")


def idx_expand_candidates(kp: KPool, rows: Rows, tbl: Table, stream=None):
    if tbl.rows != rows.rows:
        raise IdxError(f"table rows {tbl.rows} != rows {rows.rows}")
    kp_c, rows_c, t_c = kp.c(), rows.c(), tbl.c()
    _check(load().idx_expand_candidates(ctypes.byref(kp_c), ctypes.byref(rows_c), ctypes.byref(t_c),
                                        _stream(stream)), "idx_expand_candidates")


def _sparse_args(q: Query, tbl: Table, T: torch.Tensor, dtype):
    if q.rows != tbl.rows:
        raise IdxError(f"query rows {q.rows} != table rows {tbl.rows}")
    _req(T, dtype, "T", rows=tbl.rows, gpu=False)
    _width(T, tbl.kb * 8, "T")
    _on_gpu(T, names=("T",))


def idx_score_sparse_paged(q: Query, kp: KPool, tbl: Table, T: torch.Tensor, ws=None, stream=None,
                           wait_ready: bool = True):
    """wait_ready=False: the call runs on the stream that built the table, so it does
    not wait on the table's ready event (a stream never waits on an event it recorded)."""
    _sparse_args(q, tbl, T, torch.float32)
    ws = _score_ws(ws, q.rows, T.device, stream, q)
    q_c, kp_c, t_c = q.c(), kp.c(), tbl.c()
    if not wait_ready:
        t_c.ready = None
    _check(load().idx_score_sparse_paged(ctypes.byref(q_c), ctypes.byref(kp_c), ctypes.byref(t_c),
                                         _ptr(T), T.stride(0), _ptr(ws), _numel(ws),
                                         _stream(stream)),
           "idx_score_sparse_paged")


def idx_score_sparse_paged_noalloc(q: Query, kp: KPool, tbl: Table, T: torch.Tensor, stream=None):
    """idx_score_sparse_paged with the folded queries in the library's static scratch
    (at most 4096 query rows): allocates nothing."""
    _sparse_args(q, tbl, T, torch.float32)
    q_c, kp_c, t_c = q.c(), kp.c(), tbl.c()
    _check(load().idx_score_sparse_paged_noalloc(ctypes.byref(q_c), ctypes.byref(kp_c),
                                                 ctypes.byref(t_c), _ptr(T), T.stride(0),
                                                 _stream(stream)),
           "idx_score_sparse_paged_noalloc")


def idx_score_sparse_paged_bf16(q: Query, kp: KPool, tbl: Table, T: torch.Tensor, ws=None,
                                stream=None):
    """T: torch.bfloat16 [rows, >= kb * 8]."""
    _sparse_args(q, tbl, T, torch.bfloat16)
    ws = _score_ws(ws, q.rows, T.device, stream, q)
    q_c, kp_c, t_c = q.c(), kp.c(), tbl.c()
    _check(load().idx_score_sparse_paged_bf16(ctypes.byref(q_c), ctypes.byref(kp_c), ctypes.byref(t_c),
                                              _ptr(T), T.stride(0), _ptr(ws), _numel(ws),
                                              _stream(stream)),
           "idx_score_sparse_paged_bf16")


def _topk_args(X, xdtype, valid, k, out, mode, blocks, pos_offset):
    _req(valid, torch.int32, "valid", gpu=False)
    n = int(valid.shape[0]) if valid.dim() == 1 else -1
    _req(X, xdtype, "X", rows=n, gpu=False)
    _req(out, torch.int32, "out", rows=n, gpu=False)
    if out.dim() != 2 or out.shape[-1] != k:
        raise IdxError("out must be [rows, k]")
    kb = 0
    if blocks is not None:
        _req(blocks, torch.int32, "blocks", rows=n, gpu=False)
        kb = int(blocks.shape[-1])
        if mode == COLS_BLOCKMAP:
            _width(X, kb * 8, "X")
    elif mode != COLS_IDENTITY:
        raise IdxError("blocks are required in the block-mapped modes")
    if pos_offset is not None:
        _req(pos_offset, torch.int32, "pos_offset", rows=n, gpu=False)
    _on_gpu(X, valid, out, blocks, pos_offset, names=("X", "valid", "out", "blocks", "pos_offset"))
    return n, kb


def idx_topk_rows_bf16(X, valid, k: int, out, mode: int = COLS_IDENTITY, blocks=None,
                       pos_offset=None, stream=None):
    """X: torch.bfloat16 rows; as idx_topk_rows otherwise."""
    n, kb = _topk_args(X, torch.bfloat16, valid, k, out, mode, blocks, pos_offset)
    _check(load().idx_topk_rows_bf16(_ptr(X), X.stride(0), _ptr(valid), n, k, mode,
                                     _ptr(blocks), kb, _ptr(pos_offset), _ptr(out), None, 0,
                                     _stream(stream)), "idx_topk_rows_bf16")


def idx_topk_rows(X, valid, k: int, out, mode: int = COLS_IDENTITY, blocks=None, pos_offset=None,
                  stream=None):
    n, kb = _topk_args(X, torch.float32, valid, k, out, mode, blocks, pos_offset)
    _check(load().idx_topk_rows(_ptr(X), X.stride(0), _ptr(valid), n, k, mode,
                                _ptr(blocks), kb, _ptr(pos_offset), _ptr(out), None, 0,
                                _stream(stream)), "idx_topk_rows")


def tail_workspace(num_req: int, device="cuda") -> torch.Tensor:
    """Workspace of idx_prefill_tail for num_req requests."""
    n = max(16, idx_workspace_bytes(OP_TAIL, num_req, 0, 0))
    return torch.empty((n,), dtype=torch.uint8, device=device)


def idx_prefill_tail(full: Table, rows_per_req, tail_len, tail: Table, ws=None, stream=None,
                     wait_full: bool = True):
    """rows_per_req, tail_len: int32 device tensors [num_req] (array-likes are copied to the
    tail table's device first, which a graph capture cannot record: pass tensors there).
    wait_full=False: the call runs on the stream that built `full`, so it does not wait
    on full's ready event (a stream never waits on an event it recorded itself)."""
    dev = tail.blocks.device
    if not isinstance(rows_per_req, torch.Tensor):
        rows_per_req = torch.as_tensor(rows_per_req, dtype=torch.int32).to(dev)
    if not isinstance(tail_len, torch.Tensor):
        tail_len = torch.as_tensor(tail_len, dtype=torch.int32).to(dev)
    _req(rows_per_req, torch.int32, "rows_per_req", gpu=False)
    num_req = int(rows_per_req.shape[0]) if rows_per_req.dim() == 1 else -1
    _req(tail_len, torch.int32, "tail_len", rows=num_req, gpu=False)
    _on_gpu(rows_per_req, tail_len, names=("rows_per_req", "tail_len"))
    if ws is None:
        ws = tail_workspace(num_req, dev)
        if stream is not None:
            ws.record_stream(stream)
    _req(ws, torch.uint8, "ws")
    f_c, t_c = full.c(), tail.c()
    if not wait_full:
        f_c.ready = None
    _check(load().idx_prefill_tail(ctypes.byref(f_c), _ptr(rows_per_req), _ptr(tail_len), num_req,
                                   ctypes.byref(t_c), _ptr(ws), ws.numel(), _stream(stream)),
           "idx_prefill_tail")
    return ws
