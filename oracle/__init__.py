"""CPU oracle of the two-level candidate indexer (DeepSeek-V4.1).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the product path never does.  It shares
no code with the HIP library; both read the bytes made by ``workloads``.

Each step follows the sglang PR "[DSv4.1] Score prefill consumer index layers
on candidate blocks with DeepGEMM" (cited below as "the prefill PR"), the
sglang PR "dsv4.1: candidate indexer library" ("the library PR") and the
vLLM sparse_attn_indexer page ("the vLLM indexer page"):

1. ``dense_scores``   the source layer's score of every reachable position
                      (C, exact, one rounding to fp32; see idx_oracle.c).
2. ``block_keys``     one key per block of 8 positions: the block's maximum,
                      the row's newest block forced to +inf; rows with at most
                      kb blocks are not keyed (prefill PR, "Level one", and the
                      block_amax.cuh contract quoted in its review thread).
3. ``select_blocks``  the kb best blocks by (key desc, block id asc), returned
                      ascending and padded with INT32_MAX; rows with at most kb
                      blocks keep every block (prefill PR, "Level one";
                      sort_candidate_blocks in the library PR summary).
4. ``expand``         pool block of each candidate and the row's count of valid
                      candidate columns (prefill PR, "Level one"/"Level two").
5. ``scores_at``      a consumer's scores at its candidate positions, column i
                      being position blocks[i // 8] * 8 + i % 8 (prefill PR,
                      "Level two").
6. ``topk_positions`` top-k columns by (score desc, column asc), mapped to
                      positions, ascending, -1 past min(k, valid) (prefill PR,
                      "Level two"; the -1 sentinel of the vLLM indexer page).
7. ``tail_rows``      the last t_j rows of each request (prefill PR, "Tail rows"
                      and the prefill_tail snippet in its review thread).

Readings where the pages are silent are listed in the repository's design
notes; the two that change results are: ties go to the lower index, and
outputs are sorted ascending.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

INT32_MAX = np.iinfo(np.int32).max
BLOCK = 8

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libidx_oracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile idx_oracle.c into libidx_oracle.so (gcc, OpenMP)."""
    import subprocess
    src = os.path.join(_HERE, "idx_oracle.c")
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11",
           "-Wall", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        # IDX_ORACLE_LIBRARY: another build of idx_oracle.c (the sanitizer build
        # of tests/test_host_sanitizers.py)
        path = os.environ.get("IDX_ORACLE_LIBRARY")
        if not path:
            if not os.path.exists(_LIB_PATH):
                build()
            path = _LIB_PATH
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.oracle_e2m1_value.restype = ctypes.c_double
        lib.oracle_e2m1_value.argtypes = [ctypes.c_int]
        lib.oracle_ue8m0_value.restype = ctypes.c_double
        lib.oracle_ue8m0_value.argtypes = [ctypes.c_int]
        lib.oracle_dense_scores.restype = i64
        lib.oracle_dense_scores.argtypes = [P, ctypes.c_int, P, P, P, ctypes.c_int, P, P, P, P,
                                            ctypes.c_int, ctypes.c_int, P, i64]
        lib.oracle_scores_at.restype = i64
        lib.oracle_scores_at.argtypes = [P, ctypes.c_int, P, P, P, ctypes.c_int, P, P, i64, P, P,
                                         ctypes.c_int, ctypes.c_int, P, i64]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def e2m1_value(nibble: int) -> float:
    return _load().oracle_e2m1_value(int(nibble))


def ue8m0_value(byte: int) -> float:
    return _load().oracle_ue8m0_value(int(byte))


def _rows(row_ids, R):
    if row_ids is None:
        return np.arange(R, dtype=np.int32)
    return np.ascontiguousarray(np.asarray(row_ids, dtype=np.int32))


# ---------------------------------------------------------------------------
# 1. dense source scores
# ---------------------------------------------------------------------------

def dense_scores(qv, qs, w, req, lens, pool, page_table, page_size=64, row_ids=None, ld=None):
    """S[i, p] = sum_h w[r,h] * max(0, q^[r,h] . k^[p]) for p < lens[r], r = row_ids[i].

    Entries at p >= lens[r] are NaN (outside the definition)."""
    H = qv.shape[1]
    rows = _rows(row_ids, qv.shape[0])
    if ld is None:
        ld = max(8, (int(lens[rows].max()) + 7) // 8 * 8) if len(rows) else 8
    out = np.full((len(rows), ld), np.nan, dtype=np.float32)
    if len(rows):
        nbad = _load().oracle_dense_scores(
            _ptr(rows), len(rows), _ptr(np.ascontiguousarray(qv)), _ptr(np.ascontiguousarray(qs)),
            _ptr(np.ascontiguousarray(w, dtype=np.float32)), H,
            _ptr(np.ascontiguousarray(req, dtype=np.int32)),
            _ptr(np.ascontiguousarray(lens, dtype=np.int32)), _ptr(np.ascontiguousarray(pool)),
            _ptr(np.ascontiguousarray(page_table, dtype=np.int32)), page_table.shape[1], page_size,
            _ptr(out), ld)
        if nbad:
            raise ValueError(f"oracle: {nbad} logits outside the exact range (scale 255 or span)")
    return out


# ---------------------------------------------------------------------------
# 2. block keys
# ---------------------------------------------------------------------------

def nblocks(lens):
    return (np.asarray(lens, dtype=np.int64) + BLOCK - 1) // BLOCK


def block_keys(S, lens, kb, ldk=None):
    """key[i, b] = max(S[i, 8b : 8b+8]) for b < nblk-1, key[i, nblk-1] = +inf.

    Rows with nblk <= kb are left NaN (they are not keyed)."""
    n = S.shape[0]
    nb = nblocks(lens)
    if ldk is None:
        ldk = max(1, int(nb.max()) if n else 1)
    keys = np.full((n, ldk), np.nan, dtype=np.float32)
    for i in range(n):
        m = int(nb[i])
        if m <= kb:
            continue
        full = S[i, : (m - 1) * BLOCK].reshape(m - 1, BLOCK)
        keys[i, : m - 1] = full.max(axis=1)
        keys[i, m - 1] = np.inf
    return keys


# ---------------------------------------------------------------------------
# 3. block selection
# ---------------------------------------------------------------------------

def select_blocks(keys, lens, kb):
    """The kb best blocks of each row by (key desc, id asc), ascending, INT32_MAX pad."""
    n = len(lens)
    nb = nblocks(lens)
    blocks = np.full((n, kb), INT32_MAX, dtype=np.int32)
    n_kept = np.zeros(n, dtype=np.int32)
    for i in range(n):
        m = int(nb[i])
        if m <= kb:
            chosen = np.arange(m)
        else:
            ids = np.arange(m)
            order = np.lexsort((ids, -keys[i, :m].astype(np.float64)))
            chosen = np.sort(order[:kb])
        blocks[i, : len(chosen)] = chosen
        n_kept[i] = len(chosen)
    return blocks, n_kept


# ---------------------------------------------------------------------------
# 4. expansion
# ---------------------------------------------------------------------------

def expand(blocks, n_kept, lens, req, page_table, page_size=64):
    """phys[i, c] = pool block (page * blocks-per-page + block-in-page) of candidate c,
    -1 past n_kept; valid_len[i] = number of candidate positions below lens[i]."""
    n, kb = blocks.shape
    bpp = page_size // BLOCK
    phys = np.full((n, kb), -1, dtype=np.int32)
    valid = np.zeros(n, dtype=np.int32)
    for i in range(n):
        m = int(n_kept[i])
        b = blocks[i, :m].astype(np.int64)
        pages = page_table[req[i], b // bpp].astype(np.int64)
        phys[i, :m] = pages * bpp + b % bpp
        pos = b[:, None] * BLOCK + np.arange(BLOCK)[None, :]
        valid[i] = int((pos < lens[i]).sum())
    return phys, valid


def candidate_positions(blocks, valid_len):
    """Column c of a row is position blocks[c // 8] * 8 + c % 8; -1 past valid_len."""
    n, kb = blocks.shape
    cols = np.arange(kb * BLOCK)
    pos = blocks[:, cols // BLOCK].astype(np.int64) * BLOCK + cols % BLOCK
    pos = np.where(cols[None, :] < np.asarray(valid_len)[:, None], pos, -1)
    return pos.astype(np.int32)


# ---------------------------------------------------------------------------
# 5. consumer scores at candidate positions
# ---------------------------------------------------------------------------

def scores_at(qv, qs, w, req, positions, pool, page_table, page_size=64, row_ids=None):
    """T[i, c] = logit of query row r = row_ids[i] at positions[i, c] (NaN where -1)."""
    H = qv.shape[1]
    rows = _rows(row_ids, qv.shape[0])
    positions = np.ascontiguousarray(positions, dtype=np.int32)
    ncol = positions.shape[1]
    out = np.full((len(rows), max(ncol, 1)), np.nan, dtype=np.float32)
    if len(rows) and ncol:
        nbad = _load().oracle_scores_at(
            _ptr(rows), len(rows), _ptr(np.ascontiguousarray(qv)), _ptr(np.ascontiguousarray(qs)),
            _ptr(np.ascontiguousarray(w, dtype=np.float32)), H,
            _ptr(np.ascontiguousarray(req, dtype=np.int32)), _ptr(positions), ncol,
            _ptr(np.ascontiguousarray(pool)), _ptr(np.ascontiguousarray(page_table, dtype=np.int32)),
            page_table.shape[1], page_size, _ptr(out), out.shape[1])
        if nbad:
            raise ValueError(f"oracle: {nbad} logits outside the exact range (scale 255 or span)")
    return out[:, :ncol]


# ---------------------------------------------------------------------------
# 6. top-k
# ---------------------------------------------------------------------------

def topk_positions(X, valid, k, colmap=None, pos_offset=None):
    """Top-k of X[i, :valid[i]] by (value desc, column asc); columns mapped by colmap
    (colmap[i, c] = position of column c; identity if None), plus pos_offset[i];
    ascending; -1 past min(k, valid[i])."""
    n = X.shape[0]
    out = np.full((n, k), -1, dtype=np.int32)
    for i in range(n):
        v = int(valid[i])
        if v <= 0:
            continue
        cols = np.arange(v)
        order = np.lexsort((cols, -X[i, :v].astype(np.float64)))
        pick = order[:k]
        pos = pick.astype(np.int64) if colmap is None else colmap[i, pick].astype(np.int64)
        if pos_offset is not None:
            pos = pos + int(pos_offset[i])
        pos = np.sort(pos)
        out[i, : len(pos)] = pos
    return out


# ---------------------------------------------------------------------------
# 7. prefill tail
# ---------------------------------------------------------------------------

def tail_rows(rows_per_req, tail_len):
    """Indices of the last tail_len[j] rows of every request j, in row order."""
    out, start = [], 0
    for n, t in zip(rows_per_req, tail_len):
        n, t = int(n), int(t)
        out.extend(range(start + n - t, start + n))
        start += n
    return np.asarray(out, dtype=np.int32)


# ---------------------------------------------------------------------------
# the whole chunk
# ---------------------------------------------------------------------------

def run_chunk(wl, row_ids=None, n_consumers=None, k_source=None, with_offset=True):
    """Source layer + consumers over the rows `row_ids` of workload `wl`.

    Returns a dict of every intermediate, all indexed by position in row_ids."""
    rows = _rows(row_ids, wl.rows)
    lens = wl.lens[rows]
    req = wl.req[rows]
    off = wl.req_start[rows] if with_offset else None
    kb, kc = wl.kb, wl.kc
    src = wl.layers[0]
    S = dense_scores(src.qv, src.qs, src.w, wl.req, wl.lens, wl.pool, wl.page_table,
                     row_ids=rows, ld=wl.ld)
    keys = block_keys(S, lens, kb, ldk=wl.ldk)
    blocks, n_kept = select_blocks(keys, lens, kb)
    phys, valid = expand(blocks, n_kept, lens, req, wl.page_table)
    pos = candidate_positions(blocks, valid)
    k_src = kc if k_source is None else k_source
    src_top = topk_positions(S, lens, k_src, pos_offset=off)
    cons = wl.layers[1:] if n_consumers is None else wl.layers[1:1 + n_consumers]
    T, sel = [], []
    for layer in cons:
        t = scores_at(layer.qv, layer.qs, layer.w, wl.req, pos, wl.pool, wl.page_table,
                      row_ids=rows)
        T.append(t)
        sel.append(topk_positions(t, valid, kc, colmap=pos, pos_offset=off))
    return dict(rows=rows, S=S, keys=keys, blocks=blocks, n_kept=n_kept, phys=phys,
                valid_len=valid, positions=pos, source_topk=src_top, T=T, consumer_topk=sel)
