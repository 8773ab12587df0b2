"""One prefill/decode chunk through the library: a source layer plus consumers.

Stream choreography of the publish/select handoff (sglang PR "dsv4.1:
candidate indexer library", Summary and review; vLLM decode page,
CandidateOverlap fork/join; prefill PR, "Level one"), in the
source_scores="rescore" form (the default for score matrices of 4 GiB and
more, as in the long chunk):

  main stream   idx_fold_queries (the source query), idx_score_dense_keys with
                no score matrix: the source's block keys only -> event
                "scores ready"
  side stream   waits "scores ready"; idx_topk_blocks_nested (the kb best
                blocks and, nested in them, the k + 1 best),
                idx_expand_candidates of the kb-block table (records
                table.ready), then the source's own top-k: expansion of the
                (k + 1)-block table, the source query's scores at those
                blocks (idx_score_sparse_paged) and their block-mapped top-k
                (idx_topk_rows), recording "source done"
  main stream   idx_fold_queries (all consumer queries, one launch, beside the
                block select), then per consumer idx_score_sparse_paged
                (waits table.ready inside the call) and idx_topk_rows;
                finally waits "source done".  The source's rescoring runs
                beside the first consumer.

The source's dense top-k lies inside its k + 1 best blocks: a block holding
one of the k best positions has at most k - 1 blocks above it (ties go to the
lower id at both levels; the newest block, +inf, is always among them), so
the top-k over the scores at those blocks equals the dense top-k.  Rescoring
4104 columns per row costs less than writing and re-reading the 16.6 GB
score matrix of the long chunk.

source_scores="dense" keeps the score matrix S (idx_score_dense_keys with S):
the side stream then runs idx_topk_blocks and the expansion, and the source's
own top-k gathers S at its candidate columns (mode GATHER, when kb >= k + 1)
or selects over the dense row (mode IDENTITY).

Every table buffer is allocated on the main stream before the fork and
record_stream'ed to the side stream that writes it, so the caching allocator
never recycles a buffer that either stream still uses; the consumers' wait on
table.ready orders every main-stream read after the side stream's writes.

With few rows (decode: fewer rows than CUs) run() also moves the consumers'
selects to a third stream: each consumer's top-k runs there behind an event
recorded after the scores it reads, while the main stream goes on to the next
consumer's sparse scores (two score buffers, the main stream waiting for the
select that last read a buffer before rewriting it); the main stream waits
for the select stream at the end.  On 64 decode rows this cut the step from
0.326 to 0.298 ms; on 2048 and 16384 rows the sparse scores fill the GPU and
moving the consumers' selects gains nothing (16384 rows: 27.90-28.05 ms
against 27.66-27.90 ms), so there they stay on the main stream.

Tail layers (prefill PR, "Tail rows"): the last `tail_layers` consumers
score only the last tail_len[j] rows of each request j.  The side stream
builds their table with idx_prefill_tail right after the expansion (it records
the tail table's own ready event), and those consumers wait on it.

If any call raises inside a block that was forked onto the side or select
stream, the main stream waits for that stream before the exception leaves
(vLLM decode page, CandidateOverlap fork/join), so that a graph capture ends
with every stream joined and reports the real error.  No call synchronises
the host, so run() can be captured into one HIP graph (capture()).
"""

from __future__ import annotations

import contextlib
import copy

import numpy as np
import torch

from . import (COLS_BLOCKMAP, COLS_GATHER, COLS_IDENTITY, KPool, Query, Rows, Table,
               idx_amax8_varlen, idx_expand_candidates, idx_fold_queries, idx_prefill_tail,
               idx_score_dense,
               idx_score_dense_keys, idx_score_sparse_paged, idx_score_sparse_paged_bf16,
               idx_topk_blocks, idx_topk_blocks_nested, idx_topk_rows, idx_topk_rows_bf16,
               score_workspace, stream_wait_table, tail_workspace)


def _dev(a, dtype, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype).contiguous()


@contextlib.contextmanager
def _forked(stream, main):
    """Run a block on `stream`; if it raises, make `main` wait for `stream`
    before the exception propagates (the fork is always joined)."""
    try:
        with torch.cuda.stream(stream):
            yield
    except BaseException:
        main.wait_stream(stream)
        raise


def tail_row_ids(rows_per_req, tail_len):
    """Row ids of the last tail_len[j] rows of every request j, in row order."""
    out, start = [], 0
    for n, t in zip(rows_per_req, tail_len):
        out.extend(range(start + int(n) - int(t), start + int(n)))
        start += int(n)
    return np.asarray(out, dtype=np.int64)


class Chunk:
    """Device copies of a workload (see the workloads package) and its buffers."""

    # run() overlaps the selects with the next sparse scores up to this many rows
    OVERLAP_MAX_ROWS = 256
    # the source's top-k by rescoring its top-(k+1) blocks pays off when the
    # score matrix it avoids is large: long chunk (17.2 GB of S) -1.0 to -1.6 ms
    # per chunk; prefill (0.5 GB) +0.09 ms and decode (16 MB) +0.02 ms per step,
    # where writing S costs next to nothing and the nested block select and
    # the rescoring do not
    RESCORE_MIN_S_BYTES = 4 << 30

    def __init__(self, wl, device="cuda", n_consumers=None, k_source=None, with_offset=True,
                 share_T=True, fused_keys=True, consumer_bf16=False, overlap_selects=None,
                 source_side=True, tail_layers=0, source_scores="auto", prefold=True):
        self.wl = wl
        self.fused_keys = fused_keys
        self.consumer_bf16 = consumer_bf16   # consumers write and select bf16 scores
        self.device = device
        self.R, self.kb, self.kc = wl.rows, wl.kb, wl.kc
        self.k_src = wl.kc if k_source is None else k_source
        # key rows padded to 4 keys, so that the block select reads them with
        # 16-byte loads whatever the longest row
        self.ld, self.ldk = wl.ld, (wl.ldk + 3) // 4 * 4
        self.kp = KPool(_dev(wl.pool, torch.uint8, device), _dev(wl.page_table, torch.int32, device))
        off = _dev(wl.req_start, torch.int32, device) if with_offset else None
        self.rows = Rows(_dev(wl.req, torch.int32, device), _dev(wl.lens, torch.int32, device), off)
        layers = wl.layers if n_consumers is None else wl.layers[:1 + n_consumers]
        self.queries = [Query(_dev(L.qv, torch.uint8, device), _dev(L.qs, torch.uint8, device),
                              _dev(L.w, torch.float32, device)) for L in layers]
        # source top-k: "rescore" its top-(k+1) blocks (keys-only dense pass, no
        # score matrix), or take it from the "dense" score matrix S; "auto":
        # rescore when S would take at least RESCORE_MIN_S_BYTES
        if source_scores not in ("auto", "rescore", "dense"):
            raise ValueError("source_scores must be 'auto', 'rescore' or 'dense'")
        if source_scores == "auto":
            big = self.R * self.ld * 4 >= self.RESCORE_MIN_S_BYTES
            source_scores = "rescore" if big else "dense"
        self.k2 = self.k_src + 1
        self.rescore = source_scores == "rescore" and fused_keys and self.k2 <= self.kb
        self.S = None if self.rescore else \
            torch.empty((self.R, self.ld), dtype=torch.float32, device=device)
        self.keys = torch.empty((self.R, self.ldk), dtype=torch.float32, device=device)
        self.table = Table(self.R, self.kb, device)
        if self.rescore:
            self.table2 = Table(self.R, self.k2, device)   # the source's top-(k+1) blocks
            self.T_src = torch.empty((self.R, self.k2 * 8), dtype=torch.float32, device=device)
            self.ws_src = score_workspace(self.R, device)  # the source fold, on the side stream
        ncons = len(self.queries) - 1
        self.overlap = (self.R <= self.OVERLAP_MAX_ROWS) if overlap_selects is None else overlap_selects
        nT = max(1, ncons) if not share_T else (min(2, max(1, ncons)) if self.overlap else 1)
        tdt = torch.bfloat16 if consumer_bf16 else torch.float32
        self.T = [torch.empty((self.R, self.kb * 8), dtype=tdt, device=device) for _ in range(nT)]
        self.src_top = torch.empty((self.R, self.k_src), dtype=torch.int32, device=device)
        # the last tail_layers consumers see only each request's tail rows
        if tail_layers and wl.tail_len is None:
            raise ValueError("tail_layers needs a workload with tail lengths")
        self.n_tail_layers = min(int(tail_layers), ncons)
        self.tail = None
        if self.n_tail_layers:
            trows = tail_row_ids(wl.rows_per_req, wl.tail_len)
            self.tail_rows = trows
            self.tail_rpr = _dev(wl.rows_per_req, torch.int32, device)
            self.tail_len = _dev(wl.tail_len, torch.int32, device)
            self.tail = Table(len(trows), self.kb, device)
            self.tail_ws = tail_workspace(len(wl.rows_per_req), device)
            self.tail_off = _dev(wl.req_start[trows], torch.int32, device) if with_offset else None
            for i in range(ncons - self.n_tail_layers, ncons):   # those layers' tail-row queries
                L = layers[1 + i]
                self.queries[1 + i] = Query(_dev(L.qv[trows], torch.uint8, device),
                                            _dev(L.qs[trows], torch.uint8, device),
                                            _dev(L.w[trows], torch.float32, device))
            self.T_tail = torch.empty((len(trows), self.kb * 8), dtype=tdt, device=device)
        self.cons_top = [torch.empty((self.R if not self._is_tail(i) else len(self.tail_rows), self.kc),
                                     dtype=torch.int32, device=device) for i in range(ncons)]
        self.ws = score_workspace(self.R, device)      # folded queries of the layer being scored
        # prefold: the layers' folded queries made by idx_fold_queries (the
        # source's first, the consumers' in one launch beside the block
        # select), which the score calls then read
        # (self.queries stay as given; the score calls use self.fq, copies that
        # carry the folded workspaces)
        self.prefold = prefold
        self.fold_ws = []
        self.fq = list(self.queries)
        if prefold:
            self.fold_ws = [score_workspace(q.rows, device) for q in self.queries]
            self.fq = []
            for q, w in zip(self.queries, self.fold_ws):
                f = copy.copy(q)
                f.folded = w
                self.fq.append(f)
        self.side = torch.cuda.Stream(device=device)
        self.scores_ready = torch.cuda.Event()
        self.sel = torch.cuda.Stream(device=device) if self.overlap else None
        self.source_side = source_side   # big tables: source top-k on the side stream
        self.source_done = torch.cuda.Event()
        self.sparse_done = [torch.cuda.Event() for _ in range(ncons)]
        self.select_done = [torch.cuda.Event() for _ in range(ncons)]
        self.recorder = None     # optional: object with mark(name) (timing only)
        self.graph = None        # run() captured by capture()

    def _is_tail(self, i: int) -> bool:
        return i >= len(self.queries) - 1 - self.n_tail_layers

    def _mark(self, name: str):
        if self.recorder is not None:
            self.recorder.mark(name)

    # -- the source layer ---------------------------------------------------
    def fold(self, layers, stream=None):
        """The folded queries of some layers in one launch (prefold): the source's
        before its dense pass; the consumers' right after the fork of the
        publish, so that it runs beside the block select on the side stream."""
        if self.prefold and layers:
            idx_fold_queries([self.queries[i] for i in layers], [self.fold_ws[i] for i in layers],
                             stream=stream)

    def score_source(self, stream=None):
        self._mark("dense<")
        if self.rescore:   # keys only; rows with more than k + 1 blocks are keyed
            idx_score_dense_keys(self.fq[0], self.kp, self.rows, None, self.keys,
                                 skip_le_blocks=self.k2, ws=self.ws, stream=stream, ld=self.ld)
        elif self.fused_keys:
            idx_score_dense_keys(self.fq[0], self.kp, self.rows, self.S, self.keys,
                                 skip_le_blocks=self.kb, ws=self.ws, stream=stream)
        else:
            idx_score_dense(self.fq[0], self.kp, self.rows, self.S, ws=self.ws, stream=stream)
        self._mark("dense>")

    def publish(self):
        """Block keys, block selection and expansion on the side stream."""
        main = torch.cuda.current_stream()
        self.scores_ready.record(main)
        self.side.wait_event(self.scores_ready)
        if not torch.cuda.is_current_stream_capturing():   # (a graph keeps its buffers alive)
            for t in (self.keys, *self.table.tensors(), self.rows.req, self.rows.len, self.src_top,
                      *((self.S,) if self.S is not None else ()),
                      *((self.rows.pos_offset,) if self.rows.pos_offset is not None else ())):
                t.record_stream(self.side)
            if self.rescore:
                for t in (*self.table2.tensors(), self.T_src, self.ws_src):
                    t.record_stream(self.side)
            if self.tail is not None:
                for t in (*self.tail.tensors(), self.tail_rpr, self.tail_len, self.tail_ws):
                    t.record_stream(self.side)
        with _forked(self.side, main):
            if not self.fused_keys:
                self._mark("amax8<")
                idx_amax8_varlen(self.S, self.rows.len, self.keys, skip_le_blocks=self.kb)
                self._mark("amax8>")
            self._mark("topk_blocks<")
            if self.rescore:
                idx_topk_blocks_nested(self.keys, self.rows.len, self.kb, self.table.blocks,
                                       self.table.n_kept, self.k2, self.table2.blocks, self.table2.n_kept)
            else:
                idx_topk_blocks(self.keys, self.rows.len, self.kb, self.table.blocks, self.table.n_kept)
            self._mark("topk_blocks>")
            idx_expand_candidates(self.kp, self.rows, self.table)   # records table.ready
            self._mark("expand>")
            if self.tail is not None:   # records tail.ready; same stream as the table
                idx_prefill_tail(self.table, self.tail_rpr, self.tail_len, self.tail, ws=self.tail_ws,
                                 wait_full=False)
                self._mark("tail>")
            if self.rescore:
                # the source's own top-k: its scores at its top-(k+1) blocks (the
                # consumers start on table.ready meanwhile)
                idx_expand_candidates(self.kp, self.rows, self.table2)
                self._mark("source_topk<")
                idx_score_sparse_paged(self.fq[0], self.kp, self.table2, self.T_src, ws=self.ws_src,
                                       wait_ready=False)
                idx_topk_rows(self.T_src, self.table2.valid_len, self.k_src, self.src_top,
                              mode=COLS_BLOCKMAP, blocks=self.table2.blocks,
                              pos_offset=self.rows.pos_offset)
                self._mark("source_topk>")
                self.source_done.record(self.side)

    def source_topk(self, same_stream_as_table=False):
        """The source's own top-k from S (waits for the table when it reads it,
        unless it runs on the stream that built the table: a stream never waits
        on an event it recorded itself, which a graph capture cannot express).
        With rescoring it was taken in publish(), on the side stream."""
        if self.rescore:
            return
        if self.kb >= self.k_src + 1:
            if not same_stream_as_table:
                stream_wait_table(self.table)
            self._mark("source_topk<")
            idx_topk_rows(self.S, self.table.valid_len, self.k_src, self.src_top, mode=COLS_GATHER,
                          blocks=self.table.blocks, pos_offset=self.rows.pos_offset)
        else:
            self._mark("source_topk<")
            idx_topk_rows(self.S, self.rows.len, self.k_src, self.src_top, mode=COLS_IDENTITY,
                          pos_offset=self.rows.pos_offset)
        self._mark("source_topk>")

    # -- a consumer layer ---------------------------------------------------
    def _layer_table(self, i: int):
        """(table, row offsets, score buffer or None) of consumer i."""
        if self._is_tail(i):
            return self.tail, self.tail_off, self.T_tail
        return self.table, self.rows.pos_offset, None

    def _score(self, i: int, T):
        score = idx_score_sparse_paged_bf16 if self.consumer_bf16 else idx_score_sparse_paged
        tbl, _, T_own = self._layer_table(i)
        self._mark(f"sparse{i}<")
        score(self.fq[1 + i], self.kp, tbl, T if T_own is None else T_own, ws=self.ws)
        self._mark(f"sparse{i}>")

    def _select(self, i: int, T):
        select = idx_topk_rows_bf16 if self.consumer_bf16 else idx_topk_rows
        tbl, off, T_own = self._layer_table(i)
        self._mark(f"topk_rows{i}<")
        select(T if T_own is None else T_own, tbl.valid_len, self.kc, self.cons_top[i],
               mode=COLS_BLOCKMAP, blocks=tbl.blocks, pos_offset=off)
        self._mark(f"topk_rows{i}>")

    def consumer(self, i: int):
        T = self.T[i % len(self.T)]
        self._score(i, T)
        self._select(i, T)

    def run(self):
        """source + publish + source top-k + every consumer, on the current stream
        (the selects on their own stream when overlap is on; the current stream
        waits for them before returning)."""
        main = torch.cuda.current_stream()
        self._mark("fold<")
        self.fold([0])
        self._mark("fold>")
        self.score_source()
        self.publish()
        try:
            self.fold(list(range(1, len(self.queries))))
            self._run_layers(main)
        finally:
            # every fork is joined, also when a call raised
            main.wait_stream(self.side)
            if self.sel is not None:
                main.wait_stream(self.sel)

    def _run_layers(self, main):
        if self.rescore:   # the source's top-k runs inside publish(), on the side stream
            self._run_consumers(main)
            main.wait_event(self.source_done)
            return
        if not self.overlap:
            if self.source_side:
                # the source's own top-k (HBM-bound: it gathers S at the
                # candidates) behind the expansion on the side stream, beside
                # the first consumer's scores (MFMA/VALU-bound)
                with _forked(self.side, main):
                    self.source_topk(same_stream_as_table=True)
                    self.source_done.record(self.side)
                for i in range(len(self.cons_top)):
                    self.consumer(i)
                main.wait_event(self.source_done)
                return
            self.source_topk()
            for i in range(len(self.cons_top)):
                self.consumer(i)
            return
        with _forked(self.sel, main):
            self.sel.wait_event(self.scores_ready)
            self.source_topk()
        self._run_consumers(main)

    def _run_consumers(self, main):
        if not self.overlap:
            for i in range(len(self.cons_top)):
                self.consumer(i)
            return
        nT = len(self.T)
        for i in range(len(self.cons_top)):
            T = self.T[i % nT]
            if i >= nT:
                main.wait_event(self.select_done[i - nT])   # the select that last read T
            self._score(i, T)
            self.sparse_done[i].record(main)
            with _forked(self.sel, main):
                self.sel.wait_event(self.sparse_done[i])
                self._select(i, T)
                self.select_done[i].record(self.sel)

    # -- run() as one HIP graph ------------------------------------------------
    def capture(self):
        """Capture run() into a HIP graph: replay() then issues the whole step
        with one launch.  Few-row steps (decode) are otherwise bound by the
        host's cost per call (64 decode rows: 0.34 ms of issue per step).  A
        replay recomputes the step from whatever this object's inputs and
        buffers hold."""
        if self.recorder is not None:
            raise RuntimeError("capture() with a recorder attached")
        warm = torch.cuda.Stream(device=self.device)
        warm.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(warm):
            self.run()
        torch.cuda.current_stream().wait_stream(warm)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        torch.cuda.synchronize()
        self.graph = g

    def replay(self):
        self.graph.replay()
