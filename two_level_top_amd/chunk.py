"""One prefill/decode chunk through the library: a source layer plus consumers.

Stream choreography of the publish/select handoff (sglang PR "dsv4.1:
candidate indexer library", Summary and review; vLLM decode page,
CandidateOverlap fork/join; prefill PR, "Level one"):

  main stream   idx_score_dense_keys (source scores and their block keys in
                one pass; or idx_score_dense) -> event "scores ready"
  side stream   waits "scores ready"; (idx_amax8_varlen when the keys were
                not fused,) idx_topk_blocks, idx_expand_candidates, which
                records table.ready
  main stream   source's own top-k (waits table.ready when it reads the
                table), then per consumer idx_score_sparse_paged (waits
                table.ready inside the call) and idx_topk_rows.

Every table buffer is allocated on the main stream before the fork and
record_stream'ed to the side stream that writes it, so the caching allocator
never recycles a buffer that either stream still uses; the consumers' wait on
table.ready orders every main-stream read after the side stream's writes.

The source's own top-k is taken over its candidate columns (mode GATHER)
when kb >= k + 1: every block holding one of the k best positions then has at
most k - 1 blocks above it, so the result equals the dense top-k; otherwise
the dense row is selected directly (mode IDENTITY).
"""

from __future__ import annotations

import torch

from . import (COLS_BLOCKMAP, COLS_GATHER, COLS_IDENTITY, KPool, Query, Rows, Table,
               idx_amax8_varlen, idx_expand_candidates, idx_score_dense, idx_score_dense_keys,
               idx_score_sparse_paged, idx_score_sparse_paged_bf16, idx_topk_blocks, idx_topk_rows,
               idx_topk_rows_bf16, score_workspace, stream_wait_table)


def _dev(a, dtype, device):
    return torch.from_numpy(a).to(device=device, dtype=dtype).contiguous()


class Chunk:
    """Device copies of a workload (see the workloads package) and its buffers."""

    def __init__(self, wl, device="cuda", n_consumers=None, k_source=None, with_offset=True,
                 share_T=True, fused_keys=True, consumer_bf16=False):
        self.wl = wl
        self.fused_keys = fused_keys
        self.consumer_bf16 = consumer_bf16   # consumers write and select bf16 scores
        self.device = device
        self.R, self.kb, self.kc = wl.rows, wl.kb, wl.kc
        self.k_src = wl.kc if k_source is None else k_source
        self.ld, self.ldk = wl.ld, wl.ldk
        self.kp = KPool(_dev(wl.pool, torch.uint8, device), _dev(wl.page_table, torch.int32, device))
        off = _dev(wl.req_start, torch.int32, device) if with_offset else None
        self.rows = Rows(_dev(wl.req, torch.int32, device), _dev(wl.lens, torch.int32, device), off)
        layers = wl.layers if n_consumers is None else wl.layers[:1 + n_consumers]
        self.queries = [Query(_dev(L.qv, torch.uint8, device), _dev(L.qs, torch.uint8, device),
                              _dev(L.w, torch.float32, device)) for L in layers]
        self.S = torch.empty((self.R, self.ld), dtype=torch.float32, device=device)
        self.keys = torch.empty((self.R, self.ldk), dtype=torch.float32, device=device)
        self.table = Table(self.R, self.kb, device)
        ncons = len(self.queries) - 1
        nT = 1 if share_T else max(1, ncons)
        tdt = torch.bfloat16 if consumer_bf16 else torch.float32
        self.T = [torch.empty((self.R, self.kb * 8), dtype=tdt, device=device) for _ in range(nT)]
        self.src_top = torch.empty((self.R, self.k_src), dtype=torch.int32, device=device)
        self.cons_top = [torch.empty((self.R, self.kc), dtype=torch.int32, device=device)
                         for _ in range(ncons)]
        self.ws = score_workspace(self.R, device)      # folded queries of the layer being scored
        self.side = torch.cuda.Stream(device=device)
        self.scores_ready = torch.cuda.Event()
        self.recorder = None     # optional: object with mark(name) (timing only)

    def _mark(self, name: str):
        if self.recorder is not None:
            self.recorder.mark(name)

    # -- the source layer ---------------------------------------------------
    def score_source(self, stream=None):
        self._mark("dense<")
        if self.fused_keys:
            idx_score_dense_keys(self.queries[0], self.kp, self.rows, self.S, self.keys,
                                 skip_le_blocks=self.kb, ws=self.ws, stream=stream)
        else:
            idx_score_dense(self.queries[0], self.kp, self.rows, self.S, ws=self.ws, stream=stream)
        self._mark("dense>")

    def publish(self):
        """Block keys, block selection and expansion on the side stream."""
        main = torch.cuda.current_stream()
        self.scores_ready.record(main)
        self.side.wait_event(self.scores_ready)
        for t in (self.S, self.keys, *self.table.tensors(), self.rows.req, self.rows.len):
            t.record_stream(self.side)
        with torch.cuda.stream(self.side):
            if not self.fused_keys:
                self._mark("amax8<")
                idx_amax8_varlen(self.S, self.rows.len, self.keys, skip_le_blocks=self.kb)
                self._mark("amax8>")
            self._mark("topk_blocks<")
            idx_topk_blocks(self.keys, self.rows.len, self.kb, self.table.blocks, self.table.n_kept)
            self._mark("topk_blocks>")
            idx_expand_candidates(self.kp, self.rows, self.table)   # records table.ready
            self._mark("expand>")

    def source_topk(self):
        """The source's own top-k (waits for the table when it reads it)."""
        if self.kb >= self.k_src + 1:
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
    def consumer(self, i: int):
        T = self.T[i % len(self.T)]
        score = idx_score_sparse_paged_bf16 if self.consumer_bf16 else idx_score_sparse_paged
        select = idx_topk_rows_bf16 if self.consumer_bf16 else idx_topk_rows
        self._mark(f"sparse{i}<")
        score(self.queries[1 + i], self.kp, self.table, T, ws=self.ws)
        self._mark(f"sparse{i}>")
        select(T, self.table.valid_len, self.kc, self.cons_top[i], mode=COLS_BLOCKMAP,
               blocks=self.table.blocks, pos_offset=self.rows.pos_offset)
        self._mark(f"topk_rows{i}>")

    def run(self):
        """source + publish + source top-k + every consumer, on the current stream."""
        self.score_source()
        self.publish()
        self.source_topk()
        for i in range(len(self.cons_top)):
            self.consumer(i)
