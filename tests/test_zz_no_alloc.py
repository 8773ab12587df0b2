"""idx_score_sparse_paged_noalloc (the folded queries in the library's static
scratch) against idx_score_sparse_paged (a workspace argument) through the C
ABI: two calls in a row, the second on fewer rows, each bit for bit equal to
the workspace call and within tolerance of the oracle on sampled rows."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-4, 1e-5


def _scores(t, ch, noalloc):
    T = torch.full((ch.R, ch.kb * 8), float("nan"), dtype=torch.float32, device="cuda")
    if noalloc:
        t.idx_score_sparse_paged_noalloc(ch.queries[1], ch.kp, ch.table, T)
    else:
        t.idx_score_sparse_paged(ch.queries[1], ch.kp, ch.table, T, ws=ch.ws)
    torch.cuda.synchronize()
    return T.cpu().numpy()


def test_noalloc_matches_workspace_call():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import two_level_top_amd as t
    from two_level_top_amd.chunk import Chunk
    full = workloads.decode(n_consumers=1)
    cases = [("decode 64 rows", full),
             ("decode 24 rows", workloads.select_rows(full, np.arange(5, 29)))]
    for name, wl in cases:
        print(f"[case] noalloc sparse scores, {name}", flush=True)
        ch = Chunk(wl, n_consumers=1)
        ch.run()
        torch.cuda.synchronize()
        got = _scores(t, ch, noalloc=True)
        ref = _scores(t, ch, noalloc=False)
        valid = ch.table.valid_len.cpu().numpy()
        inside = np.arange(ch.kb * 8)[None, :] < valid[:, None]
        assert np.array_equal(got[inside].view(np.uint32), ref[inside].view(np.uint32)), name
        assert np.isnan(got[~inside]).all(), f"{name}: written past valid_len"
        rows = np.arange(0, wl.rows, 5)
        blocks = ch.table.blocks.cpu().numpy()
        pos = oracle.candidate_positions(blocks, valid)[rows]
        L = wl.layers[1]
        want = oracle.scores_at(L.qv, L.qs, L.w, wl.req, pos, wl.pool, wl.page_table, row_ids=rows)
        m = pos >= 0
        err = np.abs(got[rows][m].astype(np.float64) - want[m])
        assert (err <= ATOL + RTOL * np.abs(want[m])).all(), f"{name}: worst {err.max():.3g}"
