"""GPU parity of the HIP path against the CPU oracle, call by call and end to end.

Selection steps (block keys, block selection, expansion, top-k) do no float
arithmetic beyond comparisons: they are checked bit for bit on inputs the
oracle also sees.  Score steps are checked within |gpu - oracle| <=
1e-4 + 1e-5 * |oracle|.  Where a selection consumes GPU scores, sets may
differ only at ties within that tolerance of the k-th value.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-4, 1e-5
INT32_MAX = np.iinfo(np.int32).max


def say(msg: str):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def idx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import two_level_top_amd as t
    t.load()
    return t


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.to(dtype)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(gpu, ora, mask, what):
    g, o = gpu[mask].astype(np.float64), ora[mask].astype(np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU values"
    err = np.abs(g - o)
    bound = ATOL + RTOL * np.abs(o)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside tolerance, worst {err.max():.3g}"


def within_tol(a, b):
    return abs(float(a) - float(b)) <= ATOL + RTOL * abs(float(b))


def assert_same_selection(gpu_row, ora_row, score_of, kth, pad, what):
    """Equal sets, or differences only at ties within tolerance of the k-th value."""
    g = set(int(x) for x in gpu_row if x != pad)
    o = set(int(x) for x in ora_row if x != pad)
    assert len(g) == len(o), f"{what}: {len(g)} vs {len(o)} picks"
    for x in g ^ o:
        s = score_of(x)
        assert s is not None and within_tol(s, kth), f"{what}: pick {x} score {s} vs k-th {kth}"
    assert list(gpu_row) == sorted(gpu_row, key=lambda v: (v == pad, v)), f"{what}: not ascending"


def kth_largest(vals, k):
    v = np.sort(vals.astype(np.float64))[::-1]
    return v[min(k, len(v)) - 1]


# ---------------------------------------------------------------------------
# idx_score_dense
# ---------------------------------------------------------------------------

def _dense_gpu(idx, wl, layer_i, ld=None):
    from two_level_top_amd.chunk import Chunk
    ch = Chunk(wl, n_consumers=0)
    L = wl.layers[layer_i]
    q = idx.Query(dev(L.qv), dev(L.qs), dev(L.w))
    S = torch.full((wl.rows, ld or wl.ld), float("nan"), dtype=torch.float32, device="cuda")
    idx.idx_score_dense(q, ch.kp, ch.rows, S)
    return host(S)


def _check_dense(idx, wl, layer_i, rows=None):
    S = _dense_gpu(idx, wl, layer_i)
    L = wl.layers[layer_i]
    rows = np.arange(wl.rows) if rows is None else np.asarray(rows)
    ref = oracle.dense_scores(L.qv, L.qs, L.w, wl.req, wl.lens, wl.pool, wl.page_table,
                              row_ids=rows, ld=wl.ld)
    valid = np.arange(wl.ld)[None, :] < wl.lens[rows][:, None]
    assert_close(S[rows], ref, valid, f"{wl.name} layer {layer_i} dense")
    # nothing written past each row's length
    assert np.isnan(S[rows][~valid]).all(), "dense scores written past len"


def test_dense_tiny(idx):
    wl = workloads.tiny()
    for i in range(3):
        say(f"dense tiny layer {i}")
        _check_dense(idx, wl, i)


@pytest.mark.parametrize("heads", [64, 8, 24])
def test_dense_ragged_requests(idx, heads):
    # ragged lengths, an empty row, pairs of rows from different requests,
    # contexts that are not multiples of a tile or page
    wl = workloads.custom("ragged", 31 + heads, heads, 4, 8, [1000, 77, 5, 300, 2100],
                          [5, 1, 2, 3, 4],
                          [[990, 996, 997, 998, 1000], [77], [0, 5], [1, 250, 300], [1, 64, 1500, 2100]],
                          n_layers=1)
    say(f"dense ragged heads={heads}")
    _check_dense(idx, wl, 0)


def test_dense_prefill_sampled(idx):
    wl = workloads.prefill(n_consumers=0)
    say("dense prefill 2048 x 65536 (sampled rows)")
    _check_dense(idx, wl, 0, rows=[0, 1, 2, 777, 1024, 2045, 2046, 2047])


# ---------------------------------------------------------------------------
# idx_amax8_varlen (bit-exact on synthetic scores)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("width,kb", [(2048, 16), (65536, 2048), (262144, 2048)])
def test_amax8_bitexact(idx, width, kb):
    rows = 64 if width <= 65536 else 32
    S = workloads.random_matrix(width, rows, width)
    # lengths whose newest block falls at, just past or just before the
    # boundaries of the kernel's wave slices and workgroups (which divide 256
    # blocks)
    bounds = [8 * (kb + 256 * m) + d for m in (1, 2, 4, 5) for d in (-8, -7, 0, 1, 9)]
    lens = workloads.random_lengths(width, rows, 0, width,
                                    extra=[0, 1, 7, 8, 9, width, width - 1, 8 * kb, 8 * kb + 1, 8 * kb - 1]
                                    + [b for b in bounds if b <= width])
    nblk = oracle.nblocks(lens)
    ldk = width // 8
    say(f"amax8 width={width} kb={kb}")
    keys_g = torch.full((rows, ldk), -7.0, dtype=torch.float32, device="cuda")
    idx.idx_amax8_varlen(dev(S), dev(lens), keys_g, skip_le_blocks=kb)
    kg = host(keys_g)
    ko = oracle.block_keys(S, lens, kb, ldk=ldk)
    for r in range(rows):
        m = int(nblk[r])
        if m <= kb:
            assert (kg[r] == -7.0).all(), f"row {r} (nblk {m} <= kb) was written"
        else:
            # equal fp32 values (+0 and -0 are the same key)
            assert np.array_equal(kg[r, :m], ko[r, :m]), f"row {r}"
            assert (kg[r, m:] == -7.0).all(), f"row {r} written past nblk"


def _e2m1_table():
    return np.array([oracle.e2m1_value(c) for c in range(16)], dtype=np.float64)


def _dequant(codes, scales):
    """[..., 64] code bytes + [..., 4] ue8m0 bytes -> [..., 128] fp64 values."""
    tab = _e2m1_table()
    lo, hi = codes & 15, codes >> 4
    v = np.stack([tab[lo], tab[hi]], axis=-1).reshape(*codes.shape[:-1], 128)
    sc = np.exp2(scales.astype(np.float64) - 127.0)
    return v * np.repeat(sc, 32, axis=-1)


@pytest.mark.parametrize("name", ["tiny", "ragged24", "long"])
def test_fold_workspace(idx, name):
    """The score calls' workspace holds sum_h (w_h/2) q_h as 16 MXFP4 terms:
    their sum equals the fp64 fold up to the greedy split's residual (each
    term shrinks a group's largest residual at least 3-fold)."""
    from two_level_top_amd.chunk import Chunk
    if name == "long":
        wl = workloads.long_chunk(n_consumers=0)
        rows = np.array([0, 1, 2, 3, 8191, 16380, 16381, 16382, 16383])
    else:
        wl, _ = _fused_case("tiny" if name == "tiny" else "ragged64")
        if name == "ragged24":
            wl, _ = _fused_case("ragged24")
        rows = np.arange(wl.rows)
    say(f"fold workspace {name}")
    ch = Chunk(wl, n_consumers=0)
    L = wl.layers[0]
    q = idx.Query(dev(L.qv), dev(L.qs), dev(L.w))
    S = torch.empty((wl.rows, wl.ld), dtype=torch.float32, device="cuda")
    ws = idx.score_workspace(wl.rows)
    idx.idx_score_dense(q, ch.kp, ch.rows, S, ws=ws)
    fold = host(ws)[: wl.rows * 1088].reshape(wl.rows, 1088)[rows]
    terms = _dequant(fold[:, :1024].reshape(-1, 16, 64), fold[:, 1024:].reshape(-1, 16, 4))
    got = terms.sum(axis=1)
    qv = _dequant(L.qv[rows], L.qs[rows])                       # [n, H, 128]
    want = np.einsum("nh,nhd->nd", 0.5 * L.w[rows].astype(np.float64), qv)
    gmax = np.abs(want).reshape(len(rows), 4, 32).max(axis=2)   # per scale group
    bound = np.repeat(gmax, 32, axis=1) * 3.0 ** -16
    err = np.abs(got - want)
    assert (err <= bound).all(), f"fold residual {err.max():.3g} above the 16-term bound"
    # the dense scorer uses the first 8 terms (two rows share one MFMA block)
    got8 = terms[:, :8].sum(axis=1)
    err8 = np.abs(got8 - want)
    assert (err8 <= np.repeat(gmax, 32, axis=1) * 3.0 ** -8).all(), \
        f"8-term fold residual {err8.max():.3g} above its bound"


# ---------------------------------------------------------------------------
# idx_q_rope_quant: the step before the score calls (bit-exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,heads,neox", [(37, 64, True), (37, 64, False), (5, 8, True),
                                             (9, 24, False), (16384, 64, True)])
def test_q_rope_quant_bitexact(idx, rows, heads, neox):
    from oracle import q_quant
    inp = workloads.q_inputs(rows + heads, rows, heads, max_pos=262144 if rows > 1000 else 4096)
    say(f"q rope quant rows={rows} heads={heads} neox={neox}")
    q = torch.from_numpy(inp.q.view(np.int16)).cuda()
    vals = torch.full((rows, heads, 64), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows, heads, 4), 0xAB, dtype=torch.uint8, device="cuda")
    w_out = torch.full((rows, heads), float("nan"), dtype=torch.float32, device="cuda")
    softmax_scale, head_scale = 128 ** -0.5, heads ** -0.5
    idx.idx_q_rope_quant(q, dev(inp.positions), dev(inp.cos_sin), dev(inp.w), neox, softmax_scale,
                         head_scale, vals, scales, w_out)
    sample = np.arange(rows) if rows <= 64 else np.unique(np.concatenate(
        [np.arange(8), np.linspace(0, rows - 1, 120).astype(int), [rows - 1]]))
    v_o, s_o, w_o = q_quant.q_rope_quant(inp.q[sample], inp.positions[sample], inp.cos_sin,
                                         inp.w[sample], neox, softmax_scale, head_scale)
    idx_t = torch.from_numpy(sample).cuda()
    assert np.array_equal(host(vals[idx_t]), v_o), "codes differ"
    assert np.array_equal(host(scales[idx_t]), s_o), "scales differ"
    assert np.array_equal(host(w_out[idx_t]).view(np.uint32), w_o.view(np.uint32)), "weights differ"


def test_q_rope_quant_edge_values(idx):
    """Exact ties of the e2m1 grid, zeros of both signs, negative values that
    round to zero and values at the top of the grid, each group scaled by its
    own power of two, at position 0 (the rotation is then the identity, so the
    quantiser sees these values as they are)."""
    from oracle import q_quant
    rows, heads = 64, 64
    rng = np.random.default_rng(5)
    specials = np.array([0.0, -0.0, 0.25, -0.25, 0.75, -0.75, 1.25, -1.25, 1.75, -1.75, 2.5, -2.5,
                         3.5, -3.5, 5.0, -5.0, 6.0, -6.0, 4.0, -3.0, 0.1, -0.1, 0.2, -0.2], np.float32)
    x = rng.choice(specials, size=(rows, heads, 128)).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 21, size=(rows, heads, 4))).repeat(32, axis=-1).astype(np.float32)
    bits, _ = workloads.to_bf16(x)
    positions = np.zeros(rows, np.int32)
    cos_sin = workloads.rope_table(4096)
    w = rng.standard_normal((rows, heads)).astype(np.float32)
    say("q rope quant edge values")
    q = torch.from_numpy(bits.view(np.int16)).cuda()
    vals = torch.full((rows, heads, 64), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows, heads, 4), 0xAB, dtype=torch.uint8, device="cuda")
    w_out = torch.full((rows, heads), float("nan"), dtype=torch.float32, device="cuda")
    for neox in (True, False):
        idx.idx_q_rope_quant(q, dev(positions), dev(cos_sin), dev(w), neox, 1.0, 1.0, vals, scales, w_out)
        v_o, s_o, _ = q_quant.q_rope_quant(bits, positions, cos_sin, w, neox, 1.0, 1.0)
        assert np.array_equal(host(vals), v_o), "codes differ"
        assert np.array_equal(host(scales), s_o), "scales differ"


# ---------------------------------------------------------------------------
# idx_score_dense_keys: the fused source pass
# ---------------------------------------------------------------------------

def _fused_case(name):
    if name == "tiny":
        return workloads.tiny(), None
    if name.startswith("ragged"):
        heads = int(name[6:])
        if heads == 24:
            return workloads.custom("ragged", 55, 24, 8, 8, [1000, 77, 5], [2, 1, 2],
                                    [[990, 1000], [77], [0, 5]], n_layers=1), None
        # keyed and keep-all rows (kb = 8 blocks), an empty row, partial newest blocks
        return workloads.custom("ragged", 31 + heads, heads, 8, 8, [1000, 77, 5, 300, 2100],
                                [5, 1, 2, 3, 4],
                                [[990, 996, 997, 998, 1000], [77], [0, 5], [1, 250, 300],
                                 [1, 64, 1500, 2100]], n_layers=1), None
    if name == "decode":
        return workloads.decode(n_consumers=0), None
    if name == "prefill":
        return workloads.prefill(n_consumers=0), [0, 1, 2, 777, 1024, 2045, 2046, 2047]
    return workloads.long_chunk(n_consumers=0), [0, 1, 8191, 16383]


@pytest.mark.parametrize("name", ["tiny", "ragged64", "ragged8", "decode", "prefill", "long"])
@pytest.mark.parametrize("skip", ["kb", 0])
def test_dense_keys_fused(idx, name, skip):
    """Keys of the fused pass equal idx_amax8_varlen on the same S (every row,
    bit for bit as numbers), S equals idx_score_dense's bit for bit, and S is
    within tolerance of the oracle on sampled rows."""
    from two_level_top_amd.chunk import Chunk
    if name == "long" and skip == 0:
        pytest.skip("the long chunk runs once, with skip = kb as benchmarked")
    wl, sample = _fused_case(name)
    sk = wl.kb if skip == "kb" else 0
    say(f"dense keys fused {name} skip={sk}")
    ch = Chunk(wl, n_consumers=0)
    L = wl.layers[0]
    q = idx.Query(dev(L.qv), dev(L.qs), dev(L.w))
    S = torch.full((wl.rows, wl.ld), float("nan"), dtype=torch.float32, device="cuda")
    keys = torch.full((wl.rows, wl.ldk), -7.0, dtype=torch.float32, device="cuda")
    idx.idx_score_dense_keys(q, ch.kp, ch.rows, S, keys, skip_le_blocks=sk)
    ref_keys = torch.full_like(keys, -7.0)
    idx.idx_amax8_varlen(S, ch.rows.len, ref_keys, skip_le_blocks=sk)
    torch.cuda.synchronize()
    assert bool((keys == ref_keys).all()), "fused keys differ from idx_amax8_varlen on the same S"
    S2 = torch.full_like(S, float("nan"))
    idx.idx_score_dense(q, ch.kp, ch.rows, S2)
    same = (S == S2) | (torch.isnan(S) & torch.isnan(S2))
    assert bool(same.all()), "fused scores differ from idx_score_dense"
    del S2
    rows = np.arange(wl.rows) if sample is None else np.asarray(sample)
    ref = oracle.dense_scores(L.qv, L.qs, L.w, wl.req, wl.lens, wl.pool, wl.page_table,
                              row_ids=rows, ld=wl.ld)
    Sg = host(S[torch.from_numpy(rows).cuda()])
    valid = np.arange(wl.ld)[None, :] < wl.lens[rows][:, None]
    assert_close(Sg, ref, valid, f"{name} fused dense")
    ko = oracle.block_keys(ref, wl.lens[rows], sk, ldk=wl.ldk)
    kg = host(keys[torch.from_numpy(rows).cuda()])
    nblk = oracle.nblocks(wl.lens[rows])
    for i, r in enumerate(rows):
        m = int(nblk[i])
        if m <= sk:
            assert (kg[i] == -7.0).all(), f"row {r}: keys written for a keep-all row"
            continue
        assert np.isposinf(kg[i, m - 1]), f"row {r}: newest block key is not +inf"
        assert (kg[i, m:] == -7.0).all(), f"row {r}: keys written past nblk"
        g, o = kg[i, :m - 1].astype(np.float64), ko[i, :m - 1].astype(np.float64)
        bad = np.abs(g - o) > ATOL + RTOL * np.abs(o)
        assert not bad.any(), f"row {r}: {bad.sum()} block keys outside tolerance of the oracle's"


# ---------------------------------------------------------------------------
# idx_topk_blocks (bit-exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kb,maxblk", [(16, 128), (2048, 32768), (2048, 8192), (3, 40), (64, 8192)])
def test_topk_blocks_bitexact(idx, kb, maxblk):
    rows = 48
    keys = workloads.random_matrix(kb + maxblk, rows, maxblk)
    nb = workloads.random_lengths(kb + maxblk, rows, 0, maxblk,
                                  extra=[0, 1, kb - 1, kb, kb + 1, 2 * kb, maxblk, maxblk - 1])
    lens = (nb * 8 - (np.arange(rows) % 8)).clip(0).astype(np.int32)   # ragged newest blocks
    nblk = oracle.nblocks(lens)
    for r in range(rows):                # a keyed row's newest block is +inf
        if nblk[r] > 0:
            keys[r, nblk[r] - 1] = np.inf
    say(f"topk_blocks kb={kb} maxblk={maxblk}")
    blocks = torch.full((rows, kb), -5, dtype=torch.int32, device="cuda")
    n_kept = torch.full((rows,), -5, dtype=torch.int32, device="cuda")
    idx.idx_topk_blocks(dev(keys), dev(lens), kb, blocks, n_kept)
    bo, no = oracle.select_blocks(keys, lens, kb)
    assert np.array_equal(host(n_kept), no)
    assert np.array_equal(host(blocks), bo)


@pytest.mark.parametrize("kb,k2,maxblk", [(2048, 513, 32768), (2048, 513, 8192), (16, 5, 128),
                                          (64, 64, 8192), (2048, 1, 4000), (3, 2, 40), (1024, 33, 1500)])
def test_topk_blocks_nested_bitexact(idx, kb, k2, maxblk):
    """idx_topk_blocks_nested: the kb best blocks exactly as idx_topk_blocks, and
    the k2 best by the same rule, including rows that keep all kb but have more
    than k2 blocks (selected from their keys) and rows with at most k2 blocks."""
    rows = 48
    keys = workloads.random_matrix(kb + maxblk + k2, rows, maxblk)
    extra = [0, 1, k2 - 1, k2, k2 + 1, kb - 1, kb, kb + 1, 2 * kb, maxblk, maxblk - 1]
    nb = workloads.random_lengths(kb + maxblk + 1, rows, 0, maxblk,
                                  extra=[e for e in extra if 0 <= e <= maxblk])
    lens = (nb * 8 - (np.arange(rows) % 8)).clip(0).astype(np.int32)
    nblk = oracle.nblocks(lens)
    for r in range(rows):
        if nblk[r] > 0:
            keys[r, nblk[r] - 1] = np.inf
    say(f"topk_blocks_nested kb={kb} k2={k2} maxblk={maxblk}")
    blocks = torch.full((rows, kb), -5, dtype=torch.int32, device="cuda")
    n_kept = torch.full((rows,), -5, dtype=torch.int32, device="cuda")
    blocks2 = torch.full((rows, k2), -5, dtype=torch.int32, device="cuda")
    n_kept2 = torch.full((rows,), -5, dtype=torch.int32, device="cuda")
    idx.idx_topk_blocks_nested(dev(keys), dev(lens), kb, blocks, n_kept, k2, blocks2, n_kept2)
    bo, no = oracle.select_blocks(keys, lens, kb)
    b2, n2 = oracle.select_blocks(keys, lens, k2)
    assert np.array_equal(host(n_kept), no)
    assert np.array_equal(host(blocks), bo)
    assert np.array_equal(host(n_kept2), n2)
    assert np.array_equal(host(blocks2), b2)


# ---------------------------------------------------------------------------
# idx_topk_rows (bit-exact, three column modes)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("width,k", [(16384, 512), (1024, 32), (70000, 512), (300, 512), (9000, 7)])
def test_topk_rows_identity(idx, width, k):
    rows = 32
    X = workloads.random_matrix(7 * width + k, rows, width)
    extra = [v for v in (0, 1, k - 1, k, k + 1, width) if v <= width]
    valid = workloads.random_lengths(width + k, rows, 0, width, extra=extra)
    off = np.arange(rows, dtype=np.int32) * 1000
    say(f"topk_rows identity width={width} k={k}")
    out = torch.full((rows, k), -9, dtype=torch.int32, device="cuda")
    idx.idx_topk_rows(dev(X), dev(valid), k, out, mode=idx.COLS_IDENTITY, pos_offset=dev(off))
    ref = oracle.topk_positions(X, valid, k, pos_offset=off)
    assert np.array_equal(host(out), ref)


def _random_blocks(seed, rows, kb, nblk_max):
    r = np.random.default_rng(seed)
    blocks = np.full((rows, kb), INT32_MAX, np.int32)
    nk = np.zeros(rows, np.int32)
    for i in range(rows):
        n = int(r.integers(0, kb + 1)) if i % 3 else kb
        b = np.sort(r.choice(nblk_max, size=n, replace=False)).astype(np.int32)
        blocks[i, :n] = b
        nk[i] = n
    return blocks, nk


@pytest.mark.parametrize("kb,k", [(2048, 512), (16, 32), (64, 8), (1024, 100)])
def test_topk_rows_blockmap_and_gather(idx, kb, k):
    rows = 24
    nblk_max = 4 * kb + 5
    blocks, nk = _random_blocks(kb, rows, kb, nblk_max)
    valid = np.maximum(nk * 8 - (np.arange(rows) % 8), 0).astype(np.int32)
    valid[nk == 0] = 0
    T = workloads.random_matrix(kb + k, rows, kb * 8)
    dense = workloads.random_matrix(kb + k + 1, rows, nblk_max * 8)
    off = (np.arange(rows, dtype=np.int32) * 7).astype(np.int32)
    pos = oracle.candidate_positions(blocks, valid)
    say(f"topk_rows blockmap kb={kb} k={k}")
    out = torch.full((rows, k), -9, dtype=torch.int32, device="cuda")
    idx.idx_topk_rows(dev(T), dev(valid), k, out, mode=idx.COLS_BLOCKMAP, blocks=dev(blocks),
                      pos_offset=dev(off))
    ref = oracle.topk_positions(T, valid, k, colmap=pos, pos_offset=off)
    assert np.array_equal(host(out), ref)
    say(f"topk_rows gather kb={kb} k={k}")
    out2 = torch.full((rows, k), -9, dtype=torch.int32, device="cuda")
    idx.idx_topk_rows(dev(dense), dev(valid), k, out2, mode=idx.COLS_GATHER, blocks=dev(blocks))
    gathered = np.take_along_axis(dense, np.maximum(pos, 0).astype(np.int64), 1)
    ref2 = oracle.topk_positions(gathered, valid, k, colmap=pos)
    assert np.array_equal(host(out2), ref2)


@pytest.mark.parametrize("kb,k", [(2048, 512), (16, 32), (64, 8)])
def test_topk_rows_bf16_bitexact(idx, kb, k):
    """The bf16 top-k against the oracle's top-k of the same (bf16) values;
    bf16 has few distinct values, so there are many exact ties."""
    rows = 24
    nblk_max = 4 * kb + 5
    blocks, nk = _random_blocks(kb + 7, rows, kb, nblk_max)
    valid = np.maximum(nk * 8 - (np.arange(rows) % 8), 0).astype(np.int32)
    valid[nk == 0] = 0
    Tbits, Tval = workloads.to_bf16(workloads.random_matrix(kb + k + 5, rows, kb * 8))
    Dbits, Dval = workloads.to_bf16(workloads.random_matrix(kb + k + 6, rows, nblk_max * 8))
    off = (np.arange(rows, dtype=np.int32) * 3).astype(np.int32)
    pos = oracle.candidate_positions(blocks, valid)
    bf = lambda bits: torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    say(f"topk_rows bf16 blockmap kb={kb} k={k}")
    out = torch.full((rows, k), -9, dtype=torch.int32, device="cuda")
    idx.idx_topk_rows_bf16(bf(Tbits), dev(valid), k, out, mode=idx.COLS_BLOCKMAP, blocks=dev(blocks),
                           pos_offset=dev(off))
    assert np.array_equal(host(out), oracle.topk_positions(Tval, valid, k, colmap=pos, pos_offset=off))
    say(f"topk_rows bf16 gather kb={kb} k={k}")
    out2 = torch.full((rows, k), -9, dtype=torch.int32, device="cuda")
    idx.idx_topk_rows_bf16(bf(Dbits), dev(valid), k, out2, mode=idx.COLS_GATHER, blocks=dev(blocks))
    gathered = np.take_along_axis(Dval, np.maximum(pos, 0).astype(np.int64), 1)
    assert np.array_equal(host(out2), oracle.topk_positions(gathered, valid, k, colmap=pos))
    say(f"topk_rows bf16 identity width={kb * 8}")
    out3 = torch.full((rows, k), -9, dtype=torch.int32, device="cuda")
    idx.idx_topk_rows_bf16(bf(Tbits), dev(valid), k, out3)
    assert np.array_equal(host(out3), oracle.topk_positions(Tval, valid, k))


# Rows whose k-th value sits in a crowd.  The selection keeps everything at or
# above the threshold's histogram bin in an LDS list when that fits, and
# otherwise refines the bin from an LDS candidate list, or from the registers
# when that overflows too: the cluster sizes below reach each of these, with
# and without exact ties at the threshold, in one chunk and across chunks.
CROWDS = [("constant", 0), ("zeros", 0), ("cluster", 3000), ("cluster", 8000), ("neginf", 0),
          ("posinf", 0), ("posinf_many", 0), ("subnormal", 0)]


@pytest.mark.parametrize("width,k", [(16384, 512), (32768, 2048), (1024, 32), (70000, 512)])
@pytest.mark.parametrize("kind,cluster", CROWDS)
def test_topk_rows_crowded_threshold(idx, width, k, kind, cluster):
    rows = 4
    X = workloads.crowded_rows(width + k + cluster, kind, rows, width, k, cluster)
    valid = np.array([width, width - 3, k + 1, width // 2], np.int32)
    say(f"topk_rows crowded {kind}/{cluster} width={width} k={k}")
    out = torch.full((rows, k), -9, dtype=torch.int32, device="cuda")
    idx.idx_topk_rows(dev(X), dev(valid), k, out)
    assert np.array_equal(host(out), oracle.topk_positions(X, valid, k))


@pytest.mark.parametrize("kind,cluster", CROWDS)
def test_topk_mapped_and_blocks_crowded(idx, kind, cluster):
    kb, k, rows = 2048, 512, 4
    nblk_max = 4 * kb + 5
    blocks, nk = _random_blocks(kb + 11, rows, kb, nblk_max)
    valid = np.maximum(nk * 8 - (np.arange(rows) % 8), 0).astype(np.int32)
    valid[nk == 0] = 0
    pos = oracle.candidate_positions(blocks, valid)
    T = workloads.crowded_rows(kb + cluster, kind, rows, kb * 8, k, cluster)
    say(f"topk_rows crowded blockmap {kind}/{cluster}")
    out = torch.full((rows, k), -9, dtype=torch.int32, device="cuda")
    idx.idx_topk_rows(dev(T), dev(valid), k, out, mode=idx.COLS_BLOCKMAP, blocks=dev(blocks))
    assert np.array_equal(host(out), oracle.topk_positions(T, valid, k, colmap=pos))
    dense = workloads.crowded_rows(kb + cluster + 1, kind, rows, nblk_max * 8, k, cluster)
    say(f"topk_rows crowded gather {kind}/{cluster}")
    out2 = torch.full((rows, k), -9, dtype=torch.int32, device="cuda")
    idx.idx_topk_rows(dev(dense), dev(valid), k, out2, mode=idx.COLS_GATHER, blocks=dev(blocks))
    gathered = np.take_along_axis(dense, np.maximum(pos, 0).astype(np.int64), 1)
    assert np.array_equal(host(out2), oracle.topk_positions(gathered, valid, k, colmap=pos))
    maxblk = 32768
    keys = workloads.crowded_rows(kb + cluster + 2, kind, rows, maxblk, kb, cluster)
    lens = np.array([maxblk * 8, maxblk * 8 - 5, (kb + 1) * 8, maxblk * 4 - 1], np.int32)
    nblk = oracle.nblocks(lens)
    for r in range(rows):
        keys[r, nblk[r] - 1] = np.inf       # a keyed row's newest block
    say(f"topk_blocks crowded {kind}/{cluster}")
    bl = torch.full((rows, kb), -5, dtype=torch.int32, device="cuda")
    n_kept = torch.full((rows,), -5, dtype=torch.int32, device="cuda")
    idx.idx_topk_blocks(dev(keys), dev(lens), kb, bl, n_kept)
    bo, no = oracle.select_blocks(keys, lens, kb)
    assert np.array_equal(host(n_kept), no)
    assert np.array_equal(host(bl), bo)
    say(f"topk_blocks_nested crowded {kind}/{cluster}")
    k2 = 513
    bl2 = torch.full((rows, k2), -5, dtype=torch.int32, device="cuda")
    nk2 = torch.full((rows,), -5, dtype=torch.int32, device="cuda")
    bl.fill_(-5)
    n_kept.fill_(-5)
    idx.idx_topk_blocks_nested(dev(keys), dev(lens), kb, bl, n_kept, k2, bl2, nk2)
    b2, n2 = oracle.select_blocks(keys, lens, k2)
    assert np.array_equal(host(bl), bo) and np.array_equal(host(n_kept), no)
    assert np.array_equal(host(nk2), n2)
    assert np.array_equal(host(bl2), b2)


# ---------------------------------------------------------------------------
# idx_expand_candidates + idx_score_sparse_paged
# ---------------------------------------------------------------------------

def _table_from_oracle(idx, ch, blocks, n_kept):
    ch.table.blocks.copy_(dev(blocks))
    ch.table.n_kept.copy_(dev(n_kept))
    idx.idx_expand_candidates(ch.kp, ch.rows, ch.table)


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_expand_and_sparse_scores(idx, name):
    from two_level_top_amd.chunk import Chunk
    wl = workloads.tiny() if name == "tiny" else workloads.decode(n_consumers=1)
    rows = np.arange(wl.rows)
    # candidate blocks from the oracle's own source scores
    L0 = wl.layers[0]
    S = oracle.dense_scores(L0.qv, L0.qs, L0.w, wl.req, wl.lens, wl.pool, wl.page_table,
                            row_ids=rows if name == "tiny" else rows[:8], ld=wl.ld)
    sub = rows if name == "tiny" else rows[:8]
    keys = oracle.block_keys(S, wl.lens[sub], wl.kb, ldk=wl.ldk)
    b_sub, n_sub = oracle.select_blocks(keys, wl.lens[sub], wl.kb)
    # rows outside the sample get keep-all or random ascending blocks
    blocks = np.full((wl.rows, wl.kb), INT32_MAX, np.int32)
    n_kept = np.zeros(wl.rows, np.int32)
    blocks[sub], n_kept[sub] = b_sub, n_sub
    rest = np.setdiff1d(rows, sub)
    if len(rest):
        k_rest = np.full((len(rest), wl.ldk), 0.0, np.float32)
        nb_rest = oracle.nblocks(wl.lens[rest])
        k_rest[np.arange(len(rest)), np.maximum(nb_rest - 1, 0)] = np.inf   # newest block kept
        b_r, n_r = oracle.select_blocks(k_rest, wl.lens[rest], wl.kb)
        blocks[rest], n_kept[rest] = b_r, n_r
    say(f"expand {name}")
    ch = Chunk(wl, n_consumers=1)
    _table_from_oracle(idx, ch, blocks, n_kept)
    phys_o, valid_o = oracle.expand(blocks, n_kept, wl.lens, wl.req, wl.page_table)
    assert np.array_equal(host(ch.table.phys), phys_o)
    assert np.array_equal(host(ch.table.valid_len), valid_o)
    assert np.array_equal(host(ch.table.len), wl.lens)
    assert np.array_equal(host(ch.table.req), wl.req)
    sched = host(ch.table.schedule).view(np.int32)
    U = (wl.kb + 63) // 64
    assert sched[0] == wl.rows * U
    pairs = sched[4:4 + 2 * sched[0]].reshape(-1, 2)
    exp = np.array([(r, 64 * u if 64 * u < n_kept[r] else -1)
                    for r in range(wl.rows) for u in range(U)]).reshape(-1, 2)
    assert np.array_equal(pairs, exp)
    say(f"sparse scores {name}")
    L1 = wl.layers[1]
    T = torch.full((wl.rows, wl.kb * 8), float("nan"), dtype=torch.float32, device="cuda")
    idx.idx_score_sparse_paged(ch.queries[1], ch.kp, ch.table, T)
    Tg = host(T)
    pos = oracle.candidate_positions(blocks, valid_o)
    check = rows if name == "tiny" else rows[::4]
    To = oracle.scores_at(L1.qv, L1.qs, L1.w, wl.req, pos[check], wl.pool, wl.page_table, row_ids=check)
    m = pos[check] >= 0
    assert_close(Tg[check], To, m, f"{name} sparse scores")
    assert np.isnan(Tg[check][~m]).all(), "sparse scores written past valid_len"
    # the bf16 variant: the fp32 score rounded to bf16, so within half a bf16
    # step of the oracle's value plus the fp32 tolerance
    say(f"sparse scores bf16 {name}")
    Tb = torch.full((wl.rows, wl.kb * 8), float("nan"), dtype=torch.bfloat16, device="cuda")
    idx.idx_score_sparse_paged_bf16(ch.queries[1], ch.kp, ch.table, Tb)
    Tbg = host(Tb.float())[check]
    o = To[m].astype(np.float64)
    half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(o), 1e-30))) - 8)
    err = np.abs(Tbg[m].astype(np.float64) - o)
    assert (err <= half_ulp + ATOL + RTOL * np.abs(o)).all(), f"bf16 scores: worst {err.max():.3g}"
    assert np.isnan(Tbg[~m]).all(), "bf16 scores written past valid_len"


def _sparse_launch(rows, kb):
    """The consumer scorer's launch shape (score_sparse.hip): units per wave, or
    waves per unit, from the number of 64-block work units."""
    U = (kb + 63) // 64
    units = rows * U
    if units >= 2048 * 4:
        # short rows not splitting into runs of 4 go whole when that still fills the GPU
        return "upw", U if (U % 4 and U <= 12 and units >= 2048 * U) else 4
    if units >= 2048:
        return "upw", units // 2048
    split = 1
    while split < 8 and units * split < 2048:
        split *= 2
    return "split", split


# (rows, kb, context, heads): every launch shape of the consumer scorer --
# split 8 / 4 / 2, one unit per wave, 2..4 units per wave, with a row's units
# dividing evenly into runs (kb = 2048: 32 units; the runs are then ordered
# run-major: run b of every row, then run b + 1) or waves spanning two rows
# (kb = 64, 192, 320, and 3 units per wave over 32-unit rows)
SPARSE_CASES = [
    (8, 1024, 9000, 64),      # split 8
    (16, 2048, 20000, 64),    # split 4
    (40, 2048, 20000, 24),    # split 2, three 16-head blocks
    (64, 2048, 20000, 8),     # one unit per wave, one 16-head block
    (160, 2048, 20000, 64),   # runs of 2 units, run-major
    (256, 2048, 20000, 64),   # runs of 4 units, run-major
    (448, 2048, 20000, 64),   # runs of 4 units, run-major, 14 waves' rows per run
    (200, 2048, 20000, 64),   # 3 units per wave: waves span rows
    (4096, 64, 2000, 64),     # 2 units per wave of 1 unit per row: two rows per wave
    (1000, 320, 4000, 64),    # 2 units per wave over 5-unit rows
    (5462, 192, 3000, 64),    # whole 3-unit rows, one per wave
    (1700, 320, 4000, 64),    # 4 units per wave over 5-unit rows: waves span rows
    (640, 832, 8000, 64),     # 4 units per wave over 13-unit rows: waves span rows
    (8193, 256, 3000, 64),    # one run of 4 units per row, run-major; the last workgroup's spare waves
    # kb not a multiple of 4 (the source's own k + 1 blocks): the flat expansion, 4 candidates a
    # thread straddling rows
    (1000, 513, 9000, 64),    # 4 units per wave over 9-unit rows: waves span rows
    (70, 33, 1100, 8),        # split 8, one 33-block unit per row
]


@pytest.mark.parametrize("rows,kb,ctx,heads", SPARSE_CASES)
def test_sparse_scores_every_launch_shape(idx, rows, kb, ctx, heads):
    """idx_expand_candidates and idx_score_sparse_paged against the oracle at
    every launch shape of the scorer: expansion bit-exact on every row, scores
    element by element on sampled rows (the first and last rows, rows where a
    wave's units change row, random rows), nothing written past valid_len."""
    from two_level_top_amd.chunk import Chunk
    nreq = 4
    per = [rows // nreq + (1 if j < rows % nreq else 0) for j in range(nreq)]
    extra = [0, 1, 7, 8, 9, 8 * kb - 1, 8 * kb, 8 * kb + 1, ctx, ctx - 1]
    lens = workloads.random_lengths(rows + kb, rows, 0, ctx, extra=[e for e in extra if e <= ctx])
    starts = np.concatenate([[0], np.cumsum(per)])
    wl = workloads.custom(f"sparse{rows}x{kb}", 70 + rows % 97, heads, kb, 32, [ctx] * nreq, per,
                          [lens[starts[j]:starts[j + 1]] for j in range(nreq)], n_layers=2)
    mode = _sparse_launch(rows, kb)
    say(f"sparse scores rows={rows} kb={kb} heads={heads} launch={mode}")
    ldk = wl.ldk
    keys = workloads.random_matrix(rows * 3 + kb, rows, ldk)
    keys[np.isposinf(keys)] = 1e30                 # +inf only on the newest block
    nblk = oracle.nblocks(wl.lens)
    for r in range(rows):
        if nblk[r] > 0:
            keys[r, nblk[r] - 1] = np.inf       # a keyed row's newest block
    blocks, n_kept = oracle.select_blocks(keys, wl.lens, kb)
    ch = Chunk(wl, n_consumers=1)
    _table_from_oracle(idx, ch, blocks, n_kept)
    phys_o, valid_o = oracle.expand(blocks, n_kept, wl.lens, wl.req, wl.page_table)
    assert np.array_equal(host(ch.table.phys), phys_o)
    assert np.array_equal(host(ch.table.valid_len), valid_o)
    assert np.array_equal(host(ch.table.len), wl.lens)
    assert np.array_equal(host(ch.table.req), wl.req)
    U = (kb + 63) // 64
    sched = host(ch.table.schedule).view(np.int32)
    assert sched[0] == rows * U
    exp = np.stack([np.repeat(np.arange(rows), U),
                    np.where(64 * np.tile(np.arange(U), rows) < np.repeat(n_kept, U),
                             64 * np.tile(np.arange(U), rows), -1)], axis=1)
    assert np.array_equal(sched[4:4 + 2 * rows * U].reshape(-1, 2), exp), "work list"
    T = torch.full((rows, kb * 8), float("nan"), dtype=torch.float32, device="cuda")
    idx.idx_score_sparse_paged(ch.queries[1], ch.kp, ch.table, T)
    Tg = host(T)
    if mode[0] == "upw":
        # rows whose units start or end inside a wave's run of units
        edges = np.unique(np.arange(0, rows * U, mode[1]) // U)
    else:
        edges = np.arange(0, rows, max(1, rows // 16))
    rng = np.random.default_rng(rows + kb)
    pick = np.concatenate([np.arange(min(rows, 12)), np.arange(max(0, rows - 6), rows),
                           edges[:48], rng.choice(rows, size=min(rows, 48), replace=False)])
    check = np.unique(pick)
    pos = oracle.candidate_positions(blocks, valid_o)
    L1 = wl.layers[1]
    To = oracle.scores_at(L1.qv, L1.qs, L1.w, wl.req, pos[check], wl.pool, wl.page_table,
                          row_ids=check)
    m = pos[check] >= 0
    assert m.any()
    assert_close(Tg[check], To, m, f"sparse rows={rows} kb={kb}")
    assert np.isnan(Tg[check][~m]).all(), "sparse scores written past valid_len"
    assert np.isnan(Tg[~(np.arange(kb * 8)[None, :] < valid_o[:, None])]).all(), \
        "sparse scores written past valid_len"


# ---------------------------------------------------------------------------
# the whole chunk
# ---------------------------------------------------------------------------

def _run_chunk(idx, wl, n_consumers=None):
    from two_level_top_amd.chunk import Chunk
    ch = Chunk(wl, n_consumers=n_consumers)
    ch.run()
    torch.cuda.synchronize()
    return ch


def _consumer_views(ch, n_cons):
    """Per consumer: (output row of each chunk row or None, its score buffer if
    that buffer still holds this consumer's scores, else None)."""
    nT = len(ch.T)
    full_last = {}
    tail_last = None
    for c in range(n_cons):
        if ch._is_tail(c):
            tail_last = c
        else:
            full_last[c % nT] = c
    out = []
    tail_pos = {int(r): i for i, r in enumerate(ch.tail_rows)} if ch.tail is not None else {}
    for c in range(n_cons):
        if ch._is_tail(c):
            out.append((tail_pos.get, ch.T_tail if tail_last == c else None))
        else:
            out.append((lambda r: r, ch.T[c % nT] if full_last.get(c % nT) == c else None))
    return out


def _check_chunk(wl, ch, rows, n_consumers):
    """Every step of a chunk against the oracle on the sampled rows: dense scores
    within tolerance; blocks, n_kept and valid lengths bit-exact (blocks up to
    ties within tolerance of the kb-th key); the source's and every consumer's
    selection up to ties within tolerance of the k-th score; and the consumer
    scores still held in the chunk's score buffers element by element."""
    res = oracle.run_chunk(wl, row_ids=rows, n_consumers=n_consumers)
    if ch.S is not None:   # (a chunk that rescores the source's candidates has no S)
        Sg = host(ch.S)[rows]
        valid = np.arange(wl.ld)[None, :] < wl.lens[rows][:, None]
        assert_close(Sg, res["S"], valid, f"{wl.name} chunk dense")
    if ch.rescore:
        # the source's top-(k+1) blocks (nested in its kb best) and their scores
        b2 = host(ch.table2.blocks)[rows]
        nk2 = host(ch.table2.n_kept)[rows]
        T2 = host(ch.T_src)[rows]
        v2 = host(ch.table2.valid_len)[rows]
        keys2 = oracle.block_keys(res["S"], wl.lens[rows], ch.k2, ldk=wl.ldk)   # keyed past k + 1
        for i, r in enumerate(rows):
            nb = int(oracle.nblocks(wl.lens[r:r + 1])[0])
            assert nk2[i] == min(nb, ch.k2), f"row {r}: {nk2[i]} nested blocks"
            kept = set(int(x) for x in b2[i, :nk2[i]])
            if nb > ch.k2:
                kth = kth_largest(keys2[i, :nb], ch.k2)
                order = np.lexsort((np.arange(nb), -keys2[i, :nb].astype(np.float64)))
                want = set(int(x) for x in order[:ch.k2])
                for x in kept ^ want:
                    assert within_tol(keys2[i, x], kth), f"row {r}: nested block {x}"
            pos = oracle.candidate_positions(b2[i:i + 1], v2[i:i + 1])[0, :v2[i]]
            assert_close(T2[i:i + 1, :v2[i]], res["S"][i:i + 1, pos], np.ones((1, v2[i]), bool),
                         f"{wl.name} row {r} rescored source scores")
    blocks_g = host(ch.table.blocks)[rows]
    n_kept_g = host(ch.table.n_kept)[rows]
    valid_g = host(ch.table.valid_len)[rows]
    src_g = host(ch.src_top)[rows]
    views = _consumer_views(ch, len(ch.cons_top))
    cons_all = [host(t) for t in ch.cons_top]
    T_all = [None if (T is None or ch.consumer_bf16) else host(T) for _, T in views]
    same_blocks = 0
    scores_checked = 0
    for i, r in enumerate(rows):
        L, nb = int(wl.lens[r]), int(oracle.nblocks(wl.lens[r:r + 1])[0])
        assert n_kept_g[i] == res["n_kept"][i]
        if nb > wl.kb:
            kth = kth_largest(res["keys"][i, :nb], wl.kb)
            assert_same_selection(blocks_g[i], res["blocks"][i], lambda b: res["keys"][i, b], kth,
                                  INT32_MAX, f"{wl.name} row {r} blocks")
        else:
            assert np.array_equal(blocks_g[i], res["blocks"][i])
        # the source's own top-k: scores are the oracle's dense row
        row_s = res["S"][i, :L]
        if L:
            kth = kth_largest(row_s, ch.k_src)
            off = int(wl.req_start[r])
            assert_same_selection(src_g[i], res["source_topk"][i],
                                  lambda p: row_s[p - off] if 0 <= p - off < L else None, kth, -1,
                                  f"{wl.name} row {r} source top-k")
        if np.array_equal(blocks_g[i], res["blocks"][i]):
            same_blocks += 1
            assert valid_g[i] == res["valid_len"][i]
            off = int(wl.req_start[r])
            v = int(valid_g[i])
            for c, (row_of, _) in enumerate(views):
                j = row_of(int(r))
                if j is None:
                    continue
                T_o = res["T"][c][i, :v]
                if T_all[c] is not None and v:
                    assert_close(T_all[c][j, :v][None], T_o[None], np.ones((1, v), bool),
                                 f"{wl.name} row {r} consumer {c} scores")
                    scores_checked += 1
                pos = res["positions"][i, :v]
                score = dict(zip((pos + off).tolist(), T_o.tolist()))
                if v:
                    kth = kth_largest(T_o, wl.kc)
                    assert_same_selection(cons_all[c][j], res["consumer_topk"][c][i], score.get, kth,
                                          -1, f"{wl.name} row {r} consumer {c}")
                else:
                    assert (cons_all[c][j] == -1).all()
    assert same_blocks >= 0.9 * len(rows), f"only {same_blocks}/{len(rows)} rows kept identical blocks"
    if not ch.consumer_bf16 and len(ch.cons_top):
        assert scores_checked > 0, "no consumer scores were compared"


def _check_bf16_agreement(wl, ch, rows, n_consumers):
    """The prefill PR's acceptance test of bf16 consumer scores: the selection
    agrees with the fp32 one on at least 95% of the positions, picks lie inside
    the candidate blocks, and every disagreement is within 2^-5 relative of the
    selection floor (the fp32 k-th score)."""
    res = oracle.run_chunk(wl, row_ids=rows, n_consumers=n_consumers)
    blocks_g = host(ch.table.blocks)[rows]
    agree = total = 0
    for c in range(len(ch.cons_top)):
        got = host(ch.cons_top[c])[rows]
        for i, r in enumerate(rows):
            if not np.array_equal(blocks_g[i], res["blocks"][i]):
                continue        # a block set that differs at a tie: compared elsewhere
            off = int(wl.req_start[r])
            valid = int(res["valid_len"][i])
            if valid == 0:
                assert (got[i] == -1).all()
                continue
            T_o = res["T"][c][i, :valid]
            pos = res["positions"][i, :valid] + off
            score = dict(zip(pos.tolist(), T_o.tolist()))
            g = set(int(x) for x in got[i] if x != -1)
            o = set(int(x) for x in res["consumer_topk"][c][i] if x != -1)
            assert len(g) == len(o)
            assert g <= set(score), f"row {r}: a pick outside the candidate blocks"
            floor = kth_largest(T_o, wl.kc)
            for x in g ^ o:
                assert abs(score[x] - floor) <= 2.0 ** -5 * abs(floor), (r, x, score[x], floor)
            agree += len(g & o)
            total += len(o)
    assert total > 0 and agree >= 0.95 * total, f"agreement {agree}/{total}"


@pytest.mark.parametrize("name", ["tiny", "decode", "long"])
def test_chunk_bf16_consumers(idx, name):
    from two_level_top_amd.chunk import Chunk
    if name == "tiny":
        wl, rows, nc = workloads.tiny(), np.arange(64), None
    elif name == "decode":
        wl, rows, nc = workloads.decode(n_consumers=2), np.arange(0, 64, 3), None
    else:
        wl, rows, nc = workloads.long_chunk(n_consumers=1), np.array([0, 4096, 16383]), 1
    say(f"chunk {name} with bf16 consumer scores")
    ch = Chunk(wl, n_consumers=nc, consumer_bf16=True)
    ch.run()
    torch.cuda.synchronize()
    _check_bf16_agreement(wl, ch, rows, nc)


@pytest.mark.parametrize("source", ["rescore", "dense"])
def test_chunk_tiny(idx, source):
    from two_level_top_amd.chunk import Chunk
    wl = workloads.tiny()
    say(f"chunk tiny, source top-k from {source}")
    ch = Chunk(wl, source_scores=source)
    ch.run()
    torch.cuda.synchronize()
    _check_chunk(wl, ch, np.arange(wl.rows), None)


@pytest.mark.parametrize("source", ["rescore", "dense"])
def test_chunk_decode(idx, source):
    from two_level_top_amd.chunk import Chunk
    wl = workloads.decode(n_consumers=2)
    say(f"chunk decode (64 requests x 1 row), source top-k from {source}")
    ch = Chunk(wl, source_scores=source)
    ch.run()
    torch.cuda.synchronize()
    _check_chunk(wl, ch, np.arange(0, 64, 4), None)


def test_chunk_long_dense_source(idx):
    """The long chunk with the source's top-k taken from the dense score matrix
    (GATHER over the candidate columns): sampled rows against the oracle."""
    from two_level_top_amd.chunk import Chunk
    wl = workloads.long_chunk(n_consumers=1)
    say("chunk long, source top-k from the dense score matrix")
    ch = Chunk(wl, source_scores="dense")
    ch.run()
    torch.cuda.synchronize()
    _check_chunk(wl, ch, np.array([0, 7, 9000, 16383]), 1)


def test_dense_keys_newest_block_edges(idx):
    """4096-position chunks (1024 rows x 64K context) with row lengths that put
    the newest block at every offset of a page and next to page and chunk
    edges, rows of a wave from one request and from two: the fused keys equal
    idx_amax8_varlen on the same S for every row, the newest block's key is
    +inf and nothing is written past it, the keys-only pass writes the same
    keys, and S is within tolerance of the oracle on rows at the edges."""
    from two_level_top_amd.chunk import Chunk
    deltas = [-4097, -4096, -4095, -65, -64, -63, -9, -8, -7, -1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9,
              63, 64, 65, 4095]
    per = [301, 256, 467]   # odd counts: some waves hold rows of two requests
    ctx = 65536
    lens, r = [], 0
    for n in per:
        L = []
        for _ in range(n):
            base = 4096 * (1 + (r // len(deltas)) % 15)
            L.append(int(min(max(base + deltas[r % len(deltas)], 1), ctx)))
            r += 1
        lens.append(L)
    wl = workloads.custom("newest_edges", 91, 64, 64, 32, [ctx] * len(per), per, lens, n_layers=1)
    say(f"dense keys, newest-block edges: {wl.rows} rows x {ctx}")
    ch = Chunk(wl, n_consumers=0)
    L0 = wl.layers[0]
    q = idx.Query(dev(L0.qv), dev(L0.qs), dev(L0.w))
    S = torch.full((wl.rows, wl.ld), float("nan"), dtype=torch.float32, device="cuda")
    keys = torch.full((wl.rows, wl.ldk), -7.0, dtype=torch.float32, device="cuda")
    idx.idx_score_dense_keys(q, ch.kp, ch.rows, S, keys, skip_le_blocks=0)
    ref_keys = torch.full_like(keys, -7.0)
    idx.idx_amax8_varlen(S, ch.rows.len, ref_keys, skip_le_blocks=0)
    k2 = torch.full_like(keys, -7.0)
    idx.idx_score_dense_keys(q, ch.kp, ch.rows, None, k2, skip_le_blocks=0, ld=wl.ld)
    torch.cuda.synchronize()
    assert bool((keys == ref_keys).all()), "fused keys differ from idx_amax8_varlen on the same S"
    assert bool((keys == k2).all()), "keys-only pass differs from the pass that writes S"
    kg = host(keys)
    nblk = oracle.nblocks(wl.lens)
    for i in range(wl.rows):
        m = int(nblk[i])
        assert np.isposinf(kg[i, m - 1]), f"row {i}: newest block key is not +inf"
        assert np.isfinite(kg[i, :m - 1]).all(), f"row {i}: a key before the newest is not finite"
        assert (kg[i, m:] == -7.0).all(), f"row {i}: keys written past nblk"
    rows = np.array([0, 1, 2, 300, 301, 302, 556, 557, 1022, 1023] +
                    [i for i in range(24, 36)])
    ref = oracle.dense_scores(L0.qv, L0.qs, L0.w, wl.req, wl.lens, wl.pool, wl.page_table,
                              row_ids=rows, ld=wl.ld)
    valid = np.arange(wl.ld)[None, :] < wl.lens[rows][:, None]
    assert_close(host(S[torch.from_numpy(rows).cuda()]), ref, valid, "newest-block edges dense")


def test_keys_only_pass_matches_keys_with_scores(idx):
    """idx_score_dense_keys without S writes the same keys as with S."""
    from two_level_top_amd.chunk import Chunk
    for wl in (workloads.tiny(), workloads.decode(n_consumers=0)):
        say(f"keys-only dense pass, {wl.name}")
        ch = Chunk(wl, n_consumers=0, source_scores="dense")
        L = wl.layers[0]
        q = idx.Query(dev(L.qv), dev(L.qs), dev(L.w))
        k1 = torch.full((wl.rows, wl.ldk), -7.0, dtype=torch.float32, device="cuda")
        k2 = torch.full_like(k1, -7.0)
        S = torch.empty((wl.rows, wl.ld), dtype=torch.float32, device="cuda")
        for skip in (0, 9):
            k1.fill_(-7.0)
            k2.fill_(-7.0)
            idx.idx_score_dense_keys(q, ch.kp, ch.rows, S, k1, skip_le_blocks=skip)
            idx.idx_score_dense_keys(q, ch.kp, ch.rows, None, k2, skip_le_blocks=skip, ld=wl.ld)
            assert bool((k1 == k2).all()), f"{wl.name} skip={skip}"


def test_fold_queries_bitexact(idx):
    """idx_fold_queries writes, for several query batches in one launch, the same
    folded queries as each score call's own fold into its workspace."""
    from two_level_top_amd.chunk import Chunk
    wls = [workloads.tiny(), workloads.decode(n_consumers=1), _fused_case("ragged24")[0]]
    qs, ref = [], []
    for wl in wls:
        ch = Chunk(wl, n_consumers=0, source_scores="dense", prefold=False)
        for L in wl.layers[:2]:
            q = idx.Query(dev(L.qv), dev(L.qs), dev(L.w))
            ws = idx.score_workspace(wl.rows)
            S = torch.empty((wl.rows, wl.ld), dtype=torch.float32, device="cuda")
            idx.idx_score_dense(q, ch.kp, ch.rows, S, ws=ws)
            qs.append(q)
            ref.append(host(ws)[: wl.rows * 1088])
    # an empty batch in the middle folds nothing and shifts nothing
    L = wls[0].layers[0]
    empty = idx.Query(dev(L.qv[:0]), dev(L.qs[:0]), dev(L.w[:0]))
    qs.insert(2, empty)
    ref.insert(2, np.zeros((0,), dtype=np.uint8))
    say(f"fold queries: {len(qs)} batches in one launch")
    out = [torch.full((max(16, q.rows * 1088),), 0xAB, dtype=torch.uint8, device="cuda") for q in qs]
    idx.idx_fold_queries(qs, out)
    for i, (o, r) in enumerate(zip(out, ref)):
        assert np.array_equal(host(o)[: len(r)], r), f"batch {i}"
    assert (host(out[2]) == 0xAB).all(), "the empty batch's workspace was written"


@pytest.mark.parametrize("name", ["tiny", "decode", "decode_mtp"])
def test_chunk_prefold_matches_call_folds(idx, name):
    """A chunk that folds every layer's query in one launch first gives the same
    outputs, bit for bit, as one whose score calls fold their own queries."""
    from two_level_top_amd.chunk import Chunk
    wl = {"tiny": workloads.tiny, "decode": workloads.decode, "decode_mtp": workloads.decode_mtp}[name]()
    say(f"prefold chunk {name}")
    outs = []
    for prefold in (False, True):
        for source in ("rescore", "dense"):
            ch = Chunk(wl, source_scores=source, prefold=prefold)
            ch.run()
            outs.append((prefold, source, host(ch.src_top), [host(c) for c in ch.cons_top],
                         host(ch.table.blocks)))
    for source in ("rescore", "dense"):
        a = [o for o in outs if o[1] == source and not o[0]][0]
        b = [o for o in outs if o[1] == source and o[0]][0]
        assert np.array_equal(a[2], b[2]), f"{name} {source}: source top-k"
        assert all(np.array_equal(x, y) for x, y in zip(a[3], b[3])), f"{name} {source}: consumers"
        assert np.array_equal(a[4], b[4]), f"{name} {source}: blocks"


def test_chunk_decode_overlap_matches_serial(idx):
    """Few rows run the selects on their own stream, behind the next consumer's
    scores, with two score buffers reused across 4 consumers; the outputs are
    those of the serial order bit for bit (the serial order is checked against
    the oracle above)."""
    from two_level_top_amd.chunk import Chunk
    wl = workloads.decode()
    say("chunk decode, 4 consumers: overlapped selects vs serial")
    a = Chunk(wl, overlap_selects=True)
    b = Chunk(wl, overlap_selects=False)
    assert a.overlap and not b.overlap and len(a.T) == 2 and len(a.cons_top) == 4
    for _ in range(2):
        a.run()
        b.run()
    torch.cuda.synchronize()
    assert np.array_equal(host(a.src_top), host(b.src_top))
    for x, y in zip(a.cons_top, b.cons_top):
        assert np.array_equal(host(x), host(y))
    for name in ("blocks", "n_kept", "phys", "valid_len"):
        assert np.array_equal(host(getattr(a.table, name)), host(getattr(b.table, name))), name


def test_chunk_graph_replay(idx):
    """The decode step captured as one HIP graph: every replay reproduces the
    eager step's outputs bit for bit, with eager work between the replays
    (every output buffer overwritten first, so a replay that skipped a call
    would show)."""
    from two_level_top_amd.chunk import Chunk
    wl = workloads.decode()
    say("chunk decode captured as a HIP graph, 3 replays")
    ch = Chunk(wl)
    ch.run()
    torch.cuda.synchronize()
    names = ("blocks", "n_kept", "phys", "valid_len")
    ref = {"src": host(ch.src_top), **{n: host(getattr(ch.table, n)) for n in names}}
    if ch.S is not None:
        ref["S"] = host(ch.S)
    ref_c = [host(t) for t in ch.cons_top]
    ch.capture()
    for _ in range(3):
        if ch.S is not None:
            ch.S.fill_(float("nan"))
        ch.src_top.fill_(-7)
        for t in ch.cons_top:
            t.fill_(-7)
        for n in names:
            getattr(ch.table, n).fill_(-7)
        torch.cuda.synchronize()
        ch.replay()
        torch.cuda.synchronize()
        valid = np.arange(wl.ld)[None, :] < wl.lens[:, None]   # S past len is never written
        if ch.S is not None:
            assert np.array_equal(host(ch.S)[valid], ref["S"][valid])
        assert np.array_equal(host(ch.src_top), ref["src"])
        for t, r in zip(ch.cons_top, ref_c):
            assert np.array_equal(host(t), r)
        for n in names:
            assert np.array_equal(host(getattr(ch.table, n)), ref[n]), n


def test_chunk_mixed_small(idx):
    wl = workloads.mixed(n_consumers=2, decode_rows=32, max_decode_ctx=65536)
    say(f"chunk mixed (rows {wl.rows}), consumer 1 on the tail rows")
    from two_level_top_amd.chunk import Chunk
    ch = Chunk(wl, tail_layers=1)
    ch.run()
    torch.cuda.synchronize()
    starts = np.concatenate([[0], np.cumsum(wl.rows_per_req)])
    rows = np.unique(np.concatenate([starts[:-1], starts[1:] - 1, np.arange(0, wl.rows, 397),
                                     ch.tail_rows[::29]]))
    rows = rows[rows < wl.rows]
    _check_chunk(wl, ch, rows, None)


def _tail_case():
    return workloads.custom("tail", 7, 16, 4, 6, [300, 200, 90, 64], [40, 3, 1, 5],
                            [[260 + i for i in range(40)], [197, 198, 199], [90], [60, 61, 62, 63, 64]],
                            n_layers=3, tail=[5, 3, 1, 0])


def test_prefill_tail(idx):
    """The tail table against the full table's rows and the oracle; the tail
    consumer's scores and selection against the oracle's on those rows."""
    import two_level_top_amd as t
    from two_level_top_amd.chunk import Chunk
    wl = _tail_case()
    say("prefill tail (device row list), a tail consumer layer")
    ch = Chunk(wl, tail_layers=1)
    ch.run()
    torch.cuda.synchronize()
    _check_chunk(wl, ch, np.arange(wl.rows), None)
    trows = oracle.tail_rows(wl.rows_per_req, wl.tail_len)
    assert np.array_equal(ch.tail_rows, trows)
    for name in ("blocks", "n_kept", "phys", "valid_len", "len", "req"):
        assert np.array_equal(host(getattr(ch.tail, name)), host(getattr(ch.table, name))[trows]), name
    # (_check_chunk above compared the tail consumer's scores and selection with
    # the oracle's on every tail row)
    sched = host(ch.tail.schedule).view(np.int32)
    assert sched[0] == len(trows) * ((wl.kb + 63) // 64)
    nk = host(ch.tail.n_kept)
    firsts = sched[4:4 + 2 * sched[0]].reshape(-1, 2)[:, 1]
    assert ((firsts >= 0).reshape(len(trows), -1).sum(1) == (nk + 63) // 64).all()
    # the call on its own, from host lists, into a fresh table: same rows;
    # tail rows beyond the tail lengths' sum come out empty
    tail = t.Table(len(trows) + 2, wl.kb)
    t.idx_prefill_tail(ch.table, wl.rows_per_req, wl.tail_len, tail)
    assert np.array_equal(host(tail.blocks)[:len(trows)], host(ch.tail.blocks))
    assert (host(tail.n_kept)[len(trows):] == 0).all() and (host(tail.valid_len)[len(trows):] == 0).all()
    assert (host(tail.phys)[len(trows):] == -1).all()
    # lengths past a request's rows are clamped to its rows
    clamped = t.Table(int(wl.rows_per_req.sum()), wl.kb)
    t.idx_prefill_tail(ch.table, wl.rows_per_req, wl.rows_per_req + 3, clamped)
    assert np.array_equal(host(clamped.blocks), host(ch.table.blocks))


def test_chunk_prefill_sampled(idx):
    wl = workloads.prefill(n_consumers=2)
    say("chunk prefill 2048 x 65536 (sampled rows)")
    ch = _run_chunk(idx, wl)
    _check_chunk(wl, ch, np.array([0, 5, 1000, 2047]), 2)


def test_chunk_long_sampled(idx):
    """The benchmarked chunk itself: 16384 rows at 262144-position context,
    source + 4 consumers, launched exactly as bench.py launches it; sampled
    rows checked against the oracle, the last consumer's scores element by
    element."""
    wl = workloads.long_chunk()
    say("chunk long 16384 x 262144, source + 4 consumers (sampled rows)")
    ch = _run_chunk(idx, wl)
    _check_chunk(wl, ch, np.array([0, 1, 2, 4095, 8192, 12345, 16382, 16383]), None)


def test_chunk_mixed_full(idx):
    """The mixed batch at full size: 8 prefill requests and 256 decode rows
    up to 262144 context, duplicated K records; the last two consumers score
    only the tail rows (min(64, n) per request) through idx_prefill_tail."""
    from two_level_top_amd.chunk import Chunk
    wl = workloads.mixed()
    say(f"chunk mixed full (rows {wl.rows}, pages {wl.num_pages}), 2 tail consumers")
    ch = Chunk(wl, tail_layers=2)
    ch.run()
    torch.cuda.synchronize()
    starts = np.concatenate([[0], np.cumsum(wl.rows_per_req)])
    rows = np.unique(np.concatenate([starts[:8], starts[1:9] - 1, starts[8] + np.arange(0, 256, 37),
                                     ch.tail_rows[::61]]))
    _check_chunk(wl, ch, rows, None)
    trows = oracle.tail_rows(wl.rows_per_req, wl.tail_len)
    for name in ("blocks", "n_kept", "phys", "valid_len", "len", "req"):
        assert np.array_equal(host(getattr(ch.tail, name)), host(getattr(ch.table, name))[trows]), name


def test_chunk_graph_with_tail(idx):
    """Publish, the tail table and the consumers (two on the full table, one on
    the tail rows) captured as one HIP graph: every replay equals the eager
    step bit for bit, with every output overwritten eagerly in between."""
    from two_level_top_amd.chunk import Chunk
    wl = workloads.mixed(n_consumers=3, decode_rows=16, max_decode_ctx=32768)
    say(f"chunk mixed (rows {wl.rows}) with a tail consumer, captured as a HIP graph")
    ch = Chunk(wl, tail_layers=1)
    ch.run()
    torch.cuda.synchronize()
    names = ("blocks", "n_kept", "phys", "valid_len")
    outs = lambda: [ch.src_top, *ch.cons_top, *(getattr(ch.table, n) for n in names),
                    *(getattr(ch.tail, n) for n in names)]
    ref = [host(x) for x in outs()]
    ch.capture()
    for _ in range(3):
        for x in outs():
            x.fill_(-7)
        torch.cuda.synchronize()
        ch.replay()
        torch.cuda.synchronize()
        for x, r in zip(outs(), ref):
            assert np.array_equal(host(x), r)


def test_publish_error_joins_side_stream(idx):
    """A host-side validation error inside publish (after the block top-k was
    already enqueued on the side stream) under graph capture: the main stream
    rejoins the side stream before the error propagates, so the capture ends
    cleanly and the library's own error is what the caller sees."""
    import two_level_top_amd as t
    from two_level_top_amd.chunk import Chunk
    wl = workloads.tiny()
    say("publish raising inside a graph capture")
    ch = Chunk(wl)
    ch.run()
    torch.cuda.synchronize()
    good = ch.table.schedule
    ch.table.schedule = torch.empty((8,), dtype=torch.uint8, device="cuda")   # too small
    g = torch.cuda.CUDAGraph()
    with pytest.raises(t.IdxError, match="schedule_bytes"):
        with torch.cuda.graph(g):
            ch.score_source()
            ch.publish()
    ch.table.schedule = good
    torch.cuda.synchronize()
    ch.run()
    torch.cuda.synchronize()
    _check_chunk(wl, ch, np.arange(0, wl.rows, 7), None)


def test_chunk_decode_mtp(idx):
    """Decode with two rows per request (multi-token prediction / verify:
    lengths C - 1 and C) against the oracle on every row; and the paired rows
    equal the same rows scored apart from each other, bit for bit."""
    from two_level_top_amd.chunk import Chunk
    wl = workloads.decode_mtp(n_consumers=2)
    say(f"chunk decode MTP ({wl.rows} rows, 2 per request)")
    ch = Chunk(wl)
    ch.run()
    torch.cuda.synchronize()
    _check_chunk(wl, ch, np.arange(wl.rows), None)
    for parity in (0, 1):
        sel = np.arange(parity, wl.rows, 2)
        sub = Chunk(workloads.select_rows(wl, sel))
        sub.run()
        torch.cuda.synchronize()
        idx_t = torch.from_numpy(sel).cuda()
        assert np.array_equal(host(sub.src_top), host(ch.src_top[idx_t]))
        for name in ("blocks", "n_kept", "valid_len"):
            assert np.array_equal(host(getattr(sub.table, name)), host(getattr(ch.table, name)[idx_t]))
        for a, b in zip(sub.cons_top, ch.cons_top):
            assert np.array_equal(host(a), host(b[idx_t]))
