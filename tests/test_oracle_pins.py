"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks one oracle step against the format definition, a closed form,
exact rational brute force, or an invariant the method guarantees.  The
mutation tests at the end plant mistakes in copies of the oracle and check
that these pins catch them.
"""

from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from workloads import PAGE, PAGE_BYTES, SCALE_BYTES, VAL_BYTES

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers written from the OCP MX format definition (not from the oracle)
# ---------------------------------------------------------------------------

def e2m1_from_bits(code: int) -> Fraction:
    """FP4 E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0."""
    s = -1 if code & 8 else 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return s * Fraction(m, 2)             # subnormal: 2^(1-1) * (m/2)
    return s * Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))


def ue8m0(byte: int) -> Fraction:
    return Fraction(2) ** (byte - 127)


def decode_vec(vals: np.ndarray, scales: np.ndarray) -> list[Fraction]:
    out = []
    for i in range(128):
        b = int(vals[i // 2])
        code = (b >> 4) if i % 2 else (b & 15)
        out.append(e2m1_from_bits(code) * ue8m0(int(scales[i // 32])))
    return out


def round_to_f32(x: Fraction) -> np.float32:
    """Correctly rounded (half to even) fp32 of an exact rational (normal range)."""
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length() - 24
    while a / Fraction(2) ** e >= 2 ** 24:
        e += 1
    while a / Fraction(2) ** e < 2 ** 23:
        e -= 1
    assert e >= -149
    m = a / Fraction(2) ** e
    q, r = divmod(m.numerator, m.denominator)
    if 2 * r > m.denominator or (2 * r == m.denominator and q % 2 == 1):
        q += 1
    return np.float32(sign * float(q) * 2.0 ** e)


def key_record(wl, req, pos):
    page = int(wl.page_table[req, pos // PAGE])
    slot = pos % PAGE
    v = wl.pool[page, slot * VAL_BYTES:(slot + 1) * VAL_BYTES]
    s = wl.pool[page, PAGE * VAL_BYTES + slot * SCALE_BYTES: PAGE * VAL_BYTES + (slot + 1) * SCALE_BYTES]
    return v, s


def small_wl(heads=4, ctx=(40, 23), seed=11, kb=2, kc=5, lowrank=False, dup=0.0, layers=2):
    rows_per_req = [3, 2]
    lens = [[ctx[0] - 3 + i for i in range(3)], [ctx[1] - 2 + i for i in range(2)]]
    return workloads.custom("small", seed, heads, kb, kc, list(ctx), rows_per_req, lens,
                            n_layers=layers, lowrank=lowrank, dup_frac=dup, keep_keys=True)


def ref_dense_f64(wl, layer):
    """Dense scores via numpy float64 on decoded operands (an independent path)."""
    lut = np.array([float(e2m1_from_bits(c)) for c in range(16)])
    R, H = layer.qv.shape[:2]

    def dec(vals, scales):
        codes = np.stack([vals & 15, vals >> 4], axis=-1).reshape(*vals.shape[:-1], 128)
        sc = np.exp2(scales.astype(np.float64) - 127)
        return lut[codes] * np.repeat(sc, 32, axis=-1)

    q = dec(layer.qv, layer.qs)                       # [R, H, 128]
    out = np.full((R, wl.ld), np.nan)
    for r in range(R):
        j = int(wl.req[r])
        kv, ks = wl.keys_logical[j]
        n = int(wl.lens[r])
        k = dec(kv[:n], ks[:n])                       # [n, 128]
        s = q[r] @ k.T                                # [H, n]
        out[r, :n] = (layer.w[r].astype(np.float64)[:, None] * np.maximum(s, 0)).sum(0)
    return out


# ---------------------------------------------------------------------------
# 1. decoding
# ---------------------------------------------------------------------------

def test_e2m1_table_matches_ocp_spec():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_ocp_mx.txt")) if not l.startswith("#")]
    assert len(rows) == 16
    for code, val in rows:
        assert oracle.e2m1_value(int(code)) == float(val)
        assert float(e2m1_from_bits(int(code))) == float(val)


def test_ue8m0_scale():
    assert oracle.ue8m0_value(127) == 1.0
    assert oracle.ue8m0_value(128) == 2.0
    assert oracle.ue8m0_value(0) == 2.0 ** -127
    assert oracle.ue8m0_value(254) == 2.0 ** 127
    assert np.isnan(oracle.ue8m0_value(255))


# ---------------------------------------------------------------------------
# 2. logits
# ---------------------------------------------------------------------------

def _one_position_wl(qvec, qsc, kvec, ksc, w):
    """A workload of 1 row, 1 position, given explicit bytes (H = len(w))."""
    wl = workloads.custom("unit", 99, len(w), 2, 1, [1], [1], [[1]], n_layers=1)
    wl.layers[0].qv[:] = qvec
    wl.layers[0].qs[:] = qsc
    wl.layers[0].w[:] = np.asarray(w, np.float32)
    page = wl.page_table[0, 0]
    wl.pool[page, :VAL_BYTES] = kvec
    wl.pool[page, PAGE * VAL_BYTES:PAGE * VAL_BYTES + SCALE_BYTES] = ksc
    return wl


def _score(wl):
    L = wl.layers[0]
    return oracle.dense_scores(L.qv, L.qs, L.w, wl.req, wl.lens, wl.pool, wl.page_table)[0, 0]


def test_logit_bruteforce_exact_rationals():
    wl = small_wl()
    L = wl.layers[0]
    S = oracle.dense_scores(L.qv, L.qs, L.w, wl.req, wl.lens, wl.pool, wl.page_table)
    H = L.qv.shape[1]
    for r in range(wl.rows):
        q = [decode_vec(L.qv[r, h], L.qs[r, h]) for h in range(H)]
        for p in range(int(wl.lens[r])):
            k = decode_vec(*key_record(wl, int(wl.req[r]), p))
            exact = Fraction(0)
            for h in range(H):
                s = sum(a * b for a, b in zip(q[h], k))
                if s > 0:
                    exact += Fraction(float(L.w[r, h])) * s
            assert S[r, p] == round_to_f32(exact), (r, p)
        assert np.isnan(S[r, int(wl.lens[r]):]).all()


def test_logit_matches_float64_reference_tiny():
    wl = workloads.tiny(keep_keys=True)
    for L in wl.layers:
        S = oracle.dense_scores(L.qv, L.qs, L.w, wl.req, wl.lens, wl.pool, wl.page_table)
        ref = ref_dense_f64(wl, L)
        m = ~np.isnan(ref)
        assert (np.isnan(S) == ~m).all()
        ulp = np.spacing(np.abs(ref[m]).astype(np.float32))
        assert (np.abs(S[m] - ref[m]) <= ulp).all()


def _bytes_from_codes(codes):
    codes = np.asarray(codes, np.uint8)
    return (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)


def test_logit_closed_forms():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, 128)
    k = _bytes_from_codes(codes)
    ksc = np.array([126, 127, 128, 125], np.uint8)
    # H = 1, w = 1, q = k: the squared norm of k^
    wl = _one_position_wl(k, ksc, k, ksc, [1.0])
    kk = decode_vec(k, ksc)
    assert _score(wl) == round_to_f32(sum(a * a for a in kk))
    # q = -k (sign bits flipped): relu(-|k|^2) = 0 for either sign of w
    neg = _bytes_from_codes(codes ^ 8)
    assert _score(_one_position_wl(neg, ksc, k, ksc, [1.0])) == 0.0
    assert _score(_one_position_wl(neg, ksc, k, ksc, [-3.0])) == 0.0
    # w = 0 gives 0
    assert _score(_one_position_wl(k, ksc, k, ksc, [0.0])) == 0.0
    # linear in w for a power-of-two factor, on a multi-head case
    H = 4
    qv = np.stack([_bytes_from_codes(rng.integers(0, 16, 128)) for _ in range(H)])
    qs = rng.integers(124, 130, (H, 4)).astype(np.uint8)
    w = rng.standard_normal(H).astype(np.float32)
    a = _score(_one_position_wl(qv, qs, k, ksc, w))
    b = _score(_one_position_wl(qv, qs, k, ksc, w * 4))
    assert b == a * 4
    # ReLU per head: only heads with a positive dot contribute
    dots = [sum(x * y for x, y in zip(decode_vec(qv[h], qs[h]), kk)) for h in range(H)]
    exact = sum(Fraction(float(w[h])) * d for h, d in enumerate(dots) if d > 0)
    assert a == round_to_f32(exact)


def test_logit_one_hot_nibble_order_and_scale():
    # q has one nonzero element at index i; k one nonzero at index j -> product iff i == j
    for i, j, expect in [(0, 0, 1), (1, 1, 1), (0, 1, 0), (33, 33, 1), (127, 127, 1)]:
        qc = np.zeros(128, np.uint8); qc[i] = 2          # 1.0
        kc = np.zeros(128, np.uint8); kc[j] = 7          # 6.0
        qs = np.full(4, 127, np.uint8); ks = np.full(4, 127, np.uint8)
        ks[j // 32] = 129                               # x4
        got = _score(_one_position_wl(_bytes_from_codes(qc), qs, _bytes_from_codes(kc), ks, [0.5]))
        assert got == (0.5 * 6.0 * 4.0 if expect else 0.0), (i, j)
    # the low nibble is the even element: byte 0 = 0x02 is element 0 = 1.0
    v = np.zeros(64, np.uint8); v[0] = 0x02
    assert decode_vec(v, np.full(4, 127, np.uint8))[0] == 1
    assert decode_vec(v, np.full(4, 127, np.uint8))[1] == 0


def test_pool_round_trip():
    wl = small_wl()
    for j in range(wl.num_req):
        kv, ks = wl.keys_logical[j]
        for p in range(int(wl.ctx[j])):
            v, s = key_record(wl, j, p)
            assert (v == kv[p]).all() and (s == ks[p]).all()
    # every pool page is used by exactly one request page
    used = wl.page_table[wl.page_table >= 0]
    assert len(np.unique(used)) == len(used) == wl.num_pages


# ---------------------------------------------------------------------------
# 3. keys, selection, expansion, top-k (pure-Python brute force)
# ---------------------------------------------------------------------------

def _brute_keys(S_row, length, kb):
    nb = -(-length // 8)
    if nb <= kb:
        return None
    keys = [max(float(x) for x in S_row[8 * b: 8 * b + 8]) for b in range(nb - 1)]
    return keys + [float("inf")]


def _brute_select(keys, nb, kb):
    if nb <= kb:
        return list(range(nb))
    ranked = sorted(range(nb), key=lambda b: (-keys[b], b))
    return sorted(ranked[:kb])


def test_keys_and_selection_bruteforce():
    wl = workloads.tiny()
    res = oracle.run_chunk(wl)
    for i in range(wl.rows):
        n = int(wl.lens[i])
        bk = _brute_keys(res["S"][i], n, wl.kb)
        nb = -(-n // 8)
        assert bk is not None
        assert np.array_equal(res["keys"][i, :nb], np.array(bk, np.float32))
        sel = _brute_select(bk, nb, wl.kb)
        assert list(res["blocks"][i, :len(sel)]) == sel
        assert (res["blocks"][i, len(sel):] == oracle.INT32_MAX).all()
        assert res["n_kept"][i] == min(nb, wl.kb)
        # newest block always kept, ids strictly ascending
        assert nb - 1 in sel
        assert all(a < b for a, b in zip(sel, sel[1:]))


def test_selection_ties_go_to_lower_id():
    keys = np.array([[1.0, 5.0, 5.0, 2.0, 5.0, np.inf]], np.float32)
    blocks, n_kept = oracle.select_blocks(keys, np.array([48]), 3)
    assert list(blocks[0]) == [1, 2, 5] and n_kept[0] == 3
    blocks, _ = oracle.select_blocks(keys, np.array([48]), 4)
    assert list(blocks[0]) == [1, 2, 4, 5]


def test_keep_all_and_empty_rows():
    keys = np.full((3, 4), np.nan, np.float32)
    lens = np.array([0, 5, 24])
    blocks, n_kept = oracle.select_blocks(keys, lens, 3)
    assert list(n_kept) == [0, 1, 3]
    assert (blocks[0] == oracle.INT32_MAX).all()
    assert list(blocks[1]) == [0, oracle.INT32_MAX, oracle.INT32_MAX]
    assert list(blocks[2]) == [0, 1, 2]
    S = np.zeros((3, 24), np.float32)
    k = oracle.block_keys(S, lens, 3)
    assert np.isnan(k).all()       # no row has more than 3 blocks: none is keyed


def test_expand_closed_form():
    wl = workloads.tiny()
    res = oracle.run_chunk(wl)
    nb = oracle.nblocks(wl.lens)
    expect = 8 * res["n_kept"] - (8 * nb - wl.lens)
    assert np.array_equal(res["valid_len"], expect)
    for i in range(wl.rows):
        for c in range(int(res["n_kept"][i])):
            b = int(res["blocks"][i, c])
            page = int(wl.page_table[0, b // 8])
            assert res["phys"][i, c] == page * 8 + b % 8
        assert (res["phys"][i, res["n_kept"][i]:] == -1).all()
        # candidate columns map to positions inside the kept blocks and below len
        pos = res["positions"][i, :res["valid_len"][i]]
        assert (pos < wl.lens[i]).all() and (pos >= 0).all()
        assert np.all(np.diff(pos) > 0)


def test_topk_bruteforce_and_ties():
    X = np.array([[3.0, 7.0, 7.0, 1.0, 7.0, 0.0, -2.0]], np.float32)
    out = oracle.topk_positions(X, np.array([7]), 2)
    assert list(out[0]) == [1, 2]
    out = oracle.topk_positions(X, np.array([7]), 4)
    assert list(out[0]) == [0, 1, 2, 4]
    out = oracle.topk_positions(X, np.array([3]), 5)          # valid < k: pad -1
    assert list(out[0]) == [0, 1, 2, -1, -1]
    out = oracle.topk_positions(X, np.array([0]), 2)
    assert list(out[0]) == [-1, -1]
    cm = np.array([[10, 11, 12, 13, 40, 41, 42]])
    out = oracle.topk_positions(X, np.array([7]), 3, colmap=cm, pos_offset=np.array([100]))
    assert list(out[0]) == [111, 112, 140]
    rng = np.random.default_rng(3)
    X = rng.integers(-3, 4, (5, 50)).astype(np.float32)      # many ties
    valid = np.array([50, 49, 7, 1, 33])
    out = oracle.topk_positions(X, valid, 9)
    for i in range(5):
        v = int(valid[i])
        ranked = sorted(range(v), key=lambda c: (-X[i, c], c))[:9]
        exp = sorted(ranked) + [-1] * (9 - min(9, v))
        assert list(out[i]) == exp


# ---------------------------------------------------------------------------
# 4. invariants of the method
# ---------------------------------------------------------------------------

def test_full_candidate_coverage_gives_dense_topk():
    """kb * 8 >= context: the consumer's top-k equals its dense top-k."""
    wl = workloads.tiny()
    wl.kb = 128                     # 128 * 8 = 1024 = context
    res = oracle.run_chunk(wl)
    assert (res["n_kept"] == oracle.nblocks(wl.lens)).all()
    for ci, L in enumerate(wl.layers[1:]):
        S = oracle.dense_scores(L.qv, L.qs, L.w, wl.req, wl.lens, wl.pool, wl.page_table)
        dense = oracle.topk_positions(S, wl.lens, wl.kc, pos_offset=wl.req_start)
        assert np.array_equal(dense, res["consumer_topk"][ci])


def test_consumer_picks_inside_candidates():
    wl = workloads.tiny()
    res = oracle.run_chunk(wl)
    for sel in res["consumer_topk"]:
        for i in range(wl.rows):
            picks = sel[i][sel[i] >= 0]
            blocks = set(int(b) for b in res["blocks"][i, :res["n_kept"][i]])
            assert all(int(p) // 8 in blocks for p in picks)
            assert len(picks) == min(wl.kc, int(res["valid_len"][i]))


def test_source_topk_inside_candidates_and_equal_to_candidate_topk():
    """If kb > k, the dense top-k of the source lies inside its own kb blocks
    (every block holding a top-k position has at most k-1 + 1 blocks above it),
    so it equals the top-k taken over the candidate columns alone."""
    t = workloads.tiny()
    t.kc = 15                       # the identity needs kb >= k + 1 (tiny has kb = 16)
    for wl in (t, small_wl(kb=3, kc=2)):
        res = oracle.run_chunk(wl)
        via = oracle.topk_positions(
            np.take_along_axis(res["S"], np.maximum(res["positions"], 0).astype(np.int64), 1),
            res["valid_len"], wl.kc, colmap=res["positions"], pos_offset=wl.req_start)
        assert np.array_equal(via, res["source_topk"])


def test_tail_table_selects_like_full():
    wl = workloads.custom("tail", 7, 8, 4, 6, [300, 200, 90], [40, 3, 1],
                          [[260 + i for i in range(40)], [197, 198, 199], [90]],
                          n_layers=2, tail=[5, 3, 1])
    full = oracle.run_chunk(wl)
    rows = oracle.tail_rows(wl.rows_per_req, wl.tail_len)
    assert list(rows) == [35, 36, 37, 38, 39, 40, 41, 42, 43]
    tail = oracle.run_chunk(wl, row_ids=rows)
    for key in ("blocks", "n_kept", "phys", "valid_len"):
        assert np.array_equal(tail[key], full[key][rows])
    assert np.array_equal(tail["consumer_topk"][0], full["consumer_topk"][0][rows])


# ---------------------------------------------------------------------------
# 5. mutation checks: planted mistakes in copies of the oracle must fail a pin
# ---------------------------------------------------------------------------

MUTANTS = {
    # (swapping the two nibbles of every byte is not listed: it permutes q and k
    # alike inside one 32-element group, so no logit can observe it)
    "query scale of group 0 used for every group": ("int e = (int)as[g] +", "int e = (int)as[0] +"),
    "magnitude code table entry wrong": ("{0, 1, 2, 3, 4, 6, 8, 12}", "{0, 1, 2, 3, 4, 6, 8, 10}"),
    "relu dropped": ("if (s > 0.0) acc +=", "acc +="),
    "scale bias off by one": ("- 254 - 2;", "- 254 - 1;"),
    "sign bit ignored": ("(n & 8u) ? -m : m", "m"),
    "paged slot ignored": ("(int64_t)(pos % page_size) * VB", "(int64_t)0 * VB"),
}


def _build_mutant(tmp_path, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "idx_oracle.c")).read()
    assert old in src, old
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(path), "-lm"],
                   check=True)
    return ctypes.CDLL(str(so))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc needed to build mutants")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_oracle_mistakes(tmp_path, name):
    old, new = MUTANTS[name]
    good = oracle._load()
    mut = _build_mutant(tmp_path, old, new)
    for fn in ("oracle_dense_scores", "oracle_scores_at", "oracle_e2m1_value"):
        getattr(mut, fn).restype = getattr(good, fn).restype
        getattr(mut, fn).argtypes = getattr(good, fn).argtypes
    oracle._lib = mut
    try:
        failures = 0
        for pin in (test_logit_bruteforce_exact_rationals, test_logit_closed_forms,
                    test_logit_one_hot_nibble_order_and_scale, test_logit_matches_float64_reference_tiny):
            try:
                pin()
            except AssertionError:
                failures += 1
        assert failures > 0, f"no pin caught mutant '{name}'"
    finally:
        oracle._lib = good


def test_pins_catch_wrong_tie_rule(monkeypatch):
    def higher_id_wins(keys, lens, kb):
        nb = oracle.nblocks(lens)
        blocks = np.full((len(lens), kb), oracle.INT32_MAX, np.int32)
        n_kept = np.zeros(len(lens), np.int32)
        for i in range(len(lens)):
            m = int(nb[i])
            ids = np.arange(m)
            chosen = ids if m <= kb else np.sort(np.lexsort((-ids, -keys[i, :m].astype(np.float64)))[:kb])
            blocks[i, :len(chosen)] = chosen
            n_kept[i] = len(chosen)
        return blocks, n_kept

    monkeypatch.setattr(oracle, "select_blocks", higher_id_wins)
    with pytest.raises(AssertionError):
        test_selection_ties_go_to_lower_id()
