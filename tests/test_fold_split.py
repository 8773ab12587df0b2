"""The folded query's greedy MXFP4 split, on the CPU.

The score kernels write relu(s) = (s + |s|) / 2, so a row's score is
sum_h (w_h/2)|q_h.k| + q_f.k with the folded query q_f = sum_h (w_h/2) q_h.
q_f is not an MXFP4 vector; the kernels feed it to the fp4 MFMA as a sum of
MXFP4 terms found greedily: per 32-element group, scale 2^ceil(log2(max|r|/6))
and the nearest e2m1 code of every element of the residual r, then r minus
that term.  The fold kernel writes 16 terms per row; both score kernels use
the first 8 (the dense kernel packs two rows' 8 terms into one 16-row MFMA
block, the sparse kernel one row's).

These tests restate that split in numpy (independently of the kernel) and
check, on the query rows of the tiny and long workloads:

* the per-term bound: after t terms every group's largest residual is at most
  3^-t times the group's largest |q_f| element (the e2m1 grid's largest gap is
  2 at the top of [3, 6], where the scaled maximum lands);
* the score error the dropped terms leave, |residual . k| over real pool
  positions: at 8 terms below a tenth of the score tolerance's absolute part
  (1e-4; about 4% on the long workload's rows), at 16 terms nil.
"""

import os

import numpy as np
import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_ocp_mx.txt")) if not l.startswith("#")]
    return np.array([float(v) for _, v in rows])


E2M1 = _e2m1()
GRID = E2M1[:8]                    # magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6


def dequant(codes, scales):
    """[..., 64] code bytes (even element low nibble) + [..., 4] ue8m0 -> [..., 128]."""
    v = np.stack([E2M1[codes & 15], E2M1[codes >> 4]], axis=-1).reshape(*codes.shape[:-1], 128)
    return v * np.repeat(np.exp2(scales.astype(np.float64) - 127.0), 32, axis=-1)


def nearest_magnitude(a):
    """Nearest grid magnitude of a in [0, 6]; ties go to the even code."""
    d = np.abs(a[..., None] - GRID)
    best = d.min(axis=-1, keepdims=True)
    tie = d == best
    # among tied codes prefer the even one (codes 0..7 are indices into GRID)
    even = tie & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=-1), even.argmax(axis=-1), tie.argmax(axis=-1))
    return GRID[idx]


def greedy_split(qf, terms):
    """Residuals after each of `terms` greedy MXFP4 terms of qf [n, 128]."""
    r = qf.copy()
    out = []
    for _ in range(terms):
        g = r.reshape(len(r), 4, 32)
        m = np.abs(g).max(axis=2, keepdims=True)
        with np.errstate(divide="ignore"):
            e = np.where(m > 0, np.ceil(np.log2(m / 6.0)), -127.0)
        e = np.clip(e, -127, 127)
        s = np.exp2(e)
        term = np.sign(g) * nearest_magnitude(np.abs(g) / s) * s
        r = (g - term).reshape(len(r), 128)
        out.append(r.copy())
    return out


def folded_queries(wl, rows):
    L = wl.layers[0]
    q = dequant(L.qv[rows], L.qs[rows])                      # [n, H, 128]
    return np.einsum("nh,nhd->nd", 0.5 * L.w[rows].astype(np.float64), q)


def pool_keys(wl, n_pages, seed=0):
    pages = np.random.default_rng(seed).choice(wl.pool.shape[0], size=n_pages, replace=False)
    pg = wl.pool[pages]
    vals = pg[:, :64 * 64].reshape(-1, 64)
    scl = pg[:, 64 * 64:].reshape(-1, 4)
    return dequant(vals, scl)                                # [n_pages * 64, 128]


def test_nearest_magnitude_ties_and_range():
    a = np.array([0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.3, 4.9])
    # ties: 0.25 -> 0 (code 0), 0.75 -> 1 (code 2), 1.25 -> 1 (code 2), 1.75 -> 2 (code 4),
    # 2.5 -> 2 (code 4), 3.5 -> 4 (code 6), 5 -> 4 (code 6)
    want = np.array([0.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 0.5, 4.0])
    assert (nearest_magnitude(a) == want).all()


def test_split_of_an_mxfp4_vector_is_exact_in_one_term():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, size=(5, 64), dtype=np.uint8)
    scales = rng.integers(120, 135, size=(5, 4), dtype=np.uint8)
    x = dequant(codes, scales)
    # a group whose largest magnitude is below 3 scale steps maps to a smaller scale;
    # it is still exact, as the grid's values divide by powers of two exactly
    r = greedy_split(x, 2)
    assert np.abs(r[-1]).max() == 0.0


@pytest.mark.parametrize("name", ["tiny", "long"])
def test_greedy_split_bound_and_score_error(name):
    if name == "tiny":
        wl = workloads.tiny()
        rows = np.arange(wl.rows)
    else:
        wl = workloads.long_chunk(n_consumers=0)
        rows = np.random.default_rng(1).choice(wl.rows, size=512, replace=False)
    qf = folded_queries(wl, rows)
    gmax = np.repeat(np.abs(qf).reshape(len(rows), 4, 32).max(axis=2), 32, axis=1)
    res = greedy_split(qf, 16)
    for t, r in enumerate(res, start=1):
        assert (np.abs(r) <= gmax * 3.0 ** -t).all(), f"term {t}: residual above 3^-{t} of the group max"
    # the score error of the terms each scorer drops, over real pool positions
    K = pool_keys(wl, min(64, wl.pool.shape[0]))
    tol = 1e-4                                               # the absolute part of the tolerance
    for t, frac in ((8, 0.1), (16, 1e-6)):
        err = np.abs(res[t - 1] @ K.T)
        assert (err <= frac * tol).all(), \
            f"{t} terms: score error {err.max():.3g} is above {frac} of the tolerance"
