"""Pins of the query RoPE + MXFP4 quantisation oracle (oracle/q_quant.py)
against facts outside it: exact rational arithmetic, rotations with known
results, the relation between the two pair layouts, the e2m1 grid of the OCP
MX specification (tests/golden/e2m1_ocp_mx.txt) and closed forms."""

from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import q_quant as Q

GOLDEN_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def f32(x):
    return np.float32(x)


def exact_nearest_bf16(x: float) -> Fraction:
    """Nearest bf16 to the fp32 value x (ties to even mantissa), by brute force."""
    fx = Fraction(float(np.float32(x)))
    if fx == 0:
        return Fraction(0)
    sign = -1 if fx < 0 else 1
    a = abs(fx)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    step = Fraction(2) ** (e - 7)              # bf16: 7 stored mantissa bits
    lo = (a // step) * step
    hi = lo + step
    if a - lo < hi - a:
        r = lo
    elif a - lo > hi - a:
        r = hi
    else:
        r = lo if (lo / step) % 2 == 0 else hi
    return sign * r


def test_bf16_round_known_values():
    one = 1.0
    assert Q.bf16_round(np.array([one + 2 ** -8], np.float32))[0] == 1.0          # tie -> even
    assert Q.bf16_round(np.array([one + 2 ** -7 + 2 ** -8], np.float32))[0] == 1.0 + 2 ** -6
    assert Q.bf16_round(np.array([one + 3 * 2 ** -9], np.float32))[0] == 1.0 + 2 ** -7
    assert Q.bf16_round(np.array([-(one + 2 ** -8 + 2 ** -20)], np.float32))[0] == -(1.0 + 2 ** -7)


def test_bf16_round_brute_force():
    r = np.random.default_rng(5)
    x = (r.standard_normal(2000) * np.exp(r.normal(0, 8, 2000))).astype(np.float32)
    got = Q.bf16_round(x)
    for a, b in zip(x, got):
        assert Fraction(float(b)) == exact_nearest_bf16(a)


def _q(seed, n=3, h=2):
    r = np.random.default_rng(seed)
    return Q.bf16_round(r.standard_normal((n, h, 128)).astype(np.float32))


@pytest.mark.parametrize("neox", [True, False])
def test_rope_identity_and_quarter_turns(neox):
    q = _q(1)
    pos = np.zeros(3, np.int32)
    ident = np.concatenate([np.ones((1, 32)), np.zeros((1, 32))], 1).astype(np.float32)
    assert np.array_equal(Q.rope(q, pos, ident, neox), q)
    quarter = np.concatenate([np.zeros((1, 32)), np.ones((1, 32))], 1).astype(np.float32)
    half = np.concatenate([-np.ones((1, 32)), np.zeros((1, 32))], 1).astype(np.float32)
    i0 = np.arange(32) if neox else np.arange(0, 64, 2)
    i1 = i0 + 32 if neox else i0 + 1
    r = Q.rope(q, pos, quarter, neox)
    assert np.array_equal(r[..., i0], -q[..., i1]) and np.array_equal(r[..., i1], q[..., i0])
    r = Q.rope(q, pos, half, neox)
    assert np.array_equal(r[..., :64], -q[..., :64])
    assert np.array_equal(r[..., 64:], q[..., 64:])      # unrotated half untouched


def test_rope_layouts_are_a_permutation_of_each_other():
    q = _q(2, n=4, h=3)
    table = workloads.rope_table(100)
    pos = np.array([0, 7, 50, 99], np.int32)
    perm = np.arange(128)
    perm[:64] = np.stack([np.arange(32), np.arange(32) + 32], 1).reshape(-1)   # (i, i+32) -> (2i, 2i+1)
    inter = Q.rope(q[..., perm], pos, table, is_neox=False)
    neox = Q.rope(q, pos, table, is_neox=True)
    assert np.array_equal(inter, neox[..., perm])


def test_rope_matches_exact_arithmetic_then_bf16():
    q = _q(3, n=2, h=1)
    table = workloads.rope_table(64)
    pos = np.array([5, 63], np.int32)
    r = Q.rope(q, pos, table, is_neox=True)
    for n in range(2):
        c, s = table[pos[n], :32], table[pos[n], 32:]
        for i in range(32):
            x0, x1 = q[n, 0, i], q[n, 0, i + 32]
            a = f32(f32(x0 * c[i]) - f32(x1 * s[i]))       # two fp32 products, one fp32 difference
            b = f32(f32(x1 * c[i]) + f32(x0 * s[i]))
            assert Fraction(float(r[n, 0, i])) == exact_nearest_bf16(a)
            assert Fraction(float(r[n, 0, i + 32])) == exact_nearest_bf16(b)


def test_grid_matches_golden_table():
    rows = [l.split() for l in open(__file__.replace("test_q_quant_pins.py", "golden/e2m1_ocp_mx.txt"))
            if l.strip() and not l.startswith("#")]
    vals = sorted({abs(float(r[-1])) for r in rows})
    assert vals == GOLDEN_GRID == list(Q.E2M1_GRID)


def test_e2m1_code_ties_and_grid():
    for c, v in enumerate(GOLDEN_GRID):
        assert Q.e2m1_code(np.array([v]))[0] == c
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for a, c in ties.items():
        assert Q.e2m1_code(np.array([a]))[0] == c, a
    assert Q.e2m1_code(np.array([0.2500001]))[0] == 1
    assert Q.e2m1_code(np.array([7.5]))[0] == 7                 # saturates at 6


def test_scale_exponent_is_the_smallest_covering_power():
    r = np.random.default_rng(7)
    amax = np.concatenate([
        np.exp(r.normal(0, 10, 3000)).astype(np.float32),
        np.float32([0.0, 1e-30, 1e-10, 6.0, 3.0, 12.0, 6.0000005, 5.9999995, 1.0, 0.75]),
    ]).astype(np.float32)
    e = Q.scale_exponent(amax)
    for a, k in zip(amax, e):
        raw = Fraction(float(f32(f32(max(a, f32(1e-10))) * f32(1.0 / 6.0))))
        assert Fraction(2) ** int(k) >= raw and Fraction(2) ** (int(k) - 1) < raw, (a, k)


def test_quantize_round_trip_and_error_bound():
    r = np.random.default_rng(9)
    # on-grid values with the group's amax fixed at 6 * 2^e: exact round trip
    e = r.integers(-20, 20, size=(50, 4))
    codes = r.integers(0, 16, size=(50, 128)).astype(np.uint8)
    codes[:, ::32] = 7                                        # amax = 6 * 2^e in every group
    mag = np.array(GOLDEN_GRID)[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    x = (mag.reshape(50, 4, 32) * np.exp2(e)[..., None]).reshape(50, 128).astype(np.float32)
    vals, scales = Q.mxfp4_quantize(x)
    want = np.where((codes & 7) == 0, 0, codes).astype(np.uint8)   # -0 is written as 0
    assert np.array_equal(vals, (want[:, 0::2] | (want[:, 1::2] << 4)).astype(np.uint8))
    assert np.array_equal(scales.astype(int) - 127, e)
    # general values: |x - dequant| <= half the local grid step times the scale
    x = (r.standard_normal((200, 128)) * np.exp(r.normal(0, 3, (200, 1)))).astype(np.float32)
    vals, scales = Q.mxfp4_quantize(x)
    c = np.stack([vals & 15, vals >> 4], -1).reshape(200, 128)
    deq = np.array(GOLDEN_GRID)[c & 7] * np.where(c & 8, -1.0, 1.0)
    s = np.repeat(np.exp2(scales.astype(float) - 127), 32, axis=1)
    a = np.abs(x) / s
    half_step = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    assert (np.abs(x / s - deq) <= half_step + 1e-12).all()


def test_weights_and_zero_heads():
    w = np.array([[1.5, -2.0]], np.float32)
    out = Q.weights_out(w, 0.125, 64 ** -0.5)
    assert np.array_equal(out, np.float32([[1.5 * 0.125 * 0.125, -2.0 * 0.125 * 0.125]]))
    inp = workloads.q_inputs(3, 2, 2, max_pos=16)
    vals, scales, _ = Q.q_rope_quant(inp.q, inp.positions, inp.cos_sin, inp.w, True, 1.0, 1.0)
    assert (vals[0, 0] == 0).all()
    assert (scales[0, 0] == 127 + int(Q.scale_exponent(np.float32([0.0]))[0])).all()
    assert int(Q.scale_exponent(np.float32([0.0]))[0]) == -35     # 2^-35 >= 1e-10 / 6 > 2^-36


# ---- planted mistakes: each must be caught by one of the pins above ----

def _fails(test, *args):
    try:
        test(*args)
    except AssertionError:
        return True
    return False


def test_pins_catch_planted_mistakes(monkeypatch):
    # the rotation with the sign of sin flipped
    orig_rope = Q.rope
    def bad_rope(q, positions, cos_sin, is_neox):
        cs = np.asarray(cos_sin, np.float32).copy()
        cs[:, 32:] = -cs[:, 32:]
        return orig_rope(q, positions, cs, is_neox)
    monkeypatch.setattr(Q, "rope", bad_rope)
    assert _fails(test_rope_identity_and_quarter_turns, True)
    monkeypatch.setattr(Q, "rope", orig_rope)
    # e2m1 ties to the odd code
    orig_code = Q.e2m1_code
    def odd_ties(a):
        a = np.minimum(np.asarray(a, np.float64), 6.0)
        d = np.abs(a[..., None] - Q.E2M1_GRID)
        return (7 - np.argmin(d[..., ::-1], axis=-1)).astype(np.uint8)   # last of the tied
    monkeypatch.setattr(Q, "e2m1_code", odd_ties)
    assert _fails(test_e2m1_code_ties_and_grid)
    monkeypatch.setattr(Q, "e2m1_code", orig_code)
    # floor instead of ceil for the scale exponent
    orig_exp = Q.scale_exponent
    def floor_exp(amax):
        raw = (np.maximum(np.asarray(amax, np.float32), np.float32(1e-10)) * np.float32(1 / 6)).astype(np.float32)
        return np.floor(np.log2(raw)).astype(np.int32)
    monkeypatch.setattr(Q, "scale_exponent", floor_exp)
    assert _fails(test_scale_exponent_is_the_smallest_covering_power)
    monkeypatch.setattr(Q, "scale_exponent", orig_exp)
    # nibble order swapped in the packing
    orig_q = Q.mxfp4_quantize
    def swapped(x):
        v, s = orig_q(x)
        return ((v >> 4) | (v << 4)).astype(np.uint8), s
    monkeypatch.setattr(Q, "mxfp4_quantize", swapped)
    assert _fails(test_quantize_round_trip_and_error_bound)
