"""CPU oracle of the step before the index layers: query RoPE, MXFP4
quantisation and head-weight scaling (the vLLM indexer page, rope_quant_q and
fused_indexer_q_rope_quant).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the smoke
check and the benchmark's CPU baseline leg may use it; the product path never
does.  Plain numpy, one step per function, in the pages' order:

1. ``rope``      rotate the first 64 of each head's 128 dimensions by the
                 position's angles: pairs (i, i + 32) in the NeoX layout,
                 (2i, 2i + 1) otherwise; r0 = x0 cos - x1 sin and
                 r1 = x1 cos + x0 sin in fp32, each rounded to bf16.
                 Dimensions 64..127 pass through.
2. ``mxfp4_quantize``  per 32-element group: amax, the ue8m0 scale
                 2^ceil(log2(max(amax, 1e-10) * (1/6))), the e2m1 code of
                 x / scale rounded to the nearest grid value (ties to the even
                 code), saturated at 6.  Even elements in the low nibble.
3. weights       w * softmax_scale * head_scale in fp32 (the q scale stays
                 with the quantised query: it is not folded into the weights
                 on the fp4 path).

Readings where the pages leave a step open (stated again in the design
notes): the rotation's products and sums are separate fp32 roundings (no
fused multiply-add); ceil(log2(.)) is taken exactly on the fp32 value of the
scaled amax; -0 is written as code 0; cos/sin come as fp32, cos in columns
0..31 and sin in 32..63 of the position's 64-wide row.
"""

from __future__ import annotations

import numpy as np

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values."""
    return (np.asarray(u16, dtype=np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> the nearest bf16 value (ties to even), as float32 (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def rope(q: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray, is_neox: bool) -> np.ndarray:
    """q float32 [n, H, 128] (bf16 values) -> the rotated query, float32 (bf16 values)."""
    q = np.asarray(q, dtype=np.float32)
    cs = np.asarray(cos_sin, dtype=np.float32)[np.asarray(positions)]
    cos = cs[:, None, :32]
    sin = cs[:, None, 32:64]
    out = q.copy()
    if is_neox:
        i0, i1 = np.arange(32), np.arange(32) + 32
    else:
        i0, i1 = np.arange(0, 64, 2), np.arange(1, 64, 2)
    x0, x1 = q[..., i0], q[..., i1]
    r0 = (x0 * cos).astype(np.float32) - (x1 * sin).astype(np.float32)
    r1 = (x1 * cos).astype(np.float32) + (x0 * sin).astype(np.float32)
    out[..., i0] = bf16_round(r0.astype(np.float32))
    out[..., i1] = bf16_round(r1.astype(np.float32))
    return out


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """e with 2^e the ue8m0 scale of a group whose largest magnitude is amax."""
    raw = (np.maximum(np.asarray(amax, dtype=np.float32), np.float32(1e-10))
           * np.float32(1.0 / 6.0)).astype(np.float32)
    m, ex = np.frexp(raw)                     # raw = m * 2^ex, m in [0.5, 1)
    return np.where(m == 0.5, ex - 1, ex).astype(np.int32)   # ceil(log2(raw))


def e2m1_code(a: np.ndarray) -> np.ndarray:
    """Magnitude code 0..7 of the grid value nearest to a >= 0 (ties to the even
    code), saturated at 6."""
    a = np.minimum(np.asarray(a, dtype=np.float64), 6.0)
    d = np.abs(a[..., None] - E2M1_GRID)
    best = d.min(axis=-1, keepdims=True)
    tied = d == best
    even = tied & (np.arange(8) % 2 == 0)
    pick = np.where(even.any(axis=-1), even.argmax(axis=-1), tied.argmax(axis=-1))
    return pick.astype(np.uint8)


def mxfp4_quantize(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """float32 [..., 128] -> (codes u8 [..., 64], ue8m0 scales u8 [..., 4])."""
    x = np.asarray(x, dtype=np.float32)
    lead = x.shape[:-1]
    g = x.reshape(-1, 4, 32)
    e = scale_exponent(np.abs(g).max(axis=-1))
    assert (e >= -127).all() and (e <= 127).all()
    y = np.ldexp(g.astype(np.float64), -e[..., None])          # exact: power-of-two scale
    code = e2m1_code(np.abs(y))
    code = np.where((y < 0) & (code != 0), code | 8, code).astype(np.uint8).reshape(-1, 128)
    vals = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    scales = (e + 127).astype(np.uint8)
    return vals.reshape(*lead, 64), scales.reshape(*lead, 4)


def weights_out(w: np.ndarray, softmax_scale: float, head_scale: float) -> np.ndarray:
    return ((np.asarray(w, dtype=np.float32) * np.float32(softmax_scale)).astype(np.float32)
            * np.float32(head_scale)).astype(np.float32)


def q_rope_quant(q_bf16: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray, w: np.ndarray,
                 is_neox: bool, softmax_scale: float, head_scale: float):
    """The whole step: (codes [n, H, 64], scales [n, H, 4], weights [n, H])."""
    r = rope(bf16_to_f32(q_bf16), positions, cos_sin, is_neox)
    vals, scales = mxfp4_quantize(r)
    return vals, scales, weights_out(w, softmax_scale, head_scale)
