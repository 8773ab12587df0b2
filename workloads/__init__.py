"""Seeded synthetic inputs for the two-level candidate indexer.

This module only *makes bytes*: Gaussian draws, an MXFP4 encoder, page
permutations and per-row lengths.  It holds none of the indexer's arithmetic
(no dequantisation, no logits, no selection), so both the CPU oracle and the
HIP library can consume what it produces without sharing any method code.

Recipes (shapes follow the prefill/decode workloads of the sglang PR
"[DSv4.1] Score prefill consumer index layers on candidate blocks with
DeepGEMM", Design and Performance sections: 16384-row chunks, 262144-position
context, 2048 candidate blocks of 8, four consumer layers, top-512):

* q, K ~ N(0, 1) per element, encoded to MXFP4: one ue8m0 scale per 32
  elements, 2^ceil(log2(amax/6)), values rounded to the e2m1 grid
  {0, .5, 1, 1.5, 2, 3, 4, 6} (ties to the even code), two codes per byte,
  the even element in the low nibble.
* head weights w ~ N(0, 1/H) in fp32.
* the long chunk adds a low-rank term to K so block maxima are uneven:
  K = G + (A * gamma_page) @ Bm, A ~ N(0,1)^{S x 8}, gamma ~ LogNormal(0, .5)
  per 64-position page, Bm ~ N(0, 1/8)^{8 x 128}.
* the mixed batch overwrites 1% of each request's positions with copies of
  other positions of the same request (whole 68-byte records), so exact
  score ties occur.
* every request's pages are scattered over the pool by a seeded permutation.

Seeds: numpy PCG64 from SeedSequence([config, layer, tensor, chunk]); the
chunking fixes the stream, so results do not depend on the thread count.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

DIM = 128                 # index head dimension
PAGE = 64                 # positions per K-pool page
VAL_BYTES = DIM // 2      # packed e2m1 bytes per position
SCALE_BYTES = DIM // 32   # ue8m0 bytes per position
REC_BYTES = VAL_BYTES + SCALE_BYTES           # 68
PAGE_BYTES = PAGE * REC_BYTES                 # 4352: values then scales

# tensor ids for the seed sequence
_T_Q, _T_W, _T_K, _T_LOWRANK, _T_PERM, _T_LEN, _T_DUP = range(7)

_THREADS = max(1, min(16, os.cpu_count() or 1))


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


# ---------------------------------------------------------------------------
# MXFP4 encoder (generator side only)
# ---------------------------------------------------------------------------

def encode_mxfp4(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Encode float32 [..., 128] into (values u8 [..., 64], scales u8 [..., 4])."""
    x = np.asarray(x, dtype=np.float32)
    lead = x.shape[:-1]
    g = x.reshape(-1, DIM // 32, 32)
    amax = np.abs(g).max(axis=-1)
    v = np.maximum(amax, np.float32(1e-10)) / np.float32(6.0)
    m, ex = np.frexp(v)                       # v = m * 2^ex, m in [0.5, 1)
    e = np.where(m == 0.5, ex - 1, ex)        # ceil(log2(v))
    e = np.clip(e, -127, 127).astype(np.int32)
    y = np.ldexp(g, -e[..., None]).astype(np.float32)
    a = np.abs(y)
    code = np.where(
        a < 2.0, np.rint(a * 2.0),
        np.where(a < 4.0, 4.0 + np.rint(a - 2.0), 6.0 + np.rint((a - 4.0) * 0.5)))
    code = np.minimum(code, 7).astype(np.uint8)
    code |= (np.signbit(y).astype(np.uint8) << 3)
    code = code.reshape(-1, DIM)
    vals = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    scales = (e + 127).astype(np.uint8).reshape(-1, DIM // 32)
    return vals.reshape(*lead, VAL_BYTES), scales.reshape(*lead, SCALE_BYTES)


def _normal_chunks(key: tuple[int, ...], n_items: int, item_shape: tuple[int, ...],
                   chunk: int, transform=None) -> list[np.ndarray]:
    """Draw n_items x item_shape N(0,1) float32 in seeded chunks of `chunk` items."""
    starts = list(range(0, n_items, chunk))

    def one(ci: int):
        s = starts[ci]
        n = min(chunk, n_items - s)
        x = _rng(*key, ci).standard_normal((n, *item_shape), dtype=np.float32)
        return transform(x, s) if transform else x

    with ThreadPoolExecutor(_THREADS) as ex:
        return list(ex.map(one, range(len(starts))))


def gen_query(cfg: int, layer: int, rows: int, heads: int):
    """MXFP4 query [rows, heads, 128] and fp32 head weights [rows, heads]."""
    def enc(x, _s):
        return encode_mxfp4(x)
    parts = _normal_chunks((cfg, layer, _T_Q), rows, (heads, DIM), 256, enc)
    qv = np.concatenate([p[0] for p in parts]) if parts else np.zeros((0, heads, VAL_BYTES), np.uint8)
    qs = np.concatenate([p[1] for p in parts]) if parts else np.zeros((0, heads, SCALE_BYTES), np.uint8)
    w = (_rng(cfg, layer, _T_W).standard_normal((rows, heads), dtype=np.float32)
         * np.float32(1.0 / np.sqrt(heads))).astype(np.float32)
    return qv.reshape(rows, heads, VAL_BYTES), qs.reshape(rows, heads, SCALE_BYTES), w


def gen_keys(cfg: int, req: int, ctx: int, lowrank: bool):
    """MXFP4 keys of one request in logical position order: ([ctx,64], [ctx,4])."""
    if lowrank:
        r = _rng(cfg, req, _T_LOWRANK)
        bm = r.standard_normal((8, DIM), dtype=np.float32) * np.float32(np.sqrt(1.0 / 8.0))
        npages = -(-ctx // PAGE)
        gamma = r.lognormal(0.0, 0.5, size=npages).astype(np.float32)

        def tr(x, s):
            n = x.shape[0]
            a = _rng(cfg, req, _T_LOWRANK, 1 + s // 4096).standard_normal((n, 8), dtype=np.float32)
            pg = gamma[(np.arange(s, s + n) // PAGE)]
            return encode_mxfp4(x + (a * pg[:, None]) @ bm)
    else:
        def tr(x, _s):
            return encode_mxfp4(x)
    parts = _normal_chunks((cfg, req, _T_K), ctx, (DIM,), 4096, tr)
    kv = np.concatenate([p[0] for p in parts]) if parts else np.zeros((0, VAL_BYTES), np.uint8)
    ks = np.concatenate([p[1] for p in parts]) if parts else np.zeros((0, SCALE_BYTES), np.uint8)
    return kv, ks


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

@dataclass
class Layer:
    qv: np.ndarray      # u8 [R, H, 64]
    qs: np.ndarray      # u8 [R, H, 4]
    w: np.ndarray       # f32 [R, H]


@dataclass
class Workload:
    name: str
    cfg: int
    heads: int
    kb: int                       # candidate_topk_blocks
    kc: int                       # consumer top-k
    ctx: np.ndarray               # i32 [num_req] compressed context per request
    rows_per_req: np.ndarray      # i32 [num_req]
    req: np.ndarray               # i32 [R] request of each row
    lens: np.ndarray              # i32 [R] compress_len of each row
    req_start: np.ndarray         # i32 [R] first flattened-K column of the row's request
    pool: np.ndarray              # u8 [num_pages, PAGE_BYTES]
    page_table: np.ndarray        # i32 [num_req, max_pages], -1 where unused
    layers: list[Layer] = field(default_factory=list)   # [source, consumer 1, ...]
    tail_len: np.ndarray | None = None                   # i32 [num_req]
    keys_logical: list | None = None                     # per request (kv, ks), kept when asked

    @property
    def rows(self) -> int:
        return int(self.req.shape[0])

    @property
    def num_req(self) -> int:
        return int(self.ctx.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.pool.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def ld(self) -> int:
        """Dense-score row stride: the longest row rounded up to 8 (32-byte blocks)."""
        m = int(self.lens.max()) if self.rows else 0
        return max(8, (m + 7) // 8 * 8)

    @property
    def ldk(self) -> int:
        """Block-key row stride: blocks of the longest row."""
        return max(1, self.ld // 8)


def _assemble(name, cfg, heads, kb, kc, ctx, rows_per_req, lens_per_req, lowrank,
              n_layers, dup_frac=0.0, tail=None, keep_keys=False) -> Workload:
    ctx = np.asarray(ctx, dtype=np.int64)
    nreq = len(ctx)
    npages_req = (ctx + PAGE - 1) // PAGE
    total_pages = int(npages_req.sum())
    perm = _rng(cfg, 0, _T_PERM).permutation(total_pages).astype(np.int32)
    max_pages = int(max(1, npages_req.max() if nreq else 1))
    page_table = np.full((max(nreq, 1), max_pages), -1, dtype=np.int32)
    pool = np.zeros((max(total_pages, 1), PAGE_BYTES), dtype=np.uint8)
    keys_logical = [] if keep_keys else None
    off = 0
    for j in range(nreq):
        n = int(npages_req[j])
        page_table[j, :n] = perm[off:off + n]
        off += n
        kv, ks = gen_keys(cfg, j, int(ctx[j]), lowrank)
        if dup_frac > 0 and ctx[j] > 1:
            r = _rng(cfg, j, _T_DUP)
            nd = max(1, int(round(dup_frac * ctx[j])))
            dst = r.choice(int(ctx[j]), size=nd, replace=False)
            src = r.integers(0, int(ctx[j]), size=nd)
            src = np.where(src == dst, (src + 1) % ctx[j], src)
            kv[dst] = kv[src]
            ks[dst] = ks[src]
        pad = n * PAGE - int(ctx[j])
        if pad:
            kv = np.concatenate([kv, np.zeros((pad, VAL_BYTES), np.uint8)])
            ks = np.concatenate([ks, np.full((pad, SCALE_BYTES), 127, np.uint8)])
        pages = page_table[j, :n]
        pool[pages, :PAGE * VAL_BYTES] = kv.reshape(n, PAGE * VAL_BYTES)
        pool[pages, PAGE * VAL_BYTES:] = ks.reshape(n, PAGE * SCALE_BYTES)
        if keep_keys:
            keys_logical.append((kv[:int(ctx[j])], ks[:int(ctx[j])]))
    req = np.concatenate([np.full(int(n), j, np.int32) for j, n in enumerate(rows_per_req)]) \
        if nreq else np.zeros(0, np.int32)
    lens = np.concatenate([np.asarray(l, np.int32) for l in lens_per_req]) if nreq else np.zeros(0, np.int32)
    starts = np.concatenate([[0], np.cumsum(ctx)[:-1]]).astype(np.int64)
    req_start = starts[req].astype(np.int32) if len(req) else np.zeros(0, np.int32)
    R = len(req)
    layers = [Layer(*gen_query(cfg, 1 + i, R, heads)) for i in range(n_layers)]
    wl = Workload(name=name, cfg=cfg, heads=heads, kb=kb, kc=kc, ctx=ctx.astype(np.int32),
                  rows_per_req=np.asarray(rows_per_req, np.int32), req=req, lens=lens,
                  req_start=req_start, pool=pool, page_table=page_table, layers=layers,
                  tail_len=None if tail is None else np.asarray(tail, np.int32),
                  keys_logical=keys_logical)
    assert (wl.lens <= wl.ctx[wl.req]).all()
    return wl


def tiny(keep_keys: bool = False) -> Workload:
    """1 request, 64 rows at positions 960..1023 of a 1024-position context, H=8."""
    R, C = 64, 1024
    return _assemble("tiny", 1, 8, 16, 32, [C], [R], [C - R + np.arange(R)], False, 3,
                     keep_keys=keep_keys)


def decode(keep_keys: bool = False, n_consumers: int = 4) -> Workload:
    """64 requests x 1 row, context ~ U{4096..65536}, H=64."""
    ctx = _rng(2, 0, _T_LEN).integers(4096, 65536, size=64, endpoint=True)
    return _assemble("decode", 2, 64, 2048, 512, ctx, [1] * 64, [[c] for c in ctx], False,
                     1 + n_consumers, keep_keys=keep_keys)


def decode_mtp(keep_keys: bool = False, n_consumers: int = 4, next_n: int = 2) -> Workload:
    """Decode with multi-token prediction / verification: 64 requests x next_n
    rows, the rows of a request seeing contexts C - next_n + 1 .. C (C - 1 and C
    for next_n = 2), C ~ U{4096..65536}, H=64."""
    ctx = _rng(6, 0, _T_LEN).integers(4096, 65536, size=64, endpoint=True)
    lens = [c - next_n + 1 + np.arange(next_n) for c in ctx]
    return _assemble("decode_mtp", 6, 64, 2048, 512, ctx, [next_n] * 64, lens, False,
                     1 + n_consumers, keep_keys=keep_keys)


def prefill(keep_keys: bool = False, n_consumers: int = 4) -> Workload:
    """1 request, 2048 rows ending at context 65536 (len = 63488 + i), H=64."""
    R, C = 2048, 65536
    return _assemble("prefill", 3, 64, 2048, 512, [C], [R], [C - R + np.arange(R)], False,
                     1 + n_consumers, keep_keys=keep_keys)


def long_chunk(keep_keys: bool = False, n_consumers: int = 4, rows: int = 16384) -> Workload:
    """16384 rows at 262144-position context (len = 245760 + i), low-rank K, H=64."""
    C = 262144
    return _assemble("long", 4, 64, 2048, 512, [C], [rows], [C - rows + np.arange(rows)], True,
                     1 + n_consumers, keep_keys=keep_keys)


def mixed(keep_keys: bool = False, n_consumers: int = 4, decode_rows: int = 256,
          max_decode_ctx: int = 262144) -> Workload:
    """8 prefill requests (rows log-U[128,4096], context log-U[8192,131072]) plus
    decode rows (context U[1024, max_decode_ctx]); 1% duplicated K records;
    tail of min(64, n) rows per request."""
    r = _rng(5, 0, _T_LEN)
    n_pre = np.exp(r.uniform(np.log(128), np.log(4096), size=8)).astype(np.int64)
    c_pre = np.exp(r.uniform(np.log(8192), np.log(131072), size=8)).astype(np.int64)
    c_pre = np.maximum(c_pre, n_pre)
    c_dec = r.integers(1024, max_decode_ctx, size=decode_rows, endpoint=True)
    ctx = np.concatenate([c_pre, c_dec])
    rows_per_req = np.concatenate([n_pre, np.ones(decode_rows, np.int64)])
    lens = [c - n + np.arange(n) for c, n in zip(ctx, rows_per_req)]
    tail = np.minimum(64, rows_per_req)
    return _assemble("mixed", 5, 64, 2048, 512, ctx, rows_per_req, lens, False, 1 + n_consumers,
                     dup_frac=0.01, tail=tail, keep_keys=keep_keys)


def custom(name: str, cfg: int, heads: int, kb: int, kc: int, ctx, rows_per_req, lens_per_req,
           n_layers: int = 2, lowrank: bool = False, dup_frac: float = 0.0, tail=None,
           keep_keys: bool = False) -> Workload:
    """Small hand-shaped workloads for edge cases (empty rows, keep-all rows, ...)."""
    return _assemble(name, cfg, heads, kb, kc, ctx, rows_per_req, lens_per_req, lowrank,
                     n_layers, dup_frac=dup_frac, tail=tail, keep_keys=keep_keys)


CONFIGS = {"tiny": tiny, "decode": decode, "decode_mtp": decode_mtp, "prefill": prefill,
           "long": long_chunk, "mixed": mixed}


def select_rows(wl: Workload, idx) -> Workload:
    """The workload restricted to rows `idx` (same pool, page table and requests;
    each layer's query rows sliced), e.g. to score rows apart from their batch."""
    idx = np.asarray(idx, dtype=np.int64)
    layers = [Layer(L.qv[idx], L.qs[idx], L.w[idx]) for L in wl.layers]
    rows_per_req = np.bincount(wl.req[idx], minlength=wl.num_req).astype(np.int32)
    return Workload(name=wl.name + "_rows", cfg=wl.cfg, heads=wl.heads, kb=wl.kb, kc=wl.kc,
                    ctx=wl.ctx, rows_per_req=rows_per_req, req=wl.req[idx], lens=wl.lens[idx],
                    req_start=wl.req_start[idx], pool=wl.pool, page_table=wl.page_table,
                    layers=layers, tail_len=None)


# ---------------------------------------------------------------------------
# synthetic score / key matrices for the selection steps alone
# ---------------------------------------------------------------------------

def random_matrix(seed: int, rows: int, width: int, ties: bool = True,
                  specials: bool = True) -> np.ndarray:
    """float32 [rows, width] ~ N(0, 8^2) with, optionally, exact ties (values
    snapped to a coarse grid on a third of the rows) and +-0 / +-inf entries."""
    r = _rng(900, seed)
    x = (r.standard_normal((rows, width), dtype=np.float32) * np.float32(8.0)).astype(np.float32)
    if ties and rows:
        sel = r.random(rows) < 0.34
        x[sel] = np.round(x[sel] * 2.0) / 2.0
    if specials and rows and width:
        n = max(1, rows * width // 500)
        ri, ci = r.integers(0, rows, n), r.integers(0, width, n)
        vals = np.array([0.0, -0.0, np.inf, -np.inf], np.float32)
        x[ri, ci] = vals[r.integers(0, 4, n)]
    return x


def crowded_rows(seed: int, kind: str, rows: int, width: int, k: int, cluster: int = 0) -> np.ndarray:
    """float32 [rows, width] whose k-th largest value sits where many values
    crowd together, positions shuffled per row.  kind:
      'constant'  every value 3.0;
      'zeros'     +0 and -0 only;
      'cluster'   `cluster` values within a few thousand ulps above 1.0, in
                  runs of three equal values, above ~N(-5, 0.3^2) filler, with
                  two values at +1e30 and two at -1e30 widening the row's span;
      'neginf'    k // 2 finite values ~ N(0, 8^2), the rest -inf;
      'posinf'    k + k // 2 values +inf, the rest ~ N(0, 8^2);
      'posinf_many'  a quarter of the row +inf, the rest ~ N(0, 8^2);
      'subnormal' multiples -300..300 of the smallest subnormal 2^-149
                  (zeros of both signs among them), so the threshold and
                  its neighbours are subnormal."""
    r = _rng(902, seed)
    x = np.empty((rows, width), np.float32)
    for i in range(rows):
        if kind == "constant":
            v = np.full(width, 3.0, np.float32)
        elif kind == "zeros":
            v = np.where(r.random(width) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        elif kind == "cluster":
            c = min(cluster, width - 4)
            ulp = np.float32(np.spacing(np.float32(1.0)))
            clus = np.float32(1.0) + ulp * (np.arange(c) // 3).astype(np.float32)
            fill = (r.standard_normal(width - 4 - c) * 0.3 - 5.0).astype(np.float32)
            v = np.concatenate([np.float32([1e30, 1e30, -1e30, -1e30]), clus, fill]).astype(np.float32)
        elif kind == "neginf":
            v = np.full(width, -np.inf, np.float32)
            nf = min(k // 2, width)
            v[:nf] = r.standard_normal(nf) * 8.0
        elif kind == "subnormal":
            m = r.integers(-300, 301, width)
            v = (m.astype(np.float64) * 2.0 ** -149).astype(np.float32)
            v[(m == 0) & (r.random(width) < 0.5)] = np.float32(-0.0)
        elif kind in ("posinf", "posinf_many"):
            v = (r.standard_normal(width) * 8.0).astype(np.float32)
            ni = min(width, k + k // 2 if kind == "posinf" else width // 4)
            v[:ni] = np.inf
        else:
            raise ValueError(kind)
        x[i] = v[r.permutation(width)]
    return x


def to_bf16(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Input construction for bf16 operands: float32 -> (bf16 bit patterns as
    uint16, the same values as float32), nearest with ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return bits, (bits.astype(np.uint32) << 16).view(np.float32)


def random_lengths(seed: int, rows: int, lo: int, hi: int, extra=()) -> np.ndarray:
    """int32 [rows] uniform in [lo, hi], the given values placed first."""
    r = _rng(901, seed)
    out = r.integers(lo, hi, size=rows, endpoint=True).astype(np.int32)
    for i, v in enumerate(extra[:rows]):
        out[i] = v
    return out


# ---------------------------------------------------------------------------
# inputs of the query RoPE + quantisation step
# ---------------------------------------------------------------------------

@dataclass
class QInputs:
    """Projected queries before RoPE/quantisation and what the step reads."""
    q: np.ndarray          # uint16 [rows, heads, 128]: bf16 bit patterns
    positions: np.ndarray  # int32 [rows]
    cos_sin: np.ndarray    # float32 [max_pos, 64]: cos in [0, 32), sin in [32, 64)
    w: np.ndarray          # float32 [rows, heads]


def rope_table(max_pos: int, base: float = 10000.0) -> np.ndarray:
    """The rotary table over 64 rotated dimensions: angle(p, i) = p * base^(-i/32)."""
    inv = base ** (-np.arange(32, dtype=np.float64) / 32.0)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def q_inputs(seed: int, rows: int, heads: int, max_pos: int = 262144,
             specials: bool = True) -> QInputs:
    """Seeded bf16 queries ~ N(0, 1) times a per-head gain (log-normal), random
    positions in [0, max_pos), the rotary table, fp32 weights ~ N(0, 1).  With
    `specials`, some heads are all zero and some hold values that round to
    e2m1 ties."""
    r = _rng(902, seed)
    gain = np.exp(r.normal(0.0, 1.0, size=(rows, heads, 1))).astype(np.float32)
    x = (r.standard_normal((rows, heads, DIM), dtype=np.float32) * gain).astype(np.float32)
    if specials and rows * heads >= 4:
        flat = x.reshape(-1, DIM)
        flat[0] = 0.0
        # exact grid values and midpoints of a group whose scale is 1 (amax 6)
        ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], dtype=np.float32)
        flat[1, 64:96] = np.resize(np.concatenate([ties, -ties]), 32)
        flat[2, :] = np.float32(1e-30)
    u = x.view(np.uint32)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)   # to bf16 (nearest even)
    pos = r.integers(0, max_pos, size=rows).astype(np.int32)
    if rows:
        pos[0] = 0
    w = r.standard_normal((rows, heads), dtype=np.float32)
    return QInputs(bits, pos, rope_table(max_pos), w)
