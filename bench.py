"""Benchmark: one 16384-row prefill chunk at 262144-position context through the
two-level candidate indexer (source layer + 4 consumer layers) on one MI355X.

A step is one whole chunk: idx_score_dense, then on a side stream
idx_amax8_varlen / idx_topk_blocks / idx_expand_candidates, the source's own
top-512, and for each of the 4 consumers idx_score_sparse_paged +
idx_topk_rows.  Inputs are resident in HBM before the timed region.

Prints one JSON line: query-rows/s and ms per chunk, the dense score kernel
against the fp4 MFMA peak (HIP events on its stream), per-kernel times, and
the CPU oracle timed on a bounded sample of the same chunk's rows.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "indexer query-rows/s + ms per 16K-row chunk at 262K context (source+4 consumers)"
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense MXFP4 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


class Recorder:
    """Records a torch event on the current stream at each named mark."""

    def __init__(self):
        import torch
        self.torch = torch
        self.events = {}

    def mark(self, name):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record(self.torch.cuda.current_stream())
        self.events.setdefault(name, []).append(ev)

    def spans(self, a, b):
        ea, eb = self.events.get(a, []), self.events.get(b, [])
        return [x.elapsed_time(y) for x, y in zip(ea, eb)]


def workload(name):
    import workloads
    if name == "long":
        return workloads.long_chunk(), "long: 16384 rows x 262144 context (len 245760+i), H=64, kb=2048, 4 consumers, top-512"
    if name == "prefill":
        return workloads.prefill(), "prefill: 2048 rows x 65536 context (len 63488+i), H=64, kb=2048, 4 consumers, top-512"
    if name == "decode":
        return workloads.decode(), "decode: 64 requests x 1 row, context U[4096,65536], H=64, kb=2048, 4 consumers, top-512"
    if name == "decode_mtp":
        return workloads.decode_mtp(), "decode MTP: 64 requests x 2 rows (len C-1, C), C U[4096,65536], H=64, kb=2048, 4 consumers, top-512"
    if name == "tiny":
        return workloads.tiny(), "tiny: 64 rows x 1024 context, H=8, kb=16, 2 consumers, top-32"
    if name == "mixed":
        wl = workloads.mixed()
        return wl, (f"mixed: 8 prefill requests (rows log-U[128,4096], context log-U[8192,131072]) + "
                    f"256 decode rows (context U[1024,262144]), {wl.rows} rows, H=64, kb=2048, 4 consumers, "
                    f"top-512")
    raise SystemExit(f"unknown config {name}")


def algorithmic_work(wl, score_bytes=4):
    """Per-launch algorithmic flops / bytes of each kernel for this workload."""
    import numpy as np
    lens = wl.lens.astype(np.int64)
    H = wl.heads
    nblk = (lens + 7) // 8
    keyed = nblk > wl.kb
    n_kept = np.minimum(nblk, wl.kb)
    valid = np.where(lens > 0, 8 * n_kept - (8 * nblk - lens), 0)
    flop_per_logit = 2 * H * 128
    return {
        "dense_flops": float(flop_per_logit * lens.sum()),
        "dense_store_bytes": float(4 * lens.sum()),
        "amax8_bytes": float((32 * (nblk[keyed] - 1) + 4 * nblk[keyed]).sum()),
        "topk_blocks_bytes": float((4 * nblk[keyed]).sum() + 4 * wl.kb * wl.rows),
        "sparse_flops": float(flop_per_logit * valid.sum()),
        "sparse_gather_bytes": float(68 * valid.sum()),
        "topk_rows_bytes": float(score_bytes * valid.sum() + 4 * wl.kc * wl.rows),
    }


def measured_traffic(config):
    """HBM bytes per dense-score launch from the committed counter summary, or None
    when the summary is for another workload or the kernel sources have changed."""
    import hashlib
    if config != "long":
        return None
    path = os.path.join(ROOT, "profiles", "score_dense_long_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", " ", "#")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in ("score_dense.hip", "score_common.h", "idx_internal.h"):
        h.update(open(os.path.join(ROOT, "two_level_top_amd", "csrc", f), "rb").read())
    if fields.get("kernel_source_sha256") != h.hexdigest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_q_rope_quant(rows, heads, reps=20):
    """The step before the score calls (RoPE + MXFP4 quantisation of one layer's
    queries) at the chunk's shape, timed apart from the chunk: device-side random
    bf16 queries, the rotary table of 262144 positions."""
    import numpy as np
    import torch
    import two_level_top_amd as t
    import workloads
    g = torch.Generator(device="cuda").manual_seed(1)
    q = torch.randn((rows, heads, 128), device="cuda", generator=g).to(torch.bfloat16).view(torch.int16)
    pos = torch.randint(0, 262144, (rows,), device="cuda", generator=g, dtype=torch.int32)
    cs = torch.from_numpy(workloads.rope_table(262144)).cuda()
    w = torch.randn((rows, heads), device="cuda", generator=g)
    vals = torch.empty((rows, heads, 64), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, heads, 4), dtype=torch.uint8, device="cuda")
    w_out = torch.empty((rows, heads), dtype=torch.float32, device="cuda")
    run = lambda: t.idx_q_rope_quant(q, pos, cs, w, True, 128 ** -0.5, heads ** -0.5, vals, scales, w_out)
    run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    nbytes = rows * heads * (256 + 4 + 64 + 4 + 4)   # bf16 query + w in; codes, scales, w out
    return {"ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "note": "query RoPE + MXFP4 quantisation before the chunk, timed apart from it"}


def time_amax8(ch, bytes_per_call, reps=5):
    """idx_amax8_varlen alone on the chunk's source score matrix (the chunk takes
    the block keys from the fused dense pass and never writes the matrix), timed
    apart from the chunk: the matrix is scored into a buffer of its own first."""
    import torch
    import two_level_top_amd as t
    S = ch.S
    if S is None:
        S = torch.empty((ch.R, ch.ld), dtype=torch.float32, device="cuda")
        t.idx_score_dense(ch.queries[0], ch.kp, ch.rows, S, ws=ch.ws)
    keys = torch.empty_like(ch.keys)
    run = lambda: t.idx_amax8_varlen(S, ch.rows.len, keys, skip_le_blocks=ch.kb)
    run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    gbs = bytes_per_call / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "note": "the unfused block-key pass over the chunk's S, timed apart from the chunk"}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, n_rows):
    """The oracle, as it stands, on n_rows evenly spaced rows of the same chunk."""
    import ctypes
    import numpy as np
    import oracle
    rows = np.unique(np.linspace(0, wl.rows - 1, n_rows).astype(np.int64))
    oracle._load()
    t0 = time.perf_counter()
    oracle.run_chunk(wl, row_ids=rows)
    dt = time.perf_counter() - t0
    try:   # the OpenMP runtime the oracle's C code runs on reports its thread count
        cores = int(ctypes.CDLL("libgomp.so.1").omp_get_max_threads())
    except OSError:
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(len(rows) / dt, 3), "unit": "query-rows/s", "cores": cores,
            "kind": "oracle", "cpu": _cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{len(rows)} evenly spaced rows of the same chunk, source + "
                      f"{len(wl.layers) - 1} consumers (all steps), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="long", choices=["long", "prefill", "decode", "decode_mtp", "tiny", "mixed"])
    ap.add_argument("--cpu-rows", type=int, default=256,
                    help="rows of the CPU oracle sample (0 = skip the CPU baseline)")
    ap.add_argument("--graph", choices=["auto", "on", "off"], default="auto",
                    help="time replays of the step captured as one HIP graph (auto: on for "
                         "tables of at most 256 rows, whose steps are bound by per-call host cost)")
    ap.add_argument("--consumer-bf16", action="store_true",
                    help="the bf16 consumer-score variant (scores and their top-k in bf16)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB (the known-size "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the indexer path is built and timed on a single "
              "MI355X (rows shard across GPUs with no collective inside the path); "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from two_level_top_amd.chunk import Chunk

    torch.cuda.set_device(0)
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n * 4}))
        return
    wl, desc = workload(args.config)
    print(f"[bench] workload ready: {desc}", file=sys.stderr, flush=True)
    ch = Chunk(wl, consumer_bf16=args.consumer_bf16)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        ch.run()
    torch.cuda.synchronize()
    print(f"[bench] {args.warmup} warmup steps done", file=sys.stderr, flush=True)

    use_graph = args.graph == "on" or (args.graph == "auto" and wl.rows <= Chunk.OVERLAP_MAX_ROWS)
    if use_graph:
        ch.capture()
        for i in range(args.warmup):
            ch.replay()
    step = ch.replay if use_graph else ch.run
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1000.0 / args.steps
    print(f"[bench] {args.steps} timed steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)

    # per-call times from events at each call's start and end, in extra steps
    # after the timed ones (recording ~25 events per step costs host time that
    # would otherwise be charged to small configs' steps).  That pass runs the
    # source's own top-k in line, not beside the first consumer as the timed
    # steps do, so that each call's events time that call alone.
    rec = Recorder()
    ch.recorder = rec
    side = ch.source_side
    ch.source_side = False
    for i in range(min(args.steps, 5)):
        ch.run()
    torch.cuda.synchronize()
    ch.recorder = None
    ch.source_side = side

    work = algorithmic_work(wl, score_bytes=2 if args.consumer_bf16 else 4)
    ncons = len(ch.cons_top)

    def avg(a, b):
        s = rec.spans(a, b)
        return float(np.mean(s)) if s else float("nan")

    t_fold = avg("fold<", "fold>") if ch.prefold else float("nan")
    t_dense = avg("dense<", "dense>")
    t_amax = avg("amax8<", "amax8>")
    t_tkb = avg("topk_blocks<", "topk_blocks>")
    t_exp = avg("topk_blocks>", "expand>")
    t_src = avg("source_topk<", "source_topk>")
    t_sp = [avg(f"sparse{i}<", f"sparse{i}>") for i in range(ncons)]
    t_tr = [avg(f"topk_rows{i}<", f"topk_rows{i}>") for i in range(ncons)]
    dense_tflops = work["dense_flops"] / (t_dense * 1e-3) / 1e12
    dense_name = ("score_dense_keys (keys only)" if ch.rescore else "score_dense_keys") \
        if ch.fused_keys else "score_dense"
    kernels = {
        **({"fold_queries": {"ms": round(t_fold, 4),
                             "note": "the source layer's folded query (the consumers' are folded in "
                                     "one launch beside the block select)"}}
           if ch.prefold else {}),
        dense_name: {"ms": round(t_dense, 4), "TFLOP/s": round(dense_tflops, 1),
                     "frac_fp4_peak": round(dense_tflops / PEAK_FP4_TFLOPS, 4)},
        **({} if ch.fused_keys else {"amax8_varlen": {
            "ms": round(t_amax, 4), "GB/s": round(work["amax8_bytes"] / (t_amax * 1e-3) / 1e9, 1)}}),
        "topk_blocks": {"ms": round(t_tkb, 4),
                        "GB/s": round(work["topk_blocks_bytes"] / (t_tkb * 1e-3) / 1e9, 1)},
        "expand_candidates": {"ms": round(t_exp, 4)},
        ("source_rescore_topk" if ch.rescore else "source_topk_rows"): {
            "ms": round(t_src, 4),
            **({"note": "the source query scored at its top-(k+1) candidate blocks, then the "
                        "block-mapped top-k; on the side stream beside the first consumer's "
                        "scores (events on that stream include the overlap)"} if ch.rescore else
               {"note": "timed in line; the timed steps run it on the side stream beside the "
                        "first consumer"} if ch.source_side and not ch.overlap else {})},
        "score_sparse_paged": {"ms": round(float(np.mean(t_sp)), 4),
                               "TFLOP/s": round(work["sparse_flops"] / (np.mean(t_sp) * 1e-3) / 1e12, 1),
                               "gather GB/s": round(work["sparse_gather_bytes"] / (np.mean(t_sp) * 1e-3) / 1e9, 1)},
        "consumer_topk_rows": {"ms": round(float(np.mean(t_tr)), 4),
                               "GB/s": round(work["topk_rows_bytes"] / (np.mean(t_tr) * 1e-3) / 1e9, 1)},
    }
    for name in ("topk_blocks", "consumer_topk_rows"):
        kernels[name]["frac_hbm_peak"] = round(kernels[name]["GB/s"] / PEAK_HBM_GBS, 4)
    if ch.fused_keys and wl.rows > Chunk.OVERLAP_MAX_ROWS:
        kernels["amax8_varlen"] = time_amax8(ch, work["amax8_bytes"])
    kernels["q_rope_quant"] = time_q_rope_quant(wl.rows, wl.heads)
    out = {
        "metric": METRIC,
        "value": round(wl.rows / (ms * 1e-3), 1),
        "unit": "query-rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": desc, "rows": wl.rows, "heads": wl.heads, "kb": wl.kb,
                   "topk": wl.kc, "consumers": ncons,
                   "consumer_scores": "bf16" if args.consumer_bf16 else "fp32",
                   "step": "one HIP graph replay" if use_graph else "eager calls"},
        "roofline": {"bound": "mfma", "kernel": dense_name,
                     "achieved": round(dense_tflops, 2), "peak": PEAK_FP4_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(dense_tflops / PEAK_FP4_TFLOPS, 4),
                     "traffic": measured_traffic(args.config)},
        "kernels": kernels,
    }
    if args.cpu_rows > 0:
        print(f"[bench] timing the CPU oracle on {args.cpu_rows} rows", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_rows)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
