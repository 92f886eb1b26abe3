"""Benchmark of the routed-MoE block on one MI355X.

Workload: the b=16 decode/verify step (H=4096, P=2048, I=1024, E=64,
top_k=4, sigmoid scoring, MXFP4 experts), synthetic seeded inputs.  One step
is one mb_moe_block call (router, routing, pooler, experts, tail, unpooler,
boundary) on inputs already resident in HBM.  The steps rotate over several
independently drawn weight sets (about 1 GB in total, four times the 256 MB
Infinity Cache), so every step streams its weights from HBM, as the 60
distinct layers of a decode step do.

Prints one JSON line: rows/s (value), microseconds per block, the achieved
algorithmic HBM bandwidth against the 8 TB/s peak (roofline), and the CPU
oracle's rate on a bounded sample of the same workload (cpu_baseline).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-block rows/s + achieved HBM GB/s (% of peak) at b=16 decode, 1 MI355X"
HBM_PEAK_GBS = 8000.0
WEIGHT_SEEDS = (1, 1001, 2001, 3001)


def algorithmic_bytes(d, n_active: int, norm_weights=(False, False, False)) -> int:
    """Bytes the block must move: the used experts' MXFP4 w13/w2 and E8M0
    scales, router weight and bias, pooler and unpooler, norm and gate
    vectors, and the block's inputs and outputs (x, stream read and write,
    x_next, ids and weights).  Intermediates that can stay on chip are not
    counted."""
    b, H, P, I, E, k = d.rows, d.hidden, d.pooled, d.inter, d.experts, d.top_k
    expert = 2 * I * P // 2 + 2 * I * P // 32 + P * I // 2 + P * I // 32
    pre, pff, win = norm_weights
    return (n_active * expert + E * H * 4 + E * 4 + 2 * P * H * 2 + P * 2 * (1 + pre)
            + H * 2 * (1 + pff + win) + b * H * 2 + 2 * b * H * 4 + b * H * 2 + b * k * 8)


# Sources whose change invalidates a stored traffic measurement of the block
# kernel (its code and its launch configuration).
KERNEL_SOURCES = ("block.hip", "block_w4a4.hip", "block_qkv.hip", "block_w4a4_qkv.hip", "block_many.hip", "api.hip", "pack.hip", "mb_block.h", "mb_device.h", "mb_sync.h", "mb_internal.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "block_kernel_c1_traffic.txt")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "routed_expert_layer_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per launch of the block kernel from the committed counter
    summary, if it was taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(line.split(":", 1) for line in fh if ":" in line)
        if kv.get("kernel_source_sha256", "").strip() != kernel_source_hash():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(blk, seconds: float, act_quant: bool = False) -> dict:
    import numpy as np  # noqa: F401

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the affinity
        threads = len(os.sched_getaffinity(0))
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.block(blk, act_quant=act_quant)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return {"value": round(blk.dims.rows * n / el, 3), "unit": "rows/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n} full b={blk.dims.rows} decode blocks (weight set 0) through the numpy "
                      f"fp64 oracle, {el:.1f} s; cores = its BLAS thread pool",
            "cpu_model": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0))}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def percentiles(us) -> dict:
    import numpy as np

    a = np.asarray(us, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 2), "p50": round(float(np.percentile(a, 50)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


def per_launch_us(torch, fn, n: int) -> list:
    """Durations of n launches one after another on the current stream, from
    an event recorded between each two (the queue stays full, so each gap is
    one launch's time on the device)."""
    cur = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(cur)
    for i in range(n):
        fn(i)
        ev[i + 1].record(cur)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n)]


# The block kernel's timeline slots (mb_block_taps.timeline): what each
# workgroup stamps, in microseconds from the launch's first workgroup start.
TIMELINE_SLOTS = {
    0: "start", 1: "first router task", 2: "first route task", 3: "first pool task",
    22: "router task done", 23: "router products summed", 12: "route task: logits seen",
    14: "route task: rows routed", 7: "pool task done", 13: "routes seen", 5: "routing state ready",
    6: "units start", 20: "wave 0's up units done", 11: "units done", 8: "first finalize task",
    19: "finalize: experts' down units seen", 21: "finalize done", 9: "first unpool task",
    16: "unpool task done", 10: "first boundary task", 17: "boundary: unpooler seen",
    18: "boundary done", 15: "end"}
# The steps after the experts, in order, for the per-launch critical chain.
TIMELINE_CHAIN = (11, 19, 21, 16, 17, 18, 15)


def timeline(launches: int, c3_rows: int = 0) -> int:
    """Per-phase breakdown of the headline block from the kernel's own
    timeline tap: the four c1 weight sets rotated as in the benchmark (or,
    with c3_rows, two weight sets of the row-bucket sweep at that many rows,
    uniform routing), warm-up, then `launches` traced launches (each after an
    untraced one).  Prints,
    per slot, how many workgroups stamped it and the p10 / p50 / p90 / max of
    their stamps over all traced launches, then the mean over launches of the
    latest and the median stamp of each step after the experts."""
    import numpy as np
    import torch

    import routed_expert_layer_amd as rel
    import synth
    from synth.device import dims_kwargs, upload, upload_weights

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if c3_rows:
        blocks = [synth.make_c3_block(None, seed=s).rows(c3_rows) for s in (3, 1003)]
    else:
        blocks = [synth.make_block("c1", seed=s) for s in WEIGHT_SEEDS]
    d = blocks[0].dims
    wt0, x, stream = upload(blocks[0], dev)
    tensors = [wt0] + [upload_weights(b, dev) for b in blocks[1:]]
    dims = rel.make_dims(**dims_kwargs(d))
    weights = [rel.make_weights(**t) for t in tensors]
    for t, w in zip(tensors, weights):
        t["experts_packed"] = rel.pack_experts(dims, w, dev)
        t["proj_packed"] = rel.pack_projections(dims, w, dev)
    weights = [rel.make_weights(**t) for t in tensors]
    ws = rel.workspace(dims, dev)
    xn = torch.zeros((d.rows, d.hidden), dtype=torch.bfloat16, device=dev)
    S = len(weights)
    for i in range(50):
        rel.mb_moe_block(dims, x, weights[i % S], stream, xn, ws)
    torch.cuda.synchronize()
    acc = {}
    chains_max, chains_p50 = [], []
    for rep_ in range(launches):
        tl = torch.zeros((1024, 32), dtype=torch.int64, device=dev)
        rel.mb_moe_block(dims, x, weights[rep_ % S], stream, xn, ws)
        rel.mb_moe_block(dims, x, weights[(rep_ + 1) % S], stream, xn, ws, taps=rel.make_taps(timeline=tl))
        torch.cuda.synchronize()
        a = tl.cpu().numpy()
        a = a[: int((a[:, 0] != 0).sum())]
        t0 = a[:, 0].min()
        per = {}
        for slot in TIMELINE_SLOTS:
            v = a[:, slot]
            v = v[v != 0]
            if v.size:
                per[slot] = (v - t0) / 100.0
                acc.setdefault(slot, []).append(per[slot])
        chains_max.append([per[s].max() if s in per else np.nan for s in TIMELINE_CHAIN])
        chains_p50.append([np.median(per[s]) if s in per else np.nan for s in TIMELINE_CHAIN])
    print(f"grid {a.shape[0]} workgroups, {launches} traced launches; us from the first workgroup start")
    print(f"{'slot':>4}  {'stamp':<36} {'wgs':>5} {'p10':>7} {'p50':>7} {'p90':>7} {'max':>7}")
    for slot in sorted(acc, key=lambda s: np.median(np.concatenate(acc[s]))):
        v = np.concatenate(acc[slot])
        print(f"{slot:>4}  {TIMELINE_SLOTS[slot]:<36} {v.size // launches:>5} {np.percentile(v, 10):7.2f} "
              f"{np.percentile(v, 50):7.2f} {np.percentile(v, 90):7.2f} {v.max():7.2f}")
    names = [TIMELINE_SLOTS[s] for s in TIMELINE_CHAIN]
    for label, ch in (("latest", chains_max), ("median", chains_p50)):
        m = np.nanmean(np.array(ch), axis=0)
        print(f"after the experts, {label} workgroup per launch (mean over launches): " +
              "; ".join(f"{n} {v:.2f}" for n, v in zip(names, m)))
    return 0


def read_probe(mib: int) -> int:
    """Time the plain HBM read kernel (libmb_readprobe.so): over one buffer
    of `mib` MiB in each variant and grid, then, in the best variant, at the
    block's own sizes, each launch reading the next of several buffers that
    together exceed the 256 MB Infinity Cache four times over; then L2-resident
    reads in the two shapes of a weight tile's wave loads.  One JSON line per
    case."""
    import ctypes

    import numpy as np
    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "routed_expert_layer_amd", "libmb_readprobe.so"))
    lib.mbp_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                             ctypes.c_void_p]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    grids = (256, 512, 1024, 2048, 4096, 8192)
    sink = torch.zeros(max(grids), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    names = ("4 words in flight, plain loads", "8 words in flight, plain loads",
             "4 words in flight, nontemporal loads", "8 words in flight, nontemporal loads")

    def run(bufs, nbytes, grid, variant, case):
        def fn(i):
            st = lib.mbp_read(bufs[i % len(bufs)].data_ptr(), nbytes, grid, variant, sink.data_ptr(), stream)
            if st != 0:
                raise RuntimeError(f"mbp_read status {st}")
        for i in range(2 * len(bufs)):
            fn(i)
        us = per_launch_us(torch, fn, max(20, 2 * len(bufs)))
        med = float(np.median(us))
        gbs = nbytes / (med * 1e-6) / 1e9
        line = {"case": case, "variant": names[variant], "workgroups": grid, "bytes": nbytes,
                "buffers_rotated": len(bufs), "us_per_launch": percentiles(us),
                "GBps_at_median": round(gbs, 1), "frac_of_8TBps": round(gbs / HBM_PEAK_GBS, 4)}
        print(json.dumps(line), flush=True)
        return line

    nbytes = mib << 20
    big = [torch.ones(nbytes // 4, dtype=torch.float32, device=dev)]
    best = None
    for variant in range(4):
        for grid in grids:
            line = run(big, nbytes, grid, variant, f"hbm read probe {mib} MiB")
            if best is None or line["GBps_at_median"] > best["GBps_at_median"]:
                best = line
    print(json.dumps({**best, "case": f"hbm read probe {mib} MiB: best"}), flush=True)
    del big
    torch.cuda.empty_cache()
    # The block's sizes: c1's algorithmic bytes (about 169 MB) and neighbours.
    for size in (64 << 20, 169095936, 512 << 20):
        n = -(-(1 << 30) // size) + 1
        bufs = [torch.ones(size // 4, dtype=torch.float32, device=dev) for _ in range(n)]
        top = None
        for variant in (2, 3):
            for grid in grids:
                line = run(bufs, size, grid, variant, f"hbm read probe {size} B")
                if top is None or line["GBps_at_median"] > top["GBps_at_median"]:
                    top = line
        print(json.dumps({**top, "case": f"hbm read probe {size} B: best"}), flush=True)
        del bufs
        torch.cuda.empty_cache()
    # The L2: a weight tile's wave loads as one contiguous kilobyte (the
    # streaming layouts) against 16 rows x 64 bytes of a row-major matrix
    # (the caller's layout), the rows as long as the pooler's (H = 7168) and
    # the unpooler's (P = 3072) bf16 rows, and one odd length.
    lib.mbp_tile_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    buf = torch.ones(16 << 18, dtype=torch.float32, device=dev)  # 16 MiB
    grid, steps = 768, 64
    for tile, nbytes, rows, row_bytes, what in (
            (0, 1 << 20, 0, 0, "contiguous 1 KB per wave load, 1 MiB buffer"),
            (0, 2 << 20, 0, 0, "contiguous 1 KB per wave load, 2 MiB buffer"),
            (1, 16 << 20, 64, 14336, "16 rows x 64 B per wave load, rows of 14336 B (64 rows)"),
            (1, 16 << 20, 64, 6144, "16 rows x 64 B per wave load, rows of 6144 B (64 rows)"),
            (1, 16 << 20, 64, 14400, "16 rows x 64 B per wave load, rows of 14400 B (64 rows)")):
        def fn(_):
            st = lib.mbp_tile_read(buf.data_ptr(), nbytes, tile, rows, row_bytes, steps, grid, sink.data_ptr(),
                                   stream)
            if st != 0:
                raise RuntimeError(f"mbp_tile_read status {st}")
        for i in range(3):
            fn(i)
        us = per_launch_us(torch, fn, 20)
        med = float(np.median(us))
        read = grid * 256 * 128 * steps
        print(json.dumps({"case": f"l2 read probe: {what}", "workgroups": grid, "bytes_read": read,
                          "us_per_launch": percentiles(us), "TBps_at_median": round(read / (med * 1e-6) / 1e12, 2)}),
              flush=True)
    return 0


def steps_around(args, rel, synth, dims_kwargs, to_tensor, prepare, n_active, timed, report_bytes):
    """The steps either side of the block at the decode size (b = 16,
    H = 4096): the attention boundary, and the next QKV projection with 32
    query and 8 KV heads of 128 (10240 rows), alone, fused into the block's
    launch and as a second launch."""
    import numpy as np
    import torch

    dev = "cuda:0"
    print("[sweep] steps around the block", file=sys.stderr, flush=True)
    b16, H16, NQ = 16, 4096, 10240
    side = synth.make_attn_side(b16, H16, NQ, 80)
    d16 = rel.make_dims(rows=b16, hidden=H16, pooled=2048, inter=1024, experts=64, top_k=4,
                        scoring="sigmoid", route_scale=2.5)
    # (A workspace sized with qkv_rows = 10240: mb_next_qkv then runs as the
    # block kernel's projection step.)
    ws16 = rel.workspace(rel.make_dims(rows=b16, hidden=H16, pooled=2048, inter=1024, experts=64, top_k=4,
                                       scoring="sigmoid", route_scale=2.5, qkv_rows=NQ), dev)
    tp = {k: to_tensor(side[k], dev) for k in ("partial", "gate", "post_attn_norm_w", "pre_ffn_norm_w", "stream")}
    xo = torch.empty((b16, H16), dtype=torch.bfloat16, device=dev)
    us = timed(lambda i: rel.mb_attn_boundary(d16, tp["partial"], tp["gate"], tp["stream"], xo,
                                              tp["post_attn_norm_w"], tp["pre_ffn_norm_w"]), 1000, 50)
    report_bytes("attention boundary b=16 H=4096", b16, us, b16 * H16 * 2 + 2 * b16 * H16 * 4 + b16 * H16 * 2 + 3 * H16 * 2)
    wq = [to_tensor(synth.make_attn_side(1, H16, NQ, 81 + i)["w_qkvg"], dev) for i in range(4)]
    q = torch.empty((b16, NQ), dtype=torch.bfloat16, device=dev)
    us = timed(lambda i: rel.mb_next_qkv(d16, xo, wq[i % 4], q, ws16), 500, 20)
    report_bytes("next qkv projection b=16 H=4096 -> 10240", b16, us, NQ * H16 * 2 + b16 * H16 * 2 + b16 * NQ * 2)
    # The c1 block followed by the next QKV projection: fused into its launch
    # (mb_dims.qkv_rows) against a second launch (mb_next_qkv); two c1 weight
    # sets and two projection weights rotated (about 0.5 GB, past the
    # Infinity Cache).
    blocks = [synth.make_block("c1", seed=s) for s in (1, 1001)]
    dq = rel.make_dims(**dims_kwargs(blocks[0].dims), qkv_rows=NQ)
    dims1, tensors1, weights1 = prepare(blocks)
    for i, t in enumerate(tensors1):
        t["next_qkv_w"] = wq[i]
    weights_q = [rel.make_weights(**t) for t in tensors1]
    x1, s1 = to_tensor(blocks[0].x, dev), to_tensor(blocks[0].stream, dev)
    wsq = rel.workspace(dq, dev)
    xn1 = torch.empty((b16, H16), dtype=torch.bfloat16, device=dev)
    tq = rel.make_taps(qkvg=q)
    bytes_block = float(np.mean([algorithmic_bytes(blocks[0].dims, n_active(dims1, x1, w, s1, wsq))
                                 for w in weights1]))
    us = timed(lambda i: rel.mb_moe_block(dims1, x1, weights1[i % 2], s1, xn1, wsq), 500, 20)
    report_bytes("c1 block alone (two weight sets)", b16, us, bytes_block)
    us = timed(lambda i: rel.mb_moe_block(dq, x1, weights_q[i % 2], s1, xn1, wsq, taps=tq), 500, 20)
    report_bytes("c1 block + next qkv 10240 fused in its launch", b16, us, bytes_block + NQ * H16 * 2 + b16 * NQ * 2)

    def two(i):
        rel.mb_moe_block(dims1, x1, weights1[i % 2], s1, xn1, wsq)
        rel.mb_next_qkv(dims1, xn1, wq[i % 2], q, wsq)

    us = timed(two, 500, 20)
    report_bytes("c1 block, then next qkv 10240 as a second launch", b16, us, bytes_block + NQ * H16 * 2 + b16 * NQ * 2)
    del wq, tp, ws16, blocks, tensors1, weights1, weights_q, wsq
    torch.cuda.empty_cache()


def sweep(args) -> int:
    """Every workload once, each on its own seeded weight sets: microseconds per
    block, rows/s and algorithmic HBM bandwidth for c0, c2 (both skew
    readings), each c3 row bucket (uniform and calibrated skew) and the
    60-layer c4 stack.  One JSON line per case on stdout."""
    import numpy as np
    import torch

    import routed_expert_layer_amd as rel
    import synth
    from synth.device import dims_kwargs, to_tensor, upload_weights

    dev = "cuda:0"
    torch.cuda.set_device(0)

    def prepare(blocks):
        dims = rel.make_dims(**dims_kwargs(blocks[0].dims), act_quant=int(args.act_quant))
        tensors = [upload_weights(b, dev) for b in blocks]
        weights = [rel.make_weights(**t) for t in tensors]
        if args.layout == "packed":
            for t, w in zip(tensors, weights):
                t["experts_packed"] = rel.pack_experts(dims, w, dev)
                t["proj_packed"] = rel.pack_projections(dims, w, dev)
            weights = [rel.make_weights(**t) for t in tensors]
        torch.cuda.synchronize()
        return dims, tensors, weights

    def n_active(dims, x, w, stream, ws):
        n = torch.zeros(1, dtype=torch.int32, device=dev)
        xn = torch.empty((x.shape[0], x.shape[1]), dtype=torch.bfloat16, device=dev)
        rel.mb_moe_block(dims, x, w, stream.clone(), xn, ws, taps=rel.make_taps(n_active=n))
        torch.cuda.synchronize()
        return int(n.item())

    def timed(fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    def report(case, d, us, actives, blocks_per_step=1, pct=None):
        b_alg = float(np.mean([algorithmic_bytes(d, a) for a in actives])) * blocks_per_step
        gbs = b_alg / (us * 1e-6) / 1e9
        line = {"case": case, "rows": d.rows, "us_per_step": round(us, 2),
                "us_per_block_percentiles": pct,
                "blocks_per_step": blocks_per_step,
                "rows_per_s": round(d.rows * blocks_per_step / (us * 1e-6), 1),
                "algorithmic_bytes_per_step": int(b_alg), "achieved_GBps": round(gbs, 1),
                "frac_of_8TBps": round(gbs / HBM_PEAK_GBS, 4), "active_experts": actives,
                "expert_layout": args.layout, "act_quant": int(args.act_quant)}
        print(json.dumps(line), flush=True)
        print(f"[sweep] {case}: {us:.1f} us/step, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}%)",
              file=sys.stderr, flush=True)

    def run_block_case(case, blocks, steps, warmup=10):
        d = blocks[0].dims
        dims, tensors, weights = prepare(blocks)
        x, stream = to_tensor(blocks[0].x, dev), to_tensor(blocks[0].stream, dev)
        ws = rel.workspace(dims, dev)
        xn = torch.empty((d.rows, d.hidden), dtype=torch.bfloat16, device=dev)
        actives = [n_active(dims, x, w, stream, ws) for w in weights]
        S = len(weights)

        def fn(i):
            rel.mb_moe_block(dims, x, weights[i % S], stream, xn, ws)

        us = timed(fn, steps, warmup)
        report(case, d, us, actives, pct=percentiles(per_launch_us(torch, fn, min(steps, 500))))

    def report_bytes(case, rows, us, b_alg):
        gbs = b_alg / (us * 1e-6) / 1e9
        line = {"case": case, "rows": rows, "us_per_step": round(us, 2), "blocks_per_step": 1,
                "rows_per_s": round(rows / (us * 1e-6), 1), "algorithmic_bytes_per_step": int(b_alg),
                "achieved_GBps": round(gbs, 1), "frac_of_8TBps": round(gbs / HBM_PEAK_GBS, 4),
                "active_experts": None, "expert_layout": None, "act_quant": None}
        print(json.dumps(line), flush=True)
        print(f"[sweep] {case}: {us:.1f} us/step, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}%)",
              file=sys.stderr, flush=True)

    cases = set(args.sweep_cases.split(","))
    if "around" in cases:
        steps_around(args, rel, synth, dims_kwargs, to_tensor, prepare, n_active, timed, report_bytes)
    if args.steps_around_only:
        return 0
    if "c0" in cases:
        print("[sweep] c0", file=sys.stderr, flush=True)
        run_block_case("c0 tiny block", [synth.make_block("c0")], 1000)
    steps = args.sweep_steps
    for skew in ("calibrated", "literal"):
        if "c2" not in cases and f"c2-{skew}" not in cases:
            continue
        print(f"[sweep] c2 {skew}: generating 2 weight sets", file=sys.stderr, flush=True)
        blocks = [synth.make_block("c2", seed=s, skew=skew) for s in (2, 1002)]
        run_block_case(f"c2 b=64 softmax, skew {skew}", blocks, steps or 200)
        del blocks
        torch.cuda.empty_cache()
    for skew in (None, "calibrated"):
        name = skew or "uniform"
        buckets = [b for b in synth.inputs.C3_BUCKETS if "c3" in cases or f"c3-{name}-{b}" in cases]
        if not buckets:
            continue
        print(f"[sweep] c3 skew={skew}: generating 2 weight sets", file=sys.stderr, flush=True)
        full = [synth.make_c3_block(skew, seed=s) for s in (3, 1003)]
        for b in buckets:
            run_block_case(f"c3 b={b} sigmoid, {name}", [f.rows(b) for f in full], steps or 200)
        del full
        torch.cuda.empty_cache()
    if "c4" not in cases:
        return 0

    # c4: the 60-layer stack, 60 distinct layer weight sets (about 54 GB of
    # experts in HBM), x_next of each layer feeding the next.  Layers are
    # drawn in threads and uploaded one by one (their caller-layout experts,
    # pooler and unpooler weights dropped once packed).
    from concurrent.futures import ThreadPoolExecutor

    n_layers = synth.inputs.C4_LAYERS
    print(f"[sweep] c4: generating and uploading {n_layers} layer weight sets", file=sys.stderr, flush=True)
    x0, s0 = synth.make_c4_stream()
    x = to_tensor(x0, dev)
    stream = to_tensor(s0, dev)
    weights, actives, dims, ws, d = [], [], None, None, None
    with ThreadPoolExecutor(4) as pool:
        futs = [pool.submit(synth.make_c4_layer, l) for l in range(n_layers)]
        for l, fu in enumerate(futs):
            blk = fu.result()
            futs[l] = None
            d = blk.dims
            dims_l, tensors, ws_l = prepare([blk])
            if args.layout == "packed":
                for n in ("w13", "w13_scale", "w2", "w2_scale", "pool_w", "unpool_w"):
                    tensors[0].pop(n, None)
                ws_l = [rel.make_weights(**tensors[0])]
            if dims is None:
                dims, ws = dims_l, rel.workspace(dims_l, dev)
            weights.append((tensors[0], ws_l[0]))
            actives.append(n_active(dims, x, ws_l[0], stream, ws))
            del blk
    xs = [x.clone(), torch.empty_like(x)]

    def layer(i):
        rel.mb_moe_block(dims, xs[i % 2], weights[i % n_layers][1], stream, xs[(i + 1) % 2], ws)

    def stack(_):
        for i in range(n_layers):
            layer(i)

    us = timed(stack, 4, 1)
    pct = percentiles(per_launch_us(torch, layer, 4 * n_layers))
    report(f"c4 {n_layers}-layer stack b=32 (per stack, {n_layers} distinct layers)", d, us, actives,
           blocks_per_step=n_layers, pct=pct)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--sets", type=int, default=len(WEIGHT_SEEDS))
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="first run one plain elementwise copy of MB MiB (reads and writes MB MiB), "
                         "the reference kernel for scaling the HBM byte counters")
    ap.add_argument("--layout", choices=("packed", "caller"), default="packed",
                    help="expert, pooler and unpooler weights streamed from mb_pack_experts' and "
                         "mb_pack_projections' layouts (prepared once per weight set, outside the timed "
                         "region) or from the caller's layout")
    ap.add_argument("--act-quant", action="store_true",
                    help="the W4A4 variant: the experts' activations quantized to MXFP4 (needs the "
                         "packed layout); not the headline line")
    ap.add_argument("--print-source-hash", action="store_true")
    ap.add_argument("--timeline", type=int, default=0, metavar="LAUNCHES",
                    help="instead of the metric, a per-phase breakdown of the headline block from the "
                         "kernel's timeline tap over LAUNCHES traced launches")
    ap.add_argument("--timeline-c3-rows", type=int, default=0, metavar="B",
                    help="with --timeline: the row-bucket sweep's dims at B rows instead of the headline block")
    ap.add_argument("--read-probe", type=int, default=0, metavar="MiB",
                    help="instead of the block, time a plain HBM read kernel over MiB MiB "
                         "(libmb_readprobe.so) in several variants and grids")
    ap.add_argument("--sweep-cases", default="around,c0,c2,c3,c4",
                    help="with --sweep: which cases (comma list of around, c0, c2, c3, c4, or single "
                         "cases c2-calibrated, c2-literal, c3-uniform-<b>, c3-calibrated-<b>)")
    ap.add_argument("--sweep-steps", type=int, default=0,
                    help="with --sweep: timed launches per c2/c3 case (default 200)")
    ap.add_argument("--steps-around-only", action="store_true",
                    help="with --sweep: only the attention boundary and the next QKV projection")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the c1 metric, time every workload (c0, c2, c3 buckets, c4 "
                         "stack) and print one JSON line per case")
    args = ap.parse_args()
    if args.act_quant and args.layout != "packed":
        ap.error("--act-quant needs --layout packed")
    if args.print_source_hash:
        print(kernel_source_hash())
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the block runs on one GPU: it has no multi-GPU path)", file=sys.stderr)
        return 2

    if args.sweep:
        return sweep(args)
    if args.read_probe > 0:
        return read_probe(args.read_probe)
    if args.timeline > 0:
        return timeline(args.timeline, args.timeline_c3_rows)

    import numpy as np
    import torch

    import routed_expert_layer_amd as rel
    import synth
    from synth.device import dims_kwargs, upload, upload_weights

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    seeds = [WEIGHT_SEEDS[i % len(WEIGHT_SEEDS)] + 10000 * (i // len(WEIGHT_SEEDS))
             for i in range(args.sets)]
    print(f"[bench] generating {len(seeds)} c1 weight sets", file=sys.stderr, flush=True)
    blocks = [synth.make_block("c1", seed=s) for s in seeds]
    d = blocks[0].dims
    wt0, x, stream = upload(blocks[0], dev)
    tensors = [wt0] + [upload_weights(b, dev) for b in blocks[1:]]
    weights = [rel.make_weights(**t) for t in tensors]
    dims = rel.make_dims(**dims_kwargs(d), act_quant=int(args.act_quant))
    if args.layout == "packed":
        # Load-time preparation: the experts, the pooler's and the unpooler's
        # weights also in the streaming layouts.
        for t, w in zip(tensors, weights):
            t["experts_packed"] = rel.pack_experts(dims, w, dev)
            t["proj_packed"] = rel.pack_projections(dims, w, dev)
        weights = [rel.make_weights(**t) for t in tensors]
        torch.cuda.synchronize()
    ws = rel.workspace(dims, dev)
    x_next = torch.zeros((d.rows, d.hidden), dtype=torch.bfloat16, device=dev)

    # Experts each weight set's routing activates (|U| of the byte count).
    n_act = torch.zeros(1, dtype=torch.int32, device=dev)
    actives = []
    for w in weights:
        s = stream.clone()
        rel.mb_moe_block(dims, x, w, s, x_next, ws, taps=rel.make_taps(n_active=n_act))
        torch.cuda.synchronize()
        actives.append(int(n_act.item()))
    nw = (blocks[0].pre_norm_w is not None, blocks[0].ffn_norm_w is not None,
          blocks[0].next_norm_w is not None)
    b_alg = float(np.mean([algorithmic_bytes(d, a, nw) for a in actives]))

    if args.copy_probe > 0:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(f"[bench] copy probe: one elementwise kernel reading and writing {args.copy_probe} MiB",
              file=sys.stderr, flush=True)
        del src, dst

    S = len(weights)
    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        rel.mb_moe_block(dims, x, weights[i % S], stream, x_next, ws)
    torch.cuda.synchronize()

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    cur = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(cur)
    for i in range(args.steps):
        rel.mb_moe_block(dims, x, weights[i % S], stream, x_next, ws)
    ev1.record(cur)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1)
    ms_step = ms / args.steps
    us_block = ms_step * 1e3
    rows_s = d.rows * args.steps / (ms / 1e3)
    achieved = b_alg / (us_block * 1e-6) / 1e9
    print(f"[bench] {us_block:.2f} us/block, {rows_s:.0f} rows/s, {achieved:.0f} GB/s "
          f"({100 * achieved / HBM_PEAK_GBS:.1f}% of 8 TB/s), wall {wall * 1e3 / args.steps:.2f} "
          f"ms/step, active experts {actives}", file=sys.stderr, flush=True)

    # Per-launch durations (a second pass, events between launches).
    each = per_launch_us(torch, lambda i: rel.mb_moe_block(dims, x, weights[i % S], stream, x_next, ws),
                         min(args.steps, 1000))
    pct = percentiles(each)
    print(f"[bench] per launch: p10 {pct['p10']} p50 {pct['p50']} p90 {pct['p90']} us", file=sys.stderr,
          flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(blocks[0], args.cpu_seconds, args.act_quant)

    out = {
        "metric": METRIC,
        "value": round(rows_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # The expert products' operand types: bf16 activations against the
        # MXFP4 weights dequantized to bf16, or both MXFP4 (--act-quant).
        "dtype": "fp4" if args.act_quant else "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode verify step b=16: H=4096 P=2048 I=1024 E=64 top_k=4 sigmoid, "
                        "MXFP4 experts, bf16 pooler/unpooler, fp32 router and stream",
            "expert_layout": args.layout,
            "activations": "mxfp4 (W4A4)" if args.act_quant else "bf16",
            "rows": d.rows, "weight_sets": S, "active_experts": actives,
            "us_per_block": round(us_block, 3),
            "us_per_launch_percentiles": pct,
            "algorithmic_bytes_per_block": int(b_alg),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "block_kernel (the single launch of mb_moe_block)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if args.act_quant else stored_traffic(),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
