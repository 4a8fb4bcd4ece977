#!/usr/bin/env python3
"""KV-cache pack/unpack benchmark on one MI355X.

Workload (the pages' shape): 48 layers, each a separate [147456][16][K,V][128] bf16 cache
(8 KiB blocks, 1.125 GiB per layer), 8 requests x 576 blocks whose block tables are runs of
64 consecutive ids; the receiver is a second 48-layer cache with random destination ids.
All caches are synthetic (seeded random words), resident in HBM before timing starts.

One step = one pass of the whole hot path over that batch:
  sender:   kvx_build_xfer_list (pack runs) -> kvx_pack (all 48 layers, one launch)
  receiver: kvx_build_xfer_list (unpack runs) -> kvx_unpack (all 48 layers, one launch)
            -> kvx_slot_mapping for each request's recomputed last prompt token
            -> kvx_reshape_and_cache of those 8 tokens into each of the 48 layers
`value` = algorithmic bytes of the step (read + write of every moved byte) / step time.
"roofline" is the slower of pack and unpack, timed by HIP events on their stream in a second
run of the same K steps ("evented_ms_per_step"; the headline steps carry no events).

Under "ops", each after evicting the Infinity Cache: the same caches under the other
block-table shape (fragmented tables for the contiguous headline), as kv-first views, the
direct cache-to-cache copy, the layer-pipelined pack beside a GEMM forward stand-in (inline
or on a copy stream, with the signal as its own launch or inside the pack's), the
asymmetric-TP head merge, a plain unpack of the same shape and the head split (32 layers,
64 KiB blocks, each on 3 placements of the destination caches in memory), and the 32-request
decode slot mapping and new-token write (rows of 8 heads, 2 KiB, and of 1 head, 256 B). The
smallest transfer (2 layers, 6 blocks of 2 KiB) is timed on an idle GPU, as calls queued back
to back (beside the host's time to issue them) and replayed from a HIP graph.
"cpu_baseline" is the CPU oracle on the whole step. "graph_ms_per_step" is the same step
captured once in a HIP graph and replayed, timed after the ops (`value` stays the eager rate:
a graph is fixed to one transfer size).

    python bench.py [--steps K] [--warmup W] [--workload contiguous|fragmented]
                    [--no-cpu-baseline] [--no-ops] [--no-pipeline] [--no-graph] [--copy-calib]
                    [--alloc-spread ROUNDS] [--tiny]
Prints one JSON line on stdout; progress goes to stderr.
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

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak
COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "block_table_contiguous_amd", "csrc", f)
                  for f in ("kvx_kernels.hip", "kvx_launch.h")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=["contiguous", "fragmented"], default="contiguous")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ops", action="store_true")
    ap.add_argument("--op-reps", type=int, default=10)
    ap.add_argument("--no-pipeline", action="store_true",
                    help="skip the layer-pipelined pack beside the forward stand-in (ops.layer_pipeline)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the step replayed from a captured HIP graph (graph_ms_per_step)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates HBM byte counters)")
    ap.add_argument("--tiny", action="store_true",
                    help="only time the smallest transfer (ops.tiny_transfer), e.g. under a kernel trace")
    ap.add_argument("--alloc-spread", type=int, default=0, metavar="ROUNDS",
                    help="only measure how rates move with where the destination caches sit in memory: "
                         "ROUNDS placements of the 48-layer receive caches and the asymmetric-TP destination "
                         "caches inside one 198 GiB pool, each timing the 48-layer unpack, the head merge and "
                         "a plain unpack of the merge's shape")
    return ap.parse_args()


class Flush:
    """Reads a 512 MiB scratch buffer to push earlier data out of the 256 MiB Infinity Cache.
    Reading leaves clean lines behind; writing it would leave dirty ones, whose write-back the
    next kernel would pay for (the 288 MB new-token write measured 59 us after a writing flush,
    47 us after a reading one, 56 us with no flush after its own earlier writes)."""

    def __init__(self, torch, dev):
        self.t = torch.full((512 << 20,), 0x3C, dtype=torch.uint8, device=dev).view(torch.int64)

    def __call__(self):
        self.t.sum()


def time_op(torch, fn, reps, flush):
    """Median and min kernel time (ms) of fn over reps, with a cache flush before each."""
    ts = []
    for _ in range(reps):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    return ts[len(ts) // 2], ts[0]


def copy_calibration(torch, dev):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 3}), flush=True)


def alloc_spread(torch, np, W, K, dev, rounds, reps=3):
    """Rates against where the destination caches sit in memory, all in one process. Sources
    stay put. One pool of 176 chunks of 1.125 GiB (198 GiB) is allocated and filled once;
    placement r puts the 48 receive layers of the 48-layer unpack in chunks [r*s, r*s + 48) and
    the 32 destination layers of the asymmetric-TP workload in the first 16 of those chunks (two
    512 MiB layers per chunk), with the stride s spreading the placements over the pool. Per
    placement, after a cache flush each: the 48-layer unpack, the head merge and a plain unpack
    of the merge's shape (median of reps). One JSON line per placement; run it under
    rocprofv3 --pmc to set counters beside each placement's rates."""
    flush = Flush(torch, dev)
    pc = W.pages_contiguous()
    sp = pc.src_spec
    L, nb, BB, N = sp.num_layers, sp.num_blocks, sp.block_bytes, pc.total_blocks
    did, ro = K.flatten_tables(pc.dst_tables, dev)
    xu, cu = K.new_xfer_list(N, dev)
    K.kvx_build_xfer_list(None, did, ro, K.MODE_UNPACK, xu, cu)
    buf = W.fill_device_random_(torch.empty(L * N * BB, dtype=torch.uint8, device=dev), pc.seed)
    ac = W.asym_tp()
    La, Na, S = ac.dst_spec.num_layers, ac.total_blocks, ac.num_src
    BBa, nba = ac.dst_spec.block_bytes, ac.dst_spec.num_blocks
    assert 2 * nba * BBa <= nb * BB and La <= 2 * L
    srcs = [W.fill_device_random_(torch.empty((La, Na, BBa // S), dtype=torch.uint8, device=dev), ac.seed * 10 + s)
            for s in range(S)]
    one = W.fill_device_random_(torch.empty((La, Na, BBa), dtype=torch.uint8, device=dev), ac.seed * 10 + 7)
    aid, aro = K.flatten_tables(ac.dst_tables, dev)
    xa, ca = K.new_xfer_list(Na, dev)
    K.kvx_build_xfer_list(None, aid, aro, K.MODE_UNPACK, xa, ca)
    chunks = 176
    pool = [W.fill_device_byte_(torch.empty((nb, BB), dtype=torch.uint8, device=dev)) for _ in range(chunks)]
    step = (chunks - L) // max(rounds - 1, 1)
    ub, mb = 2 * L * N * BB, 2 * La * Na * BBa
    torch.cuda.synchronize()
    for rnd in range(rounds):
        first = min(rnd * step, chunks - L)
        dst = pool[first:first + L]
        adst = [dst[i // 2].view(-1)[(i % 2) * nba * BBa:(i % 2 + 1) * nba * BBa].view(nba, BBa) for i in range(La)]
        db, adb = K.layer_base_table(dst), K.layer_base_table(adst)
        rates = {}
        for name, nbytes, fn in (
                ("unpack_48layer", ub, lambda: K.kvx_unpack([buf], db, BB, nb, 1, xu, cu, N)),
                ("merge_asym_tp", mb, lambda: K.kvx_unpack(srcs, adb, BBa, nba, ac.rows_per_block, xa, ca, Na)),
                ("unpack_asym_tp_shape", mb, lambda: K.kvx_unpack([one], adb, BBa, nba, 1, xa, ca, Na))):
            med, _ = time_op(torch, fn, reps, flush)
            rates[name] = round(nbytes / (med * 1e-3) / 1e9, 1)
        print(json.dumps({"round": rnd, "chunks": [first, first + L - 1], "GB/s": rates}), flush=True)


def traffic_from_counters(name: str, launches_bytes: int):
    """HBM bytes per launch of `name` from the committed rocprofv3 counter summary, scaled by
    the copy-kernel calibration; None if absent or taken on other kernel sources."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256_16") != kernel_source_hash() or name not in c.get("kernels", {}):
        return None
    k = c["kernels"][name]
    cal = c["copy_calibration"]
    f_fetch = cal["bytes"] / (cal["FETCH_SIZE_KiB"] * 1024.0)
    f_write = cal["bytes"] / (cal["WRITE_SIZE_KiB"] * 1024.0)
    return int(k["FETCH_SIZE_KiB"] * 1024.0 * f_fetch + k["WRITE_SIZE_KiB"] * 1024.0 * f_write)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this path is measured on one GPU only (no second GPU, collective or "
              "sharded run is part of it); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    from block_table_contiguous_amd import kvx as K

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calib:
        copy_calibration(torch, dev)
        return
    if args.alloc_spread:
        alloc_spread(torch, np, W, K, dev, args.alloc_spread)
        return
    if args.tiny:
        print(json.dumps({"tiny_transfer": tiny_transfer(torch, np, W, K, dev)}), flush=True)
        return

    case = W.pages_contiguous() if args.workload == "contiguous" else W.pages_fragmented()
    spec = case.src_spec
    L, nb, BB, N = spec.num_layers, spec.num_blocks, spec.block_bytes, case.total_blocks
    log(f"workload {case.name}: {L} layers x {nb} blocks x {BB} B, {len(case.src_tables)} requests, N={N}")

    src = [torch.empty((nb, BB), dtype=torch.uint8, device=dev) for _ in range(L)]
    dst = [torch.empty((nb, BB), dtype=torch.uint8, device=dev) for _ in range(L)]
    for l in range(L):
        W.fill_device_random_(src[l], case.seed * 1000 + l)
        W.fill_device_byte_(dst[l])
    buf = torch.empty(L * N * BB, dtype=torch.uint8, device=dev)
    src_bases, dst_bases = K.layer_base_table(src), K.layer_base_table(dst)
    sid, ro = K.flatten_tables(case.src_tables, dev)
    did, _ = K.flatten_tables(case.dst_tables, dev)
    xp, cp = K.new_xfer_list(N, dev)
    xu, cu = K.new_xfer_list(N, dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    # receiver's recompute of each request's last prompt token (one token per request)
    R = len(case.dst_tables)
    row = spec.row_bytes
    d_table_h = W.pad_table(case.dst_tables, max(len(t) for t in case.dst_tables))
    r_idx_h = np.arange(R, dtype=np.int32)
    r_pos_h = np.array([n - 1 for n in case.lengths], dtype=np.int64)
    d_table, r_idx, r_pos = (torch.from_numpy(x).to(dev) for x in (d_table_h, r_idx_h, r_pos_h))
    r_slots = torch.empty(R, dtype=torch.int64, device=dev)
    rng = np.random.default_rng(case.seed + 7)
    new_k_h = W.bf16_normal_bits(rng, (L, R, row // 2))
    new_v_h = W.bf16_normal_bits(rng, (L, R, row // 2))
    new_k, new_v = torch.from_numpy(new_k_h).to(dev), torch.from_numpy(new_v_h).to(dev)
    cnb, cbs, bst, tst, kst = K.cache_strides(
        dst[0].view(torch.int16).view(nb, spec.block_size, 2, spec.num_kv_heads, spec.head_dim))
    torch.cuda.synchronize()
    log("inputs resident")

    ev = {}

    def timed(name, fn, record):
        if record:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ev.setdefault(name, []).append((a, b))
        else:
            fn()

    def step(record=False):
        timed("build_pack", lambda: K.kvx_build_xfer_list(sid, None, ro, K.MODE_PACK, xp, cp, err), record)
        timed("pack", lambda: K.kvx_pack(src_bases, BB, nb, xp, cp, N, buf, err), record)
        timed("build_unpack", lambda: K.kvx_build_xfer_list(None, did, ro, K.MODE_UNPACK, xu, cu, err), record)
        timed("unpack", lambda: K.kvx_unpack([buf], dst_bases, BB, nb, 1, xu, cu, N, err), record)
        K.kvx_slot_mapping(d_table, r_idx, r_pos, spec.block_size, r_slots, err)
        for l in range(L):
            K.kvx_reshape_and_cache(new_k[l], new_v[l], r_slots, dst[l], cnb, cbs, bst, tst, kst, err)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(err.item()) == 0, "device error flag raised"
    log(f"warmup done ({args.warmup} steps)")

    def timed_steps(record):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(record=record)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    # The headline steps carry no timing events (the eight per step cost about 40 us); the
    # per-kernel times of the roofline come from a second run of the same steps with events
    # around the run lists, pack and unpack.
    ms_per_step = timed_steps(False)
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step")
    evented_ms = timed_steps(True)
    log(f"the same steps with timing events around the run lists, pack and unpack: {evented_ms:.4f} ms/step")

    def graph_replay_ms():
        """The same step captured once in a HIP graph and replayed: ms per replay."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        log(f"graph replay: {ms:.4f} ms/step")
        assert int(err.item()) == 0, "device error flag raised"
        return ms

    copy_bytes = 2 * L * N * BB                    # pack and unpack: each byte read once, written once
    write_bytes = L * R * (2 * 2 * row + 8)        # new-token write: K,V read+write + slot
    slot_bytes = R * (4 + 8 + 4 + 8)               # req index, position, table entry, slot
    step_bytes = 2 * copy_bytes + write_bytes + slot_bytes
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    def avg_ms(name):
        xs = [a.elapsed_time(b) for a, b in ev[name]]
        return sum(xs) / len(xs)

    kern = {n: avg_ms(n) for n in ("build_pack", "pack", "build_unpack", "unpack")}
    dominant = max(("pack", "unpack"), key=lambda n: kern[n])
    achieved = copy_bytes / (kern[dominant] * 1e-3) / 1e9
    roofline = {
        "bound": "hbm", "kernel": f"kvx_{dominant}", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
        "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
        "traffic": traffic_from_counters(f"{dominant}_{case.name}", copy_bytes),
        "algorithmic_bytes": copy_bytes, "avg_launch_ms": round(kern[dominant], 5),
        "events": "HIP events around each kernel on its stream, over a second run of the same "
                  "K steps (evented_ms_per_step); the headline steps carry none",
    }
    out_ops = {n: {"avg_ms": round(v, 5)} for n, v in kern.items()}
    for n in ("pack", "unpack"):
        out_ops[n]["GB/s"] = round(copy_bytes / (kern[n] * 1e-3) / 1e9, 1)
        out_ops[n]["frac_of_peak"] = round(copy_bytes / (kern[n] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        out_ops[n]["traffic"] = traffic_from_counters(f"{n}_{case.name}", copy_bytes)
    e2e = [a.elapsed_time(b) for (a, _), (_, b) in zip(ev["build_pack"], ev["pack"])]
    out_ops["build_plus_pack"] = {"avg_ms": round(sum(e2e) / len(e2e), 5),
                                  "about": "start of the run-list build to the end of the pack, same steps"}
    runs_pack, runs_unpack = int(cp.item()), int(cu.item())
    for n, runs in (("build_pack", runs_pack), ("pack", runs_pack * L),
                    ("build_unpack", runs_unpack), ("unpack", runs_unpack * L)):
        out_ops[n]["runs"] = runs  # descriptors the op reads or writes (per layer for the copies)
        out_ops[n]["ns_per_run"] = round(kern[n] * 1e6 / max(runs, 1), 2)

    if not args.no_ops:
        flush = Flush(torch, dev)
        med, mn = time_op(torch, lambda: buf[: L * N * BB // 2].copy_(buf[L * N * BB // 2:]), args.op_reps, flush)
        out_ops["d2d_copy_ceiling"] = {"bytes": L * N * BB, "median_ms": round(med, 5),
                                       "GB/s": round(L * N * BB / (med * 1e-3) / 1e9, 1)}
        for n, fn in (("pack", lambda: K.kvx_pack(src_bases, BB, nb, xp, cp, N, buf, err)),
                      ("unpack", lambda: K.kvx_unpack([buf], dst_bases, BB, nb, 1, xu, cu, N, err))):
            med, mn = time_op(torch, fn, args.op_reps, flush)
            out_ops[n]["flushed_median_ms"] = round(med, 5)
            out_ops[n]["flushed_min_ms"] = round(mn, 5)
            out_ops[n]["flushed_GB/s"] = round(copy_bytes / (med * 1e-3) / 1e9, 1)
        # the same 48 allocations viewed as kv-first caches: (K plane, V plane) of 4 KiB segments
        seg = BB // 2
        for n, fn in (("pack_kv_first", lambda: K.kvx_pack_kv_first(src_bases, seg, nb * seg, nb, ro, xp, cp, N,
                                                                     buf, err)),
                      ("unpack_kv_first", lambda: K.kvx_unpack_kv_first(buf, dst_bases, seg, nb * seg, nb, ro, xu,
                                                                         cu, N, err))):
            med, mn = time_op(torch, fn, args.op_reps, flush)
            out_ops[n] = {"workload": f"{case.name}, kv-first view: 48 x (2, {nb}, {seg} B)",
                          "median_ms": round(med, 5), "GB/s": round(copy_bytes / (med * 1e-3) / 1e9, 1),
                          "frac_of_peak": round(copy_bytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                          "traffic": traffic_from_counters(f"{n}_{case.name}", copy_bytes)}
        # the same transfer with no send buffer: direct-mode runs, cache to cache
        xd, cd = K.new_xfer_list(N, dev)
        K.kvx_build_xfer_list(sid, did, ro, K.MODE_DIRECT, xd, cd, err)
        med, mn = time_op(torch, lambda: K.kvx_copy_direct(src_bases, dst_bases, BB, nb, nb, xd, cd, N, err),
                          args.op_reps, flush)
        direct_bytes = copy_bytes  # each listed block read once from the source, written once
        out_ops["copy_direct"] = {
            "workload": f"{case.name}: the same 48 layers and tables, cache to cache with no send buffer",
            "runs": int(cd.item()) * L, "median_ms": round(med, 5),
            "GB/s": round(direct_bytes / (med * 1e-3) / 1e9, 1),
            "frac_of_peak": round(direct_bytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "traffic": traffic_from_counters(f"direct_{case.name}", direct_bytes),
            "vs_pack_plus_unpack": round((out_ops["pack"]["flushed_median_ms"] + out_ops["unpack"]["flushed_median_ms"]) / med, 3)}
        torch.cuda.synchronize()
        assert int(err.item()) == 0, "device error flag raised"
        other = W.pages_fragmented() if case.name == "contiguous" else W.pages_contiguous()
        out_ops[other.name] = other_tables(torch, K, dev, flush, args.op_reps, other, src_bases, dst_bases,
                                           buf, L, nb, BB, err)
        if not args.no_pipeline:
            out_ops["layer_pipeline"] = layer_pipeline(torch, K, dev, L, nb, BB, N, src_bases, buf, xp, cp, err,
                                                       max(3, args.op_reps // 2))

    # Captured and replayed after the op timings and the layer pipeline: once a process has
    # replayed a HIP graph, the pipeline's forward and copy streams overlap worse (the
    # copy-stream schedule measured 9.48 ms after a replay, 8.56 ms in a process without one).
    graph_ms = None if args.no_graph else graph_replay_ms()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(np, W, case, src, d_table_h, r_idx_h, r_pos_h, new_k_h, new_v_h,
                           (cnb, cbs, bst, tst, kst))

    if not args.no_ops:
        # The workloads the headline batch does not exercise (asymmetric-TP merge and split,
        # decode writes) run last, after the 110 GiB of 48-layer caches are released, as on a
        # receiving GPU that does not also hold the sender's caches.
        del src, dst, buf, src_bases, dst_bases
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        out_ops.update(other_workloads(torch, np, W, K, dev, flush, args.op_reps))

    result = {
        "metric": "KV pack/unpack effective HBM GB/s (R+W) and % of MI355X peak, 1 GPU",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {
            "workload": f"{case.name}: 48 layers x [147456][16][K,V][128] bf16 (8 KiB blocks), "
                        f"8 requests x 576 blocks, unpacked to random ids in a second 48-layer cache",
            "layers": L, "blocks_per_layer": nb, "block_bytes": BB, "requests": R,
            "blocks_per_request": N // R, "cache_dtype": "bf16", "step_bytes": step_bytes,
            "parallelism": "single GPU",
        },
        "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        "evented_ms_per_step": round(evented_ms, 5),
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ops": out_ops,
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    print(json.dumps(result), flush=True)


def other_tables(torch, K, dev, flush, reps, case, src_bases, dst_bases, buf, L, nb, BB, err):
    """The same 48-layer caches under the other block-table shape (for the contiguous headline:
    the fragmented tables, geometric(0.5) run lengths, about 2,300 pack runs against 72): both
    run-list builds, pack and unpack, each timed after evicting the Infinity Cache."""
    N = case.total_blocks
    sid, ro = K.flatten_tables(case.src_tables, dev)
    did, _ = K.flatten_tables(case.dst_tables, dev)
    xp, cp = K.new_xfer_list(N, dev)
    xu, cu = K.new_xfer_list(N, dev)
    nbytes = 2 * L * N * BB
    out = {"workload": f"{case.name}: the same {L} caches, 8 requests x 576 blocks, "
                       + ("geometric(0.5) run lengths" if case.name == "fragmented" else "runs of 64"),
           "bytes": nbytes}
    for name, fn in (("build_pack", lambda: K.kvx_build_xfer_list(sid, None, ro, K.MODE_PACK, xp, cp, err)),
                     ("build_unpack", lambda: K.kvx_build_xfer_list(None, did, ro, K.MODE_UNPACK, xu, cu, err))):
        med, mn = time_op(torch, fn, reps, flush)
        out[name] = {"median_ms": round(med, 5)}
    torch.cuda.synchronize()
    runs = {"pack": int(cp.item()), "unpack": int(cu.item())}
    out["build_pack"]["runs"], out["build_unpack"]["runs"] = runs["pack"], runs["unpack"]
    for name, fn in (("pack", lambda: K.kvx_pack(src_bases, BB, nb, xp, cp, N, buf, err)),
                     ("unpack", lambda: K.kvx_unpack([buf], dst_bases, BB, nb, 1, xu, cu, N, err))):
        med, mn = time_op(torch, fn, reps, flush)
        out[name] = {"median_ms": round(med, 5), "min_ms": round(mn, 5),
                     "GB/s": round(nbytes / (med * 1e-3) / 1e9, 1),
                     "frac_of_peak": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "runs": runs[name] * L, "ns_per_run": round(med * 1e6 / max(runs[name] * L, 1), 2),
                     "traffic": traffic_from_counters(f"{name}_{case.name}", nbytes)}
    torch.cuda.synchronize()
    assert int(err.item()) == 0, "device error flag raised"
    log(f"{case.name} tables: pack {out['pack']['GB/s']} GB/s, unpack {out['unpack']['GB/s']} GB/s, "
        f"{runs['pack']} / {runs['unpack']} runs")
    return out


def layer_pipeline(torch, K, dev, L, nb, BB, N, src_bases, buf, xp, cp, err, reps):
    """The sender's side of a layer-pipelined transfer. One bf16 [8192 x 4096] x [4096 x 4096]
    product per layer on the forward stream stands in for that layer's forward pass (it is not
    part of the path): each layer has its own weight, and its output is the next layer's input,
    so no layer finds the previous layer's operands in cache. Schedules, each timed from a start
    event to the end of all streams:
      forward_only  the 48 products;
      serial        the 48 products, then one pack of all layers on the forward stream;
      inline        per layer on the forward stream: the product, the pack of that layer into
                    its slice of the send buffer, and a signal add (the count a transport, or a
                    receiver's signal wait, follows layer by layer);
      inline_fused  the same, with the signal carried by the pack's own launch
                    (kvx_pack_signal) instead of a separate signal kernel;
      pipelined     per layer: the product, then an event on the forward stream; on a copy
                    stream, a wait for that event, the layer's pack and the signal add. The
                    forward stream never waits for a copy;
      pipelined_fused  the same on the copy stream with the signal carried by the pack's own
                    launch (kvx_pack_signal): one launch per layer beside the forward.
    Per schedule: the total, the tail (end of the last product to the end of the packing) and
    mean_ready (start to the moment a layer's packed bytes are complete, averaged over the
    layers: when a transport could begin sending each layer). The receiver's unpack is left
    out: it runs on the other GPU of a real transfer, not beside the sender's forward pass."""
    m, k = 8192, 4096
    # activations stay 0.5 exactly: each output element is k * 0.5 * 2^-12
    acts = [torch.full((m, k), 0.5, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    weights = torch.full((L, k, k), 2.0 ** -12, dtype=torch.bfloat16, device=dev)

    def layer_forward(l):
        torch.mm(acts[l % 2], weights[l], out=acts[(l + 1) % 2])
    fwd, cpy = torch.cuda.Stream(), torch.cuda.Stream()
    counter = torch.zeros(1, dtype=torch.int64, device=dev)
    bufv = buf[: L * N * BB].view(L, N, BB)
    evs = [torch.cuda.Event() for _ in range(L)]
    pack_l = [src_bases[l:l + 1] for l in range(L)]

    def forward_only(f_ev, rdy):
        with torch.cuda.stream(fwd):
            for l in range(L):
                layer_forward(l)
            f_ev.record(fwd)

    def serial(f_ev, rdy):
        with torch.cuda.stream(fwd):
            for l in range(L):
                layer_forward(l)
            f_ev.record(fwd)
            K.kvx_pack(src_bases, BB, nb, xp, cp, N, buf, err, stream=fwd)

    def inline(f_ev, rdy):
        with torch.cuda.stream(fwd):
            for l in range(L):
                layer_forward(l)
                if l == L - 1:
                    f_ev.record(fwd)
                K.kvx_pack(pack_l[l], BB, nb, xp, cp, N, bufv[l], err, stream=fwd)
                K.kvx_signal_add(counter, 1, stream=fwd)
                rdy[l].record(fwd)

    arrivals = K.new_arrivals(dev)

    def inline_fused(f_ev, rdy):
        with torch.cuda.stream(fwd):
            for l in range(L):
                layer_forward(l)
                if l == L - 1:
                    f_ev.record(fwd)
                K.kvx_pack_signal(pack_l[l], BB, nb, xp, cp, N, bufv[l], counter, arrivals, 1, err, stream=fwd)
                rdy[l].record(fwd)

    def pipelined(f_ev, rdy):
        for l in range(L):
            with torch.cuda.stream(fwd):
                layer_forward(l)
                evs[l].record(fwd)
            cpy.wait_event(evs[l])
            K.kvx_pack(pack_l[l], BB, nb, xp, cp, N, bufv[l], err, stream=cpy)
            K.kvx_signal_add(counter, 1, stream=cpy)
            rdy[l].record(cpy)
        f_ev.record(fwd)

    def pipelined_fused(f_ev, rdy):
        for l in range(L):
            with torch.cuda.stream(fwd):
                layer_forward(l)
                evs[l].record(fwd)
            cpy.wait_event(evs[l])
            K.kvx_pack_signal(pack_l[l], BB, nb, xp, cp, N, bufv[l], counter, arrivals, 1, err, stream=cpy)
            rdy[l].record(cpy)
        f_ev.record(fwd)

    def run(fn):
        torch.cuda.synchronize()
        s_ev, f_ev, e_ev = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        rdy = [torch.cuda.Event(enable_timing=True) for _ in range(L)]
        s_ev.record(fwd)
        cpy.wait_stream(fwd)
        fn(f_ev, rdy)
        fwd.wait_stream(cpy)
        e_ev.record(fwd)
        torch.cuda.synchronize()
        total = s_ev.elapsed_time(e_ev)
        # one launch packs every layer in the schedules without per-layer events: all of its
        # layers are complete when it ends
        ready = (sum(s_ev.elapsed_time(r) for r in rdy) / L) if fn in (inline, inline_fused, pipelined, pipelined_fused) else total
        return total, f_ev.elapsed_time(e_ev), ready

    out = {"workload": f"{L} layers; forward stream: one bf16 [{m}x{k}]x[{k}x{k}] product per layer with "
                       "its own weight, output feeding the next layer (forward stand-in); per layer: that "
                       "layer's pack, then a signal add (inline on the forward stream or pipelined on a copy "
                       "stream; each either as a separate signal kernel or carried by the pack's own launch)"}
    for name, fn in (("forward_only", forward_only), ("serial", serial), ("inline", inline),
                     ("inline_fused", inline_fused), ("pipelined", pipelined),
                     ("pipelined_fused", pipelined_fused)):
        run(fn)  # warm
        ts = sorted(run(fn) for _ in range(reps))
        total, tail, ready = ts[len(ts) // 2]
        out[f"{name}_ms"] = round(total, 4)
        if name != "forward_only":
            out[f"{name}_tail_ms"] = round(tail, 4)
            out[f"{name}_mean_ready_ms"] = round(ready, 4)
        log(f"layer pipeline {name}: {total:.4f} ms, tail after the forward {tail:.4f} ms, "
            f"mean layer ready {ready:.4f} ms")
    torch.cuda.synchronize()
    assert int(err.item()) == 0, "device error flag raised"
    assert int(counter.item()) == 4 * L * (reps + 1), "signal count"
    assert not bool(arrivals.any()), "arrivals workspace left non-zero"
    return out


def tiny_transfer(torch, np, W, K, dev, iters=200):
    """The smallest transfer (2 layers, requests of 17, 40 and 5 tokens, 2 KiB blocks, 6 blocks):
    how long one transfer takes when nothing else is queued, what each call costs when launches
    follow each other (with the host time the Python calls take to enqueue them), and how long
    the transfer takes replayed from a HIP graph, with no host work between its kernels."""
    case = W.tiny_roundtrip()
    spec = case.src_spec
    L, nb, BB, N = spec.num_layers, spec.num_blocks, spec.block_bytes, case.total_blocks
    src = [torch.from_numpy(np.ascontiguousarray(c).view(np.uint8).reshape(nb, BB)).to(dev) for c in case.src_caches]
    dst = [torch.from_numpy(np.ascontiguousarray(c).view(np.uint8).reshape(nb, BB)).to(dev) for c in case.dst_caches]
    sb, db = K.layer_base_table(src), K.layer_base_table(dst)
    sid, ro = K.flatten_tables(case.src_tables, dev)
    did, _ = K.flatten_tables(case.dst_tables, dev)
    xp, cp = K.new_xfer_list(N, dev)
    xu, cu = K.new_xfer_list(N, dev)
    buf = torch.empty(L * N * BB, dtype=torch.uint8, device=dev)
    calls = {"build_pack": lambda: K.kvx_build_xfer_list(sid, None, ro, K.MODE_PACK, xp, cp),
             "pack": lambda: K.kvx_pack(sb, BB, nb, xp, cp, N, buf),
             "build_unpack": lambda: K.kvx_build_xfer_list(None, did, ro, K.MODE_UNPACK, xu, cu),
             "unpack": lambda: K.kvx_unpack([buf], db, BB, nb, 1, xu, cu, N)}

    def transfer():
        for fn in calls.values():
            fn()
    transfer()
    torch.cuda.synchronize()
    lat = []
    for _ in range(51):  # one transfer on an idle GPU: start event, the four calls, end event
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        transfer()
        b.record()
        b.synchronize()
        lat.append(a.elapsed_time(b) * 1e3)
    per_call, host_per_call = {}, {}
    for name, fn in calls.items():  # the same call queued `iters` times in a row
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        t0 = time.perf_counter()
        for _ in range(iters):
            fn()
        host_per_call[name] = round((time.perf_counter() - t0) * 1e6 / iters, 2)
        b.record()
        b.synchronize()
        per_call[name] = round(a.elapsed_time(b) * 1e3 / iters, 2)
    lat.sort()
    # The four calls captured once in a HIP graph and replayed: one transfer with no host work
    # (Python, argument checks, launch calls) between its kernels. Each replay must leave the
    # same bytes as the eager transfer.
    want_buf, want_dst = buf.clone(), [t.clone() for t in dst]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        transfer()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        transfer()
    g.replay()
    torch.cuda.synchronize()
    glat = []
    for _ in range(51):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        glat.append(a.elapsed_time(b) * 1e3)
    same = bool(torch.equal(buf, want_buf) and all(torch.equal(t, w) for t, w in zip(dst, want_dst)))
    if not same:
        log("WARNING: the graph-replayed tiny transfer left different bytes than the eager one")
    glat.sort()
    return {"workload": f"{L} layers x {N} blocks of {BB} B (requests of 17, 40 and 5 tokens)",
            "bytes": 2 * 2 * L * N * BB, "transfer_us_median": round(lat[len(lat) // 2], 2),
            "transfer_us_min": round(lat[0], 2), "queued_us_per_call": per_call,
            "host_us_per_call": host_per_call,
            "graph_transfer_us_median": round(glat[len(glat) // 2], 2),
            "graph_transfer_us_min": round(glat[0], 2), "graph_bytes_identical_to_eager": same}


def other_workloads(torch, np, W, K, dev, flush, reps, allocs=3):
    """The rows the headline batch does not exercise, each on its own workload."""
    out = {"tiny_transfer": tiny_transfer(torch, np, W, K, dev)}
    # asymmetric-TP receive: 2 sources x 4 heads -> 8-head caches, 32 layers x 4096 blocks.
    # Rates of this shape move by up to +-10% with the physical pages an allocation lands on
    # (5.3-6.6 TB/s for the same code in one process), so the destination caches are placed
    # `allocs` times and each op reports the median over the placements of its median over
    # reps, with every placement's rate beside it. Placement i is allocated while a spacer of
    # i * 24 GiB is held, so the placements take different regions of memory (a free and a
    # fresh allocation of the same size can get the same pages back).
    case = W.asym_tp()
    L, N, S = case.dst_spec.num_layers, case.total_blocks, case.num_src
    BB, nb = case.dst_spec.block_bytes, case.dst_spec.num_blocks
    srcs = [torch.empty((L, N, BB // S), dtype=torch.uint8, device=dev) for _ in range(S)]
    for s_, t in enumerate(srcs):
        W.fill_device_random_(t, case.seed * 10 + s_)
    one = torch.empty((L, N, BB), dtype=torch.uint8, device=dev)
    W.fill_device_random_(one, case.seed * 10 + 7)
    ids, ro = K.flatten_tables(case.dst_tables, dev)
    x, c = K.new_xfer_list(N, dev)
    K.kvx_build_xfer_list(None, ids, ro, K.MODE_UNPACK, x, c)
    xs, cs = K.new_xfer_list(N, dev)
    K.kvx_build_xfer_list(ids, None, ro, K.MODE_PACK, xs, cs)
    nbytes = 2 * L * N * BB
    per = {"merge": [], "plain": [], "split": []}
    for i in range(allocs):
        spacer = [torch.empty(1 << 30, dtype=torch.uint8, device=dev) for _ in range(24 * i)]
        dst = [W.fill_device_byte_(torch.empty((nb, BB), dtype=torch.uint8, device=dev)) for _ in range(L)]
        bases = K.layer_base_table(dst)
        for name, fn in (("merge", lambda: K.kvx_unpack(srcs, bases, BB, nb, case.rows_per_block, x, c, N)),
                         ("plain", lambda: K.kvx_unpack([one], bases, BB, nb, 1, x, c, N)),
                         ("split", lambda: K.kvx_pack_split(bases, BB, nb, case.rows_per_block, xs, cs, N, srcs))):
            med, _ = time_op(torch, fn, reps, flush)
            per[name].append(med)
        del dst, bases, spacer
        torch.cuda.empty_cache()
    del srcs, one
    torch.cuda.empty_cache()

    def shape_op(name, workload, counters):
        ms = sorted(per[name])
        med = ms[len(ms) // 2]
        return {"workload": workload, "bytes": nbytes, "placements": allocs, "median_ms": round(med, 4),
                "GB/s": round(nbytes / (med * 1e-3) / 1e9, 1),
                "frac_of_peak": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "per_placement_GB/s": [round(nbytes / (t * 1e-3) / 1e9, 1) for t in per[name]],
                "traffic": traffic_from_counters(counters, nbytes)}
    out["merge_unpack_asym_tp"] = shape_op(
        "merge", "2 sources x 4 of 8 heads, 32 layers x 16 requests x 256 blocks -> [8192][16][K,V][8][128] bf16",
        "merge_asym_tp")
    # the same destination blocks and bytes from one full-head buffer: a plain unpack, the
    # merge's own shape without the head interleave (its cost against the merge's)
    out["unpack_asym_tp_shape"] = shape_op(
        "plain", "one buffer of all 8 heads, 32 layers x 16 requests x 256 blocks -> the same [8192][16][K,V][8][128] "
                 "bf16 caches and destination ids as the merge", "unpack_asym_tp_shape")
    # the sender side of the same shapes: full-head caches split into 2 head shards
    out["split_pack_asym_tp"] = shape_op(
        "split", "32 layers of [8192][16][K,V][8][128] bf16, 16 requests x 256 blocks -> 2 shards x 4 heads",
        "split_asym_tp")
    # decode write: 32 requests of 1..2048 tokens into a [4096][16][K,V][8][128] bf16 cache
    d = W.decode_write()
    T = len(d.req_idx)
    bt, rq, pos = (torch.from_numpy(a).to(dev) for a in (d.block_table, d.req_idx, d.positions))
    slots = torch.empty(T, dtype=torch.int64, device=dev)
    cache = torch.full(d.spec.shape5, -1, dtype=torch.int16, device=dev)
    key, val = torch.from_numpy(d.key).to(dev), torch.from_numpy(d.value).to(dev)
    cnb, cbs, bst, tst, kst = K.cache_strides(cache)
    med, mn = time_op(torch, lambda: K.kvx_slot_mapping(bt, rq, pos, 16, slots), reps, flush)
    sbytes = T * (4 + 8 + 4 + 8)
    out["slot_mapping_decode"] = {"tokens": T, "bytes": sbytes, "median_ms": round(med, 5),
                                  "GB/s": round(sbytes / (med * 1e-3) / 1e9, 1)}
    med, mn = time_op(torch, lambda: K.kvx_reshape_and_cache(key, val, slots, cache, cnb, cbs, bst, tst, kst),
                      reps, flush)
    wbytes = T * (4 * d.spec.row_bytes + 8)
    out["reshape_and_cache_decode"] = {
        "tokens": T, "bytes": wbytes, "median_ms": round(med, 5),
        "GB/s": round(wbytes / (med * 1e-3) / 1e9, 1), "frac_of_peak": round(wbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "traffic": traffic_from_counters("write_decode", wbytes)}
    del cache, key, val
    # the same tokens with the 48-layer caches' rows: 1 head x 128 bf16 = 256 B per K or V row
    d1 = W.decode_write(num_kv_heads=1)
    cache1 = torch.full(d1.spec.shape5, -1, dtype=torch.int16, device=dev)
    key1, val1 = torch.from_numpy(d1.key).to(dev), torch.from_numpy(d1.value).to(dev)
    cnb, cbs, bst, tst, kst = K.cache_strides(cache1)
    med, mn = time_op(torch, lambda: K.kvx_reshape_and_cache(key1, val1, slots, cache1, cnb, cbs, bst, tst, kst),
                      reps, flush)
    wbytes = T * (4 * d1.spec.row_bytes + 8)
    out["reshape_and_cache_decode_1head"] = {
        "workload": f"the same {T} tokens and slots, rows of 1 head x 128 bf16 (256 B) into [4096][16][K,V][1][128]",
        "tokens": T, "bytes": wbytes, "median_ms": round(med, 5),
        "GB/s": round(wbytes / (med * 1e-3) / 1e9, 1), "frac_of_peak": round(wbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "traffic": traffic_from_counters("write_decode_1head", wbytes)}
    return out


def cpu_baseline(np, W, case, src_dev, table_h, req_h, pos_h, new_k_h, new_v_h, strides, sample_layers=48):
    """The CPU oracle, as it stands, on a bounded sample of the same step: both run lists and
    the slot mapping once, then for `sample_layers` of the 48 layers the layer's pack, its
    unpack into a receive layer filled like the benchmark's, and the write of each request's
    recomputed last prompt token into it (host copies of the real source layers). Value = the
    sample's step bytes over the oracle's time; copies to the host are not timed."""
    import oracle as O

    spec = case.src_spec
    nb, BB, bs, row = spec.num_blocks, spec.block_bytes, spec.block_size, spec.row_bytes
    R, N = len(case.dst_tables), case.total_blocks
    _, _, bst, tst, kst = strides
    stride = max(1, spec.num_layers // sample_layers)
    layers = list(range(0, spec.num_layers, stride))[:sample_layers]
    t0 = time.perf_counter()
    O.xfer_list(case.src_tables, case.dst_tables, O.MODE_PACK)
    O.xfer_list(case.src_tables, case.dst_tables, O.MODE_UNPACK)
    slots, _ = O.slot_mapping(table_h, req_h, pos_h, bs)
    t_oracle = time.perf_counter() - t0
    for l in layers:
        src_l = src_dev[l].cpu().numpy()
        before = np.full((nb, BB), W.FILL_BYTE, np.uint8)
        t0 = time.perf_counter()
        buf, _ = O.pack([src_l], case.src_tables)
        out, _ = O.unpack([buf], [before], case.dst_tables)
        O.reshape_and_cache(out[0], new_k_h[l], new_v_h[l], slots, nb, bs, bst, tst, kst)
        t_oracle += time.perf_counter() - t0
        del src_l, before, buf, out
    nbytes = len(layers) * (2 * 2 * N * BB + R * (4 * row + 8)) + R * (4 + 8 + 4 + 8)
    try:
        cores_avail = len(os.sched_getaffinity(0))
    except AttributeError:
        cores_avail = os.cpu_count()
    cpu_model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(nbytes / t_oracle / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the oracle's step on {len(layers)} of {spec.num_layers} layers: both run lists and the "
                      f"slot mapping once, then per layer pack, unpack and the new-token write "
                      f"({nbytes} algorithmic bytes, {t_oracle:.2f} s; numpy, single thread: 1 of "
                      f"{cores_avail} host cores available, {os.cpu_count()} online, {cpu_model})"}


if __name__ == "__main__":
    main()
