#!/usr/bin/env python3
"""Decode-attention benchmark for libpagedattn on one MI355X.

A step is one paged_attn_decode call over the whole batch (phase 1 with the
tier dispatch, then phase 2).  The default workload is long-context decode:
4 sequences x 102400 tokens (automatic partitions: 16 of 6400 tokens, one
workgroup per CU), 24 query / 4 KV heads, head_dim 256, 16-token pages, fp16,
q = 8 N(0,1) so the softmax is peaked.  `--workload prefill` times the chunked
prefill kernel instead (TFLOP/s).

Prints one JSON line.  `value` is the effective KV-cache read bandwidth of the
whole step (sum of seq_len x KV heads x head_dim x 2 bytes x 2 (K and V),
divided by the step time), with every input already resident in HBM.
`roofline` is the phase-1 kernel (the dominant one) timed with HIP events on
the launch stream.  `cpu_baseline` is the fp64 CPU oracle timed on this host.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0       # MI355X dense f16/bf16 MFMA
COUNTERS = os.path.join(ROOT, "profiles", "pa_phase1_kernel_long-4x102400_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "gqa_aware_paged_amd", "csrc", f)
                  for f in ("pa_kernels.h", "pa_stream.h", "pagedattn.hip")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def elapsed_ms(self, a: int, b: int) -> float:
        assert self.hip.hipEventSynchronize(ctypes.c_void_p(b)) == 0
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                            ctypes.c_void_p(b)) == 0
        return ms.value

    def destroy(self, ev: int):
        self.hip.hipEventDestroy(ctypes.c_void_p(ev))


def traffic_from_counters(units_bytes):
    """HBM bytes per phase-1 launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on different kernel sources."""
    if not os.path.exists(COUNTERS):
        return None
    c = json.load(open(COUNTERS))
    if c.get("kernel_sources_sha256_16") != kernel_hash():
        return None
    fetch = c["FETCH_SIZE_KiB_per_dispatch"] * 1024 * c["fetch_scale"]
    write = c["WRITE_SIZE_KiB_per_dispatch"] * 1024 * c["write_scale"]
    return fetch + write


def default_command(args) -> bool:
    """True when the run is the configuration the committed counters were taken on
    (the long workload with automatic partitions and the host-side length total)."""
    return (args.workload == "long" and args.partition_size == 0
            and args.single_pass_max_len is None and not args.per_query_head
            and not args.fused and not args.no_hint and args.num_cus == 0
            and args.head_dim == 256 and args.block_size == 16 and args.xcd_skew == 0
            and args.piece_cost == 0 and args.stream_walk == 0 and not args.head_sequential)


def read_ceiling(torch, pa, dev, w, gib: int = 4, reps: int = 10):
    """Read bandwidth the device delivers to phase 1's access pattern (the library's
    read probe): `gib` GiB read in order, and the same bytes as chunks of one
    (page, KV head) block each (block_size x head_dim x 2 bytes) in a random order,
    256 workgroups as in phase 1; median of `reps` timed launches each."""
    chunk = w.block_size * w.head_dim * 2
    if chunk not in (4096, 8192, 16384):
        return None
    n = (gib << 30) // chunk
    src = torch.empty(n * chunk, dtype=torch.uint8, device=dev).fill_(7)
    g = torch.Generator(device=dev).manual_seed(5)
    order = torch.randperm(n, generator=g, device=dev)
    sink = torch.empty(256, dtype=torch.int32, device=dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for name, o in (("contiguous_gbs", None), ("gather_gbs", order)):
        for _ in range(2):
            pa.read_probe(src, chunk, o, sink=sink)
        ms = []
        for _ in range(reps):
            start.record()
            pa.read_probe(src, chunk, o, sink=sink)
            stop.record()
            torch.cuda.synchronize()
            ms.append(start.elapsed_time(stop))
        res[name] = round(n * chunk / (sorted(ms)[reps // 2] * 1e-3) / 1e9, 1)
    del src, order
    torch.cuda.empty_cache()
    res.update({"bytes": n * chunk, "chunk_bytes": chunk, "workgroups": 256,
                "kernel": "pa_read_probe_kernel (nontemporal 16-byte loads, 1 KiB per "
                          "instruction, two chunks in flight per wave)"})
    log(f"read ceiling: contiguous {res['contiguous_gbs']} GB/s, "
        f"{chunk}-byte chunks shuffled {res['gather_gbs']} GB/s")
    return res


def cpu_baseline(w, nseqs: int):
    """Time the fp64 oracle (as it stands) on the first `nseqs` sequences, all heads."""
    import oracle
    seqs = list(range(min(nseqs, w.num_seqs)))
    kp, vp, bt, sl = w.host_pages(seqs)
    q = w.q[seqs].cpu()
    t0 = time.perf_counter()
    _, threads = oracle.decode(q, kp, vp, bt, sl, w.scale, w.dtype, return_threads=True)
    dt = time.perf_counter() - t0
    kvb = int(sl.astype("int64").sum()) * w.num_kv_heads * w.head_dim * 2 * 2
    full = w.kv_bytes / kvb
    return {"value": kvb / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(seqs)} of {w.num_seqs} sequences, all {w.num_heads} query heads, "
                      f"fp64 C oracle with OpenMP ({dt:.2f} s)",
            "seconds": dt, "us_per_step_extrapolated": dt * full * 1e6}


def prefill_units(w):
    """(new token, query head, key) triples of a prefill step: token n of a sequence
    with C cached tokens sees C + n + 1 keys.  Each costs 4 * head_dim flop (the
    q.k dot product and the p*v accumulation, a multiply and an add each)."""
    keys = 0
    for C, Q in zip(w.ctx.seq_lens_host.clip(0), w.q_lens_host):
        keys += int(Q) * int(C) + int(Q) * (int(Q) + 1) // 2
    return keys * w.ctx.num_heads


def run_prefill(args, torch, pa, workloads):
    """Chunked prefill over a paged context: one JSON line in TFLOP/s."""
    import numpy as np
    log("generating workload prefill")
    w = workloads.prefill_chunk(device="cuda", head_dim=args.head_dim, dtype=args.dtype,
                                block_size=args.block_size)
    c = w.ctx
    out = torch.empty_like(w.q)
    stream = torch.cuda.current_stream()

    def step():
        pa.prefill(w.q, w.k_new, w.v_new, c.key_cache, c.value_cache, c.block_tables,
                   c.seq_lens, w.query_start, c.scale, w.max_q_len, c.max_seq_len, out=out)

    settle_steps = settle(torch, step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    units = prefill_units(w)
    flops = units * 4 * c.head_dim
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"timed {args.steps} steps: {ms * 1e3:.1f} us/step, {tflops:.1f} TFLOP/s")
    rec = {
        "metric": "prefill attention TFLOP/s (causal chunk over a paged context), 1 GPU",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "ms_per_step": round(ms, 5), "us_per_step": round(ms * 1e3, 2),
        "timing": "hot", "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": c.dtype, "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": c.num_seqs,
                   "ctx_lens": f"all {int(c.seq_lens_host[0])}",
                   "q_lens": f"all {int(w.q_lens_host[0])}", "num_heads": c.num_heads,
                   "num_kv_heads": c.num_kv_heads, "head_dim": c.head_dim,
                   "block_size": c.block_size, "parallelism": "single GPU"},
        # the step is one launch of pa_prefill_kernel, timed with events on its stream
        "roofline": {"bound": "mfma", "kernel": "pa_prefill_kernel", "achieved": round(tflops, 2),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops_per_launch": flops,
                     "flops_per_unit": 4 * c.head_dim, "units_per_launch": units,
                     "avg_launch_us": round(ms * 1e3, 2)},
    }
    if not args.no_cpu:
        import oracle
        # sample: every head of the first 32 new tokens of sequence 0 (each sees the
        # whole cached context)
        r0 = int(w.query_start_host[0])
        rows = [(r0 + n, h) for n in range(32) for h in range(c.num_heads)]
        t0 = time.perf_counter()
        _, threads = oracle.prefill(w.q, w.k_new, w.v_new, c.key_cache, c.value_cache,
                                    c.block_tables_host, c.seq_lens_host, w.query_start_host,
                                    c.scale, c.dtype, rows=rows, return_threads=True)
        dt = time.perf_counter() - t0
        ctx0 = int(c.seq_lens_host[0])
        sample_flops = sum((ctx0 + n + 1) for n in range(32)) * c.num_heads * 4 * c.head_dim
        rec["cpu_baseline"] = {
            "value": sample_flops / dt / 1e12, "unit": "TFLOP/s",
            "cores": int(threads),
            "kind": "oracle",
            "sample": f"32 new tokens x {c.num_heads} heads of sequence 0 ({dt:.2f} s), fp64 C "
                      "oracle with OpenMP",
            "seconds": dt}
    print(json.dumps(rec), flush=True)


def settle(torch, step, ms: float) -> int:
    """Untimed steps of the workload itself until `ms` of wall time have passed.  For
    the first ~10-25 ms of a memory-bound workload on a freshly loaded MI355X the step
    times wander by up to 25 % before they settle (a fill kernel of the same duration
    does not remove it; the workload's own steps do), so the timed steps follow this."""
    n = 0
    t0 = time.perf_counter()
    while ms > 0 and time.perf_counter() - t0 < ms * 1e-3:
        step()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def copy_probe(args, torch, dev):
    """One device-to-device copy of a known size, for scaling the byte counters of a
    profiled run (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)."""
    if args.copy_probe_mib <= 0:
        return
    n = args.copy_probe_mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy probe: {n} bytes read, {n} bytes written")
    del src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="untimed steps of the workload for this long before the warmup "
                         "steps (0 = none)")
    ap.add_argument("--workload", default="long",
                    choices=["tiny", "batch", "long", "mixed", "saturation", "prefill"])
    ap.add_argument("--partition-size", type=int, default=0,
                    help="tokens per partition; 0 = automatic (one workgroup per CU)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the context timings (the plain call without the host-side "
                         "length total, the pages' explicit partition sizes)")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the read-ceiling measurement")
    ap.add_argument("--single-pass-max-len", type=int, default=None)
    ap.add_argument("--per-query-head", action="store_true",
                    help="ablation: one workgroup per query head (KV read once per query head)")
    ap.add_argument("--head-sequential", action="store_true",
                    help="ablation: the group's query heads taken one after another per tile")
    ap.add_argument("--stream-walk", type=int, default=0,
                    help="-1: one workgroup per piece instead of per-wave streams")
    ap.add_argument("--fused", action="store_true",
                    help="merge partitions inside phase 1 (atomic ticket) instead of a phase-2 launch")
    ap.add_argument("--head-dim", type=int, default=256,
                    help="long and prefill workloads only: head_dim for shape sweeps")
    ap.add_argument("--block-size", type=int, default=16,
                    help="long and prefill workloads only: block_size for shape sweeps")
    ap.add_argument("--dtype", default="f16", choices=["f16", "bf16"],
                    help="prefill workload only: element type")
    ap.add_argument("--no-hint", action="store_true",
                    help="do not pass the host-side total of seq_lens to the planner")
    ap.add_argument("--num-cus", type=int, default=0,
                    help="compute units assumed by the automatic choices (0 = 256)")
    ap.add_argument("--cpu-seqs", type=int, default=4,
                    help="sequences of the workload the CPU oracle is timed on")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--piece-cost", type=int, default=0,
                    help="balanced split: tiles a piece start counts as (0 = library default, "
                         "-1 = none)")
    ap.add_argument("--xcd-skew", type=int, default=0,
                    help="automatic splits: permille the even-XCD share of a pair takes "
                         "above the mean (0 = library default, -1 = equal shares)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one device copy of this size first (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path runs on a single MI355X and has no "
              "multi-GPU mode; use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.dtype != "f16" and args.workload != "prefill":
        print("--dtype applies to the prefill workload only; the decode workloads are f16",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gqa_aware_paged_amd as pa
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.lib()

    if args.workload == "prefill":
        copy_probe(args, torch, dev)
        run_prefill(args, torch, pa, workloads)
        return
    log(f"generating workload {args.workload}")
    if args.workload == "long":
        w = workloads.long_context(device="cuda", head_dim=args.head_dim,
                                   block_size=args.block_size)
    else:
        w = workloads.NAMED[args.workload](device="cuda")
    torch.cuda.synchronize()

    def decoder(P, hint=None):
        return pa.Decoder(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size,
                          w.max_blocks_per_seq, w.q.dtype, max_seq_len=w.max_seq_len,
                          partition_size=P, single_pass_max_len=args.single_pass_max_len,
                          num_cus=args.num_cus,
                          total_tokens_hint=total if hint is None else hint,
                          per_query_head=args.per_query_head, fused_combine=args.fused,
                          xcd_skew=args.xcd_skew, piece_cost=args.piece_cost,
                          stream_walk=args.stream_walk, head_sequential=args.head_sequential)

    P = args.partition_size
    # the caller knows its sequence lengths on the host: pass their sum
    total = 0 if args.no_hint else int(w.seq_lens_host.clip(0).astype("int64").sum())
    dec = decoder(P)
    info = pa.plan(list(w.seq_lens_host), w.num_heads, w.num_kv_heads, w.head_dim,
                   w.block_size, w.max_blocks_per_seq, w.max_seq_len, P,
                   single_pass_max_len=args.single_pass_max_len, num_cus=args.num_cus,
                   total_tokens_hint=total, per_query_head=args.per_query_head,
                   fused_combine=args.fused, xcd_skew=args.xcd_skew,
                   piece_cost=args.piece_cost, stream_walk=args.stream_walk,
                   head_sequential=args.head_sequential)
    log(f"plan: {info}")

    copy_probe(args, torch, dev)

    ev = HipEvents()
    stream = torch.cuda.current_stream(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def step(d, events=None):
        d(w.q, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale, events=events)

    def timed(d, n, with_events=False):
        """n back-to-back steps between events on the launch stream; returns ms/step and,
        with_events, the phase-1 durations (ms) from HIP events around each launch."""
        pairs = [(ev.create(), ev.create()) for _ in range(n)] if with_events else None
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(n):
            step(d, pairs[i] if pairs else None)
        stop.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / n
        ph1 = None
        if pairs:
            ph1 = [ev.elapsed_ms(a, b) for a, b in pairs]
            for a, b in pairs:
                ev.destroy(a)
                ev.destroy(b)
        return ms, ph1

    settle_steps = settle(torch, lambda: step(dec), args.settle_ms)
    for _ in range(args.warmup):
        step(dec)
    torch.cuda.synchronize()
    log(f"settle {settle_steps} steps ({args.settle_ms} ms), warmup done ({args.warmup} steps)")

    # timed region 1: K plain steps -> ms_per_step
    t0 = time.perf_counter()
    step_ms, _ = timed(dec, args.steps)
    wall = time.perf_counter() - t0
    # timed region 2: K steps with HIP events around each phase-1 launch
    step_ms_ev, ph1 = timed(dec, args.steps, with_events=True)
    ph1 = sorted(ph1)
    ph1_avg = sum(ph1) / len(ph1)
    log(f"timed {args.steps} steps: {step_ms * 1e3:.1f} us/step (wall {wall:.3f} s); with "
        f"phase-1 events {step_ms_ev * 1e3:.1f} us/step, phase-1 avg {ph1_avg * 1e3:.1f} us, "
        f"median {ph1[len(ph1) // 2] * 1e3:.1f} us")
    # timed region 3 (cold): each step alone, after a 1 GiB device write that evicts
    # the step's K/V from L2 and the 256 MB Infinity Cache; median over the steps
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(min(args.steps, 50)):
        flush.fill_(i & 255)
        start.record(stream)
        step(dec)
        stop.record(stream)
        torch.cuda.synchronize()
        cold.append(start.elapsed_time(stop))
    del flush
    cold_ms = sorted(cold)[len(cold) // 2]
    log(f"cold: median {cold_ms * 1e3:.1f} us/step over {len(cold)} steps")
    # context on the same inputs: the plain call (paged_attn_decode's defaults: no
    # host-side length total, so partition_size 0 is the length-balanced split) and
    # the pages' explicit partition sizes
    variants = {}
    if not args.no_variants:
        if total and P == 0:
            variants["plain_call"] = dict(P=0, hint=0)
        sweep = [256, 512, 1024] if args.workload == "mixed" else [512]
        for p in sweep:
            if p != P:
                variants[f"partition_{p}"] = dict(P=p, hint=total)
    variant_us = {}
    for name, v in variants.items():
        d = decoder(v["P"], v["hint"])
        for _ in range(args.warmup):
            step(d)
        ms, _ = timed(d, args.steps)
        variant_us[name] = round(ms * 1e3, 2)
        log(f"{name}: {ms * 1e3:.1f} us/step ({w.kv_bytes / (ms * 1e-3) / 1e9:.0f} GB/s)")
        del d
    ceiling = None if args.no_read_probe else read_ceiling(torch, pa, dev, w)

    # algorithmic bytes: one unit = one (token, KV head); it reads a K row and a V row
    units = int(w.seq_lens_host.clip(0).astype("int64").sum()) * w.num_kv_heads
    bytes_per_unit = 2 * w.head_dim * 2
    kv = units * bytes_per_unit
    assert kv == w.kv_bytes
    # the tiny and batch workloads' K/V fits (or nearly fits) in the caches, so their
    # headline is the cold step; the larger ones stream from HBM either way (hot)
    timing = "cold" if args.workload in ("tiny", "batch") else "hot"
    head_ms = cold_ms if timing == "cold" else step_ms
    eff = kv / (head_ms * 1e-3) / 1e9
    achieved = kv / (ph1_avg * 1e-3) / 1e9
    rec = {
        "metric": "decode attention us/step + effective KV-cache GB/s (% of HBM peak), 1 GPU",
        "value": round(eff, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "ms_per_step": round(head_ms, 5),
        "us_per_step": round(head_ms * 1e3, 2),
        "timing": timing,
        "us_per_step_hot": round(step_ms * 1e3, 2),
        "us_per_step_cold": round(cold_ms * 1e3, 2),
        "pct_hbm_peak": round(100 * eff / HBM_PEAK_GBS, 2),
        "us_per_step_variants": variant_us,
        "read_ceiling": ceiling,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs,
                   "seq_lens": "all 102400" if args.workload == "long" else
                   f"{int(w.seq_lens_host.min())}..{int(w.seq_lens_host.max())}",
                   "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size,
                   "partition_size": info["partition_size"],
                   "partition_size_arg": P,
                   "single_pass_max_len": info["single_pass_max_len"],
                   "split": "balanced" if info["balanced"] else "fixed partitions",
                   "xcd_skew_permille": info["xcd_skew"],
                   "piece_cost_tiles": info["piece_cost"] if info["balanced"] else None,
                   "grid": "per query head (ablation)" if args.per_query_head else
                   ("per KV head, heads in turn (ablation)" if args.head_sequential
                    else "per KV head"),
                   "walk": "per-wave streams" if info["stream"] else "workgroup per piece",
                   "combine": "fused in phase 1" if info["fused"] else
                   ("phase-2 kernel" if info["phase2_workgroups"] else "none (one pass)"),
                   "kv_bytes_per_step": kv, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm",
                     "kernel": "pa_phase1_stream_kernel" if info["stream"] else
                     ("pa_phase1_balanced_kernel" if info["balanced"] else "pa_phase1_kernel"),
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     # the committed counters cover the default command only
                     "traffic": traffic_from_counters(kv) if default_command(args) else None,
                     "algorithmic_bytes_per_launch": kv, "bytes_per_unit": bytes_per_unit,
                     "units_per_launch": units,
                     "avg_launch_us": round(ph1_avg * 1e3, 2),
                     "frac_of_read_ceiling": None if not ceiling else
                     round(achieved / ceiling["gather_gbs"], 4)},
    }
    if not args.no_cpu:
        log(f"timing the CPU oracle on {min(args.cpu_seqs, w.num_seqs)} sequences")
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seqs)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
