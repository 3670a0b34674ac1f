"""GSA decode benchmark on one MI355X.

One step = one gsa_decode call (gist scoring, top-k select, unfolded
attention, merge) over one batch of the workload, with the caches already
resident in HBM.  Several copies of the caches are rotated so that no call
finds the previous call's bytes in the 256 MB Infinity Cache (the copies
together are far larger than it).

Prints one JSON line: queries/s (batch x q-heads per second), algorithmic
HBM GB/s against the 8 TB/s peak, and the CPU oracle on the host cores as a
reported baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np
import torch

import long_context_sparse_gist_amd as gsa
from long_context_sparse_gist_amd import inputs as gi

HBM_PEAK_GBPS = 8000.0
METRIC = "GSA decode queries/sec (batch\u00d7q-heads) and achieved HBM GB/s vs peak at 128K ctx"
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL = "gsa_fused_kernel"
# sources of the single-launch kernel: measured HBM traffic is reported only
# while they are unchanged since the counters were taken
KERNEL_SOURCES = ["fused.hip", "gsa_internal.h", "gsa_lists.h", "gsa_mfma_core.h", "gsa_select.h"]


def kernel_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "long_context_sparse_gist_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter profile of this
    workload, or None if it is missing or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{KERNEL}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_hash():
        return None
    return t["bytes_per_launch"]


def alg_bytes(wl: gi.Workload) -> int:
    """Bytes the method must read per call: every attended gist K/V, the
    selected chunks' raw K/V (H-GSA: meta K/V, candidate gist K, selected gist
    V) plus q and the output."""
    e, d, G = wl.elem_bytes, wl.head_dim, wl.group
    units = wl.batch * wl.num_kv_heads
    M, C, k = wl.num_chunks, wl.chunk_size, wl.top_k
    if wl.hgsa:
        Mm, R, k1 = wl.num_meta, wl.gists_per_meta, wl.top_k_meta
        per = e * d * (2 * Mm + k1 * R + k + 2 * k * C) + 2 * G * d * e
    else:
        per = e * d * (2 * M + 2 * k * C) + 2 * G * d * e
    return units * per


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=gi.QWEN7B_128K.name, choices=sorted(gi.BY_NAME))
    ap.add_argument("--score", default="sum_logits", choices=["sum_logits", "sum_probs"],
                    help="group routing key (flat GSA): sum of the heads' logits, or of their "
                         "softmax probabilities over the gists (multi-launch kernels)")
    ap.add_argument("--top-p", type=float, default=0.0,
                    help="top-p selection with this probability mass, top_k as its cap "
                         "(flat GSA, multi-launch kernels); 0: top-k")
    ap.add_argument("--copies", type=int, default=6,
                    help="cache copies rotated between calls (defeats the Infinity Cache)")
    ap.add_argument("--cpu-baseline", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="before timing, run 5 plain device copies of this many bytes "
                         "(the reference kernel for scaling HBM byte counters)")
    return ap.parse_args()


def cpu_baseline(inp, seconds: float, flags: int = 0, top_p: float = 0.0):
    """The oracle, as it stands, on the host cores: the whole batch, repeated
    until `seconds` of wall time (at least one run)."""
    import oracle
    from tests import _util as U  # oracle glue (storage formats only)
    wl = inp.wl
    q = U.np_raw(inp.q)
    kc = U.np_raw(inp.k_cache)
    vc = U.np_raw(inp.v_cache)
    bt = U.np_raw(inp.block_table)
    sl = U.np_raw(inp.seq_lens)
    cfg = U.cfg_of(inp, flags=flags | (oracle.SELECT_TOP_P if top_p > 0.0 else 0), top_p=top_p)
    threads = oracle.max_threads()
    times = []
    t_end = time.perf_counter() + seconds
    while True:
        t0 = time.perf_counter()
        if wl.hgsa:
            oracle.hgsa_decode(cfg, q, kc, vc, bt, sl, U.np_raw(inp.k_meta), U.np_raw(inp.v_meta))
        else:
            oracle.gsa_decode(cfg, q, kc, vc, bt, sl)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() > t_end or len(times) >= 50:
            break
    t = statistics.median(times)
    queries = wl.batch * wl.num_q_heads
    return {"value": queries / t, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"whole batch of the workload ({queries} queries), median of "
                      f"{len(times)} runs, OpenMP over (batch, kv-head) units"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the decode path has "
              f"no multi-GPU mode in this build", file=sys.stderr)
        sys.exit(2)
    wl = gi.BY_NAME[args.workload]
    flags = 0
    if args.score == "sum_probs":
        if wl.hgsa or wl.dtype != gi.BF16:
            print("--score sum_probs applies to the flat bf16 workloads", file=sys.stderr)
            sys.exit(2)
        flags = gsa.GSA_SCORE_SUM_PROBS
    if args.top_p > 0.0 and (wl.hgsa or flags):
        print("--top-p applies to the flat workloads with the default key", file=sys.stderr)
        sys.exit(2)
    # one launch per call (the bf16 default key, top-k); else the multi-launch kernels
    single = wl.dtype == gi.BF16 and flags == 0 and args.top_p == 0.0
    idx = gi.WORKLOADS.index(wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gsa.lib()

    inp = gi.make_inputs(wl, gi.seed_of(idx), device=dev)
    copies = [inp]
    for _ in range(max(1, args.copies) - 1):
        copies.append(gi.GsaInputs(wl, inp.q, inp.k_cache.clone(), inp.v_cache.clone(),
                                   inp.block_table, inp.seq_lens, inp.planted,
                                   None if inp.k_meta is None else inp.k_meta.clone(),
                                   None if inp.v_meta is None else inp.v_meta.clone()))
    out = torch.empty_like(inp.q)
    stream = torch.cuda.current_stream(dev)

    # one prepared call per cache copy: arguments are marshalled once, so the
    # host enqueues faster than the device runs a call
    def prepare(c):
        if wl.hgsa:
            return gsa.prepare_hgsa_decode(
                c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, c.k_meta, c.v_meta,
                num_chunks=wl.num_chunks, chunk_size=wl.chunk_size, page_chunks=wl.page_chunks,
                gists_per_meta=wl.gists_per_meta, top_k_meta=wl.top_k_meta, top_k=wl.top_k,
                out=out, stream=stream)
        return gsa.prepare_gsa_decode(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens,
                                      num_chunks=wl.num_chunks, chunk_size=wl.chunk_size,
                                      page_chunks=wl.page_chunks, top_k=wl.top_k, out=out,
                                      flags=flags, top_p=args.top_p, stream=stream)
    calls = [prepare(c) for c in copies]

    def step(i):
        calls[i % len(calls)]()

    if args.copy_calib > 0:
        n = args.copy_calib // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly `steps` calls, bracketed by device syncs; one HIP
    # event pair on the launch stream gives the device time per launch (the
    # host enqueues faster than the device runs, so launches run back to back)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_call_s = e0.elapsed_time(e1) / 1e3 / args.steps

    # spread of single launches, each between its own events (after the timed region)
    n_spread = min(50, args.steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_spread)]
    for i in range(n_spread):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(b) for a, b in ev]

    queries = wl.batch * wl.num_q_heads
    nbytes = alg_bytes(wl)
    if args.top_p > 0.0:
        # top-p keeps a different number of chunks per unit: count them
        sel = torch.full((wl.batch, wl.num_kv_heads, wl.top_k), -1, dtype=torch.int32, device=dev)
        gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens,
                       num_chunks=wl.num_chunks, chunk_size=wl.chunk_size,
                       page_chunks=wl.page_chunks, top_k=wl.top_k, top_p=args.top_p, sel_idx=sel)
        kept = int((sel >= 0).sum().item())
        units = wl.batch * wl.num_kv_heads
        e, d, G = wl.elem_bytes, wl.head_dim, wl.group
        nbytes = units * (e * d * 2 * wl.num_chunks + 2 * G * d * e) + kept * 2 * wl.chunk_size * d * e
    ms_per_step = wall / args.steps * 1e3
    value = queries * args.steps / wall
    achieved = nbytes / mean_call_s / 1e9
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == gi.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "q_heads": wl.num_q_heads,
                   "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "context_tokens": wl.raw_tokens, "chunk_size": wl.chunk_size,
                   "top_k": wl.top_k, "page_chunks": wl.page_chunks,
                   "score": args.score, "top_p": args.top_p or None,
                   "cache_copies": len(copies)},
        "hbm_gbps_alg": achieved,
        "launch_us": mean_call_s * 1e6,
        "single_launch_us": {"mean": statistics.fmean(call_ms) * 1e3,
                    "median": statistics.median(call_ms) * 1e3,
                    "p10": float(np.percentile(call_ms, 10)) * 1e3,
                    "p90": float(np.percentile(call_ms, 90)) * 1e3},
        "roofline": {"bound": "hbm", "kernel": KERNEL if single else
                     ("hgsa_decode launches" if wl.hgsa else "gsa_decode launches (multi-launch)"),
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(wl.name) if single and not wl.hgsa else None,
                     "alg_bytes_per_launch": nbytes, "kernel_hash": kernel_hash()},
    }
    if args.cpu_baseline:
        del copies, calls
        torch.cuda.empty_cache()
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, flags, args.top_p)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
