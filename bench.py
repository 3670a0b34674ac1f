"""GSA decode benchmark on one MI355X.

One step = one decode call (gist scoring, top-k select, unfolded attention,
merge; for the hierarchy workloads every level's scoring and select) over one
batch of the workload, with the caches already resident in HBM.  Several
copies of the caches are rotated so that no call finds the previous call's
bytes in the 256 MB Infinity Cache (the copies together are far larger).

Prints one JSON line: queries/s (batch x q-heads per second), algorithmic HBM
GB/s against the 8 TB/s peak and against a device copy measured in the same
run, and the CPU oracle on the host cores (single thread and all threads) as a
reported baseline.  --level-sweep instead prints one JSON line per (context
length, hierarchy depth): bytes per query and time per call from 128K to 16M
tokens.
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
METRIC = "GSA decode queries/sec (batch×q-heads) and achieved HBM GB/s vs peak at 128K ctx"
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


def alg_bytes(wl: gi.Workload, selected_gists: bool = False) -> int:
    """Bytes the method must read per call: every attended gist K/V, the
    selected chunks' raw K/V (H-GSA: meta K/V, candidate gist K, selected gist
    V) plus q and the output.  Selected-gists set: the gists' K (scoring) and
    the selected chunks' gist V and raw K/V."""
    e, d, G = wl.elem_bytes, wl.head_dim, wl.group
    units = wl.batch * wl.num_kv_heads
    M, C, k = wl.num_chunks, wl.chunk_size, wl.top_k
    if wl.hgsa:
        Mm, R, k1 = wl.num_meta, wl.gists_per_meta, wl.top_k_meta
        per = e * d * (2 * Mm + k1 * R + k + 2 * k * C) + 2 * G * d * e
    elif selected_gists:
        per = e * d * (M + 2 * k * (C + 1)) + 2 * G * d * e
    else:
        per = e * d * (2 * M + 2 * k * C) + 2 * G * d * e
    return units * per


def alg_bytes_levels(wl: gi.Workload, fanouts, tops) -> int:
    """Bytes a hierarchy call must read: K and V of every top-level entry; at
    each level below, K of its candidates (the kept entries' children) and V of
    its kept entries (their K was read as candidates); the kept chunks' raw K/V;
    q and the output.  Full-length sequences (no entries past a last group)."""
    e, d, G, C = wl.elem_bytes, wl.head_dim, wl.group, wl.chunk_size
    cnt = [wl.num_chunks] + gi.level_sizes(wl.num_chunks, fanouts)
    ks = [wl.top_k] + list(tops)
    L = len(fanouts)
    rows = 2 * cnt[L]
    for l in range(L - 1, -1, -1):
        kept_above = min(ks[l + 1], cnt[l + 1])
        cand = kept_above * fanouts[l]
        rows += cand + min(ks[l], cand)
    rows += 2 * min(ks[0], cnt[0] if L == 0 else min(ks[1], cnt[1]) * fanouts[0]) * C
    return wl.batch * wl.num_kv_heads * (e * d * rows + 2 * G * d * e)


def prefill_flops(wl: gi.Workload, T: int, q_start: int) -> int:
    """Multiply-add flops of one prefill step: per query head 2*d for the score
    and 2*d for the weighted value of every key its mask admits (the gists of
    earlier chunks and its own chunk's slots up to itself)."""
    C = wl.chunk_size
    s = np.arange(q_start, q_start + T)
    keys = s // (C + 1) + s % (C + 1) + 1
    return int(keys.sum()) * 4 * wl.head_dim * wl.num_q_heads * wl.batch


def prefill_bench(args, step, dev):
    """Time gsa_prefill on the last `step.queries` slots of every sequence
    (bound: bf16 MFMA; 2.5 PFLOP/s dense peak)."""
    wl, T = step.wl, step.queries
    cap = wl.num_chunks * (wl.chunk_size + 1)
    inp = gi.make_inputs_large(wl, 1500, dev)
    g = torch.Generator(device=dev).manual_seed(9)
    q = torch.randn(wl.batch, T, wl.num_q_heads, wl.head_dim, generator=g, device=dev).to(torch.bfloat16)
    qs = torch.full((wl.batch,), cap - T, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = torch.empty_like(q)
    caches = [(inp.k_cache, inp.v_cache)] + [(inp.k_cache.clone(), inp.v_cache.clone())
                                              for _ in range(max(1, args.copies) - 1)]
    calls = [gsa.prepare_gsa_prefill(q, k, v, inp.block_table, qs, chunk_size=wl.chunk_size,
                                     page_chunks=wl.page_chunks, out=out, stream=stream)
             for k, v in caches]
    for i in range(args.warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        calls[i % len(calls)]()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_s = e0.elapsed_time(e1) / 1e3 / args.steps
    flops = prefill_flops(wl, T, cap - T)
    achieved = flops / call_s / 1e12
    res = {"metric": "GSA prefill query-heads/sec under the gist causal mask (multi-query side)",
           "value": wl.batch * T * wl.num_q_heads * args.steps / wall, "unit": "query-heads/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": step.name, "batch": wl.batch, "q_heads": wl.num_q_heads,
                      "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                      "context_tokens": wl.raw_tokens, "chunk_size": wl.chunk_size,
                      "queries": T, "first_query_slot": cap - T, "cache_copies": len(caches)},
           "launch_us": call_s * 1e6,
           "roofline": {"bound": "mfma", "kernel": "prefill_kernel", "achieved": achieved,
                        "peak": 2500.0, "unit": "TFLOP/s", "frac": achieved / 2500.0,
                        "traffic": None, "flops_per_launch": flops}}
    if args.cpu_baseline:
        del calls, caches
        torch.cuda.empty_cache()
        import oracle
        from tests import _util as U
        cpu_q = q[:, :8].cpu()   # a bounded sample: the first 8 queries of every sequence
        cfg = U.cfg_of(inp, top_k=0)
        kc, vc, bt = U.np_raw(inp.k_cache), U.np_raw(inp.v_cache), U.np_raw(inp.block_table)
        st = np.full(wl.batch, cap - T, np.int32)
        times = []
        for _ in range(3):
            t1 = time.perf_counter()
            oracle.prefill(cfg, U.np_raw(cpu_q), kc, vc, bt, st)
            times.append(time.perf_counter() - t1)
        rows = wl.batch * 8 * wl.num_q_heads
        res["cpu_baseline"] = {"value": rows / statistics.median(times), "unit": "query-heads/s",
                               "cores": oracle.max_threads(), "kind": "oracle",
                               "sample": f"the first 8 queries of each sequence ({rows} query "
                                         f"heads), median of 3 runs, fp64, OpenMP over rows"}
    print(json.dumps(res), flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=gi.QWEN7B_128K.name,
                    choices=sorted(gi.BY_NAME) + sorted(gi.HIER_BY_NAME) + sorted(gi.PREFILL_BY_NAME))
    ap.add_argument("--score", default="sum_logits", choices=["sum_logits", "sum_probs"],
                    help="group routing key (flat GSA): sum of the heads' logits, or of their "
                         "softmax probabilities over the gists (multi-launch kernels)")
    ap.add_argument("--set", dest="attn_set", default="all_gists",
                    choices=["all_gists", "selected_gists"],
                    help="attention set (flat GSA): every gist plus the selected chunks' raw "
                         "tokens, or only the selected chunks' gists and raw tokens (SG+SR)")
    ap.add_argument("--top-p", type=float, default=0.0,
                    help="top-p selection with this probability mass, top_k as its cap "
                         "(flat GSA, multi-launch kernels); 0: top-k")
    ap.add_argument("--copies", type=int, default=6,
                    help="cache copies rotated between calls (defeats the Infinity Cache)")
    ap.add_argument("--cpu-baseline", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="wall time of each CPU baseline mode (single thread, all threads)")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="before timing, run 5 plain device copies of this many bytes "
                         "(the reference kernel for scaling HBM byte counters)")
    ap.add_argument("--level-sweep", action="store_true",
                    help="time the hierarchy at depths 0-3 over contexts of 128K to 16M tokens "
                         "(one JSON line each) instead of the benchmark")
    return ap.parse_args()


def copy_peak_gbps(dev, nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Read+write GB/s of a plain device-to-device copy of nbytes, the best of
    `reps` (each timed with events on the current stream)."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        best = max(best, 2 * nbytes / (a.elapsed_time(b) / 1e3) / 1e9)
    del src, dst
    torch.cuda.empty_cache()
    return best


def cpu_baseline(inp, seconds: float, flags: int = 0, top_p: float = 0.0, hier=None):
    """The oracle, as it stands (fp64 accumulation), on the host cores: the
    whole batch, repeated until `seconds` of wall time (at least one run),
    single-threaded and with OpenMP over units on every host thread."""
    import oracle
    from tests import _util as U  # oracle glue (storage formats only)
    wl = inp.wl
    q, kc, vc = U.np_raw(inp.q), U.np_raw(inp.k_cache), U.np_raw(inp.v_cache)
    bt, sl = U.np_raw(inp.block_table), U.np_raw(inp.seq_lens)
    cfg = U.cfg_of(inp, flags=flags | (oracle.SELECT_TOP_P if top_p > 0.0 else 0), top_p=top_p)
    lv = None
    if hier is not None:
        lv = [(U.np_raw(k), U.np_raw(v), R, t) for k, v, R, t in hier]
    km = vm = None
    if inp.k_meta is not None:
        km, vm = U.np_raw(inp.k_meta), U.np_raw(inp.v_meta)

    def run(nthreads):
        if lv is not None:
            oracle.mgsa_decode(cfg, q, kc, vc, bt, sl, lv, nthreads=nthreads)
        elif km is not None:
            oracle.hgsa_decode(cfg, q, kc, vc, bt, sl, km, vm, nthreads=nthreads)
        else:
            oracle.gsa_decode(cfg, q, kc, vc, bt, sl, nthreads=nthreads)

    def timed(nthreads):
        times = []
        t_end = time.perf_counter() + seconds
        while True:
            t0 = time.perf_counter()
            run(nthreads)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() > t_end or len(times) >= 50:
                return statistics.median(times), len(times)

    threads = oracle.max_threads()
    queries = wl.batch * wl.num_q_heads
    t1, n1 = timed(1)
    tn, nn = timed(threads)
    return {"value": queries / tn, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "single_thread": queries / t1,
            "sample": f"whole batch of the workload ({queries} queries), fp64 accumulation; "
                      f"median of {nn} runs with OpenMP over (batch, kv-head) units on {threads} "
                      f"threads (value), median of {n1} runs on one thread (single_thread)"}


def level_sweep(dev):
    """Per context length (128K..16M tokens, one sequence, Hq 32 / Hkv 8, d 128,
    C 16) and depth (0..3 meta levels of fanout 16, keeping 32, 16, 8 going up,
    64 chunks unfolded): algorithmic bytes per query and time per call, each
    call timed alone with a 1 GiB buffer read before it (the caches' touched
    rows are not left in the Infinity Cache), and back to back."""
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for ctx in (1 << 17, 1 << 20, 1 << 22, 1 << 24):
        M = ctx // 16
        wl = gi.Workload(f"sweep-{ctx >> 10}k", gi.BF16, 1, 32, 8, 128, 16, M, 64, 16,
                         plant="align", plant_count=16)
        inp = gi.make_inputs_large(wl, 1100 + ctx.bit_length(), dev)
        for depth in range(4):
            fanouts = (16,) * depth
            tops = (32, 16, 8)[:depth]
            made = gi.make_levels(inp, fanouts, 1200 + depth) if depth else []
            lv = [(k, v, R, t) for (k, v), R, t in zip(made, fanouts, tops)]
            call = gsa.prepare_mgsa_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_table,
                                           inp.seq_lens, lv, num_chunks=M, chunk_size=16,
                                           page_chunks=16, top_k=64, stream=stream)
            for _ in range(3):
                call()
            torch.cuda.synchronize()
            cold = []
            for _ in range(10):
                float(flush.sum())
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                call()
                b.record(stream)
                torch.cuda.synchronize()
                cold.append(a.elapsed_time(b) * 1e3)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(20):
                call()
            b.record(stream)
            torch.cuda.synchronize()
            warm = a.elapsed_time(b) * 1e3 / 20
            nbytes = alg_bytes_levels(wl, fanouts, tops)
            queries = wl.batch * wl.num_q_heads
            print(json.dumps({"sweep": "hierarchy", "context_tokens": ctx, "levels": depth,
                              "fanouts": list(fanouts), "kept": [64] + list(tops),
                              "alg_bytes_per_query": nbytes / queries,
                              "us_per_call_cold_median": statistics.median(cold),
                              "us_per_call_back_to_back": warm,
                              "alg_gbps_cold": nbytes / (statistics.median(cold) * 1e3),
                              "units": wl.batch * wl.num_kv_heads}), flush=True)
            del call, lv, made
        del inp
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the decode path has "
              f"no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gsa.lib()
    if args.level_sweep:
        level_sweep(dev)
        return
    if args.workload in gi.PREFILL_BY_NAME:
        prefill_bench(args, gi.PREFILL_BY_NAME[args.workload], dev)
        return
    hier = gi.HIER_BY_NAME.get(args.workload)
    wl = hier.wl if hier is not None else gi.BY_NAME[args.workload]
    flags = 0
    if args.score == "sum_probs":
        if wl.hgsa or hier or wl.dtype != gi.BF16:
            print("--score sum_probs applies to the flat bf16 workloads", file=sys.stderr)
            sys.exit(2)
        flags = gsa.GSA_SCORE_SUM_PROBS
    if args.attn_set == "selected_gists":
        if wl.hgsa or hier:
            print("--set selected_gists applies to the flat workloads", file=sys.stderr)
            sys.exit(2)
        flags |= gsa.GSA_SET_SELECTED_GISTS
    if args.top_p > 0.0 and (wl.hgsa or hier or (flags & gsa.GSA_SCORE_SUM_PROBS)):
        print("--top-p applies to the flat workloads with the default key", file=sys.stderr)
        sys.exit(2)
    # one launch per call (the bf16 default key, flat or two-level; top-p and the
    # sum-of-probabilities key with the all-gists set while the flat grid -- max(gist slices, 1 + ceil(unfolded
    # blocks / 4)) tasks per unit -- is resident at once on 1024 slots and a unit
    # has at most 32 gist slices, as the library plans it); else the
    # multi-launch kernels
    single = hier is None and wl.dtype == gi.BF16
    if single and (args.top_p > 0.0 or (flags & gsa.GSA_SCORE_SUM_PROBS)):
        # (the sum-of-probabilities key likewise, up to 64 gist slices per unit)
        n_a = -(-wl.num_chunks // 256)
        cap2 = min(wl.top_k, wl.num_chunks) * wl.chunk_size + wl.chunk_size - 1
        need = 1 + -(-(-(-cap2 // 32)) // 4)
        single = not (flags & gsa.GSA_SET_SELECTED_GISTS) and not wl.hgsa \
            and n_a <= (32 if args.top_p > 0.0 else 64) \
            and wl.batch * wl.num_kv_heads * max(n_a, need) <= 1024
    seed = 1010 if hier is not None else gi.seed_of(gi.WORKLOADS.index(wl))
    peak_copy = copy_peak_gbps(dev)

    inp = gi.make_inputs(wl, seed, device=dev)
    levels = None
    if hier is not None:
        made = gi.make_levels(inp, hier.fanouts, seed + 1)
        levels = [(k, v, R, t) for (k, v), R, t in zip(made, hier.fanouts, hier.tops)]
    copies = [(inp, levels)]
    for _ in range(max(1, args.copies) - 1):
        c = gi.GsaInputs(wl, inp.q, inp.k_cache.clone(), inp.v_cache.clone(), inp.block_table,
                         inp.seq_lens, inp.planted,
                         None if inp.k_meta is None else inp.k_meta.clone(),
                         None if inp.v_meta is None else inp.v_meta.clone())
        lv = None if levels is None else [(k.clone(), v.clone(), R, t) for k, v, R, t in levels]
        copies.append((c, lv))
    out = torch.empty_like(inp.q)
    stream = torch.cuda.current_stream(dev)

    # one prepared call per cache copy: arguments are marshalled once, so the
    # host enqueues faster than the device runs a call
    def prepare(c, lv):
        if lv is not None:
            return gsa.prepare_mgsa_decode(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, lv,
                                           num_chunks=wl.num_chunks, chunk_size=wl.chunk_size,
                                           page_chunks=wl.page_chunks, top_k=wl.top_k, out=out,
                                           stream=stream)
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
    calls = [prepare(c, lv) for c, lv in copies]

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
    # event pair on the launch stream gives the device time per call (the
    # host enqueues faster than the device runs, so calls run back to back)
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

    # spread of single calls, each between its own events (after the timed region)
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
    if hier is not None:
        nbytes = alg_bytes_levels(wl, hier.fanouts, hier.tops)
    else:
        nbytes = alg_bytes(wl, bool(flags & gsa.GSA_SET_SELECTED_GISTS))
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
    if hier is not None:
        kname = "mgsa_decode launches"
    elif single:
        kname = KERNEL
    else:
        kname = "hgsa_decode launches" if wl.hgsa else "gsa_decode launches (multi-launch)"
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
                   "score": args.score, "set": args.attn_set, "top_p": args.top_p or None,
                   "levels": None if hier is None else {"fanouts": list(hier.fanouts),
                                                        "kept": list(hier.tops)},
                   "cache_copies": len(copies)},
        "hbm_gbps_alg": achieved,
        "launch_us": mean_call_s * 1e6,
        "single_launch_us": {"mean": statistics.fmean(call_ms) * 1e3,
                    "median": statistics.median(call_ms) * 1e3,
                    "p10": float(np.percentile(call_ms, 10)) * 1e3,
                    "p90": float(np.percentile(call_ms, 90)) * 1e3},
        "roofline": {"bound": "hbm", "kernel": kname,
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     # counters were taken for the default key and set of each single-launch
                     # workload (flat and two-level), not for the variants
                     "traffic": measured_traffic(wl.name)
                     if single and flags == 0 and args.top_p <= 0.0 and hier is None else None,
                     "alg_bytes_per_launch": nbytes, "kernel_hash": kernel_hash(),
                     "copy_peak_gbps": peak_copy, "frac_of_copy_peak": achieved / peak_copy},
    }
    if args.cpu_baseline:
        del copies, calls
        torch.cuda.empty_cache()
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, flags, args.top_p,
                                           hier=levels)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
