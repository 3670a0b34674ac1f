"""GPU-side glue for the parity tests: run the library through its C ABI and
compare with the oracle under the selection gap rule.

Gap rule (one selection per (batch, kv-head)): with the oracle's keys sorted
descending, if S_(k) - S_(k+1) > GAP the GPU's set must equal the oracle's;
otherwise every GPU-selected key must be >= S_(k) - GAP and every unselected
key <= S_(k+1) + GAP, and outputs are compared with the oracle rerun on the
GPU's set.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import long_context_sparse_gist_amd as gsa
from long_context_sparse_gist_amd import inputs as gi
from tests import _util as U

GAP = 1e-3
TOL = {gi.BF16: (2e-2, 1e-2), gi.F32: (1e-4, 1e-4)}   # (atol, rtol)
KEY_TOL = (1e-3, 1e-4)
# sum-of-probabilities keys are probabilities: relative tolerance, and the gap
# rule applies to the keys divided by the unit's largest key
KEY_TOL_PROBS = (1e-7, 1e-3)


def to(inp, device):
    f = {}
    for fld in dataclasses.fields(inp):
        v = getattr(inp, fld.name)
        f[fld.name] = v.to(device) if isinstance(v, torch.Tensor) else v
    return gi.GsaInputs(**f)


def run_gpu(inp, top_k=None, flags=0, sm_scale=0.0, want_scores=True, top_p=0.0):
    wl = inp.wl
    k = wl.top_k if top_k is None else top_k
    B, Hkv = wl.batch, wl.num_kv_heads
    dev = inp.q.device
    sel = torch.full((B, Hkv, k), -7, dtype=torch.int32, device=dev)
    sc = torch.full((B, Hkv, wl.num_chunks), 7.0, dtype=torch.float32, device=dev) \
        if want_scores else None
    out = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens,
                         num_chunks=wl.num_chunks, chunk_size=wl.chunk_size,
                         page_chunks=wl.page_chunks, top_k=k, sm_scale=sm_scale, flags=flags,
                         top_p=top_p,
                         sel_idx=sel, scores=sc)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy(), sel.cpu().numpy(),
            None if sc is None else sc.cpu().numpy())


def run_gpu_h(inp, top_k=None, top_k_meta=None, flags=0):
    wl = inp.wl
    k2 = wl.top_k if top_k is None else top_k
    k1 = wl.top_k_meta if top_k_meta is None else top_k_meta
    B, Hkv = wl.batch, wl.num_kv_heads
    dev = inp.q.device
    s1 = torch.full((B, Hkv, k1), -7, dtype=torch.int32, device=dev)
    s2 = torch.full((B, Hkv, k2), -7, dtype=torch.int32, device=dev)
    out = gsa.hgsa_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens,
                          inp.k_meta, inp.v_meta, num_chunks=wl.num_chunks,
                          chunk_size=wl.chunk_size, page_chunks=wl.page_chunks,
                          gists_per_meta=wl.gists_per_meta, top_k_meta=k1, top_k=k2,
                          flags=flags, sel_meta=s1, sel_idx=s2)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), s1.cpu().numpy(), s2.cpu().numpy()


def check_set(gpu_sel, keys, k, ids=None):
    """Gap rule for one unit.  keys: the oracle's float keys of the candidates
    (ids: their chunk ids, default 0..n-1).  Returns True when the GPU set
    equals the oracle's, False when it differs but is valid; asserts otherwise."""
    keys = np.asarray(keys, np.float64)
    n = len(keys)
    ids = np.arange(n) if ids is None else np.asarray(ids)
    keff = min(k, n)
    got = np.asarray(gpu_sel[:keff])
    assert np.all(np.asarray(gpu_sel[keff:]) == -1), "unused selection slots must be -1"
    assert np.all(np.diff(got) > 0), "selection must be strictly ascending"
    want = U.np_topk(keys, k, ids)
    if np.array_equal(got, want):
        return True
    assert keff < n
    order = np.sort(keys)[::-1]
    sk, sk1 = order[keff - 1], order[keff]
    assert sk - sk1 <= GAP, f"clear gap {sk - sk1:.3g} but the sets differ"
    pos = {int(m): i for i, m in enumerate(ids)}
    chosen = np.zeros(n, bool)
    for m in got:
        chosen[pos[int(m)]] = True
    assert np.all(keys[chosen] >= sk - GAP) and np.all(keys[~chosen] <= sk1 + GAP)
    return False


def assert_close(gpu, ref, dtype, what=""):
    atol, rtol = TOL[dtype]
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                           f"max abs err {err.max():.3g}")


def unit_inputs(inp, b, g):
    """The inputs of unit (b, g) alone: batch 1, one kv-head, its G query heads
    and only the pages sequence b maps (pure indexing)."""
    wl = inp.wl
    G = wl.group
    bt = inp.block_table[b].long()
    kc = inp.k_cache[bt, g:g + 1].contiguous()
    vc = inp.v_cache[bt, g:g + 1].contiguous()
    wl1 = wl.replace(batch=1, num_q_heads=G, num_kv_heads=1)
    q = inp.q[b:b + 1, g * G:(g + 1) * G].contiguous()
    btn = torch.arange(bt.numel(), dtype=torch.int32, device=bt.device).view(1, -1)
    km = vm = None
    if inp.k_meta is not None:
        km = inp.k_meta[b:b + 1, g:g + 1].contiguous()
        vm = inp.v_meta[b:b + 1, g:g + 1].contiguous()
    return gi.GsaInputs(wl1, q, kc, vc, btn, inp.seq_lens[b:b + 1].clone(),
                        inp.planted[b:b + 1, g:g + 1], km, vm)


def check_gsa(inp, gpu_res, units=None, top_k=None, flags=0, sm_scale=0.0):
    """Compare a GPU run with the oracle on `units` (default: all).
    Returns the number of units whose set differed within the gap rule."""
    wl = inp.wl
    out, sel, sc = gpu_res
    k = wl.top_k if top_k is None else top_k
    G = wl.group
    if units is None:
        units = [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    differ = 0
    for b, g in units:
        sub = to(unit_inputs(inp, b, g), "cpu")
        o_out, o_sel, o_sc = U.run_oracle(sub, top_k=k, flags=flags, sm_scale=sm_scale)
        n = int(sub.seq_lens[0]) // wl.chunk_size
        probs = bool(flags & gsa.GSA_SCORE_SUM_PROBS)
        if sc is not None:
            assert np.all(np.isneginf(sc[b, g, n:]))
            atol, rtol = KEY_TOL_PROBS if probs else KEY_TOL
            d = np.abs(sc[b, g, :n].astype(np.float64) - o_sc[0, 0, :n])
            assert np.all(d <= atol + rtol * np.abs(o_sc[0, 0, :n])), \
                f"unit {(b, g)}: key error {d.max():.3g}"
        gk = o_sc[0, 0, :n].astype(np.float64)
        if probs and n:
            gk = gk / max(float(np.max(gk)), 1e-30)
        same = check_set(sel[b, g], gk, k)
        if not same:
            differ += 1
            o_out, _, _ = U.run_oracle(sub, top_k=k, flags=flags, sm_scale=sm_scale,
                                       ext_sel=sel[b:b + 1, g:g + 1])
        assert_close(out[b, g * G:(g + 1) * G], o_out[0], wl.dtype, f"unit {(b, g)}")
    return differ


TOL_P = 1e-4  # top-p: running sums within this of p may fall either way


def check_gsa_topp(inp, gpu_res, p, cap, units=None):
    """Top-p: the GPU's count must be a valid cut of the oracle's running sum
    of selection probabilities (exactly the oracle's where p is clear of the
    sums on both sides), its set the top entries by key (gap rule), and the
    output the oracle's on the GPU's set."""
    import oracle
    wl = inp.wl
    out, sel, sc = gpu_res
    G = wl.group
    if units is None:
        units = [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    for b, g in units:
        sub = to(unit_inputs(inp, b, g), "cpu")
        _, o_sel, o_sc = U.run_oracle(sub, top_k=cap, flags=oracle.SELECT_TOP_P, top_p=p)
        n = int(sub.seq_lens[0]) // wl.chunk_size
        kk = min(cap, n)
        got = [int(x) for x in sel[b, g] if x >= 0]
        N = len(got)
        assert np.all(sel[b, g][N:] == -1), f"unit {(b, g)}: -1 padding"
        keys = o_sc[0, 0, :n].astype(np.float64)
        if n:
            order = sorted(range(n), key=lambda i: (-keys[i], i))
            w = np.exp(keys - keys.max())
            cum = np.cumsum(w[order] / w.sum())
            assert 1 <= N <= kk, f"unit {(b, g)}: count {N}"
            assert N == 1 or cum[N - 2] < p + TOL_P, f"unit {(b, g)}: kept past p"
            assert cum[N - 1] >= p - TOL_P or N == kk, f"unit {(b, g)}: stopped before p"
            want = [int(x) for x in o_sel[0, 0] if x >= 0]
            lo = cum[len(want) - 2] if len(want) >= 2 else 0.0
            clear = (p - lo > TOL_P) and (cum[len(want) - 1] - p > TOL_P or len(want) == kk)
            if clear:
                assert N == len(want), f"unit {(b, g)}: count {N}, oracle {len(want)}"
            check_set(np.array(got, np.int32), keys, N)
        else:
            assert N == 0
        o_out, _, _ = U.run_oracle(sub, top_k=cap, ext_sel=sel[b:b + 1, g:g + 1])
        assert_close(out[b, g * G:(g + 1) * G], o_out[0], wl.dtype, f"unit {(b, g)}")


def check_hgsa(inp, gpu_res, units=None, top_k=None, top_k_meta=None):
    wl = inp.wl
    out, s1, s2 = gpu_res
    k2 = wl.top_k if top_k is None else top_k
    k1 = wl.top_k_meta if top_k_meta is None else top_k_meta
    G, R = wl.group, wl.gists_per_meta
    if units is None:
        units = [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    differ = 0
    for b, g in units:
        sub = to(unit_inputs(inp, b, g), "cpu")
        kw = dict(top_k=k2, top_k_meta=k1)
        o_out, o_s1, o_s2, o_ms, o_gs = U.run_oracle_h(sub, **kw)
        n = int(sub.seq_lens[0]) // wl.chunk_size
        nm = n // R
        same1 = check_set(s1[b, g], o_ms[0, 0, :nm], k1)
        ext1 = None if same1 else s1[b:b + 1, g:g + 1]
        if ext1 is not None:
            o_out, o_s1, o_s2, o_ms, o_gs = U.run_oracle_h(sub, ext_sel_meta=ext1, **kw)
        kept = [int(r) for r in s1[b, g] if r >= 0]
        cand = np.array([r * R + j for r in kept for j in range(R)] +
                        list(range(nm * R, n)), np.int64)
        same2 = check_set(s2[b, g], o_gs[0, 0, cand], k2, ids=cand)
        if not (same1 and same2):
            differ += 1
            o_out, *_ = U.run_oracle_h(sub, ext_sel_meta=s1[b:b + 1, g:g + 1],
                                       ext_sel=s2[b:b + 1, g:g + 1], **kw)
        assert_close(out[b, g * G:(g + 1) * G], o_out[0], wl.dtype, f"unit {(b, g)}")
    return differ
