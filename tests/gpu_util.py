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


_WS = {}


def checked_workspace(nbytes, device):
    """The parity tests' own workspace (zero-filled, grown as needed): every
    call made through run_gpu / run_gpu_h uses it, and check_control runs
    after each one."""
    t = _WS.get(str(device))
    if t is None or t.numel() < nbytes:
        t = torch.zeros(max(nbytes, gsa.WORKSPACE_CONTROL_BYTES), dtype=torch.uint8, device=device)
        _WS[str(device)] = t
    return t


def check_control(ws, what=""):
    """After a call has completed: no wait gave up (the error word reads 0
    through the ABI) and the control block is zero again."""
    st = gsa.gsa_workspace_status(ws)
    assert st == 0, f"{what}: gsa_workspace_status = {gsa.STATUS.get(st, st)}"
    nz = int(ws[:gsa.WORKSPACE_CONTROL_BYTES].count_nonzero())
    assert nz == 0, f"{what}: {nz} control-block bytes left non-zero"


def run_gpu(inp, top_k=None, flags=0, sm_scale=0.0, want_scores=True, top_p=0.0):
    wl = inp.wl
    k = wl.top_k if top_k is None else top_k
    B, Hkv = wl.batch, wl.num_kv_heads
    dev = inp.q.device
    sel = torch.full((B, Hkv, k), -7, dtype=torch.int32, device=dev)
    sc = torch.full((B, Hkv, wl.num_chunks), 7.0, dtype=torch.float32, device=dev) \
        if want_scores else None
    p = gsa.make_params(inp.q, Hkv, k, sm_scale, flags, top_p)
    kv = gsa.make_kv(inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens, wl.num_chunks,
                     wl.chunk_size, wl.page_chunks)
    ws = checked_workspace(gsa.gsa_workspace_size(p, kv), dev)
    out = gsa.gsa_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens,
                         num_chunks=wl.num_chunks, chunk_size=wl.chunk_size,
                         page_chunks=wl.page_chunks, top_k=k, sm_scale=sm_scale, flags=flags,
                         top_p=top_p, sel_idx=sel, scores=sc, ws=ws)
    torch.cuda.synchronize()
    check_control(ws, f"gsa_decode {wl.name}")
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
    p = gsa.make_params(inp.q, Hkv, k2, 0.0, flags)
    kv = gsa.make_kv(inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens, wl.num_chunks,
                     wl.chunk_size, wl.page_chunks)
    m = gsa.make_meta(inp.k_meta, inp.v_meta, wl.gists_per_meta, k1)
    ws = checked_workspace(gsa.hgsa_workspace_size(p, kv, m), dev)
    out = gsa.hgsa_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens,
                          inp.k_meta, inp.v_meta, num_chunks=wl.num_chunks,
                          chunk_size=wl.chunk_size, page_chunks=wl.page_chunks,
                          gists_per_meta=wl.gists_per_meta, top_k_meta=k1, top_k=k2,
                          flags=flags, sel_meta=s1, sel_idx=s2, ws=ws)
    torch.cuda.synchronize()
    check_control(ws, f"hgsa_decode {wl.name}")
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


def _cpu(inp):
    return inp if inp.q.device.type == "cpu" else to(inp, "cpu")


def _all_units(wl, units):
    if units is None:
        return [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    return units


def check_gsa(inp, gpu_res, units=None, top_k=None, flags=0, sm_scale=0.0):
    """Compare a GPU run with the oracle on `units` (default: every unit).
    The oracle runs on the whole batch (one host copy of the inputs): once with
    its own selection (keys, gap rule) and once with the GPU's selection, whose
    outputs every unit is compared with.  Returns the number of units whose
    set differed within the gap rule."""
    wl = inp.wl
    out, sel, sc = gpu_res
    k = wl.top_k if top_k is None else top_k
    G = wl.group
    cpu = _cpu(inp)
    _, _, o_sc = U.run_oracle(cpu, top_k=k, flags=flags, sm_scale=sm_scale)
    n_all, _ = U.shapes(cpu)
    probs = bool(flags & gsa.GSA_SCORE_SUM_PROBS)
    differ = 0
    units = _all_units(wl, units)
    for b, g in units:
        n = int(n_all[b])
        if sc is not None:
            assert np.all(np.isneginf(sc[b, g, n:]))
            atol, rtol = KEY_TOL_PROBS if probs else KEY_TOL
            d = np.abs(sc[b, g, :n].astype(np.float64) - o_sc[b, g, :n])
            assert np.all(d <= atol + rtol * np.abs(o_sc[b, g, :n])), \
                f"unit {(b, g)}: key error {d.max():.3g}"
        gk = o_sc[b, g, :n].astype(np.float64)
        if probs and n:
            gk = gk / max(float(np.max(gk)), 1e-30)
        differ += not check_set(sel[b, g], gk, k)
    e_out, _, _ = U.run_oracle(cpu, top_k=k, flags=flags, sm_scale=sm_scale,
                               ext_sel=np.ascontiguousarray(sel, np.int32))
    for b, g in units:
        assert_close(out[b, g * G:(g + 1) * G], e_out[b, g * G:(g + 1) * G], wl.dtype,
                     f"unit {(b, g)}")
    return differ


TOL_P = 1e-4      # top-p: the GPU's cut against running sums of its own keys
TOL_P_ORA = 3e-3  # top-p: how far p must lie from the oracle's running sums for
                  # the counts to agree (keys within KEY_TOL move sums by ~1e-3)


def _topp_sums(keys, n):
    order = sorted(range(n), key=lambda i: (-keys[i], i))
    w = np.exp(keys - keys.max())
    return order, np.cumsum(w[order] / w.sum())


def check_gsa_topp(inp, gpu_res, p, cap, units=None):
    """Top-p: the GPU's count must be a valid cut of the running sum of the
    selection probabilities made from its own keys, equal to the oracle's
    where p is clear of the oracle's sums on both sides of its cut, its set
    the top entries by key (gap rule on the oracle's keys), and the output the
    oracle's on the GPU's set."""
    import oracle
    wl = inp.wl
    out, sel, sc = gpu_res
    G = wl.group
    cpu = _cpu(inp)
    _, o_sel, o_sc = U.run_oracle(cpu, top_k=cap, flags=oracle.SELECT_TOP_P, top_p=p)
    n_all, _ = U.shapes(cpu)
    units = _all_units(wl, units)
    for b, g in units:
        n = int(n_all[b])
        kk = min(cap, n)
        got = [int(x) for x in sel[b, g] if x >= 0]
        N = len(got)
        assert np.all(sel[b, g][N:] == -1), f"unit {(b, g)}: -1 padding"
        keys = o_sc[b, g, :n].astype(np.float64)
        if n:
            assert 1 <= N <= kk, f"unit {(b, g)}: count {N}"
            if sc is not None:  # the cut on the GPU's own keys
                _, cum = _topp_sums(sc[b, g, :n].astype(np.float64), n)
                assert N == 1 or cum[N - 2] < p + TOL_P, f"unit {(b, g)}: kept past p"
                assert cum[N - 1] >= p - TOL_P or N == kk, f"unit {(b, g)}: stopped before p"
            _, cum = _topp_sums(keys, n)
            want = [int(x) for x in o_sel[b, g] if x >= 0]
            lo = cum[len(want) - 2] if len(want) >= 2 else 0.0
            clear = (p - lo > TOL_P_ORA) and (cum[len(want) - 1] - p > TOL_P_ORA or len(want) == kk)
            if clear:
                assert N == len(want), f"unit {(b, g)}: count {N}, oracle {len(want)}"
            check_set(np.array(got, np.int32), keys, N)
        else:
            assert N == 0
    e_out, _, _ = U.run_oracle(cpu, top_k=cap, ext_sel=np.ascontiguousarray(sel, np.int32))
    for b, g in units:
        assert_close(out[b, g * G:(g + 1) * G], e_out[b, g * G:(g + 1) * G], wl.dtype,
                     f"unit {(b, g)}")


def check_hgsa(inp, gpu_res, units=None, top_k=None, top_k_meta=None):
    """H-GSA: the gap rule at both levels (the gist level over the candidates
    of the GPU's kept meta-groups), outputs against the oracle run with the
    GPU's selections at both levels, for `units` (default: every unit)."""
    wl = inp.wl
    out, s1, s2 = gpu_res
    k2 = wl.top_k if top_k is None else top_k
    k1 = wl.top_k_meta if top_k_meta is None else top_k_meta
    G, R = wl.group, wl.gists_per_meta
    cpu = _cpu(inp)
    kw = dict(top_k=k2, top_k_meta=k1)
    _, _, _, o_ms, o_gs = U.run_oracle_h(cpu, **kw)
    n_all, _ = U.shapes(cpu)
    units = _all_units(wl, units)
    differ = 0
    for b, g in units:
        n = int(n_all[b])
        nm = n // R
        same1 = check_set(s1[b, g], o_ms[b, g, :nm], k1)
        kept = [int(r) for r in s1[b, g] if r >= 0]
        cand = np.array([r * R + j for r in kept for j in range(R)] +
                        list(range(nm * R, n)), np.int64)
        same2 = check_set(s2[b, g], o_gs[b, g, cand], k2, ids=cand)
        differ += not (same1 and same2)
    e_out, *_ = U.run_oracle_h(cpu, ext_sel_meta=np.ascontiguousarray(s1, np.int32),
                               ext_sel=np.ascontiguousarray(s2, np.int32), **kw)
    for b, g in units:
        assert_close(out[b, g * G:(g + 1) * G], e_out[b, g * G:(g + 1) * G], wl.dtype,
                     f"unit {(b, g)}")
    return differ


def run_gpu_m(inp, levels, top_k=None):
    """mgsa_decode through the C ABI with the checked workspace.  levels:
    [(k, v, fanout, top_k)] on the device.  Returns (out, sels[l] numpy)."""
    wl = inp.wl
    k0 = wl.top_k if top_k is None else top_k
    B, Hkv = wl.batch, wl.num_kv_heads
    dev = inp.q.device
    sels = [torch.full((B, Hkv, max(k, 0)), -7, dtype=torch.int32, device=dev)
            for k in [k0] + [t for _, _, _, t in levels]]
    p = gsa.make_params(inp.q, Hkv, k0)
    kv = gsa.make_kv(inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens, wl.num_chunks,
                     wl.chunk_size, wl.page_chunks)
    ws = checked_workspace(gsa.mgsa_workspace_size(p, kv, gsa.make_levels(levels), len(levels)), dev)
    out = gsa.mgsa_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens, levels,
                          num_chunks=wl.num_chunks, chunk_size=wl.chunk_size,
                          page_chunks=wl.page_chunks, top_k=k0, sel=sels, ws=ws)
    torch.cuda.synchronize()
    check_control(ws, f"mgsa_decode {wl.name}")
    return out.float().cpu().numpy(), [s.cpu().numpy() for s in sels]


def check_mgsa(inp, levels, gpu_res, top_k=None, units=None):
    """The hierarchy of any depth: the gap rule at every level (candidates: all
    top-level entries, below them the children of the GPU's kept entries one
    level up plus the entries past the level's last complete group), outputs
    against the oracle run with the GPU's selections at every level.
    Returns the number of units with a differing set at some level."""
    wl = inp.wl
    out, sels = gpu_res
    k0 = wl.top_k if top_k is None else top_k
    G, C = wl.group, wl.chunk_size
    L = len(levels)
    cpu = _cpu(inp)
    lv = [(U.np_raw(k), U.np_raw(v), R, t) for k, v, R, t in levels]
    cfg = U.cfg_of(cpu, top_k=k0)
    args = (U.np_raw(cpu.q), U.np_raw(cpu.k_cache), U.np_raw(cpu.v_cache),
            U.np_raw(cpu.block_table), U.np_raw(cpu.seq_lens))
    import oracle
    _, _, okeys = oracle.mgsa_decode(cfg, *args, lv)
    n_all, _ = U.shapes(cpu)
    tops = [k0] + [t for _, _, _, t in levels]
    Rs = [None] + [R for _, _, R, _ in levels]
    units = _all_units(wl, units)
    differ = 0
    for b, g in units:
        cnt = [int(n_all[b])]
        for R in Rs[1:]:
            cnt.append(cnt[-1] // R)
        cand = np.arange(cnt[L])
        same = True
        for l in range(L, -1, -1):
            same &= check_set(sels[l][b, g], okeys[l][b, g, cand], tops[l], ids=cand)
            if l > 0:
                kept = [int(r) for r in sels[l][b, g] if r >= 0]
                R = Rs[l]
                cand = np.array([r * R + j for r in kept for j in range(R)] +
                                list(range(cnt[l] * R, cnt[l - 1])), np.int64)
        differ += not same
    e_out, _, _ = oracle.mgsa_decode(cfg, *args, lv,
                                     ext=[np.ascontiguousarray(s, np.int32) for s in sels])
    for b, g in units:
        assert_close(out[b, g * G:(g + 1) * G], e_out[b, g * G:(g + 1) * G], wl.dtype,
                     f"unit {(b, g)}")
    return differ
