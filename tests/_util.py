"""Test glue: tensors -> oracle arrays, plus numpy fp64 brute-force references.

The brute-force functions here are independent of oracle/ (vectorised numpy,
written from the definitions: dot-product routing keys, top-k by sort, softmax
attention over a masked token set) and are what the oracle is pinned to.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def np_raw(t: torch.Tensor) -> np.ndarray:
    """torch tensor -> numpy in the oracle's storage format (bf16 as uint16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().double().numpy()


def cfg_of(inp, top_k=None, flags=0, sm_scale=0.0, top_k_meta=None, top_p=0.0) -> dict:
    wl = inp.wl
    c = dict(top_p=top_p, batch=wl.batch, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
             head_dim=wl.head_dim, top_k=wl.top_k if top_k is None else top_k,
             sm_scale=sm_scale, dtype=wl.dtype, flags=flags, num_chunks=wl.num_chunks,
             chunk_size=wl.chunk_size, page_chunks=wl.page_chunks, num_pages=inp.num_pages,
             max_pages=inp.block_table.shape[1])
    if inp.k_meta is not None:
        c.update(gists_per_meta=wl.gists_per_meta,
                 top_k_meta=wl.top_k_meta if top_k_meta is None else top_k_meta,
                 max_meta=inp.k_meta.shape[2])
    return c


# Oracle build the pins run against (a test may swap in a variant of it).
ORACLE_LIB = None


def run_oracle(inp, ext_sel=None, nthreads=0, **kw):
    c = cfg_of(inp, **kw)
    return oracle.gsa_decode(c, np_raw(inp.q), np_raw(inp.k_cache), np_raw(inp.v_cache),
                             np_raw(inp.block_table), np_raw(inp.seq_lens), ext_sel=ext_sel,
                             nthreads=nthreads, lib=ORACLE_LIB)


def run_oracle_h(inp, ext_sel_meta=None, ext_sel=None, nthreads=0, **kw):
    c = cfg_of(inp, **kw)
    return oracle.hgsa_decode(c, np_raw(inp.q), np_raw(inp.k_cache), np_raw(inp.v_cache),
                              np_raw(inp.block_table), np_raw(inp.seq_lens), np_raw(inp.k_meta),
                              np_raw(inp.v_meta), ext_sel_meta=ext_sel_meta, ext_sel=ext_sel,
                              nthreads=nthreads, lib=ORACLE_LIB)


# ---------------- numpy fp64 brute force ----------------

def tau_of(d: int, sm_scale: float = 0.0) -> float:
    return float(sm_scale) if sm_scale > 0 else float(np.float32(1.0 / np.sqrt(d)))


def logical(inp, which: str) -> np.ndarray:
    """Cache rows in logical slot order: fp64 [B][Hkv][max_pages*spp][d]."""
    cache = f64(inp.k_cache if which == "k" else inp.v_cache)
    bt = inp.block_table.cpu().numpy()
    Hkv, d = cache.shape[1], cache.shape[3]
    return np.stack([cache[bt[b]].transpose(1, 0, 2, 3).reshape(Hkv, -1, d)
                     for b in range(bt.shape[0])])


def shapes(inp):
    C = inp.wl.chunk_size
    L = inp.seq_lens.cpu().numpy().astype(np.int64)
    return L // C, L % C


def gist_slots(n: int, C: int) -> np.ndarray:
    return np.arange(n) * (C + 1) + C


def np_keys(inp, sm_scale=0.0, probs=False) -> list:
    """Routing keys per (b, g): list of float32 arrays of length n_b."""
    wl = inp.wl
    G, C = wl.group, wl.chunk_size
    tau = tau_of(wl.head_dim, sm_scale)
    q = f64(inp.q)
    K = logical(inp, "k")
    n, _ = shapes(inp)
    res = []
    for b in range(wl.batch):
        row = []
        for g in range(wl.num_kv_heads):
            kg = K[b, g, gist_slots(n[b], C)]                  # [n][d]
            z = tau * kg @ q[b, g * G:(g + 1) * G].T           # [n][G]
            if probs:
                z = z - z.max(axis=0, keepdims=True)
                p = np.exp(z) / np.exp(z).sum(axis=0, keepdims=True)
                row.append(p.sum(axis=1).astype(np.float32))
            else:
                row.append(z.sum(axis=1).astype(np.float32))
        res.append(row)
    return res


def np_topk(S: np.ndarray, k: int, ids=None) -> np.ndarray:
    """Top-k by (key desc, id asc), returned ascending."""
    ids = np.arange(len(S)) if ids is None else np.asarray(ids)
    order = np.lexsort((ids, -S.astype(np.float64)))
    return np.sort(ids[order[:min(k, len(S))]])


def gsa_mask(n: int, tail: int, C: int, sel, slots: int, all_gists=True) -> np.ndarray:
    m = np.zeros(slots, bool)
    if all_gists:
        m[gist_slots(n, C)] = True
    for c in sel:
        if c < 0:
            continue
        m[c * (C + 1): c * (C + 1) + C + 1] = True
    m[n * (C + 1): n * (C + 1) + tail] = True
    return m


def np_attend(qh: np.ndarray, K: np.ndarray, V: np.ndarray, tau: float) -> np.ndarray:
    """softmax(tau * K qh) V for one head over the given rows; zeros if empty."""
    if len(K) == 0:
        return np.zeros(qh.shape[-1])
    z = tau * K @ qh
    p = np.exp(z - z.max())
    return (p / p.sum()) @ V


def np_gsa_out(inp, sel, sm_scale=0.0, all_gists=True) -> np.ndarray:
    """Attention restricted to the set defined by `sel` ([B][Hkv][k])."""
    wl = inp.wl
    G, C = wl.group, wl.chunk_size
    tau = tau_of(wl.head_dim, sm_scale)
    q = f64(inp.q)
    K, V = logical(inp, "k"), logical(inp, "v")
    n, tail = shapes(inp)
    out = np.zeros(q.shape)
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            m = gsa_mask(n[b], tail[b], C, sel[b][g], K.shape[2], all_gists)
            for j in range(G):
                h = g * G + j
                out[b, h] = np_attend(q[b, h], K[b, g][m], V[b, g][m], tau)
    return out


def close(a, b, atol, rtol) -> bool:
    return bool(np.all(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))
                       <= atol + rtol * np.abs(np.asarray(b, np.float64))))
