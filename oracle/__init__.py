"""ctypes front end of the CPU oracle (gsa_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It takes plain numpy
arrays (bf16 data as uint16 bit patterns) and knows nothing of the HIP path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

SCORE_SUM_PROBS = 0x1
SET_SELECTED_GISTS = 0x2
SELECT_TOP_P = 0x4


class OracleCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("batch", "num_q_heads", "num_kv_heads", "head_dim", "top_k")] + [
        ("sm_scale", ctypes.c_float)] + [(n, ctypes.c_int) for n in
        ("dtype", "flags", "num_chunks", "chunk_size", "page_chunks", "num_pages",
         "max_pages", "gists_per_meta", "top_k_meta", "max_meta")] + [
        ("top_p", ctypes.c_float)]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP over units)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        compile_source(_SRC, tmp)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def load(path: str) -> ctypes.CDLL:
    """Load an oracle build (the default one, or a test's variant of it)."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.gsa_oracle_decode.argtypes = [ctypes.POINTER(OracleCfg)] + [P] * 9 + [ctypes.c_int]
    lib.gsa_oracle_decode.restype = ctypes.c_int
    lib.hgsa_oracle_decode.argtypes = [ctypes.POINTER(OracleCfg)] + [P] * 14 + [ctypes.c_int]
    lib.hgsa_oracle_decode.restype = ctypes.c_int
    PP = ctypes.POINTER(ctypes.c_void_p)
    IP = ctypes.POINTER(ctypes.c_int)
    lib.mgsa_oracle_decode.argtypes = ([ctypes.POINTER(OracleCfg)] + [P] * 5 + [ctypes.c_int] +
                                       [PP, PP, IP, IP, IP, P, PP, PP, PP, ctypes.c_int])
    lib.mgsa_oracle_decode.restype = ctypes.c_int
    lib.gsa_prefill_oracle.argtypes = [ctypes.POINTER(OracleCfg)] + [P] * 5 + [ctypes.c_int, P,
                                                                            ctypes.c_int]
    lib.gsa_prefill_oracle.restype = ctypes.c_int
    lib.gsa_oracle_threads.restype = ctypes.c_int
    return lib


def compile_source(src: str, dst: str) -> str:
    """Compile oracle C source `src` into shared library `dst`."""
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                           "-Wall", "-Wno-unused-function", src, "-o", dst, "-lm"])
    return dst


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = load(_LIB)
    return _lib


def max_threads() -> int:
    return _load().gsa_oracle_threads()


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def _data(a, dtype):
    a = np.ascontiguousarray(a)
    want = np.float32 if dtype == 0 else np.uint16
    assert a.dtype == want, (a.dtype, want)
    return a


def _cfg(cfg: dict) -> OracleCfg:
    c = OracleCfg()
    for name, _ in OracleCfg._fields_:
        setattr(c, name, cfg.get(name, 0))
    return c


def gsa_decode(cfg: dict, q, k_cache, v_cache, block_table, seq_lens,
               ext_sel=None, nthreads: int = 0, lib=None):
    """Returns (out float64 [B][Hq][d], sel int32 [B][Hkv][top_k],
    scores float32 [B][Hkv][num_chunks])."""
    lib = lib or _load()
    c = _cfg(cfg)
    B, Hq, Hkv, d = c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim
    q, k_cache, v_cache = (_data(x, c.dtype) for x in (q, k_cache, v_cache))
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    es = _c(ext_sel, np.int32)
    out = np.zeros((B, Hq, d), np.float64)
    sel = np.zeros((B, Hkv, max(c.top_k, 0)), np.int32)
    sc = np.zeros((B, Hkv, c.num_chunks), np.float32)
    rc = lib.gsa_oracle_decode(ctypes.byref(c), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(bt), _ptr(sl), _ptr(out), _ptr(sel), _ptr(sc), _ptr(es),
                               nthreads)
    if rc:
        raise ValueError(f"oracle rejected the configuration (code {rc})")
    return out, sel, sc


def hgsa_decode(cfg: dict, q, k_cache, v_cache, block_table, seq_lens, k_meta, v_meta,
                ext_sel_meta=None, ext_sel=None, nthreads: int = 0, lib=None):
    """Returns (out, sel_meta [B][Hkv][k1], sel [B][Hkv][k2],
    meta_scores [B][Hkv][max_meta], gist_scores [B][Hkv][num_chunks])."""
    lib = lib or _load()
    c = _cfg(cfg)
    B, Hq, Hkv, d = c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim
    q, k_cache, v_cache, k_meta, v_meta = (_data(x, c.dtype) for x in
                                           (q, k_cache, v_cache, k_meta, v_meta))
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    e1 = _c(ext_sel_meta, np.int32)
    e2 = _c(ext_sel, np.int32)
    out = np.zeros((B, Hq, d), np.float64)
    s1 = np.zeros((B, Hkv, max(c.top_k_meta, 0)), np.int32)
    s2 = np.zeros((B, Hkv, max(c.top_k, 0)), np.int32)
    ms = np.zeros((B, Hkv, c.max_meta), np.float32)
    gs = np.zeros((B, Hkv, c.num_chunks), np.float32)
    rc = lib.hgsa_oracle_decode(ctypes.byref(c), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                _ptr(bt), _ptr(sl), _ptr(k_meta), _ptr(v_meta), _ptr(out),
                                _ptr(s1), _ptr(s2), _ptr(ms), _ptr(gs), _ptr(e1), _ptr(e2),
                                nthreads)
    if rc:
        raise ValueError(f"oracle rejected the configuration (code {rc})")
    return out, s1, s2, ms, gs


def _ptr_array(arrs):
    """ctypes array of data pointers (None -> NULL)."""
    return (ctypes.c_void_p * max(1, len(arrs)))(*[None if a is None else a.ctypes.data
                                                    for a in arrs])


def mgsa_decode(cfg: dict, q, k_cache, v_cache, block_table, seq_lens, levels,
                ext=None, nthreads: int = 0, lib=None):
    """Hierarchy of len(levels) meta-gist levels above the gists.  levels[l-1]
    = (k [B][Hkv][max][d], v, fanout, top_k) for level l = 1..L; cfg's top_k
    is the gist level's k.  ext: None or L + 1 arrays/None (level 0 first).
    Returns (out float64 [B][Hq][d], sels, keys): sels[l] int32
    [B][Hkv][k_l] ascending -1 padded, keys[l] float32 [B][Hkv][max_l] of
    every entry (level 0: [B][Hkv][num_chunks])."""
    lib = lib or _load()
    c = _cfg(cfg)
    B, Hq, Hkv, d = c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim
    L = len(levels)
    q, k_cache, v_cache = (_data(x, c.dtype) for x in (q, k_cache, v_cache))
    ks = [_data(lv[0], c.dtype) for lv in levels]
    vs = [_data(lv[1], c.dtype) for lv in levels]
    maxs = (ctypes.c_int * max(1, L))(*[k.shape[2] for k in ks])
    fans = (ctypes.c_int * max(1, L))(*[int(lv[2]) for lv in levels])
    tops = (ctypes.c_int * max(1, L))(*[int(lv[3]) for lv in levels])
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    out = np.zeros((B, Hq, d), np.float64)
    kk = [max(c.top_k, 0)] + [max(int(lv[3]), 0) for lv in levels]
    caps = [c.num_chunks] + [k.shape[2] for k in ks]
    sels = [np.zeros((B, Hkv, kk[l]), np.int32) for l in range(L + 1)]
    keys = [np.zeros((B, Hkv, caps[l]), np.float32) for l in range(L + 1)]
    exts = None
    if ext is not None:
        exts = [None if e is None else _c(e, np.int32) for e in ext]
        assert len(exts) == L + 1
    rc = lib.mgsa_oracle_decode(ctypes.byref(c), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt),
                                _ptr(sl), L, _ptr_array(ks), _ptr_array(vs), maxs, fans, tops,
                                _ptr(out), _ptr_array(sels), _ptr_array(keys),
                                None if exts is None else _ptr_array(exts), nthreads)
    if rc:
        raise ValueError(f"oracle rejected the configuration (code {rc})")
    return out, sels, keys


def prefill(cfg: dict, q, k_cache, v_cache, block_table, q_start, nthreads: int = 0, lib=None):
    """Multi-query attention under the gist causal mask: q [B][T][Hq][d] are
    the queries of logical slots q_start[b] .. q_start[b] + T - 1.  Returns
    out float64 [B][T][Hq][d]."""
    lib = lib or _load()
    c = _cfg(cfg)
    q, k_cache, v_cache = (_data(x, c.dtype) for x in (q, k_cache, v_cache))
    B, T, Hq, d = q.shape
    out = np.zeros((B, T, Hq, d), np.float64)
    rc = lib.gsa_prefill_oracle(ctypes.byref(c), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                _ptr(_c(block_table, np.int32)), _ptr(_c(q_start, np.int32)), T,
                                _ptr(out), nthreads)
    if rc:
        raise ValueError(f"oracle rejected the configuration (code {rc})")
    return out
