"""Python binding of libgsa.so, the MI355X gist sparse attention decode library.

Argument marshalling only: every step of the decode runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  The library
is loaded on first use and a missing or unloadable library raises; there is no
fallback path.

Names mirror the C ABI in include/gsa.h: gsa_decode, hgsa_decode,
gsa_decode_noalloc, mgsa_decode, gsa_prefill, gsa_workspace_size, hgsa_workspace_size,
mgsa_workspace_size, gsa_workspace_status, gsa_workspace_reset, gsa_status_string, gsa_version.

Streams: a call runs on `stream` (default: the current stream of q's
device).  The output and the cached workspace are allocated, and the
workspace zero-filled, on that stream, and the workspace cache is kept per
(device, stream), so calls on different streams never share a control block
and every allocation is ordered before the kernels that use it.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgsa.so")

GSA_F32 = 0
GSA_BF16 = 1
GSA_SCORE_SUM_LOGITS = 0x0
GSA_SCORE_SUM_PROBS = 0x1
GSA_SET_ALL_GISTS = 0x0
GSA_SET_SELECTED_GISTS = 0x2
GSA_SELECT_TOP_P = 0x4
GSA_PATH_PORTABLE = 0x100
# bytes at the start of every workspace that must be zero between calls
WORKSPACE_CONTROL_BYTES = 16384 + 512 * 25088
# byte offset of the control block's error word (nonzero: a wait gave up)
WORKSPACE_ERROR_OFFSET = 8
# the library-owned workspace of gsa_decode_noalloc
NOALLOC_WORKSPACE_BYTES = 64 << 20

STATUS = {0: "GSA_OK", 1: "GSA_ERR_NULL_ARG", 2: "GSA_ERR_BAD_SHAPE", 3: "GSA_ERR_BAD_DTYPE",
          4: "GSA_ERR_BAD_FLAGS", 5: "GSA_ERR_WORKSPACE", 6: "GSA_ERR_DEVICE",
          7: "GSA_ERR_LAUNCH", 8: "GSA_ERR_WAIT"}


class GsaParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32), ("top_p", ctypes.c_float)]


class GsaKV(ctypes.Structure):
    _fields_ = [("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("num_chunks", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
                ("page_chunks", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages", ctypes.c_int32)]


class HgsaMeta(ctypes.Structure):
    _fields_ = [("k_meta", ctypes.c_void_p), ("v_meta", ctypes.c_void_p),
                ("max_meta", ctypes.c_int32), ("gists_per_meta", ctypes.c_int32),
                ("top_k_meta", ctypes.c_int32)]


class GsaLevel(ctypes.Structure):
    _fields_ = [("k_meta", ctypes.c_void_p), ("v_meta", ctypes.c_void_p),
                ("max_meta", ctypes.c_int32), ("fanout", ctypes.c_int32), ("top_k", ctypes.c_int32)]


MAX_LEVELS = 8


class GsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({gsa_status_string(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libgsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m long_context_sparse_gist_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.gsa_workspace_size.argtypes = [ctypes.POINTER(GsaParams), ctypes.POINTER(GsaKV)]
        L.gsa_workspace_size.restype = ctypes.c_size_t
        L.hgsa_workspace_size.argtypes = [ctypes.POINTER(GsaParams), ctypes.POINTER(GsaKV),
                                          ctypes.POINTER(HgsaMeta)]
        L.hgsa_workspace_size.restype = ctypes.c_size_t
        L.gsa_decode.argtypes = [ctypes.POINTER(GsaParams), ctypes.POINTER(GsaKV), P, P, P, P,
                                 P, ctypes.c_size_t, P]
        L.gsa_decode.restype = ctypes.c_int
        L.hgsa_decode.argtypes = [ctypes.POINTER(GsaParams), ctypes.POINTER(GsaKV),
                                  ctypes.POINTER(HgsaMeta), P, P, P, P, P, ctypes.c_size_t, P]
        L.hgsa_decode.restype = ctypes.c_int
        L.gsa_decode_noalloc.argtypes = [ctypes.POINTER(GsaParams), ctypes.POINTER(GsaKV), P, P,
                                         P, P, P]
        L.gsa_decode_noalloc.restype = ctypes.c_int
        L.mgsa_workspace_size.argtypes = [ctypes.POINTER(GsaParams), ctypes.POINTER(GsaKV),
                                          ctypes.POINTER(GsaLevel), ctypes.c_int32]
        L.mgsa_workspace_size.restype = ctypes.c_size_t
        L.mgsa_decode.argtypes = [ctypes.POINTER(GsaParams), ctypes.POINTER(GsaKV),
                                  ctypes.POINTER(GsaLevel), ctypes.c_int32, P, P,
                                  ctypes.POINTER(ctypes.c_void_p), P, ctypes.c_size_t, P]
        L.mgsa_decode.restype = ctypes.c_int
        L.gsa_prefill.argtypes = [ctypes.POINTER(GsaParams), ctypes.POINTER(GsaKV), P,
                                  ctypes.c_int32, P, P, P]
        L.gsa_prefill.restype = ctypes.c_int
        L.gsa_workspace_status.argtypes = [P, ctypes.c_size_t, P]
        L.gsa_workspace_status.restype = ctypes.c_int
        L.gsa_workspace_reset.argtypes = [P, ctypes.c_size_t, P]
        L.gsa_workspace_reset.restype = ctypes.c_int
        L.gsa_status_string.argtypes = [ctypes.c_int]
        L.gsa_status_string.restype = ctypes.c_char_p
        L.gsa_version.restype = ctypes.c_int
        _lib = L
    return _lib


def gsa_status_string(status: int) -> str:
    return lib().gsa_status_string(status).decode()


def gsa_version() -> int:
    return lib().gsa_version()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GSA_F32
    if t.dtype == torch.bfloat16:
        return GSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def make_params(q: torch.Tensor, num_kv_heads: int, top_k: int, sm_scale: float = 0.0,
                flags: int = 0, top_p: float = 0.0) -> GsaParams:
    """top_p > 0 selects top-p selection (GSA_SELECT_TOP_P), top_k its cap."""
    B, Hq, d = q.shape
    if top_p > 0.0:
        flags |= GSA_SELECT_TOP_P
    return GsaParams(B, Hq, num_kv_heads, d, top_k, sm_scale, _dtype_code(q), flags, top_p)


def make_kv(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
            seq_lens: Optional[torch.Tensor], num_chunks: int, chunk_size: int,
            page_chunks: int) -> GsaKV:
    return GsaKV(_ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), num_chunks,
                 chunk_size, page_chunks, k_cache.shape[0], block_table.shape[1])


def make_meta(k_meta: torch.Tensor, v_meta: torch.Tensor, gists_per_meta: int,
              top_k_meta: int) -> HgsaMeta:
    return HgsaMeta(_ptr(k_meta), _ptr(v_meta), k_meta.shape[2], gists_per_meta, top_k_meta)


def gsa_workspace_size(params: GsaParams, kv: GsaKV) -> int:
    return lib().gsa_workspace_size(ctypes.byref(params), ctypes.byref(kv))


def hgsa_workspace_size(params: GsaParams, kv: GsaKV, meta: HgsaMeta) -> int:
    return lib().hgsa_workspace_size(ctypes.byref(params), ctypes.byref(kv), ctypes.byref(meta))


_ws_cache: dict = {}


def _stream_of(stream, device) -> "torch.cuda.Stream":
    return stream if stream is not None else torch.cuda.current_stream(device)


def workspace(nbytes: int, device, stream=None) -> torch.Tensor:
    """A zero-filled workspace of at least nbytes on `device` for calls on
    `stream` (default: the device's current stream), reused across calls on
    that stream.  It is allocated and zero-filled on that stream, so the fill
    is ordered before the calls; a replaced one returns to the allocator's
    pool for that stream, whose later users are ordered after the calls that
    used it."""
    dev = torch.device(device)
    s = _stream_of(stream, dev)
    key = (dev.type, dev.index, s.cuda_stream)
    t = _ws_cache.get(key)
    if t is None or t.numel() < nbytes:
        with torch.cuda.stream(s):
            t = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _ws_cache[key] = t
    return t


def gsa_workspace_status(ws: torch.Tensor, stream=None) -> int:
    """Wait for `stream`, then read the workspace's error word: 0 (GSA_OK) or
    8 (GSA_ERR_WAIT, a wait in the single-launch kernel gave up)."""
    return lib().gsa_workspace_status(_ptr(ws), ws.numel() * ws.element_size(),
                                      _stream_ptr(stream, ws.device))


def gsa_workspace_reset(ws: torch.Tensor, stream=None) -> None:
    """Enqueue the zeroing of the workspace's control block on `stream`."""
    st = lib().gsa_workspace_reset(_ptr(ws), ws.numel() * ws.element_size(),
                                   _stream_ptr(stream, ws.device))
    if st != 0:
        raise GsaError(st, "gsa_workspace_reset")


def _alloc_out(q: torch.Tensor, stream) -> torch.Tensor:
    with torch.cuda.stream(_stream_of(stream, q.device)):
        return torch.empty_like(q)


def _check(q, k_cache, v_cache, block_table, seq_lens):
    for t in (q, k_cache, v_cache, block_table):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, caches and block_table must be contiguous device tensors")
    if block_table.dtype != torch.int32:
        raise TypeError("block_table must be int32")
    if seq_lens is not None and (seq_lens.dtype != torch.int32 or not seq_lens.is_cuda):
        raise TypeError("seq_lens must be an int32 device tensor")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")


def _stream_ptr(stream, device):
    return ctypes.c_void_p(_stream_of(stream, device).cuda_stream)


class PreparedCall:
    """A decode call whose arguments were marshalled once: each call enqueues
    the same launch again, reading the tensors it was built from (which must
    stay alive, unmoved) as they are at that time.  For loops over one shape,
    where per-call argument marshalling would cost more host time than the
    kernel takes on the device."""

    def __init__(self, fn, args, keep, name):
        self._fn, self._args, self._keep, self._name = fn, args, keep, name

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            raise GsaError(st, self._name)


def prepare_gsa_decode(q, k_cache, v_cache, block_table, seq_lens, *, num_chunks: int,
                       chunk_size: int, page_chunks: int, top_k: int, sm_scale: float = 0.0,
                       flags: int = 0, top_p: float = 0.0, out=None, sel_idx=None, scores=None,
                       ws=None, stream=None) -> PreparedCall:
    """gsa_decode's arguments marshalled into a PreparedCall; `out` is
    allocated here if not given and can be read back as `.out`."""
    _check(q, k_cache, v_cache, block_table, seq_lens)
    Hkv = k_cache.shape[1]
    p = make_params(q, Hkv, top_k, sm_scale, flags, top_p)
    kv = make_kv(k_cache, v_cache, block_table, seq_lens, num_chunks, chunk_size, page_chunks)
    if out is None:
        out = _alloc_out(q, stream)
    nbytes = gsa_workspace_size(p, kv)
    if nbytes == 0:
        raise GsaError(2, "gsa_workspace_size")
    if ws is None:
        ws = workspace(nbytes, q.device, stream)
    args = (ctypes.byref(p), ctypes.byref(kv), _ptr(q), _ptr(out), _ptr(sel_idx), _ptr(scores),
            _ptr(ws), ws.numel() * ws.element_size(), _stream_ptr(stream, q.device))
    call = PreparedCall(lib().gsa_decode, args,
                        (p, kv, q, k_cache, v_cache, block_table, seq_lens, out, sel_idx, scores, ws),
                        "gsa_decode")
    call.out = out
    return call


def prepare_hgsa_decode(q, k_cache, v_cache, block_table, seq_lens, k_meta, v_meta, *,
                        num_chunks: int, chunk_size: int, page_chunks: int, gists_per_meta: int,
                        top_k_meta: int, top_k: int, sm_scale: float = 0.0, flags: int = 0,
                        out=None, sel_meta=None, sel_idx=None, ws=None,
                        stream=None) -> PreparedCall:
    """hgsa_decode's arguments marshalled into a PreparedCall."""
    _check(q, k_cache, v_cache, block_table, seq_lens)
    Hkv = k_cache.shape[1]
    p = make_params(q, Hkv, top_k, sm_scale, flags)
    kv = make_kv(k_cache, v_cache, block_table, seq_lens, num_chunks, chunk_size, page_chunks)
    m = make_meta(k_meta, v_meta, gists_per_meta, top_k_meta)
    if out is None:
        out = _alloc_out(q, stream)
    nbytes = hgsa_workspace_size(p, kv, m)
    if nbytes == 0:
        raise GsaError(2, "hgsa_workspace_size")
    if ws is None:
        ws = workspace(nbytes, q.device, stream)
    args = (ctypes.byref(p), ctypes.byref(kv), ctypes.byref(m), _ptr(q), _ptr(out),
            _ptr(sel_meta), _ptr(sel_idx), _ptr(ws), ws.numel() * ws.element_size(),
            _stream_ptr(stream, q.device))
    call = PreparedCall(lib().hgsa_decode, args,
                        (p, kv, m, q, k_cache, v_cache, block_table, seq_lens, k_meta, v_meta, out,
                         sel_meta, sel_idx, ws), "hgsa_decode")
    call.out = out
    return call


def gsa_decode(q, k_cache, v_cache, block_table, seq_lens, *, num_chunks: int,
               chunk_size: int, page_chunks: int, top_k: int, sm_scale: float = 0.0,
               flags: int = 0, top_p: float = 0.0, out=None, sel_idx=None, scores=None,
               ws=None, stream=None):
    """One GSA decode step (see gsa_decode in include/gsa.h).

    q [B][Hq][d]; k_cache, v_cache [num_pages][Hkv][page_chunks*(C+1)][d];
    block_table int32 [B][max_pages]; seq_lens int32 [B] or None.  top_p > 0:
    top-p selection with top_k as its cap.
    Returns out [B][Hq][d] (allocated if not given)."""
    _check(q, k_cache, v_cache, block_table, seq_lens)
    Hkv = k_cache.shape[1]
    p = make_params(q, Hkv, top_k, sm_scale, flags, top_p)
    kv = make_kv(k_cache, v_cache, block_table, seq_lens, num_chunks, chunk_size, page_chunks)
    if out is None:
        out = _alloc_out(q, stream)
    nbytes = gsa_workspace_size(p, kv)
    if nbytes == 0:
        raise GsaError(2, "gsa_workspace_size")
    if ws is None:
        ws = workspace(nbytes, q.device, stream)
    st = lib().gsa_decode(ctypes.byref(p), ctypes.byref(kv), _ptr(q), _ptr(out), _ptr(sel_idx),
                          _ptr(scores), _ptr(ws), ws.numel() * ws.element_size(),
                          _stream_ptr(stream, q.device))
    if st != 0:
        raise GsaError(st, "gsa_decode")
    return out


def gsa_decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, *, num_chunks: int,
                       chunk_size: int, page_chunks: int, top_k: int, sm_scale: float = 0.0,
                       flags: int = 0, top_p: float = 0.0, out, sel_idx=None, scores=None,
                       stream=None):
    """gsa_decode on the library-owned workspace (see gsa_decode_noalloc in
    include/gsa.h).  `out` must be given: this path allocates nothing."""
    _check(q, k_cache, v_cache, block_table, seq_lens)
    p = make_params(q, k_cache.shape[1], top_k, sm_scale, flags, top_p)
    kv = make_kv(k_cache, v_cache, block_table, seq_lens, num_chunks, chunk_size, page_chunks)
    st = lib().gsa_decode_noalloc(ctypes.byref(p), ctypes.byref(kv), _ptr(q), _ptr(out),
                                  _ptr(sel_idx), _ptr(scores), _stream_ptr(stream, q.device))
    if st != 0:
        raise GsaError(st, "gsa_decode_noalloc")
    return out


def hgsa_decode(q, k_cache, v_cache, block_table, seq_lens, k_meta, v_meta, *, num_chunks: int,
                chunk_size: int, page_chunks: int, gists_per_meta: int, top_k_meta: int,
                top_k: int, sm_scale: float = 0.0, flags: int = 0, out=None, sel_meta=None,
                sel_idx=None, ws=None, stream=None):
    """One H-GSA decode step (see hgsa_decode in include/gsa.h).
    k_meta, v_meta [B][Hkv][max_meta][d]."""
    _check(q, k_cache, v_cache, block_table, seq_lens)
    for t in (k_meta, v_meta):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError("meta caches must be contiguous device tensors of q's dtype")
    Hkv = k_cache.shape[1]
    p = make_params(q, Hkv, top_k, sm_scale, flags)
    kv = make_kv(k_cache, v_cache, block_table, seq_lens, num_chunks, chunk_size, page_chunks)
    m = make_meta(k_meta, v_meta, gists_per_meta, top_k_meta)
    if out is None:
        out = _alloc_out(q, stream)
    nbytes = hgsa_workspace_size(p, kv, m)
    if nbytes == 0:
        raise GsaError(2, "hgsa_workspace_size")
    if ws is None:
        ws = workspace(nbytes, q.device, stream)
    st = lib().hgsa_decode(ctypes.byref(p), ctypes.byref(kv), ctypes.byref(m), _ptr(q), _ptr(out),
                           _ptr(sel_meta), _ptr(sel_idx), _ptr(ws), ws.numel() * ws.element_size(),
                           _stream_ptr(stream, q.device))
    if st != 0:
        raise GsaError(st, "hgsa_decode")
    return out


def make_levels(levels) -> "ctypes.Array":
    """levels: [(k_meta, v_meta, fanout, top_k)], level 1 first, each meta
    array [B][Hkv][max_meta][d] -> a gsa_level_t array."""
    arr = (GsaLevel * max(1, len(levels)))()
    for i, (k, v, R, kk) in enumerate(levels):
        arr[i] = GsaLevel(_ptr(k), _ptr(v), k.shape[2], R, kk)
    return arr


def mgsa_workspace_size(params: GsaParams, kv: GsaKV, levels_arr, num_levels: int) -> int:
    return lib().mgsa_workspace_size(ctypes.byref(params), ctypes.byref(kv), levels_arr,
                                     num_levels)


def prepare_mgsa_decode(q, k_cache, v_cache, block_table, seq_lens, levels, *, num_chunks: int,
                        chunk_size: int, page_chunks: int, top_k: int, sm_scale: float = 0.0,
                        out=None, sel=None, ws=None, stream=None) -> PreparedCall:
    """mgsa_decode's arguments marshalled into a PreparedCall.  levels:
    [(k_meta, v_meta, fanout, top_k)], level 1 first; sel: None or
    len(levels) + 1 int32 tensors / None (the gist level first)."""
    _check(q, k_cache, v_cache, block_table, seq_lens)
    for k, v, _, _ in levels:
        if not k.is_cuda or not k.is_contiguous() or not v.is_contiguous() or k.dtype != q.dtype:
            raise ValueError("level arrays must be contiguous device tensors of q's dtype")
    p = make_params(q, k_cache.shape[1], top_k, sm_scale)
    kv = make_kv(k_cache, v_cache, block_table, seq_lens, num_chunks, chunk_size, page_chunks)
    lv = make_levels(levels)
    L = len(levels)
    if out is None:
        out = _alloc_out(q, stream)
    nbytes = mgsa_workspace_size(p, kv, lv, L)
    if nbytes == 0:
        raise GsaError(2, "mgsa_workspace_size")
    if ws is None:
        ws = workspace(nbytes, q.device, stream)
    sel_arr = None
    if sel is not None:
        if len(sel) != L + 1:
            raise ValueError("sel needs one entry per level plus the gist level")
        sel_arr = (ctypes.c_void_p * (L + 1))(*[None if t is None else t.data_ptr() for t in sel])
    args = (ctypes.byref(p), ctypes.byref(kv), lv, L, _ptr(q), _ptr(out), sel_arr, _ptr(ws),
            ws.numel() * ws.element_size(), _stream_ptr(stream, q.device))
    call = PreparedCall(lib().mgsa_decode, args,
                        (p, kv, lv, q, k_cache, v_cache, block_table, seq_lens, levels, out, sel,
                         sel_arr, ws), "mgsa_decode")
    call.out = out
    return call


def mgsa_decode(q, k_cache, v_cache, block_table, seq_lens, levels, *, num_chunks: int,
                chunk_size: int, page_chunks: int, top_k: int, sm_scale: float = 0.0, out=None,
                sel=None, ws=None, stream=None):
    """One decode step over a hierarchy of len(levels) meta-gist levels (see
    mgsa_decode in include/gsa.h).  Returns out [B][Hq][d]."""
    call = prepare_mgsa_decode(q, k_cache, v_cache, block_table, seq_lens, levels,
                               num_chunks=num_chunks, chunk_size=chunk_size,
                               page_chunks=page_chunks, top_k=top_k, sm_scale=sm_scale, out=out,
                               sel=sel, ws=ws, stream=stream)
    call()
    return call.out


def prepare_gsa_prefill(q, k_cache, v_cache, block_table, q_start, *, chunk_size: int,
                        page_chunks: int, sm_scale: float = 0.0, out=None,
                        stream=None) -> PreparedCall:
    """gsa_prefill's arguments marshalled into a PreparedCall.  q [B][T][Hq][d]
    are the queries of slots q_start[b] .. q_start[b] + T - 1 (q_start: int32
    device [B])."""
    for t in (q, k_cache, v_cache, block_table, q_start):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, caches, block_table and q_start must be contiguous device tensors")
    if block_table.dtype != torch.int32 or q_start.dtype != torch.int32:
        raise TypeError("block_table and q_start must be int32")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    B, T, Hq, d = q.shape
    p = GsaParams(B, Hq, k_cache.shape[1], d, 0, sm_scale, _dtype_code(q), 0, 0.0)
    cap_chunks = block_table.shape[1] * page_chunks
    kv = make_kv(k_cache, v_cache, block_table, None, cap_chunks, chunk_size, page_chunks)
    if out is None:
        out = _alloc_out(q, stream)
    args = (ctypes.byref(p), ctypes.byref(kv), _ptr(q_start), T, _ptr(q), _ptr(out),
            _stream_ptr(stream, q.device))
    call = PreparedCall(lib().gsa_prefill, args,
                        (p, kv, q, k_cache, v_cache, block_table, q_start, out), "gsa_prefill")
    call.out = out
    return call


def gsa_prefill(q, k_cache, v_cache, block_table, q_start, *, chunk_size: int, page_chunks: int,
                sm_scale: float = 0.0, out=None, stream=None):
    """Attention of T consecutive slots per sequence under the gist causal mask
    (see gsa_prefill in include/gsa.h).  Returns out [B][T][Hq][d]."""
    call = prepare_gsa_prefill(q, k_cache, v_cache, block_table, q_start, chunk_size=chunk_size,
                               page_chunks=page_chunks, sm_scale=sm_scale, out=out, stream=stream)
    call()
    return call.out
