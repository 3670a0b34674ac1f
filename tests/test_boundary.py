"""The C ABI without a GPU: the library loads, exports every function that
include/gsa.h declares, validates every argument on the host before touching
the device, and sizes its workspace consistently.

No call here reaches a kernel: every case is invalid in at least one field
(fake device pointers are never dereferenced), and the one fully valid call
runs only when no GPU is visible, where it must report GSA_ERR_DEVICE.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import long_context_sparse_gist_amd as gsa
from long_context_sparse_gist_amd import build as gbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gsa.h")
FAKE = 0x7F0000000000  # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gsa.LIB_PATH):
        gbuild.build()
    return gsa.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "return", "sizeof")))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "gsa_workspace_size", "hgsa_workspace_size", "gsa_decode", "hgsa_decode",
        "gsa_decode_noalloc", "mgsa_workspace_size", "mgsa_decode", "gsa_prefill",
        "gsa_workspace_status",
        "gsa_workspace_reset", "gsa_status_string", "gsa_version"])


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", gsa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if " T " in line)
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings_and_version(lib):
    for code, name in gsa.STATUS.items():
        assert gsa.gsa_status_string(code)
    assert gsa.gsa_status_string(99) == "unknown status"
    assert gsa.gsa_version() >= 100


def params(**kw):
    d = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, top_k=4, sm_scale=0.0,
             dtype=gsa.GSA_BF16, flags=0)
    d.update(kw)
    return gsa.GsaParams(**d)


def kvs(**kw):
    d = dict(k_cache=FAKE, v_cache=FAKE, block_table=FAKE, seq_lens=None, num_chunks=64,
             chunk_size=16, page_chunks=16, num_pages=8, max_pages=5)
    d.update(kw)
    return gsa.GsaKV(**d)


def meta(**kw):
    d = dict(k_meta=FAKE, v_meta=FAKE, max_meta=4, gists_per_meta=16, top_k_meta=2)
    d.update(kw)
    return gsa.HgsaMeta(**d)


def call(lib, p, kv, q=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib.gsa_decode(ctypes.byref(p), ctypes.byref(kv), ctypes.c_void_p(q),
                          ctypes.c_void_p(out), None, None, ctypes.c_void_p(ws), ws_bytes, None)


def call_h(lib, p, kv, m, ws_bytes=1 << 30):
    return lib.hgsa_decode(ctypes.byref(p), ctypes.byref(kv), ctypes.byref(m),
                           ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None, None,
                           ctypes.c_void_p(FAKE), ws_bytes, None)


BAD_PARAMS = [
    (dict(batch=0), 2), (dict(num_q_heads=0), 2), (dict(num_kv_heads=0), 2),
    (dict(num_q_heads=7), 2), (dict(num_q_heads=34), 2), (dict(head_dim=96), 2),
    (dict(top_k=-1), 2), (dict(sm_scale=float("nan")), 2), (dict(sm_scale=float("inf")), 2),
    (dict(dtype=2), 3), (dict(flags=0x40), 4),
    # top-p: 0 < top_p <= 1, the default key only, a cap of at most 2048
    (dict(flags=0x4, top_p=0.0), 2), (dict(flags=0x4, top_p=1.5), 2),
    (dict(flags=0x4, top_p=float("nan")), 2), (dict(flags=0x5, top_p=0.5), 4),
    (dict(flags=0x4, top_p=0.5, top_k=4096), 2),
]
BAD_KV = [
    (dict(chunk_size=0), 2), (dict(page_chunks=0), 2), (dict(num_chunks=-1), 2),
    (dict(num_pages=0), 2), (dict(max_pages=0), 2), (dict(max_pages=3), 2),
]


@pytest.mark.parametrize("kw,code", BAD_PARAMS)
def test_bad_params_rejected(lib, kw, code):
    assert call(lib, params(**kw), kvs()) == code
    assert lib.gsa_workspace_size(ctypes.byref(params(**kw)), ctypes.byref(kvs())) == 0


@pytest.mark.parametrize("kw,code", BAD_KV)
def test_bad_kv_rejected(lib, kw, code):
    assert call(lib, params(), kvs(**kw)) == code


def test_null_arguments(lib):
    p, kv = params(), kvs()
    assert lib.gsa_decode(None, ctypes.byref(kv), None, None, None, None, None, 0, None) == 1
    assert lib.gsa_decode(ctypes.byref(p), None, None, None, None, None, None, 0, None) == 1
    assert call(lib, p, kv, q=0) == 1
    assert call(lib, p, kv, out=0) == 1
    assert call(lib, p, kvs(k_cache=0)) == 1
    assert call(lib, p, kvs(v_cache=0)) == 1
    assert call(lib, p, kvs(block_table=0)) == 1
    assert call_h(lib, p, kv, meta(k_meta=0)) == 1
    assert lib.hgsa_decode(ctypes.byref(p), ctypes.byref(kv), None, None, None, None, None,
                           None, 0, None) == 1


def test_workspace_checks(lib):
    p, kv = params(), kvs()
    need = lib.gsa_workspace_size(ctypes.byref(p), ctypes.byref(kv))
    assert need > 0 and need % 256 == 0
    assert call(lib, p, kv, ws=0) == 5
    assert call(lib, p, kv, ws=FAKE + 16) == 5          # misaligned
    assert call(lib, p, kv, ws_bytes=need - 1) == 5     # too small


def test_workspace_size_monotone(lib):
    base = lib.gsa_workspace_size(ctypes.byref(params()), ctypes.byref(kvs()))
    for p, kv in [(params(batch=3), kvs()), (params(top_k=40), kvs()),
                  (params(num_q_heads=16), kvs()), (params(), kvs(num_chunks=80, max_pages=6))]:
        assert lib.gsa_workspace_size(ctypes.byref(p), ctypes.byref(kv)) >= base
    # top_k past the chunk count costs only the selection output
    a = lib.gsa_workspace_size(ctypes.byref(params(top_k=64)), ctypes.byref(kvs()))
    b = lib.gsa_workspace_size(ctypes.byref(params(top_k=6400)), ctypes.byref(kvs()))
    assert b - a <= 4 * 2 * 2 * 6400 + 512


def test_hgsa_validation(lib):
    p, kv = params(), kvs()
    assert lib.hgsa_workspace_size(ctypes.byref(p), ctypes.byref(kv), ctypes.byref(meta())) > 0
    assert call_h(lib, p, kv, meta(gists_per_meta=0)) == 2
    assert call_h(lib, p, kv, meta(top_k_meta=-1)) == 2
    assert call_h(lib, p, kv, meta(max_meta=3)) == 2
    assert call_h(lib, params(flags=gsa.GSA_SET_SELECTED_GISTS), kv, meta()) == 4
    assert call_h(lib, params(flags=gsa.GSA_SCORE_SUM_PROBS), kv, meta()) == 4  # flat GSA only
    assert call_h(lib, params(flags=gsa.GSA_SELECT_TOP_P, top_p=0.5), kv, meta()) == 4
    assert call_h(lib, params(head_dim=32), kv, meta()) == 2
    need = lib.hgsa_workspace_size(ctypes.byref(p), ctypes.byref(kv), ctypes.byref(meta()))
    assert call_h(lib, p, kv, meta(), ws_bytes=need - 1) == 5


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is visible")
def test_valid_call_without_device_reports_device_error(lib):
    assert call(lib, params(), kvs()) == 6
    assert call_h(lib, params(), kvs(), meta()) == 6


def call_na(lib, p, kv, q=FAKE, out=FAKE):
    return lib.gsa_decode_noalloc(ctypes.byref(p), ctypes.byref(kv), ctypes.c_void_p(q),
                                  ctypes.c_void_p(out), None, None, None)


def test_noalloc_validation(lib):
    """The allocation-free entry point validates like gsa_decode and rejects
    shapes whose workspace exceeds its fixed array."""
    for kw, code in BAD_PARAMS:
        assert call_na(lib, params(**kw), kvs()) == code
    for kw, code in BAD_KV:
        assert call_na(lib, params(), kvs(**kw)) == code
    assert call_na(lib, params(), kvs(), q=0) == 1
    assert call_na(lib, params(), kvs(), out=0) == 1
    # 16 x 16 units of 65536 chunks: keys alone take 64 MiB
    big_p, big_kv = params(batch=16, num_kv_heads=16, num_q_heads=16), kvs(num_chunks=65536,
                                                                            max_pages=4097)
    assert lib.gsa_workspace_size(ctypes.byref(big_p), ctypes.byref(big_kv)) > \
        gsa.NOALLOC_WORKSPACE_BYTES
    assert call_na(lib, big_p, big_kv) == 5
    m = re.search(r"#define GSA_NOALLOC_WORKSPACE_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                  open(HEADER).read())
    assert m is not None and int(m[1]) << int(m[2]) == gsa.NOALLOC_WORKSPACE_BYTES


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is visible")
def test_noalloc_without_device_reports_device_error(lib):
    assert call_na(lib, params(), kvs()) == 6


def lvl(**kw):
    d = dict(k_meta=FAKE, v_meta=FAKE, max_meta=16, fanout=4, top_k=2)
    d.update(kw)
    return gsa.GsaLevel(**d)


def call_m(lib, p, kv, levels, n=None, ws_bytes=1 << 30):
    arr = (gsa.GsaLevel * max(1, len(levels)))(*levels)
    return lib.mgsa_decode(ctypes.byref(p), ctypes.byref(kv), arr, len(levels) if n is None else n,
                           ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None,
                           ctypes.c_void_p(FAKE), ws_bytes, None)


def test_mgsa_validation(lib):
    """The hierarchy of any depth: level count, fanouts, capacities, dtype and
    flags are checked before anything is enqueued."""
    p, kv = params(), kvs()   # 64 chunks: 16 entries at fanout 4, 4 at 4 x 4
    two = [lvl(), lvl(max_meta=4)]
    arr = (gsa.GsaLevel * 2)(*two)
    need = lib.mgsa_workspace_size(ctypes.byref(p), ctypes.byref(kv), arr, 2)
    assert need > gsa.WORKSPACE_CONTROL_BYTES and need % 256 == 0
    assert lib.mgsa_workspace_size(ctypes.byref(p), ctypes.byref(kv), None, 0) > 0
    assert call_m(lib, p, kv, two, n=9) == 2                           # > GSA_MAX_LEVELS
    assert call_m(lib, p, kv, two, n=-1) == 2
    assert call_m(lib, p, kv, [lvl(fanout=0)]) == 2
    assert call_m(lib, p, kv, [lvl(top_k=-1)]) == 2
    assert call_m(lib, p, kv, [lvl(), lvl(max_meta=3)]) == 2           # level 2 holds 4
    assert call_m(lib, p, kv, [lvl(max_meta=15)]) == 2
    assert call_m(lib, params(dtype=gsa.GSA_F32), kv, two) == 3
    assert call_m(lib, params(flags=gsa.GSA_SET_SELECTED_GISTS), kv, two) == 4
    assert call_m(lib, p, kv, [lvl(k_meta=0)]) == 1
    assert lib.mgsa_decode(ctypes.byref(p), ctypes.byref(kv), None, 1, ctypes.c_void_p(FAKE),
                           ctypes.c_void_p(FAKE), None, ctypes.c_void_p(FAKE), 1 << 30, None) == 1
    assert call_m(lib, p, kv, two, ws_bytes=need - 1) == 5
    assert call_m(lib, params(batch=0), kv, two) == 2


def call_p(lib, p, kv, T=4, q_start=FAKE, q=FAKE, out=FAKE):
    return lib.gsa_prefill(ctypes.byref(p), ctypes.byref(kv), ctypes.c_void_p(q_start), T,
                           ctypes.c_void_p(q), ctypes.c_void_p(out), None)


def test_prefill_validation(lib):
    """gsa_prefill checks shapes, dtype, flags and pointers before anything is
    enqueued."""
    p, kv = params(), kvs()
    for kw, code in BAD_PARAMS:
        if "top_p" in kw:
            continue
        assert call_p(lib, params(**kw), kv) == code
    assert call_p(lib, params(dtype=gsa.GSA_F32), kv) == 3
    assert call_p(lib, params(flags=gsa.GSA_SET_SELECTED_GISTS), kv) == 4
    assert call_p(lib, p, kv, T=-1) == 2
    assert call_p(lib, p, kv, T=5 * 16 * 17 + 1) == 2    # more queries than the row holds
    assert call_p(lib, p, kv, q_start=0) == 1
    assert call_p(lib, p, kv, q=0) == 1
    assert call_p(lib, p, kv, out=0) == 1
    assert call_p(lib, p, kvs(k_cache=0)) == 1


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is visible")
def test_prefill_without_device_reports_device_error(lib):
    assert call_p(lib, params(), kvs()) == 6


def test_workspace_status_and_reset_validation(lib):
    need = gsa.WORKSPACE_CONTROL_BYTES
    for fn in (lib.gsa_workspace_status, lib.gsa_workspace_reset):
        assert fn(None, need, None) == 1
        assert fn(ctypes.c_void_p(FAKE + 16), need, None) == 5    # misaligned
        assert fn(ctypes.c_void_p(FAKE), need - 1, None) == 5     # smaller than the control block


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is visible")
def test_workspace_status_without_device_reports_device_error(lib):
    need = gsa.WORKSPACE_CONTROL_BYTES
    assert lib.gsa_workspace_status(ctypes.c_void_p(FAKE), need, None) == 6
    assert lib.gsa_workspace_reset(ctypes.c_void_p(FAKE), need, None) == 6


def test_error_word_offset_matches_header():
    m = re.search(r"#define GSA_WORKSPACE_ERROR_OFFSET \(\(size_t\)(\d+)\)", open(HEADER).read())
    assert m is not None and int(m[1]) == gsa.WORKSPACE_ERROR_OFFSET
    assert gsa.STATUS[8] == "GSA_ERR_WAIT" and "GSA_ERR_WAIT = 8" in open(HEADER).read()


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(gsa, "_lib", None)
    monkeypatch.setattr(gsa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        gsa.lib()


def test_control_block_size_matches_header():
    txt = open(HEADER).read()
    m = re.search(r"#define GSA_WORKSPACE_CONTROL_BYTES \(\(size_t\)(\d+) \+ \(size_t\)(\d+) \* (\d+)\)",
                  txt)
    assert m is not None
    assert int(m[1]) + int(m[2]) * int(m[3]) == gsa.WORKSPACE_CONTROL_BYTES


def test_workspace_covers_control_block(lib):
    p, kv = params(), kvs()
    assert lib.gsa_workspace_size(ctypes.byref(p), ctypes.byref(kv)) > gsa.WORKSPACE_CONTROL_BYTES


def test_params_layout_matches_header(tmp_path):
    """The binding's gsa_params_t / gsa_kv_t / hgsa_meta_t match the header's
    layout (sizes and field offsets, from a C program built with gcc)."""
    structs = {"gsa_params_t": gsa.GsaParams, "gsa_kv_t": gsa.GsaKV, "hgsa_meta_t": gsa.HgsaMeta}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "gsa.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'    printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'    printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["    return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), "-o", str(exe), str(src)], check=True)
    got = {}
    for ln in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n"):
        if ln:
            cname, what, val = ln.split()
            got[(cname, what)] = int(val)
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)
