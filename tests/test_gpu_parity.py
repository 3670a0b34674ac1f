"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small cases span several splits with ragged tails; the full-size workloads
run in the launch configuration the benchmark times.  Every unit of every
case is compared: the oracle runs on the whole batch from one host copy of
the inputs.  Selections follow the gap rule, outputs the dtype's tolerance
(bf16: 2e-2 abs / 1e-2 rel; fp32: 1e-4 / 1e-4), keys 1e-3 abs / 1e-4 rel.
"""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_gist_amd as gsa
from long_context_sparse_gist_amd import inputs as gi
from tests import gpu_util as GU

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


SMALL = {
    "b3-g4-d64-c8": gi.Workload("b3-g4-d64-c8", gi.BF16, 3, 8, 2, 64, 8, 300, 20, 16,
                                plant="align", plant_count=4),
    "b2-g7-d128-c16": gi.Workload("b2-g7-d128-c16", gi.BF16, 2, 14, 2, 128, 16, 333, 37, 8,
                                  plant="align", plant_count=5),
    "b2-g4-d128-c32": gi.Workload("b2-g4-d128-c32", gi.BF16, 2, 8, 2, 128, 32, 150, 9, 4,
                                  plant="doc_bias", n_docs=5),
    "b1-g1-d128-c16": gi.Workload("b1-g1-d128-c16", gi.BF16, 1, 3, 3, 128, 16, 260, 11, 16),
    "b2-g16-d64-c4": gi.Workload("b2-g16-d64-c4", gi.BF16, 2, 16, 1, 64, 4, 700, 50, 64),
    "f32-b2-g3-d64": gi.Workload("f32-b2-g3-d64", gi.F32, 2, 6, 2, 64, 16, 200, 12, 16,
                                 plant="align", plant_count=3),
    # 512 units: just as many single-launch tasks as the GPU holds at once
    # (two per unit), then more, so that the plan puts every unit's gist
    # slices first and the unfolded tasks after
    "b128-g2-d64-c4-fit": gi.Workload("b128-g2-d64-c4-fit", gi.BF16, 128, 8, 4, 64, 4, 300, 20, 16,
                                      plant="align", plant_count=3),
    "b128-g2-d64-c4-many": gi.Workload("b128-g2-d64-c4-many", gi.BF16, 128, 8, 4, 64, 4, 300, 40, 16,
                                       plant="align", plant_count=3),
    "b64-g2-d128-c8-many": gi.Workload("b64-g2-d128-c8-many", gi.BF16, 64, 16, 8, 128, 8, 270, 24, 16,
                                       plant="doc_bias", n_docs=3),
}


def lens_for(wl, kind, seed=0):
    M, C = wl.num_chunks, wl.chunk_size
    if kind == "full":
        return None
    rng = np.random.default_rng(seed)
    L = [int(x) for x in rng.integers(1, M * C + C - 1, size=wl.batch)]
    if kind == "edge":
        L[0] = 0                     # empty sequence
        if wl.batch > 1:
            L[1] = C - 1             # no gist yet, raw tail only
        if wl.batch > 2:
            L[2] = 3 * C             # fewer chunks than top_k
    return L


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("lens", ["full", "ragged", "edge"])
def test_small_all_units(gpu, name, lens):
    wl = SMALL[name]
    say(f"[parity] {name} lens={lens}")
    inp = gi.make_inputs(wl, 100 + len(name), seq_lens=lens_for(wl, lens, 3), spare_pages=2)
    g_inp = GU.to(inp, gpu)
    res = GU.run_gpu(g_inp)
    GU.check_gsa(inp, res)


@pytest.mark.parametrize("name", ["b3-g4-d64-c8", "b2-g7-d128-c16"])
@pytest.mark.parametrize("top_k", [0, 1, 10 ** 6])
def test_small_topk_extremes(gpu, name, top_k):
    wl = SMALL[name]
    say(f"[parity] {name} top_k={top_k}")
    inp = gi.make_inputs(wl, 7, seq_lens=lens_for(wl, "ragged", 1))
    res = GU.run_gpu(GU.to(inp, gpu), top_k=top_k)
    GU.check_gsa(inp, res, top_k=top_k)


@pytest.mark.parametrize("name", ["b3-g4-d64-c8", "b2-g7-d128-c16", "f32-b2-g3-d64"])
def test_small_selected_gists_set(gpu, name):
    wl = SMALL[name]
    say(f"[parity] {name} selected-gists set")
    inp = gi.make_inputs(wl, 9, seq_lens=lens_for(wl, "edge", 2))
    flags = gsa.GSA_SET_SELECTED_GISTS
    res = GU.run_gpu(GU.to(inp, gpu), flags=flags)
    GU.check_gsa(inp, res, flags=flags)


@pytest.mark.parametrize("name", ["b3-g4-d64-c8", "b2-g7-d128-c16", "b2-g16-d64-c4", "f32-b2-g3-d64"])
@pytest.mark.parametrize("lens", ["full", "edge"])
def test_small_sum_probs_key(gpu, name, lens):
    wl = SMALL[name]
    say(f"[parity] {name} sum-of-probabilities key lens={lens}")
    inp = gi.make_inputs(wl, 21, seq_lens=lens_for(wl, lens, 6))
    flags = gsa.GSA_SCORE_SUM_PROBS
    res = GU.run_gpu(GU.to(inp, gpu), flags=flags)
    GU.check_gsa(inp, res, flags=flags)


def test_sum_probs_key_multi_launch(gpu):
    # 512 units: the single launch would need two records per unit, so the
    # MFMA multi-launch kernels run (keys from each gist split's unrounded sums)
    wl = SMALL["b128-g2-d64-c4-fit"]
    say(f"[parity] {wl.name} sum-of-probabilities key, multi-launch")
    inp = gi.make_inputs(wl, 22, seq_lens=lens_for(wl, "ragged", 8))
    flags = gsa.GSA_SCORE_SUM_PROBS
    res = GU.run_gpu(GU.to(inp, gpu), flags=flags)
    GU.check_gsa(inp, res, flags=flags)


@pytest.mark.parametrize("extra", ["selected-gists", "portable"])
def test_sum_probs_key_combined(gpu, extra):
    wl = SMALL["b2-g7-d128-c16"]
    say(f"[parity] sum-of-probabilities key + {extra}")
    inp = gi.make_inputs(wl, 23, seq_lens=lens_for(wl, "ragged", 7))
    flags = gsa.GSA_SCORE_SUM_PROBS | (gsa.GSA_SET_SELECTED_GISTS if extra == "selected-gists"
                                       else gsa.GSA_PATH_PORTABLE)
    res = GU.run_gpu(GU.to(inp, gpu), flags=flags)
    GU.check_gsa(inp, res, flags=flags & ~gsa.GSA_PATH_PORTABLE)


@pytest.mark.timeout(300)
def test_sum_probs_key_full_workload(gpu):
    wl = gi.QWEN7B_128K
    say(f"[parity] full {wl.name} sum-of-probabilities key, every unit")
    inp = gi.make_inputs(wl, gi.seed_of(2), device=gpu)
    flags = gsa.GSA_SCORE_SUM_PROBS
    res = GU.run_gpu(inp, flags=flags)
    GU.check_gsa(inp, res, flags=flags)
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["b3-g4-d64-c8", "b2-g7-d128-c16", "f32-b2-g3-d64"])
@pytest.mark.parametrize("p", [0.3, 0.9])
@pytest.mark.parametrize("lens", ["full", "edge"])
def test_small_top_p(gpu, name, p, lens):
    wl = SMALL[name]
    say(f"[parity] {name} top-p {p} lens={lens}")
    inp = gi.make_inputs(wl, 41, seq_lens=lens_for(wl, lens, 9))
    res = GU.run_gpu(GU.to(inp, gpu), top_p=p)
    GU.check_gsa_topp(inp, res, p, wl.top_k)


@pytest.mark.parametrize("extra", ["selected-gists", "portable"])
def test_top_p_combined(gpu, extra):
    wl = SMALL["b2-g7-d128-c16"]
    say(f"[parity] top-p + {extra}")
    inp = gi.make_inputs(wl, 43, seq_lens=lens_for(wl, "ragged", 3))
    flags = gsa.GSA_SET_SELECTED_GISTS if extra == "selected-gists" else gsa.GSA_PATH_PORTABLE
    res = GU.run_gpu(GU.to(inp, gpu), top_p=0.8, flags=flags)
    if extra == "selected-gists":
        # the set rule changes the output only: the oracle on the GPU's set,
        # with the same rule (the cut itself is checked by the other cases)
        out, sel, _ = res
        for b in range(wl.batch):
            for g in range(wl.num_kv_heads):
                sub = GU.to(GU.unit_inputs(inp, b, g), "cpu")
                o_out, _, _ = GU.U.run_oracle(sub, top_k=wl.top_k, flags=flags,
                                              ext_sel=sel[b:b + 1, g:g + 1])
                GU.assert_close(out[b, g * wl.group:(g + 1) * wl.group], o_out[0], wl.dtype,
                                f"unit {(b, g)}")
    else:
        GU.check_gsa_topp(inp, res, 0.8, wl.top_k)


@pytest.mark.timeout(300)
def test_top_p_full_workload(gpu):
    wl = gi.QWEN7B_128K
    say(f"[parity] full {wl.name} top-p 0.9, every unit")
    inp = gi.make_inputs(wl, gi.seed_of(2), device=gpu)
    res = GU.run_gpu(inp, top_p=0.9)
    GU.check_gsa_topp(inp, res, 0.9, wl.top_k)
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("flags,top_p", [(0, 0.0), (0, 1.5), (1, 0.5)])
def test_top_p_rejected(gpu, flags, top_p):
    """top-p needs 0 < p <= 1 and the default key; H-GSA does not take it."""
    wl = SMALL["b3-g4-d64-c8"]
    inp = GU.to(gi.make_inputs(wl, 3), gpu)
    p = gsa.make_params(inp.q, wl.num_kv_heads, wl.top_k, 0.0, flags | gsa.GSA_SELECT_TOP_P, 0.0)
    p.top_p = top_p
    kv = gsa.make_kv(inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens, wl.num_chunks,
                     wl.chunk_size, wl.page_chunks)
    assert gsa.gsa_workspace_size(p, kv) == 0
    wh = SMALL_H["h-b2-g4-d64-r4"]
    ih = GU.to(gi.make_inputs(wh, 3), gpu)
    with pytest.raises(gsa.GsaError):
        gsa.hgsa_decode(ih.q, ih.k_cache, ih.v_cache, ih.block_table, ih.seq_lens,
                        ih.k_meta, ih.v_meta, num_chunks=wh.num_chunks,
                        chunk_size=wh.chunk_size, page_chunks=wh.page_chunks,
                        gists_per_meta=wh.gists_per_meta, top_k_meta=wh.top_k_meta,
                        top_k=wh.top_k, flags=gsa.GSA_SELECT_TOP_P)


def test_sum_probs_key_rejected_by_hgsa(gpu):
    wl = SMALL_H["h-b2-g4-d64-r4"]
    inp = GU.to(gi.make_inputs(wl, 3), gpu)
    with pytest.raises(gsa.GsaError):
        gsa.hgsa_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens,
                        inp.k_meta, inp.v_meta, num_chunks=wl.num_chunks,
                        chunk_size=wl.chunk_size, page_chunks=wl.page_chunks,
                        gists_per_meta=wl.gists_per_meta, top_k_meta=wl.top_k_meta,
                        top_k=wl.top_k, flags=gsa.GSA_SCORE_SUM_PROBS)


@pytest.mark.parametrize("name", ["b3-g4-d64-c8", "b2-g7-d128-c16"])
def test_portable_path_on_bf16(gpu, name):
    wl = SMALL[name]
    say(f"[parity] {name} portable kernels")
    inp = gi.make_inputs(wl, 5, seq_lens=lens_for(wl, "ragged", 4))
    res = GU.run_gpu(GU.to(inp, gpu), flags=gsa.GSA_PATH_PORTABLE)
    GU.check_gsa(inp, res)


def test_custom_scale(gpu):
    wl = SMALL["b2-g7-d128-c16"]
    say("[parity] sm_scale=0.05")
    inp = gi.make_inputs(wl, 15)
    res = GU.run_gpu(GU.to(inp, gpu), sm_scale=0.05)
    GU.check_gsa(inp, res, sm_scale=0.05)


def test_shared_and_shuffled_pages(gpu):
    wl = SMALL["b3-g4-d64-c8"]
    say("[parity] shared pages")
    inp = gi.make_inputs(wl, 21, seq_lens=[2000, 1500, 2400])
    inp = gi.share_pages(inp, 0, 2)
    res = GU.run_gpu(GU.to(inp, gpu))
    GU.check_gsa(inp, res)
    inp2 = gi.make_inputs(wl, 21, seq_lens=[2000, 1500, 2400], shuffle_pages=False)
    res2 = GU.run_gpu(GU.to(inp2, gpu))
    GU.check_gsa(inp2, res2)


def test_tiny_f32_workload(gpu):
    wl = gi.TINY_F32
    say(f"[parity] {wl.name}")
    inp = gi.make_inputs(wl, gi.seed_of(0))
    res = GU.run_gpu(GU.to(inp, gpu))
    assert GU.check_gsa(inp, res) == 0
    assert set(inp.planted[0, 0].tolist()) <= set(res[1][0, 0].tolist())


def test_deterministic(gpu):
    wl = SMALL["b2-g7-d128-c16"]
    say("[parity] determinism")
    g_inp = GU.to(gi.make_inputs(wl, 3, seq_lens=lens_for(wl, "ragged", 7)), gpu)
    first = GU.run_gpu(g_inp)
    for _ in range(5):
        again = GU.run_gpu(g_inp)
        for x, y in zip(first, again):
            assert np.array_equal(x, y)


FULL = [gi.LLAMA1B_32K, gi.QWEN7B_128K, gi.MULTIDOC_120K]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("idx", [1, 2, 3])
def test_full_workload_every_unit(gpu, idx):
    wl = gi.WORKLOADS[idx]
    say(f"[parity] full {wl.name}, every unit")
    inp = gi.make_inputs(wl, gi.seed_of(idx), device=gpu)
    res = GU.run_gpu(inp)
    GU.check_gsa(inp, res)
    # planted chunks are routed to (align planting: every planted chunk kept)
    if wl.plant == "align":
        sel = res[1]
        for b in range(wl.batch):
            for g in range(wl.num_kv_heads):
                assert set(inp.planted[b, g].tolist()) <= set(sel[b, g].tolist())
    del inp
    torch.cuda.empty_cache()


def plant_raw_rows(inp, offset=3.0):
    """Make the unfolded rows carry the result: the raw tokens of every
    planted chunk get keys aligned with the group's query (as the planted gist
    keys are) and values shifted by `offset` in every coordinate (pure
    indexing on the device).  The raw tokens of the selected chunks then hold
    most of the softmax mass, so reading a wrong chunk, page or row moves the
    outputs by a large fraction of `offset`."""
    wl = inp.wl
    C, spp, d = wl.chunk_size, wl.slots_per_page, wl.head_dim
    qdir = gi.group_direction(inp.q.float(), wl.num_kv_heads)          # [B][Hkv][d]
    gen = torch.Generator(device=inp.q.device).manual_seed(9)
    B, Hkv, P = inp.planted.shape
    slots = inp.planted.view(B, Hkv, P, 1) * (C + 1) + torch.arange(C, device=inp.q.device)
    bidx = torch.arange(B, device=inp.q.device).view(B, 1, 1, 1).expand_as(slots)
    gidx = torch.arange(Hkv, device=inp.q.device).view(1, Hkv, 1, 1).expand_as(slots)
    page = inp.block_table.long()[bidx, slots // spp]
    off = slots % spp
    noise = 0.1 * torch.randn(*slots.shape, d, generator=gen, device=inp.q.device)
    kk = 2.0 * math.sqrt(d) * qdir.view(B, Hkv, 1, 1, d) + noise
    inp.k_cache[page, gidx, off] = kk.to(inp.k_cache.dtype)
    vv = inp.v_cache[page, gidx, off].float() + offset
    inp.v_cache[page, gidx, off] = vv.to(inp.v_cache.dtype)


@pytest.mark.timeout(300)
def test_full_workload_unfolded_rows_carry_the_output(gpu):
    """qwen2-7b shape with the planted chunks' raw rows aligned with the query
    and their values shifted by 3: the output is dominated by the unfolded
    rows, so a wrong gather fails by far more than the bf16 tolerance."""
    wl = gi.QWEN7B_128K
    say(f"[parity] full {wl.name}, unfolded rows carry the output")
    inp = gi.make_inputs(wl, gi.seed_of(2), device=gpu)
    plant_raw_rows(inp)
    res = GU.run_gpu(inp)
    GU.check_gsa(inp, res)
    out, sel = res[0], res[1]
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            assert set(inp.planted[b, g].tolist()) <= set(sel[b, g].tolist())
    # the shifted rows carry much of the mass: output coordinates sit near the offset
    means = out.mean(axis=-1)
    assert float(np.mean(means)) > 2.0 and float(np.min(means)) > 0.5
    del inp
    torch.cuda.empty_cache()


# ---------------- H-GSA ----------------

SMALL_H = {
    "h-b2-g4-d64-r4": gi.Workload("h-b2-g4-d64-r4", gi.BF16, 2, 8, 2, 64, 8, 400, 12, 16,
                                  plant="align_meta", plant_count=3, gists_per_meta=4,
                                  top_k_meta=6),
    "h-b1-g7-d128-r16": gi.Workload("h-b1-g7-d128-r16", gi.BF16, 1, 7, 1, 128, 16, 600, 20, 16,
                                    plant="align_meta", plant_count=2, gists_per_meta=16,
                                    top_k_meta=5),
    "h-f32-b2-g2-r8": gi.Workload("h-f32-b2-g2-r8", gi.F32, 2, 4, 2, 64, 4, 256, 10, 16,
                                  plant="align_meta", plant_count=2, gists_per_meta=8,
                                  top_k_meta=3),
}


@pytest.mark.parametrize("name", sorted(SMALL_H))
@pytest.mark.parametrize("lens", ["full", "ragged", "edge"])
def test_hgsa_small(gpu, name, lens):
    wl = SMALL_H[name]
    say(f"[parity] {name} lens={lens}")
    inp = gi.make_inputs(wl, 200 + len(name), seq_lens=lens_for(wl, lens, 5))
    res = GU.run_gpu_h(GU.to(inp, gpu))
    GU.check_hgsa(inp, res)


@pytest.mark.parametrize("k1,k2", [(0, 5), (2, 0), (10 ** 5, 10 ** 5)])
def test_hgsa_extremes(gpu, k1, k2):
    wl = SMALL_H["h-b2-g4-d64-r4"]
    say(f"[parity] hgsa k1={k1} k2={k2}")
    inp = gi.make_inputs(wl, 17, seq_lens=lens_for(wl, "ragged", 8))
    res = GU.run_gpu_h(GU.to(inp, gpu), top_k=k2, top_k_meta=k1)
    GU.check_hgsa(inp, res, top_k=k2, top_k_meta=k1)


@pytest.mark.timeout(300)
def test_hgsa_full_workload_every_unit(gpu):
    wl = gi.HGSA_1M
    say(f"[parity] full {wl.name}, every unit")
    inp = gi.make_inputs(wl, gi.seed_of(4), device=gpu)
    res = GU.run_gpu_h(inp)
    GU.check_hgsa(inp, res)
    # planted meta-groups and chunks are routed to
    s1, s2 = res[1], res[2]
    R = wl.gists_per_meta
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            pl = inp.planted[b, g].tolist()
            assert {m // R for m in pl} <= set(s1[b, g].tolist())
            assert set(pl) <= set(s2[b, g].tolist())
    del inp
    torch.cuda.empty_cache()


def test_workspace_reuse_across_shapes(gpu):
    """One zero-filled workspace shared by calls of different shapes and paths
    (single-launch and multi-launch) in a row: the control block stays zero."""
    say("[parity] workspace reuse across shapes")
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=gpu)
    cases = [("b2-g7-d128-c16", 0), ("b3-g4-d64-c8", gsa.GSA_PATH_PORTABLE),
             ("b2-g16-d64-c4", 0), ("b3-g4-d64-c8", 0), ("b2-g7-d128-c16", 0)]
    for i, (name, flags) in enumerate(cases):
        wl = SMALL[name]
        inp = gi.make_inputs(wl, 300 + i, seq_lens=lens_for(wl, "ragged", i))
        g_inp = GU.to(inp, gpu)
        k = wl.top_k
        sel = torch.full((wl.batch, wl.num_kv_heads, k), -7, dtype=torch.int32, device=gpu)
        out = gsa.gsa_decode(g_inp.q, g_inp.k_cache, g_inp.v_cache, g_inp.block_table,
                             g_inp.seq_lens, num_chunks=wl.num_chunks, chunk_size=wl.chunk_size,
                             page_chunks=wl.page_chunks, top_k=k, flags=flags, sel_idx=sel, ws=ws)
        torch.cuda.synchronize()
        GU.check_gsa(inp, (out.float().cpu().numpy(), sel.cpu().numpy(), None))
        assert int(ws[:gsa.WORKSPACE_CONTROL_BYTES].count_nonzero()) == 0


def test_workspace_reuse_degenerate_selections(gpu):
    """One workspace shared by calls whose selections are empty, complete or
    absent (k = 0, the selected-gists set, H-GSA with no kept group or no
    selected chunk): after every call the control block is zero again and the
    next call is right."""
    say("[parity] workspace reuse, degenerate selections")
    ws = torch.zeros(96 << 20, dtype=torch.uint8, device=gpu)
    flat = [("b2-g7-d128-c16", 0, 0), ("b2-g7-d128-c16", gsa.GSA_SET_SELECTED_GISTS, 0),
            ("b2-g7-d128-c16", gsa.GSA_SET_SELECTED_GISTS, 5), ("b3-g4-d64-c8", 0, 10 ** 5),
            ("b2-g7-d128-c16", 0, 8)]
    hier = [(0, 5), (2, 0), (0, 0), (10 ** 5, 10 ** 5), (6, 12)]
    for i, (name, flags, k) in enumerate(flat):
        wl = SMALL[name]
        inp = gi.make_inputs(wl, 400 + i, seq_lens=lens_for(wl, "edge" if i % 2 else "ragged", i))
        g_inp = GU.to(inp, gpu)
        sel = torch.full((wl.batch, wl.num_kv_heads, max(k, 1)), -7, dtype=torch.int32, device=gpu)
        out = gsa.gsa_decode(g_inp.q, g_inp.k_cache, g_inp.v_cache, g_inp.block_table,
                             g_inp.seq_lens, num_chunks=wl.num_chunks, chunk_size=wl.chunk_size,
                             page_chunks=wl.page_chunks, top_k=k, flags=flags,
                             sel_idx=sel if k > 0 else None, ws=ws)
        torch.cuda.synchronize()
        if k > 0:
            GU.check_gsa(inp, (out.float().cpu().numpy(), sel.cpu().numpy(), None), top_k=k, flags=flags)
        assert int(ws[:gsa.WORKSPACE_CONTROL_BYTES].count_nonzero()) == 0, (name, flags, k)
    wl = SMALL_H["h-b2-g4-d64-r4"]
    for i, (k1, k2) in enumerate(hier):
        inp = gi.make_inputs(wl, 500 + i, seq_lens=lens_for(wl, "ragged", 20 + i))
        g_inp = GU.to(inp, gpu)
        s1 = torch.full((wl.batch, wl.num_kv_heads, max(k1, 1)), -7, dtype=torch.int32, device=gpu)
        s2 = torch.full((wl.batch, wl.num_kv_heads, max(k2, 1)), -7, dtype=torch.int32, device=gpu)
        out = gsa.hgsa_decode(g_inp.q, g_inp.k_cache, g_inp.v_cache, g_inp.block_table,
                              g_inp.seq_lens, g_inp.k_meta, g_inp.v_meta, num_chunks=wl.num_chunks,
                              chunk_size=wl.chunk_size, page_chunks=wl.page_chunks,
                              gists_per_meta=wl.gists_per_meta, top_k_meta=k1, top_k=k2,
                              sel_meta=s1 if k1 > 0 else None, sel_idx=s2 if k2 > 0 else None, ws=ws)
        torch.cuda.synchronize()
        if k1 > 0 and k2 > 0:
            GU.check_hgsa(inp, (out.float().cpu().numpy(), s1.cpu().numpy(), s2.cpu().numpy()),
                          top_k=k2, top_k_meta=k1)
        assert int(ws[:gsa.WORKSPACE_CONTROL_BYTES].count_nonzero()) == 0, ("hgsa", k1, k2)


def test_prepared_call_matches(gpu):
    """A prepared call gives the same bits as gsa_decode, call after call."""
    wl = SMALL["b2-g7-d128-c16"]
    say("[parity] prepared call")
    g_inp = GU.to(gi.make_inputs(wl, 31, seq_lens=lens_for(wl, "ragged", 2)), gpu)
    want = gsa.gsa_decode(g_inp.q, g_inp.k_cache, g_inp.v_cache, g_inp.block_table, g_inp.seq_lens,
                          num_chunks=wl.num_chunks, chunk_size=wl.chunk_size,
                          page_chunks=wl.page_chunks, top_k=wl.top_k)
    call = gsa.prepare_gsa_decode(g_inp.q, g_inp.k_cache, g_inp.v_cache, g_inp.block_table,
                                  g_inp.seq_lens, num_chunks=wl.num_chunks,
                                  chunk_size=wl.chunk_size, page_chunks=wl.page_chunks,
                                  top_k=wl.top_k)
    for _ in range(3):
        call()
        torch.cuda.synchronize()
        assert torch.equal(call.out, want)


@pytest.mark.parametrize("batch", [32, 33])
def test_unit_limits(gpu, batch):
    """H-GSA at 256 units (the single launch's limit: two control records per
    unit, the last ones at the end of the control block) and at 264 (the
    multi-launch path), flat GSA at the same batches (512 and 528 units, the
    flat limit and past it): the first and the last units against the oracle,
    and the control block zero afterwards."""
    say(f"[parity] unit limits batch={batch}")
    ws = torch.zeros(256 << 20, dtype=torch.uint8, device=gpu)
    wl = gi.Workload(f"h-limit-b{batch}", gi.BF16, batch, 8, 8, 64, 4, 96, 6, 16,
                     plant="align_meta", plant_count=2, gists_per_meta=4, top_k_meta=3)
    inp = gi.make_inputs(wl, 700 + batch, seq_lens=lens_for(wl, "ragged", 30 + batch))
    g = GU.to(inp, gpu)
    B, H = wl.batch, wl.num_kv_heads
    s1 = torch.full((B, H, wl.top_k_meta), -7, dtype=torch.int32, device=gpu)
    s2 = torch.full((B, H, wl.top_k), -7, dtype=torch.int32, device=gpu)
    out = gsa.hgsa_decode(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.k_meta, g.v_meta,
                          num_chunks=wl.num_chunks, chunk_size=wl.chunk_size, page_chunks=wl.page_chunks,
                          gists_per_meta=wl.gists_per_meta, top_k_meta=wl.top_k_meta, top_k=wl.top_k,
                          sel_meta=s1, sel_idx=s2, ws=ws)
    torch.cuda.synchronize()
    ends = [(0, 0), (B // 2, 3), (B - 1, H - 2), (B - 1, H - 1)]
    GU.check_hgsa(inp, (out.float().cpu().numpy(), s1.cpu().numpy(), s2.cpu().numpy()), units=ends)
    assert int(ws[:gsa.WORKSPACE_CONTROL_BYTES].count_nonzero()) == 0
    wl = gi.Workload(f"limit-b{batch}", gi.BF16, batch, 16, 16, 64, 4, 96, 6, 16)
    inp = gi.make_inputs(wl, 800 + batch, seq_lens=lens_for(wl, "ragged", 40 + batch))
    g = GU.to(inp, gpu)
    B, H = wl.batch, wl.num_kv_heads
    sel = torch.full((B, H, wl.top_k), -7, dtype=torch.int32, device=gpu)
    out = gsa.gsa_decode(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens,
                         num_chunks=wl.num_chunks, chunk_size=wl.chunk_size, page_chunks=wl.page_chunks,
                         top_k=wl.top_k, sel_idx=sel, ws=ws)
    torch.cuda.synchronize()
    ends = [(0, 0), (B // 2, 7), (B - 1, H - 2), (B - 1, H - 1)]
    GU.check_gsa(inp, (out.float().cpu().numpy(), sel.cpu().numpy(), None), units=ends)
    assert int(ws[:gsa.WORKSPACE_CONTROL_BYTES].count_nonzero()) == 0


# Block-table rows around the lengths the kernels keep in LDS: the flat select
# keeps a row of up to 768 pages; H-GSA's candidate tasks keep a row of up to
# 4096 pages (head_dim 64) or 8192 (head_dim 128).  One chunk per page: a row
# holds num_chunks + 1 pages (chunk size 2) or num_chunks (chunk size 1).
LONG_ROWS = {
    "rows-flat-768": gi.Workload("rows-flat-768", gi.BF16, 2, 8, 2, 64, 2, 767, 20, 1,
                                 plant="align", plant_count=3),
    "rows-flat-1001": gi.Workload("rows-flat-1001", gi.BF16, 2, 8, 2, 64, 2, 1000, 20, 1,
                                  plant="align", plant_count=3),
    "rows-h-d64-4096": gi.Workload("rows-h-d64-4096", gi.BF16, 1, 8, 2, 64, 2, 4095, 16, 1,
                                   plant="align_meta", plant_count=2, gists_per_meta=16,
                                   top_k_meta=6),
    "rows-h-d64-4201": gi.Workload("rows-h-d64-4201", gi.BF16, 1, 8, 2, 64, 2, 4200, 16, 1,
                                   plant="align_meta", plant_count=2, gists_per_meta=16,
                                   top_k_meta=6),
    "rows-h-d128-8192": gi.Workload("rows-h-d128-8192", gi.BF16, 1, 4, 1, 128, 1, 8192, 16, 1,
                                    plant="align_meta", plant_count=2, gists_per_meta=16,
                                    top_k_meta=6),
    "rows-h-d128-8300": gi.Workload("rows-h-d128-8300", gi.BF16, 1, 4, 1, 128, 1, 8300, 16, 1,
                                    plant="align_meta", plant_count=2, gists_per_meta=16,
                                    top_k_meta=6),
}


@pytest.mark.parametrize("name", sorted(LONG_ROWS))
def test_long_block_table_rows(gpu, name):
    wl = LONG_ROWS[name]
    say(f"[parity] {name} max_pages={wl.max_pages}")
    inp = gi.make_inputs(wl, 300 + len(name), seq_lens=lens_for(wl, "ragged", 11))
    if wl.hgsa:
        GU.check_hgsa(inp, GU.run_gpu_h(GU.to(inp, gpu)))
    else:
        GU.check_gsa(inp, GU.run_gpu(GU.to(inp, gpu)))


# ---------------- the boundary on the device ----------------

def test_device_is_gfx950(gpu):
    """The library's device check agrees with the device's own name: calls
    succeed on this gfx950 (every other GPU test depends on that)."""
    assert torch.cuda.get_device_properties(gpu).gcnArchName.startswith("gfx950")


def test_call_on_a_side_stream(gpu):
    """A call on a stream that is not the current one: the binding allocates
    the output and the cached workspace on that stream (the zero fill ordered
    before the kernel), results equal the current-stream call bit for bit, and
    that stream's workspace is left with a zero control block."""
    wl = SMALL["b2-g7-d128-c16"]
    say("[parity] side stream")
    g_inp = GU.to(gi.make_inputs(wl, 77, seq_lens=lens_for(wl, "ragged", 12)), gpu)
    want = gsa.gsa_decode(g_inp.q, g_inp.k_cache, g_inp.v_cache, g_inp.block_table, g_inp.seq_lens,
                          num_chunks=wl.num_chunks, chunk_size=wl.chunk_size,
                          page_chunks=wl.page_chunks, top_k=wl.top_k)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=gpu)
    side.wait_stream(torch.cuda.current_stream(gpu))
    for _ in range(3):
        got = gsa.gsa_decode(g_inp.q, g_inp.k_cache, g_inp.v_cache, g_inp.block_table,
                             g_inp.seq_lens, num_chunks=wl.num_chunks, chunk_size=wl.chunk_size,
                             page_chunks=wl.page_chunks, top_k=wl.top_k, stream=side)
        side.synchronize()
        assert torch.equal(got, want)
    p = gsa.make_params(g_inp.q, wl.num_kv_heads, wl.top_k)
    kv = gsa.make_kv(g_inp.k_cache, g_inp.v_cache, g_inp.block_table, g_inp.seq_lens,
                     wl.num_chunks, wl.chunk_size, wl.page_chunks)
    ws = gsa.workspace(gsa.gsa_workspace_size(p, kv), gpu, side)
    assert ws is not gsa.workspace(0, gpu)  # its own control block
    GU.check_control(ws, "side stream")


def test_workspace_status_and_reset(gpu):
    """The error word reads through gsa_workspace_status; gsa_workspace_reset
    zeroes a dirtied control block (the recovery step), after which calls are
    right again."""
    wl = SMALL["b3-g4-d64-c8"]
    say("[parity] workspace status and reset")
    ws = torch.zeros(gsa.WORKSPACE_CONTROL_BYTES + (8 << 20), dtype=torch.uint8, device=gpu)
    assert gsa.gsa_workspace_status(ws) == 0
    ws[:gsa.WORKSPACE_CONTROL_BYTES].fill_(0x5A)         # as if a call had left it dirty
    assert gsa.gsa_workspace_status(ws) == 8
    gsa.gsa_workspace_reset(ws)
    assert gsa.gsa_workspace_status(ws) == 0
    assert int(ws[:gsa.WORKSPACE_CONTROL_BYTES].count_nonzero()) == 0
    inp = gi.make_inputs(wl, 78, seq_lens=lens_for(wl, "ragged", 13))
    g = GU.to(inp, gpu)
    sel = torch.full((wl.batch, wl.num_kv_heads, wl.top_k), -7, dtype=torch.int32, device=gpu)
    out = gsa.gsa_decode(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens,
                         num_chunks=wl.num_chunks, chunk_size=wl.chunk_size,
                         page_chunks=wl.page_chunks, top_k=wl.top_k, sel_idx=sel, ws=ws)
    torch.cuda.synchronize()
    GU.check_control(ws, "after reset")
    GU.check_gsa(inp, (out.float().cpu().numpy(), sel.cpu().numpy(), None))
