"""Parity of mgsa_decode (the hierarchy of any depth, through the C ABI)
with the oracle: every unit, the gap rule at every level, outputs against the
oracle run with the GPU's selections (bf16: 2e-2 abs / 1e-2 rel)."""
import numpy as np
import pytest
import torch

import long_context_sparse_gist_amd as gsa
from long_context_sparse_gist_amd import inputs as gi
from tests import gpu_util as GU
from tests import test_oracle_levels as PL

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


SMALL = {
    "lv-b2-g4-d64-c8": gi.Workload("lv-b2-g4-d64-c8", gi.BF16, 2, 8, 2, 64, 8, 700, 12, 16,
                                   plant="align", plant_count=3),
    "lv-b2-g7-d128-c16": gi.Workload("lv-b2-g7-d128-c16", gi.BF16, 2, 14, 2, 128, 16, 1100, 20, 16,
                                     plant="align", plant_count=4),
    "lv-b3-g1-d128-c4": gi.Workload("lv-b3-g1-d128-c4", gi.BF16, 3, 3, 3, 128, 4, 900, 9, 32,
                                    plant="align", plant_count=2),
}
# (fanouts, kept per level, level 1 first)
SHAPES = {0: ((), ()), 1: ((8,), (6,)), 2: ((4, 4), (5, 3)), 3: ((4, 3, 3), (6, 4, 2))}


def lens_for(wl, kind, seed):
    M, C = wl.num_chunks, wl.chunk_size
    if kind == "full":
        return None
    rng = np.random.default_rng(seed)
    L = [int(x) for x in rng.integers(1, M * C + C - 1, size=wl.batch)]
    if kind == "edge":
        L[0] = 0
        if wl.batch > 1:
            L[1] = 5 * C + 1     # fewer chunks than one group at the upper levels
    return L


def levels_on(inp, fanouts, tops, seed, dev):
    return [(k.to(dev), v.to(dev), R, t) for k, v, R, t in PL.with_levels(inp, fanouts, tops, seed)]


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("depth", [0, 1, 2, 3])
@pytest.mark.parametrize("lens", ["full", "ragged", "edge"])
def test_levels_small(gpu, name, depth, lens):
    wl = SMALL[name]
    say(f"[levels] {name} depth={depth} lens={lens}")
    inp = gi.make_inputs(wl, 900 + depth, seq_lens=lens_for(wl, lens, 7 + depth))
    fanouts, tops = SHAPES[depth]
    g = GU.to(inp, gpu)
    lv = levels_on(inp, fanouts, tops, 40 + depth, gpu)
    res = GU.run_gpu_m(g, lv)
    GU.check_mgsa(inp, [(k.cpu(), v.cpu(), R, t) for k, v, R, t in lv], res)


@pytest.mark.parametrize("tops", [(0, 3), (100, 100), (2, 0)])
def test_levels_extreme_k(gpu, tops):
    wl = SMALL["lv-b2-g4-d64-c8"]
    say(f"[levels] extreme k {tops}")
    inp = gi.make_inputs(wl, 931, seq_lens=lens_for(wl, "ragged", 3))
    lv = levels_on(inp, (4, 4), tops, 44, gpu)
    for k0 in (0, 5, 10 ** 5):
        res = GU.run_gpu_m(GU.to(inp, gpu), lv, top_k=k0)
        GU.check_mgsa(inp, [(k.cpu(), v.cpu(), R, t) for k, v, R, t in lv], res, top_k=k0)


@pytest.mark.parametrize("name", sorted(PL.CASES))
def test_levels_hand_worked_bf16(gpu, name):
    """The hand-worked three-level examples in bf16 (head_dim 64): the
    selections exactly, the output within 2 % of the exact fraction (bf16
    rounding of the logarithms and of the output) and within the bf16
    tolerance of the oracle on the same rounded inputs; a read of any slot or
    entry no example may read (V = 999) would move it far past either."""
    import oracle
    case = PL.CASES[name]
    c = case["cfg"]
    say(f"[levels golden bf16] {name}")
    q, k, v, bt, sl, levels = PL.golden_arrays(case, 64)
    t = lambda x: torch.from_numpy(x).to(gpu).to(torch.bfloat16)  # noqa: E731
    lv = [(t(km), t(vm), R, kk) for km, vm, R, kk in levels]
    qg, kg, vg = t(q), t(k), t(v)
    btg, slg = torch.from_numpy(bt).to(gpu), torch.from_numpy(sl).to(gpu)
    sels = [torch.full((1, 1, kk), -7, dtype=torch.int32, device=gpu)
            for kk in [c["top_k"]] + [x[3] for x in levels]]
    out = gsa.mgsa_decode(qg, kg, vg, btg, slg, lv, num_chunks=c["num_chunks"],
                          chunk_size=c["chunk_size"], page_chunks=c["page_chunks"],
                          top_k=c["top_k"], sm_scale=1.0, sel=sels)
    torch.cuda.synchronize()
    for l, key in enumerate(["expect_sel", "expect_sel_l1", "expect_sel_l2"]):
        got = sels[l][0, 0].tolist()
        assert got[:len(case[key])] == case[key] and all(x == -1 for x in got[len(case[key]):])
    o = out[0, 0].float().cpu().numpy()
    np.testing.assert_allclose(o[:2], case["expect_out"], rtol=2e-2, atol=2e-2)
    bf = lambda x: x.cpu().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    cfg = dict(PL.golden_cfg(case, 64), dtype=1)
    ref, _, _ = oracle.mgsa_decode(cfg, bf(qg), bf(kg), bf(vg), bt, sl,
                                   [(bf(a), bf(b_), R, kk) for a, b_, R, kk in lv])
    np.testing.assert_allclose(o, ref[0, 0], rtol=1e-2, atol=2e-2)
    assert np.all(o[2:] == 0.0)


DEEP = {5: ((2, 2, 2, 2, 2), (40, 20, 10, 6, 4)),
        8: ((2,) * 8, (30, 16, 8, 6, 4, 3, 2, 2))}


@pytest.mark.parametrize("depth", sorted(DEEP))
@pytest.mark.parametrize("lens", ["full", "edge"])
def test_levels_deep(gpu, depth, lens):
    """Five and eight (the most the ABI takes) meta levels of fanout 2 above
    1100 gists: every level's kept ids and the final list's segments of every
    level, every unit."""
    wl = SMALL["lv-b2-g7-d128-c16"]
    say(f"[levels] deep {depth} lens={lens}")
    inp = gi.make_inputs(wl, 950 + depth, seq_lens=lens_for(wl, lens, 17 + depth))
    fanouts, tops = DEEP[depth]
    g = GU.to(inp, gpu)
    lv = levels_on(inp, fanouts, tops, 70 + depth, gpu)
    res = GU.run_gpu_m(g, lv)
    GU.check_mgsa(inp, [(k.cpu(), v.cpu(), R, t) for k, v, R, t in lv], res)


LONG_TOP = gi.Workload("lv-long-top", gi.BF16, 2, 8, 2, 128, 16, 20000, 24, 16,
                       plant="align", plant_count=4)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("depth", [0, 1])
@pytest.mark.parametrize("lens", ["full", "ragged"])
def test_levels_long_top(gpu, depth, lens):
    """A top level longer than the top-level pass's workgroups cover one block
    each (20000 gists, or 10000 meta entries of fanout 2): each workgroup
    folds several 128-row blocks with its online softmax, and ragged lengths
    leave some of a unit's workgroups without a block."""
    wl = LONG_TOP
    say(f"[levels] long top depth={depth} lens={lens}")
    inp = gi.make_inputs(wl, 1300 + depth, seq_lens=lens_for(wl, lens, 31 + depth))
    fanouts, tops = ((), ()) if depth == 0 else ((2,), (40,))
    g = GU.to(inp, gpu)
    lv = levels_on(inp, fanouts, tops, 60 + depth, gpu)
    res = GU.run_gpu_m(g, lv)
    GU.check_mgsa(inp, [(k.cpu(), v.cpu(), R, t) for k, v, R, t in lv], res)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("lens", ["full", "ragged"])
def test_levels_long_candidates(gpu, lens):
    """A candidate list longer than one wavefront selects (100 kept entries of
    fanout 16 above 20000 gists: 1600 candidates), selected by the whole
    workgroup from the lists the chain keeps in LDS."""
    wl = LONG_TOP
    say(f"[levels] long candidate list lens={lens}")
    inp = gi.make_inputs(wl, 1320, seq_lens=lens_for(wl, lens, 41))
    g = GU.to(inp, gpu)
    lv = levels_on(inp, (16,), (100,), 80, gpu)
    res = GU.run_gpu_m(g, lv)
    GU.check_mgsa(inp, [(k.cpu(), v.cpu(), R, t) for k, v, R, t in lv], res)


MGSA_1M = gi.Workload("mgsa-1m-c16-r16x16", gi.BF16, 4, 32, 8, 128, 16, 65536, 64, 16,
                      plant="align", plant_count=16)


@pytest.mark.timeout(300)
def test_levels_full_1m_three_levels(gpu):
    """The 1M-token H-GSA shape with a third level (4096 level-1 entries under
    256 level-2 entries, keeping 16, 32 and 64 going down): every unit, and the
    planted chunks and their ancestors are kept."""
    wl = MGSA_1M
    say(f"[levels] full {wl.name}")
    inp = gi.make_inputs(wl, 1010, device=gpu)
    lv = [(k, v, R, t) for (k, v), R, t in zip(gi.make_levels(inp, (16, 16), 1011), (16, 16), (32, 16))]
    res = GU.run_gpu_m(inp, lv)
    GU.check_mgsa(inp, lv, res)
    out, sels = res
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            pl = inp.planted[b, g].tolist()
            assert set(pl) <= set(sels[0][b, g].tolist())
            assert {m // 16 for m in pl} <= set(sels[1][b, g].tolist())
            assert {m // 256 for m in pl} <= set(sels[2][b, g].tolist())
    del inp, lv
    torch.cuda.empty_cache()
