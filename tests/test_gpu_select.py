"""Selection stress cases of the single-launch path, through the C ABI.

The gist keys are shaped so that every branch of the select runs: slices that
hold many of the largest keys (a second read round), fewer up-front keys than
k, a boundary bucket wider than the candidate buffer (the general select),
exact ties and NaN keys.  Each selection is checked exactly against the
top-k of the GPU's own routing keys (larger key first, ties to the lower
chunk index, NaN last), and the whole result against the oracle under the
gap rule of the parity tests.
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


def set_gist_k(inp, b, g, chunks, rows):
    """Overwrite the gist key rows of `chunks` of unit (b, g) (pure indexing)."""
    wl = inp.wl
    C, spp = wl.chunk_size, wl.slots_per_page
    bt = inp.block_table[b].long().cpu()
    for m, r in zip(chunks, rows):
        s = int(m) * (C + 1) + C
        inp.k_cache[int(bt[s // spp]), g, s % spp] = r.to(inp.k_cache.dtype)


def order_key(x):
    """Order-preserving uint32 image of float32 keys: NaN lowest, -0 == +0."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = np.where(u == 0x80000000, 0, u)
    k = np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000)
    return np.where(np.isnan(np.asarray(x, np.float32)), 0, k)


def exact_topk(keys, k):
    """Ascending ids of the k largest keys: larger order key first, then lower id."""
    ok = order_key(keys)
    idx = np.arange(len(keys))
    order = np.lexsort((idx, -ok.astype(np.int64)))
    return np.sort(order[:min(k, len(keys))])


def check_exact(wl, sel, sc, top_k, lens=None):
    C = wl.chunk_size
    for b in range(wl.batch):
        n = wl.num_chunks if lens is None else lens[b] // C
        for g in range(wl.num_kv_heads):
            want = exact_topk(sc[b, g, :n], top_k)
            keff = len(want)
            got = sel[b, g, :keff]
            assert np.array_equal(got, want), f"unit ({b},{g}): selection is not the exact top-k"
            assert np.all(sel[b, g, keff:] == -1)


def base(name, num_chunks, top_k, batch=2):
    return gi.Workload(name, gi.BF16, batch, 8, 2, 128, 16, num_chunks, top_k, 16)


def case_cluster():
    # 100 of the largest keys in one slice of 256 gists (slice 1), the others
    # spread: slice 1 holds more than the keys read up front
    wl = base("sel-cluster", 1000, 100)
    inp = gi.make_inputs(wl, 501)
    qdir = gi.group_direction(inp.q.float(), wl.num_kv_heads)
    gen = torch.Generator().manual_seed(7)
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            ms = list(range(256, 356)) if g == 0 else list(range(5, 1000, 10))
            noise = 0.3 * torch.randn(len(ms), wl.head_dim, generator=gen)
            set_gist_k(inp, b, g, ms, 2.0 * math.sqrt(wl.head_dim) * qdir[b, g] + noise)
    return wl, inp, wl.top_k


def case_few_upfront():
    # top_k above the keys read up front (2 slices x 32 < 200 < 300 gists)
    wl = base("sel-few", 300, 200)
    return wl, gi.make_inputs(wl, 502), wl.top_k


def _all_equal(name, num_chunks, top_k, seed):
    wl = base(name, num_chunks, top_k)
    inp = gi.make_inputs(wl, seed)
    gen = torch.Generator().manual_seed(seed)
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            r = torch.randn(wl.head_dim, generator=gen)
            set_gist_k(inp, b, g, range(num_chunks), r.expand(num_chunks, -1))
    return wl, inp, top_k


def case_ties():
    # every key equal: the lowest chunk ids win
    return _all_equal("sel-ties", 1000, 100, 503)


def case_ties_wide():
    # every key equal and more of them than the candidate buffer holds
    return _all_equal("sel-ties-wide", 3000, 100, 504)


def case_tie_groups():
    # three distinct keys, each shared by about a third of the gists
    wl = base("sel-groups", 2000, 700)
    inp = gi.make_inputs(wl, 505)
    gen = torch.Generator().manual_seed(505)
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            vecs = torch.randn(3, wl.head_dim, generator=gen)
            which = torch.randint(0, 3, (wl.num_chunks,), generator=gen)
            set_gist_k(inp, b, g, range(wl.num_chunks), vecs[which])
    return wl, inp, wl.top_k


CASES = {"cluster": case_cluster, "few_upfront": case_few_upfront, "ties": case_ties,
         "ties_wide": case_ties_wide, "tie_groups": case_tie_groups}


@pytest.mark.parametrize("case", sorted(CASES))
def test_select_stress(gpu, case):
    say(f"[select] {case}")
    wl, inp, top_k = CASES[case]()
    res = GU.run_gpu(GU.to(inp, gpu), top_k=top_k)
    out, sel, sc = res
    check_exact(wl, sel, sc, top_k)
    if case.startswith("ties"):
        assert np.all(sel[:, :, :top_k] == np.arange(top_k)), "equal keys: the lowest ids win"
    GU.check_gsa(inp, res, top_k=top_k)


@pytest.mark.parametrize("case", ["cluster", "few_upfront", "ties_wide", "tie_groups"])
def test_select_stress_top_p(gpu, case):
    # top-p after each branch of the select (the second round, the general
    # select, tied boundary keys): the kept entries are the exact top N of the
    # GPU's own keys, N a valid cut, and the output the oracle's on that set
    say(f"[select] {case}, top-p 0.5")
    wl, inp, top_k = CASES[case]()
    p = 0.5
    res = GU.run_gpu(GU.to(inp, gpu), top_k=top_k, flags=gsa.GSA_SELECT_TOP_P, top_p=p)
    out, sel, sc = res
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            got = sel[b, g][sel[b, g] >= 0]
            assert np.array_equal(got, exact_topk(sc[b, g, :wl.num_chunks], len(got))), \
                f"unit ({b},{g}): kept entries are not the top of the GPU's keys"
    GU.check_gsa_topp(inp, res, p, top_k)


def test_select_nan_keys(gpu):
    # NaN keys rank below every number; the selection is checked exactly (the
    # attended NaN gists make the outputs NaN, which carry no information)
    wl = base("sel-nan", 600, 50)
    inp = gi.make_inputs(wl, 506)
    gen = torch.Generator().manual_seed(506)
    nan_ids = {}
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            ms = torch.randperm(wl.num_chunks, generator=gen)[:40].tolist()
            nan_ids[(b, g)] = set(ms)
            set_gist_k(inp, b, g, ms, torch.full((len(ms), wl.head_dim), float("nan")))
    say("[select] nan")
    out, sel, sc = GU.run_gpu(GU.to(inp, gpu), top_k=wl.top_k)
    check_exact(wl, sel, sc, wl.top_k)
    for (b, g), ids in nan_ids.items():
        assert np.all(np.isnan(sc[b, g, sorted(ids)]))
        assert not (set(sel[b, g].tolist()) & ids), "a NaN key was selected"


def test_select_nan_fill(gpu):
    # more NaN keys than non-NaN ones: the NaN keys fill the rest, lowest ids first
    wl = base("sel-nan-fill", 400, 100)
    inp = gi.make_inputs(wl, 507)
    keep = {}
    gen = torch.Generator().manual_seed(507)
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            ms = torch.randperm(wl.num_chunks, generator=gen)[:350].tolist()
            keep[(b, g)] = sorted(set(range(wl.num_chunks)) - set(ms))
            set_gist_k(inp, b, g, ms, torch.full((len(ms), wl.head_dim), float("nan")))
    say("[select] nan fill")
    out, sel, sc = GU.run_gpu(GU.to(inp, gpu), top_k=wl.top_k)
    check_exact(wl, sel, sc, wl.top_k)
    for (b, g), ids in keep.items():
        assert set(ids) <= set(sel[b, g].tolist()), "every non-NaN key must be selected"


@pytest.mark.parametrize("top_k, tail, tasks", [(504, 5, 64), (600, 3, 76), (63, 0, 8)])
def test_unfolded_task_counts(gpu, top_k, tail, tasks):
    # many unfolded tasks per unit (their partials all merge into one output),
    # with ragged and exact last tasks
    wl = gi.Workload("many-tasks", gi.BF16, 1, 4, 2, 128, 16, 600, top_k, 16)
    L = wl.num_chunks * wl.chunk_size + tail
    inp = gi.make_inputs(wl, 600 + tasks, seq_lens=[L])
    assert -(-(top_k * wl.chunk_size + tail) // 128) == tasks
    say(f"[select] unfolded tasks {tasks}")
    res = GU.run_gpu(GU.to(inp, gpu), top_k=top_k)
    check_exact(wl, res[1], res[2], top_k, lens=[L])
    GU.check_gsa(inp, res, top_k=top_k)


@pytest.mark.parametrize("name", ["llama3.2-1b-32k-c8", "qwen2-7b-128k-c16", "multidoc-120k-c32"])
def test_full_workload_every_unit_exact(gpu, name):
    # every unit of the full-size workloads, two calls sharing one workspace:
    # the selection equals the top-k of the GPU's own routing keys (the
    # oracle comparison of sampled units lives in the parity tests)
    wl = gi.BY_NAME[name]
    inp = gi.make_inputs(wl, gi.seed_of(gi.WORKLOADS.index(wl)), device=gpu)
    for call in range(2):
        say(f"[select] full {name} call {call}")
        out, sel, sc = GU.run_gpu(inp)
        check_exact(wl, sel, sc, wl.top_k)
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seq_mode", ["full", "ragged"])
def test_two_block_unfolded_tasks(gpu, seq_mode):
    # 512 units with 6 unfolded 128-token tasks each exceed the launch's
    # 2048-task limit, so the unfolded tasks take 256 tokens (two blocks per
    # wavefront); ragged lengths leave tasks with one block, a partial second
    # block, or a partial first block only
    wl = gi.Workload("two-block", gi.BF16, 64, 8, 8, 64, 16, 300, 40, 16)
    lens = None
    if seq_mode == "ragged":
        gen = torch.Generator().manual_seed(611)
        lens = torch.randint(40 * 16, 300 * 16 + 15, (wl.batch,), generator=gen).tolist()
    inp = gi.make_inputs(wl, 610 + (seq_mode == "ragged"), seq_lens=lens)
    units = wl.batch * wl.num_kv_heads
    assert units * -(-(wl.top_k * wl.chunk_size + wl.chunk_size - 1) // 128) > 2048
    say(f"[select] two-block unfolded tasks ({seq_mode})")
    res = GU.run_gpu(GU.to(inp, gpu))
    check_exact(wl, res[1], res[2], wl.top_k, lens=lens)
    GU.check_gsa(inp, res, units=[(b, g) for b in range(0, wl.batch, 7) for g in range(wl.num_kv_heads)])
