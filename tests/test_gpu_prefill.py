"""Parity of gsa_prefill (the multi-query side under the gist causal mask,
through the C ABI) with the oracle: every output of small and medium shapes
(query runs crossing chunk boundaries, starting at a chunk, mid-chunk and in
the raw tail, one to hundreds of queries), sampled query rows of a chunked-
prefill step at the end of a 128K-token context, and the hand-worked example.
bf16 tolerance: 2e-2 abs / 1e-2 rel."""
import numpy as np
import pytest
import torch

import long_context_sparse_gist_amd as gsa
from long_context_sparse_gist_amd import inputs as gi
from tests import _util as U
from tests import gpu_util as GU
from tests import test_oracle_prefill as PP

import oracle

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


SHAPES = {
    "pf-b2-g4-d64-c8": gi.Workload("pf-b2-g4-d64-c8", gi.BF16, 2, 8, 2, 64, 8, 90, 0, 8),
    "pf-b2-g7-d128-c16": gi.Workload("pf-b2-g7-d128-c16", gi.BF16, 2, 14, 2, 128, 16, 80, 0, 16),
    "pf-b1-g16-d128-c4": gi.Workload("pf-b1-g16-d128-c4", gi.BF16, 1, 16, 1, 128, 4, 120, 0, 8),
    "pf-b3-g1-d64-c32": gi.Workload("pf-b3-g1-d64-c32", gi.BF16, 3, 3, 3, 64, 32, 40, 0, 4),
}


def queries(wl, T, seed, device):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(wl.batch, T, wl.num_q_heads, wl.head_dim, generator=g).to(torch.bfloat16).to(device)


def starts_for(wl, T, kind, seed):
    C = wl.chunk_size
    cap = wl.max_pages * wl.slots_per_page
    rng = np.random.default_rng(seed)
    if kind == "chunk":
        return [int(rng.integers(0, (cap - T) // (C + 1) + 1)) * (C + 1) for _ in range(wl.batch)]
    if kind == "mid":
        return [int(rng.integers(0, cap - T + 1)) for _ in range(wl.batch)]
    return [cap - T] * wl.batch  # the last T slots: the raw tail after the last full chunk included


def run(inp, q, starts):
    wl = inp.wl
    qs = torch.tensor(starts, dtype=torch.int32, device=q.device)
    out = gsa.gsa_prefill(q, inp.k_cache, inp.v_cache, inp.block_table, qs, chunk_size=wl.chunk_size,
                          page_chunks=wl.page_chunks)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


@pytest.mark.parametrize("name", sorted(SHAPES))
@pytest.mark.parametrize("T", [1, 3, 37, 300])
@pytest.mark.parametrize("kind", ["chunk", "mid", "end"])
def test_prefill_every_output(gpu, name, T, kind):
    wl = SHAPES[name]
    say(f"[prefill] {name} T={T} {kind}")
    inp = gi.make_inputs(wl, 1300 + T)
    q = queries(wl, T, T + 7, gpu)
    starts = starts_for(wl, T, kind, T)
    got = run(GU.to(inp, gpu), q, starts)
    ref = PP.run_prefill(inp, q.cpu(), starts)
    GU.assert_close(got, ref, wl.dtype, f"{name} T={T} {kind}")


LONG_BT = gi.Workload("pf-long-bt", gi.BF16, 1, 2, 1, 64, 4, 8000, 0, 1)


@pytest.mark.parametrize("kind", ["mid", "end"])
def test_prefill_block_table_in_memory(gpu, kind):
    """A block-table row longer than the kernel keeps in LDS (8000 one-chunk
    pages): the row is read from memory."""
    wl = LONG_BT
    say(f"[prefill] {wl.name} {kind}")
    inp = gi.make_inputs(wl, 1500)
    q = queries(wl, 37, 11, gpu)
    starts = starts_for(wl, 37, kind, 5)
    got = run(GU.to(inp, gpu), q, starts)
    ref = PP.run_prefill(inp, q.cpu(), starts)
    GU.assert_close(got, ref, wl.dtype, f"{wl.name} {kind}")


def test_prefill_repeat_is_bitwise(gpu):
    wl = SHAPES["pf-b2-g7-d128-c16"]
    inp = GU.to(gi.make_inputs(wl, 1401), gpu)
    q = queries(wl, 200, 5, gpu)
    starts = starts_for(wl, 200, "mid", 3)
    a = run(inp, q, starts)
    for _ in range(3):
        assert np.array_equal(a, run(inp, q, starts))


PREFILL_128K = gi.Workload("prefill-qwen2-7b-128k", gi.BF16, 8, 28, 4, 128, 16, 8192, 0, 16,
                           plant="align", plant_count=16)


@pytest.mark.timeout(300)
def test_prefill_chunk_step_at_128k_sampled_rows(gpu):
    """A chunked-prefill step of 2040 slots (120 chunks with their gists) at the
    end of a 128K-token context, qwen2-7b shape: 96 sampled (sequence, query)
    rows, all heads, against the oracle run on those queries one by one."""
    wl = PREFILL_128K
    say(f"[prefill] {wl.name} T=2040, sampled rows")
    inp = gi.make_inputs_large(wl, 1500, gpu)
    T = 2040
    cap = wl.num_chunks * (wl.chunk_size + 1)
    starts = [cap - T] * wl.batch
    q = queries(wl, T, 9, gpu)
    got = run(inp, q, starts)
    cpu = GU.to(inp, "cpu")
    rng = np.random.default_rng(4)
    picks = [(int(rng.integers(wl.batch)), int(t)) for t in rng.choice(T, 96, replace=False)]
    picks += [(0, 0), (wl.batch - 1, T - 1), (1, 16), (2, 17)]  # chunk edges, the last slot
    cfg = U.cfg_of(cpu, top_k=0)
    kc, vc, bt = U.np_raw(cpu.k_cache), U.np_raw(cpu.v_cache), U.np_raw(cpu.block_table)
    qh = q.cpu()
    for b, t in picks:
        c1 = dict(cfg, batch=1)
        ref = oracle.prefill(c1, U.np_raw(qh[b:b + 1, t:t + 1].contiguous()), kc, vc,
                             np.ascontiguousarray(bt[b:b + 1]), np.array([starts[b] + t], np.int32))
        GU.assert_close(got[b, t], ref[0, 0], wl.dtype, f"row {(b, t)}")
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", sorted(PP.CASES))
def test_prefill_hand_worked_bf16(gpu, name):
    """The hand-worked example in bf16 (head_dim 64): within 2 % of the exact
    fractions (bf16 rounding of the logarithms and of the output) and within
    the bf16 tolerance of the oracle on the same rounded inputs; a read of any
    slot the mask excludes (V = 999) would move it far past either."""
    case = PP.CASES[name]
    q, k, v, bt, qs = PP.golden_arrays(case, 64)
    t = lambda x: torch.from_numpy(x).to(gpu)  # noqa: E731
    qg, kg, vg = (t(x).to(torch.bfloat16) for x in (q, k, v))
    out = gsa.gsa_prefill(qg, kg, vg, t(bt), t(qs), chunk_size=case["cfg"]["chunk_size"],
                          page_chunks=case["cfg"]["page_chunks"], sm_scale=1.0)
    torch.cuda.synchronize()
    o = out[0, :, 0].float().cpu().numpy()
    np.testing.assert_allclose(o[:, :2], case["expect_out"], rtol=2e-2, atol=2e-2)
    bf = lambda x: x.cpu().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    ref = oracle.prefill(dict(PP.golden_cfg(case, 64), dtype=1), bf(qg), bf(kg), bf(vg), bt, qs)
    np.testing.assert_allclose(o, ref[0, :, 0], rtol=1e-2, atol=2e-2)
    assert np.all(o[:, 2:] == 0.0)
