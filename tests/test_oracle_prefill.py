"""Pins of the oracle's multi-query side (O8: T consecutive slots of the
interleaved sequence under the gist causal mask; "Forget, Then Recall" ja page
2.1 item 1, nl page Het Proces / Compressie), against what fixes it
independently of the oracle:

  brute force  numpy fp64: the mask written as a matrix over logical slots from
               its definition, and dense attention under it (ragged starts,
               queries crossing chunk boundaries and the raw tail).
  decode       a query in the raw tail sees every gist and the tail up to
               itself: the (separately pinned) decode oracle with top_k = 0 on
               the sequence that ends at that query.
  special      the first slot sees only itself (out = its V exactly); the first
               gist sees exactly the causal prefix of chunk 0.
  layout       page order does not change any result (bitwise).
  hand-worked  tests/golden/hand_worked_prefill.txt: exact fractions.
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

from long_context_sparse_gist_amd import inputs as gi
from tests import _util as U

import oracle

SMALL = gi.Workload("prefill-small", gi.BF16, 2, 6, 2, 64, 4, 40, 0, 4, plant="align",
                    plant_count=3)
SMALL_F32 = gi.Workload("prefill-small-f32", gi.F32, 1, 4, 1, 64, 8, 30, 0, 8)


def make_q(wl, T, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(wl.batch, T, wl.num_q_heads, wl.head_dim, generator=g).to(dtype)


def run_prefill(inp, q, q_start, lib=None):
    c = U.cfg_of(inp, top_k=0)
    return oracle.prefill(c, U.np_raw(q), U.np_raw(inp.k_cache), U.np_raw(inp.v_cache),
                          U.np_raw(inp.block_table), np.asarray(q_start, np.int32),
                          lib=lib or U.ORACLE_LIB)


def np_mask(s, nslots, C):
    """Keys of query slot s, from the definition: gist slots of earlier chunks,
    and the slots of its own chunk up to s."""
    j = np.arange(nslots)
    same = (j // (C + 1)) == (s // (C + 1))
    earlier_gist = ((j % (C + 1)) == C) & ((j // (C + 1)) < (s // (C + 1)))
    return (same & (j <= s)) | earlier_gist


def np_prefill(inp, q, q_start):
    wl = inp.wl
    C, G = wl.chunk_size, wl.group
    tau = U.tau_of(wl.head_dim)
    K, V = U.logical(inp, "k"), U.logical(inp, "v")
    qq = q.double().numpy()
    B, T, Hq, d = qq.shape
    out = np.zeros((B, T, Hq, d))
    for b in range(B):
        for t in range(T):
            m = np_mask(q_start[b] + t, K.shape[2], C)
            for h in range(Hq):
                out[b, t, h] = U.np_attend(qq[b, t, h], K[b, h // G][m], V[b, h // G][m], tau)
    return out


@pytest.mark.parametrize("wl", [SMALL, SMALL_F32], ids=lambda w: w.name)
@pytest.mark.parametrize("start", ["chunk", "mid", "tail"])
def test_prefill_matches_masked_dense(wl, start):
    inp = gi.make_inputs(wl, 51)
    C = wl.chunk_size
    T = 3 * (C + 1) + 2
    cap = wl.max_pages * wl.slots_per_page
    if start == "chunk":
        q_start = [0, 5 * (C + 1)][:wl.batch]
    elif start == "mid":
        q_start = [7 * (C + 1) + 1, 2][:wl.batch]
    else:  # the last queries reach the slots past the last full chunk
        q_start = [wl.num_chunks * (C + 1) + C - 1 - T] * wl.batch
    assert max(q_start) + T <= cap
    q = make_q(wl, T, 3, inp.q.dtype)
    out = run_prefill(inp, q, q_start)
    assert np.allclose(out, np_prefill(inp, q, q_start), rtol=1e-10, atol=1e-12)


def test_prefill_tail_query_is_decode_with_no_chunk_unfolded():
    wl = SMALL
    inp = gi.make_inputs(wl, 52)
    C = wl.chunk_size
    n = 23
    for c in range(C - 1):
        s = n * (C + 1) + c
        q = make_q(wl, 1, 10 + c, inp.q.dtype)
        out = run_prefill(inp, q, [s] * wl.batch)
        dec = dataclasses.replace(inp, q=q[:, 0].contiguous(),
                                  seq_lens=torch.full((wl.batch,), n * C + c + 1, dtype=torch.int32))
        d_out, _, _ = U.run_oracle(dec, top_k=0)
        assert np.allclose(out[:, 0], d_out, rtol=1e-12, atol=1e-12)


def test_prefill_first_slot_and_first_gist():
    wl = SMALL_F32
    inp = gi.make_inputs(wl, 53)
    C = wl.chunk_size
    q = make_q(wl, C + 1, 4, inp.q.dtype)
    out = run_prefill(inp, q, [0])
    V = U.logical(inp, "v")
    K = U.logical(inp, "k")
    assert np.array_equal(out[0, 0], np.repeat(V[0, 0, 0][None], wl.num_q_heads, 0))
    tau = U.tau_of(wl.head_dim)
    for h in range(wl.num_q_heads):
        ref = U.np_attend(q[0, C, h].double().numpy(), K[0, 0, :C + 1], V[0, 0, :C + 1], tau)
        assert np.allclose(out[0, C, h], ref, rtol=1e-12, atol=1e-12)


def test_prefill_page_order_invariant():
    wl = SMALL
    inp = gi.make_inputs(wl, 54, spare_pages=2)
    C = wl.chunk_size
    q = make_q(wl, 2 * (C + 1), 5, inp.q.dtype)
    starts = [3 * (C + 1) + 2, 11]
    base = run_prefill(inp, q, starts)
    perm = torch.randperm(inp.num_pages, generator=torch.Generator().manual_seed(2))
    inv = torch.argsort(perm)
    inp2 = dataclasses.replace(inp, k_cache=inp.k_cache[perm].contiguous(),
                               v_cache=inp.v_cache[perm].contiguous(),
                               block_table=inv[inp.block_table.long()].to(torch.int32))
    assert np.array_equal(base, run_prefill(inp2, q, starts))


def test_prefill_rejects_bad_starts():
    wl = SMALL
    inp = gi.make_inputs(wl, 55)
    q = make_q(wl, 4, 6, inp.q.dtype)
    cap = wl.max_pages * wl.slots_per_page
    for starts in ([-1, 0], [0, cap - 3]):
        with pytest.raises(ValueError):
            run_prefill(inp, q, starts)


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked_prefill.txt")
FILL_K, FILL_V = float(np.log(1000.0)), 999.0


def load_cases(path=GOLDEN):
    cases, cur = {}, None
    for raw in open(path):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "case":
            cur = {"name": tok[1], "slots": {}, "q": [], "expect_out": []}
        elif tok[0] == "end":
            cases[cur["name"]] = cur
        elif tok[0] == "cite":
            cur["cite"] = " ".join(tok[1:])
        elif tok[0] == "config":
            cur["cfg"] = {k: int(v) for k, v in (t.split("=") for t in tok[1:])}
        elif tok[0] == "queries":
            cur["first"], cur["count"] = int(tok[1]), int(tok[2])
        elif tok[0] == "q":
            cur["q"].append([float(x) for x in tok[1:]])
        elif tok[0] == "slot":
            cur["slots"][int(tok[1])] = [float(x) for x in tok[3:]]
        elif tok[0] == "expect_out":
            cur["expect_out"].append([float(x) for x in tok[1:]])
        else:
            raise ValueError(f"unknown fixture line: {line}")
    return cases


CASES = load_cases()


def golden_arrays(case, d):
    c = case["cfg"]
    spp = c["page_chunks"] * (c["chunk_size"] + 1)
    k = np.zeros((1, 1, spp, d), np.float32)
    v = np.zeros((1, 1, spp, d), np.float32)
    k[0, 0, :, 0], v[0, 0, :, 0], v[0, 0, :, 1] = FILL_K, FILL_V, FILL_V
    for s, (k0, k1, v0, v1) in case["slots"].items():
        k[0, 0, s, :2] = (k0, k1)
        v[0, 0, s, :2] = (v0, v1)
    q = np.zeros((1, case["count"], 1, d), np.float32)
    for t, qq in enumerate(case["q"]):
        q[0, t, 0, :2] = qq
    return q, k, v, np.zeros((1, 1), np.int32), np.array([case["first"]], np.int32)


def golden_cfg(case, d):
    c = case["cfg"]
    return dict(batch=1, num_q_heads=1, num_kv_heads=1, head_dim=d, top_k=0, sm_scale=1.0,
                dtype=0, flags=0, num_chunks=c["page_chunks"], chunk_size=c["chunk_size"],
                page_chunks=c["page_chunks"], num_pages=1, max_pages=1)


def test_prefill_fixture_is_complete():
    assert set(CASES) == {"prefill-c2"}
    for case in CASES.values():
        assert case["cite"] and len(case["expect_out"]) == case["count"] == len(case["q"])


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_hand_worked(name):
    case = CASES[name]
    q, k, v, bt, qs = golden_arrays(case, 2)
    out = oracle.prefill(golden_cfg(case, 2), q, k, v, bt, qs, lib=U.ORACLE_LIB)
    np.testing.assert_allclose(out[0, :, 0, :2], case["expect_out"], rtol=1e-6, atol=1e-6)
