"""Pins of the oracle's hierarchy of any depth (O7: meta-gists built again
over meta-gists, selection coarse to fine; "Forget, Then Recall" ja page,
section 2.2; nl page, Hierarchische Uitbreiding), against what fixes it
independently of the oracle:

  reductions   no meta level is flat GSA, one level is two-level H-GSA: both
               bitwise equal to the oracle's own, separately pinned, paths.
  brute force  numpy fp64 selection at every level and masked dense attention
               over the set, two and three meta levels, full and ragged
               sequences (levels with entries past their last complete group).
  closed form  every entry kept at every level: dense attention over every
               level's entries and the whole interleaved sequence.
  hand-worked  tests/golden/hand_worked_levels.txt: exact fractions.
  caller sets  a caller's selection at any level replaces that level's top-k.
"""
import os

import numpy as np
import pytest

from long_context_sparse_gist_amd import inputs as gi
from tests import _util as U

import oracle

SMALL_L = gi.Workload("small-levels", gi.BF16, 2, 6, 2, 64, 4, 150, 5, 8,
                      plant="align", plant_count=3)
SMALL_L_F32 = gi.Workload("small-levels-f32", gi.F32, 1, 4, 2, 64, 2, 97, 4, 16,
                          plant="align", plant_count=2)


def run_levels(inp, levels, top_k=None, ext=None):
    """levels: [(k, v, fanout, top_k)] as tensors; runs the oracle (or the
    build a test swapped in)."""
    c = U.cfg_of(inp, top_k=top_k)
    lv = [(U.np_raw(k), U.np_raw(v), R, kk) for k, v, R, kk in levels]
    return oracle.mgsa_decode(c, U.np_raw(inp.q), U.np_raw(inp.k_cache), U.np_raw(inp.v_cache),
                              U.np_raw(inp.block_table), U.np_raw(inp.seq_lens), lv, ext=ext,
                              lib=U.ORACLE_LIB)


def with_levels(inp, fanouts, tops, seed):
    made = gi.make_levels(inp, fanouts, seed)
    return [(k, v, R, t) for (k, v), R, t in zip(made, fanouts, tops)]


def np_mgsa(inp, levels, k0, ext=None):
    """numpy fp64 brute force of the hierarchy.  Returns (out, sels) with
    sels[(b, g)][l] the kept ids of level l (0: chunks)."""
    wl = inp.wl
    C, G = wl.chunk_size, wl.group
    tau = U.tau_of(wl.head_dim)
    q = U.f64(inp.q)
    K, V = U.logical(inp, "k"), U.logical(inp, "v")
    Ks = [U.f64(k) for k, _, _, _ in levels]
    Vs = [U.f64(v) for _, v, _, _ in levels]
    Rs = [R for _, _, R, _ in levels]
    tops = [k0] + [t for _, _, _, t in levels]
    L = len(levels)
    n, tail = U.shapes(inp)
    out = np.zeros(q.shape)
    sels = {}
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            cnt = [int(n[b])]
            for R in Rs:
                cnt.append(cnt[-1] // R)
            qg = q[b, g * G:(g + 1) * G]

            def krows(l, ids):
                ids = np.asarray(ids, np.int64)
                return K[b, g][ids * (C + 1) + C] if l == 0 else Ks[l - 1][b, g][ids]

            def vrows(l, ids):
                ids = np.asarray(ids, np.int64)
                return V[b, g][ids * (C + 1) + C] if l == 0 else Vs[l - 1][b, g][ids]

            cand = np.arange(cnt[L])
            kept = [None] * (L + 1)
            for l in range(L, -1, -1):
                S = (tau * krows(l, cand) @ qg.T).sum(1).astype(np.float32) if len(cand) else \
                    np.zeros(0, np.float32)
                s = U.np_topk(S, tops[l], ids=cand) if len(cand) else np.zeros(0, np.int64)
                if ext is not None and ext[l] is not None:
                    s = np.array(sorted(int(x) for x in ext[l][b][g] if 0 <= x < cnt[l]), np.int64)
                kept[l] = s
                if l > 0:
                    R = Rs[l - 1]
                    cand = np.array([r * R + j for r in s for j in range(R)] +
                                    list(range(cnt[l] * R, cnt[l - 1])), np.int64)
            Kset, Vset = [], []
            for l in range(L, 0, -1):
                if l == L:
                    ids = list(range(cnt[L]))
                else:
                    past = cnt[l + 1] * Rs[l]
                    ids = sorted(set(int(x) for x in kept[l]) | set(range(past, cnt[l])))
                if ids:
                    Kset.append(krows(l, ids))
                    Vset.append(vrows(l, ids))
            m = U.gsa_mask(int(n[b]), int(tail[b]), C, kept[0], K.shape[2], all_gists=(L == 0))
            if L > 0:
                m[np.arange(cnt[1] * Rs[0], cnt[0]) * (C + 1) + C] = True
            Kset.append(K[b, g][m])
            Vset.append(V[b, g][m])
            Ka, Va = np.concatenate(Kset), np.concatenate(Vset)
            for j in range(G):
                out[b, g * G + j] = U.np_attend(q[b, g * G + j], Ka, Va, tau)
            sels[(b, g)] = kept
    return out, sels


def _ragged(wl, seed):
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(wl.chunk_size, wl.num_chunks * wl.chunk_size + wl.chunk_size - 1,
                                         size=wl.batch)]


def test_no_meta_level_is_flat_gsa():
    inp = gi.make_inputs(SMALL_L, 71, seq_lens=_ragged(SMALL_L, 1))
    out, sels, keys = run_levels(inp, [])
    f_out, f_sel, f_sc = U.run_oracle(inp)
    assert np.array_equal(out, f_out) and np.array_equal(sels[0], f_sel)
    assert np.array_equal(keys[0], f_sc)


def test_one_meta_level_is_two_level_hgsa():
    wl = SMALL_L.replace(plant="align_meta", gists_per_meta=4, top_k_meta=3)
    inp = gi.make_inputs(wl, 72, seq_lens=_ragged(wl, 2))
    lv = [(inp.k_meta, inp.v_meta, wl.gists_per_meta, wl.top_k_meta)]
    out, sels, keys = run_levels(inp, lv)
    h_out, h_s1, h_s2, h_ms, h_gs = U.run_oracle_h(inp)
    assert np.array_equal(out, h_out)
    assert np.array_equal(sels[1], h_s1) and np.array_equal(sels[0], h_s2)
    assert np.array_equal(keys[1], h_ms) and np.array_equal(keys[0], h_gs)


@pytest.mark.parametrize("fanouts,tops", [((4, 3), (5, 2)), ((3, 2, 2), (4, 3, 2)),
                                          ((2, 2, 2), (3, 2, 1))])
@pytest.mark.parametrize("lens", ["full", "ragged"])
def test_levels_match_brute_force(fanouts, tops, lens):
    wl = SMALL_L
    inp = gi.make_inputs(wl, 73 + len(fanouts), seq_lens=None if lens == "full" else _ragged(wl, 3))
    lv = with_levels(inp, fanouts, tops, 9)
    out, sels, keys = run_levels(inp, lv)
    ref, rsel = np_mgsa(inp, lv, wl.top_k)
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-12)
    for (b, g), kept in rsel.items():
        for l, s in enumerate(kept):
            got = sels[l][b, g]
            assert np.array_equal(got[got >= 0], s), (b, g, l)


SMALL_DEEP = gi.Workload("small-deep", gi.BF16, 2, 6, 2, 64, 4, 600, 5, 8,
                         plant="align", plant_count=3)


@pytest.mark.parametrize("wl", [SMALL_DEEP, SMALL_L], ids=["600-gists", "150-gists-empty-top"])
@pytest.mark.parametrize("lens", ["full", "ragged"])
def test_eight_levels_match_brute_force(wl, lens):
    """Eight meta levels of fanout 2 (the most the library's entry point
    takes) against the numpy brute force; above 150 gists the eighth level is
    empty, so every level-7 entry lies past its last complete group."""
    tops = (6, 5, 4, 3, 3, 2, 2, 1)
    inp = gi.make_inputs(wl, 81, seq_lens=None if lens == "full" else _ragged(wl, 5))
    lv = with_levels(inp, (2,) * 8, tops, 15)
    out, sels, _ = run_levels(inp, lv)
    ref, rsel = np_mgsa(inp, lv, wl.top_k)
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-12)
    for (b, g), kept in rsel.items():
        for l, s in enumerate(kept):
            got = sels[l][b, g]
            assert np.array_equal(got[got >= 0], s), (b, g, l)


def test_levels_f32_and_planted_ancestors():
    """fp32 storage; the planted chunks' ancestors are kept at every level and
    the planted chunks themselves selected."""
    wl = SMALL_L_F32
    inp = gi.make_inputs(wl, 77)
    lv = with_levels(inp, (4, 3), (3, 2), 11)
    out, sels, _ = run_levels(inp, lv)
    ref, _ = np_mgsa(inp, lv, wl.top_k)
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-12)
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            pl = inp.planted[b, g].tolist()
            assert set(pl) <= set(sels[0][b, g].tolist())
            assert {m // 4 for m in pl} <= set(sels[1][b, g].tolist())
            assert {m // 12 for m in pl} <= set(sels[2][b, g].tolist())


def test_everything_kept_is_dense_over_all_levels():
    wl = SMALL_L
    inp = gi.make_inputs(wl, 79, seq_lens=_ragged(wl, 4))
    fanouts = (3, 2, 2)
    sizes = gi.level_sizes(wl.num_chunks, fanouts)
    lv = with_levels(inp, fanouts, [s for s in sizes], 12)
    out, _, _ = run_levels(inp, lv, top_k=wl.num_chunks)
    q = U.f64(inp.q)
    K, V = U.logical(inp, "k"), U.logical(inp, "v")
    n, tail = U.shapes(inp)
    tau = U.tau_of(wl.head_dim)
    for b in range(wl.batch):
        cnt = [int(n[b])]
        for R in fanouts:
            cnt.append(cnt[-1] // R)
        Lseq = int(n[b]) * (wl.chunk_size + 1) + int(tail[b])
        for h in range(wl.num_q_heads):
            g = h // wl.group
            Ka = np.concatenate([U.f64(lv[l][0])[b, g, :cnt[l + 1]] for l in range(3)] + [K[b, g, :Lseq]])
            Va = np.concatenate([U.f64(lv[l][1])[b, g, :cnt[l + 1]] for l in range(3)] + [V[b, g, :Lseq]])
            assert np.allclose(out[b, h], U.np_attend(q[b, h], Ka, Va, tau), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("which", [0, 1, 2])
def test_caller_selection_at_a_level(which):
    """O6 for the hierarchy: a caller's set (lowest keys, -1 padded, an id
    past the level's entries) at level `which` replaces its top-k; the levels
    below follow it."""
    wl = SMALL_L
    inp = gi.make_inputs(wl, 81, seq_lens=_ragged(wl, 6))
    fanouts, tops = (3, 2), (4, 2)
    lv = with_levels(inp, fanouts, tops, 13)
    _, own, keys = run_levels(inp, lv)
    n, _ = U.shapes(inp)
    k = [wl.top_k, *tops][which]
    ext = [None, None, None]
    e = np.full((wl.batch, wl.num_kv_heads, k), -1, np.int32)
    for b in range(wl.batch):
        cnt = [int(n[b])]
        for R in fanouts:
            cnt.append(cnt[-1] // R)
        for g in range(wl.num_kv_heads):
            low = np.argsort(keys[which][b, g, :cnt[which]], kind="stable")[:max(0, k - 2)]
            e[b, g, :len(low)] = low
            e[b, g, k - 1] = cnt[which] + 1
    ext[which] = e
    out, sels, _ = run_levels(inp, lv, ext=ext)
    ref, rsel = np_mgsa(inp, lv, wl.top_k, ext=ext)
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-12)
    moved = 0
    for (b, g), kept in rsel.items():
        for l, s in enumerate(kept):
            got = sels[l][b, g]
            assert np.array_equal(got[got >= 0], s)
        moved += not np.array_equal(sels[which][b, g], own[which][b, g])
    assert moved == wl.batch * wl.num_kv_heads


# ---------------- hand-worked ----------------

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked_levels.txt")
FILL_K, FILL_V = float(np.log(1000.0)), 999.0


def load_cases(path=GOLDEN):
    cases, cur = {}, None
    for raw in open(path):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "case":
            cur = {"name": tok[1], "slots": {}, "levels": {}}
        elif tok[0] == "end":
            cases[cur["name"]] = cur
        elif tok[0] == "cite":
            cur["cite"] = " ".join(tok[1:])
        elif tok[0] == "config":
            cur["cfg"] = {k: int(v) for k, v in (t.split("=") for t in tok[1:])}
        elif tok[0] == "q":
            cur["q"] = [float(x) for x in tok[1:]]
        elif tok[0] == "slot":
            cur["slots"][int(tok[1])] = [float(x) for x in tok[3:]]
        elif tok[0] == "level":
            cur["levels"].setdefault(int(tok[1]), {})[int(tok[2])] = [float(x) for x in tok[3:]]
        elif tok[0].startswith("expect_sel"):
            cur[tok[0]] = [int(x) for x in tok[1:]]
        elif tok[0] == "expect_out":
            cur["expect_out"] = [float(x) for x in tok[1:]]
        else:
            raise ValueError(f"unknown fixture line: {line}")
    return cases


CASES = load_cases()


def golden_arrays(case, d, dtype=np.float32):
    """(q, k, v, bt, sl, levels[(k, v, fanout, top_k)]) as numpy, head_dim d."""
    c = case["cfg"]
    spp = c["page_chunks"] * (c["chunk_size"] + 1)
    k = np.zeros((1, 1, spp, d), np.float32)
    v = np.zeros((1, 1, spp, d), np.float32)
    k[0, 0, :, 0], v[0, 0, :, 0], v[0, 0, :, 1] = FILL_K, FILL_V, FILL_V
    for s, (k0, k1, v0, v1) in case["slots"].items():
        k[0, 0, s, :2] = (k0, k1)
        v[0, 0, s, :2] = (v0, v1)
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, :2] = case["q"]
    levels = []
    for l in range(1, c["levels"] + 1):
        mx = c[f"max{l}"]
        km = np.zeros((1, 1, mx, d), np.float32)
        vm = np.zeros((1, 1, mx, d), np.float32)
        km[0, 0, :, 0], vm[0, 0, :, 0], vm[0, 0, :, 1] = FILL_K, FILL_V, FILL_V
        for r, (k0, k1, v0, v1) in case["levels"][l].items():
            km[0, 0, r, :2] = (k0, k1)
            vm[0, 0, r, :2] = (v0, v1)
        levels.append((km, vm, c[f"fanout{l}"], c[f"top_k{l}"]))
    return q, k, v, np.zeros((1, 1), np.int32), np.array([c["seq_len"]], np.int32), levels


def golden_cfg(case, d):
    c = case["cfg"]
    return dict(batch=1, num_q_heads=1, num_kv_heads=1, head_dim=d, top_k=c["top_k"],
                sm_scale=1.0, dtype=0, flags=0, num_chunks=c["num_chunks"],
                chunk_size=c["chunk_size"], page_chunks=c["page_chunks"], num_pages=1, max_pages=1)


def test_levels_fixture_is_complete():
    assert set(CASES) == {"mlevel-k1", "mlevel-k2"}
    for case in CASES.values():
        assert case["cite"] and case["expect_out"] and case["expect_sel"]
        assert case["expect_sel_l1"] and case["expect_sel_l2"]


@pytest.mark.parametrize("name", sorted(CASES))
def test_levels_hand_worked(name):
    case = CASES[name]
    q, k, v, bt, sl, levels = golden_arrays(case, 2)
    out, sels, _ = oracle.mgsa_decode(golden_cfg(case, 2), q, k, v, bt, sl, levels, lib=U.ORACLE_LIB)
    for l, key in enumerate(["expect_sel", "expect_sel_l1", "expect_sel_l2"]):
        want = case[key]
        assert sels[l][0, 0].tolist()[:len(want)] == want
        assert all(x == -1 for x in sels[l][0, 0].tolist()[len(want):])
    np.testing.assert_allclose(out[0, 0, :2], case["expect_out"], rtol=1e-6, atol=1e-6)
