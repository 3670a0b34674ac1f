"""gsa_decode_noalloc (the allocation-free variant of gsa_decode, on the
library's own device array) against gsa_decode, through the C ABI: two calls
in a row on one GPU, the second with a smaller input, and a multi-launch
(fp32) call; the selections and routing keys must be identical and the
outputs equal within the dtype's tolerance (the kernels are the same, so in
practice they are bit-identical)."""
import numpy as np
import pytest
import torch

import long_context_sparse_gist_amd as gsa
from long_context_sparse_gist_amd import inputs as gi
from tests import gpu_util as GU

pytestmark = pytest.mark.gpu


def _both(inp, flags=0):
    wl = inp.wl
    kw = dict(num_chunks=wl.num_chunks, chunk_size=wl.chunk_size, page_chunks=wl.page_chunks,
              top_k=wl.top_k, flags=flags)
    res = []
    for noalloc in (False, True):
        sel = torch.full((wl.batch, wl.num_kv_heads, wl.top_k), -7, dtype=torch.int32,
                         device=inp.q.device)
        sc = torch.full((wl.batch, wl.num_kv_heads, wl.num_chunks), 7.0, dtype=torch.float32,
                        device=inp.q.device)
        out = torch.full_like(inp.q, 5.0)
        fn = gsa.gsa_decode_noalloc if noalloc else gsa.gsa_decode
        fn(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens, out=out,
           sel_idx=sel, scores=sc, **kw)
        torch.cuda.synchronize()
        res.append((out.float().cpu().numpy(), sel.cpu().numpy(), sc.cpu().numpy()))
    return res


def _check(inp, flags=0):
    (o_ref, s_ref, k_ref), (o, s, k) = _both(inp, flags)
    assert np.array_equal(s, s_ref)
    assert np.array_equal(k, k_ref)
    GU.assert_close(o, o_ref, inp.wl.dtype, "noalloc vs gsa_decode")


def test_noalloc_two_calls_then_smaller(gpu):
    print("[noalloc] qwen2-7b-128k-c16, then a smaller ragged shape", flush=True)
    wl = gi.QWEN7B_128K
    inp = gi.make_inputs(wl, gi.seed_of(2), device=gpu)
    _check(inp)
    del inp
    small = gi.Workload("na-small", gi.BF16, 3, 8, 2, 64, 8, 300, 20, 16, plant="align",
                        plant_count=4)
    inp2 = GU.to(gi.make_inputs(small, 901, seq_lens=[2000, 17, 2399]), gpu)
    _check(inp2)


def test_noalloc_multi_launch_path(gpu):
    print("[noalloc] fp32 (multi-launch kernels)", flush=True)
    wl = gi.Workload("na-f32", gi.F32, 2, 6, 2, 64, 16, 200, 12, 16, plant="align",
                     plant_count=3)
    _check(GU.to(gi.make_inputs(wl, 902, seq_lens=[3000, 1234]), gpu))


def test_noalloc_rejects_oversized(gpu):
    wl = gi.Workload("na-big", gi.BF16, 64, 16, 16, 64, 4, 16384, 16, 16)
    p = gsa.make_params(torch.empty(64, 16, 64, dtype=torch.bfloat16), 16, 16)
    kv = gsa.GsaKV(None, None, None, None, wl.num_chunks, wl.chunk_size, wl.page_chunks, 1,
                   wl.max_pages)
    assert gsa.gsa_workspace_size(p, kv) > gsa.NOALLOC_WORKSPACE_BYTES
    q = torch.zeros(64, 16, 64, dtype=torch.bfloat16, device=gpu)
    dummy = torch.zeros(1, 16, 64, dtype=torch.bfloat16, device=gpu)
    bt = torch.zeros(64, wl.max_pages, dtype=torch.int32, device=gpu)
    with pytest.raises(gsa.GsaError) as e:
        gsa.gsa_decode_noalloc(q, dummy.view(1, 16, 1, 64).expand(1, 16, 1, 64).contiguous(),
                               dummy.view(1, 16, 1, 64).contiguous(), bt, None,
                               num_chunks=wl.num_chunks, chunk_size=wl.chunk_size,
                               page_chunks=wl.page_chunks, top_k=16, out=torch.empty_like(q))
    assert e.value.status == 5
