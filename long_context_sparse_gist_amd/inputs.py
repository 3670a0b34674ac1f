"""Seeded synthetic inputs for GSA / H-GSA decode.

This module only draws random numbers and lays them out in memory. It holds
none of the method's arithmetic (no scoring, selection or attention), so both
the HIP path and the CPU oracle can be fed from it.

Workloads follow the five decode shapes of the gist sparse attention pages
(chunk size 16, 8x-32x compression; "Forget, Then Recall", technical summary,
sections on method and results) plus the Llama-3.2-1B / Qwen2-7B model shapes
the summaries evaluate on.  All values are N(0, 1); planted chunks carry gist
keys aligned with the query so that a known set of chunks must be routed to.

KV layout (the boundary's paged interleaved layout):
    k_cache, v_cache : [num_pages][num_kv_heads][page_chunks*(C+1)][head_dim]
    logical slot of raw token c of chunk m : m*(C+1) + c     (c < C)
    logical slot of the gist of chunk m    : m*(C+1) + C
    logical page p of sequence b lives in physical page block_table[b][p]
Meta-gists (H-GSA): k_meta, v_meta : [batch][num_kv_heads][max_meta][head_dim],
meta-gist r summarising gists [r*R, r*R + R).

Draw order for one seed (torch.Generator on the target device):
    q; physical page permutation; planted positions; then per batch entry b:
    K[b] (fp32), its planting noise; then per b: V[b]; then per b: meta K[b],
    its planting noise; then per b: meta V[b].
Values are drawn in fp32 and rounded to the storage dtype (round to nearest
even for bf16).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

F32 = 0
BF16 = 1

_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one decode call."""

    name: str
    dtype: int            # F32 or BF16 for q, caches and output
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    chunk_size: int       # C raw tokens per gist
    num_chunks: int       # gists per sequence (capacity and default length)
    top_k: int            # chunks unfolded (k2 for H-GSA)
    page_chunks: int      # chunks per physical page
    plant: str = "none"   # none | align | doc_bias | align_meta
    plant_count: int = 0  # planted chunks per (batch, kv-head)
    n_docs: int = 0       # doc_bias: documents the context is split into
    gists_per_meta: int = 0   # R (H-GSA only)
    top_k_meta: int = 0       # k1 (H-GSA only)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def hgsa(self) -> bool:
        return self.gists_per_meta > 0

    @property
    def num_meta(self) -> int:
        return self.num_chunks // self.gists_per_meta if self.hgsa else 0

    @property
    def raw_tokens(self) -> int:
        return self.num_chunks * self.chunk_size

    @property
    def slots_per_page(self) -> int:
        return self.page_chunks * (self.chunk_size + 1)

    @property
    def max_pages(self) -> int:
        # one spare slot range so that a raw tail after the last full chunk fits
        return -(-(self.num_chunks * (self.chunk_size + 1) + self.chunk_size - 1)
                 // self.slots_per_page)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five decode workloads.  Page sizes hold about 256 logical slots.
TINY_F32 = Workload("tiny-f32-4k", F32, 1, 1, 1, 64, 16, 256, 8, 16,
                    plant="align", plant_count=4)
LLAMA1B_32K = Workload("llama3.2-1b-32k-c8", BF16, 16, 32, 8, 64, 8, 4096, 64, 32,
                       plant="align", plant_count=8)
QWEN7B_128K = Workload("qwen2-7b-128k-c16", BF16, 8, 28, 4, 128, 16, 8192, 128, 16,
                       plant="align", plant_count=16)
MULTIDOC_120K = Workload("multidoc-120k-c32", BF16, 32, 32, 8, 128, 32, 3840, 128, 8,
                         plant="doc_bias", n_docs=20)
HGSA_1M = Workload("hgsa-1m-c16-r16", BF16, 4, 32, 8, 128, 16, 65536, 64, 16,
                   plant="align_meta", plant_count=16, gists_per_meta=16, top_k_meta=32)

WORKLOADS = [TINY_F32, LLAMA1B_32K, QWEN7B_128K, MULTIDOC_120K, HGSA_1M]
BY_NAME = {w.name: w for w in WORKLOADS}


@dataclasses.dataclass(frozen=True)
class Hierarchy:
    """A decode shape with meta-gist levels above the gists: fanouts and kept
    entries per level, level 1 first (the gist level keeps wl.top_k)."""

    wl: Workload
    fanouts: tuple
    tops: tuple

    @property
    def name(self) -> str:
        return self.wl.name


# The 1M-token H-GSA shape with a third level: 4096 level-1 entries under 256
# level-2 entries; 16 kept at the top, 32 below, 64 chunks unfolded.
MGSA_1M = Hierarchy(Workload("mgsa-1m-c16-r16x16", BF16, 4, 32, 8, 128, 16, 65536, 64, 16,
                             plant="align", plant_count=16), (16, 16), (32, 16))
HIERARCHIES = [MGSA_1M]
HIER_BY_NAME = {h.name: h for h in HIERARCHIES}


@dataclasses.dataclass(frozen=True)
class PrefillStep:
    """A multi-query step: the last `queries` slots of full-length sequences
    of `wl` attend under the gist causal mask."""

    wl: Workload
    queries: int

    @property
    def name(self) -> str:
        return f"{self.wl.name}-t{self.queries}"


# A chunked-prefill step of 120 chunks (1920 raw tokens and their 120 gists) at
# the end of a 128K-token context, Qwen2-7B shape.
PREFILL_128K = PrefillStep(Workload("prefill-qwen2-7b-128k", BF16, 8, 28, 4, 128, 16, 8192, 0, 16,
                                    plant="align", plant_count=16), 2040)
PREFILLS = [PREFILL_128K]
PREFILL_BY_NAME = {p.name: p for p in PREFILLS}


def seed_of(index: int) -> int:
    """Seed of workload `index` in WORKLOADS."""
    return 1000 + index


@dataclasses.dataclass
class GsaInputs:
    wl: Workload
    q: torch.Tensor            # [B][Hq][d] dtype
    k_cache: torch.Tensor      # [num_pages][Hkv][P*(C+1)][d] dtype
    v_cache: torch.Tensor
    block_table: torch.Tensor  # [B][max_pages] int32
    seq_lens: torch.Tensor     # [B] int32, raw tokens per sequence
    planted: torch.Tensor      # [B][Hkv][plant_count] int64 chunk ids (or doc id)
    k_meta: Optional[torch.Tensor] = None   # [B][Hkv][num_meta][d]
    v_meta: Optional[torch.Tensor] = None

    @property
    def num_pages(self) -> int:
        return self.k_cache.shape[0]


def _unit(v: torch.Tensor) -> torch.Tensor:
    return v / v.norm(dim=-1, keepdim=True)


def group_direction(q32: torch.Tensor, num_kv_heads: int) -> torch.Tensor:
    """Unit vector of the summed query of each GQA group: [B][Hkv][d] fp32."""
    B, Hq, d = q32.shape
    return _unit(q32.view(B, num_kv_heads, Hq // num_kv_heads, d).sum(2))


def make_inputs(wl: Workload, seed: int, device="cpu",
                seq_lens: Optional[list] = None,
                shuffle_pages: bool = True,
                spare_pages: int = 0) -> GsaInputs:
    """Draw one batch of `wl` with generator seed `seed` on `device`.

    seq_lens: optional per-sequence raw token counts (each at most
    num_chunks*C + C-1); default num_chunks*C for every sequence.
    spare_pages: physical pages that no sequence maps (left N(0,1) garbage
    that must never be read).
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    B, Hq, Hkv, d, C = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.chunk_size
    G = wl.group
    tdt = _TORCH_DTYPE[wl.dtype]
    spp = wl.slots_per_page
    max_pages = wl.max_pages
    num_pages = B * max_pages + spare_pages

    q32 = torch.randn(B, Hq, d, generator=g, device=dev, dtype=torch.float32)
    q = q32.to(tdt)
    qdir = group_direction(q.float(), Hkv)                     # [B][Hkv][d]

    perm = (torch.randperm(num_pages, generator=g, device=dev) if shuffle_pages
            else torch.arange(num_pages, device=dev))
    block_table = perm[: B * max_pages].view(B, max_pages).to(torch.int32)

    M = wl.num_chunks
    if wl.plant in ("align", "align_meta"):
        if wl.plant == "align":
            planted = torch.stack([torch.randperm(M, generator=g, device=dev)[: wl.plant_count]
                                   for _ in range(B * Hkv)]).view(B, Hkv, -1)
        else:
            R = wl.gists_per_meta
            groups = torch.stack([torch.randperm(M // R, generator=g, device=dev)[: wl.plant_count]
                                  for _ in range(B * Hkv)]).view(B, Hkv, -1)
            inner = torch.randint(0, R, groups.shape, generator=g, device=dev)
            planted = groups * R + inner
    elif wl.plant == "doc_bias":
        planted = torch.randint(0, wl.n_docs, (B, Hkv, 1), generator=g, device=dev)
    else:
        planted = torch.zeros(B, Hkv, 0, dtype=torch.int64, device=dev)

    k_cache = torch.empty(num_pages, Hkv, spp, d, dtype=tdt, device=dev)
    v_cache = torch.empty_like(k_cache)
    if spare_pages:
        k_cache.normal_(generator=g)
        v_cache.normal_(generator=g)
    slots = max_pages * spp
    gist_slot = lambda m: m * (C + 1) + C  # noqa: E731

    for which, cache in ((0, k_cache), (1, v_cache)):
        for b in range(B):
            x = torch.randn(Hkv, slots, d, generator=g, device=dev, dtype=torch.float32)
            if which == 0 and wl.plant in ("align", "align_meta") and wl.plant_count:
                for h in range(Hkv):
                    ms = planted[b, h]
                    noise = 0.1 * torch.randn(ms.numel(), d, generator=g, device=dev)
                    x[h, gist_slot(ms)] = 2.0 * math.sqrt(d) * qdir[b, h] + noise
            if which == 0 and wl.plant == "doc_bias":
                per_doc = M // wl.n_docs
                for h in range(Hkv):
                    doc = int(planted[b, h, 0])
                    ms = torch.arange(doc * per_doc, (doc + 1) * per_doc, device=dev)
                    x[h, gist_slot(ms)] += 1.5 * qdir[b, h]
            # logical pages -> physical pages of this sequence
            xp = x.view(Hkv, max_pages, spp, d).transpose(0, 1).to(tdt)
            cache.index_copy_(0, block_table[b].long(), xp)

    k_meta = v_meta = None
    if wl.hgsa:
        Mm = wl.num_meta
        k_meta = torch.empty(B, Hkv, Mm, d, dtype=tdt, device=dev)
        v_meta = torch.empty_like(k_meta)
        for b in range(B):
            x = torch.randn(Hkv, Mm, d, generator=g, device=dev, dtype=torch.float32)
            if wl.plant == "align_meta":
                for h in range(Hkv):
                    rs = planted[b, h] // wl.gists_per_meta
                    noise = 0.1 * torch.randn(rs.numel(), d, generator=g, device=dev)
                    x[h, rs] = 2.0 * math.sqrt(d) * qdir[b, h] + noise
            k_meta[b] = x.to(tdt)
        for b in range(B):
            v_meta[b] = torch.randn(Hkv, Mm, d, generator=g, device=dev,
                                    dtype=torch.float32).to(tdt)

    if seq_lens is None:
        seq_lens = [M * C] * B
    assert len(seq_lens) == B
    for L in seq_lens:
        assert 0 <= L <= M * C + C - 1, L
    sl = torch.tensor(seq_lens, dtype=torch.int32, device=dev)
    return GsaInputs(wl, q, k_cache, v_cache, block_table, sl, planted, k_meta, v_meta)


def share_pages(inp: GsaInputs, src_b: int, dst_b: int) -> GsaInputs:
    """Make sequence dst_b map the same physical pages as src_b (same prefix
    reused across requests), returning new inputs that alias the caches."""
    bt = inp.block_table.clone()
    bt[dst_b] = bt[src_b]
    return dataclasses.replace(inp, block_table=bt)


def level_sizes(num_chunks: int, fanouts) -> list:
    """Entries of each meta-gist level above `num_chunks` gists (complete
    groups only): level l has floor(entries of level l-1 / fanouts[l-1])."""
    out, n = [], num_chunks
    for R in fanouts:
        n //= R
        out.append(n)
    return out


def make_levels(inp: GsaInputs, fanouts, seed: int, plant: bool = True) -> list:
    """Meta-gist levels for a hierarchy above the gists of `inp`: a list of
    (k, v) pairs, level 1 first, each [B][Hkv][entries][d] in the inputs'
    dtype, N(0, 1) drawn on the inputs' device with generator seed `seed`
    (per level: K, then its planting noise, then V).  With `plant`, the
    ancestors of every planted chunk at every level get keys aligned with the
    group's summed query, as the planted gists have (2*sqrt(d)*q_dir + N(0, 0.1))."""
    wl = inp.wl
    dev = inp.q.device
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    B, Hkv, d = wl.batch, wl.num_kv_heads, wl.head_dim
    tdt = _TORCH_DTYPE[wl.dtype]
    qdir = group_direction(inp.q.float(), Hkv)
    chunks = inp.planted if (plant and wl.plant in ("align", "align_meta")) else None
    levels, span = [], 1
    for R, n in zip(fanouts, level_sizes(wl.num_chunks, fanouts)):
        span *= R
        x = torch.randn(B, Hkv, max(n, 1), d, generator=g, device=dev, dtype=torch.float32)
        if chunks is not None and chunks.numel() and n > 0:
            anc = torch.div(chunks, span, rounding_mode="floor")          # [B][Hkv][P]
            noise = 0.1 * torch.randn(*anc.shape, d, generator=g, device=dev)
            val = 2.0 * math.sqrt(d) * qdir.unsqueeze(2) + noise
            ok = anc < n
            bi = torch.arange(B, device=dev).view(B, 1, 1).expand_as(anc)[ok]
            hi = torch.arange(Hkv, device=dev).view(1, Hkv, 1).expand_as(anc)[ok]
            x[bi, hi, anc[ok]] = val[ok]
        v = torch.randn(B, Hkv, max(n, 1), d, generator=g, device=dev, dtype=torch.float32)
        levels.append((x.to(tdt), v.to(tdt)))
    return levels


def make_inputs_large(wl: Workload, seed: int, device) -> GsaInputs:
    """Inputs for long full-length contexts: the layout of make_inputs, with the
    bf16 caches drawn N(0, 1) in place (no fp32 copy of a whole sequence) from
    a generator seeded with `seed` (caches, then q, then planted positions and
    their noise), pages shuffled, and the planted chunks' gist keys aligned
    with the group's summed query as in make_inputs."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    B, Hq, Hkv, d, C = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.chunk_size
    tdt = _TORCH_DTYPE[wl.dtype]
    spp, max_pages = wl.slots_per_page, wl.max_pages
    num_pages = B * max_pages
    k_cache = torch.empty(num_pages, Hkv, spp, d, dtype=tdt, device=dev)
    v_cache = torch.empty_like(k_cache)
    for cache in (k_cache, v_cache):
        for p0 in range(0, num_pages, 4096):
            cache[p0:p0 + 4096].normal_(generator=g)
    q = torch.randn(B, Hq, d, generator=g, device=dev, dtype=torch.float32).to(tdt)
    qdir = group_direction(q.float(), Hkv)
    block_table = torch.randperm(num_pages, generator=g, device=dev).view(B, max_pages).to(torch.int32)
    M = wl.num_chunks
    P = wl.plant_count if wl.plant == "align" else 0
    planted = torch.stack([torch.randperm(M, generator=g, device=dev)[:P]
                           for _ in range(B * Hkv)]).view(B, Hkv, -1)
    if P:
        slots = planted * (C + 1) + C                                     # [B][Hkv][P]
        bi = torch.arange(B, device=dev).view(B, 1, 1).expand_as(slots)
        hi = torch.arange(Hkv, device=dev).view(1, Hkv, 1).expand_as(slots)
        page = block_table.long()[bi, slots // spp]
        noise = 0.1 * torch.randn(B, Hkv, P, d, generator=g, device=dev)
        k_cache[page, hi, slots % spp] = (2.0 * math.sqrt(d) * qdir.unsqueeze(2) + noise).to(tdt)
    sl = torch.full((B,), M * C, dtype=torch.int32, device=dev)
    return GsaInputs(wl, q, k_cache, v_cache, block_table, sl, planted)
