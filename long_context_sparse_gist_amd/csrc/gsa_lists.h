// Token lists walked by the attention kernels.
//
// Every kernel works on a list of cache rows of one (batch, kv-head) unit:
//   kListGists    gist m (m < n) at logical slot m*(C+1)+C        -> keys (+ attention)
//   kListMeta     meta-gist r (r < nm) of the meta arrays          -> keys + attention
//   kListCand     candidate gists of the kept meta-groups, then the
//                 gists after the last complete group              -> keys only
//   kListUnfolded raw tokens of the selected chunks, then the raw
//                 tail after the last gist, then the gist entries
//                 the set needs beyond the all-gists list          -> attention only
// The gist entries of the unfolded list are: none (flat GSA, all gists
// attended through kListGists); the selected gists (flat GSA, selected-gists
// set); the selected gists of complete meta-groups followed by every gist
// past the last complete group (H-GSA).
#pragma once

#include "gsa_internal.h"

namespace gsa {

struct ListCtx {
    int b, g, u;
    int n, tail;   // chunks with a gist, raw tokens after the last gist
    int nm;        // complete meta-groups (H-GSA)
    int ns;        // selected chunks (flat) / selected gists (H-GSA)
    int ns1;       // kept meta-groups (H-GSA)
    int e1;        // H-GSA: selected gists inside complete meta-groups
    int len;       // list length
};

// Length of each list.  `e1` must already be known for H-GSA unfolded lists.
__device__ inline int list_len(const Args& a, int kind, const ListCtx& c, bool hier) {
    switch (kind) {
        case kListGists: return c.n;
        case kListMeta: return c.nm;
        case kListCand: return c.ns1 * a.R + (c.n - c.nm * a.R);
        default: {
            int base = c.ns * a.C + c.tail;
            if (hier) return base + c.e1 + (c.n - c.nm * a.R);
            return base + ((a.flags & kFlagSelectedGists) ? c.ns : 0);
        }
    }
}

// Block-uniform context.  Must be called by every thread of the block (it may
// synchronise to count selected gists).
__device__ inline void make_ctx(const Args& a, int kind, int u, bool hier, ListCtx& c) {
    c.u = u;
    c.b = u / a.Hkv;
    c.g = u - c.b * a.Hkv;
    seq_shape(a, c.b, c.n, c.tail);
    c.nm = hier ? c.n / a.R : 0;
    c.ns1 = hier ? min(a.top_k_meta, c.nm) : 0;
    if (hier) {
        int nc = c.ns1 * a.R + (c.n - c.nm * a.R);
        c.ns = min(a.top_k, nc);
    } else {
        c.ns = min(a.top_k, c.n);
        if (a.nsel) c.ns = min(c.ns, a.nsel[u]);  // top-p: the unit's own count
    }
    c.e1 = 0;
    if (hier && kind == kListUnfolded) {
        int cnt = 0;
        const int32_t* sel = a.sel + (size_t)u * a.top_k;
        for (int i = threadIdx.x; i < c.ns; i += blockDim.x) cnt += (sel[i] < c.nm * a.R);
        __shared__ int s_cnt;
        if (threadIdx.x == 0) s_cnt = 0;
        __syncthreads();
        if (cnt) atomicAdd(&s_cnt, cnt);
        __syncthreads();
        c.e1 = s_cnt;
        __syncthreads();
    }
    c.len = list_len(a, kind, c, hier);
}

// Gist id of candidate position p (H-GSA).
__device__ inline int cand_gist(const Args& a, const ListCtx& c, int p) {
    int head = c.ns1 * a.R;
    if (p < head) {
        int r = a.sel_meta[(size_t)c.u * a.top_k_meta + p / a.R];
        return r * a.R + (p - (p / a.R) * a.R);
    }
    return c.nm * a.R + (p - head);
}

// Selection entry i of unit u, clamped into [0, n).  `coherent`: read with a
// device-scope load (written by another workgroup of the same kernel).
__device__ inline int sel_at(const Args& a, const ListCtx& c, int i, bool coherent) {
    const int32_t* p = a.sel + (size_t)c.u * a.top_k + i;
    int v = coherent ? __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT)
                     : *p;
    return min(max(v, 0), max(c.n - 1, 0));
}

// Source rows of list position p (0 <= p < c.len): element offset of the row
// in *kbase / *vbase.
__device__ inline size_t list_row(const Args& a, int kind, const ListCtx& c, bool hier, int p,
                                  const void** kbase, const void** vbase,
                                  bool coherent = false) {
    const int C = a.C;
    if (kind == kListMeta) {
        *kbase = a.km;
        *vbase = a.vm;
        return (((size_t)c.b * a.Hkv + c.g) * a.max_meta + p) * (size_t)a.D;
    }
    *kbase = a.kc;
    *vbase = a.vc;
    int slot;
    if (kind == kListGists) {
        slot = p * (C + 1) + C;
    } else if (kind == kListCand) {
        slot = cand_gist(a, c, p) * (C + 1) + C;
    } else {
        int raw = c.ns * C;
        if (p < raw) {
            int j = p / C;
            slot = sel_at(a, c, j, coherent) * (C + 1) + (p - j * C);
        } else if (p < raw + c.tail) {
            slot = c.n * (C + 1) + (p - raw);
        } else {
            int q = p - raw - c.tail;
            int m;
            if (!hier) m = sel_at(a, c, q, coherent);
            else if (q < c.e1) m = sel_at(a, c, q, coherent);
            else m = c.nm * a.R + (q - c.e1);
            slot = m * (C + 1) + C;
        }
    }
    return slot_offset(a, c.b, c.g, slot);
}

// Partial slot of split `split` of list `kind`.
__device__ inline int partial_slot(const Args& a, int kind, int split) {
    return (kind == kListUnfolded ? a.S1 : 0) + split;
}

}  // namespace gsa
