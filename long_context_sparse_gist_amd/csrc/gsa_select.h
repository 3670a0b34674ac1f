// Block-wide top-k with deterministic tie-break on the lower index.
//
// Keys become order-preserving uint32 (larger float -> larger key, -0 == +0,
// NaN smallest).  The k-th largest key T is found by radix select over the
// digits [31:21], [20:10], [9:0]: each pass histograms (LDS atomics) the keys
// that share the already fixed high digits, and the bucket holding the k-th
// largest key fixes the next digit; a pass stops the search early when the
// keys above a bucket boundary are exactly k.  Selection = keys above T's
// bucket range, plus the lowest-index keys inside it when it is a single
// value.  The selected ids are written in ascending index order by an ordered
// scan over per-key flags (threads own contiguous index ranges).
#pragma once

#include "gsa_internal.h"

namespace gsa {

constexpr int kSelCache = 8192;  // keys kept in LDS; longer lists are re-read

template <int NT>
struct SelectSmem {
    uint32_t keys[kSelCache];
    uint8_t flags[kSelCache];
    int hist[2048];
    int wsum[NT / 64];
    int bstar, above, cnt;
};

// Loads a key.  `coherent`: read with device-scope atomic loads (data written
// by other workgroups of the same kernel).
__device__ inline float load_key(const float* p, bool coherent) {
    return coherent ? __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT)
                    : *p;
}

template <int NT>
__device__ inline int block_excl_scan(int x, int* total, int* wsum) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        int v = wsum[i];
        base += (i < w) ? v : 0;
        tot += v;
    }
    __syncthreads();
    *total = tot;
    return base + incl - x;
}

// Top-k of keys[0..n) (ids[i] or i), written ascending to out[0..k) with -1
// in unused slots.  Every thread of the block (NT threads) must call it.
// Returns min(k, n).
template <int NT>
__device__ int block_topk(const float* keys, const int32_t* ids, int n, int k, int32_t* out,
                          bool coherent, SelectSmem<NT>& sh) {
    const int tid = threadIdx.x;
    const int keff = min(k, n);
    for (int i = keff + tid; i < k; i += NT) out[i] = -1;
    if (keff == n) {
        for (int i = tid; i < n; i += NT) out[i] = ids ? ids[i] : i;
        return keff;
    }
    if (keff == 0) return 0;
    const bool cached = n <= kSelCache;
    if (cached)
        for (int i = tid; i < n; i += NT) sh.keys[i] = order_key(load_key(keys + i, coherent));
    __syncthreads();
    auto key_at = [&](int i) -> uint32_t {
        return cached ? sh.keys[i] : order_key(load_key(keys + i, coherent));
    };

    const int lane = tid & 63, w = tid >> 6;
    uint32_t prefix = 0;   // fixed high digits of T
    int above = 0;         // keys above the current bucket range
    int fixed = 0;         // number of fixed high bits
    bool take_all = false;
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
        const int width = widths[pass];
        const int shift = 32 - fixed - width;
        const int nb = 1 << width;
        for (int i = tid; i < nb; i += NT) sh.hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += NT) {
            uint32_t x = key_at(i);
            bool match = fixed == 0 || (x >> (32 - fixed)) == (prefix >> (32 - fixed));
            if (match) atomicAdd(&sh.hist[(x >> shift) & (nb - 1)], 1);
        }
        __syncthreads();
        if (w == 0) {
            const int need = keff - above;
            const int per = nb / 64;
            int s = 0;
            for (int j = 0; j < per; ++j) s += sh.hist[lane * per + j];
            int incl = s;  // sum over this lane and the higher lanes
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                int y = __shfl_down(incl, off);
                if (lane + off < 64) incl += y;
            }
            int higher = incl - s;
            if (higher < need && higher + s >= need) {
                int acc = higher;
                for (int j = per - 1; j >= 0; --j) {
                    int h = sh.hist[lane * per + j];
                    if (acc + h >= need) {
                        sh.bstar = lane * per + j;
                        sh.above = acc;
                        sh.cnt = h;
                        break;
                    }
                    acc += h;
                }
            }
        }
        __syncthreads();
        const int bstar = sh.bstar, add = sh.above, cnt = sh.cnt;
        __syncthreads();
        above += add;
        prefix |= (uint32_t)bstar << shift;
        fixed += width;
        if (above + cnt == keff) {
            take_all = true;
            break;
        }
    }
    const uint32_t lo = prefix;
    const uint32_t hi = fixed >= 32 ? prefix : (prefix | ((1u << (32 - fixed)) - 1u));
    const int need_eq = keff - above;

    // flags: 1 = above the range, 2 = inside it
    auto flag_of = [&](uint32_t x) -> int { return x > hi ? 1 : (x >= lo ? 2 : 0); };
    if (cached) {
        for (int i = tid; i < n; i += NT) sh.flags[i] = (uint8_t)flag_of(sh.keys[i]);
        __syncthreads();
    }
    const int per = (n + NT - 1) / NT;
    const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
    int c1 = 0, c2 = 0;
    for (int i = i0; i < i1; ++i) {
        int f = cached ? sh.flags[i] : flag_of(key_at(i));
        c1 += f == 1;
        c2 += f == 2;
    }
    int tot;
    const int e2 = block_excl_scan<NT>(c2, &tot, sh.wsum);
    const int take2 = take_all ? c2 : max(0, min(c2, need_eq - e2));
    int pos = block_excl_scan<NT>(c1 + take2, &tot, sh.wsum);
    int seen2 = 0;
    for (int i = i0; i < i1; ++i) {
        int f = cached ? sh.flags[i] : flag_of(key_at(i));
        bool s = f == 1 || (f == 2 && seen2++ < take2);
        if (s) out[pos++] = ids ? ids[i] : i;
    }
    __syncthreads();
    return keff;
}

}  // namespace gsa
