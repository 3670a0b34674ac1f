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

constexpr int kSelCache = 4096;   // general path: keys kept in LDS; longer lists are re-read
constexpr int kSelFast = 8192;    // fast path: longest list
constexpr int kSelCandCap = 1536;    // fast path: largest boundary bucket


template <int NT>
struct SelectSmem {
    union {
        uint32_t keys[kSelCache];  // general path: order keys, then per-key flags
        struct {
            uint64_t selbits[kSelFast / 64];  // selected keys, one bit per index
            uint32_t tiebits[kSelFast / 32];  // keys equal to the threshold
            uint32_t ckey[kSelCandCap];          // boundary-bucket candidates
            int cidx[kSelCandCap];
        } f;
    };
    int hist[2048];
    int wsum[NT / 64];
    int wcnt[NT / 64];
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
    lds_barrier();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        int v = wsum[i];
        base += (i < w) ? v : 0;
        tot += v;
    }
    lds_barrier();
    *total = tot;
    return base + incl - x;
}

// General top-k: radix select over the whole key list, ordered output through
// per-key flags.  Serves long lists and large k; block_topk below is the fast
// path for the common shapes.
template <int NT>
__device__ int block_topk_general(const float* keys, const int32_t* ids, int n, int k, int32_t* out,
                                  bool coherent, SelectSmem<NT>& sh) {
    const int tid = threadIdx.x;
    const int keff = min(k, n);
    auto put = [&](int i, int v) {
        if (coherent) __hip_atomic_store(out + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else out[i] = v;
    };
    for (int i = keff + tid; i < k; i += NT) put(i, -1);
    if (keff == n) {
        for (int i = tid; i < n; i += NT) put(i, ids ? ids[i] : i);
        return keff;
    }
    if (keff == 0) return 0;
    const bool cached = n <= kSelCache;
    if (cached) {
        // eight loads in flight per thread
        for (int i0 = tid; i0 < n; i0 += 8 * NT) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = (i0 + j * NT < n) ? load_key(keys + i0 + j * NT, coherent) : 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (i0 + j * NT < n) sh.keys[i0 + j * NT] = order_key(v[j]);
        }
    }
    __syncthreads();
    auto key_at = [&](int i) -> uint32_t {
        return cached ? sh.keys[i] : order_key(load_key(keys + i, coherent));
    };

    const int lane = tid & 63, w = tid >> 6;
    uint32_t prefix = 0;   // fixed high digits of T
    int above = 0;         // keys above the current bucket range
    int fixed = 0;         // number of fixed high bits
    bool take_all = false;
    for (int pass = 0; pass < 3; ++pass) {
        const int width = pass < 2 ? 11 : 10;
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
        for (int i = tid; i < n; i += NT) sh.keys[i] = (uint32_t)flag_of(sh.keys[i]);
        __syncthreads();
    }
    const int per = (n + NT - 1) / NT;
    const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
    int c1 = 0, c2 = 0;
    for (int i = i0; i < i1; ++i) {
        int f = cached ? (int)sh.keys[i] : flag_of(key_at(i));
        c1 += f == 1;
        c2 += f == 2;
    }
    int tot;
    const int e2 = block_excl_scan<NT>(c2, &tot, sh.wsum);
    const int take2 = take_all ? c2 : max(0, min(c2, need_eq - e2));
    int pos = block_excl_scan<NT>(c1 + take2, &tot, sh.wsum);
    int seen2 = 0;
    for (int i = i0; i < i1; ++i) {
        int f = cached ? (int)sh.keys[i] : flag_of(key_at(i));
        bool s = f == 1 || (f == 2 && seen2++ < take2);
        if (s) put(pos++, ids ? ids[i] : i);
    }
    __syncthreads();
    return keff;
}


// Suffix scan of hist[0..NB) over the block: finds the bucket b* holding the
// need-th largest key (need >= 1, at most the histogram total) and the count
// of keys in buckets above it.  Results in sh.bstar / sh.above / sh.cnt.
template <int NT, int NB, typename Smem>
__device__ inline void find_bucket(int need, Smem& sh) {
    constexpr int PER = (NB + NT - 1) / NT;  // consecutive buckets per thread
    const int tid = threadIdx.x;
    int h[PER];
    int s = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int bi = tid * PER + j;
        h[j] = bi < NB ? sh.hist[bi] : 0;
        s += h[j];
    }
    // exclusive scan from the top: sum over higher threads
    const int lane = tid & 63, w = tid >> 6;
    int incl = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_down(incl, off);
        if (lane + off < 64) incl += y;
    }
    if (lane == 0) sh.wsum[w] = incl;  // wave total
    __syncthreads();
    int higher = incl - s;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) higher += i > w ? sh.wsum[i] : 0;
    if (higher < need && higher + s >= need) {
        int acc = higher;
        bool found = false;
#pragma unroll
        for (int j = PER - 1; j >= 0; --j) {
            if (!found && acc + h[j] >= need) {
                found = true;
                sh.bstar = tid * PER + j;
                sh.above = acc;
                sh.cnt = h[j];
            }
            acc += h[j];
        }
    }
    __syncthreads();
}

// Top-k of keys[0..n) (ids[i] or i), written ascending to out[0..k) with -1
// in unused slots.  Every thread of the block (NT threads) must call it.
// Returns min(k, n).  `coherent`: keys are read and out is written with
// device-scope atomics (other workgroups of the kernel produce / consume them).
//
// Fast path (n <= kSelFast): keys sit in registers (key i = tid + j*NT in
// thread tid, so one wavefront's j-th keys are 64 consecutive indices).
//   1. histogram of the top 11 bits of every key; bucket b0 holds the k-th
//      largest key.
//   2. keys above b0 are marked in the selection bitmap (one ballot per
//      wavefront and j, no atomics); keys in b0 are compacted into an LDS
//      candidate list (longer buckets: general path).
//   3. radix passes over the candidates' bits [20:10] and [9:0] fix the k-th
//      largest key T; candidates above T join the bitmap, those equal to T go
//      to a tie bitmap of which the lowest indices are taken.
//   4. a popcount scan of the bitmap emits the ids in ascending index order.
// A pass whose boundary bucket is taken whole ends the search early.
template <int NT>
__device__ int block_topk(const float* keys, const int32_t* ids, int n, int k, int32_t* out,
                          bool coherent, SelectSmem<NT>& sh) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int keff = min(k, n);
    if (n > kSelFast || keff == n || keff == 0)
        return block_topk_general<NT>(keys, ids, n, k, out, coherent, sh);
    constexpr int KPT = kSelFast / NT;
    constexpr int WORDS = kSelFast / 32;
    uint32_t kr[KPT];
    {
        float v[KPT];
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            v[j] = (tid + j * NT < n) ? load_key(keys + tid + j * NT, coherent) : 0.f;
#pragma unroll
        for (int j = 0; j < KPT; ++j) kr[j] = order_key(v[j]);
    }
    // 1. top-digit histogram
    for (int i = tid; i < 2048; i += NT) sh.hist[i] = 0;
    for (int i = tid; i < WORDS; i += NT) sh.f.tiebits[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        if (tid + j * NT < n) atomicAdd(&sh.hist[kr[j] >> 21], 1);
    __syncthreads();
    find_bucket<NT, 2048>(keff, sh);
    const uint32_t b0 = (uint32_t)sh.bstar;
    int above = sh.above;
    const int cnt0 = sh.cnt;
    if (cnt0 > kSelCandCap) {
        // boundary bucket too long for the candidate list
        __syncthreads();
        return block_topk_general<NT>(keys, ids, n, k, out, coherent, sh);
    }
    const bool all0 = above + cnt0 == keff;
    // 2. classify: bitmap words by ballot, candidate count per wavefront
    int nmine = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const bool valid = tid + j * NT < n;
        const uint32_t top = kr[j] >> 21;
        const uint64_t sel = __ballot(valid && (top > b0 || (all0 && top == b0)));
        if (lane == 0) sh.f.selbits[(j * NT + 64 * w) >> 6] = sel;
        nmine += __popcll(__ballot(valid && !all0 && top == b0));
    }
    if (!all0) {
        if (lane == 0) sh.wcnt[w] = nmine;
        __syncthreads();
        int pos = 0;
#pragma unroll
        for (int i = 0; i < NT / 64; ++i) pos += i < w ? sh.wcnt[i] : 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const bool eq = tid + j * NT < n && (kr[j] >> 21) == b0;
            const uint64_t m = __ballot(eq);
            if (eq) {
                const int at = pos + __popcll(m & ((1ull << lane) - 1ull));
                sh.f.ckey[at] = kr[j];
                sh.f.cidx[at] = tid + j * NT;
            }
            pos += __popcll(m);
        }
    }
    __syncthreads();
    if (!all0) {
        // 3. radix passes over the candidates
        uint32_t prefix = b0 << 21;
        int fixed = 11;
        bool take_all = false;
#pragma unroll
        for (int pass = 1; pass < 3; ++pass) {
            const int width = pass == 1 ? 11 : 10;
            const int shift = 32 - fixed - width;
            for (int i = tid; i < (1 << width); i += NT) sh.hist[i] = 0;
            __syncthreads();
            for (int c = tid; c < cnt0; c += NT) {
                const uint32_t x = sh.f.ckey[c];
                if ((x >> (32 - fixed)) == (prefix >> (32 - fixed)))
                    atomicAdd(&sh.hist[(x >> shift) & ((1 << width) - 1)], 1);
            }
            __syncthreads();
            if (pass == 1) find_bucket<NT, 2048>(keff - above, sh);
            else find_bucket<NT, 1024>(keff - above, sh);
            above += sh.above;
            prefix |= (uint32_t)sh.bstar << shift;
            fixed += width;
            const int cnt = sh.cnt;
            __syncthreads();
            if (above + cnt == keff) {
                take_all = true;
                break;
            }
        }
        const uint32_t lo = prefix;
        const uint32_t hi = fixed >= 32 ? prefix : (prefix | ((1u << (32 - fixed)) - 1u));
        for (int c = tid; c < cnt0; c += NT) {
            const uint32_t x = sh.f.ckey[c];
            const int i = sh.f.cidx[c];
            if (x > hi || (take_all && x >= lo))
                atomicOr((unsigned long long*)&sh.f.selbits[i >> 6], 1ull << (i & 63));
            else if (x >= lo)
                atomicOr(&sh.f.tiebits[i >> 5], 1u << (i & 31));
        }
        __syncthreads();
        if (!take_all) {
            // the (keff - above) lowest-index keys equal to T join the selection
            const int need_eq = keff - above;
            const int wd = tid < WORDS ? tid : -1;
            const uint32_t tb = wd >= 0 ? sh.f.tiebits[wd] : 0u;
            int tot;
            int before = block_excl_scan<NT>(__popc(tb), &tot, sh.wsum);
            if (wd >= 0 && tb) {
                uint32_t add = 0u, rest = tb;
                while (rest && before < need_eq) {
                    const uint32_t bit = rest & (~rest + 1u);
                    add |= bit;
                    rest ^= bit;
                    ++before;
                }
                if (add) atomicOr((unsigned long long*)&sh.f.selbits[wd >> 1], (uint64_t)add << (32 * (wd & 1)));
            }
            __syncthreads();
        }
    }
    // 4. ascending output: popcount scan over the bitmap words
    auto put = [&](int i, int v) {
        if (coherent) __hip_atomic_store(out + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else out[i] = v;
    };
    for (int i = keff + tid; i < k; i += NT) put(i, -1);
    {
        const int wd = tid < WORDS ? tid : -1;
        uint32_t sb = wd >= 0 ? (uint32_t)(sh.f.selbits[wd >> 1] >> (32 * (wd & 1))) : 0u;
        int tot;
        int pos = block_excl_scan<NT>(__popc(sb), &tot, sh.wsum);
        while (sb) {
            const int bit = __ffs(sb) - 1;
            sb &= sb - 1u;
            const int i = wd * 32 + bit;
            put(pos++, ids ? ids[i] : i);
        }
    }
    __syncthreads();
    return keff;
}

}  // namespace gsa
