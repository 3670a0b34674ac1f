// Top-k of a short list by one wavefront (no LDS, no barriers): the same
// selection rule as block_topk in gsa_select.h.
#pragma once

#include "gsa_internal.h"

namespace gsa {

// Top-k of keys[0..n) (ids[i] or i) by one wavefront, for n <= 64 * KPW:
// the same selection as block_topk (ties to the lower index, NaN smallest),
// written ascending to out[0..k) with -1 in unused slots; returns min(k, n).
// Lane l holds keys l + 64j (and their ids) in registers, loaded together up
// front; no LDS and no barrier.  The k-th largest order key T is found bit by
// bit from the top: T | 2^b is kept when at least k keys reach it (one
// compare, ballot and popcount per register key); when exactly k keys reach
// a probe they are the selection.  Otherwise keys above T are selected, then
// the lowest-index keys equal to T.  A key's output position is the number
// of selected keys below its index (popcounts of the selection masks).
// Every lane of the wavefront must call it with the same arguments.
template <int KPW, typename KeyPtr, typename IdPtr, typename OutPtr>
__device__ int wave_topk(KeyPtr keys, IdPtr ids, int n, int k, OutPtr out) {
    const int lane = threadIdx.x & 63;
    const int keff = min(k, n);
    for (int i = keff + lane; i < k; i += 64) out[i] = -1;
    if (keff == 0) return 0;
    uint32_t x[KPW];
    int id[KPW];
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
        const int i = lane + 64 * j;
        const int ic = i < n ? i : n - 1;  // in bounds: every load issues unconditionally
        x[j] = order_key(keys[ic]);
        id[j] = ids ? ids[ic] : i;
    }
#pragma unroll
    for (int j = 0; j < KPW; ++j)
        if (lane + 64 * j >= n) x[j] = 0u;  // absent keys: 0, below every probe
    uint32_t T = 0u;
    bool exact = false;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = T | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < KPW; ++j) cnt += __popcll(__ballot(x[j] >= c));
        if (cnt >= keff) {
            T = c;
            if (cnt == keff) {
                exact = true;
                break;
            }
        }
    }
    // selection masks: keys reaching T (exact), or keys above T, then the
    // lowest-index keys equal to T (absent keys are excluded by their index;
    // NaN keys equal T = 0 only when fewer than k keys are numbers)
    uint64_t selm[KPW];
    int need = keff;
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
        selm[j] = exact ? __ballot(x[j] >= T) : __ballot(x[j] > T);
        need -= __popcll(selm[j]);
    }
    if (need > 0) {
#pragma unroll
        for (int j = 0; j < KPW; ++j) {
            uint64_t e = __ballot(x[j] == T && lane + 64 * j < n);
            if (need > 0 && e) {
                if (__popcll(e) <= need) {
                    selm[j] |= e;
                    need -= __popcll(e);
                } else {
                    while (need > 0) {
                        const uint64_t low = e & (~e + 1ull);
                        selm[j] |= low;
                        e ^= low;
                        --need;
                    }
                }
            }
        }
    }
    const uint64_t below = (1ull << lane) - 1ull;
    int base = 0;
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
        const uint64_t m = selm[j];
        if ((m >> lane) & 1ull) out[base + __popcll(m & below)] = id[j];
        base += __popcll(m);
    }
    return keff;
}

}  // namespace gsa
