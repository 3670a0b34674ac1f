// Standalone per-unit top-k select kernel (one workgroup per unit) for the
// multi-launch paths; the selection itself is block_topk.
#include "gsa_lists.h"
#include "gsa_select.h"

namespace gsa {
namespace {

constexpr int kThreads = 512;
constexpr int kKeyParts = 8;  // workgroups per unit making sum-of-probabilities keys

// Block-wide max / sum of one value per thread (every thread gets the result).
__device__ inline float block_reduce(float x, bool is_max, float* red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int o = 32; o > 0; o >>= 1) {
        const float y = __shfl_xor(x, o);
        x = is_max ? fmaxf(x, y) : x + y;
    }
    __syncthreads();  // the previous use of red is over
    if (lane == 0) red[w] = x;
    __syncthreads();
    x = red[0];
    for (int i = 1; i < kThreads / 64; ++i) x = is_max ? fmaxf(x, red[i]) : x + red[i];
    return x;
}

// Block-wide max / sum of 16 values per thread at once (every thread gets the
// results).  red: [kThreads / 64][16].
__device__ inline void block_reduce16(float (&x)[16], bool is_max, float* red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int h = 0; h < 16; ++h)
        for (int o = 32; o > 0; o >>= 1) {
            const float y = __shfl_xor(x[h], o);
            x[h] = is_max ? fmaxf(x[h], y) : x[h] + y;
        }
    __syncthreads();  // the previous use of red is over
    if (lane < 16) {
#pragma unroll
        for (int h = 0; h < 16; ++h)
            if (h == lane) red[16 * w + h] = x[h];
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 16; ++h) {
        float v = red[h];
        for (int i = 1; i < kThreads / 64; ++i) v = is_max ? fmaxf(v, red[16 * i + h]) : v + red[16 * i + h];
        x[h] = v;
    }
}

// Sum-of-probabilities routing key of the unit's n gists: for each head of the
// group, the softmax of its logits over the gists; the key of a gist is the sum
// of its probabilities over the heads.  Overwrites the sum-of-logits keys.  All
// heads go through each pass together and four gists per thread are unrolled,
// so a pass takes a few load round trips.  Used with the selected-gists set
// (no gist attention partials); otherwise probs_keys_kernel makes the keys.
__device__ void sum_probs_keys(const Args& a, int u, int n, float* kw, float* red) {
    const int G = a.G;  // <= 16
    const size_t hs = a.key_stride;
    const float* z = a.hlog + (size_t)u * G * hs;
    float m[16], l[16];
#pragma unroll
    for (int h = 0; h < 16; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
    }
#pragma unroll 4
    for (int i = threadIdx.x; i < n; i += kThreads) {
#pragma unroll
        for (int h = 0; h < 16; ++h)
            if (h < G) m[h] = fmaxf(m[h], z[h * hs + i]);
    }
    block_reduce16(m, true, red);
#pragma unroll 4
    for (int i = threadIdx.x; i < n; i += kThreads) {
#pragma unroll
        for (int h = 0; h < 16; ++h)
            if (h < G) l[h] += expf(z[h * hs + i] - m[h]);
    }
    block_reduce16(l, false, red);
#pragma unroll 4
    for (int i = threadIdx.x; i < n; i += kThreads) {
        float key = 0.f;
#pragma unroll
        for (int h = 0; h < 16; ++h)
            if (h < G) key += expf(z[h * hs + i] - m[h]) / l[h];
        kw[i] = key;
    }
    __syncthreads();
}

// Sum-of-probabilities keys with the all-gists set (grid: kKeyParts x units):
// each workgroup folds its unit's gist attention partials into every head's
// softmax maximum and normaliser (base-2 domain) and writes the keys of its
// part of the gists.  A few parts per unit: the fold is repeated per part.
// The logits of the part's keys are loaded first, so that their round trip
// overlaps the fold's; each thread holds its splits' (max, sum) pairs for both
// reductions.
__global__ __launch_bounds__(kThreads) void probs_keys_kernel(Args a) {
    __shared__ float red[16 * (kThreads / 64)];
    const int u = blockIdx.y;
    int n, tail;
    seq_shape(a, u / a.Hkv, n, tail);
    const int per = (n + (int)gridDim.x - 1) / (int)gridDim.x;
    const int p0 = blockIdx.x * per;
    if (p0 >= n) return;  // block-uniform
    const int G = a.G;    // <= 16
    const int ns = (n + a.SL - 1) / a.SL;
    const float2* ml = a.part_ml + (size_t)u * a.NS * G;
    // each split's normaliser: its sum of unrounded probabilities where the
    // attention kernel kept one (the MFMA kernels' part_ml sums the bf16 PV
    // operand), else part_ml's (exact on the fp32 kernels)
    const float* es = a.hsum ? a.hsum + (size_t)u * a.NS * G : nullptr;
    auto split_l = [&](int sp, int h, float y) { return es ? es[(size_t)sp * G + h] : y; };
    const size_t hs = a.key_stride;
    const float* zl = a.hlog + (size_t)u * G * hs;
    float* kw = a.keys + (size_t)u * hs;
    const int end = min(n, p0 + per);
    // this thread's keys: gists p0 + tid + kThreads * q (q < KQ); more than
    // KQ per thread loop below
    constexpr int KQ = 2;
    float zv[KQ][16];
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
        const int i = p0 + threadIdx.x + q * kThreads;
#pragma unroll
        for (int h = 0; h < 16; ++h) zv[q][h] = (h < G && i < end) ? zl[h * hs + i] : 0.f;
    }
    // the splits' pairs: sp = tid + kThreads * r (r < SR)
    constexpr int SR = 2;
    float m[16], l[16];
    float2 pr[SR][16];
#pragma unroll
    for (int r = 0; r < SR; ++r) {
        const int sp = threadIdx.x + r * kThreads;
#pragma unroll
        for (int h = 0; h < 16; ++h) {
            pr[r][h] = (h < G && sp < ns) ? ml[(size_t)sp * G + h] : make_float2(-INFINITY, 0.f);
            if (h < G && sp < ns) pr[r][h].y = split_l(sp, h, pr[r][h].y);
        }
    }
#pragma unroll
    for (int h = 0; h < 16; ++h) m[h] = fmaxf(pr[0][h].x, pr[1][h].x);
    for (int sp = threadIdx.x + SR * kThreads; sp < ns; sp += kThreads) {
#pragma unroll
        for (int h = 0; h < 16; ++h)
            if (h < G) m[h] = fmaxf(m[h], ml[(size_t)sp * G + h].x);
    }
    block_reduce16(m, true, red);
#pragma unroll
    for (int h = 0; h < 16; ++h) {
        l[h] = 0.f;
#pragma unroll
        for (int r = 0; r < SR; ++r)
            if (pr[r][h].x != -INFINITY) l[h] += pr[r][h].y * exp2f(pr[r][h].x - m[h]);
    }
    for (int sp = threadIdx.x + SR * kThreads; sp < ns; sp += kThreads) {
#pragma unroll
        for (int h = 0; h < 16; ++h)
            if (h < G) l[h] += split_l(sp, h, ml[(size_t)sp * G + h].y) * exp2f(ml[(size_t)sp * G + h].x - m[h]);
    }
    block_reduce16(l, false, red);
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
        const int i = p0 + threadIdx.x + q * kThreads;
        if (i >= end) continue;
        float key = 0.f;
#pragma unroll
        for (int h = 0; h < 16; ++h)
            if (h < G) key += exp2f(zv[q][h] * 1.4426950408889634f - m[h]) / l[h];
        kw[i] = key;
    }
    for (int i = p0 + threadIdx.x + KQ * kThreads; i < end; i += kThreads) {
        float key = 0.f;
#pragma unroll
        for (int h = 0; h < 16; ++h)
            if (h < G) key += exp2f(zl[h * hs + i] * 1.4426950408889634f - m[h]) / l[h];
        kw[i] = key;
    }
}

__global__ __launch_bounds__(kThreads) void select_kernel(Args a, int mode) {
    __shared__ SelectSmem<kThreads> sh;
    __shared__ float red[16 * (kThreads / 64)];
    const int u = blockIdx.x;
    ListCtx c;
    make_ctx(a, mode == kSelCand ? kListCand : kListGists, u, mode != kSelGists, c);
    if (mode == kSelGists) {
        // scores past the sequence's gists read -inf
        float* kw = a.keys + (size_t)u * a.key_stride;
        if (a.hlog && (a.flags & kFlagSelectedGists)) sum_probs_keys(a, u, c.n, kw, red);  // (else done by probs_keys_kernel)
        for (int i = c.n + threadIdx.x; i < a.num_chunks; i += kThreads) kw[i] = -INFINITY;
        block_topk<kThreads>(a.keys + (size_t)u * a.key_stride, nullptr, c.n, a.top_k,
                             a.sel + (size_t)u * a.top_k, false, sh);
    } else if (mode == kSelMeta) {
        block_topk<kThreads>(a.mkeys + (size_t)u * a.max_meta, nullptr, c.nm, a.top_k_meta,
                             a.sel_meta + (size_t)u * a.top_k_meta, false, sh);
    } else {
        block_topk<kThreads>(a.ckeys + (size_t)u * a.cand_stride,
                             a.cand + (size_t)u * a.cand_stride, c.len, a.top_k,
                             a.sel + (size_t)u * a.top_k, false, sh);
    }
}

// Top-p: trims the unit's top-k selection (k = top_k, the cap; ascending ids,
// -1 padded) to the shortest prefix of key order (largest first, ties to the
// lower id, NaN last) whose selection probabilities reach top_p, rewrites it
// ascending and stores its length in nsel.  A chunk's selection probability
// is the softmax of its key over the sequence's gists (NaN: 0).  The softmax
// maximum and normaliser come from one streaming pass over the keys (each
// thread rescales its running sum as its maximum grows); entry ranks are
// counted by every thread over a share of the others; the prefix is summed in
// key order (chunks of ranks per lane, then a prefix over lanes) and the kept
// entries are packed with a block scan.
__global__ __launch_bounds__(kThreads) void topp_trim_kernel(Args a) {
    __shared__ uint32_t okey[kTopPMaxK];
    __shared__ int oid[kTopPMaxK];
    __shared__ float wr[kTopPMaxK];  // selection weights in key order
    __shared__ int rk[kTopPMaxK];    // key-order rank of selection entry i
    __shared__ float red[kThreads / 64];
    __shared__ int wsum[kThreads / 64];
    __shared__ int s_need;
    const int u = blockIdx.x, tid = threadIdx.x;
    int n, tail;
    seq_shape(a, u / a.Hkv, n, tail);
    const int kk = min(a.top_k, n);
    const float* kw = a.keys + (size_t)u * a.key_stride;
    int32_t* sel = a.sel + (size_t)u * a.top_k;
    // the selection's entries and keys (loads issued with the key pass's)
    constexpr int EPT = kTopPMaxK / kThreads;  // entries per thread: i = EPT * tid + e
    int myid[EPT];
    float mykey[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = EPT * tid + e;
        myid[e] = i < kk ? sel[i] : 0;
    }
    // running maximum and sum of exp over this thread's keys
    constexpr int kBatch = 16;
    float m = -INFINITY, z = 0.f;
    for (int i0 = tid; i0 < n; i0 += kBatch * kThreads) {
        float v[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int i = i0 + k * kThreads;
            v[k] = i < n ? kw[i] : NAN;
        }
        float bm = -INFINITY;
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
            if (!isnan(v[k])) bm = fmaxf(bm, v[k]);
        if (bm == -INFINITY) continue;  // nothing above -inf in the batch
        const float mn = fmaxf(m, bm);
        float zb = 0.f;
        if (isfinite(mn)) {
#pragma unroll
            for (int k = 0; k < kBatch; ++k) zb += isnan(v[k]) ? 0.f : expf(v[k] - mn);
        }
        z = (m == -INFINITY || !isfinite(mn) ? 0.f : z * expf(m - mn)) + zb;
        m = mn;
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = EPT * tid + e;
        mykey[e] = i < kk ? kw[myid[e]] : 0.f;
        if (i < kk) {
            oid[i] = myid[e];
            okey[i] = order_key(mykey[e]);
            rk[i] = 0;
        }
    }
    const float M = block_reduce(m, true, red);
    const bool usable = isfinite(M);
    z = block_reduce(usable && m != -INFINITY ? z * expf(m - M) : 0.f, false, red);
    __syncthreads();  // okey, oid, rk in place
    // ranks: thread t counts, for entry t % kk (and those kThreads apart),
    // the entries of its share of the others that come first in key order
    {
        const int reps = kk > 0 ? max(1, kThreads / kk) : 1;  // threads per entry
        const int i0 = tid % max(kk, 1), part = tid / max(kk, 1);
        if (kk > 0 && part < reps) {
            const int per = (kk + reps - 1) / reps, jb = part * per, je = min(kk, jb + per);
            for (int i = i0; i < kk; i += kThreads) {
                const uint32_t oi = okey[i];
                const int di = oid[i];
                int r = 0;
                for (int j = jb; j < je; ++j) r += okey[j] > oi || (okey[j] == oi && oid[j] < di);
                atomicAdd(&rk[i], r);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = EPT * tid + e;
        if (i < kk) wr[rk[i]] = (usable && !isnan(mykey[e])) ? expf(mykey[e] - M) : 0.f;
    }
    __syncthreads();
    if (tid < 64) {
        // wavefront 0: lane l sums ranks [l*per, (l+1)*per), a prefix over the
        // lanes finds the chunk where the running sum reaches the target, and
        // that lane walks its chunk to the cut
        const int per = (kk + 63) / 64, b0 = tid * per, e0 = min(kk, b0 + per);
        float cs = 0.f;
        for (int r = b0; r < e0; ++r) cs += wr[r];
        float incl = cs;
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(incl, o);
            if (tid >= o) incl += y;
        }
        const float target = a.top_p * z;
        const uint64_t hit = __ballot(usable && b0 < e0 && incl >= target);
        int need = kk;
        if (hit) {
            const int lc = __ffsll((unsigned long long)hit) - 1;
            int nl = e0;  // (rounding: the chunk's end if the walk falls short)
            float cum = incl - cs;
            for (int r = b0; r < e0; ++r) {
                cum += wr[r];
                if (cum >= target) {
                    nl = r + 1;
                    break;
                }
            }
            need = __shfl(nl, lc);
        }
        if (tid == 0) {
            s_need = need;
            a.nsel[u] = need;
        }
    }
    __syncthreads();
    const int need = s_need;
    // keep the entries ranked below `need`, in their (ascending id) order
    int keep = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) keep += (EPT * tid + e < kk && rk[EPT * tid + e] < need) ? 1 : 0;
    int tot;
    int pos = block_excl_scan<kThreads>(keep, &tot, wsum);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = EPT * tid + e;
        if (i < kk && rk[i] < need) sel[pos++] = myid[e];
    }
    for (int i = need + tid; i < a.top_k; i += kThreads) sel[i] = -1;
}

}  // namespace

hipError_t launch_probs_keys(const Args& a, hipStream_t st) {
    hipLaunchKernelGGL(probs_keys_kernel, dim3(kKeyParts, a.B * a.Hkv), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_topp_trim(const Args& a, hipStream_t st) {
    hipLaunchKernelGGL(topp_trim_kernel, dim3(a.B * a.Hkv), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_select(const Args& a, int mode, hipStream_t st) {
    hipLaunchKernelGGL(select_kernel, dim3(a.B * a.Hkv), dim3(kThreads), 0, st, a, mode);
    return hipGetLastError();
}

}  // namespace gsa
