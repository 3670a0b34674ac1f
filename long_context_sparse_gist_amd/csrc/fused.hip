// Single-launch GSA decode (bf16, MFMA): one kernel, one task per workgroup.
//
// Workgroup t runs task t.  Tasks are numbered gist slices first (every unit,
// unit-major), then unfolded-list tasks:
//   gist slice (u, i)  scores gists [i*TA, (i+1)*TA) of unit u, writes their
//                      routing keys, publishes them sorted by the top 11 bits
//                      of their order key (bucket), largest first (the
//                      leading ones also into the unit's record), and
//                      (all-gists set) one softmax partial.  The unit's
//                      last slice runs the top-k select over the sorted
//                      slices as soon as its own keys and partial are
//                      written, and publishes the selection.
//   unfolded (u, j)    folds gist-slice partials i = j, j+nB, ... while the
//                      select runs, polls its chunks' row offsets (written
//                      by the select into the unit's record), attends tokens
//                      [j*TB, (j+1)*TB) of the unfolded list (raw tokens of
//                      the selected chunks, raw tail, selected gists) and
//                      writes one partial.  The unit's last unfolded task
//                      keeps its own partial in registers, waits for the
//                      others' partials, merges them into the output and
//                      returns the unit's record to zero.
// Waits: unfolded tasks on gist slices, the merging task on the unit's other
// unfolded tasks (all of them smaller workgroup ids), and the selecting slice
// of a unit (its last) on the unit's other slices: every task waits only on
// tasks with smaller workgroup ids.  The device dispatches each XCD's
// workgroups in id order, so while the smallest unfinished task is not yet
// running, every workgroup ahead of it on its XCD has finished and freed its
// slot; it is then dispatched, and everything it waits on has finished.  By
// induction every task runs and every wait ends.  A wait is nevertheless bounded; giving up sets the
// error word of the control block.  Several workgroups per CU hide
// each task's serial latencies (table lookups, drains) behind the others'
// streaming, and the unfolded tasks of early units overlap the gist slices of
// later ones.  Data passed between workgroups is written and read with
// device-scope atomics (coherent across the XCDs' L2s); a producer waits for
// its stores to complete before it bumps a counter.  The selection's row
// offsets need no such wait: each is one 64-bit word, nonzero once written,
// that its readers poll.  The unit's merging task returns the unit's record
// to zero.
//
// Select.  A wavefront issues at most one instruction every few cycles, so a
// single workgroup that touches every key of a unit several times is slow
// (thousands of keys per wavefront).  The per-key work is done where the keys
// are made instead: each slice (one key per thread) sorts its keys by bucket.
// The select then needs only the first few keys of every slice, plus the rest
// of the rare slice that holds many of the largest keys (select_fused).
#include "gsa_lists.h"
#include "gsa_mfma_core.h"
#include "gsa_select.h"

namespace gsa {
namespace {

constexpr int kThreads = 256;
constexpr unsigned kSpinLimit = 1u << 24;
constexpr int kFSelMaxSlices = kRecSlices;  // slices the bucketed select merges
constexpr int kFSelMaxN = 16384;     // gists per unit the bucketed select handles
constexpr int kFSelBt = 768;         // block-table entries the select keeps in LDS
constexpr int kFSelCand = 1024;      // largest boundary bucket (else the general select)
constexpr int kFSelL = kRecLead;     // keys per slice the select reads up front

__device__ inline void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(int32_t* p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(int64_t* p, int64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_dev(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline unsigned ld_dev(const unsigned* p) {
    return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int32_t ld_dev(const int32_t* p) {
    return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t ld_dev(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int64_t ld_dev(const int64_t* p) {
    return __hip_atomic_load(const_cast<int64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline unsigned add_dev(unsigned* p, unsigned v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until this thread's memory operations have completed
__device__ inline void drain() { __builtin_amdgcn_s_waitcnt(0); }
// wait until the 100 MHz wall clock reaches t (pacing only: no data depends on it)
__device__ inline void hold_until(unsigned long long t) {
    while (wall_clock64() < t) __builtin_amdgcn_s_sleep(8);
}

// Buffer view of `bytes` bytes at p (raw, 32-bit data format word).  A load at
// an offset at or past the end reads 0 and touches no memory: the folds use
// that instead of a lane-masked branch around every load.
__device__ inline __amdgpu_buffer_rsrc_t buf_view(const void* p, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr unsigned kBufOut = 0x40000000u;  // an offset part that keeps a load past the end
// 4-byte load with the cache policy of ld_dev (device scope: sc1)
__device__ inline float ld_dev_buf(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 16));
}

// Thread 0 waits until *p >= target (bounded; giving up sets the error word).
// The caller synchronises the block afterwards.  Polls are spaced out
// (SLEEP * 64 cycles): hundreds of waiting workgroups polling a few counter
// lines back to back load one memory channel enough to slow every other
// access that maps to it.
template <int SLEEP>
__device__ inline void wait_at_least(const unsigned* p, unsigned target, unsigned* err) {
    if (threadIdx.x != 0) return;
    unsigned it = 0;
    while (ld_dev(p) < target) {
        __builtin_amdgcn_s_sleep(SLEEP);
        if (++it >= kSpinLimit) {
            st_dev(err, 1u);
            break;
        }
    }
}

// As wait_at_least, polling every SLEEP * 64 cycles while more than two counts
// are missing and every 128 cycles after: many waiting workgroups poll
// rarely, the ones about to proceed see the last counts soon.
template <int SLEEP>
__device__ inline void wait_at_least_close(const unsigned* p, unsigned target, unsigned* err) {
    if (threadIdx.x != 0) return;
    unsigned it = 0;
    for (unsigned v = ld_dev(p); v < target; v = ld_dev(p)) {
        if (v + 2u < target)
            __builtin_amdgcn_s_sleep(SLEEP);
        else
            __builtin_amdgcn_s_sleep(2);
        if (++it >= kSpinLimit) {
            st_dev(err, 1u);
            break;
        }
    }
}

// Folding state of one partial: per-head running max (exp2 domain) and sum,
// and the factors of the round being folded.
constexpr int kFoldRound = 16;  // partials folded per round
struct __attribute__((aligned(16))) FoldHdr {
    float m[16], l[16], f_self[16], fg[16], fb[16];
    float f[16][kFoldRound];  // [head][slot of the round]
};

constexpr int kFSelKQ = kFSelMaxSlices * kFSelL / kThreads;  // up-front keys per thread
constexpr int kFSelKB = kFSelBt / kThreads;                   // block-table entries per thread

// The unit's block-table row, loaded by the selecting slice as soon as its
// own stream is done: the round trip overlaps its bucket sort and partial.
// (Loading the other slices' leading keys that early finds many not yet
// written and costs a poll more than it saves.)
struct SelPre {
    int bt[kFSelKB];
};

// LDS of the top-k select (last gist slice of a unit).
struct FSelSmem {
    uint64_t selbits[kFSelMaxN / 64];  // selected chunk ids, one bit each
    uint32_t tiebits[kFSelMaxN / 32];  // candidates equal to the k-th largest key
    uint32_t ckey[kFSelCand];          // boundary-bucket candidates: order key, chunk id
    int cidx[kFSelCand];
    int bt[kFSelBt];                   // the unit's block-table row
    int uh[kBins];                     // bucket histogram of the candidates
    int coarse[kBins / 32];            // its sums over 32 buckets
    int hist[128];                     // 7-bit digit histogram of the candidate passes
    uint64_t needmask;                 // slices whose boundary keys run past kFSelL
    int wsum[kThreads / 64];
    int ncand;
    int nr2;                           // keys kept from the second round
};

// Dynamic LDS layout (bytes), uses separated in time:
//   [0, vt)        V tiles of the attention blocks, parked routing keys
//   [0, kBins*4+)  a slice's bucket histogram and staged keys
//   [0, red)       wavefront combination
//   [0, sel)       top-k select (last gist slice of a unit)
struct Lds {
    // V tiles of the 4 wavefronts, then 64 parked routing keys per wavefront
    static constexpr int vt(int D) { return 4 * (32 * D * 2) + 4 * 64 * 4; }
    static constexpr int stash(int D) { return 4 * (32 * D * 2); }
    static constexpr int red(int G, int D) { return 4 * G * D * 4; }
    static int bytes(int G, int D) {
        int m = vt(D);
        m = m > red(G, D) ? m : red(G, D);
        m = m > kBins * 4 + kFusedTA * 8 ? m : kBins * 4 + kFusedTA * 8;  // histogram, staged keys
        m = m > (int)sizeof(FSelSmem) ? m : (int)sizeof(FSelSmem);
        m = m > (int)sizeof(SelectSmem<kThreads>) ? m : (int)sizeof(SelectSmem<kThreads>);
        return m;
    }
};

// Fold partial slots s0, s0 + st, ... (ns of them) of unit u into (acc, fh): acc[j] holds
// element threadIdx.x + j*kThreads of the G x D accumulator.  Eight slots per
// round, every load of a round in flight together.
template <int EJ>
__device__ __forceinline__ void fold_regs(const Args& a, int u, int s0, int st, int ns, float (&acc)[EJ], FoldHdr& fh) {
    const int G = a.G, GD = a.G * a.D;
    const size_t base = (size_t)u * a.NS;
    const __amdgpu_buffer_rsrc_t racc = buf_view(a.part_acc + base * GD, 4u * a.NS * GD);
    const __amdgpu_buffer_rsrc_t rml = buf_view(a.part_ml + base * G, 8u * a.NS * G);
    constexpr int NR = EJ >= 8 ? kFoldRound / 2 : kFoldRound;  // slots per round (registers)
    constexpr int HR = NR / 2;
    for (int r0 = 0; r0 < ns; r0 += NR) {
        const int nr = min(NR, ns - r0);
        // two half-round arrays (kept in registers), every load issued up front;
        // a slot past the round or an element past G x D reads 0 (offset past
        // the unit's partials)
        float va[EJ][HR], vb[EJ][HR];
        unsigned eo[EJ];
#pragma unroll
        for (int j = 0; j < EJ; ++j) {
            const int e = threadIdx.x + j * kThreads;
            eo[j] = e < GD ? 4u * e : kBufOut;
        }
#pragma unroll
        for (int i = 0; i < HR; ++i) {
            const unsigned oa = i < nr ? 4u * (unsigned)((s0 + (r0 + i) * st) * GD) : kBufOut;
            const unsigned ob = HR + i < nr ? 4u * (unsigned)((s0 + (r0 + HR + i) * st) * GD) : kBufOut;
#pragma unroll
            for (int j = 0; j < EJ; ++j) {
                va[j][i] = ld_dev_buf(racc, eo[j] + oa);
                vb[j][i] = ld_dev_buf(racc, eo[j] + ob);
            }
        }
        {
            // factors: the 16 lanes of row h hold slots 0..15 of head h
            const int h = threadIdx.x >> 4, i = threadIdx.x & 15;
            const unsigned om = h < G && i < nr ? 8u * (unsigned)((s0 + (r0 + i) * st) * G + h) : kBufOut;
            float x = ld_dev_buf(rml, om), y = ld_dev_buf(rml, om + 4u);
            x = h < G && i < nr ? x : -INFINITY;
            const float mold = h < G ? fh.m[h] : -INFINITY;
            const float lold = h < G ? fh.l[h] : 0.f;
            const float M = fmaxf(mold, rowmax16(x));
            const float fi = x == -INFINITY ? 0.f : exp2f(x - M);
            const float fself = mold == -INFINITY ? 0.f : exp2f(mold - M);
            const float L = lold * fself + rowsum16(y * fi);
            if (h < G) {
                fh.f[h][i] = fi;
                if (i == 0) {
                    fh.f_self[h] = fself;
                    fh.m[h] = M;
                    fh.l[h] = L;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < EJ; ++j) {
            const int e = threadIdx.x + j * kThreads;
            if (e < GD) {
                const int h = e / a.D;
                float f[NR];  // the head's factors, 16 bytes per LDS read
#pragma unroll
                for (int q = 0; q < NR / 4; ++q) {
                    const float4 v = ((const float4*)fh.f[h])[q];
                    f[4 * q] = v.x;
                    f[4 * q + 1] = v.y;
                    f[4 * q + 2] = v.z;
                    f[4 * q + 3] = v.w;
                }
                float x = acc[j] * fh.f_self[h];
#pragma unroll
                for (int i = 0; i < HR; ++i) x += va[j][i] * f[i] + vb[j][i] * f[HR + i];
                acc[j] = x;
            }
        }
        __syncthreads();
    }
}

// Bucket sort of one slice's keys, one per thread: kv (the key) and pos (its
// position in the slice, -1: none).  Publishes the keys (order key | list
// index << 32) in descending bucket order to `pairs`, staged in LDS and written
// as whole contiguous lines (the stores write through to memory, and a
// partially written line costs the memory a read-modify-write); with `lead`,
// also the first kFSelL of them (the slice's place in the unit's record).
__device__ __forceinline__ void bucket_slice(uint64_t* pairs, uint64_t* lead, int p0, float kv, int pos,
                             unsigned char* smem, int* wsum) {
    constexpr int PER = kBins / kThreads;  // consecutive buckets per thread
    int* hist = (int*)smem;
    uint64_t* pair_st = (uint64_t*)(smem + kBins * 4);  // kFusedTA pairs
    const int tid = threadIdx.x;
    for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
    lds_barrier();
    const uint32_t ok = order_key(kv);
    if (pos >= 0) atomicAdd(&hist[ok >> 21], 1);
    lds_barrier();
    int h[PER];
    int s = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        h[i] = hist[PER * tid + i];
        s += h[i];
    }
    int tot;
    const int below = block_excl_scan<kThreads>(s, &tot, wsum);
    int run = tot - below - s;  // keys in the buckets of higher threads
    int cur[PER];
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
        cur[i] = run;  // keys in buckets above bucket PER*tid + i
        run += h[i];
    }
    lds_barrier();  // histogram reads done
#pragma unroll
    for (int i = 0; i < PER; ++i) hist[PER * tid + i] = cur[i];
    lds_barrier();
    if (pos >= 0) {
        const int at = atomicAdd(&hist[ok >> 21], 1);
        pair_st[at] = (uint64_t)ok | ((uint64_t)(uint32_t)(p0 + pos) << 32);
    }
    lds_barrier();
    static_assert(kFusedTA == kThreads, "one pair per thread");
    if (tid < tot) st_dev(pairs + tid, pair_st[tid]);
    // the leading keys again, into the unit's record, index + 1: nonzero once written
    if (lead && tid < min(tot, kFSelL)) st_dev(lead + tid, pair_st[tid] + (1ull << 32));
    lds_barrier();  // the staged pairs are read (the stores need not have landed)
}

// Top-k of unit u (ascending chunk ids, -1 padded) and each selected chunk's
// first-row offset.  nA: gist slices of the unit, keys: the routing keys.
//
// Every slice left its keys sorted by bucket (the top 11 bits of the order
// key), largest first.  One round trip reads the first kFSelL keys of every
// slice and the block-table row; an LDS histogram of these candidates gives
// the bucket bT of their k-th largest key.  The k-th largest key overall lies
// in a bucket >= bT, and a slice whose kFSelL-th key lies below bT has all
// its keys of buckets >= bT among the candidates.  The keys of buckets >= bT
// past kFSelL in the other slices are read in a second round and join the
// histogram, which is then exact from bT up and gives the bucket b0 of the
// k-th largest key.  Keys above b0 are selected, keys in b0 are candidates.
// Wavefront 0 alone then runs three 7-bit radix passes over the candidates'
// low 21 bits, resolves ties to the lower chunk id and writes the selection
// ascending from the bitmap: a single wavefront needs no block barriers, and
// the candidates are few.
// Whether the bucketed select serves this list (else the general select),
// and whether it keeps the block-table row in LDS.
template <int KIND>
__device__ inline void select_plan(const Args& a, int n, int nA, bool& fast, bool& btl) {
    const int k = KIND == kListMeta ? a.top_k_meta : a.top_k, keff = min(k, n);
    fast = keff > 0 && keff < n && nA <= kFSelMaxSlices && n <= kFSelMaxN;
    btl = fast && KIND != kListMeta && a.max_pages <= kFSelBt;
}

// Issue the select's block-table loads (SelPre).
template <int KIND>
__device__ inline void select_prefetch(const Args& a, const ListCtx& c, int n, int nA, SelPre& pre) {
    bool fast, btl;
    select_plan<KIND>(a, n, nA, fast, btl);
    const int tid = threadIdx.x;
    if (btl) {
        const int32_t* btrow = a.bt + (size_t)c.b * a.max_pages;
#pragma unroll
        for (int j = 0; j < kFSelKB; ++j) {
            const int i = tid + j * kThreads;
            pre.bt[j] = i < a.max_pages ? btrow[i] : 0;
        }
    }
}

// The drained() of a caller with nothing to do once its stores have landed:
// the bucketed path then skips that wait (the paths that read stored keys
// wait for them themselves).
struct NoDrain {
    __device__ void operator()() const {}
};

// drained(): called by every thread once every wavefront's earlier stores
// have completed (at most once; maybe not at all; never with NoDrain).  pre: the block-table row
// loaded by select_prefetch.  Slice `own` (the calling one) is not bucket
// sorted: every thread brings its key (ownk: order key | list index << 32,
// ownv: present), so that slice is complete among the candidates.  own < 0:
// the caller owns no slice (every slice published its sorted keys).
template <int KIND, int PER = 1, typename Drained>
__device__ __forceinline__ bool select_fused(const Args& a, const Sched& sc, const ListCtx& c, int n, int nA,
                                             const float* keys, unsigned char* smem, SelPre& pre, int own,
                                             uint64_t ownk, bool ownv, Drained drained) {
    constexpr int KQ = kFSelKQ;   // up-front keys per thread
    constexpr int KR = kFSelCand / kThreads;                 // second-round keys per thread
    constexpr int WPL = kFSelMaxN / 32 / 64;                 // 32-bit bitmap words per lane of wavefront 0
    static_assert(kBins == 64 * 32, "64 coarse buckets of 32");
    static_assert(kFSelMaxN / 64 == kThreads, "one 64-bit bitmap word per thread");
    FSelSmem& sh = *(FSelSmem*)smem;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int u = c.u;
    constexpr bool meta = KIND == kListMeta, cand = KIND == kListCand;
    const int k = meta ? a.top_k_meta : a.top_k, keff = min(k, n);
    int32_t* out = (meta ? a.sel_meta : a.sel) + (size_t)u * k;
    int64_t* ro = unit_rowoff(a, u);  // one plus each selected chunk's first-row offset
    unsigned* mo = unit_meta(a, u);   // one plus each kept meta-group
    const uint64_t* pairs = cand ? a.spairs_c + (size_t)u * sc.S3 * kFusedTA : a.spairs + (size_t)u * sc.S1 * kFusedTA;
    const uint64_t* lead = cand ? unit_lead_c(a, u) : unit_lead(a, u);
    const int32_t* btrow = a.bt + (size_t)c.b * a.max_pages;
    bool fast, btl;
    select_plan<KIND>(a, n, nA, fast, btl);
    // candidate list index -> chunk id: the gists of the kept meta-groups,
    // then the gists past the last complete group (ascending either way)
    const int head = c.ns1 * a.R;
    unsigned kept[kRecMeta / kThreads];  // this thread's share of the kept groups (+1)
    if (cand) {
#pragma unroll
        for (int j = 0; j < kRecMeta / kThreads; ++j) {
            const int i = tid + j * kThreads;
            kept[j] = i < c.ns1 ? ld_dev(mo + i) : 1u;
        }
    }
    auto slice_n = [&](int sl) { return min(sc.TA, n - sl * sc.TA); };
    // everything but the leading keys waits for every other slice to be
    // done, and for this slice's own stores to have landed
    auto wait_slices = [&]() {
        drain();
        // (PER counts per slice: a slice that counts in per wavefront, 4; with
        // the sum-of-probabilities key there cntA counts the slices' per-head
        // pairs and cntS their keys)
        if (PER == 4 && KIND == kListGists && (a.flags & kFlagSumProbs))
            wait_at_least<8>(unit_cntS(a, u), (unsigned)PER * (own >= 0 ? nA - 1 : nA), sc.err);
        else
            wait_at_least<8>(cand ? unit_cntC(a, u) : unit_cntA(a, u), (unsigned)PER * (own >= 0 ? nA - 1 : nA),
                             sc.err);
        __syncthreads();
    };
    if (!fast && n > 0) {
        wait_slices();
        drained();
    }
    // round trip 1: the slices' leading keys, polled (a slice may still be
    // writing its own); 1 << 32 marks an unused slot.  Key slots j >= JQ
    // belong to no slice of this list: skipped with one scalar branch each.
    const int JQ = min(KQ, (nA * kFSelL + kThreads - 1) / kThreads);
    uint64_t pv[KQ];
    if (fast) {
#pragma unroll
        for (int j = 0; j < KQ; ++j) {
            pv[j] = 1ull << 32;
            if (j < JQ) {
                const int q = tid + j * kThreads, sl = q / kFSelL, p = q - sl * kFSelL;
                if (sl < nA && sl != own && p < slice_n(sl)) pv[j] = ld_dev(lead + q);
            }
        }
    }
    if (btl) {
#pragma unroll
        for (int j = 0; j < kFSelKB; ++j)
            if (tid + j * kThreads < a.max_pages) sh.bt[tid + j * kThreads] = pre.bt[j];
    }
    if (fast) {
        // clear the LDS state while the keys are in flight
        *(int4*)&sh.uh[8 * tid] = make_int4(0, 0, 0, 0);
        *(int4*)&sh.uh[8 * tid + 4] = make_int4(0, 0, 0, 0);
        sh.selbits[tid] = 0ull;
        for (int i = tid; i < kFSelMaxN / 32; i += kThreads) sh.tiebits[i] = 0u;
        if (tid == 0) {
            sh.ncand = 0;
            sh.nr2 = 0;
            sh.needmask = 0ull;
        }
        for (unsigned it = 0;; ++it) {
            bool miss = false;
#pragma unroll
            for (int j = 0; j < KQ; ++j) miss |= pv[j] == 0ull;
            if (!__ballot(miss)) break;
            if (it >= kSpinLimit) {  // never expected: report, continue with chunk 0
                if (lane == 0) st_dev(sc.err, 1u);
#pragma unroll
                for (int j = 0; j < KQ; ++j) pv[j] = pv[j] ? pv[j] : (1ull << 32);
                break;
            }
            __builtin_amdgcn_s_sleep(8);
#pragma unroll
            for (int j = 0; j < KQ; ++j)
                if (j < JQ && pv[j] == 0ull) pv[j] = ld_dev(lead + tid + j * kThreads);
        }
#pragma unroll
        for (int j = 0; j < KQ; ++j) pv[j] -= 1ull << 32;
    }
    auto row_of = [&](int m) -> int64_t {  // element offset of chunk m's first raw row
        const int lp = chunk_page(a, m);
        const int phys = btl ? sh.bt[lp] : btrow[lp];
        return (((int64_t)phys * a.Hkv + c.g) * a.spp + (int64_t)(m - lp * a.page_chunks) * (a.C + 1)) * a.D;
    };
    const int* kept_lds = (const int*)((FSelSmem*)smem)->cidx;  // kept groups (cand), filled before the output
    auto emit = [&](int pos, int m) {
        if (meta) {
            st_dev(out + pos, (int32_t)m);
            st_dev(mo + pos, (unsigned)m + 1u);
            return;
        }
        const int ch = !cand ? m : (m < head ? kept_lds[m / a.R] * a.R + (m - (m / a.R) * a.R) : c.nm * a.R + (m - head));
        st_dev(out + pos, (int32_t)ch);
        st_dev(ro + pos, (row_of(ch) + 1) | (cand && ch >= c.nm * a.R ? (int64_t)kRowPastGroups : 0));
    };
    // the kept groups into LDS for the candidate output (no other use of cidx then)
    auto park_kept = [&]() {
        if (!cand) return;
#pragma unroll
        for (int j = 0; j < kRecMeta / kThreads; ++j) {
            const int i = tid + j * kThreads;
            if (i < c.ns1) {
                unsigned v = kept[j];
                for (unsigned it = 0; v == 0u && it < kSpinLimit; ++it) {  // written before any candidate
                    __builtin_amdgcn_s_sleep(2);                          // task could start; never expected
                    v = ld_dev(mo + i);
                }
                ((int*)((FSelSmem*)smem)->cidx)[i] = (int)v - 1;
            }
        }
        __syncthreads();
    };
    for (int i = keff + tid; i < k; i += kThreads) st_dev(out + i, (int32_t)-1);
    if (keff == 0) return fast;
    // Top-p (flat GSA, per-slice layout): the top-k selection in idl
    // (ascending list indices, keff of them, in LDS) is cut to the shortest
    // prefix of key order (larger first, ties to the lower index, NaN last)
    // whose selection probabilities -- the softmax of the keys over the
    // sequence's gists, from every slice's (max, sum of exp) pair -- reach
    // top_p; the kept entries are emitted ascending, the others get -1 and a
    // row offset that marks them skipped.
    constexpr bool kTopP = KIND == kListGists && PER == 4;
    const bool topp = kTopP && (a.flags & kFlagTopP);
    // place(tc): writes every selected entry's order key << 32 | ~list index
    // at its index in idl (ascending) into tc, from keys held in registers,
    // and says whether it did (else the keys are read back from memory)
    auto topp_emit = [&](const int* idl, auto&& place) {
        float* fred = (float*)sh.hist;     // the softmax maximum and normaliser
        uint64_t* tc = (uint64_t*)sh.uh;   // the selection: order key << 32 | ~list index
        int* trk = (int*)sh.ckey;          // their ranks in key order (in idl's place)
        float* twr = (float*)sh.cidx;      // selection weights by rank
        static_assert(2 * kRecRowOffs <= kBins && kRecRowOffs <= kFSelCand, "top-p arrays");
        constexpr int EPT = kRecRowOffs / kThreads;
        // this thread's entries of idl (each read by the thread that then
        // zeroes its rank there)
        int ids_[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) ids_[e] = EPT * tid + e < keff ? idl[EPT * tid + e] : 0;
        // the slices' pairs, each written right after its K pass (all in
        // wavefront 0: at most kTopPSlices slices)
        const uint64_t* tp = unit_topp(a, u);
        float pm = -INFINITY, pz = 0.f;
        if (tid < nA) {
            uint64_t x = ld_dev(tp + tid);
            for (unsigned it = 0; x == 0ull; ++it) {
                if (it >= kSpinLimit) {  // never expected: report, count the slice empty
                    st_dev(sc.err, 1u);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
                x = ld_dev(tp + tid);
            }
            if (x != 0ull) {
                pm = __uint_as_float((uint32_t)x);
                const float zz = __uint_as_float((uint32_t)(x >> 32));
                pz = zz > 0.f ? zz : 0.f;
            }
        }
        // the selected keys: from the threads' registers, or from memory once
        // every other slice's wavefronts have counted in (their key stores
        // have landed; this slice's own drained too)
        if (!place(tc)) {
            if (tid == 0 && nA > 1) {
                unsigned it = 0;
                while (ld_dev(unit_cntA(a, u)) < (unsigned)PER * (nA - 1)) {
                    __builtin_amdgcn_s_sleep(2);
                    if (++it >= kSpinLimit) {  // never expected: report, read the keys there are
                        st_dev(sc.err, 1u);
                        break;
                    }
                }
            }
            drain();
            __syncthreads();
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                const int i = EPT * tid + e;
                if (i < keff)
                    tc[i] = ((uint64_t)order_key(ld_dev(keys + ids_[e])) << 32) | (uint32_t)~ids_[e];
            }
        }
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            if (EPT * tid + e < keff) trk[EPT * tid + e] = 0;
        if (w == 0) {  // M: the largest key; Z: the sum of exp(key - M) over the gists
            float x = pm;
            for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
            float z = isfinite(x) && pm != -INFINITY ? pz * expf(pm - x) : 0.f;
            for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
            if (lane == 0) {
                fred[0] = x;
                fred[1] = z;
            }
        }
        lds_barrier();
        const float M = fred[0], Z = fred[1];
        const bool usable = isfinite(M);
        float kvs[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int i = EPT * tid + e;
            kvs[e] = i < keff ? order_key_value((uint32_t)(tc[i] >> 32)) : 0.f;
        }
        {
            // entry t % keff's rank (the entries before it: larger keys, or
            // equal ones of lower index: larger composites), counted by
            // threads over shares of the others (multiples of 8 entries, read
            // 16 bytes at a time, four reads in flight)
            const int reps = max(1, kThreads / keff), i0 = tid % keff, part = tid / keff;
            if (part < reps) {
                const int per = (((keff + reps - 1) / reps) + 7) & ~7;
                const int jb = min(keff, part * per), je = min(keff, jb + per);
                for (int i = i0; i < keff; i += kThreads) {
                    const uint64_t ci = tc[i];
                    auto gt = [&](unsigned lo, unsigned hi) { return ((((uint64_t)hi) << 32) | lo) > ci ? 1 : 0; };
                    int r = 0, j = jb;
                    for (; j + 8 <= je; j += 8) {
                        const uint4 q0 = *(const uint4*)&tc[j], q1 = *(const uint4*)&tc[j + 2];
                        const uint4 q2 = *(const uint4*)&tc[j + 4], q3 = *(const uint4*)&tc[j + 6];
                        r += gt(q0.x, q0.y) + gt(q0.z, q0.w) + gt(q1.x, q1.y) + gt(q1.z, q1.w) +
                             gt(q2.x, q2.y) + gt(q2.z, q2.w) + gt(q3.x, q3.y) + gt(q3.z, q3.w);
                    }
                    for (; j < je; ++j) r += tc[j] > ci ? 1 : 0;
                    atomicAdd(&trk[i], r);
                }
            }
        }
        lds_barrier();
        // the weights by rank; wavefront 0 cuts: lane l sums ranks
        // [l*per, (l+1)*per), a prefix over the lanes finds the chunk where
        // the running sum reaches the target, and that lane walks its chunk
        auto weights = [&]() {
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                const int i = EPT * tid + e;
                if (i < keff) twr[trk[i]] = (usable && !isnan(kvs[e])) ? expf(kvs[e] - M) : 0.f;
            }
        };
        auto cut = [&]() {  // (wavefront 0) the kept count, in every lane
            const int per = (keff + 63) / 64, b0 = lane * per, e0 = min(keff, b0 + per);
            float cs = 0.f;
            for (int r = b0; r < e0; ++r) cs += twr[r];
            float incl = cs;
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_up(incl, o);
                if (lane >= o) incl += y;
            }
            const float target = a.top_p * Z;
            const uint64_t hit = __ballot(usable && b0 < e0 && incl >= target);
            int need = keff;
            if (hit) {
                const int lc = __ffsll((unsigned long long)hit) - 1;
                int nl = e0;  // (rounding: the chunk's end if the walk falls short)
                float cum = incl - cs;
                for (int r = b0; r < e0; ++r) {
                    cum += twr[r];
                    if (cum >= target) {
                        nl = r + 1;
                        break;
                    }
                }
                need = __shfl(nl, lc);
            }
            return need;
        };
        // then the kept entries ascending into LDS (the weights' place) and
        // one entry per thread out, the cut ones marked skipped
        int* kept_ids = (int*)sh.cidx;
        int need;
        if (keff <= 64 * EPT) {
            // every entry is wavefront 0's: no block barrier until the output
            if (w == 0) {
                weights();
                lds_fence();
                need = cut();
                int keep = 0;
#pragma unroll
                for (int e = 0; e < EPT; ++e) keep += (EPT * tid + e < keff && trk[EPT * tid + e] < need) ? 1 : 0;
                int pos = wave_prefix_incl_dpp(keep) - keep;
                lds_fence();  // (the cut's reads of the weights are done)
#pragma unroll
                for (int e = 0; e < EPT; ++e) {
                    const int i = EPT * tid + e;
                    if (i < keff && trk[i] < need) kept_ids[pos++] = ids_[e];
                }
                if (lane == 0) sh.ncand = need;
            }
        } else {
            weights();
            lds_barrier();
            if (w == 0) {
                need = cut();
                if (lane == 0) sh.ncand = need;
            }
            lds_barrier();
            need = sh.ncand;
            int keep = 0;
#pragma unroll
            for (int e = 0; e < EPT; ++e) keep += (EPT * tid + e < keff && trk[EPT * tid + e] < need) ? 1 : 0;
            int ktot;
            int pos = block_excl_scan<kThreads>(keep, &ktot, sh.wsum);
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                const int i = EPT * tid + e;
                if (i < keff && trk[i] < need) kept_ids[pos++] = ids_[e];
            }
        }
        lds_barrier();
        need = sh.ncand;
        for (int i = tid; i < keff; i += kThreads) {
            if (i < need) {
                emit(i, kept_ids[i]);
            } else {
                st_dev(out + i, (int32_t)-1);
                st_dev(ro + i, (int64_t)kRowSkip);
            }
        }
    };
    if (keff == n) {
        park_kept();
        if constexpr (kTopP) {
            if (topp) {
                int* idl = (int*)sh.ckey;
                for (int i = tid; i < n; i += kThreads) idl[i] = i;
                lds_barrier();
                topp_emit(idl, [](uint64_t*) { return false; });
                return fast;
            }
        }
        for (int i = tid; i < n; i += kThreads) emit(i, i);
        return fast;
    }
    // bucket b0 of the keff-th largest key in the LDS histogram (whose counts
    // must be exact from that bucket up), the keys above it and in it.  Every
    // wavefront sums the 64 coarse buckets of 32 itself (lane l: coarse bucket
    // 63 - l, its 16-byte reads staggered over the banks) and scans them, then
    // the 32 buckets of the coarse one holding it: no barrier.
    int b0 = 0, above0 = 0, cnt0 = 0;
    auto find_boundary = [&]() {
        const int4* hp = (const int4*)&sh.uh[32 * (63 - lane)];
        int cv = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int4 h = hp[(i + lane) & 7];
            cv += h.x + h.y + h.z + h.w;
        }
        const int cp = wave_prefix_incl_dpp(cv);   // keys in coarse buckets >= 63 - lane
        const uint64_t reach = __ballot(cp >= keff);
        if (!reach) {  // fewer than keff keys in the histogram: every bucket counts
            b0 = 0;
            cnt0 = 0;
            above0 = 0;
            return;
        }
        const int lc = __ffsll((unsigned long long)reach) - 1;
        const int B0 = 63 - lc;
        const int abovec = __builtin_amdgcn_readlane(cp, lc) - __builtin_amdgcn_readlane(cv, lc);
        const int fv = lane < 32 ? sh.uh[32 * B0 + 31 - lane] : 0;
        const int fp = wave_prefix_incl_dpp(fv) + abovec;
        const int lf = __ffsll((unsigned long long)__ballot(lane < 32 && fp >= keff)) - 1;
        b0 = 32 * B0 + 31 - lf;
        cnt0 = __builtin_amdgcn_readlane(fv, lf);
        above0 = __builtin_amdgcn_readlane(fp, lf) - cnt0;
    };
    // one key against b0: above -> selected, in b0 -> candidate (slots taken
    // with one LDS atomic per wavefront)
    auto take = [&](uint32_t key, int id, bool valid) {
        const uint32_t bk = key >> 21;
        if (valid && bk > (uint32_t)b0)
            atomicOr((unsigned long long*)&sh.selbits[id >> 6], 1ull << (id & 63));
        const bool cand = valid && bk == (uint32_t)b0;
        const uint64_t m = __ballot(cand);
        int base = 0;
        if (lane == 0 && m) base = atomicAdd(&sh.ncand, __popcll(m));
        base = __builtin_amdgcn_readfirstlane(base);
        const int ci = base + __popcll(m & ((1ull << lane) - 1ull));
        if (cand && ci < kFSelCand) {
            sh.ckey[ci] = key;
            sh.cidx[ci] = id;
        }
    };
    // the up-front keys: one LDS atomic per wavefront reserves all their
    // candidate slots
    // up-front key j of this thread (j == KQ: its key of slice `own`)
    auto up_key = [&](int j) { return j < KQ ? pv[j] : ownk; };
    auto up_valid = [&](int j) {
        const int q = tid + j * kThreads, sl = q / kFSelL, p = q - sl * kFSelL;
        return j < KQ ? sl < nA && sl != own && p < slice_n(sl) : ownv;
    };
    auto up_used = [&](int j) { return j == KQ || j < JQ; };  // uniform
    auto take_upfront = [&]() {
        uint64_t cm[KQ + 1];
        int wtot = 0;
#pragma unroll
        for (int j = 0; j <= KQ; ++j) {
            cm[j] = 0ull;
            if (!up_used(j)) continue;
            const uint64_t x = up_key(j);
            const bool valid = up_valid(j);
            const uint32_t bk = (uint32_t)x >> 21;
            if (valid && bk > (uint32_t)b0) {
                const int id = (int)(x >> 32);
                atomicOr((unsigned long long*)&sh.selbits[id >> 6], 1ull << (id & 63));
            }
            cm[j] = __ballot(valid && bk == (uint32_t)b0);
            wtot += __popcll(cm[j]);
        }
        int base = 0;
        if (lane == 0 && wtot) base = atomicAdd(&sh.ncand, wtot);
        base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
        for (int j = 0; j <= KQ; ++j) {
            if (!up_used(j)) continue;
            const uint64_t x = up_key(j);
            const int ci = base + __popcll(cm[j] & ((1ull << lane) - 1ull));
            if (((cm[j] >> lane) & 1ull) && ci < kFSelCand) {
                sh.ckey[ci] = (uint32_t)x;
                sh.cidx[ci] = (int)(x >> 32);
            }
            base += __popcll(cm[j]);
        }
    };
    bool general = !fast;
    uint32_t rk[KR];  // this thread's share of the second round's parked keys
    int ri[KR];
    int nr2k = 0;      // how many were parked (0: no second round)
    if (fast) {
        constexpr bool kDrain = !__is_same(Drained, NoDrain);
        if (kDrain) {
            drain();  // (the polls above have waited for nearly all of it)
            __syncthreads();
        } else {
            lds_barrier();  // every thread's part of the LDS state is clear
        }
        if (kDrain) drained();
#pragma unroll
        for (int j = 0; j <= KQ; ++j)
            if (up_used(j) && up_valid(j)) atomicAdd(&sh.uh[(uint32_t)up_key(j) >> 21], 1);
        lds_barrier();
        find_boundary();  // bT: the bucket of the keff-th largest candidate
        // classify against bT; a slice whose kFSelL-th key is in a bucket >= bT
        // may hold more such keys: then a second round, and classify again
        take_upfront();
        // lanes 31 and 63 of wavefront w hold the last up-front key of slices
        // 8j + 2w and 8j + 2w + 1: one ballot per key slot, one LDS atomic
        static_assert(kThreads == 256 && kFSelL == 32, "slice of a lane");
        uint64_t wneed = 0ull;
#pragma unroll
        for (int j = 0; j < KQ; ++j) {
            if (j >= JQ) continue;
            const int q = tid + j * kThreads, sl = q / kFSelL, p = q - sl * kFSelL;
            const uint64_t bm = __ballot(p == kFSelL - 1 && sl < nA && sl != own && slice_n(sl) > kFSelL &&
                                         ((uint32_t)pv[j] >> 21) >= (uint32_t)b0);
            wneed |= (((bm >> 31) & 1ull) << (8 * j + 2 * w)) | (((bm >> 63) & 1ull) << (8 * j + 2 * w + 1));
        }
        if (lane == 0 && wneed) atomicOr((unsigned long long*)&sh.needmask, wneed);
        lds_barrier();
        const uint64_t needmask = sh.needmask;
        if (needmask) {
            // round trip 2: the keys of buckets >= bT past kFSelL of those
            // slices join the histogram and are parked in the candidate arrays
            const uint32_t bT = (uint32_t)b0;
            sh.selbits[tid] = 0ull;
            if (tid == 0) sh.ncand = 0;
            wait_slices();
            const int nneed = __popcll(needmask);
            constexpr int R = kFusedTA - kFSelL;  // keys past kFSelL per slice
            for (int q0 = 0; q0 < nneed * R; q0 += kThreads) {
                const int q = q0 + tid, i = q / R, p = kFSelL + (q - i * R);
                int sl = 0;
                if (q < nneed * R) {
                    uint64_t m = needmask;
                    for (int t = 0; t < i; ++t) m &= m - 1ull;
                    sl = __ffsll((unsigned long long)m) - 1;
                }
                const bool ok = q < nneed * R && p < slice_n(sl);
                const uint64_t pr = ok ? ld_dev(pairs + (size_t)sl * kFusedTA + p) : 0ull;
                const bool keep = ok && ((uint32_t)pr >> 21) >= bT;
                const uint64_t km = __ballot(keep);
                int base = 0;
                if (lane == 0 && km) base = atomicAdd(&sh.nr2, __popcll(km));
                base = __builtin_amdgcn_readfirstlane(base);
                const int at = base + __popcll(km & ((1ull << lane) - 1ull));
                if (keep) {
                    atomicAdd(&sh.uh[(uint32_t)pr >> 21], 1);
                    if (at < kFSelCand) {
                        sh.ckey[at] = (uint32_t)pr;
                        sh.cidx[at] = (int)(pr >> 32);
                    }
                }
            }
            __syncthreads();
            find_boundary();  // exact from bT up: b0
            const int nr2 = sh.nr2;
            nr2k = nr2 <= kFSelCand ? nr2 : 0;
            if (nr2 > kFSelCand) {
                general = true;
            } else {
#pragma unroll
                for (int j = 0; j < KR; ++j) {
                    const int q = tid + j * kThreads;
                    rk[j] = q < nr2 ? sh.ckey[q] : 0u;
                    ri[j] = q < nr2 ? sh.cidx[q] : 0;
                }
                __syncthreads();  // the candidate arrays are free
                take_upfront();
#pragma unroll
                for (int j = 0; j < KR; ++j) take(rk[j], ri[j], tid + j * kThreads < nr2);
                __syncthreads();
            }
        }
        general = general || cnt0 > kFSelCand;
    }
    if (general) {
        // wide boundary bucket, long list or many slices: select over the keys
        if (fast && !sh.needmask) wait_slices();  // (else done above)
        __syncthreads();
        btl = false;  // the select reuses the LDS
        SelectSmem<kThreads>& ssh = *(SelectSmem<kThreads>*)smem;
        block_topk_general<kThreads>(keys, nullptr, n, k, out, true, ssh);
        drain();
        __syncthreads();
        int mi[kRecRowOffs / kThreads];  // this thread's list indices (keff <= kRecRowOffs)
#pragma unroll
        for (int j = 0; j < kRecRowOffs / kThreads; ++j) {
            const int i = tid + j * kThreads;
            mi[j] = i < keff ? ld_dev(out + i) : 0;
        }
        __syncthreads();  // the LDS is the select's no more
        park_kept();
        if constexpr (kTopP) {
            if (topp) {
                int* idl = (int*)sh.ckey;
#pragma unroll
                for (int j = 0; j < kRecRowOffs / kThreads; ++j)
                    if (tid + j * kThreads < keff) idl[tid + j * kThreads] = mi[j];
                lds_barrier();
                topp_emit(idl, [](uint64_t*) { return false; });
                return fast;
            }
        }
#pragma unroll
        for (int j = 0; j < kRecRowOffs / kThreads; ++j)
            if (tid + j * kThreads < keff) emit(tid + j * kThreads, mi[j]);
        return fast;
    }
    int* ids = (int*)sh.ckey;  // the selection, ascending (written by wavefront 0)
    static_assert(kRecRowOffs <= kFSelCand, "the selection fits the candidate arrays");
    static_assert(kRecMeta <= kFSelCand && kRecMeta % kThreads == 0, "the kept groups fit the candidate ids");
    if (w == 0) {
        // wavefront 0: radix passes over the candidates' bits [20:14], [13:7], [6:0]
        int above = above0;
        uint32_t prefix = (uint32_t)b0 << 21;
        int fixed = 11;
        bool take_all = above + cnt0 == keff;
        for (int pass = 0; pass < 3 && !take_all; ++pass) {
            const int shift = 14 - 7 * pass;
            sh.hist[lane] = 0;
            sh.hist[lane + 64] = 0;
            lds_fence();
            for (int ci = lane; ci < cnt0; ci += 64) {
                const uint32_t x = sh.ckey[ci];
                if ((x >> (32 - fixed)) == (prefix >> (32 - fixed))) atomicAdd(&sh.hist[(x >> shift) & 127u], 1);
            }
            lds_fence();
            const int h0 = sh.hist[2 * lane], h1 = sh.hist[2 * lane + 1];
            const int s2 = h0 + h1;
            const int pi = wave_prefix_incl_dpp(s2);
            const int higher = __builtin_amdgcn_readlane(pi, 63) - pi;  // keys in higher digit pairs
            const int need = keff - above;
            const bool mine = higher < need && higher + s2 >= need;
            int bsel = 0, abv = 0, cn = 0;
            if (mine) {
                if (higher + h1 >= need) {
                    bsel = 2 * lane + 1;
                    abv = higher;
                    cn = h1;
                } else {
                    bsel = 2 * lane;
                    abv = higher + h1;
                    cn = h0;
                }
            }
            const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
            bsel = __builtin_amdgcn_readlane(bsel, src);
            abv = __builtin_amdgcn_readlane(abv, src);
            cn = __builtin_amdgcn_readlane(cn, src);
            above += abv;
            prefix |= (uint32_t)bsel << shift;
            fixed += 7;
            if (above + cn == keff) take_all = true;
        }
        const uint32_t lo = prefix;
        const uint32_t hi = fixed >= 32 ? prefix : (prefix | ((1u << (32 - fixed)) - 1u));
        for (int ci = lane; ci < cnt0; ci += 64) {
            const uint32_t x = sh.ckey[ci];
            const int id = sh.cidx[ci];
            if (x > hi || (take_all && x >= lo))
                atomicOr((unsigned long long*)&sh.selbits[id >> 6], 1ull << (id & 63));
            else if (x >= lo)
                atomicOr(&sh.tiebits[id >> 5], 1u << (id & 31));
        }
        lds_fence();
        if (!take_all) {
            const int nw = (n + 31) / 32;
            // the (keff - above) lowest-index keys equal to the k-th largest
            const int need_eq = keff - above;
            uint32_t tb[WPL];
            int c1 = 0;
#pragma unroll
            for (int i = 0; i < WPL; ++i) {
                const int wd = WPL * lane + i;
                tb[i] = wd < nw ? sh.tiebits[wd] : 0u;
                c1 += __popc(tb[i]);
            }
            int before = wave_prefix_incl_dpp(c1) - c1;
#pragma unroll
            for (int i = 0; i < WPL; ++i) {
                uint32_t add = 0u, rest = tb[i];
                while (rest && before < need_eq) {
                    const uint32_t bit = rest & (~rest + 1u);
                    add |= bit;
                    rest ^= bit;
                    ++before;
                }
                const int wd = WPL * lane + i;
                if (add) atomicOr((unsigned long long*)&sh.selbits[wd >> 1], (uint64_t)add << (32 * (wd & 1)));
            }
            lds_fence();
        }
        // the selection in ascending order: a popcount scan over the bitmap
        // (the candidate arrays are free now)
        constexpr int WL = kFSelMaxN / 64 / 64;  // 64-bit bitmap words per lane
        const int nw64 = (n + 63) / 64;
        uint64_t sb[WL];
        int c2 = 0;
#pragma unroll
        for (int i = 0; i < WL; ++i) {
            const int wd = WL * lane + i;
            sb[i] = wd < nw64 ? sh.selbits[wd] : 0ull;
            c2 += __popcll(sb[i]);
        }
        int pos = wave_prefix_incl_dpp(c2) - c2;
        int* wpre = (int*)sh.tiebits;  // (top-p) selected ids before each bitmap word
#pragma unroll
        for (int i = 0; i < WL; ++i) {
            uint64_t x = sb[i];
            if (kTopP && topp) wpre[WL * lane + i] = pos;
            while (x) {
                const int bit = __ffsll((unsigned long long)x) - 1;
                x &= x - 1ull;
                ids[pos++] = (WL * lane + i) * 64 + bit;
            }
        }
    }  // wavefront 0
    lds_barrier();
    park_kept();
    if constexpr (kTopP) {
        if (topp) {
            // every selected entry is a candidate some thread holds (up front,
            // of its own slice, or parked in the second round); its index in
            // ids: the selected ids before its bitmap word and below it there
            topp_emit(ids, [&](uint64_t* tc) {
                const int* wpre = (const int*)sh.tiebits;
                auto put = [&](uint32_t key, int id) {
                    const uint64_t wb = sh.selbits[id >> 6], bit = 1ull << (id & 63);
                    if (wb & bit)
                        tc[wpre[id >> 6] + __popcll(wb & (bit - 1ull))] = ((uint64_t)key << 32) | (uint32_t)~id;
                };
#pragma unroll
                for (int j = 0; j <= KQ; ++j)
                    if (up_used(j) && up_valid(j)) put((uint32_t)up_key(j), (int)(up_key(j) >> 32));
#pragma unroll
                for (int j = 0; j < KR; ++j)
                    if (tid + j * kThreads < nr2k) put(rk[j], ri[j]);
                return true;
            });
            return fast;
        }
    }
    for (int i = tid; i < keff; i += kThreads) emit(i, ids[i]);
    return fast;
}

// One slice (TA rows) of a scored list of unit u: the gists (flat GSA), the
// meta-gists or the candidate gists (H-GSA).  Scores the rows (routing keys),
// attends them when the set needs them (all gists, all meta-gists), publishes
// the keys sorted by bucket and its partial.  The list's last slice runs the
// list's select as soon as its partial is written: it counts the partial in
// at the select's first barrier, once its stores have completed anyway.
template <int D, int EJ, int KIND>
__device__ __forceinline__ void task_slices(const Args& a, const Sched& s, int u, int idx,
                                            unsigned char* smem, CombineSmem& cs, int* wsum) {
    constexpr int kind = KIND;
    // 32-token blocks per wavefront: rows per task / 128 (H-GSA's lists: 1)
    constexpr int NBW = (KIND == kListMeta || KIND == kListCand ? kFusedTAH : kFusedTA) / 128;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int G = a.G, C = a.C;
    const int b = u / a.Hkv, g = u - b * a.Hkv;
    const int p0 = idx * s.TA;
    constexpr bool meta = kind == kListMeta, cand = kind == kListCand;
    auto row_p = [&](int j, int t) { return p0 + 32 * (w + 4 * j) + 16 * t + lr; };
    // gist rows of the flat list: block-table lookups issued with the length load
    size_t off[NBW][2];
    if (kind == kListGists) {
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int p = min(row_p(j, t), a.num_chunks - 1);
                off[j][t] = slot_offset(a, b, g, max(p, 0) * (C + 1) + C);
            }
    }
    ListCtx c;
    make_ctx(a, kind, u, kind != kListGists, c);
    const int n = c.len;
    const int nA = max(1, (n + s.TA - 1) / s.TA);
    if (idx >= nA) return;
    const int cnt = max(0, min(s.TA, n - p0));
    if (meta) {
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int p = max(min(row_p(j, t), n - 1), 0);
                off[j][t] = (((size_t)b * a.Hkv + g) * a.max_meta + p) * (size_t)D;
            }
    } else if (cand && cnt > 0) {
        // the gists of the kept meta-groups (the meta select's entries in the
        // unit's record, polled), then the gists past the last complete group.
        // The sequence's block-table row goes into the (unused) V-tile LDS while
        // the meta select runs, so the page lookups cost no round trip after it.
        const bool btc = a.max_pages <= Lds::stash(D) / 4;
        int* bl = (int*)smem;
        if (btc) {
            const int32_t* btrow = a.bt + (size_t)b * a.max_pages;
            for (int e0 = 64 * w; e0 < a.max_pages; e0 += 64 * 4) {
                // lane l writes entry e0 + l (a lane past the row rereads its last entry)
                const int e = min(e0 + lane, a.max_pages - 1);
                __builtin_amdgcn_global_load_lds(btrow + e, (lds_void_t*)(smem + 4 * e0), 4, 0, 0);
            }
        }
        const unsigned* mo = unit_meta(a, u);
        const int head = c.ns1 * a.R;
        unsigned grp[NBW][2];
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int p = min(row_p(j, t), n - 1);
                grp[j][t] = p < head ? ld_dev(mo + p / a.R) : 1u;
            }
        for (unsigned it = 0;; ++it) {
            bool miss = false;
#pragma unroll
            for (int j = 0; j < NBW; ++j) miss |= grp[j][0] == 0u || grp[j][1] == 0u;
            if (!__ballot(miss)) break;
            if (it >= kSpinLimit) {  // never expected: report, read group 0
                if (lane == 0) st_dev(s.err, 1u);
#pragma unroll
                for (int j = 0; j < NBW; ++j)
#pragma unroll
                    for (int t = 0; t < 2; ++t) grp[j][t] = grp[j][t] ? grp[j][t] : 1u;
                break;
            }
            __builtin_amdgcn_s_sleep(8);
#pragma unroll
            for (int j = 0; j < NBW; ++j)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    if (grp[j][t] == 0u) grp[j][t] = ld_dev(mo + min(row_p(j, t), n - 1) / a.R);
        }
        if (btc) {  // every wavefront's row entries are in LDS
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int p = min(row_p(j, t), n - 1);
                const int r = p / a.R;
                const int gist = p < head ? (int)(grp[j][t] - 1u) * a.R + (p - r * a.R) : c.nm * a.R + (p - head);
                const int sl = gist * (C + 1) + C, lp = sl / a.spp;
                const int phys = btc ? bl[lp] : a.bt[(size_t)b * a.max_pages + lp];
                off[j][t] = (((size_t)phys * a.Hkv + g) * a.spp + (sl - lp * a.spp)) * (size_t)D;
            }
    }
    const bool attn = meta || (kind == kListGists && !(a.flags & kFlagSelectedGists));
    const bool selector = idx == nA - 1;
    SelPre pre;  // the selecting slice's block-table row
    bool prefetched = false;
    uint64_t ownk = 0;  // the selecting slice's key of this thread (not bucket sorted)
    bool ownv = false;
    float* keys = meta ? a.mkeys + (size_t)u * a.max_meta
                : cand ? a.ckeys + (size_t)u * a.cand_stride : a.keys + (size_t)u * a.key_stride;
    WaveAttnL<D> wa;
    unsigned char* tile = smem + (size_t)w * WaveAttnL<D>::TILE_BYTES;
    bf16x8_t mP[NBW];  // meta slices: the K pass's probabilities (the PV operand)
    int nbw = 0;
    // this slice's partial (its wavefronts' states combined; stores in flight)
    auto publish = [&]() {
        const size_t pbase = ((size_t)u * a.NS + idx) * G;
        combine_waves<D>(
            wa, a.tau_log2e, G, (float*)smem, cs,
            [&](int h, int d, float v) { st_dev(a.part_acc + (pbase + h) * D + d, v); },
            [&](int h, float m2, float l) {
                float* p = (float*)(a.part_ml + pbase + h);
                st_dev(p, m2);
                st_dev(p + 1, l);
            });
    };

    if (cnt > 0) {
        int nval[NBW];
        const int nblk = (cnt + 31) / 32;
        nbw = nblk > w ? (nblk - w + 3) / 4 : 0;
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            nval[j] = max(0, min(32, cnt - 32 * (w + 4 * j)));
            // a token past the end reads the block's first row (in range)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                if (16 * t + lr >= nval[j]) off[j][t] = __shfl(off[j][0], lane & 48);
        }
        wa.init((const __bf16*)a.q + ((size_t)c.b * a.Hq + (size_t)c.g * G) * D, G, lr, lg);
        float* stash = (float*)(smem + Lds::stash(D)) + 64 * w;
        const float tau = a.tau;
        auto on_scores = [&](int j, const f32x4_t sc[2]) {
            // routing keys: tau * sum over the group's heads (padding heads are 0)
            float kv = 0.f;
            int kt = -1;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float x = rowsum16(sc[t][r]);
                    if (4 * t + r == lr) {
                        kv = x * tau;
                        kt = 16 * t + 4 * lg + r;
                    }
                }
            // park the key in LDS (no global store here: a store in
            // flight would hold up the next wait on this wavefront's loads)
            if (kt >= 0 && kt < nval[j]) stash[32 * j + kt] = kv;
        };
        if (meta) {
            // meta slices: K rows first, keys out, then the V rows (every
            // slice's K loads go ahead of any V load, so the meta select,
            // which waits for all of a unit's keys, starts about half a
            // stream earlier)
            wa.template kpass<NBW>((const __bf16*)a.km, off, nval, nbw, a.tau_log2e, lg, mP, on_scores);
        } else {
            wa.template stream<NBW>((const __bf16*)a.kc, (const __bf16*)a.vc, off, nval, nbw, attn,
                                    a.tau_log2e, lr, lg, tile, on_scores);
        }
        if (selector) {
            select_prefetch<KIND>(a, c, n, nA, pre);
            prefetched = true;
        }
        // thread t takes key slot t % 64 of wavefront t / 64 (slots past NBW * 32
        // hold no row: kpos >= cnt there)
        static_assert(NBW * 32 * 4 <= kThreads, "one key slot per thread");
        lds_barrier();
        const int ws = threadIdx.x >> 6, slot = threadIdx.x & 63;
        const int kpos = 32 * (ws + 4 * (slot >> 5)) + (slot & 31);
        const float kv = kpos < cnt ? ((const float*)(smem + Lds::stash(D)))[64 * ws + slot] : 0.f;
        if (kpos < cnt) st_dev(keys + p0 + kpos, kv);
        lds_barrier();  // the tiles are free (the key stores need not have landed)
        uint64_t* pairs = cand ? a.spairs_c + ((size_t)u * s.S3 + idx) * kFusedTA
                               : a.spairs + ((size_t)u * s.S1 + idx) * kFusedTA;
        uint64_t* lead = nA > kRecSlices ? nullptr : (cand ? unit_lead_c(a, u) : unit_lead(a, u)) + idx * kFSelL;
        if (!selector) {
            bucket_slice(pairs, lead, p0, kv, kpos < cnt ? kpos : -1, smem, wsum);
            // (the bucket sort's LDS is free: its last barrier)
            if (meta) wa.template vpass<NBW>((const __bf16*)a.vm, off, nbw, mP, tile, []() {});
        } else {  // the select takes this slice's keys as they are
            ownk = (uint64_t)order_key(kv) | ((uint64_t)(uint32_t)(p0 + kpos) << 32);
            ownv = kpos < cnt;
        }
        // (a meta selector's V rows and partial follow its select)
        if (attn && !(meta && selector)) publish();
    }
    if (!selector) {
        drain();
        __syncthreads();
        if (threadIdx.x == 0) add_dev(cand ? unit_cntC(a, u) : unit_cntA(a, u), 1u);
        return;
    }

    // select and publish (ahead of the streaming workgroups sharing this CU:
    // everything of the unit waits for it); the other slices' leading keys
    // are polled
    __builtin_amdgcn_s_setprio(2);
    if (kind == kListGists)
        for (int i = c.n + threadIdx.x; i < a.num_chunks; i += kThreads) keys[i] = -INFINITY;
    // the partial's count (cntP): by thread 0 once every wavefront has
    // drained, at the select's first barrier (the unfolded task that folds
    // this partial waits for it)
    const bool partial = attn && cnt > 0;
    bool counted = false;
    auto count_partial = [&]() {
        if (partial && threadIdx.x == 0) add_dev(unit_cntP(a, u), 1u);
        counted = true;
    };
    if (!prefetched) select_prefetch<KIND>(a, c, n, nA, pre);
    if (meta)  // its partial is not made yet
        select_fused<KIND>(a, s, c, n, nA, keys, smem, pre, idx, ownk, ownv, NoDrain{});
    else
        select_fused<KIND>(a, s, c, n, nA, keys, smem, pre, idx, ownk, ownv, count_partial);
    // return the leading keys in the record to zero: each has been read by the
    // select, or every slice is done (the select waited for it)
    if (nA <= kRecSlices) {
        uint64_t* lead = cand ? unit_lead_c(a, u) : unit_lead(a, u);
        for (int i = threadIdx.x; i < nA * kFSelL; i += kThreads) {
            const int sl = i / kFSelL;
            if (i - sl * kFSelL < min(s.TA, n - sl * s.TA)) st_dev(lead + i, 0ull);
        }
    }
    if (meta && partial) {
        // the V rows after the select (only the K pass's probabilities,
        // running maximum and sum were live across it: O is still zero)
        __builtin_amdgcn_s_setprio(0);
        lds_barrier();  // the select's LDS is free for the V tiles
#pragma unroll
        for (int db = 0; db < WaveAttnL<D>::DB; ++db) wa.o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        wa.template vpass<NBW>((const __bf16*)a.vm, off, nbw, mP, tile, []() {});
        publish();
    }
    // the record entries this select wrote or cleared are in place: the
    // unit's merging task resets the record only after every select says so
    drain();
    __syncthreads();
    if (!counted) count_partial();
    if (threadIdx.x == 0) add_dev(unit_cntS(a, u), 1u);
}

// Combine the 4 wavefronts' online-softmax states with the folded gist state
// (fh.m / fh.l, gacc) and publish the result as partial slot `slot` of unit u,
// or (LOCAL) leave it in (gacc, fh.m, fh.l) for a fold to continue from.  The
// partial's stores may still be in flight on return: a caller drains before
// counting it in.
template <int D, int EJ, bool LOCAL, typename WA>
__device__ __forceinline__ void combine_publish(WA& wa, const Args& a, int u, int slot, float (&gacc)[EJ],
                                FoldHdr& fh, float* red, CombineSmem& cs) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int G = a.G, GD = a.G * D;
    const float tl = a.tau_log2e;
    float l = wa.l;
    l = rows4_sum(l);
    if (lg == 0) {
        cs.wm[w][lr] = wa.m;
        cs.wl[w][lr] = l;
    }
    lds_barrier();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = 4 * lg + r;
        const float M = fmaxf(fmaxf(cs.wm[0][h], cs.wm[1][h]), fmaxf(cs.wm[2][h], cs.wm[3][h]));
        const float sc = (cs.wm[w][h] == -INFINITY) ? 0.f : exp2f((cs.wm[w][h] - M) * tl);
        if (h < G) {
#pragma unroll
            for (int db = 0; db < WA::DB; ++db)
                red[((size_t)w * G + h) * D + 16 * db + lr] = wa.o[db][r] * sc;
        }
    }
    const size_t pbase = ((size_t)u * a.NS + slot) * G;
    if (threadIdx.x < (unsigned)G) {
        const int h = threadIdx.x;
        const float M = fmaxf(fmaxf(cs.wm[0][h], cs.wm[1][h]), fmaxf(cs.wm[2][h], cs.wm[3][h]));
        float Lb = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (cs.wm[i][h] != -INFINITY) Lb += cs.wl[i][h] * exp2f((cs.wm[i][h] - M) * tl);
        const float mb = M == -INFINITY ? -INFINITY : M * tl;
        const float Mt = fmaxf(fh.m[h], mb);
        const float fg = fh.m[h] == -INFINITY ? 0.f : exp2f(fh.m[h] - Mt);
        const float fb = mb == -INFINITY ? 0.f : exp2f(mb - Mt);
        fh.fg[h] = fg;
        fh.fb[h] = fb;
        const float L = fh.l[h] * fg + Lb * fb;
        if (LOCAL) {
            fh.m[h] = Mt;
            fh.l[h] = L;
        } else {
            float* p = (float*)(a.part_ml + pbase + h);
            st_dev(p, Mt);
            st_dev(p + 1, L);
        }
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < EJ; ++j) {
        const int e = threadIdx.x + j * kThreads;
        if (e < GD) {
            const int h = e / D, d = e - h * D;
            const float bs = red[(size_t)h * D + d] + red[((size_t)G + h) * D + d] +
                             red[((size_t)2 * G + h) * D + d] + red[((size_t)3 * G + h) * D + d];
            const float v = gacc[j] * fh.fg[h] + bs * fh.fb[h];
            if (LOCAL)
                gacc[j] = v;
            else
                st_dev(a.part_acc + pbase * D + e, v);
        }
    }
}

// EJ: accumulator elements per thread, EJ * kThreads >= G * D.
template <int D, int EJ, bool HIER, int NBB>
__device__ __forceinline__ void task_unfolded(const Args& a, const Sched& s, int u, int idx, unsigned char* smem,
                              CombineSmem& cs, FoldHdr& fh, int* s_flag) {
    const int G = a.G, C = a.C;
    constexpr bool hier = HIER;
    // the list: raw tokens of the selected chunks, the raw tail, then (H-GSA)
    // the gists past the last complete meta-group and one entry per selected
    // chunk for its gist, attended only when the chunk lies in a complete
    // group (those come first: the selection is ascending), or (flat GSA,
    // selected-gists set) the selected gists
    ListCtx c;
    make_ctx(a, hier ? kListMeta : kListUnfolded, u, hier, c);
    const int ninc = hier ? c.n - c.nm * a.R : 0;
    const int len = hier ? c.ns * C + c.tail + ninc + c.ns : c.len;
    const int nB = max(1, (len + s.TB - 1) / s.TB);
    if (idx >= nB) return;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int p0 = idx * s.TB;
    const int cnt = max(0, min(s.TB, len - p0));
    const int raw = c.ns * C;
    // first raw-tail row (the tail lies in one page): known before the selection
    const int64_t tail_off = c.tail > 0 ? (int64_t)slot_offset(a, c.b, c.g, c.n * (C + 1)) : 0;
    // fold the partials of the sliced list (gists, or meta-gists) idx, idx + nB,
    // ... once every slice is done
    const bool attn = hier || !(a.flags & kFlagSelectedGists);
    const int n1 = hier ? c.nm : c.n;                  // rows of the sliced list
    const int nAt = max(1, (n1 + s.TA - 1) / s.TA);   // its slice tasks
    const int nA = attn ? (n1 + s.TA - 1) / s.TA : 0;  // slices that wrote a partial
    const int nf = idx < nA ? (nA - idx + nB - 1) / nB : 0;
    // the list's last slice (the selecting one) counts its partial in apart
    // from the others
    const bool owner = nA > 0 && (nA - 1) % nB == idx;
    float gacc[EJ];
#pragma unroll
    for (int j = 0; j < EJ; ++j) gacc[j] = 0.f;
    if (threadIdx.x < 16) {
        fh.m[threadIdx.x] = -INFINITY;
        fh.l[threadIdx.x] = 0.f;
    }
    if (nf > 0) {
        wait_at_least_close<32>(unit_cntA(a, u), (unsigned)(nAt - 1), s.err);
        if (owner) wait_at_least<8>(unit_cntP(a, u), 1u, s.err);
        __syncthreads();
        fold_regs<EJ>(a, u, idx, nB, nf, gacc, fh);
    }
    __builtin_amdgcn_s_setprio(1);  // the unit's result waits for this task
    WaveAttnL<D> wa;
    wa.init((const __bf16*)a.q + ((size_t)c.b * a.Hq + (size_t)c.g * G) * D, G, lr, lg);
    if (cnt > 0) {
        // each token row: the raw tail (known), or a row of a selected chunk,
        // whose offset the wavefront polls in the unit's record until the
        // select has written it (one plus the offset; 0 before)
        const int64_t* ro = unit_rowoff(a, u);
        // NBB 32-token blocks per wavefront (tasks of 128 NBB tokens): block j
        // of wavefront w is the task's block w + 4j
        constexpr int nbb = NBB;
        size_t off[NBB][2];
        int nval[NBB];
        int jr[NBB][2];      // selection entry of the row, -1 for a known row
        int64_t o[NBB][2];   // one plus the base offset (H-GSA: past-groups flag), 0 while unknown
        int64_t add[NBB][2]; // offset of the row from that base
        bool gsec[NBB][2];   // the row is a selected chunk's gist
#pragma unroll
        for (int j = 0; j < NBB; ++j)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                // a token past the end reads the task's first row (in range)
                const int rel = 32 * (w + 4 * j) + 16 * t + lr;
                const int p = p0 + (rel < cnt ? rel : 0);
                gsec[j][t] = false;
                jr[j][t] = -1;
                add[j][t] = 0;
                o[j][t] = 1;
                if (j >= nbb) continue;
                if (p < raw) {
                    jr[j][t] = p / C;
                    add[j][t] = (int64_t)(p - jr[j][t] * C) * D;
                } else if (p < raw + c.tail) {
                    o[j][t] = tail_off + (int64_t)(p - raw) * D + 1;
                } else if (p < raw + c.tail + ninc) {
                    const int m = c.nm * a.R + (p - raw - c.tail);
                    o[j][t] = (int64_t)slot_offset(a, c.b, c.g, m * (C + 1) + C) + 1;
                } else {
                    jr[j][t] = p - raw - c.tail - ninc;
                    add[j][t] = (int64_t)C * D;
                    gsec[j][t] = true;
                }
                if (jr[j][t] >= 0) o[j][t] = ld_dev(ro + jr[j][t]);
            }
        for (unsigned it = 0;; ++it) {
            bool miss = false;
#pragma unroll
            for (int j = 0; j < NBB; ++j) miss |= o[j][0] == 0 || o[j][1] == 0;
            if (!__ballot(miss)) break;
            if (it >= kSpinLimit) {  // never expected: report, read a row in range
                if (lane == 0) st_dev(s.err, 1u);
#pragma unroll
                for (int j = 0; j < NBB; ++j)
#pragma unroll
                    for (int t = 0; t < 2; ++t) o[j][t] = o[j][t] == 0 ? 1 : o[j][t];
                break;
            }
            __builtin_amdgcn_s_sleep(8);
#pragma unroll
            for (int j = 0; j < NBB; ++j)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    if (o[j][t] == 0) o[j][t] = ld_dev(ro + jr[j][t]);
        }
        // rows a block attends: before the end, and (H-GSA) a selected
        // chunk's gist only inside a complete group; they form a prefix of
        // the task's list, so a block's count is its length and a wavefront's
        // blocks with rows come first
        int nbw = 0;
#pragma unroll
        for (int j = 0; j < NBB; ++j) {
            int nv = 0;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const bool valid = j < nbb && 32 * (w + 4 * j) + 16 * t + lr < cnt &&
                                   !(gsec[j][t] && (o[j][t] & (int64_t)kRowPastGroups));
                nv += __popcll(__ballot(valid && lg == 0));
                off[j][t] = (size_t)((o[j][t] & ~(int64_t)kRowPastGroups) - 1 + add[j][t]);
            }
            nval[j] = nv;
            nbw += nv > 0 ? 1 : 0;
        }
        unsigned char* tile = smem + (size_t)w * WaveAttnL<D>::TILE_BYTES;
        wa.template stream<NBB>((const __bf16*)a.kc, (const __bf16*)a.vc, off, nval, nbw, true, a.tau_log2e,
                                lr, lg, tile,
                              [](int, const f32x4_t*) {});
    }
    __syncthreads();
    // the unit's last unfolded task (the last one dispatched) merges; the
    // others publish their partials and count themselves in
    if (idx != nB - 1) {
        combine_publish<D, EJ, false>(wa, a, u, s.S1 + idx, gacc, fh, (float*)smem, cs);
        drain();
        __syncthreads();
        if (threadIdx.x == 0) add_dev(unit_cntB(a, u), 1u);
        return;
    }

    // merge: this task's own partial stays in registers, the others' are
    // folded into it; then write the output and return the unit's record to
    // zero.  The reset needs every slice, candidate task and select counted
    // in: read the counts now, the fold hides the round trip.
    combine_publish<D, EJ, true>(wa, a, u, s.S1 + idx, gacc, fh, (float*)smem, cs);
    unsigned seen[3] = {0u, 0u, 0u};
    if (threadIdx.x == 0) {
        seen[0] = ld_dev(unit_cntA(a, u));
        seen[1] = ld_dev(unit_cntS(a, u));
        if (hier) seen[2] = ld_dev(unit_cntC(a, u));
        wait_at_least<8>(unit_cntB(a, u), (unsigned)(nB - 1), s.err);
    }
    __syncthreads();
    fold_regs<EJ>(a, u, s.S1, 1, nB - 1, gacc, fh);
    // the counts are compared only here: without this the compares move up
    // to the loads and the fold's loads wait for their round trip
    asm volatile("" : "+v"(seen[0]), "+v"(seen[1]), "+v"(seen[2])::"memory");
    __bf16* out = (__bf16*)a.out + ((size_t)c.b * a.Hq + (size_t)c.g * G) * D;
#pragma unroll
    for (int j = 0; j < EJ; ++j) {
        const int e = threadIdx.x + j * kThreads;
        if (e < G * D) {
            const int h = e / D;
            const float L = fh.l[h];
            out[e] = (__bf16)((fh.m[h] == -INFINITY || L == 0.f) ? 0.f : gacc[j] / L);
        }
    }
    // every unfolded task has read the selection; wait until every slice and
    // candidate task has counted in and every select has finished writing the
    // record (long done in practice: nothing else orders them before this
    // point when the selection is empty), then return the record to zero
    if (threadIdx.x == 0) {
        // (the selecting slice's partial count is in: its folding task saw it)
        if (seen[0] < (unsigned)(nAt - 1)) wait_at_least<8>(unit_cntA(a, u), (unsigned)(nAt - 1), s.err);
        if (seen[1] < (hier ? 2u : 1u)) wait_at_least<8>(unit_cntS(a, u), hier ? 2u : 1u, s.err);
        if (hier) {
            const unsigned nCt = (unsigned)max(1, (c.ns1 * a.R + ninc + s.TA - 1) / s.TA);
            if (seen[2] < nCt - 1) wait_at_least<8>(unit_cntC(a, u), nCt - 1, s.err);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < c.ns; i += kThreads) st_dev(unit_rowoff(a, u) + i, (int64_t)0);
    if (hier)
        for (int i = threadIdx.x; i < c.ns1; i += kThreads) st_dev(unit_meta(a, u) + i, 0u);
    if (threadIdx.x == 0) {
        st_dev(unit_cntA(a, u), 0u);
        st_dev(unit_cntB(a, u), 0u);
        st_dev(unit_cntS(a, u), 0u);
        st_dev(unit_cntP(a, u), 0u);
        if (hier) st_dev(unit_cntC(a, u), 0u);
    }
}

// Flat GSA: task idx of unit u, S = s.S1 tasks per unit.  Tasks idx < nA own
// a slice of 256 gists each; the last of them, nA - 1, is the unit's selector;
// every other task is an unfolded worker.
//   slice     K pass over its gists (routing keys; with the all-gists set also
//             the blocks' softmax probabilities against their maximum), keys
//             out and -- but for the selector -- bucket-sorted and published;
//             then its V pass, each wavefront counting in (cntA) once its
//             stores have landed (only the select's slower paths read cntA).
//   selector  keeps its slice's keys in registers and runs the top-k select
//             over the slices' sorted keys as soon as they are published
//             (select_fused), which writes the selection and each selected
//             chunk's first-row offset into the unit's record; then its V pass
//             and partial, and the merge.
//   workers   after their V pass (if any), 32-row blocks of the unfolded list
//             (raw tokens of the selected chunks, raw tail, selected gists of
//             the selected-gists set): block jb goes to worker wave jb mod 4W
//             (W = S - 1 workers), spread over the tasks first.  A worker polls
//             its blocks' row offsets (written by the select, in practice
//             while the V passes stream), attends them into the same
//             online-softmax state and publishes one partial (slot idx).
//   merge     every task publishes its partial (slot idx) and counts in
//             (cntB); the last R to count in (R = min(4, EJ)) each fold one
//             R-th of the output's elements from all S partials in slot order
//             (merge_part) once the count is full, and the last of them to
//             finish (cntP) returns the unit's record to zero.
// Waits go one way within a unit (the select waits for its slices' keys, the
// workers for the select, the mergers for the last task to count in), and
// only within it.  Tasks are numbered unit by
// unit and each XCD dispatches its workgroups in id order, so on every XCD the
// smallest unfinished unit's tasks come before any later unit's: slots held by
// earlier units free up as those finish, all of its tasks become resident
// together (a unit's tasks are far fewer than an XCD's slots) and it
// finishes; by induction every unit does.

// Merge the elements j = jr + R k (k < JS) of unit u's G x D output (element
// threadIdx.x + j * kThreads) from all S partials, in slot order, and write
// them to out; every partial is in memory.  A wavefront's elements of one j
// belong to one head (D is a multiple of 64): lane i takes slot i's (max, sum)
// of that head, wavefront reductions give the common max and the sum, and the
// slots' factors reach every lane by readlane -- no LDS and no barrier between
// the (max, sum) loads and the accumulator loads, which go out together.
// Slots in groups of 64, each rescaled to the running maximum; within a group
// NB slots' loads are in flight while the NB before are folded.  The order
// (hence every bit of the output) does not depend on which task merges.
template <int D, int JS>
__device__ __forceinline__ void merge_part(const Args& a, int u, int S, int jr, int R, __bf16* out) {
    static_assert(D % 64 == 0, "one head per wavefront and j");
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int G = a.G, GD = G * D;
    const size_t base = (size_t)u * a.NS;
    const __amdgpu_buffer_rsrc_t racc = buf_view(a.part_acc + base * GD, 4u * a.NS * GD);
    const __amdgpu_buffer_rsrc_t rml = buf_view(a.part_ml + base * G, 8u * a.NS * G);
    unsigned eo[JS];
    int hh[JS];
    float acc[JS], M[JS], L[JS];
#pragma unroll
    for (int k = 0; k < JS; ++k) {
        const int e0 = 64 * w + (jr + R * k) * kThreads;  // the wavefront's first element
        hh[k] = e0 / D;
        eo[k] = e0 + lane < GD ? 4u * (unsigned)(e0 + lane) : kBufOut;
        acc[k] = 0.f;
        M[k] = -INFINITY;
        L[k] = 0.f;
    }
    constexpr int NB = 32 / JS;  // slots per batch (2 NB divides 64)
    // a slot past the group or an element past G x D reads 0
    auto issue = [&](float (&v)[JS][NB], int g0, int ng, int s0) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const unsigned os = s0 + i < ng ? 4u * (unsigned)((g0 + s0 + i) * GD) : kBufOut;
#pragma unroll
            for (int k = 0; k < JS; ++k) v[k][i] = ld_dev_buf(racc, eo[k] + os);
        }
    };
    for (int g0 = 0; g0 < S; g0 += 64) {
        const int ng = min(64, S - g0);
        float x[JS], y[JS];
#pragma unroll
        for (int k = 0; k < JS; ++k) {
            const bool on = lane < ng && hh[k] < G;
            const unsigned om = on ? 8u * (unsigned)((g0 + lane) * G + hh[k]) : kBufOut;
            x[k] = ld_dev_buf(rml, om);
            y[k] = ld_dev_buf(rml, om + 4u);
            x[k] = on ? x[k] : -INFINITY;
        }
        float va[JS][NB], vb[JS][NB];
        issue(va, g0, ng, 0);
        float f[JS];  // this lane's slot factor
#pragma unroll
        for (int k = 0; k < JS; ++k) {
            float mx = x[k];
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            const float Mn = fmaxf(M[k], mx);
            f[k] = x[k] == -INFINITY ? 0.f : exp2f(x[k] - Mn);
            const float r = M[k] == -INFINITY ? 0.f : exp2f(M[k] - Mn);
            float ls = y[k] * f[k];
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o);
            L[k] = L[k] * r + ls;
            acc[k] *= r;
            M[k] = Mn;
        }
        auto fold = [&](const float (&v)[JS][NB], int s0) {
#pragma unroll
            for (int k = 0; k < JS; ++k) {
                float t = acc[k];
#pragma unroll
                for (int i = 0; i < NB; ++i)
                    t += v[k][i] * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f[k]), s0 + i));
                acc[k] = t;
            }
        };
        for (int s0 = 0; s0 < ng; s0 += 2 * NB) {
            if (s0 + NB < ng) issue(vb, g0, ng, s0 + NB);
            fold(va, s0);
            if (s0 + 2 * NB < ng) issue(va, g0, ng, s0 + 2 * NB);
            if (s0 + NB < ng) fold(vb, s0 + NB);
        }
    }
#pragma unroll
    for (int k = 0; k < JS; ++k) {
        const int e = 64 * w + (jr + R * k) * kThreads + lane;
        if (e < GD) out[e] = (__bf16)((M[k] == -INFINITY || L[k] == 0.f) ? 0.f : acc[k] / L[k]);
    }
}

template <int D, int EJ, bool PROBS>
__device__ __forceinline__ void task_flat(const Args& a, const Sched& s, int u, int idx, unsigned char* smem,
                                          CombineSmem& cs, FoldHdr& fh, int* wsum) {
    constexpr int NBW = kFusedTA / 128;  // 32-row gist blocks per wavefront
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int G = a.G, C = a.C;
    const int b = u / a.Hkv, g = u - b * a.Hkv;
    const int S = s.S1, W = S - 1;
    const int p0 = idx * kFusedTA;
    auto row_p = [&](int j, int t) { return p0 + 32 * (w + 4 * j) + 16 * t + lr; };
    // gist rows: block-table lookups issued with the length load
    size_t off[NBW][2];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int p = min(row_p(j, t), a.num_chunks - 1);
            off[j][t] = slot_offset(a, b, g, max(p, 0) * (C + 1) + C);
        }
    ListCtx c;
    make_ctx(a, kListGists, u, false, c);
    const int n = c.n;
    const int nA = max(1, (n + kFusedTA - 1) / kFusedTA);  // gist slices (<= S)
    const int sel = nA - 1;
    const bool selector = idx == sel;
    const int cnt = max(0, min(kFusedTA, n - p0));
    const bool attn = !(a.flags & kFlagSelectedGists);
    const bool topp = a.flags & kFlagTopP;      // (with the all-gists set only)
    constexpr bool probs = PROBS;  // the sum-of-probabilities key (with the all-gists set only)
    const int ulen = c.ns * C + c.tail + (attn ? 0 : c.ns);  // unfolded list
    const int nUB = (ulen + 31) / 32;
    const int widx = idx < sel ? idx : idx - 1;
    const unsigned long long t_start = wall_clock64();
    float* keys = a.keys + (size_t)u * a.key_stride;

    WaveAttnL<D> wa;
    wa.init((const __bf16*)a.q + ((size_t)b * a.Hq + (size_t)g * G) * D, G, lr, lg);
    unsigned char* tile = smem + (size_t)w * WaveAttnL<D>::TILE_BYTES;
    SelPre pre;
    uint64_t ownk = 0;  // the selector's key of this thread (its slice is not bucket sorted)
    bool ownv = false;
    int nval[NBW], nbw = 0;
    bf16x8_t P[NBW];
    if (cnt > 0) {
        const int nblk = (cnt + 31) / 32;
        nbw = nblk > w ? (nblk - w + 3) / 4 : 0;
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            nval[j] = max(0, min(32, cnt - 32 * (w + 4 * j)));
            // a token past the end reads the block's first row (in range)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                if (16 * t + lr >= nval[j]) off[j][t] = __shfl(off[j][0], lane & 48);
        }
        float* stash = (float*)(smem + Lds::stash(D)) + 64 * w;
        const float tau = a.tau;
        // sum-of-probabilities key: this lane's raw scores (head lr, token
        // 16t + 4lg + r of block j), kept until every slice's per-head
        // maximum and sum are known
        float zk[NBW][8];
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) zk[j][e] = 0.f;
        auto on_scores = [&](int j, const f32x4_t sc[2]) {
            if (probs) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) zk[j][4 * t + r] = sc[t][r];
                return;
            }
            // routing keys: tau * sum over the group's heads (padding heads are 0)
            float kv = 0.f;
            int kt = -1;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = rowsum16(sc[t][r]);
                    if (4 * t + r == lr) {
                        kv = x * tau;
                        kt = 16 * t + 4 * lg + r;
                    }
                }
            if (kt >= 0 && kt < nval[j]) stash[32 * j + kt] = kv;
        };
        if (attn)
            wa.template kpass<NBW>((const __bf16*)a.kc, off, nval, nbw, a.tau_log2e, lg, P, on_scores);
        else
            wa.template stream<NBW>((const __bf16*)a.kc, (const __bf16*)a.vc, off, nval, nbw, false,
                                    a.tau_log2e, lr, lg, tile, on_scores);
        if (probs) {
            // the sum-of-probabilities key (each head's softmax of the logits
            // z = tau q.k over the sequence's gists, summed over the group):
            // (1) this slice's per-head maximum and sum of exp, published
            auto zvalid = [&](int j, int e) { return 16 * (e >> 2) + 4 * lg + (e & 3) < nval[j]; };
            float hm = -INFINITY;
#pragma unroll
            for (int j = 0; j < NBW; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (zvalid(j, e)) hm = fmaxf(hm, zk[j][e] * tau);
            hm = fmaxf(hm, __shfl_xor(hm, 16));
            hm = fmaxf(hm, __shfl_xor(hm, 32));
            if (lg == 0) cs.wm[w][lr] = hm;
            lds_barrier();
            const float Mh = fmaxf(fmaxf(cs.wm[0][lr], cs.wm[1][lr]), fmaxf(cs.wm[2][lr], cs.wm[3][lr]));
            float hl = 0.f;
            if (isfinite(Mh)) {
#pragma unroll
                for (int j = 0; j < NBW; ++j)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (zvalid(j, e)) hl += expf(zk[j][e] * tau - Mh);
            }
            hl += __shfl_xor(hl, 16);
            hl += __shfl_xor(hl, 32);
            if (lg == 0) cs.wl[w][lr] = hl;
            lds_barrier();
            uint64_t* hp = unit_hpairs(a, u);
            if (w == 0 && lg == 0 && lr < G) {
                const float Ls = (cs.wl[0][lr] + cs.wl[1][lr]) + (cs.wl[2][lr] + cs.wl[3][lr]);
                st_dev(hp + idx * G + lr,
                       ((uint64_t)(__float_as_uint(Ls) | 0x80000000u) << 32) | __float_as_uint(Mh));
            }
            // (2) every slice's pairs, each word polled until written: each
            // head's maximum and sum over the sequence (the keys, and the
            // select, wait for the slowest slice's K pass: the V passes, which
            // do not, follow)
            float2* pl = (float2*)smem;  // (the V tiles are not in use yet)
            for (int i = threadIdx.x; i < nA * G; i += kThreads) {
                uint64_t x = ld_dev(hp + i);
                for (unsigned it = 0; x == 0ull; ++it) {
                    if (it >= kSpinLimit) {  // never expected: report, fold what is there
                        st_dev(s.err, 1u);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                    x = ld_dev(hp + i);
                }
                pl[i] = make_float2(__uint_as_float((uint32_t)x), __uint_as_float((uint32_t)(x >> 32) & 0x7fffffffu));
            }
            lds_barrier();
            if (threadIdx.x < (unsigned)G) {
                float M = -INFINITY, L = 0.f;
                for (int sl = 0; sl < nA; ++sl) M = fmaxf(M, pl[sl * G + threadIdx.x].x);
                if (isfinite(M))
                    for (int sl = 0; sl < nA; ++sl) {
                        const float2 v = pl[sl * G + threadIdx.x];
                        if (v.x != -INFINITY) L += v.y * expf(v.x - M);
                    }
                cs.wm[0][threadIdx.x] = M;
                cs.wl[0][threadIdx.x] = L;
            }
            lds_barrier();
            // (4) the keys: the sum over the heads of each head's probability
            const float Mg = lr < G ? cs.wm[0][lr] : 0.f, Lg = lr < G ? cs.wl[0][lr] : 0.f;
            const bool hok = lr < G && isfinite(Mg) && Lg > 0.f;
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                float kvp = 0.f;
                int kt = -1;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = rowsum16(hok ? expf(zk[j][e] * tau - Mg) / Lg : 0.f);
                    if (e == lr) {
                        kvp = x;
                        kt = 16 * (e >> 2) + 4 * lg + (e & 3);
                    }
                }
                if (kt >= 0 && kt < nval[j]) stash[32 * j + kt] = kvp;
            }
        }
        if (selector) select_prefetch<kListGists>(a, c, n, nA, pre);
        // thread t takes key slot t % 64 of wavefront t / 64
        static_assert(NBW * 32 * 4 <= kThreads, "one key slot per thread");
        lds_barrier();
        const int ws = threadIdx.x >> 6, slot = threadIdx.x & 63;
        const int kpos = 32 * (ws + 4 * (slot >> 5)) + (slot & 31);
        const float kv = kpos < cnt ? ((const float*)(smem + Lds::stash(D)))[64 * ws + slot] : 0.f;
        if (kpos < cnt) st_dev(keys + p0 + kpos, kv);
        if (topp) {
            // this slice's softmax maximum and sum of exp over its keys (NaN
            // keys left out), for the top-p cut
            const bool ok = kpos < cnt && !isnan(kv);
            float x = ok ? kv : -INFINITY;
            for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
            if (lane == 0) fh.m[w] = x;
            lds_barrier();
            const float ms = fmaxf(fmaxf(fh.m[0], fh.m[1]), fmaxf(fh.m[2], fh.m[3]));
            float z = ok && isfinite(ms) ? expf(kv - ms) : 0.f;
            for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
            if (lane == 0) fh.l[w] = z;
            lds_barrier();
            const float zs = (fh.l[0] + fh.l[1]) + (fh.l[2] + fh.l[3]);
            if (threadIdx.x == 0)
                st_dev(unit_topp(a, u) + idx,
                       ((uint64_t)__float_as_uint(zs > 0.f ? zs : -1.f) << 32) | __float_as_uint(ms));
        }
        lds_barrier();  // the stash is read (the key stores need not have landed)
        if (!selector) {
            uint64_t* pairs = a.spairs + ((size_t)u * s.S1 + idx) * kFusedTA;
            uint64_t* lead = nA > kRecSlices ? nullptr : unit_lead(a, u) + idx * kFSelL;
            bucket_slice(pairs, lead, p0, kv, kpos < cnt ? kpos : -1, smem, wsum);
            hold_until(t_start + s.vhold);  // (V-pass pacing: the launch's K rows go first)
            // V pass over this slice's gists; each wavefront counts itself in
            // (cntA) once its stores have landed, which the wait for its first
            // V block covers
            auto count_in = [&]() {
                if (lane == 0) add_dev(unit_cntA(a, u), 1u);
            };
            if (probs) {  // the V pass, each wavefront counting its keys in on cntS
                wa.template vpass<NBW>((const __bf16*)a.vc, off, nbw, P, tile, [&]() {
                    if (lane == 0) add_dev(unit_cntS(a, u), 1u);
                });
            } else if (attn) {
                wa.template vpass<NBW>((const __bf16*)a.vc, off, nbw, P, tile, count_in);
            } else {
                drain();
                count_in();
            }
        } else {
            ownk = (uint64_t)order_key(kv) | ((uint64_t)(uint32_t)(p0 + kpos) << 32);
            ownv = kpos < cnt;
        }
    } else if (selector) {
        select_prefetch<kListGists>(a, c, n, nA, pre);
    }
    if (selector) {
        // the select as soon as the slices' keys are in (only the K pass's
        // probabilities, running max and sum stay live across it: O is still
        // zero and is re-initialised after)
        lds_barrier();
        __builtin_amdgcn_s_setprio(2);  // everything of the unit waits for the select
        for (int i = n + threadIdx.x; i < a.num_chunks; i += kThreads) keys[i] = -INFINITY;
        select_fused<kListGists, 4>(a, s, c, n, nA, keys, smem, pre, idx, ownk, ownv, NoDrain{});
        if (nA <= kRecSlices) {  // the leading keys back to zero: each has been read
            uint64_t* lead = unit_lead(a, u);
            for (int i = threadIdx.x; i < nA * kFSelL; i += kThreads) {
                const int sl = i / kFSelL;
                if (i - sl * kFSelL < min(kFusedTA, n - sl * kFusedTA)) st_dev(lead + i, 0ull);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        lds_barrier();  // the select's LDS is free for the V tiles
#pragma unroll
        for (int db = 0; db < WaveAttnL<D>::DB; ++db) wa.o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        if (attn && cnt > 0) wa.template vpass<NBW>((const __bf16*)a.vc, off, nbw, P, tile, []() {});
    }

    // unfolded blocks of this wavefront (workers)
    if (!selector && nUB > 0) {
        __builtin_amdgcn_s_setprio(1);  // the unit's result waits for these rows
        const int64_t* ro = unit_rowoff(a, u);
        const int raw = c.ns * C;
        const int64_t tail_off = c.tail > 0 ? (int64_t)slot_offset(a, b, g, n * (C + 1)) : 0;
        for (int jb = w * W + widx; jb < nUB; jb += 4 * W) {
            size_t uoff[1][2];
            int unval[1];
            int jr[2];
            int64_t o[2], add[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rel = 32 * jb + 16 * t + lr;
                const int p = rel < ulen ? rel : 32 * jb;  // a row past the end reads the block's first
                jr[t] = -1;
                add[t] = 0;
                o[t] = 1;
                if (topp) {
                    // top-p: the raw tail first, then the selected chunks'
                    // rows, so that the rows the cut keeps come first
                    if (p < c.tail) {
                        o[t] = tail_off + (int64_t)p * D + 1;
                    } else {
                        jr[t] = (p - c.tail) / C;
                        add[t] = (int64_t)(p - c.tail - jr[t] * C) * D;
                    }
                } else if (p < raw) {
                    jr[t] = p / C;
                    add[t] = (int64_t)(p - jr[t] * C) * D;
                } else if (p < raw + c.tail) {
                    o[t] = tail_off + (int64_t)(p - raw) * D + 1;
                } else {
                    jr[t] = p - raw - c.tail;
                    add[t] = (int64_t)C * D;  // the selected chunk's gist
                }
                if (jr[t] >= 0) o[t] = ld_dev(ro + jr[t]);
            }
            for (unsigned it = 0;; ++it) {
                if (!__ballot(o[0] == 0 || o[1] == 0)) break;
                if (it >= kSpinLimit) {  // never expected: report, read a row in range
                    if (lane == 0) st_dev(s.err, 1u);
                    o[0] = o[0] == 0 ? 1 : o[0];
                    o[1] = o[1] == 0 ? 1 : o[1];
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    if (o[t] == 0) o[t] = ld_dev(ro + jr[t]);
            }
            if (topp) {
                // rows of chunks the cut dropped (and rows past the end) are
                // the block's last: its length is the count of the others
                int nv = 0;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const bool valid = 32 * jb + 16 * t + lr < ulen && !((uint64_t)o[t] & kRowSkip);
                    nv += __popcll(__ballot(valid && lg == 0));
                    if (!valid) {  // an in-range row
                        o[t] = 1;
                        add[t] = 0;
                    }
                }
                if (nv == 0) continue;
                unval[0] = nv;
            } else {
                unval[0] = min(32, ulen - 32 * jb);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) uoff[0][t] = (size_t)(o[t] - 1 + add[t]);
            wa.template stream<1>((const __bf16*)a.kc, (const __bf16*)a.vc, uoff, unval, 1, true,
                                  a.tau_log2e, lr, lg, tile, [](int, const f32x4_t*) {});
        }
    }
    // publish this task's partial (slot idx) and count in; the last to count
    // in merges
    lds_barrier();
    {
        float gacc[EJ];
#pragma unroll
        for (int j = 0; j < EJ; ++j) gacc[j] = 0.f;
        if (threadIdx.x < 16) {
            fh.m[threadIdx.x] = -INFINITY;
            fh.l[threadIdx.x] = 0.f;
        }
        combine_publish<D, EJ, false>(wa, a, u, idx, gacc, fh, (float*)smem, cs);
    }
    drain();
    __syncthreads();
    if (threadIdx.x == 0) wsum[0] = (int)add_dev(unit_cntB(a, u), 1u);
    __syncthreads();
    // the last R tasks to count in merge, element block j to the one of rank
    // j mod R; all but the last wait for it (a short wait: they are the last)
    constexpr int R = EJ < 4 ? EJ : 4;
    const int rank = wsum[0] - (S - R);
    const bool few = S < R;  // fewer tasks than mergers: the last merges all
    if (rank < 0 || (few && rank != R - 1)) return;
    if (rank != R - 1) {
        wait_at_least<1>(unit_cntB(a, u), (unsigned)S, s.err);
        __syncthreads();
    }
    __bf16* out = (__bf16*)a.out + ((size_t)b * a.Hq + (size_t)g * G) * D;
    if (few) {
        for (int jr = 0; jr < R; ++jr) merge_part<D, EJ / R>(a, u, S, jr, R, out);
    } else {
        merge_part<D, EJ / R>(a, u, S, rank, R, out);
    }
    // the last merger to finish returns the record to zero (every task has
    // read the selection before counting in, every merger has seen the count;
    // the output's stores need not have landed)
    lds_barrier();
    if (threadIdx.x == 0) wsum[0] = (int)add_dev(unit_cntP(a, u), 1u);
    __syncthreads();
    if (wsum[0] != (few ? 0 : R - 1)) return;
    for (int i = threadIdx.x; i < c.ns; i += kThreads) st_dev(unit_rowoff(a, u) + i, (int64_t)0);
    if (topp)
        for (int i = threadIdx.x; i < nA; i += kThreads) st_dev(unit_topp(a, u) + i, 0ull);
    if (probs)
        for (int i = threadIdx.x; i < nA * G; i += kThreads) st_dev(unit_hpairs(a, u) + i, 0ull);
    if (threadIdx.x == 0) {
        st_dev(unit_cntA(a, u), 0u);
        st_dev(unit_cntB(a, u), 0u);
        st_dev(unit_cntP(a, u), 0u);
        st_dev(unit_cntS(a, u), 0u);
    }
}

template <int D, int EJ, bool HIER, int NBB>
__global__ __launch_bounds__(kThreads, 4) void gsa_fused_kernel(Args a, Sched s) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ CombineSmem cs;
    __shared__ FoldHdr fh;
    __shared__ int wsum[kThreads / 64];
    __shared__ int s_flag;
    const int nA = s.units * s.S1, nC = s.units * s.S3;
    const int t = blockIdx.x;
    if constexpr (!HIER && (NBB == 0 || NBB == 3)) {  // flat GSA, every task a gist slice or unfolded blocks
        const int u = t / s.S1;
        task_flat<D, EJ, NBB == 3>(a, s, u, t - u * s.S1, smem, cs, fh, wsum);
    } else if (t < nA) {
        const int u = t / s.S1;
        task_slices<D, EJ, HIER ? kListMeta : kListGists>(a, s, u, t - u * s.S1, smem, cs, wsum);
    } else if (HIER && t < nA + nC) {
        const int u = (t - nA) / s.S3;
        task_slices<D, EJ, kListCand>(a, s, u, t - nA - u * s.S3, smem, cs, wsum);
    } else {
        const int u = (t - nA - nC) / s.S2;
        task_unfolded<D, EJ, HIER, NBB>(a, s, u, t - nA - nC - u * s.S2, smem, cs, fh, &s_flag);
    }
}

}  // namespace

namespace {
template <int D, int EJ>
void launch_fused_t(const Args& a, const Sched& s, int lds, hipStream_t st) {
    // NBB: 32-token blocks per wavefront of an unfolded task; 0: the flat
    // kernel whose every task is a gist slice or a set of unfolded blocks, 3:
    // the same with the sum-of-probabilities key
    if (s.hier)
        hipLaunchKernelGGL((gsa_fused_kernel<D, EJ, true, 1>), dim3(s.total), dim3(kThreads), lds, st, a, s);
    else if (s.flat && (a.flags & kFlagSumProbs))
        hipLaunchKernelGGL((gsa_fused_kernel<D, EJ, false, 3>), dim3(s.total), dim3(kThreads), lds, st, a, s);
    else if (s.flat)
        hipLaunchKernelGGL((gsa_fused_kernel<D, EJ, false, 0>), dim3(s.total), dim3(kThreads), lds, st, a, s);
    else if (s.TB == 2 * kFusedTB)
        hipLaunchKernelGGL((gsa_fused_kernel<D, EJ, false, 2>), dim3(s.total), dim3(kThreads), lds, st, a, s);
    else
        hipLaunchKernelGGL((gsa_fused_kernel<D, EJ, false, 1>), dim3(s.total), dim3(kThreads), lds, st, a, s);
}
}  // namespace

hipError_t launch_fused(const Args& a, const Sched& s, hipStream_t st) {
    const int lds = Lds::bytes(a.G, a.D);
    const int ej = (a.G * a.D + kThreads - 1) / kThreads;  // 1 .. 8
    if (a.D == 64) {
        if (ej <= 1) launch_fused_t<64, 1>(a, s, lds, st);
        else if (ej <= 2) launch_fused_t<64, 2>(a, s, lds, st);
        else launch_fused_t<64, 4>(a, s, lds, st);
    } else {
        if (ej <= 1) launch_fused_t<128, 1>(a, s, lds, st);
        else if (ej <= 2) launch_fused_t<128, 2>(a, s, lds, st);
        else if (ej <= 4) launch_fused_t<128, 4>(a, s, lds, st);
        else launch_fused_t<128, 8>(a, s, lds, st);
    }
    return hipGetLastError();
}

}  // namespace gsa
