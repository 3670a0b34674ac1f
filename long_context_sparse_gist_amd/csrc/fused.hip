// Single-launch GSA decode (bf16, MFMA): one kernel, one task per workgroup.
//
// Workgroup t runs task t.  Tasks are numbered gist slices first (every unit,
// unit-major), then unfolded-list tasks:
//   gist slice (u, i)  scores gists [i*TA, (i+1)*TA) of unit u, writes their
//                      routing keys and (all-gists set) one softmax partial.
//                      The unit's last slice to finish runs its top-k select
//                      and publishes the selection.
//   unfolded (u, j)    waits for unit u's selection, attends tokens
//                      [j*TB, (j+1)*TB) of the unfolded list (raw tokens of
//                      the selected chunks, raw tail, selected gists), folds
//                      gist-slice partials i = j, j+nB, ... into its own and
//                      writes one partial.  The unit's last one merges them
//                      into the output and resets the unit's counters.
// Only unfolded tasks wait, and only on gist-slice tasks, which have smaller
// workgroup ids: the device dispatches each XCD's workgroups in id order, so
// every slice a waiting task depends on has been dispatched and runs to
// completion (it never waits).  A wait is nevertheless bounded; giving up
// sets the error word of the control block.  Several workgroups per CU hide
// each task's serial latencies (table lookups, drains) behind the others'
// streaming, and the unfolded tasks of early units overlap the gist slices of
// later ones.  Data passed between workgroups is written and read with
// device-scope atomics (coherent across the XCDs' L2s); a producer waits for
// its stores to complete before it bumps a counter or sets a flag, and the
// unit's merging task returns the unit's counters to zero.
#include "gsa_lists.h"
#include "gsa_mfma_core.h"
#include "gsa_select.h"

namespace gsa {
namespace {

constexpr int kThreads = 256;
constexpr unsigned kSpinLimit = 1u << 24;

__device__ inline void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_dev(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline unsigned ld_dev(const unsigned* p) {
    return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline unsigned add_dev(unsigned* p, unsigned v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until this thread's memory operations have completed
__device__ inline void drain() { __builtin_amdgcn_s_waitcnt(0); }

// Folding state of one partial: small per-head arrays (the G*D accumulator
// lives in dynamic LDS next to it).
constexpr int kFoldRound = 8;  // partials folded per round
struct FoldHdr {
    float m[16], l[16], f_self[16];
    float f[kFoldRound][16];
    float2 ml[kFoldRound][16];
};

// Dynamic LDS layout (bytes), uses separated in time:
//   [0, vt)                          V transpose tiles (attention blocks)
//   [0, red) [red, +acc) [.., +hdr)  wavefront combination, folding state
//   [0, sel)                         top-k select (last gist slice of a unit)
struct Lds {
    static constexpr int vt(int D) { return 4 * (D * (32 + 4) * 2); }
    static constexpr int red(int G, int D) { return 4 * G * D * 4; }
    static constexpr int acc_off(int G, int D) { return red(G, D); }
    static constexpr int hdr_off(int G, int D) { return acc_off(G, D) + G * D * 4; }
    static constexpr int sel() { return (int)sizeof(SelectSmem<kThreads>); }
    static int bytes(int G, int D) {
        int a = vt(D), b = hdr_off(G, D) + (int)sizeof(FoldHdr), c = sel();
        int m = a > b ? a : b;
        return m > c ? m : c;
    }
};

// Fold partial slots slot_of(0..ns) of unit u into (acc, hdr), eight per
// round; within a round every load of a thread's element chunk is in flight
// together.
template <int D, typename SlotFn>
__device__ void fold_slots(const Args& a, int u, SlotFn slot_of, int ns, float* acc, FoldHdr& fh) {
    constexpr int EC = 4;  // elements per thread per chunk
    const int G = a.G;
    const size_t base = (size_t)u * a.NS;
    for (int r0 = 0; r0 < ns; r0 += kFoldRound) {
        const int nr = min(kFoldRound, ns - r0);
        for (int e = threadIdx.x; e < nr * G; e += kThreads) {
            int i = e / G, h = e - i * G;
            const float* p = (const float*)(a.part_ml + (base + slot_of(r0 + i)) * G + h);
            fh.ml[i][h] = make_float2(ld_dev(p), ld_dev(p + 1));
        }
        __syncthreads();
        if (threadIdx.x < (unsigned)G) {
            const int h = threadIdx.x;
            float M = fh.m[h];
            for (int i = 0; i < nr; ++i) M = fmaxf(M, fh.ml[i][h].x);
            float fself = (fh.m[h] == -INFINITY) ? 0.f : exp2f(fh.m[h] - M);
            float L = fh.l[h] * fself;
            for (int i = 0; i < kFoldRound; ++i) {
                float fi = (i >= nr || fh.ml[i][h].x == -INFINITY) ? 0.f : exp2f(fh.ml[i][h].x - M);
                fh.f[i][h] = fi;
                if (i < nr) L += fh.ml[i][h].y * fi;
            }
            fh.f_self[h] = fself;
            fh.m[h] = M;
            fh.l[h] = L;
        }
        __syncthreads();
        for (int e0 = threadIdx.x; e0 < G * D; e0 += EC * kThreads) {
            float v[EC][kFoldRound];
#pragma unroll
            for (int j = 0; j < EC; ++j) {
                const int e = e0 + j * kThreads;
#pragma unroll
                for (int i = 0; i < kFoldRound; ++i)
                    v[j][i] = (e < G * D && i < nr)
                                  ? ld_dev(a.part_acc + (base + slot_of(r0 + i)) * G * D + e)
                                  : 0.f;
            }
#pragma unroll
            for (int j = 0; j < EC; ++j) {
                const int e = e0 + j * kThreads;
                if (e < G * D) {
                    const int h = e / D;
                    float x = acc[e] * fh.f_self[h];
#pragma unroll
                    for (int i = 0; i < kFoldRound; ++i) x += v[j][i] * fh.f[i][h];
                    acc[e] = x;
                }
            }
        }
        __syncthreads();
    }
}

__device__ inline void fold_init(float* acc, FoldHdr& fh, int G, int D) {
    for (int e = threadIdx.x; e < G * D; e += kThreads) acc[e] = 0.f;
    if (threadIdx.x < 16) {
        fh.m[threadIdx.x] = -INFINITY;
        fh.l[threadIdx.x] = 0.f;
    }
}

// One 32-token block per wavefront: wavefront w owns tokens [32w, 32w+32) of
// the task.  off[t], ok[t]: element offset of this lane's K/V row (token
// 16*t + lr) and whether that token is real.  Returns the scores through sc.
template <int D>
__device__ inline void wave_block(WaveAttn<D>& wa, const Args& a, const size_t* off, const bool* ok,
                                  int nvalid, bool attn, int lr, int lg, __bf16* vt, f32x4_t sc[2]) {
    constexpr int KK = WaveAttn<D>::KK;
    // a token past the end reads q (valid memory); its score is masked out
    const __bf16* kb[2];
    const __bf16* vb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        kb[t] = ok[t] ? (const __bf16*)a.kc + off[t] : (const __bf16*)a.q;
        vb[t] = ok[t] ? (const __bf16*)a.vc + off[t] : (const __bf16*)a.q;
    }
    bf16x8_t kA[2][KK], vA[2][KK];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) kA[t][kk] = *(const bf16x8_t*)(kb[t] + 32 * kk + 8 * lg);
    if (attn) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) vA[t][kk] = *(const bf16x8_t*)(vb[t] + 32 * kk + 8 * lg);
    }
    wa.scores(kA, sc);
    if (attn && nvalid > 0) {
        bf16x8_t P = wa.softmax_stage(sc, vA, nvalid, a.tau_log2e, lr, lg, vt);
        wa.pv_stage(P, lr, lg, vt);
    }
}

template <int D>
__device__ void task_gists(const Args& a, const Sched& s, int u, int idx, unsigned char* smem,
                           CombineSmem& cs, int* s_flag) {
    constexpr int NBW = kFusedTA / 128;  // 32-token blocks per wavefront
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int G = a.G, C = a.C;
    const int b = u / a.Hkv, g = u - b * a.Hkv;
    const int p0 = idx * s.TA;
    // block-table lookups of this lane's tokens (blocks w, w+4, ...), issued
    // together with the length load
    size_t off[NBW][2];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            int p = min(p0 + 32 * (w + 4 * j) + 16 * t + lr, a.num_chunks - 1);
            off[j][t] = slot_offset(a, b, g, max(p, 0) * (C + 1) + C);
        }
    ListCtx c;
    make_ctx(a, kListGists, u, false, c);
    const int nA = max(1, (c.n + s.TA - 1) / s.TA);
    if (idx >= nA) return;
    const bool attn = !(a.flags & kFlagSelectedGists);
    const int cnt = max(0, min(s.TA, c.n - p0));
    float* keys = a.keys + (size_t)u * a.key_stride;

    if (cnt > 0) {
        int nval[NBW];
        const int nblk = (cnt + 31) / 32;
        const int nbw = nblk > w ? (nblk - w + 3) / 4 : 0;
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            nval[j] = max(0, min(32, cnt - 32 * (w + 4 * j)));
            // a token past the end reads the block's first row (in range)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                if (16 * t + lr >= nval[j]) off[j][t] = __shfl(off[j][0], lane & 48);
        }
        WaveAttn<D> wa;
        wa.init((const __bf16*)a.q + ((size_t)c.b * a.Hq + (size_t)c.g * G) * D, G, lr, lg);
        __bf16* vt = (__bf16*)smem + (size_t)w * (D * (32 + 4));
        const float tau = a.tau;
        wa.template stream<NBW, false>(
            (const __bf16*)a.kc, (const __bf16*)a.vc, off, nval, nbw, attn, a.tau_log2e, lr, lg,
            vt, [&](int j, const f32x4_t sc[2]) {
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
                if (kt >= 0 && kt < nval[j]) st_dev(keys + p0 + 32 * (w + 4 * j) + kt, kv);
            });
        if (attn) {
            __syncthreads();
            const size_t pbase = ((size_t)u * a.NS + idx) * G;
            combine_waves<D>(
                wa, a.tau_log2e, G, (float*)smem, cs,
                [&](int h, int d, float v) { st_dev(a.part_acc + (pbase + h) * D + d, v); },
                [&](int h, float m2, float l) {
                    float* p = (float*)(a.part_ml + pbase + h);
                    st_dev(p, m2);
                    st_dev(p + 1, l);
                });
        }
    }
    drain();
    __syncthreads();
    if (threadIdx.x == 0) *s_flag = add_dev(s.cntA + u, 1u) == (unsigned)(nA - 1);
    __syncthreads();
    if (!*s_flag) return;

    // last slice of the unit: select and publish
    for (int i = c.n + threadIdx.x; i < a.num_chunks; i += kThreads) keys[i] = -INFINITY;
    SelectSmem<kThreads>& ssh = *(SelectSmem<kThreads>*)smem;
    block_topk<kThreads>(keys, nullptr, c.n, a.top_k, a.sel + (size_t)u * a.top_k, true, ssh);
    drain();
    __syncthreads();
    if (threadIdx.x == 0) st_dev(s.ready + u, 1u);
}

template <int D>
__device__ void task_unfolded(const Args& a, const Sched& s, int u, int idx, unsigned char* smem,
                              CombineSmem& cs, int* s_flag) {
    const int G = a.G;
    float* facc = (float*)(smem + Lds::acc_off(G, D));
    FoldHdr& fh = *(FoldHdr*)(smem + Lds::hdr_off(G, D));
    ListCtx c;
    make_ctx(a, kListUnfolded, u, false, c);
    const int nB = max(1, (c.len + s.TB - 1) / s.TB);
    if (idx >= nB) return;
    // wait for the unit's selection
    if (threadIdx.x == 0) {
        unsigned it = 0;
        while (ld_dev(s.ready + u) == 0u) {
            __builtin_amdgcn_s_sleep(2);
            if (++it >= kSpinLimit) {
                st_dev(s.err, 1u);
                break;
            }
        }
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int p0 = idx * s.TB;
    const int cnt = max(0, min(s.TB, c.len - p0));

    if (cnt == 0) fold_init(facc, fh, G, D);
    if (cnt > 0) {
        constexpr int NBW = kFusedTB / 128;
        const int nblk = (cnt + 31) / 32;
        const int nbw = nblk > w ? (nblk - w + 3) / 4 : 0;
        size_t off[NBW][2];
        int nval[NBW];
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            nval[j] = max(0, min(32, cnt - 32 * (w + 4 * j)));
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                // a token past the end reads the task's first row (in range)
                int rel = 32 * (w + 4 * j) + 16 * t + lr;
                const void *kb, *vb;
                off[j][t] = list_row(a, kListUnfolded, c, false, p0 + (rel < cnt ? rel : 0), &kb, &vb,
                                     true);
            }
        }
        WaveAttn<D> wa;
        wa.init((const __bf16*)a.q + ((size_t)c.b * a.Hq + (size_t)c.g * G) * D, G, lr, lg);
        __bf16* vt = (__bf16*)smem + (size_t)w * (D * (32 + 4));
        wa.template stream<NBW, false>((const __bf16*)a.kc, (const __bf16*)a.vc, off, nval, nbw, true,
                                a.tau_log2e, lr, lg, vt, [](int, const f32x4_t*) {});
        __syncthreads();
        combine_waves<D>(
            wa, a.tau_log2e, G, (float*)smem, cs, [&](int h, int d, float v) { facc[h * D + d] = v; },
            [&](int h, float m2, float l) {
                fh.m[h] = m2;
                fh.l[h] = l;
            });
    }
    __syncthreads();
    // fold the gist-slice partials i = idx, idx + nB, ...
    const bool attn = !(a.flags & kFlagSelectedGists);
    const int nA = attn ? (c.n + s.TA - 1) / s.TA : 0;
    const int nf = idx < nA ? (nA - idx + nB - 1) / nB : 0;
    if (nf) fold_slots<D>(a, u, [&](int i) { return idx + i * nB; }, nf, facc, fh);
    // publish this task's partial
    const size_t pbase = ((size_t)u * a.NS + s.S1 + idx) * G;
    for (int e = threadIdx.x; e < G * D; e += kThreads) st_dev(a.part_acc + pbase * D + e, facc[e]);
    if (threadIdx.x < (unsigned)G) {
        float* p = (float*)(a.part_ml + pbase + threadIdx.x);
        st_dev(p, fh.m[threadIdx.x]);
        st_dev(p + 1, fh.l[threadIdx.x]);
    }
    drain();
    __syncthreads();
    if (threadIdx.x == 0) *s_flag = add_dev(s.cntB + u, 1u) == (unsigned)(nB - 1);
    __syncthreads();
    if (!*s_flag) return;

    // last unfolded task of the unit: merge and reset the unit's counters
    fold_init(facc, fh, G, D);
    __syncthreads();
    fold_slots<D>(a, u, [&](int i) { return s.S1 + i; }, nB, facc, fh);
    __bf16* out = (__bf16*)a.out + ((size_t)c.b * a.Hq + (size_t)c.g * G) * D;
    for (int e = threadIdx.x; e < G * D; e += kThreads) {
        const int h = e / D;
        float L = fh.l[h];
        out[e] = (__bf16)((fh.m[h] == -INFINITY || L == 0.f) ? 0.f : facc[e] / L);
    }
    if (threadIdx.x == 0) {
        st_dev(s.cntA + u, 0u);
        st_dev(s.cntB + u, 0u);
        st_dev(s.ready + u, 0u);
    }
}

template <int D>
__global__ __launch_bounds__(kThreads, 4) void gsa_fused_kernel(Args a, Sched s) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ CombineSmem cs;
    __shared__ int s_flag;
    const int nA = s.units * s.S1;
    const int t = blockIdx.x;
    if (t < nA) {
        const int u = t / s.S1;
        task_gists<D>(a, s, u, t - u * s.S1, smem, cs, &s_flag);
    } else {
        const int u = (t - nA) / s.S2;
        task_unfolded<D>(a, s, u, t - nA - u * s.S2, smem, cs, &s_flag);
    }
}

}  // namespace

hipError_t launch_fused(const Args& a, const Sched& s, hipStream_t st) {
    const int lds = Lds::bytes(a.G, a.D);
    dim3 grid(s.total);
    if (a.D == 64)
        hipLaunchKernelGGL((gsa_fused_kernel<64>), grid, dim3(kThreads), lds, st, a, s);
    else
        hipLaunchKernelGGL((gsa_fused_kernel<128>), grid, dim3(kThreads), lds, st, a, s);
    return hipGetLastError();
}

}  // namespace gsa
