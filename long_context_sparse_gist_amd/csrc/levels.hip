// Gist sparse attention decode over a hierarchy of any depth: L levels of
// meta-gists above the gists, level l entry r summarising entries
// [r*R_l, (r+1)*R_l) of level l-1 (the recursive gist-of-gist structure of
// "Forget, Then Recall", ja page section 2.2 and nl page "Hierarchische
// Uitbreiding": coarse-to-fine selection, logarithmic decoding cost).
//
// Per (batch, kv-head) unit, from the top level L down to the gists:
//   scores   every entry of level L (and attends it), then the candidates of
//            each level below: the children of the entries kept one level up
//            plus the entries past that level's last complete group;
//   select   the top-k_l candidates (ties to the lower id, NaN last);
//   attend   the kept entries and the past-the-last-group entries of every
//            level below the top, the kept chunks' raw tokens and the raw tail.
// Launches (bf16, MFMA):
//   - a top level longer than kFoldTop entries: its keys and attention
//     (lv_top_kernel, at most kTopSplits workgroups per unit, each folding its
//     128-row blocks with an online softmax);
//   - the select chain (lv_chain_kernel), one workgroup per unit: a short top
//     level's keys, then per level the top-k and the next level's candidates'
//     ids and keys (MFMA), down to the gist level's select, which writes the
//     final attention list (with a short top level's entries in it);
//   - the final attention (lv_attn_final_kernel), 128 rows of the list per
//     workgroup, whose last workgroup per unit merges the unit's partials (a
//     separate merge launch when the arrival counters do not fit the control
//     block).
// Every list is a per-unit array of row descriptors (array id << 56 | element
// offset), so the attention reads rows of any level and of the paged cache
// alike.
#include "gsa_lists.h"
#include "gsa_levels.h"
#include "gsa_select.h"
#include "gsa_wave_select.h"

namespace gsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kRows = 32 * kWaves;  // rows per attention workgroup
constexpr int kSelThreads = 512;
constexpr int64_t kOffMask = (1ll << kDescShift) - 1;

// Data handed between workgroups of one launch (the final attention's
// partials, read by the unit's merging workgroup) goes through device-scope
// accesses, coherent across the XCDs' L2s without cache-wide fences.
__device__ inline void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t ld_dev(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float2 ld_dev2(const float2* p) {
    const uint64_t v = ld_dev((const uint64_t*)p);
    return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}
__device__ inline void st_dev2(float2* p, float2 v) {
    st_dev((uint64_t*)p, (uint64_t)__float_as_uint(v.x) | ((uint64_t)__float_as_uint(v.y) << 32));
}

__device__ inline float dpp_sum_step(float x, int ctrl) {
    int v = __builtin_bit_cast(int, x), r;
    switch (ctrl) {
        case 0: r = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); break;   // quad [1,0,3,2]
        case 1: r = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); break;   // quad [2,3,0,1]
        case 2: r = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false); break;  // row half mirror
        default: r = __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); break; // row mirror
    }
    return x + __builtin_bit_cast(float, r);
}

// Sum over the 16 lanes of a row; every lane of the row gets the total.
__device__ inline float row16_sum(float x) {
    x = dpp_sum_step(x, 0);
    x = dpp_sum_step(x, 1);
    x = dpp_sum_step(x, 2);
    return dpp_sum_step(x, 3);
}

// Entries per level of batch row b (level 0: its gists), and its raw tail.
__device__ inline void level_counts(const LvArgs& A, int b, int (&cnt)[kMaxLevels + 1], int& tail) {
    int n;
    seq_shape(A.a, b, n, tail);
    cnt[0] = n;
#pragma unroll
    for (int l = 1; l <= kMaxLevels; ++l) cnt[l] = l <= A.L ? cnt[l - 1] / A.fan[l] : 0;
}

// Entries of the top level of batch row b.
__device__ inline int top_count(const LvArgs& A, int b) {
    int n, tail;
    seq_shape(A.a, b, n, tail);
    for (int l = 1; l <= A.L; ++l) n /= A.fan[l];
    return n;
}

// Descriptor of entry `id` of level l of unit (b, g): level 0 is a gist in the
// paged cache, a level l >= 1 entry a row of that level's array.
__device__ inline int64_t entry_desc(const LvArgs& A, int l, int b, int g, int id) {
    if (l == 0) return (int64_t)slot_offset(A.a, b, g, id * (A.a.C + 1) + A.a.C);
    const size_t off = (((size_t)b * A.a.Hkv + g) * A.maxe[l] + id) * (size_t)A.a.D;
    return ((int64_t)l << kDescShift) | (int64_t)off;
}

// q of the group's heads of unit (b, g) as MFMA B operands: lane (lr, lg)
// holds head lr's elements [32kk + 8lg, 32kk + 8lg + 8); heads past G are 0.
template <int D>
__device__ inline void load_q(const Args& a, int b, int g, int lr, int lg, bf16x8_t (&qB)[D / 32]) {
    const __bf16* qp = (const __bf16*)a.q + ((size_t)b * a.Hq + (size_t)g * a.G + lr) * D;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        if (lr < a.G) {
            qB[kk] = *(const bf16x8_t*)(qp + 32 * kk + 8 * lg);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) qB[kk][i] = (__bf16)0.0f;
        }
    }
}

// Routing keys of 32 rows (two MFMA tiles of 16) from the lane's K operands:
// s[t][r] = q_{head lr} . k_{row 16t + 4lg + r}.  Lanes lr < 8 return the key
// of row 16t + 4lg + r with 4t + r == lr (the row sum over the group's heads,
// padding heads scoring 0) and set rel to that row; other lanes set rel = -1.
__device__ inline float tile_keys(const f32x4_t (&s)[2], int lr, int lg, float tau, int& rel) {
    float kv = 0.f;
    rel = -1;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = row16_sum(s[t][r]) * tau;
            if (4 * t + r == lr) {
                kv = x;
                rel = 16 * t + 4 * lg + r;
            }
        }
    return kv;
}

// Merge of unit u's partial slots [0, NS) into the output (bf16, rounded to
// nearest even) by one workgroup of 256 threads (G <= 16 heads): per head the
// largest maximum M and the normaliser sum_i l_i 2^(m_i - M), then each output
// element sum_i acc_i 2^(m_i - M) / normaliser.  An empty set gives zeros.
// sc: LDS for the scale factors 2^(m_i - M) of up to sc_slots slots (past
// that they are recomputed from the maxima).  The loads go out together: each
// thread's (max, sum) words of up to 32 slots and its first output pair's
// accumulators of up to 16 slots at the start, the rest eight slots at a time.
__device__ void merge_unit_block(const LvArgs& A, int u, float* sc, int sc_slots) {
    constexpr int PF = 16;  // slots of the first output pair loaded up front
    __shared__ float s_M[16], s_inv[16];
    const Args& a = A.a;
    const int b = u / a.Hkv, g = u - b * a.Hkv;
    const int G = a.G, D = a.D, NS = A.NS;
    const float2* ml = a.part_ml + (size_t)u * NS * G;
    const float* acc = a.part_acc + (size_t)u * NS * G * D;
    const int half = D / 2;
    const int e0 = threadIdx.x;
    const bool has0 = e0 < G * half;
    const int hh0 = has0 ? e0 / half : 0, d0 = 2 * (e0 - hh0 * half);
    float2 pv[PF];
#pragma unroll
    for (int t = 0; t < PF; ++t)
        pv[t] = has0 && t < NS ? ld_dev2((const float2*)(acc + ((size_t)t * G + hh0) * D + d0))
                               : make_float2(0.f, 0.f);
    {
        const int h = threadIdx.x >> 4, j = threadIdx.x & 15;
        float2 mv[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
            mv[t] = h < G && j + 16 * t < NS ? ld_dev2(ml + (size_t)(j + 16 * t) * G + h)
                                             : make_float2(-INFINITY, 0.f);
        float m = fmaxf(mv[0].x, mv[1].x);
        if (h < G)
            for (int i = j + 32; i < NS; i += 16) m = fmaxf(m, ld_dev2(ml + (size_t)i * G + h).x);
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        float l = 0.f;
        if (h < G) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int i = j + 16 * t;
                const float f = (m != -INFINITY && mv[t].x != -INFINITY) ? exp2f(mv[t].x - m) : 0.f;
                l += mv[t].y * f;
                if (i < NS && i < sc_slots) sc[i * 16 + h] = f;
            }
            for (int i = j + 32; i < NS; i += 16) {
                const float2 v = ld_dev2(ml + (size_t)i * G + h);
                const float f = (m != -INFINITY && v.x != -INFINITY) ? exp2f(v.x - m) : 0.f;
                l += v.y * f;
                if (i < sc_slots) sc[i * 16 + h] = f;
            }
        }
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) l += __shfl_xor(l, off);
        if (h < G && j == 0) {
            s_M[h] = m;
            s_inv[h] = (m != -INFINITY && l > 0.f) ? 1.f / l : 0.f;
        }
    }
    __syncthreads();
    __bf16* out = (__bf16*)a.out + ((size_t)b * a.Hq + (size_t)g * G) * D;
    auto scale = [&](int i, int hh, float M) -> float {
        if (i < sc_slots) return sc[i * 16 + hh];
        const float mi = ld_dev2(ml + (size_t)i * G + hh).x;
        return (M != -INFINITY && mi != -INFINITY) ? exp2f(mi - M) : 0.f;
    };
    for (int e = e0; e < G * half; e += blockDim.x) {
        const int hh = e / half, d = 2 * (e - hh * half);
        const float M = s_M[hh];
        float ox = 0.f, oy = 0.f;
        int i0 = 0;
        if (e == e0) {
#pragma unroll
            for (int t = 0; t < PF; ++t)
                if (t < NS) {
                    const float f = scale(t, hh, M);
                    ox += pv[t].x * f;
                    oy += pv[t].y * f;
                }
            i0 = PF;
        }
        for (; i0 < NS; i0 += 8) {
            float2 v[8];
#pragma unroll
            for (int t = 0; t < 8; ++t)
                v[t] = i0 + t < NS ? ld_dev2((const float2*)(acc + ((size_t)(i0 + t) * G + hh) * D + d))
                                   : make_float2(0.f, 0.f);
#pragma unroll
            for (int t = 0; t < 8; ++t)
                if (i0 + t < NS) {
                    const float f = scale(i0 + t, hh, M);
                    ox += v[t].x * f;
                    oy += v[t].y * f;
                }
        }
        out[hh * D + d] = (__bf16)(ox * s_inv[hh]);
        out[hh * D + d + 1] = (__bf16)(oy * s_inv[hh]);
    }
}

// Attention over the final list of each unit, one partial per 128-row split
// into partial slot slot0 + split (an empty split writes an empty partial);
// with arrival counters, the unit's last workgroup to finish merges the
// unit's partials and clears its counter.
template <int D>
__device__ __forceinline__ void lv_attn_body(const LvArgs& A, int slot0) {
    constexpr int KK = D / 32, DB = D / 16, LDW = 32 + 4;
    constexpr int VT = kWaves * D * LDW * 2, RED = kWaves * 16 * D * 4;
    __shared__ __attribute__((aligned(16))) unsigned char smem[VT > RED ? VT : RED];
    __shared__ float s_max[kWaves][16], s_sum[kWaves][16];
    __shared__ int s_last;
    const Args& a = A.a;
    const int u = blockIdx.y, split = blockIdx.x;
    const int b = u / a.Hkv, g = u - b * a.Hkv;
    const int G = a.G;
    const int len = A.nfin[u];
    const int p0 = split * kRows;
    const int count = min(kRows, len - p0);
    const size_t pbase = ((size_t)u * A.NS + slot0 + split) * G;
    const bool dev = A.uctr != nullptr;  // partials read by this launch's merging workgroup
    auto put_acc = [&](size_t i, float v) {
        if (dev) st_dev(a.part_acc + i, v);
        else a.part_acc[i] = v;
    };
    auto put_ml = [&](size_t i, float2 v) {
        if (dev) st_dev2(a.part_ml + i, v);
        else a.part_ml[i] = v;
    };
    if (count <= 0) {
        for (int e = threadIdx.x; e < G * D; e += blockDim.x) put_acc(pbase * D + e, 0.f);
        if (threadIdx.x < (unsigned)G) put_ml(pbase + threadIdx.x, make_float2(-INFINITY, 0.f));
    } else {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 15, lg = lane >> 4;
        bf16x8_t qB[KK];
        load_q<D>(a, b, g, lr, lg, qB);
        // rows of this lane: half t -> list position p0 + 32*w + 16*t + lr (a
        // position past the end reads the split's first row)
        const __bf16* krow[2];
        const __bf16* vrow[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int rel = 32 * w + 16 * t + lr;
            const int p = p0 + (rel < count ? rel : 0);
            const int64_t d = A.fdesc[(size_t)u * A.fcap + p];
            const int arr = (int)(d >> kDescShift);
            const size_t off = (size_t)(d & kOffMask);
            krow[t] = (const __bf16*)(arr ? A.lk[arr] : a.kc) + off;
            vrow[t] = (const __bf16*)(arr ? A.lv[arr] : a.vc) + off;
        }
        bf16x8_t kA[2][KK], vA[2][KK];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) kA[t][kk] = *(const bf16x8_t*)(krow[t] + 32 * kk + 8 * lg);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) vA[t][kk] = *(const bf16x8_t*)(vrow[t] + 32 * kk + 8 * lg);
        // s[t][r] = q_{head lr} . k_{row 32w + 16t + 4lg + r}
        f32x4_t s[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA[t][kk], qB[kk], acc, 0, 0, 0);
            s[t] = acc;
        }
        auto rel_of = [&](int t, int r) { return 32 * w + 16 * t + 4 * lg + r; };
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (rel_of(t, r) < count) mx = fmaxf(mx, s[t][r]);
        mx = rows4_max(mx);
        if (lg == 0) s_max[w][lr] = mx;
        __syncthreads();
        float mh = s_max[0][lr];
#pragma unroll
        for (int i = 1; i < kWaves; ++i) mh = fmaxf(mh, s_max[i][lr]);
        const float m2 = mh * a.tau_log2e;
        bf16x8_t P;
        float lsum = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pv = rel_of(t, r) < count ? exp2f(s[t][r] * a.tau_log2e - m2) : 0.f;
                const __bf16 pb = (__bf16)pv;
                lsum += (float)pb;
                P[4 * t + r] = pb;
            }
        lsum = rows4_sum(lsum);
        f32x4_t o[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        // V transposed through LDS: V[row 16t + lr][32kk + 8lg + i] -> vt[d][16t + lr]
        __bf16* vt = (__bf16*)smem + (size_t)w * D * LDW;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                for (int i = 0; i < 8; ++i) vt[(32 * kk + 8 * lg + i) * LDW + 16 * t + lr] = vA[t][kk][i];
        __syncthreads();
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const __bf16* col = vt + (16 * db + lr) * LDW;
            const bf16x4_t lo = *(const bf16x4_t*)(col + 4 * lg);
            const bf16x4_t hi = *(const bf16x4_t*)(col + 16 + 4 * lg);
            bf16x8_t vb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vb[i] = lo[i];
                vb[4 + i] = hi[i];
            }
            o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(P, vb, o[db], 0, 0, 0);
        }
        __syncthreads();
        // the wavefronts' sums: o[db][r] is head 4lg + r, column 16db + lr
        float* red = (float*)smem;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = 4 * lg + r;
                if (h < G) red[((size_t)w * 16 + h) * D + 16 * db + lr] = o[db][r];
            }
        if (lg == 0) s_sum[w][lr] = lsum;
        __syncthreads();
        for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
            const int h = e / D, d = e - h * D;
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < kWaves; ++i) acc += red[((size_t)i * 16 + h) * D + d];
            put_acc(pbase * D + e, acc);
        }
        if (threadIdx.x < (unsigned)G) {
            const int h = threadIdx.x;
            float l = 0.f, mm = s_max[0][h];
#pragma unroll
            for (int i = 0; i < kWaves; ++i) {
                l += s_sum[i][h];
                mm = fmaxf(mm, s_max[i][h]);
            }
            put_ml(pbase + h, make_float2(mm * a.tau_log2e, l));
        }
    }
    if (!dev) return;  // grid-uniform
    // count this workgroup in once its partial's stores have completed; the
    // unit's last one merges
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev =
            __hip_atomic_fetch_add(A.uctr + u, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev + 1 == gridDim.x;
    }
    __syncthreads();
    if (!s_last) return;
    merge_unit_block(A, u, (float*)smem, (int)(sizeof(smem) / (16 * sizeof(float))));
    if (threadIdx.x == 0) st_dev(A.uctr + u, 0u);  // zero again for the next call
}

// The top level's keys and attention: every top-level row (the whole gist
// list when there is no meta level).  Workgroup `split` of a unit takes the
// 128-row blocks split, split + S_top, ...; each wavefront keeps a running
// per-head maximum, normaliser and output over its 32 rows of every block
// (online softmax, the output rescaled when the maximum moves), and the four
// wavefronts' states are combined into the workgroup's partial at the end.
// S_top is capped, so a long top level gives few partials to merge.
template <int D>
__global__ __launch_bounds__(256) void lv_top_kernel(LvArgs A) {
    constexpr int KK = D / 32, DB = D / 16, LDW = 32 + 4;
    constexpr int VT = kWaves * D * LDW * 2, RED = kWaves * 16 * D * 4;
    __shared__ __attribute__((aligned(16))) unsigned char smem[VT > RED ? VT : RED];
    __shared__ float s_max[kWaves][16], s_sum[kWaves][16];
    const Args& a = A.a;
    const int u = blockIdx.y, split = blockIdx.x;
    const int b = u / a.Hkv, g = u - b * a.Hkv;
    const int G = a.G;
    const int len = top_count(A, b);
    const int nblk = (len + kRows - 1) / kRows;
    const size_t pbase = ((size_t)u * A.NS + split) * G;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 15, lg = lane >> 4;
    float* keys = A.keys + ((size_t)A.L * a.B * a.Hkv + u) * A.cap;
    bf16x8_t qB[KK];
    load_q<D>(a, b, g, lr, lg, qB);
    float m_run = -INFINITY, l_run = 0.f;  // head lr, exp2 domain
    f32x4_t o[DB];                          // o[db][r]: head 4lg + r, column 16db + lr
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    __bf16* vt = (__bf16*)smem + (size_t)w * D * LDW;
    for (int blk = split; blk < nblk; blk += gridDim.x) {
        const int p0 = blk * kRows;
        const int count = min(kRows, len - p0);
        const __bf16* krow[2];
        const __bf16* vrow[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int rel = 32 * w + 16 * t + lr;
            const int64_t d = entry_desc(A, A.L, b, g, p0 + (rel < count ? rel : 0));
            const int arr = (int)(d >> kDescShift);
            const size_t off = (size_t)(d & kOffMask);
            krow[t] = (const __bf16*)(arr ? A.lk[arr] : a.kc) + off;
            vrow[t] = (const __bf16*)(arr ? A.lv[arr] : a.vc) + off;
        }
        bf16x8_t kA[2][KK], vA[2][KK];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) kA[t][kk] = *(const bf16x8_t*)(krow[t] + 32 * kk + 8 * lg);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) vA[t][kk] = *(const bf16x8_t*)(vrow[t] + 32 * kk + 8 * lg);
        f32x4_t s[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA[t][kk], qB[kk], acc, 0, 0, 0);
            s[t] = acc;
        }
        {
            int krel;
            const float kv = tile_keys(s, lr, lg, a.tau, krel);
            if (krel >= 0 && 32 * w + krel < count) keys[p0 + 32 * w + krel] = kv;
        }
        auto rel_of = [&](int t, int r) { return 32 * w + 16 * t + 4 * lg + r; };
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (rel_of(t, r) < count) mx = fmaxf(mx, s[t][r]);
        mx = rows4_max(mx) * a.tau_log2e;
        const float m_new = fmaxf(m_run, mx);
        // the factor that moves this head's state to the new maximum (1 while
        // the wavefront has seen no row)
        const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
        bf16x8_t P;
        float lsum = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pv = rel_of(t, r) < count ? exp2f(s[t][r] * a.tau_log2e - m_new) : 0.f;
                const __bf16 pb = (__bf16)pv;
                lsum += (float)pb;
                P[4 * t + r] = pb;
            }
        l_run = l_run * alpha + rows4_sum(lsum);
        m_run = m_new;
        // the output's rows are heads 4lg + r: their factors from lanes 4lg + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float ar = __shfl(alpha, 4 * lg + r);
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db][r] *= ar;
        }
        // V transposed through this wavefront's LDS tile
        __syncthreads();  // the previous block's reads of the tile are done
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                for (int i = 0; i < 8; ++i) vt[(32 * kk + 8 * lg + i) * LDW + 16 * t + lr] = vA[t][kk][i];
        __syncthreads();
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const __bf16* col = vt + (16 * db + lr) * LDW;
            const bf16x4_t lo = *(const bf16x4_t*)(col + 4 * lg);
            const bf16x4_t hi = *(const bf16x4_t*)(col + 16 + 4 * lg);
            bf16x8_t vb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vb[i] = lo[i];
                vb[4 + i] = hi[i];
            }
            o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(P, vb, o[db], 0, 0, 0);
        }
    }
    // combine the wavefronts: per head the largest maximum, the others' sums
    // and outputs rescaled to it
    __syncthreads();  // the V tiles are free
    if (lg == 0) {
        s_max[w][lr] = m_run;
        s_sum[w][lr] = l_run;
    }
    __syncthreads();
    float* red = (float*)smem;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = 4 * lg + r;
        if (h < G) {
            float M = s_max[0][h];
#pragma unroll
            for (int i = 1; i < kWaves; ++i) M = fmaxf(M, s_max[i][h]);
            const float f = s_max[w][h] == -INFINITY ? 0.f : exp2f(s_max[w][h] - M);
#pragma unroll
            for (int db = 0; db < DB; ++db) red[((size_t)w * 16 + h) * D + 16 * db + lr] = o[db][r] * f;
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
        const int h = e / D, d = e - h * D;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) acc += red[((size_t)i * 16 + h) * D + d];
        a.part_acc[pbase * D + e] = acc;
    }
    if (threadIdx.x < (unsigned)G) {
        const int h = threadIdx.x;
        float M = s_max[0][h];
#pragma unroll
        for (int i = 1; i < kWaves; ++i) M = fmaxf(M, s_max[i][h]);
        float l = 0.f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i)
            if (s_max[i][h] != -INFINITY) l += s_sum[i][h] * exp2f(s_max[i][h] - M);
        a.part_ml[pbase + h] = make_float2(M, l);
    }
}

template <int D>
__global__ __launch_bounds__(256) void lv_attn_final_kernel(LvArgs A, int slot0) {
    lv_attn_body<D>(A, slot0);
}

// Number of ascending entries of sel[0..k) below `bound`.
__device__ inline int count_below(const int32_t* sel, int k, int bound) {
    int lo = 0, hi = k;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sel[mid] < bound) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}


// Top-k of one list by the chain's workgroup: lists of up to 1024 keys by
// wavefront 0 alone (wave_topk: no barriers), longer ones by the whole block.
// The result count goes through LDS; on return every thread has it and the
// selection is written.
template <typename KeyPtr, typename IdPtr, typename OutPtr>
__device__ inline int chain_topk(KeyPtr keys, IdPtr ids, int n, int k, OutPtr out,
                                 SelectSmem<kSelThreads>& sh, int* s_keff) {
    if (n > 1024) return block_topk<kSelThreads>(keys, ids, n, k, out, false, sh);
    if (threadIdx.x < 64) {
        int r;
        if (n <= 256) r = wave_topk<4>(keys, ids, n, k, out);
        else if (n <= 512) r = wave_topk<8>(keys, ids, n, k, out);
        else r = wave_topk<16>(keys, ids, n, k, out);
        if (threadIdx.x == 0) *s_keff = r;
    }
    __syncthreads();
    return *s_keff;
}

// The select chain of one unit, one workgroup of 512 threads: from the top
// level down, the level's top-k (its keys from the top-level pass or from the
// previous iteration), then the next level's candidates (the children of the
// kept entries, ascending, then the entries past the level's last complete
// group): their ids and routing keys (MFMA; each wavefront issues the loads
// of up to 64 rows at once); at the gists, the final attention list.
// Segments of the final list: raw rows of the kept chunks, the raw tail,
// (L >= 1) the kept gists inside complete groups and the gists past the last
// one, then for each level 1 <= l' < L its kept entries inside complete
// groups and its entries past the last one.
// Below the top level the lists live in LDS when every candidate list fits
// (cap <= kChainCap) and the kept ids of all levels do (A.chain_lds): the
// chain then touches global memory only for the top level's keys, the
// candidates' K rows and its outputs.  Otherwise every level has key, id and
// selection buffers of its own in the workspace (no address is written twice
// in the kernel).  The unit's block-table row is read into LDS up front when
// it has at most kChainBt pages.
template <int D, bool LDS, bool BTL>
__global__ __launch_bounds__(kSelThreads) void lv_chain_kernel(LvArgs A) {
    constexpr int KK = D / 32, NW = kSelThreads / 64, U = 4;  // U tiles of 16 rows per wavefront
    __shared__ SelectSmem<kSelThreads> sh;
    __shared__ int seg[2 * kMaxLevels + 8];
    __shared__ int cnt[kMaxLevels + 2];  // entries per level, then the raw tail
    __shared__ int kept[kMaxLevels + 1];  // kept entries per level
    __shared__ int s_keff;
    __shared__ float s_keys[kChainCap];
    __shared__ int32_t s_ids[kChainCap];
    __shared__ int32_t s_sel[kChainSel];
    __shared__ int32_t s_bt[kChainBt];
    const Args& a = A.a;
    const int u = blockIdx.x, tid = threadIdx.x;
    const int b = u / a.Hkv, g = u - b * a.Hkv;
    const int lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
    const size_t units = (size_t)a.B * a.Hkv;
    constexpr bool lds = LDS;
    const int32_t* btg = a.bt + (size_t)b * a.max_pages;
    if (BTL)
        for (int i = tid; i < a.max_pages; i += kSelThreads) s_bt[i] = btg[i];
    if (tid == 0) {
        int c[kMaxLevels + 1], t;
        level_counts(A, b, c, t);
#pragma unroll
        for (int l = 0; l <= kMaxLevels; ++l) cnt[l] = c[l];
        cnt[kMaxLevels + 1] = t;
    }
    __syncthreads();
    const int tail = cnt[kMaxLevels + 1];
    // element offset of logical slot s of this unit (block-table row btrow)
    auto slot_off = [&](int s) -> size_t {
        const int lp = s / a.spp, off = s - lp * a.spp;
        const int phys = BTL ? s_bt[lp] : btg[lp];
        return (((size_t)phys * a.Hkv + g) * a.spp + off) * (size_t)a.D;
    };
    auto desc_of = [&](int l, int id) -> int64_t {
        if (l == 0) return (int64_t)slot_off(id * (a.C + 1) + a.C);
        return entry_desc(A, l, b, g, id);
    };
    // kept ids of level l: in LDS at the sum of the lower levels' k
    auto sel_of = [&](int l) -> int32_t* {
        if (!lds) return A.sel[l] + (size_t)u * A.topk[l];
        int o = 0;
        for (int i = 0; i < l; ++i) o += A.topk[i];
        return s_sel + o;
    };
    bf16x8_t qB[KK];
    load_q<D>(a, b, g, lr, lg, qB);
    // Routing keys (and, with iout, ids) of positions [0, nc) of a list of
    // level cl entries, position p holding entry id_at(p): every wavefront
    // issues the loads of up to 16U rows at once, then scores them on MFMA.
    auto score = [&](int cl, int nc, auto id_at, float* kout, int32_t* iout) {
        for (int p0 = 16 * U * w; p0 < nc; p0 += 16 * U * NW) {
            int id[U];
#pragma unroll
            for (int t = 0; t < U; ++t) {
                const int rel = 16 * t + lr;
                id[t] = id_at(p0 + rel < nc ? p0 + rel : p0);  // past the end: the pass's first row
            }
            const __bf16* krow[U];
#pragma unroll
            for (int t = 0; t < U; ++t) {
                const int64_t d = desc_of(cl, id[t]);
                const int arr = (int)(d >> kDescShift);
                krow[t] = (const __bf16*)(arr ? A.lk[arr] : a.kc) + (size_t)(d & kOffMask);
            }
            bf16x8_t kA[U][KK];
#pragma unroll
            for (int t = 0; t < U; ++t)
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) kA[t][kk] = *(const bf16x8_t*)(krow[t] + 32 * kk + 8 * lg);
            if (iout) {
#pragma unroll
                for (int t = 0; t < U; ++t)
                    if (lg == 0 && p0 + 16 * t + lr < nc) iout[p0 + 16 * t + lr] = id[t];
            }
#pragma unroll
            for (int h2 = 0; h2 < U / 2; ++h2) {
                f32x4_t s[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA[2 * h2 + t][kk], qB[kk], acc, 0, 0, 0);
                    s[t] = acc;
                }
                int krel;
                const float kv = tile_keys(s, lr, lg, a.tau, krel);
                const int q = p0 + 32 * h2 + krel;
                if (krel >= 0 && q < nc) kout[q] = kv;
            }
        }
        __syncthreads();  // the list's keys and ids are written
    };
    float* const top_keys = A.keys + ((size_t)A.L * units + u) * A.cap;
    if (A.fold_top)  // the top level's keys here (its attention is in the final list)
        score(A.L, cnt[A.L], [](int p) { return p; }, lds ? s_keys : top_keys, (int32_t*)nullptr);
    int n = cnt[A.L], keff = 0;
    for (int l = A.L; l >= 0; --l) {
        const int k = A.topk[l];
        int32_t* sel = sel_of(l);
        if (l == A.L && !(lds && A.fold_top))
            keff = chain_topk(top_keys, (const int32_t*)nullptr, n, k, sel, sh, &s_keff);
        else if (l == A.L)
            keff = chain_topk(s_keys, (const int32_t*)nullptr, n, k, sel, sh, &s_keff);
        else if (lds)
            keff = chain_topk(s_keys, s_ids, n, k, sel, sh, &s_keff);
        else
            keff = chain_topk(A.keys + ((size_t)l * units + u) * A.cap,
                              A.cid + ((size_t)l * units + u) * A.cap, n, k, sel, sh, &s_keff);
        if (tid == 0) kept[l] = keff;
        __syncthreads();  // every thread's entries of sel are written
        if (l == 0) break;
        const int cl = l - 1, R = A.fan[l];
        const int nk = keff * R, past = cnt[l] * R;
        const int nc = nk + (cnt[cl] - past);
        score(cl, nc, [&](int p) { return p < nk ? sel[p / R] * R + (p - (p / R) * R) : past + (p - nk); },
              lds ? s_keys : A.keys + ((size_t)cl * units + u) * A.cap,
              lds ? s_ids : A.cid + ((size_t)cl * units + u) * A.cap);
        n = nc;
    }
    // the gists: the final list
    const int32_t* sel = sel_of(0);
    const int C = a.C, n0 = cnt[0];
    if (tid == 0) {
        int at = keff * C + tail;
        seg[0] = at;
        if (A.L >= 1) {
            const int past0 = cnt[1] * A.fan[1];
            const int e0 = count_below(sel, keff, past0);
            seg[1] = e0;
            seg[2] = past0;
            at += e0 + (n0 - past0);
            for (int lp = 1; lp < A.L; ++lp) {
                // the kept entries of level lp are a prefix of its selection (-1 padded)
                const int32_t* sl = sel_of(lp);
                const int past = cnt[lp + 1] * A.fan[lp + 1];
                const int e = count_below(sl, kept[lp], past);
                seg[2 + 2 * lp] = at;
                seg[3 + 2 * lp] = e;
                at += e + (cnt[lp] - past);
            }
        }
        seg[2 * kMaxLevels + 6] = at;  // (folded top level) its entries
        if (A.fold_top) at += cnt[A.L];
        seg[2 * kMaxLevels + 7] = at;
    }
    __syncthreads();
    int64_t* fd = A.fdesc + (size_t)u * A.fcap;
    const int nraw = keff * C;
    for (int p = tid; p < nraw + tail; p += kSelThreads) {
        int slot;
        if (p < nraw) {
            const int i = p / C;
            slot = sel[i] * (C + 1) + (p - i * C);
        } else {
            slot = n0 * (C + 1) + (p - nraw);
        }
        fd[p] = (int64_t)slot_off(slot);
    }
    if (A.L >= 1) {
        const int base = nraw + tail, e0 = seg[1], past0 = seg[2];
        for (int p = tid; p < e0 + (n0 - past0); p += kSelThreads)
            fd[base + p] = desc_of(0, p < e0 ? sel[p] : past0 + (p - e0));
        for (int lp = 1; lp < A.L; ++lp) {
            const int32_t* sl = sel_of(lp);
            const int at = seg[2 + 2 * lp], e = seg[3 + 2 * lp];
            const int past = cnt[lp + 1] * A.fan[lp + 1];
            for (int p = tid; p < e + (cnt[lp] - past); p += kSelThreads)
                fd[at + p] = entry_desc(A, lp, b, g, p < e ? sl[p] : past + (p - e));
        }
    }
    if (A.fold_top) {
        const int at = seg[2 * kMaxLevels + 6];
        for (int p = tid; p < cnt[A.L]; p += kSelThreads) fd[at + p] = desc_of(A.L, p);
    }
    if (tid == 0) A.nfin[u] = seg[2 * kMaxLevels + 7];
    // the caller's copies of the kept ids
    for (int l = 0; l <= A.L; ++l)
        if (A.usel[l]) {
            const int32_t* sl = sel_of(l);
            for (int i = tid; i < A.topk[l]; i += kSelThreads) A.usel[l][(size_t)u * A.topk[l] + i] = sl[i];
        }
}

// Max-rescale merge of a unit's partial slots [0, NS) into the output (bf16,
// rounded to nearest even); an empty set gives zeros.  One workgroup per
// (head, unit).
__global__ __launch_bounds__(256) void lv_merge_kernel(LvArgs A) {
    __shared__ float2 red[4][64];
    __shared__ float s_m[4], s_l[4];
    const Args& a = A.a;
    const int h = blockIdx.x, u = blockIdx.y;
    const int b = u / a.Hkv, g = u - b * a.Hkv;
    const int G = a.G, D = a.D, NS = A.NS;
    const float2* ml = a.part_ml + (size_t)u * NS * G;
    const float* acc = a.part_acc + (size_t)u * NS * G * D;
    const int sg = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float m = -INFINITY;
    for (int i = threadIdx.x; i < NS; i += blockDim.x) m = fmaxf(m, ml[(size_t)i * G + h].x);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) s_m[sg] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    float l = 0.f;
    if (M != -INFINITY)
        for (int i = threadIdx.x; i < NS; i += blockDim.x) {
            const float2 v = ml[(size_t)i * G + h];
            if (v.x != -INFINITY) l += v.y * exp2f(v.x - M);
        }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) s_l[sg] = l;
    __syncthreads();
    const float lam = s_l[0] + s_l[1] + s_l[2] + s_l[3];
    float2 o = make_float2(0.f, 0.f);
    if (M != -INFINITY && 2 * lane < D) {
        for (int i = sg; i < NS; i += 4) {
            const float mi = ml[(size_t)i * G + h].x;
            if (mi == -INFINITY) continue;
            const float sc = exp2f(mi - M);
            const float2 v = *(const float2*)(acc + ((size_t)i * G + h) * D + 2 * lane);
            o.x += v.x * sc;
            o.y += v.y * sc;
        }
    }
    red[sg][lane] = o;
    __syncthreads();
    if (sg == 0 && 2 * lane < D) {
        float2 t = red[0][lane];
        for (int j = 1; j < 4; ++j) {
            t.x += red[j][lane].x;
            t.y += red[j][lane].y;
        }
        const float inv = (M != -INFINITY && lam > 0.f) ? 1.f / lam : 0.f;
        __bf16* out = (__bf16*)a.out + ((size_t)b * a.Hq + (size_t)g * G + h) * D;
        out[2 * lane] = (__bf16)(t.x * inv);
        out[2 * lane + 1] = (__bf16)(t.y * inv);
    }
}

template <int D>
hipError_t launch_d(const LvArgs& A, hipStream_t st) {
    const int units = A.a.B * A.a.Hkv;
    hipError_t e;
    if (!A.fold_top) {
        // the top level: keys and attention over all its entries
        hipLaunchKernelGGL((lv_top_kernel<D>), dim3(A.S_top, units), dim3(256), 0, st, A);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const bool btl = A.a.max_pages <= kChainBt;
    if (A.chain_lds) {
        if (btl)
            hipLaunchKernelGGL((lv_chain_kernel<D, true, true>), dim3(units), dim3(kSelThreads), 0, st, A);
        else
            hipLaunchKernelGGL((lv_chain_kernel<D, true, false>), dim3(units), dim3(kSelThreads), 0, st, A);
    } else {
        if (btl)
            hipLaunchKernelGGL((lv_chain_kernel<D, false, true>), dim3(units), dim3(kSelThreads), 0, st, A);
        else
            hipLaunchKernelGGL((lv_chain_kernel<D, false, false>), dim3(units), dim3(kSelThreads), 0, st, A);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((lv_attn_final_kernel<D>), dim3(A.S_fin, units), dim3(256), 0, st, A, A.S_top);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (!A.uctr) hipLaunchKernelGGL(lv_merge_kernel, dim3(A.a.G, units), dim3(256), 0, st, A);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_levels(const LvArgs& A, hipStream_t st) {
    return A.a.D == 64 ? launch_d<64>(A, st) : launch_d<128>(A, st);
}

}  // namespace gsa
