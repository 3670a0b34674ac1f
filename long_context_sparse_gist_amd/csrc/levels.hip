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
// Launches (bf16, MFMA): the top level's attention and keys, then per level a
// select that writes the next level's candidate list as row descriptors,
// a keys-only pass over it, ..., the gist-level select writes the final
// attention list, one attention pass over it, and a merge of the partials.
// Every list is a per-unit array of row descriptors (array id << 56 | element
// offset), so one attention kernel serves every level and the final set.
#include "gsa_lists.h"
#include "gsa_levels.h"
#include "gsa_select.h"

namespace gsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kRows = 32 * kWaves;  // rows per attention workgroup
constexpr int kSelThreads = 512;
constexpr int64_t kOffMask = (1ll << kDescShift) - 1;

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

// Descriptor of entry `id` of level l of unit (b, g): level 0 is a gist in the
// paged cache, a level l >= 1 entry a row of that level's array.
__device__ inline int64_t entry_desc(const LvArgs& A, int l, int b, int g, int id) {
    if (l == 0) return (int64_t)slot_offset(A.a, b, g, id * (A.a.C + 1) + A.a.C);
    const size_t off = (((size_t)b * A.a.Hkv + g) * A.maxe[l] + id) * (size_t)A.a.D;
    return ((int64_t)l << kDescShift) | (int64_t)off;
}

// Attention and / or routing keys over one list per unit.
//   list < 0   dense: every entry of level -list - 1 (the top level)
//   list 0, 1  the candidate list in ping-pong buffer `list`
//   list 2     the final attention list
// keys: routing keys of the list's rows into A.keys; attn: one partial per
// split into partial slot slot0 + split (an empty split writes an empty one).
template <int D>
__global__ __launch_bounds__(256) void lv_attn_kernel(LvArgs A, int list, int keys, int attn,
                                                      int slot0) {
    constexpr int KK = D / 32, DB = D / 16, LDW = 32 + 4;
    constexpr int VT = kWaves * D * LDW * 2, RED = kWaves * 16 * D * 4;
    __shared__ __attribute__((aligned(16))) unsigned char smem[VT > RED ? VT : RED];
    __shared__ float s_max[kWaves][16], s_sum[kWaves][16];
    const Args& a = A.a;
    const int u = blockIdx.y, split = blockIdx.x;
    const int b = u / a.Hkv, g = u - b * a.Hkv;
    const int G = a.G;
    int cnt[kMaxLevels + 1], tail;
    level_counts(A, b, cnt, tail);
    int len;
    if (list < 0) len = cnt[-list - 1];
    else if (list < 2) len = A.ncand[list][u];
    else len = A.nfin[u];
    const int p0 = split * kRows;
    const int count = min(kRows, len - p0);
    const size_t pbase = ((size_t)u * A.NS + slot0 + split) * G;
    if (count <= 0) {
        if (attn) {
            for (int e = threadIdx.x; e < G * D; e += blockDim.x) a.part_acc[pbase * D + e] = 0.f;
            if (threadIdx.x < (unsigned)G) a.part_ml[pbase + threadIdx.x] = make_float2(-INFINITY, 0.f);
        }
        return;
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 15, lg = lane >> 4;

    bf16x8_t qB[KK];
    {
        const __bf16* qp = (const __bf16*)a.q + ((size_t)b * a.Hq + (size_t)g * G + lr) * D;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            if (lr < G) {
                qB[kk] = *(const bf16x8_t*)(qp + 32 * kk + 8 * lg);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) qB[kk][i] = (__bf16)0.0f;
            }
        }
    }
    // rows of this lane: half t -> list position p0 + 32*w + 16*t + lr (a
    // position past the end reads the split's first row)
    const __bf16* krow[2];
    const __bf16* vrow[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int rel = 32 * w + 16 * t + lr;
        const int p = p0 + (rel < count ? rel : 0);
        int64_t d;
        if (list < 0) d = entry_desc(A, -list - 1, b, g, p);
        else if (list < 2) d = A.desc[list][(size_t)u * A.cap + p];
        else d = A.fdesc[(size_t)u * A.fcap + p];
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
    if (attn) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) vA[t][kk] = *(const bf16x8_t*)(vrow[t] + 32 * kk + 8 * lg);
    }
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
    if (keys) {
        // lanes lr < 8 keep one key each: row rel_of(t, r) with 4t + r == lr,
        // the row sum over the group's heads (padding heads score 0)
        float kv = 0.f;
        int krel = -1;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = row16_sum(s[t][r]) * a.tau;
                if (4 * t + r == lr) {
                    kv = x;
                    krel = rel_of(t, r);
                }
            }
        if (krel >= 0 && krel < count) A.keys[(size_t)u * A.cap + p0 + krel] = kv;
    }
    if (!attn) return;  // block-uniform

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
        a.part_acc[pbase * D + e] = acc;
    }
    if (threadIdx.x < (unsigned)G) {
        const int h = threadIdx.x;
        float l = 0.f, mm = s_max[0][h];
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            l += s_sum[i][h];
            mm = fmaxf(mm, s_max[i][h]);
        }
        a.part_ml[pbase + h] = make_float2(mm * a.tau_log2e, l);
    }
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

// Top-k of level l's current list (src < 0: the dense top level; else the
// candidate list in buffer src), then the next list: level l-1's candidates
// into buffer src ^ 1 (the top level writes buffer 0), or, at the gists, the
// final attention list.
__global__ __launch_bounds__(kSelThreads) void lv_select_kernel(LvArgs A, int l, int src) {
    __shared__ SelectSmem<kSelThreads> sh;
    __shared__ int seg[2 * kMaxLevels + 8];
    const Args& a = A.a;
    const int u = blockIdx.x, tid = threadIdx.x;
    const int b = u / a.Hkv, g = u - b * a.Hkv;
    int cnt[kMaxLevels + 1], tail;
    level_counts(A, b, cnt, tail);
    const int k = A.topk[l];
    const int n = src < 0 ? cnt[l] : A.ncand[src][u];
    const float* keys = A.keys + (size_t)u * A.cap;
    const int32_t* ids = src < 0 ? nullptr : A.cid[src] + (size_t)u * A.cap;
    int32_t* sel = A.sel[l] + (size_t)u * k;
    const int keff = block_topk<kSelThreads>(keys, ids, n, k, sel, false, sh);
    __syncthreads();  // every thread's entries of sel are written
    if (A.usel[l])
        for (int i = tid; i < k; i += kSelThreads) A.usel[l][(size_t)u * k + i] = sel[i];
    if (l > 0) {
        // children of the kept entries (ascending), then the entries past the
        // last complete group of level l
        const int R = A.fan[l], dst = src < 0 ? 0 : src ^ 1;
        const int past = cnt[l] * R, ntail = cnt[l - 1] - past;
        int64_t* desc = A.desc[dst] + (size_t)u * A.cap;
        int32_t* cid = A.cid[dst] + (size_t)u * A.cap;
        const int nn = keff * R + ntail;
        for (int p = tid; p < nn; p += kSelThreads) {
            const int id = p < keff * R ? sel[p / R] * R + (p - (p / R) * R) : past + (p - keff * R);
            desc[p] = entry_desc(A, l - 1, b, g, id);
            cid[p] = id;
        }
        if (tid == 0) A.ncand[dst][u] = nn;
        return;
    }
    // the gists: the final list.  Segments: raw rows of the kept chunks, the
    // raw tail, (L >= 1) the kept gists inside complete groups and the gists
    // past the last one, then for each level 1 <= l' < L its kept entries
    // inside complete groups and its entries past the last one.
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
                const int kl = min(A.topk[lp], cnt[lp]);
                // the kept entries of level lp are a prefix of its selection (-1 padded)
                const int32_t* sl = A.sel[lp] + (size_t)u * A.topk[lp];
                const int past = cnt[lp + 1] * A.fan[lp + 1];
                int kk = 0;
                while (kk < kl && sl[kk] >= 0) ++kk;
                const int e = count_below(sl, kk, past);
                seg[2 + 2 * lp] = at;
                seg[3 + 2 * lp] = e;
                at += e + (cnt[lp] - past);
            }
        }
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
        fd[p] = (int64_t)slot_offset(a, b, g, slot);
    }
    if (A.L >= 1) {
        const int base = nraw + tail, e0 = seg[1], past0 = seg[2];
        for (int p = tid; p < e0 + (n0 - past0); p += kSelThreads)
            fd[base + p] = entry_desc(A, 0, b, g, p < e0 ? sel[p] : past0 + (p - e0));
        for (int lp = 1; lp < A.L; ++lp) {
            const int32_t* sl = A.sel[lp] + (size_t)u * A.topk[lp];
            const int at = seg[2 + 2 * lp], e = seg[3 + 2 * lp];
            const int past = cnt[lp + 1] * A.fan[lp + 1];
            for (int p = tid; p < e + (cnt[lp] - past); p += kSelThreads)
                fd[at + p] = entry_desc(A, lp, b, g, p < e ? sl[p] : past + (p - e));
        }
    }
    if (tid == 0) A.nfin[u] = seg[2 * kMaxLevels + 7];
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
hipError_t launch_attn_lv(const LvArgs& A, int list, int splits, int keys, int attn, int slot0,
                          hipStream_t st) {
    hipLaunchKernelGGL((lv_attn_kernel<D>), dim3(splits, A.a.B * A.a.Hkv), dim3(256), 0, st, A, list,
                       keys, attn, slot0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_levels(const LvArgs& A, hipStream_t st) {
    const int units = A.a.B * A.a.Hkv;
    auto attn = [&](int list, int splits, int keys, int att, int slot0) {
        return A.a.D == 64 ? launch_attn_lv<64>(A, list, splits, keys, att, slot0, st)
                           : launch_attn_lv<128>(A, list, splits, keys, att, slot0, st);
    };
    hipError_t e;
    // the top level: keys and attention over all its entries
    if ((e = attn(-A.L - 1, A.S_top, 1, 1, 0)) != hipSuccess) return e;
    int src = -1;
    for (int l = A.L; l >= 0; --l) {
        hipLaunchKernelGGL(lv_select_kernel, dim3(units), dim3(kSelThreads), 0, st, A, l, src);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (l == 0) break;
        src = src < 0 ? 0 : src ^ 1;
        // keys of level l-1's candidates
        if ((e = attn(src, A.S_cand, 1, 0, 0)) != hipSuccess) return e;
    }
    if ((e = attn(2, A.S_fin, 0, 1, A.S_top)) != hipSuccess) return e;
    hipLaunchKernelGGL(lv_merge_kernel, dim3(A.a.G, units), dim3(256), 0, st, A);
    return hipGetLastError();
}

}  // namespace gsa
