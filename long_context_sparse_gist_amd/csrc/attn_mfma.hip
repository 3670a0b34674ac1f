// Group-batched MFMA attention over a token list (bf16 caches, fp32 math).
//
// One workgroup = 4 wavefronts = one split of one unit's token list.  Each
// wavefront owns NB blocks of 32 tokens.  For the G query heads of a GQA
// group (padded to 16) the scores are one 16x16x32 MFMA contraction per 16
// tokens and 32 head-dim elements:
//     S^T[token][head] = K[token][:] . Q^T[:][head]
// so the K rows feed the A operand straight from global memory (lane l reads
// 16 contiguous bytes of row l%16).  The routing key of a gist is the row sum
// of S^T over the real heads times the softmax scale.  The probabilities P
// (rounded to bf16) then multiply V as a second contraction
//     O[head][d] = P[head][token] . V[token][d]
// whose B operand needs 8 tokens of one V column per lane; V is transposed
// through LDS for that.  Softmax is two-pass inside the split (the split's
// scores are all in registers), so no running rescale is needed; splits are
// combined later by the online-softmax merge.
#include "gsa_lists.h"

namespace gsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kNB = 1;  // 32-token blocks per wavefront

__device__ inline float dpp_f(float x, int ctrl_id) {
    int v = __builtin_bit_cast(int, x);
    int r;
    switch (ctrl_id) {
        case 0: r = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); break;   // quad [1,0,3,2]
        case 1: r = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); break;   // quad [2,3,0,1]
        case 2: r = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false); break;  // row half mirror
        default: r = __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); break; // row mirror
    }
    return __builtin_bit_cast(float, r);
}

// Sum over the 16 lanes of a row; every lane of the row gets the total.
__device__ inline float rowsum16(float x) {
    x += dpp_f(x, 0);
    x += dpp_f(x, 1);
    x += dpp_f(x, 2);
    x += dpp_f(x, 3);
    return x;
}

template <int D, int NB>
__global__ __launch_bounds__(256) void attn_mfma_kernel(Args a, int kind, int hier) {
    constexpr int KK = D / 32;       // k-steps over head_dim
    constexpr int DB = D / 16;       // 16-wide output column blocks
    constexpr int TW = 32 * NB;      // tokens per wavefront
    constexpr int TB = kWaves * TW;  // tokens per workgroup
    constexpr int LDW = 32 + 4;      // row length (bf16) of transposed V in LDS
    constexpr int VT_BYTES = kWaves * D * LDW * 2;
    constexpr int RED_BYTES = kWaves * 16 * D * 4;
    constexpr int SMEM = VT_BYTES > RED_BYTES ? VT_BYTES : RED_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
    __shared__ float s_max[kWaves][16];
    __shared__ float s_sum[kWaves][16];
    __shared__ float s_esum[kWaves][16];

    const int u = blockIdx.y;
    const int split = blockIdx.x;
    ListCtx c;
    make_ctx(a, kind, u, hier != 0, c);
    const int p0 = split * TB;
    const int count = min(TB, c.len - p0);
    if (count <= 0) return;  // block-uniform

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int G = a.G;

    const bool want_keys = kind != kListUnfolded;
    const bool want_attn = kind == kListUnfolded || kind == kListMeta ||
                           (kind == kListGists && !(a.flags & kFlagSelectedGists));

    // Q^T operand: column = head lr (zero for padding heads), k = 8*lg + i
    bf16x8_t qB[KK];
    {
        const __bf16* qp = (const __bf16*)a.q + ((size_t)c.b * a.Hq + (size_t)c.g * G + lr) * D;
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

    // rows of this lane: block blk, half t -> list position p0 + w*TW + 32*blk + 16*t + lr
    const __bf16* krow[NB][2];
    const __bf16* vrow[NB][2];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            int rel = w * TW + 32 * blk + 16 * t + lr;
            int p = p0 + (rel < count ? rel : 0);
            const void *kb, *vb;
            size_t off = list_row(a, kind, c, hier != 0, p, &kb, &vb);
            krow[blk][t] = (const __bf16*)kb + off;
            vrow[blk][t] = (const __bf16*)vb + off;
        }

    bf16x8_t kA[NB][2][KK];
    bf16x8_t vA[NB][2][KK];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                kA[blk][t][kk] = *(const bf16x8_t*)(krow[blk][t] + 32 * kk + 8 * lg);
    if (want_attn) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    vA[blk][t][kk] = *(const bf16x8_t*)(vrow[blk][t] + 32 * kk + 8 * lg);
    }

    // scores: s[blk][t][r] = q_{head lr} . k_{token (blk, t, row 4*lg + r)}
    f32x4_t s[NB][2];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA[blk][t][kk], qB[kk], acc, 0, 0, 0);
            s[blk][t] = acc;
        }

    auto rel_of = [&](int blk, int t, int r) { return w * TW + 32 * blk + 16 * t + 4 * lg + r; };

    if (want_keys) {
        // routing key: tau * sum over the group's heads (padding heads are 0)
        float kv = 0.f;
        int krel = -1;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float x = rowsum16(s[blk][t][r]) * a.tau;
                    int v = blk * 8 + t * 4 + r;
                    if (v == lr) { kv = x; krel = rel_of(blk, t, r); }
                }
        if (kind == kListGists && a.hlog && lr < G) {
            // per-head logits for the sum-of-probabilities key (this lane: head lr)
            float* hl = a.hlog + ((size_t)u * G + lr) * a.key_stride + p0;
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (rel_of(blk, t, r) < count) hl[rel_of(blk, t, r)] = s[blk][t][r] * a.tau;
        }
        if (krel >= 0 && krel < count) {
            int p = p0 + krel;
            if (kind == kListGists) {
                a.keys[(size_t)u * a.key_stride + p] = kv;
            } else if (kind == kListMeta) {
                a.mkeys[(size_t)u * a.max_meta + p] = kv;
            } else {
                a.ckeys[(size_t)u * a.cand_stride + p] = kv;
                a.cand[(size_t)u * a.cand_stride + p] = cand_gist(a, c, p);
            }
        }
    }
    if (!want_attn) return;  // block-uniform

    // per-head maximum over the split (raw dot units)
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (rel_of(blk, t, r) < count) mx = fmaxf(mx, s[blk][t][r]);
    mx = rows4_max(mx);
    if (lg == 0) s_max[w][lr] = mx;
    __syncthreads();
    float mh = s_max[0][lr];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) mh = fmaxf(mh, s_max[i][lr]);
    const float m2 = mh * a.tau_log2e;

    // probabilities as the PV A operand: row = head lr, k = 8*lg + j <-> token (t=j/4, row 4*lg + j%4)
    bf16x8_t P[NB];
    float lsum = 0.f, esum = 0.f;  // sums of the bf16 PV operand and of the unrounded probabilities
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float pv = (rel_of(blk, t, r) < count) ? exp2f(s[blk][t][r] * a.tau_log2e - m2) : 0.f;
                __bf16 pb = (__bf16)pv;
                lsum += (float)pb;
                esum += pv;
                P[blk][4 * t + r] = pb;
            }
    lsum = rows4_sum(lsum);
    esum = rows4_sum(esum);

    f32x4_t o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    __bf16* vt = (__bf16*)smem + (size_t)w * D * LDW;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
        // transpose: V[token (t, row lr)][32*kk + 8*lg + i] -> vt[d][16*t + lr]
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    vt[(32 * kk + 8 * lg + i) * LDW + 16 * t + lr] = vA[blk][t][kk][i];
        __syncthreads();
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const __bf16* col = vt + (16 * db + lr) * LDW;
            bf16x4_t lo = *(const bf16x4_t*)(col + 4 * lg);
            bf16x4_t hi = *(const bf16x4_t*)(col + 16 + 4 * lg);
            bf16x8_t vb;
#pragma unroll
            for (int i = 0; i < 4; ++i) { vb[i] = lo[i]; vb[4 + i] = hi[i]; }
            o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(P[blk], vb, o[db], 0, 0, 0);
        }
        __syncthreads();
    }

    // combine the wavefronts: o[db][r] is head 4*lg + r, column 16*db + lr
    float* red = (float*)smem;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int h = 4 * lg + r;
            if (h < G) red[((size_t)w * 16 + h) * D + 16 * db + lr] = o[db][r];
        }
    if (lg == 0) {
        s_sum[w][lr] = lsum;
        s_esum[w][lr] = esum;
    }
    __syncthreads();
    const int slot = partial_slot(a, kind, split);
    const size_t pbase = ((size_t)u * a.NS + slot) * G;
    for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
        int h = e / D, d = e - h * D;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) acc += red[((size_t)i * 16 + h) * D + d];
        a.part_acc[(pbase + h) * D + d] = acc;
    }
    if (threadIdx.x < G) {
        int h = threadIdx.x;
        float l = 0.f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) l += s_sum[i][h];
        float mm = s_max[0][h];
#pragma unroll
        for (int i = 1; i < kWaves; ++i) mm = fmaxf(mm, s_max[i][h]);
        a.part_ml[pbase + h] = make_float2(mm * a.tau_log2e, l);
        if (kind == kListGists && a.hsum) {
            float le = 0.f;
#pragma unroll
            for (int i = 0; i < kWaves; ++i) le += s_esum[i][h];
            a.hsum[pbase + h] = le;
        }
    }
}

}  // namespace

int mfma_tokens_per_block(int /*D*/) { return kWaves * 32 * kNB; }

hipError_t launch_attn_mfma(const Args& a, int kind, int splits, hipStream_t st) {
    dim3 grid(splits, a.B * a.Hkv);
    int hier = a.km != nullptr;
    if (a.D == 64)
        hipLaunchKernelGGL((attn_mfma_kernel<64, kNB>), grid, dim3(256), 0, st, a, kind, hier);
    else
        hipLaunchKernelGGL((attn_mfma_kernel<128, kNB>), grid, dim3(256), 0, st, a, kind, hier);
    return hipGetLastError();
}

}  // namespace gsa
