// Per-wavefront MFMA attention core (bf16 caches, fp32 math).
//
// A wavefront streams blocks of 32 tokens.  For the G query heads of one GQA
// group (padded to 16 MFMA columns with zero queries) the scores of 16 tokens
// are one 16x16x32 MFMA chain over the head dimension:
//     S^T[token][head] = K[token][:] . Q^T[:][head]
// so the K rows feed the A operand straight from global memory (lane l reads
// 16 contiguous bytes of row l%16).  The probabilities, rounded to bf16, then
// multiply V as a second contraction
//     O[head][d] += P[head][token] . V[token][d]
// whose B operand needs 8 tokens of one V column per lane: V is transposed
// through a wavefront-private LDS tile.  Softmax runs online across blocks
// (running max per head, rescale of O when it grows).
//
// Lane layout (lane = 16*lg + lr):
//   score s[t][r]   head lr, token 16*t + 4*lg + r of the block
//   P operand       row head lr, k = 8*lg + j <-> token 16*(j/4) + 4*lg + j%4
//   O accumulator   o[db][r]: head 4*lg + r, column 16*db + lr
#pragma once

#include "gsa_internal.h"

namespace gsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ inline float dpp_row(float x, int which) {
    int v = __builtin_bit_cast(int, x);
    int r;
    switch (which) {
        case 0: r = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); break;   // quad [1,0,3,2]
        case 1: r = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); break;   // quad [2,3,0,1]
        case 2: r = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false); break;  // row half mirror
        default: r = __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); break; // row mirror
    }
    return __builtin_bit_cast(float, r);
}

// Max over the 16 lanes of a row; every lane of the row gets it.
__device__ inline float rowmax16(float x) {
    x = fmaxf(x, dpp_row(x, 0));
    x = fmaxf(x, dpp_row(x, 1));
    x = fmaxf(x, dpp_row(x, 2));
    x = fmaxf(x, dpp_row(x, 3));
    return x;
}

// Inclusive prefix sum over the 64 lanes of a wavefront (DPP row shifts, then
// row broadcasts of lanes 15 and 31).
// exp2 on the hardware instruction (v_exp_f32: exp2(-inf) = 0, results below
// 2^-126 flush to 0), for softmax weights that are rounded to bf16 anyway
__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline int wave_prefix_incl_dpp(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Sum over the 16 lanes of a row; every lane of the row gets the total.
__device__ inline float rowsum16(float x) {
    x += dpp_row(x, 0);
    x += dpp_row(x, 1);
    x += dpp_row(x, 2);
    x += dpp_row(x, 3);
    return x;
}

// Keep the compiler from moving memory accesses across this point and wait
// for this wavefront's LDS accesses to complete.
__device__ inline void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int D>
struct WaveAttn {
    static constexpr int KK = D / 32;    // k-steps over the head dimension
    static constexpr int DB = D / 16;    // 16-wide output column blocks
    static constexpr int LDW = 32 + 4;   // LDS row length (bf16) of transposed V
    static constexpr int LDS_BYTES = D * LDW * 2;

    bf16x8_t qB[KK];
    f32x4_t o[DB];
    float m;   // running max of the raw dot products of head lr
    float l;   // lane-local running sum of this lane's probabilities

    __device__ inline void init(const __bf16* qgroup, int G, int lr, int lg) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            if (lr < G) {
                qB[kk] = *(const bf16x8_t*)(qgroup + (size_t)lr * D + 32 * kk + 8 * lg);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) qB[kk][i] = (__bf16)0.0f;
            }
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        m = -INFINITY;
        l = 0.f;
    }

    // Scores of one 32-token block from its K operands (token 16*t + lr).
    __device__ inline void scores(const bf16x8_t kA[2][KK], f32x4_t s[2]) const {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA[t][kk], qB[kk], acc, 0, 0, 0);
            s[t] = acc;
        }
    }

    // Online-softmax update for one block and the transpose of its V into the
    // wavefront's LDS tile vt.  nvalid: tokens [0, nvalid) are real (>= 1).
    // Returns the block's probabilities as the PV A operand.
    __device__ inline bf16x8_t softmax_stage(const f32x4_t s[2], const bf16x8_t vA[2][KK],
                                             int nvalid, float tau_log2e, int lr, int lg,
                                             __bf16* vt) {
        float bm = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (16 * t + 4 * lg + r < nvalid) bm = fmaxf(bm, s[t][r]);
        bm = rows4_max(bm);
        const float mnew = fmaxf(m, bm);  // finite: the block has a real token
        const float alpha = exp2_hw((m - mnew) * tau_log2e);  // 0 on the first block
        const float mb = mnew * tau_log2e;
        bf16x8_t P;
        float ls = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float pv = (16 * t + 4 * lg + r < nvalid) ? exp2_hw(s[t][r] * tau_log2e - mb) : 0.f;
                __bf16 pb = (__bf16)pv;
                ls += (float)pb;
                P[4 * t + r] = pb;
            }
        l = l * alpha + ls;
        m = mnew;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float ar = __shfl(alpha, 4 * lg + r);
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db][r] *= ar;
        }
        // V[token 16*t + lr][32*kk + 8*lg + i] -> vt[d][16*t + lr]
        lds_fence();
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    vt[(32 * kk + 8 * lg + i) * LDW + 16 * t + lr] = vA[t][kk][i];
        lds_fence();
        return P;
    }

    // PV product of one block from the transposed V tile.
    __device__ inline void pv_stage(const bf16x8_t& P, int lr, int lg, const __bf16* vt) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const __bf16* col = vt + (16 * db + lr) * LDW;
            bf16x4_t lo = *(const bf16x4_t*)(col + 4 * lg);
            bf16x4_t hi = *(const bf16x4_t*)(col + 16 + 4 * lg);
            bf16x8_t vb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vb[i] = lo[i];
                vb[4 + i] = hi[i];
            }
            o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(P, vb, o[db], 0, 0, 0);
        }
    }

    __device__ static inline void load_rows(const __bf16* base, const size_t off[2], int lg,
                                            bf16x8_t x[2][KK]) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                x[t][kk] = *(const bf16x8_t*)(base + off[t] + 32 * kk + 8 * lg);
    }

    // Stream this wavefront's blocks j < nbw (<= NBW): block j's rows sit at
    // element offsets off[j][t] of kbase / vbase and its first nval[j] tokens
    // are real.  PIPE: K of block j+1 is loaded while block j is scored and V
    // of block j+1 once V of block j sits in LDS (more registers); otherwise
    // each block's loads are issued when its turn comes.  on_scores(j, s) sees
    // every block's scores; attn = false skips V and the PV product.
    template <int NBW, bool PIPE, typename OnScores>
    __device__ inline void stream(const __bf16* kbase, const __bf16* vbase,
                                  const size_t (&off)[NBW][2], const int (&nval)[NBW], int nbw,
                                  bool attn, float tau_log2e, int lr, int lg, __bf16* vt,
                                  OnScores on_scores) {
        if (nbw <= 0) return;
        if constexpr (!PIPE) {
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                if (j >= nbw) break;
                bf16x8_t kb[2][KK], vb[2][KK];
                load_rows(kbase, off[j], lg, kb);
                if (attn) load_rows(vbase, off[j], lg, vb);
                f32x4_t s[2];
                scores(kb, s);
                on_scores(j, s);
                if (attn) {
                    bf16x8_t P = softmax_stage(s, vb, nval[j], tau_log2e, lr, lg, vt);
                    pv_stage(P, lr, lg, vt);
                }
            }
        } else {
            bf16x8_t kb[2][2][KK];
            bf16x8_t vb[2][2][KK];
            load_rows(kbase, off[0], lg, kb[0]);
            if (attn) load_rows(vbase, off[0], lg, vb[0]);
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                if (j >= nbw) break;
                const int cur = j & 1, nxt = (j + 1) & 1;
                const bool more = j + 1 < NBW && j + 1 < nbw;
                if (more) load_rows(kbase, off[j + 1], lg, kb[nxt]);
                f32x4_t s[2];
                scores(kb[cur], s);
                on_scores(j, s);
                if (attn) {
                    bf16x8_t P = softmax_stage(s, vb[cur], nval[j], tau_log2e, lr, lg, vt);
                    if (more) load_rows(vbase, off[j + 1], lg, vb[nxt]);
                    pv_stage(P, lr, lg, vt);
                }
            }
        }
    }
};

// Shared memory of one workgroup's wavefront combination.
struct CombineSmem {
    float wm[4][16];
    float wl[4][16];
};

// Combine the 4 wavefronts' online-softmax states into one partial
// (max in the exp2 domain, sum, weighted V sum) and hand each element to
// `emit_acc(h, d, value)` / `emit_ml(h, m2, l)`.  red: >= 4*G*D floats of LDS
// (may alias the V tiles: a barrier separates their uses).
template <int D, typename WA, typename EmitAcc, typename EmitMl>
__device__ inline void combine_waves(WA& wa, float tau_log2e, int G, float* red,
                                     CombineSmem& cs, EmitAcc emit_acc, EmitMl emit_ml) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    float l = wa.l;
    l = rows4_sum(l);
    if (lg == 0) {
        cs.wm[w][lr] = wa.m;
        cs.wl[w][lr] = l;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = 4 * lg + r;
        float M = fmaxf(fmaxf(cs.wm[0][h], cs.wm[1][h]), fmaxf(cs.wm[2][h], cs.wm[3][h]));
        float sc = (cs.wm[w][h] == -INFINITY) ? 0.f : exp2f((cs.wm[w][h] - M) * tau_log2e);
        if (h < G) {
#pragma unroll
            for (int db = 0; db < WA::DB; ++db)
                red[((size_t)w * G + h) * D + 16 * db + lr] = wa.o[db][r] * sc;
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
        int h = e / D, d = e - h * D;
        emit_acc(h, d, red[(size_t)h * D + d] + red[((size_t)G + h) * D + d] +
                           red[((size_t)2 * G + h) * D + d] + red[((size_t)3 * G + h) * D + d]);
    }
    if (threadIdx.x < (unsigned)G) {
        const int h = threadIdx.x;
        float M = fmaxf(fmaxf(cs.wm[0][h], cs.wm[1][h]), fmaxf(cs.wm[2][h], cs.wm[3][h]));
        float L = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (cs.wm[i][h] != -INFINITY) L += cs.wl[i][h] * exp2f((cs.wm[i][h] - M) * tau_log2e);
        emit_ml(h, M * tau_log2e, L);
    }
    __syncthreads();
}

}  // namespace gsa

namespace gsa {

typedef short v4s16_t __attribute__((ext_vector_type(4)));
typedef short v8s16_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Per-wavefront attention core with V staged through LDS.
//
// A block's 32 V rows go from global memory straight into a wavefront tile
// (global_load_lds_dwordx4: lane l of an instruction writes the tile's 16-byte
// chunk 64*q + l, holding no registers), and the PV product reads its B
// operand back transposed (ds_read_b64_tr_b16: within a group of 16 lanes,
// lane j receives element j%4 of the 8 bytes read by lanes j/4 + 4i, i < 4).
// Tile rows are D bf16; chunk c of row r sits at 16-byte position
// c ^ 2(r mod CPR/2), so the four rows one 16-lane group reads hit different
// banks.  Scores, online softmax and the P operand are those of WaveAttn.
template <int D>
struct WaveAttnL {
    static constexpr int KK = D / 32;        // k-steps over the head dimension
    static constexpr int DB = D / 16;        // 16-wide output column blocks
    static constexpr int CPR = D / 8;        // 16-byte chunks per V row
    static constexpr int TILE_BYTES = 32 * D * 2;

    bf16x8_t qB[KK];
    f32x4_t o[DB];
    float m, l;

    __device__ static inline int swz(int r) { return 2 * (r % (CPR / 2)); }

    __device__ inline void init(const __bf16* qgroup, int G, int lr, int lg) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            if (lr < G) {
                qB[kk] = *(const bf16x8_t*)(qgroup + (size_t)lr * D + 32 * kk + 8 * lg);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) qB[kk][i] = (__bf16)0.0f;
            }
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        m = -INFINITY;
        l = 0.f;
    }

    // Scores of one 32-token block from its K operands (token 16*t + lr).
    __device__ inline void scores(const bf16x8_t kA[2][KK], f32x4_t s[2]) const {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA[t][kk], qB[kk], acc, 0, 0, 0);
            s[t] = acc;
        }
    }

    // Issue the direct loads of one block's V rows into `tile`.  off0 / off1:
    // element offsets (from vbase) of this lane's rows lr and 16 + lr; row r's
    // offset is taken from lane r % 16.
    __device__ inline void load_v(const __bf16* vbase, size_t off0, size_t off1,
                                  unsigned char* tile) const {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int q = 0; q < CPR / 2; ++q) {
            const int f = 64 * q + lane, r = f / CPR, p = f % CPR, c = p ^ swz(r);
            const size_t src = (64 * q) / CPR < 16 ? off0 : off1;  // uniform per q
            const unsigned lo = __shfl((unsigned)src, r % 16), hi = __shfl((unsigned)(src >> 32), r % 16);
            const size_t ro = ((size_t)hi << 32) | lo;
            __builtin_amdgcn_global_load_lds(vbase + ro + 8 * c, (lds_void_t*)(tile + 1024 * q), 16, 0, 0);
        }
    }

    // Online-softmax update for one block; returns its probabilities as the
    // PV A operand.  nvalid: tokens [0, nvalid) are real (>= 1).
    __device__ inline bf16x8_t softmax(const f32x4_t s[2], int nvalid, float tau_log2e, int lg) {
        float bm = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (16 * t + 4 * lg + r < nvalid) bm = fmaxf(bm, s[t][r]);
        bm = rows4_max(bm);
        const float mnew = fmaxf(m, bm);  // finite: the block has a real token
        const float alpha = exp2_hw((m - mnew) * tau_log2e);  // 0 on the first block
        const float mb = mnew * tau_log2e;
        bf16x8_t P;
        float ls = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float pv = (16 * t + 4 * lg + r < nvalid) ? exp2_hw(s[t][r] * tau_log2e - mb) : 0.f;
                __bf16 pb = (__bf16)pv;
                ls += (float)pb;
                P[4 * t + r] = pb;
            }
        const bool first = m == -INFINITY;
        l = l * alpha + ls;
        m = mnew;
        if (!first) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float ar = __shfl(alpha, 4 * lg + r);
#pragma unroll
                for (int db = 0; db < DB; ++db) o[db][r] *= ar;
            }
        }
        return P;
    }

    // PV product of one block from its tile (the tile's loads have completed).
    __device__ inline void pv(const bf16x8_t& P, const unsigned char* tile) {
        const int lane = threadIdx.x & 63, kq = lane >> 4, s = lane & 15;
        int rowb[2], x[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 16 * h + 4 * kq + (s >> 2);
            rowb[h] = r * 2 * D + 16 * ((s & 3) >> 1) + 8 * (s & 1);
            x[h] = r % (CPR / 2);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            v4s16_t hv[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
                hv[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4s16_t*)(tile + rowb[h] + 32 * (db ^ x[h])));
            // whole-vector reinterpretation (element-wise bf16 inserts of the
            // 16-bit lanes were lowered to wrong byte permutes)
            const v8s16_t both = __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, both);
            o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(P, vb, o[db], 0, 0, 0);
        }
    }

    // K half of a two-pass stream over this wavefront's blocks j < nbw (<=
    // NBW): every block's K rows are loaded (all in flight together), scored
    // (on_scores(j, s) sees them) and turned into probabilities against the
    // running maximum over all of them, P[j] (the PV A operand), with the
    // running sum l updated and O rescaled.  vpass then multiplies them into O.
    template <int NBW, typename OnScores>
    __device__ inline void kpass(const __bf16* kbase, const size_t (&off)[NBW][2], const int (&nval)[NBW],
                                 int nbw, float tau_log2e, int lg, bf16x8_t (&P)[NBW], OnScores on_scores) {
        f32x4_t s[NBW][2];
        float bm = -INFINITY;
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            if (j < nbw) {
                bf16x8_t kb[2][KK];
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk)
                        kb[t][kk] = *(const bf16x8_t*)(kbase + off[j][t] + 32 * kk + 8 * lg);
                scores(kb, s[j]);
                on_scores(j, s[j]);
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (16 * t + 4 * lg + r < nval[j]) bm = fmaxf(bm, s[j][t][r]);
            }
        }
        if (nbw <= 0) return;
        bm = rows4_max(bm);
        const float mnew = fmaxf(m, bm);  // finite: a block has a real token
        const float alpha = exp2_hw((m - mnew) * tau_log2e);  // 0 on an empty state
        const float mb = mnew * tau_log2e;
        float ls = 0.f;
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float pv = (j < nbw && 16 * t + 4 * lg + r < nval[j]) ? exp2_hw(s[j][t][r] * tau_log2e - mb)
                                                                                 : 0.f;
                    const __bf16 pb = (__bf16)pv;
                    ls += (float)pb;
                    P[j][4 * t + r] = pb;
                }
        }
        const bool first = m == -INFINITY;
        l = l * alpha + ls;
        m = mnew;
        if (!first) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * lg + r);
#pragma unroll
                for (int db = 0; db < DB; ++db) o[db][r] *= ar;
            }
        }
    }

    // V half: block j's V rows through the tile, O += P[j] . V.  landed() runs
    // (in every lane) once every earlier store of this wavefront has landed:
    // after the first block's wait, which covers them, or at once without
    // blocks.
    template <int NBW, typename Landed>
    __device__ inline void vpass(const __bf16* vbase, const size_t (&off)[NBW][2], int nbw,
                                 const bf16x8_t (&P)[NBW], unsigned char* tile, Landed landed) {
        if (nbw <= 0) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            landed();
        }
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            if (j < nbw) {
                load_v(vbase, off[j][0], off[j][1], tile);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the tile is loaded
                if (j == 0) landed();
                pv(P[j], tile);
                // the next block's loads overwrite the tile: its reads are done
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
        }
    }

    // Stream this wavefront's blocks j < nbw (<= NBW): block j's rows sit at
    // element offsets off[j][t] and its first nval[j] tokens are real.
    // on_scores(j, s) sees every block's scores; attn = false skips V and PV.
    template <int NBW, typename OnScores>
    __device__ inline void stream(const __bf16* kbase, const __bf16* vbase,
                                  const size_t (&off)[NBW][2], const int (&nval)[NBW], int nbw,
                                  bool attn, float tau_log2e, int lr, int lg, unsigned char* tile,
                                  OnScores on_scores) {
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            if (j < nbw) {
                bf16x8_t kb[2][KK];
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk)
                        kb[t][kk] = *(const bf16x8_t*)(kbase + off[j][t] + 32 * kk + 8 * lg);
                if (attn) load_v(vbase, off[j][0], off[j][1], tile);
                f32x4_t s[2];
                scores(kb, s);
                on_scores(j, s);
                if (attn) {
                    bf16x8_t P = softmax(s, nval[j], tau_log2e, lg);
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the tile is loaded
                    pv(P, tile);
                    // the next block's loads overwrite the tile: its reads are done
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                }
            }
        }
    }
};

}  // namespace gsa
