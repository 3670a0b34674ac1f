// The multi-query side of gist sparse attention: T consecutive slots of the
// interleaved sequence (a chunked-prefill step, or several draft tokens
// checked at once) attend under the gist causal mask ("Forget, Then Recall",
// ja page section 2.1 item 1; nl page "Het Proces", Compressie): the query at
// slot s of chunk m = s / (C+1) sees the gists of chunks m' < m and the slots
// of its own chunk up to s.  The caller has written the queries' own K/V rows
// into the paged cache.
//
// Many queries share the same gist rows, so this is a dense contraction and
// runs on MFMA.  A workgroup owns 128 columns of one (batch, kv-head) unit --
// column j is query t = j / G, head j % G of the GQA group -- as 8 blocks of 16
// (one per wavefront: few enough registers for 4 wavefronts per SIMD, two
// workgroups per compute unit, each key block serving 128 columns).  It
// streams key blocks of 32 rows: first the gists of every chunk up to the last
// query's, then the slots of the chunks its queries lie in.  Each block's K
// and V rows go from global memory straight into LDS (global_load_lds, the
// wavefronts sharing the loads and the tiles; double-buffered, so block i+1
// loads while block i is used); every wavefront reads its K operand from the
// K tile (rows 16-byte-swizzled so the 16 rows one instruction reads hit
// different banks) and its V operand transposed from the V tile.  Scores
// S^T[key][column] = K.Q^T, the mask as each column's inclusive key range
// (compares and selects: a short-circuit test per element compiled to
// branches that cost more than the MFMAs), online softmax per column in the
// exp2 domain, P (bf16) . V accumulated in fp32, and the output written once
// at the end: no partials, no workspace.
#include "gsa_mfma_core.h"

namespace gsa {

// Kernel arguments of one prefill launch.
struct PrefillArgs {
    const void* q;        // [B][T][Hq][D]
    void* out;            // [B][T][Hq][D]
    const void* kc;
    const void* vc;
    const int32_t* bt;    // [B][max_pages]
    const int32_t* q_start;  // [B] first query slot
    int B, Hq, Hkv, G, C, T, spp, max_pages, ncols;  // ncols = T * G
    uint64_t spp_inv;     // ceil(2^32 / spp): slot -> logical page by multiply
    float tau_log2e;
};

namespace {

constexpr int kPWaves = 8;                // wavefronts per workgroup
constexpr int kPThreads = 64 * kPWaves;
constexpr int kNCB = 1;                   // 16-column blocks per wavefront
constexpr int kPCols = kPWaves * kNCB * 16;  // columns per workgroup
constexpr int kPBtLds = 7936;             // block-table entries kept in LDS (64 KB in all at d = 128)

// Wait for this wavefront's outstanding memory operations (global loads into
// LDS and LDS reads).
__device__ inline void wait_mem() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

template <int D>
struct PTiles {
    static constexpr int TILE = 32 * D * 2;
    static constexpr int bytes(int max_pages) {
        return 4 * TILE + 4 * (max_pages <= kPBtLds ? max_pages : 0);
    }
};

// Issue part w of one key block's tile loads (1 KB per instruction: 64 lanes
// x 16 bytes into consecutive LDS), for wavefronts w < CPR / 2: lane l loads
// the 16-byte chunk p = (64w + l) % CPR of row r = (64w + l) / CPR, whose
// element offset is ro.  K: position p of row r holds the row's chunk
// p ^ (r mod CPR); V: the layout WaveAttnL::pv reads.
template <int D, bool BTL>
__device__ __forceinline__ void issue_part(const PrefillArgs& a, size_t ro, int r, int p, unsigned char* kt,
                                           unsigned char* vt, int w) {
    constexpr int CPR = D / 8;
    __builtin_amdgcn_global_load_lds((const __bf16*)a.kc + ro + 8 * (p ^ (r % CPR)),
                                     (lds_void_t*)(kt + 1024 * w), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const __bf16*)a.vc + ro + 8 * (p ^ WaveAttnL<D>::swz(r)),
                                     (lds_void_t*)(vt + 1024 * w), 16, 0, 0);
}

// BTL: the block-table row is kept in LDS (at most kPBtLds pages).
template <int D, bool BTL>
__global__ __launch_bounds__(kPThreads, 4) void prefill_kernel(PrefillArgs a) {  // (4 wavefronts per SIMD)
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int KK = D / 32, DB = D / 16, CPR = D / 8, TILE = PTiles<D>::TILE;
    unsigned char* ktile = smem;             // 2 buffers
    unsigned char* vtile = smem + 2 * TILE;  // 2 buffers
    int* btl = (int*)(smem + 4 * TILE);
    const int u = blockIdx.y, b = u / a.Hkv, g = u - b * a.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // (wave-uniform: scalar branches)
    const int G = a.G, C = a.C, T = a.T;
    // the queries' slots, clamped into the block-table row
    const int cap = a.max_pages * a.spp;
    const int s0 = min(max(a.q_start[b], 0), max(cap - T, 0));
    const int jw = blockIdx.x * kPCols;
    const int t_lo = jw / G, t_hi = min(T - 1, (jw + kPCols - 1) / G);
    const int m_lo = (s0 + t_lo) / (C + 1), m_hi = (s0 + t_hi) / (C + 1);
    const int s_hi = s0 + t_hi, l0 = m_lo * (C + 1);
    const int32_t* btrow = a.bt + (size_t)b * a.max_pages;
    if (BTL)
        for (int i = tid; i < a.max_pages; i += kPThreads) btl[i] = btrow[i];
    __syncthreads();
    // slots number below 2^30, so slot * ceil(2^32 / spp) / 2^32 exceeds
    // slot / spp by less than 1/4: the quotient is exact or one too large
    auto slot_off = [&](int slot) -> size_t {
        int p = (int)(((uint64_t)(uint32_t)slot * a.spp_inv) >> 32);
        p -= p * a.spp > slot;
        const int phys = BTL ? btl[p] : btrow[p];
        return (((size_t)phys * a.Hkv + g) * a.spp + (slot - p * a.spp)) * (size_t)D;
    };

    // this lane's column (lr) of each of the wavefront's column blocks
    WaveAttnL<D> wa[kNCB];
    // lsum[cb][r]: the sum of column 4lg + r's bf16 weights, accumulated on
    // MFMA (the weights times a column of ones) and rescaled with the output
    f32x4_t lsum[kNCB];
    bf16x8_t ones;
#pragma unroll
    for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;
    int colm[kNCB], cols[kNCB];
    bool colv[kNCB];
    int glo[kNCB], ghi[kNCB], slo[kNCB], shi[kNCB];  // keys a column sees: gists [glo, ghi], slots [slo, shi]
#pragma unroll
    for (int cb = 0; cb < kNCB; ++cb) {
        const int j = jw + (w * kNCB + cb) * 16 + lr;
        colv[cb] = j < a.ncols;
        const int t = colv[cb] ? j / G : 0, h = j - (j / G) * G;
        cols[cb] = s0 + t;
        colm[cb] = cols[cb] / (C + 1);
        // the gists of the chunks before the column's chunk, the slots of its
        // chunk up to its own (an empty range for a column past the end)
        glo[cb] = colv[cb] ? 0 : 1;
        ghi[cb] = colv[cb] ? colm[cb] - 1 : 0;
        slo[cb] = colv[cb] ? colm[cb] * (C + 1) : 1;
        shi[cb] = colv[cb] ? cols[cb] : 0;
        const __bf16* qp = (const __bf16*)a.q + (((size_t)b * T + t) * a.Hq + (size_t)g * G + h) * D;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            if (colv[cb]) {
                wa[cb].qB[kk] = *(const bf16x8_t*)(qp + 32 * kk + 8 * lg);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) wa[cb].qB[kk][i] = (__bf16)0.0f;
            }
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) wa[cb].o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        wa[cb].m = -INFINITY;
        wa[cb].l = 0.f;
        lsum[cb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    }

    // key blocks: the gists of chunks [0, m_hi), then the slots [l0, s_hi]
    const int nA = (m_hi + 31) / 32;
    const int nblk = nA + (s_hi - l0 + 1 + 31) / 32;
    // Each block's tiles are loaded by wavefronts w < CPR / 2, every lane one
    // 16-byte chunk of row ir; the row's element offset for block i + 2 is
    // computed during block i (its block-table read and arithmetic overlap
    // that block's work) and used when block i + 1 starts.
    const bool issuer = w < CPR / 2;  // (wave-uniform)
    const int ir = issuer ? (64 * w + lane) / CPR : 0, ip = (64 * w + lane) % CPR;
    // element offset of row ir of block i (a row past the end repeats the
    // last real one: it is masked)
    auto row_off = [&](int i) -> size_t {
        const int k = 32 * i + ir;
        return slot_off(i < nA ? min(k, m_hi - 1) * (C + 1) + C : min(l0 + k - 32 * nA, s_hi));
    };
    const float tl = a.tau_log2e;
    size_t nxt = 0;
    if (issuer) {
        if (nblk > 0) issue_part<D, BTL>(a, row_off(0), ir, ip, ktile, vtile, w);
        if (nblk > 1) nxt = row_off(1);
    }
    wait_mem();
    for (int i = 0; i < nblk; ++i) {
        __syncthreads();  // block i's tiles are in LDS; buffer (i+1)&1 is free
        if (issuer && i + 1 < nblk)
            issue_part<D, BTL>(a, nxt, ir, ip, ktile + ((i + 1) & 1) * TILE, vtile + ((i + 1) & 1) * TILE, w);
        const unsigned char* kt = ktile + (i & 1) * TILE;
        const unsigned char* vt = vtile + (i & 1) * TILE;
        bf16x8_t kA[2][KK];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int r = 16 * t + lr;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                kA[t][kk] = *(const bf16x8_t*)(kt + r * 2 * D + 16 * ((4 * kk + lg) ^ (r % CPR)));
        }
        const bool gist_blk = i < nA;
        // a gist block before the first query's chunk is visible to every
        // column: no mask (block-uniform)
        const bool full = gist_blk && 32 * i + 32 <= m_lo;
        const int kbase = gist_blk ? 32 * i : l0 + 32 * (i - nA);
        if (issuer && i + 2 < nblk) nxt = row_off(i + 2);
#pragma unroll
        for (int cb = 0; cb < kNCB; ++cb) {
            f32x4_t sc[2];
            wa[cb].scores(kA, sc);
            // key 16t + 4lg + r against column lr: inside the column's range
            // (compares and selects, no branch)
            const int lo = gist_blk ? glo[cb] : slo[cb], hi = gist_blk ? ghi[cb] : shi[cb];
            bool ok[2][4];
            float bm = -INFINITY;
            if (full) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) bm = fmaxf(bm, sc[t][r]);
            } else {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = kbase + 16 * t + 4 * lg + r;
                        ok[t][r] = (key >= lo) & (key <= hi);
                        bm = fmaxf(bm, ok[t][r] ? sc[t][r] : -INFINITY);
                    }
            }
            bm = rows4_max(bm);
            // the column's reference maximum moves only when the block's
            // exceeds it by more than 2^8 in probability (the weights stay
            // below 256, exact in bf16 to the same relative precision), so
            // most blocks rescale nothing; the output is the same ratio
            const float mold = wa[cb].m;
            const bool up = (bm - mold) * tl > 8.f;  // (false for bm = -inf; true from -inf)
            const float mnew = up ? bm : mold;
            if (__ballot(up)) {
                // (the hardware exp2: exp2(-inf) = 0)
                const float alpha = up ? __builtin_amdgcn_exp2f((mold - mnew) * tl) : 1.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ar = __shfl(alpha, 4 * lg + r);
#pragma unroll
                    for (int db = 0; db < DB; ++db) wa[cb].o[db][r] *= ar;
                    lsum[cb][r] *= ar;
                }
            }
            const float mb = mnew * tl;  // (arguments of the kept keys are <= 8)
            bf16x8_t P;
            if (full) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) P[4 * t + r] = (__bf16)__builtin_amdgcn_exp2f(sc[t][r] * tl - mb);
            } else {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float e = __builtin_amdgcn_exp2f(sc[t][r] * tl - mb);
                        P[4 * t + r] = (__bf16)(ok[t][r] ? e : 0.f);
                    }
            }
            wa[cb].m = mnew;
            wa[cb].pv(P, vt);
            lsum[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(P, ones, lsum[cb], 0, 0, 0);
        }
        // this block's LDS reads are done and block i+1's tiles have landed
        wait_mem();
    }
    // out[column 4lg + r][16db + lr] = o[db][r] / l(column 4lg + r)
#pragma unroll
    for (int cb = 0; cb < kNCB; ++cb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float L = lsum[cb][r];
            const int j = jw + (w * kNCB + cb) * 16 + 4 * lg + r;
            if (j >= a.ncols) continue;
            const int t = j / G, h = j - t * G;
            __bf16* op = (__bf16*)a.out + (((size_t)b * T + t) * a.Hq + (size_t)g * G + h) * D;
            const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
            for (int db = 0; db < DB; ++db) op[16 * db + lr] = (__bf16)(wa[cb].o[db][r] * inv);
        }
    }
}

}  // namespace

hipError_t launch_prefill(const void* q, void* out, const void* kc, const void* vc, const int32_t* bt,
                          const int32_t* q_start, int B, int Hq, int Hkv, int D, int C, int T, int spp,
                          int max_pages, float tau, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    PrefillArgs a;
    a.q = q;
    a.out = out;
    a.kc = kc;
    a.vc = vc;
    a.bt = bt;
    a.q_start = q_start;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.C = C;
    a.T = T;
    a.spp = spp;
    a.max_pages = max_pages;
    a.ncols = T * a.G;
    a.spp_inv = ((1ull << 32) + (uint64_t)spp - 1) / (uint64_t)spp;
    a.tau_log2e = (float)((double)tau * 1.4426950408889634);
    dim3 grid((a.ncols + kPCols - 1) / kPCols, B * Hkv);
    const bool btl = max_pages <= kPBtLds;
    if (D == 64) {
        if (btl)
            hipLaunchKernelGGL((prefill_kernel<64, true>), grid, dim3(kPThreads), PTiles<64>::bytes(max_pages), st, a);
        else
            hipLaunchKernelGGL((prefill_kernel<64, false>), grid, dim3(kPThreads), PTiles<64>::bytes(max_pages), st, a);
    } else {
        if (btl)
            hipLaunchKernelGGL((prefill_kernel<128, true>), grid, dim3(kPThreads), PTiles<128>::bytes(max_pages), st, a);
        else
            hipLaunchKernelGGL((prefill_kernel<128, false>), grid, dim3(kPThreads), PTiles<128>::bytes(max_pages), st, a);
    }
    return hipGetLastError();
}

}  // namespace gsa
