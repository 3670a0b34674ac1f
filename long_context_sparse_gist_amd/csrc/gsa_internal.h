// Internal declarations of the GSA decode library: kernel argument block,
// device helpers and the host launchers each kernel file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gsa {

// Block barrier that orders LDS accesses only.  __syncthreads() also makes the
// wavefronts wait for every global load and store they have in flight (its
// fences cover all memory); where a barrier guards nothing but LDS data, that
// wait costs a memory round trip for nothing.  Global accesses are not
// ordered across this barrier.
__device__ inline void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr unsigned kFlagSumProbs = 0x1u;
constexpr unsigned kFlagSelectedGists = 0x2u;
constexpr unsigned kFlagTopP = 0x4u;
constexpr unsigned kFlagPortable = 0x100u;

// Everything a kernel needs to walk one decode call.  Built once on the host,
// passed by value.
struct Args {
    // shapes
    int B, Hq, Hkv, G, D, C;
    int num_chunks, page_chunks, num_pages, max_pages, spp;  // spp: slots per page
    int top_k;
    float tau;        // softmax scale
    float tau_log2e;  // tau * log2(e): logits in the exp2 domain
    unsigned flags;
    int dtype;        // 0 f32, 1 bf16
    // inputs
    const void* q;
    const void* kc;
    const void* vc;
    const int32_t* bt;
    const int32_t* seq_lens;
    // H-GSA inputs (null for flat GSA)
    const void* km;
    const void* vm;
    int R, top_k_meta, max_meta;
    // work buffers
    float* keys;      // [units][key_stride] routing keys
    int key_stride;
    float* hlog;      // [units][G][key_stride] per-head gist logits (sum-of-probabilities key), else null
    float* hsum;      // [units][NS][G] with hlog on the MFMA kernels: each gist split's per-head sum of
                      // unrounded probabilities (part_ml's sum is of the bf16 PV operand), else null
    float top_p;      // top-p selection: probability mass to keep
    int32_t* nsel;    // [units] selected chunks per unit (top-p), else null: min(top_k, n)
    int32_t* sel;     // [units][top_k] selected chunk ids, ascending, -1 padded
    int32_t* sel_meta;   // [units][top_k_meta] (H-GSA)
    float* mkeys;     // [units][max_meta] meta routing keys (H-GSA)
    float* ckeys;     // [units][cand_stride] candidate routing keys (H-GSA)
    int32_t* cand;    // [units][cand_stride] candidate chunk ids (H-GSA)
    int cand_stride;
    float2* part_ml;  // [units][NS][G] (max in exp2 domain, sum)
    float* part_acc;  // [units][NS][G][D]
    int NS;           // partial slots per unit
    int S1;           // token-list splits of the "all gists" / meta list
    int SL;           // tokens per split of that list
    int SR;           // tokens per split of the unfolded list
    // single-launch path only
    unsigned* urec;   // [units][recs_per_unit][kUnitRec] per-unit control records, zero between calls
    int recs_per_unit;
    uint64_t* spairs; // [units][S1][kFusedTA] slice keys by bucket: order key | id << 32
    uint64_t* spairs_c;  // [units][S3][kFusedTA] the same for the candidate tasks (H-GSA)
    uint64_t pc_inv;  // ceil(2^32 / page_chunks): chunk -> logical page by multiply
    void* out;        // [B][Hq][D]
};

// Length of sequence b in chunks and raw tail, clamped so that nothing past
// the block-table row is ever read.
__device__ inline void seq_shape(const Args& a, int b, int& n, int& tail) {
    long L = a.seq_lens ? (long)a.seq_lens[b] : (long)a.num_chunks * a.C;
    long maxL = (long)a.num_chunks * a.C + a.C - 1;
    L = L < 0 ? 0 : (L > maxL ? maxL : L);
    n = (int)(L / a.C);
    tail = (int)(L - (long)n * a.C);
    if (n > a.num_chunks) { n = a.num_chunks; tail = 0; }
    long cap = (long)a.max_pages * a.spp - (long)n * (a.C + 1);
    if (tail > cap) tail = (int)cap;
}

// Logical page of chunk m.  Slots number below 2^30, so m < 2^29 and
// m * ceil(2^32 / page_chunks) / 2^32 exceeds m / page_chunks by less than
// 1/4: the quotient is exact or one too large, and one compare corrects it.
__device__ inline int chunk_page(const Args& a, int m) {
    const int q = (int)(((uint64_t)(uint32_t)m * a.pc_inv) >> 32);
    return q * a.page_chunks > m ? q - 1 : q;
}

// Element offset of logical slot s of sequence b, kv-head g in the paged cache.
__device__ inline size_t slot_offset(const Args& a, int b, int g, int s) {
    int lp = s / a.spp;
    int off = s - lp * a.spp;
    int phys = a.bt[(size_t)b * a.max_pages + lp];
    return (((size_t)phys * a.Hkv + g) * a.spp + off) * (size_t)a.D;
}

// Order-preserving 32-bit key of a float: larger float -> larger key; -0 and
// +0 map to one key; NaN maps to the smallest key.
__device__ inline uint32_t order_key(float f) {
    if (f != f) return 0u;
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// The float an order key was made from (0: a NaN; -0 comes back as +0).
__device__ inline float order_key_value(uint32_t k) {
    if (k == 0u) return __uint_as_float(0x7fc00000u);
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Sum / max over the four 16-lane rows at one column (lanes l, l^16, l^32,
// l^48); every one of them gets the result.  A lane swap between the wave's
// halves, then between the rows of each half (VALU, no LDS round trip): with
// both operands the same value, the two results of a swap hold the lane's
// value and its partner's.
__device__ inline float rows4_sum(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ inline float rows4_max(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Number of unfolded (non-"all gists") list tokens of a sequence with `ns`
// selected chunks and `tail` raw tokens after its last gist.
__device__ inline int unfolded_len(const Args& a, int ns, int tail) {
    return ns * a.C + tail + ((a.flags & kFlagSelectedGists) ? ns : 0);
}

// ---- host launchers (one per kernel family) ----
enum ListKind { kListGists = 0, kListUnfolded = 1, kListMeta = 2, kListCand = 3 };

hipError_t launch_attn_mfma(const Args& a, int kind, int splits, hipStream_t st);
hipError_t launch_attn_portable(const Args& a, int kind, int splits, hipStream_t st);
int mfma_tokens_per_block(int D);
int portable_tokens_per_block();

// Work-queue state and geometry of the single-launch kernel.  The counters
// live in the caller's workspace and are zero between calls.
struct Sched {
    unsigned* err;     // set if a wait gave up (never expected)
    int units;
    int S1, S3, S2;    // task slots per unit (capacity): gist / meta slices, candidate tasks, unfolded tasks
    int TA, TB;        // tokens per task
    int total;         // workgroups
    int hier;          // H-GSA
    int flat;          // flat GSA, one launch: 1 = every task owns a gist slice or only
                       // unfolded blocks (S1 tasks per unit, the grid resident at once),
                       // 0 = gist slices of every unit first, then unfolded tasks
    unsigned vhold;    // V-pass pacing of the per-slice layout's gist slices: a slice
                       // starts its V rows no earlier than this many ticks of the 100 MHz
                       // clock after it started (0: at once)
};
hipError_t launch_fused(const Args& a, const Sched& s, hipStream_t st);
constexpr int kFusedTA = 256;  // gists per gist-slice task (two 32-token blocks per wavefront);
                               // also the sorted-key capacity of every slice
constexpr int kFusedTAH = 128; // rows per meta slice or candidate task (H-GSA: one block per wavefront)
constexpr int kFusedTB = 128;  // tokens per unfolded task (one 32-token block per wavefront; twice
                               // that for launches with many unfolded tasks)
constexpr int kBins = 2048;    // buckets of a routing key's top 11 bits
// Control record of one unit (words): the counts of finished gist (or
// meta-gist) slices and candidate tasks (the selecting one, the list's last,
// not included), of finished unfolded tasks and of finished selects, each in
// a 64-byte sector of its own (the selecting slice's published partial
// shares the last one); from word 64 the selection's row
// offsets (entry i: one plus the element offset of the i-th selected chunk's
// first raw row, bit 62 set when the chunk lies past the last complete
// meta-group); then the leading keys of every gist or meta-gist slice
// (kRecLead per slice: order key | (list index + 1) << 32).  An H-GSA unit
// owns two consecutive records: the second one's leading-key region holds
// the candidate tasks' leading keys and its row-offset region the kept
// meta-groups (entry i: one plus the i-th kept group).  An entry is 0 until
// written, and its readers poll it; the unit's last tasks return every entry
// to 0.  Records are 24.5 KiB apart, so the words that waiting workgroups
// poll spread over memory channels instead of queueing on one.
constexpr int kRecRowOffs = 1024;  // selected chunks (or kept meta-groups) a record holds
constexpr int kRecSlices = 64;     // slices whose leading keys a record holds
constexpr int kRecLead = 32;       // leading keys per slice
constexpr int kRecMeta = kRecRowOffs;
constexpr int kUnitRec = 6272;
static_assert(64 + 2 * kRecRowOffs + 2 * kRecSlices * kRecLead <= kUnitRec, "control record");
constexpr uint64_t kRowPastGroups = 1ull << 62;  // row-offset flag (H-GSA)
constexpr uint64_t kRowSkip = 1ull << 61;        // row-offset flag: a chunk cut by top-p
// Top-p in the single launch: each gist slice's (softmax maximum, sum of exp)
// of its keys, one 64-bit word per slice after the leading keys of the record
// (nonzero once written: the sum's bits, or those of -1 for none, above the
// maximum's).
constexpr int kRecTopP = 64 + 2 * kRecRowOffs + 2 * kRecSlices * kRecLead;
constexpr int kTopPSlices = (kUnitRec - kRecTopP) / 2;
// The sum-of-probabilities key in the single launch: each gist slice's
// per-head logit maximum and sum of exp (natural units), one 64-bit word per
// (slice, head) from word 64 of the unit's second record: the maximum's bits,
// above them the sum's with the sign bit set (nonzero once written).
constexpr int kRecHeadPairs = (kUnitRec - 64) / 2;
// records per unit: 1 (flat GSA), 2 (H-GSA; flat GSA with the
// sum-of-probabilities key)
__device__ inline unsigned* unit_rec(const Args& a, int u, int second = 0) {
    return a.urec + ((size_t)u * a.recs_per_unit + second) * kUnitRec;
}
__device__ inline unsigned* unit_cntA(const Args& a, int u) { return unit_rec(a, u); }       // finished gist / meta slices
__device__ inline unsigned* unit_cntB(const Args& a, int u) { return unit_rec(a, u) + 16; }  // finished unfolded tasks
__device__ inline unsigned* unit_cntC(const Args& a, int u) { return unit_rec(a, u) + 32; }  // finished candidate tasks
__device__ inline unsigned* unit_cntS(const Args& a, int u) { return unit_rec(a, u) + 48; }  // selects done writing the record
__device__ inline unsigned* unit_cntP(const Args& a, int u) { return unit_rec(a, u) + 56; }  // selecting slice's partial published
__device__ inline int64_t* unit_rowoff(const Args& a, int u) { return (int64_t*)(unit_rec(a, u) + 64); }
__device__ inline uint64_t* unit_lead(const Args& a, int u) { return (uint64_t*)(unit_rec(a, u) + 64 + 2 * kRecRowOffs); }
__device__ inline uint64_t* unit_topp(const Args& a, int u) { return (uint64_t*)(unit_rec(a, u) + kRecTopP); }
__device__ inline uint64_t* unit_lead_c(const Args& a, int u) {
    return (uint64_t*)(unit_rec(a, u, 1) + 64 + 2 * kRecRowOffs);
}
__device__ inline unsigned* unit_meta(const Args& a, int u) { return unit_rec(a, u, 1) + 64; }
__device__ inline uint64_t* unit_hpairs(const Args& a, int u) { return (uint64_t*)(unit_rec(a, u, 1) + 64); }

enum SelectMode { kSelGists = 0, kSelMeta = 1, kSelCand = 2 };
hipError_t launch_select(const Args& a, int mode, hipStream_t st);
hipError_t launch_topp_trim(const Args& a, hipStream_t st);
hipError_t launch_probs_keys(const Args& a, hipStream_t st);
constexpr int kTopPMaxK = 2048;  // largest top_k (the cap) with top-p selection
hipError_t launch_merge(const Args& a, int hier, hipStream_t st);
hipError_t launch_cand_keys(const Args& a, hipStream_t st);
hipError_t launch_prefill(const void* q, void* out, const void* kc, const void* vc, const int32_t* bt,
                          const int32_t* q_start, int B, int Hq, int Hkv, int D, int C, int T, int spp,
                          int max_pages, float tau, hipStream_t st);

}  // namespace gsa
