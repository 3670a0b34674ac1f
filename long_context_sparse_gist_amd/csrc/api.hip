// C ABI of the GSA decode library: argument validation, workspace layout and
// launch sequencing.  Every check runs on the host before anything is
// enqueued; on error nothing is launched and no output is touched.
#include <math.h>
#include <string.h>

#include "gsa.h"
#include "gsa_internal.h"

namespace {

using gsa::Args;

constexpr size_t kAlign = 256;
constexpr int kMaxGroup = 16;
constexpr long kMaxTopK = 1L << 20;
constexpr int kVersion = 100;  // 0.1.0
// Control block at the start of every workspace layout: the single-launch
// kernel's error word (first 16 KiB) and per-unit records (counters and the
// selection's row offsets), zero between calls.  No layout writes scratch data below its end, so reusing one
// workspace across shapes keeps it zero.
constexpr size_t kCtlWords = GSA_WORKSPACE_CONTROL_BYTES / 4;
constexpr size_t kHdrWords = 4096;  // header: error word
constexpr long kMaxFusedUnits = 512;
static_assert(kHdrWords + (size_t)kMaxFusedUnits * gsa::kUnitRec <= kCtlWords, "control block");

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
    Args a;
    gsa::Sched sc;
    bool hier;
    bool mfma;
    bool fused;        // single-launch work-queue kernel
    int TB;            // tokens per split of every list
    int S1;            // splits of the gist (flat) / meta (H-GSA) list
    int Sc;            // splits of the candidate list (H-GSA)
    int S2;            // splits of the unfolded list
    int cand_cap;      // candidate list capacity (H-GSA)
    size_t off_ctl, off_keys, off_sel, off_selm, off_mkeys, off_ckeys, off_cand, off_ml, off_acc,
        off_spairs, off_spairs_c, off_hlog, off_nsel, total;
};

gsa_status_t check_params(const gsa_params_t* p, const gsa_kv_t* kv) {
    if (!p || !kv) return GSA_ERR_NULL_ARG;
    if (p->dtype != GSA_F32 && p->dtype != GSA_BF16) return GSA_ERR_BAD_DTYPE;
    if (p->batch < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1) return GSA_ERR_BAD_SHAPE;
    if (p->num_q_heads % p->num_kv_heads) return GSA_ERR_BAD_SHAPE;
    if (p->num_q_heads / p->num_kv_heads > kMaxGroup) return GSA_ERR_BAD_SHAPE;
    if (p->head_dim != 64 && p->head_dim != 128) return GSA_ERR_BAD_SHAPE;
    if (p->top_k < 0 || p->top_k > kMaxTopK) return GSA_ERR_BAD_SHAPE;
    if (!(p->sm_scale == p->sm_scale) || isinf(p->sm_scale)) return GSA_ERR_BAD_SHAPE;
    const unsigned known = GSA_SCORE_SUM_PROBS | GSA_SET_SELECTED_GISTS | GSA_SELECT_TOP_P | gsa::kFlagPortable;
    if (p->flags & ~known) return GSA_ERR_BAD_FLAGS;
    if (p->flags & GSA_SELECT_TOP_P) {
        if (p->flags & GSA_SCORE_SUM_PROBS) return GSA_ERR_BAD_FLAGS;  // default key only
        if (!(p->top_p > 0.0f && p->top_p <= 1.0f)) return GSA_ERR_BAD_SHAPE;
        if (p->top_k > gsa::kTopPMaxK) return GSA_ERR_BAD_SHAPE;
    }
    if (kv->chunk_size < 1 || kv->page_chunks < 1 || kv->num_chunks < 0) return GSA_ERR_BAD_SHAPE;
    if (kv->num_pages < 1 || kv->max_pages < 1) return GSA_ERR_BAD_SHAPE;
    long spp = (long)kv->page_chunks * (kv->chunk_size + 1);
    if (spp > (1L << 30)) return GSA_ERR_BAD_SHAPE;
    if ((long)kv->max_pages * spp > (1L << 30)) return GSA_ERR_BAD_SHAPE;  // slot ids fit int
    if ((long)kv->max_pages * kv->page_chunks < kv->num_chunks) return GSA_ERR_BAD_SHAPE;
    if ((long)kv->num_pages * p->num_kv_heads * spp > (1L << 40)) return GSA_ERR_BAD_SHAPE;
    if ((long)p->batch * kv->max_pages > (1L << 31) - 1) return GSA_ERR_BAD_SHAPE;
    return GSA_OK;
}

gsa_status_t check_meta(const gsa_params_t* p, const gsa_kv_t* kv, const hgsa_meta_t* m) {
    if (!m) return GSA_ERR_NULL_ARG;
    if (m->gists_per_meta < 1 || m->top_k_meta < 0 || m->top_k_meta > kMaxTopK) return GSA_ERR_BAD_SHAPE;
    if (m->max_meta < kv->num_chunks / m->gists_per_meta) return GSA_ERR_BAD_SHAPE;
    if ((long)p->batch * p->num_kv_heads * (long)m->max_meta > (1L << 40)) return GSA_ERR_BAD_SHAPE;
    if (p->flags & GSA_SET_SELECTED_GISTS) return GSA_ERR_BAD_FLAGS;
    if (p->flags & (GSA_SCORE_SUM_PROBS | GSA_SELECT_TOP_P)) return GSA_ERR_BAD_FLAGS;  // flat GSA only
    return GSA_OK;
}

// Shapes -> launch geometry and workspace layout (pointers left null).
void make_plan(const gsa_params_t* p, const gsa_kv_t* kv, const hgsa_meta_t* m, Plan& pl) {
    memset(&pl, 0, sizeof(pl));
    Args& a = pl.a;
    a.B = p->batch;
    a.Hq = p->num_q_heads;
    a.Hkv = p->num_kv_heads;
    a.G = a.Hq / a.Hkv;
    a.D = p->head_dim;
    a.C = kv->chunk_size;
    a.num_chunks = kv->num_chunks;
    a.page_chunks = kv->page_chunks;
    a.num_pages = kv->num_pages;
    a.max_pages = kv->max_pages;
    a.spp = kv->page_chunks * (kv->chunk_size + 1);
    a.pc_inv = ((1ull << 32) + (uint64_t)kv->page_chunks - 1) / (uint64_t)kv->page_chunks;
    a.top_k = p->top_k;
    a.tau = p->sm_scale > 0.f ? p->sm_scale : (float)(1.0 / sqrt((double)a.D));
    a.tau_log2e = (float)((double)a.tau * 1.4426950408889634);
    a.flags = p->flags;
    a.dtype = p->dtype;
    pl.hier = m != nullptr;
    pl.mfma = p->dtype == GSA_BF16 && !(p->flags & gsa::kFlagPortable);
    pl.TB = pl.mfma ? gsa::mfma_tokens_per_block(a.D) : gsa::portable_tokens_per_block();
    const long M = kv->num_chunks, C = a.C;
    const long units = (long)a.B * a.Hkv;
    long cap1, cap2;
    if (!pl.hier) {
        cap1 = M;
        long k = p->top_k < M ? p->top_k : M;
        cap2 = k * C + (C - 1) + ((p->flags & GSA_SET_SELECTED_GISTS) ? k : 0);
        pl.cand_cap = 0;
    } else {
        a.R = m->gists_per_meta;
        a.top_k_meta = m->top_k_meta;
        a.max_meta = m->max_meta;
        long nm = M / a.R;
        cap1 = nm;
        long k1 = m->top_k_meta < nm ? m->top_k_meta : nm;
        long cc = k1 * a.R + (a.R - 1);
        if (cc > M) cc = M;
        pl.cand_cap = (int)cc;
        long k2 = p->top_k < cc ? p->top_k : cc;
        cap2 = k2 * C + (C - 1) + k2 + (a.R - 1);
    }
    // single launch while the record holds the selection (and the kept meta-groups)
    {
        const long kc = pl.hier ? pl.cand_cap : M;
        const long ksel = p->top_k < kc ? p->top_k : kc;
        const long kmeta = pl.hier ? (m->top_k_meta < cap1 ? m->top_k_meta : cap1) : 0;
        // (the sum-of-probabilities key needs every gist's logits before any key:
        // multi-launch path)
        pl.fused = pl.mfma && units * (pl.hier ? 2 : 1) <= kMaxFusedUnits && ksel <= gsa::kRecRowOffs &&
                   kmeta <= gsa::kRecMeta && !(p->flags & (GSA_SCORE_SUM_PROBS | GSA_SELECT_TOP_P));
        a.recs_per_unit = pl.hier ? 2 : 1;
    }
    // H-GSA's meta slices and candidate tasks take half as many rows: its
    // launch is a chain of latency-bound steps, not a bandwidth-bound stream
    const int TA = pl.fused ? (pl.hier ? gsa::kFusedTAH : gsa::kFusedTA) : pl.TB;
    // unfolded tasks: one block per wavefront, or (flat GSA) two when a
    // launch would hold more than 2048 of them (per-task work then outweighs
    // the tail)
    int TB = pl.fused ? gsa::kFusedTB : pl.TB;
    if (pl.fused && !pl.hier && units * ((cap2 + TB - 1) / TB) > 2048) TB = 2 * gsa::kFusedTB;
    pl.S1 = (int)((cap1 + TA - 1) / TA);
    pl.Sc = (int)((pl.cand_cap + TA - 1) / TA);
    pl.S2 = (int)((cap2 + TB - 1) / TB);
    if (pl.fused) {  // every unit owns at least one task of each kind
        pl.S1 = pl.S1 > 0 ? pl.S1 : 1;
        pl.S2 = pl.S2 > 0 ? pl.S2 : 1;
        if (pl.hier) pl.Sc = pl.Sc > 0 ? pl.Sc : 1;
    }
    a.S1 = pl.S1;
    a.SL = TA;
    a.SR = TB;
    a.NS = pl.S1 + pl.S2;
    pl.sc.units = (int)units;
    pl.sc.S1 = pl.S1;
    pl.sc.S3 = pl.fused && pl.hier ? pl.Sc : 0;
    pl.sc.S2 = pl.S2;
    pl.sc.TA = TA;
    pl.sc.TB = TB;
    pl.sc.total = (int)(units * (pl.S1 + pl.sc.S3 + pl.S2));
    pl.sc.hier = pl.hier ? 1 : 0;
    a.key_stride = kv->num_chunks;
    a.cand_stride = pl.cand_cap;
    size_t off = 0;
    pl.off_ctl = off;   off += sizeof(unsigned) * kCtlWords;
    pl.off_keys = off;  off += align_up(sizeof(float) * units * (pl.hier ? 0 : M));
    pl.off_sel = off;   off += align_up(sizeof(int32_t) * units * p->top_k);
    pl.off_selm = off;  off += align_up(sizeof(int32_t) * units * (pl.hier ? m->top_k_meta : 0));
    pl.off_mkeys = off; off += align_up(sizeof(float) * units * (pl.hier ? m->max_meta : 0));
    pl.off_ckeys = off; off += align_up(sizeof(float) * units * pl.cand_cap);
    pl.off_cand = off;  off += align_up(sizeof(int32_t) * units * pl.cand_cap);
    pl.off_ml = off;    off += align_up(sizeof(float) * 2 * units * a.NS * a.G);
    pl.off_acc = off;   off += align_up(sizeof(float) * units * a.NS * a.G * a.D);
    const size_t fslices = pl.fused ? (size_t)units * pl.S1 : 0;
    pl.off_spairs = off; off += align_up(sizeof(uint64_t) * fslices * gsa::kFusedTA);
    pl.off_spairs_c = off; off += align_up(sizeof(uint64_t) * (size_t)units * pl.sc.S3 * gsa::kFusedTA);
    const bool probs = !pl.hier && (p->flags & GSA_SCORE_SUM_PROBS);
    pl.off_hlog = off;  off += align_up(sizeof(float) * (probs ? (size_t)units * a.G * M : 0));
    const bool topp = !pl.hier && (p->flags & GSA_SELECT_TOP_P);
    pl.off_nsel = off;  off += align_up(sizeof(int32_t) * (topp ? (size_t)units : 0));
    pl.total = off;
}

gsa_status_t check_device() {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        return GSA_ERR_DEVICE;
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return GSA_ERR_DEVICE;
    }
    return GSA_OK;
}

gsa_status_t check_workspace(const Plan& pl, void* ws, size_t bytes) {
    if (!ws) return GSA_ERR_WORKSPACE;
    if (((uintptr_t)ws) % kAlign) return GSA_ERR_WORKSPACE;
    if (bytes < pl.total) return GSA_ERR_WORKSPACE;
    return GSA_OK;
}

#define GSA_LAUNCH(expr)                                   \
    do {                                                   \
        if ((expr) != hipSuccess) return GSA_ERR_LAUNCH;   \
    } while (0)

gsa_status_t run_attn(const Plan& pl, int kind, int splits, hipStream_t st) {
    if (splits <= 0) return GSA_OK;
    if (pl.mfma) GSA_LAUNCH(gsa::launch_attn_mfma(pl.a, kind, splits, st));
    else GSA_LAUNCH(gsa::launch_attn_portable(pl.a, kind, splits, st));
    return GSA_OK;
}

}  // namespace

extern "C" {

size_t gsa_workspace_size(const gsa_params_t* p, const gsa_kv_t* kv) {
    if (check_params(p, kv) != GSA_OK) return 0;
    Plan pl;
    make_plan(p, kv, nullptr, pl);
    return pl.total;
}

size_t hgsa_workspace_size(const gsa_params_t* p, const gsa_kv_t* kv, const hgsa_meta_t* m) {
    if (check_params(p, kv) != GSA_OK || check_meta(p, kv, m) != GSA_OK) return 0;
    Plan pl;
    make_plan(p, kv, m, pl);
    return pl.total;
}

gsa_status_t gsa_decode(const gsa_params_t* p, const gsa_kv_t* kv, const void* q, void* out,
                        int32_t* sel_idx, float* scores, void* workspace, size_t workspace_bytes,
                        void* stream) {
    gsa_status_t s = check_params(p, kv);
    if (s != GSA_OK) return s;
    if (!q || !out || !kv->k_cache || !kv->v_cache || !kv->block_table) return GSA_ERR_NULL_ARG;
    Plan pl;
    make_plan(p, kv, nullptr, pl);
    if ((s = check_workspace(pl, workspace, workspace_bytes)) != GSA_OK) return s;
    if ((s = check_device()) != GSA_OK) return s;

    Args& a = pl.a;
    char* ws = (char*)workspace;
    a.q = q;
    a.kc = kv->k_cache;
    a.vc = kv->v_cache;
    a.bt = kv->block_table;
    a.seq_lens = kv->seq_lens;
    a.keys = scores ? scores : (float*)(ws + pl.off_keys);
    a.sel = sel_idx ? sel_idx : (int32_t*)(ws + pl.off_sel);
    a.hlog = (p->flags & GSA_SCORE_SUM_PROBS) ? (float*)(ws + pl.off_hlog) : nullptr;
    a.top_p = (p->flags & GSA_SELECT_TOP_P) ? p->top_p : 0.f;
    a.nsel = nullptr;  // set once the top-p counts are written
    a.part_ml = (float2*)(ws + pl.off_ml);
    a.part_acc = (float*)(ws + pl.off_acc);
    a.out = out;
    hipStream_t st = (hipStream_t)stream;

    if (pl.fused) {
        unsigned* ctl = (unsigned*)(ws + pl.off_ctl);
        pl.sc.err = ctl + 2;
        a.urec = ctl + kHdrWords;
        a.spairs = (uint64_t*)(ws + pl.off_spairs);
        GSA_LAUNCH(gsa::launch_fused(a, pl.sc, st));
        return GSA_OK;
    }
    if ((s = run_attn(pl, gsa::kListGists, pl.S1, st)) != GSA_OK) return s;
    if ((p->flags & GSA_SCORE_SUM_PROBS) && !(p->flags & GSA_SET_SELECTED_GISTS) && pl.S1 > 0)
        GSA_LAUNCH(gsa::launch_probs_keys(a, st));  // (the selected-gists set: in the select)
    GSA_LAUNCH(gsa::launch_select(a, gsa::kSelGists, st));
    if (p->flags & GSA_SELECT_TOP_P) {
        a.nsel = (int32_t*)(ws + pl.off_nsel);
        GSA_LAUNCH(gsa::launch_topp_trim(a, st));
    }
    if ((s = run_attn(pl, gsa::kListUnfolded, pl.S2, st)) != GSA_OK) return s;
    GSA_LAUNCH(gsa::launch_merge(a, 0, st));
    return GSA_OK;
}

gsa_status_t hgsa_decode(const gsa_params_t* p, const gsa_kv_t* kv, const hgsa_meta_t* m,
                         const void* q, void* out, int32_t* sel_meta, int32_t* sel_idx,
                         void* workspace, size_t workspace_bytes, void* stream) {
    gsa_status_t s = check_params(p, kv);
    if (s != GSA_OK) return s;
    if ((s = check_meta(p, kv, m)) != GSA_OK) return s;
    if (!q || !out || !kv->k_cache || !kv->v_cache || !kv->block_table || !m->k_meta || !m->v_meta)
        return GSA_ERR_NULL_ARG;
    Plan pl;
    make_plan(p, kv, m, pl);
    if ((s = check_workspace(pl, workspace, workspace_bytes)) != GSA_OK) return s;
    if ((s = check_device()) != GSA_OK) return s;

    Args& a = pl.a;
    char* ws = (char*)workspace;
    a.q = q;
    a.kc = kv->k_cache;
    a.vc = kv->v_cache;
    a.bt = kv->block_table;
    a.seq_lens = kv->seq_lens;
    a.km = m->k_meta;
    a.vm = m->v_meta;
    a.sel = sel_idx ? sel_idx : (int32_t*)(ws + pl.off_sel);
    a.sel_meta = sel_meta ? sel_meta : (int32_t*)(ws + pl.off_selm);
    a.mkeys = (float*)(ws + pl.off_mkeys);
    a.ckeys = (float*)(ws + pl.off_ckeys);
    a.cand = (int32_t*)(ws + pl.off_cand);
    a.part_ml = (float2*)(ws + pl.off_ml);
    a.part_acc = (float*)(ws + pl.off_acc);
    a.out = out;
    hipStream_t st = (hipStream_t)stream;

    if (pl.fused) {
        unsigned* ctl = (unsigned*)(ws + pl.off_ctl);
        pl.sc.err = ctl + 2;
        a.urec = ctl + kHdrWords;
        a.spairs = (uint64_t*)(ws + pl.off_spairs);
        a.spairs_c = (uint64_t*)(ws + pl.off_spairs_c);
        GSA_LAUNCH(gsa::launch_fused(a, pl.sc, st));
        return GSA_OK;
    }
    if ((s = run_attn(pl, gsa::kListMeta, pl.S1, st)) != GSA_OK) return s;
    GSA_LAUNCH(gsa::launch_select(a, gsa::kSelMeta, st));
    if ((s = run_attn(pl, gsa::kListCand, pl.Sc, st)) != GSA_OK) return s;
    GSA_LAUNCH(gsa::launch_select(a, gsa::kSelCand, st));
    if ((s = run_attn(pl, gsa::kListUnfolded, pl.S2, st)) != GSA_OK) return s;
    GSA_LAUNCH(gsa::launch_merge(a, 1, st));
    return GSA_OK;
}

const char* gsa_status_string(gsa_status_t s) {
    switch (s) {
        case GSA_OK: return "ok";
        case GSA_ERR_NULL_ARG: return "a required pointer is NULL";
        case GSA_ERR_BAD_SHAPE: return "a size or count is out of range";
        case GSA_ERR_BAD_DTYPE: return "unsupported dtype";
        case GSA_ERR_BAD_FLAGS: return "unknown or unsupported flags";
        case GSA_ERR_WORKSPACE: return "workspace NULL, misaligned or too small";
        case GSA_ERR_DEVICE: return "no usable HIP device";
        case GSA_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

int gsa_version(void) { return kVersion; }

}  // extern "C"
