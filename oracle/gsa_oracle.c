/*
 * CPU oracle for gist sparse attention (GSA) decode and its two-level
 * gist-of-gist variant (H-GSA).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: it is used by tests/, by the smoke check and by the
 * benchmark's CPU-baseline leg.  It shares no code with the HIP library.
 *
 * Plain, slow, obviously correct: naive loops, a full sort for top-k and a
 * two-pass softmax.  Each step follows the method as described on the pages
 * "Forget, Then Recall: Learnable Compression and Selective Unfolding via Gist
 * Sparse Attention" (gist.science technical summaries, ja / ko / nl):
 *
 *   O1 score   s_{t,m} = q_t . k_{g_m}  (nl page, Methodologie, "Het Proces",
 *              Scoring: the one formula the pages print), scaled by the softmax
 *              scale tau and summed over the query heads of a GQA group, so one
 *              selection is shared per (batch, kv-head).  Accumulated in double
 *              and rounded once to float: the selection decision is taken on
 *              float keys, the precision the GPU path decides in.
 *   O2 select  top-k chunks by score (ja page, section 2.1 item 3; nl page,
 *              "Selectie"); ties go to the lower chunk index; NaN keys last.
 *              With ORACLE_SELECT_TOP_P: the top-p (nucleus) alternative the
 *              ja page's ablation (section 4) and the nl page's results
 *              ("Stabiliteit") compare against top-k: the shortest prefix of
 *              that order whose selection probabilities (softmax of the keys)
 *              reach top_p, top_k at most.
 *   O3 set     all gist tokens plus the raw tokens of the selected chunks
 *              (ja page, 2.1 items 3-4; nl page, "Selectieve Ontvouwing"),
 *              plus the raw tokens after the last gist (not yet compressed).
 *              With ORACLE_SET_SELECTED_GISTS only the selected chunks' gists
 *              are kept (the SG+SR rule of the ja page's ablation, section 4).
 *   O4 attend  per query head: softmax(tau * q.K_j) over the set, then the
 *              weighted sum of V_j; two passes (max, then sums), in double.
 *   O5 H-GSA   coarse to fine (ja page 2.2; nl page "Hierarchische
 *              Uitbreiding"): score meta-gists, keep top-k1, score the gists of
 *              the kept groups, keep top-k2, unfold their raw tokens; attend to
 *              all meta-gists, the kept gists and their raw tokens.
 *   O7 levels  the recursive hierarchy (ja page 2.2: meta-gists built again
 *              over meta-gists into a multi-level structure, coarse-to-fine
 *              selection, O(log n) decoding; nl page "Hierarchische
 *              Uitbreiding"): L levels of meta-gists above the gists, level l
 *              entry r summarising entries [r*R_l, (r+1)*R_l) of level l-1.
 *              Every entry of the top level is scored and attended; going
 *              down, the candidates of a level are the children of the entries
 *              kept one level up plus the entries past that level's last
 *              complete group; the top-k of the candidates are kept.  Set:
 *              every top-level entry, the kept entries and the past-the-last-
 *              group entries of each level below it, the kept chunks' raw
 *              tokens, the raw tail.  L = 1 is O5, L = 0 is O1-O4.
 *   O8 prefill the multi-query side: T consecutive slots of the interleaved
 *              sequence (chunked prefill, or several draft tokens checked at
 *              once) attend under the gist causal mask (ja page 2.1 item 1; nl
 *              page "Het Proces", Compressie: a gist sees only its own chunk
 *              and the gists before it).  Reading for raw tokens, which the
 *              pages leave open: they see the gists of earlier chunks and the
 *              slots of their own chunk up to themselves (earlier chunks are
 *              present only through their gists, which stand in for their raw
 *              tokens' cache).  Query at slot s in chunk m = s / (C+1): keys =
 *              gists of chunks m' < m plus slots m*(C+1) .. s.
 *   O6         O3-O5 with the selection supplied by the caller: its ids that
 *              lie in the sequence (chunk ids in [0, n), meta-group ids in
 *              [0, n/R)) in place of the top-k at that level, in any order;
 *              -1 and other ids are ignored.  H-GSA's candidates follow the
 *              caller's meta-groups.
 *
 * Parity pins (tests/test_oracle_*.py) check this file against numpy fp64
 * brute force, closed forms and invariants; see the tests for which pin
 * covers which step.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_SCORE_SUM_PROBS 0x1
#define ORACLE_SET_SELECTED_GISTS 0x2
#define ORACLE_SELECT_TOP_P 0x4

typedef struct {
    int batch, num_q_heads, num_kv_heads, head_dim;
    int top_k;          /* chunks unfolded (k2 for H-GSA) */
    float sm_scale;     /* <= 0 selects 1/sqrt(head_dim) rounded to float */
    int dtype;          /* 0: float32, 1: bfloat16 stored as uint16 */
    int flags;
    int num_chunks, chunk_size, page_chunks, num_pages, max_pages;
    int gists_per_meta, top_k_meta, max_meta; /* H-GSA only */
    float top_p;        /* with ORACLE_SELECT_TOP_P: probability mass to keep, (0, 1] */
} oracle_cfg;

/* ---- element access (bf16 -> float widening is exact) ---------------- */

static double ld(const void *p, size_t i, int dtype) {
    if (dtype == 0) return (double)((const float *)p)[i];
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

typedef struct {
    const oracle_cfg *c;
    const void *k, *v;
    const int32_t *bt;
    int b, g;
} seqview;

/* flat element index of dimension 0 of logical slot s of sequence b, kv-head g */
static size_t slot_base(const seqview *sv, long s) {
    const oracle_cfg *c = sv->c;
    long spp = (long)c->page_chunks * (c->chunk_size + 1);
    long page = s / spp, off = s % spp;
    long phys = sv->bt[(long)sv->b * c->max_pages + page];
    return (((size_t)phys * c->num_kv_heads + sv->g) * spp + off) * c->head_dim;
}

static double tau_of(const oracle_cfg *c) {
    if (c->sm_scale > 0.f) return (double)c->sm_scale;
    return (double)(float)(1.0 / sqrt((double)c->head_dim));
}

/* q_h . x for query head h (global head index) and a K row at flat index kb */
static double dot_q(const oracle_cfg *c, const void *q, int b, int h,
                    const void *kv, size_t kb) {
    double acc = 0.0;
    size_t qb = ((size_t)b * c->num_q_heads + h) * c->head_dim;
    for (int i = 0; i < c->head_dim; i++)
        acc += ld(q, qb + i, c->dtype) * ld(kv, kb + i, c->dtype);
    return acc;
}

/* ---- O1: group routing key of one gist row ---------------------------- */

/* logits z_h = tau * q_h . k for the G heads of kv-head g */
static void group_logits(const oracle_cfg *c, const void *q, int b, int g,
                         const void *kv, size_t kb, double *z) {
    int G = c->num_q_heads / c->num_kv_heads;
    double tau = tau_of(c);
    for (int j = 0; j < G; j++) z[j] = tau * dot_q(c, q, b, g * G + j, kv, kb);
}

/* Keys of n rows. Row r sits at flat index rows[r] of array kv.
 * Default: S_r = sum_h z_hr.  Sum-of-probs: S_r = sum_h softmax_r(z_h.)_r,
 * the softmax taken over the n rows. */
static void routing_keys(const oracle_cfg *c, const void *q, int b, int g,
                         const void *kv, const size_t *rows, int n, float *S) {
    int G = c->num_q_heads / c->num_kv_heads;
    double *z = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * G);
    for (int r = 0; r < n; r++) group_logits(c, q, b, g, kv, rows[r], z + (size_t)r * G);
    if (!(c->flags & ORACLE_SCORE_SUM_PROBS)) {
        for (int r = 0; r < n; r++) {
            double s = 0.0;
            for (int j = 0; j < G; j++) s += z[(size_t)r * G + j];
            S[r] = (float)s;
        }
    } else {
        double *acc = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
        for (int j = 0; j < G; j++) {
            double mx = -INFINITY, den = 0.0;
            for (int r = 0; r < n; r++) mx = fmax(mx, z[(size_t)r * G + j]);
            for (int r = 0; r < n; r++) den += exp(z[(size_t)r * G + j] - mx);
            for (int r = 0; r < n; r++) acc[r] += exp(z[(size_t)r * G + j] - mx) / den;
        }
        for (int r = 0; r < n; r++) S[r] = (float)acc[r];
        free(acc);
    }
    free(z);
}

/* ---- O2: top-k with lower-index tie-break ----------------------------- */

typedef struct { float s; int id; } keyed;

static int cmp_keyed(const void *pa, const void *pb) {
    const keyed *a = (const keyed *)pa, *b = (const keyed *)pb;
    int na = isnan(a->s), nb = isnan(b->s);
    if (na != nb) return na ? 1 : -1;           /* NaN keys last */
    if (!na) {
        if (a->s > b->s) return -1;
        if (a->s < b->s) return 1;
    }
    return (a->id < b->id) ? -1 : (a->id > b->id);
}

static int cmp_int(const void *pa, const void *pb) {
    int a = *(const int *)pa, b = *(const int *)pb;
    return (a > b) - (a < b);
}

/* Select min(k, n) of the n candidates (ids[r], S[r]); write them sorted
 * ascending to out; return the count. */
static int topk(const float *S, const int *ids, int n, int k, int *out) {
    keyed *v = (keyed *)malloc(sizeof(keyed) * (size_t)(n > 0 ? n : 1));
    for (int r = 0; r < n; r++) { v[r].s = S[r]; v[r].id = ids[r]; }
    qsort(v, (size_t)n, sizeof(keyed), cmp_keyed);
    int kk = k < n ? k : n;
    for (int i = 0; i < kk; i++) out[i] = v[i].id;
    qsort(out, (size_t)kk, sizeof(int), cmp_int);
    free(v);
    return kk;
}

/* ---- O2': top-p (nucleus) selection ----------------------------------- */

/* The chunks in key order (largest first, ties to the lower index, NaN last)
 * up to and including the first at which the running sum of their selection
 * probabilities reaches p; at most k of them.  A chunk's selection
 * probability is the softmax of its key over the n candidates (a NaN key:
 * probability 0).  Without a usable softmax (no finite largest key) the first
 * min(k, n) are taken.  Writes them ascending to out; returns the count. */
static int topp(const float *S, const int *ids, int n, int k, double p, int *out) {
    keyed *v = (keyed *)malloc(sizeof(keyed) * (size_t)(n > 0 ? n : 1));
    for (int r = 0; r < n; r++) { v[r].s = S[r]; v[r].id = ids[r]; }
    qsort(v, (size_t)n, sizeof(keyed), cmp_keyed);
    int kk = k < n ? k : n;
    double mx = -INFINITY;
    for (int r = 0; r < n; r++)
        if (!isnan(v[r].s) && v[r].s > mx) mx = v[r].s;
    if (isfinite(mx)) {
        double z = 0.0;
        for (int r = 0; r < n; r++) z += isnan(v[r].s) ? 0.0 : exp(v[r].s - mx);
        double cum = 0.0;
        int need = kk;
        for (int r = 0; r < kk; r++) {
            cum += isnan(v[r].s) ? 0.0 : exp(v[r].s - mx);
            if (cum >= p * z) { need = r + 1; break; }
        }
        kk = need;
    }
    for (int i = 0; i < kk; i++) out[i] = v[i].id;
    qsort(out, (size_t)kk, sizeof(int), cmp_int);
    free(v);
    return kk;
}

/* ---- O4: softmax attention of the G heads over a token list ------------ */

typedef struct {
    const void *arr_k, *arr_v;  /* arrays the row index refers to */
    size_t row;                 /* flat index of element 0 */
} tokref;

static void attend(const oracle_cfg *c, const void *q, int b, int g,
                   const tokref *T, long nT, double *out /* [G][d] */) {
    int G = c->num_q_heads / c->num_kv_heads, d = c->head_dim;
    double tau = tau_of(c);
    double *z = (double *)malloc(sizeof(double) * (size_t)(nT > 0 ? nT : 1));
    for (int j = 0; j < G; j++) {
        int h = g * G + j;
        double *o = out + (size_t)j * d;
        for (int i = 0; i < d; i++) o[i] = 0.0;
        if (nT == 0) continue;  /* empty set: zero output */
        double mu = -INFINITY;
        for (long t = 0; t < nT; t++) {                 /* pass 1: logits, max */
            z[t] = tau * dot_q(c, q, b, h, T[t].arr_k, T[t].row);
            if (z[t] > mu) mu = z[t];
        }
        double lam = 0.0;
        for (long t = 0; t < nT; t++) {                 /* pass 2: sums */
            double p = exp(z[t] - mu);
            lam += p;
            for (int i = 0; i < d; i++) o[i] += p * ld(T[t].arr_v, T[t].row + i, c->dtype);
        }
        for (int i = 0; i < d; i++) o[i] /= lam;
    }
    free(z);
}

/* ---- validation -------------------------------------------------------- */

static int check_cfg(const oracle_cfg *c, int hier) {
    if (c->batch < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1 || c->head_dim < 1) return 2;
    if (c->num_q_heads % c->num_kv_heads) return 2;
    if (c->top_k < 0 || c->num_chunks < 0 || c->chunk_size < 1 || c->page_chunks < 1) return 2;
    if (c->max_pages < 1 || c->num_pages < 1) return 2;
    if ((long)c->max_pages * c->page_chunks < c->num_chunks) return 2;
    if (c->dtype != 0 && c->dtype != 1) return 3;
    if (c->flags & ~(ORACLE_SCORE_SUM_PROBS | ORACLE_SET_SELECTED_GISTS | ORACLE_SELECT_TOP_P)) return 4;
    if (c->flags & ORACLE_SELECT_TOP_P) {
        if (hier || (c->flags & ORACLE_SCORE_SUM_PROBS)) return 4;
        if (!(c->top_p > 0.0f && c->top_p <= 1.0f)) return 2;
    }
    if (hier) {
        if (c->gists_per_meta < 1 || c->top_k_meta < 0) return 2;
        if (c->max_meta < c->num_chunks / c->gists_per_meta) return 2;
        if (c->flags & ORACLE_SET_SELECTED_GISTS) return 4;
    }
    return 0;
}

/* valid lengths only: 0 <= len <= num_chunks*C + C-1, pages covering it */
static int seq_shape(const oracle_cfg *c, const int32_t *seq_lens, int b,
                     int *n, int *tail) {
    long L = seq_lens ? seq_lens[b] : (long)c->num_chunks * c->chunk_size;
    if (L < 0) return 2;
    *n = (int)(L / c->chunk_size);
    *tail = (int)(L % c->chunk_size);
    if (*n > c->num_chunks) return 2;
    long slots = (long)(*n) * (c->chunk_size + 1) + *tail;
    if (slots > (long)c->max_pages * c->page_chunks * (c->chunk_size + 1)) return 2;
    return 0;
}

/* ---- GSA decode -------------------------------------------------------- */

static void gsa_unit(const oracle_cfg *c, const void *q, const void *kc, const void *vc,
                     const int32_t *bt, int b, int g, int n, int tail,
                     double *out, int32_t *sel_out, float *scores_out,
                     const int32_t *ext_sel) {
    int C = c->chunk_size, G = c->num_q_heads / c->num_kv_heads, d = c->head_dim;
    seqview sv = {c, kc, vc, bt, b, g};
    /* O1 */
    size_t *rows = (size_t *)malloc(sizeof(size_t) * (size_t)(n > 0 ? n : 1));
    int *ids = (int *)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    float *S = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    for (int m = 0; m < n; m++) {
        rows[m] = slot_base(&sv, (long)m * (C + 1) + C);
        ids[m] = m;
    }
    routing_keys(c, q, b, g, kc, rows, n, S);
    if (scores_out) {
        for (int m = 0; m < c->num_chunks; m++) scores_out[m] = m < n ? S[m] : -INFINITY;
    }
    /* O2 (or O6: caller's selection) */
    int *sel = (int *)malloc(sizeof(int) * (size_t)(c->top_k > 0 ? c->top_k : 1));
    int ns;
    if (ext_sel) {
        ns = 0;
        for (int i = 0; i < c->top_k; i++)
            if (ext_sel[i] >= 0 && ext_sel[i] < n) sel[ns++] = ext_sel[i];
        qsort(sel, (size_t)ns, sizeof(int), cmp_int);
    } else if (c->flags & ORACLE_SELECT_TOP_P) {
        ns = topp(S, ids, n, c->top_k, (double)c->top_p, sel);
    } else {
        ns = topk(S, ids, n, c->top_k, sel);
    }
    if (sel_out)
        for (int i = 0; i < c->top_k; i++) sel_out[i] = i < ns ? sel[i] : -1;
    /* O3: token set in ascending slot order */
    char *is_sel = (char *)calloc((size_t)(n > 0 ? n : 1), 1);
    for (int i = 0; i < ns; i++) is_sel[sel[i]] = 1;
    long cap = (long)n * (C + 1) + tail;
    tokref *T = (tokref *)malloc(sizeof(tokref) * (size_t)(cap > 0 ? cap : 1));
    long nT = 0;
    int all_gists = !(c->flags & ORACLE_SET_SELECTED_GISTS);
    for (int m = 0; m < n; m++) {
        long s0 = (long)m * (C + 1);
        if (is_sel[m])
            for (int r = 0; r < C; r++) { T[nT].arr_k = kc; T[nT].arr_v = vc; T[nT].row = slot_base(&sv, s0 + r); nT++; }
        if (is_sel[m] || all_gists) { T[nT].arr_k = kc; T[nT].arr_v = vc; T[nT].row = slot_base(&sv, s0 + C); nT++; }
    }
    for (int r = 0; r < tail; r++) { T[nT].arr_k = kc; T[nT].arr_v = vc; T[nT].row = slot_base(&sv, (long)n * (C + 1) + r); nT++; }
    /* O4 */
    attend(c, q, b, g, T, nT, out);
    (void)G; (void)d;
    free(T); free(is_sel); free(sel); free(S); free(ids); free(rows);
}

/* out: [B][Hq][d] double.  sel_idx: NULL or [B][Hkv][top_k] (ascending,
 * -1 padded).  scores: NULL or [B][Hkv][num_chunks] (-inf past each
 * sequence's gists).  ext_sel: NULL or [B][Hkv][top_k] caller selection
 * (entries < 0 ignored).  nthreads <= 0: OpenMP default.
 * Returns 0, or 2 bad shape, 3 bad dtype, 4 bad flags, 1 null pointer. */
int gsa_oracle_decode(const oracle_cfg *c, const void *q, const void *k_cache,
                      const void *v_cache, const int32_t *block_table,
                      const int32_t *seq_lens, double *out, int32_t *sel_idx,
                      float *scores, const int32_t *ext_sel, int nthreads) {
    if (!c || !q || !k_cache || !v_cache || !block_table || !out) return 1;
    int e = check_cfg(c, 0);
    if (e) return e;
    for (int b = 0; b < c->batch; b++) {
        int n, t;
        if ((e = seq_shape(c, seq_lens, b, &n, &t))) return e;
    }
    int units = c->batch * c->num_kv_heads;
    int G = c->num_q_heads / c->num_kv_heads, d = c->head_dim;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int u = 0; u < units; u++) {
        int b = u / c->num_kv_heads, g = u % c->num_kv_heads, n, tail;
        seq_shape(c, seq_lens, b, &n, &tail);
        gsa_unit(c, q, k_cache, v_cache, block_table, b, g, n, tail,
                 out + ((size_t)b * c->num_q_heads + (size_t)g * G) * d,
                 sel_idx ? sel_idx + (size_t)u * c->top_k : NULL,
                 scores ? scores + (size_t)u * c->num_chunks : NULL,
                 ext_sel ? ext_sel + (size_t)u * c->top_k : NULL);
    }
    (void)nthreads;
    return 0;
}

/* ---- H-GSA decode ------------------------------------------------------ */

static void hgsa_unit(const oracle_cfg *c, const void *q, const void *kc, const void *vc,
                      const int32_t *bt, const void *km, const void *vm, int b, int g,
                      int n, int tail, double *out, int32_t *sel1_out, int32_t *sel2_out,
                      float *mscores_out, float *gscores_out,
                      const int32_t *ext1, const int32_t *ext2) {
    int C = c->chunk_size, R = c->gists_per_meta, d = c->head_dim;
    int k1 = c->top_k_meta, k2 = c->top_k;
    int nm = n / R;                 /* complete meta-groups */
    seqview sv = {c, kc, vc, bt, b, g};
    size_t mbase = ((size_t)b * c->num_kv_heads + g) * (size_t)c->max_meta * d;
    /* level 1: meta-gist keys, top-k1 */
    size_t *mrows = (size_t *)malloc(sizeof(size_t) * (size_t)(nm > 0 ? nm : 1));
    int *mids = (int *)malloc(sizeof(int) * (size_t)(nm > 0 ? nm : 1));
    float *SM = (float *)malloc(sizeof(float) * (size_t)(nm > 0 ? nm : 1));
    for (int r = 0; r < nm; r++) { mrows[r] = mbase + (size_t)r * d; mids[r] = r; }
    routing_keys(c, q, b, g, km, mrows, nm, SM);
    if (mscores_out)
        for (int r = 0; r < c->max_meta; r++) mscores_out[r] = r < nm ? SM[r] : -INFINITY;
    int *sel1 = (int *)malloc(sizeof(int) * (size_t)(k1 > 0 ? k1 : 1));
    int ns1;
    if (ext1) {
        ns1 = 0;
        for (int i = 0; i < k1; i++) if (ext1[i] >= 0 && ext1[i] < nm) sel1[ns1++] = ext1[i];
        qsort(sel1, (size_t)ns1, sizeof(int), cmp_int);
    } else {
        ns1 = topk(SM, mids, nm, k1, sel1);
    }
    if (sel1_out) for (int i = 0; i < k1; i++) sel1_out[i] = i < ns1 ? sel1[i] : -1;
    /* level 2: candidate gists = gists of kept groups + gists past the last
     * complete group; their keys, top-k2 */
    int ncand_max = ns1 * R + (n - nm * R);
    size_t *crows = (size_t *)malloc(sizeof(size_t) * (size_t)(ncand_max > 0 ? ncand_max : 1));
    int *cids = (int *)malloc(sizeof(int) * (size_t)(ncand_max > 0 ? ncand_max : 1));
    float *SC = (float *)malloc(sizeof(float) * (size_t)(ncand_max > 0 ? ncand_max : 1));
    int nc = 0;
    for (int i = 0; i < ns1; i++)
        for (int j = 0; j < R; j++) cids[nc++] = sel1[i] * R + j;
    for (int m = nm * R; m < n; m++) cids[nc++] = m;
    for (int i = 0; i < nc; i++) crows[i] = slot_base(&sv, (long)cids[i] * (C + 1) + C);
    if (gscores_out) {
        /* every gist's key, for tests (candidates or not) */
        size_t *arows = (size_t *)malloc(sizeof(size_t) * (size_t)(n > 0 ? n : 1));
        float *SA = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
        for (int m = 0; m < n; m++) arows[m] = slot_base(&sv, (long)m * (C + 1) + C);
        oracle_cfg c2 = *c;
        c2.flags &= ~ORACLE_SCORE_SUM_PROBS;
        routing_keys(&c2, q, b, g, kc, arows, n, SA);
        for (int m = 0; m < c->num_chunks; m++) gscores_out[m] = m < n ? SA[m] : -INFINITY;
        free(arows); free(SA);
    }
    routing_keys(c, q, b, g, kc, crows, nc, SC);
    int *sel2 = (int *)malloc(sizeof(int) * (size_t)(k2 > 0 ? k2 : 1));
    int ns2;
    if (ext2) {
        ns2 = 0;
        for (int i = 0; i < k2; i++) if (ext2[i] >= 0 && ext2[i] < n) sel2[ns2++] = ext2[i];
        qsort(sel2, (size_t)ns2, sizeof(int), cmp_int);
    } else {
        ns2 = topk(SC, cids, nc, k2, sel2);
    }
    if (sel2_out) for (int i = 0; i < k2; i++) sel2_out[i] = i < ns2 ? sel2[i] : -1;
    /* set: all meta-gists, kept gists + their raw tokens, gists past the last
     * complete group, raw tail */
    char *is_sel = (char *)calloc((size_t)(n > 0 ? n : 1), 1);
    for (int i = 0; i < ns2; i++) is_sel[sel2[i]] = 1;
    long cap = nm + (long)n * (C + 1) + tail;
    tokref *T = (tokref *)malloc(sizeof(tokref) * (size_t)(cap > 0 ? cap : 1));
    long nT = 0;
    for (int r = 0; r < nm; r++) { T[nT].arr_k = km; T[nT].arr_v = vm; T[nT].row = mbase + (size_t)r * d; nT++; }
    for (int m = 0; m < n; m++) {
        long s0 = (long)m * (C + 1);
        if (is_sel[m])
            for (int r = 0; r < C; r++) { T[nT].arr_k = kc; T[nT].arr_v = vc; T[nT].row = slot_base(&sv, s0 + r); nT++; }
        if (is_sel[m] || m >= nm * R) { T[nT].arr_k = kc; T[nT].arr_v = vc; T[nT].row = slot_base(&sv, s0 + C); nT++; }
    }
    for (int r = 0; r < tail; r++) { T[nT].arr_k = kc; T[nT].arr_v = vc; T[nT].row = slot_base(&sv, (long)n * (C + 1) + r); nT++; }
    attend(c, q, b, g, T, nT, out);
    free(T); free(is_sel); free(sel2); free(SC); free(cids); free(crows);
    free(sel1); free(SM); free(mids); free(mrows);
}

/* k_meta, v_meta: [B][Hkv][max_meta][d].  sel_meta: NULL or [B][Hkv][k1];
 * sel_idx: NULL or [B][Hkv][k2]; meta_scores: NULL or [B][Hkv][max_meta];
 * gist_scores: NULL or [B][Hkv][num_chunks] (plain logit-sum keys of every
 * gist).  ext_sel_meta / ext_sel: NULL or caller selections. */
int hgsa_oracle_decode(const oracle_cfg *c, const void *q, const void *k_cache,
                       const void *v_cache, const int32_t *block_table,
                       const int32_t *seq_lens, const void *k_meta, const void *v_meta,
                       double *out, int32_t *sel_meta, int32_t *sel_idx,
                       float *meta_scores, float *gist_scores,
                       const int32_t *ext_sel_meta, const int32_t *ext_sel, int nthreads) {
    if (!c || !q || !k_cache || !v_cache || !block_table || !k_meta || !v_meta || !out) return 1;
    int e = check_cfg(c, 1);
    if (e) return e;
    for (int b = 0; b < c->batch; b++) {
        int n, t;
        if ((e = seq_shape(c, seq_lens, b, &n, &t))) return e;
    }
    int units = c->batch * c->num_kv_heads;
    int G = c->num_q_heads / c->num_kv_heads, d = c->head_dim;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int u = 0; u < units; u++) {
        int b = u / c->num_kv_heads, g = u % c->num_kv_heads, n, tail;
        seq_shape(c, seq_lens, b, &n, &tail);
        hgsa_unit(c, q, k_cache, v_cache, block_table, k_meta, v_meta, b, g, n, tail,
                  out + ((size_t)b * c->num_q_heads + (size_t)g * G) * d,
                  sel_meta ? sel_meta + (size_t)u * c->top_k_meta : NULL,
                  sel_idx ? sel_idx + (size_t)u * c->top_k : NULL,
                  meta_scores ? meta_scores + (size_t)u * c->max_meta : NULL,
                  gist_scores ? gist_scores + (size_t)u * c->num_chunks : NULL,
                  ext_sel_meta ? ext_sel_meta + (size_t)u * c->top_k_meta : NULL,
                  ext_sel ? ext_sel + (size_t)u * c->top_k : NULL);
    }
    (void)nthreads;
    return 0;
}

/* ---- O7: hierarchy of L levels ----------------------------------------- */

/* one level of meta-gists (level l >= 1; level 0 is the gists themselves) */
typedef struct {
    const void *k, *v;   /* [B][Hkv][max_entries][d] */
    int max_entries;     /* >= entries of the level below / fanout */
    int fanout;          /* R_l >= 1 */
    int top_k;           /* k_l >= 0 entries kept */
} oracle_level;

/* Keep the ids of an external selection that lie in [0, count), ascending. */
static int ext_filter(const int32_t *ext, int k, int count, int *sel) {
    int ns = 0;
    for (int i = 0; i < k; i++) if (ext[i] >= 0 && ext[i] < count) sel[ns++] = ext[i];
    qsort(sel, (size_t)ns, sizeof(int), cmp_int);
    return ns;
}

static void mgsa_unit(const oracle_cfg *c, const void *q, const void *kc, const void *vc,
                      const int32_t *bt, const oracle_level *lv, int L, int b, int g,
                      int n, int tail, double *out, int32_t *const *sel_out, float *const *key_out,
                      const int32_t *const *ext, size_t u) {
    int C = c->chunk_size, d = c->head_dim;
    seqview sv = {c, kc, vc, bt, b, g};
    int cnt[33];                 /* entries per level */
    cnt[0] = n;
    for (int l = 1; l <= L; l++) cnt[l] = cnt[l - 1] / lv[l - 1].fanout;
    /* flat index of entry r of level l (level 0: the gist row in the cache) */
#define ROW_OF(l, r) ((l) == 0 ? slot_base(&sv, (long)(r) * (C + 1) + C) \
                     : ((size_t)b * c->num_kv_heads + g) * (size_t)lv[(l) - 1].max_entries * d + (size_t)(r) * d)
#define ARR_K(l) ((l) == 0 ? kc : lv[(l) - 1].k)
#define ARR_V(l) ((l) == 0 ? vc : lv[(l) - 1].v)
    /* keys of every entry of every level (tests), plain logit sums */
    for (int l = 0; l <= L; l++) {
        if (!key_out || !key_out[l]) continue;
        int nl = cnt[l], cap = l == 0 ? c->num_chunks : lv[l - 1].max_entries;
        size_t *rows = (size_t *)malloc(sizeof(size_t) * (size_t)(nl > 0 ? nl : 1));
        float *S = (float *)malloc(sizeof(float) * (size_t)(nl > 0 ? nl : 1));
        for (int r = 0; r < nl; r++) rows[r] = ROW_OF(l, r);
        routing_keys(c, q, b, g, ARR_K(l), rows, nl, S);
        for (int r = 0; r < cap; r++) key_out[l][u * cap + r] = r < nl ? S[r] : -INFINITY;
        free(rows); free(S);
    }
    /* coarse to fine: candidates of the top level are all its entries */
    int *sel[33];
    int nsel[33];
    int *cand = (int *)malloc(sizeof(int) * (size_t)(cnt[L] > 0 ? cnt[L] : 1));
    int nc = cnt[L];
    for (int r = 0; r < nc; r++) cand[r] = r;
    for (int l = L; l >= 0; l--) {
        int k = l == 0 ? c->top_k : lv[l - 1].top_k;
        size_t *rows = (size_t *)malloc(sizeof(size_t) * (size_t)(nc > 0 ? nc : 1));
        float *S = (float *)malloc(sizeof(float) * (size_t)(nc > 0 ? nc : 1));
        for (int i = 0; i < nc; i++) rows[i] = ROW_OF(l, cand[i]);
        routing_keys(c, q, b, g, ARR_K(l), rows, nc, S);
        sel[l] = (int *)malloc(sizeof(int) * (size_t)(k > 0 ? k : 1));
        if (ext && ext[l]) nsel[l] = ext_filter(ext[l] + u * k, k, cnt[l], sel[l]);
        else nsel[l] = topk(S, cand, nc, k, sel[l]);
        if (sel_out && sel_out[l])
            for (int i = 0; i < k; i++) sel_out[l][u * k + i] = i < nsel[l] ? sel[l][i] : -1;
        free(rows); free(S);
        if (l > 0) {  /* children of the kept entries, then the entries past the last group */
            int R = lv[l - 1].fanout;
            int nn = nsel[l] * R + (cnt[l - 1] - cnt[l] * R);
            free(cand);
            cand = (int *)malloc(sizeof(int) * (size_t)(nn > 0 ? nn : 1));
            nc = 0;
            for (int i = 0; i < nsel[l]; i++)
                for (int j = 0; j < R; j++) cand[nc++] = sel[l][i] * R + j;
            for (int r = cnt[l] * R; r < cnt[l - 1]; r++) cand[nc++] = r;
        }
    }
    free(cand);
    /* the set */
    long cap = (long)n * (C + 1) + tail;
    for (int l = 1; l <= L; l++) cap += cnt[l];
    tokref *T = (tokref *)malloc(sizeof(tokref) * (size_t)(cap > 0 ? cap : 1));
    long nT = 0;
    for (int l = L; l >= 1; l--) {
        /* top level: every entry; below: kept or past the last complete group */
        char *in = (char *)calloc((size_t)(cnt[l] > 0 ? cnt[l] : 1), 1);
        for (int i = 0; i < nsel[l]; i++) in[sel[l][i]] = 1;
        int past = l == L ? 0 : cnt[l + 1] * lv[l].fanout;
        for (int r = 0; r < cnt[l]; r++)
            if (l == L || in[r] || r >= past) {
                T[nT].arr_k = ARR_K(l); T[nT].arr_v = ARR_V(l); T[nT].row = ROW_OF(l, r); nT++;
            }
        free(in);
    }
    char *is_sel = (char *)calloc((size_t)(n > 0 ? n : 1), 1);
    for (int i = 0; i < nsel[0]; i++) is_sel[sel[0][i]] = 1;
    int past0 = L == 0 ? 0 : cnt[1] * lv[0].fanout;
    for (int m = 0; m < n; m++) {
        long s0 = (long)m * (C + 1);
        if (is_sel[m])
            for (int r = 0; r < C; r++) { T[nT].arr_k = kc; T[nT].arr_v = vc; T[nT].row = slot_base(&sv, s0 + r); nT++; }
        if (L == 0 || is_sel[m] || m >= past0) { T[nT].arr_k = kc; T[nT].arr_v = vc; T[nT].row = slot_base(&sv, s0 + C); nT++; }
    }
    for (int r = 0; r < tail; r++) { T[nT].arr_k = kc; T[nT].arr_v = vc; T[nT].row = slot_base(&sv, (long)n * (C + 1) + r); nT++; }
    attend(c, q, b, g, T, nT, out);
    free(T); free(is_sel);
    for (int l = 0; l <= L; l++) free(sel[l]);
#undef ROW_OF
#undef ARR_K
#undef ARR_V
}

/* L (0..32) levels of meta-gists above the gists.  Level arrays are indexed
 * by level l = 1..L at [l - 1]: k_levels / v_levels [B][Hkv][max_entries][d],
 * fanout R_l, top_k_levels k_l.  sel / keys / ext: NULL, or L + 1 pointers
 * (each NULL or an array), level 0 (the gists) first: sel[0] [B][Hkv][top_k],
 * sel[l] [B][Hkv][k_l]; keys[0] [B][Hkv][num_chunks], keys[l]
 * [B][Hkv][max_entries_l] (plain logit-sum keys of every entry, -inf past
 * the sequence's entries); ext[l]: caller selections, as sel.
 * Returns 0, or 1 null pointer, 2 bad shape, 3 bad dtype, 4 bad flags. */
int mgsa_oracle_decode(const oracle_cfg *c, const void *q, const void *k_cache,
                       const void *v_cache, const int32_t *block_table, const int32_t *seq_lens,
                       int num_levels, const void *const *k_levels, const void *const *v_levels,
                       const int *max_entries, const int *fanout, const int *top_k_levels,
                       double *out, int32_t *const *sel, float *const *keys,
                       const int32_t *const *ext, int nthreads) {
    if (!c || !q || !k_cache || !v_cache || !block_table || !out) return 1;
    if (num_levels < 0 || num_levels > 32) return 2;
    int e = check_cfg(c, 0);
    if (e) return e;
    if (num_levels > 0 && (c->flags & (ORACLE_SET_SELECTED_GISTS | ORACLE_SCORE_SUM_PROBS |
                                       ORACLE_SELECT_TOP_P))) return 4;
    oracle_level lv[32];
    long below = c->num_chunks;
    for (int l = 0; l < num_levels; l++) {
        if (!k_levels || !v_levels || !max_entries || !fanout || !top_k_levels) return 1;
        if (!k_levels[l] || !v_levels[l]) return 1;
        lv[l].k = k_levels[l]; lv[l].v = v_levels[l];
        lv[l].max_entries = max_entries[l]; lv[l].fanout = fanout[l]; lv[l].top_k = top_k_levels[l];
        if (lv[l].fanout < 1 || lv[l].top_k < 0) return 2;
        below /= lv[l].fanout;
        if (lv[l].max_entries < below) return 2;
    }
    for (int b = 0; b < c->batch; b++) {
        int n, t;
        if ((e = seq_shape(c, seq_lens, b, &n, &t))) return e;
    }
    int units = c->batch * c->num_kv_heads;
    int G = c->num_q_heads / c->num_kv_heads, d = c->head_dim;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int u = 0; u < units; u++) {
        int b = u / c->num_kv_heads, g = u % c->num_kv_heads, n, tail;
        seq_shape(c, seq_lens, b, &n, &tail);
        mgsa_unit(c, q, k_cache, v_cache, block_table, lv, num_levels, b, g, n, tail,
                  out + ((size_t)b * c->num_q_heads + (size_t)g * G) * d, sel, keys, ext, (size_t)u);
    }
    (void)nthreads;
    return 0;
}

/* ---- O8: prefill under the gist causal mask ---------------------------- */

/* q, out: [B][T][Hq][d] (out double).  q_start: [B] logical slot of each
 * sequence's first query; every query slot q_start[b] + t must lie within the
 * block-table row.  Returns 0, or 1 null pointer, 2 bad shape, 3 bad dtype. */
int gsa_prefill_oracle(const oracle_cfg *c, const void *q, const void *k_cache,
                       const void *v_cache, const int32_t *block_table, const int32_t *q_start,
                       int T, double *out, int nthreads) {
    if (!c || !q || !k_cache || !v_cache || !block_table || !q_start || !out) return 1;
    if (c->batch < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1 || c->head_dim < 1) return 2;
    if (c->num_q_heads % c->num_kv_heads || c->chunk_size < 1 || c->page_chunks < 1) return 2;
    if (c->max_pages < 1 || T < 0) return 2;
    if (c->dtype != 0 && c->dtype != 1) return 3;
    long spp = (long)c->page_chunks * (c->chunk_size + 1);
    for (int b = 0; b < c->batch; b++)
        if (q_start[b] < 0 || (long)q_start[b] + T > (long)c->max_pages * spp) return 2;
    int C = c->chunk_size, d = c->head_dim, Hq = c->num_q_heads;
    int G = Hq / c->num_kv_heads;
    double tau = tau_of(c);
    long rows = (long)c->batch * T * Hq;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
#endif
    for (long i = 0; i < rows; i++) {
        int h = (int)(i % Hq), t = (int)((i / Hq) % T), b = (int)(i / ((long)Hq * T));
        seqview sv = {c, k_cache, v_cache, block_table, b, h / G};
        long s = (long)q_start[b] + t;
        long m = s / (C + 1);
        long nk = m + (s - m * (C + 1)) + 1;
        size_t *krow = (size_t *)malloc(sizeof(size_t) * (size_t)nk);
        double *z = (double *)malloc(sizeof(double) * (size_t)nk);
        long j = 0;
        for (long mp = 0; mp < m; mp++) krow[j++] = slot_base(&sv, mp * (C + 1) + C);
        for (long sp = m * (C + 1); sp <= s; sp++) krow[j++] = slot_base(&sv, sp);
        size_t qb = (((size_t)b * T + t) * Hq + h) * d;
        double mu = -INFINITY;
        for (j = 0; j < nk; j++) {                     /* pass 1: logits, max */
            double acc = 0.0;
            for (int e = 0; e < d; e++) acc += ld(q, qb + e, c->dtype) * ld(k_cache, krow[j] + e, c->dtype);
            z[j] = tau * acc;
            if (z[j] > mu) mu = z[j];
        }
        double lam = 0.0, *o = out + qb;
        for (int e = 0; e < d; e++) o[e] = 0.0;
        for (j = 0; j < nk; j++) {                     /* pass 2: sums */
            double p = exp(z[j] - mu);
            lam += p;
            for (int e = 0; e < d; e++) o[e] += p * ld(v_cache, krow[j] + e, c->dtype);
        }
        for (int e = 0; e < d; e++) o[e] /= lam;
        free(krow); free(z);
    }
    (void)nthreads;
    return 0;
}

int gsa_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
