/*
 * gsa.h -- C ABI of the gist sparse attention (GSA) decode library for
 * MI355X (gfx950).
 *
 * One decode step of "Forget, Then Recall: Learnable Compression and
 * Selective Unfolding via Gist Sparse Attention", as described on the
 * gist.science technical summaries of that paper (ja / ko / nl pages):
 *
 *   1. score every gist of the cached context against the current query,
 *      s_{t,m} = q_t . k_{g_m}  (nl page, Methodologie, "Het Proces",
 *      Scoring; ja page, section 2.1 item 2);
 *   2. keep the top-k chunks (ja page 2.1 item 3; nl page, "Selectie");
 *   3. unfold the raw tokens of those chunks (nl page, "Selectieve
 *      Ontvouwing");
 *   4. attend over the gist tokens plus the unfolded raw tokens (ja page 2.1
 *      item 4, "hybrid attention"; ko page, methodology, hybrid attention).
 * hgsa_decode adds the coarse-to-fine gist-of-gist level (ja page 2.2; nl
 * page, "Hierarchische Uitbreiding").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensors are caller-owned device memory (HIP device pointers), dense
 *    row-major with the shapes given below.  The library allocates nothing,
 *    keeps no pointer after a call returns and has no global mutable state.
 *  - Every host-side argument is validated before anything is enqueued.  On
 *    an error nothing is launched, no output is touched and the status is
 *    returned; nothing aborts or throws across this ABI.
 *  - GSA_OK means the work has been enqueued on `stream` (a hipStream_t;
 *    NULL is the null stream); results are ready after the caller
 *    synchronises with that stream.  Device faults surface there.
 *  - Sequence lengths and block tables are device arrays read by the
 *    kernels; their contents must satisfy the constraints stated below (the
 *    host cannot check device memory without a synchronisation).  Lengths
 *    outside [0, num_chunks*C + C-1] are clamped into that range.
 *  - Two calls that share one workspace must not overlap in time.
 */
#ifndef GSA_H_
#define GSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GSA_OK = 0,
    GSA_ERR_NULL_ARG = 1,   /* a required pointer is NULL */
    GSA_ERR_BAD_SHAPE = 2,  /* a size or count is out of range */
    GSA_ERR_BAD_DTYPE = 3,  /* dtype not GSA_F32 / GSA_BF16 */
    GSA_ERR_BAD_FLAGS = 4,  /* unknown or unsupported flag bits */
    GSA_ERR_WORKSPACE = 5,  /* workspace NULL, too small or misaligned */
    GSA_ERR_DEVICE = 6,     /* no usable HIP device / the current device is not gfx950 */
    GSA_ERR_LAUNCH = 7,     /* a kernel launch failed */
    GSA_ERR_WAIT = 8        /* gsa_workspace_status: a bounded wait inside the
                               single-launch kernel gave up (see below) */
} gsa_status_t;

typedef enum { GSA_F32 = 0, GSA_BF16 = 1 } gsa_dtype_t;

/* Routing key shared by the query heads of one GQA group (one selection per
 * (batch, kv-head)).  Default: the sum over the group of the scaled logits
 * sm_scale * q_h . k_gist.  SUM_PROBS: the sum over the group of each head's
 * softmax probability of the gist, the softmax taken over the sequence's gists
 * (gsa_decode only; it needs every gist's logits before any key, so the call
 * runs the multi-launch kernels). */
#define GSA_SCORE_SUM_LOGITS 0x0u
#define GSA_SCORE_SUM_PROBS 0x1u
/* Attention set.  Default: every gist plus the raw tokens of the selected
 * chunks.  SELECTED_GISTS: only the selected chunks' gists plus their raw
 * tokens (the "SG+SR" rule of the ja page's ablation, section 4). */
#define GSA_SET_ALL_GISTS 0x0u
#define GSA_SET_SELECTED_GISTS 0x2u
/* Selection rule.  Default: the top_k largest keys.  SELECT_TOP_P: top-p
 * (nucleus) selection, the alternative the ja page's ablation (section 4) and
 * the nl page's results ("Stabiliteit") compare with top-k: the chunks in key
 * order (largest first, ties to the lower index, NaN last) up to and including
 * the first at which the running sum of their selection probabilities reaches
 * top_p, at most top_k of them (top_k <= 2048 then).  A chunk's selection
 * probability is the softmax of its key over the sequence's gists (NaN keys:
 * 0); with no finite largest key the first min(top_k, n) are taken.  Default
 * key only; gsa_decode only; runs the multi-launch kernels.  sel_idx then holds
 * a variable number of ids per (batch, kv-head), -1 padded. */
#define GSA_SELECT_TOP_P 0x4u
/* Run the portable fp32-VALU kernels instead of the MFMA kernels (the fp32
 * dtype always uses them); a cross-check of the bf16 MFMA path. */
#define GSA_PATH_PORTABLE 0x100u

typedef struct {
    int32_t batch;         /* B >= 1 */
    int32_t num_q_heads;   /* Hq >= 1, a multiple of num_kv_heads */
    int32_t num_kv_heads;  /* Hkv >= 1; query head h reads kv-head h / (Hq/Hkv) */
    int32_t head_dim;      /* d: 64 or 128 */
    int32_t top_k;         /* chunks unfolded per (batch, kv-head), >= 0; clamped
                              per sequence to its gist count; 0 = gists only.
                              For hgsa_decode: k2, the gist-level top-k. */
    float sm_scale;        /* softmax scale tau; <= 0 selects 1/sqrt(d) */
    int32_t dtype;         /* gsa_dtype_t of q, caches, meta caches and out */
    uint32_t flags;        /* GSA_SCORE_* | GSA_SET_* | GSA_SELECT_* | GSA_PATH_* */
    float top_p;           /* with GSA_SELECT_TOP_P: probability mass to keep, in (0, 1];
                              ignored otherwise */
} gsa_params_t;

/* Paged interleaved raw+gist KV cache.
 *   k_cache, v_cache : [num_pages][num_kv_heads][page_chunks*(chunk_size+1)][head_dim]
 * Logical slot s of a sequence holds raw token c of chunk m at
 * s = m*(C+1) + c (c < C) and the gist of chunk m at s = m*(C+1) + C, i.e. one
 * gist token after every chunk of C raw tokens (ja page 2.1 item 1).  Logical
 * page p = s / (page_chunks*(C+1)) of sequence b is physical page
 * block_table[b*max_pages + p]; pages may be shared between sequences.
 *   block_table : int32 [batch][max_pages], entries in [0, num_pages)
 *   seq_lens    : int32 [batch] raw tokens per sequence, or NULL meaning
 *                 num_chunks*chunk_size for all.  A sequence of L raw tokens
 *                 has L/C complete chunks (each with its gist) and L%C raw
 *                 tokens after its last gist, which are always attended.
 *                 Its block-table row must map every page those
 *                 (L/C)*(C+1) + L%C slots touch. */
typedef struct {
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_table;
    const int32_t* seq_lens;
    int32_t num_chunks;    /* capacity in chunks (>= L/C of every sequence) */
    int32_t chunk_size;    /* C >= 1 */
    int32_t page_chunks;   /* chunks per page >= 1 */
    int32_t num_pages;     /* physical pages in the caches >= 1 */
    int32_t max_pages;     /* block-table row length >= 1 */
} gsa_kv_t;

/* Meta-gists for hgsa_decode.  Meta-gist r of a sequence summarises gists
 * [r*R, r*R + R) and exists once all R of them exist; gists after the last
 * complete group are always attended and are always candidates.
 *   k_meta, v_meta : [batch][num_kv_heads][max_meta][head_dim]  */
typedef struct {
    const void* k_meta;
    const void* v_meta;
    int32_t max_meta;        /* >= num_chunks / gists_per_meta */
    int32_t gists_per_meta;  /* R >= 1 */
    int32_t top_k_meta;      /* k1 >= 0 meta-gists kept per (batch, kv-head) */
} hgsa_meta_t;

/* Size of the control block at the start of every workspace: an error word
 * and the per-(batch, kv-head) counters of the single-launch path and of
 * mgsa_decode's final attention. */
#define GSA_WORKSPACE_CONTROL_BYTES ((size_t)16384 + (size_t)512 * 25088)
/* Byte offset (in the control block) of the 32-bit error word.  The
 * single-launch kernel's workgroups hand data to each other through the
 * control block and wait for it with bounded polls; a wait that gives up
 * (never expected: it would take a device that stops dispatching queued
 * workgroups) sets this word to 1 and the kernel finishes with partial data.
 * The call's outputs are then unreliable and the control block may be left
 * non-zero.  gsa_workspace_status reads the word; gsa_workspace_reset clears
 * the control block again, after which the workspace is usable. */
#define GSA_WORKSPACE_ERROR_OFFSET ((size_t)8)

/* Bytes of device workspace gsa_decode needs for these shapes (0 if the
 * shapes are invalid).  The workspace must be 256-byte aligned and its first
 * GSA_WORKSPACE_CONTROL_BYTES (the control block) must be zero before its
 * first use; every call that completes leaves that block zero again and uses
 * the rest as scratch, so one zero-filled allocation serves any number of
 * sequential calls, of any shapes that fit it. */
size_t gsa_workspace_size(const gsa_params_t* p, const gsa_kv_t* kv);

/* As gsa_workspace_size, for hgsa_decode. */
size_t hgsa_workspace_size(const gsa_params_t* p, const gsa_kv_t* kv,
                           const hgsa_meta_t* meta);

/* One GSA decode step for every (batch, query head).
 *   q       : [batch][num_q_heads][head_dim], dtype
 *   out     : [batch][num_q_heads][head_dim], dtype (rounded to nearest even
 *             from the fp32 result for bf16)
 *   sel_idx : NULL, or int32 [batch][num_kv_heads][top_k]: selected chunk
 *             ids in ascending order, -1 in unused slots
 *   scores  : NULL, or float [batch][num_kv_heads][num_chunks]: routing key
 *             of every gist, -inf past each sequence's gists
 * Selection: the top_k largest keys, ties to the lower chunk index, NaN keys
 * last. */
gsa_status_t gsa_decode(const gsa_params_t* p, const gsa_kv_t* kv, const void* q,
                        void* out, int32_t* sel_idx, float* scores,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Size of the library-owned workspace of gsa_decode_noalloc (64 MiB per GPU). */
#define GSA_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)

/* gsa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and results as gsa_decode, without the workspace: the call uses a
 * library-owned device array of GSA_NOALLOC_WORKSPACE_BYTES that each GPU
 * holds from the library's first use on it until the process ends, and calls
 * no allocating routine.  Shapes whose gsa_workspace_size exceeds that size
 * return GSA_ERR_WORKSPACE (nothing enqueued).  Each call first clears, with a
 * fill kernel on `stream`, the part of the array's control block it uses, so
 * it does not depend on earlier calls (a given-up wait is not reported).
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (two streams, two threads) race and must be serialised by the
 * caller. */
gsa_status_t gsa_decode_noalloc(const gsa_params_t* p, const gsa_kv_t* kv, const void* q,
                                void* out, int32_t* sel_idx, float* scores, void* stream);

/* One H-GSA decode step: keep the top_k_meta meta-gists by routing key, score
 * the gists of the kept groups (plus the gists after the last complete
 * group), keep the top_k of those, and attend over every meta-gist, the kept
 * gists, the gists after the last complete group, the raw tokens of the kept
 * chunks and the raw tokens after the last gist.  flags: 0 (the default key
 * and set) or GSA_PATH_PORTABLE; other flags return GSA_ERR_BAD_FLAGS.
 *   sel_meta : NULL, or int32 [batch][num_kv_heads][top_k_meta] ascending, -1 padded
 *   sel_idx  : NULL, or int32 [batch][num_kv_heads][top_k] ascending, -1 padded */
gsa_status_t hgsa_decode(const gsa_params_t* p, const gsa_kv_t* kv,
                         const hgsa_meta_t* meta, const void* q, void* out,
                         int32_t* sel_meta, int32_t* sel_idx, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Waits for `stream` (a hipStream_t, NULL: the null stream), then reads the
 * error word of `workspace`: GSA_OK if it is zero, GSA_ERR_WAIT if a wait of
 * some call since the last reset gave up.  GSA_ERR_NULL_ARG / GSA_ERR_WORKSPACE
 * for a NULL, misaligned or too-small (< GSA_WORKSPACE_CONTROL_BYTES)
 * workspace; GSA_ERR_DEVICE if the wait or the read fails. */
gsa_status_t gsa_workspace_status(const void* workspace, size_t workspace_bytes, void* stream);

/* Enqueues on `stream` the zeroing of the control block of `workspace` (a
 * fill kernel, so the call can be captured in a HIP graph): the recovery step
 * after GSA_ERR_WAIT, or the first-use preparation of a fresh workspace.
 * Must not overlap a decode call that uses the same workspace. */
gsa_status_t gsa_workspace_reset(void* workspace, size_t workspace_bytes, void* stream);

/* Hierarchy of any depth.  One level of meta-gists: level 1 lies over the
 * gists, level l over level l-1; entry r of level l summarises entries
 * [r*fanout, (r+1)*fanout) of the level below and exists once all of them do
 * (the gist-of-gist structure built recursively, ja page 2.2; nl page,
 * "Hierarchische Uitbreiding").
 *   k_meta, v_meta : [batch][num_kv_heads][max_meta][head_dim], dtype */
typedef struct {
    const void* k_meta;
    const void* v_meta;
    int32_t max_meta;   /* >= the level's entries at full capacity: num_chunks
                           divided (rounding down) by the fanouts up to this level */
    int32_t fanout;     /* R_l >= 1 */
    int32_t top_k;      /* k_l >= 0 entries kept at this level */
} gsa_level_t;

#define GSA_MAX_LEVELS 8

/* Bytes of workspace mgsa_decode needs (0 if the shapes are invalid); the
 * same rules as gsa_workspace_size: 256-byte aligned, the control block first,
 * zero before the first use and left zero by every call that completes (the
 * call counts its final attention's workgroups there, one word per
 * (batch, kv-head)). */
size_t mgsa_workspace_size(const gsa_params_t* p, const gsa_kv_t* kv, const gsa_level_t* levels,
                           int32_t num_levels);

/* One decode step over num_levels (0 .. GSA_MAX_LEVELS) levels of meta-gists
 * above the gists, coarse to fine: every entry of the top level is scored and
 * attended and its top-k kept; at each level below, the candidates are the
 * children of the entries kept one level up plus the entries past the level's
 * last complete group, and their top-k is kept (the gist level's k is
 * p->top_k); the kept chunks' raw tokens are unfolded.  Attention set: every
 * top-level entry, the kept entries and the past-the-last-group entries of
 * each level below the top (gists included), the kept chunks' raw tokens and
 * the raw tail.  num_levels = 0 is flat GSA, 1 the two-level H-GSA of
 * hgsa_decode.  bf16 only, default key and set (flags 0).
 *   levels : [num_levels], level 1 first (NULL if num_levels = 0)
 *   sel    : NULL, or num_levels + 1 pointers (each NULL or int32
 *            [batch][num_kv_heads][k]), the gist level first (k = p->top_k),
 *            then level l (k = levels[l-1].top_k): kept ids ascending, -1 padded */
gsa_status_t mgsa_decode(const gsa_params_t* p, const gsa_kv_t* kv, const gsa_level_t* levels,
                         int32_t num_levels, const void* q, void* out, int32_t* const* sel,
                         void* workspace, size_t workspace_bytes, void* stream);

/* The multi-query side: num_queries consecutive slots of each sequence's
 * interleaved layout attend under the gist causal mask (ja page 2.1 item 1:
 * gists trained under a causal mask to summarise their chunk; nl page, "Het
 * Proces", Compressie: a gist sees only its own chunk and the gists before
 * it).  The query at slot s of chunk m = s / (C+1) attends to the gists of
 * chunks before m and to the slots of chunk m up to and including s (raw
 * tokens of earlier chunks are present only through their gists).  This is
 * the step that builds the interleaved cache (chunked prefill, one chunk of
 * slots at a time) and the one that checks several draft tokens at once; the
 * caller writes the queries' own K/V rows into the cache first.
 *   q_start : int32 device [batch], first query slot of each sequence, with
 *             q_start[b] + num_queries <= max_pages * page_chunks * (C+1)
 *             (clamped into that range)
 *   q, out  : [batch][num_queries][num_q_heads][head_dim], bf16
 * Uses kv's caches, block table, chunk size and page geometry; seq_lens,
 * top_k and num_chunks (beyond validation) are not used.  bf16 only, flags 0.
 * No workspace: the kernel keeps every query's state on chip. */
gsa_status_t gsa_prefill(const gsa_params_t* p, const gsa_kv_t* kv, const int32_t* q_start,
                         int32_t num_queries, const void* q, void* out, void* stream);

/* Static description of a status code. */
const char* gsa_status_string(gsa_status_t s);

/* Library version, major*10000 + minor*100 + patch. */
int gsa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GSA_H_ */
