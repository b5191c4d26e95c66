/*
 * tri.h -- C ABI of the TriAttention online KV-eviction pass for MI355X
 * (gfx950): score every cached key of every layer and KV head, keep the
 * top-B keys per head, compact K, V and positions in place.
 *
 * The method (cited by page title and section):
 *   - "TriAttention" paper review, romaanj.github.io, section "Method":
 *     offline calibration gives per-band pre-RoPE query centres E[q_f], mean
 *     norms and mean resultant lengths R_f; online, each cached key gets a
 *     trigonometric distance-preference term plus a norm term weighted by
 *     (1 - R_f), averaged over geometric future offsets; every 128 decoded
 *     tokens the cache is pruned back to the budget; figure 4 caption: the
 *     pruning step retains the highest-scoring keys.
 *   - "TriAttention ... Review", dimensionstp.github.io, section 2-2 (the
 *     RoPE logit as a per-band cosine series in query-key distance) and
 *     section 3-2 items 2)-5) (the cached key's position and pre-RoPE form
 *     give its score; score = S_tri + S_norm; window-based pruning keeps the
 *     top-budget keys); section 4-3 item 5 and section 6 item 1 name scoring,
 *     pruning and cache compaction as the kernel work.
 *
 * Conventions shared by every call:
 *   - Band f of a head_dim-d vector x is x[f] + i*x[f + d/2] (the rotate-half
 *     RoPE layout); RoPE at position p turns band f by w_f * p.
 *   - A cache of one sequence is K and V, each [n_layers][n_kv_heads][cap]
 *     [head_dim] rows, plus int32 positions [n_layers][n_kv_heads][cap].  Rows
 *     [0, len) of every head are in use; their positions are strictly
 *     ascending in slot order (the kernels break score ties by the lower slot,
 *     which is the lower position under this invariant).
 *   - All device pointers are owned by the caller.  The library owns only
 *     the calibration tables inside a tri_ctx.
 *   - The per-step calls (tri_score, tri_score_ws, tri_select_topb,
 *     tri_select_topb_ws, tri_compact_kv, tri_select_shared,
 *     tri_compact_kv_counts, tri_compact_kv_counts_noalloc) and
 *     tri_calibrate_stats / tri_distance_curve enqueue work on the given
 *     stream (a hipStream_t; NULL is the null stream) and never synchronise.
 *     Argument errors are reported synchronously before anything is
 *     enqueued.  The device current on the calling thread must be the
 *     context's device.  None of them allocates: scratch memory, where a
 *     call needs it, is a caller-owned workspace of the size its
 *     *_workspace_bytes call gives (tri_compact_kv_counts_noalloc uses the
 *     library's static device scratch instead).  They launch kernels only,
 *     so a caller may capture them in a HIP graph.
 *   - A head fires iff len > budget + window; the calls with a budget skip
 *     sequences that do not fire.  With head-specific budgets
 *     (tri_select_shared) a whole layer fires or not; see there.
 */
#ifndef TRI_H
#define TRI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TRI_OK = 0,
    TRI_E_INVAL = 1,        /* NULL pointer, size out of range, misaligned pointer, wrong device */
    TRI_E_UNSUPPORTED = 2,  /* head_dim / dtype combination not built (head_dim 64 or 128; f32 or bf16) */
    TRI_E_HIP = 3,          /* a HIP runtime call or launch failed; see tri_last_hip_error() */
    TRI_E_NOMEM = 4,        /* device or host allocation for the context failed */
    TRI_E_SCRATCH = 5       /* an allocation-free call needs more than the library's static scratch */
} tri_status;

typedef enum { TRI_F32 = 0, TRI_BF16 = 1 } tri_dtype;

/* Calibration statistics per (layer, KV head, band), read from host memory
 * during tri_calibrate_load and copied; the caller keeps ownership.
 * Source: romaanj.github.io review, section "Method" (per-band query centre,
 * mean norm and mean resultant length from an offline calibration pass;
 * geometric future offsets). */
typedef struct {
    int32_t n_layers;             /* >= 1 */
    int32_t n_kv_heads;           /* >= 1 */
    int32_t head_dim;             /* 64 or 128 */
    double rope_theta;            /* > 0; band frequency theta^(-2f/head_dim) when inv_freq is NULL */
    const double* inv_freq;       /* host [head_dim/2] explicit band frequencies (> 0, finite), or NULL */
    const int64_t* offsets;       /* host [n_offsets] future offsets D, each in [0, 2^40] */
    int32_t n_offsets;            /* >= 1 */
    const double* qc_re;          /* host [n_layers][n_q_heads][head_dim/2]: Re E[q_f] (pre-RoPE) */
    const double* qc_im;          /* host, same shape: Im E[q_f] */
    const double* q_mean_norm;    /* host, same shape: E|q_f| >= 0 */
    const double* q_mrl;          /* host, same shape: mean resultant length R_f in [0, 1] */
    int32_t n_q_heads;            /* query heads per layer: 0 or n_kv_heads for one query table per
                                     KV head; otherwise G * n_kv_heads with G in [2, 8] (GQA: query
                                     heads j*G .. j*G+G-1 share KV head j) */
} tri_calib_desc;

typedef struct tri_ctx tri_ctx;   /* opaque; immutable after tri_calibrate_load */

/* One sequence's cache.  Device pointers, caller-owned. */
typedef struct {
    void* k;          /* [n_layers][n_kv_heads][cap][head_dim], 16-byte aligned */
    void* v;          /* same shape and dtype as k, 16-byte aligned (read by the compaction calls only) */
    int32_t* pos;     /* [n_layers][n_kv_heads][cap] (read and written by the compaction calls only) */
    int32_t cap;      /* rows allocated per head, >= len */
    int32_t len;      /* rows in use per head (with head_len: an upper bound on every head's rows,
                         and the per-head stride of the score layout); tri_compact_kv sets it to
                         budget when it fires.  len * head_dim * 4 < 2^31 (at most 4,194,303
                         keys per head at head_dim 128), else TRI_E_INVAL */
    int64_t p_now;    /* position of the newest cached token; future queries sit at p_now + delta */
    int32_t* head_len;/* NULL: every head holds len rows.  Otherwise device int32
                         [n_layers][n_kv_heads], 4-byte aligned: head (l, h) holds rows
                         [0, min(head_len[l][h], len)) (a ragged cache, as head-specific budgets
                         leave it).  Read by tri_score / tri_score_ws / tri_select_shared, written
                         by tri_compact_kv_counts; tri_select_topb and tri_compact_kv need NULL. */
} tri_seq;

/*
 * Loads a calibration table: validates it on the host, copies it to
 * `device`, and derives there in fp64, once, the band frequencies w_f, the
 * offset-averaged phasors A_f = mean over D of exp(i*w_f*delta), the
 * products E[q_f]*A_f and the norm weights (1 - R_f) * E|q_f|.
 * Synchronous.  On success *out holds a new context; on failure *out is NULL.
 * Errors: TRI_E_INVAL (NULL pointer, non-finite or out-of-range value),
 * TRI_E_UNSUPPORTED (head_dim), TRI_E_NOMEM, TRI_E_HIP.
 * Source: romaanj.github.io review, section "Method"; reading: the norm
 * weight is (1 - R_f) * E|q_f| and the offset average is the plain mean.
 */
tri_status tri_calibrate_load(const tri_calib_desc* desc, int device, tri_ctx** out);

/*
 * Calibration statistics of query heads from pre-RoPE query samples, on the
 * device: for every head h and band f, over the n_samples samples,
 *   E[q_f]  = mean of  q[f] + i*q[f + d/2]
 *   E|q_f|  = mean of |q[f] + i*q[f + d/2]|
 *   R_f     = |E[q_f]| / E|q_f|   (0 when E|q_f| = 0),
 * accumulated in fp64 in a fixed order (two runs give identical bits).  The
 * outputs are the tables tri_calib_desc takes; copy them to the host to load
 * a context.  One workgroup per head reads that head's samples once.
 *   q       device [n_samples][n_heads][head_dim] (dtype), 16-byte aligned;
 *           n_heads counts the query heads of every layer (n_layers * n_q_heads)
 *   qc_re, qc_im, q_mean_norm, q_mrl  device fp64 [n_heads][head_dim/2] outputs,
 *           8-byte aligned, caller-owned
 * Enqueued on `stream` (NULL: the null stream), no synchronisation; uses the
 * device current on the calling thread.
 * Errors: TRI_E_INVAL (NULL or misaligned pointer, n_samples < 1, n_heads < 1),
 * TRI_E_UNSUPPORTED (head_dim or dtype), TRI_E_HIP.
 * Source: romaanj.github.io review, section "Method" (per band: pre-RoPE query
 * centre, mean norm, mean resultant length, from an offline calibration
 * pass); dimensionstp.github.io review, section 3 (the calibration phase;
 * concentration measured as MRL).  Reading: R_f = |E[q_f]| / E|q_f|, the
 * resultant length of the mean band vector relative to the mean length.
 */
tri_status tri_calibrate_stats(tri_dtype dtype, const void* q, int64_t n_samples, int32_t n_heads,
                               int32_t head_dim, double* qc_re, double* qc_im,
                               double* q_mean_norm, double* q_mrl, void* stream);

/*
 * Distance-preference curves: for every query head of the context (all
 * layers; the G query heads of a KV head in GQA contexts) and every distance
 * delta_j,
 *   curve[qh][j] = sum_f Re( E[q_f] * conj(kc_f) * exp(i*w_f*delta_j) ),
 * the RoPE logit of a query at the query head's calibrated centre E[q_f] and
 * a key at its KV head's pre-RoPE key centre kc_f, delta_j positions earlier
 * (delta may be negative).  Computed in fp64; each entry sums its bands in
 * order, and the phasors exp(i*w_f*delta_j) are evaluated once per tile of
 * 64 query heads.
 *   kc_re, kc_im  device fp64 [n_layers*n_kv_heads][head_dim/2] key centres
 *                 (e.g. tri_calibrate_stats of pre-RoPE key samples)
 *   deltas        device int64 [n_delta], |delta| <= 2^40
 *   curve         device fp64 [n_layers*n_q_heads][n_delta] output
 * Enqueued on `stream`, no synchronisation.  Errors: TRI_E_INVAL, TRI_E_HIP.
 * Source: dimensionstp.github.io review, section 2-1 item 2 (Q/K centres
 * give a distance preference curve), section 2-2 (the RoPE logit as a
 * per-band cosine series of the distance), section 6 item 2 (per-head
 * curves show local, sink-like or retrieval-like heads).
 */
tri_status tri_distance_curve(const tri_ctx* ctx, const double* kc_re, const double* kc_im,
                              const int64_t* deltas, int32_t n_delta, double* curve, void* stream);

/*
 * Future-offset sets for tri_calib_desc.offsets (host only, no GPU):
 *   kind 0, geometric: 1, 2, 4, ... up to max_distance (the pages' default is
 *           {1, 2, ..., 2^16}: max_distance 65536);
 *   kind 1, linear: round(max_distance * k / count) for k = 1..count (halves
 *           round up), at least 1.
 * Writes min(cap, size) offsets to out (host) and returns the set's size,
 * or -1 on bad arguments (max_distance outside [1, 2^40], count outside
 * [1, 2^20] for kind 1, unknown kind, out NULL with cap > 0).
 * Source: romaanj.github.io review, section "Method" (geometric offsets);
 * dimensionstp.github.io review, section 4-3 "Future offset design" (the
 * maximum distance and the spacing change the result; geometric spacing is
 * reported better than linear).
 */
int32_t tri_offset_set(int32_t kind, int64_t max_distance, int32_t count, int64_t* out,
                       int32_t cap);

/* Frees a context (NULL is allowed).  Work enqueued with it must be complete. */
void tri_ctx_destroy(tri_ctx* ctx);

/* Static text for a status code. */
const char* tri_status_str(tri_status s);

/* hipError_t of the last TRI_E_HIP returned on the calling thread (0 if none). */
int tri_last_hip_error(void);

/* Number of fp32 score slots tri_score writes: sum over seqs of
 * n_layers * n_kv_heads * len.  Returns -1 on bad arguments. */
int64_t tri_scores_count(const tri_ctx* ctx, const tri_seq* seqs, int32_t n_seq);

/*
 * Scores every cached key: for the key in slot i of a head, with stored
 * (post-RoPE) bands K_f,
 *   score = mean over delta of sum_f Re(E[q_f] * conj(k_f) * exp(i*w_f*(p_now + delta - p_i)))
 *         + sum_f (1 - R_f) * E|q_f| * |k_f|,
 * where k_f = K_f * exp(-i*w_f*p_i) is the key un-rotated to pre-RoPE form.
 * The un-rotation and the distance share p_i and cancel, so the kernel folds
 * C_f = E[q_f] * A_f * exp(i*w_f*p_now) once per head in fp64 and takes
 * score = sum_f (Re C_f * K[f] + Im C_f * K[f + d/2]) + sum_f w_f * |K_f|
 * from the stored row, accumulating in fp32.  A key whose stored row holds
 * an infinite or NaN element scores NaN (so every selection ranks it last);
 * so does a finite row whose fp32 evaluation overflows (elements of magnitude
 * above ~1e18).
 * GQA contexts (n_q_heads > n_kv_heads) need tri_score_ws; tri_score
 * returns TRI_E_INVAL for them.
 *   dtype   element type of every seq's K (TRI_F32 or TRI_BF16)
 *   scores  device fp32, tri_scores_count() slots: the scores of sequence s
 *           start after those of sequences 0..s-1, each sequence laid out
 *           [n_layers][n_kv_heads][len]
 * Reads K rows [0, len) of every head (with head_len, the head's own rows;
 * score slots past a head's length are left untouched); positions are not
 * read.
 * Errors: TRI_E_INVAL, TRI_E_UNSUPPORTED, TRI_E_HIP.
 * Source: romaanj.github.io review, section "Method" (trig term per band
 * ||E[q_f]||*||k_f||*cos(w_f*distance + phase difference), norm term,
 * offsets averaged); dimensionstp.github.io review, sections 2-2 and 3-2
 * items 2)-4).
 */
tri_status tri_score(const tri_ctx* ctx, tri_dtype dtype, const tri_seq* seqs, int32_t n_seq,
                     float* scores, void* stream);

/* Device workspace bytes tri_score_ws needs for these sequences: 0 for a
 * context with one query table per KV head; for GQA contexts 4 * G bytes per
 * cached key plus per-tile statistics and 8 KB per (layer, KV head) of
 * prepared constants.  Returns -1 on bad arguments. */
int64_t tri_score_workspace_bytes(const tri_ctx* ctx, const tri_seq* seqs, int32_t n_seq);

/*
 * tri_score with a caller-owned device workspace (16-byte aligned, at least
 * tri_score_workspace_bytes(); may be NULL when that is 0).  Contexts with
 * one query table per KV head score exactly as tri_score.  For GQA contexts
 * (G query heads per KV head) every key first gets G scores, one per query
 * head of its KV head, each the score above with that query head's table;
 * each query head's scores are z-normalized over the head's cached keys,
 *   z_g = (s_g - mean_g) / sd_g   (mean and population deviation of the finite s_g),
 * and the key's score is the largest z_g.  K is read once.  With GQA
 * contexts `scores` may be NULL: then only the raw scores and their per-tile
 * partial sums are computed, into the workspace, for tri_select_topb_ws.
 * Readings: a
 * deviation at most 1e-9 of the largest |s_g| counts as zero and gives
 * z_g = 0; a non-finite s_g gives NaN, which loses to every number; mean_g
 * and sd_g are accumulated in fp64 in a fixed order (the result does not
 * depend on scheduling).  Output layout as tri_score; the workspace holds
 * intermediates only and is overwritten.  Calls sharing a workspace must not
 * overlap in time.
 * Errors: TRI_E_INVAL (also: GQA context with a missing or short workspace),
 * TRI_E_UNSUPPORTED, TRI_E_HIP.
 * Source: dimensionstp.github.io review, section 3-2 item 6 (per query head
 * z-score normalization, then max aggregation over the query heads sharing
 * a KV head); romaanj.github.io review, section "Method".
 */
tri_status tri_score_ws(const tri_ctx* ctx, tri_dtype dtype, const tri_seq* seqs, int32_t n_seq,
                        float* scores, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Selects, for every head of every firing sequence, the `budget` keys with
 * the largest scores; equal scores go to the lower slot; NaN ranks below
 * every number and -0 equals +0.  Needs head_len == NULL.  Writes the kept slots in ascending order
 * to kept[s][layer][kv_head][0..budget) (device int32, n_seq * n_layers *
 * n_kv_heads * budget slots; entries of sequences that do not fire are left
 * untouched).
 *   scores   device fp32 in the layout tri_score writes
 *   budget   >= 1;  window >= 0;  a sequence fires iff len > budget + window
 * Errors: TRI_E_INVAL, TRI_E_HIP.
 * Source: romaanj.github.io review, section "Method" and figure 4 caption;
 * dimensionstp.github.io review, section 3-2 item 5 (top-budget keys kept).
 * Reading: ties by lower position.
 */
tri_status tri_select_topb(const tri_ctx* ctx, const tri_seq* seqs, int32_t n_seq,
                           const float* scores, int32_t budget, int32_t window,
                           int32_t* kept, void* stream);

/*
 * tri_select_topb for GQA contexts without the normalized score array: the
 * keys are ranked by the GQA score of tri_score_ws (the largest z-normalized
 * per-query-head score), formed on the fly from the raw per-query-head
 * scores and per-tile partial sums that a tri_score_ws call on the same
 * sequences, with scores == NULL, left in `workspace` (the statistics are
 * summed from them in the same fixed order).  The kept lists are those
 * tri_select_topb gives on the scores tri_score_ws would have written (the
 * same fp64 operations, rounded once to fp32).  Saves writing and reading
 * back the normalized scores, and the statistics launch.
 *   scores     NULL, unless a firing sequence holds more than 32768 keys per
 *              head: then device fp32 in the layout of tri_score, where the
 *              normalized scores of those sequences are written first
 *   workspace  the workspace of that tri_score_ws call, unchanged since
 *              (16-byte aligned, at least tri_score_workspace_bytes())
 *   budget, window, kept, the fire rule: as tri_select_topb (head_len NULL)
 * Errors: TRI_E_INVAL (also: a context with one query table per KV head, a
 * missing or short workspace), TRI_E_HIP.
 * Source: dimensionstp.github.io review, section 3-2 items 5 and 6 (top-budget
 * keys; per query head z-score, then the max over the query heads of a KV
 * head); romaanj.github.io review, section "Method".
 */
tri_status tri_select_topb_ws(const tri_ctx* ctx, const tri_seq* seqs, int32_t n_seq,
                              float* scores, const void* workspace, int64_t workspace_bytes,
                              int32_t budget, int32_t window, int32_t* kept, void* stream);

/*
 * Evicts in place (head_len must be NULL): for every head of every firing
 * sequence, rows r < budget
 * of K, V and positions become the rows at kept[r] (stable: the kept rows
 * keep their slot order).  Then sets seqs[s].len = budget for every firing
 * sequence (at enqueue time).  Rows [budget, cap) hold unspecified data
 * afterwards.  Not failure-atomic: if a launch fails, the cache contents are
 * undefined.
 *   kept  device int32 in the layout tri_select_topb writes; every list must
 *         be strictly ascending with entries in [0, len)
 * Errors: TRI_E_INVAL, TRI_E_UNSUPPORTED, TRI_E_HIP.
 * Source: dimensionstp.github.io review, section 3-2 item 5 (evict the rest)
 * and section 6 item 1 (cache compaction).
 */
tri_status tri_compact_kv(const tri_ctx* ctx, tri_dtype dtype, tri_seq* seqs, int32_t n_seq,
                          const int32_t* kept, int32_t budget, int32_t window, void* stream);

/* Device workspace bytes tri_select_shared needs: per sequence, 16 bytes
 * and two histogram rows of 16,640 bytes per (layer, KV head) plus 192 bytes
 * per layer, rounded up (9.6 MB for 36 layers x 8 KV heads).  -1 on bad
 * arguments. */
int64_t tri_select_shared_workspace_bytes(const tri_ctx* ctx, int32_t n_seq);

/*
 * Head-specific budgets: the KV heads of a layer share one budget of
 * total = budget * n_kv_heads slots instead of holding `budget` each.
 * Reading: every head first reserves its `floor` best keys (its own order:
 * higher score, then lower slot; a head with at most `floor` keys reserves
 * all); the remaining slots go to the best remaining keys of the whole layer
 * under one threshold, equal scores to the lower head and then the lower
 * slot.  NaN ranks below every number; -0 equals +0.
 * A layer fires iff the sum of its heads' lengths exceeds
 * total + n_kv_heads * window.  For layer l of sequence s:
 *   kept_count[s][l][h]  number of keys head h keeps, or -1 if the layer
 *                        does not fire (then its kept rows hold unspecified
 *                        data: they serve as scratch)
 *   kept[s][l][h][0..kept_count)  the kept slots, ascending (stride total)
 * so the sum of the counts of a firing layer is exactly total.
 *   scores     device fp32, layout of tri_score: [n_layers][n_kv_heads][len]
 *              per sequence; entries at or past a head's length are not read
 *   budget     >= 1 (slots per head on average);  window >= 0
 *   floor      in [0, budget] (keys every head keeps for itself)
 *   kept       device int32, n_seq * n_layers * n_kv_heads * total slots
 *   kept_count device int32, n_seq * n_layers * n_kv_heads slots (always written)
 *   workspace  device, 16-byte aligned, >= tri_select_shared_workspace_bytes
 * The firing decision is taken on the device (head lengths may live only
 * there).  n_kv_heads <= 128.  Calls sharing a workspace must not overlap.
 * Errors: TRI_E_INVAL, TRI_E_UNSUPPORTED (n_kv_heads > 128), TRI_E_HIP.
 * Source: romaanj.github.io review, section "Future work" (refined
 * compression with head-specific budgets); section "Method" and figure 4
 * caption (the highest-scoring keys are retained).
 */
tri_status tri_select_shared(const tri_ctx* ctx, const tri_seq* seqs, int32_t n_seq,
                             const float* scores, int32_t budget, int32_t floor, int32_t window,
                             int32_t* kept, int32_t* kept_count, void* workspace,
                             int64_t workspace_bytes, void* stream);

/*
 * Evicts in place with a kept count per head: for every head whose
 * kept_count c >= 0, rows r < c of K, V and positions become the rows at
 * kept[r] (stable), and head_len of that head becomes c; heads with
 * c == -1 are left as they are.  seqs[s].len is not changed (it stays an
 * upper bound on every head's rows; a caller that knows a smaller bound may
 * lower it).  Rows [c, cap) hold unspecified data afterwards.  Not
 * failure-atomic.
 *   kept        device int32 [n_seq][n_layers][n_kv_heads][kept_stride],
 *               every list strictly ascending within the head's rows
 *   kept_count  device int32 [n_seq][n_layers][n_kv_heads], -1 or in
 *               [0, kept_stride]
 *   every sequence needs head_len != NULL
 *   workspace   device, 4-byte aligned, >= tri_compact_kv_counts_workspace_bytes;
 *               calls sharing a workspace must not overlap
 * Errors: TRI_E_INVAL, TRI_E_UNSUPPORTED, TRI_E_HIP.
 * Source: dimensionstp.github.io review, section 3-2 item 5 (evict the rest)
 * and section 6 item 1 (cache compaction); romaanj.github.io review,
 * section "Future work" (head-specific budgets).
 */
tri_status tri_compact_kv_counts(const tri_ctx* ctx, tri_dtype dtype, tri_seq* seqs,
                                 int32_t n_seq, const int32_t* kept, int32_t kept_stride,
                                 const int32_t* kept_count, void* workspace,
                                 int64_t workspace_bytes, void* stream);

/*
 * tri_compact_kv_counts without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the queue of column parts lives in a
 * static device array of the library, one copy per GPU, held from the first
 * context loaded on that GPU until the process ends.  Arguments, effects and
 * results are those of tri_compact_kv_counts.  The array holds the queue of
 * at most 65,536 (layer, KV head) streams per context (n_layers *
 * n_kv_heads <= 65536, 2 MiB); larger contexts get TRI_E_SCRATCH before
 * anything is enqueued.  Every call on one GPU shares that GPU's array (each
 * call's first kernel re-initialises it), so calls that overlap in time on
 * one GPU, from any stream or thread, race and must not be issued.  Makes no
 * HIP allocation of any kind.
 * Errors: TRI_E_INVAL, TRI_E_UNSUPPORTED, TRI_E_SCRATCH, TRI_E_HIP.
 */
tri_status tri_compact_kv_counts_noalloc(const tri_ctx* ctx, tri_dtype dtype, tri_seq* seqs,
                                         int32_t n_seq, const int32_t* kept, int32_t kept_stride,
                                         const int32_t* kept_count, void* stream);

/* Device workspace bytes tri_compact_kv_counts needs (it orders the column
 * parts of the heads' K and V rows there, longest first):
 * 8 + 32 * n_layers * n_kv_heads, whatever the number of sequences.  -1 on
 * bad arguments. */
int64_t tri_compact_kv_counts_workspace_bytes(const tri_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* TRI_H */
