/*
 * tri_oracle.c -- plain, slow fp64 CPU oracle of the TriAttention online
 * KV-eviction pass: score every cached key, keep the top-B keys per KV head,
 * gather the kept rows.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may use it.  It shares no code, header, table or constant
 * with the HIP path.
 *
 * Sources (cited by page title and section; no code exists on the pages):
 *   [R1] "TriAttention" paper review, romaanj.github.io, section "Method":
 *        the per-band trigonometric term ||E[q_f]||*||k_f||*cos(w_f*D + phi_f),
 *        the norm term weighted by (1 - R_f), averaging over geometrically
 *        spaced future offsets {1,2,4,...,2^16}, pruning to the budget every
 *        128 decoded tokens; figure 4 caption (the prune retains the
 *        highest-scoring keys).
 *   [R2] "TriAttention ... Review", dimensionstp.github.io, section 2-2
 *        (RoPE logit as a sum over bands of r_q*r_k*cos((i-j)*theta_f+phi_f)),
 *        section 3-2 items 2)-5) (cached key has a known position and
 *        pre-RoPE form; score = S_tri + S_norm; window-based pruning keeps
 *        the top-budget keys), section 3-2 item 6 (GQA: per query head
 *        z-score normalization, then max aggregation over the query heads
 *        that share a KV head).
 *
 * Readings taken where the pages leave a step open (each is listed in the
 * design notes of the repository):
 *   - band f of a head_dim-d vector x is the complex number
 *     x[f] + i*x[f + d/2] (half-split pairing), and RoPE at position p
 *     multiplies band f by exp(i*w_f*p);
 *   - w_f = theta^(-2f/d) unless the caller gives explicit frequencies;
 *   - the norm-term weight of band f is (1 - R_f) * E|q_f|;
 *   - the average over offsets is the plain arithmetic mean;
 *   - the trig and norm terms are added unscaled;
 *   - a key whose stored row holds an infinite or NaN element scores NaN;
 *   - GQA: query heads [h*G, (h+1)*G) share KV head h; each query head's
 *     score row is z-normalized with the mean and population standard
 *     deviation of its finite scores over the head's cached keys; a
 *     deviation of at most 1e-9 of the row's largest |score| (rounding
 *     level) counts as zero and gives z = 0; a non-finite score stays NaN
 *     and loses to any number in the max over the group;
 *   - a head fires iff n > budget + window; top-B orders keys by
 *     (score descending, position ascending), NaN below every number,
 *     -0 equal to +0; kept slots are returned in ascending slot order.
 *
 * Everything is computed literally in the order the pages state it:
 * un-rotate the stored key, then average the per-band trigonometric term
 * over every future offset, then add the norm term.
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* RoPE band frequency w_f = theta^(-2f/d) (standard RoPE; reading). */
double tri_oracle_omega(int f, int d, double theta)
{
    return pow(theta, -2.0 * (double)f / (double)d);
}

/* Pre-RoPE band f of one stored (post-RoPE) key row K at position p:
 * k_f = (K[f] + i*K[f+d/2]) * exp(-i*w_f*p).  [R2 3-2 item 2: the cached key
 * has a known position and a pre-RoPE representation.] */
static double complex unrotate_band(const double* K, int d, int f,
                                    int64_t p, const double* omega)
{
    double complex stored = K[f] + I * K[f + d / 2];
    return stored * cexp(-I * omega[f] * (double)p);
}

/* Writes the d/2 pre-RoPE bands of one stored key row. */
void tri_oracle_unrotate(int d, const double* K, int64_t p,
                         const double* omega, double* k_re, double* k_im)
{
    for (int f = 0; f < d / 2; ++f) {
        double complex k = unrotate_band(K, d, f, p, omega);
        k_re[f] = creal(k);
        k_im[f] = cimag(k);
    }
}

/*
 * Scores the n keys of one (layer, KV head).
 *   K       [n][d] stored post-RoPE key rows, upcast to fp64
 *   pos     [n]    position of each key
 *   p_now          position of the newest cached token; future queries
 *                  sit at p_now + delta for each delta in offsets
 *   omega   [d/2]  band frequencies
 *   offsets [n_off]
 *   qc_re, qc_im [d/2]  calibrated pre-RoPE query centre E[q_f]
 *   q_mean_norm  [d/2]  E|q_f|
 *   q_mrl        [d/2]  mean resultant length R_f
 * Outputs trig[n], norm[n], score[n] (any may be NULL).
 *
 * trig_i = mean over delta of  sum_f Re( qc_f * conj(k_f) *
 *                                         exp(i*w_f*(p_now + delta - p_i)) )
 *   which is, band by band, |qc_f|*|k_f|*cos(w_f*dist + phase difference)
 *   [R1 Method; R2 2-2, 3-2 item 2];
 * norm_i = sum_f (1 - R_f) * E|q_f| * |k_f|      [R1 Method; R2 3-2 items 3-4];
 * score_i = trig_i + norm_i                       [R2 3-2 item 4].
 */
void tri_oracle_score_head(int d, int n, const double* K, const int64_t* pos,
                           int64_t p_now, const double* omega,
                           const int64_t* offsets, int n_off,
                           const double* qc_re, const double* qc_im,
                           const double* q_mean_norm, const double* q_mrl,
                           double* trig, double* norm, double* score)
{
    const int half = d / 2;
    double complex* k = (double complex*)malloc(sizeof(double complex) * (size_t)half);
    for (int i = 0; i < n; ++i) {
        const double* row = K + (size_t)i * (size_t)d;

        /* A stored row with an infinite or NaN element has no score: it gets
           NaN, which the selection ranks below every number (reading; the
           pages define the score for finite keys only). */
        int finite_row = 1;
        for (int j = 0; j < d; ++j)
            if (!isfinite(row[j])) finite_row = 0;
        if (!finite_row) {
            if (trig) trig[i] = NAN;
            if (norm) norm[i] = NAN;
            if (score) score[i] = NAN;
            continue;
        }

        for (int f = 0; f < half; ++f)
            k[f] = unrotate_band(row, d, f, pos[i], omega);

        /* trigonometric distance-preference series, averaged over offsets */
        double trig_sum = 0.0;
        for (int o = 0; o < n_off; ++o) {
            int64_t dist = p_now + offsets[o] - pos[i];
            double at_offset = 0.0;
            for (int f = 0; f < half; ++f) {
                double complex q = qc_re[f] + I * qc_im[f];
                at_offset += creal(q * conj(k[f]) * cexp(I * omega[f] * (double)dist));
            }
            trig_sum += at_offset;
        }
        double t = trig_sum / (double)n_off;

        /* concentration-weighted norm term */
        double nm = 0.0;
        for (int f = 0; f < half; ++f)
            nm += (1.0 - q_mrl[f]) * q_mean_norm[f] * cabs(k[f]);

        if (trig) trig[i] = t;
        if (norm) norm[i] = nm;
        if (score) score[i] = t + nm;
    }
    free(k);
}

/*
 * Per-key magnitude bound M_i = sum_f (|qc_f| * |A_f| + w_f) * |k_f| with
 * A_f = mean over delta of exp(i*w_f*delta) and w_f = (1 - R_f) * E|q_f|.
 * |score_i| <= M_i, and M_i is the scale of the rounding error of any
 * evaluation of the score, so parity tolerances are stated relative to it.
 * This is a tolerance scale, not part of the score.
 */
void tri_oracle_bound_head(int d, int n, const double* K, const double* omega,
                           const int64_t* offsets, int n_off,
                           const double* qc_re, const double* qc_im,
                           const double* q_mean_norm, const double* q_mrl,
                           double* bound)
{
    const int half = d / 2;
    double* coef = (double*)malloc(sizeof(double) * (size_t)half);
    for (int f = 0; f < half; ++f) {
        double complex a = 0.0;
        for (int o = 0; o < n_off; ++o)
            a += cexp(I * omega[f] * (double)offsets[o]);
        a /= (double)n_off;
        coef[f] = cabs(qc_re[f] + I * qc_im[f]) * cabs(a)
                + (1.0 - q_mrl[f]) * q_mean_norm[f];
    }
    for (int i = 0; i < n; ++i) {
        const double* row = K + (size_t)i * (size_t)d;
        double m = 0.0;
        for (int f = 0; f < half; ++f)
            m += coef[f] * hypot(row[f], row[f + half]);   /* |k_f| = |K_f| */
        bound[i] = m;
    }
    free(coef);
}

/* ---- distance-preference curve and offset sets -------------------------- */

/*
 * Distance-preference curve of one head [R2 section 2-1 item 2 (Q/K centres
 * give a distance preference curve), section 2-2 (the RoPE logit as a
 * per-band cosine series of the query-key distance), section 6 item 2 (the
 * per-head curve as an analysis tool)]: with the pre-RoPE query centre
 * qc_f and key centre kc_f of every band,
 *   curve[j] = sum_f Re( qc_f * conj(kc_f) * exp(i*w_f*deltas[j]) ),
 * the logit of a query at the centre and a key at the centre deltas[j]
 * positions before it.  Returns 0, or -1 on bad arguments.
 */
int tri_oracle_distance_curve(int d, const double* omega, const double* qc_re,
                              const double* qc_im, const double* kc_re, const double* kc_im,
                              const int64_t* deltas, int n_delta, double* curve)
{
    if (d < 2 || n_delta < 0) return -1;
    const int half = d / 2;
    for (int j = 0; j < n_delta; ++j) {
        double s = 0.0;
        for (int f = 0; f < half; ++f) {
            const double complex q = qc_re[f] + I * qc_im[f];
            const double complex k = kc_re[f] + I * kc_im[f];
            s += creal(q * conj(k) * cexp(I * omega[f] * (double)deltas[j]));
        }
        curve[j] = s;
    }
    return 0;
}

/*
 * Future-offset sets [R1 Method (geometric offsets {1, 2, 4, ..., 2^16});
 * R2 section 4-3 "Future offset design" (the maximum distance and the
 * spacing change the result, geometric spacing beats linear)].
 *   kind 0, geometric: 1, 2, 4, ... up to max_distance (powers of two)
 *   kind 1, linear:    max_distance * k / count for k = 1..count (rounded
 *                      to the nearest integer, at least 1)
 * Writes at most `cap` offsets and returns how many the set has, or -1 on
 * bad arguments.
 */
int tri_oracle_offset_set(int kind, int64_t max_distance, int count, int64_t* out, int cap)
{
    if (max_distance < 1) return -1;
    int n = 0;
    if (kind == 0) {
        for (int64_t x = 1; x <= max_distance; x *= 2) {
            if (n < cap) out[n] = x;
            ++n;
        }
        return n;
    }
    if (kind == 1) {
        if (count < 1) return -1;
        for (int k = 1; k <= count; ++k) {
            int64_t x = (int64_t)floor((double)max_distance * (double)k / (double)count + 0.5);
            if (x < 1) x = 1;
            if (n < cap) out[n] = x;
            ++n;
        }
        return n;
    }
    return -1;
}

/* ---- calibration statistics from query samples --------------------------- */

/*
 * Per-band calibration statistics of one query head from n pre-RoPE query
 * samples Q [n][d] [R1 Method: the offline pass estimates, per frequency
 * band, the pre-RoPE query centre E[q_f], the mean norm and the mean
 * resultant length R_f; R2 section 3 (the calibration phase computes head-
 * and band-wise centre, expected norm and concentration, measured as MRL)]:
 *   qc_f  = mean over samples of q_f = Q[t][f] + i*Q[t][f+d/2]
 *   m_f   = mean over samples of |q_f|
 *   R_f   = |qc_f| / m_f   (0 when m_f = 0)
 * Reading: R_f is the resultant length of the mean band vector relative to
 * the mean length (the mean resultant length of the band's phases, weighted
 * by magnitude); with samples of equal magnitude it is the plain mean
 * resultant length of the phases.  Returns 0, or -1 on bad arguments.
 */
int tri_oracle_calib_stats(int d, long n, const double* Q, double* qc_re, double* qc_im,
                           double* mean_norm, double* mrl)
{
    if (d < 2 || n < 1) return -1;
    const int half = d / 2;
    for (int f = 0; f < half; ++f) {
        double complex sum = 0.0;
        double norm_sum = 0.0;
        for (long t = 0; t < n; ++t) {
            const double complex q = Q[(size_t)t * d + f] + I * Q[(size_t)t * d + f + half];
            sum += q;
            norm_sum += cabs(q);
        }
        const double complex centre = sum / (double)n;
        const double m = norm_sum / (double)n;
        qc_re[f] = creal(centre);
        qc_im[f] = cimag(centre);
        mean_norm[f] = m;
        mrl[f] = m > 0.0 ? cabs(centre) / m : 0.0;
    }
    return 0;
}

/* ---- GQA: normalize, then aggregate ------------------------------------ */

/*
 * Score of the n keys of one KV head shared by `group` query heads
 * [R2 3-2 item 6; R1 Method]: query head g scores every key with its own
 * calibration (exactly tri_oracle_score_head), its row s_g is z-normalized
 * over the head's cached keys, z_g = (s_g - mean_g) / std_g, and a key's
 * score is the largest z_g over the group, so a key that any query head
 * ranks highly survives.
 *   qc_re, qc_im, q_mean_norm, q_mrl  [group][d/2]  query head g's table
 *   raw    [group][n]  out: s_g (may be NULL)
 *   zrow   [group][n]  out: z_g (may be NULL)
 *   score  [n]         out: max over g of z_g
 * mean_g and std_g (population: divided by the count) run over the finite
 * entries of s_g; a row whose std_g is at most GQA_FLAT times its largest
 * |score| counts as constant (mathematically equal scores leave a deviation
 * of a few ulps in fp64 sums) and gets z_g = 0; a non-finite s_g gives
 * z_g = NaN, and NaN loses to every number in the max.  Returns 0, or -1 on
 * bad arguments.
 */
#define GQA_FLAT 1e-9

int tri_oracle_gqa_head(int d, int n, const double* K, const int64_t* pos,
                        int64_t p_now, const double* omega,
                        const int64_t* offsets, int n_off, int group,
                        const double* qc_re, const double* qc_im,
                        const double* q_mean_norm, const double* q_mrl,
                        double* raw, double* zrow, double* score)
{
    if (d < 2 || n < 0 || group < 1 || n_off < 1) return -1;
    const int half = d / 2;
    double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int i = 0; i < n; ++i) score[i] = NAN;
    for (int g = 0; g < group; ++g) {
        tri_oracle_score_head(d, n, K, pos, p_now, omega, offsets, n_off,
                              qc_re + (size_t)g * half, qc_im + (size_t)g * half,
                              q_mean_norm + (size_t)g * half, q_mrl + (size_t)g * half,
                              NULL, NULL, s);
        if (raw) memcpy(raw + (size_t)g * n, s, sizeof(double) * (size_t)n);

        /* mean and population standard deviation of the finite scores */
        double sum = 0.0, big = 0.0;
        long count = 0;
        for (int i = 0; i < n; ++i)
            if (isfinite(s[i])) { sum += s[i]; ++count; if (fabs(s[i]) > big) big = fabs(s[i]); }
        const double mean = count ? sum / (double)count : 0.0;
        double sq = 0.0;
        for (int i = 0; i < n; ++i)
            if (isfinite(s[i])) { const double e = s[i] - mean; sq += e * e; }
        const double sd = count ? sqrt(sq / (double)count) : 0.0;
        /* a row that varies by no more than rounding counts as constant */
        const int flat = sd <= GQA_FLAT * big;

        for (int i = 0; i < n; ++i) {
            double z = NAN;
            if (isfinite(s[i])) z = flat ? 0.0 : (s[i] - mean) / sd;
            if (zrow) zrow[(size_t)g * n + i] = z;
            if (!isnan(z) && (isnan(score[i]) || z > score[i])) score[i] = z;
        }
    }
    free(s);
    return 0;
}

/* ---- top-B selection ---------------------------------------------------- */

typedef struct { double s; int64_t p; int32_t slot; } ranked;

/* Order: score descending, NaN below every number, then position ascending,
 * then slot ascending (positions are distinct in a cache, the slot only makes
 * the order total). -0 and +0 compare equal under C's ordinary comparison. */
static int by_rank(const void* a_, const void* b_)
{
    const ranked* a = (const ranked*)a_;
    const ranked* b = (const ranked*)b_;
    int an = isnan(a->s), bn = isnan(b->s);
    if (an != bn) return an ? 1 : -1;
    if (!an) {
        if (a->s > b->s) return -1;
        if (a->s < b->s) return 1;
    }
    if (a->p != b->p) return a->p < b->p ? -1 : 1;
    return a->slot < b->slot ? -1 : (a->slot > b->slot ? 1 : 0);
}

static int by_int32(const void* a_, const void* b_)
{
    int32_t a = *(const int32_t*)a_, b = *(const int32_t*)b_;
    return (a > b) - (a < b);
}

/*
 * Top-B of one head [R1 Method and figure 4 caption; R2 3-2 item 5].
 * The head fires iff n > budget + window.  When it fires, writes the budget
 * kept slots in ascending slot order to kept[] and returns budget; otherwise
 * returns 0 and writes nothing.  Returns -1 on bad arguments.
 */
int tri_oracle_select_head(int n, const double* score, const int64_t* pos,
                           int budget, int window, int32_t* kept)
{
    if (n < 0 || budget <= 0 || window < 0) return -1;
    if ((int64_t)n <= (int64_t)budget + (int64_t)window) return 0;
    ranked* r = (ranked*)malloc(sizeof(ranked) * (size_t)n);
    for (int i = 0; i < n; ++i) { r[i].s = score[i]; r[i].p = pos[i]; r[i].slot = i; }
    qsort(r, (size_t)n, sizeof(ranked), by_rank);
    for (int j = 0; j < budget; ++j) kept[j] = r[j].slot;
    qsort(kept, (size_t)budget, sizeof(int32_t), by_int32);
    free(r);
    return budget;
}

/* ---- head-specific budgets: one shared budget per layer ------------------ */

typedef struct { double s; int32_t head; int64_t p; int32_t slot; int reserved; } ranked_h;

/* Layer order: reserved keys first, then score descending (NaN below every
 * number), then lower head, lower position, lower slot. */
static int by_layer_rank(const void* a_, const void* b_)
{
    const ranked_h* a = (const ranked_h*)a_;
    const ranked_h* b = (const ranked_h*)b_;
    if (a->reserved != b->reserved) return a->reserved ? -1 : 1;
    int an = isnan(a->s), bn = isnan(b->s);
    if (an != bn) return an ? 1 : -1;   /* NaN below every number */
    if (!an) {
        if (a->s > b->s) return -1;
        if (a->s < b->s) return 1;
    }
    if (a->head != b->head) return a->head < b->head ? -1 : 1;
    if (a->p != b->p) return (a->p < b->p) ? -1 : 1;   /* then the lower position */
    return a->slot < b->slot ? -1 : (a->slot > b->slot ? 1 : 0);
}

/*
 * Head-specific budgets for the n_head KV heads of one layer [R1 "Future
 * work": refined compression strategies including head-specific budgets].
 * Reading: the heads share `total` slots (a per-head budget times the
 * heads); every head first keeps its `floor` best keys (its own order of
 * tri_oracle_select_head), and the remaining slots go to the best remaining
 * keys of the whole layer, one threshold across heads, ties to the lower
 * head and then the lower position.
 *   head h has n[h] keys: score[h*stride + i], pos[h*stride + i], i < n[h]
 *   the layer fires iff sum n[h] > total + n_head * window
 * When it fires, writes head h's kept slots in ascending order to
 * kept[h*total + r], r < count[h], and returns total; otherwise returns 0
 * and writes nothing.  Returns -1 on bad arguments (floor * n_head > total
 * among them).
 */
int tri_oracle_select_shared(int n_head, const int* n, int stride, const double* score,
                             const int64_t* pos, int total, int floor_, int window,
                             int32_t* kept, int32_t* count)
{
    if (n_head < 1 || total < 1 || floor_ < 0 || window < 0) return -1;
    if ((int64_t)floor_ * n_head > total) return -1;
    int64_t all = 0;
    for (int h = 0; h < n_head; ++h) {
        if (n[h] < 0 || n[h] > stride) return -1;
        all += n[h];
    }
    if (all <= (int64_t)total + (int64_t)n_head * window) return 0;

    ranked_h* r = (ranked_h*)malloc(sizeof(ranked_h) * (size_t)all);
    ranked* one = (ranked*)malloc(sizeof(ranked) * (size_t)(stride > 0 ? stride : 1));
    int64_t m = 0;
    for (int h = 0; h < n_head; ++h) {
        /* the head's own order decides which of its keys are reserved */
        for (int i = 0; i < n[h]; ++i) {
            one[i].s = score[(size_t)h * stride + i];
            one[i].p = pos[(size_t)h * stride + i];
            one[i].slot = i;
        }
        qsort(one, (size_t)n[h], sizeof(ranked), by_rank);
        for (int j = 0; j < n[h]; ++j) {
            r[m].s = one[j].s;
            r[m].head = h;
            r[m].p = one[j].p;
            r[m].slot = one[j].slot;
            r[m].reserved = j < floor_;
            ++m;
        }
    }
    qsort(r, (size_t)all, sizeof(ranked_h), by_layer_rank);
    for (int h = 0; h < n_head; ++h) count[h] = 0;
    for (int j = 0; j < total; ++j) {
        const int h = r[j].head;
        kept[(size_t)h * total + count[h]++] = r[j].slot;
    }
    for (int h = 0; h < n_head; ++h)
        qsort(kept + (size_t)h * total, (size_t)count[h], sizeof(int32_t), by_int32);
    free(one);
    free(r);
    return total;
}

/* Gathers rows: dst[r] = src[kept[r]] for r < n_kept (row_bytes each).
 * The eviction keeps exactly the selected rows, in ascending slot order. */
void tri_oracle_gather_rows(int n_kept, const int32_t* kept, int64_t row_bytes,
                            const void* src, void* dst)
{
    const unsigned char* s = (const unsigned char*)src;
    unsigned char* o = (unsigned char*)dst;
    for (int r = 0; r < n_kept; ++r)
        memcpy(o + (size_t)r * (size_t)row_bytes,
               s + (size_t)kept[r] * (size_t)row_bytes, (size_t)row_bytes);
}
