/*
 * A prune step driven from C through the C ABI alone (no Python, no torch),
 * checked against the fp64 oracle's C functions.  Test infrastructure: it
 * links both libtri.so and the oracle, as the Python tests do through their
 * bindings; neither library includes anything of the other.
 *
 * The cache: 1 layer x 3 KV heads x head_dim 64, fp32, 700 keys at
 * positions 0..699, budget 128, window 128, offsets 1, 2, 4, ..., 4096,
 * theta 1e4; rows and calibration tables drawn from a seeded splitmix64 /
 * Box-Muller generator (inputs only; none of the method's arithmetic).
 *
 * Checks (the bars of the GPU parity tests):
 *   - a call with budget 0 returns TRI_E_INVAL before anything is enqueued;
 *   - every GPU score is within 2e-3 * M_i of the oracle's;
 *   - every head keeps exactly B slots, ascending, and they are the top-B of
 *     the GPU's own scores with ties to the lower slot;
 *   - the oracle's clearly kept keys are kept and clearly evicted keys
 *     evicted (band 2e-3 * (M_i + M_t) around the oracle's B-th score t);
 *   - compacted K, V and positions are bit-exact copies of the input rows at
 *     the GPU's kept list, and seq.len becomes B.
 * Exit status 0 when every check holds.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tri.h"

/* the oracle's C functions (oracle/tri_oracle.c) */
double tri_oracle_omega(int f, int d, double theta);
void tri_oracle_score_head(int d, int n, const double* K, const int64_t* pos, int64_t p_now,
                           const double* omega, const int64_t* offsets, int n_off,
                           const double* qc_re, const double* qc_im, const double* q_mean_norm,
                           const double* q_mrl, double* trig, double* norm, double* score);
void tri_oracle_bound_head(int d, int n, const double* K, const double* omega,
                           const int64_t* offsets, int n_off, const double* qc_re,
                           const double* qc_im, const double* q_mean_norm, const double* q_mrl,
                           double* bound);
int tri_oracle_select_head(int n, const double* score, const int64_t* pos, int budget, int window,
                           int32_t* kept);

enum { L = 1, H = 3, D = 64, HALF = 32, N = 700, B = 128, W = 128, N_OFF = 13 };

static uint64_t rng_state = 20240601u;

static uint64_t splitmix64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double uniform(void) { return ((double)(splitmix64() >> 11) + 0.5) / 9007199254740992.0; }

static double normal(void)
{
    const double u = uniform(), v = uniform();
    return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}

static int failures = 0;

static void check(int ok, const char* what, int head)
{
    if (!ok) {
        fprintf(stderr, "FAILED: %s (head %d)\n", what, head);
        ++failures;
    }
}

#define HIP_OK(x)                                                                    \
    do {                                                                             \
        hipError_t e_ = (x);                                                         \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__);        \
            return 2;                                                                \
        }                                                                            \
    } while (0)

#define TRI_OK_(x)                                                                   \
    do {                                                                             \
        tri_status s_ = (x);                                                         \
        if (s_ != TRI_OK) {                                                          \
            fprintf(stderr, "tri call failed: %s at line %d\n", tri_status_str(s_), __LINE__); \
            return 2;                                                                \
        }                                                                            \
    } while (0)

int main(void)
{
    static float k[L * H * N * D], v[L * H * N * D], k_out[L * H * N * D], v_out[L * H * N * D];
    static int32_t pos[L * H * N], pos_out[L * H * N], kept[L * H * B];
    static float scores[L * H * N];
    static double qc_re[L * H * HALF], qc_im[L * H * HALF], qm[L * H * HALF], qr[L * H * HALF];
    int64_t offsets[N_OFF];
    for (int o = 0; o < N_OFF; ++o) offsets[o] = (int64_t)1 << o;

    /* inputs */
    for (int i = 0; i < L * H * HALF; ++i) {
        qc_re[i] = normal();
        qc_im[i] = normal();
        const double c = hypot(qc_re[i], qc_im[i]);
        qm[i] = c * (1.0 + 0.5 * uniform());
        qr[i] = qm[i] > 0.0 ? c / qm[i] : 0.0;
    }
    for (int i = 0; i < L * H * N * D; ++i) {
        k[i] = (float)normal();
        v[i] = (float)normal();
    }
    for (int h = 0; h < L * H; ++h)
        for (int i = 0; i < N; ++i) pos[h * N + i] = i;

    /* the library */
    int n_dev = 0;
    HIP_OK(hipGetDeviceCount(&n_dev));
    if (n_dev < 1) {
        fprintf(stderr, "no GPU\n");
        return 2;
    }
    HIP_OK(hipSetDevice(0));
    tri_calib_desc desc;
    memset(&desc, 0, sizeof(desc));
    desc.n_layers = L;
    desc.n_kv_heads = H;
    desc.head_dim = D;
    desc.rope_theta = 1e4;
    desc.offsets = offsets;
    desc.n_offsets = N_OFF;
    desc.qc_re = qc_re;
    desc.qc_im = qc_im;
    desc.q_mean_norm = qm;
    desc.q_mrl = qr;
    tri_ctx* ctx = NULL;
    TRI_OK_(tri_calibrate_load(&desc, 0, &ctx));

    void *dk, *dv, *dpos, *dscores, *dkept;
    HIP_OK(hipMalloc(&dk, sizeof(k)));
    HIP_OK(hipMalloc(&dv, sizeof(v)));
    HIP_OK(hipMalloc(&dpos, sizeof(pos)));
    HIP_OK(hipMalloc(&dscores, sizeof(scores)));
    HIP_OK(hipMalloc(&dkept, sizeof(kept)));
    HIP_OK(hipMemcpy(dk, k, sizeof(k), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dv, v, sizeof(v), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dpos, pos, sizeof(pos), hipMemcpyHostToDevice));

    tri_seq seq;
    memset(&seq, 0, sizeof(seq));
    seq.k = dk;
    seq.v = dv;
    seq.pos = (int32_t*)dpos;
    seq.cap = N;
    seq.len = N;
    seq.p_now = N - 1;
    seq.head_len = NULL;

    check(tri_select_topb(ctx, &seq, 1, (const float*)dscores, 0, W, (int32_t*)dkept, NULL) ==
              TRI_E_INVAL, "budget 0 is an argument error", -1);
    TRI_OK_(tri_score(ctx, TRI_F32, &seq, 1, (float*)dscores, NULL));
    TRI_OK_(tri_select_topb(ctx, &seq, 1, (const float*)dscores, B, W, (int32_t*)dkept, NULL));
    TRI_OK_(tri_compact_kv(ctx, TRI_F32, &seq, 1, (const int32_t*)dkept, B, W, NULL));
    HIP_OK(hipDeviceSynchronize());
    check(seq.len == B, "the compaction sets len to the budget", -1);
    HIP_OK(hipMemcpy(scores, dscores, sizeof(scores), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(kept, dkept, sizeof(kept), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(k_out, dk, sizeof(k), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(v_out, dv, sizeof(v), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(pos_out, dpos, sizeof(pos), hipMemcpyDeviceToHost));

    /* the oracle, head by head */
    double omega[HALF];
    for (int f = 0; f < HALF; ++f) omega[f] = tri_oracle_omega(f, D, 1e4);
    static double kd[N * D], trig[N], norm[N], ref[N], bound[N];
    static int64_t p64[N];
    static int32_t kept_ref[B];
    double worst = 0.0;
    int disagreements = 0;
    for (int h = 0; h < L * H; ++h) {
        for (int i = 0; i < N * D; ++i) kd[i] = (double)k[(size_t)h * N * D + i];
        for (int i = 0; i < N; ++i) p64[i] = pos[h * N + i];
        const double *cr = qc_re + h * HALF, *ci = qc_im + h * HALF;
        const double *m = qm + h * HALF, *r = qr + h * HALF;
        tri_oracle_score_head(D, N, kd, p64, N - 1, omega, offsets, N_OFF, cr, ci, m, r, trig, norm,
                              ref);
        tri_oracle_bound_head(D, N, kd, omega, offsets, N_OFF, cr, ci, m, r, bound);
        const float* s = scores + h * N;
        for (int i = 0; i < N; ++i) {
            const double e = fabs((double)s[i] - ref[i]) / bound[i];
            if (e > worst) worst = e;
            check(e <= 2e-3, "score within 2e-3 * M", h);
        }
        /* kept list: B slots, ascending, the top-B of the GPU's own scores */
        const int32_t* kg = kept + h * B;
        static char sel[N];
        memset(sel, 0, sizeof(sel));
        for (int j = 0; j < B; ++j) {
            check(kg[j] >= 0 && kg[j] < N, "kept slot in range", h);
            if (j > 0) check(kg[j] > kg[j - 1], "kept slots ascending", h);
            if (kg[j] >= 0 && kg[j] < N) sel[kg[j]] = 1;
        }
        float kmin = INFINITY, emax = -INFINITY;
        int last_kept_at_min = -1, first_evicted_at_max = N;
        for (int i = 0; i < N; ++i) {
            if (sel[i] && s[i] < kmin) kmin = s[i];
            if (!sel[i] && s[i] > emax) emax = s[i];
        }
        check(kmin >= emax, "no kept key scores below an evicted one", h);
        if (kmin == emax) {
            for (int i = 0; i < N; ++i) {
                if (sel[i] && s[i] == kmin) last_kept_at_min = i;
                if (!sel[i] && s[i] == emax && i < first_evicted_at_max) first_evicted_at_max = i;
            }
            check(last_kept_at_min < first_evicted_at_max, "ties go to the lower slot", h);
        }
        /* against the oracle's kept set, outside the tolerance band */
        check(tri_oracle_select_head(N, ref, p64, B, W, kept_ref) == B, "the oracle fires", h);
        double t = INFINITY, mt = 0.0;
        for (int j = 0; j < B; ++j)
            if (ref[kept_ref[j]] < t) {
                t = ref[kept_ref[j]];
                mt = bound[kept_ref[j]];
            }
        for (int i = 0; i < N; ++i) {
            const double tau = 2e-3 * (bound[i] + mt);
            if (ref[i] > t + tau) check(sel[i], "a clearly kept key is kept", h);
            if (ref[i] < t - tau) check(!sel[i], "a clearly evicted key is evicted", h);
        }
        for (int j = 0; j < B; ++j) disagreements += !sel[kept_ref[j]];
        /* compaction: rows r < B are the input rows at kept[r], bit for bit */
        for (int j = 0; j < B; ++j) {
            const size_t dst = ((size_t)h * N + j) * D, src = ((size_t)h * N + kg[j]) * D;
            check(memcmp(k_out + dst, k + src, D * sizeof(float)) == 0, "compacted K row", h);
            check(memcmp(v_out + dst, v + src, D * sizeof(float)) == 0, "compacted V row", h);
            check(pos_out[h * N + j] == pos[h * N + kg[j]], "compacted position", h);
        }
    }
    printf("prune step from C: %d heads, max |ds|/M = %.3g, kept-set disagreements with the oracle %d, "
           "%d failed checks\n", L * H, worst, disagreements, failures);

    (void)hipFree(dk);
    (void)hipFree(dv);
    (void)hipFree(dpos);
    (void)hipFree(dscores);
    (void)hipFree(dkept);
    tri_ctx_destroy(ctx);
    return failures == 0 ? 0 : 1;
}
