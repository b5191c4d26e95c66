// Host side of the C ABI declared in include/tri.h: argument validation,
// calibration context, and the launches of one prune step's kernels on the
// caller's stream.  Validation runs entirely on the host and returns before
// any HIP call, so argument errors are reported synchronously and without a
// device.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "tri_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

tri_status hip_fail(hipError_t e)
{
    g_last_hip_error = (int)e;
    return TRI_E_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool supported(int head_dim, tri_dtype dtype)
{
    return (head_dim == 64 || head_dim == 128) && (dtype == TRI_F32 || dtype == TRI_BF16);
}

int elem_size(tri_dtype dtype) { return dtype == TRI_F32 ? 4 : 2; }

// The device current on this thread must be the context's.
tri_status check_device(const tri_ctx* ctx)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    return dev == ctx->device ? TRI_OK : TRI_E_INVAL;
}

// Shape checks common to every per-step call.
tri_status check_seqs(const tri_ctx* ctx, const tri_seq* seqs, int32_t n_seq, bool need_kv)
{
    if (!ctx || n_seq < 0 || (n_seq > 0 && !seqs)) return TRI_E_INVAL;
    for (int32_t s = 0; s < n_seq; ++s) {
        const tri_seq& q = seqs[s];
        if (q.cap < 0 || q.len < 0 || q.len > q.cap) return TRI_E_INVAL;
        // the kernels address a head's rows with 32-bit byte offsets
        if ((int64_t)q.len * ctx->head_dim * 4 >= (int64_t(1) << 31)) return TRI_E_INVAL;
        if (q.p_now < -(int64_t(1) << 52) || q.p_now > (int64_t(1) << 52)) return TRI_E_INVAL;
        if ((uintptr_t)q.head_len & 3u) return TRI_E_INVAL;
        if (q.len == 0) continue;
        if (!q.k || !aligned16(q.k)) return TRI_E_INVAL;
        if (need_kv && (!q.v || !aligned16(q.v) || !q.pos || ((uintptr_t)q.pos & 3u)))
            return TRI_E_INVAL;
    }
    return TRI_OK;
}

bool fires(const tri_seq& q, int32_t budget, int32_t window)
{
    return (int64_t)q.len > (int64_t)budget + (int64_t)window;
}

// Uniform budgets keep every head at one length: no per-head lengths.
bool any_ragged(const tri_seq* seqs, int32_t n_seq)
{
    for (int32_t s = 0; s < n_seq; ++s)
        if (seqs[s].head_len) return true;
    return false;
}

}  // namespace

extern "C" {

const char* tri_status_str(tri_status s)
{
    switch (s) {
    case TRI_OK: return "ok";
    case TRI_E_INVAL: return "invalid argument";
    case TRI_E_UNSUPPORTED: return "unsupported head_dim or dtype";
    case TRI_E_HIP: return "HIP runtime error";
    case TRI_E_NOMEM: return "out of memory";
    case TRI_E_SCRATCH: return "the call needs more scratch than the library's static buffer holds";
    }
    return "unknown status";
}

int tri_last_hip_error(void) { return g_last_hip_error; }

void tri_ctx_destroy(tri_ctx* ctx)
{
    if (!ctx) return;
    int prev = -1;
    const bool have_prev = hipGetDevice(&prev) == hipSuccess;
    if (hipSetDevice(ctx->device) == hipSuccess) {
        (void)hipFree(ctx->omega);
        (void)hipFree(ctx->qa);
        (void)hipFree(ctx->w);
        (void)hipFree(ctx->qc);
    }
    if (have_prev) (void)hipSetDevice(prev);
    delete ctx;
}

tri_status tri_calibrate_load(const tri_calib_desc* d, int device, tri_ctx** out)
{
    if (!out) return TRI_E_INVAL;
    *out = nullptr;
    if (!d) return TRI_E_INVAL;
    if (d->head_dim != 64 && d->head_dim != 128) return TRI_E_UNSUPPORTED;
    if (d->n_layers < 1 || d->n_kv_heads < 1 || d->n_offsets < 1 || device < 0) return TRI_E_INVAL;
    if ((int64_t)d->n_layers * d->n_kv_heads > (1 << 24)) return TRI_E_INVAL;
    if (!d->offsets || !d->qc_re || !d->qc_im || !d->q_mean_norm || !d->q_mrl) return TRI_E_INVAL;
    // query heads per KV head: 1, or a GQA group of 2..8
    const int n_q = d->n_q_heads == 0 ? d->n_kv_heads : d->n_q_heads;
    if (n_q < d->n_kv_heads || n_q % d->n_kv_heads != 0) return TRI_E_INVAL;
    const int group = n_q / d->n_kv_heads;
    if (group > 8) return TRI_E_UNSUPPORTED;
    const int half = d->head_dim / 2;
    const int n_heads = d->n_layers * d->n_kv_heads;
    const size_t nb = (size_t)n_heads * group * half;   // query tables, [head][g][band]
    if (d->inv_freq) {
        for (int f = 0; f < half; ++f)
            if (!std::isfinite(d->inv_freq[f]) || !(d->inv_freq[f] > 0.0)) return TRI_E_INVAL;
    } else if (!std::isfinite(d->rope_theta) || !(d->rope_theta > 0.0)) {
        return TRI_E_INVAL;
    }
    for (int o = 0; o < d->n_offsets; ++o)
        if (d->offsets[o] < 0 || d->offsets[o] > (int64_t(1) << 40)) return TRI_E_INVAL;
    for (size_t i = 0; i < nb; ++i) {
        if (!std::isfinite(d->qc_re[i]) || !std::isfinite(d->qc_im[i])) return TRI_E_INVAL;
        if (!std::isfinite(d->q_mean_norm[i]) || d->q_mean_norm[i] < 0.0) return TRI_E_INVAL;
        if (!(d->q_mrl[i] >= 0.0 && d->q_mrl[i] <= 1.0)) return TRI_E_INVAL;
    }

    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e != hipSuccess) return hip_fail(e);
    e = hipSetDevice(device);
    if (e != hipSuccess) return hip_fail(e);

    tri_ctx* ctx = new (std::nothrow) tri_ctx{};
    if (!ctx) {
        (void)hipSetDevice(prev);
        return TRI_E_NOMEM;
    }
    ctx->device = device;
    ctx->n_layers = d->n_layers;
    ctx->n_kv_heads = d->n_kv_heads;
    ctx->head_dim = d->head_dim;
    ctx->n_heads = n_heads;
    ctx->group = group;

    // raw table staged on the device, derived tables computed there in fp64
    double *r_inv = nullptr, *r_re = nullptr, *r_im = nullptr, *r_m = nullptr, *r_R = nullptr;
    int64_t* r_off = nullptr;
    tri_status st = TRI_OK;
    auto alloc = [&](void** p, size_t bytes) {
        if (st != TRI_OK) return;
        hipError_t a = hipMalloc(p, bytes);
        if (a != hipSuccess) {
            g_last_hip_error = (int)a;
            st = a == hipErrorOutOfMemory ? TRI_E_NOMEM : TRI_E_HIP;
        }
    };
    auto put = [&](void* dst, const void* src, size_t bytes) {
        if (st != TRI_OK) return;
        hipError_t c = hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice);
        if (c != hipSuccess) st = hip_fail(c);
    };
    alloc((void**)&ctx->omega, sizeof(double) * half);
    alloc((void**)&ctx->qa, sizeof(double2) * nb);
    alloc((void**)&ctx->w, sizeof(float) * nb);
    alloc((void**)&ctx->qc, sizeof(double2) * nb);
    if (d->inv_freq) alloc((void**)&r_inv, sizeof(double) * half);
    alloc((void**)&r_off, sizeof(int64_t) * d->n_offsets);
    alloc((void**)&r_re, sizeof(double) * nb);
    alloc((void**)&r_im, sizeof(double) * nb);
    alloc((void**)&r_m, sizeof(double) * nb);
    alloc((void**)&r_R, sizeof(double) * nb);
    if (d->inv_freq) put(r_inv, d->inv_freq, sizeof(double) * half);
    put(r_off, d->offsets, sizeof(int64_t) * d->n_offsets);
    put(r_re, d->qc_re, sizeof(double) * nb);
    put(r_im, d->qc_im, sizeof(double) * nb);
    put(r_m, d->q_mean_norm, sizeof(double) * nb);
    put(r_R, d->q_mrl, sizeof(double) * nb);
    if (st == TRI_OK) {   // the query centres as loaded, interleaved (re, im)
        std::vector<double> qc(2 * nb);
        for (size_t i = 0; i < nb; ++i) {
            qc[2 * i] = d->qc_re[i];
            qc[2 * i + 1] = d->qc_im[i];
        }
        put(ctx->qc, qc.data(), sizeof(double2) * nb);
    }
    if (st == TRI_OK) {   // this device's static scratch (allocation-free calls), once per device
        e = tri::scratch_address(device, &ctx->scratch);
        if (e != hipSuccess) st = hip_fail(e);
    }
    if (st == TRI_OK) {
        e = tri::launch_calibrate(n_heads * group, d->head_dim, d->rope_theta, r_inv, r_off, d->n_offsets,
                                  r_re, r_im, r_m, r_R, ctx->omega, ctx->qa, ctx->w, nullptr);
        if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
        if (e != hipSuccess) st = hip_fail(e);
    }
    (void)hipFree(r_inv);
    (void)hipFree(r_off);
    (void)hipFree(r_re);
    (void)hipFree(r_im);
    (void)hipFree(r_m);
    (void)hipFree(r_R);
    if (st != TRI_OK) {
        (void)hipFree(ctx->omega);
        (void)hipFree(ctx->qa);
        (void)hipFree(ctx->w);
        (void)hipFree(ctx->qc);
        delete ctx;
        (void)hipSetDevice(prev);
        return st;
    }
    (void)hipSetDevice(prev);
    *out = ctx;
    return TRI_OK;
}

tri_status tri_calibrate_stats(tri_dtype dtype, const void* q, int64_t n_samples, int32_t n_heads,
                               int32_t head_dim, double* qc_re, double* qc_im,
                               double* q_mean_norm, double* q_mrl, void* stream)
{
    if (!q || !aligned16(q) || n_samples < 1 || n_heads < 1) return TRI_E_INVAL;
    for (const double* p : {qc_re, qc_im, q_mean_norm, q_mrl})
        if (!p || ((uintptr_t)p & 7u)) return TRI_E_INVAL;
    if (!supported(head_dim, dtype)) return TRI_E_UNSUPPORTED;
    hipError_t e = tri::launch_calib_stats(dtype, head_dim, q, n_samples, n_heads, qc_re, qc_im,
                                           q_mean_norm, q_mrl, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TRI_OK : hip_fail(e);
}

tri_status tri_distance_curve(const tri_ctx* ctx, const double* kc_re, const double* kc_im,
                              const int64_t* deltas, int32_t n_delta, double* curve, void* stream)
{
    if (!ctx || n_delta < 0) return TRI_E_INVAL;
    if (n_delta == 0) return TRI_OK;
    for (const void* p : {(const void*)kc_re, (const void*)kc_im, (const void*)deltas, (const void*)curve})
        if (!p || ((uintptr_t)p & 7u)) return TRI_E_INVAL;
    tri_status st = check_device(ctx);
    if (st != TRI_OK) return st;
    hipError_t e = tri::launch_distance_curve(ctx->n_heads * ctx->group, ctx->group, ctx->head_dim,
                                              ctx->omega, ctx->qc, kc_re, kc_im, deltas, n_delta,
                                              curve, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TRI_OK : hip_fail(e);
}

int32_t tri_offset_set(int32_t kind, int64_t max_distance, int32_t count, int64_t* out, int32_t cap)
{
    if (max_distance < 1 || max_distance > (int64_t(1) << 40) || cap < 0 || (cap > 0 && !out))
        return -1;
    int32_t n = 0;
    auto emit = [&](int64_t x) {
        if (n < cap) out[n] = x;
        ++n;
    };
    if (kind == 0) {                     // geometric: powers of two up to max_distance
        for (int64_t x = 1; x <= max_distance; x <<= 1) emit(x);
        return n;
    }
    if (kind == 1) {                     // linear: count evenly spaced, ending at max_distance
        if (count < 1 || count > (1 << 20)) return -1;
        for (int32_t k = 1; k <= count; ++k) {
            // round(max_distance * k / count) in integers: (2*m*k + count) / (2*count)
            const __int128 num = (__int128)2 * max_distance * k + count;
            int64_t x = (int64_t)(num / (2 * (__int128)count));
            emit(x < 1 ? 1 : x);
        }
        return n;
    }
    return -1;
}

int64_t tri_scores_count(const tri_ctx* ctx, const tri_seq* seqs, int32_t n_seq)
{
    if (!ctx || n_seq < 0 || (n_seq > 0 && !seqs)) return -1;
    int64_t total = 0;
    for (int32_t s = 0; s < n_seq; ++s) {
        if (seqs[s].len < 0) return -1;
        total += (int64_t)ctx->n_heads * seqs[s].len;
    }
    return total;
}

int64_t tri_score_workspace_bytes(const tri_ctx* ctx, const tri_seq* seqs, int32_t n_seq)
{
    if (!ctx || n_seq < 0 || (n_seq > 0 && !seqs)) return -1;
    if (ctx->group == 1) return 0;
    int64_t total = 0;
    for (int32_t s = 0; s < n_seq; ++s) {
        if (seqs[s].len < 0) return -1;
        if (seqs[s].len > 0) total += tri::gqa_workspace_bytes(ctx->n_heads, seqs[s].len, ctx->group);
    }
    return total;
}

tri_status tri_score_ws(const tri_ctx* ctx, tri_dtype dtype, const tri_seq* seqs, int32_t n_seq,
                        float* scores, void* workspace, int64_t workspace_bytes, void* stream)
{
    tri_status st = check_seqs(ctx, seqs, n_seq, false);
    if (st != TRI_OK) return st;
    if (!supported(ctx->head_dim, dtype)) return TRI_E_UNSUPPORTED;
    const int64_t total = tri_scores_count(ctx, seqs, n_seq);
    // GQA contexts may pass no score array: the workspace then holds the raw
    // scores and their statistics for tri_select_topb_ws
    if (total > 0 && ((!scores && ctx->group == 1) || ((uintptr_t)scores & 3u))) return TRI_E_INVAL;
    const int64_t need = tri_score_workspace_bytes(ctx, seqs, n_seq);
    if (need > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < need))
        return TRI_E_INVAL;
    if (total == 0) return TRI_OK;
    st = check_device(ctx);
    if (st != TRI_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int64_t off = 0;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    for (int32_t s = 0; s < n_seq; ++s) {
        const tri_seq& q = seqs[s];
        if (q.len > 0) {
            hipError_t e;
            if (ctx->group == 1) {
                e = tri::launch_score(dtype, ctx->head_dim, q.k, q.cap, q.len, ctx->n_heads, q.p_now,
                                      ctx->omega, ctx->qa, ctx->w, scores + off, q.head_len, hs);
            } else {
                e = tri::launch_gqa_score(dtype, ctx->head_dim, ctx->group, q.k, q.cap, q.len,
                                          ctx->n_heads, q.p_now, ctx->omega, ctx->qa, ctx->w, ws,
                                          scores ? scores + off : nullptr, q.head_len, hs);
                ws += tri::gqa_workspace_bytes(ctx->n_heads, q.len, ctx->group);
            }
            if (e != hipSuccess) return hip_fail(e);
        }
        off += (int64_t)ctx->n_heads * q.len;
    }
    return TRI_OK;
}

tri_status tri_score(const tri_ctx* ctx, tri_dtype dtype, const tri_seq* seqs, int32_t n_seq,
                     float* scores, void* stream)
{
    if (ctx && ctx->group != 1) return TRI_E_INVAL;   // GQA needs tri_score_ws
    return tri_score_ws(ctx, dtype, seqs, n_seq, scores, nullptr, 0, stream);
}

tri_status tri_select_topb(const tri_ctx* ctx, const tri_seq* seqs, int32_t n_seq,
                           const float* scores, int32_t budget, int32_t window, int32_t* kept,
                           void* stream)
{
    tri_status st = check_seqs(ctx, seqs, n_seq, false);
    if (st != TRI_OK) return st;
    if (budget < 1 || window < 0 || any_ragged(seqs, n_seq)) return TRI_E_INVAL;
    bool any = false;
    for (int32_t s = 0; s < n_seq; ++s) any = any || fires(seqs[s], budget, window);
    if (!any) return TRI_OK;
    if (!scores || !kept || ((uintptr_t)scores & 3u) || ((uintptr_t)kept & 3u)) return TRI_E_INVAL;
    st = check_device(ctx);
    if (st != TRI_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (n_seq == 1) {
        hipError_t e = tri::launch_select(scores, seqs[0].len, ctx->n_heads, budget, kept, budget,
                                          nullptr, hs);
        return e == hipSuccess ? TRI_OK : hip_fail(e);
    }
    // several sequences: one table of the firing ones, as few launches as
    // their length classes allow
    std::vector<const float*> sc;
    std::vector<int32_t*> kp;
    std::vector<int> n;
    int64_t off = 0;
    for (int32_t s = 0; s < n_seq; ++s) {
        const tri_seq& q = seqs[s];
        if (fires(q, budget, window)) {
            sc.push_back(scores + off);
            kp.push_back(kept + (int64_t)s * ctx->n_heads * budget);
            n.push_back(q.len);
        }
        off += (int64_t)ctx->n_heads * q.len;
    }
    hipError_t e = tri::launch_select_batch((int)n.size(), sc.data(), kp.data(), n.data(),
                                            ctx->n_heads, budget, hs);
    return e == hipSuccess ? TRI_OK : hip_fail(e);
}

tri_status tri_select_topb_ws(const tri_ctx* ctx, const tri_seq* seqs, int32_t n_seq,
                              float* scores, const void* workspace, int64_t workspace_bytes,
                              int32_t budget, int32_t window, int32_t* kept, void* stream)
{
    tri_status st = check_seqs(ctx, seqs, n_seq, false);
    if (st != TRI_OK) return st;
    if (ctx->group == 1 || budget < 1 || window < 0 || any_ragged(seqs, n_seq)) return TRI_E_INVAL;
    bool any = false, long_heads = false;
    for (int32_t s = 0; s < n_seq; ++s) {
        if (!fires(seqs[s], budget, window)) continue;
        any = true;
        long_heads = long_heads || seqs[s].len > 32768;
    }
    if (!any) return TRI_OK;
    const int64_t need = tri_score_workspace_bytes(ctx, seqs, n_seq);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need) return TRI_E_INVAL;
    if (!kept || ((uintptr_t)kept & 3u)) return TRI_E_INVAL;
    if ((long_heads && !scores) || ((uintptr_t)scores & 3u)) return TRI_E_INVAL;
    st = check_device(ctx);
    if (st != TRI_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    // the workspace is sliced per sequence exactly as tri_score_ws slices it
    unsigned char* ws = static_cast<unsigned char*>(const_cast<void*>(workspace));
    int64_t off = 0;
    for (int32_t s = 0; s < n_seq; ++s) {
        const tri_seq& q = seqs[s];
        if (q.len > 0 && fires(q, budget, window)) {
            float* raw = nullptr;
            double* partial = nullptr;
            double2* stats = nullptr;
            tri::gqa_workspace_views(ws, ctx->n_heads, q.len, ctx->group, &raw, &partial, &stats);
            int32_t* kp = kept + (int64_t)s * ctx->n_heads * budget;
            hipError_t e;
            if (q.len <= 32768) {
                e = tri::launch_select_gqa(ctx->group, raw, partial, q.len, ctx->n_heads, budget,
                                           kp, budget, hs);
            } else {
                // longer heads: the statistics and the normalized scores first,
                // then the plain selection
                e = tri::launch_gqa_stats(ctx->group, partial, q.len, ctx->n_heads, stats, hs);
                if (e == hipSuccess)
                    e = tri::launch_gqa_normalize(ctx->group, raw, stats, q.len, ctx->n_heads,
                                                  scores + off, hs);
                if (e == hipSuccess)
                    e = tri::launch_select(scores + off, q.len, ctx->n_heads, budget, kp, budget,
                                           nullptr, hs);
            }
            if (e != hipSuccess) return hip_fail(e);
        }
        if (q.len > 0) ws += tri::gqa_workspace_bytes(ctx->n_heads, q.len, ctx->group);
        off += (int64_t)ctx->n_heads * q.len;
    }
    return TRI_OK;
}

tri_status tri_compact_kv(const tri_ctx* ctx, tri_dtype dtype, tri_seq* seqs, int32_t n_seq,
                          const int32_t* kept, int32_t budget, int32_t window, void* stream)
{
    tri_status st = check_seqs(ctx, seqs, n_seq, true);
    if (st != TRI_OK) return st;
    if (!supported(ctx->head_dim, dtype)) return TRI_E_UNSUPPORTED;
    if (budget < 1 || window < 0 || any_ragged(seqs, n_seq)) return TRI_E_INVAL;
    bool any = false;
    for (int32_t s = 0; s < n_seq; ++s) any = any || fires(seqs[s], budget, window);
    if (!any) return TRI_OK;
    if (!kept || ((uintptr_t)kept & 3u)) return TRI_E_INVAL;
    st = check_device(ctx);
    if (st != TRI_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int row_bytes = ctx->head_dim * elem_size(dtype);
    if (n_seq == 1) {
        tri_seq& q = seqs[0];
        hipError_t e = tri::launch_compact(row_bytes, q.k, q.v, q.pos, q.cap, q.len, ctx->n_heads,
                                           kept, budget, budget, nullptr, nullptr, nullptr, hs);
        if (e != hipSuccess) return hip_fail(e);
        q.len = budget;
        return TRI_OK;
    }
    // several sequences: the firing ones in one table
    std::vector<void*> k, v;
    std::vector<int32_t*> pos;
    std::vector<int> cap, len;
    std::vector<const int32_t*> kp;
    for (int32_t s = 0; s < n_seq; ++s) {
        const tri_seq& q = seqs[s];
        if (!fires(q, budget, window)) continue;
        k.push_back(q.k);
        v.push_back(q.v);
        pos.push_back(q.pos);
        cap.push_back(q.cap);
        len.push_back(q.len);
        kp.push_back(kept + (int64_t)s * ctx->n_heads * budget);
    }
    hipError_t e = tri::launch_compact_batch(row_bytes, (int)k.size(), k.data(), v.data(),
                                             pos.data(), cap.data(), len.data(), kp.data(),
                                             ctx->n_heads, budget, hs);
    if (e != hipSuccess) return hip_fail(e);
    for (int32_t s = 0; s < n_seq; ++s)
        if (fires(seqs[s], budget, window)) seqs[s].len = budget;
    return TRI_OK;
}

int64_t tri_select_shared_workspace_bytes(const tri_ctx* ctx, int32_t n_seq)
{
    if (!ctx || n_seq < 0) return -1;
    return tri::shared_workspace_bytes(n_seq, ctx->n_layers, ctx->n_kv_heads);
}

tri_status tri_select_shared(const tri_ctx* ctx, const tri_seq* seqs, int32_t n_seq,
                             const float* scores, int32_t budget, int32_t floor, int32_t window,
                             int32_t* kept, int32_t* kept_count, void* workspace,
                             int64_t workspace_bytes, void* stream)
{
    tri_status st = check_seqs(ctx, seqs, n_seq, false);
    if (st != TRI_OK) return st;
    if (budget < 1 || window < 0 || floor < 0 || floor > budget) return TRI_E_INVAL;
    if ((int64_t)budget * ctx->n_kv_heads > INT32_MAX) return TRI_E_INVAL;
    if (ctx->n_kv_heads > 128) return TRI_E_UNSUPPORTED;
    if (n_seq == 0) return TRI_OK;
    const int64_t need = tri::shared_workspace_bytes(n_seq, ctx->n_layers, ctx->n_kv_heads);
    if (!kept || !kept_count || ((uintptr_t)kept & 3u) || ((uintptr_t)kept_count & 3u) ||
        !workspace || !aligned16(workspace) || workspace_bytes < need)
        return TRI_E_INVAL;
    bool any_keys = false;
    for (int32_t s = 0; s < n_seq; ++s) any_keys = any_keys || seqs[s].len > 0;
    if (any_keys && (!scores || ((uintptr_t)scores & 3u))) return TRI_E_INVAL;
    st = check_device(ctx);
    if (st != TRI_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int64_t total = (int64_t)budget * ctx->n_kv_heads;
    const int64_t heads = ctx->n_heads;                      // n_layers * n_kv_heads
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    const int64_t ws_seq = tri::shared_workspace_bytes(1, ctx->n_layers, ctx->n_kv_heads);
    int64_t off = 0;
    for (int32_t s = 0; s < n_seq; ++s) {
        const tri_seq& q = seqs[s];
        hipError_t e = tri::launch_select_shared(
            scores ? scores + off : nullptr, q.len, ctx->n_layers, ctx->n_kv_heads, q.head_len,
            budget, floor, window, kept + s * heads * total, kept_count + s * heads,
            ws + s * ws_seq, hs);
        if (e != hipSuccess) return hip_fail(e);
        off += heads * q.len;
    }
    return TRI_OK;
}

int64_t tri_compact_kv_counts_workspace_bytes(const tri_ctx* ctx)
{
    if (!ctx) return -1;
    return tri::compact_queue_bytes(ctx->n_heads);
}

}  // extern "C"

namespace {

// Argument checks of the counted compaction (everything but the workspace).
tri_status check_compact_counts(const tri_ctx* ctx, tri_dtype dtype, const tri_seq* seqs,
                                int32_t n_seq, const int32_t* kept, int32_t kept_stride,
                                const int32_t* kept_count)
{
    tri_status st = check_seqs(ctx, seqs, n_seq, true);
    if (st != TRI_OK) return st;
    if (!supported(ctx->head_dim, dtype)) return TRI_E_UNSUPPORTED;
    if (kept_stride < 1) return TRI_E_INVAL;
    if (n_seq == 0) return TRI_OK;
    for (int32_t s = 0; s < n_seq; ++s)
        if (!seqs[s].head_len) return TRI_E_INVAL;
    if (!kept || !kept_count || ((uintptr_t)kept & 3u) || ((uintptr_t)kept_count & 3u))
        return TRI_E_INVAL;
    return TRI_OK;
}

// The counted compaction's launches, with the queue at `queue`.
tri_status compact_counts(const tri_ctx* ctx, tri_dtype dtype, tri_seq* seqs, int32_t n_seq,
                          const int32_t* kept, int32_t kept_stride, const int32_t* kept_count,
                          void* queue, void* stream)
{
    tri_status st = check_device(ctx);
    if (st != TRI_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int row_bytes = ctx->head_dim * elem_size(dtype);
    const int64_t heads = ctx->n_heads;
    for (int32_t s = 0; s < n_seq; ++s) {
        tri_seq& q = seqs[s];
        if (q.len == 0) continue;        // no rows: every count is 0 or -1 and head_len stays
        hipError_t e = tri::launch_compact(row_bytes, q.k, q.v, q.pos, q.cap, q.len, ctx->n_heads,
                                           kept + s * heads * kept_stride, 0, kept_stride,
                                           kept_count + s * heads, q.head_len,
                                           static_cast<uint32_t*>(queue), hs);
        if (e != hipSuccess) return hip_fail(e);
    }
    return TRI_OK;
}

}  // namespace

extern "C" {

tri_status tri_compact_kv_counts(const tri_ctx* ctx, tri_dtype dtype, tri_seq* seqs,
                                 int32_t n_seq, const int32_t* kept, int32_t kept_stride,
                                 const int32_t* kept_count, void* workspace,
                                 int64_t workspace_bytes, void* stream)
{
    tri_status st = check_compact_counts(ctx, dtype, seqs, n_seq, kept, kept_stride, kept_count);
    if (st != TRI_OK || n_seq == 0) return st;
    if (!workspace || ((uintptr_t)workspace & 3u) ||
        workspace_bytes < tri::compact_queue_bytes(ctx->n_heads))
        return TRI_E_INVAL;
    return compact_counts(ctx, dtype, seqs, n_seq, kept, kept_stride, kept_count, workspace, stream);
}

tri_status tri_compact_kv_counts_noalloc(const tri_ctx* ctx, tri_dtype dtype, tri_seq* seqs,
                                         int32_t n_seq, const int32_t* kept, int32_t kept_stride,
                                         const int32_t* kept_count, void* stream)
{
    tri_status st = check_compact_counts(ctx, dtype, seqs, n_seq, kept, kept_stride, kept_count);
    if (st != TRI_OK || n_seq == 0) return st;
    if (tri::compact_queue_bytes(ctx->n_heads) > tri::scratch_bytes() || !ctx->scratch)
        return TRI_E_SCRATCH;
    return compact_counts(ctx, dtype, seqs, n_seq, kept, kept_stride, kept_count, ctx->scratch,
                          stream);
}

}  // extern "C"
