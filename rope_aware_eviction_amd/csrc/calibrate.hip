// Derivation of the per-head constant tables from a calibration table, in
// fp64, once per tri_calibrate_load.
//
// Source: romaanj.github.io "TriAttention" review, section "Method": the
// calibration gives per band the pre-RoPE query centre E[q_f], the mean norm
// and the mean resultant length R_f; the online score averages over the
// geometric future offsets.  Averaging exp(i*w_f*(p_now + delta - p)) over
// delta factors into exp(i*w_f*(p_now - p)) * A_f with
// A_f = mean_delta exp(i*w_f*delta), which does not depend on the key or the
// step, so it is computed here once and multiplied into the centre.
#include "tri_internal.h"

namespace tri {
namespace {

// One thread per (head, band).
__global__ void calibrate_kernel(int n_heads, int head_dim, double rope_theta,
                                 const double* __restrict__ inv_freq,
                                 const int64_t* __restrict__ offsets, int n_offsets,
                                 const double* __restrict__ qc_re, const double* __restrict__ qc_im,
                                 const double* __restrict__ q_mean_norm,
                                 const double* __restrict__ q_mrl, double* __restrict__ omega,
                                 double2* __restrict__ qa, float* __restrict__ w)
{
    const int half = head_dim / 2;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_heads * half) return;
    const int f = i % half;
    const int h = i / half;

    // standard RoPE band frequency unless the caller gave explicit ones
    const double om = inv_freq ? inv_freq[f] : pow(rope_theta, -2.0 * (double)f / (double)head_dim);
    if (h == 0) omega[f] = om;

    double a_re = 0.0, a_im = 0.0;
    for (int o = 0; o < n_offsets; ++o) {
        double s, c;
        sincos(om * (double)offsets[o], &s, &c);
        a_re += c;
        a_im += s;
    }
    a_re /= (double)n_offsets;
    a_im /= (double)n_offsets;

    const double q_re = qc_re[i], q_im = qc_im[i];
    qa[i] = make_double2(q_re * a_re - q_im * a_im, q_re * a_im + q_im * a_re);
    w[i] = (float)((1.0 - q_mrl[i]) * q_mean_norm[i]);
}

// Distance-preference curves: curve[qh][j] = sum_f Re(E[q_f] * conj(kc_f) *
// exp(i*w_f*delta_j)) in fp64.
// Source: dimensionstp.github.io "TriAttention ... Review", section 2-1
// item 2 and section 2-2 (Q/K centres turn the RoPE logit into a curve of
// the query-key distance), section 6 item 2 (per-head curves).
//
// The phasor exp(i*w_f*delta_j) does not depend on the query head, so each
// workgroup takes a tile of kCurveTile distances x kCurveTile query heads:
// for kBandChunk bands at a time it evaluates the tile's phasors (one sincos
// per distance and band) and the products E[q_f] * conj(kc_f) of its heads
// into LDS, and every thread accumulates a 4 x 4 block of entries over the
// bands in order.  The band chunks keep the LDS of a workgroup at 32 KB, so
// several workgroups share a compute unit and hide each other's latency.
constexpr int kCurveTile = 64;
constexpr int kCurveBlock = 256;
constexpr int kBandChunk = 16;
static_assert(kCurveTile * kCurveTile == 16 * kCurveBlock, "a 4 x 4 block of entries per thread");

__global__ __launch_bounds__(kCurveBlock) void distance_curve_kernel(
    int n_q_heads, int group, int half, const double* __restrict__ omega,
    const double2* __restrict__ qc, const double* __restrict__ kc_re,
    const double* __restrict__ kc_im, const int64_t* __restrict__ deltas, int n_delta,
    double* __restrict__ curve)
{
    __shared__ double2 s_ph[kBandChunk][kCurveTile];   // (cos, sin) of w_f * delta_j
    __shared__ double2 s_qk[kBandChunk][kCurveTile];   // E[q_f] * conj(kc_f) of the tile's heads
    const int j0 = blockIdx.x * kCurveTile;
    const int h0 = blockIdx.y * kCurveTile;
    const int tid = threadIdx.x;
    const int hb = (tid / 16) * 4;   // the thread's four query heads in the tile
    const int jb = (tid % 16) * 4;   // and its four distances
    double acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
    for (int f0 = 0; f0 < half; f0 += kBandChunk) {
        if (f0 > 0) __syncthreads();   // the previous chunk has been read
        for (int i = tid; i < kBandChunk * kCurveTile; i += kCurveBlock) {
            const int fc = i / kCurveTile, t = i - fc * kCurveTile;
            const int f = f0 + fc;
            const int j = j0 + t;
            double sn = 0.0, cs = 0.0;
            if (f < half && j < n_delta) sincos(omega[f] * (double)deltas[j], &sn, &cs);
            s_ph[fc][t] = make_double2(cs, sn);
            const int qh = h0 + t;
            double pr = 0.0, pi = 0.0;
            if (f < half && qh < n_q_heads) {
                const double2 q = qc[(size_t)qh * half + f];
                const int kv = qh / group;
                const double kr = kc_re[(size_t)kv * half + f], ki = kc_im[(size_t)kv * half + f];
                // q * conj(k) = (q.x*kr + q.y*ki) + i*(q.y*kr - q.x*ki)
                pr = q.x * kr + q.y * ki;
                pi = q.y * kr - q.x * ki;
            }
            s_qk[fc][t] = make_double2(pr, pi);
        }
        __syncthreads();
        const int nf = min(kBandChunk, half - f0);
        for (int fc = 0; fc < nf; ++fc) {
            double2 ph[4], qk[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                ph[x] = s_ph[fc][jb + x];
                qk[x] = s_qk[fc][hb + x];
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] += qk[a].x * ph[b].x - qk[a].y * ph[b].y;
        }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int qh = h0 + hb + a;
        if (qh >= n_q_heads) continue;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int j = j0 + jb + b;
            if (j < n_delta) curve[(size_t)qh * n_delta + j] = acc[a][b];
        }
    }
}

}  // namespace

hipError_t launch_distance_curve(int n_q_heads, int group, int head_dim, const double* omega,
                                 const double2* qc, const double* kc_re, const double* kc_im,
                                 const int64_t* deltas, int n_delta, double* curve,
                                 hipStream_t stream)
{
    if (n_q_heads <= 0 || n_delta <= 0) return hipSuccess;
    const int half = head_dim / 2;
    const int64_t gx = ((int64_t)n_delta + kCurveTile - 1) / kCurveTile;
    const int64_t gy = ((int64_t)n_q_heads + kCurveTile - 1) / kCurveTile;
    if (gx > 0x7FFFFFFF || gy > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(distance_curve_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(kCurveBlock),
                       0, stream, n_q_heads, group, half, omega, qc, kc_re, kc_im, deltas, n_delta,
                       curve);
    return hipGetLastError();
}

hipError_t launch_calibrate(int n_heads, int head_dim, double rope_theta, const double* inv_freq,
                            const int64_t* offsets, int n_offsets, const double* qc_re,
                            const double* qc_im, const double* q_mean_norm, const double* q_mrl,
                            double* omega, double2* qa, float* w, hipStream_t stream)
{
    const int total = n_heads * (head_dim / 2);
    const int block = 256;
    const int grid = (total + block - 1) / block;
    hipLaunchKernelGGL(calibrate_kernel, dim3(grid), dim3(block), 0, stream, n_heads, head_dim,
                       rope_theta, inv_freq, offsets, n_offsets, qc_re, qc_im, q_mean_norm, q_mrl,
                       omega, qa, w);
    return hipGetLastError();
}

}  // namespace tri
