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

// One thread per (query head, distance): the distance-preference curve
// sum_f Re(E[q_f] * conj(kc_f) * exp(i*w_f*delta)) in fp64.
// Source: dimensionstp.github.io "TriAttention ... Review", section 2-1
// item 2 and section 2-2 (Q/K centres turn the RoPE logit into a curve of
// the query-key distance), section 6 item 2 (per-head curves).
__global__ void distance_curve_kernel(int n_q_heads, int group, int half,
                                      const double* __restrict__ omega,
                                      const double2* __restrict__ qc,
                                      const double* __restrict__ kc_re,
                                      const double* __restrict__ kc_im,
                                      const int64_t* __restrict__ deltas, int n_delta,
                                      double* __restrict__ curve)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)n_q_heads * n_delta) return;
    const int qh = (int)(i / n_delta);
    const int j = (int)(i - (int64_t)qh * n_delta);
    const int kv = qh / group;
    const double dl = (double)deltas[j];
    double s = 0.0;
    for (int f = 0; f < half; ++f) {
        const double2 q = qc[(size_t)qh * half + f];
        const double kr = kc_re[(size_t)kv * half + f], ki = kc_im[(size_t)kv * half + f];
        // q * conj(k) = (q.x*kr + q.y*ki) + i*(q.y*kr - q.x*ki)
        const double pr = q.x * kr + q.y * ki, pi = q.y * kr - q.x * ki;
        double sn, cs;
        sincos(omega[f] * dl, &sn, &cs);
        s += pr * cs - pi * sn;
    }
    curve[i] = s;
}

}  // namespace

hipError_t launch_distance_curve(int n_q_heads, int group, int head_dim, const double* omega,
                                 const double2* qc, const double* kc_re, const double* kc_im,
                                 const int64_t* deltas, int n_delta, double* curve,
                                 hipStream_t stream)
{
    const int64_t total = (int64_t)n_q_heads * n_delta;
    if (total <= 0) return hipSuccess;
    const int block = 256;
    const int64_t grid = (total + block - 1) / block;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(distance_curve_kernel, dim3((unsigned)grid), dim3(block), 0, stream,
                       n_q_heads, group, head_dim / 2, omega, qc, kc_re, kc_im, deltas, n_delta,
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
