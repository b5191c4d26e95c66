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

}  // namespace

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
