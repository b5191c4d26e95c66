// Calibration statistics from pre-RoPE query samples, on the device.
//
// Source: romaanj.github.io "TriAttention" review, section "Method" (an
// offline calibration pass estimates, per frequency band, the pre-RoPE query
// centre E[q_f], the mean norm and the mean resultant length R_f);
// dimensionstp.github.io "TriAttention ... Review", section 3 (the
// calibration phase computes head- and band-wise centre, expected norm and
// concentration, measured as MRL).  Reading: band f of a sample is
// q[f] + i*q[f + d/2]; R_f = |E[q_f]| / E|q_f| (0 when E|q_f| = 0).
//
// One workgroup per query head streams that head's samples.  A sample row is
// split like a key row in the score kernel: LPR lanes cover it, lane j holds
// 16 bytes of the real half and the matching 16 bytes of the imaginary half,
// i.e. E bands.  Each lane accumulates, in fp64, the sums of the real parts,
// the imaginary parts and the magnitudes of its bands over its samples; the
// lanes that share bands are then combined by a fixed tree in LDS, so the
// result does not depend on scheduling.
#include "tri_internal.h"

namespace tri {
namespace {

constexpr int kBlock = 256;
constexpr int kUnroll = 4;   // samples per lane in flight

template <int D, bool BF16>
__global__ __launch_bounds__(kBlock) void calib_stats_kernel(
    const unsigned char* __restrict__ q, int64_t n_samples, int n_heads,
    double* __restrict__ qc_re, double* __restrict__ qc_im, double* __restrict__ mean_norm,
    double* __restrict__ mrl)
{
    constexpr int kElem = BF16 ? 2 : 4;
    constexpr int kHalf = D / 2;
    constexpr int kRowBytes = D * kElem;
    constexpr int kHalfBytes = kRowBytes / 2;
    constexpr int LPR = kHalfBytes / 16;   // lanes per sample row
    constexpr int E = 16 / kElem;          // bands per lane
    constexpr int SPB = kBlock / LPR;      // samples per workgroup step
    static_assert(SPB * LPR == kBlock, "whole rows per step");

    __shared__ double s_acc[3][SPB][kHalf];   // per sample slot: sums over its samples

    const int head = blockIdx.x;
    const int tid = threadIdx.x;
    const int j = tid % LPR;
    const int slot = tid / LPR;
    const size_t row_stride = (size_t)n_heads * kRowBytes;
    const unsigned char* base = q + (size_t)head * kRowBytes + 16 * j;

    double sre[E], sim[E], snm[E];
#pragma unroll
    for (int e = 0; e < E; ++e) sre[e] = sim[e] = snm[e] = 0.0;

    auto unpack = [&](const u32x4& v, float* out) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        if constexpr (BF16) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                out[2 * m] = __uint_as_float(w[m] << 16);
                out[2 * m + 1] = __uint_as_float(w[m] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int m = 0; m < 4; ++m) out[m] = __uint_as_float(w[m]);
        }
    };

    // samples slot, slot + SPB, ... in order; kUnroll of them in flight
    for (int64_t t0 = slot; t0 < n_samples; t0 += (int64_t)SPB * kUnroll) {
        u32x4 re[kUnroll], im[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t t = min(t0 + (int64_t)u * SPB, n_samples - 1);
            const u32x4* p = reinterpret_cast<const u32x4*>(base + (size_t)t * row_stride);
            re[u] = __builtin_nontemporal_load(p);
            im[u] = __builtin_nontemporal_load(p + kHalfBytes / 16);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (t0 + (int64_t)u * SPB >= n_samples) break;
            float a[E], b[E];
            unpack(re[u], a);
            unpack(im[u], b);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const double x = a[e], y = b[e];
                sre[e] += x;
                sim[e] += y;
                snm[e] += sqrt(x * x + y * y);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        s_acc[0][slot][j * E + e] = sre[e];
        s_acc[1][slot][j * E + e] = sim[e];
        s_acc[2][slot][j * E + e] = snm[e];
    }
    __syncthreads();
    // fixed pairwise tree over the sample slots
    for (int width = SPB / 2; width >= 1; width /= 2) {
        for (int i = tid; i < 3 * width * kHalf; i += kBlock) {
            const int c = i / (width * kHalf);
            const int r = i - c * width * kHalf;
            const int sl = r / kHalf, f = r - sl * kHalf;
            s_acc[c][sl][f] += s_acc[c][sl + width][f];
        }
        __syncthreads();
    }
    if (tid < kHalf) {
        const double n = (double)n_samples;
        const double cr = s_acc[0][0][tid] / n, ci = s_acc[1][0][tid] / n;
        const double m = s_acc[2][0][tid] / n;
        const size_t o = (size_t)head * kHalf + tid;
        qc_re[o] = cr;
        qc_im[o] = ci;
        mean_norm[o] = m;
        mrl[o] = m > 0.0 ? sqrt(cr * cr + ci * ci) / m : 0.0;
    }
}

template <int D, bool BF16>
hipError_t launch(const void* q, int64_t n_samples, int n_heads, double* qc_re, double* qc_im,
                  double* mean_norm, double* mrl, hipStream_t stream)
{
    hipLaunchKernelGGL((calib_stats_kernel<D, BF16>), dim3(n_heads), dim3(kBlock), 0, stream,
                       static_cast<const unsigned char*>(q), n_samples, n_heads, qc_re, qc_im,
                       mean_norm, mrl);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_calib_stats(tri_dtype dtype, int head_dim, const void* q, int64_t n_samples,
                              int n_heads, double* qc_re, double* qc_im, double* mean_norm,
                              double* mrl, hipStream_t stream)
{
    if (n_heads <= 0 || n_samples <= 0) return hipSuccess;
    if (dtype == TRI_BF16 && head_dim == 128)
        return launch<128, true>(q, n_samples, n_heads, qc_re, qc_im, mean_norm, mrl, stream);
    if (dtype == TRI_F32 && head_dim == 64)
        return launch<64, false>(q, n_samples, n_heads, qc_re, qc_im, mean_norm, mrl, stream);
    if (dtype == TRI_BF16 && head_dim == 64)
        return launch<64, true>(q, n_samples, n_heads, qc_re, qc_im, mean_norm, mrl, stream);
    if (dtype == TRI_F32 && head_dim == 128)
        return launch<128, false>(q, n_samples, n_heads, qc_re, qc_im, mean_norm, mrl, stream);
    return hipErrorInvalidValue;
}

}  // namespace tri
