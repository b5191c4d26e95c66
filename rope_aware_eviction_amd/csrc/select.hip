// Per-head top-B selection with a deterministic tie-break.
//
// Source: romaanj.github.io "TriAttention" review, section "Method" (prune
// back to the budget) and figure 4 caption (only the top-scoring keys
// survive); dimensionstp.github.io review, section 3-2 item 5 (keep the
// top-budget keys, evict the rest).  Reading: equal scores go to the lower
// position, which is the lower slot because positions ascend with slots;
// NaN ranks below every number; -0 equals +0.
//
// One workgroup of 1024 threads per head.  Scores map to order-preserving
// uint32 keys.  A radix select finds the key T of the B-th largest score and
// how many keys equal to T are still needed: it starts at the highest bit in
// which the head's keys differ (so the first 11-bit histogram spreads over
// the populated range instead of piling into a few exponent bins) and stops
// early when a whole histogram bin is kept.  Histograms live in LDS; when
// the head's keys fit, they are staged in LDS once and every pass reads
// them from there.  The output pass gives each wave a contiguous segment of
// slots; ballots and popcounts give every kept key its rank among the kept
// keys in slot order, so the kept list comes out ascending with no sort.
#include "tri_internal.h"

namespace tri {
namespace {

constexpr int kBlock = 1024;
constexpr int kWaves = kBlock / 64;
constexpr int kMaxDigitBits = 11;
constexpr int kHistBins = 1 << kMaxDigitBits;
// keys of a head staged in LDS up to this many (4 bytes each, plus the
// 8 KB histogram, within the 160 KB LDS of a gfx950 workgroup)
constexpr int kLdsKeysMax = 36864;

__device__ __forceinline__ uint32_t ordered_key(float x)
{
    if (x != x) return 0u;                   // NaN below every number
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;            // -0 equals +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <bool kInLds>
__device__ __forceinline__ uint32_t key_at(const uint32_t* lds_keys, const float* sc, int i)
{
    if constexpr (kInLds) return lds_keys[i];
    else return ordered_key(sc[i]);
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
    return v;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
    return v;
}

template <bool kInLds>
__global__ __launch_bounds__(kBlock) void select_kernel(const float* __restrict__ scores, int n,
                                                        int budget, int32_t* __restrict__ kept)
{
    extern __shared__ uint32_t smem[];
    uint32_t* hist = smem;                             // [kHistBins]
    uint32_t* lds_keys = smem + kHistBins;             // [n] when kInLds
    __shared__ uint32_t s_wmin[kWaves], s_wmax[kWaves];
    __shared__ uint32_t s_wgt[kWaves], s_weq[kWaves];
    __shared__ uint32_t s_digit, s_above;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const float* sc = scores + (size_t)blockIdx.x * (size_t)n;
    int32_t* out = kept + (size_t)blockIdx.x * (size_t)budget;

    // stage keys (when they fit) and find the key range of the head
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for (int i = tid; i < n; i += kBlock) {
        const uint32_t key = ordered_key(sc[i]);
        if constexpr (kInLds) lds_keys[i] = key;
        kmin = min(kmin, key);
        kmax = max(kmax, key);
    }
    kmin = wave_min(kmin);
    kmax = wave_max(kmax);
    if (lane == 0) {
        s_wmin[wave] = kmin;
        s_wmax[wave] = kmax;
    }
    __syncthreads();
    kmin = s_wmin[0];
    kmax = s_wmax[0];
    for (int x = 1; x < kWaves; ++x) {
        kmin = min(kmin, s_wmin[x]);
        kmax = max(kmax, s_wmax[x]);
    }

    // radix select: T is the key of the B-th largest score; need_eq keys
    // equal to T are kept (lowest slots first)
    uint32_t T;
    uint32_t need_eq;
    const uint32_t diff = kmin ^ kmax;
    if (diff == 0u) {
        T = kmin;                 // every key equal: keep slots 0..B-1
        need_eq = (uint32_t)budget;
    } else {
        int lo_bit = 32 - __clz((int)diff);            // bits [lo_bit, 32) are common
        uint32_t pmask = lo_bit >= 32 ? 0u : ~((1u << lo_bit) - 1u);
        uint32_t prefix = kmin & pmask;
        uint32_t rem = (uint32_t)budget;
        bool exact = true;
        while (lo_bit > 0) {
            const int nb = min(kMaxDigitBits, lo_bit);
            const int shift = lo_bit - nb;
            const uint32_t nbins = 1u << nb;
            const uint32_t dmask = nbins - 1u;
            for (uint32_t b = tid; b < nbins; b += kBlock) hist[b] = 0u;
            __syncthreads();
            for (int i = tid; i < n; i += kBlock) {
                const uint32_t key = key_at<kInLds>(lds_keys, sc, i);
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
            }
            __syncthreads();
            if (wave == 0) {
                // lane l owns a run of bins counted from the top
                const uint32_t per = nbins >= 64u ? nbins / 64u : 1u;
                const uint32_t hi = (uint32_t)lane * per;          // bins [nbins-hi-per, nbins-hi)
                uint32_t sum = 0u;
                if (hi < nbins)
                    for (uint32_t t = 0; t < per; ++t) sum += hist[nbins - 1u - hi - t];
                uint32_t incl = sum;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const uint32_t v = (uint32_t)__shfl_up((int)incl, o);
                    if (lane >= o) incl += v;
                }
                const unsigned long long hit = __ballot(incl >= rem);
                const int L = __ffsll((long long)hit) - 1;
                if (lane == L) {
                    uint32_t acc = incl - sum;
                    for (uint32_t t = 0; t < per; ++t) {
                        const uint32_t b = nbins - 1u - hi - t;
                        if (acc + hist[b] >= rem) {
                            s_digit = b;
                            s_above = acc;
                            break;
                        }
                        acc += hist[b];
                    }
                }
            }
            __syncthreads();
            const uint32_t d = s_digit & dmask;
            rem -= s_above;
            prefix |= d << shift;
            pmask |= dmask << shift;
            lo_bit = shift;
            const uint32_t in_bin = hist[d];
            __syncthreads();   // hist is cleared by the next pass
            if (rem == in_bin && prefix != 0u) {
                exact = false; // the whole bin is kept: keep every key >= prefix
                break;
            }
        }
        if (exact) {
            T = prefix;
            need_eq = rem;
        } else {
            T = prefix - 1u;
            need_eq = 0u;
        }
    }

    // stable output: wave w owns slots [w*seg, (w+1)*seg)
    const int seg = ((n + kWaves - 1) / kWaves + 63) & ~63;
    const int s0 = wave * seg;
    const int s1 = min(n, s0 + seg);
    uint32_t cgt = 0u, ceq = 0u;
    for (int i0 = s0; i0 < s1; i0 += 64) {
        const int i = i0 + lane;
        const uint32_t key = i < s1 ? key_at<kInLds>(lds_keys, sc, i) : 0u;
        cgt += __popcll(__ballot(i < s1 && key > T));
        ceq += __popcll(__ballot(i < s1 && key == T));
    }
    if (lane == 0) {
        s_wgt[wave] = cgt;
        s_weq[wave] = ceq;
    }
    __syncthreads();
    uint32_t gt_before = 0u, eq_before = 0u;
    for (int x = 0; x < wave; ++x) {
        gt_before += s_wgt[x];
        eq_before += s_weq[x];
    }
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int i0 = s0; i0 < s1; i0 += 64) {
        const int i = i0 + lane;
        const uint32_t key = i < s1 ? key_at<kInLds>(lds_keys, sc, i) : 0u;
        const bool gt = i < s1 && key > T;
        const bool eq = i < s1 && key == T;
        const unsigned long long mgt = __ballot(gt);
        const unsigned long long meq = __ballot(eq);
        const uint32_t my_gt = gt_before + (uint32_t)__popcll(mgt & below);
        const uint32_t my_eq = eq_before + (uint32_t)__popcll(meq & below);
        const uint32_t at = my_gt + min(my_eq, need_eq);
        if ((gt || (eq && my_eq < need_eq)) && at < (uint32_t)budget) out[at] = i;
        gt_before += (uint32_t)__popcll(mgt);
        eq_before += (uint32_t)__popcll(meq);
    }
}

}  // namespace

hipError_t launch_select(const float* scores, int n, int n_heads, int budget, int32_t* kept,
                         hipStream_t stream)
{
    if (n_heads <= 0 || n <= budget) return hipSuccess;
    if (n <= kLdsKeysMax) {
        const size_t lds = (size_t)(kHistBins + n) * sizeof(uint32_t);
        static bool attr_set = false;
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute((const void*)select_kernel<true>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)((kHistBins + kLdsKeysMax) * sizeof(uint32_t)));
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        hipLaunchKernelGGL(select_kernel<true>, dim3(n_heads), dim3(kBlock), lds, stream, scores, n,
                           budget, kept);
    } else {
        const size_t lds = (size_t)kHistBins * sizeof(uint32_t);
        hipLaunchKernelGGL(select_kernel<false>, dim3(n_heads), dim3(kBlock), lds, stream, scores,
                           n, budget, kept);
    }
    return hipGetLastError();
}

}  // namespace tri
