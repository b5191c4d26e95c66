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
// which the head's keys differ (so the first histogram spreads over
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
constexpr int kBatch = 8;        // keys per thread loaded before any is used
// word 3 of a raw buffer resource on gfx9-family parts: 32-bit data format
constexpr int kBufferWord3 = 0x00020000;
// stands for every key above the candidate range once phase A has run
// (no score maps to it: +inf maps to 0xFF800000)
constexpr uint32_t kTopKey = 0xFFFFFFFFu;
constexpr int kHistBins = 1 << kMaxDigitBits;
// digit width of the register-resident selection's histogram passes
constexpr int kRegDigitBits = 12;
// keys of a head staged in LDS up to this many (4 bytes each, plus the
// 8 KB histogram, within the 160 KB LDS of a gfx950 workgroup)
constexpr int kLdsKeysMax = 36864;

// Order-preserving map of fp32 scores to uint32 keys.  Key 0 is never
// produced (it marks slots past the end of a head, below every real key).
__device__ __forceinline__ uint32_t ordered_key(float x)
{
    if (x != x) return 1u;                   // NaN below every number
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;            // -0 equals +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of ordered_key for keys of numbers (key >= 2).
__device__ __forceinline__ float key_to_float(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
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

__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += (uint32_t)__shfl_xor((int)v, o);
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
    for (int i0 = tid; i0 < n; i0 += kBlock * kBatch) {
        float x[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) x[u] = sc[min(i0 + u * kBlock, n - 1)];   // kBatch loads in flight
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = i0 + u * kBlock;
            if (i < n) {
                const uint32_t key = ordered_key(x[u]);
                if constexpr (kInLds) lds_keys[i] = key;
                kmin = min(kmin, key);
                kmax = max(kmax, key);
            }
        }
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
            for (int i0 = tid; i0 < n; i0 += kBlock * kBatch) {
                uint32_t key[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) key[u] = key_at<kInLds>(lds_keys, sc, min(i0 + u * kBlock, n - 1));
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    if (i0 + u * kBlock < n && (key[u] & pmask) == prefix)
                        atomicAdd(&hist[(key[u] >> shift) & dmask], 1u);
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

// Digit holding the rem-th largest counted key, found by the whole
// workgroup: thread t owns a run of `per` bins counted from the top (thread 0
// the highest), the run sums are scanned within each wave and across the
// waves' totals, and the one thread whose run crosses rem walks its bins.
// Writes the digit, the count in higher bins and the count in the digit's
// bin; the caller's barrier publishes them.  Requires rem <= the number of
// counted keys.
template <int NT>
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t nbins, uint32_t rem,
                                           int tid, int lane, int wave, uint32_t* s_run,
                                           uint32_t* s_digit, uint32_t* s_above,
                                           uint32_t* s_inbin)
{
    const uint32_t per = nbins > (uint32_t)NT ? nbins / (uint32_t)NT : 1u;
    const uint32_t first = (uint32_t)tid * per;
    const bool active = first < nbins;
    uint32_t sum = 0u;
    if (active)
        for (uint32_t t = 0; t < per; ++t) sum += hist[nbins - 1u - first - t];
    uint32_t incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = (uint32_t)__shfl_up((int)incl, o);
        if (lane >= o) incl += v;
    }
    if (lane == 63) s_run[wave] = incl;
    __syncthreads();
    for (int x = 0; x < wave; ++x) incl += s_run[x];
    const uint32_t excl = incl - sum;
    if (active && excl < rem && rem <= incl) {
        uint32_t acc = excl;
        for (uint32_t t = 0; t < per; ++t) {
            const uint32_t b = nbins - 1u - first - t;
            const uint32_t h = hist[b];
            if (acc + h >= rem) {
                *s_digit = b;
                *s_above = acc;
                *s_inbin = h;
                break;
            }
            acc += h;
        }
    }
}

// Sorts one value per lane of a wave in descending order (bitonic network).
__device__ __forceinline__ uint32_t wave_sort_desc(uint32_t v, int lane)
{
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint32_t p = (uint32_t)__shfl_xor((int)v, j);
            const bool first = (lane & k) == 0;        // block sorted descending
            const bool lower = (lane & j) == 0;        // lower lane of the pair
            v = (first == lower) ? max(v, p) : min(v, p);
        }
    }
    return v;
}

// Register-resident variant for heads of at most NT * KPT keys (NT threads):
// lane l of wave w holds the keys of slots w*64*KPT + c*64 + l, c < KPT,
// which is the order the output sweep consumes them in.  LDS holds only the
// histogram and a short candidate list.
//
// Radix select on offsets: all live keys lie in [base, base + 2^wb); each
// pass histograms (key - base) >> (wb - 12) into 4096 bins, so the bins
// always span the populated key range (the keys of concentrated scores sit
// in a narrow range, often straddling a power of two, and a bit-aligned
// digit would pile them into a few bins).  Keys above the chosen bin are
// kept, keys below it evicted.  Once at most 64 candidates are left, one
// wave sorts them in registers and reads off the threshold.  The result is
// either "keep every key >= Tlo" (exactly B keys) or, when equal keys
// straddle the threshold, "keep keys > T and the first need_eq keys == T in
// slot order".
template <int KPT, int NT>
__global__ __launch_bounds__(NT) void select_reg_kernel(const float* __restrict__ scores,
                                                        int n, int budget,
                                                        int32_t* __restrict__ kept)
{
    constexpr int kW = NT / 64;
    __shared__ uint32_t hist[1 << kRegDigitBits];
    __shared__ uint32_t s_cand[64];
    __shared__ uint32_t s_wa[kW], s_wb[kW], s_run[kW];
    __shared__ uint32_t s_digit, s_above, s_inbin, s_ncand;
    __shared__ uint32_t s_T, s_need, s_tie;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const float* sc = scores + (size_t)blockIdx.x * (size_t)n;
    int32_t* out = kept + (size_t)blockIdx.x * (size_t)budget;
    const int seg0 = wave * (64 * KPT) + lane;     // slot of key[0]

    // Slots past the head's end hold key 0, below every real key (ordered_key
    // never returns 0): with budget < n they are never kept.
    uint32_t key[KPT];
    {
        // bounds-checked buffer loads: one offset register for all KPT loads
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)sc, 0, n * 4, kBufferWord3);
        uint32_t x[KPT];
#pragma unroll
        for (int c = 0; c < KPT; ++c)
            x[c] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (seg0 + 64 * c) * 4, 0, 0);
#pragma unroll
        for (int c = 0; c < KPT; ++c)
            key[c] = seg0 + 64 * c < n ? ordered_key(__uint_as_float(x[c])) : 0u;
    }

    uint32_t kmin, kmax;
    {
        uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
        for (int c = 0; c < KPT; ++c) {
            lo = min(lo, key[c] ? key[c] : 0xFFFFFFFFu);
            hi = max(hi, key[c]);
        }
        lo = wave_min(lo);
        hi = wave_max(hi);
        if (lane == 0) {
            s_wa[wave] = lo;
            s_wb[wave] = hi;
        }
        __syncthreads();
        kmin = s_wa[0];
        kmax = s_wb[0];
        for (int x = 1; x < kW; ++x) {
            kmin = min(kmin, s_wa[x]);
            kmax = max(kmax, s_wb[x]);
        }
    }

    // Decision: tie = false -> keep key >= T (exactly budget keys);
    //           tie = true  -> keep key > T, then the first need_eq keys == T.
    uint32_t T, need_eq;
    bool tie;
    if (kmin == kmax) {
        T = kmin;
        need_eq = (uint32_t)budget;
        tie = true;
    } else {
        uint32_t base = kmin;
        int wb = 32 - __clz((int)(kmax - kmin));       // live keys: [base, base + 2^wb)
        uint32_t rem = (uint32_t)budget;
        for (;;) {
            const int nb = min(kRegDigitBits, wb);
            const int sh = wb - nb;
            const uint32_t nbins = 1u << nb;
            const uint32_t span = wb >= 32 ? 0xFFFFFFFFu : (1u << wb) - 1u;
            __syncthreads();                            // previous readers of hist / s_*
            for (uint32_t b = tid; b < nbins; b += NT) hist[b] = 0u;
            if (tid == 0) s_ncand = 0u;
            __syncthreads();
            // padding keys (0) are skipped; the comparison value is opaque so
            // the compiler recomputes the KPT masks per pass instead of
            // keeping them live in scalar registers across passes
            uint32_t pad = 0u;
            asm volatile("" : "+v"(pad));
#pragma unroll
            for (int c = 0; c < KPT; ++c) {
                const uint32_t off = key[c] - base;
                if (off <= span && key[c] != pad) atomicAdd(&hist[off >> sh], 1u);
            }
            __syncthreads();
            find_digit<NT>(hist, nbins, rem, tid, lane, wave, s_run, &s_digit, &s_above, &s_inbin);
            __syncthreads();
            const uint32_t d = s_digit & (nbins - 1u);
            const uint32_t in_bin = s_inbin;
            rem -= s_above;
            base += d << sh;
            wb = sh;
            if (rem == in_bin) {            // the whole bin is kept
                T = base;
                need_eq = 0u;
                tie = false;
                break;
            }
            if (wb == 0) {                  // the bin is one key value: equal keys straddle
                T = base;
                need_eq = rem;
                tie = true;
                break;
            }
            if (in_bin <= 64u) {
                // stage the few candidates and let one wave sort them
                const uint32_t cspan = (1u << wb) - 1u;
#pragma unroll
                for (int c = 0; c < KPT; ++c) {
                    const uint32_t off = key[c] - base;
                    if (off <= cspan && key[c] != pad) {
                        const uint32_t at = atomicAdd(&s_ncand, 1u);
                        if (at < 64u) s_cand[at] = key[c];
                    }
                }
                __syncthreads();
                if (wave == 0) {
                    const uint32_t v = wave_sort_desc((uint32_t)lane < in_bin ? s_cand[lane] : 0u, lane);
                    const uint32_t t = (uint32_t)__shfl((int)v, (int)rem - 1);
                    const uint32_t g = (uint32_t)__popcll(__ballot(v > t));
                    const uint32_t e = (uint32_t)__popcll(__ballot(v == t));
                    if (lane == 0) {
                        s_T = t;
                        s_need = rem - g;
                        s_tie = (rem - g) != e;
                    }
                }
                __syncthreads();
                T = s_T;
                need_eq = s_need;
                tie = s_tie != 0u;
                break;
            }
        }
    }

    // ---- output sweeps
    // an opaque copy of T keeps the compiler from carrying the counting
    // sweep's comparison masks over into the writing sweep
    uint32_t T2 = T;
    asm volatile("" : "+v"(T2));
    const unsigned long long below = (1ull << lane) - 1ull;
    if (!tie) {
        uint32_t cnt = 0u;
#pragma unroll
        for (int c = 0; c < KPT; ++c) cnt += key[c] >= T ? 1u : 0u;
        cnt = wave_sum(cnt);
        __syncthreads();
        if (lane == 0) s_wa[wave] = cnt;
        __syncthreads();
        uint32_t at0 = 0u;
        for (int x = 0; x < wave; ++x) at0 += s_wa[x];
#pragma unroll
        for (int c = 0; c < KPT; ++c) {
            const bool keep = key[c] >= T2;
            const unsigned long long m = __ballot(keep);
            const uint32_t at = at0 + (uint32_t)__popcll(m & below);
            if (keep && at < (uint32_t)budget) out[at] = seg0 + 64 * c;
            at0 += (uint32_t)__popcll(m);
        }
    } else {
        uint32_t cgt = 0u, ceq = 0u;
#pragma unroll
        for (int c = 0; c < KPT; ++c) {
            cgt += key[c] > T ? 1u : 0u;
            ceq += key[c] == T ? 1u : 0u;
        }
        cgt = wave_sum(cgt);
        ceq = wave_sum(ceq);
        __syncthreads();
        if (lane == 0) {
            s_wa[wave] = cgt;
            s_wb[wave] = ceq;
        }
        __syncthreads();
        uint32_t gt_before = 0u, eq_before = 0u;
        for (int x = 0; x < wave; ++x) {
            gt_before += s_wa[x];
            eq_before += s_wb[x];
        }
#pragma unroll
        for (int c = 0; c < KPT; ++c) {
            const bool gt = key[c] > T2;
            const bool eq = key[c] == T2;
            const unsigned long long mgt = __ballot(gt);
            const unsigned long long meq = __ballot(eq);
            const uint32_t my_gt = gt_before + (uint32_t)__popcll(mgt & below);
            const uint32_t my_eq = eq_before + (uint32_t)__popcll(meq & below);
            const uint32_t at = my_gt + min(my_eq, need_eq);
            if ((gt || (eq && my_eq < need_eq)) && at < (uint32_t)budget) out[at] = seg0 + 64 * c;
            gt_before += (uint32_t)__popcll(mgt);
            eq_before += (uint32_t)__popcll(meq);
        }
    }
}

}  // namespace

hipError_t launch_select(const float* scores, int n, int n_heads, int budget, int32_t* kept,
                         hipStream_t stream)
{
    if (n_heads <= 0 || n <= budget) return hipSuccess;
    if (n <= kBlock * 8) {
        hipLaunchKernelGGL((select_reg_kernel<8, kBlock>), dim3(n_heads), dim3(kBlock), 0, stream,
                           scores, n, budget, kept);
    } else if (n <= kBlock * 16) {
        hipLaunchKernelGGL((select_reg_kernel<16, kBlock>), dim3(n_heads), dim3(kBlock), 0, stream,
                           scores, n, budget, kept);
    } else if (n <= kBlock * 32) {
        hipLaunchKernelGGL((select_reg_kernel<32, kBlock>), dim3(n_heads), dim3(kBlock), 0, stream,
                           scores, n, budget, kept);
    } else if (n <= kLdsKeysMax) {
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
