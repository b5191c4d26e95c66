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
__global__ __launch_bounds__(kBlock) void select_kernel(const float* __restrict__ scores,
                                                        int stride, int budget,
                                                        int32_t* __restrict__ kept,
                                                        int kept_stride,
                                                        const int32_t* __restrict__ head_len)
{
    extern __shared__ uint32_t smem[];
    uint32_t* hist = smem;                             // [kHistBins]
    uint32_t* lds_keys = smem + kHistBins;             // [n] when kInLds
    __shared__ uint32_t s_wmin[kWaves], s_wmax[kWaves];
    __shared__ uint32_t s_wgt[kWaves], s_weq[kWaves];
    __shared__ uint32_t s_digit, s_above;

    // keys of this head: all `stride`, or its own length (ragged heads); a
    // head with at most `budget` keys keeps them all and gets no list
    const int n = head_len ? max(0, min(head_len[blockIdx.x], stride)) : stride;
    if (n <= budget) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const float* sc = scores + (size_t)blockIdx.x * (size_t)stride;
    int32_t* out = kept + (size_t)blockIdx.x * (size_t)kept_stride;

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
                                                        int stride, int budget,
                                                        int32_t* __restrict__ kept,
                                                        int kept_stride,
                                                        const int32_t* __restrict__ head_len)
{
    constexpr int kW = NT / 64;
    __shared__ uint32_t hist[1 << kRegDigitBits];
    __shared__ uint32_t s_cand[64];
    __shared__ uint32_t s_wa[kW], s_wb[kW], s_run[kW];
    __shared__ uint32_t s_digit, s_above, s_inbin, s_ncand;
    __shared__ uint32_t s_T, s_need, s_tie;

    // keys of this head: all `stride`, or its own length (ragged heads); a
    // head with at most `budget` keys keeps them all and gets no list
    const int n = head_len ? max(0, min(head_len[blockIdx.x], stride)) : stride;
    if (n <= budget) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const float* sc = scores + (size_t)blockIdx.x * (size_t)stride;
    int32_t* out = kept + (size_t)blockIdx.x * (size_t)kept_stride;
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


// ---------------------------------------------------------------------------
// Head-specific budgets: the n_kv heads of a layer share total = budget *
// n_kv slots.  Every head reserves its `floor` best keys (found per head by
// the selection above, run with budget = floor); the remaining slots go to
// the best remaining keys of the layer, ties to the lower head and then the
// lower slot.
//
// A head's reserved set is exactly "key > Th, or key == Th and slot <= Sh",
// where Th is the smallest key on its reserved list and Sh the largest
// reserved slot holding Th: the list holds every key above its smallest key
// and the lowest slots among the keys equal to it.  So the reserved set is
// a pointwise test and needs no flag array.
//
// shared_layer_kernel (one workgroup per layer) takes the firing decision,
// derives (Th, Sh) per head, then runs the offset radix select of the
// register-resident kernel over the layer's unreserved keys, re-reading
// them from memory each pass, for rem = total - (reserved keys) slots.  When
// equal keys straddle the threshold it counts them per head and hands them
// out in head order.  shared_write_kernel (one workgroup per head) then
// writes each head's kept list in slot order and its count.

constexpr int kMaxSharedHeads = 128;

__device__ __forceinline__ int wave_max_i(int v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

// Calls f(key, unreserved) for every key of the layer's heads (slot
// i < s_n[h]), kBatch loads in flight per thread; head h's reserved set is
// key > s_th[h], or key == s_th[h] and i <= s_sh[h].
template <typename F>
__device__ __forceinline__ void for_layer_keys(const float* sc, int stride, int n_kv,
                                               const int* s_n, const uint32_t* s_th,
                                               const int* s_sh, int tid, F&& f)
{
    for (int h = 0; h < n_kv; ++h) {
        const int n = s_n[h];
        const uint32_t th = s_th[h];
        const int sh = s_sh[h];
        const float* hs = sc + (size_t)h * (size_t)stride;
        for (int i0 = tid; i0 < n; i0 += kBlock * kBatch) {
            float x[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) x[u] = hs[min(i0 + u * kBlock, n - 1)];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int i = i0 + u * kBlock;
                const uint32_t key = ordered_key(x[u]);
                if (i < n) f(key, !(key > th || (key == th && i <= sh)));
            }
        }
    }
}

__global__ __launch_bounds__(kBlock) void shared_layer_kernel(
    const float* __restrict__ scores, int stride, int n_kv, const int32_t* __restrict__ head_len,
    int total, int floor_, int window, const int32_t* __restrict__ kept,
    uint4* __restrict__ ws_head, uint4* __restrict__ ws_layer)
{
    __shared__ uint32_t hist[1 << kRegDigitBits];
    __shared__ int s_n[kMaxSharedHeads];
    __shared__ uint32_t s_Th[kMaxSharedHeads];
    __shared__ int s_Sh[kMaxSharedHeads];
    __shared__ uint32_t s_eq[kMaxSharedHeads];
    __shared__ uint32_t s_wa[kWaves], s_wb[kWaves], s_run[kWaves];
    __shared__ uint32_t s_digit, s_above, s_inbin;

    const int layer = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const float* sc = scores + (size_t)layer * (size_t)n_kv * (size_t)stride;
    const int32_t* lists = kept + (size_t)layer * (size_t)n_kv * (size_t)total;
    uint4* wh = ws_head + (size_t)layer * (size_t)n_kv;

    for (int h = tid; h < n_kv; h += kBlock) {
        s_n[h] = head_len ? max(0, min(head_len[(size_t)layer * n_kv + h], stride)) : stride;
        s_eq[h] = 0u;
    }
    __syncthreads();
    int64_t all = 0;
    for (int h = 0; h < n_kv; ++h) all += s_n[h];
    if (all <= (int64_t)total + (int64_t)n_kv * window) {      // the layer keeps every key
        if (tid == 0) ws_layer[layer] = make_uint4(0u, 0u, 0u, 0u);
        return;
    }

    // reserved sets: (Th, Sh) per head from its reserved list
    for (int h = wave; h < n_kv; h += kWaves) {
        const int n = s_n[h];
        uint32_t th;
        int sh;
        if (floor_ == 0) {
            th = kTopKey;                 // no key is above it: nothing reserved
            sh = -1;
        } else if (n <= floor_) {
            th = 0u;                      // every real key is above it: all reserved
            sh = -1;
        } else {
            const int32_t* l = lists + (size_t)h * (size_t)total;
            const float* hs = sc + (size_t)h * (size_t)stride;
            uint32_t mn = 0xFFFFFFFFu;
            for (int j = lane; j < floor_; j += 64)
                mn = min(mn, ordered_key(hs[min(max(l[j], 0), n - 1)]));
            mn = wave_min(mn);
            int mx = -1;
            for (int j = lane; j < floor_; j += 64) {
                const int slot = min(max(l[j], 0), n - 1);
                if (ordered_key(hs[slot]) == mn) mx = max(mx, slot);
            }
            th = mn;
            sh = wave_max_i(mx);
        }
        if (lane == 0) {
            s_Th[h] = th;
            s_Sh[h] = sh;
        }
    }
    __syncthreads();
    int64_t reserved = 0;
    for (int h = 0; h < n_kv; ++h) reserved += min(s_n[h], floor_);
    uint32_t rem = (uint32_t)((int64_t)total - reserved);   // floor * n_kv <= total

    uint32_t T = kTopKey, need_eq = 0u;
    bool tie = false;
    if (rem > 0u) {
        // key range of the unreserved keys (more than rem of them: the layer fires)
        uint32_t lo = 0xFFFFFFFFu, hi = 0u;
        for_layer_keys(sc, stride, n_kv, s_n, s_Th, s_Sh, tid, [&](uint32_t key, bool unres) {
            if (unres) {
                lo = min(lo, key);
                hi = max(hi, key);
            }
        });
        lo = wave_min(lo);
        hi = wave_max(hi);
        if (lane == 0) {
            s_wa[wave] = lo;
            s_wb[wave] = hi;
        }
        __syncthreads();
        uint32_t kmin = s_wa[0], kmax = s_wb[0];
        for (int x = 1; x < kWaves; ++x) {
            kmin = min(kmin, s_wa[x]);
            kmax = max(kmax, s_wb[x]);
        }
        if (kmin == kmax) {
            T = kmin;
            need_eq = rem;
            tie = true;
        } else {
            uint32_t base = kmin;
            int wb = 32 - __clz((int)(kmax - kmin));    // live keys: [base, base + 2^wb)
            for (;;) {
                const int nb = min(kRegDigitBits, wb);
                const int shift = wb - nb;
                const uint32_t nbins = 1u << nb;
                const uint32_t span = wb >= 32 ? 0xFFFFFFFFu : (1u << wb) - 1u;
                __syncthreads();                         // previous readers of hist / s_*
                for (uint32_t b = tid; b < nbins; b += kBlock) hist[b] = 0u;
                __syncthreads();
                for_layer_keys(sc, stride, n_kv, s_n, s_Th, s_Sh, tid, [&](uint32_t key, bool unres) {
                    const uint32_t off = key - base;
                    if (off <= span && unres) atomicAdd(&hist[off >> shift], 1u);
                });
                __syncthreads();
                find_digit<kBlock>(hist, nbins, rem, tid, lane, wave, s_run, &s_digit, &s_above,
                                   &s_inbin);
                __syncthreads();
                const uint32_t d = s_digit & (nbins - 1u);
                const uint32_t in_bin = s_inbin;
                rem -= s_above;
                base += d << shift;
                wb = shift;
                if (rem == in_bin) {                     // the whole bin is kept
                    T = base;
                    tie = false;
                    break;
                }
                if (wb == 0) {                           // one key value straddles
                    T = base;
                    need_eq = rem;
                    tie = true;
                    break;
                }
            }
        }
        if (tie) {
            // equal keys per head, handed out in head order
            for (int h = 0; h < n_kv; ++h) {
                const int n = s_n[h];
                const uint32_t th = s_Th[h];
                const int sh = s_Sh[h];
                const float* hs = sc + (size_t)h * (size_t)stride;
                uint32_t c = 0u;
                for (int i = tid; i < n; i += kBlock) {
                    const uint32_t key = ordered_key(hs[i]);
                    c += (key == T && !(key > th || (key == th && i <= sh))) ? 1u : 0u;
                }
                c = wave_sum(c);
                if (lane == 0 && c) atomicAdd(&s_eq[h], c);
            }
            __syncthreads();
        }
    }
    if (tid == 0) {
        uint32_t left = need_eq;
        for (int h = 0; h < n_kv; ++h) {
            const uint32_t take = tie ? min(s_eq[h], left) : 0u;
            left -= take;
            wh[h] = make_uint4(s_Th[h], (uint32_t)s_Sh[h], take, 0u);
        }
        ws_layer[layer] = make_uint4(T, tie ? 1u : 0u, 1u, 0u);
    }
}

// One workgroup per head: the kept list of the head in slot order and its
// count (-1 when the layer does not fire).  Wave w owns slots
// [w*seg, (w+1)*seg); a counting sweep gives every wave its offset.
__global__ __launch_bounds__(kBlock) void shared_write_kernel(
    const float* __restrict__ scores, int stride, int n_kv, const int32_t* __restrict__ head_len,
    int total, const uint4* __restrict__ ws_head, const uint4* __restrict__ ws_layer,
    int32_t* __restrict__ kept, int32_t* __restrict__ kept_count)
{
    __shared__ uint32_t s_wgt[kWaves], s_weq[kWaves];
    const int lh = blockIdx.x;
    const int layer = lh / n_kv;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint4 lw = ws_layer[layer];
    if (lw.z == 0u) {
        if (tid == 0) kept_count[lh] = -1;
        return;
    }
    const uint4 hw = ws_head[lh];
    const uint32_t th = hw.x;
    const int sh = (int)hw.y;
    const uint32_t take = hw.z;
    const uint32_t T = lw.x;
    const bool tie = lw.y != 0u;
    const int n = head_len ? max(0, min(head_len[lh], stride)) : stride;
    const float* sc = scores + (size_t)lh * (size_t)stride;
    int32_t* out = kept + (size_t)lh * (size_t)total;

    // gt: kept outright (reserved, or above the layer threshold);
    // eq: unreserved and equal to T when equal keys straddle it
    auto classify = [&](int i, bool& gt, bool& eq) {
        const uint32_t key = i < n ? ordered_key(sc[i]) : 0u;
        const bool res = i < n && (key > th || (key == th && i <= sh));
        gt = res || (i < n && (tie ? key > T : key >= T));
        eq = !res && tie && i < n && key == T;
    };
    const int seg = ((n + kWaves - 1) / kWaves + 63) & ~63;
    const int s0 = wave * seg;
    const int s1 = min(n, s0 + seg);
    uint32_t cgt = 0u, ceq = 0u;
    for (int i0 = s0; i0 < s1; i0 += 64) {
        bool gt, eq;
        classify(i0 + lane < s1 ? i0 + lane : n, gt, eq);
        cgt += (uint32_t)__popcll(__ballot(gt));
        ceq += (uint32_t)__popcll(__ballot(eq));
    }
    if (lane == 0) {
        s_wgt[wave] = cgt;
        s_weq[wave] = ceq;
    }
    __syncthreads();
    uint32_t gt_before = 0u, eq_before = 0u, gt_all = 0u, eq_all = 0u;
    for (int x = 0; x < kWaves; ++x) {
        if (x < wave) {
            gt_before += s_wgt[x];
            eq_before += s_weq[x];
        }
        gt_all += s_wgt[x];
        eq_all += s_weq[x];
    }
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int i0 = s0; i0 < s1; i0 += 64) {
        const int i = i0 + lane;
        bool gt, eq;
        classify(i < s1 ? i : n, gt, eq);
        const unsigned long long mgt = __ballot(gt);
        const unsigned long long meq = __ballot(eq);
        const uint32_t my_gt = gt_before + (uint32_t)__popcll(mgt & below);
        const uint32_t my_eq = eq_before + (uint32_t)__popcll(meq & below);
        const uint32_t at = my_gt + min(my_eq, take);
        if ((gt || (eq && my_eq < take)) && at < (uint32_t)total) out[at] = i;
        gt_before += (uint32_t)__popcll(mgt);
        eq_before += (uint32_t)__popcll(meq);
    }
    if (tid == 0) kept_count[lh] = (int32_t)min(gt_all + min(eq_all, take), (uint32_t)total);
}

}  // namespace

hipError_t launch_select(const float* scores, int n, int n_heads, int budget, int32_t* kept,
                         int kept_stride, const int32_t* head_len, hipStream_t stream)
{
    if (n_heads <= 0 || n <= budget) return hipSuccess;
    if (n <= kBlock * 8) {
        hipLaunchKernelGGL((select_reg_kernel<8, kBlock>), dim3(n_heads), dim3(kBlock), 0, stream,
                           scores, n, budget, kept, kept_stride, head_len);
    } else if (n <= kBlock * 16) {
        hipLaunchKernelGGL((select_reg_kernel<16, kBlock>), dim3(n_heads), dim3(kBlock), 0, stream,
                           scores, n, budget, kept, kept_stride, head_len);
    } else if (n <= kBlock * 32) {
        hipLaunchKernelGGL((select_reg_kernel<32, kBlock>), dim3(n_heads), dim3(kBlock), 0, stream,
                           scores, n, budget, kept, kept_stride, head_len);
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
                           budget, kept, kept_stride, head_len);
    } else {
        const size_t lds = (size_t)kHistBins * sizeof(uint32_t);
        hipLaunchKernelGGL(select_kernel<false>, dim3(n_heads), dim3(kBlock), lds, stream, scores,
                           n, budget, kept, kept_stride, head_len);
    }
    return hipGetLastError();
}


int64_t shared_workspace_bytes(int64_t n_seq, int64_t n_layers, int64_t n_kv)
{
    auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    return up(n_seq * n_layers * n_kv * 16) + up(n_seq * n_layers * 16);
}

hipError_t launch_select_shared(const float* scores, int stride, int n_layers, int n_kv,
                                const int32_t* head_len, int budget, int floor_, int window,
                                int32_t* kept, int32_t* kept_count, void* ws_head, void* ws_layer,
                                hipStream_t stream)
{
    if (n_layers <= 0 || n_kv <= 0) return hipSuccess;
    if (n_kv > kMaxSharedHeads) return hipErrorInvalidValue;
    const int64_t total = (int64_t)budget * n_kv;
    if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (floor_ > 0 && stride > floor_) {
        // each head's reserved list, into the head's kept row (stride total)
        hipError_t e = launch_select(scores, stride, n_layers * n_kv, floor_, kept, (int)total,
                                     head_len, stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(shared_layer_kernel, dim3(n_layers), dim3(kBlock), 0, stream, scores,
                       stride, n_kv, head_len, (int)total, floor_, window, kept,
                       static_cast<uint4*>(ws_head), static_cast<uint4*>(ws_layer));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(shared_write_kernel, dim3(n_layers * n_kv), dim3(kBlock), 0, stream,
                       scores, stride, n_kv, head_len, (int)total,
                       static_cast<const uint4*>(ws_head), static_cast<const uint4*>(ws_layer),
                       kept, kept_count);
    return hipGetLastError();
}

}  // namespace tri
