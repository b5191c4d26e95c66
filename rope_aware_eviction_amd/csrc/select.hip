// Per-head top-B selection with a deterministic tie-break.
//
// Source: romaanj.github.io "TriAttention" review, section "Method" (prune
// back to the budget) and figure 4 caption (the prune retains the
// highest-scoring keys); dimensionstp.github.io review, section 3-2 item 5 (keep the
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
#include <algorithm>
#include <vector>

#include "gqa_stats.h"
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
// a per-head histogram row in the shared-budget workspace: the 4096 bins,
// then the sums of their 64 groups of 64 consecutive bins
constexpr int kHistRow = (1 << kRegDigitBits) + 64;
// keys of a head staged in LDS up to this many (4 bytes each, plus the
// 8 KB histogram, within the 160 KB LDS of a gfx950 workgroup)
constexpr int kLdsKeysMax = 36864;
// sequences per launch of the batched selection (the table travels in the
// kernel arguments: 24 bytes per sequence)
constexpr int kSelectBatch = 64;

// Order-preserving map of fp32 scores to uint32 keys.  Key 0 is never
// produced (it marks slots past the end of a head, below every real key).
__device__ __forceinline__ uint32_t ordered_key(float x)
{
    if (x != x) return 1u;                   // NaN below every number
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

// Wave-wide reductions and scan (every lane active).  DPP moves inside each
// 16-lane row (quad permutations, then the half-row and row mirrors pair
// every lane with one of the other half), then the four row results are
// combined from scalar registers: no LDS round trip.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

__device__ __forceinline__ uint32_t lane_u(uint32_t x, int l)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)x, l);
}

template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op)
{
    v = op(v, dpp_u<0xB1>(v));                  // quad_perm [1,0,3,2]
    v = op(v, dpp_u<0x4E>(v));                  // quad_perm [2,3,0,1]
    v = op(v, dpp_u<0x141>(v));                 // row_half_mirror
    v = op(v, dpp_u<0x140>(v));                 // row_mirror: the row's result in every lane
    return op(op(lane_u(v, 0), lane_u(v, 16)), op(lane_u(v, 32), lane_u(v, 48)));
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v)
{
    return wave_reduce(v, [](uint32_t a, uint32_t b) { return min(a, b); });
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
    return wave_reduce(v, [](uint32_t a, uint32_t b) { return a + b; });
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v)
{
    return wave_reduce(v, [](uint32_t a, uint32_t b) { return max(a, b); });
}

// The 64 group sums of an LDS histogram of nbins <= 4096 bins, out[g] =
// bins [64g, 64g + 64) below nbins.  Every thread of a 1024-thread workgroup
// calls it once the histogram is complete: thread t adds bins 4t..4t+3, and
// the 16 threads of a DPP row add their sums.
__device__ __forceinline__ void write_group_sums(const uint32_t* h, uint32_t nbins, uint32_t* out,
                                                 int tid)
{
    uint32_t p = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t b = 4u * (uint32_t)tid + (uint32_t)j;
        p += b < nbins ? h[b] : 0u;
    }
    p += dpp_u<0xB1>(p);
    p += dpp_u<0x4E>(p);
    p += dpp_u<0x141>(p);
    p += dpp_u<0x140>(p);
    if ((tid & 15) == 0) out[tid >> 4] = p;
}

// Inclusive prefix sum over the lanes of a wave: shift-and-add inside each
// row (row_shr fills the lanes it shifts past with 0), then the totals of
// the rows below.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane)
{
    x += dpp_u<0x111>(x);                       // row_shr:1
    x += dpp_u<0x112>(x);                       // row_shr:2
    x += dpp_u<0x114>(x);                       // row_shr:4
    x += dpp_u<0x118>(x);                       // row_shr:8
    const uint32_t r0 = lane_u(x, 15), r1 = lane_u(x, 31), r2 = lane_u(x, 47);
    const int row = lane >> 4;
    return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// The selection of one head of n > budget keys at sc into out, with
// kHistBins words of LDS at smem for the histogram (kInLds: then n more for
// the staged keys).  Every thread of the workgroup calls it.
template <bool kInLds>
__device__ __forceinline__ void select_lds_head(uint32_t* smem, const float* __restrict__ sc, int n,
                                                int budget, int32_t* __restrict__ out)
{
    uint32_t* hist = smem;                             // [kHistBins]
    uint32_t* lds_keys = smem + kHistBins;             // [n] when kInLds
    __shared__ uint32_t s_wmin[kWaves], s_wmax[kWaves];
    __shared__ uint32_t s_wgt[kWaves], s_weq[kWaves];
    __shared__ uint32_t s_digit, s_above;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

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
                const uint32_t incl = wave_incl_scan(sum, lane);
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

template <bool kInLds>
__global__ __launch_bounds__(kBlock) void select_kernel(const float* __restrict__ scores,
                                                        int stride, int budget,
                                                        int32_t* __restrict__ kept,
                                                        int kept_stride,
                                                        const int32_t* __restrict__ head_len)
{
    extern __shared__ uint32_t smem[];
    // keys of this head: all `stride`, or its own length (ragged heads); a
    // head with at most `budget` keys keeps them all and gets no list
    const int n = head_len ? max(0, min(head_len[blockIdx.x], stride)) : stride;
    if (n <= budget) return;
    select_lds_head<kInLds>(smem, scores + (size_t)blockIdx.x * (size_t)stride, n, budget,
                            kept + (size_t)blockIdx.x * (size_t)kept_stride);
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
    uint32_t incl = wave_incl_scan(sum, lane);
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
// wave ranks them (each counts the candidates above it and equal to it)
// and reads off the threshold.  The result is either "keep every key >= T"
// (exactly B keys) or, when equal keys straddle the threshold, "keep keys
// > T and the first need_eq keys == T in slot order".
//
// RESERVE (head-specific budgets, budget = the per-head floor): instead of
// the kept list, writes rec[head] = {Th, Sh, min, max}: the kept set as the
// pointwise test "key > Th, or key == Th and slot <= Sh", and the range of
// the keys outside it (min > max when there are none); and hist_out[head],
// the histogram of the keys outside it by their top 12 bits (the first
// radix digit of the layer-wide selection, whose binning needs no range).
// LDS of one register-resident selection.
template <int NT>
struct RegLds {
    uint32_t hist[1 << kRegDigitBits];
    uint32_t cand[64];
    uint32_t wa[NT / 64], wb[NT / 64], run[NT / 64];
    uint32_t digit, above, inbin, ncand, T, need, tie;
};

// The keys a register-resident selection ranks: key[c] of lane l of wave w
// is the order-preserving key of slot w * 64 * KPT + 64 * c + l, or 0 (below
// every real key) for slots past the head's n keys.
//
// ScoreKeys: the fp32 scores of the head.
struct ScoreKeys {
    const float* sc;
    template <int KPT>
    __device__ __forceinline__ void load(uint32_t (&key)[KPT], int seg0, int n) const
    {
        // bounds-checked buffer loads: one offset register for all KPT loads
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)sc, 0, n * 4, kBufferWord3);
        uint32_t x[KPT];
#pragma unroll
        for (int c = 0; c < KPT; ++c)
            x[c] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (seg0 + 64 * c) * 4, 0, 0);
        // a mask rather than a select, so the key is computed with no branch
#pragma unroll
        for (int c = 0; c < KPT; ++c)
            key[c] = ordered_key(__uint_as_float(x[c])) & (0u - (seg0 + 64 * c < n ? 1u : 0u));
    }
};

// GqaKeys<G>: the GQA score of the head formed on the fly from its G raw
// per-query-head scores [n][G] and their statistics (mean, deviation): the
// largest z_g = (s_g - mean_g) / deviation_g over the finite s_g (z_g = 0
// for a flat row, deviation 0), in fp64 and rounded once to fp32 in the same
// operations as the GQA normalize kernel, so the key equals the one of the
// score that kernel writes; NaN when no s_g is finite.
template <int G>
struct GqaKeys {
    const float* raw;          // the head's raw scores, [n][G]
    const double2* stats;      // the head's [G] (mean, deviation)
    template <int KPT>
    __device__ __forceinline__ void load(uint32_t (&key)[KPT], int seg0, int n) const
    {
        double mean[G], inv[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const double2 st = stats[g];
            mean[g] = st.x;
            inv[g] = st.y > 0.0 ? 1.0 / st.y : 0.0;
        }
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)raw, 0, n * G * 4, kBufferWord3);
        // Rows in flight per lane.  With G <= 4 each group's loads are pinned
        // ahead of its arithmetic by scheduling barriers (with more query
        // heads they would push the kernel into spills).  Left alone, the
        // compiler merges a row's G loads into one and interleaves them with
        // the fp64 work, keeping only 1-4 rows in flight, so a head alone on
        // a compute unit (the second round of a launch with more heads than
        // compute units) paid about ten memory round trips for its 32 rows
        // per lane.  Measured on the 288-head GQA cache (G = 4): 66.6 us
        // against 69.8 us; 8 rows per group 67.0 us, two groups of 8 in turn
        // 68.0 us.
        constexpr int kRows = G <= 4 ? (KPT % 16 == 0 ? 16 : 8) : 4;
        static_assert(KPT % kRows == 0, "whole groups of rows");
#pragma unroll
        for (int c0 = 0; c0 < KPT; c0 += kRows) {
            uint32_t x[kRows][G];
#pragma unroll
            for (int c = 0; c < kRows; ++c)
#pragma unroll
                for (int g = 0; g < G; ++g)
                    x[c][g] = __builtin_amdgcn_raw_buffer_load_b32(
                        rsrc, ((seg0 + 64 * (c0 + c)) * G + g) * 4, 0, 0);
            if constexpr (G <= 4) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int c = 0; c < kRows; ++c) {
                double best = __longlong_as_double(0x7FF8000000000000ll);   // NaN
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const double sg = (double)__uint_as_float(x[c][g]);
                    if (isfinite(sg)) {
                        const double z = (sg - mean[g]) * inv[g];
                        if (isnan(best) || z > best) best = z;
                    }
                }
                key[c0 + c] = ordered_key((float)best) &
                              (0u - (seg0 + 64 * (c0 + c) < n ? 1u : 0u));
            }
            if constexpr (G <= 4) __builtin_amdgcn_sched_barrier(0);
        }
    }
};

// The selection of one head of n keys (from `keys`): the kept list goes to
// out (RESERVE: the record to *rec and the histogram row to hist_row).  Every
// thread of the workgroup calls it.
template <int KPT, int NT, bool RESERVE, class Keys>
__device__ __forceinline__ void select_reg_head(RegLds<NT>& L, const Keys& keys, int n,
                                                int budget, int32_t* __restrict__ out,
                                                uint4* __restrict__ rec,
                                                uint32_t* __restrict__ hist_row)
{
    constexpr int kW = NT / 64;
    uint32_t* hist = L.hist;
    uint32_t* s_cand = L.cand;
    uint32_t* s_wa = L.wa;
    uint32_t* s_wb = L.wb;
    uint32_t* s_run = L.run;
    uint32_t& s_digit = L.digit;
    uint32_t& s_above = L.above;
    uint32_t& s_inbin = L.inbin;
    uint32_t& s_ncand = L.ncand;
    uint32_t& s_T = L.T;
    uint32_t& s_need = L.need;
    uint32_t& s_tie = L.tie;

    // a head with at most `budget` keys keeps them all and gets no list
    if (n <= budget) {
        // RESERVE: every key is reserved (Th = 0 lies below every real key)
        if constexpr (RESERVE) {
            for (int b = threadIdx.x; b < kHistRow; b += NT) hist_row[b] = 0u;
            if (threadIdx.x == 0) *rec = make_uint4(0u, 0xFFFFFFFFu, 0xFFFFFFFFu, 0u);
        }
        return;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int seg0 = wave * (64 * KPT) + lane;     // slot of key[0]

    // Slots past the head's end hold key 0, below every real key (ordered_key
    // never returns 0): with budget < n they are never kept.
    uint32_t key[KPT];
    keys.template load<KPT>(key, seg0, n);

    uint32_t kmin, kmax;
    {
        // the minimum of key - 1 skips key 0 (it wraps to the top) with no
        // comparison; the head has a real key, so adding 1 back is exact
        uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
        for (int c = 0; c < KPT; ++c) {
            lo = min(lo, key[c] - 1u);
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
        kmin += 1u;
    }

    // RESERVE: the range and the top-12-bit histogram of the keys outside
    // the reserved set "key > th, or key == th and slot <= sh"
    auto reserve_tail = [&](uint32_t th, int sh) {
        __syncthreads();                                // earlier readers of hist / s_*
        for (uint32_t b = tid; b < (1u << kRegDigitBits); b += NT) hist[b] = 0u;
        __syncthreads();
        uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
        for (int c = 0; c < KPT; ++c) {
            const uint32_t k = key[c];
            const bool res = k > th || (k == th && seg0 + 64 * c <= sh);
            const bool live = k != 0u && !res;
            lo = min(lo, live ? k : 0xFFFFFFFFu);
            hi = max(hi, live ? k : 0u);
            if (live) atomicAdd(&hist[k >> (32 - kRegDigitBits)], 1u);
        }
        lo = wave_min(lo);
        hi = wave_max(hi);
        if (lane == 0) {
            s_wa[wave] = lo;
            s_wb[wave] = hi;
        }
        __syncthreads();
        for (uint32_t b = tid; b < (1u << kRegDigitBits); b += NT) hist_row[b] = hist[b];
        static_assert(!RESERVE || NT == 1024, "group sums assume 1024 threads");
        write_group_sums(hist, 1u << kRegDigitBits, hist_row + (1 << kRegDigitBits), tid);
        if (tid == 0) {
            for (int x = 0; x < kW; ++x) {
                lo = min(lo, s_wa[x]);
                hi = max(hi, s_wb[x]);
            }
            *rec = make_uint4(th, (uint32_t)sh, lo, hi);
        }
    };

    if (RESERVE && budget == 0) {
        reserve_tail(kTopKey, -1);                      // nothing reserved
        return;
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
            // Only keys in the live range are added (padding keys, 0, never
            // are).  The adds are masked, not redirected: after the first
            // pass most keys lie outside the range, and sending them to spill
            // bins made every add a full-wave LDS operation, which was slower
            // wherever the keys in range pile into a few bins.  The padding
            // value is opaque so that the compiler recomputes the masks per
            // pass instead of keeping them live in scalar registers.
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
                // stage the few candidates and let one wave rank them
                const uint32_t cspan = (1u << wb) - 1u;
                // an opaque zero, so the padding test is made here and not
                // kept live in scalar registers from elsewhere
                uint32_t pad = 0u;
                asm volatile("" : "+v"(pad));
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
                    // each candidate counts the candidates above it and equal
                    // to it; the rem-th largest is one with gt < rem <= gt + eq
                    const uint32_t v = (uint32_t)lane < in_bin ? s_cand[lane] : 0u;
                    uint32_t gt = 0u, eq = 0u;
                    for (uint32_t j = 0; j < in_bin; ++j) {
                        const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)v, (int)j);
                        gt += o > v ? 1u : 0u;
                        eq += o == v ? 1u : 0u;
                    }
                    const bool hit = (uint32_t)lane < in_bin && gt < rem && rem <= gt + eq;
                    const int src = __ffsll((unsigned long long)__ballot(hit)) - 1;   // one exists
                    const uint32_t t = (uint32_t)__builtin_amdgcn_readlane((int)v, src);
                    const uint32_t g = (uint32_t)__builtin_amdgcn_readlane((int)gt, src);
                    const uint32_t e = (uint32_t)__builtin_amdgcn_readlane((int)eq, src);
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

    if constexpr (RESERVE) {
        // (Th, Sh): "key >= T" is "key > T - 1"; with a tie, Sh is the slot
        // of the need_eq-th key equal to T in slot order
        const unsigned long long below_r = (1ull << lane) - 1ull;
        uint32_t th = T - 1u;
        int sh = -1;
        if (tie) {
            th = T;
            uint32_t ceq = 0u;
#pragma unroll
            for (int c = 0; c < KPT; ++c) ceq += key[c] == T ? 1u : 0u;
            ceq = wave_sum(ceq);
            __syncthreads();
            if (lane == 0) s_wb[wave] = ceq;
            if (tid == 0) s_T = 0xFFFFFFFFu;           // Sh + 1 (0: no key equal to T reserved)
            __syncthreads();
            uint32_t eq_before = 0u;
            for (int x = 0; x < wave; ++x) eq_before += s_wb[x];
#pragma unroll
            for (int c = 0; c < KPT; ++c) {
                const bool eq = key[c] == T;
                const unsigned long long meq = __ballot(eq);
                const uint32_t my_eq = eq_before + (uint32_t)__popcll(meq & below_r);
                if (eq && my_eq + 1u == need_eq) s_T = (uint32_t)(seg0 + 64 * c);
                eq_before += (uint32_t)__popcll(meq);
            }
            __syncthreads();
            sh = need_eq == 0u ? -1 : (int)s_T;
        }
        reserve_tail(th, sh);
        return;
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


// One workgroup per head of one sequence: heads of `stride` keys (with
// head_len, head h has its own length up to stride); kept lists of head h
// start at kept + h * kept_stride (RESERVE: rec[h] and hist_out row h).
template <int KPT, int NT, bool RESERVE = false>
__global__ __launch_bounds__(NT) void select_reg_kernel(const float* __restrict__ scores,
                                                        int stride, int budget,
                                                        int32_t* __restrict__ kept,
                                                        int kept_stride,
                                                        const int32_t* __restrict__ head_len,
                                                        uint4* __restrict__ rec = nullptr,
                                                        uint32_t* __restrict__ hist_out = nullptr)
{
    __shared__ RegLds<NT> L;
    const int n = head_len ? max(0, min(head_len[blockIdx.x], stride)) : stride;
    select_reg_head<KPT, NT, RESERVE>(
        L, ScoreKeys{scores + (size_t)blockIdx.x * (size_t)stride}, n, budget,
        RESERVE ? nullptr : kept + (size_t)blockIdx.x * (size_t)kept_stride,
        RESERVE ? rec + blockIdx.x : nullptr,
        RESERVE ? hist_out + (size_t)blockIdx.x * kHistRow : nullptr);
}

// GQA without the normalized score array: one workgroup per head of `len`
// keys selects on the max-z keys formed from the raw per-query-head scores
// [head][len][G] (GqaKeys); wave g first forms query head g's statistics
// from the per-tile partial sums [head][tiles][G][4] exactly as the
// statistics kernel does.
template <int KPT, int G>
__global__ __launch_bounds__(kBlock) void select_gqa_kernel(const float* __restrict__ raw,
                                                            const double* __restrict__ partial,
                                                            int tiles, int len, int budget,
                                                            int32_t* __restrict__ kept,
                                                            int kept_stride)
{
    __shared__ RegLds<kBlock> L;
    __shared__ double2 s_stats[G];
    const int h = blockIdx.x;
    static_assert(G <= kBlock / 64, "one wave per query head");
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    if (wave < G) {   // wave g forms query head g's statistics
        const double2 st = gqa_query_head_stats(partial + (size_t)h * tiles * G * 4, tiles, G, wave,
                                                lane);
        if (lane == 0) s_stats[wave] = st;
    }
    __syncthreads();
    select_reg_head<KPT, kBlock, false>(
        L, GqaKeys<G>{raw + (size_t)h * (size_t)len * G, s_stats}, len, budget,
        kept + (size_t)h * (size_t)kept_stride, nullptr, nullptr);
}

// A ragged batch in one launch: the heads of up to kSelectBatch sequences of
// the same length class (at most 64 * KPT * NT / 64 keys each), one
// workgroup per head.  Workgroup w selects head w % heads of sequence
// w / heads of the table; the caller orders the table longest first, so the
// long heads are dispatched first.
struct SelectSeq {
    const float* scores;   // the sequence's scores, [heads][n]
    int32_t* kept;         // its kept lists, [heads][budget]
    int32_t n;             // keys per head
    int32_t pad;
};
struct SelectBatch {
    SelectSeq seq[kSelectBatch];
};

template <int KPT>
__global__ __launch_bounds__(kBlock) void select_batch_kernel(const SelectBatch b, int heads,
                                                              int budget)
{
    __shared__ RegLds<kBlock> L;
    const int s = blockIdx.x / heads;
    const int h = blockIdx.x - s * heads;
    const float* sc = b.seq[s].scores;
    int32_t* kept = b.seq[s].kept;
    const int n = b.seq[s].n;
    select_reg_head<KPT, kBlock, false>(L, ScoreKeys{sc + (size_t)h * (size_t)n}, n, budget,
                                        kept + (size_t)h * (size_t)budget, nullptr, nullptr);
}


// ---------------------------------------------------------------------------
// Heads longer than the register-resident selection takes (more than 32768
// keys, up to kWideMax), with one read of the scores:
//
// 1. A fixed sample of kSample keys: kSampleRuns runs of kSampleRun
//    consecutive slots, run c at a hashed offset inside the c-th
//    1/kSampleRuns of the head (stratified, and jittered so that scores that
//    vary periodically with the position, as the distance preference makes
//    them, are not sampled at one phase).  With r the number of sample keys
//    expected among the head's top B (B * kSample / n, rounded up) and
//    delta = max(32, 10 sqrt(r)), two levels of 4096-bin histograms of the
//    sample find the bins of its (r - delta)-th and (r + delta)-th largest
//    keys: hi is the top of the first, lo the bottom of the second.  The
//    bracket [lo, hi] holds the head's B-th largest key unless the sample
//    misrepresents the head.
// 2. One pass over the scores: keys above hi set a bit in the "above"
//    bitmap; keys in [lo, hi] are candidates: a bit in the candidate bitmap,
//    and (key, slot) appended to the wave's own segment of an LDS list while
//    it has room (the count is wave-uniform, so appending needs no atomics).
// 3. If fewer than B keys lie above hi, at least B at or above lo, and the
//    candidates fit the list (or lo == hi: then they all equal the
//    threshold), the threshold T is found among the candidates alone
//    (offset-radix passes over the LDS list, then one wave ranks the last 64
//    or fewer); candidates above T (T and above
//    when equal keys do not straddle it) join the "above" bitmap and those
//    equal to T make up the candidate bitmap.  Otherwise the head is selected
//    by the general path (select_lds_head, which reads the scores again), so
//    the result never depends on the sample.
// 4. The kept list comes from the two bitmaps in slot order: every "above"
//    slot and the first need_eq slots equal to T.  Each lane takes a
//    contiguous run of 64-slot blocks; scans of the per-lane counts give
//    every lane its place in the list.
// Dynamic LDS: the two bitmaps (ceil(n / 64) 64-bit words each), a 4096-bin
// histogram, and the candidate list (cmax keys, then cmax slots, in kWaves
// equal segments).
constexpr int kWideMax = 1 << 18;
constexpr int kSampleRuns = 512;
constexpr int kSampleRun = 32;
constexpr int kSample = kSampleRuns * kSampleRun;
constexpr int kSamplePerThread = kSample / kBlock;
static_assert(kSample == kSamplePerThread * kBlock, "whole sample keys per thread");
constexpr int kWideBins = 1 << kRegDigitBits;
constexpr int kWideLdsBytes = 155648;          // dynamic LDS of the wide selection
constexpr int kPassBatch = 16;                 // score loads per thread in flight in the pass
static_assert(kWideLdsBytes >= kHistBins * 4, "room for the general path's histogram");

__global__ __launch_bounds__(kBlock) void select_wide_kernel(const float* __restrict__ scores,
                                                             int n, int budget,
                                                             int32_t* __restrict__ kept,
                                                             int kept_stride, int cmax)
{
    // 16-byte aligned: the bitmaps are 64-bit words, and LDS atomics on them
    // (ds_or_b64) need natural alignment
    extern __shared__ __align__(16) uint32_t smem[];
    __shared__ uint32_t s_wa[kWaves], s_wb[kWaves], s_run[kWaves], s_cnt[kWaves];
    __shared__ uint32_t s_cand[64];
    __shared__ uint32_t s_digit, s_above, s_inbin, s_nc, s_T, s_need, s_tie;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const float* sc = scores + (size_t)blockIdx.x * (size_t)n;
    int32_t* out = kept + (size_t)blockIdx.x * (size_t)kept_stride;
    const int W64 = (n + 63) / 64;                       // 64-slot blocks
    unsigned long long* above_bm = reinterpret_cast<unsigned long long*>(smem);
    unsigned long long* cand_bm = above_bm + W64;
    uint32_t* hist = reinterpret_cast<uint32_t*>(cand_bm + W64);
    uint32_t* ckey = hist + kWideBins;
    uint32_t* cslot = ckey + cmax;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)sc, 0, n * 4, kBufferWord3);
    const unsigned long long below = (1ull << lane) - 1ull;

    // ---- 1. the bracket from the sample
    uint32_t lo, hi;
    {
        // sample key q = tid + kBlock * u is key q % kSampleRun of run
        // q / kSampleRun, which starts at a hashed offset inside the run's
        // 1/kSampleRuns of the head (a wave reads two whole runs per load)
        const int stride = n / kSampleRuns;
        uint32_t sk[kSamplePerThread];
#pragma unroll
        for (int u = 0; u < kSamplePerThread; ++u) {
            const int q = tid + kBlock * u;
            const int run = q / kSampleRun;
            uint32_t hsh = (uint32_t)run * 0x9E3779B1u + 0x7F4A7C15u;
            hsh ^= hsh >> 15;
            hsh *= 0x2C1B3C6Du;
            hsh ^= hsh >> 12;
            const int start = run * stride + (int)(hsh % (uint32_t)(stride - kSampleRun + 1));
            sk[u] = ordered_key(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rsrc, (start + q % kSampleRun) * 4, 0, 0)));
        }
        uint32_t smn = 0xFFFFFFFFu, smx = 0u;
#pragma unroll
        for (int u = 0; u < kSamplePerThread; ++u) {
            smn = min(smn, sk[u]);
            smx = max(smx, sk[u]);
        }
        smn = wave_min(smn);
        smx = wave_max(smx);
        if (lane == 0) {
            s_wa[wave] = smn;
            s_wb[wave] = smx;
        }
        __syncthreads();
        smn = s_wa[0];
        smx = s_wb[0];
        for (int x = 1; x < kWaves; ++x) {
            smn = min(smn, s_wa[x]);
            smx = max(smx, s_wb[x]);
        }
        // sample ranks (from the top) of the bracket's ends, then two levels
        // of histograms narrow [base, top] down to the bins that hold them
        const int64_t r = ((int64_t)budget * kSample + n - 1) / n;
        const int64_t delta = max((int64_t)32, (int64_t)ceil(10.0 * sqrt((double)r)));
        uint32_t r_hi = (uint32_t)max((int64_t)1, r - delta);
        uint32_t r_lo = (uint32_t)min((int64_t)kSample, r + delta);
        uint32_t base = smn, top = smx;
        for (int level = 0; level < 2 && base != top; ++level) {
            const int wb = 32 - __clz((int)(top - base));
            const int nb = min(kRegDigitBits, wb);
            const int sh = wb - nb;
            const uint32_t nbins = 1u << nb;
            __syncthreads();                            // previous readers of hist / s_*
            for (uint32_t b = tid; b < nbins; b += kBlock) hist[b] = 0u;
            __syncthreads();
#pragma unroll
            for (int u = 0; u < kSamplePerThread; ++u)
                if (sk[u] >= base && sk[u] <= top) atomicAdd(&hist[(sk[u] - base) >> sh], 1u);
            __syncthreads();
            find_digit<kBlock>(hist, nbins, r_hi, tid, lane, wave, s_run, &s_digit, &s_above, &s_inbin);
            __syncthreads();
            const uint32_t d_hi = s_digit;
            const uint32_t a_hi = s_above;
            __syncthreads();
            find_digit<kBlock>(hist, nbins, r_lo, tid, lane, wave, s_run, &s_digit, &s_above, &s_inbin);
            __syncthreads();
            const uint32_t d_lo = s_digit;
            top = (uint32_t)min((uint64_t)top, (uint64_t)base + ((uint64_t)(d_hi + 1u) << sh) - 1u);
            base = base + (d_lo << sh);
            r_hi -= a_hi;                               // sample keys above top are no longer counted
            r_lo -= a_hi;
        }
        lo = base;
        hi = top;
    }

    // ---- 2. one pass: "above" and candidate bitmaps; each wave appends its
    // candidates to a segment of the list of its own, counted in a register
    // (no atomics: every lane of the wave holds the same count)
    const uint32_t segcap = (uint32_t)cmax / kWaves;
    uint32_t* wkey = ckey + wave * segcap;
    uint32_t* wslot = cslot + wave * segcap;
    uint32_t n_above = 0u, n_cw = 0u;                   // this wave's counts
    for (int i0 = 0; i0 < n; i0 += kBlock * kPassBatch) {
        uint32_t x[kPassBatch];
#pragma unroll
        for (int u = 0; u < kPassBatch; ++u)
            x[u] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (i0 + u * kBlock + tid) * 4, 0, 0);
#pragma unroll
        for (int u = 0; u < kPassBatch; ++u) {
            const int blk = i0 + u * kBlock + wave * 64;   // the wave's 64 slots
            const int i = blk + lane;
            const uint32_t key = ordered_key(__uint_as_float(x[u]));
            const bool valid = i < n;
            const bool ab = valid && key > hi;
            const bool cd = valid && !ab && key >= lo;
            const unsigned long long ma = __ballot(ab);
            const unsigned long long mc = __ballot(cd);
            if (lane == 0 && blk < n) {
                above_bm[blk >> 6] = ma;
                cand_bm[blk >> 6] = mc;
            }
            n_above += (uint32_t)__popcll(ma);
            const uint32_t at = n_cw + (uint32_t)__popcll(mc & below);
            if (cd && at < segcap) {
                wkey[at] = key;
                wslot[at] = (uint32_t)i;
            }
            n_cw += (uint32_t)__popcll(mc);
        }
    }
    if (lane == 0) {
        s_wa[wave] = n_above;
        s_cnt[wave] = n_cw;
    }
    __syncthreads();
    uint32_t total_above = 0u, n_cand = 0u, max_cw = 0u;
    for (int x = 0; x < kWaves; ++x) {
        total_above += s_wa[x];
        n_cand += s_cnt[x];
        max_cw = max(max_cw, s_cnt[x]);
    }
    const bool bracket = total_above < (uint32_t)budget && total_above + n_cand >= (uint32_t)budget &&
                         (lo == hi || max_cw <= segcap);
    if (!bracket) {
        __syncthreads();                                // every thread is done with the bitmaps
        select_lds_head<false>(smem, sc, n, budget, out);
        return;
    }

    // ---- 3. the threshold among the candidates
    uint32_t T, need_eq;
    bool tie;
    const uint32_t rem0 = (uint32_t)budget - total_above;     // in [1, n_cand]
    if (lo == hi) {
        T = lo;                                          // every candidate equals T
        need_eq = rem0;
        tie = true;
    } else {
        const uint32_t my_cnt = s_cnt[wave];            // <= segcap here
        uint32_t base = lo;
        int wb = 32 - __clz((int)(hi - lo));            // candidates lie in [base, base + 2^wb)
        uint32_t rem = rem0;
        for (;;) {
            const int nb = min(kRegDigitBits, wb);
            const int sh = wb - nb;
            const uint32_t nbins = 1u << nb;
            const uint32_t span = wb >= 32 ? 0xFFFFFFFFu : (1u << wb) - 1u;
            __syncthreads();                            // previous readers of hist / s_*
            for (uint32_t b = tid; b < nbins; b += kBlock) hist[b] = 0u;
            if (tid == 0) s_nc = 0u;
            __syncthreads();
            for (uint32_t c = lane; c < my_cnt; c += 64) {
                const uint32_t off = wkey[c] - base;
                if (off <= span) atomicAdd(&hist[off >> sh], 1u);
            }
            __syncthreads();
            find_digit<kBlock>(hist, nbins, rem, tid, lane, wave, s_run, &s_digit, &s_above, &s_inbin);
            __syncthreads();
            const uint32_t d = s_digit & (nbins - 1u);
            const uint32_t in_bin = s_inbin;
            rem -= s_above;
            base += d << sh;
            wb = sh;
            if (rem == in_bin) {                        // the whole bin is kept
                T = base;
                need_eq = 0u;
                tie = false;
                break;
            }
            if (wb == 0) {                              // one key value straddles the budget
                T = base;
                need_eq = rem;
                tie = true;
                break;
            }
            if (in_bin <= 64u) {
                // the few candidates left: one wave ranks them (each counts
                // those above it and equal to it; the rem-th largest has
                // gt < rem <= gt + eq)
                const uint32_t cspan = (1u << wb) - 1u;
                for (uint32_t c = lane; c < my_cnt; c += 64) {
                    const uint32_t k = wkey[c];
                    if (k - base <= cspan) {
                        const uint32_t at = atomicAdd(&s_nc, 1u);
                        if (at < 64u) s_cand[at] = k;
                    }
                }
                __syncthreads();
                if (wave == 0) {
                    const uint32_t v = (uint32_t)lane < in_bin ? s_cand[lane] : 0u;
                    uint32_t gt = 0u, eq = 0u;
                    for (uint32_t j = 0; j < in_bin; ++j) {
                        const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)v, (int)j);
                        gt += o > v ? 1u : 0u;
                        eq += o == v ? 1u : 0u;
                    }
                    const bool hit = (uint32_t)lane < in_bin && gt < rem && rem <= gt + eq;
                    const int src = __ffsll((unsigned long long)__ballot(hit)) - 1;   // one exists
                    const uint32_t t = (uint32_t)__builtin_amdgcn_readlane((int)v, src);
                    const uint32_t g = (uint32_t)__builtin_amdgcn_readlane((int)gt, src);
                    const uint32_t e = (uint32_t)__builtin_amdgcn_readlane((int)eq, src);
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
        // candidates above T (or at least T) join "above"; those equal to T
        // (with a tie) become the candidate bitmap
        __syncthreads();
        for (int w = tid; w < W64; w += kBlock) cand_bm[w] = 0ull;
        __syncthreads();
        for (uint32_t c = lane; c < my_cnt; c += 64) {
            const uint32_t key = wkey[c];
            const uint32_t slot = wslot[c];
            if (tie ? key > T : key >= T) atomicOr(&above_bm[slot >> 6], 1ull << (slot & 63u));
            else if (tie && key == T) atomicOr(&cand_bm[slot >> 6], 1ull << (slot & 63u));
        }
    }
    __syncthreads();

    // ---- 4. the kept list in slot order: wave w owns a run of 64-slot
    // blocks, and each lane a contiguous part of it; the kept slots before a
    // lane's part come from a scan of the per-lane counts
    const int per_wave = (W64 + kWaves - 1) / kWaves;
    const int per_lane = (per_wave + 63) / 64;
    const int lb0 = min(W64, wave * per_wave + lane * per_lane);
    const int lb1 = min(min(W64, (wave + 1) * per_wave), lb0 + per_lane);
    uint32_t ca = 0u, ce = 0u;
    for (int b = lb0; b < lb1; ++b) {
        ca += (uint32_t)__popcll(above_bm[b]);
        ce += (uint32_t)__popcll(cand_bm[b]);
    }
    const uint32_t ia = wave_incl_scan(ca, lane);
    const uint32_t ie = wave_incl_scan(ce, lane);
    if (lane == 63) {
        s_wa[wave] = ia;
        s_wb[wave] = ie;
    }
    __syncthreads();
    uint32_t a_before = ia - ca, e_before = ie - ce;
    for (int x = 0; x < wave; ++x) {
        a_before += s_wa[x];
        e_before += s_wb[x];
    }
    for (int b = lb0; b < lb1; ++b) {
        const unsigned long long ma = above_bm[b];
        unsigned long long m = ma | cand_bm[b];
        while (m) {
            const int bit = __ffsll(m) - 1;
            m &= m - 1ull;
            uint32_t at = 0xFFFFFFFFu;
            if ((ma >> bit) & 1ull) {
                at = a_before + min(e_before, need_eq);
                ++a_before;
            } else {
                if (e_before < need_eq) at = a_before + e_before;
                ++e_before;
            }
            if (at < (uint32_t)budget) out[at] = 64 * b + bit;
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
// The layer-wide threshold is a radix select (12-bit digits) over the
// layer's unreserved keys, spread over one workgroup per head so that every
// compute unit works: in each pass every head histograms its own unreserved
// keys into a histogram of its own in the workspace, with the sums of its
// 64-bin groups, and the next launch adds up the layer's histograms (every
// workgroup of the layer does the same sums and takes the same decision):
// first the group sums, to find the group of the deciding digit, then the
// 64 bins of that group.  The digits are the
// key's bits 31..20, 19..8 and 7..0, so the first needs no key range and is
// histogrammed by the reserve step itself.  When equal keys straddle the
// threshold, the bin counts of the deciding pass give each head's equal
// keys, handed out in head order.
//   select_reg_kernel<.., true> / shared_reserve_kernel
//                          (Th, Sh), the range and the first-digit histogram
//                          of the unreserved keys
//   shared_pass_kernel     (twice) decide the previous digit, histogram the next
//   shared_write_kernel    decide the last digit, write each head's list

constexpr int kMaxSharedHeads = 128;
constexpr int kSharedBins = 1 << kRegDigitBits;
static_assert(kSharedBins % kBlock == 0, "whole bins per thread");

// Selection state of one layer after a pass (identical in every workgroup
// of the layer; the first head's workgroup stores it for the next launch).
struct LayerState {
    uint32_t fired;      // the layer prunes
    uint32_t done;       // T decided
    uint32_t base;       // unreserved keys still in play: [base, base + 2^wb)
    uint32_t wb;
    uint32_t rem;        // slots still to fill from the keys in play
    uint32_t T;          // keep unreserved keys >= T (tie: > T, plus need_eq == T)
    uint32_t tie;
    uint32_t need_eq;
    uint32_t res_pass;   // tie: pass that decided it (0: every unreserved key equals T)
    uint32_t eq_bin;     // tie: bin of T in that pass's histograms
    uint32_t pad0, pad1, pad2, pad3, pad4, pad5;
};
static_assert(sizeof(LayerState) == 64, "layer state layout");

__device__ __forceinline__ int head_rows(const int32_t* head_len, int64_t idx, int stride)
{
    return head_len ? max(0, min(head_len[idx], stride)) : stride;
}

__device__ __forceinline__ bool is_reserved(uint32_t key, int i, uint32_t th, int sh)
{
    return key > th || (key == th && i <= sh);
}

// Block-wide min / max over uint32 (every thread gets the result).
__device__ __forceinline__ uint32_t block_min(uint32_t v, uint32_t* s_w, int lane, int wave)
{
    v = wave_min(v);
    __syncthreads();
    if (lane == 0) s_w[wave] = v;
    __syncthreads();
    uint32_t r = s_w[0];
    for (int x = 1; x < kWaves; ++x) r = min(r, s_w[x]);
    return r;
}

__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* s_w, int lane, int wave)
{
    v = wave_max(v);
    __syncthreads();
    if (lane == 0) s_w[wave] = v;
    __syncthreads();
    uint32_t r = s_w[0];
    for (int x = 1; x < kWaves; ++x) r = max(r, s_w[x]);
    return r;
}

// Calls f(i, key) for the n keys of one head, kHeadBatch loads in flight per
// thread.
constexpr int kHeadBatch = 8;
template <typename F>
__device__ __forceinline__ void for_head_keys(const float* sc, int n, int tid, F&& f)
{
    for (int i0 = tid; i0 < n; i0 += kBlock * kHeadBatch) {
        float x[kHeadBatch];
#pragma unroll
        for (int u = 0; u < kHeadBatch; ++u) x[u] = sc[min(i0 + u * kBlock, n - 1)];
#pragma unroll
        for (int u = 0; u < kHeadBatch; ++u) {
            const int i = i0 + u * kBlock;
            if (i < n) f(i, ordered_key(x[u]));
        }
    }
}

// Heads of more than 32768 keys: one workgroup per head takes (Th, Sh) from
// the head's reserved list (written by the list-making selection) and writes
// rec[head] = {Th, Sh, min, max} of its unreserved keys (min > max when there
// are none) and their first-digit histogram, as the register-resident
// reserve step does.
__global__ __launch_bounds__(kBlock) void shared_reserve_kernel(
    const float* __restrict__ scores, int stride, const int32_t* __restrict__ head_len,
    int total, int floor_, const int32_t* __restrict__ kept, uint4* __restrict__ rec,
    uint32_t* __restrict__ hist_out)
{
    __shared__ uint32_t s_w[kWaves];
    __shared__ uint32_t lhist[1 << kRegDigitBits];
    const int head = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = head_rows(head_len, head, stride);
    const float* sc = scores + (size_t)head * (size_t)stride;
    uint32_t th;
    int sh;
    if (floor_ == 0) {
        th = kTopKey;                     // no key is above it: nothing reserved
        sh = -1;
    } else if (n <= floor_) {
        th = 0u;                          // every real key is above it: all reserved
        sh = -1;
    } else {
        const int32_t* l = kept + (size_t)head * (size_t)total;
        uint32_t mn = 0xFFFFFFFFu;
        for (int j = tid; j < floor_; j += kBlock) mn = min(mn, ordered_key(sc[min(max(l[j], 0), n - 1)]));
        th = block_min(mn, s_w, lane, wave);
        int mx = -1;
        for (int j = tid; j < floor_; j += kBlock) {
            const int slot = min(max(l[j], 0), n - 1);
            if (ordered_key(sc[slot]) == th) mx = max(mx, slot);
        }
        sh = (int)block_max((uint32_t)(mx + 1), s_w, lane, wave) - 1;
    }
    for (int b = tid; b < (1 << kRegDigitBits); b += kBlock) lhist[b] = 0u;
    __syncthreads();
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for_head_keys(sc, n, tid, [&](int i, uint32_t key) {
        if (!is_reserved(key, i, th, sh)) {
            lo = min(lo, key);
            hi = max(hi, key);
            atomicAdd(&lhist[key >> (32 - kRegDigitBits)], 1u);
        }
    });
    lo = block_min(lo, s_w, lane, wave);
    hi = block_max(hi, s_w, lane, wave);
    uint32_t* ho = hist_out + (size_t)head * kHistRow;
    for (int b = tid; b < (1 << kRegDigitBits); b += kBlock) ho[b] = lhist[b];
    write_group_sums(lhist, 1u << kRegDigitBits, ho + (1 << kRegDigitBits), tid);
    if (tid == 0) rec[head] = make_uint4(th, (uint32_t)sh, lo, hi);
}

// State after the reserve step: the firing rule, the slots left and the
// range of the layer's unreserved keys.
__device__ __forceinline__ LayerState layer_init(const uint4* __restrict__ rec_l,
                                                 const int32_t* __restrict__ hl_l, int stride,
                                                 int n_kv, int total, int floor_, int window)
{
    LayerState S = {};
    int64_t all = 0, reserved = 0;
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int h = 0; h < n_kv; ++h) {
        const int n = head_rows(hl_l, h, stride);
        all += n;
        reserved += min(n, floor_);
        const uint4 r = rec_l[h];
        lo = min(lo, r.z);
        hi = max(hi, r.w);
    }
    S.fired = all > (int64_t)total + (int64_t)n_kv * window ? 1u : 0u;
    if (!S.fired) {
        S.done = 1u;
        return S;
    }
    S.rem = (uint32_t)((int64_t)total - reserved);        // floor * n_kv <= total
    if (S.rem == 0u) {                                     // the reserved keys fill the layer
        S.done = 1u;
        S.T = kTopKey;
    } else if (lo == hi) {                                 // one unreserved key value
        S.done = 1u;
        S.T = lo;
        S.tie = 1u;
        S.need_eq = S.rem;
        S.res_pass = 0u;
    } else {
        // the first digit is the top 12 bits of the key: the reserve step
        // has already histogrammed it, with no range needed
        S.base = 0u;
        S.wb = 32u;
    }
    return S;
}

// Decides pass `pass` from the layer's per-head histogram rows (hist_l:
// n_kv rows of kHistRow).  Every thread of the workgroup calls it; wave 0
// finds the digit in two steps, each a 64-lane scan counted from the top:
// the group of 64 bins that holds the rem-th key (from the rows' group
// sums), then the bin inside it, so a workgroup reads 2 x 64 x n_kv words
// of the rows instead of all 4096 x n_kv.
__device__ __forceinline__ void layer_resolve(LayerState& S, uint32_t pass,
                                              const uint32_t* __restrict__ hist_l, int n_kv,
                                              uint32_t* s_dig, int lane, int wave)
{
    const int nb = min(kRegDigitBits, (int)S.wb);
    const int shift = (int)S.wb - nb;
    const uint32_t nbins = 1u << nb;
    if (wave == 0) {
        // the n_kv rows' words at one column, summed (loads in flight 8 at a time)
        auto column = [&](uint32_t col, bool live) {
            uint32_t acc = 0u;
            int h = 0;
            for (; h + 8 <= n_kv; h += 8) {
                uint32_t v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = live ? hist_l[(size_t)(h + u) * kHistRow + col] : 0u;
#pragma unroll
                for (int u = 0; u < 8; ++u) acc += v[u];
            }
            for (; h < n_kv; ++h) acc += live ? hist_l[(size_t)h * kHistRow + col] : 0u;
            return acc;
        };
        // lane j: group 63 - j (groups past nbins sum to 0)
        const uint32_t g = 63u - (uint32_t)lane;
        const uint32_t cg_sum = column((uint32_t)kSharedBins + g, true);
        const uint32_t cg_incl = wave_incl_scan(cg_sum, lane);
        const int lg = __ffsll((unsigned long long)__ballot(cg_incl >= S.rem)) - 1;
        const uint32_t grp = 63u - (uint32_t)lg;
        const uint32_t above_g = lane_u(cg_incl - cg_sum, lg);
        // lane j: bin 64 * grp + 63 - j
        const uint32_t bin = 64u * grp + 63u - (uint32_t)lane;
        const uint32_t b_sum = column(bin, bin < nbins);
        const uint32_t b_incl = wave_incl_scan(b_sum, lane);
        const int lb = __ffsll((unsigned long long)__ballot(above_g + b_incl >= S.rem)) - 1;
        // lane reads with every lane active (a value computed under a
        // one-lane mask would hold garbage in the other lanes)
        const uint32_t above_b = lane_u(b_incl - b_sum, lb);
        const uint32_t in_b = lane_u(b_sum, lb);
        if (lane == 0) {
            s_dig[0] = 64u * grp + 63u - (uint32_t)lb;
            s_dig[1] = above_g + above_b;
            s_dig[2] = in_b;
        }
    }
    __syncthreads();
    const uint32_t d = s_dig[0] & (nbins - 1u);
    const uint32_t in_bin = s_dig[2];
    S.rem -= s_dig[1];
    S.base += d << shift;
    S.wb = (uint32_t)shift;
    // the whole bin is kept, or the bin is one key value that straddles
    // (selects rather than branches keep the state in registers)
    const bool whole = S.rem == in_bin;
    const bool straddle = !whole && shift == 0;
    S.done = (whole || straddle) ? 1u : 0u;
    S.T = (whole || straddle) ? S.base : S.T;
    S.tie = straddle ? 1u : S.tie;
    S.need_eq = straddle ? S.rem : S.need_eq;
    S.res_pass = straddle ? pass : S.res_pass;
    S.eq_bin = straddle ? d : S.eq_bin;
    __syncthreads();                     // s_dig is reused
}

// Launch `pass` (2 or 3): decide pass - 1 (pass 1's histograms come from the
// reserve step), then histogram this head's unreserved keys for pass `pass`.
// KPT > 0: every thread loads its KPT keys at once (lane l of wave w: slots
// w*64*KPT + c*64 + l); KPT == 0: batches of kHeadBatch.
template <int KPT>
__global__ __launch_bounds__(kBlock) void shared_pass_kernel(
    int pass, const float* __restrict__ scores, int stride, int n_layers, int n_kv,
    const int32_t* __restrict__ head_len, int total, int floor_, int window,
    const uint4* __restrict__ rec, uint32_t* __restrict__ hist, LayerState* __restrict__ state)
{
    __shared__ uint32_t lhist[kSharedBins];
    __shared__ uint32_t s_dig[3];
    const int head = blockIdx.x;
    const int layer = head / n_kv;
    const int h = head - layer * n_kv;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const size_t heads = (size_t)n_layers * (size_t)n_kv;
    // the state before pass - 1: set up from the reserve step (pass 2) or
    // stored by the previous launch
    LayerState S = pass == 2
        ? layer_init(rec + (size_t)layer * n_kv, head_len ? head_len + (size_t)layer * n_kv : nullptr,
                     stride, n_kv, total, floor_, window)
        : state[(size_t)(pass - 2) * n_layers + layer];
    if (!S.done)
        layer_resolve(S, (uint32_t)(pass - 1),
                      hist + (size_t)((pass - 2) & 1) * heads * kHistRow +
                          (size_t)layer * n_kv * kHistRow,
                      n_kv, s_dig, lane, wave);
    if (h == 0 && tid == 0) state[(size_t)(pass - 1) * n_layers + layer] = S;
    if (S.done) return;

    const int nb = min(kRegDigitBits, (int)S.wb);
    const int shift = (int)S.wb - nb;
    const uint32_t nbins = 1u << nb;
    const uint32_t span = S.wb >= 32u ? 0xFFFFFFFFu : (1u << S.wb) - 1u;
    for (uint32_t b = tid; b < nbins; b += kBlock) lhist[b] = 0u;
    __syncthreads();
    const uint4 r = rec[head];
    const uint32_t th = r.x;
    const int sh = (int)r.y;
    const uint32_t base = S.base;
    const int n = head_rows(head_len, head, stride);
    const float* sc = scores + (size_t)head * (size_t)stride;
    auto add = [&](int i, uint32_t key) {
        const uint32_t off = key - base;
        if (i < n && off <= span && !is_reserved(key, i, th, sh)) atomicAdd(&lhist[off >> shift], 1u);
    };
    if constexpr (KPT > 0) {
        const int seg0 = wave * (64 * KPT) + lane;
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)sc, 0, n * 4, kBufferWord3);
        uint32_t x[KPT];
#pragma unroll
        for (int c = 0; c < KPT; ++c)
            x[c] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (seg0 + 64 * c) * 4, 0, 0);
#pragma unroll
        for (int c = 0; c < KPT; ++c) add(seg0 + 64 * c, ordered_key(__uint_as_float(x[c])));
    } else {
        for_head_keys(sc, n, tid, add);
    }
    __syncthreads();
    uint32_t* out = hist + (size_t)((pass - 1) & 1) * heads * kHistRow + (size_t)head * kHistRow;
    for (uint32_t b = tid; b < nbins; b += kBlock) out[b] = lhist[b];
    write_group_sums(lhist, nbins, out + kSharedBins, tid);
}

// One workgroup per head: decide the last pass if needed, then the kept list
// of the head in slot order and its count (-1 when the layer does not fire).
// KPT > 0: the head's keys sit in registers as in the register-resident
// selection (lane l of wave w holds slots w*64*KPT + c*64 + l); KPT == 0:
// wave w owns slots [w*seg, (w+1)*seg) and reads them from memory twice.  A
// counting sweep gives every wave its offset in the list.
template <int KPT>
__global__ __launch_bounds__(kBlock) void shared_write_kernel(
    const float* __restrict__ scores, int stride, int n_layers, int n_kv,
    const int32_t* __restrict__ head_len, int total, int floor_, const uint4* __restrict__ rec,
    const uint32_t* __restrict__ hist, const LayerState* __restrict__ state,
    int32_t* __restrict__ kept, int32_t* __restrict__ kept_count)
{
    __shared__ uint32_t s_dig[3];
    __shared__ uint32_t s_wgt[kWaves], s_weq[kWaves];
    const int lh = blockIdx.x;
    const int layer = lh / n_kv;
    const int hh = lh - layer * n_kv;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const size_t heads = (size_t)n_layers * (size_t)n_kv;
    LayerState S = state[(size_t)2 * n_layers + layer];
    if (!S.done)
        layer_resolve(S, 3u, hist + (size_t)layer * n_kv * kHistRow, n_kv, s_dig, lane, wave);
    if (!S.fired) {
        if (tid == 0) kept_count[lh] = -1;
        return;
    }
    // equal keys taken by this head: what is left after the lower heads
    uint32_t take = 0u;
    if (S.tie) {
        const int32_t* hl_l = head_len ? head_len + (size_t)layer * n_kv : nullptr;
        const uint32_t* bins = hist + (size_t)((S.res_pass - 1u) & 1u) * heads * kHistRow +
                               (size_t)layer * n_kv * kHistRow + S.eq_bin;
        uint32_t left = S.need_eq;
        for (int h = 0; h <= hh; ++h) {
            uint32_t eq;
            if (S.res_pass == 0u) {
                const int n = head_rows(hl_l, h, stride);
                eq = (uint32_t)(n - min(n, floor_));
            } else {
                eq = bins[(size_t)h * kHistRow];
            }
            const uint32_t t = min(eq, left);
            if (h == hh) take = t;
            left -= t;
        }
    }
    const uint4 r = rec[lh];
    const uint32_t th = r.x;
    const int sh = (int)r.y;
    const uint32_t T = S.T;
    const bool tie = S.tie != 0u;
    const int n = head_rows(head_len, lh, stride);
    const float* sc = scores + (size_t)lh * (size_t)stride;
    int32_t* out = kept + (size_t)lh * (size_t)total;
    const unsigned long long below = (1ull << lane) - 1ull;

    // gt: kept outright (reserved, or above the layer threshold);
    // eq: unreserved and equal to T when equal keys straddle it.  Key 0
    // marks a slot past the head's end.
    auto classify = [&](int i, uint32_t key, bool& gt, bool& eq) {
        const bool real = key != 0u;
        const bool res = real && is_reserved(key, i, th, sh);
        gt = res || (real && (tie ? key > T : key >= T));
        eq = !res && tie && real && key == T;
    };

    if constexpr (KPT > 0) {
        static_assert(KPT <= 32, "one bit per key in a 32-bit mask");
        const int seg0 = wave * (64 * KPT) + lane;
        // classify every key once; bit c of gtb / eqb is key c's class.  The
        // tests are 0/1 words combined with bit operations, so the sweep is
        // straight-line code (the same classes as classify below)
        uint32_t gtb = 0u, eqb = 0u;
        {
            const __amdgpu_buffer_rsrc_t rsrc =
                __builtin_amdgcn_make_buffer_rsrc((void*)sc, 0, n * 4, kBufferWord3);
            uint32_t x[KPT];
#pragma unroll
            for (int c = 0; c < KPT; ++c)
                x[c] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (seg0 + 64 * c) * 4, 0, 0);
            const uint32_t tie_w = tie ? 1u : 0u;
#pragma unroll
            for (int c = 0; c < KPT; ++c) {
                const int slot = seg0 + 64 * c;
                const uint32_t key = ordered_key(__uint_as_float(x[c]));
                const uint32_t real = slot < n ? 1u : 0u;
                const uint32_t at_th = key == th ? 1u : 0u;
                const uint32_t low_slot = slot <= sh ? 1u : 0u;
                const uint32_t res = real & ((key > th ? 1u : 0u) | (at_th & low_slot));
                const uint32_t at_t = key == T ? 1u : 0u;
                const uint32_t above = (key > T ? 1u : 0u) | (at_t & (tie_w ^ 1u));
                gtb |= (res | (real & above)) << c;
                eqb |= ((res ^ 1u) & real & tie_w & at_t) << c;
            }
        }
        uint32_t cgt = (uint32_t)__popc(gtb), ceq = (uint32_t)__popc(eqb);
        cgt = wave_sum(cgt);
        ceq = wave_sum(ceq);
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
        // a partly unrolled sweep: a full unroll keeps every ballot mask of
        // the 32 rounds live at once and spills scalar registers
#pragma unroll 4
        for (int c = 0; c < KPT; ++c) {
            const bool gt = (gtb >> c) & 1u;
            const bool eq = (eqb >> c) & 1u;
            const unsigned long long mgt = __ballot(gt);
            const unsigned long long meq = __ballot(eq);
            const uint32_t my_gt = gt_before + (uint32_t)__popcll(mgt & below);
            const uint32_t my_eq = eq_before + (uint32_t)__popcll(meq & below);
            const uint32_t at = my_gt + min(my_eq, take);
            if ((gt || (eq && my_eq < take)) && at < (uint32_t)total) out[at] = seg0 + 64 * c;
            gt_before += (uint32_t)__popcll(mgt);
            eq_before += (uint32_t)__popcll(meq);
        }
        if (tid == 0) kept_count[lh] = (int32_t)min(gt_all + min(eq_all, take), (uint32_t)total);
    } else {
        const int seg = ((n + kWaves - 1) / kWaves + 63) & ~63;
        const int s0 = wave * seg;
        const int s1 = min(n, s0 + seg);
        auto key_at = [&](int i) { return i < s1 ? ordered_key(sc[i]) : 0u; };
        uint32_t cgt = 0u, ceq = 0u;
        for (int i0 = s0; i0 < s1; i0 += 64) {
            bool gt, eq;
            classify(i0 + lane, key_at(i0 + lane), gt, eq);
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
        for (int i0 = s0; i0 < s1; i0 += 64) {
            const int i = i0 + lane;
            bool gt, eq;
            classify(i, key_at(i), gt, eq);
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
    } else if (n <= kBlock * 24) {
        hipLaunchKernelGGL((select_reg_kernel<24, kBlock>), dim3(n_heads), dim3(kBlock), 0, stream,
                           scores, n, budget, kept, kept_stride, head_len);
    } else if (n <= kBlock * 32) {
        hipLaunchKernelGGL((select_reg_kernel<32, kBlock>), dim3(n_heads), dim3(kBlock), 0, stream,
                           scores, n, budget, kept, kept_stride, head_len);
    } else if (n <= kWideMax && !head_len) {
        // dynamic LDS: two bitmaps, the histogram, then the candidate list
        const int64_t words = 2 * 2 * (((int64_t)n + 63) / 64) + kWideBins;   // two 64-bit bitmaps
        const int cmax = (int)((kWideLdsBytes / 4 - words) / 2);
        if (cmax < 1024) return hipErrorInvalidValue;
        // the attribute belongs to the current device: set it on every call
        hipError_t e = hipFuncSetAttribute((const void*)select_wide_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kWideLdsBytes);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(select_wide_kernel, dim3(n_heads), dim3(kBlock), (size_t)kWideLdsBytes,
                           stream, scores, n, budget, kept, kept_stride, cmax);
    } else if (n <= kLdsKeysMax) {
        const size_t lds = (size_t)(kHistBins + n) * sizeof(uint32_t);
        // the attribute belongs to the current device: set it on every call
        hipError_t e = hipFuncSetAttribute((const void*)select_kernel<true>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)((kHistBins + kLdsKeysMax) * sizeof(uint32_t)));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(select_kernel<true>, dim3(n_heads), dim3(kBlock), lds, stream, scores, n,
                           budget, kept, kept_stride, head_len);
    } else {
        const size_t lds = (size_t)kHistBins * sizeof(uint32_t);
        hipLaunchKernelGGL(select_kernel<false>, dim3(n_heads), dim3(kBlock), lds, stream, scores,
                           n, budget, kept, kept_stride, head_len);
    }
    return hipGetLastError();
}


hipError_t launch_select_gqa(int group, const float* raw, const double* partial, int len,
                             int n_heads, int budget, int32_t* kept, int kept_stride,
                             hipStream_t stream)
{
    if (n_heads <= 0 || len <= budget) return hipSuccess;
    if (len > kBlock * 32) return hipErrorInvalidValue;
    const int tiles = (len + kGqaTileRows - 1) / kGqaTileRows;
    const dim3 grid((unsigned)n_heads), block(kBlock);
#define TRI_GQA_SEL(KPT, G)                                                                       \
    hipLaunchKernelGGL((select_gqa_kernel<KPT, G>), grid, block, 0, stream, raw, partial, tiles,  \
                       len, budget, kept, kept_stride)
#define TRI_GQA_SEL_G(KPT)                                                                        \
    switch (group) {                                                                              \
    case 2: TRI_GQA_SEL(KPT, 2); break;                                                           \
    case 3: TRI_GQA_SEL(KPT, 3); break;                                                           \
    case 4: TRI_GQA_SEL(KPT, 4); break;                                                           \
    case 5: TRI_GQA_SEL(KPT, 5); break;                                                           \
    case 6: TRI_GQA_SEL(KPT, 6); break;                                                           \
    case 7: TRI_GQA_SEL(KPT, 7); break;                                                           \
    case 8: TRI_GQA_SEL(KPT, 8); break;                                                           \
    default: return hipErrorInvalidValue;                                                         \
    }
    if (len <= kBlock * 8) {
        TRI_GQA_SEL_G(8)
    } else if (len <= kBlock * 16) {
        TRI_GQA_SEL_G(16)
    } else if (len <= kBlock * 24) {
        TRI_GQA_SEL_G(24)
    } else {
        TRI_GQA_SEL_G(32)
    }
#undef TRI_GQA_SEL_G
#undef TRI_GQA_SEL
    return hipGetLastError();
}

hipError_t launch_select_batch(int n_seq, const float* const* scores, int32_t* const* kept,
                               const int* n, int n_heads, int budget, hipStream_t stream)
{
    if (n_heads <= 0) return hipSuccess;
    // register-resident length classes; longer heads go one sequence at a time
    std::vector<int> cls[4];
    for (int s = 0; s < n_seq; ++s) {
        if (n[s] <= budget) continue;
        if (n[s] <= kBlock * 8) cls[0].push_back(s);
        else if (n[s] <= kBlock * 16) cls[1].push_back(s);
        else if (n[s] <= kBlock * 24) cls[2].push_back(s);
        else if (n[s] <= kBlock * 32) cls[3].push_back(s);
        else {
            hipError_t e = launch_select(scores[s], n[s], n_heads, budget, kept[s], budget, nullptr,
                                         stream);
            if (e != hipSuccess) return e;
        }
    }
    for (int c = 3; c >= 0; --c) {
        std::vector<int>& v = cls[c];
        // longest heads first: the dispatcher hands out workgroups in order
        std::stable_sort(v.begin(), v.end(), [&](int a, int b) { return n[a] > n[b]; });
        for (size_t i0 = 0; i0 < v.size(); i0 += kSelectBatch) {
            const int cnt = (int)std::min<size_t>(kSelectBatch, v.size() - i0);
            if ((int64_t)cnt * n_heads > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
            SelectBatch b{};
            for (int j = 0; j < cnt; ++j) {
                const int s = v[i0 + j];
                b.seq[j] = SelectSeq{scores[s], kept[s], n[s], 0};
            }
            const dim3 grid((unsigned)(cnt * n_heads)), block(kBlock);
            if (c == 0) hipLaunchKernelGGL(select_batch_kernel<8>, grid, block, 0, stream, b, n_heads, budget);
            else if (c == 1) hipLaunchKernelGGL(select_batch_kernel<16>, grid, block, 0, stream, b, n_heads, budget);
            else if (c == 2) hipLaunchKernelGGL(select_batch_kernel<24>, grid, block, 0, stream, b, n_heads, budget);
            else hipLaunchKernelGGL(select_batch_kernel<32>, grid, block, 0, stream, b, n_heads, budget);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

// Workspace of one sequence: per-head records, two banks of per-head
// histograms, the layer states of three passes.
int64_t shared_workspace_bytes(int64_t n_seq, int64_t n_layers, int64_t n_kv)
{
    auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    const int64_t heads = n_layers * n_kv;
    return n_seq * (up(heads * 16) + up(2 * heads * kHistRow * 4) +
                    up(3 * n_layers * (int64_t)sizeof(LayerState)));
}

hipError_t launch_select_shared(const float* scores, int stride, int n_layers, int n_kv,
                                const int32_t* head_len, int budget, int floor_, int window,
                                int32_t* kept, int32_t* kept_count, void* workspace,
                                hipStream_t stream)
{
    if (n_layers <= 0 || n_kv <= 0) return hipSuccess;
    if (n_kv > kMaxSharedHeads) return hipErrorInvalidValue;
    const int64_t total = (int64_t)budget * n_kv;
    const int64_t heads = (int64_t)n_layers * n_kv;
    if (total > 0x7FFFFFFF || heads > 0x7FFFFFFF) return hipErrorInvalidValue;
    auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    uint4* rec = reinterpret_cast<uint4*>(ws);
    uint32_t* hist = reinterpret_cast<uint32_t*>(ws + up(heads * 16));
    LayerState* state = reinterpret_cast<LayerState*>(ws + up(heads * 16) +
                                                      up(2 * heads * kHistRow * 4));
    const dim3 grid((unsigned)heads), block(kBlock);
    hipError_t e = hipSuccess;
    if (stride <= kBlock * 32) {
        // register-resident: the floor selection writes the reserved sets directly
#define TRI_RESERVE(KPT)                                                                          \
        hipLaunchKernelGGL((select_reg_kernel<KPT, kBlock, true>), grid, block, 0, stream, scores, \
                           stride, floor_, nullptr, 0, head_len, rec, hist)
        if (stride <= kBlock * 8) TRI_RESERVE(8);
        else if (stride <= kBlock * 16) TRI_RESERVE(16);
        else TRI_RESERVE(32);
#undef TRI_RESERVE
    } else {
        if (floor_ > 0 && stride > floor_) {
            // each head's reserved list, into the head's kept row (stride total)
            e = launch_select(scores, stride, (int)heads, floor_, kept, (int)total, head_len,
                              stream);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(shared_reserve_kernel, grid, block, 0, stream, scores, stride,
                           head_len, (int)total, floor_, kept, rec, hist);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    for (int pass = 2; pass <= 3; ++pass) {
#define TRI_PASS(KPT)                                                                             \
        hipLaunchKernelGGL(shared_pass_kernel<KPT>, grid, block, 0, stream, pass, scores, stride,  \
                           n_layers, n_kv, head_len, (int)total, floor_, window,                  \
                           static_cast<const uint4*>(rec), hist, state)
        if (stride <= kBlock * 8) TRI_PASS(8);
        else if (stride <= kBlock * 16) TRI_PASS(16);
        else if (stride <= kBlock * 32) TRI_PASS(32);
        else TRI_PASS(0);
#undef TRI_PASS
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
#define TRI_WRITE(KPT)                                                                            \
    hipLaunchKernelGGL(shared_write_kernel<KPT>, grid, block, 0, stream, scores, stride,           \
                       n_layers, n_kv, head_len, (int)total, floor_,                               \
                       static_cast<const uint4*>(rec), static_cast<const uint32_t*>(hist),         \
                       static_cast<const LayerState*>(state), kept, kept_count)
    if (stride <= kBlock * 8) TRI_WRITE(8);
    else if (stride <= kBlock * 16) TRI_WRITE(16);
    else if (stride <= kBlock * 32) TRI_WRITE(32);
    else TRI_WRITE(0);
#undef TRI_WRITE
    return hipGetLastError();
}

}  // namespace tri
