// GQA normalize-then-aggregate scoring: G query heads share each KV head.
//
// Source: dimensionstp.github.io "TriAttention ... Review", section 3-2
// item 6 (each query head's key scores are z-score normalized, then the max
// over the query heads of a KV head is the key's score), and romaanj.github.io
// "TriAttention" review, section "Method" (GQA: per-head z-score, then max).
// Readings: the mean and the population standard deviation run over the
// finite scores of the head's cached keys; a deviation of at most 1e-9 of
// the largest |score| counts as zero and gives z = 0; a non-finite score
// gives NaN, which loses to every number in the max.
//
// Launches per sequence:
//   1. One pass over K.  Every row gets G raw scores (the score of the
//      single-query-head kernel with query head g's folded constants); the
//      band magnitudes |K_f| are shared by the G norm terms.  Raw scores go
//      to the workspace [head][row][g]; per 512-row tile and query head the
//      pass also writes fp64 partial statistics (sum, sum of squares, count
//      of finite scores, largest |score|).  bf16 K: gqa_prep_kernel folds
//      the constants into matrix-core operands, gqa_mfma_kernel scores;
//      f32 K: gqa_score_kernel.
//   With a score array:
//   2. gqa_stats_kernel: per (head, g), the partials summed in tile order
//      (deterministic) into the mean and the deviation (0 when flat).
//   3. gqa_norm_kernel: z = (s - mean) / sd per query head in fp64, the max
//      over the group, rounded once to fp32 into the caller's score array.
//   Without one, the GQA selection forms the statistics (gqa_stats.h) and
//   the max-z keys from the workspace itself (select_gqa_kernel).
#include <type_traits>

#include "gqa_stats.h"
#include "tri_internal.h"

namespace tri {
namespace {

constexpr int kBlock = 256;
constexpr int kTileRows = kGqaTileRows;
constexpr int kBufferWord3 = 0x00020000;   // raw buffer resource word 3, gfx9 family
constexpr int kSC1 = 16;                   // cache-policy bits: sc1
constexpr int kNT = 2;                     // cache-policy bits: non-temporal
// matrix-core B operands of one head: at most 8 k-blocks x 64 lanes x 16 bytes
constexpr int64_t kBopBytesPerHead = 8 * 64 * 16;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPR consecutive lanes; every lane of the group
// receives the total.
template <int LPR>
__device__ __forceinline__ float group_sum(float x)
{
    static_assert(LPR == 4 || LPR == 8 || LPR == 16 || LPR == 32 || LPR == 64, "lanes per row");
    x += dpp<0xB1>(x);                          // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp<0x4E>(x);                          // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (LPR >= 8) x += dpp<0x141>(x);   // row_half_mirror: quads of an 8-lane half
    if constexpr (LPR >= 16) x += dpp<0x140>(x);  // row_mirror: halves of a 16-lane row
    if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
    if constexpr (LPR >= 64) x += __shfl_xor(x, 32);
    return x;
}

// Partner value at lane distance S inside aligned groups (the pairing of
// each step of the reductions below): xor for 32, 16, 2 and 1; a mirror of
// the 16-lane row for 8 and of the 8-lane half for 4.  Each pairs a lane
// whose bit S is clear with one whose bit S is set.
template <int S>
__device__ __forceinline__ float partner(float x)
{
    if constexpr (S == 32 || S == 16) return __shfl_xor(x, S);
    else if constexpr (S == 8) return dpp<0x140>(x);   // row_mirror
    else if constexpr (S == 4) return dpp<0x141>(x);   // row_half_mirror
    else if constexpr (S == 2) return dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    else return dpp<0xB1>(x);                          // quad_perm [1,0,3,2]
}

// Sums M values per lane over aligned groups of LPR lanes, M a power of two
// <= LPR, with the values split between partners: at each of the first
// log2(M) steps a lane keeps one half of its values, sends the other half
// and adds what its partner sends, so the work halves every step.  Lane j of
// a group ends with the group total of value g = j / (LPR / M) (the lanes
// of one g hold the same total).
template <int LPR, int S, int M>
__device__ __forceinline__ float split_reduce(float* v, int j)
{
    if constexpr (S == 0) {
        return v[0];
    } else if constexpr (M > 1) {
        const bool lower = (j & S) == 0;
#pragma unroll
        for (int k = 0; k < M / 2; ++k) {
            const float keep = lower ? v[k] : v[M / 2 + k];
            const float send = lower ? v[M / 2 + k] : v[k];
            v[k] = keep + partner<S>(send);
        }
        return split_reduce<LPR, S / 2, M / 2>(v, j);
    } else {
        v[0] += partner<S>(v[0]);
        return split_reduce<LPR, S / 2, 1>(v, j);
    }
}

constexpr int pow2_at_least(int x)
{
    int p = 1;
    while (p < x) p *= 2;
    return p;
}

__device__ __forceinline__ double wave_sum_d(double v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ double wave_max_d(double v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o));
    return v;
}

// EB bytes of one half-row per lane, unpacked to fp32 bands.
template <bool BF16, int EB>
struct Chunk {
    static constexpr int kElem = BF16 ? 2 : 4;
    static constexpr int E = EB / kElem;        // bands per lane
    static constexpr int W = EB / 4;            // 32-bit words per lane
    uint32_t w[W];
    __device__ __forceinline__ void load(const unsigned char* p)
    {
        if constexpr (W == 2) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
            w[0] = v.x;
            w[1] = v.y;
        } else {
            w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
        }
    }
    __device__ __forceinline__ void unpack(float* out) const
    {
#pragma unroll
        for (int m = 0; m < W; ++m) {
            if constexpr (BF16) {
                out[2 * m] = __uint_as_float(w[m] << 16);
                out[2 * m + 1] = __uint_as_float(w[m] & 0xFFFF0000u);
            } else {
                out[m] = __uint_as_float(w[m]);
            }
        }
    }
};

// The end of a score tile: its raw scores (rows [tile_start, row_end) x G,
// staged in s_raw) leave in one contiguous sweep, and per query head the
// fp64 partial statistics of the tile (sum, sum of squares, count of finite
// scores, largest |score|) are reduced in a fixed order.
template <int G>
__device__ __forceinline__ void tile_epilogue(const float* s_raw, double (*s_red)[4],
                                              float* __restrict__ raw,
                                              double* __restrict__ partial, int head, int tile,
                                              int tiles_per_head, int len, int tile_start,
                                              int row_end, int tid, int lane, int wave)
{
    const int n_out = (row_end - tile_start) * G;
    float* out = raw + ((size_t)head * (size_t)len + tile_start) * G;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(out, 0, n_out * 4, kBufferWord3);
    for (int i = tid; i < n_out; i += kBlock)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s_raw[i]), ro, i * 4, 0, kSC1);

    double* pt = partial + (((size_t)head * tiles_per_head + tile) * G) * 4;
    const int n_rows = row_end - tile_start;
    for (int g = 0; g < G; ++g) {
        double s1 = 0.0, s2 = 0.0, cnt = 0.0, big = 0.0;
        for (int r = tid; r < n_rows; r += kBlock) {
            const double x = (double)s_raw[r * G + g];
            if (isfinite(x)) {
                s1 += x;
                s2 += x * x;
                cnt += 1.0;
                big = fmax(big, fabs(x));
            }
        }
        s1 = wave_sum_d(s1);
        s2 = wave_sum_d(s2);
        cnt = wave_sum_d(cnt);
        big = wave_max_d(big);
        if (lane == 0) {
            s_red[wave][0] = s1;
            s_red[wave][1] = s2;
            s_red[wave][2] = cnt;
            s_red[wave][3] = big;
        }
        __syncthreads();
        if (tid == 0) {
            double a1 = 0.0, a2 = 0.0, ac = 0.0, ab = 0.0;
            for (int x = 0; x < kBlock / 64; ++x) {
                a1 += s_red[x][0];
                a2 += s_red[x][1];
                ac += s_red[x][2];
                ab = fmax(ab, s_red[x][3]);
            }
            pt[g * 4 + 0] = a1;
            pt[g * 4 + 1] = a2;
            pt[g * 4 + 2] = ac;
            pt[g * 4 + 3] = ab;
        }
        __syncthreads();
    }
}

template <int D, bool BF16, int G>
struct GqaShape {
    static constexpr int kElem = BF16 ? 2 : 4;
    static constexpr int kHalf = D / 2;
    static constexpr int kRowBytes = D * kElem;
    static constexpr int kHalfBytes = kRowBytes / 2;
    // 8 bytes per lane and half row while G * 3 * bands fits in 48 registers
    static constexpr int EB = (3 * G * (8 / kElem) <= 48 && kHalfBytes / 8 <= 64) ? 8 : 4;
    static constexpr int LPR = kHalfBytes / EB;   // lanes per row
    static constexpr int E = EB / kElem;          // bands per lane
    static constexpr int RPI = 64 / LPR;          // rows per wave instruction
    static constexpr int GR = kBlock / LPR;       // rows per workgroup step
    static constexpr int kUnroll = 64 / EB;       // rows per lane in flight (64 bytes)
    static_assert(LPR >= 4 && LPR <= 64 && E >= 1, "lane layout");
    static_assert(3 * G * E <= 48, "folded constants fit in registers");
    static_assert(kTileRows % (GR * kUnroll) == 0, "a tile is whole iterations");
};

template <int D, bool BF16, int G>
__global__ __launch_bounds__(kBlock) void gqa_score_kernel(
    const unsigned char* __restrict__ k, int64_t cap, int len, int tiles_per_head, double p_now,
    const double* __restrict__ omega, const double2* __restrict__ qa, const float* __restrict__ w,
    float* __restrict__ raw, double* __restrict__ partial, const int32_t* __restrict__ head_len)
{
    using S = GqaShape<D, BF16, G>;
    constexpr int kHalf = S::kHalf, LPR = S::LPR, E = S::E, GR = S::GR, kUnroll = S::kUnroll;
    constexpr int GP = pow2_at_least(G);      // query heads padded to a power of two
    static_assert(GP <= LPR, "one lane per query head in a row group");
    constexpr int kRowBytes = S::kRowBytes, kHalfBytes = S::kHalfBytes, EB = S::EB;

    __shared__ float s_u[G][D];
    __shared__ float s_w[G][kHalf];
    __shared__ float s_raw[kTileRows * G];
    __shared__ double s_red[kBlock / 64][4];

    const int head = blockIdx.x / tiles_per_head;
    const int tile = blockIdx.x - head * tiles_per_head;
    // rows in use of this head: all `len`, or its own length (ragged heads);
    // tiles past it are skipped and left out of the statistics
    const int n_h = head_len ? max(0, min(head_len[head], len)) : len;
    if (tile * kTileRows >= n_h) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = tid % LPR;   // lane within the row
    const int g0 = tid / LPR;  // row within a workgroup step
    const unsigned char* base = k + (size_t)head * (size_t)cap * kRowBytes + EB * j;
    const int tile_start = tile * kTileRows;
    const int row_end = min(n_h, tile_start + kTileRows);

    Chunk<BF16, EB> re[kUnroll], im[kUnroll];
    auto load_row = [&](int u, int row) {
        const unsigned char* p = base + (size_t)min(row, row_end - 1) * kRowBytes;
        re[u].load(p);
        im[u].load(p + kHalfBytes);
    };
    const int iters = (row_end - tile_start + GR * kUnroll - 1) / (GR * kUnroll);
    int r0 = tile_start + g0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) load_row(u, r0 + u * GR);   // in flight during the fold

    // fold C_f = E[q_f] A_f e^{i w_f p_now} of each query head in fp64
    for (int t = tid; t < G * kHalf; t += kBlock) {
        const int g = t / kHalf, f = t - g * kHalf;
        double sn, cs;
        sincos(omega[f] * p_now, &sn, &cs);
        const double2 a = qa[((size_t)head * G + g) * kHalf + f];
        s_u[g][f] = (float)(a.x * cs - a.y * sn);
        s_u[g][f + kHalf] = (float)(a.x * sn + a.y * cs);
        s_w[g][f] = w[((size_t)head * G + g) * kHalf + f];
    }
    __syncthreads();
    float u_re[G][E], u_im[G][E], wt[G][E];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < E; ++e) {
            u_re[g][e] = s_u[g][j * E + e];
            u_im[g][e] = s_u[g][kHalf + j * E + e];
            wt[g][e] = s_w[g][j * E + e];
        }

    // rolling pipeline as in the single-query-head kernel
    for (int it = 0; it < iters; ++it) {
        const int r_next = r0 + GR * kUnroll;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float a[E], b[E];
            re[u].unpack(a);
            im[u].unpack(b);
            load_row(u, r_next + u * GR);
            __builtin_amdgcn_sched_barrier(0);
            float mag[E];
#pragma unroll
            for (int e = 0; e < E; ++e) mag[e] = __builtin_amdgcn_sqrtf(fmaf(a[e], a[e], b[e] * b[e]));
            float part[GP];
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                float t = 0.f;
                if (g < G) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        t = fmaf(u_re[g][e], a[e], t);
                        t = fmaf(u_im[g][e], b[e], t);
                    }
                    float nrm = 0.f;
#pragma unroll
                    for (int e = 0; e < E; ++e) nrm = fmaf(wt[g][e], mag[e], nrm);
                    t += nrm;
                }
                part[g] = t;
            }
            const float total = split_reduce<LPR, LPR / 2, GP>(part, j);
            const int gq = j / (LPR / GP);           // query head whose total this lane holds
            if (j % (LPR / GP) == 0 && gq < G)
                s_raw[(r0 + u * GR - tile_start) * G + gq] = total;   // < kTileRows * G
            __builtin_amdgcn_sched_barrier(0);
        }
        r0 = r_next;
    }
    __syncthreads();

    tile_epilogue<G>(s_raw, s_red, raw, partial, head, tile, tiles_per_head, len, tile_start,
                     row_end, tid, lane, wave);
}

// MFMA variant for bf16 K (D = 64 or 128): the G dot products and the G
// norm sums of 16 rows are one small contraction,
//   raw[row][g] = sum_k K[row][k] u_g[k] + sum_f |K_f|[row] w_g[f],
// which v_mfma_f32_16x16x32_bf16 evaluates with the rows as M, the query
// heads as N and [K | |K|] as the contraction.  Its operands are bf16: K is
// stored in bf16 (exact); the folded constants u_g, the weights w_g and the
// magnitudes |K_f| are fp32 and enter as a sum of two bf16 numbers,
// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), which leaves an error
// of at most 2^-16 |x|.  Columns g < G carry the hi parts of the constants,
// columns G + g their lo parts, and raw[row][g] is the sum of columns g and
// G + g:
//   column g:     K . u_hi  +  |K|_hi . w_hi  +  |K|_lo . w_hi
//   column G + g: K . u_lo  +  |K|_hi . w_lo
// (the dropped |K|_lo . w_lo is below 2^-16 of the norm term).  Products of
// bf16 numbers are exact and the MFMA accumulates in fp32.
//
// Lane layout of the 16x16x32 operands (checked on the device): lane l holds
// A[l % 16][8 (l / 16) + i] and B[8 (l / 16) + i][l % 16], i < 8, and result
// rows 4 (l / 16) + i of column l % 16, i < 4.  So lane l loads 16 bytes of
// row l % 16 at byte 16 (l / 16) of each 64-byte k-block: a row's real half
// and imaginary half land in the same lane (k-blocks m and m + KB / 2), which
// gives the band magnitudes with no data exchange.
//
// gqa_prep_kernel folds the constants once per head (fp64) and writes every
// lane's B operands, [head][k-block][lane] x 16 bytes, to the workspace;
// gqa_mfma_kernel reads them at the start of each tile.
template <int D>
struct MfmaShape {
    static constexpr int kHalf = D / 2;
    static constexpr int kRowBytes = D * 2;
    static constexpr int KB = kRowBytes / 64;   // k-blocks of a K row
    static constexpr int KM = KB / 2;           // k-blocks of the band magnitudes
    static constexpr int NT = KB + 2 * KM;      // k-blocks of the contraction
    static_assert(KB >= 2 && KB % 2 == 0, "row of whole k-block pairs");
};

// B operands of one head: one wave; lane l's entries of column l % 16.
template <int D, int G>
__global__ __launch_bounds__(64) void gqa_prep_kernel(double p_now, const double* __restrict__ omega,
                                                      const double2* __restrict__ qa,
                                                      const float* __restrict__ w,
                                                      u32x4* __restrict__ bops)
{
    using S = MfmaShape<D>;
    constexpr int kHalf = S::kHalf, KB = S::KB, KM = S::KM, NT = S::NT;
    static_assert(2 * G <= 16, "hi and lo columns of every query head fit in 16");
    __shared__ float s_u[G][D];
    __shared__ float s_w[G][kHalf];
    const int head = blockIdx.x;
    const int lane = threadIdx.x;
    // one rotation e^{i w_f p_now} per band, shared by the G query heads
    for (int f = lane; f < kHalf; f += 64) {
        double sn, cs;
        sincos(omega[f] * p_now, &sn, &cs);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const double2 a = qa[((size_t)head * G + g) * kHalf + f];
            s_u[g][f] = (float)(a.x * cs - a.y * sn);
            s_u[g][f + kHalf] = (float)(a.x * sn + a.y * cs);
            s_w[g][f] = w[((size_t)head * G + g) * kHalf + f];
        }
    }
    __syncthreads();
    const int q = lane >> 4, rl = lane & 15;
    const bool col_hi = rl < G, col_lo = rl >= G && rl < 2 * G;
    const int g = col_hi ? rl : (col_lo ? rl - G : 0);
    for (int t = 0; t < NT; ++t) {
        bf16x8 v;
        for (int i = 0; i < 8; ++i) {
            float x;
            bool take_lo = col_lo;
            bool use = col_hi || col_lo;
            if (t < KB) {
                x = s_u[g][t * 32 + 8 * q + i];
            } else if (t < KB + KM) {
                x = s_w[g][(t - KB) * 32 + 8 * q + i];
            } else {
                x = s_w[g][(t - KB - KM) * 32 + 8 * q + i];
                use = col_hi;               // |K|_lo meets w_hi only
                take_lo = false;
            }
            const __bf16 h = (__bf16)x;
            v[i] = !use ? (__bf16)0.0f : (take_lo ? (__bf16)(x - (float)h) : h);
        }
        bops[((size_t)head * NT + t) * 64 + lane] = __builtin_bit_cast(u32x4, v);
    }
}

// Squares of the two bands held in the low and the high halves of a bf16
// pair register: the real and imaginary parts are paired by a byte permute
// and squared and summed by one dot instruction (exact products).
__device__ __forceinline__ void band_energy(uint32_t re2, uint32_t im2, float& e0, float& e1)
{
    const uint32_t p0 = __builtin_amdgcn_perm(im2, re2, 0x05040100u);   // (re lo, im lo)
    const uint32_t p1 = __builtin_amdgcn_perm(im2, re2, 0x07060302u);   // (re hi, im hi)
    const bf16x2 a0 = __builtin_bit_cast(bf16x2, p0), a1 = __builtin_bit_cast(bf16x2, p1);
    e0 = __builtin_amdgcn_fdot2_f32_bf16(a0, a0, 0.0f, false);
    e1 = __builtin_amdgcn_fdot2_f32_bf16(a1, a1, 0.0f, false);
}

// Each wave takes 16-row groups w, w + 4, ... of the tile, R of them in flight.
template <int D, int G>
__global__ __launch_bounds__(kBlock) void gqa_mfma_kernel(
    const unsigned char* __restrict__ k, int64_t cap, int len, int tiles_per_head,
    const u32x4* __restrict__ bops, float* __restrict__ raw, double* __restrict__ partial,
    const int32_t* __restrict__ head_len)
{
    using S = MfmaShape<D>;
    constexpr int kRowBytes = S::kRowBytes, KB = S::KB, KM = S::KM, NT = S::NT;
    // R = 4, P = 2 measured 422.8 us per pass on the 36 x 8 x 32768 cache
    // with G = 4, against 427.5 us for R = 2, P = 1 (the same code otherwise)
    constexpr int R = 4;                      // 16-row groups in registers per wave
    constexpr int P = 2;                      // groups computed together
    static_assert(R % P == 0, "whole steps");
    constexpr int kWaves = kBlock / 64;
    constexpr int kGroupsPerWave = kTileRows / 16 / kWaves;
    static_assert(kGroupsPerWave % R == 0, "whole rounds of groups per wave");

    __shared__ float s_raw[kTileRows * G];
    __shared__ double s_red[kBlock / 64][4];
    __shared__ __attribute__((aligned(16))) unsigned char s_stage[kWaves * 16 * (kRowBytes + 16)];

    const int head = blockIdx.x / tiles_per_head;
    const int tile = blockIdx.x - head * tiles_per_head;
    const int n_h = head_len ? max(0, min(head_len[head], len)) : len;
    if (tile * kTileRows >= n_h) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int q = lane >> 4;                  // 16-byte chunk within a k-block
    const int rl = lane & 15;                 // row within a group; result column
    const int tile_start = tile * kTileRows;
    const int row_end = min(n_h, tile_start + kTileRows);

    bf16x8 bop[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        bop[t] = __builtin_bit_cast(bf16x8, bops[((size_t)head * NT + t) * 64 + lane]);

    // K rows through a bounds-checked buffer resource that spans exactly
    // the tile's rows: loads of groups past the tile's end fall outside it
    // and the hardware drops them (zeros, no traffic), so every wave issues
    // the same loads in the same order and the waits can count them
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(k + ((size_t)head * (size_t)cap + tile_start) * kRowBytes), 0,
        (row_end - tile_start) * kRowBytes, kBufferWord3);
    // A wave instruction reads whole rows (RPI rows of CPR 16-byte chunks,
    // every 128-byte line complete); the rows then pass through LDS, where
    // each lane picks up the chunks the MFMA layout gives it.
    constexpr int CPR = kRowBytes / 16;       // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;             // rows per wave instruction
    constexpr int NI = 16 / RPI;              // instructions per 16-row group
    static_assert(NI == KB, "a group is one load per k-block");
    u32x4 buf[R][KB];
    auto load_group = [&](u32x4* b, int gi) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            // lane l: row l / CPR of the instruction's RPI rows, chunk l % CPR
            // (a row is CPR chunks of 16 bytes, so that is byte 16 l)
            const uint32_t off = (uint32_t)(gi * 16 + j * RPI) * kRowBytes + lane * 16;
            b[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kNT));
        }
    };
    // staging rows padded by 16 bytes: the MFMA-layout reads (16 rows at
    // one chunk offset) fall into 16 different 4-bank groups
    constexpr int kStageRow = kRowBytes + 16;
    unsigned char* stage = s_stage + wave * (16 * kStageRow);
#pragma unroll
    for (int r = 0; r < R; ++r) load_group(buf[r], wave + r * kWaves);

    // P groups at a time: their magnitude work and their MFMA chains are
    // independent, which gives the scheduler work to overlap with each
    // chain's latency
    auto compute = [&](const u32x4 (*bl)[KB], const int* gi) {
        u32x4 b[P][KB];
#pragma unroll
        for (int p = 0; p < P; ++p) {
#pragma unroll
            for (int j = 0; j < NI; ++j)
                *reinterpret_cast<u32x4*>(stage + (j * RPI + lane / CPR) * kStageRow + (lane % CPR) * 16) =
                    bl[p][j];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                b[p][kb] = *reinterpret_cast<const u32x4*>(stage + rl * kStageRow + (kb * 4 + q) * 16);
        }
        u32x4 mh[P][KM], ml[P][KM];   // band magnitudes: bf16 hi and lo parts, in pairs
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int m = 0; m < KM; ++m)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    float e0, e1;
                    band_energy(b[p][m][c], b[p][m + KM][c], e0, e1);
                    const float m0 = __builtin_amdgcn_sqrtf(e0), m1 = __builtin_amdgcn_sqrtf(e1);
                    // hi parts packed in one conversion; their fp32 values
                    // are the halves of that word
                    const uint32_t hw = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)m0, (__bf16)m1});
                    const float h0 = __uint_as_float(hw << 16), h1 = __uint_as_float(hw & 0xFFFF0000u);
                    mh[p][m][c] = hw;
                    ml[p][m][c] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)(m0 - h0), (__bf16)(m1 - h1)});
                }
        f32x4 acc[P];
#pragma unroll
        for (int p = 0; p < P; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KB; ++t)
#pragma unroll
            for (int p = 0; p < P; ++p)
                acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b[p][t]),
                                                                 bop[t], acc[p], 0, 0, 0);
#pragma unroll
        for (int m = 0; m < KM; ++m)
#pragma unroll
            for (int p = 0; p < P; ++p)
                acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, mh[p][m]),
                                                                 bop[KB + m], acc[p], 0, 0, 0);
#pragma unroll
        for (int m = 0; m < KM; ++m)
#pragma unroll
            for (int p = 0; p < P; ++p)
                acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ml[p][m]),
                                                                 bop[KB + KM + m], acc[p], 0, 0, 0);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)   // + column G + rl, same rows: row_shl:G within the 16 lanes
                v[i] = acc[p][i] + __int_as_float(__builtin_amdgcn_update_dpp(
                                       0, __float_as_int(acc[p][i]), 0x100 + G, 0xF, 0xF, false));
            // rows past the tile's end (zero rows) land in s_raw entries the
            // epilogue does not read
            if (rl < G) {
#pragma unroll
                for (int i = 0; i < 4; ++i) s_raw[(gi[p] * 16 + 4 * q + i) * G + rl] = v[i];
            }
        }
    };

    // scheduling barriers pin every step's loads right after the compute
    // that frees their registers, so R - P groups stay in flight
#pragma unroll
    for (int o = 0; o < kGroupsPerWave; o += R) {
#pragma unroll
        for (int r = 0; r < R; r += P) {
            int gi[P];
#pragma unroll
            for (int p = 0; p < P; ++p) gi[p] = wave + (o + r + p) * kWaves;
            __builtin_amdgcn_sched_barrier(0);
            compute(&buf[r], gi);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int p = 0; p < P; ++p) load_group(buf[r + p], gi[p] + R * kWaves);
        }
    }
    __syncthreads();
    tile_epilogue<G>(s_raw, s_red, raw, partial, head, tile, tiles_per_head, len, tile_start,
                     row_end, tid, lane, wave);
}

// mean and deviation per (head, query head): one wave per head; lane t sums
// tiles t, t + 64, ... in order, then a fixed butterfly combines the lanes,
// so the result does not depend on scheduling
__global__ __launch_bounds__(64) void gqa_stats_kernel(const double* __restrict__ partial,
                                                       int tiles_per_head, int group, int len,
                                                       const int32_t* __restrict__ head_len,
                                                       double2* __restrict__ stats)
{
    const int head = blockIdx.x;
    const int lane = threadIdx.x;
    const int n_h = head_len ? max(0, min(head_len[head], len)) : len;
    const int tiles = (n_h + kTileRows - 1) / kTileRows;   // tiles the score kernel wrote
    const double* ph = partial + (size_t)head * tiles_per_head * group * 4;
    for (int g = 0; g < group; ++g) {
        const double2 st = gqa_query_head_stats(ph, tiles, group, g, lane);
        if (lane == 0) stats[(size_t)head * group + g] = st;
    }
}

// z per query head in fp64, max over the group, rounded once to fp32
template <int G>
__global__ __launch_bounds__(kBlock) void gqa_norm_kernel(const float* __restrict__ raw,
                                                          const double2* __restrict__ stats,
                                                          int len, int tiles_per_head,
                                                          float* __restrict__ scores,
                                                          const int32_t* __restrict__ head_len)
{
    __shared__ double s_mean[G], s_inv[G];   // s_inv = 0: flat row, z = 0
    const int head = blockIdx.x / tiles_per_head;
    const int tile = blockIdx.x - head * tiles_per_head;
    if (threadIdx.x < G) {
        const double2 st = stats[(size_t)head * G + threadIdx.x];
        s_mean[threadIdx.x] = st.x;
        s_inv[threadIdx.x] = st.y > 0.0 ? 1.0 / st.y : 0.0;
    }
    __syncthreads();
    const int n_h = head_len ? max(0, min(head_len[head], len)) : len;
    const int row_end = min(n_h, (tile + 1) * kTileRows);
    for (int r = tile * kTileRows + threadIdx.x; r < row_end; r += kBlock) {
        const float* p = raw + ((size_t)head * len + r) * G;
        float x[G];
#pragma unroll
        for (int g = 0; g < G; ++g) x[g] = __builtin_nontemporal_load(p + g);
        double best = NAN;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const double s = (double)x[g];
            if (isfinite(s)) {
                const double z = (s - s_mean[g]) * s_inv[g];
                if (isnan(best) || z > best) best = z;
            }
        }
        scores[(size_t)head * len + r] = (float)best;
    }
}

template <int D, bool BF16, int G>
hipError_t launch_g(const void* k, int64_t cap, int len, int n_heads, int64_t p_now,
                    const double* omega, const double2* qa, const float* w, float* raw,
                    double* partial, double2* stats, float* scores, const int32_t* head_len,
                    u32x4* bops, hipStream_t stream)
{
    const int tiles = (len + kTileRows - 1) / kTileRows;
    const int64_t grid = (int64_t)tiles * n_heads;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if constexpr (BF16) {
        // bf16 K: the G dot products and norm sums on the matrix cores, their
        // operands prepared once per head
        hipLaunchKernelGGL((gqa_prep_kernel<D, G>), dim3((unsigned)n_heads), dim3(64), 0, stream,
                           (double)p_now, omega, qa, w, bops);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((gqa_mfma_kernel<D, G>), dim3((unsigned)grid), dim3(kBlock), 0, stream,
                           static_cast<const unsigned char*>(k), cap, len, tiles,
                           static_cast<const u32x4*>(bops), raw, partial, head_len);
    } else {
        hipLaunchKernelGGL((gqa_score_kernel<D, BF16, G>), dim3((unsigned)grid), dim3(kBlock), 0,
                           stream, static_cast<const unsigned char*>(k), cap, len, tiles,
                           (double)p_now, omega, qa, w, raw, partial, head_len);
    }
    hipError_t e = hipGetLastError();
    // no score array: the raw scores and the per-tile partial sums only (the
    // GQA selection forms the statistics itself)
    if (e != hipSuccess || !scores) return e;
    hipLaunchKernelGGL(gqa_stats_kernel, dim3(n_heads), dim3(64), 0, stream, partial, tiles, G,
                       len, head_len, stats);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gqa_norm_kernel<G>), dim3((unsigned)grid), dim3(kBlock), 0, stream, raw,
                       stats, len, tiles, scores, head_len);
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_d(int group, const void* k, int64_t cap, int len, int n_heads, int64_t p_now,
                    const double* omega, const double2* qa, const float* w, float* raw,
                    double* partial, double2* stats, float* scores, const int32_t* head_len,
                    u32x4* bops, hipStream_t stream)
{
#define TRI_GQA_CASE(G)                                                                           \
    case G:                                                                                       \
        return launch_g<D, BF16, G>(k, cap, len, n_heads, p_now, omega, qa, w, raw, partial,      \
                                    stats, scores, head_len, bops, stream);
    switch (group) {
        TRI_GQA_CASE(2)
        TRI_GQA_CASE(3)
        TRI_GQA_CASE(4)
        TRI_GQA_CASE(5)
        TRI_GQA_CASE(6)
        TRI_GQA_CASE(7)
        TRI_GQA_CASE(8)
    default: return hipErrorInvalidValue;
    }
#undef TRI_GQA_CASE
}

}  // namespace

int64_t gqa_workspace_bytes(int64_t n_heads, int64_t len, int group)
{
    auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    const int64_t tiles = (len + kTileRows - 1) / kTileRows;
    return up(n_heads * len * group * 4) + up(n_heads * tiles * group * 4 * 8) +
           up(n_heads * group * 16) + up(n_heads * kBopBytesPerHead);
}

void gqa_workspace_views(void* workspace, int64_t n_heads, int64_t len, int group, float** raw,
                         double** partial, double2** stats)
{
    auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    const int64_t tiles = (len + kTileRows - 1) / kTileRows;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    *raw = reinterpret_cast<float*>(ws);
    *partial = reinterpret_cast<double*>(ws + up(n_heads * len * group * 4));
    *stats = reinterpret_cast<double2*>(ws + up(n_heads * len * group * 4) +
                                        up(n_heads * tiles * group * 4 * 8));
}

hipError_t launch_gqa_stats(int group, const double* partial, int len, int n_heads,
                            double2* stats, hipStream_t stream)
{
    if (len <= 0 || n_heads <= 0) return hipSuccess;
    const int tiles = (len + kTileRows - 1) / kTileRows;
    hipLaunchKernelGGL(gqa_stats_kernel, dim3(n_heads), dim3(64), 0, stream, partial, tiles, group,
                       len, nullptr, stats);
    return hipGetLastError();
}

hipError_t launch_gqa_normalize(int group, const float* raw, const double2* stats, int len,
                                int n_heads, float* scores, hipStream_t stream)
{
    if (len <= 0 || n_heads <= 0) return hipSuccess;
    const int tiles = (len + kTileRows - 1) / kTileRows;
    const int64_t grid = (int64_t)tiles * n_heads;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
#define TRI_NORM_CASE(G)                                                                          \
    case G:                                                                                       \
        hipLaunchKernelGGL((gqa_norm_kernel<G>), dim3((unsigned)grid), dim3(kBlock), 0, stream,   \
                           raw, stats, len, tiles, scores, nullptr);                              \
        break;
    switch (group) {
        TRI_NORM_CASE(2)
        TRI_NORM_CASE(3)
        TRI_NORM_CASE(4)
        TRI_NORM_CASE(5)
        TRI_NORM_CASE(6)
        TRI_NORM_CASE(7)
        TRI_NORM_CASE(8)
    default: return hipErrorInvalidValue;
    }
#undef TRI_NORM_CASE
    return hipGetLastError();
}

hipError_t launch_gqa_score(tri_dtype dtype, int head_dim, int group, const void* k, int64_t cap,
                            int len, int n_heads, int64_t p_now, const double* omega,
                            const double2* qa, const float* w, void* workspace, float* scores,
                            const int32_t* head_len, hipStream_t stream)
{
    if (len <= 0 || n_heads <= 0) return hipSuccess;
    // the matrix-core kernel addresses a head's rows with 32-bit buffer offsets
    if (dtype == TRI_BF16 && (int64_t)len * head_dim * 2 >= (int64_t(1) << 31))
        return hipErrorInvalidValue;
    auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    const int64_t tiles = (len + kTileRows - 1) / kTileRows;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* raw = reinterpret_cast<float*>(ws);
    double* partial = reinterpret_cast<double*>(ws + up((int64_t)n_heads * len * group * 4));
    double2* stats = reinterpret_cast<double2*>(ws + up((int64_t)n_heads * len * group * 4) +
                                                up((int64_t)n_heads * tiles * group * 4 * 8));
    u32x4* bops = reinterpret_cast<u32x4*>(ws + up((int64_t)n_heads * len * group * 4) +
                                           up((int64_t)n_heads * tiles * group * 4 * 8) +
                                           up((int64_t)n_heads * group * 16));
    if (dtype == TRI_BF16 && head_dim == 128)
        return launch_d<128, true>(group, k, cap, len, n_heads, p_now, omega, qa, w, raw, partial,
                                   stats, scores, head_len, bops, stream);
    if (dtype == TRI_F32 && head_dim == 64)
        return launch_d<64, false>(group, k, cap, len, n_heads, p_now, omega, qa, w, raw, partial,
                                   stats, scores, head_len, bops, stream);
    if (dtype == TRI_BF16 && head_dim == 64)
        return launch_d<64, true>(group, k, cap, len, n_heads, p_now, omega, qa, w, raw, partial,
                                  stats, scores, head_len, bops, stream);
    if (dtype == TRI_F32 && head_dim == 128)
        return launch_d<128, false>(group, k, cap, len, n_heads, p_now, omega, qa, w, raw, partial,
                                    stats, scores, head_len, bops, stream);
    return hipErrorInvalidValue;
}

}  // namespace tri
