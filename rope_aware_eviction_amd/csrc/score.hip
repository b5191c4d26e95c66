// Fused key-score kernel: per cached key, the offset-averaged trigonometric
// distance-preference series plus the concentration-weighted norm term.
//
// Source: romaanj.github.io "TriAttention" review, section "Method" (trig
// term per band |E q_f| |k_f| cos(w_f * distance + phase difference), norm
// term weighted by (1 - R_f), averaging over future offsets);
// dimensionstp.github.io review, section 2-2 (RoPE logit as a per-band
// cosine series of the query-key distance) and section 3-2 items 2)-4).
//
// Algebra.  With the stored (post-RoPE) band K_f = k_f * e^{i w_f p}, the
// un-rotation e^{-i w_f p} and the distance factor e^{i w_f (p_now + delta - p)}
// cancel in p, so
//     trig = sum_f Re( C_f * conj(K_f) ),  C_f = E[q_f] * A_f * e^{i w_f p_now},
// i.e. the plain dot product of u = [Re C ; Im C] with the stored row, and
// |k_f| = |K_f|.  C_f is folded in fp64 (w_0 * p_now reaches 1e5 rad, where
// an fp32 angle would be off by ~1e-2 rad) and rounded to fp32 once per
// workgroup; each key then costs d FMAs for the dot product, d/2 band
// energies, d/2 square roots and d/2 FMAs for the norm term, in fp32.
//
// Layout.  A row of head_dim elements is two halves (real parts, imaginary
// parts).  LPR lanes cover one row; lane j loads 16 bytes of each half at
// byte offset 16*j, so one wave instruction reads 64/LPR whole half-rows,
// fully coalesced 128-byte lines, and every lane holds matching real and
// imaginary parts of E = 16/elem_size bands: no cross-lane exchange is needed
// until the final row sum, which is a DPP butterfly within the LPR lanes.
#include "tri_internal.h"

namespace tri {
namespace {

constexpr int kBlock = 256;      // threads per workgroup
// Rows of one head per workgroup: at least kMinTileRows, and whole batches
// of kUnroll rows per lane (see TileRows).  Measured on the 36 x 8 x 32768
// bf16 cache: 371 us with 128-row tiles, 381 with 256, 385 with 512, 386
// with 1024; 64 rows with 2 rows per lane in flight take 385 us, 256 rows
// with 8 in flight 389.
constexpr int kMinTileRows = 128;
constexpr int kUnroll = 4;       // rows per lane kept in flight
constexpr int kLineFloats = 32;            // scores per 128-byte cache line
constexpr int kBufferWord3 = 0x00020000;   // raw buffer resource word 3, gfx9 family
constexpr int kSC1 = 16;                   // cache-policy bits: sc1

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
    static_assert(LPR == 4 || LPR == 8 || LPR == 16 || LPR == 32, "lanes per row");
    x += dpp<0xB1>(x);                          // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp<0x4E>(x);                          // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (LPR >= 8) x += dpp<0x141>(x);   // row_half_mirror: quads of an 8-lane half
    if constexpr (LPR >= 16) x += dpp<0x140>(x);  // row_mirror: halves of a 16-lane row
    if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
    return x;
}

template <bool BF16>
struct Elem;

template <>
struct Elem<true> {
    static constexpr int kSize = 2;
    // 16 bytes = 8 bf16; element 2m sits in the low half of word m.
    __device__ static __forceinline__ void unpack(const u32x4& v, float* out)
    {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            out[2 * m] = __uint_as_float(w[m] << 16);
            out[2 * m + 1] = __uint_as_float(w[m] & 0xFFFF0000u);
        }
    }
};

template <>
struct Elem<false> {
    static constexpr int kSize = 4;
    __device__ static __forceinline__ void unpack(const u32x4& v, float* out)
    {
        out[0] = __uint_as_float(v.x);
        out[1] = __uint_as_float(v.y);
        out[2] = __uint_as_float(v.z);
        out[3] = __uint_as_float(v.w);
    }
};

// A row is LPR lanes (16 bytes of each half per lane); a workgroup step
// covers kBlock / LPR rows and a batch kUnroll steps.  The tile is one
// batch, or kMinTileRows when a batch is smaller (then a tile is whole
// batches).
template <int D, bool BF16>
struct TileRows {
    static constexpr int kLpr = D * Elem<BF16>::kSize / 2 / 16;
    static constexpr int kBatch = kBlock / kLpr * kUnroll;
    static constexpr int value = kBatch >= kMinTileRows ? kBatch : kMinTileRows;
    static_assert(value % kBatch == 0, "a tile is whole batches");
};

template <int D, bool BF16>
__global__ __launch_bounds__(kBlock) void score_kernel(
    const unsigned char* __restrict__ k, int64_t cap, int len, int tiles_per_head, int lead_tile,
    double p_now,
    const double* __restrict__ omega, const double2* __restrict__ qa, const float* __restrict__ w,
    float* __restrict__ scores, const int32_t* __restrict__ head_len)
{
    constexpr int kHalf = D / 2;
    constexpr int kElem = Elem<BF16>::kSize;
    constexpr int kRowBytes = D * kElem;
    constexpr int kHalfBytes = kRowBytes / 2;
    constexpr int LPR = kHalfBytes / 16;   // lanes per row
    constexpr int E = 16 / kElem;          // bands per lane
    constexpr int G = kBlock / LPR;        // rows per workgroup step
    constexpr int kTileRows = TileRows<D, BF16>::value;
    static_assert(kTileRows % (G * kUnroll) == 0, "rows of every batch stay inside the tile");

    __shared__ float s_u[D];
    __shared__ float s_w[kHalf];
    __shared__ float s_out[kTileRows];

    const int head = blockIdx.x / tiles_per_head;
    const int tile = blockIdx.x - head * tiles_per_head;
    // rows in use of this head: all `len`, or its own length (ragged heads)
    const int n_h = head_len ? max(0, min(head_len[head], len)) : len;
    float* out = scores + (size_t)head * (size_t)len;
    // Tile boundaries fall on 128-byte lines of the score array, so every
    // line is written, whole, by one workgroup: a line that two workgroups
    // write in parts measured 4% slower over the whole kernel (heads of
    // 32,751 keys against 32,768).  When a head's scores do not start on a
    // line (lead_tile), tile 0 takes the rows up to its first line boundary
    // and tile t >= 1 the kTileRows rows after tile t - 1.
    int tile_start = tile * kTileRows, tile_stop = tile_start + kTileRows;
    if (lead_tile) {
        const int lead = (kLineFloats - (int)(((uintptr_t)out >> 2) % kLineFloats)) % kLineFloats;
        tile_start = tile == 0 ? 0 : lead + (tile - 1) * kTileRows;
        tile_stop = tile == 0 ? lead : tile_start + kTileRows;
    }
    const int row_end = min(n_h, tile_stop);
    if (tile_start >= row_end) return;   // whole workgroup: nothing of this head here
    const int tid = threadIdx.x;
    const int j = tid % LPR;   // lane within the row
    const int g = tid / LPR;   // row group within the workgroup
    const unsigned char* base = k + (size_t)head * (size_t)cap * kRowBytes + 16 * j;

    // K is streamed once: non-temporal loads keep it from displacing the
    // scores and constants in the caches.  Rows past the end of the tile
    // re-read its last row (in bounds, cache hits; their sums are dropped).
    u32x4 re[kUnroll], im[kUnroll];
    auto load_row = [&](int u, int row) {
        const u32x4* p = reinterpret_cast<const u32x4*>(base + (size_t)min(row, row_end - 1) * kRowBytes);
        re[u] = __builtin_nontemporal_load(p);
        im[u] = __builtin_nontemporal_load(p + kHalfBytes / 16);
    };
    const int iters = (row_end - tile_start + G * kUnroll - 1) / (G * kUnroll);   // uniform
    int r0 = tile_start + g;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) load_row(u, r0 + u * G);   // in flight during the fold

    // fold C_f = E[q_f] * A_f * e^{i w_f p_now} in fp64, once per workgroup
    if (tid < kHalf) {
        double sn, cs;
        sincos(omega[tid] * p_now, &sn, &cs);
        const double2 a = qa[(size_t)head * kHalf + tid];
        s_u[tid] = (float)(a.x * cs - a.y * sn);
        s_u[tid + kHalf] = (float)(a.x * sn + a.y * cs);
        s_w[tid] = w[(size_t)head * kHalf + tid];
    }
    __syncthreads();
    float u_re[E], u_im[E], wt[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        u_re[e] = s_u[j * E + e];
        u_im[e] = s_u[kHalf + j * E + e];
        wt[e] = s_w[j * E + e];
    }

    // Scores of the tile are staged in LDS and leave in one coalesced sweep
    // at the end: a store inside the loop would share the in-order memory
    // counter with the row loads, so every wait for a row would also wait
    // for earlier partial-line score writes to be acknowledged.
    // Rolling pipeline: as soon as row u of this batch is consumed, the same
    // registers start loading row u of the next batch, so every wave keeps
    // kUnroll - 1 to kUnroll rows in flight while it computes.
    for (int it = 0; it < iters; ++it) {
        const int r_next = r0 + G * kUnroll;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float a[E], b[E];
            Elem<BF16>::unpack(re[u], a);
            Elem<BF16>::unpack(im[u], b);
            load_row(u, r_next + u * G);
            // keep the scheduler from regrouping the stages (it would drain
            // every load first and issue the next batch after the compute)
            __builtin_amdgcn_sched_barrier(0);
            float dot = 0.f, nrm = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                dot = fmaf(u_re[e], a[e], dot);
                dot = fmaf(u_im[e], b[e], dot);
                const float energy = fmaf(a[e], a[e], b[e] * b[e]);
                nrm = fmaf(wt[e], __builtin_amdgcn_sqrtf(energy), nrm);
            }
            const float total = group_sum<LPR>(dot + nrm);
            if (j == 0) s_out[r0 + u * G - tile_start] = total;   // row < tile_start + kTileRows
            __builtin_amdgcn_sched_barrier(0);
        }
        r0 = r_next;
    }
    __syncthreads();
    // sc1 stores: measured to cost the read stream far less than default
    // write-back stores, while the scores stay cached for the selection
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(out, 0, len * 4, kBufferWord3);
    // A row with an infinite or NaN element has no score: any non-finite
    // total (an infinite element alone gives +inf or -inf) is stored as NaN,
    // which every selection ranks below all numbers.
    for (int i = tid; i < row_end - tile_start; i += kBlock) {
        uint32_t x = __float_as_uint(s_out[i]);
        if ((x & 0x7F800000u) == 0x7F800000u) x = 0x7FC00000u;
        __builtin_amdgcn_raw_buffer_store_b32(x, ro, (tile_start + i) * 4, 0, kSC1);
    }
}

template <int D, bool BF16>
hipError_t launch(const void* k, int64_t cap, int len, int n_heads, int64_t p_now,
                  const double* omega, const double2* qa, const float* w, float* scores,
                  const int32_t* head_len, hipStream_t stream)
{
    constexpr int kTileRows = TileRows<D, BF16>::value;
    // a lead tile per head unless every head's scores start on a line (len a
    // multiple of the line and the array line-aligned)
    const int lead_tile = (len % kLineFloats != 0 ||
                           ((uintptr_t)scores >> 2) % kLineFloats != 0) ? 1 : 0;
    const int tiles = (len + kTileRows - 1) / kTileRows + lead_tile;
    const int64_t grid = (int64_t)tiles * n_heads;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((score_kernel<D, BF16>), dim3((unsigned)grid), dim3(kBlock), 0, stream,
                       static_cast<const unsigned char*>(k), cap, len, tiles, lead_tile, (double)p_now, omega,
                       qa, w, scores, head_len);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_score(tri_dtype dtype, int head_dim, const void* k, int64_t cap, int len,
                        int n_heads, int64_t p_now, const double* omega, const double2* qa,
                        const float* w, float* scores, const int32_t* head_len, hipStream_t stream)
{
    if (len <= 0 || n_heads <= 0) return hipSuccess;
    if (dtype == TRI_BF16 && head_dim == 128)
        return launch<128, true>(k, cap, len, n_heads, p_now, omega, qa, w, scores, head_len, stream);
    if (dtype == TRI_F32 && head_dim == 64)
        return launch<64, false>(k, cap, len, n_heads, p_now, omega, qa, w, scores, head_len, stream);
    if (dtype == TRI_BF16 && head_dim == 64)
        return launch<64, true>(k, cap, len, n_heads, p_now, omega, qa, w, scores, head_len, stream);
    if (dtype == TRI_F32 && head_dim == 128)
        return launch<128, false>(k, cap, len, n_heads, p_now, omega, qa, w, scores, head_len, stream);
    return hipErrorInvalidValue;
}

}  // namespace tri
