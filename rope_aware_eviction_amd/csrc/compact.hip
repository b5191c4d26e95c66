// Stable in-place eviction: rows r < B of K, V and positions become the rows
// at kept[r].
//
// Source: dimensionstp.github.io "TriAttention ... Review", section 3-2
// item 5 (keep the top-budget keys, evict the rest) and section 6 item 1
// (cache compaction is part of the kernel work the method needs).
//
// Hazard.  kept[] is strictly ascending, so kept[r] >= r: row r is only ever
// filled from itself or from a later row, and writing row r can only destroy
// a source needed by a destination r' <= r.  Destinations are processed in
// ascending tiles of T rows: tile t reads rows >= tT and writes rows
// [tT, (t+1)T).  Its writes may destroy sources of tiles <= t only, so a
// tile is written once the reads of every tile up to it have landed; reads
// of later tiles never touch rows written so far.  A workgroup owns one
// (head, K or V) stream at a time and walks its tiles in order, then takes
// its next stream; positions travel with K.
//
// Pipeline.  The loads of tile t+1 are issued before the stores of tile t,
// then the workgroup waits until those loads (not the stores, which share
// the in-order memory counter) have landed and meets at a barrier.  Every
// load and store is an unconditional bounds-checked buffer access (rows that
// need no move get an offset past the buffer, which the hardware drops), so
// the number of memory instructions per tile is fixed and the wait can
// count them exactly.  The head's kept list is staged in LDS so index reads
// stay off the memory counter.  Rows are moved with non-temporal accesses:
// every byte is touched once.
//
// Counted lists (head-specific budgets) differ in length from head to head,
// by up to the whole shared total, so a fixed assignment of streams to
// workgroups leaves most of them idle while a few move the long streams.
// There every stream is cut into 128-byte column parts of its rows (a row's
// column c only ever comes from column c of another row, so the parts are
// independent and each keeps the hazard rule above on its own), a small
// kernel orders the parts by size class (largest first) and the workgroups
// take parts from that order through an atomic counter: the longest parts
// start first and the short ones fill in.
#include <algorithm>
#include <mutex>

#include "tri_internal.h"

// Scratch memory of the allocation-free counted compaction
// (tri_compact_kv_counts_noalloc): the queue of column parts of up to
// tri::kScratchHeads (layer, KV head) streams.  One copy per GPU, alive until
// the process ends.  Host code never uses this name as an address: the
// device address of each GPU's copy comes from hipGetSymbolAddress
// (tri::scratch_address).
static __device__ __align__(256) uint32_t scratch[2 + 2 * 4 * tri::kScratchHeads];

namespace tri {
namespace {

constexpr int kBlock = 1024;
constexpr int kUnroll = 8;
constexpr int kIdxChunk = 8192;                 // kept entries staged in LDS at a time
constexpr uint32_t kDrop = 0xFFFFFFC0u;          // buffer offset that is always out of range
constexpr int kBufferWord3 = 0x00020000;         // raw buffer resource word 3, gfx9 family
constexpr int kNT = 2;                           // cache-policy bits: non-temporal
// sequences per launch of the batched compaction (the table travels in the
// kernel arguments: 40 bytes per sequence)
constexpr int kCompactBatch = 32;

// s_waitcnt with only the vector-memory count bounded (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Moves one column part (PARTS = 1: the whole rows) of one K or V stream in
// place: rows r < n_keep become the rows at idx[r] (strictly ascending, in
// [0, len)); with moves_pos the positions move with them.  Every thread of
// the workgroup calls it; s_idx is the workgroup's LDS index buffer.
template <int ROWB, int PARTS>
__device__ __forceinline__ void move_stream(unsigned char* __restrict__ rows,
                                            int32_t* __restrict__ hpos,
                                            const int32_t* __restrict__ idx, int n_keep, int len,
                                            int part, bool moves_pos, int32_t* s_idx)
{
    constexpr int kChunks = ROWB / 16;                  // 16-byte chunks per row
    constexpr int kCpp = kChunks / PARTS;               // chunks per column part
    static_assert(kCpp * PARTS == kChunks, "parts split the row evenly");
    constexpr int kRowsPerStep = kBlock / kCpp;
    constexpr int kTile = kRowsPerStep * kUnroll;
    constexpr int kPosPerThread = (kTile + kBlock - 1) / kBlock;
    constexpr int kStores = kUnroll + kPosPerThread;    // memory stores per thread per tile
    static_assert(kIdxChunk % kTile == 0, "tiles never straddle an index chunk");

    const __amdgpu_buffer_rsrc_t rrows =
        __builtin_amdgcn_make_buffer_rsrc(rows, 0, len * ROWB, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rpos =
        __builtin_amdgcn_make_buffer_rsrc(hpos, 0, len * 4, kBufferWord3);

    const int tid = threadIdx.x;
    const int c = part * kCpp + tid % kCpp;
    const int rs = tid / kCpp;

    // one tile's data in flight: rows, their destinations, positions
    struct Tile {
        u32x4 buf[kUnroll];
        uint32_t dst[kUnroll];
        uint32_t pval[kPosPerThread];
        uint32_t pdst[kPosPerThread];
    };
    Tile ta, tb;

    auto load = [&](Tile& t, int t0, int c0) {
        // all of the tile's indices first, so the LDS reads overlap
        int srcs[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int r = t0 + u * kRowsPerStep + rs;
            srcs[u] = s_idx[min(r, c0 + kIdxChunk - 1) - c0];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int r = t0 + u * kRowsPerStep + rs;
            const int src = r < n_keep ? srcs[u] : r;
            const bool mv = r < n_keep && src != r && (unsigned)src < (unsigned)len;
            const uint32_t from = mv ? (uint32_t)src * ROWB + 16u * c : kDrop;
            t.dst[u] = mv ? (uint32_t)r * ROWB + 16u * c : kDrop;
            t.buf[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rrows, from, 0, kNT));
        }
#pragma unroll
        for (int q = 0; q < kPosPerThread; ++q) {
            const int i = q * kBlock + tid;
            const int r = t0 + i;
            const int src = (i < kTile && r < n_keep) ? s_idx[r - c0] : r;
            const bool mv = moves_pos && i < kTile && r < n_keep && src != r && (unsigned)src < (unsigned)len;
            t.pdst[q] = mv ? (uint32_t)r * 4u : kDrop;
            t.pval[q] = __builtin_amdgcn_raw_buffer_load_b32(rpos, mv ? (uint32_t)src * 4u : kDrop, 0, 0);
        }
    };
    auto store = [&](const Tile& t) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            __builtin_amdgcn_raw_buffer_store_b128(t.buf[u], rrows, t.dst[u], 0, kNT);
#pragma unroll
        for (int q = 0; q < kPosPerThread; ++q)
            __builtin_amdgcn_raw_buffer_store_b32(t.pval[q], rpos, t.pdst[q], 0, 0);
    };

    for (int c0 = 0; c0 < n_keep; c0 += kIdxChunk) {
        const int c1 = min(n_keep, c0 + kIdxChunk);
        __syncthreads();                               // previous chunk's index reads done
        for (int i = c0 + tid; i < c1; i += kBlock) s_idx[i - c0] = idx[i];
        __syncthreads();
        const int n_tiles = (c1 - c0 + kTile - 1) / kTile;
        load(ta, c0, c0);
        wait_vmcnt<0>();
        __syncthreads();
        // tiles alternate between the two register sets
        // (the scheduling barriers keep every load of the next tile ahead of
        // the stores, which the exact wait count relies on)
        for (int t = 0; t < n_tiles; t += 2) {
            const int t0 = c0 + t * kTile;
            if (t + 1 < n_tiles) load(tb, t0 + kTile, c0);
            __builtin_amdgcn_sched_barrier(0);
            store(ta);
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<kStores>();                     // tile t+1's reads have landed
            __syncthreads();
            if (t + 1 >= n_tiles) break;
            if (t + 2 < n_tiles) load(ta, t0 + 2 * kTile, c0);
            __builtin_amdgcn_sched_barrier(0);
            store(tb);
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<kStores>();
            __syncthreads();
        }
    }
}

template <int ROWB, int PARTS>
__global__ __launch_bounds__(kBlock) void compact_kernel(unsigned char* __restrict__ k,
                                                         unsigned char* __restrict__ v,
                                                         int32_t* __restrict__ pos, int64_t cap,
                                                         int len,
                                                         const int32_t* __restrict__ kept,
                                                         int budget, int kept_stride, int n_heads,
                                                         const int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ head_len,
                                                         uint32_t* __restrict__ queue)
{
    __shared__ int32_t s_idx[kIdxChunk];
    __shared__ int s_item;

    // queue: [0] the counter, [1] the number of parts, [2..] their order
    const int n_items = queue ? (int)queue[1] : 2 * n_heads * PARTS;
    auto next_item = [&](int item) {
        if (!queue) return item + (int)gridDim.x;
        __syncthreads();                                   // every thread has read s_item
        if (threadIdx.x == 0) s_item = (int)atomicAdd(&queue[0], 1u);
        __syncthreads();
        return s_item;
    };
    for (int item = queue ? next_item(0) : (int)blockIdx.x; item < n_items; item = next_item(item)) {
        const int work = queue ? (int)queue[2 + item] : item;
        const int stream_id = work / PARTS;
        const int part = work - stream_id * PARTS;
        const int head = stream_id >> 1;
        const bool is_v = (stream_id & 1) != 0;
        const bool moves_pos = !is_v && part == 0;      // positions travel with K's first part
        // rows this head keeps: `budget`, or its own count (-1: the head is
        // left as it is; head_len takes the new count)
        const int n_keep = counts ? min(counts[head], kept_stride) : budget;
        if (n_keep < 0) continue;
        if (counts && moves_pos && threadIdx.x == 0) head_len[head] = n_keep;
        move_stream<ROWB, PARTS>((is_v ? v : k) + (size_t)head * (size_t)cap * ROWB,
                                 pos + (size_t)head * (size_t)cap,
                                 kept + (size_t)head * (size_t)kept_stride, n_keep, len, part,
                                 moves_pos, s_idx);
    }
}

// A ragged batch of sequences with uniform budgets in one launch: the K and
// V streams of every head of every sequence in the table, all `budget` rows
// long, taken by the workgroups in turn (stream i by workgroup i mod grid).
struct CompactSeq {
    unsigned char* k;
    unsigned char* v;
    int32_t* pos;
    const int32_t* kept;   // the sequence's kept lists, [heads][budget]
    int32_t cap;
    int32_t len;
};
struct CompactBatch {
    CompactSeq seq[kCompactBatch];
};

template <int ROWB>
__global__ __launch_bounds__(kBlock) void compact_batch_kernel(const CompactBatch b, int n_seq,
                                                               int n_heads, int budget)
{
    __shared__ int32_t s_idx[kIdxChunk];
    const int per_seq = 2 * n_heads;
    const int items = n_seq * per_seq;
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int s = item / per_seq;
        const int stream_id = item - s * per_seq;
        const int head = stream_id >> 1;
        const bool is_v = (stream_id & 1) != 0;
        const int64_t cap = b.seq[s].cap;
        move_stream<ROWB, 1>((is_v ? b.seq[s].v : b.seq[s].k) + (size_t)head * (size_t)cap * ROWB,
                             b.seq[s].pos + (size_t)head * (size_t)cap,
                             b.seq[s].kept + (size_t)head * (size_t)budget, budget, b.seq[s].len, 0,
                             !is_v, s_idx);
    }
}

// Orders the column parts of the K and V streams of heads with a count >= 0
// by size class (bit length of the count), largest first, into queue[2..];
// queue[1] gets their number and the counter queue[0] is cleared.  Work item
// w is part w % parts of stream w / parts.  One workgroup.
__global__ __launch_bounds__(kBlock) void order_kernel(const int32_t* __restrict__ counts,
                                                       int n_heads, int parts,
                                                       uint32_t* __restrict__ queue)
{
    __shared__ uint32_t s_start[33];
    const int tid = threadIdx.x;
    if (tid < 33) s_start[tid] = 0u;
    __syncthreads();
    auto cls = [](int c) { return c <= 0 ? 0 : 32 - __clz(c); };   // 0..31
    const int items = 2 * n_heads * parts;
    for (int i = tid; i < items; i += kBlock) {
        const int c = counts[(i / parts) >> 1];
        if (c >= 0) atomicAdd(&s_start[cls(c)], 1u);
    }
    __syncthreads();
    if (tid == 0) {
        uint32_t at = 0u;
        for (int b = 31; b >= 0; --b) {
            const uint32_t m = s_start[b];
            s_start[b] = at;
            at += m;
        }
        queue[0] = 0u;
        queue[1] = at;
    }
    __syncthreads();
    for (int i = tid; i < items; i += kBlock) {
        const int c = counts[(i / parts) >> 1];
        if (c >= 0) queue[2 + atomicAdd(&s_start[cls(c)], 1u)] = (uint32_t)i;
    }
}

template <int ROWB>
hipError_t launch(void* k, void* v, int32_t* pos, int64_t cap, int len, int n_heads,
                  const int32_t* kept, int budget, int kept_stride, const int32_t* counts,
                  int32_t* head_len, uint32_t* queue, hipStream_t stream)
{
    // Each workgroup walks whole K or V streams one after another, at most
    // one workgroup per compute unit, every workgroup the same number of
    // streams.  Measured on the 36 x 8 x 32768 cache (576 streams of 4096
    // rows): 192 workgroups of three streams move the rows in 225 us, one
    // 512-thread workgroup per stream in 250 us, and more streams in flight
    // at once is slower still.  On the 32 x 8 x 8192 cache (512 streams of
    // 2048 rows) 256 workgroups of two streams take 98 us (one per stream:
    // 97.5 us).
    // compute units of the current device (a cheap query, done per call so
    // that every device gets its own count)
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return hipErrorInvalidDevice;
    const int streams = 2 * n_heads;
    if (queue) {
        // counted lists: 128-byte column parts taken in order by workgroups
        // on three quarters of the compute units.  Measured on the 36 x 8 x
        // 32768 cache with head-specific budgets (floor 1024): 192
        // workgroups move the rows in 232 us, 160 in 242, 224 in 244, 256
        // in 254 and 128 in 268; whole streams instead of column parts
        // (one per workgroup in turn) take 333 us.
        constexpr int kParts = ROWB / 128;
        hipLaunchKernelGGL(order_kernel, dim3(1), dim3(kBlock), 0, stream, counts, n_heads,
                           kParts, queue);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int workers = std::max(1, cus * 3 / 4);
        hipLaunchKernelGGL((compact_kernel<ROWB, kParts>), dim3(std::min(streams * kParts, workers)),
                           dim3(kBlock), 0, stream, static_cast<unsigned char*>(k),
                           static_cast<unsigned char*>(v), pos, cap, len, kept, budget,
                           kept_stride, n_heads, counts, head_len, queue);
        return hipGetLastError();
    }
    const int per_block = (streams + cus - 1) / cus;
    const int grid = (streams + per_block - 1) / per_block;
    hipLaunchKernelGGL((compact_kernel<ROWB, 1>), dim3(grid), dim3(kBlock), 0, stream,
                       static_cast<unsigned char*>(k), static_cast<unsigned char*>(v), pos, cap,
                       len, kept, budget, kept_stride, n_heads, counts, head_len, queue);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_compact_batch(int row_bytes, int n_seq, void* const* k, void* const* v,
                                int32_t* const* pos, const int* cap, const int* len,
                                const int32_t* const* kept, int n_heads, int budget,
                                hipStream_t stream)
{
    if (n_heads <= 0 || budget <= 0 || n_seq <= 0) return hipSuccess;
    for (int s = 0; s < n_seq; ++s)
        if ((int64_t)len[s] * row_bytes >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return hipErrorInvalidDevice;
    for (int s0 = 0; s0 < n_seq; s0 += kCompactBatch) {
        const int cnt = std::min(kCompactBatch, n_seq - s0);
        const int64_t streams = (int64_t)cnt * 2 * n_heads;
        if (streams > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        CompactBatch b{};
        for (int j = 0; j < cnt; ++j) {
            const int s = s0 + j;
            b.seq[j] = CompactSeq{static_cast<unsigned char*>(k[s]), static_cast<unsigned char*>(v[s]),
                                  pos[s], kept[s], cap[s], len[s]};
        }
        // streams of equal length taken in turn by workgroups on three
        // quarters of the compute units (as for one sequence, fewer copy
        // streams in flight move the rows faster)
        const int grid = (int)std::min<int64_t>(streams, std::max(1, cus * 3 / 4));
        switch (row_bytes) {
        case 128: hipLaunchKernelGGL(compact_batch_kernel<128>, dim3(grid), dim3(kBlock), 0, stream, b, cnt, n_heads, budget); break;
        case 256: hipLaunchKernelGGL(compact_batch_kernel<256>, dim3(grid), dim3(kBlock), 0, stream, b, cnt, n_heads, budget); break;
        case 512: hipLaunchKernelGGL(compact_batch_kernel<512>, dim3(grid), dim3(kBlock), 0, stream, b, cnt, n_heads, budget); break;
        default: return hipErrorInvalidValue;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// counter, item count and one entry per column part (at most 512 / 128 per stream)
int64_t compact_queue_bytes(int64_t n_heads) { return 8 + 4 * 2 * 4 * n_heads; }

static_assert(sizeof(scratch) == 8 + 4 * 2 * 4 * kScratchHeads, "scratch holds the queue of kScratchHeads");

int64_t scratch_bytes() { return (int64_t)sizeof(scratch); }

// Device address of the current device's copy of `scratch`, looked up once
// per device (the first call with that device current) and kept.
hipError_t scratch_address(int device, void** out)
{
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    *out = nullptr;
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device]) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[device] = p;
    }
    *out = addr[device];
    return hipSuccess;
}

hipError_t launch_compact(int row_bytes, void* k, void* v, int32_t* pos, int64_t cap, int len,
                          int n_heads, const int32_t* kept, int budget, int kept_stride,
                          const int32_t* counts, int32_t* head_len, uint32_t* queue,
                          hipStream_t stream)
{
    if (n_heads <= 0 || kept_stride <= 0 || (!counts && budget <= 0)) return hipSuccess;
    if (counts && (!head_len || !queue)) return hipErrorInvalidValue;
    // buffer offsets are 32-bit: a head's rows must span less than 2 GiB
    if ((int64_t)len * row_bytes >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    switch (row_bytes) {
    case 128: return launch<128>(k, v, pos, cap, len, n_heads, kept, budget, kept_stride, counts,
                                 head_len, queue, stream);
    case 256: return launch<256>(k, v, pos, cap, len, n_heads, kept, budget, kept_stride, counts,
                                 head_len, queue, stream);
    case 512: return launch<512>(k, v, pos, cap, len, n_heads, kept, budget, kept_stride, counts,
                                 head_len, queue, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace tri
