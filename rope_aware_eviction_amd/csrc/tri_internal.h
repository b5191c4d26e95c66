// Internal declarations shared by the HIP translation units of libtri.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tri.h"

struct tri_ctx {
    int device;
    int n_layers;
    int n_kv_heads;
    int head_dim;
    int n_heads;          // n_layers * n_kv_heads
    int group;            // query heads per KV head (1: one query table per KV head)
    double* omega;        // device [head_dim/2]        band frequencies
    double2* qa;          // device [n_heads][group][head_dim/2] E[q_f] * A_f (complex, fp64)
    float* w;             // device [n_heads][group][head_dim/2] (1 - R_f) * E|q_f|
    double2* qc;          // device [n_heads][group][head_dim/2] E[q_f] as loaded (complex, fp64)
    void* scratch;        // device address of this device's static scratch (allocation-free calls)
};

namespace tri {

// 16-byte native vector: loads and stores of it are single dwordx4 memory
// instructions, and arrays of it stay in registers.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Launchers (one per kernel family).  Each enqueues on `stream` and returns
// the launch's hipError_t.

hipError_t launch_calibrate(int n_heads, int head_dim, double rope_theta, const double* inv_freq,
                            const int64_t* offsets, int n_offsets, const double* qc_re,
                            const double* qc_im, const double* q_mean_norm, const double* q_mrl,
                            double* omega, double2* qa, float* w, hipStream_t stream);

// Per-band calibration statistics of n_heads query heads from samples
// [n_samples][n_heads][head_dim].
hipError_t launch_calib_stats(tri_dtype dtype, int head_dim, const void* q, int64_t n_samples,
                              int n_heads, double* qc_re, double* qc_im, double* mean_norm,
                              double* mrl, hipStream_t stream);

// Distance-preference curves: one thread per (query head, distance).
hipError_t launch_distance_curve(int n_q_heads, int group, int head_dim, const double* omega,
                                 const double2* qc, const double* kc_re, const double* kc_im,
                                 const int64_t* deltas, int n_delta, double* curve,
                                 hipStream_t stream);

// Scores rows [0, len) of n_heads heads of one sequence.
hipError_t launch_score(tri_dtype dtype, int head_dim, const void* k, int64_t cap, int len,
                        int n_heads, int64_t p_now, const double* omega, const double2* qa,
                        const float* w, float* scores, const int32_t* head_len,
                        hipStream_t stream);

// GQA (group >= 2): G raw scores per key, per-query-head statistics, then
// the normalized max into `scores`.  `workspace` holds gqa_workspace_bytes.
int64_t gqa_workspace_bytes(int64_t n_heads, int64_t len, int group);
hipError_t launch_gqa_score(tri_dtype dtype, int head_dim, int group, const void* k, int64_t cap,
                            int len, int n_heads, int64_t p_now, const double* omega,
                            const double2* qa, const float* w, void* workspace, float* scores,
                            const int32_t* head_len, hipStream_t stream);
// The raw scores [n_heads][len][group], per-tile partial sums
// [n_heads][tiles][group][4] and statistics [n_heads][group] in a GQA
// workspace laid out by launch_gqa_score (scores == nullptr there stops after
// the raw scores and partial sums: launch_gqa_stats then forms the
// statistics); launch_gqa_normalize writes the normalized scores of such a
// workspace.
void gqa_workspace_views(void* workspace, int64_t n_heads, int64_t len, int group, float** raw,
                         double** partial, double2** stats);
hipError_t launch_gqa_stats(int group, const double* partial, int len, int n_heads,
                            double2* stats, hipStream_t stream);
hipError_t launch_gqa_normalize(int group, const float* raw, const double2* stats, int len,
                                int n_heads, float* scores, hipStream_t stream);
// Top-`budget` of heads of len <= 32768 keys, keyed by the normalized GQA
// score formed from a workspace's raw scores and per-tile partial sums (each
// workgroup forms its head's statistics as the statistics kernel does).
hipError_t launch_select_gqa(int group, const float* raw, const double* partial, int len,
                             int n_heads, int budget, int32_t* kept, int kept_stride,
                             hipStream_t stream);

// Top-`budget` of each of n_heads score rows of length n.
// Heads of `n` keys (stride n; with head_len, head h has its own length up
// to n and heads of at most `budget` keys get no list); kept lists of head h
// start at kept + h * kept_stride.
hipError_t launch_select(const float* scores, int n, int n_heads, int budget, int32_t* kept,
                         int kept_stride, const int32_t* head_len, hipStream_t stream);

// Top-`budget` of the n_heads heads of each of n_seq sequences (host
// arrays: scores[s], kept[s] and n[s] keys per head; sequences with
// n[s] <= budget are skipped), in as few launches as the length classes allow.
hipError_t launch_select_batch(int n_seq, const float* const* scores, int32_t* const* kept,
                               const int* n, int n_heads, int budget, hipStream_t stream);

// Head-specific budgets over one sequence's n_layers x n_kv heads.
int64_t shared_workspace_bytes(int64_t n_seq, int64_t n_layers, int64_t n_kv);
hipError_t launch_select_shared(const float* scores, int stride, int n_layers, int n_kv,
                                const int32_t* head_len, int budget, int floor_, int window,
                                int32_t* kept, int32_t* kept_count, void* workspace,
                                hipStream_t stream);

// In-place stable gather of the first `budget` rows of every head (kept
// lists at stride kept_stride); with counts, head h keeps counts[h] rows
// (-1: untouched) and head_len[h] takes that count.
// queue: device scratch of compact_queue_bytes(n_heads), needed with counts.
int64_t compact_queue_bytes(int64_t n_heads);

// The allocation-free counted compaction keeps its queue in a static device
// array of scratch_bytes() (= compact_queue_bytes(kScratchHeads)), one copy
// per GPU; scratch_address gives the copy of `device` (which must be the
// current device on the first call for it).
constexpr int64_t kScratchHeads = 65536;
constexpr int kMaxDevices = 64;
int64_t scratch_bytes();
hipError_t scratch_address(int device, void** out);
hipError_t launch_compact(int row_bytes, void* k, void* v, int32_t* pos, int64_t cap, int len,
                          int n_heads, const int32_t* kept, int budget, int kept_stride,
                          const int32_t* counts, int32_t* head_len, uint32_t* queue,
                          hipStream_t stream);

// Uniform-budget compaction of n_seq sequences in as few launches as the
// kernel-argument table allows (host arrays, one entry per firing sequence;
// kept[s] holds that sequence's [n_heads][budget] lists).
hipError_t launch_compact_batch(int row_bytes, int n_seq, void* const* k, void* const* v,
                                int32_t* const* pos, const int* cap, const int* len,
                                const int32_t* const* kept, int n_heads, int budget,
                                hipStream_t stream);

}  // namespace tri
