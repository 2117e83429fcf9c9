// Balanced split of the decode work over waves (used by the matrix-core family).
//
// The key lists of all (sequence b, KV head kh) units are laid end to end,
// unit u = b*KV + kh, each as n_sub(b) = ceil(L_b/16) + ceil(NQ/16) "sub-pages"
// of 16 keys (cached keys first, then the step's new rows). The concatenation
// (W sub-pages) is cut into segments of sigma = max(min_seg, ceil(W / n_seg))
// sub-pages; wave g of the grid attends segment g. The intersection of a
// segment with a unit is a "piece". A unit covered by a single piece is
// finished by that wave (output written directly); otherwise each piece's
// online-softmax state goes to workspace slot u + g (one-to-one, because
// segments and units are both ordered along the same axis) and the combine
// kernel merges the unit's slots. This is the partition/merge scheme of the
// docs.rs page "onnxruntime-ep-mlx 0.31.1: src/ops/paged_attention.rs"
// (VECTOR_PARTIALS, PARTIALS_REDUCE) with the cut placed by work rather than
// by a fixed key stride, so ragged batches keep every wave equally busy.
#pragma once

#include "pa_device.hpp"

namespace pa {

constexpr int kMaxSplitBatch = 8192;  // sequences per call for the balanced split

struct SplitGeometry {
    int B, KV, NQ, max_tokens;  // max_tokens = max_blocks_per_seq * block_size
    int n_seg;                  // segments the grid provides (waves)
    int min_seg;                // minimum segment length, in sub-pages
};

// s_pref[b] = sum_{b' < b} n_sub(b'), b = 0..B (exclusive prefix in LDS).
// Every thread of the workgroup must call this; ends with __syncthreads.
__device__ __forceinline__ void build_prefix(const int32_t* context_lens, const SplitGeometry& g,
                                             int* s_pref) {
    __shared__ int s_part[256];
    const int nnew = (g.NQ + 15) / 16;
    const int per = (g.B + 255) / 256;
    const int b0 = threadIdx.x * per;
    int sum = 0;
    for (int i = 0; i < per; ++i) {
        const int b = b0 + i;
        if (b < g.B) {
            const int L = min(max(context_lens[b], 0), g.max_tokens);
            sum += (L + 15) / 16 + nnew;
        }
    }
    s_part[threadIdx.x] = sum;
    __syncthreads();
    // exclusive scan of the 256 partial sums (Hillis-Steele in LDS)
    for (int off = 1; off < 256; off <<= 1) {
        const int v = threadIdx.x >= off ? s_part[threadIdx.x - off] : 0;
        __syncthreads();
        s_part[threadIdx.x] += v;
        __syncthreads();
    }
    int run = threadIdx.x > 0 ? s_part[threadIdx.x - 1] : 0;
    for (int i = 0; i < per; ++i) {
        const int b = b0 + i;
        if (b < g.B) {
            s_pref[b] = run;
            const int L = min(max(context_lens[b], 0), g.max_tokens);
            run += (L + 15) / 16 + nnew;
        }
    }
    if (threadIdx.x == 255) s_pref[g.B] = s_part[255];
    __syncthreads();
}

__device__ __forceinline__ int64_t split_total(const SplitGeometry& g, const int* s_pref) {
    return (int64_t)g.KV * s_pref[g.B];
}

__device__ __forceinline__ int64_t split_sigma(const SplitGeometry& g, int64_t W) {
    const int64_t s = (W + g.n_seg - 1) / g.n_seg;
    return s > g.min_seg ? s : g.min_seg;
}

// Sequence whose units contain position x: largest b with KV*s_pref[b] <= x.
__device__ __forceinline__ int split_find_seq(const SplitGeometry& g, const int* s_pref,
                                              int64_t x) {
    int lo = 0, hi = g.B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)g.KV * s_pref[mid] <= x) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

}  // namespace pa
