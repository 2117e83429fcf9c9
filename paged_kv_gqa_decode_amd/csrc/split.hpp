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

// s_pref[b] = sum_{b' < b} n_sub(b'), b = 0..B (exclusive prefix in LDS), and
// s_len[b] = the cached length of sequence b clamped to [0, max_tokens].
// Every thread of the workgroup must call this; the first wave scans 64
// sequences per round (8 rounds' loads in flight at once), one barrier at the end.
__device__ __forceinline__ void build_prefix(const int32_t* context_lens, const SplitGeometry& g,
                                             int* s_pref, int* s_len) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int nnew = (g.NQ + 15) / 16;
        int carry = 0;
        for (int base = 0; base < g.B; base += 512) {
            int n[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int b = base + 64 * r + lane;
                const int L = b < g.B ? min(max(context_lens[b], 0), g.max_tokens) : 0;
                if (b < g.B) s_len[b] = L;
                n[r] = b < g.B ? (L + 15) / 16 + nnew : 0;
            }
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                int incl = n[r];  // inclusive scan over the wave
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int v = __shfl_up(incl, off);
                    if (lane >= off) incl += v;
                }
                const int b = base + 64 * r + lane;
                if (b < g.B) s_pref[b] = carry + incl - n[r];
                carry += __shfl(incl, 63);
            }
        }
        if (lane == 0) s_pref[g.B] = carry;
    }
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
