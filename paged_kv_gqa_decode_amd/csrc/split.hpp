// Balanced split of the decode work (used by the matrix-core family).
//
// The sequences are laid end to end along one axis, sequence b as n_sub(b) =
// ceil(L_b/16) + ceil(NQ/16) positions (16-key "sub-pages": cached keys first,
// then the step's new rows). The axis (W positions) is cut into n_grp groups
// at positions start(g) = floor(g*W/n_grp), so group sizes differ by at most
// one. Group g is attended by KV consecutive waves of the grid, wave (g, kh)
// taking KV head kh of every position of the group: the KV waves of a group
// stream the same pages at the same time, which keeps the pool reads of one
// page (all heads of a token are adjacent in memory) close together.
// The intersection of a group with a sequence is a "piece". A sequence inside
// a single group is finished by that group's waves (output written directly);
// otherwise each piece's online-softmax state of head kh goes to workspace slot
// (b + g)*KV + kh (one-to-one: groups and sequences are ordered along the same
// axis, so b + g grows at every new intersection) and the combine kernel merges
// the slots of each (sequence, head). This is the partition/merge scheme of the
// docs.rs page "onnxruntime-ep-mlx 0.31.1: src/ops/paged_attention.rs"
// (VECTOR_PARTIALS, PARTIALS_REDUCE) with cuts placed by work rather than by a
// fixed key stride, so ragged batches keep every wave equally busy.
#pragma once

#include "pa_device.hpp"

namespace pa {

constexpr int kMaxSplitBatch = 8192;  // sequences per call for the balanced split

struct SplitGeometry {
    int B, KV, NQ, max_tokens;  // max_tokens = max_blocks_per_seq * block_size
    int n_grp;                  // groups the grid provides (KV waves each)
    int min_seg;                // minimum group length, in positions
    int seq_pad;                // cost of a sequence beyond its positions, in positions
};

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS round trips): within each 16-lane row by shifts of 1,
// 2, 4 and 8, then lane 15 of each row into the next and lane 31 into the
// upper half.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// s_pref[b] = sum_{b' < b} n_sub(b'), b = 0..B (exclusive prefix in LDS), and
// s_len[b] = the cached length of sequence b clamped to [0, max_tokens].
// Every thread of the workgroup must call this; the first wave loads 512
// lengths per round (all 8 loads in flight at once) and scans only the
// 64-lane slices that hold sequences; one barrier at the end.
__device__ __forceinline__ void build_prefix(const int32_t* context_lens, const SplitGeometry& g,
                                             int* s_pref, int* s_len) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int nnew = (g.NQ + 15) / 16;
        int carry = 0;
        for (int base = 0; base < g.B; base += 512) {
            int raw[8];
#pragma unroll
            for (int r = 0; r < 8; ++r)  // unconditional (clamped index): all 8 loads in flight
                raw[r] = context_lens[min(base + 64 * r + lane, g.B - 1)];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if (base + 64 * r >= g.B) break;  // uniform: no sequences left
                const int b = base + 64 * r + lane;
                const int L = b < g.B ? min(max(raw[r], 0), g.max_tokens) : 0;
                const int n = b < g.B ? (L + 15) / 16 + nnew : 0;
                const int incl = wave_inclusive_scan(n);
                if (b < g.B) {
                    s_len[b] = L;
                    s_pref[b] = carry + incl - n;
                }
                carry += __builtin_amdgcn_readlane(incl, 63);
            }
        }
        if (lane == 0) s_pref[g.B] = carry;
    }
    __syncthreads();
}

// The cut of the axis into groups by cost: a sequence costs its n_sub
// positions plus seq_pad (its fixed work: Q loads, the piece's state, the
// switch), so the axis is C = W + seq_pad * B cost units, sequence b taking
// [pref(b) + seq_pad * b, pref(b + 1) + seq_pad * b + seq_pad) with its pad
// after its positions. Group g takes the cost units from floor(g*C/n): its
// first position is that of cost unit floor(g*C/n), a unit of a pad standing
// for the next sequence's first position. Groups differ by at most one cost
// unit; a group inside a pad has no position (and is skipped).
struct Cut {
    int64_t W, C;
    int64_t n;  // groups in use: n_grp, fewer when groups would be shorter than min_seg
    int pad;
    __device__ __forceinline__ Cut(const SplitGeometry& g, int64_t total)
        : W(total), C(total + (int64_t)g.seq_pad * g.B), pad(g.seq_pad) {
        int64_t m = g.min_seg > 1 ? C / g.min_seg : C;
        if (m < 1) m = 1;
        n = m < g.n_grp ? m : g.n_grp;
    }
    // first position of group grp (grp <= n; start(n) = W)
    template <typename SEQ>
    __device__ __forceinline__ int64_t start(int64_t grp, const SEQ& seq, const SplitGeometry& g) const {
        const int64_t c = grp * C / n;
        if (pad == 0 || c >= C) return c >= C ? W : c;
        const int b = seq.find_cost(g, c, pad);
        const int64_t p0 = seq.pref(b);
        const int64_t p1 = seq.pref(b + 1);
        const int64_t off = c - (p0 + (int64_t)pad * b);
        return off < p1 - p0 ? p0 + off : p1;
    }
    // the group holding position x of sequence b (largest g with start(g) <= x)
    __device__ __forceinline__ int64_t group_of(int64_t x, int b) const {
        return ((x + (int64_t)pad * b + 1) * n - 1) / C;
    }
};

// Sequence holding position x: largest b with s_pref[b] + pad*b <= x (pad = 0:
// the position axis; pad > 0: the cost axis of Cut).
__device__ __forceinline__ int split_find_seq(const SplitGeometry& g, const int* s_pref,
                                              int64_t x, int pad = 0) {
    int lo = 0, hi = g.B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)s_pref[mid] + (int64_t)pad * mid <= x) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The batch's sequence table as the streams read it: pref(b) = sum of n_sub
// over sequences before b (pref(B) = W), len(b) = the clamped cached length,
// find(x) = the sequence holding axis position x.
// SeqTableLds: built in LDS by build_prefix, any batch size.
struct SeqTableLds {
    const int* s_pref;
    const int* s_len;
    int B;
    __device__ __forceinline__ int pref(int b) const { return s_pref[b]; }
    __device__ __forceinline__ int len(int b) const { return s_len[b]; }
    __device__ __forceinline__ int total() const { return s_pref[B]; }
    __device__ __forceinline__ int find(const SplitGeometry& g, int64_t x) const {
        return split_find_seq(g, s_pref, x);
    }
    __device__ __forceinline__ int find_cost(const SplitGeometry& g, int64_t c, int pad) const {
        return split_find_seq(g, s_pref, c, pad);
    }
};

// SeqTableRegs: batches of at most 64 sequences, held in registers: lane b of
// each wave keeps sequence b's prefix and length (every wave builds its own
// copy with one load and a wave scan: no LDS and no barrier), read back with
// readlane at the wave-uniform sequence index.
constexpr int kRegTableMaxBatch = 64;
struct SeqTableRegs {
    int v_pref, v_len;  // this lane's sequence (lane < B)
    int W, B;
    __device__ __forceinline__ SeqTableRegs(const int32_t* context_lens, const SplitGeometry& g)
        : B(g.B) {
        const int lane = threadIdx.x & 63;
        const int nnew = (g.NQ + 15) / 16;
        const int raw = lane < g.B ? context_lens[lane] : 0;
        const int L = lane < g.B ? min(max(raw, 0), g.max_tokens) : 0;
        const int n = lane < g.B ? (L + 15) / 16 + nnew : 0;
        const int incl = wave_inclusive_scan(n);
        v_pref = incl - n;
        v_len = L;
        W = __builtin_amdgcn_readlane(incl, 63);
    }
    __device__ __forceinline__ int pref(int b) const {
        return b < B ? __builtin_amdgcn_readlane(v_pref, b) : W;
    }
    __device__ __forceinline__ int len(int b) const { return __builtin_amdgcn_readlane(v_len, b); }
    __device__ __forceinline__ int total() const { return W; }
    __device__ __forceinline__ int find(const SplitGeometry&, int64_t x) const {
        const int lane = threadIdx.x & 63;
        // lanes of sequences starting at or before x; lane 0 always (pref(0) = 0)
        const uint64_t m = __ballot(lane < B && (int64_t)v_pref <= x);
        return 63 - __builtin_clzll(m);
    }
    // the sequence holding cost unit c of Cut (largest b with pref(b) + pad*b <= c)
    __device__ __forceinline__ int find_cost(const SplitGeometry&, int64_t c, int pad) const {
        const int lane = threadIdx.x & 63;
        const uint64_t m = __ballot(lane < B && (int64_t)v_pref + (int64_t)pad * lane <= c);
        return 63 - __builtin_clzll(m);
    }
};

}  // namespace pa
