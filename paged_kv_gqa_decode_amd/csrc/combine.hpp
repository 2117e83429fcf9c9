// Merge of key-partition states (gfx950): the role of PARTIALS_REDUCE on the
// docs.rs page "onnxruntime-ep-mlx 0.31.1: src/ops/paged_attention.rs".
// One wave per output row (b, h, r). For the n partitions the row's sequence
// used: M = max_p m_p, w_p = 2^(m_p - M), out = sum_p w_p o_p / sum_p w_p l_p
// (0 if the denominator is 0), rounded to nearest-even into the I/O dtype.
// Sequences that fit in one partition were finished by pass 1 and are skipped.
#pragma once

#include "epilogue.hpp"
#include "split.hpp"

namespace pa {

template <typename T>
struct CombineArgs {
    const float* ws_o;
    const float* ws_ml;
    const int32_t* context_lens;
    T* out;
    int64_t rows;      // B * H * NQ
    int rows_per_seq;  // H * NQ
    int n_parts;
    int chunk;
    int max_tokens;    // max_blocks_per_seq * block_size
};

template <typename T, int D>
__global__ __launch_bounds__(256) void combine_partitions(CombineArgs<T> a) {
    using E = Elem<T>;
    constexpr int PER = D / 64;  // output elements per lane
    static_assert(D % 64 == 0, "D");
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.rows) return;
    const int b = (int)(row / a.rows_per_seq);
    const int L = min(a.context_lens[b], a.max_tokens);
    const int n = partitions_of(L, a.chunk, a.n_parts);
    if (n <= 1) return;

    // Lane p holds partition p's (m, l) and its weight 2^(m_p - M); the
    // partial outputs are summed with the weights taken by readlane, four
    // partitions' loads in flight at a time.
    const float* ml = a.ws_ml + row * a.n_parts * 2;
    const float* po = a.ws_o + row * a.n_parts * D + lane * PER;
    float M = kNegMax;
    for (int p = lane; p < n; p += 64) M = fmaxf(M, ml[2 * p]);
    M = wave_max(M);
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float lsum = 0.f;
    for (int p0 = 0; p0 < n; p0 += 64) {
        const int cnt = min(64, n - p0);
        const float w = lane < cnt ? fast_exp2(ml[2 * (p0 + lane)] - M) : 0.f;
        if (lane < cnt) lsum = fmaf(w, ml[2 * (p0 + lane) + 1], lsum);
        auto weight = [&](int j) {
            return __builtin_bit_cast(float,
                                      __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
        };
        int p = 0;
        for (; p + 4 <= cnt; p += 4) {
            float ov[4][PER];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < PER; ++e) ov[j][e] = po[(int64_t)(p0 + p + j) * D + e];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float wj = weight(p + j);
#pragma unroll
                for (int e = 0; e < PER; ++e) acc[e] = fmaf(wj, ov[j][e], acc[e]);
            }
        }
        for (; p < cnt; ++p) {
            const float wj = weight(p);
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] = fmaf(wj, po[(int64_t)(p0 + p) * D + e], acc[e]);
        }
    }
    lsum = wave_sum(lsum);
    T* dst = a.out + row * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) E::store(dst + e, lsum != 0.f ? acc[e] / lsum : 0.f);
}

}  // namespace pa

namespace pa {

// Merge for the balanced per-wave split (split.hpp): row (b, h, r) of unit
// u = b*KV + h/G has one state per segment s in [s0, s1] that overlaps the unit,
// stored in slot u + s. Units inside a single segment were finished by pass 1.
template <typename T>
struct SplitCombineArgs {
    const float* ws_o;   // [slots][R][D]
    const float* ws_ml;  // [slots][R][2]
    const int32_t* context_lens;
    T* out;
    SplitGeometry g;
    int H, R;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void combine_split(SplitCombineArgs<T> a) {
    using E = Elem<T>;
    constexpr int PER = D / 64;
    static_assert(D % 64 == 0, "D");
    __shared__ int s_pref[kMaxSplitBatch + 1];
    build_prefix(a.context_lens, a.g, s_pref);
    const int64_t W = split_total(a.g, s_pref);
    const int64_t sigma = split_sigma(a.g, W);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int KV = a.g.KV, NQ = a.g.NQ, G = a.H / KV, R = a.R;
    const int64_t rows = (int64_t)a.g.B * a.H * NQ;
    for (int64_t row = (int64_t)blockIdx.x * 4 + wave; row < rows; row += (int64_t)gridDim.x * 4) {
        const int b = (int)(row / ((int64_t)a.H * NQ));
        const int h = (int)((row / NQ) % a.H);
        const int r = (int)(row % NQ);
        const int kh = h / G, rho = (h % G) * NQ + r;
        const int nsub = s_pref[b + 1] - s_pref[b];
        const int64_t ustart = (int64_t)KV * s_pref[b] + (int64_t)kh * nsub;
        const int64_t s0 = ustart / sigma, s1 = (ustart + nsub - 1) / sigma;
        if (s0 == s1) continue;
        const int n = (int)(s1 - s0 + 1);
        const int64_t first = (int64_t)b * KV + kh + s0;  // slot of the first piece
        auto m_of = [&](int p) { return a.ws_ml[((first + p) * R + rho) * 2]; };
        auto l_of = [&](int p) { return a.ws_ml[((first + p) * R + rho) * 2 + 1]; };
        const float* po = a.ws_o + (first * R + rho) * D + lane * PER;
        const int64_t pstride = (int64_t)R * D;
        float M = kNegMax;
        for (int p = lane; p < n; p += 64) M = fmaxf(M, m_of(p));
        M = wave_max(M);
        float acc[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = 0.f;
        float lsum = 0.f;
        for (int p0 = 0; p0 < n; p0 += 64) {
            const int cnt = min(64, n - p0);
            const float w = lane < cnt ? fast_exp2(m_of(p0 + lane) - M) : 0.f;
            if (lane < cnt) lsum = fmaf(w, l_of(p0 + lane), lsum);
            for (int p = 0; p < cnt; ++p) {
                const float wj = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), p));
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    acc[e] = fmaf(wj, po[(int64_t)(p0 + p) * pstride + e], acc[e]);
            }
        }
        lsum = wave_sum(lsum);
        T* dst = a.out + row * D + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) E::store(dst + e, lsum != 0.f ? acc[e] / lsum : 0.f);
    }
}

}  // namespace pa
