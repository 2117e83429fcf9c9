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

// Merge for the balanced per-wave split (split.hpp): unit u = b*KV + h/G has one
// state per segment s in [s0, s1] that overlaps it, stored in slot u + s; pass 1
// recorded (s0, s1) per unit. Units inside one segment were finished by pass 1.
// RPW = 4: a workgroup takes 4 rows of one unit, one wave per row, each wave
// summing every piece with 8 pieces' loads in flight (few pieces per unit).
// RPW = 1: a workgroup takes one row; its 4 waves take every 4th piece and are
// merged through LDS (many pieces per unit, e.g. a few very long sequences).
template <typename T>
struct SplitCombineArgs {
    const float* ws_o;     // [slots][R][D]
    const float* ws_ml;    // [slots][R][2]
    const int32_t* meta;   // [B*KV][2]  first and last segment of each unit
    T* out;
    int KV, H, NQ, R;
};

template <typename T, int D, int RPW>
__global__ __launch_bounds__(256) void combine_split(SplitCombineArgs<T> a) {
    using E = Elem<T>;
    constexpr int PER = D / 64;
    constexpr int BATCH = 8;
    constexpr int WAVES_PER_ROW = 4 / RPW;
    static_assert(D % 64 == 0 && (RPW == 1 || RPW == 4), "shape");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tiles = (a.R + RPW - 1) / RPW;
    const int64_t u = blockIdx.x / tiles;
    const int rho = (int)(blockIdx.x % tiles) * RPW + (RPW == 4 ? wave : 0);
    const int s0 = a.meta[2 * u], s1 = a.meta[2 * u + 1];
    if (s0 == s1) return;  // finished by pass 1 (whole workgroup)
    const int n = s1 - s0 + 1, R = a.R;
    const int64_t first = u + s0;
    const int b = (int)(u / a.KV), kh = (int)(u % a.KV);
    const int64_t grow = ((int64_t)b * a.H + (int64_t)kh * (a.H / a.KV)) * a.NQ + rho;
    const bool active = rho < R;  // RPW = 4: the unit's last tile may be short
    const float* ml = a.ws_ml + (first * R + rho) * 2;
    const int64_t mstride = (int64_t)R * 2;
    const float* po = a.ws_o + (first * R + rho) * D + lane * PER;
    const int64_t ostride = (int64_t)R * D;
    const int pw = RPW == 4 ? 0 : wave;  // first piece of this wave

    float M = kNegMax;
    if (active)
        for (int p = pw * 64 + lane; p < n; p += 64 * WAVES_PER_ROW)
            M = fmaxf(M, ml[p * mstride]);
    M = wave_max(M);
    __shared__ float s_max[4], s_l[4];
    __shared__ float s_o[4][D];
    if constexpr (RPW == 1) {
        if (lane == 0) s_max[wave] = M;
        __syncthreads();
        M = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    }
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float lsum = 0.f;
    if (active) {
        for (int p0 = pw; p0 < n; p0 += WAVES_PER_ROW * BATCH) {
            float ov[BATCH][PER], mv[BATCH], lv[BATCH];
#pragma unroll
            for (int j = 0; j < BATCH; ++j) {
                const int p = p0 + WAVES_PER_ROW * j;
                const bool ok = p < n;
#pragma unroll
                for (int e = 0; e < PER; ++e) ov[j][e] = ok ? po[p * ostride + e] : 0.f;
                mv[j] = ok ? ml[p * mstride] : kNegMax;
                lv[j] = ok ? ml[p * mstride + 1] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < BATCH; ++j) {
                const float w = fast_exp2(mv[j] - M);
                lsum = fmaf(w, lv[j], lsum);
#pragma unroll
                for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, ov[j][e], acc[e]);
            }
        }
    }
    if constexpr (RPW == 1) {
#pragma unroll
        for (int e = 0; e < PER; ++e) s_o[wave][lane * PER + e] = acc[e];
        if (lane == 0) s_l[wave] = lsum;
        __syncthreads();
        if (threadIdx.x < D) {
            const int d = threadIdx.x;
            const float lt = (s_l[0] + s_l[1]) + (s_l[2] + s_l[3]);
            const float o = (s_o[0][d] + s_o[1][d]) + (s_o[2][d] + s_o[3][d]);
            E::store(a.out + grow * D + d, lt != 0.f ? o / lt : 0.f);
        }
    } else if (active) {
        T* dst = a.out + grow * D + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) E::store(dst + e, lsum != 0.f ? acc[e] / lsum : 0.f);
    }
}

}  // namespace pa
