// Merge of key-partition states (gfx950): the role of PARTIALS_REDUCE on the
// docs.rs page "onnxruntime-ep-mlx 0.31.1: src/ops/paged_attention.rs".
// One wave per output row (b, h, r). For the n partitions the row's sequence
// used: M = max_p m_p, w_p = 2^(m_p - M), out = sum_p w_p o_p / sum_p w_p l_p
// (0 if the denominator is 0), rounded to nearest-even into the I/O dtype.
// Sequences that fit in one partition were finished by pass 1 and are skipped.
#pragma once

#include "pa_device.hpp"

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
    const int L = a.context_lens[b];
    int n = L > 0 ? (L - 1) / a.chunk + 1 : 1;
    n = n < a.n_parts ? n : a.n_parts;
    if (n <= 1) return;

    const float* ml = a.ws_ml + row * a.n_parts * 2;
    float M = kNegMax;
    for (int p = lane; p < n; p += 64) M = fmaxf(M, ml[2 * p]);
    M = wave_max(M);
    float lsum = 0.f;
    for (int p = lane; p < n; p += 64) lsum = fmaf(fast_exp2(ml[2 * p] - M), ml[2 * p + 1], lsum);
    lsum = wave_sum(lsum);

    const float* po = a.ws_o + row * a.n_parts * D + lane * PER;
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    for (int p = 0; p < n; ++p) {
        const float w = fast_exp2(ml[2 * p] - M);
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, po[(int64_t)p * D + e], acc[e]);
    }
    T* dst = a.out + row * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) E::store(dst + e, lsum != 0.f ? acc[e] / lsum : 0.f);
}

}  // namespace pa
