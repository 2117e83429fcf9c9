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

// Merge for the balanced split (split.hpp): (sequence b, KV head kh) has one
// state per group g in [g0, g1] that overlaps sequence b, stored in slot
// (b + g)*KV + kh; pass 1 recorded (g0, g1) per sequence. Sequences inside one
// group were finished by pass 1.
// The merge is PARTIALS_REDUCE of the docs.rs page "onnxruntime-ep-mlx 0.31.1:
// src/ops/paged_attention.rs" in base 2: out = sum_g 2^(m_g - M) o_g /
// sum_g 2^(m_g - M) l_g with M = max_g m_g.
// WPR waves share one output row (WPR = 1: a workgroup takes 4*RPW rows of a
// (sequence, head), RPW per wave; WPR = 4: one row, its pieces dealt to 4 waves
// in contiguous runs and the four partial merges combined through LDS). Each
// wave loads the (m, l) of up to 64 pieces lane-parallel and the partial outputs
// of up to kBatch pieces at once, for all of its rows before any is reduced, so
// a wave's rows cost two dependent memory latencies after the metadata together
// (RPW = 2: half the waves, each with twice the loads in flight).
template <typename T>
struct SplitCombineArgs {
    const typename Partial<T>::type* ws_o;  // [slots][R][D] (Partial<T>)
    const float* ws_ml;    // [slots][R][2]
    const int32_t* meta;   // [B][2]     first and last group of each sequence
    T* out;
    int KV, H, NQ, R;
};

// The PER fp16 partial-output elements of a lane, read as one 32-bit word or as
// zero-extended 16-bit words, so that no load writes half a register and has to
// wait for the one before it.
template <int PER>
__device__ __forceinline__ void load_partial(const _Float16* src, float (&o)[PER]) {
    if constexpr (PER == 2) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(src);
        o[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
        o[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    } else {
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const uint32_t w = *reinterpret_cast<const uint16_t*>(src + e);
            o[e] = (float)__builtin_bit_cast(_Float16, (uint16_t)w);
        }
    }
}

template <typename T, int D, int WPR, int RPW = 1, int kBatch = 16>
__global__ __launch_bounds__(256) void combine_split(SplitCombineArgs<T> a) {
    using E = Elem<T>;
    constexpr int PER = D / 64;      // output elements per lane
    // kBatch: partial outputs in flight per wave and row
    constexpr int RPB = 4 * RPW / WPR;  // rows per workgroup
    static_assert(D % 64 == 0 && (WPR == 1 || (WPR == 4 && RPW == 1)), "shape");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int R = a.R;
    const int tiles = (R + RPB - 1) / RPB;
    const int64_t u = blockIdx.x / tiles;  // b * KV + kh
    const int rho0 = (int)(blockIdx.x % tiles) * RPB + (WPR == 1 ? wave * RPW : 0);
    const int64_t b = u / a.KV;
    const int s0 = a.meta[2 * b], s1 = a.meta[2 * b + 1];
    if (s0 == s1) return;  // finished by pass 1 (whole workgroup)
    const int n = s1 - s0 + 1;
    // WPR = 1: rows past R (the last tile may be short) read row R - 1 and store nothing
    bool active[RPW];
    int rho[RPW];
    bool any = false;
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
        active[k] = rho0 + k < R;
        rho[k] = min(rho0 + k, R - 1);
        any = any || active[k];
    }
    // this wave's pieces [p0, p1) of the row
    const int per_w = (n + WPR - 1) / WPR;
    const int p0 = WPR == 1 ? 0 : min(n, wave * per_w), p1 = WPR == 1 ? n : min(n, p0 + per_w);
    const int64_t first = (b + s0) * a.KV + (u - b * a.KV);  // slot of piece g0
    const float* ml[RPW];
    const typename Partial<T>::type* po[RPW];
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
        ml[k] = a.ws_ml + (first * R + rho[k]) * 2;
        po[k] = a.ws_o + (first * R + rho[k]) * D + lane * PER;
    }
    // consecutive groups of one (sequence, head) are KV slots apart
    const int64_t mstride = (int64_t)a.KV * R * 2, ostride = (int64_t)a.KV * R * D;

    float M[RPW], Lw[RPW];
    float acc[RPW][PER];
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
        M[k] = kNegMax;
        Lw[k] = 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[k][e] = 0.f;
    }
    auto load_batch = [&](int k, int c0, int j0, int cn, float (&ov)[kBatch][PER]) {
        // (fp16: pieces past the run read the last one again, with weight 0)
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if constexpr (Partial<T>::kNorm)
                load_partial<PER>(po[k] + (c0 + min(j0 + j, cn - 1)) * ostride, ov[j]);
            else
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    ov[j][e] = j0 + j < cn ? po[k][(c0 + j0 + j) * ostride + e] : 0.f;
        }
    };
    if (WPR == 4 || any) {
        for (int c0 = p0; c0 < p1; c0 += 64) {  // runs of up to 64 pieces
            const int cn = min(64, p1 - c0);
            // partial outputs of every row's first batch, issued before the (m, l) are used
            float ov[RPW][kBatch][PER];
#pragma unroll
            for (int k = 0; k < RPW; ++k) load_batch(k, c0, 0, cn, ov[k]);
            const bool mine = lane < cn;
            float mp[RPW], lp[RPW], wo[RPW];
#pragma unroll
            for (int k = 0; k < RPW; ++k) {
                mp[k] = mine ? ml[k][(c0 + lane) * mstride] : kNegMax;
                lp[k] = mine ? ml[k][(c0 + lane) * mstride + 1] : 0.f;
            }
#pragma unroll
            for (int k = 0; k < RPW; ++k) {
                const float Mr = wave_max(mp[k]);
                const float Mn = fmaxf(M[k], Mr);
                const float sc = fast_exp2(M[k] - Mn);  // rescale what earlier runs gathered
                Lw[k] *= sc;
#pragma unroll
                for (int e = 0; e < PER; ++e) acc[k][e] *= sc;
                M[k] = Mn;
                const float wp = mine ? fast_exp2(mp[k] - M[k]) : 0.f;
                Lw[k] += wave_sum(wp * lp[k]);
                wo[k] = Partial<T>::kNorm ? wp * lp[k] : wp;  // weight of the stored o
            }
            for (int j0 = 0; j0 < cn; j0 += kBatch) {
                if (j0 > 0) {
#pragma unroll
                    for (int k = 0; k < RPW; ++k) load_batch(k, c0, j0, cn, ov[k]);
                }
#pragma unroll
                for (int k = 0; k < RPW; ++k)
#pragma unroll
                    for (int j = 0; j < kBatch; ++j) {
                        // weight of piece j0 + j (lane j0 + j; 0 past the run's end)
                        const float w = __builtin_bit_cast(
                            float,
                            __builtin_amdgcn_readlane(__builtin_bit_cast(int, wo[k]), (j0 + j) & 63));
#pragma unroll
                        for (int e = 0; e < PER; ++e) acc[k][e] = fmaf(w, ov[k][j][e], acc[k][e]);
                    }
            }
        }
    }
    const int kh = (int)(u % a.KV);
    if constexpr (WPR == 4) {
        __shared__ float s_m[4], s_l[4];
        __shared__ float s_o[4][D];
        if (lane == 0) {
            s_m[wave] = M[0];
            s_l[wave] = Lw[0];
        }
#pragma unroll
        for (int e = 0; e < PER; ++e) s_o[wave][lane * PER + e] = acc[0][e];
        __syncthreads();
        if (threadIdx.x < D) {
            const int d = threadIdx.x;
            const float Mt = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
            float o = 0.f, lt = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float f = fast_exp2(s_m[w] - Mt);
                o = fmaf(f, s_o[w][d], o);
                lt = fmaf(f, s_l[w], lt);
            }
            const int64_t grow = (b * a.H + (int64_t)kh * (a.H / a.KV)) * a.NQ + rho[0];
            E::store(a.out + grow * D + d, lt != 0.f ? o / lt : 0.f);
        }
    } else {
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
            if (!active[k]) continue;
            const int64_t grow = (b * a.H + (int64_t)kh * (a.H / a.KV)) * a.NQ + rho[k];
            T* dst = a.out + grow * D + lane * PER;
#pragma unroll
            for (int e = 0; e < PER; ++e) E::store(dst + e, Lw[k] != 0.f ? acc[k][e] / Lw[k] : 0.f);
        }
    }
}

}  // namespace pa
