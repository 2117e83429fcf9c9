// Dense (prefill) GQA attention forward on the matrix cores (gfx950, fp16/bf16).
//
// Operation: the forward half of the docs.rs page "onnxruntime-ep-mlx 0.31.1:
// src/ops/attention_vjp/dense.rs", execute(): scores scale * q k^T, plus an
// optional boolean or additive mask broadcast over [B, HQ, SQ, SK] (keys past a
// shorter mask width hidden), the top-left causal limit (key j visible to query
// i only if j <= i), softmax, rows with no visible key set to zero, times V.
// GQA: query head h = kh*G + g reads KV head kh.
//
// A workgroup takes (sequence b, KV head kh, a block of P = 16*NW*NRT/G query
// positions), so it holds R = G*P <= 16*NW*NRT rows: every query head of the
// group at those positions, and each K/V tile of the KV head is read once for
// all of them. The keys stream through a ring of kRing 16-key LDS slots as in
// the cooperative decode kernel (NW waves of NRT row tiles, the issuing waves
// sharing every slot's loads, one barrier per slot); the causal limit and the
// mask width shorten the stream. Mask values are read per score element from
// global memory: waiting for them drains the wave's ring, so masked runs are
// correct but not tuned.
#pragma once

#include "decode_mfma.hpp"

namespace pa {

struct DenseGeometry {
    int B, HQ, HK, SQ, SK;
    int G, P, nblk;  // heads per KV head, query positions per workgroup, blocks per (b, kh)
    int causal;
};

template <typename T>
struct DenseArgs {
    const T* q;        // [B, HQ, SQ, D]
    const T* k;        // [B, HK, SK, D]
    const T* v;
    T* out;            // [B, HQ, SQ, D]
    const void* mask;  // uint8 (nonzero = visible) or float32 bias, dims [mb, mh, mq, mw]
    int mb, mh, mq, mw;
    DenseGeometry g;
    float qscale;      // scale * log2(e)
    // statistics pass of the backward (STATS): out is not written; per query
    // row (index (b*HQ + h)*SQ + i) lse = log2 of sum_j 2^(s_j * log2 e) (+inf
    // for a row with no visible key) and delta = sum_d Y_d * dout_d, Y in fp32
    const T* dout;
    float* lse;
    float* delta;
};

// Mask bias of score (b, h, qi, kj) in base-2 units (0 or -inf for a boolean
// mask, value * log2(e) for an additive one); indices already inside the
// mask's broadcast shape (kj < mw unless mw == 1).
template <int MASK, typename T>
__device__ __forceinline__ float mask_bias2(const DenseArgs<T>& d, int b, int h, int qi, int kj) {
    const int64_t mi = (((int64_t)(d.mb == 1 ? 0 : b) * d.mh + (d.mh == 1 ? 0 : h)) * d.mq +
                        (d.mq == 1 ? 0 : qi)) * d.mw + (d.mw == 1 ? 0 : kj);
    if constexpr (MASK == 1)
        return static_cast<const uint8_t*>(d.mask)[mi] ? 0.f : -__builtin_inff();
    else
        return static_cast<const float*>(d.mask)[mi] * 1.4426950408889634f;
}

// Backward statistics of the finished rows of a RowTiles (rows 16*(rt0 + rt)
// + 4*g16 + i held in acc[rt][*][i]): lse = m + log2(l) per row (+inf when l =
// 0, so that every recomputed probability of the row is 0) and delta = sum_d
// (acc / l)_d * dout_d, reduced over the 16 lanes of a row group. off(r) is the
// element offset of row r from row index `first` * D (-1: no such row).
template <int D, typename Rows, typename T, typename F>
__device__ __forceinline__ void dense_row_stats(const Rows& rows, const DenseArgs<T>& d,
                                                int64_t first, F&& off) {
    constexpr int NT = D / 16;
    const int c16 = rows.c16, g16 = rows.g16;
#pragma unroll
    for (int rt = 0; rt < (int)(sizeof(rows.m) / sizeof(rows.m[0])); ++rt) {
        float lrow = rows.lsum[rt];
        lrow += __shfl_xor(lrow, 16);
        lrow += __shfl_xor(lrow, 32);  // l of row 16*(rt0+rt) + c16
        const int rc = 16 * (rows.rt0 + rt) + c16;
        const int64_t oc = off(rc);
        if (g16 == 0 && oc >= 0)
            d.lse[first + oc / D] = lrow > 0.f ? rows.m[rt] + __builtin_log2f(lrow)
                                               : __builtin_inff();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * (rows.rt0 + rt) + 4 * g16 + i;
            const float l_r = __shfl(lrow, 4 * g16 + i);
            const int64_t o = off(r);  // the same in the 16 lanes of the group
            float part = 0.f;
            if (o >= 0) {
                const T* gy = d.dout + first * D + o + c16;
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    part = fmaf(rows.acc[rt][t][i], Elem<T>::load(gy + 16 * t), part);
            }
            part += __shfl_xor(part, 1);
            part += __shfl_xor(part, 2);
            part += __shfl_xor(part, 4);
            part += __shfl_xor(part, 8);
            if (o >= 0 && c16 == 0) d.delta[first + o / D] = l_r > 0.f ? part / l_r : 0.f;
        }
    }
}

// MASK: 0 none, 1 boolean, 2 additive. PAIR: workgroup w takes blocks w and
// nblk - 1 - w of its (sequence, KV head), one after the other, so that under
// the causal limit every workgroup has the same number of keys to attend.
// STATS: write the backward's row statistics (DenseArgs::lse, ::delta) instead
// of the output.
template <typename T, int D, int NW, int NRT, int kRing, int MASK, bool PAIR, bool STATS = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dense_mfma(DenseArgs<T> d) {
    using Lay = SlotLayout<T, D>;
    using Rows = RowTiles<T, D, NRT, true>;
    constexpr int KS = D / 32;
    constexpr int NWI = NW < KS ? NW : KS;  // waves that issue loads
    constexpr int IPW = KS / NWI;           // instructions per half per issuing wave
    static_assert(D % 32 == 0 && Lay::kOps == KS && KS % NWI == 0, "shape");
    static_assert(kRing >= 3 && 2 * IPW * (kRing - 2) <= 63, "ring");

    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int lane = threadIdx.x & 63, c16 = lane & 15, g16 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const DenseGeometry& g = d.g;
    const int nw = PAIR ? (g.nblk + 1) / 2 : g.nblk;  // workgroups per (b, kh)
    const int w = blockIdx.x % nw;
    const int kh = (blockIdx.x / nw) % g.HK;
    const int b = blockIdx.x / (nw * g.HK);
    for (int half = 0; half < (PAIR ? 2 : 1); ++half) {
    const int blk = half == 0 ? w : g.nblk - 1 - w;
    if (half == 1) {
        if (blk == w) break;  // odd block count: the middle block has no partner
        asm volatile("" ::: "memory");
        __syncthreads();      // every wave is done with the ring before it is refilled
    }
    const int i0 = blk * g.P;                // first query position of the block
    const int R = g.G * g.P;                 // rows: r = gg*P + p -> head kh*G + gg, position i0 + p
    const int pend = min(g.P, g.SQ - i0);    // positions of the block that exist (>= 1)
    int kend = g.SK;                         // keys any row of the block may see
    if (g.causal) kend = min(kend, i0 + pend);
    if (MASK && d.mw != 1 && d.mw < g.SK) kend = min(kend, d.mw);
    const int n_sub = (kend + 15) / 16;
    const bool issues = wave < NWI;
    const bool has_rows = 16 * NRT * wave < R;

    // The row tiles take the row count and the score scale from split arguments.
    SplitArgs<T> sa{};
    sa.R = R;
    sa.qscale = d.qscale;
    sa.g.NQ = 1;
    sa.g.KV = 1;
    sa.H = 1;
    Rows rows(sa, lane, wave * NRT);

    // This lane's S^T row of tile rt (row c16 of the tile), clamped to a real one.
    int srow_p[NRT], srow_h[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int r = min(16 * (wave * NRT + rt) + c16, R - 1);
        srow_p[rt] = min(r % g.P, pend - 1);
        srow_h[rt] = kh * g.G + r / g.P;
    }
    const int64_t head0 = (int64_t)b * g.HQ + (int64_t)kh * g.G;  // first query head of the group
    if (has_rows) {
        uint32_t qoff[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
            qoff[rt] = (uint32_t)(((srow_h[rt] - kh * g.G) * g.SQ + i0 + srow_p[rt]) * D);
        rows.load_q_at(d.q + head0 * g.SQ * D, qoff);  // older than the ring's loads
    }
    const int64_t kv0 = ((int64_t)b * g.HK + kh) * g.SK * D;
    const T* const kb = d.k + kv0;
    const T* const vb = d.v + kv0;
    for (int s = 0; s < kRing - 1 && s < n_sub; ++s)
        if (issues)
            fetch_rows<T, D, IPW>(kb + (int64_t)16 * s * D, vb + (int64_t)16 * s * D,
                                  min(15, g.SK - 1 - 16 * s), smem + s * Lay::kBytes, lane, wave, NWI);
    rows.reset();
    bool q_pending = has_rows;
    for (int i = 0; i < n_sub; ++i) {
        const int ahead = min(kRing - 2, n_sub - 1 - i);  // sub-pages fetched after i
        if (issues) wait_ahead<2 * IPW, kRing - 2>(ahead);
        else __builtin_amdgcn_s_waitcnt(kWaitVm0);
        if (q_pending) {
            rows.q_ready();
            q_pending = false;
        }
        // every wave's part of sub-page i is in; slot i - 1 is read out
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int nxt = i + kRing - 1;
        if (nxt < n_sub && issues)
            fetch_rows<T, D, IPW>(kb + (int64_t)16 * nxt * D, vb + (int64_t)16 * nxt * D,
                                  min(15, g.SK - 1 - 16 * nxt), smem + (nxt % kRing) * Lay::kBytes,
                                  lane, wave, NWI);
        if (!has_rows) continue;
        const char* slot = smem + (i % kRing) * Lay::kBytes;
        u32x4_t kop[KS];
        u32x2_t vt[D / 16];
        rows.read_k(slot, kop);
        rows.read_v(slot, vt);
        Rows::lds_wait(vt);
        const int key0 = 16 * i;
        const int valid = min(16, kend - key0);
        int lim[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
            lim[rt] = g.causal ? max(0, min(valid, i0 + srow_p[rt] - key0 + 1)) : valid;
        if constexpr (MASK != 0) {
            float bias[NRT][4];
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    bias[rt][e] = mask_bias2<MASK>(d, b, srow_h[rt], i0 + srow_p[rt],
                                                   min(key0 + 4 * g16 + e, d.mw - 1));
            rows.template scores<true>(kop, lim, false, bias);
        } else {
            // every key visible to every row: whole sub-page, and causally
            // below the block's first query
            const bool full = valid == 16 && (!g.causal || key0 + 15 <= i0);
            rows.scores(kop, lim, full);
        }
        rows.accumulate(vt, valid);
    }
    // Q is still in flight when there were no keys; otherwise nothing is (the
    // loop waited for every sub-page), so this costs nothing and leaves no path
    // on which the rows' registers are read before a wait.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    rows.flush();
    auto row_off = [&](int r) -> int64_t {  // element offset of row r from head0's first row
        if (r >= R || r % g.P >= pend) return -1;
        return ((int64_t)(r / g.P) * g.SQ + i0 + r % g.P) * D;
    };
    if (has_rows) {
        if constexpr (STATS)
            dense_row_stats<D>(rows, d, head0 * g.SQ, row_off);
        else
            rows.emit_rows(d.out + head0 * g.SQ * D, row_off);
    }
    }  // blocks of this workgroup
}

}  // namespace pa
