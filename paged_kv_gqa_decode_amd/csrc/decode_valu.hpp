// Pass 1 of paged GQA decode attention on the vector ALU (gfx950, wave64).
//
// Operation: docs.rs page "onnxruntime-ep-mlx 0.31.1: src/ops/paged_attention.rs",
// VECTOR_BODY (scores, per-key online softmax, accumulation), VECTOR_REDUCE
// (merge of the per-simdgroup states) and VECTOR_PARTIALS (partition states).
// What differs from that Apple-GPU kernel:
//   * one workgroup per (sequence, KV head, row tile, key partition) holds all
//     G*NQ query rows of the KV head, so every K/V page is fetched once per GQA
//     group instead of once per query head;
//   * partitions are contiguous page-aligned chunks of the cached keys (the page
//     strides keys across partitions); the new rows go to the last partition;
//   * the running max is updated once per page of keys, not once per key, and
//     exponentials are base 2 with log2(e) folded into q;
//   * each 16-byte lane load covers 8 (16-bit) or 4 (fp32) elements of one key
//     row; a wave covers 64*16 bytes = several whole rows, so page reads are
//     fully coalesced; q.k partial sums are reduced across the lanes of a row
//     with DPP.
// Lane layout within a wave: lane = g * LPR + j, where j selects a 16-byte
// slice of the head dimension and g a key of the page (keys g, g+TPI, ...).
// Each key group g keeps its own online-softmax state; the TPI groups and the
// 4 waves are merged once at the end of the chunk.
#pragma once

#include "epilogue.hpp"

namespace pa {

enum { kModeFull = 0, kModePartial = 1, kModeNew = 2 };

// Attend NTOK keys per lane (one page, or a tile of new rows) for RT rows.
template <typename T, int LPR, int TPI, int NTOK, int RT, int MODE>
__device__ __forceinline__ void valu_attend(const uint4 (&kr)[NTOK], const uint4 (&vr)[NTOK],
                                            const float (&qf)[RT][Elem<T>::kVec], float (&m)[RT],
                                            float (&l)[RT], float (&o)[RT][Elem<T>::kVec],
                                            int g, int valid, int t0, int nq, int causal,
                                            int row0) {
    using E = Elem<T>;
    constexpr int VEC = E::kVec;
    float s[NTOK][RT];
#pragma unroll
    for (int i = 0; i < NTOK; ++i) {
        float kf[VEC];
        E::unpack(kr[i], kf);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc = fmaf(qf[r][e], kf[e], acc);
            s[i][r] = acc;
        }
    }
#pragma unroll
    for (int i = 0; i < NTOK; ++i)
#pragma unroll
        for (int r = 0; r < RT; ++r) s[i][r] = group_sum<LPR>(s[i][r]);

    float vf[NTOK][VEC];
#pragma unroll
    for (int i = 0; i < NTOK; ++i) E::unpack(vr[i], vf[i]);

    if constexpr (MODE != kModeFull) {
#pragma unroll
        for (int i = 0; i < NTOK; ++i) {
            const int t = (MODE == kModeNew ? t0 : 0) + g + TPI * i;
            const bool tok_ok = MODE == kModePartial ? (t < valid) : (t < nq);
            if (!tok_ok) {
                // unused slots may hold anything (NaN included): never let them in
#pragma unroll
                for (int e = 0; e < VEC; ++e) vf[i][e] = 0.f;
            }
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                bool vis = tok_ok;
                if constexpr (MODE == kModeNew) vis = vis && (!causal || t <= (row0 + r) % nq);
                if (!vis) s[i][r] = -__builtin_inff();
            }
        }
    }

#pragma unroll
    for (int r = 0; r < RT; ++r) {
        float mx = m[r];
#pragma unroll
        for (int i = 0; i < NTOK; ++i) mx = fmaxf(mx, s[i][r]);
        const float alpha = fast_exp2(m[r] - mx);
        m[r] = mx;
        float p[NTOK];
        float ls = 0.f;
#pragma unroll
        for (int i = 0; i < NTOK; ++i) {
            p[i] = fast_exp2(s[i][r] - mx);
            ls += p[i];
        }
        l[r] = fmaf(l[r], alpha, ls);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            float acc = o[r][e] * alpha;
#pragma unroll
            for (int i = 0; i < NTOK; ++i) acc = fmaf(p[i], vf[i][e], acc);
            o[r][e] = acc;
        }
    }
}

template <typename T, int D, int BS, int RT, bool APPEND>
__global__ __launch_bounds__(256) void decode_valu(DecodeArgs<T> a) {
    using E = Elem<T>;
    constexpr int VEC = E::kVec;
    constexpr int LPR = D / VEC;    // lanes per key row
    constexpr int TPI = 64 / LPR;   // key rows per wave load
    constexpr int NTOK = BS / TPI;  // keys per lane per page
    static_assert(D % VEC == 0 && 64 % LPR == 0 && BS % TPI == 0, "layout");

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPR, j = lane % LPR;
    const int part = blockIdx.x;
    const int kh = blockIdx.y / a.n_tiles, tile = blockIdx.y % a.n_tiles;
    const int b = blockIdx.z;
    const int G = a.H / a.KV, R = G * a.NQ;
    // cached length, never beyond what the block table can address
    const int L = min(a.context_lens[b], a.max_blocks * BS);
    const int n_seq = partitions_of(L, a.chunk, a.n_parts);
    if (part >= n_seq) return;  // whole workgroup leaves
    const int tok_begin = part * a.chunk;
    const int tok_end = min(tok_begin + a.chunk, L);
    const int row0 = tile * RT;
    // Rows of one (b, kh) are contiguous in q/out: ((b*H + kh*G)*NQ + rho)*D.
    const int64_t grow0 = ((int64_t)b * a.H + (int64_t)kh * G) * a.NQ + row0;

    float qf[RT][VEC];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        if (row0 + r < R) {
            E::unpack(load16(a.q + (grow0 + r) * D + j * VEC), qf[r]);
#pragma unroll
            for (int e = 0; e < VEC; ++e) qf[r][e] *= a.qscale;
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) qf[r][e] = 0.f;
        }
    }
    float m[RT], l[RT], o[RT][VEC];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        m[r] = kNegMax;
        l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[r][e] = 0.f;
    }

    // ---- cached keys: pages of this chunk, round-robin over the 4 waves ----
    const int64_t tstride = (int64_t)a.KV * D;  // elements between keys of a page
    const int32_t* trow = a.block_table + (int64_t)b * a.max_blocks;
    const int pg_begin = tok_begin / BS;
    const int pg_end = tok_end > tok_begin ? (tok_end + BS - 1) / BS : pg_begin;
    int n = pg_begin + wave;
    if (n < pg_end) {
        // Slot-patched step: a key whose pool slot a new row of the sequence
        // names reads that row (the last one naming it) instead of the pool.
        const int32_t* sl = APPEND ? a.ap.slots + (int64_t)b * a.NQ : nullptr;
        const int64_t nrow0 = ((int64_t)b * a.KV + kh) * a.NQ;
        auto load_page = [&](int page, uint4(&kr)[NTOK], uint4(&vr)[NTOK]) {
            const int64_t phys = trow[page];
            const int64_t off = (phys * BS * a.KV + kh) * D + j * VEC;
#pragma unroll
            for (int i = 0; i < NTOK; ++i) {
                const int64_t t = g + TPI * i;
                int src = -1;
                if constexpr (APPEND)
                    for (int jn = 0; jn < a.NQ; ++jn)
                        if (sl[jn] == phys * BS + t) src = jn;
                if (src < 0) {
                    kr[i] = load16(a.k_pool + off + t * tstride);
                    vr[i] = load16(a.v_pool + off + t * tstride);
                } else {
                    kr[i] = load16(a.new_k + (nrow0 + src) * D + j * VEC);
                    vr[i] = load16(a.new_v + (nrow0 + src) * D + j * VEC);
                }
            }
        };
        uint4 kr[NTOK], vr[NTOK];
        load_page(n, kr, vr);
        while (true) {
            const int nn = n + 4;
            const bool more = nn < pg_end;
            uint4 kn[NTOK], vn[NTOK];
            if (more) load_page(nn, kn, vn);
            const int valid = min(BS, tok_end - n * BS);
            if (valid == BS)
                valu_attend<T, LPR, TPI, NTOK, RT, kModeFull>(kr, vr, qf, m, l, o, g, BS, 0, a.NQ,
                                                             a.causal, row0);
            else
                valu_attend<T, LPR, TPI, NTOK, RT, kModePartial>(kr, vr, qf, m, l, o, g, valid, 0,
                                                                a.NQ, a.causal, row0);
            if (!more) break;
#pragma unroll
            for (int i = 0; i < NTOK; ++i) {
                kr[i] = kn[i];
                vr[i] = vn[i];
            }
            n = nn;
        }
    }

    // ---- this step's new rows, attended directly by the last partition ----
    if (part == n_seq - 1 && wave == 0) {
        const int64_t nbase = (((int64_t)b * a.KV + kh) * a.NQ) * D + j * VEC;
        for (int t0 = 0; t0 < a.NQ; t0 += TPI * NTOK) {
            uint4 kr[NTOK], vr[NTOK];
#pragma unroll
            for (int i = 0; i < NTOK; ++i) {
                const int t = t0 + g + TPI * i;
                if (t < a.NQ) {
                    kr[i] = load16(a.new_k + nbase + (int64_t)t * D);
                    vr[i] = load16(a.new_v + nbase + (int64_t)t * D);
                    // slot-patched step: row t into its pool slot (one tile stores it)
                    if (APPEND && tile == 0) {
                        const int32_t* sr = a.ap.slots + (int64_t)b * a.NQ;
                        if (stores_row(sr, a.NQ, t, a.ap.n_slot)) {
                            const int64_t dst = ((int64_t)sr[t] * a.KV + kh) * D + j * VEC;
                            *reinterpret_cast<uint4*>(static_cast<T*>(a.ap.k_dst) + dst) = kr[i];
                            *reinterpret_cast<uint4*>(static_cast<T*>(a.ap.v_dst) + dst) = vr[i];
                        }
                    }
                } else {
                    kr[i] = make_uint4(0, 0, 0, 0);
                    vr[i] = make_uint4(0, 0, 0, 0);
                }
            }
            valu_attend<T, LPR, TPI, NTOK, RT, kModeNew>(kr, vr, qf, m, l, o, g, 0, t0, a.NQ,
                                                        a.causal, row0);
        }
    }

    // ---- merge: key groups of the wave, then the 4 waves through LDS ----
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const float M = across_groups_max<LPR>(m[r]);
        const float w = fast_exp2(m[r] - M);
        l[r] = across_groups_sum<LPR>(l[r] * w);
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[r][e] = across_groups_sum<LPR>(o[r][e] * w);
        m[r] = M;
    }
    __shared__ float s_o[4][RT][D];
    __shared__ float s_m[4][RT], s_l[4][RT];
    if (g == 0) {
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int e = 0; e < VEC; ++e) s_o[wave][r][j * VEC + e] = o[r][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            s_m[wave][r] = m[r];
            s_l[wave][r] = l[r];
        }
    }
    __syncthreads();

    const int nrows = min(RT, R - row0);
    const bool single = n_seq == 1;
    emit_rows<T, D, RT>(a, s_o, s_m, s_l, nrows, grow0, part, single);
}

}  // namespace pa
