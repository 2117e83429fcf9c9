// Dense (training) GQA attention backward on the matrix cores (gfx950,
// fp16/bf16): the gradient half of execute() on the docs.rs page
// "onnxruntime-ep-mlx 0.31.1: src/ops/attention_vjp/dense.rs". With P the
// recomputed softmax (masks and the top-left causal limit as in the forward),
// Y = P V and dY the output gradient:
//   dP = dY V^T,  delta = rowsum(Y * dY),  dS = P * (dP - delta),
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dY,
// dK and dV of KV head kh summed over the G query heads h = kh*G + g.
//
// Launches: the forward kernel in its statistics form (per query row the
// base-2 log-sum-exp of the scores and delta, Y kept in fp32 and never stored),
// then the two kernels below, which recompute P from those statistics:
//   dense_bwd_dq   - a workgroup per (sequence, KV head, block of positions),
//                    the forward's rows layout; K and V stream through a ring;
//   dense_bwd_dkdv - a workgroup per (sequence, KV head, 16*NW keys), each wave
//                    holding 16 keys; the Q/dY rows of all G heads stream
//                    through a ring, so the group sums stay in registers (one
//                    writer per dK/dV row, no atomics); under the causal limit
//                    (G >= 2) each workgroup takes half the heads of two key
//                    blocks and dense_bwd_sum_halves adds the two halves.
// Every streamed tile of 16 rows (K and V, or Q and dY) is loaded once into a
// slot whose two halves both use the layout the transposing LDS read needs;
// rows are read from the same layout (slot_read_rows_v), so each half serves
// both operand forms its products take.
#pragma once

#include "dense_mfma.hpp"

namespace pa {

template <typename T>
struct BwdArgs {
    const T* dout;  // dY [B, HQ, SQ, D]
    T* dq;          // [B, HQ, SQ, D]
    T* dk;          // [B, HK, SK, D]
    T* dv;
    float scale;
    // causal, G >= 2 (SPLIT): fp32 sums of the two head halves, [2][B*HK*SK*D]
    // each for dK (already scaled) and dV; dense_bwd_sum_halves adds them
    float* part_dk;
    float* part_dv;
    int64_t part_n;  // B*HK*SK*D
};

// The 16-byte chunks 32*kk + 8*g16 of one row of D elements (an operand whose
// lane holds that row): plain global loads.
template <typename T, int D>
__device__ __forceinline__ void frag_load(const T* row, int g16, u32x4_t (&op)[D / 32]) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        const uint4 v = load16(row + 32 * kk + 8 * g16);
        op[kk] = u32x4_t{v.x, v.y, v.z, v.w};
    }
}

// Value j of four wave-uniform values for the lanes of group j (mask[j] all
// ones there, zero elsewhere): bitwise, exact for every value.
__device__ __forceinline__ float pick4(float a, float b, float c, float d,
                                       const uint32_t (&mask)[4]) {
    return __uint_as_float((__float_as_uint(a) & mask[0]) | (__float_as_uint(b) & mask[1]) |
                           (__float_as_uint(c) & mask[2]) | (__float_as_uint(d) & mask[3]));
}

// dQ: rows as in dense_mfma (R = G*P rows of one (b, kh) and P positions, NRT
// 16-row tiles per wave); per 16-key tile, S^T = K Q^T and dP^T = V dY^T give
// this lane's row c16 against keys 4*g16 + e, then dS and dQ += dS K.
template <typename T, int D, int NW, int NRT, int kRing, int MASK, bool PAIR>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dense_bwd_dq(DenseArgs<T> d, BwdArgs<T> w, const float* __restrict__ lse,
                  const float* __restrict__ delta) {
    using Lay = SlotLayout<T, D>;
    using M = Mfma<T>;
    constexpr int KS = D / 32, NT = D / 16;
    constexpr int NWI = NW < KS ? NW : KS;  // waves that issue loads
    constexpr int IPW = KS / NWI;           // instructions per half per issuing wave
    constexpr int OPS = 2 * IPW;            // per key tile: two halves
    constexpr int TB = Lay::kBytes;         // bytes of one key tile
    static_assert(D % 32 == 0 && Lay::kOps == KS && KS % NWI == 0, "shape");
    static_assert(kRing >= 3 && OPS * (kRing - 2) <= 63, "ring");

    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int lane = threadIdx.x & 63, c16 = lane & 15, g16 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const DenseGeometry& g = d.g;
    const int nw = PAIR ? (g.nblk + 1) / 2 : g.nblk;  // workgroups per (b, kh)
    const int wg = blockIdx.x % nw;
    const int kh = (blockIdx.x / nw) % g.HK;
    const int b = blockIdx.x / (nw * g.HK);
    const int64_t kv0 = ((int64_t)b * g.HK + kh) * g.SK * D;
    const T* const kb = d.k + kv0;
    const T* const vb = d.v + kv0;
    const int64_t head0 = (int64_t)b * g.HQ + (int64_t)kh * g.G;  // first query head of the group
    const bool issues = wave < NWI;

    for (int half = 0; half < (PAIR ? 2 : 1); ++half) {
    const int blk = half == 0 ? wg : g.nblk - 1 - wg;
    if (half == 1) {
        if (blk == wg) break;  // odd block count: the middle block has no partner
        asm volatile("" ::: "memory");
        __syncthreads();      // every wave is done with the ring before it is refilled
    }
    const int i0 = blk * g.P;
    const int R = g.G * g.P;
    const int pend = min(g.P, g.SQ - i0);
    int kend = g.SK;
    if (g.causal) kend = min(kend, i0 + pend);
    if (MASK && d.mw != 1 && d.mw < g.SK) kend = min(kend, d.mw);
    const int n_sub = (kend + 15) / 16;
    const bool has_rows = 16 * NRT * wave < R;

    // this lane's row of tile rt (row c16), clamped to a real one
    int srow_p[NRT], srow_h[NRT];
    u32x4_t qop[NRT][KS], gop[NRT][KS];
    float lse_r[NRT], dl_r[NRT];
    f32x4_t acc[NRT][NT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int r = min(16 * (wave * NRT + rt) + c16, R - 1);
        srow_p[rt] = min(r % g.P, pend - 1);
        srow_h[rt] = kh * g.G + r / g.P;
        const int64_t row = ((int64_t)b * g.HQ + srow_h[rt]) * g.SQ + i0 + srow_p[rt];
        frag_load<T, D>(d.q + row * D, g16, qop[rt]);
        frag_load<T, D>(w.dout + row * D, g16, gop[rt]);
        lse_r[rt] = lse[row];
        dl_r[rt] = delta[row];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[rt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // the row operands, before the ring's loads

    // key tile s: K | V, both halves in the transposable layout
    auto fetch_tile = [&](int s) {
        const int64_t o = (int64_t)16 * s * D;
        const int rmax = min(15, g.SK - 1 - 16 * s);
        fetch_rows<T, D, IPW, true>(kb + o, vb + o, rmax, smem + (s % kRing) * TB, lane, wave,
                                    NWI);
    };
    for (int s = 0; s < kRing - 1 && s < n_sub; ++s)
        if (issues) fetch_tile(s);
    for (int i = 0; i < n_sub; ++i) {
        const int ahead = min(kRing - 2, n_sub - 1 - i);  // tiles fetched after i
        if (issues) wait_ahead<OPS, kRing - 2>(ahead);
        else __builtin_amdgcn_s_waitcnt(kWaitVm0);
        // every wave's part of tile i is in; slot i - 1 is read out
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int nxt = i + kRing - 1;
        if (nxt < n_sub && issues) fetch_tile(nxt);
        if (!has_rows) continue;
        const char* sa = smem + (i % kRing) * TB;
        u32x4_t kop[KS], vop[KS];
        u32x2_t kt[NT];
        slot_read_rows_v<T, D>(sa, c16, g16, kop);
        slot_read_rows_v<T, D>(sa + Lay::kKBytes, c16, g16, vop);
        slot_read_cols_at<T, D>(sa, c16, g16, kt);
        slot_lds_wait<D>(kt);
        const int key0 = 16 * i;
        const int valid = min(16, kend - key0);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            f32x4_t st = f32x4_t{0.f, 0.f, 0.f, 0.f}, dpt = st;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                st = M::qk(kop[kk], qop[rt][kk], st);
                dpt = M::qk(vop[kk], gop[rt][kk], dpt);
            }
            const int lim = g.causal ? max(0, min(valid, i0 + srow_p[rt] - key0 + 1)) : valid;
            float ds[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * g16 + e;
                float x = st[e] * d.qscale;
                if constexpr (MASK != 0)
                    x += mask_bias2<MASK>(d, b, srow_h[rt], i0 + srow_p[rt],
                                          min(key0 + j, d.mw - 1));
                const float p = j < lim ? fast_exp2(x - lse_r[rt]) : 0.f;
                ds[e] = p * (dpt[e] - dl_r[rt]);
            }
            u32x2_t phi, plo;
            M::make_p(ds, phi, plo);
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[rt][t] = M::pv(phi, plo, kt[t], acc[rt][t]);
        }
    }
    if (has_rows) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * (wave * NRT + rt) + 4 * g16 + i;
                if (r >= R || r % g.P >= pend) continue;
                T* dst = w.dq + ((head0 + r / g.P) * g.SQ + i0 + r % g.P) * D + c16;
#pragma unroll
                for (int t = 0; t < NT; ++t) Elem<T>::store(dst + 16 * t, acc[rt][t][i] * w.scale);
            }
    }
    }  // blocks of this workgroup
}

// dK, dV: key wave kw (0..NW-1) of a workgroup holds keys kw0 .. kw0 + 15 of
// (b, kh) as operands (K, V rows); two sets of NW waves hold the same keys and
// take alternate tiles of the Q/dY rows of the G query heads (16 rows a tile),
// so two waves share each SIMD. Per tile, S = Q K^T and dP = dY
// V^T give query rows 4*g16 + e against this lane's key c16, then dV += P^T dY
// and dK += dS^T Q. At the end the second set hands its accumulators to the
// first through LDS. The tile's 16 log-sum-exps and deltas are read with
// scalar loads (lse and delta are read-only here), which the vector-memory
// counter of the ring does not see; the statistics arrays hold 16 entries of
// padding past the last row.
// Tiles run position-major from the last position tile down, heads inside, so
// that the workgroups of every key block of (b, kh) start on the same tile and
// read the same rows at about the same time (under the causal limit each stops
// at its own first tile).
// SPLIT (causal, G >= 2): under the causal limit key block kb has tiles in
// proportion to nkb - kb, so workgroup pair (2*w, 2*w + 1) takes the query heads
// [0, G/2) and [G/2, G) of key block w and then of key block nkb - 1 - w: every
// workgroup has the same work. Sums go to BwdArgs::part_* (fp32).
template <typename T, int D, int NW, int kRing, int MASK, bool SPLIT>
__global__ __launch_bounds__(128 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dense_bwd_dkdv(DenseArgs<T> d, BwdArgs<T> w, const float* __restrict__ lse,
                    const float* __restrict__ delta) {
    using Lay = SlotLayout<T, D>;
    using M = Mfma<T>;
    constexpr int NSET = 2;                 // wave sets (alternate query tiles)
    constexpr int KS = D / 32, NT = D / 16;
    constexpr int NWI = NW < KS ? NW : KS;  // waves of a set that issue its loads
    constexpr int IPW = KS / NWI;
    constexpr int OPS = 2 * IPW;            // per tile: two halves
    constexpr int TB = Lay::kBytes;         // bytes of one tile
    static_assert(D % 32 == 0 && Lay::kOps == KS && KS % NWI == 0, "shape");
    static_assert(kRing >= 3 && OPS * (kRing - 2) <= 63, "ring");
    static_assert(NW * 2 * NT * 4 * 64 * 4 <= kRing * NSET * TB, "hand-off fits the ring");

    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int lane = threadIdx.x & 63, c16 = lane & 15, g16 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int set = wave / NW, kw = wave % NW;
    const DenseGeometry& g = d.g;
    const int nkb = (g.SK + 16 * NW - 1) / (16 * NW);  // key blocks per (b, kh)
    const int npair = SPLIT ? (nkb + 1) / 2 : nkb;      // workgroup (pairs) per (b, kh)
    const int part = SPLIT ? (int)(blockIdx.x & 1) : 0;
    const int wgi = SPLIT ? (int)(blockIdx.x >> 1) : (int)blockIdx.x;
    const int wblk = wgi % npair;
    const int kh = (wgi / npair) % g.HK;
    const int b = wgi / (npair * g.HK);
    const int64_t kv0 = ((int64_t)b * g.HK + kh) * g.SK;
    const int64_t head0 = (int64_t)b * g.HQ + (int64_t)kh * g.G;
    const bool issues = kw < NWI;
    const int g_lo = SPLIT ? part * (g.G / 2) : 0;  // the heads [g_lo, g_lo + GH) of the group
    const int GH = SPLIT ? (part == 0 ? g.G / 2 : g.G - g.G / 2) : g.G;
    // all-ones for the lane's 16-lane group g16, zero for the others (opaque to
    // the optimizer, which would otherwise turn the pick into an indexed
    // private array)
    uint32_t gmask[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        gmask[j] = g16 == j ? 0xffffffffu : 0u;
        asm volatile("" : "+v"(gmask[j]));
    }

    for (int half = 0; half < (SPLIT ? 2 : 1); ++half) {
    const int kblk = half == 0 ? wblk : nkb - 1 - wblk;
    if (half == 1) {
        if (kblk == wblk) break;  // odd block count: the middle block has no partner
        asm volatile("" ::: "memory");
        __syncthreads();          // the first block's hand-off is read out
    }
    const int kw0 = kblk * 16 * NW + 16 * kw;  // this wave's first key
    const bool has_keys = kw0 < g.SK;
    u32x4_t kfr[KS], vfr[KS];
    {
        const int64_t kr = kv0 + min(kw0 + c16, g.SK - 1);
        frag_load<T, D>(d.k + kr * D, g16, kfr);
        frag_load<T, D>(d.v + kr * D, g16, vfr);
    }
    f32x4_t dk[NT], dv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) dk[t] = dv[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_s_waitcnt(kWaitVm0);

    // query tiles: head gg of the group, positions 16*it .. +15; under the
    // causal limit positions before the block's first key see none of its keys.
    // Tile t: position tile ntile - 1 - t / GH, head g_lo + t % GH. Iteration u
    // holds tiles 2u (set 0) and 2u + 1 (set 1).
    const int ntile = (g.SQ + 15) / 16;
    const int it0 = g.causal ? min(ntile, kblk * NW) : 0;
    const int nit = ntile - it0;
    const int n_t = GH * nit;
    const int n_u = (n_t + 1) / 2;
    // a set past the last tile loads the last one again, so every issuing wave
    // has the same loads in flight per iteration
    auto fetch = [&](int u) {
        const int t = min(2 * u + set, n_t - 1);
        const int tp = t / GH;
        const int gg = g_lo + t - tp * GH, q0 = 16 * (ntile - 1 - tp);
        const int64_t r0 = (head0 + gg) * g.SQ + q0;
        fetch_rows<T, D, IPW, true>(d.q + r0 * D, w.dout + r0 * D, min(15, g.SQ - 1 - q0),
                                    smem + ((u % kRing) * NSET + set) * TB, lane, kw, NWI);
    };
    for (int u = 0; u < kRing - 1 && u < n_u; ++u)
        if (issues) fetch(u);
    const float* const lse0 = lse + head0 * g.SQ;  // statistics of the group's first row
    const float* const dl0 = delta + head0 * g.SQ;
    for (int u = 0; u < n_u; ++u) {
        const int t = 2 * u + set;
        const int tc = min(t, n_t - 1);
        const int tp = tc / GH;
        const int gg = g_lo + tc - tp * GH;    // head of the group
        const int q0 = 16 * (ntile - 1 - tp);  // first query position of the tile
        const int hq = kh * g.G + gg;
        const int sr = __builtin_amdgcn_readfirstlane(gg * g.SQ + q0);  // < 2^31 (checked)
        const float* ls = lse0 + sr;
        const float* dl = dl0 + sr;
        float lv[16], dv16[16];  // uniform loads of all 16 rows, then a per-lane pick
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            lv[j] = ls[j];
            dv16[j] = dl[j];
        }
        float lr[4], dr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // row 4*g16 + e of the tile
            lr[e] = pick4(lv[e], lv[4 + e], lv[8 + e], lv[12 + e], gmask);
            dr[e] = pick4(dv16[e], dv16[4 + e], dv16[8 + e], dv16[12 + e], gmask);
        }
        const int ahead = min(kRing - 2, n_u - 1 - u);
        if (issues) wait_ahead<OPS, kRing - 2>(ahead);
        else __builtin_amdgcn_s_waitcnt(kWaitVm0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int nxt = u + kRing - 1;
        if (nxt < n_u && issues) fetch(nxt);
        if (t >= n_t || !has_keys || (g.causal && kw0 > q0 + 15)) continue;  // nothing visible
        const char* sl = smem + ((u % kRing) * NSET + set) * TB;
        u32x4_t qa[KS], ga[KS];
        u32x2_t gt[NT], qt[NT];
        slot_read_rows_v<T, D>(sl, c16, g16, qa);
        slot_read_rows_v<T, D>(sl + Lay::kKBytes, c16, g16, ga);
        slot_read_cols_at<T, D>(sl, c16, g16, qt);
        slot_read_cols_at<T, D>(sl + Lay::kKBytes, c16, g16, gt);
        slot_lds_wait<D>(gt);
        slot_lds_wait<D>(qt);
        f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f}, dp = s;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            s = M::qk(qa[kk], kfr[kk], s);
            dp = M::qk(ga[kk], vfr[kk], dp);
        }
        const int kj = kw0 + c16;
        float p[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int qi = q0 + 4 * g16 + e;
            bool vis = kj < g.SK && qi < g.SQ && (!g.causal || kj <= qi);
            float x = s[e] * d.qscale;
            if constexpr (MASK != 0) {
                vis = vis && (d.mw == 1 || kj < d.mw);
                x += mask_bias2<MASK>(d, b, hq, min(qi, g.SQ - 1), min(kj, d.mw - 1));
            }
            p[e] = vis ? fast_exp2(x - lr[e]) : 0.f;
            ds[e] = p[e] * (dp[e] - dr[e]);
        }
        u32x2_t phi, plo, dhi, dlo;
        M::make_p(p, phi, plo);
        M::make_p(ds, dhi, dlo);
#pragma unroll
        for (int v = 0; v < NT; ++v) {
            dv[v] = M::pv(phi, plo, gt[v], dv[v]);
            dk[v] = M::pv(dhi, dlo, qt[v], dk[v]);
        }
    }
    // the second set's sums go to the first through the (now idle) ring
    asm volatile("" ::: "memory");
    __syncthreads();
    float* const red = reinterpret_cast<float*>(smem) + (size_t)kw * 2 * NT * 4 * 64;
    if (set == 1 && has_keys) {
#pragma unroll
        for (int v = 0; v < NT; ++v)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                red[(v * 4 + i) * 64 + lane] = dk[v][i];
                red[((NT + v) * 4 + i) * 64 + lane] = dv[v][i];
            }
    }
    __syncthreads();
    if (set == 0 && has_keys) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = kw0 + 4 * g16 + i;
            if (key >= g.SK) continue;
            const int64_t o = (kv0 + key) * D + c16;
#pragma unroll
            for (int v = 0; v < NT; ++v) {
                const float ks = (dk[v][i] + red[(v * 4 + i) * 64 + lane]) * w.scale;
                const float vs = dv[v][i] + red[((NT + v) * 4 + i) * 64 + lane];
                if constexpr (SPLIT) {
                    w.part_dk[part * w.part_n + o + 16 * v] = ks;
                    w.part_dv[part * w.part_n + o + 16 * v] = vs;
                } else {
                    Elem<T>::store(w.dk + o + 16 * v, ks);
                    Elem<T>::store(w.dv + o + 16 * v, vs);
                }
            }
        }
    }
    }  // key blocks of this workgroup
}

// dK = part_dk[0] + part_dk[1], dV likewise, rounded once to the I/O dtype;
// four elements per thread (part_n is a multiple of 64).
template <typename T>
__global__ __launch_bounds__(256) void dense_bwd_sum_halves(BwdArgs<T> w) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= 2 * w.part_n) return;
    const bool is_v = e >= w.part_n;
    const int64_t o = is_v ? e - w.part_n : e;
    const float* p = is_v ? w.part_dv : w.part_dk;
    const float4 a = *reinterpret_cast<const float4*>(p + o);
    const float4 c = *reinterpret_cast<const float4*>(p + w.part_n + o);
    T* dst = (is_v ? w.dv : w.dk) + o;
    Elem<T>::store(dst + 0, a.x + c.x);
    Elem<T>::store(dst + 1, a.y + c.y);
    Elem<T>::store(dst + 2, a.z + c.z);
    Elem<T>::store(dst + 3, a.w + c.w);
}

}  // namespace pa
