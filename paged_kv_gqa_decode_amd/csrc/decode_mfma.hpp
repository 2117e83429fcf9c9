// Pass 1 of paged GQA decode attention on the matrix cores (gfx950, fp16/bf16),
// with the work cut into equal per-wave segments (split.hpp).
//
// Operation: docs.rs page "onnxruntime-ep-mlx 0.31.1: src/ops/paged_attention.rs",
// VECTOR_BODY (scores, online softmax, accumulation) and VECTOR_PARTIALS.
//
// A wave attends one piece (a run of 16-key sub-pages of one (sequence, KV
// head) unit) at a time, for all R = G*NQ query rows of the KV head in row
// tiles of 16, so each K/V page is fetched from HBM once per GQA group:
//   scores  S^T[16 keys x 16 rows] = K Q^T  : v_mfma_f32_16x16x32 (D/32 steps);
//           A = K: lane l holds key l%16, 8 elements of d; B = Q: row l%16
//   softmax fp32 on the VALU; the D-layout of S^T (key 4*(l/16)+i, row l%16)
//           is exactly the A layout of the next product, so P stays in lane
//   output  O[16 rows x 16 d] += P V        : v_mfma_f32_16x16x16 per 16 d;
//           B = V: lane l needs keys 4*(l/16)..+3 at one d. Each lane loads the
//           dword (d, d+1) of its 4 keys and v_perm splits it into the
//           operands of two d-columns, so output tile 2j holds d = 32j + 2c and
//           tile 2j+1 holds d = 32j + 2c + 1 for column c.
// bf16 probabilities are split into hi + lo bf16 parts (two products), so P
// keeps ~16 significant bits; fp16 P keeps 11. The reference max moves only
// when a score exceeds it by more than 2^kSlack (probabilities stay <= 256),
// so the accumulators are rescaled almost never.
// Block-table entries of a piece are read 64 pages at a time into one VGPR
// (lane i = page i) and taken with readlane. K/V sub-pages are staged through
// LDS: each wave owns one sub-page slot; buffer loads write it directly
// (no VGPRs held by loads in flight), the wave copies it to registers in the
// MFMA operand layout and immediately issues the next sub-page into the slot,
// so one sub-page per wave is always in flight while the previous is computed.
// Small register footprint -> 4 waves per SIMD; many waves, each with one
// sub-page in flight, is what keeps HBM busy on this part.
#pragma once

#include "split.hpp"

namespace pa {

typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

template <typename T> struct Mfma;

template <> struct Mfma<_Float16> {
    static constexpr bool kSplitP = false;
    __device__ static __forceinline__ f32x4_t qk(u32x4_t k, u32x4_t q, f32x4_t acc) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, k),
                                                      __builtin_bit_cast(f16x8_t, q), acc, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4_t pv(u32x2_t p, u32x2_t v, f32x4_t acc) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, p),
                                                     __builtin_bit_cast(f16x4_t, v), acc, 0, 0, 0);
    }
    __device__ static __forceinline__ unsigned pack2(float lo, float hi) {
        return (unsigned)__builtin_bit_cast(uint16_t, (_Float16)lo) |
               ((unsigned)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
    }
};

template <> struct Mfma<bf16_t> {
    static constexpr bool kSplitP = true;
    __device__ static __forceinline__ f32x4_t qk(u32x4_t k, u32x4_t q, f32x4_t acc) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k),
                                                       __builtin_bit_cast(bf16x8_t, q), acc, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4_t pv(u32x2_t p, u32x2_t v, f32x4_t acc) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, p),
                                                         __builtin_bit_cast(i16x4_t, v), acc, 0, 0, 0);
    }
    __device__ static __forceinline__ unsigned pack2(float lo, float hi) {
        return (unsigned)f32_to_bf16_rne(lo) | ((unsigned)f32_to_bf16_rne(hi) << 16);
    }
};

__device__ __forceinline__ float bf16_round(float x) {
    return __uint_as_float((unsigned)f32_to_bf16_rne(x) << 16);
}

// Raw buffer descriptor over `bytes` bytes at p (GFX9-family format word).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// s_waitcnt immediates (GFX9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8]
// | vmcnt[5:4] << 14): wait for all vector-memory operations, or for all LDS ops.
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;

// Slack of the lazy reference max, in log2 units (probabilities stay <= 256).
constexpr float kSlack = 8.0f;

template <typename T>
struct SplitArgs {
    const T* q;
    const T* k_pool;
    const T* v_pool;
    const int32_t* block_table;
    const int32_t* context_lens;
    const T* new_k;
    const T* new_v;
    T* out;
    float* ws_o;   // [slots][R][D]  unnormalised partial outputs
    float* ws_ml;  // [slots][R][2]  (max, sum) in base-2 units
    int32_t* meta; // [B*KV][2]      first and last segment overlapping each unit
    SplitGeometry g;
    int H, causal, max_blocks, R;
    float qscale;  // scale * log2(e)
};

template <int KS, int NP>
struct SubPage {
    u32x4_t k[KS];      // key c16, d = 32*kk + 8*g16 .. +8
    unsigned v[NP][4];  // keys 4*g16 + j, d = 32*np + 2*c16 .. +1
};

// LDS layout of one sub-page slot (16 keys): K operands first, one 16-byte
// chunk per lane per score step (kk*1024 + lane*16); then V, one 16-byte chunk
// per lane per output tile pair holding the dwords of keys 4*g16 + 0..3.
template <typename T, int D>
struct SlotLayout {
    static constexpr int kKBytes = 16 * D * (int)sizeof(T);
    static constexpr int kBytes = 2 * kKBytes;
};

template <typename T, int D, int BS, int NRT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NRT == 1 ? 4 : 1, 4)))
void decode_mfma(SplitArgs<T> a) {
    using M = Mfma<T>;
    constexpr int KS = D / 32;    // score MFMA steps over d
    constexpr int NT = D / 16;    // output tiles over d
    constexpr int NP = D / 32;    // output tile pairs
    constexpr int SUB = BS / 16;  // 16-key sub-pages per page
    static_assert(D % 32 == 0 && BS % 16 == 0, "shape");

    using Slot = SlotLayout<T, D>;
    extern __shared__ __attribute__((aligned(16))) char smem[];  // 4 slots, then the prefix
    int* s_pref = reinterpret_cast<int*>(smem + 4 * Slot::kBytes);
    build_prefix(a.context_lens, a.g, s_pref);
    const int64_t W = split_total(a.g, s_pref);
    const int64_t sigma = split_sigma(a.g, W);

    // The wave index is uniform within a wave; saying so keeps every per-piece
    // quantity (sequence, head, page, descriptors, LDS slot) in scalar registers.
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    char* slot_lds = smem + wave * Slot::kBytes;
    const int c16 = lane & 15, g16 = lane >> 4;
    const int gw = blockIdx.x * 4 + wave;  // this wave's segment
    int64_t x = (int64_t)gw * sigma;
    const int64_t x_end = min(W, x + sigma);
    if (x >= W) return;  // no barrier follows
    const int KV = a.g.KV, NQ = a.g.NQ, R = a.R;
    const int G = a.H / KV;
    const int nnew = (NQ + 15) / 16;
    const int64_t tstride = (int64_t)KV * D;

    int b = split_find_seq(a.g, s_pref, x);
    while (x < x_end) {
        while ((int64_t)KV * s_pref[b + 1] <= x) ++b;
        const int nsub = s_pref[b + 1] - s_pref[b];
        const int64_t seq_start = (int64_t)KV * s_pref[b];
        const int kh = (int)((x - seq_start) / nsub);
        const int64_t ustart = seq_start + (int64_t)kh * nsub;
        const int64_t pend = min(x_end, ustart + nsub);
        const int j0 = (int)(x - ustart), j1 = (int)(pend - ustart);
        const int L = min(max(a.context_lens[b], 0), a.g.max_tokens);
        const int nc = nsub - nnew;  // cached sub-pages = ceil(L / 16)
        const int64_t grow0 = ((int64_t)b * a.H + (int64_t)kh * G) * NQ;
        if (j0 == 0 && lane == 0 && a.meta) {  // the unit's first piece records its segments
            int32_t* mt = a.meta + 2 * ((int64_t)b * KV + kh);
            mt[0] = (int32_t)(ustart / sigma);
            mt[1] = (int32_t)((ustart + nsub - 1) / sigma);
        }

        // Q operand (B of S^T = K Q^T): row 16*rt + c16, d = 32*kk + 8*g16 .. +8
        u32x4_t qop[NRT][KS];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const int row = 16 * rt + c16;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                qop[rt][kk] = row < R ? *reinterpret_cast<const u32x4_t*>(
                                            a.q + (grow0 + row) * D + 32 * kk + 8 * g16)
                                      : u32x4_t{0, 0, 0, 0};
        }
        float m[NRT], lsum[NRT];
        f32x4_t acc[NRT][NT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            m[rt] = kNegMax;
            lsum[rt] = 0.f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }

        // Attend one 16-key sub-page: keys [0, valid) exist. For new rows
        // (is_new) key tau is new row t0 + tau, visible to query rows by causality.
        // kop(kk): K operand of score step kk; vquad(np): this lane's dwords of
        // keys 4*g16 + 0..3 at d = 32*np + 2*c16. Both read just before use.
        auto attend = [&](auto&& kop, auto&& vquad, int valid, bool is_new, int t0) {
            // V operands of output tiles 2*np and 2*np+1, built right before use
            auto vops = [&](int np, u32x2_t& lo, u32x2_t& hi) {
                const u32x4_t q4 = vquad(np);
                unsigned v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = (4 * g16 + j < valid) ? q4[j] : 0u;  // unused slots may be NaN
                lo = u32x2_t{__builtin_amdgcn_perm(v[1], v[0], 0x05040100u),
                             __builtin_amdgcn_perm(v[3], v[2], 0x05040100u)};
                hi = u32x2_t{__builtin_amdgcn_perm(v[1], v[0], 0x07060302u),
                             __builtin_amdgcn_perm(v[3], v[2], 0x07060302u)};
            };
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) s = M::qk(kop(kk), qop[rt][kk], s);
                float sv[4];
                const int row = 16 * rt + c16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tau = 4 * g16 + i;
                    bool vis = tau < valid;
                    if (is_new) vis = vis && (!a.causal || t0 + tau <= row % NQ);
                    sv[i] = vis ? s[i] * a.qscale : -__builtin_inff();
                }
                // m[rt] is the same in the 4 lanes of a row (lanes c16 + 16*g).
                float tm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
                if (__any(tm > m[rt] + kSlack)) {
                    tm = fmaxf(tm, __shfl_xor(tm, 16));
                    tm = fmaxf(tm, __shfl_xor(tm, 32));  // exact max of the row's 16 keys
                    const float mn = tm > m[rt] + kSlack ? tm : m[rt];
                    const float alpha = fast_exp2(m[rt] - mn);
                    m[rt] = mn;
                    lsum[rt] *= alpha;
                    float ai[4];  // output rows 4*g16 + i take the factor of that row
#pragma unroll
                    for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * g16 + i);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[rt][nt][i] *= ai[i];
                }
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sv[i] - m[rt]);
                lsum[rt] += (p[0] + p[1]) + (p[2] + p[3]);
                if constexpr (!M::kSplitP) {
                    const u32x2_t pop = u32x2_t{M::pack2(p[0], p[1]), M::pack2(p[2], p[3])};
#pragma unroll
                    for (int np = 0; np < NP; ++np) {
                        u32x2_t vlo, vhi;
                        vops(np, vlo, vhi);
                        acc[rt][2 * np] = M::pv(pop, vlo, acc[rt][2 * np]);
                        acc[rt][2 * np + 1] = M::pv(pop, vhi, acc[rt][2 * np + 1]);
                    }
                } else {
                    float hi[4], lo[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        hi[i] = bf16_round(p[i]);
                        lo[i] = p[i] - hi[i];
                    }
                    const u32x2_t phi = u32x2_t{M::pack2(hi[0], hi[1]), M::pack2(hi[2], hi[3])};
                    const u32x2_t plo = u32x2_t{M::pack2(lo[0], lo[1]), M::pack2(lo[2], lo[3])};
#pragma unroll
                    for (int np = 0; np < NP; ++np) {
                        u32x2_t vlo, vhi;
                        vops(np, vlo, vhi);
                        acc[rt][2 * np] = M::pv(phi, vlo, acc[rt][2 * np]);
                        acc[rt][2 * np] = M::pv(plo, vlo, acc[rt][2 * np]);
                        acc[rt][2 * np + 1] = M::pv(phi, vhi, acc[rt][2 * np + 1]);
                        acc[rt][2 * np + 1] = M::pv(plo, vhi, acc[rt][2 * np + 1]);
                    }
                }
            }
        };

        // ---- cached sub-pages [j0, jc) of this unit ----
        const int jc = min(j1, nc);
        if (j0 < jc) {
            const T* kpool = a.k_pool + (int64_t)kh * D;
            const T* vpool = a.v_pool + (int64_t)kh * D;
            const int32_t* trow = a.block_table + (int64_t)b * a.max_blocks;
            const int npages = (L + BS - 1) / BS;
            int pbase = -1000000, phys_lane = 0;  // lane i: block of page pbase + i
            // One buffer descriptor per sub-page (wave-uniform, scalar registers).
            // K: lane l fetches key c16, d = 32*kk + 8*g16 (16 bytes) into
            // kk*1024 + l*16. V: for output tile pair np and key quad i, lane l
            // fetches the dword of key 4*i + (l&3) at d = 32*np + 2*(l>>2) into
            // K_bytes + np*1024 + i*256 + l*4, which puts lane L's dwords of keys
            // 4*(L/16)+0..3 at K_bytes + np*1024 + L*16.
            const uint32_t koff = (uint32_t)((c16 * tstride + 8 * g16) * sizeof(T));
            const uint32_t voff = (uint32_t)(((lane & 3) * tstride + 2 * (lane >> 2)) * sizeof(T));
            const uint32_t quad = (uint32_t)(4 * tstride * sizeof(T));
            const int span = (int)(16 * tstride * sizeof(T));  // bytes a sub-page spans
            typedef __attribute__((address_space(3))) void lds_void;
            auto issue = [&](int j) {
                const int page = j / SUB, sub = j % SUB;
                if (page >= pbase + 64) {
                    pbase = page;
                    phys_lane = page + lane < npages ? trow[page + lane] : 0;
                }
                const int64_t phys = __builtin_amdgcn_readlane(phys_lane, page - pbase);
                const int64_t row0 = phys * BS + 16 * sub;
                const __amdgpu_buffer_rsrc_t kr = make_rsrc(kpool + row0 * tstride, span);
                const __amdgpu_buffer_rsrc_t vr = make_rsrc(vpool + row0 * tstride, span);
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        kr, (lds_void*)(slot_lds + kk * 1024), 16, koff, 64 * kk, 0, 0);
#pragma unroll
                for (int np = 0; np < NP; ++np)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            vr, (lds_void*)(slot_lds + Slot::kKBytes + np * 1024 + i * 256), 4,
                            voff, i * quad + 64 * np, 0, 0);
            };
            auto kop_lds = [&](int kk) {
                return *reinterpret_cast<const u32x4_t*>(slot_lds + kk * 1024 + lane * 16);
            };
            auto vquad_lds = [&](int np) {
                return *reinterpret_cast<const u32x4_t*>(slot_lds + Slot::kKBytes + np * 1024 +
                                                         lane * 16);
            };
            issue(j0);
            for (int j = j0; j < jc; ++j) {
                __builtin_amdgcn_s_waitcnt(kWaitVm0);    // sub-page j has landed in the slot
                attend(kop_lds, vquad_lds, min(16, L - 16 * j), false, 0);
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // slot read out: free for j + 1
                if (j + 1 < jc) issue(j + 1);
            }
        }

        // ---- new-row tiles [max(j0, nc), j1) of this unit ----
        const int64_t nbase = ((int64_t)b * KV + kh) * NQ;
        for (int j = max(j0, nc); j < j1; ++j) {
            const int t0 = 16 * (j - nc);
            SubPage<KS, NP> sp;
            const int tk = t0 + c16;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                sp.k[kk] = tk < NQ ? *reinterpret_cast<const u32x4_t*>(
                                         a.new_k + (nbase + tk) * D + 32 * kk + 8 * g16)
                                   : u32x4_t{0, 0, 0, 0};
#pragma unroll
            for (int np = 0; np < NP; ++np)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int tv = t0 + 4 * g16 + jj;
                    sp.v[np][jj] = tv < NQ ? *reinterpret_cast<const unsigned*>(
                                                 a.new_v + (nbase + tv) * D + 32 * np + 2 * c16)
                                           : 0u;
                }
            attend([&](int kk) { return sp.k[kk]; },
                   [&](int np) {
                       return u32x4_t{sp.v[np][0], sp.v[np][1], sp.v[np][2], sp.v[np][3]};
                   },
                   min(16, NQ - t0), true, t0);
        }

        // ---- emit: the finished output, or this piece's state for the combine ----
        const bool whole = (j0 == 0 && j1 == nsub);
        const int64_t slot = (int64_t)b * KV + kh + gw;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            float lrow = lsum[rt];
            lrow += __shfl_xor(lrow, 16);
            lrow += __shfl_xor(lrow, 32);  // l of row 16*rt + c16
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * rt + 4 * g16 + i;  // output row held in acc[rt][*][i]
                const float l_r = __shfl(lrow, 4 * g16 + i);
                if (r >= R) continue;
                if (whole) {
                    const float inv = l_r != 0.f ? 1.f / l_r : 0.f;
                    unsigned* dst = reinterpret_cast<unsigned*>(a.out + (grow0 + r) * D + 2 * c16);
#pragma unroll
                    for (int np = 0; np < NP; ++np)
                        dst[16 * np] = M::pack2(acc[rt][2 * np][i] * inv, acc[rt][2 * np + 1][i] * inv);
                } else {
                    f32x2_t* dst = reinterpret_cast<f32x2_t*>(a.ws_o + (slot * R + r) * D + 2 * c16);
#pragma unroll
                    for (int np = 0; np < NP; ++np)
                        dst[16 * np] = f32x2_t{acc[rt][2 * np][i], acc[rt][2 * np + 1][i]};
                }
            }
            if (!whole && g16 == 0 && 16 * rt + c16 < R) {
                float* ml = a.ws_ml + (slot * R + 16 * rt + c16) * 2;
                ml[0] = m[rt];
                ml[1] = lrow;
            }
        }
        x = pend;
    }
}

}  // namespace pa
