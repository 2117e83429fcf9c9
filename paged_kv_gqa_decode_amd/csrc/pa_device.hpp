// Device helpers for the gfx950 paged decode kernels: element conversion,
// 16-byte vector loads, DPP/shuffle reductions and base-2 exponentials.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Storage type for bfloat16 elements (only its bits are used).
struct bf16_t {
    uint16_t bits;
};

constexpr float kLog2e = 1.4426950408889634f;
// Finite "minus infinity" for running maxima: exp2(x - kNegMax) never produces
// NaN, and an empty state (m = kNegMax, l = 0) merges with weight 0.
constexpr float kNegMax = -3.402823466e+38f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest-even float -> bfloat16 bits; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Element traits: how one 16-byte lane load unpacks into fp32 values, and how
// an fp32 result is stored with round-to-nearest-even.
template <typename T> struct Elem;

template <> struct Elem<float> {
    static constexpr int kVec = 4;
    __device__ static __forceinline__ void unpack(const uint4& r, float* f) {
        f[0] = __uint_as_float(r.x);
        f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z);
        f[3] = __uint_as_float(r.w);
    }
    __device__ static __forceinline__ void store(float* p, float v) { *p = v; }
    __device__ static __forceinline__ float load(const float* p) { return *p; }
};

template <> struct Elem<_Float16> {
    static constexpr int kVec = 8;
    __device__ static __forceinline__ void unpack_word(uint32_t w, float* f) {
        f[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
        f[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
    __device__ static __forceinline__ void unpack(const uint4& r, float* f) {
        unpack_word(r.x, f + 0);
        unpack_word(r.y, f + 2);
        unpack_word(r.z, f + 4);
        unpack_word(r.w, f + 6);
    }
    __device__ static __forceinline__ void store(_Float16* p, float v) { *p = (_Float16)v; }
    __device__ static __forceinline__ float load(const _Float16* p) { return (float)*p; }
};

template <> struct Elem<bf16_t> {
    static constexpr int kVec = 8;
    __device__ static __forceinline__ void unpack_word(uint32_t w, float* f) {
        f[0] = __uint_as_float(w << 16);
        f[1] = __uint_as_float(w & 0xffff0000u);
    }
    __device__ static __forceinline__ void unpack(const uint4& r, float* f) {
        unpack_word(r.x, f + 0);
        unpack_word(r.y, f + 2);
        unpack_word(r.z, f + 4);
        unpack_word(r.w, f + 6);
    }
    __device__ static __forceinline__ void store(bf16_t* p, float v) {
        p->bits = f32_to_bf16_rne(v);
    }
    __device__ static __forceinline__ float load(const bf16_t* p) {
        return __uint_as_float((uint32_t)p->bits << 16);
    }
};

// Partial outputs of the matrix-core family's split pieces. fp16 I/O: o / l
// stored as fp16 (|o / l| <= max |v|, which fp16 holds; 2^-12 relative), half
// the bytes of the workspace round trip; the merge weighs piece p by 2^(m_p -
// M) * l_p. Other types: the unnormalised fp32 o, weighed by 2^(m_p - M).
template <typename T> struct Partial {
    using type = float;
    static constexpr bool kNorm = false;
};
template <> struct Partial<_Float16> {
    using type = _Float16;
    static constexpr bool kNorm = true;
};

__device__ __forceinline__ uint4 load16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// ---------------------------------------------------------------------------
// Cross-lane reductions. DPP controls (GFX9 encoding): quad_perm selectors in
// bits [7:0]; row_ror:n = 0x120 + n; row_half_mirror = 0x141.
// ---------------------------------------------------------------------------
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, true));
}
constexpr int kDppXor1 = 0xb1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4e;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i of an 8-lane half <- lane 7-i
constexpr int kDppRor4 = 0x124;       // rotate a 16-lane row by 4
constexpr int kDppRor8 = 0x128;       // rotate a 16-lane row by 8

// Sum over aligned groups of N consecutive lanes; every lane of a group gets
// the group's total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "N");
    if constexpr (N >= 2) x += dpp<kDppXor1>(x);
    if constexpr (N >= 4) x += dpp<kDppXor2>(x);
    if constexpr (N == 8) x += dpp<kDppHalfMirror>(x);
    if constexpr (N >= 16) {
        x += dpp<kDppRor4>(x);
        x += dpp<kDppRor8>(x);
    }
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    if constexpr (N >= 64) x += __shfl_xor(x, 32);
    return x;
}

// Max / sum across lanes that differ only in the bits of [kFrom, 64): combines
// the groups of kFrom consecutive lanes.
template <int kFrom>
__device__ __forceinline__ float across_groups_max(float x) {
#pragma unroll
    for (int m = kFrom; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}
template <int kFrom>
__device__ __forceinline__ float across_groups_sum(float x) {
#pragma unroll
    for (int m = kFrom; m < 64; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

__device__ __forceinline__ float wave_max(float x) { return across_groups_max<1>(x); }
__device__ __forceinline__ float wave_sum(float x) { return across_groups_sum<1>(x); }

// The slot-patched step (docs.rs page "onnxruntime-ep-mlx 0.31.1:
// src/ops/paged_attention.rs", VECTOR_BODY's `position` slots; the page
// "onnxruntime-ep-mlx 0.31.1: src/engine.rs", write_back_input_patches): new row j of sequence b is stored into token
// slot slots[b*NQ + j] (block * BS + offset) of both pools, every KV head, and
// a cached position of sequence b whose slot one of its new rows names reads
// that row instead of the pool (the highest such j). Slots outside [0, n_slot)
// are neither stored nor read.
struct AppendArgs {
    const int32_t* slots;  // [B][NQ]; nullptr: the plain step (pools read only)
    void* k_dst;           // the pools, written (the same memory as k_pool / v_pool)
    void* v_dst;
    int64_t n_slot;        // num_blocks * block_size
};

// New row j is the one stored in slot s: s is a real slot and no later new row
// of the sequence names it (sl = the sequence's NQ slots).
__device__ __forceinline__ bool stores_row(const int32_t* sl, int NQ, int j, int64_t n_slot) {
    const int32_t s = sl[j];
    if (s < 0 || s >= n_slot) return false;
    for (int jj = j + 1; jj < NQ; ++jj)
        if (sl[jj] == s) return false;
    return true;
}

}  // namespace pa
