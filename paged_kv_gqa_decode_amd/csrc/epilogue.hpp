// End of pass 1, shared by the kernel families: merge the online-softmax
// states of the 4 waves of a workgroup (the role of VECTOR_REDUCE on the docs.rs
// page "onnxruntime-ep-mlx 0.31.1: src/ops/paged_attention.rs"), then either
// write the normalised output (sequence fits one partition) or the partition's
// state (VECTOR_PARTIALS), which the combine kernel merges (PARTIALS_REDUCE).
// The merge is a separate launch on purpose: making one workgroup's states
// visible to another inside a launch needs a device-scope release/acquire,
// which on this part writes back and invalidates the XCD's L2; issued once per
// workgroup it cost more than the whole decode step.
#pragma once

#include "pa_device.hpp"

namespace pa {

template <typename T>
struct DecodeArgs {
    const T* q;
    const T* k_pool;
    const T* v_pool;
    const int32_t* block_table;
    const int32_t* context_lens;
    const T* new_k;
    const T* new_v;
    T* out;
    float* ws_o;         // [rows][n_parts][D]  unnormalised partial outputs
    float* ws_ml;        // [rows][n_parts][2]  (max, sum) in base-2 units
    int H, KV, NQ, causal, max_blocks, chunk, n_parts, n_tiles;
    float qscale;        // scale * log2(e)
    AppendArgs ap;       // slot-patched step (ap.slots == nullptr: plain step)
};

// Partitions sequence b uses: one per `chunk` cached keys (at least one, for
// the new rows), never more than the launch provides.
__device__ __forceinline__ int partitions_of(int L, int chunk, int n_parts) {
    const int n = L > 0 ? (L - 1) / chunk + 1 : 1;
    return n < n_parts ? n : n_parts;
}

// Merge the 4 waves' states held in LDS for ROWS rows (rows >= nrows are
// padding) and emit them: the output when `single`, else this partition's
// state. Every thread of the workgroup calls this.
template <typename T, int D, int ROWS>
__device__ __forceinline__ void emit_rows(const DecodeArgs<T>& a, const float (*s_o)[ROWS][D],
                                          const float (*s_m)[ROWS], const float (*s_l)[ROWS],
                                          int nrows, int64_t grow0, int part, bool single) {
    for (int idx = threadIdx.x; idx < ROWS * D; idx += 256) {
        const int r = idx / D, d = idx % D;
        if (r >= nrows) continue;
        float M = s_m[0][r];
#pragma unroll
        for (int w = 1; w < 4; ++w) M = fmaxf(M, s_m[w][r]);
        float acc = 0.f, lt = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float wt = fast_exp2(s_m[w][r] - M);
            acc = fmaf(wt, s_o[w][r][d], acc);
            lt = fmaf(wt, s_l[w][r], lt);
        }
        const int64_t grow = grow0 + r;
        if (single) {
            Elem<T>::store(a.out + grow * D + d, lt != 0.f ? acc / lt : 0.f);
        } else {
            const int64_t slot = grow * a.n_parts + part;
            a.ws_o[slot * D + d] = acc;
            if (d == 0) {
                a.ws_ml[slot * 2 + 0] = M;
                a.ws_ml[slot * 2 + 1] = lt;
            }
        }
    }
}

}  // namespace pa
