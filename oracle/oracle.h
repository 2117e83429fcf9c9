/*
 * Reference oracle for paged-KV grouped-query decode attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls
 * this library: only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark do. It shares no code, header or constant with the HIP library.
 *
 * What it computes is the plain definition of the operation described on the
 * docs.rs source page "onnxruntime-ep-mlx 0.31.1: src/ops/paged_attention.rs"
 * (the VECTOR_BODY kernel text and the vector() launcher): for every sequence b,
 * query head h and new row r, gather the visible keys and values in logical
 * order (cached positions through the block table, then the step's new rows),
 * then apply a textbook max-subtracted softmax, all in double precision.
 *
 * Element types are given by a code: 0 = IEEE binary32, 1 = IEEE binary16,
 * 2 = bfloat16. Every stored element is widened exactly to double.
 *
 * Layouts (all row-major, contiguous):
 *   q, out       [B, H, NQ, D]
 *   k/v pool     [num_blocks, BS, KV, D]
 *   block_table  int32 [B, max_blocks]
 *   context_lens int32 [B]   cached (past) length, new rows excluded
 *   new_k/new_v  [B, KV, NQ, D]
 *   slot_mapping int32 [B, NQ] token slot of each new row, negative = none
 * Return value: 0 on success, a negative number on a malformed argument (no
 * partial output is guaranteed in that case).
 */
#ifndef PAGED_DECODE_ORACLE_H
#define PAGED_DECODE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Single-pass definition: gather, then softmax in double. out is double [B,H,NQ,D]. */
int oracle_paged_decode(int B, int H, int KV, int D, int BS, int max_blocks, int NQ,
                        int causal, int dtype, const void* q, const void* k_pool,
                        const void* v_pool, const int32_t* block_table,
                        const int32_t* context_lens, const void* new_k,
                        const void* new_v, float scale, double* out);

/*
 * Partitioned form: the visible keys of each row are cut into consecutive
 * chunks of `chunk` keys; each chunk yields (max m_c, sum Z_c, unnormalised
 * o_c); the chunks are merged with weights exp(m_c - M). Same output layout.
 * If part_m/part_z/part_o are non-NULL they receive each chunk's state, for
 * row index ((b*H + h)*NQ + r) and chunk c at [row*max_chunks + c] (part_o
 * additionally times D); chunks that do not exist are written as m = -inf,
 * Z = 0, o = 0.
 */
int oracle_paged_decode_partitioned(int B, int H, int KV, int D, int BS, int max_blocks,
                                    int NQ, int causal, int dtype, const void* q,
                                    const void* k_pool, const void* v_pool,
                                    const int32_t* block_table,
                                    const int32_t* context_lens, const void* new_k,
                                    const void* new_v, float scale, int chunk,
                                    int max_chunks, double* part_m, double* part_z,
                                    double* part_o, double* out);

/*
 * Stores this step's new rows into the pools: for b = 0..B-1, then j =
 * 0..NQ-1 (later stores replace earlier ones), if 0 <= slot_mapping[b*NQ + j]
 * < num_blocks*BS, token slot s = slot_mapping[b*NQ + j] (block s / BS, offset
 * s % BS) receives new row j of sequence b for every KV head. Decoding the
 * updated pools with oracle_paged_decode is the page's slot-patched read.
 */
int oracle_kv_append(int B, int KV, int D, int BS, int num_blocks, int NQ, int dtype,
                     void* k_pool, void* v_pool, const void* new_k, const void* new_v,
                     const int32_t* slot_mapping);

/*
 * Dense GQA attention forward (docs.rs page "onnxruntime-ep-mlx 0.31.1:
 * src/ops/attention_vjp/dense.rs", execute()): q [B, HQ, SQ, D], k/v
 * [B, HK, SK, D], out double [B, HQ, SQ, D]. s = scale * <q_i, k_j> plus the
 * mask bias (mask_kind 0: none; 1: boolean bytes, nonzero = visible; 2:
 * additive binary32) broadcast from dims mask_dims[4] = [mb, mh, mq, mw] (each
 * 1 or the full size; keys j >= mw masked when 1 < mw < SK); causal: j <= i
 * only. Rows whose every key is masked give zeros.
 */
int oracle_dense_attention(int B, int HQ, int HK, int SQ, int SK, int D, int dtype,
                           const void* q, const void* k, const void* v, int mask_kind,
                           const void* mask, const int32_t* mask_dims, int causal,
                           float scale, double* out);

/*
 * Dense GQA attention backward (the same page, execute()'s gradients): given
 * dout = dY [B, HQ, SQ, D] of the forward above (same inputs, mask and causal
 * flag), dq [B, HQ, SQ, D], dk and dv [B, HK, SK, D] (double) receive the
 * gradients: dS = P * (dY V^T - rowsum(Y * dY)), dQ = scale dS K, dK = scale
 * dS^T Q and dV = P^T dY, dK and dV summed over the G query heads of a KV head.
 */
int oracle_dense_attention_backward(int B, int HQ, int HK, int SQ, int SK, int D, int dtype,
                                    const void* q, const void* k, const void* v,
                                    const void* dout, int mask_kind, const void* mask,
                                    const int32_t* mask_dims, int causal, float scale,
                                    double* dq, double* dk, double* dv);

/* Exact widening of one stored element (exported so tests can pin it). */
double oracle_widen(const void* base, int64_t index, int dtype);

/* Number of OpenMP threads the oracle uses (1 when built without OpenMP). */
int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
