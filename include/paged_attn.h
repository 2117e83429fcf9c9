/*
 * paged_attn.h: C ABI of the MI355X (gfx950) paged-KV grouped-query decode
 * attention library, libpaged_attn.so.
 *
 * The operation is the one the docs.rs source page "onnxruntime-ep-mlx 0.31.1:
 * src/ops/paged_attention.rs" implements for Apple GPUs (kernel text
 * VECTOR_BODY, VECTOR_REDUCE, VECTOR_PARTIALS, PARTIALS_REDUCE; host launcher
 * vector()). For every sequence b, query head h and new row r:
 *
 *   kh       = h / (H / KV)                         (GQA: a group of H/KV query
 *                                                    heads shares KV head kh)
 *   visible  = cached positions i < L_b, read through the block table, then
 *              new rows j of this step: j <= r when causal, all NQ otherwise
 *   s_i      = scale * <q[b,h,r,:], k_i>
 *   out      = sum_i softmax(s)_i * v_i             (0 if nothing is visible)
 *
 * computed with an fp32 online softmax (running max and sum), optionally split
 * into key partitions whose partial states are merged by a second kernel.
 *
 * Conventions shared by every entry point
 *   - All pointers to tensors are DEVICE pointers owned by the caller; the
 *     library never allocates, frees, copies to the host or synchronises in
 *     paged_attn_decode / paged_attn_decode_append / paged_attn_combine.
 *     Tensors are contiguous row-major.
 *   - Element type of q, pools, new_k, new_v and out: pa_problem.dtype.
 *   - Layouts:
 *       q, out        [batch, num_heads, nq, head_dim]
 *       k_pool/v_pool [num_blocks, block_size, num_kv_heads, head_dim]
 *       block_table   int32 [batch, max_blocks_per_seq]; entry [b, n] is the
 *                     physical block holding cached positions n*block_size ..
 *       context_lens  int32 [batch]: cached (past) length of each sequence,
 *                     the nq new rows NOT included
 *       new_k/new_v   [batch, num_kv_heads, nq, head_dim]: this step's rows,
 *                     attended directly (they are not read from the pool)
 *   - Alignment: tensor pointers 16-byte aligned, block_table/context_lens
 *     4-byte aligned, workspace 16-byte aligned.
 *   - Device-side contract (not checked on the hot path):
 *       0 <= context_lens[b] <= max_context_len <= max_blocks_per_seq*block_size
 *       0 <= block_table[b, n] < num_blocks for n < ceil(context_lens[b]/block_size)
 *     Table entries past a sequence's last page and the unused slots of its
 *     last page are never read. Pools are read-only, so one physical block may
 *     appear in several sequences' tables.
 *   - Errors: every call returns a pa_status; on failure a thread-local
 *     message (paged_attn_last_error) says what was wrong and what to verify.
 *     Argument checks run on the host before any HIP call.
 *   - Supported shapes: head_dim 64 or 128; block_size 16 or 32; nq >= 1;
 *     (num_heads/num_kv_heads)*nq <= 128; dtype PA_F32, PA_F16 or PA_BF16.
 *     Device: gfx950 (MI355X) only.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. NULL selects the null stream of the current device. */
typedef struct ihipStream_t* pa_stream_t;

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, inconsistent sizes */
    PA_ERR_UNSUPPORTED = 2, /* well-formed but outside the supported shapes */
    PA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    PA_ERR_DEVICE = 4,      /* no usable device, or the device is not gfx950 */
    PA_ERR_LAUNCH = 5       /* the HIP runtime reported a launch failure */
} pa_status;

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

/* Kernel family for pass 1 (pa_problem.kernel and pa_plan_ex output). */
typedef enum {
    PA_KERNEL_AUTO = 0, /* chosen by the launch heuristic */
    PA_KERNEL_VALU = 1, /* vector-ALU scores and PV, DPP reductions */
    PA_KERNEL_MFMA = 2  /* matrix-core scores and PV (16-bit dtypes only) */
} pa_kernel;

/*
 * Problem description. The fields mirror the compile-time constants of the
 * page's vector() launcher (H, KV, D, BLOCK, MAX_BLOCKS, NQ, CAUSAL and the
 * `length` the partition count is chosen from), plus a batch dimension.
 */
typedef struct {
    int32_t batch;              /* B >= 0 (0: nothing to do) */
    int32_t num_heads;          /* H >= 1 */
    int32_t num_kv_heads;       /* KV >= 1, H % KV == 0 */
    int32_t head_dim;           /* D: 64 or 128 */
    int32_t block_size;         /* BS: tokens per page, 16 or 32 */
    int32_t num_blocks;         /* pool capacity (dim 0 of k_pool/v_pool), >= 1 */
    int32_t max_blocks_per_seq; /* block_table row stride, >= 0 */
    int32_t nq;                 /* new rows per sequence, >= 1 */
    int32_t causal;             /* 1: new row r sees new rows 0..r; 0: all nq */
    int32_t dtype;              /* pa_dtype */
    int32_t max_context_len;    /* host-side upper bound of context_lens, >= 0 */
    int32_t num_partitions;     /* 0: heuristic; 1: single pass; > 1: at most this many
                                   key partitions per sequence (tests, tuning) */
    int32_t kernel;             /* pa_kernel; PA_KERNEL_AUTO unless forcing a family.
                                   PA_KERNEL_MFMA needs fp16/bf16 and (H/KV)*nq <= 64 */
    int32_t flags;              /* bitwise OR of pa_flag values, 0 by default */
} pa_problem;

typedef enum {
    /* paged_attn_decode enqueues pass 1 only; the caller enqueues paged_attn_combine
       (same problem, context_lens and workspace) on the same stream afterwards, e.g.
       to time the two kernels separately. Without this flag decode does both. */
    PA_FLAG_DEFER_COMBINE = 1
} pa_flag;

/*
 * Launch plan, a pure host function of the problem and the number of compute
 * units of the device (the page's partitions() plays this role: it picks the
 * partition count from the context length and the number of query rows).
 * Outputs: kernel = pa_kernel family used for pass 1; for PA_KERNEL_MFMA,
 * partitions = groups the batch's sequence axis is cut into (all sequences
 * laid end to end in 16-key positions; each group is attended by one stream
 * per KV head, so partitions = resident streams / num_kv_heads; 1 = no merge)
 * and chunk_tokens = 16 * the minimum group length in positions; for
 * PA_KERNEL_VALU, partitions = key partitions per sequence (1 = single pass)
 * and chunk_tokens = cached tokens per partition (a multiple of block_size).
 * num_partitions > 0 in the problem fixes `partitions`.
 * Any output pointer may be NULL. No HIP call is made.
 */
int pa_plan_ex(const pa_problem* problem, int32_t num_cus, int32_t* partitions,
               int32_t* chunk_tokens, int32_t* kernel);

/* pa_plan_ex for the current HIP device (its compute-unit count is queried once
 * per device and cached). Fails with PA_ERR_DEVICE if the device is not gfx950. */
int pa_plan(const pa_problem* problem, int32_t* partitions, int32_t* chunk_tokens,
            int32_t* kernel);

/*
 * Workspace bytes paged_attn_decode needs on the current device: 0 for a plan
 * that needs no merge. No initial contents are required. The workspace holds
 * online-softmax states (the page's VECTOR_PARTIALS state, in base-2 units):
 * o = sum_i 2^(t_i - m) v_i (unnormalised), m = max_i t_i and
 * l = sum_i 2^(t_i - m), with t_i = s_i * log2(e) over some keys of a row;
 * m and l are fp32, o is fp32 except as noted below.
 *   PA_KERNEL_MFMA (balanced split): the sequences laid end to end in
 *   positions of 16 keys (ceil(L_b/16) cached, then ceil(nq/16) new) are cut
 *   into `partitions` groups of equal length (+-1); the piece of sequence b in
 *   group g, for KV head kh, is slot (b + g)*num_kv_heads + kh. Layout:
 *   o[slots][R][head_dim] (for PA_F16 stored as o / l in fp16), ml[slots][R][2],
 *   then int32 [B][2] = first and last group of each sequence (written by pass
 *   1); slots = (B + partitions) * num_kv_heads, R = (H/KV)*nq (rows of one KV
 *   head, r_local = (h % G)*nq + r).
 *   PA_KERNEL_VALU (chunks of chunk_tokens cached keys per sequence):
 *   o[rows][P][head_dim], ml[rows][P][2] with rows = B*H*nq, row = (b*H + h)*nq + r.
 * States that are not needed (a unit or sequence done in one piece) are not
 * written; those outputs are final after pass 1. pa_workspace_size_ex is the
 * same for a device with num_cus compute units (pure host).
 */
int pa_workspace_size(const pa_problem* problem, size_t* bytes);
int pa_workspace_size_ex(const pa_problem* problem, int32_t num_cus, size_t* bytes);

/*
 * One decode-attention step (page: vector(), which issues pass 1 and, when
 * partitioned, the merge). Enqueues pass 1 on `stream` and, when the plan has
 * more than one partition, paged_attn_combine's kernel after it. Asynchronous:
 * returns once the work is enqueued. `scale` multiplies q.k (binary32, as the
 * page passes the scale's fp32 bits). `workspace` may be NULL when
 * pa_workspace_size reports 0; otherwise it must hold that many bytes. Calls
 * sharing a workspace must not run concurrently. q/new_k/new_v/pools/tables
 * are only read; `out` and the workspace are written.
 */
int paged_attn_decode(const pa_problem* problem, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_table,
                      const int32_t* context_lens, const void* new_k, const void* new_v,
                      float scale, void* out, void* workspace, size_t workspace_bytes,
                      pa_stream_t stream);

/*
 * The slot-patched step: one decode-attention step that also stores this
 * step's new rows into the pools (page: VECTOR_BODY's `position` slots, where
 * a cached position whose token slot is named by a new row reads that row;
 * the docs.rs page "onnxruntime-ep-mlx 0.31.1: src/engine.rs",
 * write_back_input_patches, copies such rows back into their cache slots, one
 * complete token row per slot).
 *   slot_mapping  int32 [batch, nq], device: token slot s = block * block_size
 *                 + offset of new row j of sequence b; negative, or >=
 *                 num_blocks * block_size: the row is neither stored nor read
 *                 back.
 * Effects, as if the rows were stored first and then the step ran:
 *   - k_pool/v_pool[s / block_size, s % block_size, kh, :] = new_k/new_v[b, kh,
 *     j, :] for every KV head; when several rows of one sequence name the same
 *     slot, the highest j is the one stored;
 *   - a cached position i < context_lens[b] of sequence b whose slot (through
 *     the block table) some new row of sequence b names reads that row (the
 *     highest such j) instead of the pool; the new rows themselves are attended
 *     exactly as in paged_attn_decode.
 * The pools are written (the other arguments as in paged_attn_decode). Caller
 * contract (not checked on the device): a slot named by one sequence is neither
 * named by nor a cached position of another sequence in the same call. Errors:
 * those of paged_attn_decode, and PA_ERR_INVALID_ARG for a NULL or misaligned
 * slot_mapping.
 */
int paged_attn_decode_append(const pa_problem* problem, const void* q, void* k_pool,
                             void* v_pool, const int32_t* block_table,
                             const int32_t* context_lens, const void* new_k, const void* new_v,
                             const int32_t* slot_mapping, float scale, void* out,
                             void* workspace, size_t workspace_bytes, pa_stream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * paged_attn_decode with the split's partial states kept in a workspace the
 * library owns, a static device array of PA_STATIC_WORKSPACE_BYTES that each
 * device holds from the library's load until the process ends. Nothing is
 * allocated or freed. Arguments, effects and errors as paged_attn_decode
 * (both kernels always run: PA_FLAG_DEFER_COMBINE is rejected with
 * PA_ERR_INVALID_ARG), plus PA_ERR_WORKSPACE when the plan needs more than
 * PA_STATIC_WORKSPACE_BYTES (pa_workspace_size reports what it needs; a
 * smaller num_partitions or batch lowers it). No initial contents are needed.
 * Every call on one device shares that device's array: calls that can overlap
 * on one device (different streams, or different host threads without
 * ordering) race on it and must not be issued.
 */
#define PA_STATIC_WORKSPACE_BYTES ((size_t)32 << 20)

int paged_attn_decode_static(const pa_problem* problem, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table,
                             const int32_t* context_lens, const void* new_k, const void* new_v,
                             float scale, void* out, pa_stream_t stream);

/*
 * Merge step alone (page: PARTIALS_REDUCE), as its own kernel. Reads the
 * partial states a partitioned paged_attn_decode left in `workspace` for the
 * same problem and
 * context_lens, and writes out = (sum_p 2^(m_p - M) o_p) / (sum_p 2^(m_p - M) l_p)
 * with M = max_p m_p over each row's partitions (0 when that sum is 0), rounded
 * to nearest-even in the I/O dtype. Rows of sequences that fit in one partition
 * were already written by pass 1 and are left untouched. For a single-pass plan
 * it does nothing and returns PA_OK.
 */
int paged_attn_combine(const pa_problem* problem, const int32_t* context_lens,
                       const void* workspace, size_t workspace_bytes, void* out,
                       pa_stream_t stream);

/*
 * Dense (prefill) GQA attention forward: the forward half of the docs.rs page
 * "onnxruntime-ep-mlx 0.31.1: src/ops/attention_vjp/dense.rs", execute()
 * (score matrix, mask bias, causal mask, softmax with fully masked rows set to
 * zero), times V. For sequence b, query head h (KV head kh = h / (HQ/HK)) and
 * query position i:
 *   s_j = scale * <q[b,h,i,:], k[b,kh,j,:]> + bias(b,h,i,j),  j < kv_len
 *   bias = 0 / -inf from a boolean mask (nonzero = visible) or the value of an
 *          additive binary32 mask, broadcast from mask_dims = [mb, mh, mq, mw]
 *          (a dim of 1 repeats; when 1 < mw < kv_len, keys j >= mw get -inf,
 *          as the page pads the mask's last axis); 0 without a mask
 *   causal: s_j = -inf for j > i (top-left alignment: query i sees keys 0..i)
 *   out[b,h,i,:] = softmax(s) . v[b,kh,:,:], or 0 where every s_j is -inf
 * Layouts: q, out [batch, num_heads, q_len, head_dim]; k, v [batch,
 * num_kv_heads, kv_len, head_dim]; mask [mb, mh, mq, mw] uint8 (PA_MASK_BOOL)
 * or float32 (PA_MASK_ADD), row-major. Device pointers owned by the caller;
 * out is written, nothing else. Asynchronous on `stream`. Supported: fp16/bf16,
 * head_dim 64/128, num_heads/num_kv_heads <= 64. Errors: PA_ERR_INVALID_ARG for
 * NULL/misaligned pointers or inconsistent sizes/mask dims, PA_ERR_UNSUPPORTED
 * outside the supported shapes (fp32 included), PA_ERR_DEVICE, PA_ERR_LAUNCH.
 */
typedef enum { PA_MASK_NONE = 0, PA_MASK_BOOL = 1, PA_MASK_ADD = 2 } pa_mask_kind;

typedef struct {
    int32_t batch;        /* >= 0 */
    int32_t num_heads;    /* HQ >= 1 */
    int32_t num_kv_heads; /* HK >= 1, HQ % HK == 0 */
    int32_t head_dim;     /* 64 or 128 */
    int32_t q_len;        /* SQ >= 0 */
    int32_t kv_len;       /* SK >= 0 */
    int32_t causal;       /* 1: key j visible to query i only if j <= i */
    int32_t dtype;        /* PA_F16 or PA_BF16 */
    int32_t mask_kind;    /* pa_mask_kind */
    int32_t mask_dims[4]; /* [mb, mh, mq, mw] when mask_kind != PA_MASK_NONE */
} pa_dense_problem;

int pa_dense_attention(const pa_dense_problem* problem, const void* q, const void* k,
                       const void* v, const void* mask, float scale, void* out,
                       pa_stream_t stream);

/*
 * Dense GQA attention backward: the gradient half of execute() on the same
 * page ("onnxruntime-ep-mlx 0.31.1: src/ops/attention_vjp/dense.rs"). For the
 * forward of pa_dense_attention on the same problem, inputs and mask, and the
 * output gradient dout = dY [batch, num_heads, q_len, head_dim], it recomputes
 * P (the softmax rows, 0 for rows with no visible key) and Y = P V, and writes
 *   dS = P * (dY V^T - rowsum(Y * dY))      (per query row)
 *   dq = scale * dS K                       [batch, num_heads, q_len, head_dim]
 *   dk = scale * sum over the group dS^T Q  [batch, num_kv_heads, kv_len, head_dim]
 *   dv = sum over the group P^T dY          [batch, num_kv_heads, kv_len, head_dim]
 * where the group of KV head kh is the query heads kh*G .. kh*G + G - 1
 * (G = num_heads / num_kv_heads). Products accumulate in fp32 and are rounded
 * once to the I/O dtype. `workspace` (device, 256-byte aligned, at least
 * pa_dense_backward_workspace_size bytes, no initial contents required) holds
 * two fp32 values per query row between the launches and, for causal problems
 * with num_heads / num_kv_heads >= 2, two fp32 halves of dk and of dv (each
 * workgroup takes half the query heads of two key blocks of complementary
 * weight; the halves are added in a fixed order); dq, dk
 * and dv are written whole; nothing else is written. Device pointers are owned by the
 * caller; asynchronous on `stream`. Supported shapes and errors as for
 * pa_dense_attention, plus PA_ERR_WORKSPACE for a missing, small or
 * misaligned workspace.
 */
int pa_dense_backward_workspace_size(const pa_dense_problem* problem, size_t* bytes);

int pa_dense_attention_backward(const pa_dense_problem* problem, const void* q, const void* k,
                                const void* v, const void* mask, const void* dout, float scale,
                                void* dq, void* dk, void* dv, void* workspace,
                                size_t workspace_bytes, pa_stream_t stream);

/* Message of the last failing call on this thread ("" if none). Valid until the
 * next call on this thread. Each message names what was wrong and ends with
 * what to verify, the form of the errors that the dispatch() function and the
 * device checks of docs.rs page "onnxruntime-ep-mlx 0.31.1:
 * src/ops/paged_attention.rs" return; here they are a pa_status code plus this
 * thread-local text (no allocation is returned to the caller). */
const char* paged_attn_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int paged_attn_version(void);  /* 105: paged_attn_decode_static */

#ifdef __cplusplus
}
#endif
#endif /* PAGED_ATTN_H */
