// Host side of libpaged_attn.so: argument validation, launch plan, kernel
// selection and the extern "C" entry points declared in paged_attn.h.
//
// The plan plays the role of partitions() and the launch shapes of vector() on
// the docs.rs page "onnxruntime-ep-mlx 0.31.1: src/ops/paged_attention.rs"; its
// constants are chosen for MI355X (256 compute units in 8 XCDs) rather than for
// Apple GPUs.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>

#include "paged_attn.h"
#include "combine.hpp"
#include "decode_mfma.hpp"
#include "decode_valu.hpp"
#include "dense_bwd.hpp"

// Workspace of paged_attn_decode_static, for callers that cannot allocate:
// every device the library runs on holds its own copy of this array until the
// process ends. In host code the name denotes a host-side stand-in, not device
// memory: the device address comes from hipGetSymbolAddress (scratch_address),
// and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[PA_STATIC_WORKSPACE_BYTES];

namespace {

thread_local std::string t_error;

int fail(int code, const char* fmt, ...) {
    char buf[640];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    t_error = buf;
    return code;
}

int succeed() {
    t_error.clear();
    return PA_OK;
}

constexpr int kMaxRows = 128;         // G * nq
constexpr int kMfmaMaxRows = 64;      // the matrix-core family keeps <= 4 row tiles of 16
constexpr int kLdsPerCu = 160 * 1024;
// A piece's saved state may be at most 1/kStateRatio of the K/V bytes it covers.
constexpr int kStateRatio = 8;
constexpr int kGroupsPerCu = 8;       // workgroups per CU the heuristic aims to keep busy
constexpr int kMinChunkTokens = 256;  // below this, partial-state traffic outweighs balance
constexpr int kMaxChunkTokens = 2048; // above this, ragged batches leave CUs idle

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

int validate_problem(const pa_problem* p) {
    if (!p) return fail(PA_ERR_INVALID_ARG, "problem is NULL; verify the pa_problem pointer");
    if (p->batch < 0)
        return fail(PA_ERR_INVALID_ARG, "batch = %d is negative; verify pa_problem.batch", p->batch);
    if (p->batch > 65535)
        return fail(PA_ERR_UNSUPPORTED, "batch = %d exceeds 65535 sequences per call; verify "
                    "pa_problem.batch or split the batch", p->batch);
    if (p->num_heads < 1 || p->num_kv_heads < 1)
        return fail(PA_ERR_INVALID_ARG, "num_heads = %d, num_kv_heads = %d must be >= 1; verify "
                    "the head counts", p->num_heads, p->num_kv_heads);
    if (p->num_heads % p->num_kv_heads != 0)
        return fail(PA_ERR_INVALID_ARG, "num_heads = %d is not a multiple of num_kv_heads = %d; "
                    "verify the GQA grouping", p->num_heads, p->num_kv_heads);
    if (p->head_dim != 64 && p->head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "head_dim = %d is not supported (64 or 128); verify "
                    "pa_problem.head_dim", p->head_dim);
    if (p->block_size != 16 && p->block_size != 32)
        return fail(PA_ERR_UNSUPPORTED, "block_size = %d is not supported (16 or 32); verify "
                    "the page size of the KV pools", p->block_size);
    if (p->nq < 1)
        return fail(PA_ERR_INVALID_ARG, "nq = %d must be >= 1; verify the number of new rows",
                    p->nq);
    if (p->causal != 0 && p->causal != 1)
        return fail(PA_ERR_INVALID_ARG, "causal = %d must be 0 or 1", p->causal);
    if (p->dtype != PA_F32 && p->dtype != PA_F16 && p->dtype != PA_BF16)
        return fail(PA_ERR_INVALID_ARG, "dtype = %d is not a pa_dtype; verify pa_problem.dtype",
                    p->dtype);
    const int64_t rows = (int64_t)(p->num_heads / p->num_kv_heads) * p->nq;
    if (rows > kMaxRows)
        return fail(PA_ERR_UNSUPPORTED, "(num_heads/num_kv_heads)*nq = %lld exceeds %d query rows "
                    "per KV head; verify nq and the GQA group size", (long long)rows, kMaxRows);
    if (p->num_blocks < 1)
        return fail(PA_ERR_INVALID_ARG, "num_blocks = %d must be >= 1; verify the pool shape",
                    p->num_blocks);
    if (p->max_blocks_per_seq < 0)
        return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq = %d is negative",
                    p->max_blocks_per_seq);
    if (p->max_context_len < 0)
        return fail(PA_ERR_INVALID_ARG, "max_context_len = %d is negative", p->max_context_len);
    if ((int64_t)p->max_context_len > (int64_t)p->max_blocks_per_seq * p->block_size)
        return fail(PA_ERR_INVALID_ARG, "max_context_len = %d exceeds the block-table capacity "
                    "max_blocks_per_seq*block_size = %lld; verify the table shape",
                    p->max_context_len, (long long)p->max_blocks_per_seq * p->block_size);
    if (p->num_partitions < 0)
        return fail(PA_ERR_INVALID_ARG, "num_partitions = %d is negative", p->num_partitions);
    if (p->flags & ~PA_FLAG_DEFER_COMBINE)
        return fail(PA_ERR_INVALID_ARG, "flags = 0x%x has unknown bits", p->flags);
    if (p->kernel != PA_KERNEL_AUTO && p->kernel != PA_KERNEL_VALU && p->kernel != PA_KERNEL_MFMA)
        return fail(PA_ERR_INVALID_ARG, "kernel = %d is not a pa_kernel", p->kernel);
    if (p->kernel == PA_KERNEL_MFMA && p->dtype == PA_F32)
        return fail(PA_ERR_UNSUPPORTED, "the matrix-core kernel family needs fp16 or bf16 I/O; "
                    "verify pa_problem.kernel");
    if (p->kernel == PA_KERNEL_MFMA && p->batch > pa::kMaxSplitBatch)
        return fail(PA_ERR_UNSUPPORTED, "the matrix-core kernel family takes at most %d sequences "
                    "per call (got %d); verify pa_problem.kernel or split the batch",
                    pa::kMaxSplitBatch, p->batch);
    {
        // 16-key groups of the whole batch at the table's capacity, counted in int32
        const int64_t cap = (int64_t)p->max_blocks_per_seq * p->block_size;
        const int64_t subpages = (int64_t)p->batch * ((cap + 15) / 16 + (p->nq + 15) / 16);
        if (subpages >= (1LL << 31))
            return fail(PA_ERR_UNSUPPORTED, "batch * context is too large for one call (%lld "
                        "16-key groups); split the batch", (long long)subpages);
    }
    if (p->kernel == PA_KERNEL_MFMA && rows > kMfmaMaxRows)
        return fail(PA_ERR_UNSUPPORTED, "the matrix-core kernel family takes at most %d query "
                    "rows per KV head (got %lld); verify pa_problem.kernel", kMfmaMaxRows,
                    (long long)rows);
    return PA_OK;
}

constexpr int kCoopSeqPad = 3;  // a sequence's fixed cost in the cooperative kernel, positions

struct Plan {
    // VALU family: parts = key partitions per sequence, chunk = cached tokens per
    // partition (multiple of block_size). Matrix-core family (balanced split):
    // parts = groups the sequence axis is cut into (KV waves each), chunk =
    // 16 * min_seg.
    int parts;
    int chunk;
    int min_seg;  // matrix-core family: minimum group length in 16-key positions
    int seq_pad;  // matrix-core family: a sequence's fixed cost, in 16-key positions
    int kernel;   // pa_kernel
    int rt;       // VALU: query rows per workgroup (power of two <= 8); MFMA: 16-row tiles (1, 2, 4)
    int n_tiles;  // workgroups per KV head along the rows (1 for MFMA)
};

// Matrix-core family launch shapes, by 16-row tiles per KV head (Plan::rt):
//   rt = 1: decode_mfma, one wave per (group, head) with one row tile;
//   rt = 2: decode_mfma with two row tiles per wave;
//   rt = 4: decode_mfma_coop, two waves of two row tiles per (group, head)
//           sharing a ring of three slots (four workgroups per CU, set by
//           registers; three slots ran 1-3 % faster than four and five on
//           batches of 16, 128 and 256 sequences);
// batches of at most 64 sequences keep the sequence table in registers in every
// shape (each wave loads and scans the lengths itself: no barrier before the
// first fetch); all at 2 waves per SIMD (slots double for D = 64, whose slots
// are half as large). Measured
// on the Llama-3-8B-shaped and ragged-serving workloads: 2 waves per SIMD with
// 2 slots each beat 4 waves with 1 slot (oldest waves hog the memory path,
// the last quarter of the kernel runs thin) and 1 wave with 4 slots; for 64
// rows, 2 waves x 2 tiles beat 4 waves x 1 tile and 1 wave x 4 tiles, and
// four workgroups per CU beat fewer with deeper rings (two of nine slots,
// three of six).
struct MfmaShape {
    int nw;      // waves per (group, head): 1, or the cooperative workgroup
    int nrt;     // row tiles per wave
    int slots;   // LDS slots per wave (nw = 1) or ring slots per workgroup
    int wps;     // waves per SIMD the kernel is built for
    bool regseq; // sequence table in registers (no prefix in LDS)
};
bool regseq_batch(const pa_problem* p) { return p->batch <= pa::kRegTableMaxBatch; }
MfmaShape mfma_shape(const pa_problem* p, int rt) {
    const int s1 = p->head_dim == 128 ? 1 : 2;  // a D = 64 slot is half as large
    if (rt == 1) return {1, 1, 2 * s1, 2, regseq_batch(p)};
    if (rt == 2) return {1, 2, 2 * s1, 2, regseq_batch(p)};
    return {2, 2, 3 * s1, 2, regseq_batch(p)};
}
int mfma_slot_bytes(int head_dim) {
    return head_dim == 64 ? pa::SlotLayout<_Float16, 64>::kBytes
                          : pa::SlotLayout<_Float16, 128>::kBytes;
}

// Dynamic LDS of one matrix-core workgroup: its slots (4 single waves' slots,
// or the cooperative ring), then the per-sequence prefix and lengths.
size_t mfma_lds_bytes(const pa_problem* p, int rt) {
    const MfmaShape sh = mfma_shape(p, rt);
    const size_t slots = sh.nw == 1 ? 4 * (size_t)sh.slots : (size_t)sh.slots;
    const size_t table = sh.regseq ? 0 : (2 * (size_t)p->batch + 1) * sizeof(int);
    return slots * mfma_slot_bytes(p->head_dim) + table;
}

// Streams (waves for nw = 1, workgroups otherwise) one CU holds at once: the
// kernel's occupancy, lowered by LDS.
int mfma_streams_per_cu(const pa_problem* p, int rt) {
    const MfmaShape sh = mfma_shape(p, rt);
    const int wg_waves = sh.nw == 1 ? 4 : sh.nw;
    int groups = (int)(kLdsPerCu / mfma_lds_bytes(p, rt));  // workgroups by LDS
    const int by_regs = 4 * sh.wps / wg_waves;
    if (groups > by_regs) groups = by_regs;
    if (groups < 1) groups = 1;
    return sh.nw == 1 ? 4 * groups : groups;
}

int plan_impl(const pa_problem* p, int num_cus, Plan* pl) {
    if (int rc = validate_problem(p)) return rc;
    if (num_cus < 1) return fail(PA_ERR_INVALID_ARG, "num_cus = %d must be >= 1", num_cus);
    const int R = (p->num_heads / p->num_kv_heads) * p->nq;
    int kernel = p->kernel;
    if (kernel == PA_KERNEL_AUTO)
        kernel = (p->dtype != PA_F32 && R <= kMfmaMaxRows && p->batch <= pa::kMaxSplitBatch)
                     ? PA_KERNEL_MFMA
                     : PA_KERNEL_VALU;
    pl->kernel = kernel;
    pl->min_seg = 1;
    pl->seq_pad = 0;
    if (kernel == PA_KERNEL_MFMA) {
        pl->rt = R <= 16 ? 1 : (R <= 32 ? 2 : 4);
        pl->n_tiles = 1;
        const int64_t elem = p->dtype == PA_F32 ? 4 : 2;
        const int64_t state = (int64_t)R * (p->head_dim + 2) * 4;
        const int64_t kv_per_group = 16 * 2 * (int64_t)p->head_dim * elem;
        if (p->num_partitions > (1 << 22))
            return fail(PA_ERR_UNSUPPORTED, "num_partitions = %d is more groups than supported "
                        "(%d)", p->num_partitions, 1 << 22);
        if (p->num_partitions > 0) {
            pl->parts = p->num_partitions;
            pl->min_seg = 1;
        } else {
            const int64_t streams = (int64_t)num_cus * mfma_streams_per_cu(p, pl->rt);
            const int64_t groups = streams / p->num_kv_heads;
            pl->parts = (int)(groups < 1 ? 1 : (groups > (1 << 22) ? (1 << 22) : groups));
            pl->min_seg = (int)ceil_div(kStateRatio * state, kv_per_group);
            // the cooperative kernel's fixed work per sequence (a drain of its
            // ring for the next Q, a 64-row piece state, the new rows) costs
            // about 3 sub-pages: charged to the sequence, the groups that hold a
            // sequence start finish with the others (multi-row causal pass 1
            // 68 -> 66 us); the one-wave kernels measured best without
            pl->seq_pad = pl->rt == 4 ? kCoopSeqPad : 0;
        }
        pl->chunk = 16 * pl->min_seg;
        return PA_OK;
    } else {
        int rt = 1;
        while (rt < R && rt < 8) rt *= 2;
        pl->rt = rt;
        pl->n_tiles = (R + rt - 1) / rt;
    }
    const int BS = p->block_size;
    const int64_t ctx = p->max_context_len;
    const int64_t full = round_up(ctx > 0 ? ctx : 1, BS);  // one chunk covering everything
    int64_t chunk;
    if (p->num_partitions == 1) {
        chunk = full;
    } else if (p->num_partitions > 1) {
        chunk = round_up(ceil_div(ctx > 0 ? ctx : 1, p->num_partitions), BS);
    } else {
        const int64_t units = (int64_t)p->batch * p->num_kv_heads * pl->n_tiles;
        const int64_t target = (int64_t)num_cus * kGroupsPerCu;
        const int64_t want = units > 0 ? ceil_div(target, units) : 1;
        chunk = round_up(ceil_div(ctx > 0 ? ctx : 1, want > 1 ? want : 1), BS);
        if (chunk < kMinChunkTokens) chunk = round_up(kMinChunkTokens, BS);
        if (chunk > kMaxChunkTokens) chunk = kMaxChunkTokens;
    }
    if (chunk > full) chunk = full;
    int64_t parts = ctx > 0 ? ceil_div(ctx, chunk) : 1;
    if (parts > 65535 * 32767LL)
        return fail(PA_ERR_UNSUPPORTED, "too many partitions (%lld)", (long long)parts);
    pl->chunk = (int)chunk;
    pl->parts = (int)parts;
    return PA_OK;
}

// Workspace: VALU family [rows][parts][D] + [rows][parts][2]; matrix-core
// family [slots][R][D] + [slots][R][2] with slots = (B + groups)*KV.
size_t state_floats(const pa_problem* p, const Plan& pl) {
    if (pl.kernel == PA_KERNEL_MFMA) {
        const size_t R = (size_t)(p->num_heads / p->num_kv_heads) * p->nq;
        const size_t slots = ((size_t)p->batch + (size_t)pl.parts) * p->num_kv_heads;
        return slots * R;
    }
    return (size_t)p->batch * p->num_heads * p->nq * (size_t)pl.parts;
}

// Bytes of one partial-output element: fp16 I/O on the matrix-core family keeps
// them as fp16 (Partial<T>), everything else as fp32.
size_t partial_bytes(const pa_problem* p, const Plan& pl) {
    return pl.kernel == PA_KERNEL_MFMA && p->dtype == PA_F16 ? 2 : 4;
}
// Byte offset of the (max, sum) pairs: after the partial outputs.
size_t ml_offset(const pa_problem* p, const Plan& pl) {
    return state_floats(p, pl) * (size_t)p->head_dim * partial_bytes(p, pl);
}
// Matrix-core family: after the states, two int32 per sequence: the first and
// last group that overlap it (written by pass 1).
size_t meta_offset(const pa_problem* p, const Plan& pl) {
    return ml_offset(p, pl) + state_floats(p, pl) * 2 * sizeof(float);
}

size_t workspace_bytes_for(const pa_problem* p, const Plan& pl) {
    if (pl.parts <= 1) return 0;
    size_t bytes = meta_offset(p, pl);
    if (pl.kernel == PA_KERNEL_MFMA) bytes += (size_t)p->batch * 2 * sizeof(int32_t);
    return bytes;
}

// Per-device property cache (compute units, gfx950 or not), filled once, and
// the device address of that device's static workspace (set on first use).
struct DeviceInfo {
    bool known = false;
    bool gfx950 = false;
    int cus = 0;
    char arch[64] = {0};
    void* scratch = nullptr;
};
std::mutex g_device_mutex;
DeviceInfo g_devices[64];

int current_device_cus(int* cus) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return fail(PA_ERR_DEVICE, "no HIP device is available; verify that a gfx950 GPU is "
                    "visible to this process");
    if (dev >= 64) return fail(PA_ERR_DEVICE, "device ordinal %d is out of range", dev);
    std::lock_guard<std::mutex> lock(g_device_mutex);
    DeviceInfo& info = g_devices[dev];
    if (!info.known) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(PA_ERR_DEVICE, "cannot read properties of device %d; verify the HIP "
                        "runtime", dev);
        info.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        info.cus = prop.multiProcessorCount;
        std::snprintf(info.arch, sizeof info.arch, "%s", prop.gcnArchName);
        info.known = true;
    }
    if (!info.gfx950)
        return fail(PA_ERR_DEVICE, "device %d is %s, not gfx950 (MI355X); verify the selected "
                    "device", dev, info.arch);
    *cus = info.cus;
    return PA_OK;
}

// Device address of the current device's copy of `scratch`, looked up once per
// device with that device current (each device holds the array at its own
// address). Call after current_device_cus has accepted the device.
int scratch_address(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return fail(PA_ERR_DEVICE, "no usable HIP device for the static workspace");
    std::lock_guard<std::mutex> lock(g_device_mutex);
    DeviceInfo& info = g_devices[dev];
    if (!info.scratch) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(PA_ERR_DEVICE, "cannot locate the static workspace on device %d: %s; "
                        "verify the HIP runtime", dev, hipGetErrorString(e));
        info.scratch = p;
    }
    *ptr = info.scratch;
    return PA_OK;
}

bool misaligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) != 0; }

int validate_tensors(const pa_problem* p, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_table, const int32_t* context_lens, const void* new_k,
                     const void* new_v, const void* out) {
    if (!q || !k_pool || !v_pool || !context_lens || !new_k || !new_v || !out)
        return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL (q %p, k_pool %p, v_pool %p, "
                    "context_lens %p, new_k %p, new_v %p, out %p); verify the arguments", q,
                    k_pool, v_pool, (const void*)context_lens, new_k, new_v, out);
    if (!block_table && p->max_blocks_per_seq > 0)
        return fail(PA_ERR_INVALID_ARG, "block_table is NULL; verify the arguments");
    const void* t16[] = {q, k_pool, v_pool, new_k, new_v, out};
    const char* n16[] = {"q", "k_pool", "v_pool", "new_k", "new_v", "out"};
    for (int i = 0; i < 6; ++i)
        if (misaligned(t16[i], 16))
            return fail(PA_ERR_INVALID_ARG, "%s (%p) is not 16-byte aligned; verify the tensor "
                        "storage offset", n16[i], t16[i]);
    if (misaligned(block_table, 4) || misaligned(context_lens, 4))
        return fail(PA_ERR_INVALID_ARG, "block_table/context_lens must be 4-byte aligned");
    return PA_OK;
}

// ---------------------------------------------------------------------------
// Kernel dispatch over the compile-time shapes.
// ---------------------------------------------------------------------------
template <typename T, int D, int BS, bool APPEND>
void launch_valu_k(const Plan& pl, dim3 grid, hipStream_t s, const pa::DecodeArgs<T>& a) {
    switch (pl.rt) {
        case 1: hipLaunchKernelGGL((pa::decode_valu<T, D, BS, 1, APPEND>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((pa::decode_valu<T, D, BS, 2, APPEND>), grid, dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL((pa::decode_valu<T, D, BS, 4, APPEND>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((pa::decode_valu<T, D, BS, 8, APPEND>), grid, dim3(256), 0, s, a); break;
    }
}

template <typename T, int D, int BS>
void launch_valu(const Plan& pl, dim3 grid, hipStream_t s, const pa::DecodeArgs<T>& a) {
    if (a.ap.slots) launch_valu_k<T, D, BS, true>(pl, grid, s, a);
    else launch_valu_k<T, D, BS, false>(pl, grid, s, a);
}

template <typename T, int D, int BS, bool APPEND>
void launch_mfma_k(const pa_problem* p, const Plan& pl, size_t lds, hipStream_t s,
                   const pa::SplitArgs<T>& a, const int32_t* table) {
    constexpr int S1 = D == 128 ? 1 : 2;  // slot counts of mfma_shape
    const int64_t streams = (int64_t)pl.parts * p->num_kv_heads;
    const bool regseq = regseq_batch(p);
    if (pl.rt <= 2) {
        const dim3 grid((unsigned)ceil_div(streams, 4));
        if (pl.rt == 1 && regseq)
            hipLaunchKernelGGL((pa::decode_mfma<T, D, BS, 1, 2 * S1, 2, APPEND, true>), grid,
                               dim3(256), lds, s, a, table, a.ap.slots);
        else if (pl.rt == 1)
            hipLaunchKernelGGL((pa::decode_mfma<T, D, BS, 1, 2 * S1, 2, APPEND, false>), grid,
                               dim3(256), lds, s, a, table, a.ap.slots);
        else if (regseq)
            hipLaunchKernelGGL((pa::decode_mfma<T, D, BS, 2, 2 * S1, 2, APPEND, true>), grid,
                               dim3(256), lds, s, a, table, a.ap.slots);
        else
            hipLaunchKernelGGL((pa::decode_mfma<T, D, BS, 2, 2 * S1, 2, APPEND, false>), grid,
                               dim3(256), lds, s, a, table, a.ap.slots);
    } else if (regseq) {
        hipLaunchKernelGGL((pa::decode_mfma_coop<T, D, BS, 2, 2, 3 * S1, 2, APPEND, true>),
                           dim3((unsigned)streams), dim3(128), lds, s, a, table, a.ap.slots);
    } else {
        hipLaunchKernelGGL((pa::decode_mfma_coop<T, D, BS, 2, 2, 3 * S1, 2, APPEND, false>),
                           dim3((unsigned)streams), dim3(128), lds, s, a, table, a.ap.slots);
    }
}

// The plain step and the slot-patched step are separate instantiations, so the
// plain kernels carry none of the patching code.
template <typename T, int D, int BS>
void launch_mfma(const pa_problem* p, const Plan& pl, size_t lds, hipStream_t s,
                 const pa::SplitArgs<T>& a, const int32_t* table) {
    if (a.ap.slots) launch_mfma_k<T, D, BS, true>(p, pl, lds, s, a, table);
    else launch_mfma_k<T, D, BS, false>(p, pl, lds, s, a, table);
}

pa::SplitGeometry split_geometry(const pa_problem* p, const Plan& pl) {
    pa::SplitGeometry g;
    g.B = p->batch;
    g.KV = p->num_kv_heads;
    g.NQ = p->nq;
    g.max_tokens = p->max_blocks_per_seq * p->block_size;
    g.n_grp = pl.parts;
    g.min_seg = pl.min_seg;
    g.seq_pad = pl.seq_pad;
    return g;
}

template <typename T>
void launch_pass1_mfma(const pa_problem* p, const Plan& pl, hipStream_t s,
                       const pa::DecodeArgs<T>& d) {
    pa::SplitArgs<T> a;
    a.q = d.q;
    a.k_pool = d.k_pool;
    a.v_pool = d.v_pool;
    a.block_table = d.block_table;
    a.context_lens = d.context_lens;
    a.new_k = d.new_k;
    a.new_v = d.new_v;
    a.out = d.out;
    char* const ws = reinterpret_cast<char*>(d.ws_o);
    a.ws_o = reinterpret_cast<typename pa::Partial<T>::type*>(ws);
    a.ws_ml = ws ? reinterpret_cast<float*>(ws + ml_offset(p, pl)) : nullptr;
    a.meta = ws ? reinterpret_cast<int32_t*>(ws + meta_offset(p, pl)) : nullptr;
    a.g = split_geometry(p, pl);
    a.H = p->num_heads;
    a.causal = p->causal;
    a.max_blocks = p->max_blocks_per_seq;
    a.R = (p->num_heads / p->num_kv_heads) * p->nq;
    a.qscale = d.qscale;
    a.ap = d.ap;
    const size_t lds = mfma_lds_bytes(p, pl.rt);
    if (p->head_dim == 64) {
        if (p->block_size == 16) launch_mfma<T, 64, 16>(p, pl, lds, s, a, d.block_table);
        else launch_mfma<T, 64, 32>(p, pl, lds, s, a, d.block_table);
    } else {
        if (p->block_size == 16) launch_mfma<T, 128, 16>(p, pl, lds, s, a, d.block_table);
        else launch_mfma<T, 128, 32>(p, pl, lds, s, a, d.block_table);
    }
}

template <typename T>
void launch_pass1(const pa_problem* p, const Plan& pl, hipStream_t s, const pa::DecodeArgs<T>& a) {
    if constexpr (!std::is_same<T, float>::value) {
        if (pl.kernel == PA_KERNEL_MFMA) {
            launch_pass1_mfma<T>(p, pl, s, a);
            return;
        }
    }
    const dim3 grid(pl.parts, p->num_kv_heads * pl.n_tiles, p->batch);
    if (p->head_dim == 64) {
        if (p->block_size == 16) launch_valu<T, 64, 16>(pl, grid, s, a);
        else launch_valu<T, 64, 32>(pl, grid, s, a);
    } else {
        if (p->block_size == 16) launch_valu<T, 128, 16>(pl, grid, s, a);
        else launch_valu<T, 128, 32>(pl, grid, s, a);
    }
}

template <typename T>
void launch_combine(const pa_problem* p, const Plan& pl, hipStream_t s, const float* ws,
                    const int32_t* lens, void* out) {
    const int64_t rows = (int64_t)p->batch * p->num_heads * p->nq;
    if (pl.kernel == PA_KERNEL_MFMA) {
        pa::SplitCombineArgs<T> c;
        const char* const wb = reinterpret_cast<const char*>(ws);
        c.ws_o = reinterpret_cast<const typename pa::Partial<T>::type*>(wb);
        c.ws_ml = reinterpret_cast<const float*>(wb + ml_offset(p, pl));
        c.meta = reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(ws) +
                                                  meta_offset(p, pl));
        c.out = static_cast<T*>(out);
        c.KV = p->num_kv_heads;
        c.H = p->num_heads;
        c.NQ = p->nq;
        c.R = (p->num_heads / p->num_kv_heads) * p->nq;
        // pieces per sequence is data dependent; groups / sequences + 1 estimates
        // it. Many pieces per row: four waves per row; else one wave per row.
        const int64_t units = (int64_t)p->batch * p->num_kv_heads;
        const int64_t pieces = pl.parts / p->batch + 1;
        if (pieces >= 48) {
            const dim3 grid((unsigned)(units * c.R));
            if (p->head_dim == 64)
                hipLaunchKernelGGL((pa::combine_split<T, 64, 4>), grid, dim3(256), 0, s, c);
            else
                hipLaunchKernelGGL((pa::combine_split<T, 128, 4>), grid, dim3(256), 0, s, c);
        } else if (c.R >= 32) {
            // many rows per (sequence, head): two rows per wave (64 rows: merge
            // 6.8-7.1 -> 6.1 us; on 4 and 8 rows it measured no faster or slower)
            const dim3 grid((unsigned)(units * ((c.R + 7) / 8)));
            if (p->head_dim == 64)
                hipLaunchKernelGGL((pa::combine_split<T, 64, 1, 2>), grid, dim3(256), 0, s, c);
            else
                hipLaunchKernelGGL((pa::combine_split<T, 128, 1, 2>), grid, dim3(256), 0, s, c);
        } else if (pieces > 8) {
            const dim3 grid((unsigned)(units * ((c.R + 3) / 4)));
            if (p->head_dim == 64)
                hipLaunchKernelGGL((pa::combine_split<T, 64, 1>), grid, dim3(256), 0, s, c);
            else
                hipLaunchKernelGGL((pa::combine_split<T, 128, 1>), grid, dim3(256), 0, s, c);
        } else {
            // few pieces per row: batches of 8 keep the waves small (38 VGPRs on
            // ragged serving, 8 waves per SIMD): its merge 10.7 -> 8.6 us
            const dim3 grid((unsigned)(units * ((c.R + 3) / 4)));
            if (p->head_dim == 64)
                hipLaunchKernelGGL((pa::combine_split<T, 64, 1, 1, 8>), grid, dim3(256), 0, s, c);
            else
                hipLaunchKernelGGL((pa::combine_split<T, 128, 1, 1, 8>), grid, dim3(256), 0, s, c);
        }
        return;
    }
    pa::CombineArgs<T> c;
    c.ws_o = ws;
    c.ws_ml = ws + rows * pl.parts * p->head_dim;
    c.context_lens = lens;
    c.out = static_cast<T*>(out);
    c.rows = rows;
    c.rows_per_seq = p->num_heads * p->nq;
    c.n_parts = pl.parts;
    c.chunk = pl.chunk;
    c.max_tokens = p->max_blocks_per_seq * p->block_size;
    const dim3 grid((unsigned)ceil_div(rows, 4));
    if (p->head_dim == 64)
        hipLaunchKernelGGL((pa::combine_partitions<T, 64>), grid, dim3(256), 0, s, c);
    else
        hipLaunchKernelGGL((pa::combine_partitions<T, 128>), grid, dim3(256), 0, s, c);
}

template <typename T>
int run_decode(const pa_problem* p, const Plan& pl, const void* q, const void* k_pool,
               const void* v_pool, const int32_t* block_table, const int32_t* context_lens,
               const void* new_k, const void* new_v, float scale, void* out, void* workspace,
               hipStream_t s, const int32_t* slots = nullptr) {
    pa::DecodeArgs<T> a;
    a.ap.slots = slots;
    a.ap.k_dst = slots ? const_cast<void*>(k_pool) : nullptr;  // written only when appending
    a.ap.v_dst = slots ? const_cast<void*>(v_pool) : nullptr;
    a.ap.n_slot = (int64_t)p->num_blocks * p->block_size;
    const int64_t rows = (int64_t)p->batch * p->num_heads * p->nq;
    a.q = static_cast<const T*>(q);
    a.k_pool = static_cast<const T*>(k_pool);
    a.v_pool = static_cast<const T*>(v_pool);
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.new_k = static_cast<const T*>(new_k);
    a.new_v = static_cast<const T*>(new_v);
    a.out = static_cast<T*>(out);
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = workspace ? static_cast<float*>(workspace) + rows * pl.parts * p->head_dim : nullptr;
    a.H = p->num_heads;
    a.KV = p->num_kv_heads;
    a.NQ = p->nq;
    a.causal = p->causal;
    a.max_blocks = p->max_blocks_per_seq;
    a.chunk = pl.chunk;
    a.n_parts = pl.parts;
    a.n_tiles = pl.n_tiles;
    a.qscale = (float)((double)scale * 1.4426950408889634);
    launch_pass1<T>(p, pl, s, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess)
        return fail(PA_ERR_LAUNCH, "pass-1 launch failed: %s; verify the device state",
                    hipGetErrorString(e));
    if (pl.parts > 1 && !(p->flags & PA_FLAG_DEFER_COMBINE)) {
        launch_combine<T>(p, pl, s, static_cast<const float*>(workspace), context_lens, out);
        if (hipError_t e = hipGetLastError(); e != hipSuccess)
            return fail(PA_ERR_LAUNCH, "combine launch failed: %s; verify the device state",
                        hipGetErrorString(e));
    }
    return succeed();
}

int decode_entry(const pa_problem* problem, const void* q, const void* k_pool,
                 const void* v_pool, const int32_t* block_table, const int32_t* context_lens,
                 const void* new_k, const void* new_v, const int32_t* slots, float scale,
                 void* out, void* workspace, size_t workspace_bytes, pa_stream_t stream) {
    if (int rc = validate_problem(problem)) return rc;
    if (problem->batch == 0) return succeed();
    if (int rc = validate_tensors(problem, q, k_pool, v_pool, block_table, context_lens, new_k,
                                  new_v, out))
        return rc;
    if (workspace && misaligned(workspace, 16))
        return fail(PA_ERR_INVALID_ARG, "workspace (%p) is not 16-byte aligned", workspace);
    int cus = 0;
    if (int rc = current_device_cus(&cus)) return rc;
    Plan pl;
    if (int rc = plan_impl(problem, cus, &pl)) return rc;
    const size_t need = workspace_bytes_for(problem, pl);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes at %p is smaller than the %zu bytes "
                    "this plan needs (%d partitions); verify pa_workspace_size",
                    workspace_bytes, workspace, need, pl.parts);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (problem->dtype) {
        case PA_F32:
            return run_decode<float>(problem, pl, q, k_pool, v_pool, block_table, context_lens,
                                     new_k, new_v, scale, out, workspace, s, slots);
        case PA_F16:
            return run_decode<_Float16>(problem, pl, q, k_pool, v_pool, block_table,
                                        context_lens, new_k, new_v, scale, out, workspace, s,
                                        slots);
        default:
            return run_decode<pa::bf16_t>(problem, pl, q, k_pool, v_pool, block_table,
                                          context_lens, new_k, new_v, scale, out, workspace, s,
                                          slots);
    }
}

// ---------------------------------------------------------------------------
// Dense GQA attention forward
// ---------------------------------------------------------------------------
int validate_dense(const pa_dense_problem* p) {
    if (!p) return fail(PA_ERR_INVALID_ARG, "problem is NULL");
    if (p->batch < 0 || p->q_len < 0 || p->kv_len < 0)
        return fail(PA_ERR_INVALID_ARG, "batch (%d), q_len (%d) and kv_len (%d) must be >= 0",
                    p->batch, p->q_len, p->kv_len);
    if (p->num_heads < 1 || p->num_kv_heads < 1 || p->num_heads % p->num_kv_heads != 0)
        return fail(PA_ERR_INVALID_ARG, "num_heads (%d) must be a positive multiple of "
                    "num_kv_heads (%d)", p->num_heads, p->num_kv_heads);
    if (p->num_heads / p->num_kv_heads > 64)
        return fail(PA_ERR_UNSUPPORTED, "at most 64 query heads per KV head (got %d)",
                    p->num_heads / p->num_kv_heads);
    if (p->head_dim != 64 && p->head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "head_dim %d: supported are 64 and 128", p->head_dim);
    if (p->dtype != PA_F16 && p->dtype != PA_BF16)
        return fail(p->dtype == PA_F32 ? PA_ERR_UNSUPPORTED : PA_ERR_INVALID_ARG,
                    "dtype %d: the dense kernel takes fp16 or bf16", p->dtype);
    if (p->causal != 0 && p->causal != 1)
        return fail(PA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (p->mask_kind < PA_MASK_NONE || p->mask_kind > PA_MASK_ADD)
        return fail(PA_ERR_INVALID_ARG, "mask_kind %d is not a pa_mask_kind", p->mask_kind);
    if (p->mask_kind != PA_MASK_NONE) {
        const int32_t* m = p->mask_dims;
        if ((m[0] != 1 && m[0] != p->batch) || (m[1] != 1 && m[1] != p->num_heads) ||
            (m[2] != 1 && m[2] != p->q_len) || m[3] < 1 || m[3] > (p->kv_len > 0 ? p->kv_len : 1))
            return fail(PA_ERR_INVALID_ARG, "mask_dims [%d, %d, %d, %d] must be [1|batch, "
                        "1|num_heads, 1|q_len, 1..kv_len]", m[0], m[1], m[2], m[3]);
    }
    // query rows of one KV head are addressed with 32-bit byte offsets
    const int64_t span = (int64_t)(p->num_heads / p->num_kv_heads) * p->q_len * p->head_dim * 2;
    if (span >= (1LL << 31))
        return fail(PA_ERR_UNSUPPORTED, "(num_heads/num_kv_heads) * q_len * head_dim is too "
                    "large for one call; split the query length");
    return PA_OK;
}

// Dense forward launch shapes: NW = 4 waves sharing a ring of 16-key slots.
// Without the causal limit every block has the same work: two 16-row tiles per
// wave (128 rows a workgroup). Causal: block p attends p + 1 tiles of keys, so
// a workgroup takes blocks p and nblk - 1 - p (the same total for everyone) with
// one tile per wave (64 rows), which keeps two workgroups per CU. Measured on a
// 2048-token prefill (32 query heads over 8 KV heads, D = 128): non-causal 568
// TFLOP/s with 128 rows, 534 with 64; causal 331 TFLOP/s paired with 64 rows,
// 302 paired with 128 (one workgroup per CU), 294 unpaired (the workgroups of a
// CU got blocks of the same weight).
constexpr int kDenseWaves = 4;
int dense_tiles(int causal) { return causal ? 1 : 2; }  // 16-row tiles per wave

template <typename T, int D, int MASK>
void launch_dense_k(const pa::DenseArgs<T>& a, unsigned grid, hipStream_t s) {
    constexpr int kRing = D == 128 ? 4 : 8;
    const size_t lds = (size_t)kRing * pa::SlotLayout<T, D>::kBytes;
    if (a.g.causal)
        hipLaunchKernelGGL((pa::dense_mfma<T, D, kDenseWaves, 1, kRing, MASK, true>), dim3(grid),
                           dim3(64 * kDenseWaves), lds, s, a);
    else
        hipLaunchKernelGGL((pa::dense_mfma<T, D, kDenseWaves, 2, kRing, MASK, false>), dim3(grid),
                           dim3(64 * kDenseWaves), lds, s, a);
}

// Kernel arguments of a dense problem (forward geometry; out, dout and the
// statistics pointers left empty).
template <typename T>
pa::DenseArgs<T> dense_args(const pa_dense_problem* p, const void* q, const void* k,
                            const void* v, const void* mask, float scale) {
    pa::DenseArgs<T> a{};
    a.q = static_cast<const T*>(q);
    a.k = static_cast<const T*>(k);
    a.v = static_cast<const T*>(v);
    a.mask = mask;
    a.mb = p->mask_dims[0];
    a.mh = p->mask_dims[1];
    a.mq = p->mask_dims[2];
    a.mw = p->mask_dims[3];
    a.g.B = p->batch;
    a.g.HQ = p->num_heads;
    a.g.HK = p->num_kv_heads;
    a.g.SQ = p->q_len;
    a.g.SK = p->kv_len;
    a.g.G = p->num_heads / p->num_kv_heads;
    a.g.P = 16 * kDenseWaves * dense_tiles(p->causal) / a.g.G;  // rows = G * P <= 64 or 128
    a.g.nblk = (int)ceil_div(p->q_len, a.g.P);
    a.g.causal = p->causal;
    a.qscale = (float)((double)scale * 1.4426950408889634);
    return a;
}

// Workgroups of the forward's row blocks (paired under the causal limit).
int64_t dense_row_grid(const pa_dense_problem* p, const pa::DenseGeometry& g) {
    const int64_t per_kv = p->causal ? (g.nblk + 1) / 2 : g.nblk;
    return (int64_t)p->batch * p->num_kv_heads * per_kv;
}

template <typename T>
int run_dense(const pa_dense_problem* p, const void* q, const void* k, const void* v,
              const void* mask, float scale, void* out, hipStream_t s) {
    pa::DenseArgs<T> a = dense_args<T>(p, q, k, v, mask, scale);
    a.out = static_cast<T*>(out);
    const int64_t grid = dense_row_grid(p, a.g);
    if (grid >= (1LL << 31))
        return fail(PA_ERR_UNSUPPORTED, "too many workgroups (%lld) for one call",
                    (long long)grid);
    const int mk = p->mask_kind;
    if (p->head_dim == 64) {
        if (mk == PA_MASK_BOOL) launch_dense_k<T, 64, 1>(a, (unsigned)grid, s);
        else if (mk == PA_MASK_ADD) launch_dense_k<T, 64, 2>(a, (unsigned)grid, s);
        else launch_dense_k<T, 64, 0>(a, (unsigned)grid, s);
    } else {
        if (mk == PA_MASK_BOOL) launch_dense_k<T, 128, 1>(a, (unsigned)grid, s);
        else if (mk == PA_MASK_ADD) launch_dense_k<T, 128, 2>(a, (unsigned)grid, s);
        else launch_dense_k<T, 128, 0>(a, (unsigned)grid, s);
    }
    if (hipError_t e = hipGetLastError(); e != hipSuccess)
        return fail(PA_ERR_LAUNCH, "dense attention launch failed: %s; verify the device state",
                    hipGetErrorString(e));
    return succeed();
}

// ---------------------------------------------------------------------------
// Dense GQA attention backward
// ---------------------------------------------------------------------------
// dK/dV: 16 keys per wave, four key waves (64 keys) per workgroup, in two sets
// that split the query tiles (eight waves).
constexpr int kBwdKeyWaves = 4;

// Bytes of one statistics array (lse or delta): a float per query row plus 16
// floats of padding (the dK/dV kernel reads whole 16-row tiles), rounded up to
// 256 bytes.
size_t dense_stats_bytes(const pa_dense_problem* p) {
    const int64_t rows = (int64_t)p->batch * p->num_heads * p->q_len;
    return (size_t)(((rows + 16) * 4 + 255) / 256 * 256);
}

// Elements of dK (and of dV): batch * num_kv_heads * kv_len * head_dim.
int64_t dense_kv_elems(const pa_dense_problem* p) {
    return (int64_t)p->batch * p->num_kv_heads * p->kv_len * p->head_dim;
}

// Causal calls with G >= 2 give each dK/dV workgroup half the query heads of two
// key blocks of complementary weight; their fp32 sums (two halves of dK and of
// dV) follow the statistics in the workspace.
bool dense_bwd_split(const pa_dense_problem* p) {
    return p->causal && p->num_heads / p->num_kv_heads >= 2;
}
size_t dense_bwd_bytes(const pa_dense_problem* p) {
    size_t n = 2 * dense_stats_bytes(p);
    if (dense_bwd_split(p)) n += (size_t)(4 * dense_kv_elems(p)) * sizeof(float);
    return n;
}

// Rings: the statistics pass uses the forward's; a backward tile is one slot
// (two halves of 16 rows), 64 KiB of them per workgroup (the dK/dV kernel's
// slots are shared by its two wave sets).
template <typename T, int D, int MASK>
void launch_dense_bwd_k(const pa::DenseArgs<T>& a, const pa::BwdArgs<T>& w, unsigned grid_rows,
                        unsigned grid_keys, hipStream_t s) {
    constexpr int kSlot = pa::SlotLayout<T, D>::kBytes;
    constexpr int kRing = D == 128 ? 4 : 8;  // forward ring
    constexpr int kRingDq = 65536 / kSlot;
    constexpr int kRingKv = 65536 / (2 * kSlot);
    const size_t lds_fwd = (size_t)kRing * kSlot;
    const size_t lds_bwd = 65536;
    const float* lse = a.lse;
    const float* dl = a.delta;
    if (grid_rows) {
        if (a.g.causal) {
            hipLaunchKernelGGL((pa::dense_mfma<T, D, kDenseWaves, 1, kRing, MASK, true, true>),
                               dim3(grid_rows), dim3(64 * kDenseWaves), lds_fwd, s, a);
            hipLaunchKernelGGL((pa::dense_bwd_dq<T, D, kDenseWaves, 1, kRingDq, MASK, true>),
                               dim3(grid_rows), dim3(64 * kDenseWaves), lds_bwd, s, a, w, lse, dl);
        } else {
            hipLaunchKernelGGL((pa::dense_mfma<T, D, kDenseWaves, 2, kRing, MASK, false, true>),
                               dim3(grid_rows), dim3(64 * kDenseWaves), lds_fwd, s, a);
            hipLaunchKernelGGL((pa::dense_bwd_dq<T, D, kDenseWaves, 2, kRingDq, MASK, false>),
                               dim3(grid_rows), dim3(64 * kDenseWaves), lds_bwd, s, a, w, lse, dl);
        }
    }
    if (grid_keys && w.part_dk) {  // grid_keys = workgroups: pairs of key blocks, two head halves
        hipLaunchKernelGGL((pa::dense_bwd_dkdv<T, D, kBwdKeyWaves, kRingKv, MASK, true>),
                           dim3(grid_keys), dim3(128 * kBwdKeyWaves), lds_bwd, s, a, w, lse, dl);
        hipLaunchKernelGGL((pa::dense_bwd_sum_halves<T>),
                           dim3((unsigned)ceil_div(2 * w.part_n, 4 * 256)), dim3(256), 0, s, w);
    } else if (grid_keys) {
        hipLaunchKernelGGL((pa::dense_bwd_dkdv<T, D, kBwdKeyWaves, kRingKv, MASK, false>),
                           dim3(grid_keys), dim3(128 * kBwdKeyWaves), lds_bwd, s, a, w, lse, dl);
    }
}

template <typename T>
int run_dense_bwd(const pa_dense_problem* p, const void* q, const void* k, const void* v,
                  const void* mask, const void* dout, float scale, void* dq, void* dk, void* dv,
                  void* workspace, hipStream_t s) {
    pa::DenseArgs<T> a = dense_args<T>(p, q, k, v, mask, scale);
    a.dout = static_cast<const T*>(dout);
    a.lse = static_cast<float*>(workspace);
    a.delta = reinterpret_cast<float*>(static_cast<char*>(workspace) + dense_stats_bytes(p));
    pa::BwdArgs<T> w{};
    w.dout = a.dout;
    w.dq = static_cast<T*>(dq);
    w.dk = static_cast<T*>(dk);
    w.dv = static_cast<T*>(dv);
    w.scale = scale;
    w.part_n = dense_kv_elems(p);
    if (dense_bwd_split(p)) {
        w.part_dk = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             2 * dense_stats_bytes(p));
        w.part_dv = w.part_dk + 2 * w.part_n;
    }
    const int64_t grid_rows = p->q_len > 0 ? dense_row_grid(p, a.g) : 0;
    const int64_t nkb = ceil_div(p->kv_len, 16 * kBwdKeyWaves);  // key blocks per (b, kh)
    const int64_t grid_keys = (int64_t)p->batch * p->num_kv_heads *
                              (dense_bwd_split(p) ? 2 * ((nkb + 1) / 2) : nkb);
    if (grid_rows >= (1LL << 31) || grid_keys >= (1LL << 31) ||
        ceil_div(2 * w.part_n, 4 * 256) >= (1LL << 31))
        return fail(PA_ERR_UNSUPPORTED, "too many workgroups (%lld, %lld) for one call",
                    (long long)grid_rows, (long long)grid_keys);
    const unsigned gr = (unsigned)grid_rows, gk = (unsigned)grid_keys;
    const int mk = p->mask_kind;
    if (p->head_dim == 64) {
        if (mk == PA_MASK_BOOL) launch_dense_bwd_k<T, 64, 1>(a, w, gr, gk, s);
        else if (mk == PA_MASK_ADD) launch_dense_bwd_k<T, 64, 2>(a, w, gr, gk, s);
        else launch_dense_bwd_k<T, 64, 0>(a, w, gr, gk, s);
    } else {
        if (mk == PA_MASK_BOOL) launch_dense_bwd_k<T, 128, 1>(a, w, gr, gk, s);
        else if (mk == PA_MASK_ADD) launch_dense_bwd_k<T, 128, 2>(a, w, gr, gk, s);
        else launch_dense_bwd_k<T, 128, 0>(a, w, gr, gk, s);
    }
    if (hipError_t e = hipGetLastError(); e != hipSuccess)
        return fail(PA_ERR_LAUNCH, "dense attention backward launch failed: %s; verify the "
                    "device state", hipGetErrorString(e));
    return succeed();
}

}  // namespace

extern "C" {

int pa_dense_attention(const pa_dense_problem* problem, const void* q, const void* k,
                       const void* v, const void* mask, float scale, void* out,
                       pa_stream_t stream) {
    if (int rc = validate_dense(problem)) return rc;
    const pa_dense_problem* p = problem;
    if (p->batch == 0 || p->q_len == 0) return succeed();
    if (!q || !out || (p->kv_len > 0 && (!k || !v)))
        return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL (q %p, k %p, v %p, out %p)", q,
                    k, v, out);
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16))
        return fail(PA_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
    if (p->mask_kind != PA_MASK_NONE &&
        (!mask || (p->mask_kind == PA_MASK_ADD && misaligned(mask, 4))))
        return fail(PA_ERR_INVALID_ARG, "mask is NULL or (additive) not 4-byte aligned");
    int cus = 0;
    if (int rc = current_device_cus(&cus)) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p->dtype == PA_F16) return run_dense<_Float16>(p, q, k, v, mask, scale, out, s);
    return run_dense<pa::bf16_t>(p, q, k, v, mask, scale, out, s);
}


int pa_dense_backward_workspace_size(const pa_dense_problem* problem, size_t* bytes) {
    if (!bytes) return fail(PA_ERR_INVALID_ARG, "bytes is NULL");
    if (int rc = validate_dense(problem)) return rc;
    *bytes = dense_bwd_bytes(problem);
    return succeed();
}

int pa_dense_attention_backward(const pa_dense_problem* problem, const void* q, const void* k,
                                const void* v, const void* mask, const void* dout, float scale,
                                void* dq, void* dk, void* dv, void* workspace,
                                size_t workspace_bytes, pa_stream_t stream) {
    if (int rc = validate_dense(problem)) return rc;
    const pa_dense_problem* p = problem;
    if (p->batch == 0 || (p->q_len == 0 && p->kv_len == 0)) return succeed();
    const bool rows = p->q_len > 0, keys = p->kv_len > 0;
    if ((rows && (!q || !dout || !dq)) || (keys && (!k || !v || !dk || !dv)))
        return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL (q %p, k %p, v %p, dout %p, "
                    "dq %p, dk %p, dv %p)", q, k, v, dout, dq, dk, dv);
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(dout, 16) ||
        misaligned(dq, 16) || misaligned(dk, 16) || misaligned(dv, 16))
        return fail(PA_ERR_INVALID_ARG, "q, k, v, dout, dq, dk and dv must be 16-byte aligned");
    if (p->mask_kind != PA_MASK_NONE &&
        (!mask || (p->mask_kind == PA_MASK_ADD && misaligned(mask, 4))))
        return fail(PA_ERR_INVALID_ARG, "mask is NULL or (additive) not 4-byte aligned");
    const size_t need = dense_bwd_bytes(p);
    if (!workspace || workspace_bytes < need || misaligned(workspace, 256))
        return fail(PA_ERR_WORKSPACE, "workspace %p of %zu bytes: need %zu bytes, 256-byte "
                    "aligned (pa_dense_backward_workspace_size)", workspace, workspace_bytes, need);
    int cus = 0;
    if (int rc = current_device_cus(&cus)) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p->dtype == PA_F16)
        return run_dense_bwd<_Float16>(p, q, k, v, mask, dout, scale, dq, dk, dv, workspace, s);
    return run_dense_bwd<pa::bf16_t>(p, q, k, v, mask, dout, scale, dq, dk, dv, workspace, s);
}

int pa_plan_ex(const pa_problem* problem, int32_t num_cus, int32_t* partitions,
               int32_t* chunk_tokens, int32_t* kernel) {
    Plan pl;
    if (int rc = plan_impl(problem, num_cus, &pl)) return rc;
    if (partitions) *partitions = pl.parts;
    if (chunk_tokens) *chunk_tokens = pl.chunk;
    if (kernel) *kernel = pl.kernel;
    return succeed();
}

int pa_plan(const pa_problem* problem, int32_t* partitions, int32_t* chunk_tokens,
            int32_t* kernel) {
    if (int rc = validate_problem(problem)) return rc;
    int cus = 0;
    if (int rc = current_device_cus(&cus)) return rc;
    return pa_plan_ex(problem, cus, partitions, chunk_tokens, kernel);
}

int pa_workspace_size_ex(const pa_problem* problem, int32_t num_cus, size_t* bytes) {
    if (!bytes) return fail(PA_ERR_INVALID_ARG, "bytes is NULL");
    Plan pl;
    if (int rc = plan_impl(problem, num_cus, &pl)) return rc;
    *bytes = workspace_bytes_for(problem, pl);
    return succeed();
}

int pa_workspace_size(const pa_problem* problem, size_t* bytes) {
    if (!bytes) return fail(PA_ERR_INVALID_ARG, "bytes is NULL");
    if (int rc = validate_problem(problem)) return rc;
    int cus = 0;
    if (int rc = current_device_cus(&cus)) return rc;
    return pa_workspace_size_ex(problem, cus, bytes);
}

int paged_attn_decode(const pa_problem* problem, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_table,
                      const int32_t* context_lens, const void* new_k, const void* new_v,
                      float scale, void* out, void* workspace, size_t workspace_bytes,
                      pa_stream_t stream) {
    return decode_entry(problem, q, k_pool, v_pool, block_table, context_lens, new_k, new_v,
                        nullptr, scale, out, workspace, workspace_bytes, stream);
}

int paged_attn_decode_append(const pa_problem* problem, const void* q, void* k_pool,
                             void* v_pool, const int32_t* block_table,
                             const int32_t* context_lens, const void* new_k, const void* new_v,
                             const int32_t* slot_mapping, float scale, void* out,
                             void* workspace, size_t workspace_bytes, pa_stream_t stream) {
    if (problem && problem->batch > 0 && !slot_mapping)
        return fail(PA_ERR_INVALID_ARG, "slot_mapping is NULL; pass int32 [batch, nq] slots "
                    "(negative = row not stored) or call paged_attn_decode");
    if (misaligned(slot_mapping, 4))
        return fail(PA_ERR_INVALID_ARG, "slot_mapping (%p) is not 4-byte aligned",
                    (const void*)slot_mapping);
    return decode_entry(problem, q, k_pool, v_pool, block_table, context_lens, new_k, new_v,
                        slot_mapping, scale, out, workspace, workspace_bytes, stream);
}

int paged_attn_decode_static(const pa_problem* problem, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table,
                             const int32_t* context_lens, const void* new_k, const void* new_v,
                             float scale, void* out, pa_stream_t stream) {
    if (int rc = validate_problem(problem)) return rc;
    if (problem->flags & PA_FLAG_DEFER_COMBINE)
        return fail(PA_ERR_INVALID_ARG, "PA_FLAG_DEFER_COMBINE is not accepted by "
                    "paged_attn_decode_static (its partial states stay in the library's static "
                    "workspace, which paged_attn_combine cannot be given); verify pa_problem.flags");
    if (problem->batch == 0) return succeed();
    int cus = 0;
    if (int rc = current_device_cus(&cus)) return rc;
    Plan pl;
    if (int rc = plan_impl(problem, cus, &pl)) return rc;
    const size_t need = workspace_bytes_for(problem, pl);
    if (need > (size_t)PA_STATIC_WORKSPACE_BYTES)
        return fail(PA_ERR_WORKSPACE, "this plan (%d partitions) needs %zu bytes of workspace, "
                    "more than the %zu-byte static workspace; call paged_attn_decode with a "
                    "workspace of pa_workspace_size bytes, or lower num_partitions or the batch",
                    pl.parts, need, (size_t)PA_STATIC_WORKSPACE_BYTES);
    void* ws = nullptr;
    if (need > 0)
        if (int rc = scratch_address(&ws)) return rc;
    return decode_entry(problem, q, k_pool, v_pool, block_table, context_lens, new_k, new_v,
                        nullptr, scale, out, ws, need > 0 ? (size_t)PA_STATIC_WORKSPACE_BYTES : 0,
                        stream);
}

int paged_attn_combine(const pa_problem* problem, const int32_t* context_lens,
                       const void* workspace, size_t workspace_bytes, void* out,
                       pa_stream_t stream) {
    if (int rc = validate_problem(problem)) return rc;
    if (problem->batch == 0) return succeed();
    if (!context_lens || !out)
        return fail(PA_ERR_INVALID_ARG, "context_lens or out is NULL; verify the arguments");
    if (misaligned(out, 16) || misaligned(context_lens, 4))
        return fail(PA_ERR_INVALID_ARG, "out must be 16-byte and context_lens 4-byte aligned");
    int cus = 0;
    if (int rc = current_device_cus(&cus)) return rc;
    Plan pl;
    if (int rc = plan_impl(problem, cus, &pl)) return rc;
    if (pl.parts <= 1) return succeed();
    const size_t need = workspace_bytes_for(problem, pl);
    if (!workspace || workspace_bytes < need || misaligned(workspace, 16))
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes at %p does not hold the %zu bytes "
                    "of partial states this plan uses; verify pa_workspace_size",
                    workspace_bytes, workspace, need);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const float* ws = static_cast<const float*>(workspace);
    switch (problem->dtype) {
        case PA_F32: launch_combine<float>(problem, pl, s, ws, context_lens, out); break;
        case PA_F16: launch_combine<_Float16>(problem, pl, s, ws, context_lens, out); break;
        default: launch_combine<pa::bf16_t>(problem, pl, s, ws, context_lens, out); break;
    }
    if (hipError_t e = hipGetLastError(); e != hipSuccess)
        return fail(PA_ERR_LAUNCH, "combine launch failed: %s; verify the device state",
                    hipGetErrorString(e));
    return succeed();
}

const char* paged_attn_last_error(void) { return t_error.c_str(); }

int paged_attn_version(void) { return 105; }

}  // extern "C"
