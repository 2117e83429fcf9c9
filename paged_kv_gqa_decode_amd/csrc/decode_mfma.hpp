// Pass 1 of paged GQA decode attention on the matrix cores (gfx950, fp16/bf16),
// with the work cut into equal groups along the sequence axis (split.hpp).
//
// Operation: docs.rs page "onnxruntime-ep-mlx 0.31.1: src/ops/paged_attention.rs",
// VECTOR_BODY (scores, online softmax, accumulation) and VECTOR_PARTIALS.
//
// One wave attends one KV head over one group's positions (16-key sub-pages)
// for all R = G*NQ query rows of that head, in NRT row tiles of 16, so each
// K/V page is fetched from HBM once per GQA group:
//   scores  S^T[16 keys x 16 rows] = K Q^T  : v_mfma_f32_16x16x32 (D/32 steps);
//           A = K: lane l holds key l%16, 8 elements of d; B = Q: row l%16
//   softmax fp32 on the VALU; the D-layout of S^T (key 4*(l/16)+i, row l%16)
//           is exactly the A layout of the next product, so P stays in lane
//   output  O[16 rows x 16 d] += P V per 16 d (Mfma<T>::pv);
//           B = V: lane l needs keys 4*(l/16)..+3 at d = 16t + l%16; one
//           transposing LDS read (ds_read_b64_tr_b16) of the row-major V slot
//           delivers exactly that, so output tile t holds d = 16t + l%16.
// The reference max moves only when a score exceeds it by more than 2^kSlack
// (probabilities stay <= 256), so the accumulators are rescaled almost never.
// Sub-pages are staged through a ring of NS LDS slots per wave by
// buffer-to-LDS loads (no VGPRs held by loads in flight, non-temporal: the pool
// is streamed once); block-table entries are scalar loads issued one fetch
// ahead of their use, so they never share the vector-memory counter with the
// loads whose completion the wave counts. The KV waves of a group read the
// heads of the same pages at the same time (the pool keeps a token's heads
// adjacent), which the memory system serves faster than one head at a time.
// Occupancy: NRT = 1 runs 4 waves per SIMD with one slot each; NRT = 2, 2
// waves with 2 slots; NRT = 4, 1 wave with 4 slots: the same bytes in flight
// per CU (D = 128), with room for the larger accumulators.
#pragma once

#include <type_traits>

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

// Mfma<T>: the two products of one 16-key sub-page and the P operand.
//   qk: S^T += K Q^T over 32 d (v_mfma_f32_16x16x32).
//   make_p: P operand(s) of 4 probabilities of a lane. fp16: one operand
//     (round to nearest). bf16: p = hi + lo with hi = p truncated to bf16 and
//     lo = the exact fp32 remainder truncated again, so P keeps ~16 bits.
//   pv: O += P V for one 16-column output tile. fp16: v_mfma_f32_16x16x16f16.
//     bf16: one v_mfma_f32_16x16x32_bf16 whose 32-long contraction holds the
//     hi parts against V and the lo parts against the same V again (lane k
//     index 8*g + j: j < 4 -> hi of key 4*g + j, j >= 4 -> lo of key 4*g + j - 4).
template <> struct Mfma<_Float16> {
    __device__ static __forceinline__ f32x4_t qk(u32x4_t k, u32x4_t q, f32x4_t acc) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, k),
                                                      __builtin_bit_cast(f16x8_t, q), acc, 0, 0, 0);
    }
    __device__ static __forceinline__ unsigned pack2(float lo, float hi) {
        return (unsigned)__builtin_bit_cast(uint16_t, (_Float16)lo) |
               ((unsigned)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
    }
    __device__ static __forceinline__ void make_p(const float (&p)[4], u32x2_t& phi, u32x2_t&) {
        phi = u32x2_t{pack2(p[0], p[1]), pack2(p[2], p[3])};
    }
    __device__ static __forceinline__ f32x4_t pv(u32x2_t phi, u32x2_t, u32x2_t v, f32x4_t acc) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, phi),
                                                     __builtin_bit_cast(f16x4_t, v), acc, 0, 0, 0);
    }
    // O += P V over two sub-pages in one 32-deep product (the same cost as one
    // 16-deep product): lane k slots 0..3 hold the first sub-page's keys
    // 4*g .. 4*g + 3, slots 4..7 the second's, in both operands.
    __device__ static __forceinline__ f32x4_t pv2(u32x2_t p0, u32x2_t p1, u32x2_t v0, u32x2_t v1,
                                                  f32x4_t acc) {
        const u32x4_t a = u32x4_t{p0[0], p0[1], p1[0], p1[1]};
        const u32x4_t b = u32x4_t{v0[0], v0[1], v1[0], v1[1]};
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), acc, 0, 0, 0);
    }
};

template <> struct Mfma<bf16_t> {
    __device__ static __forceinline__ f32x4_t qk(u32x4_t k, u32x4_t q, f32x4_t acc) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k),
                                                       __builtin_bit_cast(bf16x8_t, q), acc, 0, 0, 0);
    }
    __device__ static __forceinline__ unsigned pack2(float lo, float hi) {
        return (unsigned)f32_to_bf16_rne(lo) | ((unsigned)f32_to_bf16_rne(hi) << 16);
    }
    // high halves of two fp32 values, packed (element 0 in the low half)
    __device__ static __forceinline__ unsigned high2(float a, float b) {
        return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
    }
    __device__ static __forceinline__ void make_p(const float (&p)[4], u32x2_t& phi, u32x2_t& plo) {
        float lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[i] = p[i] - __uint_as_float(__float_as_uint(p[i]) & 0xffff0000u);
        phi = u32x2_t{high2(p[0], p[1]), high2(p[2], p[3])};
        plo = u32x2_t{high2(lo[0], lo[1]), high2(lo[2], lo[3])};
    }
    __device__ static __forceinline__ f32x4_t pv(u32x2_t phi, u32x2_t plo, u32x2_t v, f32x4_t acc) {
        const u32x4_t a = u32x4_t{phi[0], phi[1], plo[0], plo[1]};
        const u32x4_t b = u32x4_t{v[0], v[1], v[0], v[1]};
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
    }
};

// Raw buffer descriptor over `bytes` bytes at p (GFX9-family format word).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// s_waitcnt immediates (GFX9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8]
// | vmcnt[5:4] << 14): wait for all vector-memory operations, or for all LDS ops.
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;
// wait until at most n vector-memory operations of this wave are outstanding
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Cache policy of the pool loads: the non-temporal bit (bit 1 of the buffer
// instruction's cache-policy operand). Every pool byte is read once per step, so
// nothing is gained by keeping it in L2 or the Infinity Cache; streaming it
// through raises the sustained read rate of this page pattern by about 12 %.
constexpr int kStreamPolicy = 2;

// Slack of the lazy reference max, in log2 units (probabilities stay <= 256).
constexpr float kSlack = 8.0f;

// Issue priority from progress: every wave of the grid has the same work (the
// balanced split), but the arbiter favours the oldest waves of a CU, so the
// workgroups dispatched first finish early and the last ones set the kernel's
// end. A wave starts at priority 3 and steps down one level per quarter of its
// sub-pages, so the waves that are behind are issued first (measured: multi-row
// causal pass 1 68 -> 66 us, ragged serving 284 -> 281 us).
struct ProgressPrio {
    int level, next, n;  // level holds while i < next = n * (4 - level) / 4
    __device__ __forceinline__ ProgressPrio(int n_total, bool on)
        : level(3), next(n_total / 4), n(n_total) {
        if (on) __builtin_amdgcn_s_setprio(3);
    }
    __device__ __forceinline__ void update(int i) {
        if (i < next) return;  // one compare per sub-page; the rest three times a wave
        do {
            --level;
            next = n * (4 - level) / 4;
        } while (level > 0 && i >= next);
        if (level == 2) __builtin_amdgcn_s_setprio(2);
        else if (level == 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
    }
};

// Logical workgroup index: the hardware hands workgroups to the 8 XCDs in turn
// (workgroup n to XCD n % 8), so logical index (n % 8) * (N / 8) + n / 8 puts
// consecutive logical indices, i.e. the KV heads of one group, on one XCD. The
// last N % 8 workgroups keep their index (the map is a bijection of [0, N)).
__device__ __forceinline__ int64_t xcd_local_block() {
    const int64_t n = gridDim.x, b = blockIdx.x;
    const int64_t full = n / 8 * 8;
    if (b >= full) return b;
    return (b % 8) * (n / 8) + b / 8;
}

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
    typename Partial<T>::type* ws_o;  // [slots][R][D]  partial outputs (Partial<T>)
    float* ws_ml;  // [slots][R][2]  (max, sum) in base-2 units
    int32_t* meta; // [B][2]         first and last group overlapping each sequence
    SplitGeometry g;
    int H, causal, max_blocks, R;
    float qscale;  // scale * log2(e)
    AppendArgs ap; // slot-patched step (ap.slots == nullptr: plain step)
};

// LDS layout of one sub-page slot (16 keys), filled by row-coalesced 16-byte
// buffer-to-LDS loads; each load instruction fills 1 KB (kKeysPerOp whole
// rows of 2*D bytes). K rows, then V rows, back to back; the 16-byte chunk c of
// key row k sits at position c ^ swz(k) (K) or c ^ vswz(k) (V), which puts the
// operand reads on distinct banks (the minimum number of passes):
//  K: a K-operand read takes one chunk of keys 0..15: swz(k) spreads them.
//  V: a transposing read (ds_read_b64_tr_b16) takes 8 bytes of 16 rows for
//     one 16-column tile: vswz(k) = 2 * (row line % (kChunks/2)) moves the
//     32-byte column pair of consecutive row lines apart.
template <typename T, int D>
struct SlotLayout {
    static constexpr int kRowBytes = D * (int)sizeof(T);
    static constexpr int kChunks = kRowBytes / 16;       // 16-byte chunks per row
    static constexpr int kKeysPerOp = 1024 / kRowBytes;  // rows per load instruction
    static constexpr int kOps = 16 / kKeysPerOp;         // load instructions per half
    static constexpr int kRowsPerBank = 256 / kRowBytes; // rows sharing one 256-byte bank line
    static constexpr int kKBytes = 16 * kRowBytes;
    static constexpr int kBytes = 2 * kKBytes;
    __device__ static __forceinline__ int swz(int k) { return (k / kRowsPerBank) % kChunks; }
    __device__ static __forceinline__ int vswz(int k) {
        return 2 * ((k / kRowsPerBank) % (kChunks / 2));
    }
    // K: byte offset of logical chunk c of key k
    __device__ static __forceinline__ int k_addr(int k, int c) {
        return k * kRowBytes + ((c ^ swz(k)) << 4);
    }
    // V (from the V half): byte offset of logical chunk c of key k
    __device__ static __forceinline__ int v_addr(int k, int c) {
        return k * kRowBytes + ((c ^ vswz(k)) << 4);
    }
    // K: the offset lane l fetches in instruction i is k_fetch_base ^ (64*i).
    // For both row sizes the instruction-i row of lane l has swz = 4*i + l/16,
    // so its chunk is ((l % kChunks) ^ (l/16)) ^ (4*i): only offset bits 6..7
    // depend on i, and the row part is a multiple of the 256- or 128-byte row.
    __device__ static __forceinline__ int k_fetch_base(int lane, int tbytes) {
        return (lane / kChunks) * tbytes + (((lane % kChunks) ^ (lane >> 4)) << 4);
    }
    // V: offset (beyond the instruction's first row) that lane l fetches in
    // instruction i: chunk (l % kChunks) ^ vswz(k) of key k = i*kKeysPerOp + l/kChunks
    __device__ static __forceinline__ int v_fetch_off(int i, int lane, int tbytes) {
        const int k = kKeysPerOp * i + lane / kChunks;
        return (lane / kChunks) * tbytes + (((lane % kChunks) ^ vswz(k)) << 4);
    }
};

typedef __attribute__((address_space(3))) void lds_void;

// Loads rows 0..15 (row stride D elements; rows past rmax repeat row rmax) of
// K and V starting at k and v into the slot at `slot` in the slot layout,
// instructions i = i0, i0 + istep, ... (COUNT of each half); 16 bytes per lane
// per instruction. All offsets are in voffset, so the descriptors cover exactly
// rmax + 1 rows.
// VV: the first half also in the second half's layout (rows read with
// slot_read_rows_v, columns with slot_read_cols_at).
template <typename T, int D, int COUNT, bool VV = false>
__device__ __forceinline__ void fetch_rows(const T* k, const T* v, int rmax, char* slot, int lane,
                                           int i0 = 0, int istep = 1) {
    using Lay = SlotLayout<T, D>;
    constexpr int kStride = D * (int)sizeof(T);
    char* const k_lds = slot;
    char* const v_lds = slot + Lay::kKBytes;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(k, (rmax + 1) * kStride);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(v, (rmax + 1) * kStride);
    int ln = lane;
    asm volatile("" : "+v"(ln));  // computed here, not kept live across the loop
#pragma unroll
    for (int t = 0; t < COUNT; ++t) {
        const int i = i0 + istep * t;
        const int row = Lay::kKeysPerOp * i + ln / Lay::kChunks;
        const int rc = min(row, rmax);
        const int koff = rc * kStride +
                         (((ln % Lay::kChunks) ^ (VV ? Lay::vswz(row) : Lay::swz(row))) << 4);
        const int voff = rc * kStride + (((ln % Lay::kChunks) ^ Lay::vswz(row)) << 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(k_lds + i * 1024), 16, koff, 0,
                                                 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(v_lds + i * 1024), 16, voff, 0,
                                                 0, 0);
    }
}

// ---- the stream of one wave's sub-pages: cursor, table entries, fetches ----
// SEQ: the sequence table (SeqTableLds or SeqTableRegs).
template <typename T, int D, int BS, typename SEQ = SeqTableLds>
struct SubPageStream {
    using Lay = SlotLayout<T, D>;
    static constexpr int KS = D / 32;    // load instructions per half (K or V)
    static constexpr int SUB = BS / 16;  // 16-key sub-pages per page
    static constexpr int kNewStride = D * (int)sizeof(T);  // row stride of new_k/new_v
    static constexpr int kOps = 2 * KS;  // vector-memory instructions of one fetch

    struct Cur {
        int b, j;       // sequence b, its sub-page j (the head is the wave's)
        int nsub, nc;   // sub-pages of the sequence; the first nc hold cached keys
        int L;          // cached keys of sequence b
    };
    struct Src {
        const T* k;  // first row of the 16-key span (head kh)
        const T* v;
        int rmax;    // last row that exists (15 for cached keys)
    };

    const SplitArgs<T>& a;
    const int32_t* __restrict__ table;  // block table; entries are read with scalar loads
    const int32_t* __restrict__ slots;  // slot-patched step: [B][NQ] (a.ap.slots), else nullptr
    SEQ seq;
    int KV, NQ, kh, nnew, tbytes, lane;
    int kfb;  // per-lane K fetch offset of a cached sub-page (instruction 0)
    int pre_phys = 0;  // table entry of the last prefetch_table() position
    int pat_b = -1;    // slot-patched step: sequence whose block range is held
    int pat_blo = 0, pat_bhi = -1;  // smallest and largest block its new rows' slots are in

    __device__ __forceinline__ SubPageStream(const SplitArgs<T>& args,
                                             const int32_t* __restrict__ tab,
                                             const int32_t* __restrict__ sl, const SEQ& sq,
                                             int head, int ln)
        : a(args), table(tab), slots(sl), seq(sq), KV(args.g.KV), NQ(args.g.NQ), kh(head),
          nnew((args.g.NQ + 15) / 16), tbytes(args.g.KV * D * (int)sizeof(T)), lane(ln) {
        kfb = Lay::k_fetch_base(lane, tbytes);
    }
    __device__ __forceinline__ void enter_seq(Cur& c) const {
        c.nsub = seq.pref(c.b + 1) - seq.pref(c.b);
        c.nc = c.nsub - nnew;
        c.L = seq.len(c.b);
    }
    __device__ __forceinline__ Cur seek(int64_t x) const {  // the sub-page at axis position x
        Cur c;
        c.b = seq.find(a.g, x);
        enter_seq(c);
        c.j = (int)(x - seq.pref(c.b));
        return c;
    }
    __device__ __forceinline__ void step(Cur& c) const {  // next position along the axis
        if (++c.j < c.nsub) return;
        c.j = 0;
        ++c.b;
        enter_seq(c);
    }
    // Block-table entry of a cached sub-page: a scalar load (wave-uniform
    // address, read-only table), counted apart from the vector loads in flight.
    __device__ __forceinline__ int table_entry(const Cur& c) const {
        return table[(int64_t)c.b * a.max_blocks + c.j / SUB];
    }
    // Table entries of the positions c, c + 1, ... (n of them, n <= N) for
    // priming a ring: their scalar loads go out back to back (one latency for
    // the run instead of one per sub-page); entries of new-row positions are 0.
    template <int N>
    __device__ __forceinline__ void run_tables(Cur c, int n, int (&phys)[N]) const {
#pragma unroll
        for (int k = 0; k < N; ++k) {
            phys[k] = k < n && c.j < c.nc ? table_entry(c) : 0;
            if (k + 1 < n) step(c);
        }
    }
    // Starts loading the table entry of c ahead of locate(c).
    __device__ __forceinline__ void prefetch_table(const Cur& c) {
        if (c.j >= c.nc) return;  // new rows: no table
        pre_phys = table_entry(c);
    }
    // Source of sub-page c; a cached one must be the position of the last
    // prefetch_table() (every fetch after the prime follows that order).
    __device__ __forceinline__ Src locate(const Cur& c) const { return locate_at(c, pre_phys); }
    // locate() with the table entry of a cached sub-page already at hand
    __device__ __forceinline__ Src locate_at(const Cur& c, int64_t phys) const {
        Src s;
        if (c.j < c.nc) {
            const int64_t row0 = phys * BS + 16 * (c.j % SUB);
            s.k = a.k_pool + (row0 * KV + kh) * D;
            s.v = a.v_pool + (row0 * KV + kh) * D;
            s.rmax = 15;
        } else {
            const int t0 = 16 * (c.j - c.nc);
            const int64_t r0 = ((int64_t)c.b * KV + kh) * NQ + t0;
            s.k = a.new_k + r0 * D;
            s.v = a.new_v + r0 * D;
            s.rmax = min(15, NQ - t0 - 1);
        }
        return s;
    }
    // Issues load instructions i = i0, i0 + istep, ... (COUNT of them, < KS) of
    // the K and of the V half of sub-page `s` into the slot at `slot`
    // (row-coalesced, 16 bytes per lane per instruction); COUNT = KS, i0 = 0,
    // istep = 1 is the whole sub-page (kOps instructions). Cached keys: pool
    // row stride, no range check needed, non-temporal. New rows: all offsets
    // in voffset and rows past nq clamped to the last one (they are masked
    // later). (Offsets go in as plain int values: an array element or a
    // dependent expression passed as is makes the host compilation pass drop
    // the kernel's launch stub.)
    template <int COUNT = KS>
    __device__ __forceinline__ void fetch(const Src& s, char* slot, bool cached, int i0 = 0,
                                          int istep = 1) const {
        char* const k_lds = slot;
        char* const v_lds = slot + Lay::kKBytes;
        if (cached) {
            const __amdgpu_buffer_rsrc_t kr = make_rsrc(s.k, 16 * tbytes);
            const __amdgpu_buffer_rsrc_t vr = make_rsrc(s.v, 16 * tbytes);
#pragma unroll
            for (int t = 0; t < COUNT; ++t) {
                const int i = i0 + istep * t;
                const int koff = kfb ^ (64 * i);
                const int soff = i * Lay::kKeysPerOp * tbytes;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(k_lds + i * 1024), 16,
                                                         koff, soff, 0, kStreamPolicy);
            }
#pragma unroll
            for (int t = 0; t < COUNT; ++t) {
                const int i = i0 + istep * t;
                const int voff = Lay::v_fetch_off(i, lane, tbytes);
                const int soff = i * Lay::kKeysPerOp * tbytes;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(v_lds + i * 1024), 16,
                                                         voff, soff, 0, kStreamPolicy);
            }
        } else {
            fetch_rows<T, D, COUNT>(s.k, s.v, s.rmax, slot, lane, i0, istep);
        }
    }

    // ---- slot-patched step (AppendArgs) ----
    // Whether a new row of sequence c.b names the slot of a valid key of cached
    // sub-page c in block `phys` (wave-uniform). The range of slots the
    // sequence's rows name is kept per sequence, so the rows themselves are
    // only compared for sub-pages inside it.
    __device__ __forceinline__ bool patched(const Cur& c, int64_t phys) {
        if (c.j >= c.nc) return false;
        const int32_t* sl = slots + (int64_t)c.b * NQ;
        if (c.b != pat_b) {  // the blocks the sequence's stored rows fall in
            pat_b = c.b;
            pat_blo = 0x7fffffff;
            pat_bhi = -1;
            for (int j = 0; j < NQ; ++j) {
                const int32_t sj = sl[j];
                if (sj < 0 || sj >= a.ap.n_slot) continue;  // neither stored nor read
                pat_blo = min(pat_blo, sj / BS);
                pat_bhi = max(pat_bhi, sj / BS);
            }
        }
        if ((int)phys < pat_blo || (int)phys > pat_bhi) return false;
        const int64_t base = phys * BS + 16 * (c.j % SUB);
        const int valid = min(16, c.L - 16 * c.j);
        bool any = false;
        for (int j = 0; j < NQ; ++j) {
            const int64_t t = (int64_t)sl[j] - base;
            any = any || (t >= 0 && t < valid);
        }
        return any;
    }
    // Overwrites, in LDS slot `slot` holding cached sub-page c, each key whose
    // pool slot a new row of the sequence names with that row (rows in order,
    // so the last one naming a slot stays). Lanes 0 .. kChunks - 1 move the K
    // row's 16-byte chunks, the next kChunks lanes the V row's. A rare, slow
    // path: it ends with every vector-memory operation of the wave complete.
    __device__ __forceinline__ void patch(const Cur& c, char* slot) const {
        typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
        const int64_t base = (int64_t)table_entry(c) * BS + 16 * (c.j % SUB);
        const int valid = min(16, c.L - 16 * c.j);
        const int32_t* sl = slots + (int64_t)c.b * NQ;
        const uint32_t slot_lds = (uint32_t)reinterpret_cast<uintptr_t>(slot);
        for (int j = 0; j < NQ; ++j) {
            const int64_t t = (int64_t)sl[j] - base;
            if (t < 0 || t >= valid) continue;
            const int64_t row = (((int64_t)c.b * KV + kh) * NQ + j) * D;
            if (lane < Lay::kChunks) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(a.new_k + row + 8 * lane);
                *(lds_u32x4*)(uintptr_t)(slot_lds + Lay::k_addr((int)t, lane)) = v;
            } else if (lane < 2 * Lay::kChunks) {
                const int ch = lane - Lay::kChunks;
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(a.new_v + row + 8 * ch);
                *(lds_u32x4*)(uintptr_t)(slot_lds + Lay::kKBytes + Lay::v_addr((int)t, ch)) = v;
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    // Copies new row t of the sub-page in LDS slot `slot` (head kh) to pool
    // slot s: lanes 0 .. kChunks - 1 move the K row's 16-byte chunks, the next
    // kChunks lanes the V row's. Not waited for.
    __device__ __forceinline__ void store_row(const char* slot, int t, int64_t s) const {
        typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4;
        const uint32_t slot_lds = (uint32_t)reinterpret_cast<uintptr_t>(slot);
        const int64_t row = (s * KV + kh) * D;
        if (lane < Lay::kChunks) {
            const u32x4_t v = *(lds_u32x4*)(uintptr_t)(slot_lds + Lay::k_addr(t, lane));
            *reinterpret_cast<u32x4_t*>(static_cast<T*>(a.ap.k_dst) + row + 8 * lane) = v;
        } else if (lane < 2 * Lay::kChunks) {
            const int ch = lane - Lay::kChunks;
            const u32x4_t v = *(lds_u32x4*)(uintptr_t)(slot_lds + Lay::kKBytes + Lay::v_addr(t, ch));
            *reinterpret_cast<u32x4_t*>(static_cast<T*>(a.ap.v_dst) + row + 8 * ch) = v;
        }
    }
    // Stores the new rows of sub-page c (new rows, in LDS slot `slot`) that the
    // step keeps into their pool slots, head kh of each: row j goes to slot s =
    // slots[b][j] when 0 <= s < n_slot and no later row of the sequence names
    // s; the stores are not waited for. Up to 16 rows (one new-row sub-page) the
    // sequence's slots are scalar loads (the wait for them does not drain the
    // wave's pool loads in flight); beyond, they are loaded once, lane l holding
    // rows l and 64 + l, the later rows found with a ballot (nq <= 128), and
    // that load is waited for at once (one drain of the wave's loads per unit).
    __device__ __forceinline__ void store_new(const Cur& c, const char* slot) const {
        const int t0 = 16 * (c.j - c.nc);
        const int valid = min(16, NQ - t0);
        const int32_t* sl = slots + (int64_t)c.b * NQ;
        if (NQ <= 16) {
            int32_t sm[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) sm[j] = j < NQ ? sl[j] : -1;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (j >= NQ) break;
                const int32_t sj = sm[j];
                bool later = false;
#pragma unroll
                for (int jj = j + 1; jj < 16; ++jj) later = later || (jj < NQ && sm[jj] == sj);
                if (sj < 0 || sj >= a.ap.n_slot || later) continue;
                store_row(slot, j, sj);
            }
            return;
        }
        int32_t m0 = lane < NQ ? sl[lane] : -1;
        int32_t m1 = 64 + lane < NQ ? sl[64 + lane] : -1;
        asm volatile("" : "+v"(m0), "+v"(m1));  // consumed here, whatever the loop below does
        for (int t = 0; t < valid; ++t) {
            const int j = t0 + t;
            const int32_t s = __builtin_amdgcn_readlane(j < 64 ? m0 : m1, j & 63);
            const bool later = __ballot(lane > j && lane < NQ && m0 == s) != 0 ||
                               __ballot(64 + lane > j && 64 + lane < NQ && m1 == s) != 0;
            if (s < 0 || s >= a.ap.n_slot || later) continue;
            store_row(slot, t, s);
        }
    }
};

// ---- operand reads from a slot (lane = 16*g16 + c16) ----
// Rows: the 16-byte chunks 4*kk + g16 of row c16 of the slot's first half, for
// kk < D/32: an MFMA operand whose lane holds row c16 and elements 32*kk +
// 8*g16 .. +7 (A of a product whose rows are the slot's rows, or B of one whose
// columns are). Chunk 4*kk + g16 of row c16 sits at c16*R + (((g16 ^ swz(c16))
// ^ 4*kk) << 4), so the address of step kk is one base XOR (kk << 6); the base
// is recomputed per call (opaque to the optimizer) rather than kept as D/32
// live registers. (LDS-space pointers: a generic pointer would become a flat
// load, which the vector-memory counter also counts, so waiting for the
// operand would wait for every pool load in flight.)
template <typename T, int D>
__device__ __forceinline__ void slot_read_rows(const char* slot, int c16, int g16,
                                               u32x4_t (&op)[D / 32]) {
    using Lay = SlotLayout<T, D>;
    typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4;
    uint32_t base = (uint32_t)reinterpret_cast<uintptr_t>(slot) + Lay::k_addr(c16, g16);
    asm volatile("" : "+v"(base));
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
        op[kk] = *(lds_u32x4*)(uintptr_t)(base ^ (uint32_t)(kk << 6));
}
// Columns of the slot's second half for the D/16 column tiles: the B operand
// of a 16-deep product whose contraction runs over the slot's rows, tile t =
// X[row 4*g16 + j][col 16*t + c16], j = 0..3, read with one transposing LDS
// read: within a 16-lane group, lane s supplies row 4*g16 + s/4, columns 16*t +
// 4*(s%4) .. +3, and lane c16 receives column c16 of the 4 rows. (Chunk 2*t + h
// of a row sits at ((2*t + h) ^ vswz) << 4 = base ^ (t << 5): one base per
// call.) The reads are issued as inline assembly: the compiler treats its
// transposing-read builtin as possibly aliasing the buffer-to-LDS loads in
// flight and would wait for all of them first. The results are only valid
// after slot_lds_wait(), which ties them to an LDS-counter wait.
template <typename T, int D>
__device__ __forceinline__ void slot_read_cols_at(const char* half, int c16, int g16,
                                                  u32x2_t (&vt)[D / 16]) {
    using Lay = SlotLayout<T, D>;
    const int s = c16;
    const int row = 4 * g16 + s / 4;
    uint32_t base = (uint32_t)reinterpret_cast<uintptr_t>(half) +
                    Lay::v_addr(row, (s & 3) >> 1) + 8 * (s & 1);
    asm volatile("" : "+v"(base));
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
        const uint32_t p = base ^ (uint32_t)(t << 5);
        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(vt[t]) : "v"(p) : "memory");
    }
}
template <typename T, int D>
__device__ __forceinline__ void slot_read_cols(const char* slot, int c16, int g16,
                                               u32x2_t (&vt)[D / 16]) {
    slot_read_cols_at<T, D>(slot + SlotLayout<T, D>::kKBytes, c16, g16, vt);
}
// Rows, as slot_read_rows, of a half in the second half's layout (`half` is
// its first byte): chunk 4*kk + g16 of row c16 sits at c16*R + (((g16 ^
// vswz(c16)) ^ 4*kk) << 4), again one base XOR (kk << 6).
template <typename T, int D>
__device__ __forceinline__ void slot_read_rows_v(const char* half, int c16, int g16,
                                                 u32x4_t (&op)[D / 32]) {
    using Lay = SlotLayout<T, D>;
    typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4;
    uint32_t base = (uint32_t)reinterpret_cast<uintptr_t>(half) + Lay::v_addr(c16, g16);
    asm volatile("" : "+v"(base));
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
        op[kk] = *(lds_u32x4*)(uintptr_t)(base ^ (uint32_t)(kk << 6));
}
// Waits for every LDS read of this wave (and its scalar loads); values read by
// slot_read_cols are used only through this call's outputs.
template <int D>
__device__ __forceinline__ void slot_lds_wait(u32x2_t (&vt)[D / 16]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int t = 0; t < D / 16; ++t) asm volatile("" : "+v"(vt[t]));
}

// ---- online-softmax state of NRT row tiles (rows 16*(rt0 + rt) + c16) ----
// PAIRPV (fp16 only): the PV product of a sub-page waits for the next one and
// both go through one 32-deep product; the pending half is added on its own
// (flush) before the accumulators are rescaled and before they are read.
template <typename T, int D, int NRT, bool PAIRPV = false>
struct RowTiles {
    using M = Mfma<T>;
    using Lay = SlotLayout<T, D>;
    static constexpr int KS = D / 32;  // score MFMA steps over d
    static constexpr int NT = D / 16;  // output tiles over d
    static constexpr int NP = D / 32;  // load instructions per half (K or V)

    const SplitArgs<T>& a;
    int lane, c16, g16, rt0;
    u32x4_t qop[NRT][KS];  // B of S^T = K Q^T: row 16*(rt0+rt) + c16, d = 32*kk + 8*g16 .. +8
    float m[NRT], lsum[NRT];
    f32x4_t acc[NRT][NT];
    u32x2_t phi[NRT], plo[NRT];
    static constexpr bool kPair = PAIRPV && std::is_same<T, _Float16>::value;
    u32x2_t pend_p[NRT], pend_v[NT];  // the sub-page whose PV waits (kPair)
    bool pv_pending = false;
    int rmod[NRT];  // query row modulo nq: its position among the new rows

    __device__ __forceinline__ RowTiles(const SplitArgs<T>& args, int ln, int first_tile)
        : a(args), lane(ln), c16(ln & 15), g16(ln >> 4), rt0(first_tile) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) rmod[rt] = (16 * (rt0 + rt) + c16) % args.g.NQ;
    }
    __device__ __forceinline__ int64_t grow0(int b, int kh) const {  // first output row of the unit
        const int G = a.H / a.g.KV;
        return ((int64_t)b * a.H + (int64_t)kh * G) * a.g.NQ;
    }
    // Q rows of (b, kh) as the B operands, issued as inline assembly so that
    // the compiler does not count them (it would wait for every pool load in
    // flight before their first use); q_ready() must follow once they have
    // landed. Rows past R load row R-1 (in bounds) and are zeroed by q_ready().
    // The address is a scalar base (the unit's first row) plus a 32-bit
    // per-lane byte offset, so no 64-bit per-lane pointer stays live.
    __device__ __forceinline__ void load_q(int b, int kh) {
        uint32_t rows[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) rows[rt] = (uint32_t)min(16 * (rt0 + rt) + c16, a.R - 1) * D;
        load_q_at(a.q + grow0(b, kh) * D, rows);
    }
    // load_q with this lane's row of tile rt at element offset row_off[rt] from
    // `first` (a wave-uniform address; offsets < 2^31 bytes).
    __device__ __forceinline__ void load_q_at(const T* first, const uint32_t (&row_off)[NRT]) {
        const uint64_t addr = reinterpret_cast<uint64_t>(first);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
        const T* base = reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const uint32_t off = (row_off[rt] + 8 * g16) * (uint32_t)sizeof(T);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                asm volatile("global_load_dwordx4 %0, %1, %2 offset:%3"
                             : "=v"(qop[rt][kk])
                             : "v"(off), "s"(base), "i"(64 * kk)
                             : "memory");
        }
    }
    // After a wait that covers load_q's loads: makes their values visible to
    // the code that follows and zeroes rows past R.
    __device__ __forceinline__ void q_ready() {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const bool live = 16 * (rt0 + rt) + c16 < a.R;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                asm volatile("" : "+v"(qop[rt][kk]));
                if (!live) qop[rt][kk] = u32x4_t{0, 0, 0, 0};
            }
        }
    }
    __device__ __forceinline__ void reset() {
        pv_pending = false;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            m[rt] = kNegMax;
            lsum[rt] = 0.f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    // K operands of one sub-page (A of S^T = K Q^T), read from a slot.
    __device__ __forceinline__ void read_k(const char* slot, u32x4_t (&kop)[KS]) const {
        slot_read_rows<T, D>(slot, c16, g16, kop);
    }
    // V operands of the NT output tiles (B of O += P V), read from a slot;
    // valid after lds_wait().
    __device__ __forceinline__ void read_v(const char* slot, u32x2_t (&vt)[NT]) const {
        slot_read_cols<T, D>(slot, c16, g16, vt);
    }
    __device__ __forceinline__ static void lds_wait(u32x2_t (&vt)[NT]) { slot_lds_wait<D>(vt); }
    // Visible-key limits of one sub-page: keys [0, valid) exist; for new rows
    // (is_new) key tau is new row t0 + tau, visible to a query row by causality.
    __device__ __forceinline__ void limits(int valid, bool is_new, int t0, int (&lim)[NRT]) const {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
            lim[rt] = is_new && a.causal ? min(valid, rmod[rt] - t0 + 1) : valid;
    }
    // S^T and the online softmax for one sub-page; leaves the P operands in
    // phi/plo. Keys 4*g16 + i >= lim[rt] are not visible to this lane's row.
    // `full`: every key of the sub-page is visible to every row (wave-uniform),
    // so no score needs masking. The score products of all row tiles are
    // issued before any is read (one tile: two independent half-chains over
    // d), so the matrix-core latency of one chain is covered by the others.
    // BIAS: bias[rt][i] (base-2 units, -inf hides) is added to the score of
    // key 4*g16 + i of this lane's row.
    template <bool BIAS = false>
    __device__ __forceinline__ void scores(const u32x4_t (&kop)[KS], const int (&lim)[NRT],
                                           bool full, const float (*bias)[4] = nullptr) {
        constexpr int NC = NRT == 1 && KS % 2 == 0 ? 2 : 1;  // chains per tile
        f32x4_t sc[NRT][NC];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int c = 0; c < NC; ++c) sc[rt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
                sc[rt][kk % NC] = M::qk(kop[kk], qop[rt][kk], sc[rt][kk % NC]);
        float sv[NRT][4], tms[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            f32x4_t s = sc[rt][0];
            if constexpr (NC == 2) s += sc[rt][1];
            if (full) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[rt][i] = s[i] * a.qscale;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sv[rt][i] = 4 * g16 + i < lim[rt] ? s[i] * a.qscale : -__builtin_inff();
            }
            if constexpr (BIAS) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[rt][i] += bias[rt][i];
            }
            // m[rt] is the same in the 4 lanes of a row (lanes c16 + 16*g).
            tms[rt] = fmaxf(fmaxf(sv[rt][0], sv[rt][1]), fmaxf(sv[rt][2], sv[rt][3]));
        }
        if constexpr (kPair) {
            // a waiting PV product is at the old references: add it before any
            // tile's accumulators are rescaled
            bool moves = false;
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) moves = moves || tms[rt] > m[rt] + kSlack;
            if (__any(moves)) flush();
        }
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            float tm = tms[rt];
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
            for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sv[rt][i] - m[rt]);
            lsum[rt] += (p[0] + p[1]) + (p[2] + p[3]);
            M::make_p(p, phi[rt], plo[rt]);
        }
    }
    // O += P V; keys [valid, 16) are zeroed first (their slot rows may hold NaN).
    // Lane key 4*g16 + j is 16-bit half j of the lane's two dwords.
    __device__ __forceinline__ void accumulate(u32x2_t (&vt)[NT], int valid) {
        if (valid < 16) {
            const int k0 = 4 * g16;
            const unsigned m0 = (k0 < valid ? 0xffffu : 0u) | (k0 + 1 < valid ? 0xffff0000u : 0u);
            const unsigned m1 = (k0 + 2 < valid ? 0xffffu : 0u) | (k0 + 3 < valid ? 0xffff0000u : 0u);
#pragma unroll
            for (int t = 0; t < NT; ++t) vt[t] = u32x2_t{vt[t][0] & m0, vt[t][1] & m1};
        }
        if constexpr (kPair) {
            if (!pv_pending) {  // wait for the next sub-page
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) pend_p[rt] = phi[rt];
#pragma unroll
                for (int t = 0; t < NT; ++t) pend_v[t] = vt[t];
                pv_pending = true;
                return;
            }
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
                    acc[rt][t] = M::pv2(pend_p[rt], phi[rt], pend_v[t], vt[t], acc[rt][t]);
            pv_pending = false;
        } else {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
                    acc[rt][t] = M::pv(phi[rt], plo[rt], vt[t], acc[rt][t]);
        }
    }
    // Adds a waiting PV product on its own (kPair; nothing otherwise).
    __device__ __forceinline__ void flush() {
        if constexpr (kPair) {
            if (!pv_pending) return;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
                    acc[rt][t] = M::pv(pend_p[rt], pend_p[rt], pend_v[t], acc[rt][t]);
            pv_pending = false;
        }
    }
    // Normalised rows (all of their keys attended): output row r, held in
    // acc[rt][*][i] for r = 16*(rt0 + rt) + 4*g16 + i, goes to `base` + off(r)
    // (elements) unless off(r) < 0; 0 where nothing was visible.
    template <typename F>
    __device__ __forceinline__ void emit_rows(T* base, F&& off) const {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            float lrow = lsum[rt];
            lrow += __shfl_xor(lrow, 16);
            lrow += __shfl_xor(lrow, 32);  // l of row 16*(rt0+rt) + c16
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float l_r = __shfl(lrow, 4 * g16 + i);
                const int64_t o = off(16 * (rt0 + rt) + 4 * g16 + i);
                if (o < 0) continue;
                const float inv = l_r != 0.f ? 1.f / l_r : 0.f;
                T* dst = base + o + c16;
#pragma unroll
                for (int t = 0; t < NT; ++t) Elem<T>::store(dst + 16 * t, acc[rt][t][i] * inv);
            }
        }
    }
    // The finished output of (b, kh) (its whole sequence attended here), or
    // this piece's state for the combine (workspace slot (b + grp)*KV + kh).
    __device__ __forceinline__ void emit(int b, int kh, int64_t grp, bool whole) const {
        const int64_t g0 = grow0(b, kh);
        const int R = a.R;
        const int64_t slot = ((int64_t)b + grp) * a.g.KV + kh;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            float lrow = lsum[rt];
            lrow += __shfl_xor(lrow, 16);
            lrow += __shfl_xor(lrow, 32);  // l of row 16*(rt0+rt) + c16
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * (rt0 + rt) + 4 * g16 + i;  // output row held in acc[rt][*][i]
                const float l_r = __shfl(lrow, 4 * g16 + i);
                if (r >= R) continue;
                // tile t holds d = 16*t + c16
                if (whole) {
                    const float inv = l_r != 0.f ? 1.f / l_r : 0.f;
                    T* dst = a.out + (g0 + r) * D + c16;
#pragma unroll
                    for (int t = 0; t < NT; ++t) Elem<T>::store(dst + 16 * t, acc[rt][t][i] * inv);
                } else if constexpr (Partial<T>::kNorm) {
                    const float inv = l_r != 0.f ? 1.f / l_r : 0.f;
                    auto* dst = a.ws_o + (slot * R + r) * D + c16;
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        dst[16 * t] = (typename Partial<T>::type)(acc[rt][t][i] * inv);
                } else {
                    auto* dst = a.ws_o + (slot * R + r) * D + c16;
#pragma unroll
                    for (int t = 0; t < NT; ++t) dst[16 * t] = acc[rt][t][i];
                }
            }
            const int row = 16 * (rt0 + rt) + c16;
            if (!whole && g16 == 0 && row < R) {
                float* ml = a.ws_ml + (slot * R + row) * 2;
                ml[0] = m[rt];
                ml[1] = lrow;
            }
        }
    }
};

// Waits until at most A vector-memory instructions of this wave are
// outstanding, for A = OPS * ahead (ahead <= MAXA; a runtime value dispatched to
// immediates).
template <int OPS, int MAXA>
__device__ __forceinline__ void wait_ahead(int ahead) {
    if constexpr (MAXA > 0) {
        if (ahead >= MAXA) {
            __builtin_amdgcn_s_waitcnt(wait_vm(OPS * MAXA));
            return;
        }
        wait_ahead<OPS, MAXA - 1>(ahead);
    } else {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
}

// ---- one wave per (group, KV head): NRT row tiles, a ring of NS slots ----
// Sub-page i of the wave's run sits in slot i % NS. Iteration i waits until
// sub-page i has landed (vector loads complete in issue order, so at most
// kOps * (fetches issued after it) may be outstanding; Q loads and workspace
// stores issued in between can only make that wait longer), reads the slot
// into registers, refills it with sub-page i + NS (i + 1 when NS = 1: issued
// before the arithmetic; otherwise after the scores, so that the next
// sequence's Q, loaded after the scores, is older than the refill), then
// computes. NS sub-pages per wave stay in flight.
template <typename T, int D, int BS, int NRT, int NS, int WPS, bool APPEND, bool REGSEQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPS, WPS)))
void decode_mfma(SplitArgs<T> a, const int32_t* __restrict__ table,
                 const int32_t* __restrict__ slots) {
    using Lay = SlotLayout<T, D>;
    using Seq = typename std::conditional<REGSEQ, SeqTableRegs, SeqTableLds>::type;
    using Stream = SubPageStream<T, D, BS, Seq>;
    using Rows = RowTiles<T, D, NRT>;
    using Cur = typename Stream::Cur;
    constexpr int KS = D / 32;
    static_assert(D % 32 == 0 && BS % 16 == 0 && Lay::kOps == KS, "shape");
    static_assert(Stream::kOps * (NS - 1) <= 63, "vmcnt range");

    // LDS: per wave NS slots, then (REGSEQ false) the prefix and lengths.
    extern __shared__ __attribute__((aligned(1024))) char smem[];  // slots start 1 KiB aligned (XOR addressing)
    const Seq seq = [&]() {
        if constexpr (REGSEQ) {
            return SeqTableRegs(a.context_lens, a.g);  // each wave its own copy: no barrier
        } else {
            int* s_pref = reinterpret_cast<int*>(smem + 4 * NS * Lay::kBytes);
            int* s_len = s_pref + a.g.B + 1;
            build_prefix(a.context_lens, a.g, s_pref, s_len);
            return SeqTableLds{s_pref, s_len, a.g.B};
        }
    }();
    const Cut cut(a.g, seq.total());

    // The wave index is uniform within a wave; saying so keeps every per-wave
    // quantity (group, head, sequence, page, descriptors, LDS slot) scalar.
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // (measured: 0.6 us faster on the Llama-3-8B batch, 1.5 us on ragged
    // serving; the cooperative kernel, whose groups span eight workgroups,
    // keeps the hardware order, which measured faster for it)
    const int64_t gw = xcd_local_block() * 4 + wave;
    const int64_t grp = gw / a.g.KV;  // the KV waves of a group are consecutive
    const int kh = (int)(gw - grp * a.g.KV);
    if (grp >= cut.n) return;  // no barrier follows
    const int64_t x0 = cut.start(grp, seq, a.g);
    const int n_total = (int)(cut.start(grp + 1, seq, a.g) - x0);  // sub-pages this wave attends
    if (n_total == 0) return;  // a group inside a sequence's pad
    char* const ring = smem + wave * NS * Lay::kBytes;

    Stream st(a, table, slots, seq, kh, lane);
    Rows rows(a, lane, 0);
    Cur cc = st.seek(x0);  // the sub-page being attended
    Cur pc = cc;           // the next sub-page to fetch
    rows.load_q(cc.b, kh);  // older than every fetch: the first wait covers it
    // prime the ring with sub-pages 0 .. min(NS, n_total) - 1
    const int nf = min(NS, n_total);
    uint32_t pmask = 0;  // bit k: the sub-page in slot k has keys to patch (slot-patched step)
    {
        int phys[NS];
        st.run_tables(cc, nf, phys);
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            if (k < nf) {
                if constexpr (APPEND)
                    if (st.patched(pc, phys[k])) pmask |= 1u << k;
                st.fetch(st.locate_at(pc, phys[k]), ring + k * Lay::kBytes, pc.j < pc.nc);
            }
            if (k + 1 < nf) st.step(pc);
        }
        if (nf < n_total) st.step(pc);
    }
    if (nf < n_total) st.prefetch_table(pc);  // its table entry, one fetch ahead
    rows.reset();
    bool piece_from_start = cc.j == 0;
    bool q_pending = true;   // load_q issued, q_ready not yet called
    int q_younger = NS;      // fetches issued after the pending Q loads (upper bound)
    ProgressPrio prio(n_total, true);
    for (int i = 0; i < n_total; ++i) {
        prio.update(i);
        const bool more = i + 1 < n_total;
        if (cc.j == 0 && kh == 0 && lane == 0 && a.meta) {
            // the first piece of a sequence records the groups it spans
            const int64_t s0 = seq.pref(cc.b);
            a.meta[2 * cc.b] = (int32_t)cut.group_of(s0, cc.b);
            a.meta[2 * cc.b + 1] = (int32_t)cut.group_of(s0 + cc.nsub - 1, cc.b);
        }
        // Sub-page i has landed once at most kOps * (fetches issued after it)
        // vector loads are outstanding; pending Q loads need at most
        // kOps * q_younger.
        const int ahead = min(NS - 1, n_total - 1 - i);
        wait_ahead<Stream::kOps, NS - 1>(q_pending ? min(ahead, q_younger) : ahead);
        if (q_pending) {
            rows.q_ready();
            q_pending = false;
        }
        char* const slot = ring + (i % NS) * Lay::kBytes;
        if constexpr (APPEND) {
            if ((pmask >> (i % NS)) & 1u) st.patch(cc, slot);  // cached keys re-written this step
            if (cc.j >= cc.nc) st.store_new(cc, slot);         // this step's rows into the pools
        }
        u32x4_t kop[KS];
        u32x2_t vt[D / 16];
        rows.read_k(slot, kop);
        rows.read_v(slot, vt);
        const bool refill = i + NS < n_total;  // sub-page i + NS exists (it is pc)
        if constexpr (NS == 1) {
            if (refill) {
                const typename Stream::Src sn = st.locate(pc);
                if constexpr (APPEND) pmask = st.patched(pc, st.pre_phys) ? 1u : 0u;
                Rows::lds_wait(vt);  // slot read out
                st.fetch(sn, slot, pc.j < pc.nc);
            } else {
                Rows::lds_wait(vt);
            }
        } else {
            Rows::lds_wait(vt);
        }
        const bool seq_ends = cc.j + 1 == cc.nsub;
        // NS > 1: the slot is read out, so it is refilled at once, unless this
        // sub-page ends its sequence: the next sequence's Q, loaded after the
        // scores (it overwrites this one's), must then be older than the refill
        const bool late = more && seq_ends;
        auto refill_slot = [&]() {
            if constexpr (APPEND) {
                const uint32_t bit = 1u << (i % NS);
                pmask = st.patched(pc, st.pre_phys) ? (pmask | bit) : (pmask & ~bit);
            }
            st.fetch(st.locate(pc), slot, pc.j < pc.nc);
            ++q_younger;
        };
        if constexpr (NS > 1)
            if (refill && !late) refill_slot();
        const bool is_new = cc.j >= cc.nc;
        const int t0 = 16 * (cc.j - cc.nc);
        const int valid = is_new ? min(16, st.NQ - t0) : min(16, cc.L - 16 * cc.j);
        int lim[NRT];
        rows.limits(valid, is_new, t0, lim);
        rows.scores(kop, lim, !is_new && valid == 16);
        if (late) {  // Q of the next sequence
            rows.load_q(cc.b + 1, kh);
            q_pending = true;
            q_younger = 0;
        }
        if constexpr (NS > 1)
            if (refill && late) refill_slot();
        if (refill && i + NS + 1 < n_total) {
            st.step(pc);
            st.prefetch_table(pc);
        }
        rows.accumulate(vt, valid);
        if (seq_ends || !more) {
            rows.emit(cc.b, kh, grp, piece_from_start && seq_ends);
            rows.reset();
            piece_from_start = true;
        }
        if (more) st.step(cc);
    }
}

// ---- NW waves per (group, KV head), NRT row tiles each, sharing a ring ----
// For R > 16 rows: the workgroup's waves split the row tiles (wave w owns tiles
// w*NRT ..) and share a ring of kRing sub-page slots, so each sub-page is read
// from HBM once and from LDS once per wave. Every wave issues its share of each
// sub-page's load instructions (NWI waves issue; vmcnt thresholds count only a
// wave's own loads); one bare s_barrier per sub-page publishes it and frees the
// slot read in the previous iteration, which is refilled at once: kRing - 1
// sub-pages per workgroup stay in flight during the arithmetic. A sequence
// switch loads the waves' new Q after the arithmetic (it is waited for at the
// next iteration, a rare full drain).
template <typename T, int D, int BS, int NW, int NRT, int kRing, int WPS, bool APPEND,
          bool REGSEQ>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPS, WPS)))
void decode_mfma_coop(SplitArgs<T> a, const int32_t* __restrict__ table,
                      const int32_t* __restrict__ slots) {
    using Lay = SlotLayout<T, D>;
    using Seq = typename std::conditional<REGSEQ, SeqTableRegs, SeqTableLds>::type;
    using Stream = SubPageStream<T, D, BS, Seq>;
    using Rows = RowTiles<T, D, NRT, true>;
    using Cur = typename Stream::Cur;
    constexpr int KS = D / 32;
    constexpr int NWI = NW < KS ? NW : KS;  // waves that issue loads
    constexpr int IPW = KS / NWI;           // instructions per half per issuing wave
    static_assert(D % 32 == 0 && BS % 16 == 0 && Lay::kOps == KS && KS % NWI == 0, "shape");
    static_assert(kRing >= 3 && 2 * IPW * (kRing - 2) <= 63, "ring");

    extern __shared__ __attribute__((aligned(1024))) char smem[];  // slots start 1 KiB aligned (XOR addressing)
    const Seq seq = [&]() {
        if constexpr (REGSEQ) {
            return SeqTableRegs(a.context_lens, a.g);  // no LDS beyond the ring
        } else {
            int* s_pref = reinterpret_cast<int*>(smem + kRing * Lay::kBytes);
            int* s_len = s_pref + a.g.B + 1;
            build_prefix(a.context_lens, a.g, s_pref, s_len);
            return SeqTableLds{s_pref, s_len, a.g.B};
        }
    }();
    const Cut cut(a.g, seq.total());

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t grp = blockIdx.x / a.g.KV;  // the KV workgroups of a group are consecutive
    const int kh = (int)(blockIdx.x - grp * a.g.KV);
    if (grp >= cut.n) return;  // uniform over the workgroup: no barrier follows
    const int64_t x0 = cut.start(grp, seq, a.g);
    const int n_total = (int)(cut.start(grp + 1, seq, a.g) - x0);
    if (n_total == 0) return;  // a group inside a sequence's pad (uniform)
    const bool issues = wave < NWI;  // this wave loads instructions wave, wave + NWI, ...
    const bool has_rows = 16 * NRT * wave < a.R;

    Stream st(a, table, slots, seq, kh, lane);
    Rows rows(a, lane, wave * NRT);
    Cur cc = st.seek(x0);
    Cur pc = cc;  // next sub-page to fetch: kRing - 1 ahead of cc once primed
    if (has_rows) rows.load_q(cc.b, kh);  // older than the ring's loads
    uint32_t pmask = 0;  // bit k: the sub-page in slot k has keys to patch (slot-patched step)
    {
        const int np = min(kRing - 1, n_total);
        int phys[kRing - 1];
        st.run_tables(cc, np, phys);
#pragma unroll
        for (int k = 0; k < kRing - 1; ++k) {
            if (k < np) {
                if constexpr (APPEND)
                    if (st.patched(pc, phys[k])) pmask |= 1u << k;
                if (issues)
                    st.template fetch<IPW>(st.locate_at(pc, phys[k]), smem + k * Lay::kBytes,
                                           pc.j < pc.nc, wave, NWI);
            }
            if (k + 1 < n_total && k + 1 <= np) st.step(pc);
        }
    }
    st.prefetch_table(pc);
    rows.reset();
    bool q_pending = has_rows;  // load_q issued, q_ready not yet called
    bool q_drain = false;       // pending Q is younger than the ring's loads
    bool piece_from_start = cc.j == 0;
    ProgressPrio prio(n_total, !APPEND);
    for (int i = 0; i < n_total; ++i) {
        if constexpr (!APPEND) prio.update(i);  // the slot-patched cooperative step measured better without
        const int ahead = min(kRing - 2, n_total - 1 - i);  // sub-pages fetched after i
        if (cc.j == 0 && lane == 0 && wave == 0 && kh == 0 && a.meta) {
            const int64_t s0 = seq.pref(cc.b);
            a.meta[2 * cc.b] = (int32_t)cut.group_of(s0, cc.b);
            a.meta[2 * cc.b + 1] = (int32_t)cut.group_of(s0 + cc.nsub - 1, cc.b);
        }
        // this wave's loads of sub-page i have landed (later ones may be in flight)
        if (issues && !q_drain) {
            wait_ahead<2 * IPW, kRing - 2>(ahead);
        } else {
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
        }
        if (q_pending) {
            rows.q_ready();
            q_pending = false;
            q_drain = false;
        }
        // Every wave's part of sub-page i is in; slot i-1 is read out. A bare
        // barrier: each wave has already waited for its own loads (LDS needs no
        // flush within the CU), and a fenced barrier would also wait for the
        // loads still in flight into the other slots.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if constexpr (APPEND) {
            char* const cur = smem + (i % kRing) * Lay::kBytes;
            if ((pmask >> (i % kRing)) & 1u) {  // cached keys re-written this step (uniform)
                if (wave == 0) st.patch(cc, cur);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
            if (cc.j >= cc.nc && wave == 0) st.store_new(cc, cur);  // into the pools
        }
        // refill the slot of sub-page i - 1 with sub-page i + kRing - 1
        const int nxt = i + kRing - 1;
        if (nxt < n_total) {
            if constexpr (APPEND) {
                const uint32_t bit = 1u << (nxt % kRing);
                pmask = st.patched(pc, st.pre_phys) ? (pmask | bit) : (pmask & ~bit);
            }
            const typename Stream::Src sn = st.locate(pc);
            if (issues)
                st.template fetch<IPW>(sn, smem + (nxt % kRing) * Lay::kBytes, pc.j < pc.nc, wave, NWI);
        }
        // the next fetch position and its table entry; the scalar load is
        // issued after this iteration's LDS wait (which would also wait for it)
        const bool adv = nxt + 1 < n_total;
        const char* slot = smem + (i % kRing) * Lay::kBytes;
        const bool is_new = cc.j >= cc.nc;
        const int t0 = 16 * (cc.j - cc.nc);
        const int valid = is_new ? min(16, st.NQ - t0) : min(16, cc.L - 16 * cc.j);
        const bool seq_ends = cc.j + 1 == cc.nsub;
        const bool piece_ends = seq_ends || i + 1 == n_total;
        if (has_rows) {
            u32x4_t kop[KS];
            u32x2_t vt[D / 16];
            rows.read_k(slot, kop);
            rows.read_v(slot, vt);
            Rows::lds_wait(vt);
            if (adv) {
                st.step(pc);
                st.prefetch_table(pc);
            }
            int lim[NRT];
            rows.limits(valid, is_new, t0, lim);
            rows.scores(kop, lim, !is_new && valid == 16);
            rows.accumulate(vt, valid);
            if (piece_ends) {
                rows.flush();
                rows.emit(cc.b, kh, grp, piece_from_start && seq_ends);
                rows.reset();
            }
        } else if (adv) {
            st.step(pc);
            st.prefetch_table(pc);
        }
        if (piece_ends) piece_from_start = true;
        if (i + 1 < n_total) {
            st.step(cc);
            if (has_rows && cc.j == 0) {  // Q of the next sequence
                rows.load_q(cc.b, kh);
                q_pending = true;
                q_drain = true;
            }
        }
    }
}

}  // namespace pa
