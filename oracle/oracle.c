/*
 * Reference oracle for paged-KV grouped-query decode attention (plain C, double).
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark; never by the product path. It shares no
 * code with the HIP library.
 *
 * Source of the definition: docs.rs source page "onnxruntime-ep-mlx 0.31.1:
 * src/ops/paged_attention.rs".
 *   - GQA head mapping, visible-key window, block-table address and the
 *     widening of stored elements to fp32: VECTOR_BODY.
 *   - Empty rows produce zeros (division skipped when the sum is zero):
 *     VECTOR_REDUCE and PARTIALS_REDUCE.
 *   - Chunk merge with weights exp(m_c - M): VECTOR_PARTIALS + PARTIALS_REDUCE.
 * The same head grouping (query head h = kh*G + g) appears on the docs.rs page
 * "onnxruntime-ep-mlx 0.31.1: src/ops/attention_vjp/dense.rs", execute().
 *
 * Readings taken where the page is silent:
 *   - context_lens[b] is the cached length only; row r additionally sees new
 *     rows 0..r when causal, all NQ new rows otherwise (VECTOR_BODY's `total`).
 *   - The softmax scale is the binary32 value passed in, widened to double
 *     (the page passes the fp32 bit pattern of the scale to the kernel).
 *   - Slot patching (oracle_kv_append): the page gives each new row j a pool
 *     slot (block * BS + offset, negative = none) and makes a cached position
 *     whose slot is one of them read that new row instead of the pool, the
 *     last such j winning; the engine page writes the rows into those slots.
 *     Both are the same as first storing every new row into its slot in
 *     order (sequence, then j ascending: later stores replace earlier ones)
 *     and then gathering as usual. Slots outside [0, num_blocks * BS) are
 *     ignored.
 * No blocking, fusion or reordering beyond gathering one (sequence, KV head)
 * once and reusing it for the G*NQ query rows that read it.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE binary16 -> double, exact (sign, 5-bit exponent, 10-bit fraction). */
static double half_bits_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exponent = (h >> 10) & 0x1f;
    int fraction = h & 0x3ff;
    double value;
    if (exponent == 0)
        value = ldexp((double)fraction, -24); /* subnormal: fraction * 2^-24 */
    else if (exponent == 31)
        value = fraction ? NAN : INFINITY;
    else
        value = ldexp((double)(fraction + 1024), exponent - 25);
    return sign ? -value : value;
}

/* bfloat16 -> double, exact: the 16 bits are the top half of a binary32. */
static double bf16_bits_to_double(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

double oracle_widen(const void* base, int64_t index, int dtype)
{
    const unsigned char* p = (const unsigned char*)base;
    if (dtype == 0) {
        float f;
        memcpy(&f, p + index * 4, 4);
        return (double)f;
    }
    uint16_t bits;
    memcpy(&bits, p + index * 2, 2);
    return dtype == 1 ? half_bits_to_double(bits) : bf16_bits_to_double(bits);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int check_args(int B, int H, int KV, int D, int BS, int max_blocks, int NQ,
                      int dtype, const int32_t* context_lens)
{
    if (B < 0 || H <= 0 || KV <= 0 || D <= 0 || BS <= 0 || max_blocks < 0 || NQ < 0)
        return -1;
    if (H % KV != 0)
        return -2;
    if (dtype < 0 || dtype > 2)
        return -3;
    for (int b = 0; b < B; ++b)
        if (context_lens[b] < 0 || context_lens[b] > (int64_t)max_blocks * BS)
            return -4;
    return 0;
}

/*
 * Gather the logical key/value sequence of (b, kh): cached positions i < L in
 * order through the block table, then the NQ new rows. Rows are D doubles.
 */
static void gather(int b, int kh, int KV, int D, int BS, int max_blocks, int NQ, int dtype,
                   const void* k_pool, const void* v_pool, const int32_t* block_table,
                   int L, const void* new_k, const void* new_v, double* K, double* V)
{
    for (int i = 0; i < L; ++i) {
        int64_t physical = block_table[(int64_t)b * max_blocks + i / BS];
        int64_t row = ((physical * BS + i % BS) * KV + kh) * (int64_t)D;
        for (int d = 0; d < D; ++d) {
            K[(int64_t)i * D + d] = oracle_widen(k_pool, row + d, dtype);
            V[(int64_t)i * D + d] = oracle_widen(v_pool, row + d, dtype);
        }
    }
    for (int j = 0; j < NQ; ++j) {
        int64_t row = (((int64_t)b * KV + kh) * NQ + j) * D;
        for (int d = 0; d < D; ++d) {
            K[(int64_t)(L + j) * D + d] = oracle_widen(new_k, row + d, dtype);
            V[(int64_t)(L + j) * D + d] = oracle_widen(new_v, row + d, dtype);
        }
    }
}

/* s_i = scale * <q, K_i> for the first n keys. */
static void scores(const double* qrow, const double* K, int n, int D, double scale, double* s)
{
    for (int i = 0; i < n; ++i) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += qrow[d] * K[(int64_t)i * D + d];
        s[i] = scale * dot;
    }
}

static int decode_impl(int B, int H, int KV, int D, int BS, int max_blocks, int NQ, int causal,
                       int dtype, const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_table, const int32_t* context_lens,
                       const void* new_k, const void* new_v, float scale, int chunk,
                       int max_chunks, double* part_m, double* part_z, double* part_o,
                       double* out)
{
    int rc = check_args(B, H, KV, D, BS, max_blocks, NQ, dtype, context_lens);
    if (rc)
        return rc;
    if (chunk < 0 || (chunk > 0 && max_chunks <= 0))
        return -5;
    const int G = H / KV;
    const double sc = (double)scale;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t unit = 0; unit < (int64_t)B * KV; ++unit) {
        const int b = (int)(unit / KV), kh = (int)(unit % KV);
        const int L = context_lens[b];
        const int64_t n_all = (int64_t)L + NQ;
        double* K = (double*)malloc(sizeof(double) * (size_t)(n_all > 0 ? n_all : 1) * D);
        double* V = (double*)malloc(sizeof(double) * (size_t)(n_all > 0 ? n_all : 1) * D);
        double* s = (double*)malloc(sizeof(double) * (size_t)(n_all > 0 ? n_all : 1));
        double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
        if (!K || !V || !s || !qrow || !acc) {
#pragma omp atomic write
            failed = 1;
            free(K); free(V); free(s); free(qrow); free(acc);
            continue;
        }
        gather(b, kh, KV, D, BS, max_blocks, NQ, dtype, k_pool, v_pool, block_table, L, new_k,
               new_v, K, V);
        for (int g = 0; g < G; ++g) {
            const int h = kh * G + g; /* query head h reads KV head h / G */
            for (int r = 0; r < NQ; ++r) {
                const int64_t orow = ((int64_t)b * H + h) * NQ + r;
                const int n = L + (causal ? r + 1 : NQ);
                for (int d = 0; d < D; ++d)
                    qrow[d] = oracle_widen(q, orow * D + d, dtype);
                scores(qrow, K, n, D, sc, s);
                double* o = out + orow * D;
                if (chunk == 0) {
                    /* textbook softmax: m = max s, w = exp(s - m), out = sum w V / sum w */
                    double m = -INFINITY, Z = 0.0;
                    for (int i = 0; i < n; ++i)
                        if (s[i] > m)
                            m = s[i];
                    for (int d = 0; d < D; ++d)
                        acc[d] = 0.0;
                    for (int i = 0; i < n; ++i) {
                        double w = exp(s[i] - m);
                        Z += w;
                        for (int d = 0; d < D; ++d)
                            acc[d] += w * V[(int64_t)i * D + d];
                    }
                    for (int d = 0; d < D; ++d)
                        o[d] = Z != 0.0 ? acc[d] / Z : 0.0;
                } else {
                    /* per-chunk states, then the merge */
                    const int n_chunks = (n + chunk - 1) / chunk;
                    double M = -INFINITY, Z = 0.0;
                    for (int d = 0; d < D; ++d)
                        acc[d] = 0.0;
                    for (int c = 0; c < max_chunks; ++c) {
                        double* po = part_o ? part_o + (orow * max_chunks + c) * D : NULL;
                        if (part_m) part_m[orow * max_chunks + c] = -INFINITY;
                        if (part_z) part_z[orow * max_chunks + c] = 0.0;
                        if (po)
                            for (int d = 0; d < D; ++d) po[d] = 0.0;
                    }
                    for (int c = 0; c < n_chunks; ++c) {
                        const int lo = c * chunk, hi = lo + chunk < n ? lo + chunk : n;
                        double mc = -INFINITY;
                        for (int i = lo; i < hi; ++i)
                            if (s[i] > mc)
                                mc = s[i];
                        if (mc > M)
                            M = mc;
                    }
                    for (int c = 0; c < n_chunks; ++c) {
                        const int lo = c * chunk, hi = lo + chunk < n ? lo + chunk : n;
                        double mc = -INFINITY, zc = 0.0;
                        for (int i = lo; i < hi; ++i)
                            if (s[i] > mc)
                                mc = s[i];
                        const double weight = exp(mc - M);
                        double* po = (part_o && c < max_chunks)
                                         ? part_o + (orow * max_chunks + c) * D
                                         : NULL;
                        for (int i = lo; i < hi; ++i) {
                            const double w = exp(s[i] - mc);
                            zc += w;
                            for (int d = 0; d < D; ++d) {
                                const double contribution = w * V[(int64_t)i * D + d];
                                acc[d] += weight * contribution;
                                if (po)
                                    po[d] += contribution;
                            }
                        }
                        Z += weight * zc;
                        if (c < max_chunks) {
                            if (part_m) part_m[orow * max_chunks + c] = mc;
                            if (part_z) part_z[orow * max_chunks + c] = zc;
                        }
                    }
                    for (int d = 0; d < D; ++d)
                        o[d] = Z != 0.0 ? acc[d] / Z : 0.0;
                }
            }
        }
        free(K); free(V); free(s); free(qrow); free(acc);
    }
    return failed ? -6 : 0;
}

int oracle_kv_append(int B, int KV, int D, int BS, int num_blocks, int NQ, int dtype,
                     void* k_pool, void* v_pool, const void* new_k, const void* new_v,
                     const int32_t* slot_mapping)
{
    if (B < 0 || KV <= 0 || D <= 0 || BS <= 0 || num_blocks < 0 || NQ < 0)
        return -1;
    if (dtype < 0 || dtype > 2)
        return -3;
    const int64_t elem = dtype == 0 ? 4 : 2;
    const int64_t row_bytes = (int64_t)KV * D * elem; /* one token: every KV head */
    const int64_t slots = (int64_t)num_blocks * BS;
    for (int b = 0; b < B; ++b) {
        for (int j = 0; j < NQ; ++j) {
            const int64_t slot = slot_mapping[(int64_t)b * NQ + j];
            if (slot < 0 || slot >= slots)
                continue;
            for (int kh = 0; kh < KV; ++kh) {
                const int64_t row = ((int64_t)b * KV + kh) * NQ + j; /* new row j of (b, kh) */
                const int64_t src = row * D * elem;
                const int64_t dst = slot * row_bytes + (int64_t)kh * D * elem;
                memcpy((char*)k_pool + dst, (const char*)new_k + src, (size_t)(D * elem));
                memcpy((char*)v_pool + dst, (const char*)new_v + src, (size_t)(D * elem));
            }
        }
    }
    return 0;
}

int oracle_paged_decode(int B, int H, int KV, int D, int BS, int max_blocks, int NQ,
                        int causal, int dtype, const void* q, const void* k_pool,
                        const void* v_pool, const int32_t* block_table,
                        const int32_t* context_lens, const void* new_k,
                        const void* new_v, float scale, double* out)
{
    return decode_impl(B, H, KV, D, BS, max_blocks, NQ, causal, dtype, q, k_pool, v_pool,
                       block_table, context_lens, new_k, new_v, scale, 0, 0, NULL, NULL,
                       NULL, out);
}

int oracle_paged_decode_partitioned(int B, int H, int KV, int D, int BS, int max_blocks,
                                    int NQ, int causal, int dtype, const void* q,
                                    const void* k_pool, const void* v_pool,
                                    const int32_t* block_table,
                                    const int32_t* context_lens, const void* new_k,
                                    const void* new_v, float scale, int chunk,
                                    int max_chunks, double* part_m, double* part_z,
                                    double* part_o, double* out)
{
    if (chunk <= 0)
        return -5;
    return decode_impl(B, H, KV, D, BS, max_blocks, NQ, causal, dtype, q, k_pool, v_pool,
                       block_table, context_lens, new_k, new_v, scale, chunk, max_chunks,
                       part_m, part_z, part_o, out);
}

/*
 * Dense GQA attention forward: the forward half of the docs.rs page
 * "onnxruntime-ep-mlx 0.31.1: src/ops/attention_vjp/dense.rs", execute() (score
 * matrix, mask bias, causal mask, softmax with empty rows set to zero; the
 * output is p V). Readings where the page leaves a step open:
 *   - the page multiplies q and k each by sqrt(scale); in exact arithmetic that
 *     is scale * <q, k>, computed here as the binary32 scale times the double
 *     dot product;
 *   - mask_kind 1 is boolean (nonzero = visible: bias 0, else -inf), 2 is an
 *     additive binary32 bias; the mask has dims [mb, mh, mq, mw], a dim of 1
 *     repeating over batch, query head, query position or key; when 1 < mw < SK
 *     keys j >= mw get -inf (the page pads the last axis with -inf);
 *   - causal: key j is visible to query i only if j <= i (the page compares the
 *     two aranges: top-left alignment).
 */
/* Mask bias of score (b, h, i, j) of the dense operation: 0 or -inf for a
 * boolean mask, the stored value for an additive one, -inf past a short mask
 * width and, when causal, for keys after the query (top-left). */
static double dense_bias(int b, int h, int i, int j, int mask_kind, const void* mask, int mb,
                         int mh, int mq, int mw, int causal)
{
    double bias = 0.0;
    if (mask_kind) {
        if (mw != 1 && j >= mw) {
            bias = -INFINITY;
        } else {
            const int64_t mi = (((int64_t)(mb == 1 ? 0 : b) * mh + (mh == 1 ? 0 : h)) * mq +
                                (mq == 1 ? 0 : i)) * mw + (mw == 1 ? 0 : j);
            if (mask_kind == 1)
                bias = ((const uint8_t*)mask)[mi] ? 0.0 : -INFINITY;
            else
                bias = (double)((const float*)mask)[mi];
        }
    }
    if (causal && j > i)
        bias = -INFINITY;
    return bias;
}

static int dense_mask_dims(int B, int HQ, int SQ, int SK, int mask_kind, const void* mask,
                           const int32_t* mask_dims, int* mb, int* mh, int* mq, int* mw)
{
    *mb = *mh = *mq = *mw = 1;
    if (!mask_kind)
        return 0;
    if (!mask || !mask_dims)
        return -7;
    *mb = mask_dims[0]; *mh = mask_dims[1]; *mq = mask_dims[2]; *mw = mask_dims[3];
    if ((*mb != 1 && *mb != B) || (*mh != 1 && *mh != HQ) || (*mq != 1 && *mq != SQ) || *mw < 1 ||
        *mw > (SK > 0 ? SK : 1))
        return -8;
    return 0;
}

int oracle_dense_attention(int B, int HQ, int HK, int SQ, int SK, int D, int dtype,
                           const void* q, const void* k, const void* v, int mask_kind,
                           const void* mask, const int32_t* mask_dims, int causal,
                           float scale, double* out)
{
    if (B < 0 || HQ <= 0 || HK <= 0 || SQ < 0 || SK < 0 || D <= 0 || HQ % HK != 0)
        return -1;
    if (dtype < 0 || dtype > 2 || mask_kind < 0 || mask_kind > 2)
        return -3;
    int mb, mh, mq, mw;
    const int mrc = dense_mask_dims(B, HQ, SQ, SK, mask_kind, mask, mask_dims, &mb, &mh, &mq, &mw);
    if (mrc)
        return mrc;
    const int G = HQ / HK;
    const double sc = (double)scale;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t row = 0; row < (int64_t)B * HQ * SQ; ++row) {
        const int b = (int)(row / ((int64_t)HQ * SQ));
        const int h = (int)(row / SQ % HQ);
        const int i = (int)(row % SQ);
        const int kh = h / G; /* query head h = kh*G + g */
        double* s = (double*)malloc(sizeof(double) * (size_t)(SK > 0 ? SK : 1));
        double* qr = (double*)malloc(sizeof(double) * (size_t)D);
        if (!s || !qr) {
#pragma omp atomic write
            failed = 1;
            free(s); free(qr);
            continue;
        }
        for (int d = 0; d < D; ++d)
            qr[d] = oracle_widen(q, row * D + d, dtype);
        double m = -INFINITY;
        for (int j = 0; j < SK; ++j) {
            const int64_t krow = ((int64_t)b * HK + kh) * SK + j;
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += qr[d] * oracle_widen(k, krow * D + d, dtype);
            s[j] = sc * dot + dense_bias(b, h, i, j, mask_kind, mask, mb, mh, mq, mw, causal);
            if (s[j] > m)
                m = s[j];
        }
        for (int d = 0; d < D; ++d)
            out[row * D + d] = 0.0;
        if (m != -INFINITY) { /* rows with every key masked stay zero */
            double z = 0.0;
            for (int j = 0; j < SK; ++j) {
                const double w = exp(s[j] - m);
                if (w == 0.0)
                    continue;
                z += w;
                const int64_t krow = ((int64_t)b * HK + kh) * SK + j;
                for (int d = 0; d < D; ++d)
                    out[row * D + d] += w * oracle_widen(v, krow * D + d, dtype);
            }
            for (int d = 0; d < D; ++d)
                out[row * D + d] /= z;
        }
        free(s); free(qr);
    }
    return failed ? -6 : 0;
}

/*
 * Dense GQA attention backward: the gradient part of execute() on the docs.rs
 * page "onnxruntime-ep-mlx 0.31.1: src/ops/attention_vjp/dense.rs". The
 * forward is recomputed exactly as oracle_dense_attention does (P, Y); then,
 * per query row, dP_j = <dY, v_j>, delta = sum_d Y_d dY_d, dS_j = P_j (dP_j -
 * delta), dQ = scale * sum_j dS_j k_j, and KV head kh collects over the G query
 * heads that read it dK_j += scale * dS_j q and dV_j += P_j dY. The page scales
 * q and k by sqrt(scale) each and multiplies the two products by sqrt(scale)
 * once more, which gives the same scale * (...) written here. Rows with every
 * key masked have P = 0 and contribute nothing. Work is split over (b, kh), so
 * each dK/dV row has one writer.
 */
int oracle_dense_attention_backward(int B, int HQ, int HK, int SQ, int SK, int D, int dtype,
                                    const void* q, const void* k, const void* v,
                                    const void* dout, int mask_kind, const void* mask,
                                    const int32_t* mask_dims, int causal, float scale,
                                    double* dq, double* dk, double* dv)
{
    if (B < 0 || HQ <= 0 || HK <= 0 || SQ < 0 || SK < 0 || D <= 0 || HQ % HK != 0)
        return -1;
    if (dtype < 0 || dtype > 2 || mask_kind < 0 || mask_kind > 2)
        return -3;
    int mb, mh, mq, mw;
    const int mrc = dense_mask_dims(B, HQ, SQ, SK, mask_kind, mask, mask_dims, &mb, &mh, &mq, &mw);
    if (mrc)
        return mrc;
    const int G = HQ / HK;
    const double sc = (double)scale;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t unit = 0; unit < (int64_t)B * HK; ++unit) {
        const int b = (int)(unit / HK), kh = (int)(unit % HK);
        const size_t nk = (size_t)(SK > 0 ? SK : 1);
        double* s = (double*)malloc(sizeof(double) * nk);    /* scores, then P */
        double* dp = (double*)malloc(sizeof(double) * nk);
        double* qr = (double*)malloc(sizeof(double) * (size_t)D);
        double* gy = (double*)malloc(sizeof(double) * (size_t)D);  /* dY row */
        double* y = (double*)malloc(sizeof(double) * (size_t)D);
        if (!s || !dp || !qr || !gy || !y) {
#pragma omp atomic write
            failed = 1;
            free(s); free(dp); free(qr); free(gy); free(y);
            continue;
        }
        const int64_t kv0 = ((int64_t)b * HK + kh) * SK; /* first key row of the unit */
        for (int64_t e = kv0 * D; e < (kv0 + SK) * D; ++e)
            dk[e] = dv[e] = 0.0;
        for (int g = 0; g < G; ++g) {
            const int h = g + kh * G; /* the G query heads that read KV head kh */
            for (int i = 0; i < SQ; ++i) {
                const int64_t row = ((int64_t)b * HQ + h) * SQ + i;
                for (int d = 0; d < D; ++d) {
                    qr[d] = oracle_widen(q, row * D + d, dtype);
                    gy[d] = oracle_widen(dout, row * D + d, dtype);
                    dq[row * D + d] = 0.0;
                }
                /* forward recompute: P (softmax of the scores) and Y */
                double m = -INFINITY;
                for (int j = 0; j < SK; ++j) {
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += qr[d] * oracle_widen(k, (kv0 + j) * D + d, dtype);
                    s[j] = sc * dot + dense_bias(b, h, i, j, mask_kind, mask, mb, mh, mq, mw, causal);
                    if (s[j] > m)
                        m = s[j];
                }
                if (m == -INFINITY)
                    continue; /* every key masked: P = 0, no gradient */
                double z = 0.0;
                for (int j = 0; j < SK; ++j) {
                    s[j] = exp(s[j] - m);
                    z += s[j];
                }
                for (int d = 0; d < D; ++d)
                    y[d] = 0.0;
                for (int j = 0; j < SK; ++j) {
                    s[j] /= z;
                    for (int d = 0; d < D; ++d)
                        y[d] += s[j] * oracle_widen(v, (kv0 + j) * D + d, dtype);
                }
                /* dP, delta, dS */
                double delta = 0.0;
                for (int d = 0; d < D; ++d)
                    delta += y[d] * gy[d];
                for (int j = 0; j < SK; ++j) {
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += gy[d] * oracle_widen(v, (kv0 + j) * D + d, dtype);
                    dp[j] = s[j] * (dot - delta); /* dS_j */
                }
                /* dQ, and this row's share of dK and dV */
                for (int j = 0; j < SK; ++j) {
                    if (s[j] == 0.0)
                        continue;
                    for (int d = 0; d < D; ++d) {
                        dq[row * D + d] += sc * dp[j] * oracle_widen(k, (kv0 + j) * D + d, dtype);
                        dk[(kv0 + j) * D + d] += sc * dp[j] * qr[d];
                        dv[(kv0 + j) * D + d] += s[j] * gy[d];
                    }
                }
            }
        }
        free(s); free(dp); free(qr); free(gy); free(y);
    }
    return failed ? -6 : 0;
}
