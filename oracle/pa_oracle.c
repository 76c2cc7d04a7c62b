/*
 * pa_oracle.c -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.
 *
 * A plain, slow, obviously-correct CPU statement, in float64, of what the paged-attention hot path
 * computes. Only the tests, the smoke check and the CPU-baseline leg of the benchmark may load it.
 * It shares no code, header, table or helper with the HIP library; the two agree only on the
 * interface facts (argument meaning and the cache layout below), each written out independently.
 *
 * Sources (a reader has the pages, so each function names the passage it follows):
 *   [MEM]  openeuler.csdn.net, "高并发 AI 服务的内存瓶颈" (memory bottleneck of high-concurrency
 *          AI serving): sections "vLLM - PagedAttention" (机制1 按需分配, 机制 2 写时复制) and
 *          "PagedAttention 在 vLLM 中的实现细节" (Block Table 数据结构; Attention 计算时的 Block 映射).
 *   [PD]   lilinji.mintlify.site lecture 32, "LLM 在线推理两阶段（Prefill vs Decode）…":
 *          §1.1 (causal factorisation), §3.1 (attention formula; decode appends k_t, v_t then
 *          attends K_{1:t}, V_{1:t}), §3.4 (GQA grouping figure), §5.4 (chunked prefill).
 *   [OV]   devpress.csdn.net/amd vLLM overview: §3 PagedAttention (3) pseudo-code (per-block
 *          accumulation over the block table), §9 FlashAttention (4) online softmax (running max
 *          and running sum of exponentials, rescaled at the end).
 *   [V1]   lilinji.mintlify.site lecture 34, "vLLM 生产级系统架构全景剖析…": §4.4 FP8 KV cache;
 *          §5.3 draft trees (EAGLE): a tree of drafted tokens is verified by the target model in
 *          one pass, each drafted token seeing the context and its own ancestors.
 *   [OFP8] the OCP 8-bit floating point specification (not one of the pages): the E4M3 format.
 *
 * Cache layout (an interface fact, fixed by the library's header, restated here on its own):
 *   k_cache, v_cache: 16-bit words, [num_blocks][num_kv_heads][16][head_dim].
 *   The token in slot s lives in physical block s/16 at in-block offset s%16 ([MEM] Block Table
 *   数据结构: position -> physical_block*block_size + offset). The pages leave the arrangement of
 *   heads inside a block open; this layout keeps each (block, kv-head) tile contiguous.
 *
 * FP8 cache variant ([V1] lecture 34 §4.4: kv_cache_dtype="fp8" stores each key and value element
 * in one E4M3 byte instead of two): caches of bytes in the same layout, each code the E4M3 value of
 * x / scale for a per-cache scale; reading multiplies the value back by the scale.
 *
 * Readings where the pages are silent (each is listed with its reason in the design notes):
 *   - seq_lens counts the token being decoded, so the decode query attends positions 0..L-1
 *     inclusive of itself ([PD] §3.1).
 *   - a prefill row at absolute position p attends keys 0..p inclusive ([PD] §1.1 causal law).
 *   - query head h reads kv head h / (H_q/H_kv): contiguous groups ([PD] §3.4 figure).
 *   - L = 0 gives a zero output row; slot < 0 means "skip this token"; copy_blocks copies the
 *     whole 16-slot block in both caches.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F16 = 0, OR_BF16 = 1 };
enum { OR_OK = 0, OR_BAD_INDEX = 1, OR_DUP_SLOT = 2, OR_BAD_MAPPING = 3, OR_BAD_ARG = 4,
       OR_NO_MEM = 5 };

#define OR_BLOCK 16

/* ---------------------------------------------------------------- O1: 16-bit -> float64 */
/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. bfloat16: the top 16 bits of an
 * IEEE binary32. Both decode exactly into a double. */
double oracle_to_double(uint16_t bits, int dtype)
{
    if (dtype == OR_BF16) {
        uint32_t u = (uint32_t)bits << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    int sign = bits >> 15;
    int e = (bits >> 10) & 0x1f;
    int m = bits & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-14 * 2^-10 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

static size_t cache_at(int blk, int kvh, int off, int d, int H_kv, int D)
{
    return (((size_t)blk * H_kv + kvh) * OR_BLOCK + off) * D + d;
}

/* ---------------------------------------------------------------- F1: E4M3 codes ([OFP8])
 * One byte: sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0. Exponent field 0 holds
 * the subnormals m * 2^-9; S.1111.111 is NaN; there are no infinities, so the largest magnitude is
 * 1.75 * 2^8 = 448 (code 0x7E). Every code decodes exactly into a double. */
double oracle_e4m3_to_double(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);                /* subnormal: (m/8) * 2^-6 */
    else
        v = ldexp((double)(8 + m), e - 10);      /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* The E4M3 code of a float: the nearest E4M3 value, a tie going to the even mantissa; magnitudes of
 * 448 and above (infinities included) saturate to 448; NaN gives the NaN code with the input's sign.
 * Below 2^-6 the grid spacing is 2^-9 (subnormals); in the binade [2^E, 2^(E+1)) it is 2^(E-3). */
uint8_t oracle_e4m3_from_float(float x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x))
        return sign | 0x7F;
    double a = fabs((double)x);
    if (a >= 448.0)
        return sign | 0x7E;
    int e;
    frexp(a, &e);                                /* a = f * 2^e, f in [0.5, 1) */
    int spacing = a < ldexp(1.0, -6) ? -9 : (e - 1) - 3;
    double n = nearbyint(ldexp(a, -spacing));    /* round half to even (default mode) */
    double v = ldexp(n, spacing);                /* the rounded magnitude, at most 448 */
    if (v == 0.0)
        return sign;
    frexp(v, &e);
    int E = e - 1;                               /* v = (1 + m/8) * 2^E, or subnormal */
    if (E < -6)
        return sign | (uint8_t)ldexp(v, 9);      /* m = v / 2^-9 */
    int m = (int)(ldexp(v, -E) * 8.0) - 8;
    return sign | (uint8_t)(((E + 7) << 3) | m);
}

/* F2: quantize one 16-bit element with a per-cache scale: the E4M3 code of x / scale, the division
 * rounded to float32 (the precision the library takes this decision in). A NaN element keeps its
 * sign in the NaN code. */
uint8_t oracle_quantize_e4m3(uint16_t bits, int dtype, float scale)
{
    float x = (float)oracle_to_double(bits, dtype);  /* exact: both formats are floats */
    if (isnan(x))
        return oracle_e4m3_from_float(x);
    float q = x / scale;
    return oracle_e4m3_from_float(q);
}

/* ---------------------------------------------------------------- O2: scatter ([PD] §3.1; [MEM])
 * For every token t with slot_mapping[t] >= 0, copy its H_kv*D key and value words into slot
 * slot_mapping[t]. A bit copy: no arithmetic on the values. Slots in one call must be distinct and
 * inside the pool, else nothing is written and an error is returned. */
int oracle_reshape_and_cache(const uint16_t *key, const uint16_t *value, uint16_t *k_cache,
                             uint16_t *v_cache, const int32_t *slot_mapping, int T,
                             int num_blocks, int H_kv, int D)
{
    if (T < 0 || num_blocks < 0 || H_kv <= 0 || D <= 0)
        return OR_BAD_ARG;
    for (int t = 0; t < T; ++t) {
        int32_t s = slot_mapping[t];
        if (s < 0)
            continue;
        if ((int64_t)s >= (int64_t)num_blocks * OR_BLOCK)
            return OR_BAD_INDEX;
        for (int u = 0; u < t; ++u)
            if (slot_mapping[u] == s)
                return OR_DUP_SLOT;
    }
    for (int t = 0; t < T; ++t) {
        int32_t s = slot_mapping[t];
        if (s < 0)
            continue;
        int blk = s / OR_BLOCK, off = s % OR_BLOCK;
        for (int g = 0; g < H_kv; ++g)
            for (int d = 0; d < D; ++d) {
                size_t src = ((size_t)t * H_kv + g) * D + d;
                k_cache[cache_at(blk, g, off, d, H_kv, D)] = key[src];
                v_cache[cache_at(blk, g, off, d, H_kv, D)] = value[src];
            }
    }
    return OR_OK;
}

/* F2 over an array of n elements (OpenMP over elements; each element is independent). */
void oracle_quantize_e4m3_n(const uint16_t *bits, long n, int dtype, float scale, uint8_t *out)
{
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (long i = 0; i < n; ++i)
        out[i] = oracle_quantize_e4m3(bits[i], dtype, scale);
}

/* F3: the scatter of O2 into E4M3 caches: the element written to the slot is the code of F2 with
 * k_scale for keys and v_scale for values ([V1] §4.4: one byte per key and value element). */
int oracle_reshape_and_cache_fp8(const uint16_t *key, const uint16_t *value, uint8_t *k_cache,
                                 uint8_t *v_cache, const int32_t *slot_mapping, int T,
                                 int num_blocks, int H_kv, int D, int dtype, float k_scale,
                                 float v_scale)
{
    if (T < 0 || num_blocks < 0 || H_kv <= 0 || D <= 0 || !(k_scale > 0) || !(v_scale > 0))
        return OR_BAD_ARG;
    for (int t = 0; t < T; ++t) {
        int32_t s = slot_mapping[t];
        if (s < 0)
            continue;
        if ((int64_t)s >= (int64_t)num_blocks * OR_BLOCK)
            return OR_BAD_INDEX;
        for (int u = 0; u < t; ++u)
            if (slot_mapping[u] == s)
                return OR_DUP_SLOT;
    }
    for (int t = 0; t < T; ++t) {
        int32_t s = slot_mapping[t];
        if (s < 0)
            continue;
        int blk = s / OR_BLOCK, off = s % OR_BLOCK;
        for (int g = 0; g < H_kv; ++g)
            for (int d = 0; d < D; ++d) {
                size_t src = ((size_t)t * H_kv + g) * D + d;
                k_cache[cache_at(blk, g, off, d, H_kv, D)] = oracle_quantize_e4m3(key[src], dtype, k_scale);
                v_cache[cache_at(blk, g, off, d, H_kv, D)] = oracle_quantize_e4m3(value[src], dtype, v_scale);
            }
    }
    return OR_OK;
}

/* ---------------------------------------------------------------- O3: copy-on-write ([MEM] 机制 2)
 * For each (src, dst) pair copy the whole physical block -- all 16 slots, all kv heads -- in both
 * caches. Destinations must be distinct and no destination may also be a source, so the result does
 * not depend on the order of the pairs. */
int oracle_copy_blocks(uint16_t *k_cache, uint16_t *v_cache, const int32_t *mapping, int n,
                       int num_blocks, int H_kv, int D)
{
    if (n < 0 || num_blocks < 0 || H_kv <= 0 || D <= 0)
        return OR_BAD_ARG;
    for (int i = 0; i < n; ++i) {
        int32_t s = mapping[2 * i], d = mapping[2 * i + 1];
        if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks)
            return OR_BAD_INDEX;
        for (int j = 0; j < n; ++j) {
            if (j != i && mapping[2 * j + 1] == d)
                return OR_BAD_MAPPING;
            if (mapping[2 * j] == d)
                return OR_BAD_MAPPING;
        }
    }
    for (int i = 0; i < n; ++i) {
        int32_t s = mapping[2 * i], d = mapping[2 * i + 1];
        for (int g = 0; g < H_kv; ++g)
            for (int off = 0; off < OR_BLOCK; ++off)
                for (int e = 0; e < D; ++e) {
                    k_cache[cache_at(d, g, off, e, H_kv, D)] = k_cache[cache_at(s, g, off, e, H_kv, D)];
                    v_cache[cache_at(d, g, off, e, H_kv, D)] = v_cache[cache_at(s, g, off, e, H_kv, D)];
                }
    }
    return OR_OK;
}

/* F4: O3 on E4M3 caches (one byte per element): the same whole-block copies. */
int oracle_copy_blocks_fp8(uint8_t *k_cache, uint8_t *v_cache, const int32_t *mapping, int n,
                           int num_blocks, int H_kv, int D)
{
    if (n < 0 || num_blocks < 0 || H_kv <= 0 || D <= 0)
        return OR_BAD_ARG;
    for (int i = 0; i < n; ++i) {
        int32_t s = mapping[2 * i], d = mapping[2 * i + 1];
        if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks)
            return OR_BAD_INDEX;
        for (int j = 0; j < n; ++j) {
            if (j != i && mapping[2 * j + 1] == d)
                return OR_BAD_MAPPING;
            if (mapping[2 * j] == d)
                return OR_BAD_MAPPING;
        }
    }
    for (int i = 0; i < n; ++i) {
        int32_t s = mapping[2 * i], d = mapping[2 * i + 1];
        for (int g = 0; g < H_kv; ++g)
            for (int off = 0; off < OR_BLOCK; ++off)
                for (int e = 0; e < D; ++e) {
                    k_cache[cache_at(d, g, off, e, H_kv, D)] = k_cache[cache_at(s, g, off, e, H_kv, D)];
                    v_cache[cache_at(d, g, off, e, H_kv, D)] = v_cache[cache_at(s, g, off, e, H_kv, D)];
                }
    }
    return OR_OK;
}

/* ---------------------------------------------------------------- O4: gather ([MEM] Block 映射)
 * Rebuild the logically contiguous rows 0..L-1 of kv head `kvh` of one sequence: position i sits in
 * logical block i/16 at offset i%16, and the table maps the logical block to a physical one. */
int oracle_gather(const uint16_t *cache, const int32_t *table_row, int L, int kvh, int num_blocks,
                  int H_kv, int D, int dtype, double *out)
{
    for (int i = 0; i < L; ++i) {
        int32_t blk = table_row[i / OR_BLOCK];
        if (blk < 0 || blk >= num_blocks)
            return OR_BAD_INDEX;
        for (int d = 0; d < D; ++d)
            out[(size_t)i * D + d] = oracle_to_double(cache[cache_at(blk, kvh, i % OR_BLOCK, d, H_kv, D)], dtype);
    }
    return OR_OK;
}

/* F5: O4 on an E4M3 cache: each element is its code's value times the cache's scale (exact in
 * double: at most 4 significant bits times a float). */
int oracle_gather_fp8(const uint8_t *cache, const int32_t *table_row, int L, int kvh,
                      int num_blocks, int H_kv, int D, double cache_scale, double *out)
{
    for (int i = 0; i < L; ++i) {
        int32_t blk = table_row[i / OR_BLOCK];
        if (blk < 0 || blk >= num_blocks)
            return OR_BAD_INDEX;
        for (int d = 0; d < D; ++d)
            out[(size_t)i * D + d] =
                oracle_e4m3_to_double(cache[cache_at(blk, kvh, i % OR_BLOCK, d, H_kv, D)]) * cache_scale;
    }
    return OR_OK;
}

/* ---------------------------------------------------------------- O5: attention ([PD] §3.1)
 * out = softmax(scale * q K^T) V over the L rows of K and V, written out as its definition in two
 * passes: scores, their maximum, the exponentials, their sum, the weighted sum of rows. The maximum
 * is subtracted only to keep exp() finite; it cancels exactly in the ratio. L = 0 gives zeros. */
int oracle_attention(const double *q, const double *K, const double *V, int L, int D,
                     double scale, double *out)
{
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    if (L <= 0)
        return OR_OK;
    double *w = (double *)malloc(sizeof(double) * (size_t)L);
    if (!w)
        return OR_NO_MEM;
    double m = -INFINITY;
    for (int j = 0; j < L; ++j) {
        double s = 0.0;
        for (int d = 0; d < D; ++d)
            s += q[d] * K[(size_t)j * D + d];
        w[j] = scale * s;
        if (w[j] > m)
            m = w[j];
    }
    double Z = 0.0;
    for (int j = 0; j < L; ++j) {
        w[j] = exp(w[j] - m);
        Z += w[j];
    }
    for (int j = 0; j < L; ++j)
        for (int d = 0; d < D; ++d)
            out[d] += w[j] * V[(size_t)j * D + d];
    for (int d = 0; d < D; ++d)
        out[d] /= Z;
    free(w);
    return OR_OK;
}

/* ---------------------------------------------------------------- O6: paged decode
 * For sequence s and query head h: gather rows 0..seq_lens[s]-1 of kv head h/(H_q/H_kv) through the
 * block table ([MEM] Block 映射, [PD] §3.4) and apply O5 to query row q[s][h] ([PD] §3.1).
 * `pairs` lists the (s, h) pairs to evaluate ([n_pairs][2]); NULL means every pair in order.
 * out is [n_pairs][D] (or [B][H_q][D] when pairs is NULL). With fp8 set the caches hold E4M3 codes
 * read through F5 with k_scale and v_scale; otherwise 16-bit words of `dtype`. */
static int gather_kv(const void *cache, int fp8, double cache_scale, const int32_t *row, int L,
                     int kvh, int num_blocks, int H_kv, int D, int dtype, double *out)
{
    if (fp8)
        return oracle_gather_fp8((const uint8_t *)cache, row, L, kvh, num_blocks, H_kv, D,
                                 cache_scale, out);
    return oracle_gather((const uint16_t *)cache, row, L, kvh, num_blocks, H_kv, D, dtype, out);
}

/* The attention outputs one call evaluates: output row `out` is O5 of query row `qrow`, head `h`,
 * over rows 0..L-1 of the gathered K and V of (sequence s, kv head g). */
typedef struct {
    int s, g, L, qrow, h;
    long out;
} or_item;

static int item_order(const void *a, const void *b)
{
    const or_item *x = (const or_item *)a, *y = (const or_item *)b;
    if (x->s != y->s)
        return x->s < y->s ? -1 : 1;
    if (x->g != y->g)
        return x->g < y->g ? -1 : 1;
    return (x->out > y->out) - (x->out < y->out);
}

/* Evaluate the items. Items of one (s, g) read the same gathered rows (O4 is exact, so gathering
 * them once and letting each item read its leading L rows gives the very doubles a per-item gather
 * would), so they are sorted by (s, g) and the gathers of a batch of keys, at most about 256 MB of
 * doubles unless one key alone is larger, are made once before its items are evaluated. */
static int run_items(or_item *it, long n, const uint16_t *query, int H_q, const void *k_cache,
                     const void *v_cache, int fp8, double k_scale, double v_scale,
                     const int32_t *block_tables, int max_blocks, int num_blocks, int H_kv, int D,
                     int dtype, double scale, int nthreads, double *out)
{
    const size_t budget = (size_t)32 << 20; /* doubles of K plus V per batch */
    int status = OR_OK;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
    qsort(it, (size_t)n, sizeof(or_item), item_order);
    long i0 = 0;
    while (i0 < n) {
        /* keys of this batch: [k0, k1) in the list of distinct (s, g) starting at item i0 */
        long *first = NULL;
        int nk = 0, cap = 0;
        size_t used = 0;
        long i = i0;
        while (i < n) {
            long j = i;
            int L = 0;
            while (j < n && it[j].s == it[i].s && it[j].g == it[i].g) {
                if (it[j].L > L)
                    L = it[j].L;
                ++j;
            }
            size_t need = (size_t)2 * (size_t)L * D;
            if (nk > 0 && used + need > budget)
                break;
            if (nk == cap) {
                cap = cap ? 2 * cap : 64;
                long *nf = (long *)realloc(first, sizeof(long) * (size_t)(cap + 1));
                if (!nf) {
                    free(first);
                    return OR_NO_MEM;
                }
                first = nf;
            }
            first[nk++] = i;
            used += need;
            i = j;
        }
        first[nk] = i; /* end of the batch's items */
        double **K = (double **)calloc((size_t)nk, sizeof(double *));
        double **V = (double **)calloc((size_t)nk, sizeof(double *));
        int *krc = (int *)calloc((size_t)nk, sizeof(int));
        if (!K || !V || !krc) {
            free(K);
            free(V);
            free(krc);
            free(first);
            return OR_NO_MEM;
        }
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
        for (int k = 0; k < nk; ++k) {
            const or_item *head = &it[first[k]];
            int L = 0;
            for (long j = first[k]; j < first[k + 1]; ++j)
                if (it[j].L > L)
                    L = it[j].L;
            K[k] = (double *)malloc(sizeof(double) * ((size_t)L * D + 1));
            V[k] = (double *)malloc(sizeof(double) * ((size_t)L * D + 1));
            if (!K[k] || !V[k]) {
                krc[k] = OR_NO_MEM;
                continue;
            }
            const int32_t *row = block_tables + (size_t)head->s * max_blocks;
            krc[k] = gather_kv(k_cache, fp8, k_scale, row, L, head->g, num_blocks, H_kv, D, dtype,
                               K[k]);
            if (krc[k] == OR_OK)
                krc[k] = gather_kv(v_cache, fp8, v_scale, row, L, head->g, num_blocks, H_kv, D,
                                   dtype, V[k]);
        }
        const long nb = first[nk] - i0;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
        for (long jj = 0; jj < nb; ++jj) {
            const long j = i0 + jj;
            int lo = 0, hi = nk - 1; /* the key whose items [first[k], first[k+1]) hold j */
            while (lo < hi) {
                int mid = (lo + hi + 1) / 2;
                if (first[mid] <= j)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            const int k = lo;
            int rc = krc[k];
            if (rc == OR_OK) {
                double *q = (double *)malloc(sizeof(double) * (size_t)D);
                if (!q) {
                    rc = OR_NO_MEM;
                } else {
                    for (int d = 0; d < D; ++d)
                        q[d] = oracle_to_double(query[((size_t)it[j].qrow * H_q + it[j].h) * D + d],
                                                dtype);
                    rc = oracle_attention(q, K[k], V[k], it[j].L, D, scale,
                                          out + (size_t)it[j].out * D);
                    free(q);
                }
            }
            if (rc != OR_OK) {
#ifdef _OPENMP
#pragma omp critical
#endif
                status = rc;
            }
        }
        for (int k = 0; k < nk; ++k) {
            free(K[k]);
            free(V[k]);
        }
        free(K);
        free(V);
        free(krc);
        i0 = first[nk];
        free(first);
    }
    return status;
}

static int decode_pairs(const uint16_t *query, const void *k_cache, const void *v_cache, int fp8,
                        double k_scale, double v_scale, const int32_t *block_tables,
                        int max_blocks, const int32_t *seq_lens, int B, int H_q, int H_kv, int D,
                        int num_blocks, int dtype, double scale, const int32_t *pairs,
                        int n_pairs, int nthreads, double *out)
{
    if (B < 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv || D <= 0)
        return OR_BAD_ARG;
    long n = pairs ? n_pairs : (long)B * H_q;
    int group = H_q / H_kv;
    or_item *it = (or_item *)malloc(sizeof(or_item) * (size_t)(n + 1));
    if (!it)
        return OR_NO_MEM;
    for (long i = 0; i < n; ++i) {
        int s = pairs ? pairs[2 * i] : (int)(i / H_q);
        int h = pairs ? pairs[2 * i + 1] : (int)(i % H_q);
        if (s < 0 || s >= B || h < 0 || h >= H_q) {
            free(it);
            return OR_BAD_ARG;
        }
        int L = seq_lens[s];
        if (L < 0 || L > max_blocks * OR_BLOCK) {
            free(it);
            return OR_BAD_INDEX;
        }
        it[i].s = s;
        it[i].g = h / group;
        it[i].L = L;
        it[i].qrow = s;
        it[i].h = h;
        it[i].out = i;
    }
    int rc = run_items(it, n, query, H_q, k_cache, v_cache, fp8, k_scale, v_scale, block_tables,
                       max_blocks, num_blocks, H_kv, D, dtype, scale, nthreads, out);
    free(it);
    return rc;
}

int oracle_decode(const uint16_t *query, const uint16_t *k_cache, const uint16_t *v_cache,
                  const int32_t *block_tables, int max_blocks, const int32_t *seq_lens, int B,
                  int H_q, int H_kv, int D, int num_blocks, int dtype, double scale,
                  const int32_t *pairs, int n_pairs, int nthreads, double *out)
{
    return decode_pairs(query, k_cache, v_cache, 0, 1.0, 1.0, block_tables, max_blocks, seq_lens,
                        B, H_q, H_kv, D, num_blocks, dtype, scale, pairs, n_pairs, nthreads, out);
}

/* F6: O6 over E4M3 caches ([V1] §4.4); query and output stay in `dtype`. */
int oracle_decode_fp8(const uint16_t *query, const uint8_t *k_cache, const uint8_t *v_cache,
                      const int32_t *block_tables, int max_blocks, const int32_t *seq_lens, int B,
                      int H_q, int H_kv, int D, int num_blocks, int dtype, double scale,
                      double k_scale, double v_scale, const int32_t *pairs, int n_pairs,
                      int nthreads, double *out)
{
    if (!(k_scale > 0) || !(v_scale > 0))
        return OR_BAD_ARG;
    return decode_pairs(query, k_cache, v_cache, 1, k_scale, v_scale, block_tables, max_blocks,
                        seq_lens, B, H_q, H_kv, D, num_blocks, dtype, scale, pairs, n_pairs,
                        nthreads, out);
}

/* ---------------------------------------------------------------- O7: paged causal prefill chunk
 * Sequence s owns query rows cu_q_lens[s] .. cu_q_lens[s+1]-1: the last q_len tokens of its
 * seq_lens[s] tokens ([PD] §5.4: a chunk attends the cached context plus the earlier part of
 * itself). Row i of the chunk sits at absolute position p = seq_lens[s] - q_len + i and attends
 * keys 0..p ([PD] §1.1). `rows` lists (row, head) pairs ([n_rows][2]); NULL means every
 * (row, head) in order. out is [n_rows][D] (or [total_q][H_q][D]). */
static int prefill_rows(const uint16_t *query, const void *k_cache, const void *v_cache, int fp8,
                        double k_scale, double v_scale, const int32_t *block_tables,
                        int max_blocks, const int32_t *seq_lens, const int32_t *cu_q_lens, int S,
                        int H_q, int H_kv, int D, int num_blocks, int dtype, double scale,
                        const int32_t *rows, int n_rows, int nthreads, double *out)
{
    if (S < 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv || D <= 0)
        return OR_BAD_ARG;
    int total_q = cu_q_lens[S];
    long n = rows ? n_rows : (long)total_q * H_q;
    int group = H_q / H_kv;
    or_item *it = (or_item *)malloc(sizeof(or_item) * (size_t)(n + 1));
    if (!it)
        return OR_NO_MEM;
    for (long i = 0; i < n; ++i) {
        int r = rows ? rows[2 * i] : (int)(i / H_q);
        int h = rows ? rows[2 * i + 1] : (int)(i % H_q);
        int s = -1;
        for (int j = 0; j < S; ++j)
            if (cu_q_lens[j] <= r && r < cu_q_lens[j + 1])
                s = j;
        if (s < 0 || h < 0 || h >= H_q) {
            free(it);
            return OR_BAD_ARG;
        }
        int q_len = cu_q_lens[s + 1] - cu_q_lens[s];
        int p = seq_lens[s] - q_len + (r - cu_q_lens[s]);
        if (p < 0 || seq_lens[s] > max_blocks * OR_BLOCK) {
            free(it);
            return OR_BAD_INDEX;
        }
        it[i].s = s;
        it[i].g = h / group;
        it[i].L = p + 1; /* the row attends positions 0..p */
        it[i].qrow = r;
        it[i].h = h;
        it[i].out = i;
    }
    int rc = run_items(it, n, query, H_q, k_cache, v_cache, fp8, k_scale, v_scale, block_tables,
                       max_blocks, num_blocks, H_kv, D, dtype, scale, nthreads, out);
    free(it);
    return rc;
}

int oracle_prefill(const uint16_t *query, const uint16_t *k_cache, const uint16_t *v_cache,
                   const int32_t *block_tables, int max_blocks, const int32_t *seq_lens,
                   const int32_t *cu_q_lens, int S, int H_q, int H_kv, int D, int num_blocks,
                   int dtype, double scale, const int32_t *rows, int n_rows, int nthreads,
                   double *out)
{
    return prefill_rows(query, k_cache, v_cache, 0, 1.0, 1.0, block_tables, max_blocks, seq_lens,
                        cu_q_lens, S, H_q, H_kv, D, num_blocks, dtype, scale, rows, n_rows,
                        nthreads, out);
}

/* F7: O7 over E4M3 caches ([V1] §4.4): the gathered rows are code value x k_scale / v_scale (F5),
 * the queries 16-bit words of dtype. */
int oracle_prefill_fp8(const uint16_t *query, const uint8_t *k_cache, const uint8_t *v_cache,
                       const int32_t *block_tables, int max_blocks, const int32_t *seq_lens,
                       const int32_t *cu_q_lens, int S, int H_q, int H_kv, int D, int num_blocks,
                       int dtype, double scale, double k_scale, double v_scale,
                       const int32_t *rows, int n_rows, int nthreads, double *out)
{
    if (!(k_scale > 0) || !(v_scale > 0))
        return OR_BAD_ARG;
    return prefill_rows(query, k_cache, v_cache, 1, k_scale, v_scale, block_tables, max_blocks,
                        seq_lens, cu_q_lens, S, H_q, H_kv, D, num_blocks, dtype, scale, rows,
                        n_rows, nthreads, out);
}


/* ---------------------------------------------------------------- T1: tree-masked prefill */
/* [V1] §5.3 (a draft tree checked in one target pass) with [PD] §5.4 (k drafted tokens verified
 * together): the q_len rows of sequence s are the drafted tokens at positions first .. L-1,
 * first = L - q_len, and row i sees every context position 0..first-1 plus chunk row j (position
 * first + j) exactly when j <= i and bit j of tree_mask[cu_q_lens[s] + i] is set. The visible rows
 * are gathered in position order and given to O5. q_len <= 64 (one 64-bit mask per row). */
int oracle_prefill_tree(const uint16_t *query, const uint16_t *k_cache, const uint16_t *v_cache,
                        const int32_t *block_tables, int max_blocks, const int32_t *seq_lens,
                        const int32_t *cu_q_lens, const uint64_t *tree_mask, int S, int H_q,
                        int H_kv, int D, int num_blocks, int dtype, double scale, int nthreads,
                        double *out)
{
    if (S < 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv || D <= 0)
        return OR_BAD_ARG;
    for (int s = 0; s < S; ++s)
        if (cu_q_lens[s + 1] - cu_q_lens[s] > 64 || cu_q_lens[s + 1] < cu_q_lens[s])
            return OR_BAD_ARG;
    int total_q = cu_q_lens[S];
    int n = total_q * H_q;
    int group = H_q / H_kv;
    int status = OR_OK;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int idx = 0; idx < n; ++idx) {
        int r = idx / H_q, h = idx % H_q;
        int rc = OR_OK;
        int s = -1;
        for (int j = 0; j < S; ++j)
            if (cu_q_lens[j] <= r && r < cu_q_lens[j + 1])
                s = j;
        int q_len = cu_q_lens[s + 1] - cu_q_lens[s];
        int i = r - cu_q_lens[s];
        int first = seq_lens[s] - q_len;
        int p = first + i;
        if (first < 0 || seq_lens[s] > max_blocks * OR_BLOCK) {
            rc = OR_BAD_INDEX;
        } else {
            int L = p + 1;
            double *K = (double *)malloc(sizeof(double) * (size_t)L * D);
            double *V = (double *)malloc(sizeof(double) * (size_t)L * D);
            double *q = (double *)malloc(sizeof(double) * (size_t)D);
            if (!K || !V || !q) {
                rc = OR_NO_MEM;
            } else {
                const int32_t *row = block_tables + (size_t)s * max_blocks;
                rc = oracle_gather(k_cache, row, L, h / group, num_blocks, H_kv, D, dtype, K);
                if (rc == OR_OK)
                    rc = oracle_gather(v_cache, row, L, h / group, num_blocks, H_kv, D, dtype, V);
                /* keep the visible positions, in order */
                int kept = 0;
                for (int pos = 0; rc == OR_OK && pos < L; ++pos) {
                    int j = pos - first;
                    int visible = j < 0 || ((tree_mask[r] >> j) & 1u);
                    if (!visible)
                        continue;
                    memmove(K + (size_t)kept * D, K + (size_t)pos * D, sizeof(double) * D);
                    memmove(V + (size_t)kept * D, V + (size_t)pos * D, sizeof(double) * D);
                    ++kept;
                }
                for (int d = 0; d < D; ++d)
                    q[d] = oracle_to_double(query[((size_t)r * H_q + h) * D + d], dtype);
                if (rc == OR_OK)
                    rc = oracle_attention(q, K, V, kept, D, scale, out + (size_t)idx * D);
            }
            free(K);
            free(V);
            free(q);
        }
        if (rc != OR_OK) {
#ifdef _OPENMP
#pragma omp critical
#endif
            status = rc;
        }
    }
    return status;
}

/* ---------------------------------------------------------------- O8: split-and-merge ([OV] §9 (4))
 * Cut the L rows into consecutive parts of `part` rows. Each part keeps its own running maximum m_p,
 * its sum of exponentials Z_p = sum exp(s_j - m_p) and its normalised output o_p; the parts are then
 * combined by rescaling every part to the global maximum M:
 *   out = sum_p exp(m_p - M) Z_p o_p / sum_p exp(m_p - M) Z_p.
 * This is the merge the split-K decode uses; it equals O5 up to rounding. */
int oracle_split_merge(const double *q, const double *K, const double *V, int L, int D,
                       double scale, int part, double *out)
{
    if (part <= 0 || L < 0 || D <= 0)
        return OR_BAD_ARG;
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    if (L == 0)
        return OR_OK;
    int np = (L + part - 1) / part;
    double *m = (double *)malloc(sizeof(double) * np);
    double *Z = (double *)malloc(sizeof(double) * np);
    double *o = (double *)malloc(sizeof(double) * (size_t)np * D);
    double *w = (double *)malloc(sizeof(double) * part);
    if (!m || !Z || !o || !w) {
        free(m); free(Z); free(o); free(w);
        return OR_NO_MEM;
    }
    for (int p = 0; p < np; ++p) {
        int a = p * part, b = a + part < L ? a + part : L;
        m[p] = -INFINITY;
        for (int j = a; j < b; ++j) {
            double s = 0.0;
            for (int d = 0; d < D; ++d)
                s += q[d] * K[(size_t)j * D + d];
            w[j - a] = scale * s;
            if (w[j - a] > m[p])
                m[p] = w[j - a];
        }
        Z[p] = 0.0;
        for (int d = 0; d < D; ++d)
            o[(size_t)p * D + d] = 0.0;
        for (int j = a; j < b; ++j) {
            double e = exp(w[j - a] - m[p]);
            Z[p] += e;
            for (int d = 0; d < D; ++d)
                o[(size_t)p * D + d] += e * V[(size_t)j * D + d];
        }
        for (int d = 0; d < D; ++d)
            o[(size_t)p * D + d] /= Z[p];
    }
    double M = -INFINITY;
    for (int p = 0; p < np; ++p)
        if (m[p] > M)
            M = m[p];
    double W = 0.0;
    for (int p = 0; p < np; ++p) {
        double wp = exp(m[p] - M) * Z[p];
        W += wp;
        for (int d = 0; d < D; ++d)
            out[d] += wp * o[(size_t)p * D + d];
    }
    for (int d = 0; d < D; ++d)
        out[d] /= W;
    free(m); free(Z); free(o); free(w);
    return OR_OK;
}

/* ---------------------------------------------------------------- test helper: poison free slots
 * Overwrite every slot of both caches that holds no valid token -- no sequence s has a position
 * i < seq_lens[s] mapped to it by its table -- with the element `pattern` (a NaN code for the
 * cache's element type). Attention must never read such a slot, so a kernel that does turns a finite
 * result into NaN. Returns the number of poisoned slots, or -1 on a bad table entry. */
static long poison_slots(void *k_cache, void *v_cache, int esize, unsigned pattern,
                         const int32_t *block_tables, int max_blocks, const int32_t *seq_lens,
                         int S, int num_blocks, int H_kv, int D)
{
    unsigned char *used = (unsigned char *)calloc((size_t)num_blocks * OR_BLOCK, 1);
    if (!used)
        return -1;
    for (int s = 0; s < S; ++s)
        for (int i = 0; i < seq_lens[s]; ++i) {
            int32_t blk = block_tables[(size_t)s * max_blocks + i / OR_BLOCK];
            if (blk < 0 || blk >= num_blocks) {
                free(used);
                return -1;
            }
            used[(size_t)blk * OR_BLOCK + i % OR_BLOCK] = 1;
        }
    long count = 0;
    for (int blk = 0; blk < num_blocks; ++blk)
        for (int off = 0; off < OR_BLOCK; ++off) {
            if (used[(size_t)blk * OR_BLOCK + off])
                continue;
            ++count;
            for (int g = 0; g < H_kv; ++g)
                for (int d = 0; d < D; ++d) {
                    size_t at = cache_at(blk, g, off, d, H_kv, D);
                    if (esize == 2) {
                        ((uint16_t *)k_cache)[at] = (uint16_t)pattern;
                        ((uint16_t *)v_cache)[at] = (uint16_t)pattern;
                    } else {
                        ((uint8_t *)k_cache)[at] = (uint8_t)pattern;
                        ((uint8_t *)v_cache)[at] = (uint8_t)pattern;
                    }
                }
        }
    free(used);
    return count;
}

long oracle_poison_free_slots(uint16_t *k_cache, uint16_t *v_cache, const int32_t *block_tables,
                              int max_blocks, const int32_t *seq_lens, int S, int num_blocks,
                              int H_kv, int D, uint16_t pattern)
{
    return poison_slots(k_cache, v_cache, 2, pattern, block_tables, max_blocks, seq_lens, S,
                        num_blocks, H_kv, D);
}

long oracle_poison_free_slots_fp8(uint8_t *k_cache, uint8_t *v_cache, const int32_t *block_tables,
                                  int max_blocks, const int32_t *seq_lens, int S, int num_blocks,
                                  int H_kv, int D, uint8_t pattern)
{
    return poison_slots(k_cache, v_cache, 1, pattern, block_tables, max_blocks, seq_lens, S,
                        num_blocks, H_kv, D);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
