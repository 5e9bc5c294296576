/*
 * Paged-attention decode oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * CPU definition that the GPU library is checked against.  Only the test
 * suite, the smoke check and the CPU-baseline leg of the benchmark load it.
 * It shares no code, header, table or helper with the GPU library, and the
 * GPU library never loads it.
 *
 * Sources (web pages), cited by title and section:
 *   [10x]  "vLLM推理加速深度解读：PagedAttention如何提升10x吞吐量"
 *          §2.1  attention equation  Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V
 *          §2.3  paged equations     Attention(Q,K_paged,V_paged) = softmax(Q K_paged^T / sqrt(d_k)) V_paged
 *                                    K_paged[i] = K_physical[BlockTable[i / B]][i mod B]
 *          §4.2  cache layout in the kernel sketch: K_cache, V_cache are
 *                [num_blocks, block_size, num_heads, head_size]; Q and the
 *                output are [num_heads, head_size] per sequence
 *          §3.3  FP8 quantisation is listed among the later optimisations; the
 *                format is not given: we use OCP FP8 E4M3 with one scale per
 *                cache (see the FP8 section below)
 *   [eng]  "深入解析LLM推理引擎：从PagedAttention到调度优化"
 *          §3.2  block table worked example (block size 4, table [0, 1, 3, ...])
 *          §3.3  the gather is driven by block_table and current_position
 *   [arch] "vLLM基础架构：核心组件、PagedAttention原理、KV Cache管理与连续批处理机制"
 *          §2.3  shared blocks are copied before a sequence writes into one
 *                (copy-on-write), then its table points at the copy
 *          §4.3  prefill and decode requests may share one batch
 *   [eng]  §4.2 a batch mixes requests in prefill with requests in decode
 *   [src]  "【硬核】啃透vLLM源码：从PagedAttention到连续批处理，大模型推理加速24倍的秘密"
 *          §三   blocks are swapped out to host memory and back in
 *
 * Arithmetic: every fp16 value is decoded exactly to double (IEEE-754
 * binary16 definition, written out below) and all arithmetic is in double.
 * The softmax is the two-pass stable form: subtract the maximum logit,
 * exponentiate, normalise.  Sums run in logical token order.
 *
 * Readings where the pages are silent:
 *   - scale is an argument (the configurations pass 1/sqrt(head_dim));
 *   - only logical positions 0 .. context_len-1 are attended;
 *   - context_len == 0 gives an all-zero output;
 *   - a slot (reshape_and_cache) is physical_block * block_size + offset;
 *     slots outside [0, num_blocks*block_size) are not written.
 *
 * Parity pins for every function here live in the CPU test suite; there is
 * no "parity unpinned" function in this file.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_ERR_ARG (-1)
#define OR_ERR_RANGE (-2)
#define OR_ERR_NOMEM (-3)

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0: subnormal, value = fraction * 2^-24; exponent 31: Inf / NaN;
 * otherwise value = (1024 + fraction) * 2^(exponent - 25). */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

/* Decode n binary16 values (used by the exhaustive decoder pin). */
void oracle_half_array_to_double(const uint16_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = oracle_half_to_double(src[i]);
}

/* Element (block, offset, head, d) of a [num_blocks, block_size, num_heads,
 * head_dim] cache ([10x] §4.2). */
static size_t cache_index(int64_t block, int64_t offset, int64_t head, int64_t d,
                          int64_t block_size, int64_t num_heads, int64_t head_dim)
{
    return (size_t)(((block * block_size + offset) * num_heads + head) * head_dim + d);
}

/*
 * The paged gather of [10x] §2.3: for logical position i of sequence s,
 * K_paged[i] = K_physical[BlockTable[i / B]][i mod B], and the same for V.
 * Writes the contiguous K_paged, V_paged rows of head h, shape
 * [context_len, head_dim], as doubles.  Returns the number of rows, or a
 * negative code when a table entry or the context length is out of range.
 */
int oracle_gather(double *k_out, double *v_out,
                  const uint16_t *k_cache, const uint16_t *v_cache,
                  const int32_t *block_tables, const int32_t *context_lens,
                  int32_t seq, int32_t head,
                  int32_t num_heads, int32_t head_dim, int32_t num_blocks,
                  int32_t block_size, int32_t max_blocks_per_seq)
{
    int32_t L = context_lens[seq];
    if (L < 0 || (int64_t)L > (int64_t)max_blocks_per_seq * block_size)
        return OR_ERR_RANGE;
    for (int32_t i = 0; i < L; ++i) {
        int32_t logical_block = i / block_size;
        int32_t offset = i % block_size;
        int32_t physical = block_tables[(int64_t)seq * max_blocks_per_seq + logical_block];
        if (physical < 0 || physical >= num_blocks)
            return OR_ERR_RANGE;
        for (int32_t d = 0; d < head_dim; ++d) {
            size_t src = cache_index(physical, offset, head, d, block_size, num_heads, head_dim);
            k_out[(int64_t)i * head_dim + d] = oracle_half_to_double(k_cache[src]);
            v_out[(int64_t)i * head_dim + d] = oracle_half_to_double(v_cache[src]);
        }
    }
    return L;
}

/*
 * softmax(q K^T * scale) V for one query row against L contiguous key/value
 * rows ([10x] §2.1 with 1/sqrt(d_k) passed in as scale).  Two-pass stable
 * softmax; out has head_dim entries.  L == 0 gives zeros.
 */
static void attend_contiguous(double *out, const double *q, const double *K, const double *V,
                              int32_t L, int32_t head_dim, double scale, double *logits)
{
    for (int32_t d = 0; d < head_dim; ++d)
        out[d] = 0.0;
    if (L == 0)
        return;
    for (int32_t i = 0; i < L; ++i) {
        double dot = 0.0;
        for (int32_t d = 0; d < head_dim; ++d)
            dot += q[d] * K[(int64_t)i * head_dim + d];
        logits[i] = dot * scale;
    }
    double m = logits[0];
    for (int32_t i = 1; i < L; ++i)
        if (logits[i] > m)
            m = logits[i];
    double Z = 0.0;
    for (int32_t i = 0; i < L; ++i) {
        logits[i] = exp(logits[i] - m);
        Z += logits[i];
    }
    for (int32_t i = 0; i < L; ++i) {
        double w = logits[i] / Z;
        for (int32_t d = 0; d < head_dim; ++d)
            out[d] += w * V[(int64_t)i * head_dim + d];
    }
}

/* The query row of (s, h) from q [num_seqs, num_heads, head_dim], decoded. */
static void load_query(double *qbuf, const uint16_t *q, int32_t s, int32_t h, int32_t num_heads,
                       int32_t head_dim)
{
    const uint16_t *qrow = q + ((int64_t)s * num_heads + h) * head_dim;
    for (int32_t d = 0; d < head_dim; ++d)
        qbuf[d] = oracle_half_to_double(qrow[d]);
}

/* One (sequence, head): gather, then attend.  Scratch buffers are owned by
 * the caller (one set per thread). */
static int decode_one(double *out, const uint16_t *q,
                      const uint16_t *k_cache, const uint16_t *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens,
                      int32_t s, int32_t h,
                      int32_t num_heads, int32_t head_dim, int32_t num_blocks,
                      int32_t block_size, int32_t max_blocks_per_seq, double scale,
                      double *Kbuf, double *Vbuf, double *qbuf, double *logits)
{
    int L = oracle_gather(Kbuf, Vbuf, k_cache, v_cache, block_tables, context_lens, s, h,
                          num_heads, head_dim, num_blocks, block_size, max_blocks_per_seq);
    if (L < 0)
        return L;
    load_query(qbuf, q, s, h, num_heads, head_dim);
    attend_contiguous(out, qbuf, Kbuf, Vbuf, L, head_dim, scale, logits);
    return OR_OK;
}

static int check_shapes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                        int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq)
{
    if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || num_blocks <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0)
        return OR_ERR_ARG;
    return OR_OK;
}

/*
 * Decode a list of (sequence, head) pairs.  pairs holds 2*num_pairs int32
 * values (s0, h0, s1, h1, ...); out is [num_pairs, head_dim] doubles.
 * q is [num_seqs, num_heads, head_dim] binary16, block_tables is
 * [num_seqs, max_blocks_per_seq] int32, context_lens is [num_seqs] int32.
 * Pairs are independent; OpenMP spreads them over the host threads.
 * *threads_used (if not NULL) receives the thread count.
 */
int oracle_decode_pairs(double *out, const int32_t *pairs, int32_t num_pairs,
                        const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                        const int32_t *block_tables, const int32_t *context_lens,
                        int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                        int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                        double scale, int32_t *threads_used)
{
    int rc = check_shapes(num_seqs, num_heads, head_dim, num_blocks, block_size,
                          max_blocks_per_seq);
    if (rc)
        return rc;
    int64_t max_len = (int64_t)max_blocks_per_seq * block_size;
    int status = OR_OK;
    int nthreads = 1;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        nthreads = omp_get_num_threads();
#endif
        double *Kbuf = malloc(sizeof(double) * (size_t)(max_len * head_dim + 1));
        double *Vbuf = malloc(sizeof(double) * (size_t)(max_len * head_dim + 1));
        double *qbuf = malloc(sizeof(double) * (size_t)head_dim);
        double *logits = malloc(sizeof(double) * (size_t)(max_len + 1));
        int local = (Kbuf && Vbuf && qbuf && logits) ? OR_OK : OR_ERR_NOMEM;
#pragma omp for schedule(dynamic, 1)
        for (int32_t p = 0; p < num_pairs; ++p) {
            if (local)
                continue;
            int32_t s = pairs[2 * p], h = pairs[2 * p + 1];
            if (s < 0 || s >= num_seqs || h < 0 || h >= num_heads) {
                local = OR_ERR_ARG;
                continue;
            }
            int r = decode_one(out + (int64_t)p * head_dim, q, k_cache, v_cache, block_tables,
                               context_lens, s, h, num_heads, head_dim, num_blocks, block_size,
                               max_blocks_per_seq, scale, Kbuf, Vbuf, qbuf, logits);
            if (r)
                local = r;
        }
        if (local) {
#pragma omp critical
            status = local;
        }
        free(Kbuf);
        free(Vbuf);
        free(qbuf);
        free(logits);
    }
    if (threads_used)
        *threads_used = nthreads;
    return status;
}

/* Decode every (sequence, head): out is [num_seqs, num_heads, head_dim]. */
int oracle_decode(double *out, const uint16_t *q, const uint16_t *k_cache,
                  const uint16_t *v_cache, const int32_t *block_tables,
                  const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                  int32_t head_dim, int32_t num_blocks, int32_t block_size,
                  int32_t max_blocks_per_seq, double scale, int32_t *threads_used)
{
    int rc = check_shapes(num_seqs, num_heads, head_dim, num_blocks, block_size,
                          max_blocks_per_seq);
    if (rc)
        return rc;
    int64_t n = (int64_t)num_seqs * num_heads;
    int32_t *pairs = malloc(sizeof(int32_t) * (size_t)(2 * n + 2));
    if (!pairs)
        return OR_ERR_NOMEM;
    for (int64_t i = 0; i < n; ++i) {
        pairs[2 * i] = (int32_t)(i / num_heads);
        pairs[2 * i + 1] = (int32_t)(i % num_heads);
    }
    rc = oracle_decode_pairs(out, pairs, (int32_t)n, q, k_cache, v_cache, block_tables,
                             context_lens, num_seqs, num_heads, head_dim, num_blocks, block_size,
                             max_blocks_per_seq, scale, threads_used);
    free(pairs);
    return rc;
}

/*
 * Write each new token's key/value into its cache slot, as raw 16-bit
 * patterns.  key, value: [num_tokens, num_heads, head_dim]; slot_mapping:
 * [num_tokens] int64, slot = physical_block * block_size + offset, the
 * position [10x] §2.3 maps a logical index to.  Slots outside
 * [0, num_blocks * block_size) are skipped.
 */
int oracle_reshape_and_cache(const uint16_t *key, const uint16_t *value,
                             uint16_t *k_cache, uint16_t *v_cache,
                             const int64_t *slot_mapping, int32_t num_tokens,
                             int32_t num_heads, int32_t head_dim, int32_t num_blocks,
                             int32_t block_size)
{
    if (num_tokens < 0 || num_heads <= 0 || head_dim <= 0 || num_blocks <= 0 || block_size <= 0)
        return OR_ERR_ARG;
    int64_t num_slots = (int64_t)num_blocks * block_size;
    for (int32_t t = 0; t < num_tokens; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0 || slot >= num_slots)
            continue;
        int64_t block = slot / block_size;
        int64_t offset = slot % block_size;
        for (int32_t h = 0; h < num_heads; ++h)
            for (int32_t d = 0; d < head_dim; ++d) {
                size_t dst = cache_index(block, offset, h, d, block_size, num_heads, head_dim);
                size_t src = (size_t)(((int64_t)t * num_heads + h) * head_dim + d);
                k_cache[dst] = key[src];
                v_cache[dst] = value[src];
            }
    }
    return OR_OK;
}

/*
 * Copy whole physical blocks inside a cache pair ([arch] §2.3 copy-on-write):
 * for each pair i, block mapping[2i+1] of k_cache and v_cache becomes a
 * bitwise copy of block mapping[2i].  block_elems = block_size * num_heads *
 * head_dim.  Pairs naming a block outside [0, num_blocks) are skipped.
 * Destinations are distinct and no destination is also a source in the same
 * call; under that precondition the pair order does not matter.
 */
int oracle_copy_blocks(uint16_t *k_cache, uint16_t *v_cache, const int64_t *mapping,
                       int32_t num_pairs, int32_t num_blocks, int64_t block_elems)
{
    if (num_pairs < 0 || num_blocks <= 0 || block_elems <= 0)
        return OR_ERR_ARG;
    for (int32_t i = 0; i < num_pairs; ++i) {
        int64_t src = mapping[2 * i], dst = mapping[2 * i + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks)
            continue;
        for (int64_t e = 0; e < block_elems; ++e) {
            k_cache[dst * block_elems + e] = k_cache[src * block_elems + e];
            v_cache[dst * block_elems + e] = v_cache[src * block_elems + e];
        }
    }
    return OR_OK;
}

/*
 * Move whole blocks between two caches of the same block shape ([src] §三:
 * swap out to host memory, swap back in): for each pair i, block
 * mapping[2i+1] of dst becomes a bitwise copy of block mapping[2i] of src.
 * Pairs outside [0, src_blocks) x [0, dst_blocks) are rejected.
 */
int oracle_swap_blocks(const uint16_t *src, uint16_t *dst, const int64_t *mapping,
                       int32_t num_pairs, int32_t src_blocks, int32_t dst_blocks,
                       int64_t block_elems)
{
    if (num_pairs < 0 || src_blocks <= 0 || dst_blocks <= 0 || block_elems <= 0)
        return OR_ERR_ARG;
    for (int32_t i = 0; i < num_pairs; ++i) {
        int64_t a = mapping[2 * i], b = mapping[2 * i + 1];
        if (a < 0 || a >= src_blocks || b < 0 || b >= dst_blocks)
            return OR_ERR_RANGE;
    }
    for (int32_t i = 0; i < num_pairs; ++i) {
        int64_t a = mapping[2 * i], b = mapping[2 * i + 1];
        for (int64_t e = 0; e < block_elems; ++e)
            dst[b * block_elems + e] = src[a * block_elems + e];
    }
    return OR_OK;
}

/* ---------------------------------------------------------------------------
 * FP8 KV cache ([10x] §3.3 names FP8 quantisation; the format is our reading:
 * OCP FP8 E4M3, 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, S.1111.111 = NaN, largest finite value 448; exponent field 0
 * holds the subnormals mantissa * 2^-9).  One float scale per cache:
 * stored code = E4M3(x * (1/scale)) and value = decode(code) * scale.
 * ------------------------------------------------------------------------- */

double oracle_e4m3_to_double(uint8_t c)
{
    int sign = c >> 7;
    int expo = (c >> 3) & 15;
    int mant = c & 7;
    double v;
    if (expo == 15 && mant == 7)
        return NAN;
    if (expo == 0)
        v = ldexp((double)mant, -9);
    else
        v = ldexp((double)(8 + mant), expo - 10); /* (1 + mant/8) * 2^(expo-7) */
    return sign ? -v : v;
}

/* Nearest E4M3 code to y, ties to the code with an even mantissa; finite
 * values beyond the largest code (and +-inf) saturate to +-448; NaN stays NaN.
 * Written as a search over the 127 non-negative finite codes, whose values
 * increase with the code. */
uint8_t oracle_float_to_e4m3(float y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    if (isnan(y))
        return (uint8_t)(sign | 0x7F);
    double a = fabs((double)y);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    int best = 0;
    for (int c = 1; c <= 0x7E; ++c) {
        double dc = fabs(oracle_e4m3_to_double((uint8_t)c) - a);
        double db = fabs(oracle_e4m3_to_double((uint8_t)best) - a);
        if (dc < db || (dc == db && (c & 1) == 0))
            best = c;
    }
    return (uint8_t)(sign | best);
}

/* The scale factor the quantiser multiplies by: 1/scale rounded to float. */
static float inverse_scale(float scale) { return (float)(1.0 / (double)scale); }

/* codes[i] = E4M3(fp16(x[i]) * (1/scale)), the product rounded to float. */
void oracle_quantize_e4m3(const uint16_t *x, uint8_t *codes, int64_t n, float scale)
{
    float inv = inverse_scale(scale);
    for (int64_t i = 0; i < n; ++i) {
        float xf = (float)oracle_half_to_double(x[i]);
        float y = xf * inv;
        codes[i] = oracle_float_to_e4m3(y);
    }
}

/* reshape_and_cache into FP8 caches: the same slots as the fp16 version,
 * each value quantised with its cache's scale. */
int oracle_reshape_and_cache_fp8(const uint16_t *key, const uint16_t *value,
                                 uint8_t *k_cache, uint8_t *v_cache,
                                 const int64_t *slot_mapping, int32_t num_tokens,
                                 int32_t num_heads, int32_t head_dim, int32_t num_blocks,
                                 int32_t block_size, float k_scale, float v_scale)
{
    if (num_tokens < 0 || num_heads <= 0 || head_dim <= 0 || num_blocks <= 0 || block_size <= 0)
        return OR_ERR_ARG;
    int64_t num_slots = (int64_t)num_blocks * block_size;
    int64_t row = (int64_t)num_heads * head_dim;
    for (int32_t t = 0; t < num_tokens; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0 || slot >= num_slots)
            continue;
        /* [NB, B, H, D]: the rows of slot = block*B + offset start at slot*H*D */
        oracle_quantize_e4m3(key + t * row, k_cache + slot * row, row, k_scale);
        oracle_quantize_e4m3(value + t * row, v_cache + slot * row, row, v_scale);
    }
    return OR_OK;
}

/* The paged gather of [10x] §2.3 over FP8 caches, dequantising each value. */
static int gather_fp8(double *k_out, double *v_out, const uint8_t *k_cache, const uint8_t *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens, int32_t seq,
                      int32_t head, int32_t num_heads, int32_t head_dim, int32_t num_blocks,
                      int32_t block_size, int32_t max_blocks_per_seq, float k_scale, float v_scale)
{
    int32_t L = context_lens[seq];
    if (L < 0 || (int64_t)L > (int64_t)max_blocks_per_seq * block_size)
        return OR_ERR_RANGE;
    for (int32_t i = 0; i < L; ++i) {
        int32_t physical = block_tables[(int64_t)seq * max_blocks_per_seq + i / block_size];
        int32_t offset = i % block_size;
        if (physical < 0 || physical >= num_blocks)
            return OR_ERR_RANGE;
        for (int32_t d = 0; d < head_dim; ++d) {
            size_t src = cache_index(physical, offset, head, d, block_size, num_heads, head_dim);
            k_out[(int64_t)i * head_dim + d] = oracle_e4m3_to_double(k_cache[src]) * (double)k_scale;
            v_out[(int64_t)i * head_dim + d] = oracle_e4m3_to_double(v_cache[src]) * (double)v_scale;
        }
    }
    return L;
}

/* Decode over FP8 caches for a list of (sequence, head) pairs; the same
 * conventions as oracle_decode_pairs, q still fp16. */
int oracle_decode_fp8_pairs(double *out, const int32_t *pairs, int32_t num_pairs,
                            const uint16_t *q, const uint8_t *k_cache, const uint8_t *v_cache,
                            const int32_t *block_tables, const int32_t *context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                            int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                            double scale, float k_scale, float v_scale, int32_t *threads_used)
{
    int rc = check_shapes(num_seqs, num_heads, head_dim, num_blocks, block_size,
                          max_blocks_per_seq);
    if (rc)
        return rc;
    int64_t max_len = (int64_t)max_blocks_per_seq * block_size;
    int status = OR_OK;
    int nthreads = 1;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        nthreads = omp_get_num_threads();
#endif
        double *Kbuf = malloc(sizeof(double) * (size_t)(max_len * head_dim + 1));
        double *Vbuf = malloc(sizeof(double) * (size_t)(max_len * head_dim + 1));
        double *qbuf = malloc(sizeof(double) * (size_t)head_dim);
        double *logits = malloc(sizeof(double) * (size_t)(max_len + 1));
        int local = (Kbuf && Vbuf && qbuf && logits) ? OR_OK : OR_ERR_NOMEM;
#pragma omp for schedule(dynamic, 1)
        for (int32_t p = 0; p < num_pairs; ++p) {
            if (local)
                continue;
            int32_t s = pairs[2 * p], h = pairs[2 * p + 1];
            if (s < 0 || s >= num_seqs || h < 0 || h >= num_heads) {
                local = OR_ERR_ARG;
                continue;
            }
            int L = gather_fp8(Kbuf, Vbuf, k_cache, v_cache, block_tables, context_lens, s, h,
                               num_heads, head_dim, num_blocks, block_size, max_blocks_per_seq,
                               k_scale, v_scale);
            if (L < 0) {
                local = L;
                continue;
            }
            load_query(qbuf, q, s, h, num_heads, head_dim);
            attend_contiguous(out + (int64_t)p * head_dim, qbuf, Kbuf, Vbuf, L, head_dim, scale,
                              logits);
        }
        if (local) {
#pragma omp critical
            status = local;
        }
        free(Kbuf);
        free(Vbuf);
        free(qbuf);
        free(logits);
    }
    if (threads_used)
        *threads_used = nthreads;
    return status;
}

/* ---------------------------------------------------------------------------
 * Multi-query paged attention ([10x] §4.3 and [eng] §4.2: prefill and
 * decode work in one batch).  Reading: sequence s brings n_s = query_start[s+1] - query_start[s]
 * query rows, the last n_s positions of its context (their K/V are already
 * in the cache); row i sits at logical position p = context_lens[s] - n_s + i
 * and attends positions 0..p (causal).  n_s = 1 is the decode step.
 * q and out are [num_tokens, num_heads, head_dim] with the rows of sequence s
 * at query_start[s] .. query_start[s+1]-1.
 * ------------------------------------------------------------------------- */
/* One body for both cache formats: fp16 caches (k_cache, v_cache), or FP8
 * codes (k8, v8, non-NULL) dequantised with k_scale, v_scale as in the FP8
 * decode. */
static int prefill_any(double *out, const uint16_t *q, const uint16_t *k_cache,
                       const uint16_t *v_cache, const uint8_t *k8, const uint8_t *v8,
                       float k_scale, float v_scale, const int32_t *block_tables,
                       const int32_t *context_lens, const int32_t *query_start,
                       int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                       int32_t head_dim, int32_t num_blocks, int32_t block_size,
                       int32_t max_blocks_per_seq, double scale, int32_t *threads_used)
{
    int rc = check_shapes(num_seqs, num_heads, head_dim, num_blocks, block_size,
                          max_blocks_per_seq);
    if (rc)
        return rc;
    if (query_start[0] != 0 || query_start[num_seqs] != num_tokens)
        return OR_ERR_ARG;
    for (int32_t s = 0; s < num_seqs; ++s) {
        int32_t n = query_start[s + 1] - query_start[s];
        if (n < 0 || n > context_lens[s])
            return OR_ERR_RANGE;
    }
    int64_t max_len = (int64_t)max_blocks_per_seq * block_size;
    int status = OR_OK;
    int nthreads = 1;
    int64_t units = (int64_t)num_seqs * num_heads;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        nthreads = omp_get_num_threads();
#endif
        double *Kbuf = malloc(sizeof(double) * (size_t)(max_len * head_dim + 1));
        double *Vbuf = malloc(sizeof(double) * (size_t)(max_len * head_dim + 1));
        double *qbuf = malloc(sizeof(double) * (size_t)head_dim);
        double *logits = malloc(sizeof(double) * (size_t)(max_len + 1));
        int local = (Kbuf && Vbuf && qbuf && logits) ? OR_OK : OR_ERR_NOMEM;
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (local)
                continue;
            int32_t s = (int32_t)(u / num_heads), h = (int32_t)(u % num_heads);
            int L = k8 ? gather_fp8(Kbuf, Vbuf, k8, v8, block_tables, context_lens, s, h,
                                    num_heads, head_dim, num_blocks, block_size,
                                    max_blocks_per_seq, k_scale, v_scale)
                       : oracle_gather(Kbuf, Vbuf, k_cache, v_cache, block_tables, context_lens,
                                       s, h, num_heads, head_dim, num_blocks, block_size,
                                       max_blocks_per_seq);
            if (L < 0) {
                local = L;
                continue;
            }
            int32_t n = query_start[s + 1] - query_start[s];
            for (int32_t i = 0; i < n; ++i) {
                int32_t row = query_start[s] + i;
                int32_t visible = L - n + i + 1; /* positions 0 .. L-n+i */
                load_query(qbuf, q, row, h, num_heads, head_dim);
                attend_contiguous(out + ((int64_t)row * num_heads + h) * head_dim, qbuf, Kbuf, Vbuf,
                                  visible, head_dim, scale, logits);
            }
        }
        if (local) {
#pragma omp critical
            status = local;
        }
        free(Kbuf);
        free(Vbuf);
        free(qbuf);
        free(logits);
    }
    if (threads_used)
        *threads_used = nthreads;
    return status;
}

int oracle_prefill(double *out, const uint16_t *q, const uint16_t *k_cache,
                   const uint16_t *v_cache, const int32_t *block_tables,
                   const int32_t *context_lens, const int32_t *query_start, int32_t num_seqs,
                   int32_t num_tokens, int32_t num_heads, int32_t head_dim, int32_t num_blocks,
                   int32_t block_size, int32_t max_blocks_per_seq, double scale,
                   int32_t *threads_used)
{
    return prefill_any(out, q, k_cache, v_cache, NULL, NULL, 1.0f, 1.0f, block_tables,
                       context_lens, query_start, num_seqs, num_tokens, num_heads, head_dim,
                       num_blocks, block_size, max_blocks_per_seq, scale, threads_used);
}

/* Multi-query paged attention over FP8 caches: oracle_prefill with each K
 * (V) value read as value(code) * k_scale (v_scale), q still fp16. */
int oracle_prefill_fp8(double *out, const uint16_t *q, const uint8_t *k_cache,
                       const uint8_t *v_cache, const int32_t *block_tables,
                       const int32_t *context_lens, const int32_t *query_start,
                       int32_t num_seqs, int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                       int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                       double scale, float k_scale, float v_scale, int32_t *threads_used)
{
    if (!k_cache || !v_cache)
        return OR_ERR_ARG;
    return prefill_any(out, q, NULL, NULL, k_cache, v_cache, k_scale, v_scale, block_tables,
                       context_lens, query_start, num_seqs, num_tokens, num_heads, head_dim,
                       num_blocks, block_size, max_blocks_per_seq, scale, threads_used);
}

/* Timing plumbing, no arithmetic: the number of host threads later calls use
 * (n <= 0: the OpenMP default).  Returns the count now in effect. */
int oracle_set_threads(int n)
{
    static int default_threads = 0;
    if (default_threads == 0)
        default_threads = omp_get_max_threads();
    omp_set_num_threads(n > 0 ? n : default_threads);
    return omp_get_max_threads();
}
