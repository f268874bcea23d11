/*
 * oracle.c -- the fp64 CPU oracle for paged-KV attention decode.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this file's library.  The GPU library shares no code,
 * header, table or helper with it.
 *
 * What it computes (plain definition, written out):
 *
 *   For every sequence s and q head h, with kv head g = h / (Hq / Hkv):
 *     1. gather: for each logical token t of the context, physical block
 *        b = block_tables[s][t / bs] and slot t % bs give the rows
 *        Kc[t] = k_cache[b][g][t % bs][:] and Vc[t] likewise.  The K/V of a
 *        sequence sit in fixed-size physical blocks found through a per-sequence
 *        logical->physical table and addressed indirectly
 *        ("架构解构：推理引擎的四层抽象", PagedAttention section; the block count
 *        ceil(n / block_size) is "LLM+Agent 全栈推理底座" 4.2, BlockManager.allocate).
 *     2. textbook scaled dot-product attention for the one query row:
 *        z[t] = scale * sum_d q[s][h][d] * Kc[t][d];  weights = softmax(z)
 *        computed stably by subtracting max z;  out = sum_t weights[t] * Vc[t]
 *        ("从零开始构建LLM推理引擎：模型执行器深度解析" 3.1, scaled_dot_product_attention:
 *        scores q k^T / sqrt(d), stable softmax, weights times v).  Decode has a
 *        single query at the newest position, so no causal mask applies.
 *     3. lse[s][h] = max z + log(sum_t exp(z[t] - max z)), natural log.
 *
 *   All arithmetic is IEEE double.  The fp16/bf16 inputs are widened exactly by
 *   decoding their bits here.  `scale` is the fp32 value the caller passes,
 *   widened.  Tokens are summed in logical order t = lo, lo+1, ..., hi-1.
 *
 *   An optional token range [tok_lo[s], tok_hi[s]) restricts step 1 to part of
 *   the context (clipped to [0, context_lens[s])).  An empty range gives
 *   out = 0 and lse = -inf.  That reading of an empty context (the pages do not
 *   speak of one) is also what the GPU library writes.
 *
 * Reduced-precision KV (oracle_paged_decode_kv with kv_dtype ORACLE_FP8): the
 * cache holds one byte per value in the OCP 8-bit floating-point format E4M3
 * (1 sign, 4 exponent bits with bias 7, 3 fraction bits; exponent field 0 is
 * subnormal; the all-ones exponent with all-ones fraction is NaN; no
 * infinities), and every (block, kv head) of K and of V carries one fp32
 * scale: the value a code stands for is its E4M3 value times the scale of its
 * block and kv head.  This is the KV-compression idea of
 * "从零开始构建LLM推理引擎：模型执行器深度解析" 5.2, KV缓存管理技巧 (historical
 * KV kept at reduced precision) carried
 * to an 8-bit format with per-block scales; the pages fix neither the format
 * nor the scale granularity.
 *
 * Return value: 0 on success; -1 if a table entry that the context reaches is
 * outside [0, num_blocks) or a context length is negative or exceeds the table
 * width times block_size; -2 on a bad argument.  No output is defined on error.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1, ORACLE_FP8 = 3 };

/* IEEE-754 binary16: 1 sign, 5 exponent, 10 fraction bits. */
static double half_bits_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 1024), e - 25);     /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent, 7 fraction bits (the top half of a binary32). */
static double bf16_bits_to_double(uint16_t b) {
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);                /* f * 2^-126 * 2^-7 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 128), e - 134);     /* (1 + f/2^7) * 2^(e-127) */
    return sign ? -v : v;
}

/* OCP E4M3: 1 sign, 4 exponent (bias 7), 3 fraction bits; S.1111.111 is NaN. */
static double e4m3_bits_to_double(uint8_t c) {
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xf;
    int f = c & 0x7;
    double v;
    if (e == 0)
        v = ldexp((double)f, -9);                  /* f/8 * 2^(1-7) */
    else if (e == 15 && f == 7)
        v = NAN;
    else
        v = ldexp((double)(f + 8), e - 10);        /* (1 + f/8) * 2^(e-7) */
    return sign ? -v : v;
}

double oracle_decode_value(uint16_t bits, int dtype) {
    if (dtype == ORACLE_FP8) return e4m3_bits_to_double((uint8_t)bits);
    return dtype == ORACLE_BF16 ? bf16_bits_to_double(bits) : half_bits_to_double(bits);
}

/* The E4M3 code nearest to x (saturating: beyond the largest finite value 448
 * the nearest finite code is 448's), ties to the code with an even last
 * fraction bit; NaN gives the NaN code.  Brute force over the 127 non-negative
 * finite codes, so it needs no rounding arithmetic of its own. */
uint8_t oracle_fp8_encode(float x) {
    if (x != x) return 0x7f;
    const uint8_t sign = signbit(x) ? 0x80 : 0;
    const double a = fabs((double)x);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c < 127; ++c) {
        const double d = fabs(e4m3_bits_to_double((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(sign | best);
}

void oracle_fp8_encode_array(const float* x, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_encode(x[i]);
}

/* Quantise one (block, kv head): the first ntok rows of a [bs][D] tile of
 * 16-bit values become E4M3 codes with one scale.  amax = max |x| over those
 * rows; scale = amax / 448 in fp32 (1 when amax is 0); code = nearest E4M3 to
 * x / scale, the division in fp32; rows from ntok on become code 0. */
void oracle_quantize_fp8(const uint16_t* src, int src_dtype, int ntok, int bs, int D,
                         uint8_t* codes, float* scale_out) {
    float amax = 0.0f;
    for (int i = 0; i < ntok * D; ++i) {
        const float x = (float)oracle_decode_value(src[i], src_dtype);
        if (fabsf(x) > amax) amax = fabsf(x);
    }
    const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    for (int i = 0; i < bs * D; ++i) {
        if (i < ntok * D) {
            const float x = (float)oracle_decode_value(src[i], src_dtype);
            const float y = x / scale;
            codes[i] = oracle_fp8_encode(y);
        } else {
            codes[i] = 0;
        }
    }
    *scale_out = scale;
}

/* One cache value: 16-bit storage decoded exactly, or an E4M3 code times the
 * scale of its (block, kv head). */
static double kv_value(const void* cache, int64_t idx, int kv_dtype, const float* scales, int64_t bg) {
    if (kv_dtype == ORACLE_FP8)
        return e4m3_bits_to_double(((const uint8_t*)cache)[idx]) * (double)scales[bg];
    return oracle_decode_value(((const uint16_t*)cache)[idx], kv_dtype);
}

int oracle_paged_decode_kv(
    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int block_size, int num_blocks, int table_stride, int table_width, int dtype, int kv_dtype,
    const uint16_t* q,            /* [B][Hq][D], dtype */
    const void* k_cache,          /* [NB][Hkv][bs][D], kv_dtype */
    const void* v_cache,          /* [NB][Hkv][bs][D], kv_dtype */
    const float* k_scale,         /* [NB][Hkv] when kv_dtype is ORACLE_FP8, else unused */
    const float* v_scale,
    const int32_t* block_tables,  /* [B][table_stride], table_width used */
    const int32_t* context_lens,  /* [B] */
    const int32_t* tok_lo,        /* nullable [B] */
    const int32_t* tok_hi,        /* nullable [B] */
    float scale,
    double* out,                  /* [B][Hq][D] */
    double* lse,                  /* [B][Hq], nullable */
    int nthreads)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || num_q_heads % num_kv_heads != 0 || table_width > table_stride ||
        (dtype != ORACLE_F16 && dtype != ORACLE_BF16) ||
        (kv_dtype == ORACLE_FP8 ? (!k_scale || !v_scale) : kv_dtype != dtype))
        return -2;
    const int B = num_seqs, Hq = num_q_heads, Hkv = num_kv_heads, D = head_dim;
    const int bs = block_size, G = Hq / Hkv;
    const double sc = (double)scale;

    /* Check every table entry a context reaches before computing anything. */
    for (int s = 0; s < B; ++s) {
        int c = context_lens[s];
        if (c < 0 || (int64_t)c > (int64_t)table_width * bs) return -1;
        for (int j = 0; j < (c + bs - 1) / bs; ++j) {
            int32_t b = block_tables[(int64_t)s * table_stride + j];
            if (b < 0 || b >= num_blocks) return -1;
        }
    }

    int status = 0;
    const int64_t npairs = (int64_t)B * Hkv;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t pair = 0; pair < npairs; ++pair) {
        const int s = (int)(pair / Hkv), g = (int)(pair % Hkv);
        int lo = 0, hi = context_lens[s];
        if (tok_lo && tok_lo[s] > lo) lo = tok_lo[s];
        if (tok_hi && tok_hi[s] < hi) hi = tok_hi[s];
        const int n = hi > lo ? hi - lo : 0;

        if (n == 0) {
            for (int hh = 0; hh < G; ++hh) {
                int h = g * G + hh;
                for (int d = 0; d < D; ++d) out[((int64_t)s * Hq + h) * D + d] = 0.0;
                if (lse) lse[(int64_t)s * Hq + h] = -INFINITY;
            }
            continue;
        }

        /* Step 1: gather this sequence's K/V rows for kv head g into contiguous
           fp64 arrays, token by token through the block table. */
        double* Kc = (double*)malloc(sizeof(double) * (size_t)n * D);
        double* Vc = (double*)malloc(sizeof(double) * (size_t)n * D);
        double* z = (double*)malloc(sizeof(double) * (size_t)n);
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
        if (!Kc || !Vc || !z || !acc) {
            free(Kc); free(Vc); free(z); free(acc);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = -2;
            continue;
        }
        for (int i = 0; i < n; ++i) {
            const int t = lo + i;
            const int64_t b = block_tables[(int64_t)s * table_stride + t / bs];
            const int64_t row = ((b * Hkv + g) * bs + (t % bs)) * D;
            for (int d = 0; d < D; ++d) {
                Kc[(int64_t)i * D + d] = kv_value(k_cache, row + d, kv_dtype, k_scale, b * Hkv + g);
                Vc[(int64_t)i * D + d] = kv_value(v_cache, row + d, kv_dtype, v_scale, b * Hkv + g);
            }
        }

        /* Steps 2-3 for each q head of the group. */
        for (int hh = 0; hh < G; ++hh) {
            const int h = g * G + hh;
            const uint16_t* qh = q + ((int64_t)s * Hq + h) * D;
            double m = -INFINITY;
            for (int i = 0; i < n; ++i) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += oracle_decode_value(qh[d], dtype) * Kc[(int64_t)i * D + d];
                z[i] = sc * dot;
                if (z[i] > m) m = z[i];
            }
            double Z = 0.0;
            for (int d = 0; d < D; ++d) acc[d] = 0.0;
            for (int i = 0; i < n; ++i) {
                const double w = exp(z[i] - m);
                Z += w;
                for (int d = 0; d < D; ++d) acc[d] += w * Vc[(int64_t)i * D + d];
            }
            for (int d = 0; d < D; ++d) out[((int64_t)s * Hq + h) * D + d] = acc[d] / Z;
            if (lse) lse[(int64_t)s * Hq + h] = m + log(Z);
        }
        free(Kc); free(Vc); free(z); free(acc);
    }
    return status;
}

/* Same-precision K/V and q (fp16 or bf16 everywhere). */
int oracle_paged_decode(
    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int block_size, int num_blocks, int table_stride, int table_width, int dtype,
    const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* tok_lo, const int32_t* tok_hi,
    float scale, double* out, double* lse, int nthreads)
{
    return oracle_paged_decode_kv(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                  table_stride, table_width, dtype, dtype, q, k_cache, v_cache, NULL, NULL,
                                  block_tables, context_lens, tok_lo, tok_hi, scale, out, lse, nthreads);
}

/* Chunked prefill ("架构解构：推理引擎的四层抽象", FlashAttention section: many
 * queries per sequence over the paged context, causal).  Sequence s has
 * context_lens[s] = n tokens in the cache, the last m = cu_q[s+1] - cu_q[s] of
 * which are this chunk; chunk query i (row cu_q[s] + i of q and out) sits at
 * position n - m + i and attends to the tokens at positions 0 .. n - m + i.
 * That is decode attention over a context of n - m + i + 1 tokens, so each
 * query row is computed by oracle_paged_decode_kv with that length.
 *   q, out : [total_q][Hq][D];  lse : [total_q][Hq] (nullable)
 * Returns -1 if some m exceeds its n or cu_q is not non-decreasing from 0. */
int oracle_paged_prefill(
    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int block_size, int num_blocks, int table_stride, int table_width, int dtype,
    const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_q,
    float scale, double* out, double* lse, int nthreads)
{
    if (num_seqs < 0 || table_width > table_stride || cu_q[0] != 0) return -1;
    const int total = cu_q[num_seqs];
    for (int s = 0; s < num_seqs; ++s) {
        const int m = cu_q[s + 1] - cu_q[s];
        if (m < 0 || m > context_lens[s]) return -1;
    }
    if (total == 0) return 0;
    int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)total * table_stride);
    int32_t* lens = (int32_t*)malloc(sizeof(int32_t) * (size_t)total);
    if (!rows || !lens) { free(rows); free(lens); return -2; }
    for (int s = 0; s < num_seqs; ++s) {
        const int n = context_lens[s], m = cu_q[s + 1] - cu_q[s];
        for (int i = 0; i < m; ++i) {
            const int r = cu_q[s] + i;
            memcpy(rows + (int64_t)r * table_stride, block_tables + (int64_t)s * table_stride,
                   sizeof(int32_t) * (size_t)table_stride);
            lens[r] = n - m + i + 1;
        }
    }
    const int rc = oracle_paged_decode_kv(total, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                          table_stride, table_width, dtype, dtype, q, k_cache, v_cache, NULL, NULL,
                                          rows, lens, NULL, NULL, scale, out, lse, nthreads);
    free(rows);
    free(lens);
    return rc;
}

/* Threads OpenMP would use for nthreads <= 0 requests (reported by the bench). */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
