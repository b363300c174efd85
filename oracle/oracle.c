/*
 * CPU oracle for paged decode attention and the slot-mapped cache write.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load
 * this file: only tests/, the smoke check and the bench's cpu_baseline leg use it.
 * It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (all floating point in IEEE binary64):
 *
 *   Paging.  The K/V of each sequence lives in fixed 16-token blocks that need not
 *   be adjacent; a per-sequence block table maps logical block j to a physical block
 *   ("vLLM ve Triton ile maliyet optimizasyonu", §03 Yöntem, steps 1 and 2;
 *   "vLLM Nedir? PagedAttention ile Production LLM Serving", section "PagedAttention").
 *   Token t of sequence b lives in physical block table[b][t / 16], row t % 16.
 *
 *   Attention.  The math is ordinary scaled dot-product attention; paging only
 *   changes where K and V are read from (same page, §03, closing paragraphs).
 *   For one query q over n gathered rows K[t], V[t]:
 *       s_t = scale * sum_i q_i K[t][i]
 *       m   = max_t s_t,  p_t = exp(s_t - m) / sum_u exp(s_u - m)
 *       o   = sum_t p_t V[t]
 *   GQA: query head h reads KV head h / (Hq / Hkv) ("Yerel LLM sistemlerinde
 *   backpressure ve ölçekleme", section "KV bütçesi", on 64 attention heads sharing
 *   8 KV heads; the page gives the counts, the contiguous grouping is our reading).
 *
 *   Split over the context.  Attention restricted to the token range of partition p
 *   gives (o_p, m_p, l_p) with l_p = sum exp(s_t - m_p); the full result is
 *   sum_p w_p o_p / sum_p w_p with w_p = exp(m_p - max_p m_p) l_p.
 *
 *   Cache write.  Each token t with slot_mapping[t] >= 0 copies the raw bits of its
 *   K/V rows into slot s = block * 16 + offset; every other byte is left alone
 *   (§03 step 3: a new token goes into the current block, a new block is taken only
 *   when the last one is full).
 *
 *   FP8 KV cache ("Yerel LLM sistemlerinde backpressure ve ölçekleme", the paragraph
 *   on KV cache quantisation: storing K/V in FP8 halves the bytes per token, at some
 *   accuracy cost on long contexts).  The page names neither the format nor a scale;
 *   our reading is the OCP e4m3 format (1 sign, 4 exponent bits with bias 7, 3 mantissa
 *   bits, no infinities, NaN = S.1111.111, largest finite 448) with one scale per
 *   tensor for K and one for V.  A stored code c stands for value(c) * scale.  Writing
 *   x: v = x / scale in IEEE binary32 (the precision the library decides in), then the
 *   code of the finite e4m3 value nearest to v, ties to the even code; so |v| > 448
 *   (infinities included) saturates to +-448.  NaN gives S.1111.111.
 *
 * Cache layout (the pages leave it open; this is the layout the library documents), for
 * blocks of BS tokens (16 by default; 8 and 32 as the block-size variants: "vLLM ve
 * Triton ...", the paragraph calling block size a tuning knob):
 *   x = 16 / element_bytes (16 for fp8, 8 for fp16/bf16, 4 for fp32)
 *   K: [num_blocks][Hkv][d / x][BS][x]   element (blk, g, t, i) at
 *        (((blk * Hkv + g) * (d / x) + i / x) * BS + t) * x + i % x
 *   V: [num_blocks][Hkv][d][BS]          element (blk, g, t, i) at
 *        ((blk * Hkv + g) * d + i) * BS + t
 *   Token t of a sequence lives in block table[t / BS], row t % BS.
 *   key/value rows: element (t, g, i) at t * row_stride + g * d + i
 *   q:              element (b, h, i) at b * q_stride + h * d + i
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math, no FMA contraction).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_FP8 = 3 };

/* IEEE 754 binary16 -> binary64, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double half_bits_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1, e = (h >> 10) & 0x1f, f = h & 0x3ff;
    double v;
    if (e == 0) v = ldexp((double)f, -24);                 /* zero / subnormal */
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(0x400 | f), e - 25);           /* (1.f) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double bf16_bits_to_f64(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* OCP e4m3 -> binary64, from the format's definition: 1 sign bit, 4 exponent bits
 * (bias 7), 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN
 * and there is no infinity. */
static double fp8_bits_to_f64(uint8_t c) {
    int sign = c >> 7, e = (c >> 3) & 0xf, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);                  /* (m/8) * 2^(1-7) */
    else v = ldexp((double)(8 | m), e - 10);               /* (1.m) * 2^(e-7) */
    return sign ? -v : v;
}

/* binary64 -> OCP e4m3: the code of the nearest finite value, ties to the even code
 * (round to nearest even on the 3-bit mantissa); larger magnitudes saturate to 448.
 * Written as a search over the 127 non-negative finite codes so that it follows the
 * definition of rounding to nearest with no bit tricks. */
static uint8_t fp8_from_f64(double v) {
    uint8_t sign = signbit(v) ? 0x80 : 0;
    if (isnan(v)) return sign | 0x7f;
    double a = fabs(v), best_d = INFINITY;
    /* 448 is the nearest finite value to any larger magnitude.  Said outright: far out
     * (1e30, inf) every distance below rounds to the same binary64 value. */
    if (a >= 448.0) return sign | 0x7e;
    int best = 0;
    for (int c = 0; c <= 0x7e; ++c) {
        double dd = fabs(a - fp8_bits_to_f64((uint8_t)c));
        if (dd < best_d || (dd == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best_d = dd;
            best = c;
        }
    }
    return sign | (uint8_t)best;
}

static double elem(const void* base, int64_t idx, int dtype) {
    if (dtype == OR_F32) return (double)((const float*)base)[idx];
    if (dtype == OR_FP8) return fp8_bits_to_f64(((const uint8_t*)base)[idx]);
    uint16_t h = ((const uint16_t*)base)[idx];
    return dtype == OR_F16 ? half_bits_to_f64(h) : bf16_bits_to_f64(h);
}

static int elem_bytes(int dtype) { return dtype == OR_F32 ? 4 : dtype == OR_FP8 ? 1 : 2; }

static int64_t k_off(int64_t blk, int g, int t, int i, int Hkv, int d, int x, int bs) {
    return (((blk * Hkv + g) * (d / x) + i / x) * bs + t) * x + i % x;
}
static int64_t v_off(int64_t blk, int g, int t, int i, int Hkv, int d, int bs) {
    return ((blk * Hkv + g) * d + i) * bs + t;
}

/* Element-wise widening, exported so tests can pin the conversions. */
void oracle_to_f64(double* dst, const void* src, int64_t n, int32_t dtype) {
    for (int64_t k = 0; k < n; ++k) dst[k] = elem(src, k, dtype);
}

/* FP8 quantisation of n elements of src (fp32/fp16/bf16): dst[k] = e4m3 code of the
 * binary32 quotient src[k] / scale. */
void oracle_fp8_quantize(uint8_t* dst, const void* src, int64_t n, int32_t src_dtype,
                         float scale) {
    for (int64_t k = 0; k < n; ++k) {
        float v = (float)elem(src, k, src_dtype);   /* exact: fp16/bf16 fit in binary32 */
        float qv = v / scale;
        dst[k] = fp8_from_f64((double)qv);
    }
}

/* The e4m3 encoder on binary64 inputs, exported for its pins. */
void oracle_fp8_encode(uint8_t* dst, const double* src, int64_t n) {
    for (int64_t k = 0; k < n; ++k) dst[k] = fp8_from_f64(src[k]);
}

/* Textbook attention of one query over n contiguous rows.
 * Writes o[d]; *m_out = max logit (natural units), *l_out = sum exp(s - m).
 * n == 0 gives o = 0, m = -inf, l = 0. */
void oracle_attend(double* o, double* m_out, double* l_out, const double* q,
                   const double* K, const double* V, int64_t n, int32_t d, double scale) {
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    if (n <= 0) {
        if (m_out) *m_out = -INFINITY;
        if (l_out) *l_out = 0.0;
        return;
    }
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
        double dot = 0.0;
        for (int i = 0; i < d; ++i) dot += q[i] * K[t * d + i];
        s[t] = scale * dot;
        if (s[t] > m) m = s[t];
    }
    double l = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        s[t] = exp(s[t] - m);
        l += s[t];
    }
    for (int64_t t = 0; t < n; ++t) {
        double p = s[t] / l;
        for (int i = 0; i < d; ++i) o[i] += p * V[t * d + i];
    }
    free(s);
    if (m_out) *m_out = m;
    if (l_out) *l_out = l;
}

/* Gather rows [t0, t1) of KV head g of one sequence through its block-table row
 * into contiguous fp64 arrays K[t1-t0][d], V[t1-t0][d], each element times its
 * cache's scale (1 unless the cache is fp8).  Returns -1 when the table points
 * outside the pool. */
int oracle_gather(double* K, double* V, const void* k_cache, const void* v_cache,
                  const int32_t* table_row, int64_t t0, int64_t t1, int32_t g,
                  int32_t Hkv, int32_t d, int64_t num_blocks, int32_t dtype,
                  double k_scale, double v_scale, int32_t bs) {
    int x = 16 / elem_bytes(dtype);
    for (int64_t t = t0; t < t1; ++t) {
        int64_t blk = table_row[t / bs];
        int off = (int)(t % bs);
        if (blk < 0 || blk >= num_blocks) return -1;
        for (int i = 0; i < d; ++i) {
            K[(t - t0) * d + i] = elem(k_cache, k_off(blk, g, off, i, Hkv, d, x, bs), dtype) * k_scale;
            V[(t - t0) * d + i] = elem(v_cache, v_off(blk, g, off, i, Hkv, d, bs), dtype) * v_scale;
        }
    }
    return 0;
}

/* Shared driver: for each requested (b, h) row and each context partition of
 * `part` tokens (part <= 0: one partition over the whole context), gather and
 * attend.  Outputs per (row, partition): o[d], m, l.  rows == NULL means every
 * (b, h) in order b * Hq + h. */
static int decode_core(double* o, double* m, double* l, const int32_t* rows, int32_t n_rows,
                       const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                       const int32_t* tables, const int32_t* seq_lens, int32_t B, int32_t Hq,
                       int32_t Hkv, int32_t d, int32_t max_blocks, int64_t num_blocks,
                       double scale, int32_t q_dtype, int32_t kv_dtype, double k_scale,
                       double v_scale, int32_t part, int32_t max_parts, int32_t nthreads,
                       int32_t bs) {
    if (Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || (d % (16 / elem_bytes(kv_dtype))) != 0) return -1;
    if (q_dtype == OR_FP8) return -1;
    int G = Hq / Hkv;
    int64_t total = rows ? n_rows : (int64_t)B * Hq;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
#endif
    for (int64_t r = 0; r < total; ++r) {
        int b = rows ? rows[2 * r] : (int)(r / Hq);
        int h = rows ? rows[2 * r + 1] : (int)(r % Hq);
        if (b < 0 || b >= B || h < 0 || h >= Hq) { bad |= 1; continue; }
        int g = h / G;
        int64_t n = seq_lens[b];
        if (n > (int64_t)max_blocks * bs) { bad |= 1; continue; }
        int64_t P = part > 0 ? part : (n > 0 ? n : 1);
        int64_t np = n > 0 ? (n + P - 1) / P : 0;
        int nslots = part > 0 ? max_parts : 1;
        if (np > nslots) { bad |= 1; continue; }
        double* qq = (double*)malloc(sizeof(double) * d);
        for (int i = 0; i < d; ++i) qq[i] = elem(q, (int64_t)b * q_stride + (int64_t)h * d + i, q_dtype);
        for (int p = 0; p < nslots; ++p) {
            double* op = o + (r * nslots + p) * d;
            double mp = -INFINITY, lp = 0.0;
            int64_t t0 = p * P, t1 = t0 + P < n ? t0 + P : n;
            if (p < np) {
                double* K = (double*)malloc(sizeof(double) * (size_t)((t1 - t0) * d));
                double* V = (double*)malloc(sizeof(double) * (size_t)((t1 - t0) * d));
                if (oracle_gather(K, V, k_cache, v_cache, tables + (int64_t)b * max_blocks,
                                  t0, t1, g, Hkv, d, num_blocks, kv_dtype, k_scale,
                                  v_scale, bs) != 0) bad |= 1;
                oracle_attend(op, &mp, &lp, qq, K, V, t1 - t0, d, scale);
                free(K);
                free(V);
            } else {
                for (int i = 0; i < d; ++i) op[i] = 0.0;
            }
            if (m) m[r * nslots + p] = mp;
            if (l) l[r * nslots + p] = lp;
        }
        free(qq);
    }
    return bad ? -1 : 0;
}

/* Single-pass decode.  out[r][d] for each requested row (all rows: r = b*Hq + h). */
int oracle_decode(double* out, const int32_t* rows, int32_t n_rows, const void* q,
                  int64_t q_stride, const void* k_cache, const void* v_cache,
                  const int32_t* tables, const int32_t* seq_lens, int32_t B, int32_t Hq,
                  int32_t Hkv, int32_t d, int32_t max_blocks, int64_t num_blocks,
                  double scale, int32_t q_dtype, int32_t kv_dtype, double k_scale,
                  double v_scale, int32_t nthreads, int32_t bs) {
    return decode_core(out, NULL, NULL, rows, n_rows, q, q_stride, k_cache, v_cache, tables,
                       seq_lens, B, Hq, Hkv, d, max_blocks, num_blocks, scale, q_dtype,
                       kv_dtype, k_scale, v_scale, 0, 1, nthreads, bs);
}

/* Per-partition results: o[r][max_parts][d], m[r][max_parts], l[r][max_parts];
 * partitions at or past ceil(n / part) hold o = 0, m = -inf, l = 0. */
int oracle_decode_partitions(double* o, double* m, double* l, const int32_t* rows,
                             int32_t n_rows, const void* q, int64_t q_stride,
                             const void* k_cache, const void* v_cache, const int32_t* tables,
                             const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                             int32_t d, int32_t max_blocks, int64_t num_blocks, double scale,
                             int32_t q_dtype, int32_t kv_dtype, double k_scale, double v_scale,
                             int32_t part, int32_t max_parts, int32_t nthreads, int32_t bs) {
    if (part <= 0 || max_parts <= 0) return -1;
    return decode_core(o, m, l, rows, n_rows, q, q_stride, k_cache, v_cache, tables, seq_lens,
                       B, Hq, Hkv, d, max_blocks, num_blocks, scale, q_dtype, kv_dtype,
                       k_scale, v_scale, part, max_parts, nthreads, bs);
}

/* Multi-query (chunked prefill) attention ("vLLM Nedir? ...", section "Chunked prefill";
 * "Yerel LLM ...", section "4. Prefill ve decode": a long prompt is processed in chunks
 * over several steps, each chunk's K/V joining the cache before the next).  Sequence b's
 * queries are rows q_start[b] .. q_start[b+1]-1 of q: the last L = q_start[b+1] -
 * q_start[b] of its n = seq_lens[b] positions, so query i sits at position n - L + i and
 * attends to positions 0 .. n - L + i (causal; the chunk's own K/V is already in the
 * cache).  A query whose position would be negative (L > n) gets a zero row.
 * out[r][h][d] for every query row r and head h (rows == NULL), or out[k][d] for the
 * (row, head) pairs rows[2k], rows[2k+1]. */
int oracle_prefill(double* out, const int32_t* rows, int32_t n_rows, const void* q,
                   int64_t q_stride, const int32_t* q_start, const void* k_cache,
                   const void* v_cache, const int32_t* tables, const int32_t* seq_lens,
                   int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t max_blocks,
                   int64_t num_blocks, double scale, int32_t q_dtype, int32_t kv_dtype,
                   double k_scale, double v_scale, int32_t nthreads, int32_t bs) {
    if (Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || q_dtype == OR_FP8 || bs <= 0) return -1;
    int G = Hq / Hkv;
    int64_t total_q = q_start[B];
    int64_t total = rows ? n_rows : total_q * Hq;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
#endif
    for (int64_t k = 0; k < total; ++k) {
        int64_t r = rows ? rows[2 * k] : k / Hq;
        int h = rows ? rows[2 * k + 1] : (int)(k % Hq);
        double* o = out + k * d;
        if (r < 0 || r >= total_q || h < 0 || h >= Hq) { bad |= 1; continue; }
        int b = 0;
        while (b < B && q_start[b + 1] <= r) ++b;           /* the sequence of row r */
        int64_t L = q_start[b + 1] - q_start[b], n = seq_lens[b];
        int64_t pos = n - L + (r - q_start[b]);
        if (n > (int64_t)max_blocks * bs) { bad |= 1; continue; }
        if (pos < 0) {
            for (int i = 0; i < d; ++i) o[i] = 0.0;
            continue;
        }
        double* qq = (double*)malloc(sizeof(double) * d);
        double* K = (double*)malloc(sizeof(double) * (size_t)((pos + 1) * d));
        double* V = (double*)malloc(sizeof(double) * (size_t)((pos + 1) * d));
        for (int i = 0; i < d; ++i) qq[i] = elem(q, r * q_stride + (int64_t)h * d + i, q_dtype);
        if (oracle_gather(K, V, k_cache, v_cache, tables + (int64_t)b * max_blocks, 0, pos + 1,
                          h / G, Hkv, d, num_blocks, kv_dtype, k_scale, v_scale, bs) != 0)
            bad |= 1;
        oracle_attend(o, NULL, NULL, qq, K, V, pos + 1, d, scale);
        free(qq);
        free(K);
        free(V);
    }
    return bad ? -1 : 0;
}

/* Merge of per-partition results for n_rows rows, each with n_parts[r] live
 * partitions: out = sum_p w_p o_p / sum_p w_p, w_p = exp(m_p - M) l_p, M = max m_p.
 * A row with no live partition gets o = 0. */
void oracle_merge(double* out, const double* o, const double* m, const double* l,
                  const int32_t* n_parts, int32_t n_rows, int32_t max_parts, int32_t d) {
    for (int64_t r = 0; r < n_rows; ++r) {
        double* dst = out + r * d;
        for (int i = 0; i < d; ++i) dst[i] = 0.0;
        int np = n_parts[r];
        if (np <= 0) continue;
        double M = -INFINITY;
        for (int p = 0; p < np; ++p)
            if (m[r * max_parts + p] > M) M = m[r * max_parts + p];
        double W = 0.0;
        for (int p = 0; p < np; ++p) {
            double w = exp(m[r * max_parts + p] - M) * l[r * max_parts + p];
            W += w;
            for (int i = 0; i < d; ++i) dst[i] += w * o[(r * max_parts + p) * d + i];
        }
        for (int i = 0; i < d; ++i) dst[i] /= W;
    }
}

/* Slot-mapped cache write.  With cache_dtype == dtype a raw bit copy; with an fp8
 * cache each element is quantised (k_scale for K, v_scale for V) as described at
 * the top.  Returns -1 (and writes nothing) if a slot lies outside the pool. */
int oracle_cache_write(const void* key, const void* value, void* k_cache, void* v_cache,
                       const int32_t* slot_mapping, int32_t num_tokens, int32_t Hkv, int32_t d,
                       int64_t num_blocks, int64_t key_stride, int64_t value_stride,
                       int32_t dtype, int32_t cache_dtype, float k_scale, float v_scale,
                       int32_t bs) {
    int e = elem_bytes(dtype), ce = elem_bytes(cache_dtype), x = 16 / ce;
    if (cache_dtype != dtype && (cache_dtype != OR_FP8 || dtype == OR_FP8)) return -1;
    if (bs <= 0) return -1;
    for (int t = 0; t < num_tokens; ++t)
        if ((int64_t)slot_mapping[t] >= num_blocks * bs) return -1;
    for (int t = 0; t < num_tokens; ++t) {
        int64_t s = slot_mapping[t];
        if (s < 0) continue;
        int64_t blk = s / bs;
        int off = (int)(s % bs);
        for (int g = 0; g < Hkv; ++g)
            for (int i = 0; i < d; ++i) {
                const char* ksrc = (const char*)key + (t * key_stride + (int64_t)g * d + i) * e;
                const char* vsrc = (const char*)value + (t * value_stride + (int64_t)g * d + i) * e;
                char* kdst = (char*)k_cache + k_off(blk, g, off, i, Hkv, d, x, bs) * ce;
                char* vdst = (char*)v_cache + v_off(blk, g, off, i, Hkv, d, bs) * ce;
                if (cache_dtype == OR_FP8) {
                    oracle_fp8_quantize((uint8_t*)kdst, ksrc, 1, dtype, k_scale);
                    oracle_fp8_quantize((uint8_t*)vdst, vsrc, 1, dtype, v_scale);
                } else {
                    memcpy(kdst, ksrc, (size_t)e);
                    memcpy(vdst, vsrc, (size_t)e);
                }
            }
    }
    return 0;
}
