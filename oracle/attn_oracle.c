/*
 * attn_oracle.c -- CPU fp64 oracle for paged grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * GPU library is checked against.  Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load it.  It shares no code,
 * header, table or constant with the GPU library (paged_kv_cache_20_amd/),
 * and the library never calls it.
 *
 * What it computes (the pages print no attention arithmetic, so the core is
 * the textbook definition of scaled dot-product attention written out):
 *
 *   for query row r of sequence s and query head h:
 *     kh    = h / (n_head / n_head_kv)           contiguous GQA groups
 *     last  = ctx_len[s] - R + r                 last key position it sees
 *     score_t = (q . k_t) / sqrt(head_dim)       t = 0 .. last
 *     out     = sum_t exp(score_t - max) v_t / sum_t exp(score_t - max)
 *
 * Problem statement taken from the pages:
 *  - "kern manifest v7" schema, $defs.Batch: a call carries `rows` rows per
 *    sequence -- 1 for a decode step, exactly 8 for a speculative round, or
 *    the chunk's row count for a prefill chunk (one sequence).
 *  - same schema, $defs.Fill "seq_len": a sequence's length counts the rows
 *    already in the state plus this call's, so the call's own rows are the
 *    last R positions of the context and row r sits at ctx_len - R + r.
 *  - same schema, $defs.Domain: a paged KV block table indexes pages of
 *    `stride` (16) token slots; token t of a sequence lives in page
 *    table[t / P] at offset t % P.
 *  - "Radiance Architecture Plugins -- declaring a model", section
 *    "Declare: the metadata": head_dim is an input, never derived from the
 *    hidden size and head count.
 *  - same page, section "Declare: buffers and KV groups": the full KV group
 *    is a paged, per-token, growing cache.
 *
 * Storage decoding is exact: a bf16 value is the top half of an IEEE single;
 * an fp8 code is decoded from the OCP E4M3 ("E4M3FN") definition -- 1 sign,
 * 4 exponent bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 is
 * NaN, exponent 0 is subnormal m * 2^-9 -- and multiplied by its page's fp32
 * scale in double precision (4 significant bits times 24 is exact).
 *
 * fp8 quantisation (the append oracle) follows the reading stated with
 * oracle_kv_append below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_KV_BF16 = 0, ORC_KV_FP8 = 1 };

static double orc_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP E4M3 value of a code, from the format definition. */
double oracle_e4m3_value(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                 /* subnormal: m/8 * 2^-6 */
    else
        v = ldexp(1.0 + m / 8.0, e - 7);         /* normal: (1 + m/8) 2^(e-7) */
    return sign ? -v : v;
}

/* Values of all 256 codes, filled from oracle_e4m3_value before use. */
static double orc_e4m3_tab[256];
static int orc_e4m3_tab_ready = 0;

static void orc_e4m3_init(void)
{
    if (orc_e4m3_tab_ready)
        return;
    for (int c = 0; c < 256; ++c)
        orc_e4m3_tab[c] = oracle_e4m3_value((uint8_t)c);
    orc_e4m3_tab_ready = 1;
}

typedef struct {
    const void *k_pool, *v_pool;
    const float *k_scale, *v_scale;
    int64_t n_pages;
    const int32_t *block_table;
    int max_pages, n_head_kv, d, P, kv_dtype;
} orc_pool;

/* One stored K or V element of token slot (page, kh, off), as a double. */
static double orc_elem(const orc_pool *pl, int is_v, int64_t page, int kh, int off, int i)
{
    int64_t idx = ((page * pl->n_head_kv + kh) * (int64_t)pl->P + off) * pl->d + i;
    if (pl->kv_dtype == ORC_KV_BF16) {
        const uint16_t *p = (const uint16_t *)(is_v ? pl->v_pool : pl->k_pool);
        return orc_bf16(p[idx]);
    } else {
        const uint8_t *p = (const uint8_t *)(is_v ? pl->v_pool : pl->k_pool);
        const float *sc = is_v ? pl->v_scale : pl->k_scale;
        return orc_e4m3_tab[p[idx]] * (double)sc[page * pl->n_head_kv + kh];
    }
}

/*
 * Attention of one query vector over key positions first..last of sequence
 * seq, kv head kh.  Writes d doubles to out.  Returns 0, or -1 when a
 * block-table entry that the row needs is outside the pool.  (scores is
 * indexed by absolute position; entries below first are not used.)
 */
static int orc_attend(const orc_pool *pl, const double *q, int seq, int64_t first, int64_t last,
                      int kh, double *scores, double *out)
{
    const int d = pl->d, P = pl->P;
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    int64_t t;
    int i;
    for (t = first; t <= last; ++t) {
        int64_t page = pl->block_table[(int64_t)seq * pl->max_pages + t / P];
        double dot = 0.0;
        if (page < 0 || page >= pl->n_pages)
            return -1;
        for (i = 0; i < d; ++i)
            dot += q[i] * orc_elem(pl, 0, page, kh, (int)(t % P), i);
        scores[t] = dot * inv_sqrt_d;
    }
    double mx = -INFINITY;
    for (t = first; t <= last; ++t)
        if (scores[t] > mx)
            mx = scores[t];
    double z = 0.0;
    for (t = first; t <= last; ++t) {
        scores[t] = exp(scores[t] - mx);
        z += scores[t];
    }
    for (i = 0; i < d; ++i)
        out[i] = 0.0;
    for (t = first; t <= last; ++t) {
        int64_t page = pl->block_table[(int64_t)seq * pl->max_pages + t / P];
        double w = scores[t] / z;
        for (i = 0; i < d; ++i)
            out[i] += w * orc_elem(pl, 1, page, kh, (int)(t % P), i);
    }
    return 0;
}

/*
 * oracle_paged_attention -- every call shape at once.
 *
 *   q         bf16 bits [n_seq][rows][n_head][head_dim]
 *   rows      R: 1 (decode), 8 (verify round), or the chunk length with
 *             n_seq = 1 (prefill chunk)
 *   ctx_lens  [n_seq] length of each sequence after this call
 *   row_mask  [n_seq*rows] nonzero = compute that row, or NULL for all rows
 *   out       fp64 [n_seq][rows][n_head][head_dim]; rows not computed are
 *             left untouched
 *
 * Returns 0, -1 for a bad shape, -2 for a row whose context is shorter than
 * the call's rows or longer than its block-table row, -3 for a block-table
 * entry outside the pool.
 */
/*
 * oracle_paged_attention_window -- the same with a lower bound on the keys
 * a row attends ("Radiance Architecture Plugins -- declaring a model",
 * section "Declare: buffers and KV groups": a KV group bounded by a window,
 * and a ring whose window floor is set at runtime).  The row at position p
 * attends keys max(kv_floor[s], p - window + 1) .. p; window 0 means no
 * window, kv_floor NULL a floor of 0.  Returns -2 also for a floor outside
 * 0 .. ctx_lens[s] - rows.  Block-table entries below a row's first key are
 * not read.
 */
int oracle_paged_attention_window(const uint16_t *q, int n_seq, int rows,
                                  const void *k_pool, const void *v_pool,
                                  const float *k_scale, const float *v_scale, int64_t n_pages,
                                  const int32_t *block_table, int max_pages,
                                  const int32_t *ctx_lens, int n_head, int n_head_kv,
                                  int head_dim, int page_size, int kv_dtype, int window,
                                  const int32_t *kv_floor, const uint8_t *row_mask, double *out,
                                  int n_threads)
{
    if (n_seq <= 0 || rows <= 0 || n_head <= 0 || n_head_kv <= 0 || head_dim <= 0 ||
        page_size <= 0 || n_head % n_head_kv != 0)
        return -1;
    orc_e4m3_init();
    orc_pool pl = {k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                   max_pages, n_head_kv, head_dim, page_size, kv_dtype};
    const int g = n_head / n_head_kv;
    int64_t max_ctx = 0;
    if (window < 0)
        return -1;
    for (int s = 0; s < n_seq; ++s) {
        if (ctx_lens[s] < rows || (int64_t)ctx_lens[s] > (int64_t)max_pages * page_size)
            return -2;
        if (kv_floor && (kv_floor[s] < 0 || kv_floor[s] > ctx_lens[s] - rows))
            return -2;
        if (ctx_lens[s] > max_ctx)
            max_ctx = ctx_lens[s];
    }
    const int64_t n_items = (int64_t)n_seq * rows * n_head;
    int status = 0;
    if (n_threads <= 0)
        n_threads = 1;
#pragma omp parallel num_threads(n_threads)
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)max_ctx);
        double *qrow = (double *)malloc(sizeof(double) * (size_t)head_dim);
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < n_items; ++it) {
            const int h = (int)(it % n_head);
            const int64_t sr = it / n_head; /* s * rows + r */
            const int r = (int)(sr % rows), s = (int)(sr / rows);
            if (row_mask && !row_mask[sr])
                continue;
            const uint16_t *qv = q + it * head_dim;
            for (int i = 0; i < head_dim; ++i)
                qrow[i] = orc_bf16(qv[i]);
            const int64_t last = (int64_t)ctx_lens[s] - rows + r;
            int64_t first = kv_floor ? kv_floor[s] : 0;
            if (window > 0 && last - window + 1 > first)
                first = last - window + 1;
            if (orc_attend(&pl, qrow, s, first, last, h / g, scores, out + it * head_dim) != 0) {
#pragma omp atomic write
                status = -3;
            }
        }
        free(scores);
        free(qrow);
    }
    return status;
}

int oracle_paged_attention(const uint16_t *q, int n_seq, int rows,
                           const void *k_pool, const void *v_pool,
                           const float *k_scale, const float *v_scale, int64_t n_pages,
                           const int32_t *block_table, int max_pages,
                           const int32_t *ctx_lens, int n_head, int n_head_kv,
                           int head_dim, int page_size, int kv_dtype,
                           const uint8_t *row_mask, double *out, int n_threads)
{
    return oracle_paged_attention_window(q, n_seq, rows, k_pool, v_pool, k_scale, v_scale,
                                         n_pages, block_table, max_pages, ctx_lens, n_head,
                                         n_head_kv, head_dim, page_size, kv_dtype, 0, NULL,
                                         row_mask, out, n_threads);
}

/* ---------------------------------------------------------------------- */
/* fp8 quantisation                                                        */
/* ---------------------------------------------------------------------- */

/*
 * Nearest E4M3 code to the fp32 value y, ties to the code with an even
 * mantissa, magnitudes above the largest finite value (448) saturating to it.
 * Plain search over the 127 non-negative finite codes, whose values increase
 * with the code.
 */
uint8_t oracle_e4m3_encode(float y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0; /* -0 keeps its sign, like any negative */
    double a = fabs((double)y);
    if (isnan(y))
        return 0x7F;
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    orc_e4m3_init();
    int lo = 0, hi = 126; /* value(lo) <= a < value(hi) once narrowed */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (orc_e4m3_tab[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    double vlo = orc_e4m3_tab[lo], vhi = orc_e4m3_tab[hi];
    int pick;
    if (a - vlo < vhi - a)
        pick = lo;
    else if (a - vlo > vhi - a)
        pick = hi;
    else
        pick = (lo & 1) ? hi : lo; /* tie: even code, i.e. even mantissa */
    return (uint8_t)(sign | pick);
}

/*
 * oracle_round_q_e4m3 -- the query vectors of an fp8 prefill, rounded to
 * E4M3 ("Radiance Architecture Plugins -- declaring a model", section
 * "Declare: the metadata": the build context carries `attn_prefill_fp8` bits
 * that the attention op takes as `prefill_fp8`).  The pages name the switch
 * only; the reading here is the plainest one that keeps every step exact
 * except the rounding itself:
 *
 *   per vector (one query row of one head, head_dim values):
 *     amax = max_d |q_d|
 *     e    = the smallest integer with amax <= 448 * 2^e, and at least -117
 *            (so every rounded value below stays a normal number; an
 *            all-zero vector takes -117)
 *     q'_d = 2^e * value(nearest E4M3 code of q_d / 2^e, ties to even)
 *
 * q_d / 2^e lies in [-448, 448], so no code saturates; q'_d has at most 4
 * significant bits and is exact in bf16.
 *
 *   q, out   bf16 bits [n_vec][head_dim]
 *   exps     [n_vec] receives e (may be NULL)
 * Returns 0, or -1 for a non-finite input element.
 */
int oracle_round_q_e4m3(const uint16_t *q, int64_t n_vec, int32_t head_dim, uint16_t *out,
                        int32_t *exps)
{
    if (!q || !out || n_vec < 0 || head_dim <= 0)
        return -1;
    for (int64_t v = 0; v < n_vec; ++v) {
        const uint16_t *x = q + v * head_dim;
        double amax = 0.0;
        for (int d = 0; d < head_dim; ++d) {
            const double a = fabs(orc_bf16(x[d]));
            if (!isfinite(a))
                return -1;
            if (a > amax)
                amax = a;
        }
        int e = -117;
        if (amax > 0.0) {
            int ex;
            const double m = frexp(amax, &ex); /* amax = m 2^ex, m in [0.5, 1) */
            /* 448 = 0.875 * 2^9: amax <= 448 * 2^e  <=>  m 2^ex <= 0.875 2^(9+e) */
            e = m <= 0.875 ? ex - 9 : ex - 8;
            if (e < -117)
                e = -117;
        }
        if (exps)
            exps[v] = e;
        for (int d = 0; d < head_dim; ++d) {
            const double y = ldexp(orc_bf16(x[d]), -e); /* exact */
            const uint8_t c = oracle_e4m3_encode((float)y);
            orc_e4m3_init();
            const float r = (float)ldexp(orc_e4m3_tab[c & 0x7F], e); /* exact */
            uint32_t u;
            memcpy(&u, &r, sizeof u);
            u |= (uint32_t)(c & 0x80) << 24;
            out[v * head_dim + d] = (uint16_t)(u >> 16);
        }
    }
    return 0;
}

/*
 * oracle_kv_append -- write n_tok new K/V rows into their token slots.
 *
 *   k_new, v_new  bf16 bits [n_tok][n_head_kv][head_dim]
 *   slot_mapping  [n_tok] slot = page * page_size + offset ("kern manifest v7"
 *                 schema, $defs.Fill "slot": a row's token slot in the paged
 *                 state); a negative slot skips the row
 *   pools         [n_pages][n_head_kv][page_size][head_dim], bf16 bits or
 *                 E4M3 codes; scales fp32 [n_pages][n_head_kv] (fp8 only)
 *
 * bf16: a plain copy into the slot.
 * fp8: one fp32 scale per (page, kv head), separately for K and for V, equal
 * to absmax / 448 ("one fp32 scale per page per KV head (absmax/448)"), where
 * absmax runs over every element of this call's rows that land in that page
 * and head.  A call that writes the page's first slot (offset 0) sets the
 * scale from its own rows (a zero absmax gives scale 1).  A call that writes
 * only later slots keeps the stored scale s while its rows fit (fp32 absmax
 * / s <= 448); otherwise the scale doubles until they fit (s' = s * 2^k,
 * the least k >= 1 with fp32 absmax / s' <= 448; a non-finite absmax never
 * grows it) and the codes already in the page's slots below the call's first
 * one are re-encoded at s': code' = nearest E4M3 to fp32(fp32(value(code) *
 * s) / s'), which is exact for every code that stays a normal number.  Each
 * new element's code is the nearest E4M3 value to the fp32 quotient x /
 * scale.
 *
 * Returns 0, or -1 for a slot outside the pool.
 */
int oracle_kv_append(const uint16_t *k_new, const uint16_t *v_new,
                     const int32_t *slot_mapping, int n_tok,
                     void *k_pool, void *v_pool, float *k_scale, float *v_scale,
                     int64_t n_pages, int n_head_kv, int head_dim, int page_size,
                     int kv_dtype)
{
    const int64_t row = (int64_t)n_head_kv * head_dim; /* elements per token */
    for (int t = 0; t < n_tok; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot >= (int64_t)n_pages * page_size)
            return -1;
    }
    if (kv_dtype == ORC_KV_BF16) {
        for (int t = 0; t < n_tok; ++t) {
            int64_t slot = slot_mapping[t];
            if (slot < 0)
                continue;
            int64_t page = slot / page_size, off = slot % page_size;
            for (int h = 0; h < n_head_kv; ++h)
                for (int i = 0; i < head_dim; ++i) {
                    int64_t dst = ((page * n_head_kv + h) * page_size + off) * head_dim + i;
                    ((uint16_t *)k_pool)[dst] = k_new[t * row + (int64_t)h * head_dim + i];
                    ((uint16_t *)v_pool)[dst] = v_new[t * row + (int64_t)h * head_dim + i];
                }
        }
        return 0;
    }
    /* fp8: first the scales of the pages this call writes: the first slot
       each page receives (page_size if none), absmax over every row of the
       call that lands in the page, then a new scale from offset 0, or a grown
       scale (with the earlier slots' codes re-encoded), or the stored one. */
    {
        int *first = (int *)malloc(sizeof(int) * (size_t)n_pages);
        float *amax = (float *)calloc((size_t)(n_pages * n_head_kv), sizeof(float));
        for (int64_t page = 0; page < n_pages; ++page)
            first[page] = page_size;
        for (int t = 0; t < n_tok; ++t) {
            int64_t slot = slot_mapping[t];
            if (slot >= 0 && slot % page_size < first[slot / page_size])
                first[slot / page_size] = (int)(slot % page_size);
        }
        for (int kv = 0; kv < 2; ++kv) {
            const uint16_t *src = kv ? v_new : k_new;
            float *scale = kv ? v_scale : k_scale;
            uint8_t *pool = (uint8_t *)(kv ? v_pool : k_pool);
            memset(amax, 0, sizeof(float) * (size_t)(n_pages * n_head_kv));
            for (int t = 0; t < n_tok; ++t) {
                int64_t slot = slot_mapping[t];
                if (slot < 0)
                    continue;
                int64_t page = slot / page_size;
                for (int h = 0; h < n_head_kv; ++h)
                    for (int i = 0; i < head_dim; ++i) {
                        float x = fabsf((float)orc_bf16(src[t * row + (int64_t)h * head_dim + i]));
                        if (x > amax[page * n_head_kv + h])
                            amax[page * n_head_kv + h] = x;
                    }
            }
            for (int64_t page = 0; page < n_pages; ++page) {
                if (first[page] == page_size)
                    continue; /* not written by this call */
                for (int h = 0; h < n_head_kv; ++h) {
                    float a = amax[page * n_head_kv + h];
                    float *sc = &scale[page * n_head_kv + h];
                    if (first[page] == 0) {
                        *sc = a > 0.0f ? a / 448.0f : 1.0f;
                    } else if (a <= 3.4028234663852886e38f && a / *sc > 448.0f) {
                        float s_old = *sc, s_new = s_old;
                        while (a / s_new > 448.0f)
                            s_new = s_new * 2.0f;
                        for (int off = 0; off < first[page]; ++off)
                            for (int i = 0; i < head_dim; ++i) {
                                uint8_t *c =
                                    &pool[((page * n_head_kv + h) * page_size + off) * head_dim + i];
                                float y = (float)oracle_e4m3_value(*c) * s_old;
                                *c = oracle_e4m3_encode(y / s_new);
                            }
                        *sc = s_new;
                    }
                }
            }
        }
        free(first);
        free(amax);
    }
    /* then every row's codes, with its page's scale. */
    for (int kv = 0; kv < 2; ++kv) {
        const uint16_t *src = kv ? v_new : k_new;
        float *scale = kv ? v_scale : k_scale;
        uint8_t *pool = (uint8_t *)(kv ? v_pool : k_pool);
        for (int t = 0; t < n_tok; ++t) {
            int64_t slot = slot_mapping[t];
            if (slot < 0)
                continue;
            int64_t page = slot / page_size, off = slot % page_size;
            for (int h = 0; h < n_head_kv; ++h) {
                float sc = scale[page * n_head_kv + h];
                for (int i = 0; i < head_dim; ++i) {
                    float x = (float)orc_bf16(src[t * row + (int64_t)h * head_dim + i]);
                    float y = x / sc;
                    pool[((page * n_head_kv + h) * page_size + off) * head_dim + i] =
                        oracle_e4m3_encode(y);
                }
            }
        }
    }
    return 0;
}

/*
 * oracle_tree_view -- the cache that row r of a tree-shaped speculative round
 * attends ("Radiance Architecture Plugins -- declaring a model", section
 * "Declare: drafters, encoders, generators": a drafter may propose a tree;
 * "TandemLLM -- Adding a model", section "The adapter path in ten steps": a
 * recorded decode replayed as trees must match row for row).
 *
 *   pools, scales  the cache, as for oracle_paged_attention
 *   table_row      the sequence's block-table row (max_pages entries)
 *   ctx_len, rows  C and R: the round's rows sit at C0 .. C0 + R - 1, C0 = C - R
 *   mask, r        bit j set = row r attends round row j; a valid mask names r
 *                  and no later row
 *   out_*          the view: pages 0 .. out_pages - 1 of a private cache whose
 *                  block table is the identity; slots past the view's length
 *                  are zero
 *
 * The view holds the context positions 0 .. C0 - 1 followed by the round rows
 * the mask names, in row order, at C0, C0 + 1, ... (the branch laid out as a
 * plain sequence).  bf16: every token's bytes are copied.  fp8: a view page
 * takes the scale of the cache page that holds its first token (its home
 * page); tokens from the home page keep their codes; a token from another
 * page (possible only where a round crosses a page boundary and the branch
 * skips rows, so a later row moves down into the earlier page) is written as
 * kv_append would write a new row into that page at a later call: its value
 * y = fp32(value(code) * its page's scale) is encoded at the view page's
 * scale, which first doubles while fp32 absmax(y) / scale > 448 (the home
 * tokens are then re-encoded too, code' = nearest E4M3 to fp32(fp32(value *
 * s) / s')).  A chain mask therefore gives the cache itself, byte for byte.
 *
 * Returns the view's length, -1 for an invalid mask or length, -2 for a page
 * outside the pool, -3 when out_pages is too small.
 */
int oracle_tree_view(const void *k_pool, const void *v_pool, const float *k_scale,
                     const float *v_scale, int64_t n_pages, const int32_t *table_row,
                     int max_pages, int ctx_len, int rows, uint32_t mask, int r, int n_head_kv,
                     int head_dim, int page_size, int kv_dtype, void *out_k, void *out_v,
                     float *out_ks, float *out_vs, int out_pages)
{
    const int P = page_size, d = head_dim, Hk = n_head_kv;
    if (rows < 1 || rows > 32 || r < 0 || r >= rows || ctx_len < rows ||
        (int64_t)ctx_len > (int64_t)max_pages * P)
        return -1;
    if (!(mask >> r & 1u) || (r + 1 < 32 && (mask >> (r + 1)) != 0))
        return -1;
    const int C0 = ctx_len - rows;
    int L = C0;
    for (int j = 0; j < rows; ++j)
        L += (int)(mask >> j & 1u);
    const int npg = (L + P - 1) / P;
    if (npg > out_pages)
        return -3;
    /* pos[t]: cache position of view position t */
    int *pos = (int *)malloc(sizeof(int) * (size_t)L);
    for (int t = 0; t < C0; ++t)
        pos[t] = t;
    for (int j = 0, t = C0; j < rows; ++j)
        if (mask >> j & 1u)
            pos[t++] = C0 + j;
    for (int t = 0; t < L; ++t) {
        const int32_t pg = table_row[pos[t] / P];
        if (pg < 0 || (int64_t)pg >= n_pages) {
            free(pos);
            return -2;
        }
    }
    const size_t eb = kv_dtype == ORC_KV_BF16 ? 2 : 1;
    const int64_t row_el = d, page_el = (int64_t)Hk * P * d;
    memset(out_k, 0, eb * (size_t)(out_pages * page_el));
    memset(out_v, 0, eb * (size_t)(out_pages * page_el));
    if (kv_dtype == ORC_KV_BF16) {
        for (int t = 0; t < L; ++t) {
            const int64_t sp = table_row[pos[t] / P], so = pos[t] % P;
            for (int h = 0; h < Hk; ++h)
                for (int i = 0; i < d; ++i) {
                    const int64_t src = (sp * Hk + h) * P * row_el + so * row_el + i;
                    const int64_t dst = ((int64_t)(t / P) * Hk + h) * P * row_el + (t % P) * row_el + i;
                    ((uint16_t *)out_k)[dst] = ((const uint16_t *)k_pool)[src];
                    ((uint16_t *)out_v)[dst] = ((const uint16_t *)v_pool)[src];
                }
        }
        free(pos);
        return L;
    }
    for (int kv = 0; kv < 2; ++kv) {
        const uint8_t *pool = (const uint8_t *)(kv ? v_pool : k_pool);
        const float *scale = kv ? v_scale : k_scale;
        uint8_t *out = (uint8_t *)(kv ? out_v : out_k);
        float *out_s = kv ? out_vs : out_ks;
        for (int vp = 0; vp < npg; ++vp) {
            const int t_lo = vp * P, t_hi = L < t_lo + P ? L : t_lo + P;
            const int64_t home = table_row[pos[t_lo] / P];
            for (int h = 0; h < Hk; ++h) {
                const float s_home = scale[home * Hk + h];
                /* absmax of the moved tokens' values */
                float a = 0.0f;
                for (int t = t_lo; t < t_hi; ++t) {
                    const int64_t sp = table_row[pos[t] / P];
                    if (sp == home)
                        continue;
                    const float s = scale[sp * Hk + h];
                    for (int i = 0; i < d; ++i) {
                        const uint8_t c = pool[((sp * Hk + h) * P + pos[t] % P) * row_el + i];
                        const float y = fabsf((float)oracle_e4m3_value(c) * s);
                        if (y > a)
                            a = y;
                    }
                }
                float s_view = s_home;
                if (a <= 3.4028234663852886e38f && a / s_home > 448.0f)
                    while (a / s_view > 448.0f)
                        s_view = s_view * 2.0f;
                const int grown = s_view != s_home;
                for (int t = t_lo; t < t_hi; ++t) {
                    const int64_t sp = table_row[pos[t] / P];
                    const float s = scale[sp * Hk + h];
                    const int moved = sp != home;
                    for (int i = 0; i < d; ++i) {
                        const uint8_t c = pool[((sp * Hk + h) * P + pos[t] % P) * row_el + i];
                        uint8_t c2 = c;
                        if (moved || grown) {
                            const float y = (float)oracle_e4m3_value(c) * s;
                            c2 = oracle_e4m3_encode(y / s_view);
                        }
                        out[(((int64_t)vp * Hk + h) * P + (t % P)) * row_el + i] = c2;
                    }
                }
                out_s[(int64_t)vp * Hk + h] = s_view;
            }
        }
        /* pages of the view past its length keep scale 1 */
        for (int vp = npg; vp < out_pages; ++vp)
            for (int h = 0; h < Hk; ++h)
                out_s[(int64_t)vp * Hk + h] = 1.0f;
    }
    free(pos);
    return L;
}
