/*
 * Oracle for paged head-dim-512 causal GQA attention.  TEST INFRASTRUCTURE
 * ONLY: the tests, the smoke check and the bench's CPU-baseline leg may call
 * it; the library under test never does, and this file shares no code with it.
 *
 * What it computes is the plain definition, written out slowly in fp32:
 *
 *   for every query row i of sequence b and query head h:
 *     pos  = q_start[b] + i            absolute position of the row
 *     n    = min(pos + 1, kv_len[b])   keys it may see (causal, bottom-right)
 *     kvh  = h / (Hq / Hkv)            consecutive GQA grouping
 *     S[j] = scale * <q[i,h,:], K[b,kvh,j,:]>   for j < n,  -inf for n <= j < kv_len
 *     o    = softmax(S) V  =  (sum_j e^{S[j]-max S} V[j]) / (sum_j e^{S[j]-max S})
 *
 * Sources for the definition:
 *  - the score row [chunk x attended_len] and its softmax are what a classical
 *    attention materialises and FlashAttention's online softmax avoids
 *    (Writing a FlashAttention Prefill Kernel for Gemma 4, intro and
 *    "The starting point"); this oracle materialises it on purpose;
 *  - a chunk attends to every key before it, including earlier chunks
 *    (pegainfer issue 1051, "Description");
 *  - keys are walked by absolute position through the page table, never by
 *    cache slot, and only the live band [0, kv_len) is read (Flash-Decoding for
 *    MQA in CUDA, "One KV head breaks the textbook");
 *  - query heads of one KV head are consecutive, so [B,1,Hq*D] and
 *    [B*Hkv, g, D] are one layout (same page and section);
 *  - FP8 keys/values are decoded from the same E4M3 bytes the kernel reads and
 *    scaled per tensor (vLLM flash-attention PR 199, review tables: errors
 *    are measured against a reference that reads the identical E4M3 data).
 *
 * The Flash-Decoding partial and merge (same page, "One KV head breaks the
 * textbook"): a key range [k0, k1) of one row gives the unnormalised
 * (O, m, l) = (sum_j e^{S[j]-m} V[j], max_j S[j], sum_j e^{S[j]-m}); partials
 * combine as  mu = max_i m_i,  o = sum_i e^{m_i-mu} O_i / sum_i e^{m_i-mu} l_i;
 * an empty range is (0, -inf, 0) and contributes nothing.
 *
 * Attention sinks and the log-sum-exp (vLLM flash-attention PR 199, second
 * review, finding F4): a head may carry a sink logit s_h, an extra softmax
 * term with no value row.  Then
 *     o   = (sum_j e^{S[j]} V[j]) / (e^{s_h} + sum_j e^{S[j]})
 *     lse = log(e^{s_h} + sum_j e^{S[j]})
 * (both evaluated around the larger of max S and s_h).  A row with no visible
 * key gives o = 0 and lse = s_h, or lse = -inf without a sink.
 *
 * Sliding-window layers and the ring cache (Flash-Decoding for MQA in CUDA,
 * "One KV head breaks the textbook": the walk is over absolute positions, the
 * slot of a position is position % capacity, and only the live band
 * [max(0, len - window), len) is read; A custom attention kernel for Gemma 4
 * on the RTX PRO 6000, "The deployment": local layers attend to the last
 * 1,024 tokens).  With a window W a row at pos sees keys
 *     max(0, pos - W + 1) <= j <= pos,  j < kv_len,
 * i.e. its own position and the W - 1 before it; with a ring of C slots, key
 * j is read from slot j % C (page table entry (j % C) / page_size), which
 * holds it as long as j >= kv_len - C.  W = 0 means no window and C = 0 an
 * unbounded cache (slot = position).
 *
 * Precision: inputs are widened exactly (bf16 -> fp32; e4m3 -> fp32, then
 * times the per-tensor scale in fp32); dot products, exponentials and sums
 * run in fp32 in plain sequential order.  Built without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { KV_BF16 = 0, KV_E4M3 = 1 };
enum { OK = 0, ERR_ARG = 1, ERR_INDEX = 2, ERR_NOMEM = 3 };

/* bf16 is the upper half of an IEEE binary32. */
static float bf16_bits_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* OCP 8-bit E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
 * no infinities; exponent 15 with mantissa 7 is NaN; exponent 0 is subnormal. */
static float e4m3_to_f32(uint8_t b) {
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 15;
    int m = b & 7;
    float mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexpf((float)m, -9);                 /* (m/8) * 2^(1-7) */
    else
        mag = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return sign ? -mag : mag;
}

void oracle_bf16_to_f32(const uint16_t* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_bits_to_f32(in[i]);
}

void oracle_e4m3_to_f32(const uint8_t* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_to_f32(in[i]);
}

typedef struct {
    const uint16_t* q;
    int64_t q_rows;
    const void* k_pool;
    const void* v_pool;
    int kv_format;
    float k_scale, v_scale;
    const int32_t* page_table;
    int max_pages, num_pages;
    const int32_t* cu_seqlens_q;
    const int32_t* q_start;
    const int32_t* kv_len;
    int batch, hq, hkv, d, page_size;
    float scale;
    int window;      /* 0: none */
    int ring_slots;  /* 0: unbounded cache */
} problem_t;

/* Index of element 0 of key (or value) row j of sequence b, KV head kvh:
 * logical key j has cache slot c = j (or j % C in a ring of C slots), which
 * lives in page page_table[b][c / page_size] at offset c % page_size. */
static int64_t kv_row_index(const problem_t* p, int b, int kvh, int j) {
    int c = p->ring_slots > 0 ? j % p->ring_slots : j;
    int page = p->page_table[(int64_t)b * p->max_pages + c / p->page_size];
    int slot = c % p->page_size;
    return (((int64_t)page * p->hkv + kvh) * p->page_size + slot) * p->d;
}

/* e4m3_to_f32 of every byte, filled once when the library is loaded: the
 * per-element decode above calls ldexpf, which made FP8 rows several times
 * slower than bf16 ones.  The table holds exactly the function's values. */
static float e4m3_table[256];
__attribute__((constructor)) static void fill_e4m3_table(void) {
    for (int b = 0; b < 256; ++b) e4m3_table[b] = e4m3_to_f32((uint8_t)b);
}

/* One stored element, dequantised to fp32. */
static float kv_load(const problem_t* p, const void* pool, int64_t idx, float tscale) {
    if (p->kv_format == KV_BF16)
        return bf16_bits_to_f32(((const uint16_t*)pool)[idx]);
    return e4m3_table[((const uint8_t*)pool)[idx]] * tscale;
}

static int seq_of_row(const problem_t* p, int64_t row) {
    int lo = 0, hi = p->batch - 1;
    while (lo < hi) { /* last b with cu[b] <= row */
        int mid = (lo + hi + 1) / 2;
        if (p->cu_seqlens_q[mid] <= row) lo = mid; else hi = mid - 1;
    }
    return lo;
}

/* Checks every page id a row could read; rejects indexes outside the pool. */
static int check_problem(const problem_t* p) {
    if (p->batch < 1 || p->hq < 1 || p->hkv < 1 || p->hq % p->hkv || p->d < 1 ||
        p->page_size < 1 || p->max_pages < 1 || p->window < 0 || p->ring_slots < 0)
        return ERR_ARG;
    if (p->cu_seqlens_q[0] != 0) return ERR_ARG;
    for (int b = 0; b < p->batch; ++b) {
        int ql = p->cu_seqlens_q[b + 1] - p->cu_seqlens_q[b];
        int L = p->kv_len[b];
        if (ql < 0 || L < 0 || p->q_start[b] < 0) return ERR_ARG;
        int slots = p->ring_slots > 0 && p->ring_slots < L ? p->ring_slots : L;
        if ((slots + p->page_size - 1) / p->page_size > p->max_pages) return ERR_INDEX;
        for (int j = 0; j < (slots + p->page_size - 1) / p->page_size; ++j) {
            int pg = p->page_table[(int64_t)b * p->max_pages + j];
            if (pg < 0 || pg >= p->num_pages) return ERR_INDEX;
        }
    }
    if (p->cu_seqlens_q[p->batch] > p->q_rows) return ERR_INDEX;
    return OK;
}

/*
 * One row, keys [k0, k1) of its sequence, unnormalised: writes O[d] and
 * returns m and l.  S is scratch of at least kv_len floats.  Keys past the
 * causal limit n carry S = -inf and weight e^{-inf} = 0.
 */
static void row_partial(const problem_t* p, int64_t row, int h, int k0, int k1, float* S,
                        float* O, float* m_out, float* l_out) {
    int b = seq_of_row(p, row);
    int i = (int)(row - p->cu_seqlens_q[b]);
    int pos = p->q_start[b] + i;
    int L = p->kv_len[b];
    int n = pos + 1 < L ? pos + 1 : L;
    int lo = p->window > 0 && pos - p->window + 1 > 0 ? pos - p->window + 1 : 0;
    int kvh = h / (p->hq / p->hkv);
    const uint16_t* qrow = p->q + (row * p->hq + h) * (int64_t)p->d;
    if (k1 > L) k1 = L;
    if (k0 < 0) k0 = 0;

    /* scores, materialised over the whole range (masked entries -inf) */
    for (int j = k0; j < k1; ++j) {
        if (j >= lo && j < n) {
            int64_t kr = kv_row_index(p, b, kvh, j);
            float dot = 0.0f;
            for (int d = 0; d < p->d; ++d)
                dot += bf16_bits_to_f32(qrow[d]) * kv_load(p, p->k_pool, kr + d, p->k_scale);
            S[j - k0] = p->scale * dot;
        } else {
            S[j - k0] = -INFINITY;
        }
    }
    float m = -INFINITY;
    for (int j = k0; j < k1; ++j)
        if (S[j - k0] > m) m = S[j - k0];
    for (int d = 0; d < p->d; ++d) O[d] = 0.0f;
    float l = 0.0f;
    if (m == -INFINITY) { /* no visible key in the range */
        *m_out = m;
        *l_out = 0.0f;
        return;
    }
    for (int j = k0; j < k1; ++j) {
        float e = expf(S[j - k0] - m);
        S[j - k0] = e;
        l += e;
    }
    /* masked keys (j < lo, j >= n) have weight exactly zero and are left out */
    for (int j = (k0 > lo ? k0 : lo); j < (k1 < n ? k1 : n); ++j) {
        float e = S[j - k0];
        int64_t vr = kv_row_index(p, b, kvh, j);
        for (int d = 0; d < p->d; ++d)
            O[d] += e * kv_load(p, p->v_pool, vr + d, p->v_scale);
    }
    *m_out = m;
    *l_out = l;
}

#define FILL_PROBLEM                                                                     \
    problem_t p = {q, q_rows, k_pool, v_pool, kv_format, k_scale, v_scale, page_table,   \
                   max_pages, num_pages, cu_seqlens_q, q_start, kv_len, batch, hq, hkv,  \
                   head_dim, page_size, softmax_scale, 0, 0};

/* Normalises one row's (O, m, l) with an optional sink logit (NAN = none):
 * writes o[d] and, when lse is not NULL, the log-sum-exp. */
static void finish_row(const float* O, float m, float l, float sink, int d_len, float* o,
                       float* lse) {
    float top = m;
    if (!isnan(sink) && sink > top) top = sink;
    if (top == -INFINITY) { /* nothing visible and no sink */
        for (int d = 0; d < d_len; ++d) o[d] = 0.0f;
        if (lse) *lse = -INFINITY;
        return;
    }
    float w = (m == -INFINITY) ? 0.0f : expf(m - top); /* rescales O and l to `top` */
    float den = w * l + (isnan(sink) ? 0.0f : expf(sink - top));
    for (int d = 0; d < d_len; ++d) o[d] = (w * O[d]) / den;
    if (lse) *lse = top + logf(den);
}

/*
 * out[r, :] = attention output of entry rows[r] = q_row * Hq + head, and, when
 * lse is not NULL, lse[r] = its log-sum-exp.  sinks (NULL = none) holds one
 * logit per query head.  A row with no visible key gives 0 (lse = the sink,
 * or -inf).  Returns 0, or an error code without writing anything when an
 * argument or a page id is out of range.
 */
int oracle_attn_rows_full(const uint16_t* q, int64_t q_rows, const void* k_pool,
                          const void* v_pool, int kv_format, float k_scale, float v_scale,
                          const int32_t* page_table, int max_pages, int num_pages,
                          const int32_t* cu_seqlens_q, const int32_t* q_start,
                          const int32_t* kv_len, int batch, int hq, int hkv, int head_dim,
                          int page_size, float softmax_scale, int window, int ring_slots,
                          const float* sinks, const int64_t* rows, int64_t n_rows, float* out,
                          float* lse, int num_threads) {
    FILL_PROBLEM
    p.window = window;
    p.ring_slots = ring_slots;
    int rc = check_problem(&p);
    if (rc) return rc;
    int total_q = cu_seqlens_q[batch];
    int maxL = 0;
    for (int b = 0; b < batch; ++b) if (kv_len[b] > maxL) maxL = kv_len[b];
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= (int64_t)total_q * hq) return ERR_INDEX;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
    int failed = 0;
#pragma omp parallel
    {
        float* S = (float*)malloc(sizeof(float) * (size_t)(maxL > 0 ? maxL : 1));
        float* O = (float*)malloc(sizeof(float) * (size_t)head_dim);
        if (!S || !O) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t row = rows[r] / hq;
                int h = (int)(rows[r] % hq);
                int b = seq_of_row(&p, row);
                float m, l;
                row_partial(&p, row, h, 0, kv_len[b], S, O, &m, &l);
                finish_row(O, m, l, sinks ? sinks[h] : NAN, head_dim,
                           out + r * (int64_t)head_dim, lse ? lse + r : NULL);
            }
        }
        free(S);
        free(O);
    }
    return failed ? ERR_NOMEM : OK;
}

/* oracle_attn_rows_full without a window, over an unbounded cache. */
int oracle_attn_rows_ex(const uint16_t* q, int64_t q_rows, const void* k_pool,
                        const void* v_pool, int kv_format, float k_scale, float v_scale,
                        const int32_t* page_table, int max_pages, int num_pages,
                        const int32_t* cu_seqlens_q, const int32_t* q_start,
                        const int32_t* kv_len, int batch, int hq, int hkv, int head_dim,
                        int page_size, float softmax_scale, const float* sinks,
                        const int64_t* rows, int64_t n_rows, float* out, float* lse,
                        int num_threads) {
    return oracle_attn_rows_full(q, q_rows, k_pool, v_pool, kv_format, k_scale, v_scale,
                                 page_table, max_pages, num_pages, cu_seqlens_q, q_start,
                                 kv_len, batch, hq, hkv, head_dim, page_size, softmax_scale, 0,
                                 0, sinks, rows, n_rows, out, lse, num_threads);
}

/* oracle_attn_rows_ex without sinks and without the log-sum-exp. */
int oracle_attn_rows(const uint16_t* q, int64_t q_rows, const void* k_pool, const void* v_pool,
                     int kv_format, float k_scale, float v_scale, const int32_t* page_table,
                     int max_pages, int num_pages, const int32_t* cu_seqlens_q,
                     const int32_t* q_start, const int32_t* kv_len, int batch, int hq, int hkv,
                     int head_dim, int page_size, float softmax_scale, const int64_t* rows,
                     int64_t n_rows, float* out, int num_threads) {
    return oracle_attn_rows_ex(q, q_rows, k_pool, v_pool, kv_format, k_scale, v_scale,
                               page_table, max_pages, num_pages, cu_seqlens_q, q_start, kv_len,
                               batch, hq, hkv, head_dim, page_size, softmax_scale, NULL, rows,
                               n_rows, out, NULL, num_threads);
}

/* Unnormalised partial of one row (q_row, head) over keys [k0, k1). */
int oracle_attn_partial(const uint16_t* q, int64_t q_rows, const void* k_pool,
                        const void* v_pool, int kv_format, float k_scale, float v_scale,
                        const int32_t* page_table, int max_pages, int num_pages,
                        const int32_t* cu_seqlens_q, const int32_t* q_start,
                        const int32_t* kv_len, int batch, int hq, int hkv, int head_dim,
                        int page_size, float softmax_scale, int64_t q_row, int head, int k0,
                        int k1, float* O, float* m, float* l) {
    FILL_PROBLEM
    int rc = check_problem(&p);
    if (rc) return rc;
    if (q_row < 0 || q_row >= cu_seqlens_q[batch] || head < 0 || head >= hq) return ERR_INDEX;
    int b = seq_of_row(&p, q_row);
    float* S = (float*)malloc(sizeof(float) * (size_t)(kv_len[b] > 0 ? kv_len[b] : 1));
    if (!S) return ERR_NOMEM;
    row_partial(&p, q_row, head, k0, k1, S, O, m, l);
    free(S);
    return OK;
}

/* Merge n partials (O_i [d], m_i, l_i) into one normalised output row, with
 * an optional sink logit (NAN = none) and log-sum-exp (lse may be NULL). */
void oracle_merge_ex(const float* O, const float* m, const float* l, int n, int head_dim,
                     float sink, float* out, float* lse) {
    float mu = -INFINITY;
    for (int i = 0; i < n; ++i) if (m[i] > mu) mu = m[i];
    float* acc = (float*)calloc((size_t)head_dim, sizeof(float));
    float den = 0.0f;
    if (mu != -INFINITY) {
        for (int i = 0; i < n; ++i) {
            if (m[i] == -INFINITY) continue; /* empty split: identity */
            float w = expf(m[i] - mu);
            den += w * l[i];
            for (int d = 0; d < head_dim; ++d) acc[d] += w * O[(int64_t)i * head_dim + d];
        }
    }
    /* the merged partial is (acc, mu, den); normalise it like one row */
    finish_row(acc, mu, den, sink, head_dim, out, lse);
    free(acc);
}

/* oracle_merge_ex without a sink and without the log-sum-exp. */
void oracle_merge(const float* O, const float* m, const float* l, int n, int head_dim,
                  float* out) {
    oracle_merge_ex(O, m, l, n, head_dim, NAN, out, NULL);
}
