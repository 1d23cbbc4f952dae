/*
 * CPU fp64 oracle for length-aware decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header, table or helper with the HIP
 * library: it is the plain definition of masked softmax attention, written
 * out, with no blocking, fusion or reordering.
 *
 * What it computes (one result per batch entry b, query i, query head h):
 *
 *   g    = h / G, G = Hq / Hkv            consecutive query heads share a KV
 *                                         head (the packed GQA group of
 *                                         ComfyUI issue "Qwen3.5 text
 *                                         generation attends over the full KV
 *                                         capacity every step…", Feature Idea)
 *   L    = clamp(kv_lens[b], 0, cap)      only the filled prefix is attended
 *                                         (same page, Feature Idea: the
 *                                         device-side seqlen bounds the read)
 *   lim  = causal ? clamp(L - n_q + i + 1, 0, L) : L
 *                                         bottom-right aligned causal window:
 *                                         each verification query sees the
 *                                         cache plus the drafts before it
 *                                         (same page, Feature Idea and
 *                                         Existing Solutions)
 *   visible set V:
 *     dense : { j in [0, lim) : keep_mask == NULL || keep_mask[b,i,g,j] != 0 }
 *             in increasing j
 *     gather: [ idx[b,i,g,t] for t in 0..W-1 if 0 <= idx < lim ] in list
 *             order (llama.cpp PR "qwen4exp: attend the selected cells
 *             instead of masking the window", PR body: the selected cells
 *             are gathered into a window of their own and the mask is taken
 *             at those cells; llama.cpp PR "qwen4exp : gather-based sparse
 *             attention for QSA decode", Overview)
 *     steps : (k_step/v_step given, dense, non-causal, no mask) the cache
 *             cells j in [0, L), then the query's own step rows t = 0..i of
 *             k_step/v_step [B, n_q, Hkv, D]: the verification drafts are
 *             not written into the cache; each query sees the whole prefix
 *             plus the drafts up to itself, and the two parts are merged
 *             (comfy-kitchen PR "Performance improvements for qwen 3.x LLM
 *             (Part 1)", commit list: causal step rows merged into prefix
 *             attention).  It equals the causal window over a cache that
 *             holds the step rows at [L, L + n_q).
 *   V empty -> o = 0, lse = -inf
 *   else      s_j = scale * sum_d q[b,i,h,d] * K[b,j,g,d]
 *             m   = max_j s_j,  e_j = exp(s_j - m),  l = sum_j e_j
 *             o_d = sum_j e_j * V[b,j,g,d] / l,  lse = m + ln(l)
 *
 * Split mode (num_splits > 0) cuts V into num_splits contiguous pieces,
 * takes (m_c, l_c, acc_c) per piece in fp64 and merges them with
 *   M = max_c m_c,  w_c = exp(m_c - M),  o = sum_c w_c acc_c / sum_c w_c l_c,
 * the merge that split-KV decoding relies on (comfy-kitchen PR "Performance
 * improvements for qwen 3.x LLM (Part 1)", section GQA decode: the KV prefix
 * is split and the splits' results are combined).  It exists to pin that
 * algebra; it must agree with the unsplit result to rounding.
 *
 * Paged INT8 cache (ck_oracle_attn_q8): K and V are stored per (token, KV
 * head) row as int8 codes with one fp32 scale, in pages of `page` tokens
 * reached through a block table (comfy-kitchen PR "Performance improvements
 * for qwen 3.x LLM (Part 1)", commit list: bounded paged INT8 decode cache
 * with rollback; the pages run 8-bit KV caches throughout, llama.cpp PR
 * "qwen4exp: attend the selected cells instead of masking the window",
 * Additional information).  Cell j of sequence b lives in page
 * block_table[b][j / page], row j % page of its KV head's block (a page is
 * [Hkv][page][D], so a head's rows in a page are contiguous; the pages leave
 * the layout open); its value is code * scale, taken
 * exactly in fp64, and the definition above applies unchanged.  A cell whose
 * page id is outside [0, num_pages) reads as zeros.  Rows are quantized in
 * fp32 (ck_oracle_q8_quantize_row): scale = amax / 127, code = x * (127 /
 * amax) rounded half to even and clamped to [-127, 127]; an all-zero row has
 * scale 0.  Rolling a sequence back is lowering its length: cells at or past
 * it are never read and are overwritten by the next append.
 *
 * Inputs are bf16 bit patterns (uint16); each is widened to fp64 exactly.
 * scale arrives as the fp32 value the GPU receives and is widened.  Cells
 * outside V are never read, so garbage (NaN/Inf bit patterns) there cannot
 * reach the result.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_NOMEM (-2)

static double bf16_to_f64(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    int B, n_q, Hq, Hkv, D, cap;
    const uint16_t *q, *k, *v;
    const uint16_t *k_step, *v_step; /* NULL unless step rows are merged */
    const int32_t *kv_lens;
    double scale;
    int causal;
    const uint8_t *keep_mask;
    const int32_t *idx;
    int W;
    long long idx_head_stride;
    int num_splits;
    double *out, *lse;
    /* paged INT8 cache; kq == NULL for the bf16 cache */
    const int8_t *kq, *vq;
    const float *ksc, *vsc;
    const int32_t *block_table;
    int page, max_pages, num_pages;
} job_t;

typedef struct {
    const job_t *job;
    long long unit_begin, unit_end;
    int status;
} worker_t;

/* Dequantized row of cell j of (b, g) in the paged INT8 cache, exactly in
   fp64; zeros when the page id is outside [0, num_pages). */
static void q8_row(const job_t *J, const int8_t *codes, const float *scales, int b, int g, int32_t j,
                   double *dst) {
    int32_t pg = J->block_table[(size_t)b * J->max_pages + (size_t)(j / J->page)];
    if (pg < 0 || pg >= J->num_pages) {
        for (int d = 0; d < J->D; ++d) dst[d] = 0.0;
        return;
    }
    size_t row = ((size_t)pg * J->Hkv + g) * J->page + (size_t)(j % J->page);
    double sc = (double)scales[row];
    for (int d = 0; d < J->D; ++d) dst[d] = (double)codes[row * J->D + d] * sc;
}

/* Row of K or V behind visible entry e of (b, g): a cache row, or step row
   e - cap. */
static const uint16_t *kv_row(const job_t *J, const uint16_t *cache, const uint16_t *step, int b,
                              int g, int32_t e) {
    if (e < J->cap) return cache + (((size_t)b * J->cap + (size_t)e) * J->Hkv + g) * (size_t)J->D;
    return step + (((size_t)b * J->n_q + (size_t)(e - J->cap)) * J->Hkv + g) * (size_t)J->D;
}

/* Visible cell list for (b, i, g), written to vis[]; returns its length. */
static int visible_cells(const job_t *J, int b, int i, int g, int32_t *vis) {
    long long L = J->kv_lens[b];
    if (L < 0) L = 0;
    if (L > J->cap) L = J->cap;
    long long lim = L;
    if (J->causal) {
        lim = L - J->n_q + i + 1;
        if (lim < 0) lim = 0;
        if (lim > L) lim = L;
    }
    int n = 0;
    if (J->idx == NULL) {
        for (long long j = 0; j < lim; ++j) {
            if (J->keep_mask != NULL) {
                size_t mo = (((size_t)b * J->n_q + i) * J->Hkv + g) * (size_t)J->cap + (size_t)j;
                if (J->keep_mask[mo] == 0) continue;
            }
            vis[n++] = (int32_t)j;
        }
        /* Step rows are listed after the cache cells as cap + t. */
        if (J->k_step != NULL)
            for (int t = 0; t <= i; ++t) vis[n++] = (int32_t)(J->cap + t);
    } else {
        const int32_t *list;
        if (J->idx_head_stride == 0)
            list = J->idx + ((size_t)b * J->n_q + i) * (size_t)J->W;
        else
            list = J->idx + ((size_t)b * J->n_q + i) * (size_t)J->Hkv * (size_t)J->idx_head_stride
                   + (size_t)g * (size_t)J->idx_head_stride;
        for (int t = 0; t < J->W; ++t) {
            long long j = list[t];
            if (j >= 0 && j < lim) vis[n++] = (int32_t)j;
        }
    }
    return n;
}

static void one_unit(const job_t *J, long long unit, int32_t *vis, double *s, double *acc,
                     double *qrow, double *rowbuf) {
    const int D = J->D;
    const int G = J->Hq / J->Hkv;
    int h = (int)(unit % J->Hq);
    int i = (int)((unit / J->Hq) % J->n_q);
    int b = (int)(unit / ((long long)J->Hq * J->n_q));
    int g = h / G;

    size_t qo = (((size_t)b * J->n_q + i) * J->Hq + h) * (size_t)D;
    double *o = J->out + qo;
    double *lse = J->lse ? J->lse + ((size_t)b * J->n_q + i) * J->Hq + h : NULL;

    int n = visible_cells(J, b, i, g, vis);
    if (n == 0) {
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (lse) *lse = -INFINITY;
        return;
    }
    for (int d = 0; d < D; ++d) qrow[d] = bf16_to_f64(J->q[qo + d]);

    /* scores over the visible list */
    for (int t = 0; t < n; ++t) {
        double dot = 0.0;
        if (J->kq != NULL) {
            q8_row(J, J->kq, J->ksc, b, g, vis[t], rowbuf);
            for (int d = 0; d < D; ++d) dot += qrow[d] * rowbuf[d];
        } else {
            const uint16_t *krow = kv_row(J, J->k, J->k_step, b, g, vis[t]);
            for (int d = 0; d < D; ++d) dot += qrow[d] * bf16_to_f64(krow[d]);
        }
        s[t] = J->scale * dot;
    }

    int S = J->num_splits > 0 ? J->num_splits : 1;
    double M = -INFINITY, den = 0.0;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    /* First pass: the overall max of the per-piece maxima. */
    double *m_c = (double *)malloc(sizeof(double) * (size_t)S);
    for (int c = 0; c < S; ++c) {
        int t0 = (int)((long long)c * n / S), t1 = (int)((long long)(c + 1) * n / S);
        double m = -INFINITY;
        for (int t = t0; t < t1; ++t)
            if (s[t] > m) m = s[t];
        m_c[c] = m;
        if (m > M) M = m;
    }
    /* Each piece: its own softmax numerator/denominator against its own max,
       then rescaled by exp(m_c - M) into the merged result. */
    for (int c = 0; c < S; ++c) {
        int t0 = (int)((long long)c * n / S), t1 = (int)((long long)(c + 1) * n / S);
        if (t1 <= t0) continue;
        double l_c = 0.0;
        for (int d = 0; d < D; ++d) acc[d] = 0.0;
        for (int t = t0; t < t1; ++t) {
            double e = exp(s[t] - m_c[c]);
            l_c += e;
            if (J->vq != NULL) {
                q8_row(J, J->vq, J->vsc, b, g, vis[t], rowbuf);
                for (int d = 0; d < D; ++d) acc[d] += e * rowbuf[d];
            } else {
                const uint16_t *vrow = kv_row(J, J->v, J->v_step, b, g, vis[t]);
                for (int d = 0; d < D; ++d) acc[d] += e * bf16_to_f64(vrow[d]);
            }
        }
        double w = exp(m_c[c] - M);
        den += w * l_c;
        for (int d = 0; d < D; ++d) o[d] += w * acc[d];
    }
    free(m_c);
    for (int d = 0; d < D; ++d) o[d] /= den;
    if (lse) *lse = M + log(den);
}

static void *worker_main(void *arg) {
    worker_t *w = (worker_t *)arg;
    const job_t *J = w->job;
    size_t vis_cap = J->idx ? (size_t)J->W : (size_t)J->cap + (J->k_step ? (size_t)J->n_q : 0);
    if (vis_cap == 0) vis_cap = 1;
    int32_t *vis = (int32_t *)malloc(sizeof(int32_t) * vis_cap);
    double *s = (double *)malloc(sizeof(double) * vis_cap);
    double *acc = (double *)malloc(sizeof(double) * (size_t)J->D);
    double *qrow = (double *)malloc(sizeof(double) * (size_t)J->D);
    double *rowbuf = (double *)malloc(sizeof(double) * (size_t)J->D);
    if (!vis || !s || !acc || !qrow || !rowbuf) {
        w->status = ORACLE_ERR_NOMEM;
    } else {
        for (long long u = w->unit_begin; u < w->unit_end; ++u) one_unit(J, u, vis, s, acc, qrow, rowbuf);
        w->status = ORACLE_OK;
    }
    free(vis);
    free(s);
    free(acc);
    free(qrow);
    free(rowbuf);
    return NULL;
}

int ck_oracle_nthreads_default(void) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/*
 * q  [B, n_q, Hq, D], k/v [B, cap, Hkv, D]: bf16 bit patterns, contiguous.
 * kv_lens [B] (host).  keep_mask [B, n_q, Hkv, cap] or NULL.
 * idx: NULL for the dense definition; else int32 lists of width W laid out
 * [B, n_q, Hkv, idx_head_stride] (idx_head_stride >= W) or, with
 * idx_head_stride == 0, one list per query shared by all its heads
 * [B, n_q, W].  out [B, n_q, Hq, D] fp64; lse [B, n_q, Hq] fp64 or NULL.
 * nthreads <= 0 uses every online host core.  Returns 0 or a negative code.
 */
static int run_job(const job_t *J, int nthreads);

int ck_oracle_attn(int B, int n_q, int Hq, int Hkv, int D, int cap, const uint16_t *q,
                   const uint16_t *k, const uint16_t *v, const int32_t *kv_lens, float scale,
                   int causal, const uint8_t *keep_mask, const int32_t *idx, int W,
                   long long idx_head_stride, int num_splits, double *out, double *lse,
                   int nthreads) {
    if (B < 1 || n_q < 1 || Hq < 1 || Hkv < 1 || D < 1 || cap < 1) return ORACLE_ERR_ARG;
    if (Hq % Hkv != 0) return ORACLE_ERR_ARG;
    if (!q || !k || !v || !kv_lens || !out) return ORACLE_ERR_ARG;
    if (idx && (W < 1 || (idx_head_stride != 0 && idx_head_stride < W))) return ORACLE_ERR_ARG;
    if (idx && keep_mask) return ORACLE_ERR_ARG;
    if (num_splits < 0) return ORACLE_ERR_ARG;

    job_t J = {B, n_q, Hq, Hkv, D, cap, q, k, v, NULL, NULL, kv_lens, (double)scale, causal ? 1 : 0,
               keep_mask, idx, W, idx_head_stride, num_splits, out, lse,
               NULL, NULL, NULL, NULL, NULL, 0, 0, 0};
    return run_job(&J, nthreads);
}

/*
 * The step-row definition: q [B, n_q, Hq, D], cache k/v [B, cap, Hkv, D],
 * k_step/v_step [B, n_q, Hkv, D] (bf16 bit patterns), kv_lens [B] (host).
 * Query i sees the cache prefix and step rows 0..i.  Arguments otherwise as
 * ck_oracle_attn.
 */
int ck_oracle_attn_steps(int B, int n_q, int Hq, int Hkv, int D, int cap, const uint16_t *q,
                         const uint16_t *k, const uint16_t *v, const int32_t *kv_lens,
                         const uint16_t *k_step, const uint16_t *v_step, float scale,
                         int num_splits, double *out, double *lse, int nthreads) {
    if (B < 1 || n_q < 1 || Hq < 1 || Hkv < 1 || D < 1 || cap < 1) return ORACLE_ERR_ARG;
    if (Hq % Hkv != 0) return ORACLE_ERR_ARG;
    if (!q || !k || !v || !kv_lens || !k_step || !v_step || !out) return ORACLE_ERR_ARG;
    if (num_splits < 0) return ORACLE_ERR_ARG;
    job_t J = {B, n_q, Hq, Hkv, D, cap, q, k, v, k_step, v_step, kv_lens, (double)scale, 0,
               NULL, NULL, 0, 0, num_splits, out, lse,
               NULL, NULL, NULL, NULL, NULL, 0, 0, 0};
    return run_job(&J, nthreads);
}

/*
 * Attention over the paged INT8 cache: q [B, n_q, Hq, D] bf16; kq/vq int8
 * [num_pages, Hkv, page, D]; ksc/vsc fp32 [num_pages, Hkv, page];
 * block_table int32 [B, max_pages]; kv_lens [B] clamped to
 * [0, max_pages * page].  Dense and causal windows as ck_oracle_attn.
 */
int ck_oracle_attn_q8(int B, int n_q, int Hq, int Hkv, int D, int page, int max_pages, int num_pages,
                      const uint16_t *q, const int8_t *kq, const int8_t *vq, const float *ksc,
                      const float *vsc, const int32_t *block_table, const int32_t *kv_lens,
                      float scale, int causal, int num_splits, double *out, double *lse,
                      int nthreads) {
    if (B < 1 || n_q < 1 || Hq < 1 || Hkv < 1 || D < 1 || page < 1 || max_pages < 1 || num_pages < 1)
        return ORACLE_ERR_ARG;
    if (Hq % Hkv != 0) return ORACLE_ERR_ARG;
    if ((long long)page * max_pages > 0x7fffffffLL) return ORACLE_ERR_ARG;
    if (!q || !kq || !vq || !ksc || !vsc || !block_table || !kv_lens || !out) return ORACLE_ERR_ARG;
    if (num_splits < 0) return ORACLE_ERR_ARG;
    job_t J = {B, n_q, Hq, Hkv, D, page * max_pages, q, NULL, NULL, NULL, NULL, kv_lens, (double)scale,
               causal ? 1 : 0, NULL, NULL, 0, 0, num_splits, out, lse,
               kq, vq, ksc, vsc, block_table, page, max_pages, num_pages};
    return run_job(&J, nthreads);
}

/* One row of D bf16 values to int8 codes and an fp32 scale (see the header
   comment); all arithmetic in fp32, rounding half to even. */
void ck_oracle_q8_quantize_row(int D, const uint16_t *x, int8_t *codes, float *scale) {
    float amax = 0.0f;
    for (int d = 0; d < D; ++d) {
        float a = fabsf((float)bf16_to_f64(x[d]));
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        for (int d = 0; d < D; ++d) codes[d] = 0;
        *scale = 0.0f;
        return;
    }
    float inv = 127.0f / amax;
    *scale = amax / 127.0f;
    for (int d = 0; d < D; ++d) {
        float c = nearbyintf((float)bf16_to_f64(x[d]) * inv);
        if (c > 127.0f) c = 127.0f;
        if (c < -127.0f) c = -127.0f;
        codes[d] = (int8_t)c;
    }
}

/* n_rows independent rows (x [n_rows, D]), as ck_oracle_q8_quantize_row. */
void ck_oracle_q8_quantize_rows(long long n_rows, int D, const uint16_t *x, int8_t *codes, float *scales) {
    for (long long r = 0; r < n_rows; ++r)
        ck_oracle_q8_quantize_row(D, x + r * D, codes + r * D, scales + r);
}

/*
 * Append n_new rows per sequence: k_new/v_new [B, n_new, Hkv, D] bf16 go to
 * positions start[b] + t (start clamped to [0, max_pages * page]); rows past
 * the capacity, or whose page id is outside [0, num_pages), are dropped.
 */
int ck_oracle_q8_append(int B, int n_new, int Hkv, int D, int page, int max_pages, int num_pages,
                        const uint16_t *k_new, const uint16_t *v_new, const int32_t *start,
                        const int32_t *block_table, int8_t *kq, int8_t *vq, float *ksc, float *vsc) {
    if (B < 1 || n_new < 1 || Hkv < 1 || D < 1 || page < 1 || max_pages < 1 || num_pages < 1)
        return ORACLE_ERR_ARG;
    if (!k_new || !v_new || !start || !block_table || !kq || !vq || !ksc || !vsc) return ORACLE_ERR_ARG;
    long long cap = (long long)page * max_pages;
    for (int b = 0; b < B; ++b) {
        long long s0 = start[b];
        if (s0 < 0) s0 = 0;
        if (s0 > cap) s0 = cap;
        for (int t = 0; t < n_new; ++t) {
            long long pos = s0 + t;
            if (pos >= cap) break;
            int32_t pg = block_table[(size_t)b * max_pages + (size_t)(pos / page)];
            if (pg < 0 || pg >= num_pages) continue;
            for (int g = 0; g < Hkv; ++g) {
                size_t row = ((size_t)pg * Hkv + g) * page + (size_t)(pos % page);
                size_t src = (((size_t)b * n_new + t) * Hkv + g) * (size_t)D;
                ck_oracle_q8_quantize_row(D, k_new + src, kq + row * D, ksc + row);
                ck_oracle_q8_quantize_row(D, v_new + src, vq + row * D, vsc + row);
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Top-k selection (ck_oracle_topk): the index lists the gather reads
 * (llama.cpp PR "qwen4exp : gather-based sparse attention for QSA decode",
 * discussion: the indexer's top-k over the whole score row every step; the
 * selection always keeps the current tail, llama.cpp PR "qwen4exp: attend the
 * selected cells instead of masking the window", PR body).  For each row
 * (b, i, h) of scores [B, n_q, Hs, cap]: L and lim as above, the tail
 * [max(0, lim - tail), lim), the candidates [0, n) with n = max(0, lim - tail).
 * The selection is the first min(k, n) candidates in the order "larger score
 * first, then smaller cell", with NaN taken as -inf (a sort serves this
 * step); the row of idx [B, n_q, Hs, k + tail] holds those cells ascending,
 * then the tail cells, then -1.
 */
typedef struct {
    double v;
    int32_t j;
} scored_t;

static int by_score_then_cell(const void *a, const void *b) {
    const scored_t *x = (const scored_t *)a, *y = (const scored_t *)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

static int by_cell(const void *a, const void *b) {
    const int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

int ck_oracle_topk(int B, int n_q, int Hs, int cap, const float *scores, const int32_t *kv_lens, int k,
                   int tail, int causal, int32_t *idx) {
    if (B < 1 || n_q < 1 || Hs < 1 || cap < 1 || k < 1 || tail < 0) return ORACLE_ERR_ARG;
    if (!scores || !kv_lens || !idx) return ORACLE_ERR_ARG;
    const int W = k + tail;
    scored_t *c = (scored_t *)malloc((size_t)cap * sizeof(scored_t));
    int32_t *sel = (int32_t *)malloc((size_t)cap * sizeof(int32_t));
    if (!c || !sel) {
        free(c);
        free(sel);
        return ORACLE_ERR_NOMEM;
    }
    for (int b = 0; b < B; ++b) {
        int L = kv_lens[b];
        if (L < 0) L = 0;
        if (L > cap) L = cap;
        for (int i = 0; i < n_q; ++i) {
            int lim = L;
            if (causal) {
                lim = L - n_q + i + 1;
                if (lim < 0) lim = 0;
                if (lim > L) lim = L;
            }
            int n = lim - tail;
            if (n < 0) n = 0;
            for (int h = 0; h < Hs; ++h) {
                const float *row = scores + (((size_t)b * n_q + i) * Hs + h) * (size_t)cap;
                for (int j = 0; j < n; ++j) {
                    double v = (double)row[j];
                    if (isnan(v)) v = -INFINITY;
                    c[j].v = v;
                    c[j].j = j;
                }
                qsort(c, (size_t)n, sizeof(scored_t), by_score_then_cell);
                int m = n < k ? n : k;
                for (int t = 0; t < m; ++t) sel[t] = c[t].j;
                qsort(sel, (size_t)m, sizeof(int32_t), by_cell);
                int32_t *out = idx + (((size_t)b * n_q + i) * Hs + h) * (size_t)W;
                int s = 0;
                for (int t = 0; t < m; ++t) out[s++] = sel[t];
                for (int j = n; j < lim; ++j) out[s++] = j;
                while (s < W) out[s++] = -1;
            }
        }
    }
    free(c);
    free(sel);
    return ORACLE_OK;
}

static int run_job(const job_t *JP, int nthreads) {
    const job_t J = *JP;
    const int B = J.B, n_q = J.n_q, Hq = J.Hq;
    long long units = (long long)B * n_q * Hq;
    if (nthreads <= 0) nthreads = ck_oracle_nthreads_default();
    if (nthreads > units) nthreads = (int)units;
    if (nthreads < 1) nthreads = 1;

    worker_t *ws = (worker_t *)calloc((size_t)nthreads, sizeof(worker_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!ws || !th) {
        free(ws);
        free(th);
        return ORACLE_ERR_NOMEM;
    }
    for (int t = 0; t < nthreads; ++t) {
        ws[t].job = &J;
        ws[t].unit_begin = units * t / nthreads;
        ws[t].unit_end = units * (t + 1) / nthreads;
    }
    int status = ORACLE_OK;
    if (nthreads == 1) {
        worker_main(&ws[0]);
        status = ws[0].status;
    } else {
        int started = 0;
        for (int t = 0; t < nthreads; ++t) {
            if (pthread_create(&th[t], NULL, worker_main, &ws[t]) != 0) break;
            ++started;
        }
        for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
        /* Any unit range whose thread failed to start runs here. */
        for (int t = started; t < nthreads; ++t) worker_main(&ws[t]);
        for (int t = 0; t < nthreads; ++t)
            if (ws[t].status != ORACLE_OK) status = ws[t].status;
    }
    free(ws);
    free(th);
    return status;
}
