/* Exercises every entry of the C oracle on small random inputs (lengths past
 * the capacity and negative, masks, gather lists with invalid and duplicate
 * entries, causal windows, split counts, step rows, paged INT8 pages with
 * ids outside the pool, appends past the capacity, top-k with ties and NaN),
 * for a build with AddressSanitizer and UndefinedBehaviorSanitizer: any
 * out-of-bounds access, use of freed memory or undefined arithmetic aborts
 * the run.  Exits 0 when every call returned and every output is finite or
 * the defined -inf/0 of an empty row. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ck_oracle_attn(int B, int n_q, int Hq, int Hkv, int D, int cap, const uint16_t *q, const uint16_t *k,
                   const uint16_t *v, const int32_t *kv_lens, float scale, int causal, const uint8_t *keep_mask,
                   const int32_t *idx, int W, long long idx_head_stride, int num_splits, double *out, double *lse,
                   int nthreads);
int ck_oracle_attn_steps(int B, int n_q, int Hq, int Hkv, int D, int cap, const uint16_t *q, const uint16_t *k,
                         const uint16_t *v, const int32_t *kv_lens, const uint16_t *k_step, const uint16_t *v_step,
                         float scale, int num_splits, double *out, double *lse, int nthreads);
int ck_oracle_attn_q8(int B, int n_q, int Hq, int Hkv, int D, int page, int max_pages, int num_pages,
                      const uint16_t *q, const int8_t *kq, const int8_t *vq, const float *ksc, const float *vsc,
                      const int32_t *block_table, const int32_t *kv_lens, float scale, int causal, int num_splits,
                      double *out, double *lse, int nthreads);
void ck_oracle_q8_quantize_rows(long long n_rows, int D, const uint16_t *x, int8_t *codes, float *scales);
int ck_oracle_q8_append(int B, int n_new, int Hkv, int D, int page, int max_pages, int num_pages,
                        const uint16_t *k_new, const uint16_t *v_new, const int32_t *start,
                        const int32_t *block_table, int8_t *kq, int8_t *vq, float *ksc, float *vsc);
int ck_oracle_topk(int B, int n_q, int Hs, int cap, const float *scores, const int32_t *kv_lens, int k, int tail,
                   int causal, int32_t *idx);

static uint64_t rng_state = 88172645463325252ull;
static uint32_t rnd(void) {  /* xorshift64 */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 16);
}
static int rint_in(int lo, int hi) { return lo + (int)(rnd() % (uint32_t)(hi - lo + 1)); }
/* N(0,1)-ish bf16 bits (sum of uniforms), occasionally garbage bits */
static uint16_t rbf16(int garbage) {
    if (garbage) return (uint16_t)rnd();
    float x = 0.f;
    for (int i = 0; i < 4; ++i) x += (float)(rnd() % 65536) / 65536.f - 0.5f;
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}
static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) exit(2);
    return p;
}
static int bad = 0;
static void check(const double *out, const double *lse, long long n_rows, int D) {
    for (long long r = 0; r < n_rows; ++r) {
        if (!(isfinite(lse[r]) || (isinf(lse[r]) && lse[r] < 0))) ++bad;
        for (int d = 0; d < D; ++d)
            if (!isfinite(out[r * D + d])) ++bad;
    }
}

int main(void) {
    for (int trial = 0; trial < 60; ++trial) {
        const int B = rint_in(1, 3), n_q = rint_in(1, 4), Hkv = rint_in(1, 3), G = rint_in(1, 4), Hq = Hkv * G;
        const int D = (int[]){4, 8, 16, 32}[rint_in(0, 3)], cap = rint_in(1, 70), causal = trial & 1;
        const size_t nq = (size_t)B * n_q * Hq * D, nkv = (size_t)B * cap * Hkv * D;
        uint16_t *q = xmalloc(nq * 2), *k = xmalloc(nkv * 2), *v = xmalloc(nkv * 2);
        int32_t *lens = xmalloc((size_t)B * 4);
        for (size_t i = 0; i < nq; ++i) q[i] = rbf16(0);
        for (int b = 0; b < B; ++b) lens[b] = rint_in(-3, cap + 3);
        for (int b = 0; b < B; ++b)
            for (int j = 0; j < cap; ++j)
                for (int e = 0; e < Hkv * D; ++e) {
                    const size_t o = ((size_t)b * cap + j) * Hkv * D + e;
                    const int past = j >= lens[b];
                    k[o] = rbf16(past);
                    v[o] = rbf16(past);
                }
        double *out = xmalloc(nq * 8), *lse = xmalloc((size_t)B * n_q * Hq * 8);
        const float scale = 1.f / sqrtf((float)D);
        const long long rows = (long long)B * n_q * Hq;
        /* dense, with split counts */
        for (int S = 0; S < 3; ++S) {
            if (ck_oracle_attn(B, n_q, Hq, Hkv, D, cap, q, k, v, lens, scale, causal, NULL, NULL, 0, 0,
                               S * 5, out, lse, 1 + S) != 0) ++bad;
            check(out, lse, rows, D);
        }
        /* keep_mask */
        uint8_t *mask = xmalloc((size_t)B * n_q * Hkv * cap);
        for (size_t i = 0; i < (size_t)B * n_q * Hkv * cap; ++i) mask[i] = (uint8_t)(rnd() % 3 == 0);
        if (ck_oracle_attn(B, n_q, Hq, Hkv, D, cap, q, k, v, lens, scale, causal, mask, NULL, 0, 0, 2, out, lse, 2))
            ++bad;
        check(out, lse, rows, D);
        /* gather lists, per head and shared, with invalid and duplicate entries */
        const int W = rint_in(1, 12);
        int32_t *idx = xmalloc((size_t)B * n_q * Hkv * (W + 3) * 4);
        for (size_t i = 0; i < (size_t)B * n_q * Hkv * (W + 3); ++i) idx[i] = rint_in(-4, cap + 4);
        if (ck_oracle_attn(B, n_q, Hq, Hkv, D, cap, q, k, v, lens, scale, causal, NULL, idx, W, W + 3, 0, out,
                           lse, 3))
            ++bad;
        check(out, lse, rows, D);
        if (ck_oracle_attn(B, n_q, Hq, Hkv, D, cap, q, k, v, lens, scale, causal, NULL, idx, W, 0, 1, out, lse, 1))
            ++bad;
        check(out, lse, rows, D);
        /* step rows */
        uint16_t *ks = xmalloc((size_t)B * n_q * Hkv * D * 2), *vs = xmalloc((size_t)B * n_q * Hkv * D * 2);
        for (size_t i = 0; i < (size_t)B * n_q * Hkv * D; ++i) {
            ks[i] = rbf16(0);
            vs[i] = rbf16(0);
        }
        if (ck_oracle_attn_steps(B, n_q, Hq, Hkv, D, cap, q, k, v, lens, ks, vs, scale, 2, out, lse, 2)) ++bad;
        check(out, lse, rows, D);
        /* paged INT8: quantize rows, append (past the capacity too), attend */
        const int page = rint_in(1, 8), max_pages = rint_in(1, 6), num_pages = rint_in(1, B * max_pages + 2);
        const size_t pool = (size_t)num_pages * Hkv * page;
        int8_t *kq = xmalloc(pool * D), *vq = xmalloc(pool * D);
        float *ksc = xmalloc(pool * 4), *vsc = xmalloc(pool * 4);
        memset(kq, 0, pool * D);
        memset(vq, 0, pool * D);
        memset(ksc, 0, pool * 4);
        memset(vsc, 0, pool * 4);
        int32_t *bt = xmalloc((size_t)B * max_pages * 4);
        for (int i = 0; i < B * max_pages; ++i) bt[i] = rint_in(-2, num_pages + 1);
        const int n_new = rint_in(1, 5);
        uint16_t *kn = xmalloc((size_t)B * n_new * Hkv * D * 2), *vn = xmalloc((size_t)B * n_new * Hkv * D * 2);
        for (size_t i = 0; i < (size_t)B * n_new * Hkv * D; ++i) {
            kn[i] = rbf16(0);
            vn[i] = rbf16(0);
        }
        int32_t *start = xmalloc((size_t)B * 4);
        for (int b = 0; b < B; ++b) start[b] = rint_in(-2, page * max_pages + 2);
        if (ck_oracle_q8_append(B, n_new, Hkv, D, page, max_pages, num_pages, kn, vn, start, bt, kq, vq, ksc, vsc))
            ++bad;
        int8_t *codes = xmalloc((size_t)B * n_new * Hkv * D);
        float *scales = xmalloc((size_t)B * n_new * Hkv * 4);
        ck_oracle_q8_quantize_rows((long long)B * n_new * Hkv, D, kn, codes, scales);
        int32_t *lq = xmalloc((size_t)B * 4);
        for (int b = 0; b < B; ++b) lq[b] = rint_in(-2, page * max_pages + 2);
        if (ck_oracle_attn_q8(B, n_q, Hq, Hkv, D, page, max_pages, num_pages, q, kq, vq, ksc, vsc, bt, lq, scale,
                              causal, 1, out, lse, 2))
            ++bad;
        check(out, lse, rows, D);
        /* top-k over scores with ties, NaN and infinities */
        const int Hs = rint_in(1, 2) == 1 ? 1 : Hkv, kk = rint_in(1, 10), tail = rint_in(0, 4);
        float *sc = xmalloc((size_t)B * n_q * Hs * cap * 4);
        for (size_t i = 0; i < (size_t)B * n_q * Hs * cap; ++i) {
            const uint32_t r = rnd() % 20;
            sc[i] = r == 0 ? NAN : r == 1 ? INFINITY : r == 2 ? -INFINITY : (float)(int)(rnd() % 5) - 2.f;
        }
        int32_t *lists = xmalloc((size_t)B * n_q * Hs * (kk + tail) * 4);
        if (ck_oracle_topk(B, n_q, Hs, cap, sc, lens, kk, tail, causal, lists)) ++bad;
        for (size_t i = 0; i < (size_t)B * n_q * Hs * (kk + tail); ++i)
            if (lists[i] < -1 || lists[i] >= cap) ++bad;
        free(q); free(k); free(v); free(lens); free(out); free(lse); free(mask); free(idx); free(ks); free(vs);
        free(kq); free(vq); free(ksc); free(vsc); free(bt); free(kn); free(vn); free(start); free(codes);
        free(scales); free(lq); free(sc); free(lists);
    }
    if (bad) {
        fprintf(stderr, "oracle driver: %d unexpected results\n", bad);
        return 1;
    }
    printf("oracle driver: ok\n");
    return 0;
}
