// Exercises the host code of the HIP library -- launch planning, the
// gather-or-scan choice, top-k planning, argument validation of every entry
// point -- over many shapes and bad arguments, for a build with
// AddressSanitizer and UndefinedBehaviorSanitizer on its host code (no GPU
// needed: no call here launches anything).
// Checks the plans' documented invariants; exits 0 when all hold.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "ck_decode_attn.h"

static int bad = 0;
#define EXPECT(c)                                                   \
    do {                                                            \
        if (!(c)) {                                                 \
            ++bad;                                                  \
            if (bad < 20) fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c); \
        }                                                           \
    } while (0)

int main() {
    // plans over a grid of shapes
    const int Bs[] = {1, 2, 7, 32, 200}, nqs[] = {1, 2, 5, 6, 7}, Hkvs[] = {1, 2, 4, 8, 32};
    const int Gs[] = {1, 3, 4, 8, 16}, Ds[] = {64, 128, 256}, caps[] = {1, 63, 1024, 24007, 32768, 4000000};
    const int Ws[] = {0, 1, 2112, 40000}, splits[] = {0, 1, 7, 64, 256, 257, -1}, cuss[] = {1, 80, 256, 304};
    long n_ok = 0;
    for (int B : Bs)
        for (int n_q : nqs)
            for (int Hkv : Hkvs)
                for (int G : Gs)
                    for (int D : Ds)
                        for (int cap : caps)
                            for (int W : Ws)
                                for (int S : splits)
                                    for (int cus : cuss) {
                                        ck_decode_shape s{B, n_q, Hkv * G, Hkv, D, cap};
                                        ck_decode_plan p;
                                        memset(&p, 0xA5, sizeof(p));
                                        const int st = ck_decode_attn_plan(&s, W, S, cus, &p);
                                        if (st != CK_OK) continue;
                                        ++n_ok;
                                        EXPECT(p.units >= 1 && p.splits >= 1 && p.splits <= CK_MAX_SPLITS);
                                        EXPECT(p.rows == (W > 0 ? G : n_q * G));
                                        EXPECT(p.rows_per_group == 16 || p.rows_per_group == 32);
                                        EXPECT(p.row_groups * p.rows_per_group >= p.rows);
                                        EXPECT(p.slices >= 1 && p.slices <= 64 && p.slices <= D / 4);
                                        EXPECT(p.granule > 0 && p.chunk_min % p.granule == 0);
                                        EXPECT(S == 0 || p.splits <= S);
                                        EXPECT((p.splits == 1) == (p.workspace_bytes == 0));
                                        int32_t path = -1;
                                        if (W > 0 && ck_decode_sparse_path(&s, W, cap, &path) == CK_OK)
                                            EXPECT(path == CK_PATH_GATHER || path == CK_PATH_SCAN);
                                    }
    EXPECT(n_ok > 1000);
    // bad plan arguments
    ck_decode_shape s{1, 1, 16, 4, 256, 24007};
    ck_decode_plan p;
    EXPECT(ck_decode_attn_plan(nullptr, 0, 0, 256, &p) == CK_ERR_ARG);
    EXPECT(ck_decode_attn_plan(&s, 0, 0, 256, nullptr) == CK_ERR_ARG);
    EXPECT(ck_decode_attn_plan(&s, -1, 0, 256, &p) == CK_ERR_ARG);
    EXPECT(ck_decode_attn_plan(&s, 0, 0, 0, &p) == CK_ERR_ARG);
    ck_decode_shape odd{1, 1, 15, 4, 256, 100};
    EXPECT(ck_decode_attn_plan(&odd, 0, 0, 256, &p) == CK_ERR_ARG);
    ck_decode_shape d64{1, 1, 16, 4, 64, 100};
    EXPECT(ck_decode_attn_plan(&d64, 0, 0, 256, &p) == CK_ERR_UNSUPPORTED);
    // top-k plans
    for (int B : Bs)
        for (int n_q : {1, 3, 6})
            for (int Hkv : {1, 2, 8})
                for (int cap : {1, 4095, 4097, 131072, 1 << 20})
                    for (int k : {1, 2048})
                        for (int tail : {0, 64})
                            for (int cus : cuss) {
                                ck_decode_shape t{B, n_q, Hkv, Hkv, 128, cap};
                                int32_t P = -1;
                                size_t bytes = 0;
                                for (int Hs : {1, Hkv})
                                    if (ck_decode_topk_plan(&t, Hs, k, tail, cus, &P, &bytes) == CK_OK) {
                                        EXPECT(P >= 1 && (long long)B * n_q * Hs * P <= (P > 1 ? cus : 1LL << 40));
                                        EXPECT((P == 1) == (bytes == 0));
                                    }
                            }
    // entry points: every call below has a bad argument and is refused by
    // the validation before any HIP call, so none launches anything
    std::vector<uint16_t> buf(1 << 16);
    std::vector<int32_t> lens(64, 10);
    void* q = buf.data();
    const int32_t* kl = lens.data();
    EXPECT(ck_decode_attn(nullptr, q, q, q, kl, 1.f, 0, nullptr, q, CK_DT_F32, nullptr, nullptr, 0, 0, nullptr) ==
           CK_ERR_ARG);
    EXPECT(ck_decode_attn(&s, nullptr, q, q, kl, 1.f, 0, nullptr, q, CK_DT_F32, nullptr, nullptr, 0, 0, nullptr) ==
           CK_ERR_ARG);
    EXPECT(ck_decode_attn(&s, q, q, q, kl, 1.f, 0, nullptr, q, 7, nullptr, nullptr, 0, 0, nullptr) == CK_ERR_ARG);
    EXPECT(ck_decode_attn(&s, (char*)q + 2, q, q, kl, 1.f, 0, nullptr, q, CK_DT_F32, nullptr, nullptr, 0, 0,
                          nullptr) == CK_ERR_ALIGN);
    EXPECT(ck_decode_attn(&s, q, q, q, kl, 1.f / 0.f, 0, nullptr, q, CK_DT_F32, nullptr, nullptr, 0, 0, nullptr) ==
           CK_ERR_ARG);
    EXPECT(ck_decode_attn(&s, q, q, q, kl, 1.f, 0, nullptr, q, CK_DT_F32, nullptr, nullptr, 0, 300, nullptr) ==
           CK_ERR_ARG);
    EXPECT(ck_decode_attn_noalloc(&d64, q, q, q, kl, 1.f, 0, nullptr, q, CK_DT_F32, nullptr, 0, nullptr) ==
           CK_ERR_UNSUPPORTED);
    const int32_t* idx = lens.data();
    EXPECT(ck_decode_attn_gather(&s, q, q, q, kl, idx, 0, 0, 1.f, 0, q, CK_DT_F32, nullptr, nullptr, 0, 0,
                                 nullptr) == CK_ERR_ARG);
    EXPECT(ck_decode_attn_gather(&s, q, q, q, kl, idx, 8, 4, 1.f, 0, q, CK_DT_F32, nullptr, nullptr, 0, 0,
                                 nullptr) == CK_ERR_ARG);
    EXPECT(ck_decode_attn_steps(&s, q, q, q, kl, nullptr, q, 1.f, q, CK_DT_F32, nullptr, nullptr, 0, 0, nullptr) ==
           CK_ERR_ARG);
    ck_q8_cache c{};
    EXPECT(ck_decode_attn_q8(&s, q, &c, kl, 1.f, 0, q, CK_DT_F32, nullptr, nullptr, 0, 0, nullptr) == CK_ERR_ARG);
    c = ck_q8_cache{q, q, (float*)q, (float*)q, kl, 60, 4, 4};
    EXPECT(ck_decode_attn_q8(&s, q, &c, kl, 1.f, 0, q, CK_DT_F32, nullptr, nullptr, 0, 0, nullptr) == CK_ERR_ARG);
    EXPECT(ck_kv_append_q8(&s, q, q, kl, nullptr, nullptr) == CK_ERR_ARG);
    EXPECT(ck_decode_topk(&s, (const float*)q, 3, kl, 8, 0, 0, (int32_t*)q, nullptr, 0, nullptr) == CK_ERR_ARG);
    EXPECT(ck_workspace_status(nullptr, nullptr, nullptr) == CK_ERR_ARG);
    EXPECT(ck_set_spin_limit(-1) == CK_ERR_ARG);
    EXPECT(ck_set_spin_limit(0) == CK_OK);
    for (int code = -7; code <= 1; ++code) EXPECT(ck_status_string(code) != nullptr);
    if (bad) {
        fprintf(stderr, "host driver: %d failed expectations\n", bad);
        return 1;
    }
    printf("host driver: ok (%ld valid plans)\n", n_ok);
    return 0;
}
