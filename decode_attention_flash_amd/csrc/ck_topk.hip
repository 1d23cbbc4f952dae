// ck_topk.hip -- top-k cell selection for the gathered decode, gfx950.
//
// For every (sequence b, query i, score head h) row of scores over the
// cache positions, pick the k highest-scoring cells of the query's window
// and emit them, with the window's last `tail` cells, as one ascending index
// list: the lists ck_decode_attn_gather reads (llama.cpp PR "qwen4exp :
// gather-based sparse attention for QSA decode", discussion: the selection
// runs over the whole score row every step and is the cost that still grows
// with the context; radix/partial top-k paths serve it on other backends).
//
// Radix select over an order-preserving 32-bit key, from the top: digits of
// 11, 11 and 10 bits.  Each level histograms the digit of the candidates
// that share the digits fixed so far, and the bin holding the k-th largest
// is kept.  P workgroups share a row: each holds a contiguous range of
// positions (its scores stay in registers across the levels), adds its LDS
// histogram into the row's histogram in the workspace, and meets the others
// at a row barrier.  Every workgroup of a row is resident at once (the host
// sizes the grid to the CU count), so the barriers never wait on a
// workgroup that is not running.  A final pass writes the selected positions
// in position order: each workgroup's output offset follows from the
// per-workgroup counts of keys above and equal to the threshold, and equal
// keys are taken lowest position first, so the result is unique.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ck_decode_attn.h"

namespace cktk {

constexpr int kThreads = 256;
constexpr int kBlock = 4 * kThreads;  // positions per block: four per thread
constexpr int kCacheBlocks = 4;       // blocks a workgroup keeps in registers
constexpr int kBins = 2048;           // widest digit: 11 bits
constexpr int kSpinLimit = 1 << 22;
constexpr uint32_t kRsrcWord3 = 0x00020000u;

// Per-row workspace, in 32-bit words: barrier and completion counters, the
// three level histograms, then (above, equal) counts per workgroup.
constexpr int kWsCounters = 64;
constexpr int kWsHist = kWsCounters;
constexpr int kWsCounts = kWsHist + 3 * kBins;
constexpr int kMaxWgPerRow = 256;
constexpr int kWsRowWords = kWsCounts + 2 * kMaxWgPerRow;

struct TParams {
    const float* scores;      // [B, n_q, Hs, cap]
    const int32_t* kv_lens;   // [B]
    int32_t* idx;             // [B, n_q, Hs, W]
    uint32_t* ws;             // rows x kWsRowWords (P > 1)
    int32_t B, n_q, Hs, cap, causal;
    int32_t k, tail, W;
    int32_t P;                // workgroups per row
    int32_t vec4;             // score rows 16-byte aligned
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

// Order-preserving key: a larger score has a larger key.  NaN ranks with
// -inf and -0 with +0, so key order is the order of the values compared as
// numbers.  Key 0 is never produced and marks "no candidate".
__device__ __forceinline__ uint32_t key_of(float x) {
    if (x != x) x = -__builtin_inff();
    if (x == 0.f) x = 0.f;
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int ld_dev(const uint32_t* p) {
    return (int)__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every store and atomic this wave issued has completed.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Exclusive prefix sum over the workgroup's threads in thread order; also
// returns the total.  `red` is LDS scratch of kThreads/64 + 1 words.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* red, uint32_t* total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(inc, d);
        if (lane >= d) inc += o;
    }
    if (lane == 63) red[wave] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        const uint32_t s = red[w];
        before += w < wave ? s : 0u;
        all += s;
    }
    __syncthreads();  // red may be reused by the next call
    *total = all;
    return before + inc - v;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const TParams p) {
    __shared__ uint32_t lh[kBins];
    __shared__ uint32_t red[kThreads / 64 + 1];
    __shared__ uint32_t pick[2];
    __shared__ uint32_t offs[2];

    const int tid = threadIdx.x;
    const int row = blockIdx.x / p.P, w = blockIdx.x % p.P;
    const int bi = row / p.Hs;  // row = (b * n_q + i) * Hs + h
    const int i = bi % p.n_q, b = bi / p.n_q;
    if (tid < 2) pick[tid] = 0u;

    const int L_raw = p.kv_lens[b];
    const int L = L_raw < 0 ? 0 : (L_raw > p.cap ? p.cap : L_raw);
    int lim = L;
    if (p.causal) {
        lim = L - p.n_q + i + 1;
        lim = lim < 0 ? 0 : (lim > L ? L : lim);
    }
    const int n_cand = max(0, lim - p.tail);  // candidates [0, n_cand), tail [n_cand, lim)
    const int n_take = min(p.k, n_cand);
    int32_t* out = p.idx + (size_t)row * p.W;

    // Positions of this workgroup: whole blocks, the same split in every
    // workgroup of the row.
    const int nblk = (n_cand + kBlock - 1) / kBlock;
    const int per = (nblk + p.P - 1) / p.P;
    const int blk0 = min(nblk, w * per), blk1 = min(nblk, blk0 + per);

    // The tail and the padding after the selection.
    if (w == 0) {
        for (int s = n_take + tid; s < p.W; s += kThreads) {
            const int c = n_cand + (s - n_take);
            out[s] = c < lim ? c : -1;
        }
    }
    if (n_cand <= p.k) {  // every candidate is selected: position j goes to slot j
        for (int pos = blk0 * kBlock + tid; pos < min(blk1 * kBlock, n_cand); pos += kThreads) out[pos] = pos;
        return;
    }

    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.scores + (size_t)row * p.cap, (uint32_t)n_cand * 4u);
    auto load_keys = [&](int blk, uint32_t kk[4]) {
        const int pos = blk * kBlock + 4 * tid;
        if (p.vec4) {
            const uint32_t off = pos < n_cand ? (uint32_t)pos * 4u : 0x80000000u;
            const float4 x = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
            kk[0] = key_of(x.x);
            kk[1] = key_of(x.y);
            kk[2] = key_of(x.z);
            kk[3] = key_of(x.w);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t off = pos + j < n_cand ? (uint32_t)(pos + j) * 4u : 0x80000000u;
                kk[j] = key_of(__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0)));
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (pos + j >= n_cand) kk[j] = 0u;
    };
    uint32_t kc[kCacheBlocks][4];
#pragma unroll
    for (int c = 0; c < kCacheBlocks; ++c) {
        if (blk0 + c < blk1) {
            load_keys(blk0 + c, kc[c]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) kc[c][j] = 0u;
        }
    }
    // Calls f(key, position) for this thread's candidates, block by block.
    auto for_keys = [&](auto&& f) {
#pragma unroll
        for (int c = 0; c < kCacheBlocks; ++c)
            if (blk0 + c < blk1) {
#pragma unroll
                for (int j = 0; j < 4; ++j) f(kc[c][j], (blk0 + c) * kBlock + 4 * tid + j);
            }
        for (int blk = blk0 + kCacheBlocks; blk < blk1; ++blk) {
            uint32_t kk[4];
            load_keys(blk, kk);
#pragma unroll
            for (int j = 0; j < 4; ++j) f(kk[j], blk * kBlock + 4 * tid + j);
        }
    };

    const bool shared_row = p.P > 1;
    uint32_t* ws = p.ws + (size_t)row * kWsRowWords;
    uint32_t* ctr = ws;  // [0] barrier arrivals, [1] completions
    int barriers = 0;
    auto row_barrier = [&]() {
        ++barriers;
        wait_stores();
        __syncthreads();
        if (tid == 0) {
            __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            int spins = 0;
            while (ld_dev(ctr) < barriers * p.P) {
                __builtin_amdgcn_s_sleep(1);
                if (++spins > kSpinLimit) break;  // cannot happen while the row's workgroups run
            }
        }
        __syncthreads();
    };

    // ---- three radix levels: 11, 11 and 10 bits of the key, from the top ----
    uint32_t prefix = 0;
    int k_rem = p.k;
#pragma unroll 1
    for (int lvl = 0; lvl < 3; ++lvl) {
        const int shift = lvl == 0 ? 21 : (lvl == 1 ? 10 : 0);
        const int nb = lvl == 2 ? 1024 : 2048;
        const int above = lvl == 0 ? 32 : (lvl == 1 ? 21 : 10);  // bits fixed so far start here
        for (int j = tid; j < nb; j += kThreads) lh[j] = 0u;
        __syncthreads();
        for_keys([&](uint32_t key, int) {
            const bool in = key != 0u && (above == 32 || (key >> above) == prefix);
            if (in) atomicAdd(&lh[(key >> shift) & (uint32_t)(nb - 1)], 1u);
        });
        __syncthreads();
        uint32_t* gh = ws + kWsHist + lvl * kBins;
        if (shared_row) {
            for (int j = tid; j < nb; j += kThreads) {
                const uint32_t c = lh[j];
                if (c) __hip_atomic_fetch_add(gh + j, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            row_barrier();
        }
        // Thread t owns bins nb-1-(t*bpt+j), j < bpt: the scan runs from the
        // largest digit down.
        const int bpt = nb / kThreads;
        uint32_t cnt[kBins / kThreads];
        uint32_t tsum = 0;
#pragma unroll
        for (int j = 0; j < kBins / kThreads; ++j) {
            uint32_t c = 0;
            if (j < bpt) {
                const int d = nb - 1 - (tid * bpt + j);
                c = shared_row ? (uint32_t)ld_dev(gh + d) : lh[d];
            }
            cnt[j] = c;
            tsum += c;
        }
        uint32_t total;
        const uint32_t before = block_scan(tsum, red, &total);
        if (before < (uint32_t)k_rem && (uint32_t)k_rem <= before + tsum) {
            uint32_t acc = before;
#pragma unroll
            for (int j = 0; j < kBins / kThreads; ++j) {
                if (j < bpt && acc + cnt[j] >= (uint32_t)k_rem && acc < (uint32_t)k_rem) {
                    pick[0] = (uint32_t)(nb - 1 - (tid * bpt + j));
                    pick[1] = acc;
                }
                acc += cnt[j];
            }
        }
        __syncthreads();
        const uint32_t digit = pick[0], n_above = pick[1];
        __syncthreads();
        prefix = (prefix << (lvl == 2 ? 10 : 11)) | digit;
        k_rem -= (int)n_above;
    }
    const uint32_t T = prefix;        // key of the k-th largest candidate
    const int n_eq_take = k_rem;      // candidates with key T to take, lowest position first

    // ---- this workgroup's counts above / equal to T, and its output offset ----
    uint32_t g_t = 0, e_t = 0;
    for_keys([&](uint32_t key, int) {
        g_t += key > T ? 1u : 0u;
        e_t += key == T ? 1u : 0u;
    });
    uint32_t g_w, e_w;
    block_scan(g_t, red, &g_w);
    block_scan(e_t, red, &e_w);
    uint32_t out_base = 0, eq_base = 0;
    if (shared_row) {
        uint32_t* counts = ws + kWsCounts;
        if (tid == 0) {
            st_dev(counts + 2 * w, g_w);
            st_dev(counts + 2 * w + 1, e_w);
        }
        row_barrier();
        // Thread t < P holds workgroup t's counts; scans give every
        // workgroup's equal-key rank start and output offset.
        const uint32_t g = tid < p.P ? (uint32_t)ld_dev(counts + 2 * tid) : 0u;
        const uint32_t e = tid < p.P ? (uint32_t)ld_dev(counts + 2 * tid + 1) : 0u;
        uint32_t dummy;
        const uint32_t E = block_scan(e, red, &dummy);
        const int left = n_eq_take - (int)E;
        const uint32_t take = g + (uint32_t)(left <= 0 ? 0 : (left < (int)e ? left : (int)e));
        const uint32_t S = block_scan(take, red, &dummy);
        if (tid == w) {
            offs[0] = S;
            offs[1] = E;
        }
        __syncthreads();
        out_base = offs[0];
        eq_base = offs[1];
    }

    // ---- write the selected positions in position order ----
    uint32_t run_sel = out_base, run_eq = eq_base;
    auto emit_block = [&](const uint32_t kk[4], int blk) {
        uint32_t ne = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) ne += kk[j] == T ? 1u : 0u;
        uint32_t eq_tot;
        uint32_t eq_rank = run_eq + block_scan(ne, red, &eq_tot);
        bool sel[4];
        uint32_t ns = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool eq = kk[j] == T;
            sel[j] = kk[j] > T || (eq && eq_rank < (uint32_t)n_eq_take);
            eq_rank += eq ? 1u : 0u;
            ns += sel[j] ? 1u : 0u;
        }
        uint32_t sel_tot;
        uint32_t slot = run_sel + block_scan(ns, red, &sel_tot);
        // (slot < n_take always holds when the counts agree; the bound keeps
        // every store inside the row whatever they read)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (sel[j]) {
                if (slot < (uint32_t)n_take) out[slot] = blk * kBlock + 4 * tid + j;
                ++slot;
            }
        run_sel += sel_tot;
        run_eq += eq_tot;
    };
#pragma unroll
    for (int c = 0; c < kCacheBlocks; ++c)
        if (blk0 + c < blk1) emit_block(kc[c], blk0 + c);
    for (int blk = blk0 + kCacheBlocks; blk < blk1; ++blk) {
        uint32_t kk[4];
        load_keys(blk, kk);
        emit_block(kk, blk);
    }

    // ---- leave the row's workspace zeroed for the next launch ----
    if (shared_row) {
        // Every workgroup passed the last barrier after reading the level
        // histograms, so they can be cleared; the counts are rewritten by
        // every launch.  The last workgroup to finish resets the counters.
        const int words = 3 * kBins;
        const int chunk = (words + p.P - 1) / p.P;
        for (int j = w * chunk + tid; j < min(words, (w + 1) * chunk); j += kThreads) st_dev(ws + kWsHist + j, 0u);
        wait_stores();
        __syncthreads();
        if (tid == 0 && __hip_atomic_fetch_add(ctr + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                            (uint32_t)(p.P - 1)) {
            st_dev(ctr, 0u);
            st_dev(ctr + 1, 0u);
        }
    }
}

static int device_cus(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CK_ERR_HIP;
    if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return CK_ERR_HIP;
    return CK_OK;
}

static int plan(const ck_decode_shape* s, int32_t Hs, int32_t k, int32_t tail, int num_cus, int32_t* P,
                size_t* ws_bytes) {
    if (!s || !P || !ws_bytes) return CK_ERR_ARG;
    if (s->B < 1 || s->n_q < 1 || s->Hkv < 1 || s->cap < 1) return CK_ERR_ARG;
    if (s->n_q > CK_MAX_NQ) return CK_ERR_UNSUPPORTED;
    if (Hs != 1 && Hs != s->Hkv) return CK_ERR_ARG;
    if (k < 1 || tail < 0 || (int64_t)k + tail >= ((int64_t)1 << 31) || num_cus < 1) return CK_ERR_ARG;
    if ((int64_t)s->cap * 4 + kBlock * 4 >= ((int64_t)1 << 31)) return CK_ERR_UNSUPPORTED;
    const int64_t rows = (int64_t)s->B * s->n_q * Hs;
    if (rows * ((int64_t)k + tail) >= ((int64_t)1 << 40)) return CK_ERR_UNSUPPORTED;
    const int64_t blocks = ((int64_t)s->cap + kBlock - 1) / kBlock;
    int64_t wg = rows >= num_cus ? 1 : num_cus / rows;  // all of a row's workgroups resident at once
    if (wg > blocks) wg = blocks;
    if (wg > kMaxWgPerRow) wg = kMaxWgPerRow;
    if (wg < 1) wg = 1;
    if (rows * wg >= ((int64_t)1 << 31)) return CK_ERR_UNSUPPORTED;
    *P = (int32_t)wg;
    *ws_bytes = wg > 1 ? (size_t)rows * kWsRowWords * sizeof(uint32_t) : 0;
    return CK_OK;
}

}  // namespace cktk

extern "C" {

int ck_decode_topk_plan(const ck_decode_shape* shape, int32_t Hs, int32_t k, int32_t tail, int num_cus,
                        int32_t* wgs_per_row, size_t* workspace_bytes) {
    return cktk::plan(shape, Hs, k, tail, num_cus, wgs_per_row, workspace_bytes);
}

int ck_decode_topk_workspace_size(const ck_decode_shape* shape, int32_t Hs, int32_t k, int32_t tail,
                                  size_t* bytes) {
    int32_t P = 0;
    int st = cktk::plan(shape, Hs, k, tail, 1, &P, bytes);
    if (st != CK_OK) return st;
    int cus = 0;
    st = cktk::device_cus(&cus);
    if (st != CK_OK) return st;
    return cktk::plan(shape, Hs, k, tail, cus, &P, bytes);
}

int ck_decode_topk(const ck_decode_shape* shape, const float* scores, int32_t Hs, const int32_t* kv_lens,
                   int32_t k, int32_t tail, int causal, int32_t* idx, void* workspace, size_t workspace_bytes,
                   void* stream) {
    int32_t P = 0;
    size_t need = 0;
    int st = cktk::plan(shape, Hs, k, tail, 1, &P, &need);
    if (st != CK_OK) return st;
    if (!scores || !kv_lens || !idx) return CK_ERR_ARG;
    if (((uintptr_t)scores & 3) || ((uintptr_t)kv_lens & 3) || ((uintptr_t)idx & 3)) return CK_ERR_ALIGN;
    int cus = 0;
    st = cktk::device_cus(&cus);
    if (st != CK_OK) return st;
    st = cktk::plan(shape, Hs, k, tail, cus, &P, &need);
    if (st != CK_OK) return st;
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return CK_ERR_WORKSPACE;
        if ((uintptr_t)workspace & 255) return CK_ERR_ALIGN;
    }
    cktk::TParams p{};
    p.scores = scores;
    p.kv_lens = kv_lens;
    p.idx = idx;
    p.ws = (uint32_t*)workspace;
    p.B = shape->B;
    p.n_q = shape->n_q;
    p.Hs = Hs;
    p.cap = shape->cap;
    p.causal = causal ? 1 : 0;
    p.k = k;
    p.tail = tail;
    p.W = k + tail;
    p.P = P;
    p.vec4 = ((uintptr_t)scores & 15) == 0 && shape->cap % 4 == 0 ? 1 : 0;
    const int rows = shape->B * shape->n_q * Hs;
    hipLaunchKernelGGL(cktk::topk_kernel, dim3((unsigned)(rows * P)), dim3(cktk::kThreads), 0,
                       (hipStream_t)stream, p);
    return hipGetLastError() == hipSuccess ? CK_OK : CK_ERR_HIP;
}

}  // extern "C"
