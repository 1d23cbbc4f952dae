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
// positions (the keys of up to 8 super-blocks of 4096 stay in registers
// across the levels), adds its LDS histogram into the row's histogram in
// the workspace, and meets the others at a row barrier.  Every workgroup of a row is resident at once (the host
// sizes the grid to the CU count), so the barriers never wait on a
// workgroup that is not running.  A final pass writes the selected positions
// in position order: each workgroup's output offset follows from the
// per-workgroup counts of keys above and equal to the threshold, and equal
// keys are taken lowest position first, so the result is unique.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ck_decode_attn.h"

namespace ckda {
int spin_limit();  // polls a bounded wait makes before it gives up (ck_decode_attn.hip)
}

namespace cktk {

constexpr int kThreads = 256;
constexpr int kPerThread = 16;                  // positions per thread in a super-block
constexpr int kSuper = kPerThread * kThreads;   // positions per super-block
constexpr int kBins = 2048;           // widest digit: 11 bits
constexpr int kAuxDevice = 16;  // sc1: served from the device's point of coherence
constexpr uint32_t kRsrcWord3 = 0x00020000u;

// Per-row workspace, in 32-bit words: a parity word naming the set the next
// launch uses and, 64 bytes apart, the barrier counters of two sets; the
// three level histograms of each set; then (above, equal) counts per
// workgroup.  A launch uses one set and clears the other one early (its
// stores overlap the score loads), and the row's last arrival at its final
// barrier flips the parity: no clearing pass or completion count at the end.
constexpr int kWsCounters = 64;
constexpr int kWsParity = 0, kWsCtr0 = 16, kWsCtrStride = 16;
constexpr int kWsHist = kWsCounters;
constexpr int kWsHistSet = 3 * kBins;
constexpr int kWsCounts = kWsHist + 2 * kWsHistSet;
constexpr int kMaxWgPerRow = 256;
constexpr int kWsCand = kWsCounts + 2 * kMaxWgPerRow;  // then (key, position) pairs, per workgroup
constexpr int kCand = 4096;                               // threshold-bin cells gathered in LDS
constexpr int kRankMax = 64;                              // a bin of at most this many keys is ranked by one wave
constexpr size_t kWsHeader = 256;                         // the status word, then the rows
// Super-blocks of a workgroup whose keys stay in registers: 1 when a
// workgroup holds one (a row split over many workgroups), else 8.  Each
// cached super-block unrolls every pass over the keys once more, and the
// larger code costs a one-block workgroup several microseconds, so each case
// gets its own kernel.
constexpr int kCacheMany = 8;

struct TParams {
    const float* scores;      // [B, n_q, Hs, cap]
    const int32_t* kv_lens;   // [B]
    int32_t* idx;             // [B, n_q, Hs, W]
    uint32_t* ws;             // rows x kWsRowWords (P > 1)
    int32_t* status;          // the workspace's status word (P > 1)
    int32_t spin_limit;       // polls at a row barrier before giving up
    int32_t B, n_q, Hs, cap, causal;
    int32_t k, tail, W;
    int32_t P;                // workgroups per row
    int32_t vec4;             // score rows 16-byte aligned
    int32_t cand_per_wg;      // pair slots per workgroup (its largest range)
    uint32_t cand_off;        // word offset of the pair slots in a row's workspace
    uint64_t ws_row_words;    // workspace words per row
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
__device__ __forceinline__ void st_dev64(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every store and atomic this wave issued has completed.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves:
// within each row of 16 lanes, shifts by 1, 2 and 3 of the input, then by 4
// and 8 of the running sum (on the lanes that have such a predecessor); then
// row 0's total goes to row 1 and row 2's to row 3 (broadcast of lane 15),
// and lane 31's running total to rows 2 and 3.  Lanes a move does not reach
// add 0.
__device__ __forceinline__ uint32_t wave_scan(uint32_t x) {
    uint32_t v = x;
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x113, 0xf, 0xf, true);  // row_shr:3
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xe, true);  // row_shr:4, lanes 4-15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xc, true);  // row_shr:8, lanes 8-15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, true);  // row_bcast:15 -> rows 1, 3
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, true);  // row_bcast:31 -> rows 2, 3
    return v;
}

// Exclusive prefix sum over the workgroup's threads in thread order; also
// returns the total.  Calls alternate between the two halves of `red`
// (2 x kThreads/64 words of LDS), so the one barrier of a call also
// orders the previous call's reads before the next call's writes.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* red, int& parity, uint32_t* total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t* r = red + parity * (kThreads / 64);
    parity ^= 1;
    const uint32_t inc = wave_scan(v);
    if (lane == 63) r[wave] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        const uint32_t s = r[w];
        before += w < wave ? s : 0u;
        all += s;
    }
    *total = all;
    return before + inc - v;
}

template <int CSB>
__global__ __launch_bounds__(kThreads) void topk_kernel(const TParams p) {
    __shared__ uint32_t lh[kBins];
    __shared__ uint32_t red[2 * (kThreads / 64)];
    int parity = 0;  // which half of red the next block_scan uses
    __shared__ uint32_t pick[3];
    __shared__ uint32_t offs[2];
    __shared__ uint32_t cpre[kMaxWgPerRow];
    __shared__ uint32_t ck_key[kCand];
    __shared__ int32_t ck_pos[kCand];

    const int tid = threadIdx.x;
    const int row = blockIdx.x / p.P, w = blockIdx.x % p.P;
    const int bi = row / p.Hs;  // row = (b * n_q + i) * Hs + h
    const int i = bi % p.n_q, b = bi / p.n_q;
    if (tid < 3) pick[tid] = 0u;

    // Positions of this workgroup: whole super-blocks of kSuper positions,
    // split by the capacity, which is known before the length arrives, so
    // the first score loads go out together with the length load.  Thread t
    // holds positions 16t .. 16t+15 of each super-block.
    const int nsb = (p.cap + kSuper - 1) / kSuper;
    const int per = (nsb + p.P - 1) / p.P;
    const int sb0 = min(nsb, w * per), sb1 = min(nsb, sb0 + per);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.scores + (size_t)row * p.cap, (uint32_t)p.cap * 4u);
    auto load_raw = [&](int sb, float x[kPerThread]) {
        const uint32_t pos = (uint32_t)(sb * kSuper + kPerThread * tid);
        if (p.vec4) {
#pragma unroll
            for (int c = 0; c < kPerThread / 4; ++c) {
                const float4 v =
                    __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, (pos + 4 * c) * 4u, 0, 0));
                x[4 * c] = v.x;
                x[4 * c + 1] = v.y;
                x[4 * c + 2] = v.z;
                x[4 * c + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kPerThread; ++j)
                x[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (pos + j) * 4u, 0, 0));
        }
    };
    // The first CSB super-blocks of the range are loaded at once (one
    // round trip) and stay in registers as keys for every pass; any further
    // ones are read again at each pass.
    float xc[CSB][kPerThread];
#pragma unroll
    for (int c = 0; c < CSB; ++c) {
        if (sb0 + c < sb1) {
            load_raw(sb0 + c, xc[c]);
        } else {
#pragma unroll
            for (int j = 0; j < kPerThread; ++j) xc[c][j] = 0.f;
        }
    }

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

    // The tail and the padding after the selection.
    if (w == 0) {
        for (int s = n_take + tid; s < p.W; s += kThreads) {
            const int c = n_cand + (s - n_take);
            out[s] = c < lim ? c : -1;
        }
    }
    if (n_cand <= p.k) {  // every candidate is selected: position j goes to slot j
        for (int pos = sb0 * kSuper + tid; pos < min(sb1 * kSuper, n_cand); pos += kThreads) out[pos] = pos;
        return;
    }

    // Keys of a super-block; positions past the candidates get key 0.
    auto to_keys = [&](const float x[kPerThread], int sb, uint32_t kk[kPerThread]) {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j)
            kk[j] = sb * kSuper + kPerThread * tid + j < n_cand ? key_of(x[j]) : 0u;
    };
    uint32_t kc[CSB][kPerThread];
#pragma unroll
    for (int c = 0; c < CSB; ++c) to_keys(xc[c], sb0 + c, kc[c]);
    // Calls f(key, position) for this thread's positions, super-block by
    // super-block (those past the register cache are read again).
    auto for_keys = [&](auto&& f) {
#pragma unroll
        for (int c = 0; c < CSB; ++c) {
            if (sb0 + c < sb1) {
#pragma unroll
                for (int j = 0; j < kPerThread; ++j) f(kc[c][j], (sb0 + c) * kSuper + kPerThread * tid + j);
            }
        }
        for (int sb = sb0 + CSB; sb < sb1; ++sb) {
            float x[kPerThread];
            uint32_t kk[kPerThread];
            load_raw(sb, x);
            to_keys(x, sb, kk);
#pragma unroll
            for (int j = 0; j < kPerThread; ++j) f(kk[j], sb * kSuper + kPerThread * tid + j);
        }
    };

    const bool shared_row = p.P > 1;
    uint32_t* ws = p.ws + (size_t)row * p.ws_row_words;
    // This launch's set, and the other set (the previous launch's) cleared
    // now: every workgroup its share of the histograms, workgroup 0 the
    // counter.  Nothing waits on these stores; the launch boundary orders
    // them before the next launch, which uses that set.
    int par = 0;
    if (shared_row) {
        par = __builtin_amdgcn_readfirstlane(ld_dev(ws + kWsParity)) & 1;
        uint32_t* other = ws + kWsHist + (par ^ 1) * kWsHistSet;
        const int chunk = (kWsHistSet + p.P - 1) / p.P;
        for (int j = w * chunk + tid; j < min(kWsHistSet, (w + 1) * chunk); j += kThreads) st_dev(other + j, 0u);
        if (w == 0 && tid == 0) st_dev(ws + kWsCtr0 + (par ^ 1) * kWsCtrStride, 0u);
    }
    uint32_t* ctr = ws + kWsCtr0 + par * kWsCtrStride;  // barrier arrivals of this launch's set
    int barriers = 0;
    // The row's last arrival at its final barrier flips the parity: every
    // workgroup of the row read it before arriving there.
    auto row_barrier = [&](bool final) {
        ++barriers;
        wait_stores();
        __syncthreads();
        if (tid == 0) {
            const uint32_t rank = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (final && rank == (uint32_t)(barriers * p.P - 1)) st_dev(ws + kWsParity, (uint32_t)(par ^ 1));
            int spins = 0;
            while (ld_dev(ctr) < barriers * p.P) {
                __builtin_amdgcn_s_sleep(1);
                // Cannot happen while the row's workgroups run: report it and
                // go on (every store below stays inside the row whatever the
                // counts say), so the kernel still ends.
                if (++spins > p.spin_limit) {
                    __hip_atomic_fetch_or(p.status, CK_WS_ERR_TOPK, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
        __syncthreads();
    };

    // Finds the digit whose bin holds the k_rem-th largest key, scanning
    // bins from the largest digit down; gh is the row's histogram in the
    // workspace (device-coherent buffer loads, all issued before the first
    // is used), or null for this workgroup's histogram in LDS.  Every thread
    // gets the digit, the count of keys in larger bins and the bin's own count.
    auto find_bin = [&](const uint32_t* gh, int nb, int k_need, uint32_t* n_above, uint32_t* n_bin) -> uint32_t {
        const int bpt = nb / kThreads;  // thread t owns bins nb-1-(t*bpt+j)
        uint32_t cnt[kBins / kThreads];
        if (gh) {
            const __amdgpu_buffer_rsrc_t rh = make_rsrc(gh, (uint32_t)nb * 4u);
#pragma unroll
            for (int j = 0; j < kBins / kThreads; ++j) {
                const uint32_t off = j < bpt ? (uint32_t)(nb - 1 - (tid * bpt + j)) * 4u : 0x80000000u;
                cnt[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rh, off, 0, kAuxDevice);
            }
        } else {
#pragma unroll
            for (int j = 0; j < kBins / kThreads; ++j) cnt[j] = j < bpt ? lh[nb - 1 - (tid * bpt + j)] : 0u;
        }
        uint32_t tsum = 0;
#pragma unroll
        for (int j = 0; j < kBins / kThreads; ++j) tsum += cnt[j];
        uint32_t total;
        const uint32_t before = block_scan(tsum, red, parity, &total);
        if (before < (uint32_t)k_need && (uint32_t)k_need <= before + tsum) {
            uint32_t acc = before;
#pragma unroll
            for (int j = 0; j < kBins / kThreads; ++j) {
                if (j < bpt && acc < (uint32_t)k_need && acc + cnt[j] >= (uint32_t)k_need) {
                    pick[0] = (uint32_t)(nb - 1 - (tid * bpt + j));
                    pick[1] = acc;
                    pick[2] = cnt[j];
                }
                acc += cnt[j];
            }
        }
        __syncthreads();
        const uint32_t d = pick[0];
        *n_above = pick[1];
        *n_bin = pick[2];
        __syncthreads();
        return d;
    };

    // One radix level over the row: histogram of the digit below `above` of
    // the keys whose higher digits equal prefix, summed over the row's
    // workgroups, then its bin search.  Returns the chosen bin's count.
    uint32_t prefix = 0;
    int k_rem = p.k;
    auto row_level = [&](int lvl) -> uint32_t {
        const int shift = lvl == 0 ? 21 : (lvl == 1 ? 10 : 0);
        const int nb = lvl == 2 ? 1024 : 2048;
        const int above = lvl == 0 ? 32 : (lvl == 1 ? 21 : 10);
        for (int j = tid; j < nb; j += kThreads) lh[j] = 0u;
        __syncthreads();
        for_keys([&](uint32_t key, int) {
            const bool in = key != 0u && (above == 32 || (key >> above) == prefix);
            if (in) atomicAdd(&lh[(key >> shift) & (uint32_t)(nb - 1)], 1u);
        });
        __syncthreads();
        uint32_t* gh = ws + kWsHist + par * kWsHistSet + lvl * kBins;
        if (shared_row) {
            for (int j = tid; j < nb; j += kThreads) {
                const uint32_t c = lh[j];
                if (c) __hip_atomic_fetch_add(gh + j, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            row_barrier(false);
        }
        uint32_t n_above, n_bin;
        const uint32_t digit = find_bin(shared_row ? gh : nullptr, nb, k_rem, &n_above, &n_bin);
        prefix = (prefix << (lvl == 2 ? 10 : 11)) | digit;
        k_rem -= (int)n_above;
        return n_bin;
    };

    // ---- level 0: the top 11 bits over the whole row ----
    const uint32_t c_bin = row_level(0);
    uint32_t T;           // key of the k-th largest candidate
    int n_eq_take;        // candidates with key T to take, lowest position first
    uint32_t out_base = 0, eq_base = 0;
    uint32_t* counts = ws + kWsCounts;

    if (shared_row && c_bin <= (uint32_t)kCand) {
        // ---- the threshold bin fits in LDS: exchange it once and finish here ----
        // Each workgroup publishes how many of its keys lie above the bin
        // (all selected) and writes the bin's (key, position) pairs to its
        // own slots; after one barrier every workgroup gathers the pairs and
        // selects among them in LDS, so all reach the same threshold.
        const uint32_t d0 = prefix;
        uint32_t a_t = 0, c_t = 0;
        for_keys([&](uint32_t key, int) {
            a_t += key != 0u && (key >> 21) > d0 ? 1u : 0u;
            c_t += key != 0u && (key >> 21) == d0 ? 1u : 0u;
        });
        uint32_t a_w, c_w;
        block_scan(a_t, red, parity, &a_w);
        uint32_t slot = block_scan(c_t, red, parity, &c_w);
        uint64_t* mine = reinterpret_cast<uint64_t*>(ws + p.cand_off) + (size_t)w * p.cand_per_wg;
        for_keys([&](uint32_t key, int pos) {
            if (key != 0u && (key >> 21) == d0) {
                // (slot < cand_per_wg always holds when the scan is right)
                if (slot < (uint32_t)p.cand_per_wg) st_dev64(mine + slot, ((uint64_t)(uint32_t)pos << 32) | key);
                ++slot;
            }
        });
        if (tid == 0) {
            st_dev(counts + 2 * w, a_w);
            st_dev(counts + 2 * w + 1, c_w);
        }
        row_barrier(true);
        const uint32_t a = tid < p.P ? (uint32_t)ld_dev(counts + 2 * tid) : 0u;
        const uint32_t c = tid < p.P ? (uint32_t)ld_dev(counts + 2 * tid + 1) : 0u;
        uint32_t a_tot, c_tot;
        const uint32_t A = block_scan(a, red, parity, &a_tot);
        const uint32_t Cp = block_scan(c, red, parity, &c_tot);
        if (tid < p.P) cpre[tid] = Cp;
        if (tid == w) offs[0] = A;
        __syncthreads();
        const int n_c = (int)min(c_tot, (uint32_t)kCand);
        // Entry e comes from workgroup t with cpre[t] <= e < cpre[t + 1].  All
        // of a thread's loads go out before the first is stored (one round trip).
        const __amdgpu_buffer_rsrc_t rc =
            make_rsrc(ws + p.cand_off, (uint32_t)((size_t)p.P * p.cand_per_wg * 8u));
        uint64_t got[kCand / kThreads];
#pragma unroll
        for (int u = 0; u < kCand / kThreads; ++u) {
            const int e = tid + u * kThreads;
            uint32_t off = 0x80000000u;
            if (e < n_c) {
                int lo = 0, hi = p.P - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (cpre[mid] <= (uint32_t)e) lo = mid;
                    else hi = mid - 1;
                }
                off = (uint32_t)(((size_t)lo * p.cand_per_wg + (size_t)(e - (int)cpre[lo])) * 8u);
            }
            got[u] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rc, off, 0, kAuxDevice));
        }
#pragma unroll
        for (int u = 0; u < kCand / kThreads; ++u) {
            const int e = tid + u * kThreads;
            if (e < n_c) {
                ck_key[e] = (uint32_t)got[u];
                ck_pos[e] = (int32_t)(got[u] >> 32);
            }
        }
        __syncthreads();
        // the remaining 21 bits in LDS: an 11-bit digit, then the last 10
        // bits of the chosen bin.  The bin usually holds a few keys (of ~2000
        // normal scores over 2048 bins): up to kRankMax of them are ranked by
        // one wave, key against key, instead of a third histogram.
        uint32_t n_bin1 = 0;
        bool ranked = false;
#pragma unroll 1
        for (int lvl = 1; lvl < 3; ++lvl) {
            if (lvl == 2 && n_bin1 <= (uint32_t)kRankMax) {
                ranked = true;
                break;
            }
            const int shift = lvl == 1 ? 10 : 0;
            const int nb = lvl == 1 ? 2048 : 1024;
            const int above = lvl == 1 ? 21 : 10;
            for (int j = tid; j < nb; j += kThreads) lh[j] = 0u;
            __syncthreads();
            for (int e = tid; e < n_c; e += kThreads) {
                const uint32_t key = ck_key[e];
                if ((key >> above) == prefix) atomicAdd(&lh[(key >> shift) & (uint32_t)(nb - 1)], 1u);
            }
            __syncthreads();
            uint32_t n_above, n_bin;
            const uint32_t digit = find_bin(nullptr, nb, k_rem, &n_above, &n_bin);
            prefix = (prefix << (lvl == 2 ? 10 : 11)) | digit;
            k_rem -= (int)n_above;
            n_bin1 = n_bin;
        }
        if (ranked) {
            // The bin's keys (their top 22 bits equal prefix) go to lh[0..),
            // counted in lh[kRankMax]; lane j of wave 0 holds key j and counts
            // the keys above it and equal to it.  The key with k_rem - 1 keys
            // above it, or fewer but with equals reaching k_rem, is T.
            if (tid == 0) lh[kRankMax] = 0u;
            __syncthreads();
            for (int e = tid; e < n_c; e += kThreads) {
                const uint32_t key = ck_key[e];
                if ((key >> 10) == prefix) {
                    const uint32_t at = atomicAdd(&lh[kRankMax], 1u);
                    if (at < (uint32_t)kRankMax) lh[at] = key;
                }
            }
            __syncthreads();
            if (tid < 64) {
                const int m = (int)n_bin1;
                const uint32_t mine = tid < m ? lh[tid] : 0u;
                uint32_t gt = 0, eq = 0;
                for (int j = 0; j < m; ++j) {
                    const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)mine, j);
                    gt += o > mine ? 1u : 0u;
                    eq += o == mine ? 1u : 0u;
                }
                if (tid < m && gt < (uint32_t)k_rem && (uint32_t)k_rem <= gt + eq) {
                    pick[0] = mine;  // every lane holding T writes the same values
                    pick[1] = (uint32_t)k_rem - gt;
                }
            }
            __syncthreads();
            T = pick[0];
            n_eq_take = (int)pick[1];
        } else {
            T = prefix;
            n_eq_take = k_rem;
        }
        // selected pairs before this workgroup's range, and equal keys there
        const int start = sb0 * kSuper;
        uint32_t gb_t = 0, eb_t = 0;
        for (int e = tid; e < n_c; e += kThreads) {
            gb_t += ck_key[e] > T && ck_pos[e] < start ? 1u : 0u;
            eb_t += ck_key[e] == T && ck_pos[e] < start ? 1u : 0u;
        }
        uint32_t gb, eb;
        block_scan(gb_t, red, parity, &gb);
        block_scan(eb_t, red, parity, &eb);
        out_base = offs[0] + gb + min(eb, (uint32_t)n_eq_take);
        eq_base = eb;
    } else {
        // ---- the next two digits over the row, then the counts exchange ----
        row_level(1);
        row_level(2);
        T = prefix;
        n_eq_take = k_rem;
        uint32_t g_t = 0, e_t = 0;
        for_keys([&](uint32_t key, int) {
            g_t += key > T ? 1u : 0u;
            e_t += key == T ? 1u : 0u;
        });
        uint32_t g_w, e_w;
        block_scan(g_t, red, parity, &g_w);
        block_scan(e_t, red, parity, &e_w);
        if (shared_row) {
            if (tid == 0) {
                st_dev(counts + 2 * w, g_w);
                st_dev(counts + 2 * w + 1, e_w);
            }
            row_barrier(true);
            // Thread t < P holds workgroup t's counts; scans give every
            // workgroup's equal-key rank start and output offset.
            const uint32_t g = tid < p.P ? (uint32_t)ld_dev(counts + 2 * tid) : 0u;
            const uint32_t e = tid < p.P ? (uint32_t)ld_dev(counts + 2 * tid + 1) : 0u;
            uint32_t dummy;
            const uint32_t E = block_scan(e, red, parity, &dummy);
            const int left = n_eq_take - (int)E;
            const uint32_t take = g + (uint32_t)(left <= 0 ? 0 : (left < (int)e ? left : (int)e));
            const uint32_t S = block_scan(take, red, parity, &dummy);
            if (tid == w) {
                offs[0] = S;
                offs[1] = E;
            }
            __syncthreads();
            out_base = offs[0];
            eq_base = offs[1];
        }
    }

    // ---- write the selected positions in position order ----
    uint32_t run_sel = out_base, run_eq = eq_base;
    auto emit = [&](const uint32_t kk[kPerThread], int sb) {
        uint32_t ne = 0;
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) ne += kk[j] == T ? 1u : 0u;
        uint32_t eq_tot;
        uint32_t eq_rank = run_eq + block_scan(ne, red, parity, &eq_tot);
        uint32_t sel = 0, ns = 0;
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const bool eq = kk[j] == T;
            const bool take = kk[j] > T || (eq && eq_rank < (uint32_t)n_eq_take);
            eq_rank += eq ? 1u : 0u;
            sel |= (take ? 1u : 0u) << j;
            ns += take ? 1u : 0u;
        }
        uint32_t sel_tot;
        uint32_t slot = run_sel + block_scan(ns, red, parity, &sel_tot);
        // (slot < n_take always holds when the counts agree; the bound keeps
        // every store inside the row whatever they read)
#pragma unroll
        for (int j = 0; j < kPerThread; ++j)
            if ((sel >> j) & 1u) {
                if (slot < (uint32_t)n_take) out[slot] = sb * kSuper + kPerThread * tid + j;
                ++slot;
            }
        run_sel += sel_tot;
        run_eq += eq_tot;
    };
#pragma unroll
    for (int c = 0; c < CSB; ++c)
        if (sb0 + c < sb1) emit(kc[c], sb0 + c);
    for (int sb = sb0 + CSB; sb < sb1; ++sb) {
        float x[kPerThread];
        uint32_t kk[kPerThread];
        load_raw(sb, x);
        to_keys(x, sb, kk);
        emit(kk, sb);
    }
}

static int device_cus(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CK_ERR_HIP;
    if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return CK_ERR_HIP;
    return CK_OK;
}

struct Plan {
    int32_t P;            // workgroups per row
    int32_t cand_per_wg;  // pair slots per workgroup
    uint64_t row_words;   // workspace words per row
    size_t ws_bytes;
};

static int plan(const ck_decode_shape* s, int32_t Hs, int32_t k, int32_t tail, int num_cus, Plan* pl) {
    if (!s || !pl) return CK_ERR_ARG;
    if (s->B < 1 || s->n_q < 1 || s->Hkv < 1 || s->cap < 1) return CK_ERR_ARG;
    if (s->n_q > CK_MAX_NQ) return CK_ERR_UNSUPPORTED;
    if (Hs != 1 && Hs != s->Hkv) return CK_ERR_ARG;
    if (k < 1 || tail < 0 || (int64_t)k + tail >= ((int64_t)1 << 31) || num_cus < 1) return CK_ERR_ARG;
    if ((int64_t)s->cap * 4 + kSuper * 4 >= ((int64_t)1 << 31)) return CK_ERR_UNSUPPORTED;
    const int64_t rows = (int64_t)s->B * s->n_q * Hs;
    if (rows * ((int64_t)k + tail) >= ((int64_t)1 << 40)) return CK_ERR_UNSUPPORTED;
    const int64_t blocks = ((int64_t)s->cap + kSuper - 1) / kSuper;
    int64_t wg = rows >= num_cus ? 1 : num_cus / rows;  // all of a row's workgroups resident at once
    // at least one super-block per workgroup: fewer workgroups meet sooner
    // at the barriers and add fewer histogram atomics
    if (wg > blocks) wg = blocks;
    if (wg > kMaxWgPerRow) wg = kMaxWgPerRow;
    if (wg < 1) wg = 1;
    if (rows * wg >= ((int64_t)1 << 31)) return CK_ERR_UNSUPPORTED;
    const int64_t per_max = (blocks + wg - 1) / wg;
    // a row's (key, position) slots are read through one 32-bit buffer range
    if (wg > 1 && wg * per_max * kSuper * 8 >= ((int64_t)1 << 31)) return CK_ERR_UNSUPPORTED;
    pl->P = (int32_t)wg;
    pl->cand_per_wg = (int32_t)(per_max * kSuper);
    pl->row_words = (uint64_t)kWsCand + (uint64_t)wg * (uint64_t)pl->cand_per_wg * 2u;
    // 256 bytes of header (the status word) before the rows
    pl->ws_bytes = wg > 1 ? kWsHeader + (size_t)rows * (size_t)pl->row_words * sizeof(uint32_t) : 0;
    return CK_OK;
}

}  // namespace cktk

extern "C" {

int ck_decode_topk_plan(const ck_decode_shape* shape, int32_t Hs, int32_t k, int32_t tail, int num_cus,
                        int32_t* wgs_per_row, size_t* workspace_bytes) {
    if (!wgs_per_row || !workspace_bytes) return CK_ERR_ARG;
    cktk::Plan pl;
    const int st = cktk::plan(shape, Hs, k, tail, num_cus, &pl);
    if (st != CK_OK) return st;
    *wgs_per_row = pl.P;
    *workspace_bytes = pl.ws_bytes;
    return CK_OK;
}

int ck_decode_topk_workspace_size(const ck_decode_shape* shape, int32_t Hs, int32_t k, int32_t tail,
                                  size_t* bytes) {
    if (!bytes) return CK_ERR_ARG;
    cktk::Plan pl;
    int st = cktk::plan(shape, Hs, k, tail, 1, &pl);
    if (st != CK_OK) return st;
    int cus = 0;
    st = cktk::device_cus(&cus);
    if (st != CK_OK) return st;
    st = cktk::plan(shape, Hs, k, tail, cus, &pl);
    if (st != CK_OK) return st;
    *bytes = pl.ws_bytes;
    return CK_OK;
}

int ck_decode_topk(const ck_decode_shape* shape, const float* scores, int32_t Hs, const int32_t* kv_lens,
                   int32_t k, int32_t tail, int causal, int32_t* idx, void* workspace, size_t workspace_bytes,
                   void* stream) {
    cktk::Plan pl;
    int st = cktk::plan(shape, Hs, k, tail, 1, &pl);
    if (st != CK_OK) return st;
    if (!scores || !kv_lens || !idx) return CK_ERR_ARG;
    if (((uintptr_t)scores & 3) || ((uintptr_t)kv_lens & 3) || ((uintptr_t)idx & 3)) return CK_ERR_ALIGN;
    int cus = 0;
    st = cktk::device_cus(&cus);
    if (st != CK_OK) return st;
    st = cktk::plan(shape, Hs, k, tail, cus, &pl);
    if (st != CK_OK) return st;
    if (pl.ws_bytes > 0) {
        if (!workspace || workspace_bytes < pl.ws_bytes) return CK_ERR_WORKSPACE;
        if ((uintptr_t)workspace & 255) return CK_ERR_ALIGN;
    }
    cktk::TParams p{};
    p.scores = scores;
    p.kv_lens = kv_lens;
    p.idx = idx;
    p.status = (int32_t*)workspace;
    p.ws = workspace ? (uint32_t*)((char*)workspace + cktk::kWsHeader) : nullptr;
    p.spin_limit = ckda::spin_limit();
    p.B = shape->B;
    p.n_q = shape->n_q;
    p.Hs = Hs;
    p.cap = shape->cap;
    p.causal = causal ? 1 : 0;
    p.k = k;
    p.tail = tail;
    p.W = k + tail;
    p.P = pl.P;
    p.vec4 = ((uintptr_t)scores & 15) == 0 && shape->cap % 4 == 0 ? 1 : 0;
    p.cand_per_wg = pl.cand_per_wg;
    p.cand_off = (uint32_t)cktk::kWsCand;
    p.ws_row_words = pl.row_words;
    const int rows = shape->B * shape->n_q * Hs;
    if (pl.cand_per_wg <= cktk::kSuper)  // one super-block per workgroup
        hipLaunchKernelGGL(cktk::topk_kernel<1>, dim3((unsigned)(rows * pl.P)), dim3(cktk::kThreads), 0,
                           (hipStream_t)stream, p);
    else
        hipLaunchKernelGGL(cktk::topk_kernel<cktk::kCacheMany>, dim3((unsigned)(rows * pl.P)),
                           dim3(cktk::kThreads), 0, (hipStream_t)stream, p);
    return hipGetLastError() == hipSuccess ? CK_OK : CK_ERR_HIP;
}

}  // extern "C"
