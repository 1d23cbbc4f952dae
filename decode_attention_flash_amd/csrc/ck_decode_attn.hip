// Length-aware split-KV GQA decode attention for gfx950 (MI355X).
//
// One workgroup (4 waves of 64 lanes) takes one (unit, split): a unit is a
// (sequence, [query,] KV head, row group), a split is a contiguous range of
// cache positions (dense) or of index-list entries (gather).  The query
// rows of the unit -- the GQA group's query heads times the causal window's
// queries -- ride as the N side of 16x16x32 bf16 MFMAs against 16-token
// tiles of K, so every K/V byte is read once for all of them (comfy-kitchen
// PR "Performance improvements for qwen 3.x LLM (Part 1)", GQA decode).
// More rows than one group holds go to several 16-row groups, whose
// workgroups run on one XCD and share each tile through its L2.
// Only positions below the device-side length are read (ComfyUI issue
// "Qwen3.5 text generation attends over the full KV capacity every step…",
// Feature Idea), an online softmax runs per split, and the workgroup that
// finishes a unit's last split merges the splits in the same launch (same
// comfy-kitchen PR, GQA decode), so the launch has a fixed shape.
//
// Per wave and tile (TT tokens, TT*D*2 = 16 KiB of K and as much of V; 8 KiB
// with one row tile, where two workgroups share a CU):
//   K,V : row-major buffer loads (each instruction reads whole cache rows,
//         which streams faster than the 16-row x 64-byte pattern of an MFMA
//         operand), staged in LDS; rows past the split or the visible limit
//         come back as zeros from the buffer range check, so garbage is never
//         read.  The next tile's loads go out as soon as this one is staged.
//   K   : read back from LDS as the MFMA A operand (lane l holds token l%16
//         of a 16-token block, 8 consecutive head-dim values).
//   S^T = K Q^T on MFMA, C layout: lane l holds query row l%16 and tokens
//         4*(l/16)+0..3 of each 16-token block.
//   softmax on those registers; P^T for PV is the same registers rounded to
//         bf16 (token order inside the 32-token k-block is permuted the same
//         way on both operands, which leaves the contraction unchanged).
//   V   : row-major buffer loads, staged in LDS, read back transposed
//         (lane: head-dim column l%16, 8 tokens) as the A operand of
//         O^T += V^T P^T, whose C layout again gives lane l query row l%16.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "ck_decode_attn.h"

namespace ckda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9 raw buffer descriptor, dword data format
constexpr uint32_t kOOB = 0x80000000u;        // an offset beyond every range we build
constexpr int kBtFirst = 4 * 64;               // block-table entries loaded with the length
constexpr int kMaxQueries = CK_MAX_NQ;         // query rows per sequence (n_q)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLn2 = 0.69314718055994530942f;
// Per unit, kCntStride ints of the workspace: a parity word naming the
// counter set the next launch uses, then two counter sets (splits started,
// splits arrived, one claim flag per merge slice), each field on its own
// 128-byte line.
constexpr int kCntStride = 512, kParity = 0, kSet0 = 128, kSetStride = 128;
constexpr int kStarted = 0, kArrived = 32, kSliceFlag = 64;
constexpr int kMaxSlices = 64;  // slice claims are collected by one wave's ballot
static_assert(kMaxSlices <= 64, "one claim per lane of a wave");
constexpr int kPlanSlices = 16;  // the plan's limit (see plan_impl)
// Short work: with an automatic split count, a unit whose span holds at most
// kSingleSplitBytes of K+V (4·D bytes per position) is streamed by one split,
// which writes the output itself: the split merge's store, arrival and
// read-back cost more than one workgroup's read of that much (head_dim 128
// at 100 / 200 tokens: 4.35 / 5.55 us against 6.9 / 7.2; 160 KiB measured
// even, 200 KiB slower).  A merge of at most kSingleSliceBytes of partials
// runs as one column slice (no helpers): their claim and polling cost more
// than they share (head_dim 128, 300-1000 tokens: 0.4-0.5 us less; 64 KiB
// was slower at head_dim 256).
constexpr int64_t kSingleSplitBytes = 128 * 1024;
constexpr int64_t kSingleSliceBytes = 32 * 1024;
static_assert(kPlanSlices <= kMaxSlices, "slices per unit");

// Bytes of K per wave tile.  With one row tile (up to 16 packed rows) the
// kernel needs under 256 VGPRs, so with 8 KiB tiles (32 tokens at D = 128,
// 16 at D = 256; under 80 KiB of LDS) two workgroups share a CU: two waves
// per SIMD, and one wave's conversions, softmax and stores run while the
// other waits for its loads.  Two row tiles need 350-510 VGPRs: one wave per
// SIMD, which takes 16 KiB tiles.
constexpr int tile_bytes(int RT) { return RT == 1 ? 8192 : 16384; }
constexpr int waves_per_simd(int RT) { return RT == 1 ? 2 : 1; }

template <int D, int TB>
struct Geo {
    static constexpr int TT = TB / (2 * D);  // tokens per wave tile
    static constexpr int MB = TT / 16;          // 16-token blocks per tile (QK M side)
    static constexpr int KS = D / 32;           // k-steps of the QK contraction
    static constexpr int KB = TT / 32;          // 32-token k-blocks of PV
    static constexpr int NB = D / 16;           // 16-wide head-dim blocks of PV
    static constexpr int CPR = D / 8;           // 16-byte chunks per cache row
    static constexpr int RPI = 64 / CPR;        // cache rows per V load instruction
    static constexpr int VI = TT / RPI;         // V load instructions per tile
    // LDS row stride of the staged V tile: 32 bytes of skew puts the four rows
    // a 16-lane group reads in one transposed load on disjoint bank ranges.
    static constexpr int RS = 2 * D + 32;
    static constexpr int VBYTES = TT * RS;  // LDS bytes per wave for staged V
    // LDS row stride of the staged K tile: 16 bytes of skew puts the 16 rows
    // that one A-operand read touches (same columns) on disjoint banks.
    static constexpr int RSK = 2 * D + 16;
    static constexpr int KBYTES = TT * RSK;
    static constexpr int STAGE = KBYTES + VBYTES;  // LDS bytes per wave
    // Paged INT8 cache: 16-byte chunks of an int8 row, rows per load
    // instruction, load instructions per tile.
    static constexpr int CPR8 = D / 16;
    static constexpr int RPI8 = 64 / CPR8;
    static constexpr int VI8 = TT / RPI8;
};

struct KParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* k_step;  // step rows [B, n_q, Hkv, D] merged into the prefix, or null
    const uint16_t* v_step;
    const int32_t* kv_lens;
    const uint8_t* keep_mask;
    const int32_t* idx;
    void* out;
    float* lse;
    float* ws_o;
    float* ws_ml;
    int32_t* ws_cnt;     // per unit kCntStride ints: counters and slice claim flags
    int32_t* ws_status;  // sticky error bits (CK_WS_*), set with an atomic OR
    int32_t spin_limit;  // polls a merge helper makes before it gives up
    uint64_t* stamps;    // phase timestamps, kStampWords per workgroup, or null
    int32_t stamp_wgs;   // workgroups the stamp buffer holds
    // paged INT8 cache (MODE 3)
    const int8_t* kq;
    const int8_t* vq;
    const float* ksc;
    const float* vsc;
    const int32_t* block_table;  // [B, max_pages]
    int32_t page, max_pages, num_pages;
    int32_t B, n_q, Hq, Hkv, G, cap;
    int32_t R, RG, rows_alloc;
    int32_t units;   // work units (grid = splits x units)
    int32_t splits;  // grid splits per unit
    int32_t S_target, c_min, c_max, gran;
    int32_t S_win, win_span;  // spans of at most win_span positions aim at S_win splits
    int32_t auto_splits;  // split count chosen by the plan (short spans take one split)
    int32_t slices;  // column slices of the merge
    int32_t W;
    int64_t idx_head_stride;  // 0: one list per query shared by its heads
    float scale_log2;         // softmax scale times log2(e)
    int32_t causal, out_bf16;
    int32_t mask_dw;     // keep_mask rows start 4-byte aligned: read 4 cells per load
    int32_t mask_skip;   // keep_mask rows start 16-byte aligned: tiles without a kept cell are skipped
    uint32_t row_bytes;  // bytes between consecutive positions of one head
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             (int)kRsrcWord3);
}

// 16-byte buffer load; out-of-range offsets read as zero.  aux 2 marks the
// access non-temporal (streamed once).
template <int AUX = 0>
__device__ __forceinline__ u32x4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}

// Device-coherent accesses (cache policy sc1): stores write through to the
// point of coherence of the whole device and loads are served from there, so
// workgroups on different XCDs (each with its own L2) see each other's data.
// They are the instructions the compiler itself uses for agent-scope relaxed
// atomic stores and loads.
constexpr int kAuxDevice = 16;

template <typename T>
__device__ __forceinline__ void store_dev(__amdgpu_buffer_rsrc_t r, uint32_t off, T v);
template <>
__device__ __forceinline__ void store_dev<f32x4>(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kAuxDevice);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <>
__device__ __forceinline__ void store_dev<f32x2>(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, kAuxDevice);
}
__device__ __forceinline__ f32x4 load_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxDevice));
}
__device__ __forceinline__ f32x2 load_dev2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kAuxDevice));
}
// Wait until every store this wave issued has completed (vmcnt = 0; the
// expcnt and lgkmcnt fields are left at their maxima).
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 lds_bf16x4;
typedef short s16x4 __attribute__((ext_vector_type(4)));
// 16x16x16 bf16 MFMA (a 16-token k-block): lane l holds 4 k-values of row
// (A) or column (B) l % 16, k-group l / 16.
__device__ __forceinline__ f32x4 mfma_k16(lds_bf16x4 a, lds_bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                     0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The low and high bf16 of a dword, widened to fp32 (exact).
__device__ __forceinline__ float bf_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

// Two bf16 products summed into an fp32 accumulator (v_dot2c_f32_bf16).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Transposed LDS read (gfx950): within each 16-lane group, lane j receives
// element j%4 of the 64-bit words read by lanes 4e+j/4, e = 0..3.
__device__ __forceinline__ lds_bf16x4 lds_read_tr(const unsigned char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) lds_bf16x4*)((__attribute__((address_space(3))) unsigned char*)(p)));
}

// Orders this wave's LDS writes before its later LDS reads (and the reverse)
// without waiting on outstanding global loads.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Phase timestamps (diagnostic instances of the kernel only, ST = true):
// thread 0 of workgroup w writes the 100 MHz real-time counter to word k of
// its kStampWords.  Words: 0 start, 1 length known, 2 first tile loaded
// (wave 0), 3 tile loop done (wave 0), 4 all waves done, 5 partial (or
// output) stores complete, 6 arrival rank known, 7 merge begins, 8 merge
// ends; 13 the slices this workgroup merged, 14 the arrival rank, 15 split
// | unit << 16 | n_active << 32 | role << 48 (1 last arrival, 2 helper that
// merged, 3 other).  Words of phases a workgroup never reaches stay as they
// were.  (A run-time switch in every kernel cost 0.5-2 us per launch: each
// test reloads the pointer from the kernel arguments and waits for it.)
constexpr int kStampWords = 16;
template <bool ST, typename P>
__device__ __forceinline__ void stamp(const P& p, int k, uint64_t v = 0, bool raw = false) {
    if constexpr (ST) {
        if (threadIdx.x == 0 && (int)blockIdx.x < p.stamp_wgs)
            p.stamps[(size_t)blockIdx.x * kStampWords + k] = raw ? v : __builtin_amdgcn_s_memrealtime();
    }
}

__device__ __forceinline__ int atomic_ld(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_st(int32_t* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Length of the range one split takes; the same arithmetic runs in every
// workgroup of a unit, so they agree on the split count.  It never yields
// more splits than the grid holds.
__device__ __forceinline__ int chunk_len(int span, const KParams& p) {
    const int S = span <= p.win_span ? p.S_win : p.S_target;
    int c = (span + S - 1) / S;
    c = (c + p.gran - 1) / p.gran * p.gran;
    if (c < p.c_min) c = p.c_min;
    if (p.c_max > 0 && c > p.c_max) c = p.c_max;
    int need = (span + p.splits - 1) / p.splits;
    need = (need + p.gran - 1) / p.gran * p.gran;
    return c < need ? need : c;
}

template <int D, int RT>
struct Acc {
    f32x4 o[RT][D / 16];
    float m[RT], l[RT];
};

// Byte K of w, sign-extended, as a float: one SDWA conversion that selects
// and sign-extends the byte itself (left to itself the compiler first shifts
// bytes 1 and 3 down with a separate instruction).
template <int K>
__device__ __forceinline__ float sbyte_f32(uint32_t w) {
    float r;
    if constexpr (K == 0)
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(w));
    else if constexpr (K == 1)
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(w));
    else if constexpr (K == 2)
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(w));
    else
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(w));
    return r;
}

// 16 int8 codes to 16 bf16 values (exact: |code| <= 128 needs 8 significant
// bits), as two 16-byte halves: per code one conversion to fp32, per pair
// one packing conversion to bf16.
__device__ __forceinline__ void i8x16_to_bf16(u32x4 w, u32x4& lo, u32x4& hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    uint32_t d[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2 a = {(__bf16)sbyte_f32<0>(w[i]), (__bf16)sbyte_f32<1>(w[i])};
        const bf16x2 c = {(__bf16)sbyte_f32<2>(w[i]), (__bf16)sbyte_f32<3>(w[i])};
        d[2 * i] = __builtin_bit_cast(uint32_t, a);
        d[2 * i + 1] = __builtin_bit_cast(uint32_t, c);
    }
    lo = u32x4{d[0], d[1], d[2], d[3]};
    hi = u32x4{d[4], d[5], d[6], d[7]};
}

// Bit e set where byte e of w is nonzero (4 keep_mask cells).
__device__ __forceinline__ uint32_t mask_bits(uint32_t w) {
    uint32_t bits = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) bits |= (uint32_t)(((w >> (8 * e)) & 0xFFu) != 0u) << e;
    return bits;
}

// Flat (b, i, h) index of packed row r of a unit.
__device__ __forceinline__ size_t out_row(const KParams& p, int b, int g, int r, int iq, bool gather) {
    int i = gather ? iq : r / p.G;
    int j = gather ? r : r % p.G;
    int h = g * p.G + j;
    return ((size_t)b * p.n_q + i) * p.Hq + h;
}

template <int D>
__device__ __forceinline__ void store4(const KParams& p, size_t row, int d, f32x4 v) {
    if (p.out_bf16) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 h;
        h[0] = (__bf16)v[0];
        h[1] = (__bf16)v[1];
        h[2] = (__bf16)v[2];
        h[3] = (__bf16)v[3];
        *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(p.out) + row * D + d) = h;
    } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + row * D + d) = v;
    }
}

struct MergeScratch {
    int flag;
    uint64_t owned;  // slices the unit's last split claimed (bit c = slice c)
};

// All-reduce over aligned groups of `span` neighbouring lanes (a power of two
// up to 64, the same in the whole wave; every lane must be active).  Steps
// inside a 16-lane row are DPP lane moves: swap neighbours, swap pairs, then
// the half-row and row mirrors, each of which pairs a lane with one of the
// other half of its group.  Wider steps go through the cross-lane permute.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <bool MAX>
__device__ __forceinline__ float group_reduce(float v, int span) {
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    if (span >= 2) v = op(v, dpp<kDppXor1>(v));
    if (span >= 4) v = op(v, dpp<kDppXor2>(v));
    if (span >= 8) v = op(v, dpp<kDppHalfMirror>(v));
    if (span >= 16) v = op(v, dpp<kDppMirror>(v));
    if (span >= 32) v = op(v, __shfl_xor(v, 16));
    if (span >= 64) v = op(v, __shfl_xor(v, 32));
    return v;
}

// The merge's reductions over groups of `span` lanes (a uniform power of
// two) as straight-line code: every DPP step runs, and a step beyond the span
// adds +0 (or takes the max with -inf) through a lane mask the compiler
// cannot turn back into a branch.  A merging wave runs this code once per
// launch, so its instruction count is its time.  Only the two cross-row
// steps sit behind one uniform branch.
__device__ __forceinline__ uint32_t opaque_mask(bool on) {
    uint32_t v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "v"(on ? ~0u : 0u));
    return v;
}
template <bool MAX>
__device__ __forceinline__ float masked_step(float v, float x, uint32_t m) {
    const uint32_t xb = __builtin_bit_cast(uint32_t, x) & m;
    if constexpr (MAX)
        return fmaxf(v, __builtin_bit_cast(float, xb | (0xFF800000u & ~m)));
    else
        return v + __builtin_bit_cast(float, xb);
}
template <bool MAX, int N>
__device__ __forceinline__ void group_reduce_masked(float (&v)[N], int span) {
    const uint32_t m2 = opaque_mask(span >= 2), m4 = opaque_mask(span >= 4);
    const uint32_t m8 = opaque_mask(span >= 8), m16 = opaque_mask(span >= 16);
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = masked_step<MAX>(v[k], dpp<kDppXor1>(v[k]), m2);
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = masked_step<MAX>(v[k], dpp<kDppXor2>(v[k]), m4);
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = masked_step<MAX>(v[k], dpp<kDppHalfMirror>(v[k]), m8);
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = masked_step<MAX>(v[k], dpp<kDppMirror>(v[k]), m16);
    if (span >= 32) {
        auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
#pragma unroll
        for (int k = 0; k < N; ++k) v[k] = op(v[k], __shfl_xor(v[k], 16));
        if (span >= 64) {
#pragma unroll
            for (int k = 0; k < N; ++k) v[k] = op(v[k], __shfl_xor(v[k], 32));
        }
    }
}

// Merge column slice `c` of `ns` for one unit from the n_active published
// partials (acc_s, m_s, l_s):  O = sum_s w_s acc_s / sum_s w_s l_s with
// w_s = 2^(m_s - max m).  Each output group (row, 4 columns) is taken by TPP
// neighbouring lanes, each lane by a strided subset of at most NS splits
// whose loads are all issued before the first use, so a pass over the
// outputs costs one round trip.  A lane takes the max of its m_s, then sums
// its weighted terms (independent exponentials, no serial chain); the TPP
// lanes then agree on the max, rescale once and sum.  The order is fixed, so
// the result does not depend on which workgroup merges or when.  NS is the
// slot count rounded up to 4, 8 or 16: every slot costs instructions whether
// or not a split fills it (a lane past the splits loads at an offset beyond
// the buffer, which reads zeros without a memory access; skipping the slots
// no lane fills, behind a uniform branch each, measured 0.1 us slower).
template <int D, int NS>
__device__ __forceinline__ void merge_slice_n(const KParams& p, int unit, int n_active, int nrows, int c, int ns,
                                              int b, int g, int iq, bool gather, int row0, int TPP) {
    constexpr int D4 = D / 4;
    const int tid = threadIdx.x;
    const int col_lo = c * D4 / ns, col_hi = (c + 1) * D4 / ns;
    const int ncol = col_hi - col_lo;
    const int P = nrows * ncol;
    const int per_pass = kThreads / TPP;
    const uint32_t unit_parts = (uint32_t)(p.splits * p.rows_alloc);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.ws_o + (size_t)unit * unit_parts * D, unit_parts * D * 4u);
    const __amdgpu_buffer_rsrc_t rml = make_rsrc(p.ws_ml + (size_t)unit * unit_parts * 2, unit_parts * 8u);
    const uint32_t sstride = (uint32_t)p.rows_alloc * D * 4u;  // bytes between splits
    const int j = tid % TPP;
    for (int pass = 0; pass * per_pass < P; ++pass) {
        const int pos = pass * per_pass + tid / TPP;
        const bool act = pos < P;
        const int rr = act ? pos / ncol : 0;
        const int col = act ? col_lo + pos % ncol : 0;
        const uint32_t xoff = (uint32_t)(rr * D + 4 * col) * 4u;
        const uint32_t moff = (uint32_t)(rr * p.splits) * 8u;
        f32x4 x[NS];
        f32x2 ml[NS];
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int s2 = j + u * TPP;
            const bool ok = act && s2 < n_active;
            x[u] = load_dev4(ro, ok ? xoff + (uint32_t)s2 * sstride : kOOB);
            ml[u] = load_dev2(rml, ok ? moff + (uint32_t)s2 * 8u : kOOB);
        }
        float M = -INFINITY;
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            ml[u][0] = (act && j + u * TPP < n_active) ? ml[u][0] : -INFINITY;
            M = fmaxf(M, ml[u][0]);
        }
        float v[5] = {0.f, 0.f, 0.f, 0.f, 0.f};  // den, acc[0..3]
        {
            const float mu = (M == -INFINITY) ? 0.f : M;
#pragma unroll
            for (int u = 0; u < NS; ++u) {
                const float w = fast_exp2(ml[u][0] - mu);
                v[0] += w * ml[u][1];
#pragma unroll
                for (int k = 0; k < 4; ++k) v[k + 1] += w * x[u][k];
            }
        }
        float mg[1] = {M};
        group_reduce_masked<true>(mg, TPP);
        const float Mg = mg[0];
        const float mu = (Mg == -INFINITY) ? 0.f : Mg;
        const float r = fast_exp2(M - mu);
#pragma unroll
        for (int k = 0; k < 5; ++k) v[k] *= r;
        group_reduce_masked<false>(v, TPP);
        if (act && j == 0) {
            const float den = v[0];
            const float inv = den > 0.f ? 1.f / den : 0.f;
            const size_t orow = out_row(p, b, g, row0 + rr, iq, gather);
            store4<D>(p, orow, 4 * col, f32x4{v[1], v[2], v[3], v[4]} * inv);
            if (col == 0 && p.lse != nullptr) p.lse[orow] = den > 0.f ? (Mg + __log2f(den)) * kLn2 : -INFINITY;
        }
    }
}

constexpr int kMergeSlots = 16;  // splits one lane of the merge holds at most
static_assert(CK_MAX_SPLITS <= 64 * kMergeSlots, "a lane holds at most kMergeSlots splits");

template <int D>
__device__ void merge_slice(const KParams& p, int unit, int n_active, int nrows, int c, int ns, int b, int g,
                            int iq, bool gather, int row0) {
    constexpr int D4 = D / 4;
    const int ncol = (c + 1) * D4 / ns - c * D4 / ns;
    const int P = nrows * ncol;
    int TPP = 1;
    while (TPP < 64 && 2 * TPP * P <= kThreads) TPP *= 2;
    while (TPP < 64 && TPP * kMergeSlots < n_active) TPP *= 2;
    const int nslot = (n_active + TPP - 1) / TPP;
    if (nslot <= 4)
        merge_slice_n<D, 4>(p, unit, n_active, nrows, c, ns, b, g, iq, gather, row0, TPP);
    else if (nslot <= 8)
        merge_slice_n<D, 8>(p, unit, n_active, nrows, c, ns, b, g, iq, gather, row0, TPP);
    else
        merge_slice_n<D, kMergeSlots>(p, unit, n_active, nrows, c, ns, b, g, iq, gather, row0, TPP);
}

// A merge that gave up: its column slice of the output (and the lse of its
// rows) reads NaN, so the failure is visible in the results as well as in
// the workspace status word.
template <int D>
__device__ void fill_slice_nan(const KParams& p, int nrows, int c, int ns, int b, int g, int iq, bool gather,
                               int row0) {
    constexpr int D4 = D / 4;
    const int col_lo = c * D4 / ns, col_hi = (c + 1) * D4 / ns, ncol = col_hi - col_lo;
    for (int k = threadIdx.x; k < nrows * ncol; k += kThreads) {
        const int rr = k / ncol, col = col_lo + k % ncol;
        const size_t orow = out_row(p, b, g, row0 + rr, iq, gather);
        store4<D>(p, orow, 4 * col, f32x4{NAN, NAN, NAN, NAN});
        if (col == 0 && p.lse != nullptr) p.lse[orow] = NAN;
    }
}

// MODE 0: dense, 1: dense with keep_mask, 2: gather, 3: dense over the paged
// INT8 cache.
// RV = 0: QK^T and PV on MFMA.  RV = 4 or 8: the alternative VALU contraction
// for up to RV packed rows (dense and gather, one row tile), kept to measure
// the choice: lane l takes row l / (64 / RV) and a slice of D / (64 / RV)
// head dims; QK^T sums bf16 pairs with v_dot2 over the slice and then over
// the row's lanes, the softmax runs in the lane, and PV takes token pairs
// (V rows paired by byte permutes) with v_dot2 into fp32 accumulators,
// which are handed to the merge in the MFMA layout.  VF: the same in plain
// fp32 (every K and V element widened, one FMA per element and token, the
// probabilities kept in fp32 instead of rounded to bf16).
template <int D, int RT, int MODE, bool CO, int RV = 0, bool ST = false, bool VF = false>
__global__ __launch_bounds__(kThreads, waves_per_simd(RT)) void decode_kernel(const KParams p) {
    static_assert(!CO || RT == 1, "row groups share tiles only with one row tile");
    static_assert(RV == 0 || ((RV == 4 || RV == 8) && RT == 1 && !CO && (MODE == 0 || MODE == 2)),
                  "the VALU contraction serves up to 8 rows of dense or gathered decode");
    static_assert(!VF || RV > 0, "the fp32 form is a VALU form");
    using Gm = Geo<D, tile_bytes(RT)>;
    constexpr int TT = Gm::TT, MB = Gm::MB, KS = Gm::KS, KB = Gm::KB, NB = Gm::NB;
    constexpr int CPR = Gm::CPR, RPI = Gm::RPI, VI = Gm::VI, RS = Gm::RS, RSK = Gm::RSK;
    constexpr bool GATHER = (MODE == 2);

    __shared__ __attribute__((aligned(16))) unsigned char smem[kWaves * Gm::STAGE];
    __shared__ float s_ml[kWaves][RT][64][2];
    __shared__ bf16x8 q_lds[RT * KS * 64];
    __shared__ MergeScratch ms;
    constexpr bool Q8 = (MODE == 3);
    // per wave: the tile's K scales, V scales and reciprocal V scales
    __shared__ float sc_lds[Q8 ? kWaves * 3 * TT : 1];

    // The wave index is uniform in its wave; saying so keeps everything
    // derived from it (tile indices, descriptors chosen per tile) in scalar
    // registers, so buffer loads never need a per-lane descriptor.
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4;
    // Split-major numbering: every unit's first split comes first and the
    // (often inactive) high splits last.  Workgroups are dealt round-robin to
    // the 8 XCDs; rotating the unit by the split index moves consecutive
    // splits of one unit to different XCDs, so each XCD gets a fair share of
    // long and short sequences.
    // CO (several 16-row groups): the row groups of one (sequence, head,
    // split) read the same tiles.  They take blocks 8 apart, so they run on
    // the same XCD and the later reads of a tile hit its L2.  Blocks come in
    // chunks of 8 x RG; the host pads the grid to whole chunks and the
    // padding blocks leave here, before any barrier.
    int s, unit;
    if constexpr (CO) {
        const int per = 8 * p.RG, within = blockIdx.x % per;
        const int idx = blockIdx.x / per * 8 + within % 8, units_nr = p.units / p.RG;
        if (idx >= units_nr * p.splits) return;
        s = idx / units_nr;
        unit = (idx % units_nr + s) % units_nr * p.RG + within / 8;
    } else {
        s = blockIdx.x / p.units;
        unit = (blockIdx.x % p.units + s) % p.units;
    }
    int t = unit;
    const int rg = t % p.RG;
    t /= p.RG;
    const int g = t % p.Hkv;
    t /= p.Hkv;
    int b, iq = 0;
    if constexpr (GATHER) {
        iq = t % p.n_q;
        b = t / p.n_q;
    } else {
        b = t;
    }
    const int row0 = rg * p.rows_alloc;
    const int nrows = min(p.rows_alloc, p.R - row0);
    stamp<ST>(p, 0);

    // ---- prologue: the length and the query rows, loaded together ----------
    // The query rows are the B operand of every QK^T MFMA.  They are the same
    // for the four waves, so the workgroup loads them once, cooperatively, into
    // LDS in operand order ([row tile][k-step][lane], 16 bytes each).
    // The unit's counter parity goes out with the length (it is needed as
    // soon as the split knows it is active); a plan with one split has no
    // workspace and no counters.
    int32_t* const ucnt = p.ws_cnt + kCntStride * unit;
    const int par_word = p.splits > 1 ? atomic_ld(ucnt + kParity) : 0;
    const int L_raw = p.kv_lens[b];
    // Paged INT8 cache: the sequence's first kBtFirst block-table entries, 16
    // bytes a lane, travel with the length.  Past the table the load reads 0.
    const __amdgpu_buffer_rsrc_t rbt =
        make_rsrc(Q8 ? p.block_table + (size_t)b * p.max_pages : p.kv_lens, Q8 ? (uint32_t)p.max_pages * 4u : 0u);
    u32x4 bt_first{0u, 0u, 0u, 0u};
    if constexpr (Q8) bt_first = bload128(rbt, (uint32_t)lane * 16u);
    constexpr int QF = RT * KS * 64 / kThreads;  // fragments per thread
    bf16x8 qfrag[QF];
    {
        const uint32_t q_bytes = (uint32_t)(p.n_q * p.Hq * D * 2);
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (size_t)b * p.n_q * p.Hq * D, q_bytes);
#pragma unroll
        for (int u = 0; u < QF; ++u) {
            const int f = tid + u * kThreads;
            const int rt = f / (KS * 64), ks = (f / 64) % KS, fl = f % 64;
            const int rr = rt * 16 + (fl & 15);
            const int r = row0 + rr;
            const int i = GATHER ? iq : r / p.G;
            const int j = GATHER ? r : r % p.G;
            // Paged INT8 cache: k-step ks of lane group q covers head dims
            // 64 (ks / 2) + 16 q + 8 (ks % 2), the order in which each lane
            // loads its K codes (16 per load) straight into MFMA operands.
            const int col = Q8 ? 64 * (ks >> 1) + 16 * (fl >> 4) + 8 * (ks & 1) : 32 * ks + 8 * (fl >> 4);
            const uint32_t qoff = rr < nrows ? (uint32_t)((i * p.Hq + g * p.G + j) * D + col) * 2u : kOOB;
            qfrag[u] = __builtin_bit_cast(bf16x8, bload128(rq, qoff));
        }
    }
    int i_r[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = row0 + rt * 16 + l16;
        i_r[rt] = GATHER ? iq : r / p.G;
    }
    const int L = L_raw < 0 ? 0 : (L_raw > p.cap ? p.cap : L_raw);
    const int span = GATHER ? p.W : L;
    const int C = p.auto_splits && (int64_t)span * 4 * D <= kSingleSplitBytes ? span : chunk_len(span, p);
    const int n_active = span > 0 ? (span + C - 1) / C : 1;
    stamp<ST>(p, 1);
    stamp<ST>(p, 15, (uint64_t)s | ((uint64_t)unit << 16) | ((uint64_t)n_active << 32) | (3ull << 48), true);
    if (s >= n_active) return;
    // The unit's counter set for this launch.  Every active split has read
    // the parity before it arrives, and only the last arrival changes it.
    const int par = __builtin_amdgcn_readfirstlane(par_word) & 1;  // uniform: the counters stay scalar
    int32_t* const cnt = ucnt + kSet0 + par * kSetStride;
    if (n_active > 1 && tid == 0) atomicAdd(cnt + kStarted, 1);  // this split has started
    const int pos_begin = s * C;
    const int pos_end = min(pos_begin + C, span);

    int lim_r[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        int lim = L;
        if (p.causal) {
            lim = L - p.n_q + i_r[rt] + 1;
            lim = lim < 0 ? 0 : (lim > L ? L : lim);
        }
        lim_r[rt] = (rt * 16 + l16) < nrows ? lim : 0;
    }

    // ---- cache views ------------------------------------------------------
    const size_t head_off = ((size_t)b * p.cap * p.Hkv + g) * D;
    int rows_lim;  // rows [0, rows_lim) of this head may be read
    int lim_g = L;
    const int32_t* list = nullptr;
    if constexpr (GATHER) {
        if (p.causal) {
            lim_g = L - p.n_q + iq + 1;
            lim_g = lim_g < 0 ? 0 : (lim_g > L ? L : lim_g);
        }
        rows_lim = lim_g;
        const int64_t hs = p.idx_head_stride;
        list = p.idx + ((size_t)b * p.n_q + iq) * (size_t)(hs == 0 ? (int64_t)p.W : (int64_t)p.Hkv * hs) +
               (size_t)(hs == 0 ? 0 : (int64_t)g * hs);
    } else {
        rows_lim = pos_end;
    }
    const uint32_t kv_bytes = rows_lim > 0 ? (uint32_t)(rows_lim - 1) * p.row_bytes + 2u * D : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + head_off, kv_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + head_off, kv_bytes);
    // Step rows (verification drafts that are not in the cache): the unit's
    // last split streams them as one extra tile, whose row t is visible to
    // query i when t <= i.
    const bool steps = MODE == 0 && RV == 0 && p.k_step != nullptr;
    const size_t step_off = ((size_t)b * p.n_q * p.Hkv + g) * D;
    const uint32_t step_bytes = (uint32_t)(p.n_q - 1) * p.row_bytes + 2u * D;
    const __amdgpu_buffer_rsrc_t rks = make_rsrc(steps ? p.k_step + step_off : p.k, steps ? step_bytes : 0u);
    const __amdgpu_buffer_rsrc_t rvs = make_rsrc(steps ? p.v_step + step_off : p.v, steps ? step_bytes : 0u);
    const size_t mask_per_b = (size_t)p.n_q * p.Hkv * p.cap;
    const __amdgpu_buffer_rsrc_t rm = MODE == 1 ? make_rsrc(p.keep_mask + (size_t)b * mask_per_b, (uint32_t)mask_per_b)
                                                : make_rsrc(p.k, 0u);

    Acc<D, RT> st;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        st.m[rt] = -INFINITY;
        st.l[rt] = 0.f;
#pragma unroll
        for (int n = 0; n < NB; ++n) st.o[rt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    unsigned char* klds = smem + wave * Gm::STAGE;
    unsigned char* vlds = klds + Gm::KBYTES;
    const int ntiles_c = (pos_end - pos_begin + TT - 1) / TT;  // cache tiles
    const int ntiles = ntiles_c + ((steps && s == n_active - 1) ? 1 : 0);
    // Whether every split of the unit has started: thread 0 reads the count
    // after its first tile's data has arrived, so the round trip hides under
    // the tile loop.  The count only grows until the unit's last arrival,
    // which cannot precede this split's own arrival.
    int started_seen = 0;

    // Gather: list entry of this lane for a tile (one entry per lane).
    auto list_entry = [&](int tile) -> int {
        const int pe = pos_begin + tile * TT + lane;
        return (tile < ntiles && lane < TT && pe < pos_end) ? list[pe] : -1;
    };
    // Paged INT8 cache: page id of a tile, read one tile ahead of its loads
    // with a vector-memory load (a scalar load would be counted with the LDS
    // accesses, and every LDS wait would then also wait for it).  Past the
    // table the load reads 0; such tiles are past the split and read nothing.
    auto page_of = [&](int tile) -> int {
        const uint32_t idx = (uint32_t)((pos_begin + tile * TT) / (Q8 ? p.page : 1));
        return __builtin_amdgcn_raw_buffer_load_b32(rbt, idx * 4u, 0, 0);
    };
    // The first tile's page comes from the entries loaded with the length
    // when it is among them, so its loads need no round trip after the
    // length is known.
    auto first_page_of = [&](int tile) -> int {
        const int idx = __builtin_amdgcn_readfirstlane((pos_begin + tile * TT) / (Q8 ? p.page : 1));
        if (idx >= kBtFirst) return page_of(tile);
        const int ln = idx >> 2, c = idx & 3;
        const uint32_t x = __builtin_amdgcn_readlane((int)bt_first[0], ln), y = __builtin_amdgcn_readlane((int)bt_first[1], ln),
                       z = __builtin_amdgcn_readlane((int)bt_first[2], ln), w = __builtin_amdgcn_readlane((int)bt_first[3], ln);
        return (int)(c == 0 ? x : c == 1 ? y : c == 2 ? z : w);
    };

    // Issue the K and V loads (and mask loads) of one tile.  Load n of a lane
    // reads 16 bytes of cache row n*RPI + lane/CPR, so one instruction covers
    // RPI whole rows.
    u32x4 kraw[VI], vraw[VI];
    u32x4 k8[Gm::VI8], v8[Gm::VI8];  // paged INT8 tile (MODE 3)
    bf16x8 kop[Q8 ? 2 * Gm::VI8 : 1];  // its K as bf16 MFMA operands, [mb][k-step]
    static_assert(Gm::VI8 * 2 == MB * KS, "one 16-code K load per two k-steps of an M block");
    float ksv = 0.f, vsv = 0.f;       // scales of token `lane` of that tile
    uint32_t mraw[RT][MB];
    constexpr bool kDeferMask = !(D == 256 && RT == 2);
    uint64_t gvalid = 0;
    auto issue = [&](int tile, int jv) {
        const bool st_tile = steps && tile == ntiles_c;
        const int tb = st_tile ? 0 : pos_begin + tile * TT;
        if constexpr (Q8) {
            // jv is the tile's page id.  The tile lies in one page (pages hold a
            // multiple of 64 tokens, tiles start at multiples of TT); the
            // descriptors cover only its readable rows, and none of an id
            // outside the pool, so such rows read as zero.
            // (Every value that shapes a descriptor goes through readfirstlane:
            // left to itself the compiler may compute one of them with vector
            // instructions, and a descriptor in vector registers makes it wrap
            // each load in a loop over the lanes.)
            const int pg = __builtin_amdgcn_readfirstlane(jv);
            const int nvalid = __builtin_amdgcn_readfirstlane(
                (pg >= 0 && pg < p.num_pages) ? max(0, min(TT, pos_end - tb)) : 0);
            const int prow_page = __builtin_amdgcn_readfirstlane(nvalid > 0 ? pg : 0);
            // pages are [Hkv][page][D]: the tile's rows of head g are contiguous
            const size_t prow = ((size_t)prow_page * p.Hkv + g) * p.page + (size_t)(tb % p.page);
            const uint32_t rstride = (uint32_t)D;
            const uint32_t cbytes =
                (uint32_t)__builtin_amdgcn_readfirstlane(nvalid > 0 ? (int)((uint32_t)(nvalid - 1) * rstride + D) : 0);
            const uint32_t sbytes = (uint32_t)__builtin_amdgcn_readfirstlane(nvalid * 4);
            const __amdgpu_buffer_rsrc_t rk8 = make_rsrc(p.kq + prow * D, cbytes);
            const __amdgpu_buffer_rsrc_t rv8 = make_rsrc(p.vq + prow * D, cbytes);
            const __amdgpu_buffer_rsrc_t rks = make_rsrc(p.ksc + prow, sbytes);
            const __amdgpu_buffer_rsrc_t rvs8 = make_rsrc(p.vsc + prow, sbytes);
            constexpr int CPR8 = Gm::CPR8, RPI8 = Gm::RPI8;
            uint32_t o8[Gm::VI8], ok8[Gm::VI8];
#pragma unroll
            for (int n = 0; n < Gm::VI8; ++n) {
                o8[n] = (uint32_t)(n * RPI8 + lane / CPR8) * rstride + (uint32_t)(lane % CPR8) * 16u;
                // K: row 16 mb + l16, head dims 64 u + 16 q4 .. + 15 (n = mb * KS / 2 + u)
                ok8[n] = (uint32_t)(16 * (n / (KS / 2)) + l16) * rstride + (uint32_t)(64 * (n % (KS / 2)) + 16 * q4);
            }
            if constexpr (CO) {  // the other row groups read these tiles again: keep them in L2
#pragma unroll
                for (int n = 0; n < Gm::VI8; ++n) k8[n] = bload128<0>(rk8, ok8[n]);
#pragma unroll
                for (int n = 0; n < Gm::VI8; ++n) v8[n] = bload128<0>(rv8, o8[n]);
            } else {
#pragma unroll
                for (int n = 0; n < Gm::VI8; ++n) k8[n] = bload128<2>(rk8, ok8[n]);
#pragma unroll
                for (int n = 0; n < Gm::VI8; ++n) v8[n] = bload128<2>(rv8, o8[n]);
            }
            const uint32_t soff = (uint32_t)lane * 4u;
            ksv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rks, soff, 0, 0));
            vsv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvs8, soff, 0, 0));
            return;
        }
        uint32_t roff[VI];
        if constexpr (GATHER) {
            const bool ok = jv >= 0 && jv < lim_g;
            const uint32_t off = ok ? (uint32_t)jv * p.row_bytes : kOOB;
            gvalid = __ballot(ok);
#pragma unroll
            for (int n = 0; n < VI; ++n) roff[n] = __shfl(off, n * RPI + lane / CPR);
        } else {
#pragma unroll
            for (int n = 0; n < VI; ++n) roff[n] = (uint32_t)(tb + n * RPI + lane / CPR) * p.row_bytes;
        }
        // Mask cells of the lane's 4 tokens per 16-token block.  An aligned
        // dword stays raw until the tile is consumed, so the issue does not
        // wait for it (except with two row tiles at D = 256, where the
        // registers are short); single bytes (unaligned rows) are reduced to
        // bits here.
        if constexpr (MODE == 1) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const uint32_t off = (rt * 16 + l16) < nrows
                                             ? (uint32_t)(i_r[rt] * p.Hkv + g) * (uint32_t)p.cap +
                                                   (uint32_t)(tb + 16 * mb + 4 * q4)
                                             : kOOB;
                    if (p.mask_dw) {  // the four bytes form one aligned dword
                        const uint32_t w = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rm, off, 0, 0);
                        mraw[rt][mb] = kDeferMask ? w : mask_bits(w);
                    } else {
                        uint32_t bits = 0;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            bits |= (uint32_t)(__builtin_amdgcn_raw_buffer_load_b8(rm, off + e, 0, 0) != 0) << e;
                        mraw[rt][mb] = bits;
                    }
                }
        }
        const uint32_t coff = (uint32_t)(lane % CPR) * 16u;
        const __amdgpu_buffer_rsrc_t rkt = st_tile ? rks : rk;
        const __amdgpu_buffer_rsrc_t rvt = st_tile ? rvs : rv;
        if constexpr (CO) {  // the other row groups read these tiles again: keep them in L2
#pragma unroll
            for (int n = 0; n < VI; ++n) kraw[n] = bload128<0>(rkt, roff[n] + coff);
#pragma unroll
            for (int n = 0; n < VI; ++n) vraw[n] = bload128<0>(rvt, roff[n] + coff);
        } else {
#pragma unroll
            for (int n = 0; n < VI; ++n) kraw[n] = bload128<2>(rkt, roff[n] + coff);
#pragma unroll
            for (int n = 0; n < VI; ++n) vraw[n] = bload128<2>(rvt, roff[n] + coff);
        }
    };

    // keep_mask: tiles that hold no kept cell of the workgroup's mask rows
    // are skipped, with neither K/V traffic nor arithmetic (they would add
    // exact zeros).  The split's tiles are taken in windows of 64: lane l
    // reads the mask cells of tile l of the window for every mask row and one
    // ballot gives the window's tile bitmap.  Every wave computes the same
    // bitmap and takes every kWaves-th set bit, so the waves share the kept
    // tiles evenly however they cluster.  When rows are not 16-byte aligned
    // every tile counts as kept.
    const int i_lo = row0 / p.G, i_hi = (row0 + nrows - 1) / p.G;
    auto window_bits = [&](int w) -> uint64_t {
        const int tile = 64 * w + lane;
        const bool in = tile < ntiles_c;
        if (!p.mask_skip) return __ballot(in);
        // All rows' loads go out before the first is used (one round trip).
        u32x4 x[kMaxQueries][TT / 16];
#pragma unroll
        for (int k = 0; k < kMaxQueries; ++k) {
            const uint32_t base =
                (uint32_t)((i_lo + k) * p.Hkv + g) * (uint32_t)p.cap + (uint32_t)(pos_begin + tile * TT);
#pragma unroll
            for (int c = 0; c < TT / 16; ++c)
                x[k][c] = k <= i_hi - i_lo ? bload128(rm, in ? base + 16u * c : kOOB) : u32x4{0u, 0u, 0u, 0u};
        }
        uint32_t any = 0;
#pragma unroll
        for (int k = 0; k < kMaxQueries; ++k)
#pragma unroll
            for (int c = 0; c < TT / 16; ++c) any |= x[k][c][0] | x[k][c][1] | x[k][c][2] | x[k][c][3];
        return __ballot(in && any != 0);
    };
    uint64_t tbits = 0;  // set bits: kept tiles of window `twin` not yet passed
    int twin = 0;
    // Drops the k lowest kept tiles still ahead, then returns the lowest one
    // left (ntiles when none): k = wave gives the wave's first tile, k =
    // kWaves its next.  Wave-uniform scalar work, except one mask round trip
    // per window crossed.
    auto pick = [&](int k) -> int {
        for (;;) {
            for (; k > 0 && tbits != 0; --k) tbits &= tbits - 1;
            if (tbits != 0) return 64 * twin + __builtin_ctzll(tbits);
            if (64 * (twin + 1) >= ntiles_c) return ntiles;
            ++twin;
            tbits = window_bits(twin);
        }
    };

    // Query fragments to LDS before the first tile's loads are issued (they
    // arrived with the length), then an LDS-only barrier after the issue.
#pragma unroll
    for (int u = 0; u < QF; ++u) q_lds[tid + u * kThreads] = qfrag[u];
    int jv_next = 0;
    int first = wave;
    if constexpr (MODE == 1) {
        tbits = window_bits(0);
        first = pick(wave);
    }
    if (first < ntiles) {
        if constexpr (GATHER) jv_next = list_entry(wave);
        if constexpr (Q8) jv_next = first_page_of(wave);
        issue(first, jv_next);
        if constexpr (GATHER) jv_next = list_entry(wave + kWaves);
        if constexpr (Q8) jv_next = page_of(wave + kWaves);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

    // VALU contraction: lane (vr, dp) holds query row vr's head dims
    // [dp * DS, dp * DS + DS) as bf16 pairs, its fp32 accumulators for those
    // dims, and the row's running max and (per lane, summed at the end) sum.
    constexpr int NDP = RV > 0 ? 64 / RV : 1, DS = D / NDP, TPL = TT / NDP;
    static_assert(RV == 0 || (TPL >= 1 && DS % 8 == 0), "VALU lane slices");
    const int vr = lane / NDP, dp = lane % NDP;
    uint32_t qv[RV > 0 && !VF ? DS / 2 : 1];
    float qf[VF ? DS : 1];
    float vacc[RV > 0 ? DS : 1];
    float m_v = -INFINITY, l_v = 0.f;
    int lim_v = 0;
    if constexpr (RV > 0) {
#pragma unroll
        for (int c = 0; c < DS / 8; ++c) {
            const int d0 = dp * DS + 8 * c;
            const u32x4 w = __builtin_bit_cast(u32x4, q_lds[(d0 / 32) * 64 + ((d0 / 8) % 4) * 16 + vr]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (VF) {
                    qf[8 * c + 2 * e] = bf_lo(w[e]);
                    qf[8 * c + 2 * e + 1] = bf_hi(w[e]);
                } else {
                    qv[4 * c + e] = w[e];
                }
            }
        }
#pragma unroll
        for (int d = 0; d < DS; ++d) vacc[d] = 0.f;
        int lim = L;
        if (p.causal) {
            lim = L - p.n_q + (GATHER ? iq : (row0 + vr) / p.G) + 1;
            lim = lim < 0 ? 0 : (lim > L ? L : lim);
        }
        lim_v = vr < nrows ? lim : 0;
    }

    if (ST && first < ntiles) {
        wait_stores();  // the first tile's loads are in
        stamp<ST>(p, 2);
    }
    for (int tile = first, next; tile < ntiles; tile = next) {
        const int tb = pos_begin + tile * TT;
        const bool st_tile = steps && tile == ntiles_c;
        const uint64_t tvalid = gvalid;
        uint32_t tmbits[RT][MB];  // keep bit e: token 16mb + 4q4 + e
        if constexpr (MODE == 1) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    tmbits[rt][mb] = (kDeferMask && p.mask_dw) ? mask_bits(mraw[rt][mb]) : mraw[rt][mb];
                }
        }
        // -- stage K and V rows in LDS, then send the next tile's loads -----
        float* scw = sc_lds + (Q8 ? wave * 3 * TT : 0);
        if constexpr (Q8) {
            // K codes become bf16 MFMA operands in registers (two k-steps per
            // load); V codes become bf16 in the LDS layout of the bf16 path;
            // the scales go beside.
            constexpr int CPR8 = Gm::CPR8, RPI8 = Gm::RPI8;
#pragma unroll
            for (int n = 0; n < Gm::VI8; ++n) {
                const int row = n * RPI8 + lane / CPR8, c8 = lane % CPR8;
                u32x4 lo, hi;
                i8x16_to_bf16(k8[n], lo, hi);
                kop[2 * n] = __builtin_bit_cast(bf16x8, lo);
                kop[2 * n + 1] = __builtin_bit_cast(bf16x8, hi);
                i8x16_to_bf16(v8[n], lo, hi);
                *reinterpret_cast<u32x4*>(vlds + row * RS + c8 * 32) = lo;
                *reinterpret_cast<u32x4*>(vlds + row * RS + c8 * 32 + 16) = hi;
            }
            if (lane < TT) {
                scw[lane] = ksv;
                scw[TT + lane] = vsv;
                scw[2 * TT + lane] = vsv > 0.f ? 1.f / vsv : 0.f;
            }
        } else {
            // keep_mask: bit t of vkeep is set when some query row of the
            // workgroup keeps token t of the tile.  V rows that no row keeps
            // are staged as zeros, so whatever those cells hold (NaN and Inf
            // included) meets only zero weights as zero values.  The 16 lanes
            // of a q4 group hold the same 4 tokens of a 16-token block for
            // different rows: their bits are OR-ed with DPP moves inside the
            // group, and lane 16 g4 of each group gives its 4 bits.  (Not
            // with two row tiles at head_dim 256, whose registers are full.)
            uint64_t vkeep = ~0ull;
            if constexpr (MODE == 1 && !(D == 256 && RT == 2)) {
                vkeep = 0;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    uint32_t a4 = 0;
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) a4 |= tmbits[rt][mb];
                    a4 |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a4, kDppXor1, 0xF, 0xF, false);
                    a4 |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a4, kDppXor2, 0xF, 0xF, false);
                    a4 |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a4, kDppHalfMirror, 0xF, 0xF, false);
                    a4 |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a4, kDppMirror, 0xF, 0xF, false);
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4)
                        vkeep |= (uint64_t)((uint32_t)__builtin_amdgcn_readlane((int)a4, 16 * g4) & 0xFu)
                                 << (16 * mb + 4 * g4);
                }
            }
#pragma unroll
            for (int n = 0; n < VI; ++n)
                *reinterpret_cast<u32x4*>(klds + (n * RPI + lane / CPR) * RSK + (lane % CPR) * 16) = kraw[n];
#pragma unroll
            for (int n = 0; n < VI; ++n) {
                const int row = n * RPI + lane / CPR;
                const bool keep = MODE != 1 || ((vkeep >> row) & 1ull);
                *reinterpret_cast<u32x4*>(vlds + row * RS + (lane % CPR) * 16) =
                    keep ? vraw[n] : u32x4{0u, 0u, 0u, 0u};
            }
        }
        wave_lds_sync();
        // The next tile's loads go out now, or after QK^T where the registers
        // of two row tiles at D = 256 would not hold them during it.
        constexpr bool kEarly = !(D == 256 && RT == 2);
        auto next_tile = [&]() -> int {
            if constexpr (MODE == 1)
                return pick(kWaves);
            else
                return tile + kWaves;
        };
        if (kEarly) next = next_tile();
        if (kEarly && next < ntiles) {
            issue(next, jv_next);
            if constexpr (GATHER) jv_next = list_entry(next + kWaves);
            if constexpr (Q8) jv_next = page_of(next + kWaves);
        }

        if constexpr (RV > 0) {
            // -- VALU: scores over the lane's head-dim slice ---------------
            float sv[TT];
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const unsigned char* kr = klds + t * RSK + dp * DS * 2;
                float a = 0.f;
#pragma unroll
                for (int c = 0; c < DS / 8; ++c) {
                    const u32x4 k4 = *reinterpret_cast<const u32x4*>(kr + 16 * c);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (VF) {
                            a = fmaf(qf[8 * c + 2 * e], bf_lo(k4[e]), a);
                            a = fmaf(qf[8 * c + 2 * e + 1], bf_hi(k4[e]), a);
                        } else {
                            a = dot2(k4[e], qv[4 * c + e], a);
                        }
                    }
                }
                sv[t] = a;
            }
            // Sum over the row's NDP lanes, scattering the tokens: at each
            // step a lane keeps half of its tokens and adds its partner's
            // copy of that half (the partner differs in the step's lane bit,
            // and keeps the other half).  Lane dp ends with the full scores
            // of tokens dp * TPL .. dp * TPL + TPL - 1.
            auto rs_step = [&](auto ctrl, int bit, int half) {
                const bool up = (dp >> bit) & 1;
#pragma unroll
                for (int i = 0; i < TT / 2; ++i) {
                    if (i < half) {
                        const float send = up ? sv[i] : sv[half + i];
                        const float keep = up ? sv[half + i] : sv[i];
                        sv[i] = keep + dpp<decltype(ctrl)::value>(send);
                    }
                }
            };
            using Mir = std::integral_constant<int, kDppMirror>;
            using HMir = std::integral_constant<int, kDppHalfMirror>;
            using X2 = std::integral_constant<int, kDppXor2>;
            using X1 = std::integral_constant<int, kDppXor1>;
            if constexpr (NDP == 16) rs_step(Mir{}, 3, TT / 2);
            rs_step(HMir{}, 2, TT / (NDP / 4));
            rs_step(X2{}, 1, TT / (NDP / 2));
            rs_step(X1{}, 0, TT / NDP);
            if (tid == 0 && tile == first && n_active > 1) started_seen = atomic_ld(cnt + kStarted);

            // -- online softmax of the lane's TPL tokens ----------------------
            const int tok0 = dp * TPL;
            const int lim_off = GATHER ? 0 : min(lim_v, pos_end) - tb;
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                const int off = tok0 + i;
                const bool ok = GATHER ? (vr < nrows && ((tvalid >> off) & 1ull)) : off < lim_off;
                const float x = ok ? sv[i] * p.scale_log2 : -INFINITY;
                sv[i] = x;
                mx = fmaxf(mx, x);
            }
            mx = group_reduce<true>(mx, NDP);
            const float m_new = fmaxf(m_v, mx);
            const float mu = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_v - mu);
            float lsum = 0.f;
            uint16_t ph[TPL];
            float pf[TPL];
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                if constexpr (VF) {
                    pf[i] = fast_exp2(sv[i] - mu);
                    lsum += pf[i];
                } else {
                    const __bf16 h = (__bf16)fast_exp2(sv[i] - mu);
                    ph[i] = __builtin_bit_cast(uint16_t, h);
                    lsum += (float)h;
                }
            }
            l_v = l_v * alpha + lsum;
            m_v = m_new;
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int d = 0; d < DS; ++d) vacc[d] *= alpha;
            }
            // The row's TT probabilities go through LDS (over the consumed K
            // tile) so that every lane of the row has them all.
            if constexpr (VF) {
                float* prowf = reinterpret_cast<float*>(klds) + vr * TT;
#pragma unroll
                for (int i = 0; i < TPL; ++i) prowf[tok0 + i] = pf[i];
                wave_lds_sync();
                float pt[TT];
#pragma unroll
                for (int c = 0; c < TT / 4; ++c) {
                    const f32x4 w = *reinterpret_cast<const f32x4*>(prowf + 4 * c);
#pragma unroll
                    for (int e = 0; e < 4; ++e) pt[4 * c + e] = w[e];
                }
                // -- O += P V, one FMA per element and token ---------------
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    const unsigned char* v0 = vlds + t * RS + dp * DS * 2;
#pragma unroll
                    for (int c = 0; c < DS / 8; ++c) {
                        const u32x4 a = *reinterpret_cast<const u32x4*>(v0 + 16 * c);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            vacc[8 * c + 2 * e] = fmaf(pt[t], bf_lo(a[e]), vacc[8 * c + 2 * e]);
                            vacc[8 * c + 2 * e + 1] = fmaf(pt[t], bf_hi(a[e]), vacc[8 * c + 2 * e + 1]);
                        }
                    }
                }
                wave_lds_sync();
                continue;
            }
            uint16_t* prow = reinterpret_cast<uint16_t*>(klds) + vr * TT;
#pragma unroll
            for (int i = 0; i < TPL; ++i) prow[tok0 + i] = ph[i];
            wave_lds_sync();
            uint32_t pp[TT / 2];
#pragma unroll
            for (int c = 0; c < TT / 8; ++c) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(prow + 8 * c);
#pragma unroll
                for (int e = 0; e < 4; ++e) pp[4 * c + e] = w[e];
            }

            // -- O += P V, two tokens per v_dot2 --------------------------
            // The bf16 pair (V[t][d], V[t+1][d]) is put together from the two
            // rows' dwords with a byte permute.
#pragma unroll
            for (int j = 0; j < TT / 2; ++j) {
                const unsigned char* v0 = vlds + (2 * j) * RS + dp * DS * 2;
#pragma unroll
                for (int c = 0; c < DS / 8; ++c) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(v0 + 16 * c);
                    const u32x4 b2 = *reinterpret_cast<const u32x4*>(v0 + RS + 16 * c);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t lo = __builtin_amdgcn_perm(b2[e], a[e], 0x05040100u);
                        const uint32_t hi = __builtin_amdgcn_perm(b2[e], a[e], 0x07060302u);
                        vacc[8 * c + 2 * e] = dot2(lo, pp[j], vacc[8 * c + 2 * e]);
                        vacc[8 * c + 2 * e + 1] = dot2(hi, pp[j], vacc[8 * c + 2 * e + 1]);
                    }
                }
            }
            wave_lds_sync();
            continue;
        }

        // -- S^T = K Q^T ---------------------------------------------------
        f32x4 sc[RT][MB];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) sc[rt][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 ka = Q8 ? kop[mb * KS + ks]
                                     : *reinterpret_cast<const bf16x8*>(klds + (16 * mb + l16) * RSK + 64 * ks + 16 * q4);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) sc[rt][mb] = mfma(ka, q_lds[(rt * KS + ks) * 64 + lane], sc[rt][mb]);
            }

        if (!kEarly) next = next_tile();
        if (!kEarly && next < ntiles) {
            issue(next, jv_next);
            if constexpr (GATHER) jv_next = list_entry(next + kWaves);
            if constexpr (Q8) jv_next = page_of(next + kWaves);
        }
        if (tid == 0 && tile == first && n_active > 1) started_seen = atomic_ld(cnt + kStarted);

        // -- online softmax (log2 domain) -----------------------------------
        bf16x8 pb[RT][KB > 0 ? KB : 1];  // PV B operands of the 32-token k-blocks
        lds_bf16x4 p16[RT];               // of a 16-token tile
        // Paged INT8 cache: the K scale multiplies the score of its token, the
        // V scale the probability that weights its codes.
        // Each probability is rounded to bf16 after the V scale is applied;
        // the denominator takes that rounded weight back over the scale, so
        // the output stays a convex combination of the dequantized rows (one
        // visible cell returns its row exactly).  A zero scale (zero row)
        // keeps the plain rounded probability.
        f32x4 kss[MB], vss[MB], ivs[MB];
        if constexpr (Q8) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                kss[mb] = *reinterpret_cast<const f32x4*>(scw + 16 * mb + 4 * q4) * p.scale_log2;
                vss[mb] = *reinterpret_cast<const f32x4*>(scw + TT + 16 * mb + 4 * q4);
                ivs[mb] = *reinterpret_cast<const f32x4*>(scw + 2 * TT + 16 * mb + 4 * q4);
            }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const bool row_ok = (rt * 16 + l16) < nrows;
            // Tokens of this tile below lim_off are visible to the lane's row:
            // the cache limit, or for the step tile the query's own index + 1.
            const int lim_off = GATHER ? 0
                                       : (st_tile ? (row_ok ? i_r[rt] + 1 : 0) : min(lim_r[rt], pos_end) - tb);
            float mx = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int off = 16 * mb + 4 * q4 + e;
                    bool ok;
                    if constexpr (GATHER) {
                        ok = row_ok && ((tvalid >> off) & 1ull);
                    } else {
                        ok = off < lim_off;
                        if constexpr (MODE == 1) ok = ok && ((tmbits[rt][mb] >> e) & 1u);
                    }
                    const float x = ok ? sc[rt][mb][e] * (Q8 ? kss[mb][e] : p.scale_log2) : -INFINITY;
                    sc[rt][mb][e] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(st.m[rt], mx);
            const float mu = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(st.m[rt] - mu);
            float lsum = 0.f;
            __bf16 ph[MB][4];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float pe = fast_exp2(sc[rt][mb][e] - mu);
                    if constexpr (Q8) {
                        const __bf16 h = (__bf16)(pe * vss[mb][e]);
                        ph[mb][e] = h;
                        lsum += vss[mb][e] > 0.f ? (float)h * ivs[mb][e] : (float)(__bf16)pe;
                    } else {
                        const __bf16 h = (__bf16)pe;
                        ph[mb][e] = h;
                        lsum += (float)h;
                    }
                }
            st.l[rt] = st.l[rt] * alpha + lsum;
            st.m[rt] = m_new;
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int n = 0; n < NB; ++n) st.o[rt][n] *= alpha;
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 8; ++e) pb[rt][kb][e] = e < 4 ? ph[2 * kb][e] : ph[2 * kb + 1][e - 4];
            if constexpr (TT == 16) p16[rt] = lds_bf16x4{ph[0][0], ph[0][1], ph[0][2], ph[0][3]};
        }

        // -- O^T += V^T P^T with V^T read transposed from LDS ---------------
        // Lane (group q4, k = l16) reads 4 head-dim values of token row
        // 32kb + 4q4 + k/4 (and + 16 for the upper half of the k-slots).  It
        // receives head-dim column l16 of tokens 32kb + 4q4 .. +3 (+16).
        wave_lds_sync();
        if constexpr (TT == 16) {
            // A 16-token tile is one k-block of 16x16x16 MFMAs: the
            // transposed read is the A operand and the lane's 4 probabilities
            // (tokens 4q4 .. 4q4+3 of its row) the B operand, unpermuted.
            const unsigned char* row_lo = vlds + (4 * q4 + (l16 >> 2)) * RS + (l16 & 3) * 8;
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                const lds_bf16x4 va = lds_read_tr(row_lo + 32 * n);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) st.o[rt][n] = mfma_k16(va, p16[rt], st.o[rt][n]);
            }
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const unsigned char* row_lo = vlds + (32 * kb + 4 * q4 + (l16 >> 2)) * RS + (l16 & 3) * 8;
            const unsigned char* row_hi = row_lo + 16 * RS;
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                const lds_bf16x4 lo = lds_read_tr(row_lo + 32 * n);
                const lds_bf16x4 hi = lds_read_tr(row_hi + 32 * n);
                const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) st.o[rt][n] = mfma(va, pb[rt][kb], st.o[rt][n]);
            }
        }
        wave_lds_sync();
    }

    stamp<ST>(p, 3);
    // Row sums were kept per lane (each lane saw 4 of every 16 tokens, or
    // with the VALU contraction TPL of every TT).
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        st.l[rt] += __shfl_xor(st.l[rt], 16);
        st.l[rt] += __shfl_xor(st.l[rt], 32);
    }
    if constexpr (RV > 0) l_v = group_reduce<false>(l_v, NDP);

    // ---- merge the four waves' states and publish ---------------------------
    // Every wave dumps its (m, l, acc) to LDS in its MFMA register layout; then
    // each thread merges a few (row, 4 columns) output groups of the valid
    // rows across the four waves and writes them: the final output when the
    // unit has a single split, else this split's partial (unnormalised acc,
    // m, l) with device-coherent stores.  Row tiles are dumped in rounds when
    // all of them do not fit in LDS at once.
    constexpr int RT_ROUND = (RT * NB * 64 * 16 <= Gm::STAGE) ? RT : 1;
    static_assert(RT_ROUND * NB * 64 * 16 <= Gm::STAGE, "a wave's dump exceeds its staging area");
    static_assert(Gm::STAGE % 16 == 0, "16-byte dump slots");
    // Wave w dumps into its own staging area, which no other wave touches, so
    // the first round's dump needs no barrier before it.
    auto dump_of = [&](int w) { return reinterpret_cast<f32x4*>(smem + w * Gm::STAGE); };
    const uint32_t unit_parts = (uint32_t)(p.splits * p.rows_alloc);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.ws_o + (size_t)unit * unit_parts * D, unit_parts * D * 4u);
    const __amdgpu_buffer_rsrc_t rml = make_rsrc(p.ws_ml + (size_t)unit * unit_parts * 2, unit_parts * 8u);
    if constexpr (RV == 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            s_ml[wave][rt][lane][0] = st.m[rt];
            s_ml[wave][rt][lane][1] = st.l[rt];
        }
    } else if (dp == 0) {
        s_ml[wave][0][vr][0] = m_v;
        s_ml[wave][0][vr][1] = l_v;
    }
#pragma unroll
    for (int rt0 = 0; rt0 < RT; rt0 += RT_ROUND) {
        if (ST || rt0 > 0) __syncthreads();  // the previous round's reads are done
        if (rt0 == 0) stamp<ST>(p, 4);
        if constexpr (RV == 0) {
#pragma unroll
            for (int rl = 0; rl < RT_ROUND; ++rl)
#pragma unroll
                for (int n = 0; n < NB; ++n)
                    dump_of(wave)[(rl * NB + n) * 64 + q4 * 16 + (l16 ^ ((4 * n + q4) & 15))] = st.o[rt0 + rl][n];
        } else {
            // the same slots as the MFMA layout: (row, 4 columns) of block n,
            // column group q
#pragma unroll
            for (int j = 0; j < DS / 4; ++j) {
                const int c0 = dp * DS + 4 * j, n = c0 >> 4, q = (c0 >> 2) & 3;
                dump_of(wave)[n * 64 + q * 16 + (vr ^ ((4 * n + q) & 15))] =
                    f32x4{vacc[4 * j], vacc[4 * j + 1], vacc[4 * j + 2], vacc[4 * j + 3]};
            }
        }
        __syncthreads();
        constexpr int D4 = D / 4;
        const int rows_here = min(nrows - rt0 * 16, RT_ROUND * 16);
        for (int k = tid; k < rows_here * D4; k += kThreads) {
            const int rl16 = k / D4, d4 = k % D4;
            const int rl = rl16 >> 4, r16 = rl16 & 15;
            const int rr = rt0 * 16 + rl16;
            // Slot of (row, 4 columns): the lane that held it, with the row index
            // XOR-swizzled by the column group so that threads reading
            // consecutive column groups of one row hit distinct banks.
            const int src = (d4 & 3) * 16 + (r16 ^ (d4 & 15));
            float mw[kWaves], M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                mw[w] = s_ml[w][rt0 + rl][r16][0];
                M = fmaxf(M, mw[w]);
            }
            const float mu = (M == -INFINITY) ? 0.f : M;
            float den = 0.f;
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float wt = fast_exp2(mw[w] - mu);
                den += wt * s_ml[w][rt0 + rl][r16][1];
                a += wt * dump_of(w)[(rl * NB + (d4 >> 2)) * 64 + src];
            }
            if (n_active == 1) {
                const size_t orow = out_row(p, b, g, row0 + rr, iq, GATHER);
                const float inv = den > 0.f ? 1.f / den : 0.f;
                store4<D>(p, orow, 4 * d4, a * inv);
                if (d4 == 0 && p.lse != nullptr) p.lse[orow] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
            } else {
                const uint32_t prow = (uint32_t)(s * p.rows_alloc + rr);
                store_dev<f32x4>(ro, (prow * D + 4 * d4) * 4u, a);
                if (d4 == 0) store_dev<f32x2>(rml, (uint32_t)(rr * p.splits + s) * 8u, f32x2{M, den});
            }
        }
    }
    if (n_active == 1) {
        if constexpr (ST) {
            wait_stores();
            stamp<ST>(p, 5);
        }
        return;
    }

    // ---- several splits: announce the arrival -----------------------------
    // Each wave waits for its own partial stores to complete before the
    // barrier, and thread 0 announces the arrival after it, so whichever
    // workgroup sees the arrival count reach n_active reads complete partials
    // with device-coherent loads (no L2 writeback or invalidate is needed).
    wait_stores();
    __syncthreads();
    stamp<ST>(p, 5);
    if (tid == 0) ms.flag = atomicAdd(cnt + kArrived, 1);  // arrival rank
    __syncthreads();
    const int rank = ms.flag;
    stamp<ST>(p, 6);
    stamp<ST>(p, 14, (uint64_t)rank, true);
    if (rank == n_active - 1 && wave == 0) {
        // Last arrival: every active split has read the parity, so the other
        // counter set (this unit's previous launch used it) is cleared for
        // the next launch and the parity points at it.  Nothing waits on
        // these stores; the launch boundary orders them before the next use.
        int32_t* const other = ucnt + kSet0 + (par ^ 1) * kSetStride;
        atomic_st(other + kSliceFlag + lane, 0);
        if (lane == 0) {
            atomic_st(other + kStarted, 0);
            atomic_st(other + kArrived, 0);
            atomic_st(ucnt + kParity, par ^ 1);
        }
    }

    // ---- merge: the unit's last split and the ns-1 splits that arrived just
    // before it share the ns column slices.  The last split always takes slice
    // 0; the split of rank n_active-1-c may take slice c, by winning that
    // slice's claim flag, but only if every split of the unit was already
    // running, so its wait for the other arrivals can never depend on a
    // workgroup that has not been scheduled.  After slice 0 the last split
    // claims and merges every slice no helper took.  A small merge is one
    // slice.
    const int ns = (int64_t)n_active * nrows * D * 4 <= kSingleSliceBytes ? 1 : min(p.slices, n_active);
    const bool last = rank == n_active - 1;
    const bool helper = !last && rank >= n_active - ns;
    if (!last && !helper) return;
    __syncthreads();  // everyone has read ms.flag
    // The slice this workgroup merges first: 0 for the last split; a helper's
    // own slice once it has won the claim and seen every arrival.
    int c = 0;
    if (!last) {
        c = n_active - 1 - rank;
        if (tid == 0) {
            // 0: not ours, 1: merge, 2: gave up waiting
            int ok = 0;
            if (started_seen == n_active && atomicExch(cnt + kSliceFlag + c, 1) == 0) {
                ok = 1;
                int spins = 0;
                while (atomic_ld(cnt + kArrived) < n_active) {
                    __builtin_amdgcn_s_sleep(2);
                    // Cannot happen while every split runs (they all started
                    // before the claim); if the GPU is held elsewhere that
                    // long, report it instead of waiting on.
                    if (++spins > p.spin_limit) {
                        ok = 2;
                        atomicOr(p.ws_status, CK_WS_ERR_MERGE);
                        break;
                    }
                }
            }
            ms.flag = ok;
        }
        __syncthreads();
        const int ok = ms.flag;
        if (ok == 2) fill_slice_nan<D>(p, nrows, c, ns, b, g, iq, GATHER, row0);
        if (ok != 1) return;
    }
    stamp<ST>(p, 7);
    stamp<ST>(p, 15,
              (uint64_t)s | ((uint64_t)unit << 16) | ((uint64_t)n_active << 32) | ((last ? 1ull : 2ull) << 48), true);
    // One call site for every slice (the merge is inlined once): the last
    // split's first slice is followed by its claims, then by each slice it
    // won.  ns <= 64: lane c of wave 0 claims slice c, one ballot collects
    // them.  The claims wait until slice 0 is merged: claimed at arrival they
    // take slices from helpers that arrived just before (their claims still
    // in flight), and merging those one after another cost 1.5-2.5 us on
    // short sequences.
    uint64_t more = 0;
    int merged = 0;
    for (bool first_slice = true;; first_slice = false) {
        merge_slice<D>(p, unit, n_active, nrows, c, ns, b, g, iq, GATHER, row0);
        ++merged;
        if (last && first_slice) {
            if (wave == 0) {
                const bool own = lane >= 1 && lane < ns && atomicExch(cnt + kSliceFlag + lane, 1) == 0;
                const uint64_t mask = __ballot(own);
                if (lane == 0) ms.owned = mask;
            }
            __syncthreads();
            const uint64_t owned = ms.owned;
            more = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(owned >> 32)) << 32) |
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)owned);
        }
        if (more == 0) break;
        c = __builtin_ctzll(more);
        more &= more - 1;
    }
    if constexpr (ST) {
        wait_stores();
        stamp<ST>(p, 8);
        stamp<ST>(p, 13, (uint64_t)merged, true);
    }
}

// ---------------------------------------------------- paged INT8 append ----
// One wave per (sequence, new token, KV head, K or V) row: the row's D bf16
// values become int8 codes and one fp32 scale, in fp32 with the rounding the
// format fixes (scale = amax / 127, code = x * (127 / amax) rounded half to
// even, clamped to +-127; an all-zero row gets scale 0), and land in page
// block_table[b][pos / page], row pos % page, with pos = clamp(start[b]) + t.
// Rows past the capacity, or whose page id is outside the pool, are dropped.
struct AppendParams {
    const uint16_t* k_new;  // [B, n_new, Hkv, D] bf16
    const uint16_t* v_new;
    const int32_t* start;   // [B]
    const int32_t* block_table;
    int8_t* kq;
    int8_t* vq;
    float* ksc;
    float* vsc;
    int32_t B, n_new, Hkv, page, max_pages, num_pages;
};

template <int D>
__global__ __launch_bounds__(kThreads) void q8_append_kernel(const AppendParams p) {
    constexpr int PER = D / 64;  // values per lane
    const int lane = threadIdx.x & 63;
    const int64_t row_id = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int64_t rows = (int64_t)p.B * p.n_new * p.Hkv * 2;
    if (row_id >= rows) return;
    const int which = (int)(row_id & 1);  // 0: K, 1: V
    int64_t r = row_id >> 1;
    const int g = (int)(r % p.Hkv);
    r /= p.Hkv;
    const int t = (int)(r % p.n_new);
    const int b = (int)(r / p.n_new);
    const int64_t cap = (int64_t)p.page * p.max_pages;
    int64_t s0 = p.start[b];
    s0 = s0 < 0 ? 0 : (s0 > cap ? cap : s0);
    const int64_t pos = s0 + t;
    if (pos >= cap) return;
    const int32_t pg = p.block_table[(size_t)b * p.max_pages + (size_t)(pos / p.page)];
    if (pg < 0 || pg >= p.num_pages) return;
    const uint16_t* src = (which ? p.v_new : p.k_new) + (((size_t)b * p.n_new + t) * p.Hkv + g) * D;
    float x[PER];
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        x[e] = __uint_as_float((uint32_t)src[lane * PER + e] << 16);
        amax = fmaxf(amax, fabsf(x[e]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const size_t row = ((size_t)pg * p.Hkv + g) * p.page + (size_t)(pos % p.page);
    int8_t* dst = (which ? p.vq : p.kq) + row * D + lane * PER;
    const float inv = amax > 0.f ? __fdiv_rn(127.f, amax) : 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        float c = __builtin_rintf(x[e] * inv);
        c = fminf(fmaxf(c, -127.f), 127.f);
        dst[e] = (int8_t)(int)c;
    }
    if (lane == 0) (which ? p.vsc : p.ksc)[row] = amax > 0.f ? __fdiv_rn(amax, 127.f) : 0.f;
}

// ------------------------------------------------------------------ host ----

constexpr int kWgPerCu = 1;

// Split boundaries fall on multiples of this many tokens, a multiple of the
// kernel's tiles with one and with two row tiles (16 and 32 tokens at
// D = 256, 32 and 64 at D = 128).
static int tile_tokens(int D) { return D == 256 ? 32 : 64; }
// When the units alone fill the chip, a long sequence is still cut into
// ranges of at most this many K+V bytes, so ragged batches balance over the
// CUs; each split then streams enough to amortise its fixed costs.
constexpr int64_t kChunkMaxBytes = 2 << 20;
static int chunk_max_tokens(int D) { return (int)(kChunkMaxBytes / (4 * D)); }
// A split publishes rows*D fp32 partials that are written and read back once,
// against 4*D bytes of K+V per token it streams: at least 5 tokens per packed
// row keeps that round trip under 40 % of the split's cache traffic.
constexpr int kTokensPerRow = 5;
// Units of 8 or more packed rows (12 with the INT8 cache) at head_dim 256
// over at most kWindowSpan positions: at most kWindowSplits active splits per
// unit (see the launch).
constexpr int kWindowSplits = 32;
constexpr int kWindowSpan = 6144;
// Fewest splits per group at which 17-32 packed rows still take two 16-row
// groups rather than one of 32 (see plan_impl).
constexpr int64_t kPairSplits = 16;

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// The workspace opens with 256 bytes whose first int32 is the status word.
constexpr size_t kWsHeader = 256;

// Polls a merge helper (or a top-k row barrier) makes before it gives up.
// At about a microsecond per poll the default is seconds: far beyond any
// launch whose workgroups all run, so it only ends a wait that cannot finish.
constexpr int32_t kDefaultSpinLimit = 1 << 22;
static std::atomic<int32_t> g_spin_limit{kDefaultSpinLimit};

int spin_limit() { return g_spin_limit.load(std::memory_order_relaxed); }

static int plan_impl(const ck_decode_shape* s, int32_t W, int num_splits, int num_cus,
                     ck_decode_plan* pl) {
    if (!s || !pl) return CK_ERR_ARG;
    if (s->B < 1 || s->n_q < 1 || s->Hq < 1 || s->Hkv < 1 || s->cap < 1) return CK_ERR_ARG;
    if (s->Hq % s->Hkv != 0) return CK_ERR_ARG;
    if (s->D != 128 && s->D != 256) return CK_ERR_UNSUPPORTED;
    if (s->n_q > CK_MAX_NQ) return CK_ERR_UNSUPPORTED;
    if (W < 0 || num_splits < 0 || num_splits > CK_MAX_SPLITS || num_cus < 1) return CK_ERR_ARG;
    const int64_t G = s->Hq / s->Hkv;
    const int TT = tile_tokens(s->D);
    // 32-bit buffer offsets: a whole head's cache, plus one tile of overhang.
    const int64_t row_bytes = (int64_t)s->Hkv * s->D * 2;
    if ((int64_t)(s->cap + TT) * row_bytes >= ((int64_t)1 << 31)) return CK_ERR_UNSUPPORTED;
    if (W == 0 && (int64_t)s->n_q * s->Hkv * s->cap + TT >= ((int64_t)1 << 31)) return CK_ERR_UNSUPPORTED;
    if ((int64_t)s->n_q * s->Hq * s->D * 2 >= ((int64_t)1 << 31)) return CK_ERR_UNSUPPORTED;
    const int64_t R = W > 0 ? G : (int64_t)s->n_q * G;
    const int64_t heads = (W > 0 ? (int64_t)s->B * s->n_q : (int64_t)s->B) * s->Hkv;
    // Rows are packed in 16-row groups (one row tile, two waves per SIMD;
    // the groups of a head read its tiles once from HBM and again from L2)
    // except for 17-32 rows on many heads: when each group would get fewer
    // than kPairSplits splits, the 32-row tile (one read of each tile, one
    // wave per SIMD) is faster on long caches.  Beyond 32 rows a 32-row
    // tile needs several groups as well, and 16-row groups are faster.
    const int64_t RG16 = (R + 15) / 16;
    const int rows_per_group =
        RG16 != 2 || (int64_t)num_cus * kWgPerCu / (heads * RG16) >= kPairSplits ? 16 : 32;
    const int64_t RG = (R + rows_per_group - 1) / rows_per_group;
    const int64_t units = heads * RG;
    const int64_t span_max = W > 0 ? W : s->cap;
    const int64_t rows_eff = R < rows_per_group ? R : rows_per_group;
    int64_t target, cmax, cmin = TT;
    if (num_splits == 0) {
        // As many splits as keep every unit's workgroups in one round (one
        // workgroup per CU): one more would leave a few workgroups for a
        // second round and double the time.  Where two workgroups fit on a
        // CU (D = 128, one row tile) the target stays one per CU: twice the
        // splits measured slower on long single sequences.
        target = (int64_t)num_cus * kWgPerCu / units;
        cmax = 2 * units >= num_cus ? chunk_max_tokens(s->D) : 0;
        cmin = (kTokensPerRow * rows_eff + TT - 1) / TT * TT;
    } else {
        target = num_splits;
        cmax = 0;
    }
    if (target < 1) target = 1;
    if (target > CK_MAX_SPLITS) target = CK_MAX_SPLITS;
    int64_t splits = target;
    if (cmax > 0) {
        const int64_t need = (span_max + cmax - 1) / cmax;
        if (need > splits) splits = need;
    }
    const int64_t most = (span_max + cmin - 1) / cmin;
    if (splits > most) splits = most;
    if (splits > CK_MAX_SPLITS) splits = CK_MAX_SPLITS;
    if (splits < 1) splits = 1;
    if (units * splits + 8 * RG >= ((int64_t)1 << 31)) return CK_ERR_UNSUPPORTED;

    pl->units = (int32_t)units;
    pl->splits = (int32_t)splits;
    pl->split_target = (int32_t)target;
    pl->chunk_min = (int32_t)cmin;
    pl->chunk_max = (int32_t)cmax;
    pl->granule = TT;
    pl->rows = (int32_t)R;
    pl->row_groups = (int32_t)RG;
    pl->rows_per_group = rows_per_group;
    // Column slices of the merge: about 16 KiB of partials each, at most one
    // per 4 columns and at most kPlanSlices.  Every slice but the first is
    // merged by a helper that polls the unit's arrival count.  A merging
    // lane's work follows the splits it holds, so smaller slices shorten the
    // merge: 16 against 32 KiB took 9.7 / 12.6 / 22.2 us against 10.3 / 13.1 /
    // 22.6 at kv_len 3000 / 8000 / 24000 (head_dim 256, 4 KV heads).  The cap
    // matters for 12-24 packed rows: 32 slices made n_q = 3 windows faster
    // (0.3-0.55 us) and n_q = 4-5 slower (0.2-0.35 us); with a prologue that
    // sent the first tile earlier, 31 helpers polling one word per unit made
    // a launch whose splits arrived spread out take 22 us instead of 10.7
    // (n_q = 3, kv_len 2000).  A cap of 8 was slower (n_q = 3 at 4000: 12.6
    // -> 14.9 us).
    const int64_t merge_bytes = splits * rows_eff * s->D * 4;
    int64_t slices = 1;
    while (slices * 16384 < merge_bytes && slices < s->D / 4 && slices < kPlanSlices) slices *= 2;
    pl->slices = (int32_t)slices;
    pl->tile = tile_bytes(rows_per_group / 16) / (2 * s->D);
    if (splits == 1) {
        pl->workspace_bytes = 0;
    } else {
        const size_t parts = (size_t)units * (size_t)splits * (size_t)rows_per_group;
        pl->workspace_bytes = kWsHeader + align256((size_t)units * kCntStride * sizeof(int32_t)) +
                              align256(parts * s->D * sizeof(float)) + align256(parts * 2 * sizeof(float));
    }
    return CK_OK;
}

static std::atomic<int> g_cus[64];

static int device_cus(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CK_ERR_HIP;
    if (dev >= 0 && dev < 64) {
        int c = g_cus[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return CK_OK;
        }
    }
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1)
        return CK_ERR_HIP;
    if (dev >= 0 && dev < 64) g_cus[dev].store(c, std::memory_order_relaxed);
    *cus = c;
    return CK_OK;
}

static bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

template <int D, int RT, int MODE, bool CO, int RV = 0, bool ST = false, bool VF = false>
static hipError_t launch_one(const KParams& kp, int grid, hipStream_t st) {
    void* args[] = {const_cast<KParams*>(&kp)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&decode_kernel<D, RT, MODE, CO, RV, ST, VF>), dim3(grid),
                           dim3(kThreads), args, 0, st);
}

// The VALU contraction (dense or gathered decode, at most 8 packed rows),
// on bf16 pairs or in fp32.
template <int MODE, bool VF>
static hipError_t launch_valu(int D, int rows, const KParams& kp, int grid, hipStream_t st) {
    if (D == 128)
        return rows <= 4 ? launch_one<128, 1, MODE, false, 4, false, VF>(kp, grid, st)
                         : launch_one<128, 1, MODE, false, 8, false, VF>(kp, grid, st);
    return rows <= 4 ? launch_one<256, 1, MODE, false, 4, false, VF>(kp, grid, st)
                     : launch_one<256, 1, MODE, false, 8, false, VF>(kp, grid, st);
}

// Process-wide phase-timestamp buffer (diagnostics; null: off).
static std::atomic<uint64_t*> g_stamps{nullptr};
static std::atomic<int64_t> g_stamp_wgs{0};

// Process-wide contraction choice for up to 8 packed rows (0: MFMA).
static std::atomic<int> g_contraction{CK_CONTRACT_MFMA};

template <int D, int MODE>
static hipError_t launch_d(int RT, bool co, const KParams& kp, int grid, hipStream_t st) {
    if (RT == 2) return launch_one<D, 2, MODE, false>(kp, grid, st);
    return co ? launch_one<D, 1, MODE, true>(kp, grid, st) : launch_one<D, 1, MODE, false>(kp, grid, st);
}

template <int MODE>
static hipError_t launch_mode(int D, int RT, bool co, const KParams& kp, int grid, hipStream_t st) {
    return D == 128 ? launch_d<128, MODE>(RT, co, kp, grid, st) : launch_d<256, MODE>(RT, co, kp, grid, st);
}

// ---- the file-scope scratch of ck_decode_attn_noalloc ----------------------
// For callers that cannot allocate: the split merge's workspace (status
// header, the counters of up to kScratchUnits units at fixed places, then
// the partial results) lives in this array, one copy per device, zero when
// the code object loads.  Every launch leaves each unit's next counter set
// at zero, so any sequence of shapes may share it; calls that overlap on
// one device race on it.
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int64_t kScratchUnits = 1024;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

// The device address of `scratch` on the current device (looked up once per
// device; the array's name is only a host-side stand-in).
static int scratch_ptr(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CK_ERR_HIP;
    if (dev < 0 || dev >= 64) return CK_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return CK_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return CK_OK;
}

static int run(const ck_decode_shape* s, const void* q, const void* k, const void* v, const int32_t* kv_lens,
               const uint8_t* keep_mask, const int32_t* idx, int32_t W, int64_t idx_head_stride, float scale,
               int causal, void* out, int out_dtype, float* lse, void* workspace, size_t workspace_bytes,
               int num_splits, void* stream, const void* k_step = nullptr, const void* v_step = nullptr,
               const ck_q8_cache* q8 = nullptr, int64_t counter_units = 0) {
    if (!s) return CK_ERR_ARG;
    ck_decode_plan pl;
    int st = plan_impl(s, W, num_splits, 1, &pl);  // shape checks only
    if (st != CK_OK) return st;
    if (q8) {
        // The paged INT8 cache replaces k and v: check it and its pointers.
        if (!q8->k_codes || !q8->v_codes || !q8->k_scales || !q8->v_scales || !q8->block_table)
            return CK_ERR_ARG;
        if (q8->page_tokens < 64 || q8->page_tokens % 64 != 0 || q8->max_pages < 1 || q8->num_pages < 1)
            return CK_ERR_ARG;
        if ((int64_t)q8->page_tokens * q8->max_pages != s->cap) return CK_ERR_ARG;
        if ((int64_t)q8->page_tokens * s->Hkv * s->D >= ((int64_t)1 << 31)) return CK_ERR_UNSUPPORTED;
        if (!aligned(q8->k_codes, 16) || !aligned(q8->v_codes, 16) || !aligned(q8->k_scales, 4) ||
            !aligned(q8->v_scales, 4) || !aligned(q8->block_table, 4))
            return CK_ERR_ALIGN;
        if (W > 0 || keep_mask || k_step) return CK_ERR_ARG;
        k = v = q;  // not read in this mode
    }
    if (!q || !k || !v || !kv_lens || !out) return CK_ERR_ARG;
    if ((k_step == nullptr) != (v_step == nullptr)) return CK_ERR_ARG;
    if (k_step && (W > 0 || keep_mask || causal)) return CK_ERR_ARG;
    if (k_step && (!aligned(k_step, 16) || !aligned(v_step, 16))) return CK_ERR_ALIGN;
    if (W > 0 && !idx) return CK_ERR_ARG;
    if (W > 0 && idx_head_stride != 0 && idx_head_stride < W) return CK_ERR_ARG;
    if (out_dtype != CK_DT_F32 && out_dtype != CK_DT_BF16) return CK_ERR_ARG;
    if (!isfinite(scale)) return CK_ERR_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return CK_ERR_ALIGN;
    if (!aligned(kv_lens, 4) || (lse && !aligned(lse, 4)) || (idx && !aligned(idx, 4))) return CK_ERR_ALIGN;

    int cus = 0;
    st = device_cus(&cus);
    if (st != CK_OK) return st;
    st = plan_impl(s, W, num_splits, cus, &pl);
    if (st != CK_OK) return st;
    // counter_units > 0: a workspace whose counter blocks are laid out for
    // that many units whatever the plan (the file-scope scratch), so that
    // unit u's counters sit at the same place for every shape.
    const size_t parts = (size_t)pl.units * pl.splits * pl.rows_per_group;
    const int64_t cnt_units = counter_units > 0 ? counter_units : pl.units;
    if (counter_units > 0 && pl.units > counter_units) return CK_ERR_SCRATCH;
    const size_t need = kWsHeader + align256((size_t)cnt_units * kCntStride * sizeof(int32_t)) +
                        align256(parts * s->D * sizeof(float)) + align256(parts * 2 * sizeof(float));
    if (pl.workspace_bytes > 0) {
        if (!workspace) return CK_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return CK_ERR_ALIGN;
        if (workspace_bytes < need) return counter_units > 0 ? CK_ERR_SCRATCH : CK_ERR_WORKSPACE;
    }

    KParams kp{};
    kp.q = static_cast<const uint16_t*>(q);
    kp.k_step = static_cast<const uint16_t*>(k_step);
    if (q8) {
        kp.kq = static_cast<const int8_t*>(q8->k_codes);
        kp.vq = static_cast<const int8_t*>(q8->v_codes);
        kp.ksc = q8->k_scales;
        kp.vsc = q8->v_scales;
        kp.block_table = q8->block_table;
        kp.page = q8->page_tokens;
        kp.max_pages = q8->max_pages;
        kp.num_pages = q8->num_pages;
    }
    kp.v_step = static_cast<const uint16_t*>(v_step);
    kp.k = static_cast<const uint16_t*>(k);
    kp.v = static_cast<const uint16_t*>(v);
    kp.kv_lens = kv_lens;
    kp.keep_mask = keep_mask;
    kp.idx = idx;
    kp.out = out;
    kp.lse = lse;
    if (pl.workspace_bytes > 0) {
        char* w = static_cast<char*>(workspace);
        kp.ws_status = reinterpret_cast<int32_t*>(w);
        w += kWsHeader;
        kp.ws_cnt = reinterpret_cast<int32_t*>(w);
        w += align256((size_t)cnt_units * kCntStride * sizeof(int32_t));
        kp.ws_o = reinterpret_cast<float*>(w);
        w += align256(parts * s->D * sizeof(float));
        kp.ws_ml = reinterpret_cast<float*>(w);
    }
    kp.B = s->B;
    kp.n_q = s->n_q;
    kp.Hq = s->Hq;
    kp.Hkv = s->Hkv;
    kp.G = s->Hq / s->Hkv;
    kp.cap = s->cap;
    kp.R = pl.rows;
    kp.RG = pl.row_groups;
    kp.rows_alloc = pl.rows_per_group;
    kp.units = pl.units;
    kp.splits = pl.splits;
    kp.S_target = pl.split_target;
    // Plain bf16 decode with one row group per head, when the units alone
    // leave most of the chip idle: three quarters of the planned splits are
    // active (the grid keeps the rest, which leave at once).  Fewer, longer
    // splits publish fewer partials, and the merge reads them back sooner.
    // Measured on the MI355X (us per layer, head_dim 256, 4 KV heads, cold):
    // kv_len 8000 14.3-14.5 -> 13.75, n_q = 3 at 4000 13.9 -> 12.7, kv_len
    // 1000 / 3000 / 24000 and n_q = 4 within noise.  Shared 16-row groups
    // (n_q 5-6) were slower with it (13.8 -> 14.5), the INT8 and masked
    // paths are left as planned.
    const bool few_units = !q8 && W == 0 && !keep_mask && num_splits == 0 && pl.row_groups == 1 &&
                           (int64_t)pl.units * pl.split_target * 2 > cus;
    if (few_units) kp.S_target = max(1, pl.split_target * 3 / 4);
    // Units of 8 or more packed rows at head_dim 256 (causal windows, step
    // rows, groups of 8 or more query heads) make partials 2-4 times those of
    // one query of a 4-head group, so up to kWindowSpan positions such a unit
    // aims at no more than kWindowSplits splits: their merge costs more than
    // the extra splits save on the stream.  Measured on the MI355X (us
    // per layer, B = 1, 4 KV heads, cold; 48 -> 32 splits): n_q = 3 at kv_len
    // 3000 / 4000 / 5000 / 6000 11.9 / 12.4 / 13.0 / 13.9 -> 11.1 / 11.7 /
    // 12.6 / 13.2, n_q = 4 at 4000 / 6000 13.2 / 14.8 -> 12.3 / 13.7, n_q =
    // 2 at 3000 10.7 -> 10.4, 2000 unchanged.  Longer spans keep the target:
    // with 32 splits n_q = 2 at 7000 took 13.8-14.2 against 13.1, n_q = 3 at
    // 8000 15.5 against 14.5.  With two sequences (a target of 24) halving
    // the splits was 1.0-1.3 us slower, so the bound is a cap, not a fraction.
    // The INT8 cache, which keeps every planned split otherwise, takes the
    // cap from 12 rows: n_q = 3 / 4 at kv_len 4000 13.1 / 13.8 -> 12.2 / 12.7
    // us, at 6000 14.4 / 15.5 -> 13.6 / 14.3, 2000 unchanged, while n_q = 2
    // was 0.05-0.5 us slower with it (kv_len 3000-6000).
    const bool q8_units = q8 && W == 0 && !keep_mask && num_splits == 0 && pl.row_groups == 1 &&
                          (int64_t)pl.units * pl.split_target * 2 > cus;
    kp.S_win = kp.S_target;
    kp.win_span = 0;
    if (((few_units && pl.rows >= 8) || (q8_units && pl.rows >= 12)) && s->D == 256) {
        kp.S_win = min(kp.S_target, kWindowSplits);
        kp.win_span = kWindowSpan;
    }
    kp.c_min = pl.chunk_min;
    kp.auto_splits = num_splits == 0 ? 1 : 0;
    kp.c_max = pl.chunk_max;
    kp.gran = pl.granule;
    kp.slices = pl.slices;
    kp.spin_limit = spin_limit();
    kp.stamps = g_stamps.load(std::memory_order_relaxed);
    const int64_t stamp_wgs = g_stamp_wgs.load(std::memory_order_relaxed);
    kp.stamp_wgs = kp.stamps ? (int32_t)(stamp_wgs < INT32_MAX ? stamp_wgs : INT32_MAX) : 0;
    kp.W = W;
    kp.idx_head_stride = idx_head_stride;
    kp.scale_log2 = (float)((double)scale * 1.4426950408889634074);
    kp.causal = causal ? 1 : 0;
    kp.out_bf16 = out_dtype == CK_DT_BF16 ? 1 : 0;
    kp.mask_dw = keep_mask != nullptr && aligned(keep_mask, 4) && s->cap % 4 == 0 ? 1 : 0;
    kp.mask_skip = keep_mask != nullptr && aligned(keep_mask, 16) && s->cap % 16 == 0 ? 1 : 0;
    kp.row_bytes = (uint32_t)(s->Hkv * s->D * 2);

    const int RT = pl.rows_per_group / 16;
    // Several 16-row groups: whole chunks of 8 x row_groups blocks (the
    // kernel's XCD co-location), the padding blocks exit at once.
    const bool co = RT == 1 && pl.row_groups > 1;
    const int grid = co ? (pl.units / pl.row_groups * pl.splits + 7) / 8 * 8 * pl.row_groups : pl.units * pl.splits;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int contraction = g_contraction.load(std::memory_order_relaxed);
    const bool valu = contraction != CK_CONTRACT_MFMA && !q8 && !keep_mask && !k_step && RT == 1 && !co &&
                      pl.rows <= 8;
    const bool vf = contraction == CK_CONTRACT_VALU_F32;
    // phase timestamps: the plain dense kernel with one row tile and one row
    // group has a stamping instance
    const bool stamped = kp.stamps != nullptr && !valu && !q8 && W == 0 && !keep_mask && RT == 1 && !co;
    hipError_t e;
    if (stamped)
        e = s->D == 128 ? launch_one<128, 1, 0, false, 0, true>(kp, grid, hs)
                        : launch_one<256, 1, 0, false, 0, true>(kp, grid, hs);
    else if (valu && vf)
        e = W > 0 ? launch_valu<2, true>(s->D, pl.rows, kp, grid, hs)
                  : launch_valu<0, true>(s->D, pl.rows, kp, grid, hs);
    else if (valu)
        e = W > 0 ? launch_valu<2, false>(s->D, pl.rows, kp, grid, hs)
                  : launch_valu<0, false>(s->D, pl.rows, kp, grid, hs);
    else if (q8)
        e = launch_mode<3>(s->D, RT, co, kp, grid, hs);
    else if (W > 0)
        e = launch_mode<2>(s->D, RT, co, kp, grid, hs);
    else if (keep_mask)
        e = launch_mode<1>(s->D, RT, co, kp, grid, hs);
    else
        e = launch_mode<0>(s->D, RT, co, kp, grid, hs);
    return e == hipSuccess ? CK_OK : CK_ERR_HIP;
}

}  // namespace ckda

extern "C" {

int ck_decode_attn_plan(const ck_decode_shape* shape, int32_t W, int num_splits, int num_cus,
                        ck_decode_plan* plan) {
    return ckda::plan_impl(shape, W, num_splits, num_cus, plan);
}

int ck_decode_sparse_path(const ck_decode_shape* shape, int32_t W, int64_t n_kv, int32_t* path) {
    if (!path || W < 1 || n_kv < 0) return CK_ERR_ARG;
    ck_decode_plan pl;
    const int st = ckda::plan_impl(shape, W, 0, 1, &pl);  // validates the shape
    if (st != CK_OK) return st;
    // Time model fitted (least relative error) to MI355X timings of both
    // paths (cold caches, B = 1, D 128 and 256, 2 and 4 KV heads, n_q 1-6,
    // n_kv 2k-64k, W 128-32k, scattered cells), in us, with a cell =
    // B * Hkv * 4 * D bytes (the K and V rows of every KV head at one
    // position):
    //   gather = 8.4 + 0.141 * MB of listed cells            (n_q * W cells)
    //   scan   = 10.2 + 0.30 * (n_q - 1) + (0.131 + 0.0167 * (n_q - 1)) * MB of window   (n_kv cells)
    // It names the faster path at 129 of the 135 measured points; the other
    // six are within 0.9 us of a tie.  The scan term is its cost with every
    // tile holding a kept cell; clustered selections make the scan cheaper
    // (skipped tiles), never the gather.
    const double cell_mb = (double)shape->B * shape->Hkv * 4.0 * shape->D / 1e6;
    const double extra_q = (double)(shape->n_q - 1);
    const double t_gather = 8.4 + 0.141 * (double)shape->n_q * (double)W * cell_mb;
    const double t_scan = 10.2 + 0.30 * extra_q + (0.131 + 0.0167 * extra_q) * (double)n_kv * cell_mb;
    *path = t_scan < t_gather ? CK_PATH_SCAN : CK_PATH_GATHER;
    return CK_OK;
}

int ck_decode_attn_workspace_size(const ck_decode_shape* shape, int32_t W, int num_splits, size_t* bytes) {
    if (!bytes) return CK_ERR_ARG;
    ck_decode_plan pl;
    int st = ckda::plan_impl(shape, W, num_splits, 1, &pl);
    if (st != CK_OK) return st;
    int cus = 0;
    st = ckda::device_cus(&cus);
    if (st != CK_OK) return st;
    st = ckda::plan_impl(shape, W, num_splits, cus, &pl);
    if (st != CK_OK) return st;
    *bytes = pl.workspace_bytes;
    return CK_OK;
}

int ck_decode_attn(const ck_decode_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* kv_lens, float scale, int causal, const uint8_t* keep_mask, void* out,
                   int out_dtype, float* lse, void* workspace, size_t workspace_bytes, int num_splits,
                   void* stream) {
    return ckda::run(shape, q, k_cache, v_cache, kv_lens, keep_mask, nullptr, 0, 0, scale, causal, out,
                     out_dtype, lse, workspace, workspace_bytes, num_splits, stream);
}

int ck_decode_attn_noalloc(const ck_decode_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* kv_lens, float scale, int causal, const uint8_t* keep_mask, void* out,
                           int out_dtype, float* lse, int num_splits, void* stream) {
    ck_decode_plan pl;
    int st = ckda::plan_impl(shape, 0, num_splits, 1, &pl);  // shape checks before any HIP call
    if (st != CK_OK) return st;
    void* ws = nullptr;
    st = ckda::scratch_ptr(&ws);
    if (st != CK_OK) return st;
    return ckda::run(shape, q, k_cache, v_cache, kv_lens, keep_mask, nullptr, 0, 0, scale, causal, out, out_dtype,
                     lse, ws, ckda::kScratchBytes, num_splits, stream, nullptr, nullptr, nullptr,
                     ckda::kScratchUnits);
}

int ck_decode_attn_gather(const ck_decode_shape* shape, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* kv_lens, const int32_t* idx, int32_t W,
                          int64_t idx_head_stride, float scale, int causal, void* out, int out_dtype,
                          float* lse, void* workspace, size_t workspace_bytes, int num_splits, void* stream) {
    if (W < 1) return CK_ERR_ARG;
    return ckda::run(shape, q, k_cache, v_cache, kv_lens, nullptr, idx, W, idx_head_stride, scale, causal, out,
                     out_dtype, lse, workspace, workspace_bytes, num_splits, stream);
}

int ck_decode_attn_steps(const ck_decode_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* kv_lens, const void* k_step, const void* v_step, float scale, void* out,
                         int out_dtype, float* lse, void* workspace, size_t workspace_bytes, int num_splits,
                         void* stream) {
    if (!k_step || !v_step) return CK_ERR_ARG;
    return ckda::run(shape, q, k_cache, v_cache, kv_lens, nullptr, nullptr, 0, 0, scale, 0, out, out_dtype, lse,
                     workspace, workspace_bytes, num_splits, stream, k_step, v_step);
}

int ck_decode_attn_q8(const ck_decode_shape* shape, const void* q, const ck_q8_cache* cache,
                      const int32_t* kv_lens, float scale, int causal, void* out, int out_dtype, float* lse,
                      void* workspace, size_t workspace_bytes, int num_splits, void* stream) {
    if (!cache) return CK_ERR_ARG;
    return ckda::run(shape, q, nullptr, nullptr, kv_lens, nullptr, nullptr, 0, 0, scale, causal, out, out_dtype, lse,
                     workspace, workspace_bytes, num_splits, stream, nullptr, nullptr, cache);
}

int ck_kv_append_q8(const ck_decode_shape* shape, const void* k_new, const void* v_new, const int32_t* start,
                    const ck_q8_cache* cache, void* stream) {
    if (!shape || !cache || !k_new || !v_new || !start) return CK_ERR_ARG;
    const ck_decode_shape& s = *shape;
    if (s.B < 1 || s.n_q < 1 || s.Hkv < 1) return CK_ERR_ARG;
    if (s.D != 128 && s.D != 256) return CK_ERR_UNSUPPORTED;
    if (!cache->k_codes || !cache->v_codes || !cache->k_scales || !cache->v_scales || !cache->block_table)
        return CK_ERR_ARG;
    if (cache->page_tokens < 64 || cache->page_tokens % 64 != 0 || cache->max_pages < 1 || cache->num_pages < 1)
        return CK_ERR_ARG;
    if ((int64_t)cache->page_tokens * cache->max_pages != s.cap) return CK_ERR_ARG;
    if (!ckda::aligned(k_new, 2) || !ckda::aligned(v_new, 2) || !ckda::aligned(start, 4) ||
        !ckda::aligned(cache->k_scales, 4) || !ckda::aligned(cache->v_scales, 4) ||
        !ckda::aligned(cache->block_table, 4))
        return CK_ERR_ALIGN;
    const int64_t rows = (int64_t)s.B * s.n_q * s.Hkv * 2;
    const int64_t blocks = (rows + ckda::kWaves - 1) / ckda::kWaves;
    if (blocks >= ((int64_t)1 << 31)) return CK_ERR_UNSUPPORTED;
    ckda::AppendParams ap{};
    ap.k_new = static_cast<const uint16_t*>(k_new);
    ap.v_new = static_cast<const uint16_t*>(v_new);
    ap.start = start;
    ap.block_table = cache->block_table;
    ap.kq = static_cast<int8_t*>(cache->k_codes);
    ap.vq = static_cast<int8_t*>(cache->v_codes);
    ap.ksc = cache->k_scales;
    ap.vsc = cache->v_scales;
    ap.B = s.B;
    ap.n_new = s.n_q;
    ap.Hkv = s.Hkv;
    ap.page = cache->page_tokens;
    ap.max_pages = cache->max_pages;
    ap.num_pages = cache->num_pages;
    void* args[] = {&ap};
    const void* fn = s.D == 128 ? reinterpret_cast<const void*>(&ckda::q8_append_kernel<128>)
                                : reinterpret_cast<const void*>(&ckda::q8_append_kernel<256>);
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(ckda::kThreads), args, 0,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CK_OK : CK_ERR_HIP;
}

int ck_workspace_status(const void* workspace, void* stream, int32_t* status) {
    if (!workspace || !status) return CK_ERR_ARG;
    if (!ckda::aligned(workspace, 256)) return CK_ERR_ALIGN;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int32_t v = 0;
    if (hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, hs) != hipSuccess) return CK_ERR_HIP;
    if (hipStreamSynchronize(hs) != hipSuccess) return CK_ERR_HIP;
    *status = v;
    return CK_OK;
}

int ck_set_spin_limit(int32_t polls) {
    if (polls < 0) return CK_ERR_ARG;
    ckda::g_spin_limit.store(polls == 0 ? ckda::kDefaultSpinLimit : polls, std::memory_order_relaxed);
    return CK_OK;
}

int ck_set_phase_stamps(void* stamps, int64_t workgroups) {
    if (workgroups < 0 || (stamps == nullptr) != (workgroups == 0)) return CK_ERR_ARG;
    if (stamps && !ckda::aligned(stamps, 8)) return CK_ERR_ALIGN;
    ckda::g_stamp_wgs.store(workgroups, std::memory_order_relaxed);
    ckda::g_stamps.store(static_cast<uint64_t*>(stamps), std::memory_order_relaxed);
    return CK_OK;
}

int ck_set_contraction(int32_t contraction) {
    if (contraction != CK_CONTRACT_MFMA && contraction != CK_CONTRACT_VALU && contraction != CK_CONTRACT_VALU_F32)
        return CK_ERR_ARG;
    ckda::g_contraction.store(contraction, std::memory_order_relaxed);
    return CK_OK;
}

const char* ck_status_string(int status) {
    switch (status) {
        case CK_OK: return "ok";
        case CK_ERR_ARG: return "invalid argument";
        case CK_ERR_UNSUPPORTED: return "unsupported shape";
        case CK_ERR_ALIGN: return "misaligned pointer";
        case CK_ERR_WORKSPACE: return "workspace missing or too small";
        case CK_ERR_HIP: return "HIP runtime error";
        case CK_ERR_SCRATCH: return "shape needs more than the no-alloc scratch holds";
        default: return "unknown status";
    }
}

}  // extern "C"
