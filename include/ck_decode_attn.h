/*
 * ck_decode_attn — length-aware split-KV GQA decode attention for AMD
 * Instinct MI355X (gfx950).  Plain C ABI: device pointers, sizes, an int
 * status.  No C++ types, no exceptions and no framework types cross it.
 *
 * The operation (ComfyUI issue "Qwen3.5 text generation attends over the
 * full KV capacity every step, so decode speed drops with max_length",
 * sections Feature Idea and Existing Solutions): every decode step attends
 * each query only over the filled prefix of a preallocated KV cache, whose
 * length is read on the device from kv_lens, so the cost follows the tokens
 * generated rather than the capacity.  The query heads of one KV head are
 * packed as rows against each KV tile (the GQA group), up to 6 queries per
 * sequence may form a bottom-right aligned causal window (MTP
 * verification), and head_dim is 128 or 256.
 *
 * For batch entry b, query i < n_q and query head h < Hq, with G = Hq/Hkv:
 *   g   = h / G                                (consecutive heads share a KV head)
 *   L   = clamp(kv_lens[b], 0, cap)
 *   lim = causal ? clamp(L - n_q + i + 1, 0, L) : L
 *   visible cells: dense  -> j in [0, lim), and keep_mask[b,i,g,j] != 0 if a
 *                            mask is given
 *                  gather -> idx[...][t] for t < W with 0 <= idx < lim, in
 *                            list order (a cell listed twice counts twice)
 *   out[b,i,h,:] = sum_j softmax_j(scale * q.K[b,j,g,:]) * V[b,j,g,:]
 *   lse[b,i,h]   = ln sum_j exp(scale * q.K[b,j,g,:])
 * A query with no visible cell gets out = 0 and lse = -inf.
 * Cell contents: cells at or past L are never read and may hold any bits
 * (NaN/Inf included).  Cells below L (the filled prefix, the causal window's
 * drafts included) are read in whole tiles, where a cell hidden from one
 * query row still meets that row's zero weight, so they must hold finite
 * values.  The exception is a cell that keep_mask excludes for every query
 * row of its KV head: it is staged as zeros and may hold any bits (except
 * at head_dim 256 when a workgroup holds 17-32 packed rows, see
 * ck_decode_plan.rows_per_group, where it must be finite as well).
 *
 * Layouts (all contiguous, row-major, bf16 = IEEE binary16 brain float):
 *   q        [B, n_q, Hq, D]   bf16
 *   k_cache  [B, cap, Hkv, D]  bf16
 *   v_cache  [B, cap, Hkv, D]  bf16
 *   kv_lens  [B]               int32, device memory, read by the kernel
 *   out      [B, n_q, Hq, D]   fp32 or bf16 (round to nearest even)
 *   lse      [B, n_q, Hq]      fp32 natural log, optional (NULL)
 *
 * Ownership: every pointer is a device pointer owned by the caller.  The
 * library never allocates, frees or synchronizes and never reads device
 * memory from the host, so kv_lens and idx are not checked on the host: the
 * clamp and validity rules above define every value.  Calls are stream
 * ordered on `stream` (a hipStream_t; NULL is the default stream).
 *
 * Workspace: when the plan splits the KV range (see
 * ck_decode_attn_workspace_size) the caller passes a device buffer of at
 * least that many bytes, 256-byte aligned.  It starts with a 256-byte header
 * whose first int32 is the status word (see ck_workspace_status), then a
 * 2 KiB block of int32 counters per unit: a parity word and two counter sets.
 * A launch uses the set the parity names, which is zero when it starts,
 * clears the other set and flips the parity for the next launch (the partial
 * results after the counters are scratch).  So a buffer ZEROED ONCE serves
 * any number of launches of the same plan (same shape, W, num_splits and
 * device), eager or replayed from a captured HIP graph without a memset
 * node.  A buffer used for one plan must be zeroed again before it serves a
 * different plan, and launches that may run concurrently (different streams,
 * or graphs replayed on different streams) need different workspaces.
 *
 * Launch shape depends only on the shape, W, num_splits and the device, never
 * on kv_lens or idx contents, so one captured launch stays valid while the
 * lengths and index lists change between replays.
 *
 * Errors: a negative status is returned synchronously and nothing is
 * launched.  CK_ERR_HIP reports a failure of the HIP launch itself.  Faults
 * inside a kernel surface at the caller's next synchronization.
 */
#ifndef CK_DECODE_ATTN_H
#define CK_DECODE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ck_decode_shape {
    int32_t B;    /* sequences                                   >= 1        */
    int32_t n_q;  /* queries per sequence (causal window rows)   1..6        */
    int32_t Hq;   /* query heads                                 multiple of Hkv */
    int32_t Hkv;  /* KV heads                                    >= 1        */
    int32_t D;    /* head dim                                    128 or 256  */
    int32_t cap;  /* cache capacity (slots per sequence)         >= 1        */
} ck_decode_shape;

enum {
    CK_DT_F32 = 0,
    CK_DT_BF16 = 1
};

enum {
    CK_OK = 0,
    CK_ERR_ARG = -1,          /* null pointer, bad count or enum, bad stride */
    CK_ERR_UNSUPPORTED = -2,  /* D not 128/256, n_q > 6, cache too large     */
    CK_ERR_ALIGN = -3,        /* pointer misaligned (see each argument)      */
    CK_ERR_WORKSPACE = -4,    /* workspace missing or too small              */
    CK_ERR_HIP = -5,          /* the HIP runtime rejected the query/launch   */
    CK_ERR_SCRATCH = -6       /* ck_decode_attn_noalloc: the shape needs more
                                 than its fixed scratch holds                 */
};

#define CK_MAX_NQ 6
#define CK_MAX_SPLITS 256

/* Launch plan, exposed so that callers and tests can see how a shape is cut.
 * units = independent (sequence, [query,] KV head, row group) work items;
 * splits = workgroups per unit along the KV range (grid = splits x units,
 * padded to whole chunks of 8 x row_groups workgroups when several 16-row
 * groups share the tiles of one head; padding workgroups exit at once);
 * rows = packed query rows per (sequence, [query,] KV head): n_q*G dense,
 * G gather.  The device cuts each unit's range from its length.  With an
 * automatic split count, a unit whose range holds at most 128 KiB of K+V
 * (4 * D bytes per position) is streamed by one split, which writes the
 * output itself (no split merge).  Plain bf16 decode (no keep_mask, no INT8
 * cache, automatic split count) with one row
 * group per head, whose units alone leave most compute units idle
 * (2 * units * split_target > CUs), aims at three quarters of split_target
 * (fewer, longer splits publish fewer partials), and at no more than 32
 * splits for 8 or more packed rows at head_dim 256 over a range of at most
 * 6144 positions (with the INT8 cache, which otherwise aims at split_target,
 * from 12 rows); the grid, and so the workspace, is that of the plan either
 * way. */
typedef struct ck_decode_plan {
    int32_t units;
    int32_t splits;          /* grid splits per unit                         */
    int32_t split_target;    /* splits aimed for when the range is long      */
    int32_t chunk_min;       /* shortest range one split takes               */
    int32_t chunk_max;       /* longest range one split takes (0: no limit)  */
    int32_t granule;         /* split ranges are multiples of this           */
    int32_t rows;            /* query rows per unit                          */
    int32_t row_groups;      /* units per (sequence, query, KV head)         */
    int32_t rows_per_group;  /* rows handled by one workgroup: 16, or 32 for
                                17-32 rows when two 16-row groups would get
                                fewer than 16 splits each                    */
    int32_t slices;          /* column slices the split merge is cut into at
                                most; a merge of at most 32 KiB of partials
                                is one slice                                 */
    int32_t tile;            /* cache positions (or list entries) per wave
                                tile: a masked scan reads whole tiles that
                                hold a kept cell and skips the others        */
    size_t workspace_bytes;  /* 0 when no launch of this plan can split      */
} ck_decode_plan;

/* Plan for `shape` on a device with `num_cus` compute units.  W = 0 plans the
 * dense entry, W >= 1 the gather entry.  num_splits = 0 picks the split count
 * automatically, otherwise it is used as given (1..CK_MAX_SPLITS).  Pure host
 * arithmetic: no HIP call.  Returns CK_OK or an argument error. */
int ck_decode_attn_plan(const ck_decode_shape* shape, int32_t W, int num_splits, int num_cus,
                        ck_decode_plan* plan);

/* Workspace bytes needed by ck_decode_attn (W = 0) or ck_decode_attn_gather
 * (W >= 1) for `shape` and `num_splits` on the current HIP device.
 * 0 means no workspace is needed (NULL may be passed). */
int ck_decode_attn_workspace_size(const ck_decode_shape* shape, int32_t W, int num_splits,
                                  size_t* bytes);

/* Dense decode over the filled prefix (see the definition above).
 *   q, k_cache, v_cache, out : 16-byte aligned.  kv_lens, lse : 4-byte aligned.
 *   scale      : softmax scale (finite), typically 1/sqrt(D).
 *   causal     : nonzero for the bottom-right aligned causal window.
 *   keep_mask  : NULL, or uint8 [B, n_q, Hkv, cap]; cells with 0 are excluded
 *                (the masked full-window scan the gather entry replaces:
 *                llama.cpp PR "qwen4exp: attend the selected cells instead of
 *                masking the window", PR body).  Only [0, lim) is scanned.
 *   out_dtype  : CK_DT_F32 or CK_DT_BF16.
 *   num_splits : 0 = automatic, else 1..CK_MAX_SPLITS. */
int ck_decode_attn(const ck_decode_shape* shape, const void* q, const void* k_cache,
                   const void* v_cache, const int32_t* kv_lens, float scale, int causal,
                   const uint8_t* keep_mask, void* out, int out_dtype, float* lse,
                   void* workspace, size_t workspace_bytes, int num_splits, void* stream);

/* For callers that cannot allocate (code under graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): ck_decode_attn without a
 * workspace argument.  The split merge uses a 32 MiB array the library holds
 * in each device's memory until the process ends: a 256-byte status header,
 * the counters of up to 1024 units at fixed places, then up to about 30 MiB
 * of partial results.  A shape whose plan needs more (more than 1024 units,
 * or more partials) returns CK_ERR_SCRATCH and launches nothing.  Every call
 * leaves the counters ready for the next call of any shape, so no memset is
 * ever needed; the array is shared by every call on the device, so calls
 * that may overlap on one device (different streams) race and must not be
 * issued.  The call allocates nothing and frees nothing; its first call on a
 * device looks the array's address up once.  Arguments, result and errors
 * as ck_decode_attn. */
int ck_decode_attn_noalloc(const ck_decode_shape* shape, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* kv_lens, float scale, int causal,
                           const uint8_t* keep_mask, void* out, int out_dtype, float* lse,
                           int num_splits, void* stream);

/* Gathered decode: each query attends a list of W selected cells read in
 * place from the cache, instead of masking the whole window (llama.cpp PR
 * "qwen4exp: attend the selected cells instead of masking the window", PR
 * body and Additional information; llama.cpp PR "qwen4exp : gather-based
 * sparse attention for QSA decode", Overview; per-token lists for MTP
 * verification in that PR's discussion).  The selected K/V rows move once,
 * straight from the cache: there is no compacted copy.
 *   idx             : int32, 4-byte aligned.  idx_head_stride == 0: one list
 *                     per query shared by its heads, layout [B, n_q, W];
 *                     idx_head_stride >= W: layout [B, n_q, Hkv,
 *                     idx_head_stride] with the list in the first W entries.
 *   W               : list length >= 1.
 * Entries < 0 or >= lim are skipped; other arguments as ck_decode_attn. */
int ck_decode_attn_gather(const ck_decode_shape* shape, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* kv_lens, const int32_t* idx,
                          int32_t W, int64_t idx_head_stride, float scale, int causal, void* out,
                          int out_dtype, float* lse, void* workspace, size_t workspace_bytes,
                          int num_splits, void* stream);

/* Gather or scan for a top-k selection: which of ck_decode_attn_gather
 * (over the index lists) and ck_decode_attn with keep_mask (a scan of the
 * window with the same cells kept) is faster for this shape on MI355X.
 * The pages gate their gather by the cache depth: the scan reads the window
 * once for all queries while their gather moves the selected cells twice,
 * so they meet at n_kv = 2 * n_tps * width (llama.cpp PR "qwen4exp: attend
 * the selected cells instead of masking the window", PR body; per-token
 * lists in the discussion of llama.cpp PR "qwen4exp : gather-based sparse
 * attention for QSA decode"), and that PR's author gates at 4 x the top-k
 * width.  The gather here moves each selected cell once, straight from the
 * cache, and has the lower fixed cost, so it is faster unless the lists
 * cover most of a long window.  The choice compares two time models fitted
 * to MI355X measurements of both entry points, with a cell = B*Hkv*4*D
 * bytes (K and V of every KV head at one position):
 *   gather: 8.4 us + 0.141 us per MB of the n_q * W listed cells
 *   scan:   10.2 us + 0.30 us * (n_q - 1)
 *           + (0.131 + 0.0167 * (n_q - 1)) us per MB of the n_kv window cells
 * and returns the smaller (the scan term assumes every tile holds a kept
 * cell; clustered selections only make the scan cheaper).
 *   shape : as for the entry points (W >= 1 selects the gather plan checks)
 *   W     : list length per query
 *   n_kv  : host-side bound of the lengths the scan would cover (the largest
 *           length, or cap); >= 0
 *   path  : receives CK_PATH_GATHER or CK_PATH_SCAN
 * Pure host arithmetic: no HIP call, nothing read from device memory, so the
 * choice is fixed for a captured graph.  Returns CK_OK or an argument error. */
#define CK_PATH_GATHER 0
#define CK_PATH_SCAN 1
int ck_decode_sparse_path(const ck_decode_shape* shape, int32_t W, int64_t n_kv, int32_t* path);

/* Top-k selection: the index lists the gather reads, from one score per
 * cache cell (llama.cpp PR "qwen4exp : gather-based sparse attention for QSA
 * decode", discussion: the selection runs over the whole score row every
 * decode step, so it is the cost that still grows with the context once the
 * attention is gathered; radix/partial top-k paths serve it on other
 * backends).  For each row (sequence b, query i, score head h):
 *   L, lim   as in the definition above (causal: the window's query limit)
 *   tail     the last `tail` cells of the window, [max(0, lim - tail), lim),
 *            are always kept (the pages' selection always keeps the current
 *            tail)
 *   selected the min(k, n) highest-scoring of the n = max(0, lim - tail)
 *            cells before the tail; equal scores are taken lowest cell first,
 *            NaN ranks with -inf and -0 with +0, so the set is unique
 *   idx row  the selected cells and then the tail cells, ascending, padded
 *            with -1 to W = k + tail entries
 * Scores at or past the window limit are never read.
 *   shape     : B, n_q (<= CK_MAX_NQ), Hkv and cap are used; Hq and D are not
 *   scores    : fp32 [B, n_q, Hs, cap], 4-byte aligned (16-byte aligned rows
 *               read 4 scores per load)
 *   Hs        : score heads: Hkv (a list per KV head) or 1 (one list per
 *               query, shared by its heads: pass idx_head_stride 0 to the gather)
 *   kv_lens   : int32 [B], device memory
 *   k, tail   : k >= 1, tail >= 0
 *   idx       : int32 [B, n_q, Hs, k + tail], device memory, written whole
 *   workspace : as for the attention entries: ck_decode_topk_workspace_size
 *               bytes (0 when one workgroup serves a row), 256-byte aligned,
 *               zeroed once.  Each row holds a parity word and two sets of
 *               barrier counters and level histograms: a launch uses the
 *               set the parity names (zero when it starts), clears the
 *               other and flips the parity, so the buffer serves any number
 *               of launches of the same plan, eager or replayed from a
 *               graph, without a memset; its 256-byte header holds the
 *               status word (ck_workspace_status).
 * Errors as for the attention entries; nothing is launched on error.
 * CK_ERR_UNSUPPORTED also when cap * 4 bytes reaches 2 GiB, or when the
 * rows' workgroups would need 2 GiB of (key, position) slots for one row
 * (about 2^28 positions). */
int ck_decode_topk(const ck_decode_shape* shape, const float* scores, int32_t Hs, const int32_t* kv_lens,
                   int32_t k, int32_t tail, int causal, int32_t* idx, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Workgroups per row and workspace bytes of ck_decode_topk for `shape` on a
 * device with num_cus compute units (pure host arithmetic).  A row's
 * workgroups meet at barriers, so rows x workgroups never exceeds num_cus
 * (one workgroup per row when the rows alone reach it). */
int ck_decode_topk_plan(const ck_decode_shape* shape, int32_t Hs, int32_t k, int32_t tail, int num_cus,
                        int32_t* wgs_per_row, size_t* workspace_bytes);

/* Workspace bytes of ck_decode_topk for `shape` on the current device. */
int ck_decode_topk_workspace_size(const ck_decode_shape* shape, int32_t Hs, int32_t k, int32_t tail,
                                  size_t* bytes);

/* Step rows merged into prefix attention: the n_q verification queries of
 * an MTP step attend the cache prefix [0, L) plus their own draft rows,
 * whose K/V are passed separately instead of being written into the cache
 * first (comfy-kitchen PR "Performance improvements for qwen 3.x LLM
 * (Part 1)", commit list: causal step rows merged into prefix attention).
 * Query i sees every cache cell j < L and step rows 0..i, so the result
 * equals ck_decode_attn with causal = 1 over a cache holding the step rows
 * at [L, L + n_q).  The unit's last split streams the step rows as one more
 * tile and the in-launch combine merges it with the prefix.
 *   k_step, v_step : bf16 [B, n_q, Hkv, D], 16-byte aligned, non-null.
 * Other arguments as ck_decode_attn (no keep_mask; the window is implied);
 * the workspace is the dense one (ck_decode_attn_workspace_size, W = 0). */
int ck_decode_attn_steps(const ck_decode_shape* shape, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* kv_lens, const void* k_step,
                         const void* v_step, float scale, void* out, int out_dtype, float* lse,
                         void* workspace, size_t workspace_bytes, int num_splits, void* stream);

/* Paged INT8 KV cache (comfy-kitchen PR "Performance improvements for qwen
 * 3.x LLM (Part 1)", commit list: bounded paged INT8 decode cache with
 * rollback; 8-bit KV caches are what the pages run, llama.cpp PR "qwen4exp:
 * attend the selected cells instead of masking the window", Additional
 * information).  Each (token, KV head) row of K and of V is D int8 codes with
 * one fp32 scale: scale = amax / 127 and code = x * (127 / amax) rounded half
 * to even and clamped to [-127, 127], in fp32 (an all-zero row has scale 0);
 * the row's value is code * scale.  Token j of sequence b lives in page
 * block_table[b * max_pages + j / page_tokens], row j % page_tokens of its
 * KV head's block: a page is [Hkv][page_tokens][D], so a head's rows in a
 * page are one contiguous run (the pages leave the layout open).  Pages
 * are owned by the caller: several sequences may share a page pool, and
 * rolling a sequence back (rejected MTP drafts) is lowering its kv_lens
 * entry, after which the next append overwrites from there.
 *   k_codes, v_codes   : int8 [num_pages, Hkv, page_tokens, D], 16-byte aligned
 *   k_scales, v_scales : fp32 [num_pages, Hkv, page_tokens], 4-byte aligned
 *   block_table        : int32 [B, max_pages], device memory; an id outside
 *                        [0, num_pages) is never dereferenced: the tokens it
 *                        would hold read as zeros, appends to it are dropped
 *   page_tokens        : a multiple of 64; shape->cap must equal
 *                        page_tokens * max_pages (the logical capacity). */
typedef struct ck_q8_cache {
    void* k_codes;
    void* v_codes;
    float* k_scales;
    float* v_scales;
    const int32_t* block_table;
    int32_t page_tokens;
    int32_t max_pages;
    int32_t num_pages;
} ck_q8_cache;

/* Dense decode (optionally the causal window) over the paged INT8 cache.
 * Arguments as ck_decode_attn, with the cache in place of k_cache/v_cache
 * (and no keep_mask); the workspace is the dense one (W = 0).  The tiles are
 * dequantized exactly to bf16 codes, the K scale multiplies each score and
 * the V scale each probability. */
int ck_decode_attn_q8(const ck_decode_shape* shape, const void* q, const ck_q8_cache* cache,
                      const int32_t* kv_lens, float scale, int causal, void* out, int out_dtype,
                      float* lse, void* workspace, size_t workspace_bytes, int num_splits,
                      void* stream);

/* Quantize and append shape->n_q new tokens per sequence: k_new, v_new bf16
 * [B, n_q, Hkv, D] (2-byte aligned) go to positions start[b] + t, with start
 * (int32 [B], device memory, usually kv_lens) clamped to [0, cap]; rows past
 * the capacity or in a page outside the pool are dropped.  shape->Hq is not
 * used.  The caller advances kv_lens afterwards.  No workspace. */
int ck_kv_append_q8(const ck_decode_shape* shape, const void* k_new, const void* v_new,
                    const int32_t* start, const ck_q8_cache* cache, void* stream);

/* Workspace status.  Every workspace (of the attention entries and of
 * ck_decode_topk) opens with 256 bytes whose first int32 is a status word of
 * sticky bits, zero after the caller zeroes the buffer.  A launch waits on
 * other workgroups of the same launch in two places: a split-merge helper
 * waits for the unit's last split to arrive (only once every split of the
 * unit has started), and a top-k row waits at barriers for the row's other
 * workgroups (all resident by construction).  Every such wait is bounded.  One that gives up sets a bit:
 *   CK_WS_ERR_MERGE : a split merge gave up; its column slice of out (and
 *                     the lse of its rows) holds NaN
 *   CK_WS_ERR_TOPK  : a top-k row barrier gave up; that launch's lists are
 *                     not valid
 * and the kernel still ends normally, leaving the counters ready for the
 * next launch.  Neither can happen while the launch's workgroups all make
 * progress; it would take the GPU being held by other work for seconds.  The
 * bits stay set until the caller zeroes the header (or the whole buffer):
 * a nonzero status means that some launch since then returned invalid
 * results.
 * ck_workspace_status copies the word to *status; it waits for the work
 * queued on `stream` before it (it synchronizes that stream), so it is not
 * for use inside a captured graph.  workspace: 256-byte aligned. */
#define CK_WS_ERR_MERGE 1
#define CK_WS_ERR_TOPK 2
int ck_workspace_status(const void* workspace, void* stream, int32_t* status);

/* Polls a bounded wait makes before it gives up (process-wide, read at each
 * launch; 0 restores the default of 2^22, about seconds).  Failure handling
 * can be exercised by lowering it: every kernel still ends normally and the
 * workspace status reports the give-up.  polls >= 0. */
int ck_set_spin_limit(int32_t polls);

/* Contraction used by the dense and gathered entries for plans of at most
 * 8 packed query rows (n_q * G rows dense, G rows gathered), process-wide
 * and read at each launch:
 *   CK_CONTRACT_MFMA (the default): QK^T and PV as bf16 MFMA tiles (16 rows,
 *     12 or 8 of which are padding at 4 or 8 rows), the probabilities rounded
 *     to bf16 for PV;
 *   CK_CONTRACT_VALU: both on the vector ALUs with v_dot2 over bf16 pairs,
 *     one row per 64 / 4 or 64 / 8 lanes, the probabilities rounded the same
 *     way;
 *   CK_CONTRACT_VALU_F32: the same lanes in plain fp32 (every K and V element
 *     widened, one FMA per element and token), the probabilities kept in fp32.
 * All read the same bytes and agree with the exact result within the stated
 * tolerances.  The VALU forms exist to measure the choice: packing the GQA
 * group's query heads as rows makes every KV tile read from HBM serve all of
 * them (comfy-kitchen PR "Performance improvements for qwen 3.x LLM
 * (Part 1)", GQA decode), which leaves 4 or 8 rows per tile, and the
 * question is whether the padded MFMA or an unpadded VALU contraction keeps
 * up with the loads; keep_mask,
 * step rows, the INT8 cache and more than 8 rows always take MFMA.
 * Returns CK_ERR_ARG for any other value. */
#define CK_CONTRACT_MFMA 0
#define CK_CONTRACT_VALU 1
#define CK_CONTRACT_VALU_F32 2
int ck_set_contraction(int32_t contraction);

/* Phase timestamps of plain dense decode, for diagnosing where a launch
 * spends its time, in particular the part of a decode step's cost that does
 * not follow the filled length (ComfyUI issue "Qwen3.5 text generation
 * attends over the full KV capacity every step, so decode speed drops with
 * max_length", Measurements) (process-wide, read at each launch).  While a buffer is
 * set, ck_decode_attn and ck_decode_attn_steps launches whose plan has one
 * 16-row group per KV head (at most 16 packed rows, no keep_mask) run a
 * stamping instance of their kernel, a little slower than the plain one;
 * other launches are unaffected and write nothing.  stamps: device buffer of
 * workgroups * 16 uint64 words, 8-byte aligned, owned by the caller, or NULL
 * (with workgroups = 0) to turn stamping off.  Thread 0 of workgroup w
 * (w < workgroups) writes the device's 100 MHz real-time counter to word
 * 16 w + k at phase k: 0 start, 1 sequence length known, 2 first KV tile in
 * registers (first wave), 3 tile loop done (first wave), 4 all waves done,
 * 5 its partial result (or, with one split, the output) stored and
 * complete, 6 arrival counted, 7 split merge begins, 8 merge ends.  Word 13
 * holds the number of column slices it merged, word 14 the arrival rank,
 * word 15 split | unit << 16 | active splits << 32 | role << 48 (1 last
 * arrival, 2 helper that merged a slice, 3 neither).  A launch writes only
 * the words of phases its workgroups reach; the grid is units * splits of
 * ck_decode_attn_plan.  The buffer must stay allocated while it is set, and
 * as long as graphs captured meanwhile are replayed (their launches keep
 * its address).  CK_ERR_ARG when exactly one of stamps and workgroups is
 * zero or workgroups < 0, CK_ERR_ALIGN for a misaligned buffer. */
int ck_set_phase_stamps(void* stamps, int64_t workgroups);

/* Static text for a status code. */
const char* ck_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* CK_DECODE_ATTN_H */
