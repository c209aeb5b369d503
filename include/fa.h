/*
 * fa.h - C ABI of libfa.so: masked scaled-dot-product attention forward on MI355X (gfx950).
 *
 *   O = softmax(scale * Q K^T + bias, masked) V,   plus the fp32 log-sum-exp of each row.
 *
 * The operation and its mask family follow the pages this library is built from:
 * - "sparseMode介绍" (CANN aolapi common parameter page): attenMask True = masked, and
 *   sparseMode 0..8 (sections sparseMode=0 .. sparseMode=8), including the varlen split
 *   modes 7/8 with their cumulative actual_seq_qlen / actual_seq_kvlen arrays.
 * - "压缩mask" (CANN ATB compressed-mask page), alibi scenario: per-head slope times a
 *   right-aligned relative-position bias; masks aligned from kvSeqLen and qSeqLen.
 * - "Ý Tưởng Tiling & Online Softmax Trong FlashAttention" (exercise page), knowledge goals:
 *   block tiling with a running row maximum and running sum, never forming the Sq x Skv
 *   matrix.
 * - "aclnnScatterPaKvCache" (ops-transformer doc), sections "函数原型" and the return-code
 *   table: the two-phase call (workspace size first, then execute on a stream) and
 *   validation with status codes before any device work. The codes below are this
 *   library's own.
 *
 * Conventions shared by every entry point:
 * - Device buffers (q, k, v, out, softmax_lse, alibi_slopes, atten_mask, workspace and the
 *   probe outputs) are allocated and owned by the caller and must be contiguous in the
 *   stated layout. The library never allocates device memory.
 * - actual_seq_qlen, actual_seq_kvlen and prefix are HOST int64 arrays, read during the call
 *   only.
 * - Every argument is validated on the host before anything is enqueued. On any error the
 *   call returns a non-zero status and writes nothing.
 * - Compute calls are asynchronous on `stream` (a hipStream_t, 0 = the null stream); the
 *   caller synchronises. Results are bitwise deterministic for identical inputs (no
 *   atomics), as the ops-transformer doc asks of its ops ("确定性计算").
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fa_status;
#define FA_OK 0
#define FA_ERR_NULLPTR 1        /* a required pointer is NULL                                */
#define FA_ERR_PARAM_INVALID 2  /* a value breaks a rule of the pages or of this ABI         */
#define FA_ERR_UNSUPPORTED 3    /* valid per the pages but not built (e.g. D > 128)          */
#define FA_ERR_HIP 4            /* the HIP runtime reported an error (launch, copy, device)  */
#define FA_ERR_WORKSPACE 5      /* workspace smaller than fa_fwd_workspace_size asked for    */

/* Tensor layouts. BNSD: [B, N, S, D]. BSND: [B, S, N, D]. TND: [T, N, D], the B sequences
 * packed back to back; sequence b occupies tokens [cum[b-1], cum[b]) of the cumulative
 * arrays (cum[-1] = 0). */
#define FA_LAYOUT_BNSD 0
#define FA_LAYOUT_BSND 1
#define FA_LAYOUT_TND 2

/* Alibi bias variants ("压缩mask", section "不同压缩mask的构造方法", alibi scenario). With
 * d = i - j + (Skv_b - Sq_b), the distance of key j from query i's bottom-right diagonal:
 *   FA_ALIBI_RIGHT: bias_ij = slope_h * (j - i - (Skv_b - Sq_b)) = -slope_h * d (right-aligned);
 *   FA_ALIBI_SQRT:  bias_ij = -slope_h * sign(d) * sqrt(|d|) (the right-aligned bias with its
 *                   magnitude square-rooted);
 *   FA_ALIBI_LEFT:  bias_ij = slope_h * (j - i) (left-aligned: zero on the top-left diagonal).
 * The page's figures with the exact values did not survive; these are the plain readings. */
#define FA_ALIBI_RIGHT 0
#define FA_ALIBI_SQRT 1
#define FA_ALIBI_LEFT 2

/* Element types of q, k, v and out (all four share one). softmax_lse is always fp32. */
#define FA_DTYPE_F32 0
#define FA_DTYPE_F16 1
#define FA_DTYPE_BF16 2

/* Problem sizes. B batches, N heads (q, k and v have the same N), head size D.
 * BNSD/BSND: every batch has Sq queries and Skv keys; T_q / T_kv are ignored.
 * TND: Sq / Skv are ignored; T_q / T_kv are the total token counts and must equal the last
 * entries of actual_seq_qlen / actual_seq_kvlen. */
typedef struct fa_dims {
    int32_t dtype;
    int64_t B, N, Sq, Skv, D;
    int64_t T_q, T_kv;
} fa_dims;

/* Mask arguments, shared by fa_fwd and fa_mask_probe.
 *
 * sparse_mode ("sparseMode介绍"):
 *   0 defaultMask: row i sees columns j with -pre_tokens <= j - i <= next_tokens (offsets from
 *     the top-left). pre/next >= max(Sq, Skv) (e.g. INT64_MAX) is "no mask". Negative
 *     next_tokens needs pre_tokens >= |next_tokens| and |next_tokens| < Skv; negative
 *     pre_tokens needs next_tokens >= |pre_tokens| and |pre_tokens| < Sq.
 *   1 allMask: atten_mask (uint8, non-zero = masked) gives every entry; pre/next ignored.
 *     Shape [B or 1, N or 1, Sq, Skv]: mask_bcast[0] / mask_bcast[1] non-zero means the batch
 *     / head dimension has size 1 and is shared. BNSD/BSND only.
 *   2 leftUpCausal: j <= i.
 *   3 rightDownCausal: j <= i + (Skv_b - Sq_b).
 *   4 band from the bottom-right: -pre <= j - i - (Skv_b - Sq_b) <= next, pre + next >= 0.
 *   5, 6 prefix: rightDownCausal, plus columns j < prefix[b] for every row.
 *   7 (TND only): the last batch with Sq_b > 0 and Skv_b > 0 uses rule 4, with
 *     pre >= Skv_b and Sq_b - Skv_b <= next <= 0; every other batch uses rule 3 and needs
 *     Sq_b <= Skv_b. No alibi.
 *   8 (TND only): the first such batch uses rule 4 with pre >= Skv_b and
 *     next >= Sq_b - Skv_b; every other batch uses rule 2. No alibi.
 * pre_tokens / next_tokens are ignored (and not checked) in modes 1, 2, 3, 5 and 6.
 * Rows with no visible column produce O = 0 and LSE = -inf. */

/* Phase 1: validate the sizes and return the workspace size fa_fwd needs (in bytes; 0 means
 * no workspace). Host only; never touches the GPU.
 * What the workspace holds: the per-batch geometry and work list in TND and prefix modes
 * (modes 5, 6), the split-KV partial results of short-query problems, and in mode 1 (on the
 * MFMA kernels) the tile map a pre-pass builds from atten_mask: per (q tile, kv tile) its
 * class, per q tile the list of kv tiles with a visible entry (the kernel loads no other), and
 * the mask bits packed in the order the kernel reads them, about an eighth of the mask's own
 * size. For mode 1 this query assumes an unbroadcast mask, the largest case; see
 * fa_fwd_mask_workspace_size. */
fa_status fa_fwd_workspace_size(const fa_dims* dims, int32_t layout, int32_t sparse_mode,
                                const int64_t* actual_seq_qlen, const int64_t* actual_seq_kvlen,
                                size_t* bytes);

/* The workspace size of a mode-1 (atten_mask) call whose mask broadcast is known: mask_bcast
 * as for fa_fwd (NULL = unbroadcast). A mask shared over batches and heads ([1, 1, Sq, Skv])
 * needs 1 / (B N) of what fa_fwd_workspace_size returns for mode 1. fa_fwd accepts any
 * workspace at least this large. Host only. */
fa_status fa_fwd_mask_workspace_size(const fa_dims* dims, int32_t layout, const int64_t* mask_bcast,
                                     size_t* bytes);

/* Phase 2: the forward pass.
 *   q, k, v, out:  device, dims->dtype, in `layout`.
 *   softmax_lse:   device fp32, [B, N, Sq] (BNSD/BSND) or [N, T_q] (TND); natural log of the
 *                  sum over visible j of exp(scale * q_i.k_j + bias_ij).
 *   alibi_slopes:  device fp32 [N] or NULL. When given, the bias of head h is slope_h times
 *                  the relative-position term alibi_mode selects; D <= 128; not with modes 7/8.
 *   alibi_mode:    FA_ALIBI_RIGHT, FA_ALIBI_SQRT or FA_ALIBI_LEFT (else FA_ERR_PARAM_INVALID);
 *                  checked even when alibi_slopes is NULL.
 *   scale:         softmax scale, finite and > 0 (e.g. 1/sqrt(D)).
 *   workspace:     device, at least fa_fwd_workspace_size bytes (may be NULL when that is 0).
 * Supported: D <= 128 for every dtype; the MFMA kernels serve fp16/bf16 with D = 64 or 128,
 * a generic kernel everything else. */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* out, float* softmax_lse,
                 const fa_dims* dims, int32_t layout, int32_t sparse_mode,
                 int64_t pre_tokens, int64_t next_tokens,
                 const int64_t* actual_seq_qlen, const int64_t* actual_seq_kvlen,
                 const int64_t* prefix, const float* alibi_slopes, int32_t alibi_mode,
                 const uint8_t* atten_mask, const int64_t* mask_bcast,
                 float scale, void* workspace, size_t workspace_bytes, void* stream);

/* fa_fwd for callers that cannot allocate device memory: code under HIP graph capture,
 * serving loops and harnesses that forbid hipMalloc. The arguments, validation, status codes
 * and results are fa_fwd's (bitwise: the same kernels run), without the workspace pair: the
 * workspace fa_fwd_workspace_size would ask for lives in a device array of this library, one
 * copy per GPU, FA_NOALLOC_SCRATCH_BYTES long and held until the process ends.
 * - A problem that needs more than FA_NOALLOC_SCRATCH_BYTES of workspace returns
 *   FA_ERR_WORKSPACE before any device work (use fa_fwd with a workspace of its own).
 * - stream must belong to the current device (else FA_ERR_PARAM_INVALID), whose copy of the
 *   array is used.
 * - The call allocates nothing (no hipMalloc, no hipFree). Every call on one GPU shares that
 *   GPU's array, and the array keeps the last call's contents: calls that overlap on one GPU
 *   (on different streams, or from several threads without ordering) race and may corrupt
 *   each other's results. Nothing in it needs to start at zero: each call writes what it
 *   reads. */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)

fa_status fa_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* softmax_lse,
                         const fa_dims* dims, int32_t layout, int32_t sparse_mode,
                         int64_t pre_tokens, int64_t next_tokens,
                         const int64_t* actual_seq_qlen, const int64_t* actual_seq_kvlen,
                         const int64_t* prefix, const float* alibi_slopes, int32_t alibi_mode,
                         const uint8_t* atten_mask, const int64_t* mask_bcast,
                         float scale, void* stream);

/* Backward pass: gradients of a loss with respect to q, k and v, given dout = dLoss/dO. No
 * page gives a backward pass; this is the derivative of the forward defined above. With P
 * recomputed from q, k, the bias and the mask, and the forward's softmax_lse:
 *   P_ij = exp(scale q_i.k_j + bias_ij - LSE_i) for visible (i, j), else 0;
 *   Delta_i = sum_d dout_id out_id;
 *   dV = P^T dout,  dP = dout V^T,  dS = P * (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q.
 *   q, k, v:          the forward's inputs; out, softmax_lse: what fa_fwd returned for them.
 *   dout:             device, dims->dtype, out's layout.
 *   dq, dk, dv:       device, dims->dtype, the layouts of q, k and v; every element is written
 *                     (zero where no visible pair contributes).
 *   workspace:        at least fa_bwd_workspace_size bytes (Delta and the LSE scaled to log2
 *                     units, each laid out like softmax_lse, and the per-batch geometry in
 *                     TND / prefix modes).
 * Every other argument, its validation and the status codes are fa_fwd's. Gradients accumulate
 * in fp32; with fp16 / bf16 inputs P and dS are rounded to that type for the products that
 * consume them. No atomics: results are bitwise deterministic. */
fa_status fa_bwd_workspace_size(const fa_dims* dims, int32_t layout, int32_t sparse_mode,
                                const int64_t* actual_seq_qlen, const int64_t* actual_seq_kvlen,
                                size_t* bytes);

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* out,
                 const float* softmax_lse, const void* dout, void* dq, void* dk, void* dv,
                 const fa_dims* dims, int32_t layout, int32_t sparse_mode,
                 int64_t pre_tokens, int64_t next_tokens,
                 const int64_t* actual_seq_qlen, const int64_t* actual_seq_kvlen,
                 const int64_t* prefix, const float* alibi_slopes, int32_t alibi_mode,
                 const uint8_t* atten_mask, const int64_t* mask_bcast,
                 float scale, void* workspace, size_t workspace_bytes, void* stream);

/* Mask probe: runs the same device mask code the forward kernels use, without any
 * attention arithmetic.
 *   row_visible_counts: device int64, laid out like softmax_lse ([B, N, Sq] or [N, T_q]):
 *                       the number of visible columns of each row.
 *   tile_class:         device uint8 or NULL, [n_qtiles_total, n_kvtiles_max] (see
 *                       fa_tile_shape): 0 = the forward kernel skips the tile (never loads
 *                       it), 1 = visited with per-element masking, 2 = visited without
 *                       masking (every in-range entry visible), 3 = outside the sequence.
 *                       Row r of the map is the q tile r of the batch-major enumeration
 *                       (batch 0's tiles first). In mode 1 the classes come from atten_mask
 *                       and differ per head: the map is [B * N * n_qtiles_per_batch,
 *                       n_kvtiles_max], rows ordered by batch, then head, then q tile; mode 1
 *                       has a map only where fa_fwd runs the pre-pass (fp16 / bf16 with
 *                       D = 64 or 128), else tile_class must be NULL (FA_ERR_UNSUPPORTED).
 * The workspace argument has fa_fwd's meaning and size. Asynchronous on `stream`. */
fa_status fa_mask_probe(const fa_dims* dims, int32_t layout, int32_t sparse_mode,
                        int64_t pre_tokens, int64_t next_tokens,
                        const int64_t* actual_seq_qlen, const int64_t* actual_seq_kvlen,
                        const int64_t* prefix, const uint8_t* atten_mask,
                        const int64_t* mask_bcast, int64_t* row_visible_counts,
                        uint8_t* tile_class, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Tile shape the forward kernel will use for these sizes: block_m query rows by block_n
 * keys, the number of q tiles (all batches) and the largest number of kv tiles of a batch.
 * Host only. */
fa_status fa_tile_shape(const fa_dims* dims, int32_t layout, const int64_t* actual_seq_qlen,
                        const int64_t* actual_seq_kvlen, int32_t* block_m, int32_t* block_n,
                        int64_t* n_qtiles_total, int64_t* n_kvtiles_max);

/* Host-side plan summary of one fa_fwd call (same validation as fa_fwd, no device work).
 * kernel: 0 = generic, 1 = ping-pong MFMA, 2 = four-wave MFMA, 3 = split-KV decode. Tile
 * counts are per head. */
typedef struct fa_plan_stats {
    int32_t kernel;
    int32_t block_m, block_n;
    int64_t work_items;        /* (batch, q tile) pairs per head; (batch, kv split) for 3 */
    int64_t kv_tiles_visited;  /* kv tiles loaded, summed over work items, per head     */
    int64_t kv_tiles_full;     /* of which need no per-element masking                  */
    int64_t kv_tiles_total;    /* kv tiles a dense pass would load, per head            */
    size_t workspace_bytes;
    int32_t launch_order;      /* prefill work-item order: 0 batch-major, 1 pair-major,
                                  2 rank-major, 3 rank-major in groups of four pairs (the
                                  last three XCD-major), 4 a work table (varlen / prefix);
                                  0 for the split-KV decode kernel */
    int32_t edge_skip;         /* 1: the ping-pong kernel's variant in which a wave skips the
                                  softmax of a kv tile none of its rows sees (chosen for bands
                                  with a lower bound and for items of at most 64 kv tiles) */
} fa_plan_stats;

fa_status fa_plan_stats_get(const fa_dims* dims, int32_t layout, int32_t sparse_mode,
                            int64_t pre_tokens, int64_t next_tokens,
                            const int64_t* actual_seq_qlen, const int64_t* actual_seq_kvlen,
                            const int64_t* prefix, int32_t has_alibi, int32_t has_mask,
                            float scale, fa_plan_stats* out);

/* A static, human-readable name for a status code. */
const char* fa_status_str(fa_status status);

/* ---------------------------------------------------------------------------------------
 * Paged KV cache ("aclnnScatterPaKvCache", sections "功能说明" and "约束说明").
 * --------------------------------------------------------------------------------------- */

/* Cache layouts. A slot is block * block_size + offset.
 *   FA_CACHE_NORM: [num_blocks, block_size, N, head_size] (the page's scenario two, "Norm");
 *   FA_CACHE_NHSD: [num_blocks, N, block_size, head_size] (scenario seven, "NHSD"). */
#define FA_CACHE_NORM 0
#define FA_CACHE_NHSD 1

typedef struct fa_kv_cache_dims {
    int64_t num_tokens;   /* tokens to write (key is [num_tokens, N, k_head_size])       */
    int64_t num_heads;    /* N                                                           */
    int64_t k_head_size;
    int64_t v_head_size;  /* ignored when value is NULL (keys only, scenario six)        */
    int64_t num_blocks;
    int64_t block_size;
    int32_t elem_bytes;   /* bytes per element of key / value / caches: 1, 2 or 4 (raw copy) */
    int32_t slot_bytes;   /* slot_mapping element: 4 (int32) or 8 (int64)                */
} fa_kv_cache_dims;

/* Scatter: for every token t and head h, key[t, h, :] goes to key_cache at slot
 * slot_mapping[t] (and value[t, h, :] to value_cache).
 *   key, value:             device, contiguous [num_tokens, N, head_size]; value may be NULL
 *                           (then value_cache must be NULL too).
 *   key_cache, value_cache: device, contiguous in cache_layout; updated in place.
 *   slot_mapping:           device int32 or int64 [num_tokens]. Slots must be distinct; a
 *                           slot outside [0, num_blocks * block_size - 1] (for example -1
 *                           for a padding token) writes nothing.
 * Errors: NULLPTR for a missing required pointer (when num_tokens > 0, or dims itself);
 * PARAM_INVALID for an unknown layout or element size or non-positive sizes; UNSUPPORTED for
 * sizes beyond 32-bit row offsets; HIP for a launch error. Asynchronous on `stream`; no
 * workspace, no allocation; deterministic. */
fa_status fa_scatter_kv_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                              const void* slot_mapping, const fa_kv_cache_dims* dims,
                              int32_t cache_layout, void* stream);

/* Where a sequence's keys live in a paged cache. Sequence b's key j (j counted from the
 * sequence's first key) is in page block_table[b * max_blocks_per_seq + j / block_size] at
 * offset j % block_size, i.e. in the slot that fa_scatter_kv_cache writes for
 * slot = page * block_size + j % block_size. The pages describe the cache and its slots; this
 * read-back rule is the plain reading of "slot = block * block_size + offset".
 *   block_table:        device int32 [B, max_blocks_per_seq]; entries past a sequence's last
 *                       page are not read. Every page a sequence uses must lie in
 *                       [0, num_blocks): an id outside it reads as zeros (no access outside
 *                       the cache), which gives a defined but meaningless result.
 *   max_blocks_per_seq: row length of block_table; max_blocks_per_seq * block_size must cover
 *                       the longest sequence.
 *   num_blocks, block_size, cache_layout: as for fa_scatter_kv_cache (FA_CACHE_NORM or
 *                       FA_CACHE_NHSD); head_size of the caches is dims->D. */
typedef struct fa_paged_kv {
    const int32_t* block_table;
    int64_t max_blocks_per_seq;
    int64_t num_blocks;
    int64_t block_size;
    int32_t cache_layout;
    int32_t reserved;      /* must be 0 */
} fa_paged_kv;

/* Workspace size of fa_fwd_paged for these sizes (host only, like fa_fwd_workspace_size; it
 * can differ from fa_fwd's because the kernel choice depends on the page size). */
fa_status fa_fwd_paged_workspace_size(const fa_dims* dims, int32_t layout, int32_t sparse_mode,
                                      const int64_t* actual_seq_qlen, const int64_t* actual_seq_kvlen,
                                      const fa_paged_kv* paged, size_t* bytes);

/* fa_fwd with K and V read from paged caches instead of contiguous tensors.
 *   q, out, softmax_lse: as for fa_fwd, in `layout`.
 *   key_cache, value_cache: device, dims->dtype, [num_blocks, block_size, N, D] (Norm) or
 *                        [num_blocks, N, block_size, D] (NHSD).
 *   dims:                as for fa_fwd; Skv (BNSD / BSND) or actual_seq_kvlen (TND) give the
 *                        key count of each sequence, T_kv must equal the last kvlen entry.
 *   workspace:           at least fa_fwd_paged_workspace_size bytes.
 * Every other argument, the status codes and the results are fa_fwd's: the output equals
 * fa_fwd's on the gathered K and V (bitwise when both calls run the same kernel). PARAM_INVALID for a bad fa_paged_kv (unknown layout, non-positive sizes,
 * reserved != 0, or a table too short for the longest sequence); NULLPTR when paged or a
 * cache or block_table is missing while some sequence has keys. */
fa_status fa_fwd_paged(const void* q, const void* key_cache, const void* value_cache, void* out,
                       float* softmax_lse, const fa_dims* dims, int32_t layout, int32_t sparse_mode,
                       int64_t pre_tokens, int64_t next_tokens,
                       const int64_t* actual_seq_qlen, const int64_t* actual_seq_kvlen,
                       const int64_t* prefix, const float* alibi_slopes, int32_t alibi_mode,
                       const uint8_t* atten_mask, const int64_t* mask_bcast,
                       const fa_paged_kv* paged, float scale, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Measurement helper: the chip's base-2 exponential throughput.
 * --------------------------------------------------------------------------------------- */

/* The online softmax of the tiling page's recurrence evaluates one exponential per computed
 * score, issued as the hardware exp2 instruction; its rate is the second roofline of the
 * forward beside the matrix cores. This call launches `blocks` workgroups of 256 threads that
 * issue nothing in their inner loop but that instruction, each thread iters * 128 times
 * across 8 independent chains x <- 2^(-x).
 *   out:             device float [blocks * 256]; thread t writes the sum of its 8 chains,
 *                    which converge to 8 times the root of x = 2^(-x) (about 5.1295).
 *   exps_per_launch: host, receives blocks * 256 * iters * 128.
 * Errors: NULLPTR for a missing pointer, PARAM_INVALID for blocks or iters outside
 * [1, 2^20], HIP for a launch error. Asynchronous on `stream`; time it with events there. */
fa_status fa_exp2_rate_probe(float* out, int32_t blocks, int32_t iters, int64_t* exps_per_launch,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
