/*
 * mla.h -- C ABI of libmla, a gfx950 (MI355X) sparse MLA attention decode
 * library for DeepSeek-V3.2-shaped attention: h_q query heads (64 or 128)
 * share one compressed KV head, d_qk = 576 (512 NoPE + 64 RoPE), d_v = 512;
 * and for the V4 / V4.1 caches, d_qk = d_v = 512.
 *
 * Operation (reference semantics: "FlashMLA 与 DSA：内核、流水线和正确性边界",
 * section 4.3; call shapes: "FlashMLA Sparse Decode 完整计算过程详解", steps 1,
 * 2.2, 2.3 and 19):
 *   for every query token (b, s) and head h, over the topk slots k with
 *   t = indices[b, s, k]:
 *     slot k is valid iff 0 <= t < num_kv_tokens  (-1 marks an empty slot);
 *     K_t = dequantised token row t (d_qk values), V_t = K_t[0:512];
 *     score_k = sm_scale * <q[b,s,h,:], K_t>        (-inf when invalid)
 *     lse[b,h,s] = ln sum_k exp(score_k)            (+inf when no slot is valid)
 *     out[b,s,h,:] = sum_k exp(score_k - lse) V_t   (0 when no slot is valid)
 *   A repeated token counts once per slot.
 *
 * KV formats:
 *   MLA_KV_FP8_656  paged cache [num_blocks, page_block_size, 1, 656] bytes; a
 *                   token row holds 512 e4m3fn NoPE codes, four little-endian
 *                   fp32 power-of-two scales (one per 128 NoPE dims) and 64
 *                   bf16 RoPE values ("FlashMLA Sparse Decode 完整计算过程详解",
 *                   steps 2.2 and 4.3).  Token t lives in page t / P at offset
 *                   t % P (step 7.2); NoPE dequant is code * scale (step 7.4).
 *                   The scales must be powers of two, as the walkthrough's
 *                   quantisation makes them (step 4.2): the GPU conversion
 *                   uses only a scale's exponent (sign and mantissa ignored).
 *   MLA_KV_BF16_576 flat cache [s_kv, 576] bf16 with logical indices (the
 *                   sparse-prefill contract of "FlashMLA 与 DSA", section 4.0).
 *   MLA_KV_V4_584,  paged struct-of-arrays caches with d_qk = 512 ("FlashMLA
 *   MLA_KV_V41_528  与 DSA" section 3.1: a page holds its data rows, then its
 *                   scale rows; e8m0 scales; 584 / 528 bytes per token;
 *                   walkthrough step 2.3: d_qk 512 selects these models).
 *                   Page n starts at kv + n * kv_stride_block; with P tokens
 *                   per page, token t = n P + o has its data row at page +
 *                   o * D and its scale row at page + P * D + o * S.
 *                   V4:   D = 576: 448 e4m3fn codes (dims 0..447), then 64
 *                         little-endian bf16 values (dims 448..511); S = 8:
 *                         7 e8m0 scales (dims 64 g .. 64 g + 63), 1 pad byte.
 *                   V4.1: D = 512 e4m3fn codes; S = 16 e8m0 scales (dims
 *                         32 g .. 32 g + 31).
 *                   An e8m0 byte e is 2^(e - 127) (0xFF: NaN); dequant is
 *                   code * scale; V = K.  The split of each token into codes,
 *                   bf16 values and scales is the one the byte counts allow
 *                   (the pages give only the counts and the group sizes).
 *
 * Work split (step 3 of the walkthrough): the topk list of every request is cut
 * into blocks of split_granularity slots; a greedy left-to-right plan assigns
 * (request, block range) pieces to num_parts partitions with a fixed per-request
 * cost of fixed_overhead blocks.  A request whose blocks land in more than one
 * partition is "split": each piece writes its normalised partial O/l and a
 * base-2 lse (step 14) into the workspace and mla_splitkv_combine merges them
 * (step 16).  A request that lands in exactly one partition is written to
 * out/lse directly.  Partial O precision: stored as bf16, packed in the
 * decode's register layout (narrower than the walkthrough's fp32 o_accum; a
 * partial is bounded by max |V| and its rounding stays inside the output
 * tolerance).  The workspace is sized for fp32 partials.
 *
 * Conventions:
 *   - Every pointer in mla_decode_args is device memory owned by the caller; the
 *     library allocates nothing, keeps no per-call state, and never frees.
 *   - Calls that take a stream are asynchronous on that stream (hipStream_t
 *     passed as void*, NULL = the default stream).  Kernel launch failures are
 *     reported as MLA_ERR_HIP.
 *   - Every argument is validated on the host before anything is launched; on
 *     error nothing is launched, the status is returned and mla_last_error()
 *     holds a message (thread-local).  The library never aborts the process.
 *   - Shape limits: b * ceil(topk / split_granularity) < 2^30, s_q <= 65535,
 *     b * s_q <= 2^24.
 *   - Calls that overlap on one stream-ordered pipeline must use distinct
 *     sched/workspace buffers if they run concurrently on different streams.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MLA_OK                0
#define MLA_ERR_INVALID_ARG  -1   /* a pointer, size, stride or shape is wrong     */
#define MLA_ERR_UNSUPPORTED  -2   /* a valid request this build does not support   */
#define MLA_ERR_WORKSPACE    -3   /* a sched or workspace buffer is too small      */
#define MLA_ERR_HIP          -4   /* the HIP runtime reported an error             */
#define MLA_ERR_NO_DEVICE    -5   /* a device property was needed and none exists  */

/* KV cache formats */
#define MLA_KV_FP8_656   0
#define MLA_KV_BF16_576  1
#define MLA_KV_V4_584    2
#define MLA_KV_V41_528   3

/* Problem shape.  All fields are plain host values. */
typedef struct mla_shape {
    int32_t b;                 /* requests (batch), >= 1                               */
    int32_t s_q;               /* query tokens per request, >= 1                       */
    int32_t h_q;               /* query heads: 64 or 128                                */
    int32_t h_kv;              /* KV heads: must be 1                                   */
    int32_t d_qk;              /* 576; 512 for MLA_KV_V4_584 and MLA_KV_V41_528         */
    int32_t d_v;               /* must be 512                                           */
    int32_t topk;              /* slots per query token, >= 1                           */
    int32_t page_block_size;   /* paged formats: tokens per page (>= 1); BF16: ignored
                                  (use 1)                                                */
    int64_t num_kv_tokens;     /* paged: num_blocks * page_block_size; BF16: s_kv; >= 1 */
    int32_t kv_format;         /* MLA_KV_FP8_656, MLA_KV_BF16_576, MLA_KV_V4_584 or
                                  MLA_KV_V41_528                                         */
    int32_t num_parts;         /* scheduler partitions (work-groups per query-token
                                  column); 0 = derive from the current device's CU count */
    int32_t split_granularity; /* topk slots per scheduler block, a multiple of 32;
                                  0 = 64 (the walkthrough's TOPK_BLOCK_SIZE)            */
    int32_t fixed_overhead;    /* per-request scheduler cost in blocks; < 0 = 5 (the
                                  walkthrough's fixed_overhead_num_blocks)              */
} mla_shape;

/* One scheduler partition (32 bytes, int32 fields).  end_req is inclusive,
 * end_block is exclusive and counts blocks of end_req; begin_split is the
 * global split index of the first piece; a partition with begin_req >= b is idle.
 * by_length is 1 in a plan made from valid lengths (mla_get_sched_meta_len):
 * a request that the partition covers whole then spans
 * ceil(topk_length[r] / split_granularity) blocks; 0 otherwise. */
typedef struct mla_sched_part {
    int32_t begin_req, end_req, begin_block, end_block;
    int32_t begin_split, first_splitted, last_splitted, by_length;
} mla_sched_part;

typedef struct mla_decode_args {
    mla_shape shape;
    float sm_scale;                     /* softmax scale; <= 0 means 1/sqrt(d_qk)         */

    const void* q;                      /* bf16 [b, s_q, h_q, d_qk], last dim contiguous   */
    int64_t q_stride_b, q_stride_s, q_stride_h;          /* in elements, multiples of 8   */

    const void* kv;                     /* FP8: [num_blocks, P, 1, 656] bytes (token stride
                                           656 B); BF16: [s_kv, kv_stride_block/2] bf16;
                                           V4 / V4.1: [num_blocks, kv_stride_block] bytes,
                                           pages as described above                        */
    int64_t kv_stride_block;            /* FP8: bytes per page (>= P*656); V4 / V4.1: bytes
                                           per page (>= P * 584 / 528, P * that < 2^31);
                                           BF16: bytes per token row (>= 1152); a multiple
                                           of 16                                           */

    const int32_t* indices;             /* [b, s_q, topk], last dim contiguous; FP8:
                                           physical token ids, BF16: row ids; -1 = empty   */
    int64_t idx_stride_b, idx_stride_s; /* in elements                                      */

    void* out;                          /* bf16 [b, s_q, h_q, 512], last dim contiguous    */
    int64_t out_stride_b, out_stride_s, out_stride_h;    /* in elements, multiples of 8   */
    float* lse;                         /* fp32 [b, h_q, s_q] contiguous, natural log      */

    const float* attn_sink;             /* NULL, or fp32 [h_q] device: one sink logit per
                                           head (natural log).  out is scaled by
                                           1 / (1 + exp(attn_sink - lse)); lse is that of
                                           the real slots ("FlashMLA 与 DSA" section 4.3,
                                           walkthrough step 13)                            */
    const int32_t* topk_length;         /* NULL, or int32 [b] device: slots at positions
                                           >= topk_length[b] are empty (clamped to
                                           [0, topk]).  A plan from mla_get_sched_meta or
                                           the closed form still covers topk slots; one
                                           from mla_get_sched_meta_len covers only the
                                           valid ones and must be used with the same
                                           lengths (its pieces follow them).  Such a plan
                                           passed with topk_length NULL is a contract
                                           error the host cannot see (the plan is device
                                           memory): the decode then writes nothing and the
                                           combine writes NaN to every out and lse element */

    const void* sched_meta;             /* from mla_get_sched_meta (same shape), or NULL   */
    const int32_t* num_splits;          /* [b + 1] split prefix from mla_get_sched_meta, or
                                           NULL.  Both NULL (only with fixed_overhead == 0):
                                           the kernels evaluate the same greedy plan in closed
                                           form (partition q takes blocks [q p, (q + 1) p) of
                                           the request-major block sequence, p = ceil(b
                                           ceil(topk / split_granularity) / num_parts)), so no
                                           scheduler launch is needed.  One NULL and one set
                                           is MLA_ERR_INVALID_ARG.                           */

    float* o_accum;                     /* workspace, >= mla_workspace_size bytes          */
    float* lse_accum;                   /* workspace, >= mla_workspace_size bytes          */
    size_t o_accum_bytes, lse_accum_bytes;               /* capacities of the two above   */
} mla_decode_args;

/* Sizes of the scheduler outputs for `shape`: meta = num_parts * 32 bytes,
 * num_splits = (b + 1) * 4 bytes.  Needs a device only when num_parts == 0. */
int mla_sched_meta_size(const mla_shape* shape, size_t* meta_bytes, size_t* num_splits_bytes);

/* Split workspace sizes: (b + num_parts) * s_q * h_q * 512 * 4 bytes for
 * o_accum and (b + num_parts) * s_q * h_q * 4 bytes for lse_accum. */
int mla_workspace_size(const mla_shape* shape, size_t* o_accum_bytes, size_t* lse_accum_bytes);

/* Resolve the defaults of `shape` (num_parts, split_granularity, fixed_overhead)
 * in place, exactly as the other calls do. */
int mla_resolve_shape(mla_shape* shape);

/* Tile scheduler ("FlashMLA Sparse Decode 完整计算过程详解", step 3): computes
 * the partition plan on the device into sched_meta_dev (num_parts
 * mla_sched_part records) and num_splits_dev (b + 1 int32 prefix), in one
 * launch of one work-group (1024 threads evaluating the greedy fill in
 * parallel; one lane filling it in order when the per-request state does not
 * fit).  It depends on the shape only, so one plan serves every layer of a
 * step. */
int mla_get_sched_meta(const mla_shape* shape, void* sched_meta_dev,
                       int32_t* num_splits_dev, void* stream);

/* The same plan computed on the host into host buffers of the same sizes. */
int mla_plan_sched_meta_host(const mla_shape* shape, void* sched_meta_host,
                             int32_t* num_splits_host);

/* Tile scheduler with per-request valid lengths ("FlashMLA Sparse Decode
 * 完整计算过程详解", step 3, where a request's block count follows its valid
 * top-k length; "FlashMLA 与 DSA" section 4.3 for topk_length): request r costs
 * ceil(min(max(topk_length_dev[r], 0), topk) / split_granularity) blocks plus
 * fixed_overhead, so short requests take fewer partitions and tiles.
 * topk_length_dev is int32 [b] device memory, 4-byte aligned, read by the
 * scheduler kernel on `stream`; the decode and combine calls must pass the
 * same array as mla_decode_args.topk_length.  One lane fills the plan
 * sequentially.  Output buffers and errors as mla_get_sched_meta, plus
 * MLA_ERR_INVALID_ARG for a NULL or misaligned topk_length_dev. */
int mla_get_sched_meta_len(const mla_shape* shape, const int32_t* topk_length_dev,
                           void* sched_meta_dev, int32_t* num_splits_dev, void* stream);

/* The same length-aware plan computed on the host; topk_length_host is int32 [b]
 * host memory. */
int mla_plan_sched_meta_len_host(const mla_shape* shape, const int32_t* topk_length_host,
                                 void* sched_meta_host, int32_t* num_splits_host);

/* Sparse decode ("FlashMLA Sparse Decode 完整计算过程详解", steps 7-14):
 * gathers and dequantises the selected rows, runs the two bf16 contractions with
 * an online softmax, and writes out/lse for unsplit requests and o_accum /
 * lse_accum (base 2) for split ones. */
int mla_sparse_decode_fwd(const mla_decode_args* args, void* stream);

/* FP4 extra cache beside a V4.1 main cache ("FlashMLA 与 DSA" section 3.1:
 * 288 bytes per token, e8m0 scales per 16 elements; section 6.1: FP4 only as
 * an extra cache, with V4.1; section 3.2: split-KV decided on topk +
 * extra_topk; section 3.5: main and extra blocks walked in one loop each).
 * A query token attends over its main slots and its extra slots in one
 * softmax.  Page n of P tokens starts at kv + n * kv_stride_block; token
 * t = n P + o has its data row (512 E2M1 values, element 2 i in the low
 * nibble of byte i: 256 bytes) at page + 256 o and its scale row (32 e8m0
 * bytes, one per 16 dims) at page + 256 P + 32 o.  The split of the 288
 * bytes, the nibble order and the e8m0 scale type (the pages name both e8m0
 * and e4m3 for FP4 scales) are readings; V = K.  All pointers are device
 * memory owned by the caller. */
typedef struct mla_extra_kv {
    const void* kv;                 /* [num_blocks, kv_stride_block] bytes, 16-byte aligned       */
    int64_t kv_stride_block;        /* bytes per page: >= P * 288, a multiple of 16, P * 288 < 2^31 */
    int32_t page_block_size;        /* P >= 1                                                      */
    int64_t num_kv_tokens;          /* num_blocks * P, in [1, 2^31)                               */
    const int32_t* indices;         /* [b, s_q, extra_topk] physical token ids of this cache, -1 =
                                       empty (ids outside [0, num_kv_tokens) are empty too);
                                       last dim contiguous, 4-byte aligned                        */
    int64_t idx_stride_b, idx_stride_s;   /* in elements                                          */
    int32_t extra_topk;             /* extra slots per query token, in [1, shape.topk)           */
    const int32_t* topk_length;     /* NULL, or int32 [b]: extra slots at positions >= it are
                                       empty (clamped to [0, extra_topk])                         */
} mla_extra_kv;

/* Sparse decode over a V4.1 main cache and an FP4 extra cache.  args is as
 * for mla_sparse_decode_fwd with kv_format MLA_KV_V41_528, except that
 * args->shape.topk counts every slot of a query token: its first
 * shape.topk - extra->extra_topk slots are the main slots (args->indices
 * rows of that many ids, args->topk_length their valid lengths), the rest
 * the extra slots.  The plan (mla_get_sched_meta, or NULL for the closed
 * form) and mla_splitkv_combine take that same args->shape; plans made from
 * valid lengths are not supported here (the decode and the combine then
 * write NaN).  MLA_ERR_UNSUPPORTED for another main format; MLA_ERR_INVALID_ARG
 * for a NULL extra or a bad extra field. */
int mla_sparse_decode_extra_fwd(const mla_decode_args* args, const mla_extra_kv* extra, void* stream);

/* Dense decode ("FlashMLA Sparse Decode 完整计算过程详解", step 1: a call
 * without indices takes block_table + cache_seqlens and walks every page of
 * a request in block-table order; the caller routes here when the context is
 * no longer than topk; "FlashMLA 与 DSA" sections 3.3 and 6.1 for the dense
 * decode and its 64-token pages): request b attends to its first
 * cache_seqlens[b] logical tokens, token t being physical token
 *   block_table[b * block_table_stride + t / 64] * 64 + t % 64
 * of the FP8 656-byte paged cache, with the same scores, softmax, out, lse,
 * split partials and attention sink as mla_sparse_decode_fwd.
 *   - args->indices must be NULL; args->topk_length holds cache_seqlens (int32
 *     [b] device memory, clamped to [0, topk]); args->shape.topk is the
 *     tokens a block-table row can name (its width * 64); page_block_size 64;
 *     the page stride below 4 GiB.
 *   - block_table: int32 device memory, rows block_table_stride (>= topk / 64)
 *     elements apart, 4-byte aligned.  An entry outside [0, num_kv_tokens / 64)
 *     makes the tokens of that page empty (like -1 in the sparse indices).
 *   - causal = 1 (with s_q > 1, multi-token decode): the s_q query tokens are
 *     the last s_q positions of the sequence, so query token j sees
 *     cache_seqlens[b] - (s_q - 1 - j) tokens; causal = 0: all of them see
 *     cache_seqlens[b].
 *   - Plans: mla_get_sched_meta_len with the cache lengths (a request then
 *     costs its own pages), mla_get_sched_meta, or the closed form; then
 *     mla_splitkv_combine with the same args.
 * MLA_ERR_UNSUPPORTED for the bf16 cache or another page size. */
int mla_dense_decode_fwd(const mla_decode_args* args, const int32_t* block_table,
                         int64_t block_table_stride, int causal, void* stream);

/* Split-KV combine (step 16): merges the partials of every split request into
 * out / lse; unsplit requests are left untouched.  args->indices is not read
 * (it may be NULL).  With the closed-form plan (plan pointers NULL) and
 * partitions that hold whole requests only, nothing is split and nothing is
 * launched. */
int mla_splitkv_combine(const mla_decode_args* args, void* stream);

/* Test hook for the gather + dequant stage (attn_sink and topk_length are not
 * used): for every (b, s, slot) writes the
 * dequantised 576-value row as the decode kernel stages it, bf16
 * [b, s_q, topk, 576] into k_rows; if v_rows is not NULL also the 512 V values
 * read back through the decode kernel's transposed V layout, bf16
 * [b, s_q, topk, 512].  Empty slots give zero rows.  Both contiguous. */
int mla_debug_gather_dequant(const mla_decode_args* args, void* k_rows, void* v_rows,
                             void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the whole
 * decode step -- the tile plan when fixed_overhead > 0 (else the closed form),
 * mla_sparse_decode_fwd and mla_splitkv_combine -- in one call that allocates
 * nothing.  args->sched_meta, num_splits, o_accum and lse_accum must be NULL
 * (MLA_ERR_INVALID_ARG otherwise); the plan and the split partials live in one
 * 64 MiB device array of the library, one per GPU, held until the process
 * ends.  A shape whose split workspace does not fit ((b + num_parts) * s_q
 * splits of 128 KB plus h_q * 4 B each) is rejected with MLA_ERR_WORKSPACE before
 * anything runs.  Every call on a GPU uses that GPU's array: calls that
 * overlap on one GPU (different streams or threads) race; calls in one
 * stream are ordered.  Outputs and errors otherwise as the calls above. */
int mla_sparse_decode_noalloc(const mla_decode_args* args, void* stream);

/* Message for the last non-OK status on this thread ("" if none). */
const char* mla_last_error(void);

/* Library version string. */
const char* mla_version(void);

/* Lightning indexer and top-k ("FlashMLA 与 DSA：内核、流水线和正确性边界",
 * sections 4.1, 4.2, 5.2, 5.3, 5.5): the step upstream of the sparse decode
 * that picks each request's topk key tokens.  All pointers are device memory
 * owned by the caller. */
typedef struct mla_indexer_args {
    int32_t b;                  /* requests (one query token each), 0 .. 65535          */
    int32_t n_heads;            /* indexer heads, 32 or 64                               */
    int32_t max_pages;          /* page-table width; logical tokens < max_pages * 64    */
    int32_t num_pages;          /* physical pages in kcache                              */
    int32_t topk;               /* K >= 1 (2048 in DeepSeek-V3.2)                        */
    const void* q;              /* e4m3 [b, n_heads, 128] contiguous, 16-byte aligned   */
    const float* weights;       /* fp32 [b, n_heads]: head weights with the q scale and
                                   1/sqrt(d) folded in (section 4.1)                     */
    const void* kcache;         /* [num_pages, 8448] bytes: per page 64 x 128 e4m3 key
                                   codes (token-major) then 64 fp32 scales (5.3)         */
    const int32_t* page_table;  /* int32 [b, max_pages]: logical page -> physical page;
                                   an entry outside [0, num_pages) makes its tokens score
                                   -inf and emit id -1                                   */
    const int32_t* seq_len;     /* int32 [b]: valid tokens, clamped to [0, max_pages*64] */
    void* scores;               /* bf16 [b, max_pages * 64], 16-byte aligned: written by
                                   mla_indexer_scores for t < seq_len of rows with
                                   seq_len > topk, read by mla_indexer_topk              */
    int32_t* indices;           /* int32 [b, topk] output of mla_indexer_topk            */
} mla_indexer_args;

/* Index scores (section 4.1, Eq. 1): scores[r][t] = bf16( scale_t *
 * sum_j weights[r][j] * max(0, q[r][j] . codes_t) ), the FP8 products summed in
 * fp32 on the matrix cores and the positive per-token scale applied after the
 * head sum (section 5.3).  Rows with seq_len <= topk are skipped (section 5.2).
 * MLA_ERR_INVALID_ARG / MLA_ERR_UNSUPPORTED for bad sizes or pointers. */
int mla_indexer_scores(const mla_indexer_args* args, void* stream);

/* Top-k (sections 4.2, 5.5): for each request the topk highest scores among its
 * first seq_len tokens, written to indices[r] as physical token ids
 * (page_table[r][t / 64] * 64 + t % 64), in no particular order; ties at the
 * threshold keep an arbitrary subset.  seq_len <= topk emits tokens
 * 0 .. seq_len - 1 then -1 (section 5.2).  Reads scores only. */
int mla_indexer_topk(const mla_indexer_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
