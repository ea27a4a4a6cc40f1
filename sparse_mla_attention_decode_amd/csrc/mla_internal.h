// Internal declarations shared by the host API and the kernels of libmla.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

// mla_shape with every default resolved.
struct ResolvedShape {
    int b, s_q, h_q, topk, page_block_size, kv_format;
    int64_t num_kv_tokens;
    int num_parts;   // partitions per query-token column
    int block;       // topk slots per scheduler block
    int overhead;    // scheduler per-request cost in blocks
};

// Division by a divisor fixed at launch: for 0 <= n < 2^31,
// n / d == (mulhi(n, m) + n) >> s with s = ceil(log2 d),
// m = floor(2^32 (2^s - d) / d) + 1 (the round-up reciprocal).
struct FastDiv {
    uint32_t m;
    int s;
};
inline FastDiv make_fastdiv(uint32_t d) {
    int s = 0;
    while ((1ull << s) < d) ++s;
    return FastDiv{(uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1), s};
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) { return (__umulhi(n, f.m) + n) >> f.s; }

// Kernel arguments (by value).
struct DecodeParams {
    const uint16_t* q;
    int64_t q_sb, q_ss, q_sh;
    const uint8_t* kv;
    int64_t kv_block_stride;        // bytes: per page (FP8) or per token row (BF16)
    const int32_t* indices;
    int64_t idx_sb, idx_ss;
    uint16_t* out;
    int64_t out_sb, out_ss, out_sh;
    float* lse;
    const int32_t* sched_meta;      // NULL: closed-form plan (plan_part / split_prefix)
    const int32_t* num_splits;
    float* o_accum;
    float* lse_accum;
    const float* attn_sink;         // [h_q] natural-log sink logits, or NULL
    const int32_t* topk_length;     // [b] valid slots per request (dense decode: the cache
                                    // lengths), or NULL
    const int32_t* block_table;     // dense decode: [b, bt_stride] logical page -> physical page;
                                    // NULL for sparse decode (ids come from `indices`)
    int64_t bt_stride;              // elements between block-table rows
    int causal;                     // dense decode with s_q > 1: query token sq sees
                                    // topk_length - (s_q - 1 - sq) tokens
    uint32_t n_pages;               // FP8 pages in the cache (n_tok / page_block_size)
    int64_t n_tok;
    uint32_t n_tok32;               // min(n_tok, 2^31 - 1): token ids are int32
    int b, s_q, h_q, topk, page_block_size, block;
    uint32_t page_magic;            // t / page_block_size == (mulhi(t, page_magic) + t) >> page_mshift
    int page_mshift;                // for 0 <= t < 2^31 (round-up reciprocal)
    uint32_t soa_scale_off;         // V4 / V4.1: byte offset of a page's scale rows (P * data row)
    // FP4 extra cache beside a V4.1 main cache (x_kv NULL: none).  Its slots
    // follow the main ones: slot k >= main_topk is extra slot k - main_topk,
    // and topk counts both.
    const uint8_t* x_kv;
    int64_t x_block_stride;
    const int32_t* x_indices;
    int64_t x_idx_sb, x_idx_ss;
    const int32_t* x_topk_length;   // NULL or [b]
    int main_topk, x_topk, x_page_block_size, x_page_mshift;
    uint32_t x_page_magic, x_scale_off, x_n_tok32;
    int kv_flat;                    // FP8 pages back to back, n_tok < 2^24 and n_tok * 656 < 2^32:
                                    // the row of token t is kv + 656 t (32-bit offset)
    // closed-form plan (per-request cost zero): B blocks per request, total
    // b * B blocks, partitions of `payload` blocks; gb = B / gcd(B, payload),
    // gp = payload / gcd(B, payload).  All below 2^31.
    uint32_t plan_nblk, plan_total, plan_payload, plan_gb, plan_gp;
    FastDiv div_nblk, div_payload, div_gb, div_gp;     // the same divisors as reciprocals
    float c;                        // sm_scale * log2(e)
    float threshold;                // log2-units gap above the reference max that
                                    // makes a piece recompute with a higher reference
};

// One partition of the plan: requests begin_req..end_req (inclusive), blocks
// [begin_block, end_block) of end_req, its first piece has split index
// begin_split; begin_req >= b marks an idle partition.  by_length: the plan
// was made from the valid lengths, so a request covered whole spans
// ceil(length / block) blocks instead of ceil(topk / block).
struct PartPlan {
    int begin_req, end_req, begin_block, end_block, begin_split, by_length;
};

// Blocks of request `req` that a partition covering it whole processes.
// (A by_length plan without lengths never gets here: see lengths_missing.)
__device__ __forceinline__ int whole_blocks(const DecodeParams& p, const PartPlan& plan, int req) {
    if (plan.by_length) {
        const int len = min(max(p.topk_length[req], 0), p.topk);
        return (len + p.block - 1) / p.block;
    }
    return (p.topk + p.block - 1) / p.block;
}

// Partition `part` of the plan, read from the scheduler's output or, with no
// scheduler output, evaluated in closed form.  With zero per-request cost the
// greedy fill ("FlashMLA Sparse Decode 完整计算过程详解", step 3) cuts the
// request-major sequence of T = b B blocks into consecutive runs of
// payload = ceil(T / num_parts) blocks: partition q holds blocks
// [q payload, min((q + 1) payload, T)).  Its pieces are the requests that run
// meets, so the pieces before it number
//   sum_{q' < q} (floor(e_q' / B) - floor(s_q' / B) + 1)
//     = q + floor((q payload - 1) / B) - #{0 < q' < q : B divides q' payload}
// (the sum telescopes; a boundary that is also a request boundary adds no
// piece), and B divides q' payload exactly when gb divides q'.
__device__ __forceinline__ PartPlan plan_part(const DecodeParams& p, int part) {
    PartPlan r;
    if (p.sched_meta != nullptr) {
        const int32_t* m = p.sched_meta + 8 * part;
        r.begin_req = m[0];
        r.end_req = m[1];
        r.begin_block = m[2];
        r.end_block = m[3];
        r.begin_split = m[4];
        r.by_length = m[7];
        return r;
    }
    const uint32_t B = p.plan_nblk, P = p.plan_payload, T = p.plan_total, q = (uint32_t)part;
    const uint32_t s0 = q * P;
    r.by_length = 0;
    if (s0 >= T) {
        r.begin_req = r.end_req = p.b;
        r.begin_block = r.end_block = r.begin_split = 0;
        return r;
    }
    const uint32_t e = min(s0 + P, T) - 1;
    // every dividend is below b B < 2^30 (checked on the host)
    const uint32_t rs = fdiv(s0, p.div_nblk), re = fdiv(e, p.div_nblk);
    r.begin_req = (int)rs;
    r.end_req = (int)re;
    r.begin_block = (int)(s0 - rs * B);
    r.end_block = (int)(e - re * B) + 1;
    r.begin_split = q == 0 ? 0 : (int)(q + fdiv(s0 - 1, p.div_nblk) - fdiv(q - 1, p.div_gb));
    return r;
}

// A plan made from valid lengths (by_length records) passed without the
// lengths it was made from.  The host cannot see this (the plan is device
// memory), so it is a contract error found on the device: the decode does
// nothing and the combine writes NaN to every output (split and unsplit
// requests alike), instead of silently mixing the two kinds of plan.
__device__ __forceinline__ bool lengths_missing(const DecodeParams& p) {
    // (also a length plan with an extra cache: such a plan covers main slots only)
    return p.sched_meta != nullptr && p.sched_meta[7] != 0 && (p.topk_length == nullptr || p.x_kv != nullptr);
}

// Split index of the first piece of request r (the number of pieces at r = b).
// Closed form as above: request r' covers partitions floor(r' B / payload) ..
// floor(((r' + 1) B - 1) / payload), so the pieces before request r number
//   r + floor((r B - 1) / payload) - #{0 < r' < r : payload divides r' B}.
__device__ __forceinline__ int split_prefix(const DecodeParams& p, int r) {
    if (p.num_splits != nullptr) return p.num_splits[r];
    if (r == 0) return 0;
    const uint32_t u = (uint32_t)r;
    return (int)(u + fdiv(u * p.plan_nblk - 1, p.div_payload) - fdiv(u - 1, p.div_gp));
}

// A tile whose max score exceeds the reference (the first valid tile's max) by
// more than this many log2 units triggers a recompute.  Below it p <= 2^64, so
// l <= topk * 2^64 and every accumulator stays far inside fp32 range.
constexpr float kRefGapLog2 = 64.0f;

hipError_t launch_sched(const ResolvedShape& s, const int32_t* lengths, int32_t* meta, int32_t* prefix,
                        hipStream_t st);
// decode_h128.hip: every cache format (656-byte, V4, V4.1 with the FP4 extra
// cache, bf16 rows), sparse and dense; the split-KV combine over its packed
// partials; the gather test hook (656-byte and bf16 rows)
hipError_t launch_decode(const DecodeParams& p, int kv_format, int num_parts, hipStream_t st);
hipError_t launch_combine(const DecodeParams& p, hipStream_t st);
hipError_t launch_gather(const DecodeParams& p, int kv_format, uint16_t* k_rows, uint16_t* v_rows,
                         hipStream_t st);

}  // namespace mla
