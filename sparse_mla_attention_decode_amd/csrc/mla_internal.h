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
    const int32_t* sched_meta;
    const int32_t* num_splits;
    float* o_accum;
    float* lse_accum;
    int64_t n_tok;
    uint32_t n_tok32;               // min(n_tok, 2^31 - 1): token ids are int32
    int b, s_q, h_q, topk, page_block_size, block;
    uint32_t page_magic;            // t / page_block_size == (mulhi(t, page_magic) + t) >> page_mshift
    int page_mshift;                // for 0 <= t < 2^31 (round-up reciprocal)
    int packed_partials;            // split partials as packed bf16 (128-head FP8 decode)
    float c;                        // sm_scale * log2(e)
    float threshold;                // log2-units gap above the reference max that
                                    // makes a piece recompute with a higher reference
};

// A tile whose max score exceeds the reference (the first valid tile's max) by
// more than this many log2 units triggers a recompute.  Below it p <= 2^64, so
// l <= topk * 2^64 and every accumulator stays far inside fp32 range.
constexpr float kRefGapLog2 = 64.0f;

hipError_t launch_sched(const ResolvedShape& s, int32_t* meta, int32_t* prefix, hipStream_t st);
hipError_t launch_decode(const DecodeParams& p, int kv_format, int num_parts, hipStream_t st);
hipError_t launch_decode_fp8_h128(const DecodeParams& p, int num_parts, hipStream_t st);
hipError_t launch_gather_fp8_h128(const DecodeParams& p, uint16_t* k_rows, uint16_t* v_rows,
                                  hipStream_t st);
hipError_t launch_combine(const DecodeParams& p, hipStream_t st);
hipError_t launch_combine_packed(const DecodeParams& p, hipStream_t st);
hipError_t launch_gather(const DecodeParams& p, int kv_format, uint16_t* k_rows, uint16_t* v_rows,
                         hipStream_t st);

}  // namespace mla
