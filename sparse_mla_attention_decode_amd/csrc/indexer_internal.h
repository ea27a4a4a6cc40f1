// Lightning indexer + top-k ("FlashMLA 与 DSA：内核、流水线和正确性边界",
// sections 4.1, 5.3, 5.5): kernel parameters, validated by the C entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct IndexerParams {
    int b, n_heads, max_pages, num_pages, topk;
    const uint8_t* q;            // e4m3 [b, n_heads, 128]
    const float* weights;        // [b, n_heads]
    const uint8_t* kcache;       // [num_pages, 8448]
    const int32_t* page_table;   // [b, max_pages]
    const int32_t* seq_len;      // [b]
    uint16_t* scores;            // bf16 [b, max_pages * 64]
    int32_t* indices;            // [b, topk]
};

hipError_t launch_indexer_scores(const IndexerParams& p, hipStream_t st);
hipError_t launch_indexer_topk(const IndexerParams& p, hipStream_t st);

}  // namespace mla
