// Greedy split-KV tile scheduler ("FlashMLA Sparse Decode 完整计算过程详解",
// step 3): the topk list of each request is cut into blocks of `block`
// slots (or, given per-request valid lengths, ceil(length / block) blocks for
// its first min(max(length, 0), topk) slots); every request costs its block
// count plus a fixed overhead; the
// payload of a partition is ceil(total / num_parts) + overhead; partitions are
// filled left to right and a request that does not fit whole is split, the
// partition taking (remaining capacity - overhead) of its blocks when that is
// positive.  One implementation serves the host export and the device kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Writes num_parts records of 8 int32 (begin_req, end_req, begin_block,
// end_block, begin_split, first_splitted, last_splitted, by_length) and the
// split prefix (b + 1 int32).  `lengths` is NULL (every request has topk slots,
// by_length = 0) or b int32 valid lengths readable by the caller (by_length =
// 1 in every record: the requests a partition covers whole have their own
// block counts).  `store` is called as store(ptr, value) so the device
// caller can route writes through vector stores.
template <typename Store>
__host__ __device__ inline void plan_schedule(int b, int topk, int block, int overhead,
                                              int num_parts, const int32_t* lengths, int32_t* meta,
                                              int32_t* prefix, Store store) {
    const int full = (topk + block - 1) / block;
    auto blocks_of = [&](int r) -> int {
        if (lengths == nullptr) return full;
        const int len = lengths[r] < 0 ? 0 : (lengths[r] > topk ? topk : lengths[r]);
        return (len + block - 1) / block;
    };
    const int flag = lengths != nullptr;
    int64_t total = 0;
    for (int r = 0; r < b; ++r) total += blocks_of(r) + overhead;
    const int payload = (int)((total + num_parts - 1) / num_parts) + overhead;
    int req = 0, done = 0, cursor = 0;
    store(prefix + 0, 0);
    for (int p = 0; p < num_parts; ++p) {
        int32_t* m = meta + 8 * p;
        if (req >= b) {
            store(m + 0, b); store(m + 1, b); store(m + 2, 0); store(m + 3, 0);
            store(m + 4, cursor); store(m + 5, 0); store(m + 6, 0); store(m + 7, flag);
            continue;
        }
        const int begin_req = req, begin_block = done;
        const int first_splitted = done > 0;
        int remain = payload;
        int end_req = req, end_block = done, last_splitted = 0;
        while (req < b) {
            const int blocks = blocks_of(req);
            const int left = blocks - done;
            if (left + overhead <= remain) {
                remain -= left + overhead;
                end_req = req; end_block = blocks; last_splitted = 0;
                ++req; done = 0;
                store(prefix + req, cursor + (req - begin_req));   // splits of requests < req
            } else {
                const int take = remain - overhead;
                if (take > 0) {
                    done += take;
                    end_req = req; end_block = done; last_splitted = 1;
                }
                break;
            }
        }
        store(m + 0, begin_req); store(m + 1, end_req); store(m + 2, begin_block);
        store(m + 3, end_block); store(m + 4, cursor); store(m + 5, first_splitted);
        store(m + 6, last_splitted); store(m + 7, flag);
        cursor += end_req - begin_req + 1;
    }
}

}  // namespace mla
