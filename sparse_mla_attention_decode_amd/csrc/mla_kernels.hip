// gfx950 tile scheduler of libmla ("FlashMLA Sparse Decode 完整计算过程详解",
// step 3): the greedy partition of (request, slot-block) work over num_parts
// partitions, as three kernels -- pointer doubling over the per-request state
// (uniform topk), a closed form plus a wave scan (zero per-request cost), and
// the sequential fill (per-request lengths, or shapes the others do not
// take).  The decode, combine and gather kernels are in decode_h128.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "mla_internal.h"
#include "sched_plan.h"

namespace mla {

// ----------------------------------------------------------------------------
// scheduler
// ----------------------------------------------------------------------------
// Every request has the same block count B, so the greedy fill is a walk on
// one small state: d = blocks of the current request already assigned when a
// partition opens.  One partition maps d to g(d) and finishes h(d) requests.
// g and h are tabulated for all d, their 2^k-fold compositions are built by
// pointer doubling, and each partition finds its opening state from the bits
// of its index.  Splits are numbered by a block-wide prefix sum.  The result
// equals the sequential left-to-right fill step by step.
constexpr int SCHED_THREADS = 1024;
constexpr int SCHED_MAX_STATES = 512;      // B = ceil(topk / block) handled here
constexpr int SCHED_LOG = 16;              // up to 65535 partitions

struct SchedStep {               // one partition opened with d blocks of request r done
    int begin_block, end_rel, end_block, last_splitted, next_d, finished;
};

__device__ __forceinline__ SchedStep sched_step(int d, int B, int ovh, int64_t payload) {
    SchedStep s;
    s.begin_block = d;
    const int64_t left = B - d;
    if (left + ovh <= payload) {
        const int64_t rem = payload - (left + ovh);
        const int64_t k = rem / (B + ovh);                  // whole requests after the first
        const int64_t x = rem - k * (B + ovh) - ovh;        // blocks of the next one
        if (x > 0) {
            s.end_rel = (int)(1 + k); s.end_block = (int)x; s.last_splitted = 1;
        } else {
            s.end_rel = (int)k; s.end_block = B; s.last_splitted = 0;
        }
        s.next_d = x > 0 ? (int)x : 0;
        s.finished = (int)(1 + k);
    } else {
        const int x = (int)(payload - ovh);
        s.end_rel = 0; s.end_block = d + x; s.last_splitted = 1;
        s.next_d = d + x;
        s.finished = 0;
    }
    return s;
}

__global__ void __launch_bounds__(SCHED_THREADS) sched_parallel_kernel(int b, int topk, int block,
                                                                     int ovh, int num_parts,
                                                                     int32_t* meta, int32_t* prefix) {
    __shared__ int16_t Gt[SCHED_LOG][SCHED_MAX_STATES];
    __shared__ int32_t Ht[SCHED_LOG][SCHED_MAX_STATES];
    __shared__ int32_t scan[SCHED_THREADS];
    const int tid = threadIdx.x;
    const int B = (topk + block - 1) / block;
    const int64_t total = (int64_t)b * (B + ovh);
    const int64_t payload = (total + num_parts - 1) / num_parts + ovh;
    int levels = 1;
    while ((1 << levels) <= num_parts && levels < SCHED_LOG) ++levels;

    for (int d = tid; d < B; d += SCHED_THREADS) {
        const SchedStep st = sched_step(d, B, ovh, payload);
        Gt[0][d] = (int16_t)st.next_d;
        Ht[0][d] = st.finished;
    }
    for (int k = 1; k < levels; ++k) {
        __syncthreads();
        for (int d = tid; d < B; d += SCHED_THREADS) {
            const int mid = Gt[k - 1][d];
            Gt[k][d] = Gt[k - 1][mid];
            Ht[k][d] = min(Ht[k - 1][d] + Ht[k - 1][mid], b);   // saturate: only r < b matters
        }
    }
    __syncthreads();

    // each thread owns a contiguous run of partitions
    const int per = (num_parts + SCHED_THREADS - 1) / SCHED_THREADS;
    const int p0 = min(tid * per, num_parts), p1 = min(p0 + per, num_parts);
    // opening state of p0
    int r = 0, d = 0;
    for (int k = 0; k < levels; ++k) {
        if ((p0 >> k) & 1) {
            r = min(r + Ht[k][d], b);
            d = Gt[k][d];
        }
    }
    // pieces of the run, then a block-wide exclusive scan of the counts
    int count = 0;
    {
        int rr = r, dd = d;
        for (int p = p0; p < p1 && rr < b; ++p) {
            const SchedStep st = sched_step(dd, B, ovh, payload);
            count += min(rr + st.end_rel, b - 1) - rr + 1;
            rr = min(rr + st.finished, b);
            dd = st.next_d;
        }
    }
    scan[tid] = count;
    __syncthreads();
    for (int off = 1; off < SCHED_THREADS; off <<= 1) {
        const int v = tid >= off ? scan[tid - off] : 0;
        __syncthreads();
        scan[tid] += v;
        __syncthreads();
    }
    int cursor = scan[tid] - count;
    const int total_pieces = scan[SCHED_THREADS - 1];
    for (int p = p0; p < p1; ++p) {
        int32_t* m = meta + 8 * p;
        if (r >= b) {
            m[0] = b; m[1] = b; m[2] = 0; m[3] = 0; m[4] = cursor; m[5] = 0; m[6] = 0; m[7] = 0;
            continue;
        }
        const SchedStep st = sched_step(d, B, ovh, payload);
        int end_req = r + st.end_rel, end_block = st.end_block, last = st.last_splitted;
        if (end_req >= b) { end_req = b - 1; end_block = B; last = 0; }
        m[0] = r; m[1] = end_req; m[2] = d; m[3] = end_block; m[4] = cursor;
        m[5] = d > 0; m[6] = last; m[7] = 0;
        for (int q = (d > 0 ? r + 1 : r); q <= end_req; ++q) prefix[q] = cursor + (q - r);
        cursor += end_req - r + 1;
        r = min(r + st.finished, b);
        d = st.next_d;
    }
    if (tid == 0) prefix[b] = total_pieces;
}

// Without a per-request overhead the greedy fill gives partition p exactly the
// blocks [p payload, min((p+1) payload, b B)) of the request-major block
// sequence, so every record has a closed form; only the split numbering needs
// a prefix sum (a wave scan plus one pass over the wave totals).
constexpr int SCHED_FLAT_THREADS = 1024;
__global__ void __launch_bounds__(SCHED_FLAT_THREADS) sched_flat_kernel(int b, int topk, int block,
                                                                        int num_parts, int32_t* meta,
                                                                        int32_t* prefix) {
    __shared__ int32_t wsum[SCHED_FLAT_THREADS / 64];
    __shared__ int32_t first_split[SCHED_FLAT_THREADS];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t B = (topk + block - 1) / block, total = (int64_t)b * B;
    const int64_t payload = (total + num_parts - 1) / num_parts;
    const int64_t s0 = (int64_t)tid * payload, s1 = min(s0 + payload, total);
    const bool busy = tid < num_parts && s0 < total;
    const int pieces = busy ? (int)((s1 - 1) / B - s0 / B + 1) : 0;
    int incl = pieces;
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int before = 0;
    for (int i = 0; i < wv; ++i) before += wsum[i];
    const int cursor = before + incl - pieces;
    first_split[tid] = cursor;
    if (tid < num_parts) {
        int32_t* m = meta + 8 * tid;
        if (!busy) {
            m[0] = b; m[1] = b; m[2] = 0; m[3] = 0; m[4] = cursor; m[5] = 0; m[6] = 0; m[7] = 0;
        } else {
            const int64_t e = s1 - 1;
            const int begin_block = (int)(s0 % B), end_block = (int)(e % B) + 1;
            m[0] = (int)(s0 / B); m[1] = (int)(e / B); m[2] = begin_block; m[3] = end_block;
            m[4] = cursor; m[5] = begin_block > 0; m[6] = end_block < B; m[7] = 0;
        }
    }
    __syncthreads();
    // request r opens in partition q = floor(r B / payload) as its piece
    // r - (first request of q)
    for (int r = tid; r < b; r += SCHED_FLAT_THREADS) {
        const int64_t q = (int64_t)r * B / payload;
        prefix[r] = first_split[q] + r - (int)(q * payload / B);
    }
    if (tid == SCHED_FLAT_THREADS - 1) {
        int all = 0;
        for (int i = 0; i < SCHED_FLAT_THREADS / 64; ++i) all += wsum[i];
        prefix[b] = all;
    }
}

// Sequential fill, one lane (used when the state table does not fit, and for
// plans made from per-request valid lengths).
__global__ void __launch_bounds__(64) sched_kernel(int b, int topk, int block, int overhead,
                                                   int num_parts, const int32_t* lengths,
                                                   int32_t* meta, int32_t* prefix) {
    if (threadIdx.x != 0) return;
    plan_schedule(b, topk, block, overhead, num_parts, lengths, meta, prefix,
                  [](int32_t* p, int32_t v) { *p = v; });
}

// ----------------------------------------------------------------------------
// launcher
// ----------------------------------------------------------------------------
hipError_t launch_sched(const ResolvedShape& s, const int32_t* lengths, int32_t* meta, int32_t* prefix,
                        hipStream_t st) {
    const int B = (s.topk + s.block - 1) / s.block;
    if (lengths != nullptr)
        hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(64), 0, st, s.b, s.topk, s.block, s.overhead,
                           s.num_parts, lengths, meta, prefix);
    else if (s.overhead == 0 && s.num_parts <= SCHED_FLAT_THREADS)
        hipLaunchKernelGGL(sched_flat_kernel, dim3(1), dim3(SCHED_FLAT_THREADS), 0, st, s.b, s.topk,
                           s.block, s.num_parts, meta, prefix);
    else if (B <= SCHED_MAX_STATES && s.num_parts < (1 << SCHED_LOG))
        hipLaunchKernelGGL(sched_parallel_kernel, dim3(1), dim3(SCHED_THREADS), 0, st, s.b, s.topk,
                           s.block, s.overhead, s.num_parts, meta, prefix);
    else
        hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(64), 0, st, s.b, s.topk, s.block, s.overhead,
                           s.num_parts, (const int32_t*)nullptr, meta, prefix);
    return hipGetLastError();
}

}  // namespace mla
