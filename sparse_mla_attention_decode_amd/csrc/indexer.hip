// Lightning indexer and top-k selection ("FlashMLA 与 DSA：内核、流水线和正确性边界",
// sections 4.1, 4.2, 5.2, 5.3, 5.5): the FP8 index scores of Eq. 1 over the
// paged key cache, stored as bf16, then the K highest per request emitted as
// physical token ids for the sparse decode.
#include "device_common.h"
#include "indexer_internal.h"

namespace mla {
namespace {

constexpr int IX_PAGE = 64;                 // tokens per key-cache page
constexpr int IX_DIM = 128;                 // e4m3 dims per key
constexpr int IX_PAGE_BYTES = IX_PAGE * IX_DIM + IX_PAGE * 4;   // codes, then fp32 scales
constexpr int IX_WAVES = 4;
constexpr int IX_PAGES_PER_WAVE = 4;        // q and the weights stay in registers across them
constexpr int TOPK_THREADS = 1024;

__device__ __forceinline__ int clamp_len(const IndexerParams& p, int r) {
    return min(max(p.seq_len[r], 0), p.max_pages * IX_PAGE);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {          // nearest, ties to even
    const uint32_t u = __float_as_uint(x);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Scores of one request's pages (Eq. 1).  Each wave takes up to four pages
// (the work-group's waves read adjacent pages at each step), each as two
// groups of 32 tokens.  The head-by-token products run on the FP8 matrix
// cores with q as the A operand (rows = heads) and the keys as B (columns =
// tokens), so every lane ends with one token's 16 head dot products per head
// tile: ReLU, the head weights and the sum over heads stay in the lane, and
// one exchange joins the two lane halves.  The contraction's k slots of lane
// half hf at step s are dims 64 hf + 8 s .. + 7 for both operands, so each
// lane reads 64 contiguous bytes of its head row and of its token row.  The
// per-token scale multiplies the head sum (it is positive, so it commutes
// with the ReLU: section 5.3).
__global__ void __launch_bounds__(IX_WAVES * 64) indexer_score_kernel(IndexerParams p) {
    const int r = blockIdx.y;
    const int len = clamp_len(p, r);
    if (len <= p.topk) return;                                   // passthrough row
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int first_page = blockIdx.x * IX_WAVES * IX_PAGES_PER_WAVE + wave;
    if (first_page * IX_PAGE >= len) return;
    const int hf = lane >> 5, col = lane & 31;
    const int nt = p.n_heads >> 5;                               // 1 or 2 head tiles

    long qa[2][8];
    float wv[2][16];
    const uint8_t* qr = p.q + (size_t)r * p.n_heads * IX_DIM;
    const float* wr = p.weights + (size_t)r * p.n_heads;
    for (int tile = 0; tile < 2; ++tile) {
        const int ht = tile < nt ? tile : 0;
        const u32x4* src = (const u32x4*)(qr + (ht * 32 + col) * IX_DIM + 64 * hf);
        for (int c = 0; c < 4; ++c) {
            const u32x4 v = src[c];
            qa[tile][2 * c] = (long)(((uint64_t)v[1] << 32) | v[0]);
            qa[tile][2 * c + 1] = (long)(((uint64_t)v[3] << 32) | v[2]);
        }
        for (int i = 0; i < 16; ++i)
            wv[tile][i] = tile < nt ? wr[ht * 32 + 8 * (i >> 2) + 4 * hf + (i & 3)] : 0.0f;
    }

    uint16_t* out = p.scores + (size_t)r * p.max_pages * IX_PAGE;
    for (int step = 0; step < IX_PAGES_PER_WAVE; ++step) {
    const int page_l = first_page + step * IX_WAVES;
    const int t0 = page_l * IX_PAGE;
    if (t0 >= len) break;                                        // page_l < max_pages below
    const int pg = p.page_table[(size_t)r * p.max_pages + page_l];
    const bool ok = pg >= 0 && pg < p.num_pages;
    const uint8_t* page = p.kcache + (size_t)(ok ? pg : 0) * IX_PAGE_BYTES;

    for (int g = 0; g < 2; ++g) {
        const int tok = g * 32 + col;
        const u32x4* ks = (const u32x4*)(page + tok * IX_DIM + 64 * hf);
        long kb[8];
        for (int c = 0; c < 4; ++c) {
            const u32x4 v = ks[c];
            kb[2 * c] = (long)(((uint64_t)v[1] << 32) | v[0]);
            kb[2 * c + 1] = (long)(((uint64_t)v[3] << 32) | v[2]);
        }
        float sum = 0.0f;
        for (int tile = 0; tile < 2; ++tile) {
            if (tile >= nt) break;
            f32x16 acc = {};
            for (int s = 0; s < 8; ++s)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(qa[tile][s], kb[s], acc, 0, 0, 0);
            for (int i = 0; i < 16; ++i) sum += wv[tile][i] * fmaxf(acc[i], 0.0f);
        }
        sum += __shfl_xor(sum, 32);
        const float scale = ((const float*)(page + IX_PAGE * IX_DIM))[tok];
        const int t = t0 + tok;
        if (hf == 0 && t < len) out[t] = ok ? to_bf16_bits(sum * scale) : (uint16_t)0xFF80u;   // -inf
    }
    }
}

__device__ __forceinline__ uint32_t order_key(uint32_t b) {     // bf16 bits -> unsigned order
    return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

__device__ __forceinline__ int phys_id(const int32_t* pt, int t, int num_pages) {
    const int pg = pt[t >> 6];
    return (pg >= 0 && pg < num_pages) ? pg * IX_PAGE + (t & 63) : -1;
}

constexpr int TK_DIGIT1 = 12;                         // first radix digit: the top 12 bits of the key
constexpr int TK_BINS = 1 << TK_DIGIT1;              // 4096
constexpr int TK_CAND = 8192;                         // tokens of the threshold bin kept in LDS

// Block-wide: the largest bin index i of hist[0 .. nbins) whose suffix count
// S(i) = sum_{j >= i} hist[j] reaches `target` (S(i) >= target > S(i + 1)),
// and S(i + 1).  nbins = 256 * g; every thread of the block calls it.
// S(0) >= target >= 1 is required (there is such a bin).
__device__ void find_threshold_bin(const uint32_t* hist, int nbins, uint32_t target, uint32_t* coarse,
                                   int* bin_out, uint32_t* above_out) {
    const int tid = threadIdx.x, g = nbins >> 8;
    if (tid < 256) {                                  // coarse group sums, then their suffix sums
        uint32_t sum = 0;
        for (int j = 0; j < g; ++j) sum += hist[tid * g + j];
        coarse[tid] = sum;
    }
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        uint32_t v = 0;
        if (tid < 256 && tid + off < 256) v = coarse[tid + off];
        __syncthreads();
        if (tid < 256) coarse[tid] += v;
        __syncthreads();
    }
    if (tid < 256) {
        const uint32_t si = coarse[tid], sn = tid < 255 ? coarse[tid + 1] : 0u;
        if (si >= target && sn < target) {            // exactly one group qualifies
            uint32_t acc = sn;
            int b = tid * g + g - 1;
            for (; b > tid * g; --b) {
                if (acc + hist[b] >= target) break;
                acc += hist[b];
            }
            *bin_out = b;
            *above_out = acc;
        }
    }
    __syncthreads();
}

// Exact top-K of one request's bf16 scores (sections 4.2, 5.5), one
// 1024-thread work-group per request, on the 16-bit order key of each score:
//   1. a 4096-bin histogram of the key's top 12 bits (sign, exponent and three
//      mantissa bits, so that scores of one magnitude spread over many bins and
//      the LDS atomics rarely collide), eight scores per 16-byte load;
//   2. the threshold bin b1: fewer than K keys lie above it, at least K at or
//      above it;
//   3. a second pass that emits every key above b1 at once and keeps the
//      tokens of bin b1 in LDS (or, if there are too many, notes that);
//   4. among those candidates, the low four bits of the key select the rest:
//      keys above the threshold key all, equal keys up to K (any of them).
// Ids are remapped through the page table as they are written; rows with
// seq_len <= K emit tokens 0 .. seq_len - 1 and -1 padding without reading
// scores (section 5.2).
__global__ void __launch_bounds__(TOPK_THREADS) indexer_topk_kernel(IndexerParams p) {
    __shared__ uint32_t hist[TK_BINS];
    __shared__ uint32_t cand[TK_CAND];
    __shared__ uint32_t coarse[256];
    __shared__ uint32_t hist2[16];
    __shared__ int bin_s;
    __shared__ uint32_t above_s, cnt_out, cnt_cand, cnt_eq;
    const int r = blockIdx.x, tid = threadIdx.x, K = p.topk;
    const int len = clamp_len(p, r);
    const int32_t* pt = p.page_table + (size_t)r * p.max_pages;
    int32_t* out = p.indices + (size_t)r * K;
    if (len <= K) {
        for (int k = tid; k < K; k += TOPK_THREADS) out[k] = k < len ? phys_id(pt, k, p.num_pages) : -1;
        return;
    }
    const uint16_t* s = p.scores + (size_t)r * p.max_pages * IX_PAGE;
    const u32x4* s16 = (const u32x4*)s;               // rows start on 128-byte boundaries
    const int n_chunks = (len + 7) >> 3;

    for (int i = tid; i < TK_BINS; i += TOPK_THREADS) hist[i] = 0;
    if (tid == 0) { cnt_out = 0; cnt_cand = 0; cnt_eq = 0; }
    if (tid < 16) hist2[tid] = 0;
    __syncthreads();
    // 1. first-digit histogram
    for (int c = tid; c < n_chunks; c += TOPK_THREADS) {
        const u32x4 v = s16[c];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = 8 * c + e;
            if (t < len) atomicAdd(&hist[order_key((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) >> 4], 1u);
        }
    }
    __syncthreads();
    // 2. threshold bin
    find_threshold_bin(hist, TK_BINS, (uint32_t)K, coarse, &bin_s, &above_s);
    const uint32_t b1 = (uint32_t)bin_s, above1 = above_s;
    const uint32_t in_bin = hist[b1];
    const bool stash = in_bin <= (uint32_t)TK_CAND;
    // 3. keys above b1 are in the top K; the tokens of bin b1 are candidates
    for (int c = tid; c < n_chunks; c += TOPK_THREADS) {
        const u32x4 v = s16[c];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = 8 * c + e;
            if (t >= len) continue;
            const uint32_t k = order_key((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
            if ((k >> 4) > b1) {
                out[atomicAdd(&cnt_out, 1u)] = phys_id(pt, t, p.num_pages);
            } else if ((k >> 4) == b1) {
                atomicAdd(&hist2[k & 15u], 1u);
                if (stash) cand[atomicAdd(&cnt_cand, 1u)] = (uint32_t)t;
            }
        }
    }
    __syncthreads();
    // 4. the threshold key T inside bin b1 and the K - above1 keys taken from it
    if (tid == 0) {
        const uint32_t need = (uint32_t)K - above1;
        uint32_t acc = 0;
        int lo = 15;
        for (; lo > 0; --lo) {
            if (acc + hist2[lo] >= need) break;
            acc += hist2[lo];
        }
        bin_s = lo;                                   // low nibble of T
        above_s = acc;                                // keys of bin b1 above T
    }
    __syncthreads();
    const uint32_t T = (b1 << 4) | (uint32_t)bin_s, n_gt = above1 + above_s, take_eq = (uint32_t)K - n_gt;
    auto take = [&](int t, uint32_t k) {
        if (k > T) {                                  // slots above1 .. n_gt - 1 (cnt_out stands at above1)
            out[atomicAdd(&cnt_out, 1u)] = phys_id(pt, t, p.num_pages);
        } else if (k == T) {
            const uint32_t e = atomicAdd(&cnt_eq, 1u);
            if (e < take_eq) out[n_gt + e] = phys_id(pt, t, p.num_pages);
        }
    };
    if (stash) {
        for (uint32_t i = tid; i < in_bin; i += TOPK_THREADS) {
            const int t = (int)cand[i];
            take(t, order_key(s[t]));
        }
    } else {                                          // the bin did not fit: scan the row again
        for (int t = tid; t < len; t += TOPK_THREADS) {
            const uint32_t k = order_key(s[t]);
            if ((k >> 4) == b1) take(t, k);
        }
    }
}

}  // namespace

hipError_t launch_indexer_scores(const IndexerParams& p, hipStream_t st) {
    if (p.b == 0) return hipSuccess;
    const int per_wg = IX_WAVES * IX_PAGES_PER_WAVE;
    const dim3 grid((p.max_pages + per_wg - 1) / per_wg, p.b);
    hipLaunchKernelGGL(indexer_score_kernel, grid, dim3(IX_WAVES * 64), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_indexer_topk(const IndexerParams& p, hipStream_t st) {
    if (p.b == 0) return hipSuccess;
    hipLaunchKernelGGL(indexer_topk_kernel, dim3(p.b), dim3(TOPK_THREADS), 0, st, p);
    return hipGetLastError();
}

}  // namespace mla
