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

__device__ __forceinline__ uint32_t order_key(uint16_t b) {     // bf16 bits -> unsigned order
    return (b & 0x8000u) ? (uint32_t)(~b & 0xFFFFu) : (uint32_t)(b | 0x8000u);
}

__device__ __forceinline__ int phys_id(const int32_t* pt, int t, int num_pages) {
    const int pg = pt[t >> 6];
    return (pg >= 0 && pg < num_pages) ? pg * IX_PAGE + (t & 63) : -1;
}

// Bin i with S(i) >= target > S(i + 1), S(i) = sum of hist[j >= i]; the
// count above the bin goes to *above.  S(0) >= target >= 1 and S(256) = 0,
// so exactly one bin qualifies.
__device__ void find_bin(uint32_t* hist, uint32_t* scan, uint32_t target, int* bin, uint32_t* above) {
    const int tid = threadIdx.x;
    if (tid < 256) scan[tid] = hist[tid];
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        uint32_t v = 0;
        if (tid < 256 && tid + off < 256) v = scan[tid + off];
        __syncthreads();
        if (tid < 256) scan[tid] += v;
        __syncthreads();
    }
    if (tid < 256) {
        const uint32_t si = scan[tid], sn = tid < 255 ? scan[tid + 1] : 0u;
        if (si >= target && sn < target) { *bin = tid; *above = sn; }
    }
    __syncthreads();
}

// Exact top-K of one request's bf16 scores by a two-pass 8-bit radix select
// (section 5.5): a histogram of the high byte of the order key picks the
// threshold bin, a histogram of the low byte inside it picks the threshold
// key T; keys above T are all kept and the first K - #above keys equal to T
// (in the order the threads reach them) fill the rest.  Ids are remapped
// through the page table as they are written; rows with seq_len <= K emit
// tokens 0 .. seq_len - 1 and -1 padding without reading scores (section 5.2).
__global__ void __launch_bounds__(TOPK_THREADS) indexer_topk_kernel(IndexerParams p) {
    __shared__ uint32_t hist[256], scan[256];
    __shared__ int bin_s;
    __shared__ uint32_t above_s, cnt_gt, cnt_eq;
    const int r = blockIdx.x, tid = threadIdx.x, K = p.topk;
    const int len = clamp_len(p, r);
    const int32_t* pt = p.page_table + (size_t)r * p.max_pages;
    int32_t* out = p.indices + (size_t)r * K;
    if (len <= K) {
        for (int k = tid; k < K; k += TOPK_THREADS) out[k] = k < len ? phys_id(pt, k, p.num_pages) : -1;
        return;
    }
    const uint16_t* s = p.scores + (size_t)r * p.max_pages * IX_PAGE;

    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int t = tid; t < len; t += TOPK_THREADS) atomicAdd(&hist[order_key(s[t]) >> 8], 1u);
    __syncthreads();
    find_bin(hist, scan, (uint32_t)K, &bin_s, &above_s);
    const uint32_t b1 = (uint32_t)bin_s, above1 = above_s;

    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int t = tid; t < len; t += TOPK_THREADS) {
        const uint32_t k = order_key(s[t]);
        if ((k >> 8) == b1) atomicAdd(&hist[k & 255u], 1u);
    }
    __syncthreads();
    find_bin(hist, scan, (uint32_t)K - above1, &bin_s, &above_s);
    const uint32_t T = (b1 << 8) | (uint32_t)bin_s;
    const uint32_t n_gt = above1 + above_s, take_eq = (uint32_t)K - n_gt;

    if (tid == 0) { cnt_gt = 0; cnt_eq = 0; }
    __syncthreads();
    for (int t = tid; t < len; t += TOPK_THREADS) {
        const uint32_t k = order_key(s[t]);
        if (k > T) {
            out[atomicAdd(&cnt_gt, 1u)] = phys_id(pt, t, p.num_pages);
        } else if (k == T) {
            const uint32_t e = atomicAdd(&cnt_eq, 1u);
            if (e < take_eq) out[n_gt + e] = phys_id(pt, t, p.num_pages);
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
