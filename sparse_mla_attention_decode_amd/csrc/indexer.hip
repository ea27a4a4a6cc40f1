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
constexpr int IX_PAGES_PER_WAVE = 11;       // 12 x 64 work-groups for 512-page rows: one round at 3 per CU
constexpr int TOPK_THREADS = 1024;

__device__ __forceinline__ int clamp_len(const IndexerParams& p, int r) {
    return min(max(p.seq_len[r], 0), p.max_pages * IX_PAGE);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 32 contiguous bytes of an operand row as the 8-dword operand of a k-64 MFMA
__device__ __forceinline__ i32x8 join8(u32x4 a, u32x4 b) {
    return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {          // nearest, ties to even
    const uint32_t u = __float_as_uint(x);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Scores of one request's pages (Eq. 1).  Each wave takes up to
// IX_PAGES_PER_WAVE pages (the work-group's waves read adjacent pages at each
// step), each as two groups of 32 tokens, with the keys of its next page in
// flight while a page is scored.  The head-by-token products run on the FP8
// matrix cores with q as the A operand (rows = heads) and the keys as B
// (columns = tokens), so every lane ends with one token's 16 head dot products
// per head tile: ReLU, the head weights and the sum over heads stay in the
// lane, and one exchange joins the two lane halves.  The contraction's k slots
// of lane half hf at step s are dims 64 hf + 32 s .. + 31 for both operands, so
// each lane reads 64 contiguous bytes of its head row and of its token row.  The
// per-token scale multiplies the head sum (it is positive, so it commutes
// with the ReLU: section 5.3).
__global__ void __launch_bounds__(IX_WAVES * 64) __attribute__((amdgpu_waves_per_eu(3))) indexer_score_kernel(IndexerParams p) {
    const int r = blockIdx.y;
    const int len = clamp_len(p, r);
    if (len <= p.topk) return;                                   // passthrough row
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int first_page = blockIdx.x * IX_WAVES * IX_PAGES_PER_WAVE + wave;
    if (first_page * IX_PAGE >= len) return;
    const int hf = lane >> 5, col = lane & 31;
    const int nt = p.n_heads >> 5;                               // 1 or 2 head tiles

    i32x8 qa[2][2];
    float wv[2][16];
    const uint8_t* qr = p.q + (size_t)r * p.n_heads * IX_DIM;
    const float* wr = p.weights + (size_t)r * p.n_heads;
    for (int tile = 0; tile < 2; ++tile) {
        const int ht = tile < nt ? tile : 0;
        const u32x4* src = (const u32x4*)(qr + (ht * 32 + col) * IX_DIM + 64 * hf);
        for (int s = 0; s < 2; ++s) qa[tile][s] = join8(src[2 * s], src[2 * s + 1]);
        for (int i = 0; i < 16; ++i)
            wv[tile][i] = tile < nt ? wr[ht * 32 + 8 * (i >> 2) + 4 * hf + (i & 3)] : 0.0f;
    }

    // the wave's page-table entries up front (one round trip; lane s holds the
    // entry of its step s), then the keys of page s + 1 in flight while page s
    // is scored (two register sets, pages taken in pairs)
    const int32_t* pt = p.page_table + (size_t)r * p.max_pages;
    const int n_steps = min(IX_PAGES_PER_WAVE, (len - first_page * IX_PAGE + IX_WAVES * IX_PAGE - 1) / (IX_WAVES * IX_PAGE));
    const int pg_lane = lane < n_steps ? pt[first_page + lane * IX_WAVES] : -1;   // below max_pages
    struct PageRegs {
        i32x8 kb[2][2];
        float scale[2];
    };
    auto load_page = [&](int step, PageRegs& d) {
        const int pg = __builtin_amdgcn_readlane(pg_lane, step);
        const bool ok = pg >= 0 && pg < p.num_pages;
        const uint8_t* page = p.kcache + (size_t)(ok ? pg : 0) * IX_PAGE_BYTES;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int tok = g * 32 + col;
            const u32x4* ks = (const u32x4*)(page + tok * IX_DIM + 64 * hf);
#pragma unroll
            for (int s = 0; s < 2; ++s) d.kb[g][s] = join8(ks[2 * s], ks[2 * s + 1]);
            d.scale[g] = ((const float*)(page + IX_PAGE * IX_DIM))[tok];
        }
    };
    uint16_t* out = p.scores + (size_t)r * p.max_pages * IX_PAGE;
    auto score_page = [&](int step, const PageRegs& cur) {
        const int t0 = (first_page + step * IX_WAVES) * IX_PAGE;
        const int pg = __builtin_amdgcn_readlane(pg_lane, step);
        const bool ok = pg >= 0 && pg < p.num_pages;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            float sum = 0.0f;
#pragma unroll
            for (int tile = 0; tile < 2; ++tile) {
                if (tile >= nt) break;
                // two k-64 steps on e4m3 operands (format code 0 for both), block
                // scales 2^0 (e8m0 code 127): plain fp8 products summed in fp32
                f32x16 acc = {};
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[tile][s], cur.kb[g][s], acc, 0, 0, 0, 127,
                                                                          0, 127);
#pragma unroll
                for (int i = 0; i < 16; ++i) sum += wv[tile][i] * fmaxf(acc[i], 0.0f);
            }
            sum += __shfl_xor(sum, 32);
            const int t = t0 + g * 32 + col;
            if (hf == 0 && t < len) out[t] = ok ? to_bf16_bits(sum * cur.scale[g]) : (uint16_t)0xFF80u;   // -inf
        }
    };
    PageRegs a, b;
    load_page(0, a);
    for (int step = 0; step < n_steps; step += 2) {
        if (step + 1 < n_steps) load_page(step + 1, b);
        score_page(step, a);
        if (step + 1 >= n_steps) break;
        if (step + 2 < n_steps) load_page(step + 2, a);
        score_page(step + 1, b);
    }
}

__device__ __forceinline__ uint32_t order_key(uint32_t b) {     // bf16 bits -> unsigned order
    return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

__device__ __forceinline__ int phys_id(const int32_t* pt, int t, int num_pages) {
    const int pg = pt[t >> 6];
    return (pg >= 0 && pg < num_pages) ? pg * IX_PAGE + (t & 63) : -1;
}

constexpr int TK_DIGIT1 = 12;                         // radix digit of the two-level path: 12 bits
constexpr int TK_BINS = 1 << TK_DIGIT1;              // 4096
constexpr int TK_LDS_KEYS = 65536;                    // rows of up to this many scores stay in LDS
constexpr int TK_LDS_PAGES = TK_LDS_KEYS / IX_PAGE;   // with their page-table entries
constexpr int TK_HIST = TK_BINS + 64;                 // and a dummy bin per lane
constexpr int TK_LDS_BYTES = TK_HIST * 4 + TK_LDS_KEYS * 2 + TK_LDS_PAGES * 4;   // 148 KB

// Block-wide: the largest bin index i of hist[0 .. 4096) whose suffix count
// S(i) = sum_{j >= i} hist[j] reaches `target` (S(i) >= target > S(i + 1))
// and S(i + 1); *bin_out = -1 when S(0) < target.  Every thread sums four
// bins and sixteen lanes join them into the sum of a group of 64 bins
// (gsum[64]); wave 0 then finds the group and the bin in it with suffix scans
// across lanes (shuffles).  Two block barriers.
__device__ void find_threshold_bin(const uint32_t* hist, uint32_t target, uint32_t* gsum, int* bin_out,
                                   uint32_t* above_out) {
    const int tid = threadIdx.x, lane = tid & 63;
    const u32x4 h = *(const u32x4*)(hist + 4 * tid);              // TOPK_THREADS * 4 == 4096 bins
    uint32_t v = h[0] + h[1] + h[2] + h[3];
    for (int off = 8; off > 0; off >>= 1) v += __shfl_xor(v, off);   // sixteen lanes = 64 bins
    if ((lane & 15) == 0) gsum[tid >> 4] = v;
    __syncthreads();
    if (tid < 64) {
        uint32_t suf = gsum[lane];                    // S over the groups >= this one
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t o = __shfl_down(suf, off);
            if (lane + off < 64) suf += o;
        }
        uint32_t next = __shfl_down(suf, 1);
        if (lane == 63) next = 0;
        const uint64_t qm = __ballot(suf >= target && next < target);
        if (qm == 0) {                                // S(0) < target
            if (lane == 0) *bin_out = -1;
        } else {
            const int g = __ffsll((unsigned long long)qm) - 1;               // the one group that qualifies
            const uint32_t above_g = __shfl(next, g); // keys in the groups above g
            uint32_t s2 = hist[64 * g + lane];        // suffix inside group g
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t o = __shfl_down(s2, off);
                if (lane + off < 64) s2 += o;
            }
            const uint64_t m2 = __ballot(above_g + s2 >= target);
            const int j = 63 - __clzll((unsigned long long)m2);              // highest qualifying bin
            const uint32_t s2n = __shfl(s2, j < 63 ? j + 1 : j);
            if (lane == 0) {
                *bin_out = 64 * g + j;
                *above_out = above_g + (j < 63 ? s2n : 0u);
            }
        }
    }
    __syncthreads();
}

// Exclusive prefix sum inside a wave of per-lane counts below 2^nbits, bit
// by bit: for each bit a ballot of the lanes that have it, and the lanes
// below this one among them (mbcnt).  No LDS round trip.  Returns the wave
// total.
__device__ __forceinline__ uint32_t wave_scan_bits(uint32_t x, int nbits, uint32_t& excl) {
    uint32_t pre = 0, tot = 0;
    for (int bit = 0; bit < nbits; ++bit) {
        const uint64_t m = __ballot((x >> bit) & 1u);
        pre += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << bit;
        tot += (uint32_t)__popcll(m) << bit;
    }
    excl = pre;
    return tot;
}

// Order keys of the two bf16 scores in a word, both halves at once (the
// unsigned order of the keys is the numeric order of the scores): negative
// scores get every bit flipped, the others the sign bit set.
__device__ __forceinline__ uint32_t order_keys2(uint32_t w) {
    return w ^ (((w >> 15) & 0x00010001u) * 0x7FFFu + 0x80008000u);
}

// Output slots for the marks of a wave: n marks in this lane (n < 64), one
// atomic on the shared counter per wave.  Returns this lane's first slot.
// Every lane of the wave calls it (rounds are uniform across a wave).
__device__ __forceinline__ uint32_t wave_slots(uint32_t n, uint32_t* counter) {
    uint32_t excl;
    const uint32_t tot = wave_scan_bits(n, 7, excl);
    uint32_t base = 0;
    if ((threadIdx.x & 63) == 0 && tot) base = atomicAdd(counter, tot);
    return (uint32_t)__shfl((int)base, 0) + excl;
}

// Exact top-K of one request's bf16 scores (sections 4.2, 5.5), one
// 1024-thread work-group per request, on the 16-bit order key of each score.
// Every pass is branch-free per key (a CU's scalar unit, which executes the
// exec-mask updates of per-key branches, is shared by its 16 waves):
//   1. the order keys of the row into LDS (with its page-table entries) for
//      rows of up to 65536 scores, four 16-byte loads in flight per thread
//      (longer rows re-read the scores in every pass);
//   2. a histogram of the key's top 12 bits (sign, exponent and three
//      mantissa bits: scores of one magnitude spread over eight bins per
//      octave), counted in the pass that copies the keys into LDS;
//   3. the threshold bin b1: fewer than K keys above it, at least K at or
//      above it (one wave, shuffle scans);
//   4. one pass that writes every token whose key lies above b1 and keeps
//      the tokens of b1 with the low 4 bits of their keys in LDS (where the
//      first histogram was);
//   5. a histogram of those low bits, the threshold key T from it, and the
//      tokens of b1: keys above T all, keys equal to T while their slot is
//      below K (any of them).
// Each thread marks its tokens in bit masks; a wave takes output slots for
// all of its marks with one atomic per counter, and each lane writes only
// its marked tokens, ids remapped through the page table.  Rows with
// seq_len <= K emit tokens 0 .. seq_len - 1 and -1 padding without reading
// scores (section 5.2).
__global__ void __launch_bounds__(TOPK_THREADS) indexer_topk_kernel(IndexerParams p) {
    extern __shared__ __attribute__((aligned(16))) uint32_t tk_lds[];
    uint32_t* hist = tk_lds;                                    // [TK_BINS + 64 dummy bins]; later the stash
    uint16_t* keys = (uint16_t*)(tk_lds + TK_HIST);              // [TK_LDS_KEYS]
    int32_t* pt_lds = (int32_t*)(keys + TK_LDS_KEYS);            // [TK_LDS_PAGES]
    __shared__ uint32_t hist2[16];                              // low 4 bits of the keys in b1
    __shared__ uint32_t gsum[64];
    __shared__ int bin_s;
    __shared__ uint32_t above_s, cnt_gt, cnt_eq, cnt_cand;
    const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, K = p.topk;
    const int len = clamp_len(p, r);
    const int32_t* pt = p.page_table + (size_t)r * p.max_pages;
    int32_t* out = p.indices + (size_t)r * K;
    if (len <= K) {
        for (int k = tid; k < K; k += TOPK_THREADS) out[k] = k < len ? phys_id(pt, k, p.num_pages) : -1;
        return;
    }
    const uint16_t* s = p.scores + (size_t)r * p.max_pages * IX_PAGE;
    const u32x4* s16 = (const u32x4*)s;               // rows start on 128-byte boundaries
    const int n_chunks = (len + 7) >> 3;              // 8 scores per 16-byte chunk (inside the row)
    // the body is compiled for rows kept in LDS and for longer ones: in the
    // first no loop holds a global load, whose wait would also wait for the
    // id stores issued before it
    auto body = [&](auto lds_c) {
    constexpr bool in_lds = decltype(lds_c)::value;
    constexpr int BATCH = 4;                          // chunks per thread per round (32 keys)
    const int n_pages = (len + IX_PAGE - 1) / IX_PAGE;
    if (in_lds)
        for (int i = tid; i < n_pages; i += TOPK_THREADS) pt_lds[i] = pt[i];
    for (int i = tid; i < TK_HIST; i += TOPK_THREADS) hist[i] = 0;
    if (tid < 16) hist2[tid] = 0;
    if (tid == 0) { cnt_gt = 0; cnt_eq = 0; cnt_cand = 0; }
    // physical id of token t (page-table entry from LDS when the row is there)
    auto phys = [&](int t) -> int {
        const int pg = in_lds ? pt_lds[t >> 6] : pt[t >> 6];
        return (pg >= 0 && pg < p.num_pages) ? pg * IX_PAGE + (t & 63) : -1;
    };
    // keys of chunk c from raw scores: two per word, 0 for tokens >= len
    auto to_keys = [&](u32x4 v, int c) -> u32x4 {
#pragma unroll
        for (int w = 0; w < 4; ++w) v[w] = order_keys2(v[w]);
        if (8 * c + 8 > len) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int t = 8 * c + 2 * w;
                v[w] = (t < len ? v[w] & 0xFFFFu : 0u) | (t + 1 < len ? v[w] & 0xFFFF0000u : 0u);
            }
        }
        return v;
    };
    // fn(cb, k) for this thread's chunks cb + u * TOPK_THREADS (u < BATCH),
    // k[u] = their keys, loaded BATCH at a time with the loads in flight
    // together (from LDS, or converted from the scores for a row too long to
    // keep).  Rounds are uniform across a wave, so fn may use wave-wide
    // ballots after its per-chunk work; fn skips chunks >= n_chunks.
    auto for_rounds = [&](auto fn) {
        for (int c0 = tid - lane; c0 < n_chunks; c0 += BATCH * TOPK_THREADS) {
            u32x4 k[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int c = c0 + lane + u * TOPK_THREADS;
                k[u] = c < n_chunks ? (in_lds ? *(const u32x4*)(keys + 8 * c) : s16[c]) : u32x4{0u, 0u, 0u, 0u};
            }
            if (!in_lds) {
#pragma unroll
                for (int u = 0; u < BATCH; ++u)
                    if (c0 + lane + u * TOPK_THREADS < n_chunks) k[u] = to_keys(k[u], c0 + lane + u * TOPK_THREADS);
            }
            fn(c0 + lane, k);
        }
    };
    auto key_of = [](const u32x4& k, int e) -> uint32_t { return (k[e >> 1] >> (16 * (e & 1))) & 0xFFFFu; };

    // first digit of one chunk's keys (only the row's last chunk can hold
    // tokens past it: the test is per chunk, so a full chunk costs an extract
    // and an atomic per key)
    auto hist_chunk = [&](const u32x4& k, int c) {
        if (8 * c + 8 <= len) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                atomicAdd(&hist[(k[w] >> 4) & 0xFFFu], 1u);
                atomicAdd(&hist[k[w] >> 20], 1u);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                atomicAdd(&hist[8 * c + e < len ? key_of(k, e) >> 4 : TK_BINS + lane], 1u);
        }
    };
    __syncthreads();                                  // histogram cleared
    // 1 + 2. keys into LDS with their first digit counted on the way (rows
    // kept in LDS), or the first digit from the scores (longer rows)
    if (in_lds) {
        for (int c0 = tid; c0 < n_chunks; c0 += BATCH * TOPK_THREADS) {
            u32x4 v[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u)
                if (c0 + u * TOPK_THREADS < n_chunks) v[u] = s16[c0 + u * TOPK_THREADS];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int c = c0 + u * TOPK_THREADS;
                if (c < n_chunks) {
                    const u32x4 k = to_keys(v[u], c);
                    *(u32x4*)(keys + 8 * c) = k;
                    hist_chunk(k, c);
                }
            }
        }
    } else {
        for_rounds([&](int cb, u32x4* k) {
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int c = cb + u * TOPK_THREADS;
                if (c >= n_chunks) break;
                hist_chunk(k[u], c);
            }
        });
    }
    __syncthreads();
    // 3. threshold bin (exists: len > K)
    find_threshold_bin(hist, (uint32_t)K, gsum, &bin_s, &above_s);
    const uint32_t b1 = (uint32_t)bin_s, above1 = above_s;
    const uint32_t in_b1 = hist[b1];
    __syncthreads();                                  // hist is the stash from here on
    const bool stash = in_b1 <= (uint32_t)TK_HIST;
    uint32_t* cand = hist;                            // (token << 4) | low 4 bits of its key
    // the key of token t (from LDS, or from the scores for long rows)
    auto key_at = [&](int t) -> uint32_t { return in_lds ? keys[t] : order_key(s[t]); };
    // 4. the tokens above b1 out; those in b1 to the stash
    // digit above b1 <=> key >= (b1 + 1) * 16; digit >= b1 <=> key >= b1 * 16
    const uint32_t thr_gt = (b1 + 1u) << 4, thr_ge = b1 << 4;
    for_rounds([&](int cb, u32x4* k) {
        uint32_t mup = 0, mge = 0;                    // bit 8 u + e: key e of round chunk u
#pragma unroll
        for (int u = BATCH - 1; u >= 0; --u) {        // bits shifted in from the top
            const int c = cb + u * TOPK_THREADS;
            if (8 * c + 8 <= len) {
#pragma unroll
                for (int e = 7; e >= 0; --e) {
                    const uint32_t key = key_of(k[u], e);
                    mup = (mup << 1) | (uint32_t)(key >= thr_gt);
                    mge = (mge << 1) | (uint32_t)(key >= thr_ge);
                }
            } else {                                  // the row's last chunk, or past the row
#pragma unroll
                for (int e = 7; e >= 0; --e) {
                    const uint32_t key = key_of(k[u], e);
                    const bool ok = 8 * c + e < len;
                    mup = (mup << 1) | (uint32_t)(ok && key >= thr_gt);
                    mge = (mge << 1) | (uint32_t)(ok && key >= thr_ge);
                }
            }
        }
        uint32_t mb1 = mge & ~mup;
        uint32_t o = wave_slots((uint32_t)__popc(mup), &cnt_gt);
        while (mup) {
            const int i = __ffs(mup) - 1;
            mup &= mup - 1;
            out[o++] = phys(8 * (cb + (i >> 3) * TOPK_THREADS) + (i & 7));
        }
        if (stash) {
            uint32_t sl = wave_slots((uint32_t)__popc(mb1), &cnt_cand);
            while (mb1) {
                const int i = __ffs(mb1) - 1;
                mb1 &= mb1 - 1;
                const int t = 8 * (cb + (i >> 3) * TOPK_THREADS) + (i & 7);
                cand[sl++] = ((uint32_t)t << 4) | (key_at(t) & 15u);
            }
        }
    });
    __syncthreads();
    // 5. the low-bit histogram of b1 (from the stash, or the keys again), the
    // threshold key T = (b1 << 4) | lo and the tokens of b1
    if (stash) {
        for (int i = tid; i < (int)in_b1; i += TOPK_THREADS) atomicAdd(&hist2[cand[i] & 15u], 1u);
    } else {
        for (int t = tid; t < len; t += TOPK_THREADS) {
            const uint32_t key = key_at(t);
            if ((key >> 4) == b1) atomicAdd(&hist2[key & 15u], 1u);
        }
    }
    __syncthreads();
    if (tid == 0) {
        const uint32_t need = (uint32_t)K - above1;
        uint32_t acc = 0;
        int lo = 15;
        for (; lo > 0; --lo) {
            if (acc + hist2[lo] >= need) break;
            acc += hist2[lo];
        }
        bin_s = lo;
        above_s = acc;                                // keys of b1 above T
    }
    __syncthreads();
    const uint32_t lo = (uint32_t)bin_s, n_gt = above1 + above_s, take_eq = (uint32_t)K - n_gt;
    // a token of b1 with low bits x: above T (out after the above1 written), or
    // equal (slot n_gt + its rank among the equal ones, below K)
    auto take_b1 = [&](uint32_t mgt, uint32_t meq, auto token_of) {
        uint32_t o = wave_slots((uint32_t)__popc(mgt), &cnt_gt);
        uint32_t q = wave_slots((uint32_t)__popc(meq), &cnt_eq);
        while (mgt) {
            const int i = __ffs(mgt) - 1;
            mgt &= mgt - 1;
            out[o++] = phys(token_of(i));
        }
        while (meq) {
            const int i = __ffs(meq) - 1;
            meq &= meq - 1;
            if (q < take_eq) out[n_gt + q] = phys(token_of(i));
            ++q;
        }
    };
    if (stash) {
        const int n_cand = (int)in_b1;
        for (int i0 = tid - lane; i0 < n_cand; i0 += BATCH * TOPK_THREADS) {
            uint32_t mgt = 0, meq = 0, e[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int i = i0 + lane + u * TOPK_THREADS;
                e[u] = i < n_cand ? cand[i] : 0u;
                mgt |= (uint32_t)(i < n_cand && (e[u] & 15u) > lo) << u;
                meq |= (uint32_t)(i < n_cand && (e[u] & 15u) == lo) << u;
            }
            take_b1(mgt, meq, [&](int u) { return (int)(e[u] >> 4); });
        }
    } else {                                          // more tokens in b1 than the stash holds
        for_rounds([&](int cb, u32x4* k) {
            uint32_t mgt = 0, meq = 0;
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int c = cb + u * TOPK_THREADS;
                if (c >= n_chunks) break;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t key = key_of(k[u], e);
                    const bool in = 8 * c + e < len && (key >> 4) == b1;
                    mgt |= (uint32_t)(in && (key & 15u) > lo) << (8 * u + e);
                    meq |= (uint32_t)(in && (key & 15u) == lo) << (8 * u + e);
                }
            }
            take_b1(mgt, meq, [&](int i) { return 8 * (cb + (i >> 3) * TOPK_THREADS) + (i & 7); });
        });
    }
    };
    if (len <= TK_LDS_KEYS) body(std::integral_constant<bool, true>{});
    else body(std::integral_constant<bool, false>{});
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
    static bool lds_allowed = false;                 // the keys of a row live in dynamic LDS (144 KB)
    if (!lds_allowed) {
        const hipError_t e = hipFuncSetAttribute((const void*)indexer_topk_kernel,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, TK_LDS_BYTES);
        if (e != hipSuccess) return e;
        lds_allowed = true;
    }
    hipLaunchKernelGGL(indexer_topk_kernel, dim3(p.b), dim3(TOPK_THREADS), TK_LDS_BYTES, st, p);
    return hipGetLastError();
}

}  // namespace mla
