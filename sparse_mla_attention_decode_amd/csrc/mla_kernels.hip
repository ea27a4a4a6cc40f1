// gfx950 kernels for sparse MLA attention: the tile scheduler, the decode and
// split-KV combine over the flat bf16 cache (sparse prefill), and a
// gather test hook.  (The FP8 656-byte cache has its own kernels in
// decode_h128.hip.)
//
// Decode work-group = NW waves of 64 lanes; wave w owns query heads
// [32w, 32w+32).  Each wave keeps Q for its heads in VGPRs (the B operand of
// the score contraction) and the transposed output accumulator O^T [512 x 32]
// in AGPRs.  The work-group walks its topk slots in tiles of 32 keys:
//
//   1. gather: the tile's 1152-byte bf16 token rows are copied HBM -> LDS by
//      direct-to-LDS loads (16 B per lane, no registers), one tile ahead of
//      the compute; empty slots are skipped;
//   2. stage: rows are copied into padded K rows [32 keys][576] in LDS;
//      empty slots become zero rows;
//   3. S^T[key][head] = K Q^T: 36 MFMA 32x32x16 bf16 per wave;
//   4. softmax in base 2 on the accumulator, masked by slot validity; every
//      lane holds 16 keys of one head so the row max needs one exchange;
//   5. O^T[dim][head] += V^T P^T: 32 MFMA per wave; P comes straight from
//      the score accumulator (its layout is the B layout) and V^T fragments
//      are read from the K rows with the LDS transpose read.
//
// The reference max of a piece is the max score of its first tile holding a
// valid key; later tiles are accumulated against it as long as no score
// exceeds it by more than 2^64 (so p <= 2^64 and all sums stay finite in
// fp32).  If one does, the piece is recomputed with the larger reference --
// equal to the exact online-softmax result, without rescaling O in place.
//
// Sources: "FlashMLA Sparse Decode 完整计算过程详解" steps 3 (scheduler), 7
// (index load, address, dequant), 8-11 (contractions, base-2 softmax with
// c = sm_scale*log2(e)), 12 and 14 (epilogue: out = O/l, lse = ln l + m/log2(e),
// +inf when l = 0; split partials O/l in fp32 and lse = log2 l + m, -inf when
// l = 0) and 16 (combine).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "mla_internal.h"
#include "sched_plan.h"

namespace mla {

constexpr int KROW = 1168;                 // LDS bytes per staged bf16 K row (1152 + 16 pad)
constexpr int KB_BYTES = TILE * KROW;      // 37376

// Per-format constants of the raw token row.  The generic kernels serve the
// bf16 cache (sparse prefill); the FP8 656-byte cache has its own kernels
// (decode_h128.hip).
template <int FMT> struct RowFmt;
template <> struct RowFmt<MLA_KV_BF16_576> {
    static constexpr int ROWB = 1152, ROPE_OFF = 1024;
};

// LDS map: [NRAW raw tiles][2 staged K-row tiles][validity masks][4 restart flags].
// Raw tiles are padded so every wave issues the same number of 1 KB
// direct-to-LDS copies per tile (exact vmcnt accounting).
template <int FMT, int NW> struct Lds {
    static constexpr int CPR = RowFmt<FMT>::ROWB / 16;                 // 16-byte chunks per row
    static constexpr int CHUNKS = TILE * CPR;                          // per tile
    static constexpr int NI = ((CHUNKS + 63) / 64 + NW - 1) / NW;      // copies per wave per tile
    static constexpr int RAW_BYTES = NI * NW * 1024;
    static constexpr int NRAW = 2;
    static constexpr int RAW = 0;
    static constexpr int KB = RAW + NRAW * RAW_BYTES;
    static constexpr int MASK = KB + 2 * KB_BYTES;                      // 4 slots
    static constexpr int FLAGS = MASK + 16;
    static constexpr int BYTES = FLAGS + 16;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};



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
// decode
// ----------------------------------------------------------------------------
// Address of token t (bytes) or nullptr when the slot is empty.
template <int FMT>
__device__ __forceinline__ const uint8_t* row_ptr(const DecodeParams& p, int t) {
    if (t < 0 || (int64_t)t >= p.n_tok) return nullptr;
    return p.kv + (int64_t)t * p.kv_block_stride;
}


// Row address (as two dwords) of slot `key` of the piece for lanes 0..31; slots
// that are empty, beyond k_end, or outside the cache get the cache base (a
// harmless dummy source whose staged row is zeroed).  Returns the validity
// bit of this lane's slot.
template <int FMT>
__device__ __forceinline__ bool slot_address(const DecodeParams& p, int t, bool in_range,
                                             uint32_t& lo, uint32_t& hi) {
    const uint8_t* rp = in_range ? row_ptr<FMT>(p, t) : nullptr;
    const uint64_t a = (uint64_t)(uintptr_t)(rp ? rp : p.kv);
    lo = (uint32_t)a;
    hi = (uint32_t)(a >> 32);
    return rp != nullptr;
}

// Gather: start the HBM -> LDS copy of the 32 rows of one tile into a raw
// buffer.  `t` holds (lanes 0..31) the token ids of the tile's slots, or -1.
// Every wave issues exactly NI 1 KB copies with all lanes active (padding
// chunks re-read row 0 of the tile into the buffer's padding), so the number
// of outstanding memory operations is the same in every iteration.  Thread 0
// records the tile's validity mask in mask slot `ms`.
template <int FMT, int NW>
__device__ __forceinline__ void gather_tile(const DecodeParams& p, int t, bool in_range,
                                            LDS_AS uint8_t* lds, int raw_off, int ms) {
    using L = Lds<FMT, NW>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t a_lo, a_hi;
    const bool ok = slot_address<FMT>(p, t, in_range && lane < 32, a_lo, a_hi);
    const uint64_t valid = __ballot(ok);
    if (threadIdx.x == 0) *(LDS_AS uint32_t*)(lds + L::MASK + 4 * ms) = (uint32_t)valid;
    const uint8_t* src[L::NI];
#pragma unroll
    for (int i = 0; i < L::NI; ++i) {
        const int f = 64 * (wave + NW * i) + lane;   // chunk index in the tile
        const int row = f < L::CHUNKS ? f / L::CPR : 0;
        const int chunk = f < L::CHUNKS ? f - row * L::CPR : 0;
        const uint32_t lo = __shfl(a_lo, row), hi = __shfl(a_hi, row);
        src[i] = (const uint8_t*)(((uint64_t)hi << 32) | lo) + 16 * chunk;
    }
    // LDS byte address of the wave's first 1 KB block (wave-uniform, so an SGPR)
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds + raw_off) + 1024u * wave;
#pragma unroll
    for (int i = 0; i < L::NI; ++i)
        dma16(src[i], __builtin_amdgcn_readfirstlane(lds_base + 1024u * NW * i));
}

// Stage: raw rows -> K rows (NoPE and RoPE copied into the padded row
// layout), branch free; empty slots become zero rows.  Split into a read half
// and a write half so the decode loop can spread it between MFMAs.
template <int FMT, int NW> struct StageRegs {
    static constexpr int NT = NW * 64;
    static constexpr int NOPE_UNITS = 32 * 64 / NT;
    static constexpr int ROPE_UNITS = (32 * 8 + NT - 1) / NT;
    u32x4 nope[NOPE_UNITS];
    u32x4 rope[ROPE_UNITS];
};

template <int FMT, int NW>
__device__ __forceinline__ void stage_read(const LDS_AS uint8_t* lds, int raw_off, StageRegs<FMT, NW>& R,
                                           int i0 = 0, int i1 = StageRegs<FMT, NW>::NOPE_UNITS + 1) {
    using SR = StageRegs<FMT, NW>;
    constexpr int ROWB = RowFmt<FMT>::ROWB;
#pragma unroll
    for (int i = i0; i < min(i1, SR::NOPE_UNITS); ++i) {
        const int u = i * SR::NT + threadIdx.x;
        const int row = u >> 6, c = u & 63;
        R.nope[i] = lds_read16(lds, raw_off + row * ROWB + 16 * c);
    }
    if (i1 <= SR::NOPE_UNITS) return;
#pragma unroll
    for (int i = 0; i < SR::ROPE_UNITS; ++i) {
        const int u = min(i * SR::NT + (int)threadIdx.x, 255);
        R.rope[i] = lds_read16(lds, raw_off + (u >> 3) * ROWB + RowFmt<FMT>::ROPE_OFF + 16 * (u & 7));
    }
}

// write NoPE unit i (or the RoPE units when i == NOPE_UNITS)
template <int FMT, int NW>
__device__ __forceinline__ void stage_write(LDS_AS uint8_t* lds, int kb_off, uint32_t valid,
                                            const StageRegs<FMT, NW>& R, int i) {
    using SR = StageRegs<FMT, NW>;
    const u32x4 zero = {0, 0, 0, 0};
    if (i < SR::NOPE_UNITS) {
        const int u = i * SR::NT + threadIdx.x;
        const int row = u >> 6, c = u & 63;
        lds_write16(lds, kb_off + row * KROW + 16 * c, ((valid >> row) & 1u) ? R.nope[i] : zero);
    } else {
#pragma unroll
        for (int r = 0; r < SR::ROPE_UNITS; ++r) {
            const int u = r * SR::NT + threadIdx.x;
            if (SR::NT * SR::ROPE_UNITS == 256 || u < 256) {
                const int row = u >> 3, c = u & 7;
                lds_write16(lds, kb_off + row * KROW + 1024 + 16 * c, ((valid >> row) & 1u) ? R.rope[r] : zero);
            }
        }
    }
}

template <int FMT, int NW>
__device__ __forceinline__ void stage_tile(LDS_AS uint8_t* lds, int raw_off, int kb_off, uint32_t valid) {
    StageRegs<FMT, NW> R;
    stage_read<FMT, NW>(lds, raw_off, R);
#pragma unroll
    for (int i = 0; i <= StageRegs<FMT, NW>::NOPE_UNITS; ++i) stage_write<FMT, NW>(lds, kb_off, valid, R, i);
}

// Byte offset (relative to a staged K-row tile) of this lane's transposing
// read for the value contraction: output block mb (dims 32mb..32mb+31),
// k-step t, half `second` (keys +8).  Lane l feeds the 8-byte row of key
// 16t + 4(l/32) + (l%16)/4 (+8) at dims 32mb + 16((l/16)%2) + 4(l%4); the
// transpose hands lane l dim 32mb + l%32 of keys 16t + 4(l/32) + 0..3 (+8),
// which is the key order the score accumulator gives P.
__device__ __forceinline__ int pv_read_base(int lane) {
    const int key = 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    return key * KROW + 2 * dim;
}


template <int FMT, int NW>
__global__ void __launch_bounds__(NW * 64, 1) decode_kernel(DecodeParams p) {
    using L = Lds<FMT, NW>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
    LDS_AS uint8_t* lds = (LDS_AS uint8_t*)lds_raw;

    const int part = blockIdx.x, sq = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 31, h = lane >> 5;
    const int head = 32 * wave + n;

    const PartPlan plan = plan_part(p, part);
    const int begin_req = plan.begin_req;
    if (begin_req >= p.b) return;
    const int end_req = plan.end_req, begin_block = plan.begin_block, end_block = plan.end_block;
    const int begin_split = plan.begin_split;
    if (plan.by_length && p.topk_length == nullptr) return;   // contract error: see lengths_missing
    const int qk_base = n * KROW + 16 * h;          // score operand: key n, dims 16j + 8h
    const int pv_base = pv_read_base(lane);
    if (threadIdx.x < 4) lds[L::FLAGS + threadIdx.x] = 0;   // ordered by the first barrier

    for (int req = begin_req; req <= end_req; ++req) {
        const int blk_lo = req == begin_req ? begin_block : 0;
        const int blk_hi = req == end_req ? end_block : whole_blocks(p, plan, req);
        const int k_lo = blk_lo * p.block;
        const int k_hi = min(blk_hi * p.block, p.topk);
        const int n_tiles = (k_hi - k_lo + TILE - 1) / TILE;
        const int32_t* idx = p.indices + (int64_t)req * p.idx_sb + (int64_t)sq * p.idx_ss;
        // raw token ids of slots k0 + lane (lanes 0..31); the load address is
        // clamped so the load is always issued (fixed vmcnt accounting) and
        // slots past the piece are masked where the ids are used
        auto load_ids = [&](int tile) -> int {
            const int k = k_lo + tile * TILE + (lane & 31);
            return idx[min(k, k_hi - 1)];
        };
        // slots past the request's valid length (topk_length) are empty too
        const int k_ok = p.topk_length ? min(k_hi, max(p.topk_length[req], 0)) : k_hi;
        auto ids_in_range = [&](int tile) -> bool {
            return tile < n_tiles && k_lo + tile * TILE + (lane & 31) < k_ok;
        };

        // Q for this wave's heads as B operands: k-step j covers dims
        // 16j + 8h .. 16j + 8h + 7, matching the K row reads
        bf16x8 qb[36];
        {
            const uint16_t* qrow = p.q + (int64_t)req * p.q_sb + (int64_t)sq * p.q_ss +
                                   (int64_t)head * p.q_sh;
#pragma unroll
            for (int j = 0; j < 36; ++j)
                qb[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * j + 8 * h));
        }

        f32x16 O[16];
        float m_ref = INIT_MAX, m_seen = -INFINITY, l_part = 0.f;
        for (int pass = 0;; ++pass) {
#pragma unroll
            for (int mb = 0; mb < 16; ++mb) O[mb] = f32x16{};
            l_part = 0.f;
            __syncthreads();                        // LDS free (previous piece / pass done)

            // prologue: tiles 0 and 1 in flight, ids of tiles 2 and 3 loaded
            const int ids0 = load_ids(0), ids1 = load_ids(1);
            gather_tile<FMT, NW>(p, ids0, ids_in_range(0), lds, L::RAW, 0);
            gather_tile<FMT, NW>(p, ids1, ids_in_range(1), lds, L::RAW + L::RAW_BYTES, 1);
            int ids_a = load_ids(2), ids_b = load_ids(3);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            stage_tile<FMT, NW>(lds, L::RAW, L::KB, *(const LDS_AS uint32_t*)(lds + L::MASK));
            __syncthreads();

            for (int it = 0; it < n_tiles; ++it) {
                const int kb_cur = L::KB + (it & 1) * KB_BYTES;
                const uint32_t vmask = *(const LDS_AS uint32_t*)(lds + L::MASK + 4 * (it & 3));
                // ---- start tile it+2 (ids loaded two iterations ago) and the ids of it+4
                // The id load goes first: vmcnt is in order, so a later wait on
                // these ids only forces copies older than them, never tile it+2.
                const int ids_new = load_ids(it + 4);
                gather_tile<FMT, NW>(p, ids_a, ids_in_range(it + 2), lds,
                                     L::RAW + ((it + 2) % L::NRAW) * L::RAW_BYTES, (it + 2) & 3);
                ids_a = ids_b;
                ids_b = ids_new;

                // ---- S^T = K Q^T, with the staging of tile it+1 spread between
                // the MFMAs (the raw rows of tile it+1 landed before the last barrier)
                StageRegs<FMT, NW> R;
                const int raw_next = L::RAW + ((it + 1) % L::NRAW) * L::RAW_BYTES;
                const int kb_next = L::KB + ((it + 1) & 1) * KB_BYTES;
                const uint32_t vmask_next = *(const LDS_AS uint32_t*)(lds + L::MASK + 4 * ((it + 1) & 3));
                constexpr int NSTAGE = StageRegs<FMT, NW>::NOPE_UNITS + 1;   // units incl. RoPE
                constexpr int SPAN = 36 / NSTAGE > 1 ? 36 / NSTAGE : 1;        // MFMAs per unit
                stage_read<FMT, NW>(lds, raw_next, R, 0, 1);
                // two alternating accumulator chains: the score MFMAs are inline
                // asm (register classes pinned), which the compiler's hazard
                // checks do not see into, so no MFMA may take the result of the
                // one issued right before it
                f32x16 Sa, Sb;
                {
                    constexpr int AHEAD = 2;
                    bf16x8 a[AHEAD];
#pragma unroll
                    for (int j = 0; j < AHEAD; ++j)
                        a[j] = __builtin_bit_cast(bf16x8, lds_read16(lds, kb_cur + qk_base + 32 * j));
#pragma unroll
                    for (int j = 0; j < 36; ++j) {
                        const bf16x8 cur = a[j % AHEAD];
                        if (j + AHEAD < 36)
                            a[j % AHEAD] = __builtin_bit_cast(bf16x8, lds_read16(lds, kb_cur + qk_base + 32 * (j + AHEAD)));
                        if (j == 0) mfma_qk_first(Sa, cur, qb[j]);
                        else if (j == 1) mfma_qk_first(Sb, cur, qb[j]);
                        else if (j & 1) mfma_qk(Sb, cur, qb[j]);
                        else mfma_qk(Sa, cur, qb[j]);
                        // staging unit u is read at MFMA SPAN*u - SPAN/2 and written at SPAN*u + SPAN-1
                        if (j % SPAN == SPAN / 2 && j / SPAN + 1 < NSTAGE)
                            stage_read<FMT, NW>(lds, raw_next, R, j / SPAN + 1, j / SPAN + 2);
                        if (j % SPAN == SPAN - 1 && j / SPAN < NSTAGE)
                            stage_write<FMT, NW>(lds, kb_next, vmask_next, R, j / SPAN);
                    }
#pragma unroll
                    for (int i = 36 / SPAN; i < NSTAGE; ++i) {
                        stage_read<FMT, NW>(lds, raw_next, R, i, i + 1);
                        stage_write<FMT, NW>(lds, kb_next, vmask_next, R, i);
                    }
                }
                mfma_result_fence2(Sa, Sb);
                f32x16 S = Sa + Sb;

                // ---- masked softmax in base 2 against the reference max
                float mx = -INFINITY;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = 8 * (v >> 2) + 4 * h + (v & 3);
                    S[v] = ((vmask >> key) & 1u) ? S[v] : -INFINITY;
                    mx = fmaxf(mx, S[v]);
                }
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float mnew = mx * p.c;
                m_seen = fmaxf(m_seen, mnew);
                if (m_ref == INIT_MAX && mnew > -INFINITY) m_ref = mnew;   // O, l still zero
                if (__any(mnew > m_ref + p.threshold) && lane == 0) lds[L::FLAGS + wave] = 1;

                float psum = 0.f;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    S[v] = __builtin_amdgcn_exp2f(S[v] * p.c - m_ref);
                    psum += S[v];
                }
                l_part += psum;
                bf16x8 pb[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    u32x4 w = {pack_bf16(S[8 * t + 0], S[8 * t + 1]), pack_bf16(S[8 * t + 2], S[8 * t + 3]),
                               pack_bf16(S[8 * t + 4], S[8 * t + 5]), pack_bf16(S[8 * t + 6], S[8 * t + 7])};
                    pb[t] = __builtin_bit_cast(bf16x8, w);
                }

                // ---- O^T += V^T P^T
                valu_to_mfma_fence(pb[0], pb[1]);
                {
                    constexpr int AHEAD = 2;
                    auto vread = [&](int st) {          // step st = (block st/2, k-step st%2)
                        const int off = kb_cur + pv_base + (st & 1) * 16 * KROW + (st >> 1) * 64;
                        const u32x2 r0 = lds_read_tr16(lds, off);
                        const u32x2 r1 = lds_read_tr16(lds, off + 8 * KROW);
                        return __builtin_bit_cast(bf16x8, u32x4{r0[0], r0[1], r1[0], r1[1]});
                    };
                    bf16x8 a[AHEAD];
#pragma unroll
                    for (int st = 0; st < AHEAD; ++st) a[st] = vread(st);
#pragma unroll
                    for (int st = 0; st < 32; ++st) {
                        const bf16x8 cur = a[st % AHEAD];
                        if (st + AHEAD < 32) a[st % AHEAD] = vread(st + AHEAD);
                        mfma_pv(O[st >> 1], cur, pb[st & 1]);
                    }
                }
                // tile it+2 (the last memory operations issued) must have landed
                // before it is staged in the next iteration
                wait_vmcnt<0>();
                __syncthreads();
            }
            // A score exceeded the reference by more than 2^threshold in some
            // wave: recompute the piece against the true max (rare).
            const uint32_t flags = *(const LDS_AS uint32_t*)(lds + L::FLAGS);
            __syncthreads();
            if (flags == 0u || pass > 0) break;          // the second pass uses the true max
            if (threadIdx.x < 4) lds[L::FLAGS + threadIdx.x] = 0;
            m_ref = m_seen;
        }

        // ---- epilogue
#pragma unroll
        for (int mb = 0; mb < 16; ++mb) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+a"(O[mb]));
        const float l_tot = l_part + __shfl_xor(l_part, 32);
        const int first_split = split_prefix(p, req);
        const int nsplit = split_prefix(p, req + 1) - first_split;
        // the final output of an unsplit request takes the attention sink as an
        // extra exp-sum term 2^(sink log2(e) - m) (split requests: in the combine)
        const float den = nsplit == 1 && p.attn_sink != nullptr
                              ? l_tot + __builtin_amdgcn_exp2f(p.attn_sink[head] * 1.4426950408889634f - m_ref)
                              : l_tot;
        const float inv = l_tot == 0.f ? 0.f : 1.0f / den;     // a NaN sum (NaN in the cache) stays NaN
        if (nsplit == 1) {
            uint16_t* orow = p.out + (int64_t)req * p.out_sb + (int64_t)sq * p.out_ss +
                             (int64_t)head * p.out_sh;
#pragma unroll
            for (int mb = 0; mb < 16; ++mb) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = 32 * mb + 8 * g + 4 * h;
                    u32x2 w = {pack_bf16(O[mb][4 * g] * inv, O[mb][4 * g + 1] * inv),
                               pack_bf16(O[mb][4 * g + 2] * inv, O[mb][4 * g + 3] * inv)};
                    *(u32x2*)(orow + d) = w;
                }
            }
            if (h == 0)
                p.lse[((int64_t)req * p.h_q + head) * p.s_q + sq] =
                    l_tot == 0.f ? INFINITY : (__log2f(l_tot) + m_ref) * 0.69314718055994531f;
        } else {
            const int split = req == begin_req ? begin_split : first_split;
            const int64_t base = ((int64_t)split * p.s_q + sq) * p.h_q + head;
            float* orow = p.o_accum + base * 512;
#pragma unroll
            for (int mb = 0; mb < 16; ++mb) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = 32 * mb + 8 * g + 4 * h;
                    *(f32x4*)(orow + d) = f32x4{O[mb][4 * g] * inv, O[mb][4 * g + 1] * inv,
                                                O[mb][4 * g + 2] * inv, O[mb][4 * g + 3] * inv};
                }
            }
            if (h == 0) p.lse_accum[base] = l_tot == 0.f ? -INFINITY : __log2f(l_tot) + m_ref;
        }
    }
}

// ----------------------------------------------------------------------------
// gather/dequant test hook: gathers and stages every tile exactly as decode
// does and reads the staged rows back through the decode kernel's two operand
// read paths (row reads for K, transposing reads for V).
// ----------------------------------------------------------------------------
template <int FMT, int NW>
__global__ void __launch_bounds__(NW * 64, 1) gather_kernel(DecodeParams p, uint16_t* k_rows,
                                                            uint16_t* v_rows) {
    using L = Lds<FMT, NW>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
    LDS_AS uint8_t* lds = (LDS_AS uint8_t*)lds_raw;
    const int qi = blockIdx.x;                    // query token = req * s_q + sq
    const int req = qi / p.s_q, sq = qi % p.s_q;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 31, h = lane >> 5;
    const int32_t* idx = p.indices + (int64_t)req * p.idx_sb + (int64_t)sq * p.idx_ss;
    const int n_tiles = (p.topk + TILE - 1) / TILE;
    for (int it = 0; it < n_tiles; ++it) {
        const int k0 = it * TILE;
        const int k = k0 + (lane & 31);
        const int t = idx[min(k, p.topk - 1)];
        __syncthreads();
        gather_tile<FMT, NW>(p, t, k < p.topk, lds, L::RAW, 0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        stage_tile<FMT, NW>(lds, L::RAW, L::KB, *(const LDS_AS uint32_t*)(lds + L::MASK));
        __syncthreads();
        if (wave == 0) {
            const int key = k0 + n;
            if (key < p.topk) {
                uint16_t* dst = k_rows + ((int64_t)qi * p.topk + key) * 576;
                for (int j = 0; j < 36; ++j)
                    *(u32x4*)(dst + 16 * j + 8 * h) = lds_read16(lds, L::KB + n * KROW + 16 * h + 32 * j);
            }
        }
        if (v_rows != nullptr && wave == NW - 1) {
            const int pv_base = pv_read_base(lane);
            for (int mb = 0; mb < 16; ++mb) {
                for (int tt = 0; tt < 2; ++tt) {
                    const int off = L::KB + pv_base + tt * 16 * KROW + mb * 64;
                    const u32x2 r0 = lds_read_tr16(lds, off);
                    const u32x2 r1 = lds_read_tr16(lds, off + 8 * KROW);
                    const uint32_t d[4] = {r0[0], r0[1], r1[0], r1[1]};
                    for (int e = 0; e < 8; ++e) {
                        const int key = k0 + 16 * tt + 8 * (e >> 2) + 4 * h + (e & 3);
                        if (key < p.topk) {
                            const uint16_t val = (uint16_t)(d[e >> 1] >> (16 * (e & 1)));
                            v_rows[((int64_t)qi * p.topk + key) * 512 + 32 * mb + n] = val;
                        }
                    }
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------
// combine: one wave per (query token, head); lanes own 8 output dims each.
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(256) combine_kernel(DecodeParams p) {
    const int qi = blockIdx.x;
    const int req = qi / p.s_q, sq = qi % p.s_q;
    const int lane = threadIdx.x & 63;
    const int head = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (head >= p.h_q) return;
    const int first = split_prefix(p, req);
    const int ns = split_prefix(p, req + 1) - first;
    bool poison = lengths_missing(p);                       // contract error: NaN everywhere
    if (ns <= 1 && !poison) return;
    auto lse_at = [&](int j) {
        return p.lse_accum[((int64_t)(first + j) * p.s_q + sq) * p.h_q + head];
    };
    // a split whose lse is NaN (NaN in the cache) makes the output NaN
    bool nan_lse = false;
    for (int j = lane; j < (poison ? 0 : ns); j += 64) nan_lse |= lse_at(j) != lse_at(j);
    poison = poison || __any(nan_lse);
    uint16_t* orow = p.out + (int64_t)req * p.out_sb + (int64_t)sq * p.out_ss + (int64_t)head * p.out_sh;
    float* lse_out = p.lse + ((int64_t)req * p.h_q + head) * p.s_q + sq;
    if (poison) {
        *(u32x4*)(orow + 8 * lane) = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
        if (lane == 0) *lse_out = __builtin_nanf("");
        return;
    }
    float mx = -INFINITY;
    for (int j = lane; j < ns; j += 64) mx = fmaxf(mx, lse_at(j));
    mx = wave_max(mx);
    if (mx == -INFINITY) {
        *(u32x4*)(orow + 8 * lane) = u32x4{0, 0, 0, 0};
        if (lane == 0) *lse_out = INFINITY;
        return;
    }
    float tot = 0.f;
    for (int j = lane; j < ns; j += 64) tot += __builtin_amdgcn_exp2f(lse_at(j) - mx);
    tot = wave_sum(tot);
    // an attention sink adds 2^(sink log2(e) - mx) to the exp-sum; lse keeps
    // the real slots only
    const float den = p.attn_sink != nullptr
                          ? tot + __builtin_amdgcn_exp2f(p.attn_sink[head] * 1.4426950408889634f - mx)
                          : tot;
    const float inv = 1.0f / den;
    f32x4 a0 = {}, a1 = {};
    for (int j = 0; j < ns; ++j) {
        const float w = __builtin_amdgcn_exp2f(lse_at(j) - mx) * inv;
        const float* src = p.o_accum + (((int64_t)(first + j) * p.s_q + sq) * p.h_q + head) * 512 + 8 * lane;
        a0 += w * *(const f32x4*)src;
        a1 += w * *(const f32x4*)(src + 4);
    }
    *(u32x4*)(orow + 8 * lane) = u32x4{pack_bf16(a0[0], a0[1]), pack_bf16(a0[2], a0[3]),
                                       pack_bf16(a1[0], a1[1]), pack_bf16(a1[2], a1[3])};
    if (lane == 0) *lse_out = (mx + __log2f(tot)) * 0.69314718055994531f;
}


// ----------------------------------------------------------------------------
// launchers
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

template <typename K>
static hipError_t allow_lds(K k, int bytes, bool& done) {
    if (done) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done = true;
    return e;
}

template <int FMT, int NW>
static hipError_t launch_decode_t(const DecodeParams& p, int num_parts, hipStream_t st) {
    auto k = decode_kernel<FMT, NW>;
    static bool done = false;
    constexpr int bytes = Lds<FMT, NW>::BYTES;
    hipError_t e = allow_lds(k, bytes, done);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(num_parts, p.s_q), dim3(NW * 64), bytes, st, p);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int kv_format, int num_parts, hipStream_t st) {
    if (kv_format != MLA_KV_BF16_576)                  // the 656-byte, V4 and V4.1 FP8 caches
        return launch_decode_fp8_h128(p, kv_format, num_parts, st);
    return p.h_q == 128 ? launch_decode_t<MLA_KV_BF16_576, 4>(p, num_parts, st)
                        : launch_decode_t<MLA_KV_BF16_576, 2>(p, num_parts, st);
}

template <int FMT>
static hipError_t launch_gather_t(const DecodeParams& p, uint16_t* k_rows, uint16_t* v_rows,
                                  hipStream_t st) {
    auto k = gather_kernel<FMT, 4>;
    static bool done = false;
    constexpr int bytes = Lds<FMT, 4>::BYTES;
    hipError_t e = allow_lds(k, bytes, done);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(p.b * p.s_q), dim3(256), bytes, st, p, k_rows, v_rows);
    return hipGetLastError();
}

hipError_t launch_gather(const DecodeParams& p, int kv_format, uint16_t* k_rows, uint16_t* v_rows,
                         hipStream_t st) {
    // the FP8 decode kernel serves 64 and 128 heads; its gather does not depend on h_q
    if (kv_format == MLA_KV_FP8_656) return launch_gather_fp8_h128(p, k_rows, v_rows, st);
    if (kv_format != MLA_KV_BF16_576) return hipErrorNotSupported;    // checked on the host first
    return launch_gather_t<MLA_KV_BF16_576>(p, k_rows, v_rows, st);
}

hipError_t launch_combine(const DecodeParams& p, hipStream_t st) {
    // the 128-head FP8 decode writes packed bf16 partials (decode_h128.hip)
    if (p.packed_partials) return launch_combine_packed(p, st);
    hipLaunchKernelGGL(combine_kernel, dim3(p.b * p.s_q, (p.h_q + 3) / 4), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace mla
