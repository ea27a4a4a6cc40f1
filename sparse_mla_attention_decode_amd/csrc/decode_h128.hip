// gfx950 sparse MLA decode for 128 or 64 query heads over the FP8 656-byte
// token cache ("FlashMLA Sparse Decode 完整计算过程详解", steps 7-14), and the
// dense decode that walks a block table instead of indices (step 1).  With 64
// query heads (the H64 instances) waves w and w + 2 split the score
// contraction of head block w % 2 by dims and the softmax by keys, and the
// value contraction covers two head blocks instead of four.
//
// One work-group of 4 waves per scheduler partition; it walks the topk slots
// of each (request, block range) piece in tiles of 32 keys.  Wave w owns
// heads [32w, 32w+32) for the score contraction and output dims
// [128w, 128w+128) of all 128 heads for the value contraction.
//
//   gather   every wave copies its 8 rows of a tile (keys 8w..8w+7) HBM -> LDS
//            with direct-to-LDS loads into a ring of two raw slots; the token
//            ids are copied into LDS the same way, so memory-counter waits are
//            explicit and wave-local.  Empty slots copy rows of a zero page.
//   stage    every wave dequantises the NoPE chunks it copied (code *
//            power-of-two scale -> bf16, exact) and moves the RoPE chunks
//            into a staged tile [32 keys][576 bf16]; three staged buffers;
//   S^T      = K Q^T over all 576 dims for the wave's 32 heads (36 MFMAs per
//            tile, two accumulator chains), so no partial scores cross waves;
//   softmax  base 2 on the accumulator, masked by slot validity, against a
//            per-head reference max (see below); P rounded to bf16 and
//            published in LDS;
//   O^T     += V^T P^T for the wave's 128 dims and all 128 heads: each V^T
//            fragment (transposing LDS read) feeds four MFMAs (32 per tile);
//            O^T [128 dims x 128 heads] lives in the 256 AGPRs.
//
// Tile loop, two parts per tile i separated by work-group barriers:
//   1. the score MFMAs of tile i+1 with the softmax of tile i (its scores
//      were computed one tile earlier), the copies of tile i+3 and the ids
//      of tile i+5 between them; P(i) -> LDS;
//   2. the value MFMAs of tile i with the dequant of tile i+2 written
//      straight into the staged buffer that tile i-1 released;
// so the VALU work runs under matrix-core work and no phase is left with
// only LDS stores.
//
// The reference max of a piece is the max score of its first tile holding a
// valid key; later tiles are accumulated against it as long as no score
// exceeds it by more than 2^64.  If one does, the piece is recomputed with the
// true max, which gives the online-softmax result without rescaling O.
//
// The same kernel reads the V4 and V4.1 caches ("FlashMLA 与 DSA：内核、流水线
// 和正确性边界" section 3.1: struct-of-arrays pages, e8m0 scales; d_qk = 512
// per the walkthrough's step 2.3).  A page of P tokens holds P data rows, then
// P scale rows.  V4: 576-byte data rows (448 e4m3 codes, then 64 bf16 values
// for dims 448..511) and 8-byte scale rows (7 e8m0 bytes, one per 64 dims,
// and a pad byte); V4.1: 512-byte data rows (512 e4m3 codes) and 16-byte
// scale rows (one e8m0 byte per 32 dims).  Only the copies and the staging
// differ: the staged tile holds all 512 dims of K in its NoPE rows, the score
// contraction takes 32 k-steps instead of 36, and V = K.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int NW = 4;                             // waves per work-group
constexpr int ROWB = 656;                         // FP8 token row
constexpr int WROWS = TILE / NW;                  // rows gathered and staged per wave
constexpr int NRAW = 2;                           // raw tiles (one being staged, one landing)
constexpr int NP = 1040;                          // staged NoPE row pitch (1024 + 16)
constexpr int ROPE_OFF = TILE * NP;               // 33280: RoPE rows of a staged tile (656-byte rows)
constexpr int IDS_SLOTS = 2;                      // token-id tiles per wave in LDS
constexpr int ZERO_ROWS = 64;                     // rows of the zero page
constexpr int KAHEAD = 3;                         // score fragments read ahead of their MFMAs
constexpr int DENSE_PAGE = 64;                    // tokens per page for dense decode
constexpr int L_RAW = 0;

// Cache formats (the kv_format values).
constexpr int F32 = MLA_KV_FP8_656;               // 656-byte rows
constexpr int F4 = MLA_KV_V4_584;                 // pages of 576-byte data rows, then 8-byte scale rows
constexpr int F41 = MLA_KV_V41_528;               // pages of 512-byte data rows, then 16-byte scale rows
constexpr int FX = 4;                             // FP4 extra cache: pages of 256-byte data rows, then 32-byte
                                                  // scale rows (read beside a V4.1 main cache)
constexpr int FB = MLA_KV_BF16_576;               // bf16 rows of 1152 bytes (576 values), one per token, at the
                                                  // cache's row stride: copied straight into the staged tile

// Per-format sizes and LDS map (bytes).  A staged tile is 32 NoPE rows of NP
// bytes (bf16 dims 0..511 and a 16-byte pad that the contractions never read)
// and, for 656-byte rows, 32 RoPE rows of 128 bytes copied straight from the
// cache, chunk c of key n in slot c ^ ((n / 2) % 8) so that the score reads
// are conflict-free.  Row 0's pad of staged buffer 0 holds the restart flags;
// the head statistics of the epilogue use the P area.  Q passes through the
// bottom of the LDS in the prologue only: 32 rows per wave of QCH chunks and
// a pad chunk (conflict-free operand reads).
// 64 query heads: P takes two head blocks, and the partial scores the two
// waves of a head block exchange take [2 head blocks][2 key halves][2][64
// lanes][16 B] (the ids of tiles 0..3 use its start in the prologue).
template <int F, bool H64 = false>
struct Lay {
    static constexpr int DB = F == F32 ? 656 : F == F4 ? 576 : F == F41 ? 512 : F == FB ? 1152 : 256;   // data row
    static constexpr int SB = F == F32 || F == FB ? 0 : F == F4 ? 8 : F == F41 ? 16 : 32;            // scale row
    static constexpr int KSTEPS = F == F32 || F == FB ? 36 : 32;       // score k-steps of 16 dims
    // bf16 rows need no conversion: the copies land in the staged tile itself
    // (one 1 KB copy per NoPE row, one for the RoPE chunks), so there are no
    // raw slots and a fourth staged buffer takes the tile copied 3 ahead
    static constexpr int WAVE_RAW = F == FB ? 0 : F == F4 ? 5184 : 4224;   // a wave's raw slice
    static constexpr int NDMA = F == F41 ? 5 : F == FX ? 3 : F == FB ? WROWS + 1 : 6;   // copies per lane per tile
    static constexpr int NLOAD = F == F41 ? 5 : F == FX ? 4 : 6;       // row loads per lane (prologue)
    static constexpr int NKB = F == FB ? 4 : 3;                         // staged tiles
    static constexpr int RAW_BYTES = NW * WAVE_RAW;
    static constexpr int KBB = F == F32 || F == FB ? ROPE_OFF + TILE * 128 : TILE * NP;
    static constexpr int L_KB = L_RAW + NRAW * RAW_BYTES;              // [NKB] staged tiles
    static constexpr int L_XP = L_KB + NKB * KBB;                      // [head blocks][2 k-steps][64][16]
    static constexpr int L_XS = L_XP + (H64 ? 2 : 4) * 2048;           // 64 heads: partial-score exchange
    static constexpr int L_IDS = L_XS + (H64 ? 8192 : 0);              // [4 waves][2 slots][32] int32
    static constexpr int L_IDS0 = H64 ? L_XS : L_IDS + NW * IDS_SLOTS * 128;   // [4 waves][4 tiles][32] (prologue)
    static constexpr int L_MREF = H64 ? L_IDS + NW * IDS_SLOTS * 128 : L_IDS0 + NW * 4 * 128;   // 64 heads:
                                                                       // [2 head blocks][2 key halves][32] maxima
    static constexpr int L_BYTES = L_MREF + (H64 ? 512 : 256);
    static constexpr int L_FLAGS = L_KB + 1024;                        // [4] restart flags (row pad)
    static constexpr int L_LM = L_XP;                                  // [128 heads] {l, m} (epilogue)
    static constexpr int QCH = 2 * KSTEPS;                             // 16-byte chunks of a head's Q
    static constexpr int QROW = 16 * (QCH + 1);
    static constexpr int QCOPIES = (32 * QROW / 16 + 63) / 64;         // whole-line copies per wave
    static constexpr int L_Q = 0;                                      // [4 waves][32 heads][QROW]
    static_assert(L_BYTES <= 160 * 1024, "LDS budget");
    static_assert(L_Q + NW * 32 * QROW <= L_IDS && (32 * QROW / 16) % 64 == 32, "Q staging");
};
static_assert(Lay<F32>::WAVE_RAW == 4 * 1024 + WROWS * 16 && Lay<F32>::QCOPIES == 37, "copy layout");
static_assert(Lay<F4>::WAVE_RAW == 5120 + WROWS * 8 && Lay<F41>::QCOPIES == 33, "copy layout");
static_assert(Lay<FX>::L_BYTES == Lay<F41>::L_BYTES && Lay<FX>::L_KB == Lay<F41>::L_KB, "one LDS map for V4.1 + FP4");
static_assert(Lay<FX, true>::L_BYTES == Lay<F41, true>::L_BYTES, "one LDS map for V4.1 + FP4");
static_assert(Lay<F32, true>::L_BYTES <= 160 * 1024 && Lay<FB, true>::L_BYTES <= 160 * 1024 &&
              Lay<F4, true>::L_BYTES <= 160 * 1024, "LDS budget, 64 heads");

// Rows copied for empty or out-of-range slots: all zero bytes (zero codes,
// zero scales, zero RoPE), so staged values of empty slots are zero without
// masking.  Spread over 64 rows so the reads do not pile onto one L2 channel.
__device__ __attribute__((aligned(256))) uint8_t g_zero_rows[ZERO_ROWS * 1152];
// The id copied for slots past the end of a piece: such slots are empty.
__device__ int32_t g_no_id[1] = {-1};

// Raw slice layout (656-byte rows, 4224 bytes): NoPE chunk c < 32 of row r at
// 1024 (c / 8) + 128 r + 16 (c % 8); the scale chunk (32) of row r at
// 4096 + 16 r.  Copy i < 4 of lane L moves chunk (L % 8) + 8 i of row L / 8,
// i.e. LDS byte 1024 i + 16 L: every 8 lanes read 128 contiguous bytes of one
// row and each lane needs one row address per tile.  The RoPE copy moves the
// 8 RoPE chunks (33..40) of every row into the staged tile; the scale copy
// moves chunk 32 of row L with lanes 0..7.
//   V4.1 (4224 bytes): the same, with the 16-byte scale row of row L in place
// of chunk 32.  V4 (5184 bytes): code chunks 0..27 as above (copy 3 by lanes
// with L % 8 < 4 only), bf16 chunk j (data chunk 28 + j) of row r at
// 4096 + 128 r + 16 j (one copy by all lanes), and the 8-byte scale row of row
// r at 5120 + 8 r (4-byte copies by lanes 0..15).  FP4 (the V4.1 slice
// size): code chunks 0..15 as above (copies 0 and 1), the 32-byte scale row
// of row r at 2048 + 32 r (16-byte copies by lanes 0..15).
// RoPE copy of lane L (row L / 8 = key 8 w + L / 8 of the tile, slot L % 8):
// it moves RoPE chunk (L % 8) ^ ((key / 2) % 8) of its row; `src` points at
// chunk L % 8 of the row.
__device__ __forceinline__ const uint8_t* rope_src(const uint8_t* src, int lane, int wave) {
    const int key = WROWS * wave + (lane >> 3), s = lane & 7;
    return src + 16 * (33 + (s ^ ((key >> 1) & 7)) - s);
}
// Byte offset of RoPE chunk c (0..7) of key n in a staged tile.
__device__ __forceinline__ int rope_off(int n, int c) { return ROPE_OFF + 128 * n + 16 * (c ^ ((n >> 1) & 7)); }

// Partitions of one request are adjacent in the plan and blocks are dealt to
// the 8 XCDs round robin: map each XCD's blocks to a contiguous partition
// range, so a request's partitions share one L2 (Q is fetched once per XCD).
__device__ __forceinline__ int xcd_part(int bid, int nb) {
    const int x = bid & 7, k = bid >> 3;
    const int q = nb >> 3, r = nb & 7;
    return x * q + min(x, r) + k;
}

// Whether slot value t names a cache row (in the piece, not -1, inside the
// cache); bitwise, so that no branch is generated.
__device__ __forceinline__ bool slot_ok(const DecodeParams& p, int t, bool in_range) {
    return in_range & ((uint32_t)t < p.n_tok32);
}
// Row address of token t when ok, else row zrow of the zero page.  FLAT:
// pages back to back and every row offset below 2^32 with t < 2^24, so the
// offset is one 24-bit multiply instead of a page division.
template <bool FLAT>
__device__ __forceinline__ const uint8_t* row_addr(const DecodeParams& p, int t, bool ok, int zrow) {
    const uint32_t tt = ok ? (uint32_t)t : 0u;
    uint64_t r;
    if (FLAT) {
        r = (uint64_t)(uintptr_t)p.kv + (uint32_t)__umul24(tt, (uint32_t)ROWB);
    } else {
        const uint32_t blk = (__umulhi(tt, p.page_magic) + tt) >> p.page_mshift;
        const uint32_t off = tt - blk * (uint32_t)p.page_block_size;
        r = (uint64_t)(uintptr_t)p.kv + (uint64_t)blk * (uint64_t)p.kv_block_stride + (uint64_t)off * ROWB;
    }
    const uint64_t z = (uint64_t)(uintptr_t)g_zero_rows + (uint32_t)zrow * ROWB;
    return (const uint8_t*)(uintptr_t)(ok ? r : z);
}

// Dense decode: row address of slot `off` (0..63) of page `entry` when ok,
// else row zrow of the zero page.  FLAT: token entry * 64 + off at 656 bytes
// per token (pages back to back); otherwise the page's own stride.
template <bool FLAT>
__device__ __forceinline__ const uint8_t* dense_row_addr(const DecodeParams& p, int entry, int off, bool ok,
                                                         int zrow) {
    if (FLAT) return row_addr<true>(p, entry * DENSE_PAGE + off, ok, zrow);
    const uint32_t e = ok ? (uint32_t)entry : 0u;
    // the page stride is below 2^32 for dense decode (checked on the host):
    // one 32 x 32 -> 64-bit multiply-add
    const uint64_t r = (uint64_t)(uintptr_t)p.kv + (uint64_t)e * (uint32_t)p.kv_block_stride + (uint32_t)off * ROWB;
    const uint64_t z = (uint64_t)(uintptr_t)g_zero_rows + (uint32_t)zrow * ROWB;
    return (const uint8_t*)(uintptr_t)(ok ? r : z);
}

// bf16 cache: the row of token t when ok, else row zrow of the zero rows
// (1152-byte rows there).
__device__ __forceinline__ const uint8_t* bf16_row(const DecodeParams& p, int t, bool ok, int zrow) {
    const uint64_t r = (uint64_t)(uintptr_t)p.kv + (uint64_t)(uint32_t)(ok ? t : 0) * (uint64_t)p.kv_block_stride;
    const uint64_t z = (uint64_t)(uintptr_t)g_zero_rows + (uint32_t)zrow * 1152u;
    return (const uint8_t*)(uintptr_t)(ok ? r : z);
}

// V4 / V4.1 rows of token t when ok, else row zrow of the zero page: the
// data row address, and the scale row as a byte offset from it (page blk at
// blk * stride, its data rows from the page start, its scale rows from
// soa_scale_off = P * data row bytes; offsets inside a page are below 2^31,
// checked on the host).  A 32-bit offset instead of a second address keeps
// one register per lane across the tile loop.
template <int F>
__device__ __forceinline__ const uint8_t* soa_row(const DecodeParams& p, int t, bool ok, int zrow, int& sdel) {
    constexpr bool X = F == FX;                   // the extra cache's own pages
    const uint32_t tt = ok ? (uint32_t)t : 0u;
    const uint32_t blk = (__umulhi(tt, X ? p.x_page_magic : p.page_magic) + tt) >> (X ? p.x_page_mshift : p.page_mshift);
    const uint32_t off = tt - blk * (uint32_t)(X ? p.x_page_block_size : p.page_block_size);
    const uint64_t d = (uint64_t)(uintptr_t)(X ? p.x_kv : p.kv) +
                       (uint64_t)blk * (uint64_t)(X ? p.x_block_stride : p.kv_block_stride) + off * (uint32_t)Lay<F>::DB;
    const uint64_t z = (uint64_t)(uintptr_t)g_zero_rows + (uint32_t)zrow * Lay<F>::DB;
    // scale row - data row: P D + o S - o D (zero page: z S - z D)
    sdel = (ok ? (int)(X ? p.x_scale_off : p.soa_scale_off) : 0) -
           (int)(ok ? off : (uint32_t)zrow) * (Lay<F>::DB - Lay<F>::SB);
    return (const uint8_t*)(uintptr_t)(ok ? d : z);
}
// Source of this lane's scale copy: V4.1 lanes 0..7 copy the scale row of row
// L, V4 lanes 0..15 dword L % 2 of the scale row of row L / 2, FP4 lanes
// 0..15 half L % 2 of the scale row of row L / 2.  `src` and `sdel` are the
// lanes' own (row L / 8: chunk L % 8 of the data row, scale offset); the
// row's values come from lane 8 r.
template <int F>
__device__ __forceinline__ const uint8_t* scale_src(const uint8_t* src, int sdel, int lane) {
    const int from = 8 * (F == F41 ? (lane & 7) : ((lane >> 1) & 7));
    const uint64_t a = (uint64_t)(uintptr_t)(src - 16 * (lane & 7));
    const uint64_t r = ((uint64_t)(uint32_t)__shfl((uint32_t)(a >> 32), from) << 32) |
                       (uint32_t)__shfl((uint32_t)a, from);
    const int del = __shfl(sdel, from);
    return (const uint8_t*)(uintptr_t)(r + (int64_t)del) + (F == F4 ? 4 * (lane & 1) : F == FX ? 16 * (lane & 1) : 0);
}
// The copies of a tile from V4 / V4.1 rows; `src` points at chunk lane % 8 of
// the lane's data row, `sdel` is its scale offset.
template <int F>
__device__ __forceinline__ void gather_soa(const uint8_t* src, int sdel, int lane, uint32_t slice) {
    const uint32_t sl = __builtin_amdgcn_readfirstlane(slice);
    const uint8_t* ssrc = scale_src<F>(src, sdel, lane);
    if constexpr (F == F41) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(src + 128 * i, sl + 1024u * i);
        if (lane < 8) dma16(ssrc, sl + 4096u);
    } else if constexpr (F == FX) {
        dma16(src, sl);
        dma16(src + 128, sl + 1024u);
        if (lane < 16) dma16(ssrc, sl + 2048u);
    } else {
#pragma unroll
        for (int i = 0; i < 3; ++i) dma16(src + 128 * i, sl + 1024u * i);
        if ((lane & 7) < 4) dma16(src + 384, sl + 3072u);
        dma16(src + 448, sl + 4096u);
        if (lane < 16) dma4(ssrc, sl + 5120u);
    }
}

// Copies of this wave's 8 rows of a tile into its raw slice; `src` points at
// chunk lane % 8 of row lane / 8 (key 8w + lane / 8).
__device__ __forceinline__ const uint8_t* tail_src(const uint8_t* src, int lane) {
    // chunk 32 (scales) of row `lane` (lanes 0..7): row starts are held by lanes 8 r
    const uint64_t row = (uint64_t)(uintptr_t)(src - 16 * (lane & 7));
    const int from = 8 * (lane & 7);
    const uint64_t rl = ((uint64_t)(uint32_t)__shfl((uint32_t)(row >> 32), from) << 32) |
                        (uint32_t)__shfl((uint32_t)row, from);
    return (const uint8_t*)(uintptr_t)rl + 16 * 32;
}
__device__ __forceinline__ void gather_tail(const uint8_t* src, int lane, uint32_t slice) {
    const uint8_t* t = tail_src(src, lane);
    const uint32_t dst = __builtin_amdgcn_readfirstlane(slice + 4096u);
    if (lane < 8) dma16(t, dst);
}
// The same with the destination given as a scalar base plus a constant.
__device__ __forceinline__ void gather_tail_at(const uint8_t* src, int lane, uint32_t base, int off) {
    const uint8_t* t = tail_src(src, lane);
    if (lane < 8) dma16_at(t, base, off);
}
// All six copies of a tile: NoPE and scales into the raw slice, RoPE into
// the staged tile whose RoPE rows of this wave start at `rope_dst`.
__device__ __forceinline__ void gather_rows(const uint8_t* src, int lane, int wave, uint32_t slice, uint32_t rope_dst) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        dma16(src + 128 * i, __builtin_amdgcn_readfirstlane(slice + 1024u * i));
    dma16(rope_src(src, lane, wave), __builtin_amdgcn_readfirstlane(rope_dst));
    gather_tail(src, lane, slice);
}
// bf16 rows: copy r (0..7) of a wave moves NoPE row 8w + r whole (1 KB: lane
// L reads its bytes 16 L ..) into that row of the staged tile at kb; the row's
// address comes from lane 8 r, which holds it (`row` is the lane's own row,
// key 8w + L / 8).  The RoPE copy moves chunk (L % 8) ^ ((key / 2) % 8) of the
// lane's row, as for 656-byte rows.
template <int R>
__device__ __forceinline__ void bf16_row_copy(const uint8_t* row, int lane, int wave, uint32_t kb_addr) {
    const uint64_t a = (uint64_t)(uintptr_t)row;
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)a, 8 * R);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(a >> 32), 8 * R);
    dma16_row(((uint64_t)hi << 32) | lo, 16u * (uint32_t)lane,
              __builtin_amdgcn_readfirstlane(kb_addr + (uint32_t)((WROWS * wave + R) * NP)));
}
__device__ __forceinline__ void bf16_rope_copy(const uint8_t* row, int lane, int wave, uint32_t kb_addr) {
    const int key = WROWS * wave + (lane >> 3), s = lane & 7;
    dma16(row + 1024 + 16 * (s ^ ((key >> 1) & 7)),
          __builtin_amdgcn_readfirstlane(kb_addr + ROPE_OFF + 1024u * wave));
}
__device__ __forceinline__ void bf16_tile_copy(const uint8_t* row, int lane, int wave, uint32_t kb_addr) {
    bf16_row_copy<0>(row, lane, wave, kb_addr);
    bf16_row_copy<1>(row, lane, wave, kb_addr);
    bf16_row_copy<2>(row, lane, wave, kb_addr);
    bf16_row_copy<3>(row, lane, wave, kb_addr);
    bf16_row_copy<4>(row, lane, wave, kb_addr);
    bf16_row_copy<5>(row, lane, wave, kb_addr);
    bf16_row_copy<6>(row, lane, wave, kb_addr);
    bf16_row_copy<7>(row, lane, wave, kb_addr);
    bf16_rope_copy(row, lane, wave, kb_addr);
}

// The copies of a tile in any format (rope_dst: 656-byte rows only; sdel:
// V4 / V4.1 only).
template <int F>
__device__ __forceinline__ void gather_tile(const uint8_t* src, int sdel, int lane, int wave, uint32_t slice,
                                            uint32_t rope_dst) {
    if constexpr (F == F32) gather_rows(src, lane, wave, slice, rope_dst);
    else gather_soa<F>(src, sdel, lane, slice);
}

// Copy the 32 token ids of a tile into an id slot; slots past the end of the
// piece receive -1 (empty), so readers test only the id.
__device__ __forceinline__ void copy_ids(const int32_t* idx, int k_lo, int k_hi, int tile, int lane,
                                         uint32_t slot_addr) {
    const int k = k_lo + tile * TILE + (lane & 31);
    const int32_t* src = k < k_hi ? idx + k : g_no_id;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(slot_addr);
    if (lane < 32) dma4(src, dst);
}

// Dense decode ("FlashMLA Sparse Decode 完整计算过程详解", step 1: the block
// table walked in order; "FlashMLA 与 DSA" section 6.1: the dense decode
// pages hold 64 tokens): slot k of a request is its logical token k.  Pieces
// start on 32-slot boundaries, so the 32 slots of a tile lie in one page;
// every slot of the id slot receives that page's block-table entry (slots past
// the piece: -1), copied the same way as sparse ids so the memory-counter
// accounting is unchanged.  dense_id turns an entry back into a token id when
// it is read.
__device__ __forceinline__ void copy_pages(const int32_t* bt_row, int k_lo, int k_hi, int tile, int lane,
                                           uint32_t slot_addr) {
    const int k0 = k_lo + tile * TILE;
    const int k = k0 + (lane & 31);
    const int32_t* src = k < k_hi ? bt_row + k0 / DENSE_PAGE : g_no_id;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(slot_addr);
    if (lane < 32) dma4(src, dst);
}


// Staging of this wave's 8 rows.  Lane L holds NoPE chunks (L % 8) + 8 i of
// row r = L / 8 (copies i = 0..3: dims 16 c .. 16 c + 15) and each chunk's
// scale: dequantised into 32 bytes of the staged NoPE row.  656-byte rows:
// chunk i has fp32 scale i; V4.1: e8m0 byte c / 2 of the row's scale row;
// V4: e8m0 byte c / 4, chunk 3 only in lanes with L % 8 < 4, and the lane's
// bf16 chunk (dims 448 + 8 (L % 8) ..) copied into the row unchanged.  Split
// into the LDS reads and the conversion + writes, so a caller can put other
// work between them.  (656-byte rows: the RoPE chunks were copied into the
// staged tile directly.)
struct StageRegs {
    u32x4 w[4];
    float sc[4];
    u32x4 rope;
};
// e8m0 byte `byte` of `word` as the conversion's scale operand.  The scaled
// conversions take only the exponent field of their f32 scale, so the float
// with exponent bits e is exactly 2^(e - 127) for every byte, 0 included,
// and NaN for 0xFF: the e8m0 values.
__device__ __forceinline__ float e8m0_scale(uint32_t word, int byte) {
    return __uint_as_float(((word >> (8 * byte)) & 0xffu) << 23);
}
// Byte `sel` of w (two e2m1 values, the first in the low nibble) times the
// scale -> two bf16 (the same exponent-only scale operand as above).
__device__ __forceinline__ uint32_t fp4_pair(uint32_t w, float scale, int sel) {
    switch (sel) {
        case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
        case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
        case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
        default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
    }
}
// Scales of a lane's four chunks from its row's scale bytes (V4.1: 4 words,
// V4: 2 words).  FP4: a lane holds two 32-dim chunks c = L % 8 and c + 8,
// each with two scales (bytes 2 c, 2 c + 1 and 2 c + 16, 2 c + 17 of the
// row), from the two words that hold them.
template <int F>
__device__ __forceinline__ void soa_scales(StageRegs& g, const uint32_t* words, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (F == F41) {
            g.sc[i] = e8m0_scale(words[i], (lane & 7) >> 1);
        } else if constexpr (F == FX) {
            g.sc[i] = e8m0_scale(words[i >> 1], 2 * (lane & 1) + (i & 1));
        } else {
            const int grp = ((lane & 7) >> 2) + 2 * i;          // 7 in lanes without a chunk 3: the pad
            g.sc[i] = e8m0_scale(words[grp >> 2], grp & 3);
        }
    }
}
// V4: the bf16 chunk of the lane (read late in the tile loop, when the
// registers of chunks 0..2 are free).
__device__ __forceinline__ u32x4 stage_load_tail(const LDS_AS uint8_t* lds, int slice, int lane) {
    return lds_read16(lds, slice + 4096 + 16 * lane);
}
// TAIL: V4 reads its bf16 chunk here too (otherwise stage_load_tail does)
template <int F, bool TAIL = true>
__device__ __forceinline__ StageRegs stage_load(const LDS_AS uint8_t* lds, int slice, int lane) {
    const int r = lane >> 3;
    StageRegs g;
#pragma unroll
    for (int i = 0; i < (F == FX ? 2 : 4); ++i) g.w[i] = lds_read16(lds, slice + 1024 * i + 16 * lane);
    if constexpr (F == F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) g.sc[i] = *(const LDS_AS float*)(lds + slice + 4096 + 16 * r + 4 * i);
    } else if constexpr (F == F41) {
        const u32x4 sw = lds_read16(lds, slice + 4096 + 16 * r);
        const uint32_t words[4] = {sw[0], sw[1], sw[2], sw[3]};
        soa_scales<F>(g, words, lane);
    } else if constexpr (F == FX) {
        const int wo = slice + 2048 + 32 * r + 4 * ((lane & 7) >> 1);
        const uint32_t words[2] = {*(const LDS_AS uint32_t*)(lds + wo), *(const LDS_AS uint32_t*)(lds + wo + 16)};
        soa_scales<F>(g, words, lane);
    } else {
        if (TAIL) g.rope = stage_load_tail(lds, slice, lane);
        const u32x2 sw = *(const LDS_AS u32x2*)(lds + slice + 5120 + 8 * r);
        const uint32_t words[2] = {sw[0], sw[1]};
        soa_scales<F>(g, words, lane);
    }
    return g;
}
// Chunk I of this wave's staging share converted and written at once (the
// target buffer is free): dims 16 (c0 + 8 I) .. +15 of row 8 wave + r.
template <int I, int F = F32>
__device__ __forceinline__ void stage_chunk(LDS_AS uint8_t* lds, const StageRegs& g, int kb, int wave, int lane) {
    const int r = lane >> 3, c0 = lane & 7;
    if constexpr (F == FX) {
        // FP4: half H = I % 2 of chunk c0 + 8 (I / 2): 16 e2m1 values in two
        // words -> dims 32 (c0 + 8 (I / 2)) + 16 H .. + 15
        const u32x4 w = g.w[I >> 1];
        const float sc = g.sc[I];
        const uint32_t a = w[2 * (I & 1)], b = w[2 * (I & 1) + 1];
        const u32x4 lo = {fp4_pair(a, sc, 0), fp4_pair(a, sc, 1), fp4_pair(a, sc, 2), fp4_pair(a, sc, 3)};
        const u32x4 hi = {fp4_pair(b, sc, 0), fp4_pair(b, sc, 1), fp4_pair(b, sc, 2), fp4_pair(b, sc, 3)};
        const int off = kb + (WROWS * wave + r) * NP + 64 * (c0 + 8 * (I >> 1)) + 32 * (I & 1);
        lds_write16(lds, off, lo);
        lds_write16(lds, off + 16, hi);
        return;
    }
    // V4 has 28 code chunks: in lanes with c0 >= 4 chunk 3 holds bf16 values,
    // whose conversion lands on dims 448.. and is overwritten by stage_tail
    const u32x4 w = g.w[I];
    const float sc = g.sc[I];
    const u32x4 lo = {dequant2<false>(w[0], sc), dequant2<true>(w[0], sc),
                      dequant2<false>(w[1], sc), dequant2<true>(w[1], sc)};
    const u32x4 hi = {dequant2<false>(w[2], sc), dequant2<true>(w[2], sc),
                      dequant2<false>(w[3], sc), dequant2<true>(w[3], sc)};
    const int off = kb + (WROWS * wave + r) * NP + 32 * (c0 + 8 * I);
    lds_write16(lds, off, lo);
    lds_write16(lds, off + 16, hi);
}
// V4: the lane's bf16 chunk into dims 448 + 8 (L % 8) .. of its row.
template <int F>
__device__ __forceinline__ void stage_tail(LDS_AS uint8_t* lds, const StageRegs& g, int kb, int wave, int lane) {
    if constexpr (F == F4) lds_write16(lds, kb + (WROWS * wave + (lane >> 3)) * NP + 896 + 16 * (lane & 7), g.rope);
}
template <int F>
__device__ __forceinline__ void stage_store(LDS_AS uint8_t* lds, const StageRegs& g, int kb, int wave, int lane) {
    stage_chunk<0, F>(lds, g, kb, wave, lane);
    stage_chunk<1, F>(lds, g, kb, wave, lane);
    stage_chunk<2, F>(lds, g, kb, wave, lane);
    stage_chunk<3, F>(lds, g, kb, wave, lane);
    stage_tail<F>(lds, g, kb, wave, lane);
}
template <int F>
__device__ __forceinline__ void stage_rows(LDS_AS uint8_t* lds, int slice, int kb, int wave, int lane) {
    stage_store<F>(lds, stage_load<F>(lds, slice, lane), kb, wave, lane);
}

// The rows of a tile loaded into registers instead of copied into a raw
// slot (the first tile of a pass, while Q still fills the LDS): lane L
// holds NoPE chunks (L % 8) + 8 i of its row (key 8 w + L / 8) and its
// scales; 656-byte rows: the row's four scales and the RoPE chunk it places
// in slot L % 8; V4.1: the 16-byte scale row; V4: the 8-byte scale row and
// bf16 chunk L % 8 (copy 3 of lanes with L % 8 >= 4 loads bf16 chunks that
// are not used).  Loaded with inline asm so the compiler neither counts nor
// waits for them: rows_wait waits for every load in flight with the
// registers tied to the wait.
struct RowRegs {
    u32x4 nope[4];
    u32x4 scales;
    u32x4 rope;
    u32x2 sc8;
    uint32_t s0, s1;                               // FP4: the two scale words of the lane
};
__device__ __forceinline__ u32x4 gload16(const uint8_t* src) {
    u32x4 v;
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(src) : "memory");
    return v;
}
__device__ __forceinline__ u32x2 gload8(const uint8_t* src) {
    u32x2 v;
    asm volatile("global_load_dwordx2 %0, %1, off" : "=v"(v) : "v"(src) : "memory");
    return v;
}
__device__ __forceinline__ uint32_t gload4(const uint8_t* src) {
    uint32_t v;
    asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(src) : "memory");
    return v;
}
// `src` points at chunk lane % 8 of the lane's row, as for gather_rows;
// `sdel` (V4 / V4.1) is the row's scale offset
template <int F>
__device__ __forceinline__ RowRegs load_rows(const uint8_t* src, int sdel, int lane, int wave) {
    const uint8_t* sown = src - 16 * (lane & 7) + sdel;
    RowRegs r;
#pragma unroll
    for (int i = 0; i < (F == FX ? 2 : 4); ++i) r.nope[i] = gload16(src + 128 * i);
    if constexpr (F == F32) {
        r.scales = gload16(src - 16 * (lane & 7) + 512);
        r.rope = gload16(rope_src(src, lane, wave));
    } else if constexpr (F == F41) {
        r.scales = gload16(sown);
    } else if constexpr (F == FX) {
        r.s0 = gload4(sown + 4 * ((lane & 7) >> 1));
        r.s1 = gload4(sown + 16 + 4 * ((lane & 7) >> 1));
    } else {
        r.rope = gload16(src + 448);
        r.sc8 = gload8(sown);
    }
    return r;
}
// Wait until at most N memory operations newer than the loads of `a` are in
// flight (so `a` has landed), with its registers tied to the wait.
template <int N, int F>
__device__ __forceinline__ void rows_wait(RowRegs& a) {
    if constexpr (F == F32)
        asm volatile("s_waitcnt vmcnt(%6)"
                     : "+v"(a.nope[0]), "+v"(a.nope[1]), "+v"(a.nope[2]), "+v"(a.nope[3]), "+v"(a.scales), "+v"(a.rope)
                     : "n"(N) : "memory");
    else if constexpr (F == F41)
        asm volatile("s_waitcnt vmcnt(%5)"
                     : "+v"(a.nope[0]), "+v"(a.nope[1]), "+v"(a.nope[2]), "+v"(a.nope[3]), "+v"(a.scales)
                     : "n"(N) : "memory");
    else if constexpr (F == FX)
        asm volatile("s_waitcnt vmcnt(%4)"
                     : "+v"(a.nope[0]), "+v"(a.nope[1]), "+v"(a.s0), "+v"(a.s1)
                     : "n"(N) : "memory");
    else
        asm volatile("s_waitcnt vmcnt(%6)"
                     : "+v"(a.nope[0]), "+v"(a.nope[1]), "+v"(a.nope[2]), "+v"(a.nope[3]), "+v"(a.rope), "+v"(a.sc8)
                     : "n"(N) : "memory");
}
// Staging of a tile from registers into the K buffer at kb: the NoPE chunks
// dequantised as in stage_chunk, the RoPE chunk (656-byte rows) written to
// its slot, the bf16 chunk (V4) into its row.
template <int F>
__device__ __forceinline__ void stage_from_regs(LDS_AS uint8_t* lds, const RowRegs& r, int kb, int wave, int lane) {
    StageRegs g;
#pragma unroll
    for (int i = 0; i < (F == FX ? 2 : 4); ++i) g.w[i] = r.nope[i];
    if constexpr (F == F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) g.sc[i] = __uint_as_float(r.scales[i]);
    } else if constexpr (F == F41) {
        const uint32_t words[4] = {r.scales[0], r.scales[1], r.scales[2], r.scales[3]};
        soa_scales<F>(g, words, lane);
    } else if constexpr (F == FX) {
        const uint32_t words[2] = {r.s0, r.s1};
        soa_scales<F>(g, words, lane);
    } else {
        g.rope = r.rope;
        const uint32_t words[2] = {r.sc8[0], r.sc8[1]};
        soa_scales<F>(g, words, lane);
    }
    stage_store<F>(lds, g, kb, wave, lane);
    if constexpr (F == F32) lds_write16(lds, kb + ROPE_OFF + 1024 * wave + 16 * lane, r.rope);
}

// Value operand (V^T fragment) of the transposing LDS read, 32 dims x 16 keys
// of k-step t.  In each 16-lane group, provider lane 4q + b points at the
// 8-byte row of key 16t + s(q) + 2h + r (s = 0, 8, 4, 12; h = lane / 32;
// r = 0 for the first read, 1 for the second) at dims 16((lane/16)%2) + 4b;
// receiver lane l then holds dim l%32 of keys s(q) + 2h + r as element
// 4r + q.  Rows are 1040 bytes apart, so each half-wave's 32 providers hit 32
// distinct 8-byte bank pairs.  P is laid out in the same key order.
__device__ __forceinline__ int pv_base(int lane) {
    const int q = (lane & 15) >> 2;
    const int key = 8 * (q & 1) + 4 * (q >> 1) + 2 * (lane >> 5);
    const int dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    return key * NP + 2 * dim;
}
__device__ __forceinline__ bf16x8 v_frag(const LDS_AS uint8_t* lds, int off) {
    const u32x2 r0 = lds_read_tr16(lds, off);
    const u32x2 r1 = lds_read_tr16(lds, off + NP);
    return __builtin_bit_cast(bf16x8, u32x4{r0[0], r0[1], r1[0], r1[1]});
}

// P of k-step t as the value contraction's B operand.  The score accumulator
// gives lane (head n, half h) keys 16t + 4h + e and 16t + 8 + 4h + e; pair_e
// packs those two.  Element 4r + q of the operand must be key s(q) + 2h + r,
// i.e. dwords {pair_2h of half 0, pair_2h of half 1, pair_2h+1 of half 0,
// pair_2h+1 of half 1}: two half-wave swaps produce exactly that.
__device__ __forceinline__ u32x4 p_fragment(const f32x16& p, int t) {
    uint32_t pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = pack_bf16(p[8 * t + e], p[8 * t + 4 + e]);
    const auto a = __builtin_amdgcn_permlane32_swap(pr[0], pr[2], false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(pr[1], pr[3], false, false);
    return u32x4{a[0], a[1], b[0], b[1]};
}

// Offset of the score A operand for k-step j (dims 16 j + 8 h .. +7 of key n)
// in a staged tile: NoPE row bytes for j < 32, the RoPE slot of chunk
// 2 (j - 32) + h otherwise.
__device__ __forceinline__ int qk_off(int lane, int j) {
    const int n = lane & 31, h = lane >> 5;
    return j < 32 ? n * NP + 32 * j + 16 * h : rope_off(n, 2 * (j - 32) + h);
}

// Packed split partials: for split s and query column sq, 128 KB of bf16 laid
// out as [wave 4][k 32][lane 64][8 bf16], where k = 2 i + half holds elements
// 8 half .. 8 half + 7 of the lane's output block i = 4 j + hb (head
// 32 hb + lane % 32, dims 128 wave + 32 j + 8 (e / 4) + 4 (lane / 32) + e % 4
// for element e).  Every store and load of a wave moves 1 KB contiguously.
__device__ __forceinline__ u32x4* packed_partial(const DecodeParams& p, int split, int sq) {
    return (u32x4*)((uint16_t*)p.o_accum + ((int64_t)split * p.s_q + sq) * (128 * 512));
}

// Lane id from the lane-mask counters (no register has to keep the thread
// id alive across the kernel).
__device__ __forceinline__ int opaque_lane() {
    int l = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(l));
    return l;
}

// This lane's 16 bytes in the P area (head block 0, k-step 0), opaque so
// that head-block and k-step offsets fold into the LDS instructions'
// immediate offsets (the area lies above 64 KB).
template <int F, bool H64>
__device__ __forceinline__ int xp_base(int lane) {
    int b = Lay<F, H64>::L_XP + 16 * lane;
    asm volatile("" : "+v"(b));
    return b;
}

template <bool FLAT, bool DENSE, bool H64, int F, bool EXTRA = false>
__global__ void __launch_bounds__(NW * 64, 1) decode_fp8_h128_kernel(DecodeParams p) {
    static_assert(F == F32 || (!FLAT && !DENSE), "V4 / V4.1: paged sparse decode only");
    static_assert(!EXTRA || F == F41, "an FP4 extra cache goes with a V4.1 main cache");
    using L = Lay<F, H64>;
    constexpr int KSTEPS = L::KSTEPS;
    // 64 heads: wave w scores head block w % 2 over half w / 2 of the k-steps
    // and runs the softmax of that block over half w / 2 of a tile's keys
    constexpr int QA = H64 ? KSTEPS / 2 : KSTEPS;                // Q k-steps a wave holds
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
    LDS_AS uint8_t* lds = (LDS_AS uint8_t*)lds_raw;

    const int part = xcd_part(blockIdx.x, gridDim.x), sq = blockIdx.y;
    // wave-uniform values live in scalar registers; lane-derived offsets are
    // recomputed where they are used (opaque_lane) instead of being held
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // 64 query heads: waves w and w + 2 share head block w % 2 (heads 32 (w %
    // 2) ..).  Wave w holds Q of dims half w / 2 (k-steps 18 (w / 2) ..) and
    // scores every tile over those dims; the partners swap the partial scores
    // of each other's key half through LDS, so wave w then holds the whole
    // scores of keys 16 (w / 2) .. +15 and runs their softmax.  The tile
    // maximum comes from both halves, so the two waves of a head keep the same
    // reference max; their exp-sums are added in the epilogue.  Every wave's
    // value contraction covers head blocks 0 and 1 only.
    const int dh = wave >> 1;                                  // 64 heads: the wave's half
    constexpr int HB = H64 ? 2 : 4;                            // head blocks of 32

    const PartPlan plan = plan_part(p, part);
    const int begin_req = plan.begin_req;
    if (begin_req >= p.b) return;
    const int end_req = plan.end_req, begin_block = plan.begin_block, end_block = plan.end_block;
    const int begin_split = plan.begin_split;
    if (plan.by_length && p.topk_length == nullptr) return;   // contract error: see lengths_missing

    const uint32_t lds0 = lds_u32(lds);
    const int slice_off = L_RAW + wave * L::WAVE_RAW;         // this wave's slice in raw slot 0
    if (wave == 0 && opaque_lane() < 4) lds[L::L_FLAGS + opaque_lane()] = 0;   // ordered by the first barrier

    for (int req = begin_req; req <= end_req; ++req) {
        const int blk_lo = req == begin_req ? begin_block : 0;
        const int blk_hi = req == end_req ? end_block : whole_blocks(p, plan, req);
        const int k_lo = blk_lo * p.block;
        const int k_hi = min(blk_hi * p.block, p.topk);
        // sparse: the request's index row; dense: its block-table row
        const int32_t* idx_main = DENSE ? p.block_table + (int64_t)req * p.bt_stride
                                        : p.indices + (int64_t)req * p.idx_sb + (int64_t)sq * p.idx_ss;
        // main slots below min(piece end, len_main) hold ids; the ones past the
        // request's valid length (topk_length; dense: the cache length, less
        // the later query tokens with causal) are empty like the ones past the
        // piece.  With an extra cache, slots from main_topk on are its slots.
        const int main_top = EXTRA ? p.main_topk : p.topk;
        const int len_main = p.topk_length ? max(p.topk_length[req] - (p.causal ? p.s_q - 1 - sq : 0), 0) : k_hi;

        // Q as B operands of the score contraction, loaded once per request:
        // lane (n, h) holds dims 16 j + 8 h .. +7 of head 32w + n for k-step j
        bf16x8 qa[QA];
        f32x16 O[16];
        float m_ref = INIT_MAX, m_seen = -INFINITY, l_part = 0.f;
        // One segment of the piece: slots [s_lo, s_hi) of one cache (the main
        // cache, or the extra cache with its slots counted from 0), slots from
        // s_ok on empty, in one format FS (the formats are never mixed inside a
        // tile loop, so each loop keeps the registers of one format only).  O,
        // l and the reference max carry over from segment to segment.
        auto segment = [&](auto fs_tag, const int s_lo, const int s_hi, const int32_t* idx, const int s_ok,
                           const int pass, const bool load_q) {
            constexpr int FS = decltype(fs_tag)::value;
            constexpr int NDMA = Lay<FS, H64>::NDMA;
            const int n_tiles = (s_hi - s_lo + TILE - 1) / TILE;
            auto tile_ids = [&](int tile, int ln, uint32_t slot_addr) {
                if (DENSE) copy_pages(idx, s_lo, s_ok, tile, ln, slot_addr);
                else copy_ids(idx, s_lo, s_ok, tile, ln, slot_addr);
            };

            // LDS slots of this wave's token ids: tile t in the ring (t % 2), the
            // first four tiles of a pass in the prologue area
            auto ring_slot = [&](int tile) -> int { return L::L_IDS + (wave * IDS_SLOTS + (tile & 1)) * 128; };
            auto first_slot = [&](int tile) -> int { return L::L_IDS0 + wave * 512 + tile * 128; };
            // ids that this lane needs from a slot: key ln % 32 (validity mask) and
            // key 8w + ln / 8 (its copy row)
            auto ids_at = [&](int slot_off, int ln) -> int2 {
                const LDS_AS int32_t* slot = (const LDS_AS int32_t*)(lds + slot_off);
                return int2{slot[ln & 31], slot[WROWS * wave + (ln >> 3)]};
            };
            // validity mask of the tile's 32 keys and the copy source of this
            // lane's row (chunk ln % 8; V4 / V4.1: and the row's scale offset in
            // sdel); tiles past the piece copy zero rows
            auto rows_from = [&](int tile, int ln, int2 id, const uint8_t*& src, int& sdel) -> uint32_t {
                const int kr = WROWS * wave + (ln >> 3);
                if (DENSE) {
                    // the id slot holds the tile's block-table entry (or -1): a
                    // key is valid when the entry names a page of the cache
                    const bool ok = (uint32_t)id.x < p.n_pages;
                    const bool okr = (uint32_t)id.y < p.n_pages;
                    src = dense_row_addr<FLAT>(p, id.y, (s_lo + tile * TILE) % DENSE_PAGE + kr, okr, kr) + 16 * (ln & 7);
                    return (uint32_t)__ballot(ok);
                }
                const uint32_t n_tok = FS == FX ? p.x_n_tok32 : p.n_tok32;   // ids name tokens of the segment's cache
                const bool ok = (uint32_t)id.x < n_tok;
                const bool okr = (uint32_t)id.y < n_tok;
                if constexpr (FS == F32) src = row_addr<FLAT>(p, id.y, okr, kr) + 16 * (ln & 7);
                else if constexpr (FS == FB) src = bf16_row(p, id.y, okr, kr);     // the row itself
                else src = soa_row<FS>(p, id.y, okr, kr, sdel) + 16 * (ln & 7);
                return (uint32_t)__ballot(ok);
            };


                // this wave's raw slice in slot 0 (copy destinations are this
                // plus constants)
                const uint32_t raw0 = lds0 + slice_off;

                // Part 1 of tile i: the 36 score MFMAs of tile i+1 (K buffer at
                // kb) for this wave's 32 heads over all 576 dims (two accumulator
                // chains) with, between them, the softmax of tile i (mask empty
                // slots, base-2 exponent against the reference max, P to LDS), the
                // ids of tile i+5 and the copies of tile i+3 (raw slot and id slot
                // 1 - par for tile parity par).  With soft == false (the prologue)
                // only the scores of tile 0.  d_c (64 heads, compile time): the
                // wave's half -- k-steps D QA .. of the scores (one MFMA every
                // other step), keys 16 D .. of the softmax, whose tile maximum
                // also takes the other half's (hm: this half's, from part 2); at
                // the end the other key half of the partial scores goes to LDS
                // for the partner wave.  128 heads: d_c is unused.
                auto part1 = [&](auto d_c, int i, int par, int kb, int kb3, int ln, bool soft, bool scores,
                                 bool copies, const uint8_t* src3, int sdel3, uint32_t vm, f32x16 S, float hm,
                                 f32x16& S_next, const StageRegs* pro_g) {
                    constexpr int D = decltype(d_c)::value & 1;
                    const int qk = kb + qk_off(ln, 0);      // NoPE k-steps: qk + 32 j
                    const int r3 = 1 - par;
                    const uint32_t raw3 = raw0 + r3 * L::RAW_BYTES;
                    f32x16 Sa, Sb;
                    bf16x8 ka[KAHEAD];
                    // K operand of k-step j: NoPE rows, or RoPE k-steps 32..35
                    // (lane-dependent slots)
                    auto kofs = [&](int j) { return j < 32 ? qk + 32 * j : kb + qk_off(ln, j); };
                    constexpr int K0 = H64 ? D * QA : 0;    // first k-step of this wave
    #pragma unroll
                    for (int j = 0; j < KAHEAD; ++j)
                        if (scores) ka[j] = __builtin_bit_cast(bf16x8, lds_read16(lds, kofs(K0 + j)));
                    if (soft && copies) tile_ids(i + 5, ln, lds0 + ring_slot(r3));
                    __builtin_amdgcn_sched_barrier(0);
                    float mx, psum = 0.f, other = 0.f;
    #pragma unroll
                    for (int js = 0; js < KSTEPS; ++js) {
                        // 128 heads: k-step js; 64 heads: k-step K0 + js / 2 on even js
                        if (scores && (!H64 || (js & 1) == 0)) {
                            const int t = H64 ? js >> 1 : js;
                            const bf16x8 cur = ka[t % KAHEAD];
                            if (t + KAHEAD < QA)
                                ka[t % KAHEAD] = __builtin_bit_cast(bf16x8, lds_read16(lds, kofs(K0 + t + KAHEAD)));
                            // two alternating accumulator chains: a score MFMA never
                            // takes the result of the one issued right before it
                            // (64 heads leave AGPRs free for the compiler: guarded MFMAs)
                            if (t == 0) mfma_qk_first<H64>(Sa, cur, qa[0]);
                            else if (t == 1) mfma_qk_first<H64>(Sb, cur, qa[1]);
                            else if (t & 1) mfma_qk<H64>(Sb, cur, qa[t]);
                            else mfma_qk<H64>(Sa, cur, qa[t]);
                        }
                        if (pro_g != nullptr) {
                            // prologue: tile 1 staged into K buffer 1 under the scores of tile 0
                            if (js == 4) stage_chunk<0, FS>(lds, *pro_g, L::L_KB + L::KBB, wave, ln);
                            if (js == 12) stage_chunk<1, FS>(lds, *pro_g, L::L_KB + L::KBB, wave, ln);
                            if (js == 20) stage_chunk<2, FS>(lds, *pro_g, L::L_KB + L::KBB, wave, ln);
                            if (js == 28) {
                                stage_chunk<3, FS>(lds, *pro_g, L::L_KB + L::KBB, wave, ln);
                                stage_tail<FS>(lds, *pro_g, L::L_KB + L::KBB, wave, ln);
                            }
                        }
                        if constexpr (FS == FB) {
                            // bf16 rows: the copies of tile i+3 straight into its staged
                            // tile (K buffer kb3), rows 0..7 at js 3, 6, .., 24, RoPE at 27
                            if (soft && copies && js >= 3 && js <= 24 && js % 3 == 0) {
                                const uint32_t kbc = lds0 + kb3;
                                if (js == 3) bf16_row_copy<0>(src3, ln, wave, kbc);
                                if (js == 6) bf16_row_copy<1>(src3, ln, wave, kbc);
                                if (js == 9) bf16_row_copy<2>(src3, ln, wave, kbc);
                                if (js == 12) bf16_row_copy<3>(src3, ln, wave, kbc);
                                if (js == 15) bf16_row_copy<4>(src3, ln, wave, kbc);
                                if (js == 18) bf16_row_copy<5>(src3, ln, wave, kbc);
                                if (js == 21) bf16_row_copy<6>(src3, ln, wave, kbc);
                                if (js == 24) bf16_row_copy<7>(src3, ln, wave, kbc);
                            }
                            if (soft && copies && js == 27) bf16_rope_copy(src3, ln, wave, lds0 + kb3);
                        } else if (soft) {
                            // copies of tile i+3: NoPE chunks into the raw slot, RoPE
                            // into the staged tile it will occupy (K buffer kb3, whose
                            // RoPE rows the scores of its previous tile no longer read);
                            // V4 / V4.1: code chunks, bf16 chunks and scale rows into
                            // the raw slot
                            if (copies && js >= 3 && js <= 18 && js % 5 == 3) {
                                if (FS == FX ? js <= 8 : FS != F4 || js < 18)
                                    dma16_at(src3 + 128 * (js / 5), raw3, 1024 * (js / 5));
                                else if (FS == F4 && (ln & 7) < 4) dma16_at(src3 + 384, raw3, 3072);
                            }
                            if (copies && js == 23) {
                                if constexpr (FS == F32)
                                    dma16_at(rope_src(src3, ln, wave), lds0 + kb3 + ROPE_OFF + 1024u * wave, 0);
                                if constexpr (FS == F4) dma16_at(src3 + 448, raw3, 4096);
                            }
                            if (copies && js == 28) {
                                if constexpr (FS == F32) gather_tail_at(src3, ln, raw3, 4096);
                                if constexpr (FS == F41) {
                                    const uint8_t* ssrc3 = scale_src<FS>(src3, sdel3, ln);
                                    if (ln < 8) dma16_at(ssrc3, raw3, 4096);
                                }
                                if constexpr (FS == F4) {
                                    const uint8_t* ssrc3 = scale_src<FS>(src3, sdel3, ln);
                                    if (ln < 16) dma4_at(ssrc3, raw3, 5120);
                                }
                                if constexpr (FS == FX) {
                                    const uint8_t* ssrc3 = scale_src<FS>(src3, sdel3, ln);
                                    if (ln < 16) dma16_at(ssrc3, raw3, 2048);
                                }
                            }
                        }
                        if (soft && H64) {
                            // 64 heads: keys 16 D .. 16 D + 15 of head block wave % 2
                            // (values 8 D .. 8 D + 7, masked in part 2)
                            if (js == 0)
                                other = *(const LDS_AS float*)(lds + L::L_MREF + 4 * (32 * (2 * (wave & 1) + 1 - D) + (ln & 31)));
                            if (js == 2) {
                                const float mnew = fmaxf(hm, other) * p.c;
                                m_seen = fmaxf(m_seen, mnew);
                                if (m_ref == INIT_MAX && mnew > -INFINITY) m_ref = mnew;   // O, l still zero
                            }
                            if (js >= 4 && js < 12) {
                                const int v = 8 * D + js - 4;
                                S[v] = __builtin_amdgcn_exp2f(S[v] * p.c - m_ref);
                                psum += S[v];
                            }
                            if (js == 14) {
                                l_part += psum;
                                lds_write16(lds, xp_base<FS, H64>(ln) + (wave & 1) * 2048 + D * 1024, p_fragment(S, D));
                            }
                        }
                        if (soft && !H64) {
                            if (js == 1 && vm != 0xffffffffu) {
                                // accumulator element v holds key 8(v/4) + 4h + v%4:
                                // lanes 0..31 test bit 8(v/4) + v%4, lanes 32..63 that + 4
    #pragma unroll
                                for (int v = 0; v < 16; ++v) {
                                    const int key = 8 * (v >> 2) + (v & 3);
                                    const uint64_t lanes = (uint64_t)(0u - ((vm >> key) & 1u)) |
                                                           ((uint64_t)(0u - ((vm >> (key + 4)) & 1u)) << 32);
                                    S[v] = __builtin_amdgcn_inverse_ballot_w64(lanes) ? S[v] : -INFINITY;
                                }
                            }
                            if (js == 2) {
                                mx = S[0];
    #pragma unroll
                                for (int v = 1; v < 16; ++v) mx = fmaxf(mx, S[v]);
                            }
                            if (js == 4) {
                                // max with the other half-wave (same head): the swap hands
                                // lanes 0..31 the upper half's value in the second result
                                // and lanes 32..63 the lower half's in the first
                                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                                mx = fmaxf(mx, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
                                const float mnew = mx * p.c;
                                m_seen = fmaxf(m_seen, mnew);
                                if (m_ref == INIT_MAX && mnew > -INFINITY) m_ref = mnew;   // O, l still zero
                            }
                            if (js >= 6 && js < 22) {
                                const int v = js - 6;
                                S[v] = __builtin_amdgcn_exp2f(S[v] * p.c - m_ref);
                                psum += S[v];
                            }
                            if (js == 24) {
                                l_part += psum;
                                lds_write16(lds, xp_base<FS, H64>(ln) + wave * 2048, p_fragment(S, 0));
                            }
                            if (js == 26) lds_write16(lds, xp_base<FS, H64>(ln) + wave * 2048 + 1024, p_fragment(S, 1));
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (scores) {
                        mfma_result_fence2(Sa, Sb);
                        S_next = Sa + Sb;
                        if constexpr (H64) {
                            // the other key half of this partial to the partner wave:
                            // [head block][key half][2][64 lanes][16 B]
                            const int xo = L::L_XS + (2 * (wave & 1) + 1 - D) * 2048 + 16 * ln;
                            constexpr int V0 = 8 * (1 - D);
                            lds_write16(lds, xo, u32x4{__float_as_uint(S_next[V0]), __float_as_uint(S_next[V0 + 1]),
                                                      __float_as_uint(S_next[V0 + 2]), __float_as_uint(S_next[V0 + 3])});
                            lds_write16(lds, xo + 1024, u32x4{__float_as_uint(S_next[V0 + 4]), __float_as_uint(S_next[V0 + 5]),
                                                             __float_as_uint(S_next[V0 + 6]), __float_as_uint(S_next[V0 + 7])});
                        }
                    }
                };
                // 64 heads, under the value steps of part 2 (xs_read, then
                // assemble): this wave's key half of the next tile's scores in S
                // (its partial plus the partner's, from LDS), masked by that
                // tile's validity vm, and its maximum (both half-waves) in hm and
                // in LDS for the partner's next part 1; the prologue does the
                // same for tile 0.
                auto xs_read = [&](auto d_c, int ln, u32x4& a, u32x4& b) {
                    constexpr int D = decltype(d_c)::value & 1;
                    const int xi = L::L_XS + (2 * (wave & 1) + D) * 2048 + 16 * ln;
                    a = lds_read16(lds, xi);
                    b = lds_read16(lds, xi + 1024);
                };
                auto assemble = [&](auto d_c, f32x16& S, const u32x4& a, const u32x4& b, uint32_t vm, float& hm, int ln) {
                    constexpr int D = decltype(d_c)::value & 1;
    #pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        S[8 * D + e] += __uint_as_float(a[e]);
                        S[8 * D + 4 + e] += __uint_as_float(b[e]);
                    }
                    if (vm != 0xffffffffu) {
                        // element v holds key 8(v/4) + 4h + v%4 (as in the 128-head mask)
    #pragma unroll
                        for (int v = 8 * D; v < 8 * D + 8; ++v) {
                            const int key = 8 * (v >> 2) + (v & 3);
                            const uint64_t lanes = (uint64_t)(0u - ((vm >> key) & 1u)) |
                                                   ((uint64_t)(0u - ((vm >> (key + 4)) & 1u)) << 32);
                            S[v] = __builtin_amdgcn_inverse_ballot_w64(lanes) ? S[v] : -INFINITY;
                        }
                    }
                    float mx = S[8 * D];
    #pragma unroll
                    for (int v = 8 * D + 1; v < 8 * D + 8; ++v) mx = fmaxf(mx, S[v]);
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                    mx = fmaxf(mx, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
                    hm = mx;
                    if (ln < 32) *(LDS_AS float*)(lds + L::L_MREF + 4 * (32 * (2 * (wave & 1) + D) + ln)) = mx;
                };
                // Part 2 of tile i: the 32 value MFMAs of tile i (O^T += V^T P^T over
                // this wave's 128 dims, all 128 heads; V from the K buffer at kbv, P
                // from LDS) with, between them, the dequant of tile i+2 (raw slot
                // par) written straight into the K buffer at kb2 (free since tile
                // i-1 is done) and the copy source of tile i+4 (id slot par).  Past
                // the piece the staged rows are zero rows.  step_hook(jv) runs at
                // the end of value step jv (64 heads: the score exchange).
                auto part2 = [&](int i, int par, int kbv, int kb2, int ln, bool stage, bool copies_out,
                                 const uint8_t*& src4, int& sdel4, uint32_t& vm4, auto&& step_hook) {
                    const int vb = kbv + pv_base(ln) + 64 * 4 * wave;
                    const int xp = xp_base<FS, H64>(ln);
                    // the copies of tile i+2 and the ids of tile i+4 have landed
                    // (1 + NDMA newer ops: the ids of tile i+5, the copies of tile
                    // i+3; none near the end of the piece)
                    // bf16 rows: nothing to stage, but tile i+2 must have landed
                    // before its scores (the next part 1)
                    constexpr bool ST = FS != FB;
                    StageRegs g;
                    if (stage) {
                        if (copies_out) wait_vmcnt<1 + NDMA>();
                        else wait_vmcnt<0>();
                        if constexpr (ST) g = stage_load<FS, false>(lds, slice_off + par * L::RAW_BYTES, ln);
                    }
                    bf16x8 va, pf[4];
    #pragma unroll
                    for (int hb = 0; hb < HB; ++hb)
                        pf[hb] = __builtin_bit_cast(bf16x8, lds_read16(lds, xp + hb * 2048));
                    va = v_frag(lds, vb);
                    __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                    for (int jv = 0; jv < 8; ++jv) {
                        // value step jv: k-step jv / 4, dim block jv % 4; the next V^T
                        // fragment is read ahead
                        bf16x8 vn;
                        if (jv + 1 < 8) vn = v_frag(lds, vb + ((jv + 1) >> 2) * 16 * NP + ((jv + 1) & 3) * 64);
    #pragma unroll
                        for (int hb = 0; hb < HB; ++hb) mfma_pv(O[4 * (jv & 3) + hb], va, pf[hb]);
                        if (jv == 3) {
    #pragma unroll
                            for (int hb = 0; hb < HB; ++hb)
                                pf[hb] = __builtin_bit_cast(bf16x8, lds_read16(lds, xp + hb * 2048 + 1024));
                        }
                        if (jv + 1 < 8) va = vn;
                        if (stage && jv == 0) vm4 = rows_from(i + 4, ln, ids_at(ring_slot(par), ln), src4, sdel4);
                        if (ST && stage && jv == 1) stage_chunk<0, FS>(lds, g, kb2, wave, ln);
                        if (ST && stage && jv == 3) stage_chunk<1, FS>(lds, g, kb2, wave, ln);
                        if (ST && stage && jv == 5) {
                            stage_chunk<2, FS>(lds, g, kb2, wave, ln);
                            if constexpr (FS == F4) g.rope = stage_load_tail(lds, slice_off + par * L::RAW_BYTES, ln);
                        }
                        if (ST && stage && jv == 7) {
                            stage_chunk<3, FS>(lds, g, kb2, wave, ln);
                            stage_tail<FS>(lds, g, kb2, wave, ln);
                        }
                        step_hook(jv);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                };

                // ---- prologue: ids of tiles 0..4; (first pass) Q through LDS and,
                // under it, the rows of tiles 0 and 1 into registers; copy sources
                // of tiles 2 and 3; the copies of tile 2 into raw slot 0; tiles 0
                // and 1 staged from the registers into K buffers 0 and 1; the
                // scores of tile 0.  (Dense decode: tiles 0 and 1 copied into the
                // raw slots after Q, tile 1 staged under the scores of tile 0;
                // bf16 rows: tiles 0..2 copied into K buffers 0..2 after Q.)
                uint32_t vm0, vm1, vm2, vm3;            // validity masks of tiles i .. i+3
                const uint8_t* src_nx;                  // this lane's copy source in tile i+3
                int sdel_nx = 0;                        // and its scale offset (V4 / V4.1)
                f32x16 S_cur;                           // scores of tile i
                float hm_cur = -INFINITY;               // 64 heads: max of this wave's key half
                {
                    const int ln = opaque_lane();
                    for (int t = 0; t < 4; ++t) tile_ids(t, ln, lds0 + first_slot(t));
                    tile_ids(4, ln, lds0 + ring_slot(4));
                    if (pass == 0 && load_q) {
                        // Q of the wave's 32 heads (with 64 query heads waves 2 and
                        // 3 take heads 0..63 again; those results are never stored)
                        // copied whole-line into LDS: region row n = head 32w + n,
                        // QROW bytes (the QCH chunks of a head's Q and a pad chunk,
                        // so the operand reads are conflict-free).  Copy m, lane l
                        // moves region chunk 64 m + l.
                        const uint16_t* q_req = p.q + (int64_t)req * p.q_sb + (int64_t)sq * p.q_ss;
                        const uint32_t qreg = lds0 + L::L_Q + wave * 32 * L::QROW;
                        int n = 0, c = ln;                  // region row and chunk of copy 0
    #pragma unroll
                        for (int m = 0; m < L::QCOPIES; ++m) {
                            const uint16_t* src = q_req + (int64_t)((32 * wave + n) & (p.h_q - 1)) * p.q_sh +
                                                  8 * (c < L::QCH ? c : 0);
                            if (m < L::QCOPIES - 1 || ln < 32) dma16(src, qreg + 1024u * m);
                            c += 64;
                            if (c >= L::QCH + 1) { c -= L::QCH + 1; n += 1; }
                        }
                        wait_vmcnt<L::QCOPIES>();           // ids of tiles 0..4 (the copies of Q are newer)
                    } else {
                        wait_vmcnt<0>();                    // ids of tiles 0..4
                    }
                    if constexpr (FS == FB) {
                        // bf16 rows: tiles 0..2 copied straight into K buffers 0..2
                        // once Q has left the LDS
                        const uint8_t* s0;
                        const uint8_t* s1;
                        const uint8_t* s2;
                        int sd = 0;
                        vm0 = rows_from(0, ln, ids_at(first_slot(0), ln), s0, sd);
                        vm1 = rows_from(1, ln, ids_at(first_slot(1), ln), s1, sd);
                        vm2 = rows_from(2, ln, ids_at(first_slot(2), ln), s2, sd);
                        vm3 = rows_from(3, ln, ids_at(first_slot(3), ln), src_nx, sdel_nx);
                        if (pass == 0 && load_q) {
                            wait_vmcnt<0>();
                            const int qr = L::L_Q + wave * 32 * L::QROW + (ln & 31) * L::QROW + 16 * (ln >> 5) +
                                           32 * (H64 ? dh * QA : 0);
    #pragma unroll
                            for (int j = 0; j < QA; ++j)
                                qa[j] = __builtin_bit_cast(bf16x8, lds_read16(lds, qr + 32 * j));
                            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
                        }
                        __syncthreads();                    // every wave's Q reads are done
                        bf16_tile_copy(s0, ln, wave, lds0 + L::L_KB);
                        bf16_tile_copy(s1, ln, wave, lds0 + L::L_KB + L::KBB);
                        bf16_tile_copy(s2, ln, wave, lds0 + L::L_KB + 2 * L::KBB);
                        wait_vmcnt<2 * NDMA>();             // the wave's copies of tile 0 (tiles 1 and 2 newer)
                    } else {
                    const uint8_t* src;
                    const uint8_t* src2;
                    int sdel = 0, sdel2 = 0;
                    vm0 = rows_from(0, ln, ids_at(first_slot(0), ln), src, sdel);
                    vm1 = rows_from(1, ln, ids_at(first_slot(1), ln), src2, sdel2);
                    // sparse decode: the rows of tiles 0 and 1 travel while Q lands
                    // (NLOAD loads per lane each, newer than the copies of Q), so
                    // no copy waits for the Q reads to free the LDS.  (Dense decode
                    // copies its tiles after Q: holding these registers across the
                    // Q reads would make its paged-address instance spill.)
                    RowRegs r0, r1;
                    if (!DENSE) {
                        r0 = load_rows<FS>(src, sdel, ln, wave);
                        r1 = load_rows<FS>(src2, sdel2, ln, wave);
                    }
                    if (pass == 0 && load_q) {
                        {
                            // Q into registers: lane (n, h) holds dims 16 j + 8 h .. +7
                            // of head 32w + n for k-step j
                            if (DENSE) wait_vmcnt<0>();
                            else wait_vmcnt<2 * Lay<FS, H64>::NLOAD>();
                            const int qr = L::L_Q + wave * 32 * L::QROW + (ln & 31) * L::QROW + 16 * (ln >> 5) +
                                           32 * (H64 ? dh * QA : 0);
    #pragma unroll
                            for (int j = 0; j < QA; ++j)
                                qa[j] = __builtin_bit_cast(bf16x8, lds_read16(lds, qr + 32 * j));
                            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
                        }
                        // every wave's reads are done before the staging reuses the area
                        __syncthreads();
                    }
                    const uint32_t rope0 = lds0 + L::L_KB + ROPE_OFF + 1024u * wave;   // K buffer 0 (656-byte rows)
                    if (DENSE) {
                        gather_rows(src, ln, wave, lds0 + slice_off, rope0);
                        gather_tile<FS>(src2, sdel2, ln, wave, lds0 + slice_off + L::RAW_BYTES, rope0 + L::KBB);
                    }
                    vm2 = rows_from(2, ln, ids_at(first_slot(2), ln), src2, sdel2);
                    vm3 = rows_from(3, ln, ids_at(first_slot(3), ln), src_nx, sdel_nx);
                    if (DENSE) {
                        wait_vmcnt<0>();                    // copies of tiles 0 and 1
                        stage_rows<FS>(lds, slice_off, L::L_KB, wave, ln);
                        // raw slot 0 is free (its values went through the conversions)
                        gather_tile<FS>(src2, sdel2, ln, wave, lds0 + slice_off, rope0 + 2 * L::KBB);
                        wait_vmcnt<NDMA>();                 // the wave's copies of tile 1 (tile 2's are newer)
                    } else {
                        // tile 2 into raw slot 0, then tiles 0 and 1 staged from registers
                        gather_tile<FS>(src2, sdel2, ln, wave, lds0 + slice_off, rope0 + 2 * L::KBB);
                        rows_wait<Lay<FS, H64>::NLOAD + NDMA, FS>(r0);   // tile 0 (tile 1, tile 2 newer)
                        stage_from_regs<FS>(lds, r0, L::L_KB, wave, ln);
                        rows_wait<NDMA, FS>(r1);            // tile 1 (the copies of tile 2 are newer)
                        stage_from_regs<FS>(lds, r1, L::L_KB + L::KBB, wave, ln);
                    }
                    }
                }
                __syncthreads();                        // tiles 0 and 1 staged (dense: tile 0)
                {
                    // the scores of tile 0
                    const int ln = opaque_lane();
                    // (dense decode: tile 1 staged under them from raw slot 1)
                    StageRegs g1;
                    if constexpr (DENSE && FS != FB) g1 = stage_load<FS>(lds, slice_off + L::RAW_BYTES, ln);
                    const StageRegs* pg = DENSE && FS != FB ? &g1 : nullptr;
                    f32x16 none = {};
                    if (!H64 || dh == 0)
                        part1(std::integral_constant<int, 0>{}, -1, 1, L::L_KB, 0, ln, false, true, false, nullptr, 0, 0u,
                              none, 0.f, S_cur, pg);
                    else if constexpr (H64)
                        part1(std::integral_constant<int, 1>{}, -1, 1, L::L_KB, 0, ln, false, true, false, nullptr, 0, 0u,
                              none, 0.f, S_cur, pg);
                    if constexpr (FS == FB) wait_vmcnt<NDMA>();   // tile 1 landed (tile 2's copies newer)
                }
                __syncthreads();                        // tile 1 staged
                if constexpr (H64) {
                    // the partner's half of the scores of tile 0; both halves' maxima
                    // in LDS before the softmax of tile 0 reads them
                    auto pro = [&](auto d_c) {
                        const int ln = opaque_lane();
                        u32x4 a, b;
                        xs_read(d_c, ln, a, b);
                        assemble(d_c, S_cur, a, b, vm0, hm_cur, ln);
                    };
                    if (dh == 0) pro(std::integral_constant<int, 0>{});
                    else pro(std::integral_constant<int, 1>{});
                    __syncthreads();
                }

                // K buffers of the values, scores and staging of tile i (buffers
                // i % 3, (i + 1) % 3, (i + 2) % 3), rotated every tile
                int kb_v = L::L_KB, kb_s = L::L_KB + L::KBB, kb_g = L::L_KB + 2 * L::KBB;
                int kb_c = L::L_KB + 3 * L::KBB;        // bf16 rows: the buffer tile i+3 is copied into
                // One tile; near the end of the piece the work for tiles past it is
                // left out: the copies of tile i+3 (and ids of i+5) from tile n-3 on,
                // the staging of tile i+2 from n-2 on, the scores of tile i+1 at n-1.
                auto tile = [&](int i, int par, auto tail_c, auto d_c) {
                    constexpr int left = decltype(tail_c)::value;   // tiles left including i, 0 = more than 3
                    constexpr bool copies = left == 0, stage = left == 0 || left == 3, scores = left != 1;
                    // lane-derived offsets are recomputed every tile (cheap VALU)
                    // rather than held in registers across the loop
                    const int ln = opaque_lane();
                    f32x16 S_next;
                    float hm_next = -INFINITY;
                    // the buffer of tile i+3's RoPE (656-byte rows: tile i's, whose
                    // NoPE rows the values still read) or of all of it (bf16 rows)
                    const int kb3 = FS == FB ? kb_c : kb_v;
                    part1(d_c, i, par, kb_s, kb3, ln, true, scores, copies, src_nx, sdel_nx, vm0, S_cur, hm_cur,
                          S_next, nullptr);
                    __syncthreads();
                    const uint8_t* src4 = src_nx;
                    int sdel4 = sdel_nx;
                    uint32_t vm4 = 0u;
                    // 64 heads, tile i + 1: the partner's half of the scores (written
                    // before the barrier above) read under the first value steps and
                    // added in the middle ones; the maxima reach the partner by the
                    // barrier below
                    u32x4 xa, xb;
                    part2(i, par, kb_v, kb_g, ln, stage, copies, src4, sdel4, vm4, [&](int jv) {
                        if constexpr (H64) {
                            if (scores && jv == 0) xs_read(d_c, ln, xa, xb);
                            if (scores && jv == 3) assemble(d_c, S_next, xa, xb, vm1, hm_next, ln);
                        }
                    });
                    __syncthreads();
                    S_cur = S_next;
                    hm_cur = hm_next;
                    src_nx = src4;
                    sdel_nx = sdel4;
                    vm0 = vm1;
                    vm1 = vm2;
                    vm2 = vm3;
                    vm3 = vm4;
                    const int t = kb_v;
                    kb_v = kb_s;
                    kb_s = kb_g;
                    if constexpr (FS == FB) {
                        kb_g = kb_c;
                        kb_c = t;
                    } else {
                        kb_g = t;
                    }
                };
                // 64 heads: one loop per key half (its part 1 and 2 are compiled
                // for it)
                auto loop = [&](auto d_c) {
                    int i = 0;
                    for (; i + 3 < n_tiles; ++i) tile(i, i & 1, std::integral_constant<int, 0>{}, d_c);
                    if (i + 2 < n_tiles) tile(i, i & 1, std::integral_constant<int, 3>{}, d_c), ++i;
                    if (i + 1 < n_tiles) tile(i, i & 1, std::integral_constant<int, 2>{}, d_c), ++i;
                    tile(i, i & 1, std::integral_constant<int, 1>{}, d_c);
                };
                if (!H64 || dh == 0) loop(std::integral_constant<int, 0>{});
                else if constexpr (H64) loop(std::integral_constant<int, 1>{});
        };

        for (int pass = 0;; ++pass) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if ((i & 3) < HB) O[i] = f32x16{};
            l_part = 0.f;
            __syncthreads();                        // LDS free (previous piece / pass done)
            const int m_hi = min(k_hi, main_top);
            if (k_lo < m_hi)
                segment(std::integral_constant<int, F>{}, k_lo, m_hi, idx_main, min(m_hi, len_main), pass, true);
            if constexpr (EXTRA) {
                if (k_hi > main_top) {
                    if (k_lo < m_hi) {
                        wait_vmcnt<0>();            // copies past the main slots
                        __syncthreads();            // LDS free for the extra segment
                    }
                    const int x_lo = max(k_lo, main_top) - main_top, x_hi = k_hi - main_top;
                    const int32_t* idx_x = p.x_indices + (int64_t)req * p.x_idx_sb + (int64_t)sq * p.x_idx_ss;
                    const int x_ok = p.x_topk_length ? min(x_hi, max(p.x_topk_length[req], 0)) : x_hi;
                    segment(std::integral_constant<int, FX>{}, x_lo, x_hi, idx_x, x_ok, pass, k_lo >= m_hi);
                }
            }
            // the reference stays fixed once set, so one test of the largest
            // score max of the pass covers every tile
            const bool restart = __any(m_seen > m_ref + p.threshold);
            if (opaque_lane() == 0) lds[L::L_FLAGS + wave] = restart ? 1 : 0;
            __syncthreads();
            wait_vmcnt<0>();                                    // copies still in flight (short pieces)
            // A score exceeded the reference by more than 2^threshold in some
            // wave: recompute the piece against the true max (rare).
            const uint32_t flags = *(const LDS_AS uint32_t*)(lds + L::L_FLAGS);
            __syncthreads();
            if (flags == 0u || pass > 0) break;
            if (wave == 0 && opaque_lane() < 4) lds[L::L_FLAGS + opaque_lane()] = 0;
            m_ref = m_seen;     // 64 heads: both waves of a head saw the same maxima
        }

        // ---- epilogue: l and m of every head through LDS
        const int lane = opaque_lane();
        const int n = lane & 31, h = lane >> 5;
        // the value MFMAs retire in order: one wait after the last (O[15])
        // covers every accumulator
        constexpr int OLAST = H64 ? 13 : 15;                   // the last accumulator written
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+a"(O[OLAST]));
#pragma unroll
        for (int i = 0; i < OLAST; ++i)
            if ((i & 3) < HB) asm volatile("" : "+a"(O[i]));
        // exp-sum over both half-waves (same head): the swap leaves a lane's
        // own value in one result and the other half's in the other
        const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
        float l_tot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
        if (lane < 32) *(LDS_AS f32x2*)(lds + L::L_LM + 8 * (32 * wave + n)) = f32x2{l_tot, m_ref};
        __syncthreads();
        // 64 heads: a head's exp-sum is split over waves w and w + 2
        if constexpr (H64) l_tot += (*(const LDS_AS f32x2*)(lds + L::L_LM + 8 * (32 * (wave ^ 2) + n)))[0];
        float inv[4];
        const int first_split = split_prefix(p, req);
        const int nsplit = split_prefix(p, req + 1) - first_split;
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
            f32x2 lm = *(const LDS_AS f32x2*)(lds + L::L_LM + 8 * (32 * hb + n));
            if (H64 && hb < 2) lm[0] += (*(const LDS_AS f32x2*)(lds + L::L_LM + 8 * (32 * (hb + 2) + n)))[0];
            // the final output of an unsplit request takes the attention sink
            // as an extra exp-sum term 2^(sink log2(e) - m) (split requests: in
            // the combine)
            float den = lm[0];
            if (nsplit == 1 && p.attn_sink != nullptr && 32 * hb + n < p.h_q)
                den += __builtin_amdgcn_exp2f(p.attn_sink[32 * hb + n] * 1.4426950408889634f - lm[1]);
            inv[hb] = lm[0] == 0.f ? 0.f : 1.0f / den;        // a NaN sum (NaN in the cache) stays NaN
        }
        const int own_head = 32 * wave + n;
        if (nsplit == 1) {
            // O/l as bf16 through LDS, so that every store writes whole
            // 256-byte row segments: the wave's 128 dims of head r at
            // 32768 w + 256 r, its 16-byte chunk c at position c ^ (r % 16)
            // (conflict-free column writes), read back four heads per
            // instruction.  The LDS below 128 KB is free here: the tiles are
            // done and the head statistics live above it.
            static_assert(L::L_LM >= NW * 32768, "epilogue transpose area");
            uint16_t* obase = p.out + (int64_t)req * p.out_sb + (int64_t)sq * p.out_ss + 128 * wave;
            const int treg = wave * 32768;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {                   // 64 heads: blocks 0 and 1 only
                const int r = 32 * hb + n;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x16& o = O[4 * j + hb];
                        const u32x2 w = {pack_bf16(o[4 * g] * inv[hb], o[4 * g + 1] * inv[hb]),
                                         pack_bf16(o[4 * g + 2] * inv[hb], o[4 * g + 3] * inv[hb])};
                        *(LDS_AS u32x2*)(lds + treg + 256 * r + 16 * ((4 * j + g) ^ (r & 15)) + 8 * h) = w;
                    }
            }
            const int k = lane & 15;
#pragma unroll
            for (int i = 0; i < 8 * HB; ++i) {
                const int r = 4 * i + (lane >> 4);
                const u32x4 v = lds_read16(lds, treg + 256 * r + 16 * (k ^ (r & 15)));
                *(u32x4*)(obase + (int64_t)r * p.out_sh + 8 * k) = v;
            }
            if (h == 0 && own_head < p.h_q)
                p.lse[((int64_t)req * p.h_q + own_head) * p.s_q + sq] =
                    l_tot == 0.f ? INFINITY : (__log2f(l_tot) + m_ref) * 0.69314718055994531f;
        } else {
            // normalised partial O/l as bf16 in the lanes' own layout (packed
            // partials, see combine_packed_kernel) and lse in base 2
            const int split = req == begin_req ? begin_split : first_split;
            const int64_t row0 = ((int64_t)split * p.s_q + sq) * p.h_q;
            u32x4* dst = packed_partial(p, split, sq) + (int64_t)wave * 32 * 64 + lane;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if ((i & 3) >= HB) continue;                   // 64 heads: blocks 0 and 1 only
                const f32x16& o = O[i];
                const float sc = inv[i & 3];
#pragma unroll
                for (int half = 0; half < 2; ++half)
                    dst[(2 * i + half) * 64] = u32x4{pack_bf16(o[8 * half] * sc, o[8 * half + 1] * sc),
                                                     pack_bf16(o[8 * half + 2] * sc, o[8 * half + 3] * sc),
                                                     pack_bf16(o[8 * half + 4] * sc, o[8 * half + 5] * sc),
                                                     pack_bf16(o[8 * half + 6] * sc, o[8 * half + 7] * sc)};
            }
            if (h == 0 && own_head < p.h_q)
                p.lse_accum[row0 + own_head] = l_tot == 0.f ? -INFINITY : __log2f(l_tot) + m_ref;
        }
        __syncthreads();                                       // head statistics read
    }
}

// Test hook: gathers and stages every tile exactly as the decode kernel does
// (656-byte rows: copies into the raw slot, dequant into the staged tile;
// bf16 rows: copies straight into the staged tile) and reads the operands
// back through its two read paths (score A operands for K, transposing reads
// for V).  Rows of empty slots are the zero page.
template <int F>
__global__ void __launch_bounds__(NW * 64, 1) gather_h128_kernel(DecodeParams p, uint16_t* k_rows,
                                                                 uint16_t* v_rows) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
    LDS_AS uint8_t* lds = (LDS_AS uint8_t*)lds_raw;
    const int qi = blockIdx.x;                    // query token = req * s_q + sq
    const int req = qi / p.s_q, sq = qi % p.s_q;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 31, h = lane >> 5;
    const int32_t* idx = p.indices + (int64_t)req * p.idx_sb + (int64_t)sq * p.idx_ss;
    const int n_tiles = (p.topk + TILE - 1) / TILE;
    using L = Lay<F>;
    const uint32_t lds0 = lds_u32(lds);
    const int slice_off = L_RAW + wave * L::WAVE_RAW;
    const LDS_AS int32_t* slot = (const LDS_AS int32_t*)(lds + L::L_IDS + wave * IDS_SLOTS * 128);
    for (int it = 0; it < n_tiles; ++it) {
        __syncthreads();
        copy_ids(idx, 0, p.topk, it, lane, lds0 + L::L_IDS + wave * IDS_SLOTS * 128);
        wait_vmcnt<0>();
        const int kr = WROWS * wave + (lane >> 3);
        const bool ok = slot_ok(p, slot[n], it * TILE + n < p.topk);
        const bool okr = slot_ok(p, slot[kr], it * TILE + kr < p.topk);
        const uint32_t vm = (uint32_t)__ballot(ok);
        if constexpr (F == FB) {
            bf16_tile_copy(bf16_row(p, slot[kr], okr, kr), lane, wave, lds0 + L::L_KB);
            wait_vmcnt<0>();
        } else {
            gather_rows(row_addr<false>(p, slot[kr], okr, kr) + 16 * (lane & 7), lane, wave, lds0 + slice_off,
                        lds0 + L::L_KB + ROPE_OFF + 1024u * wave);
            wait_vmcnt<0>();
            stage_rows<F32>(lds, slice_off, L::L_KB, wave, lane);
        }
        __syncthreads();
        const int key = it * TILE + n;
        if (wave < 2 && key < p.topk) {
            uint16_t* dst = k_rows + ((int64_t)qi * p.topk + key) * 576 + 288 * wave + 8 * h;
            const bool kok = (vm >> n) & 1u;
            for (int j = 0; j < 18; ++j) {
                // the score operand read of k-step 18 w + j
                u32x4 v = lds_read16(lds, L::L_KB + qk_off(lane, 18 * wave + j));
                if (!kok) v = u32x4{0, 0, 0, 0};
                *(u32x4*)(dst + 16 * j) = v;
            }
        }
        if (v_rows != nullptr && wave >= 2) {
            const int vb = L::L_KB + pv_base(lane);
            for (int mb = 8 * (wave - 2); mb < 8 * (wave - 1); ++mb) {
                for (int tt = 0; tt < 2; ++tt) {
                    const u32x4 r = __builtin_bit_cast(u32x4, v_frag(lds, vb + tt * 16 * NP + mb * 64));
                    for (int e = 0; e < 8; ++e) {
                        const int q = e & 3, rr = e >> 2;
                        const int k = it * TILE + 16 * tt + 8 * (q & 1) + 4 * (q >> 1) + 2 * h + rr;
                        if (k < p.topk) {
                            const uint16_t val = (uint16_t)(r[e >> 1] >> (16 * (e & 1)));
                            v_rows[((int64_t)qi * p.topk + k) * 512 + 32 * mb + n] = val;
                        }
                    }
                }
            }
        }
    }
}

// Split-KV combine over packed partials ("FlashMLA Sparse Decode 完整计算过程详解",
// step 16): one wave per (query column, output block i = 4 j + hb of decode
// wave w), 64 waves per column (32 with 64 heads).  M = max_s lse_s (base 2),
// w_s = 2^(lse_s - M) / sum, out = sum_s w_s O_s, lse = (M + log2 sum) ln 2; out 0 and lse +inf
// when no split saw a valid key.  Splits are taken four at a time with their
// lse and partial loads issued together (one memory round trip per batch);
// a later batch with a larger max rescales what was accumulated so far.
// The work items (query column, piece) are taken query-major through the same
// XCD mapping as the decode's partitions, so a request's partials are read
// back on the XCD whose L2 received them (for b a multiple of 8 and a uniform
// plan exactly, otherwise approximately).
__global__ void __launch_bounds__(64) combine_packed_kernel(DecodeParams p) {
    const int item = xcd_part(blockIdx.x, gridDim.x);
    // 128 heads: 64 pieces per column (piece = 16 w + 4 j + hb); 64 heads: the
    // 32 of head blocks 0 and 1 only (8 w + 2 j + hb)
    const bool h64 = p.h_q == 64;
    const int qi = h64 ? item >> 5 : item >> 6;
    const int piece = h64 ? (((item >> 1) & 15) << 2) | (item & 1) : item & 63;
    const int req = qi / p.s_q, sq = qi % p.s_q;
    const int first = split_prefix(p, req);
    const int ns = split_prefix(p, req + 1) - first;
    const bool poison = lengths_missing(p);                  // contract error: NaN everywhere
    if (ns <= 1 && !poison) return;
    const int lane = threadIdx.x, n = lane & 31, h = lane >> 5;
    const int w = piece >> 4, j = (piece >> 2) & 3, hb = piece & 3;
    const int head = 32 * hb + n;
    const float* lse_col = p.lse_accum + (int64_t)first * p.s_q * p.h_q + (int64_t)sq * p.h_q + head;
    const int64_t lse_step = (int64_t)p.s_q * p.h_q;
    const int64_t kofs = (int64_t)w * 32 * 64 + (2 * (4 * j + hb)) * 64 + lane;
    float M = -INFINITY, W = 0.f;
    bool nan_lse = false;                                    // a split saw NaN (NaN in the cache)
    f32x16 acc = {};
    for (int s0 = 0; s0 < (poison ? 0 : ns); s0 += 4) {
        float lv[4];
        u32x4 raw[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int s = min(s0 + u, ns - 1);
            lv[u] = lse_col[s * lse_step];
            const u32x4* src = packed_partial(p, first + s, sq) + kofs;
            raw[u][0] = src[0];
            raw[u][1] = src[64];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (s0 + u >= ns) lv[u] = -INFINITY;
            nan_lse |= lv[u] != lv[u];
        }
        const float Mn = fmaxf(fmaxf(M, fmaxf(lv[0], lv[1])), fmaxf(lv[2], lv[3]));
        if (Mn == -INFINITY) continue;                     // no valid key so far
        const float keep = __builtin_amdgcn_exp2f(M - Mn);  // 0 while M is -inf
        W *= keep;
        acc *= keep;
        M = Mn;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float ws = __builtin_amdgcn_exp2f(lv[u] - M);
            W += ws;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t word = raw[u][e >> 3][(e >> 1) & 3];
                const float x = __builtin_bit_cast(float, (e & 1) ? (word & 0xffff0000u) : (word << 16));
                acc[e] += ws * x;
            }
        }
    }
    // an attention sink adds 2^(sink log2(e) - M) to the exp-sum (base 2, in
    // units of 2^M); lse stays that of the real slots
    const float den = p.attn_sink != nullptr && W > 0.f
                          ? W + __builtin_amdgcn_exp2f(p.attn_sink[head] * 1.4426950408889634f - M)
                          : W;
    const bool nan_out = poison || nan_lse;
    const float inv = nan_out ? __builtin_nanf("") : W > 0.f ? 1.0f / den : 0.f;
    // lane (n, h) holds dims 8 g + 4 h .. + 3 (g < 4) of the piece's 32; one
    // swap between the half-waves gives lane (n, h) dims 16 h .. 16 h + 15,
    // written as two 16-byte stores
    uint32_t wd[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        wd[2 * g] = pack_bf16(acc[4 * g] * inv, acc[4 * g + 1] * inv);
        wd[2 * g + 1] = pack_bf16(acc[4 * g + 2] * inv, acc[4 * g + 3] * inv);
    }
    uint32_t mine[4], theirs[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t send = h ? wd[k] : wd[4 + k];      // the other half's dims
        const auto sw = __builtin_amdgcn_permlane32_swap(send, send, false, false);
        theirs[k] = h ? sw[0] : sw[1];
        mine[k] = h ? wd[4 + k] : wd[k];
    }
    uint16_t* orow = p.out + (int64_t)req * p.out_sb + (int64_t)sq * p.out_ss + (int64_t)head * p.out_sh +
                     128 * w + 32 * j + 16 * h;
#pragma unroll
    for (int q = 0; q < 2; ++q)
        *(u32x4*)(orow + 8 * q) = h ? u32x4{theirs[2 * q], theirs[2 * q + 1], mine[2 * q], mine[2 * q + 1]}
                                    : u32x4{mine[2 * q], mine[2 * q + 1], theirs[2 * q], theirs[2 * q + 1]};
    if (w == 0 && j == 0 && h == 0)
        p.lse[((int64_t)req * p.h_q + head) * p.s_q + sq] =
            nan_out ? __builtin_nanf("") : M == -INFINITY ? INFINITY : (M + __log2f(W)) * 0.69314718055994531f;
}

// per instance: dynamic LDS size allowed (FLAT, DENSE, H64, format 656 / V4 / V4.1 / V4.1 + FP4)
bool g_lds_decode[2][2][2][5] = {}, g_lds_gather[2] = {};

template <typename K>
hipError_t allow_lds_once(K k, bool& done, int bytes) {
    if (done) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done = true;
    return e;
}

template <bool FLAT, bool DENSE, bool H64, int F, bool EXTRA = false>
hipError_t launch_h128(const DecodeParams& p, int num_parts, hipStream_t st) {
    constexpr int fi = F == F32 ? 0 : F == F4 ? 1 : F == FB ? 4 : EXTRA ? 3 : 2;
    constexpr int bytes = Lay<F, H64>::L_BYTES;
    hipError_t e = allow_lds_once(decode_fp8_h128_kernel<FLAT, DENSE, H64, F, EXTRA>,
                                  g_lds_decode[FLAT][DENSE][H64][fi], bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_fp8_h128_kernel<FLAT, DENSE, H64, F, EXTRA>), dim3(num_parts, p.s_q), dim3(NW * 64),
                       bytes, st, p);
    return hipGetLastError();
}
template <int F>
hipError_t launch_gather_t(const DecodeParams& p, uint16_t* k_rows, uint16_t* v_rows, hipStream_t st) {
    hipError_t e = allow_lds_once(gather_h128_kernel<F>, g_lds_gather[F == FB], Lay<F>::L_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gather_h128_kernel<F>, dim3(p.b * p.s_q), dim3(NW * 64), Lay<F>::L_BYTES, st, p, k_rows,
                       v_rows);
    return hipGetLastError();
}
template <bool FLAT, bool DENSE, int F = F32, bool EXTRA = false>
hipError_t launch_h128_heads(const DecodeParams& p, int num_parts, hipStream_t st) {
    return p.h_q == 64 ? launch_h128<FLAT, DENSE, true, F, EXTRA>(p, num_parts, st)
                       : launch_h128<FLAT, DENSE, false, F, EXTRA>(p, num_parts, st);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int kv_format, int num_parts, hipStream_t st) {
    if (kv_format == MLA_KV_BF16_576) return launch_h128_heads<false, false, FB>(p, num_parts, st);
    if (kv_format == MLA_KV_V4_584) return launch_h128_heads<false, false, F4>(p, num_parts, st);
    if (kv_format == MLA_KV_V41_528)
        return p.x_kv != nullptr ? launch_h128_heads<false, false, F41, true>(p, num_parts, st)
                                 : launch_h128_heads<false, false, F41>(p, num_parts, st);
    const bool dense = p.block_table != nullptr;
    if (p.kv_flat)
        return dense ? launch_h128_heads<true, true>(p, num_parts, st) : launch_h128_heads<true, false>(p, num_parts, st);
    return dense ? launch_h128_heads<false, true>(p, num_parts, st) : launch_h128_heads<false, false>(p, num_parts, st);
}

hipError_t launch_combine(const DecodeParams& p, hipStream_t st) {
    hipLaunchKernelGGL(combine_packed_kernel, dim3(p.b * p.s_q * (p.h_q == 64 ? 32 : 64)), dim3(64), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_gather(const DecodeParams& p, int kv_format, uint16_t* k_rows, uint16_t* v_rows,
                         hipStream_t st) {
    return kv_format == MLA_KV_BF16_576 ? launch_gather_t<FB>(p, k_rows, v_rows, st)
                                        : launch_gather_t<F32>(p, k_rows, v_rows, st);
}

}  // namespace mla
