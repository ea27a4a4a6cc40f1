"""CPU oracle for DeepSeek-V3.2-style sparse MLA decode.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
__graft_entry__ and the CPU-baseline leg of bench.py may import this module.
The product path (the HIP library and its Python binding) never calls it, and
this module shares no code, table or constant generator with that path.

Everything here is the plain definition, written out slowly in float64 with
numpy (a matrix product, max, exp and log from the library are the only
primitives used; no blocking, fusion or online rescaling):

* e4m3fn decode -- the pages give the FP8 format as 1 sign, 4 exponent and
  3 mantissa bits with range +-448 ("FlashMLA Sparse Decode 完整计算过程详解",
  step 4.3, hardware note).  Subnormals (exponent field 0) and the NaN codes
  (S.1111.111) are not spelled out there; the OCP E4M3 "fn" encoding is taken
  (bias 7, subnormal = m/8 * 2^-6, no infinities).
* 656-byte token row -- same page, step 2.2 and step 4.3: bytes [0,512) e4m3
  NoPE codes, [512,528) four little-endian fp32 scales (one per 128 NoPE
  dims), [528,656) 64 little-endian bf16 RoPE values.  Dequant is
  code * scale (step 7.4); K = [NoPE || RoPE] (576 dims) and V = NoPE (512).
* paged addressing -- step 7.2: block = idx // page_block_size,
  offset = idx % page_block_size.  An index names a physical token; -1 is an
  empty slot (step 1, step 7.7).  Indices outside [0, num_tokens) are treated
  as empty as well (the sparse-prefill contract in "FlashMLA 与 DSA：内核、
  流水线和正确性边界" section 4.0 calls -1 or out-of-range invalid).
* attention -- "FlashMLA 与 DSA：内核、流水线和正确性边界" section 4.3 gives
  the reference semantics: gather the selected rows, scores = q K^T * sm_scale,
  invalid slots -> -inf, lse = logsumexp(scores), out = exp(scores - lse) V.
  A slot that repeats a token counts once per slot.  When no slot is valid the
  sparse-decode walkthrough (step 14.2) writes lse = +inf; out is then 0.
* valid length and attention sink -- "FlashMLA 与 DSA" section 4.3: a slot
  whose position is at or past topk_length[b] is invalid like -1, and an
  attention sink (one logit per head, natural log) scales the output by
  1 / (1 + exp(attn_sink - lse)) while lse stays the log-sum-exp of the real
  slots.  Walkthrough step 13 gives the same as an extra "sink" token whose
  value row is zero (output scale 1 / (l + 2^(sink log2(e) - m)) in base-2
  terms).  Lengths are clamped to [0, topk] (the pages do not say what a
  negative or larger length means; this reading makes them none / all).
* dense decode -- walkthrough step 1 (no indices: block_table +
  cache_seqlens, every page of the request walked in block-table order) and
  "FlashMLA 与 DSA" section 3.3.  Request b sees its first cache_seqlens[b]
  logical tokens (clamped to the block table's capacity); with causal and
  s_q > 1 the query tokens are the last s_q positions, token j seeing
  cache_seqlens[b] - (s_q - 1 - j) of them (the pages do not spell this
  out; it is the plain reading of multi-token decode).
* V4 / V4.1 caches (d_qk = 512) -- "FlashMLA 与 DSA：内核、流水线和正确性
  边界" section 3.1 gives only this: the pages are struct-of-arrays (a page
  block holds its data rows first, then its scale rows), the scale type is
  float8_e8m0, the groups shrink to 64 (V4) and 32 (V4.1) elements, and a
  token takes 584 (V4) or 528 (V4.1) bytes.  The sparse-decode walkthrough,
  step 2.3, has the model type follow d_qk (576: V3.2, 512: the newer
  model), so d_qk = 512; "FlashMLA 与 DSA" section 6.1 limits sparse decode
  to d_qk of 512 or 576 with d_v = 512.  Readings taken (the byte counts admit
  no other split): V4 data row = 448 e4m3 codes (dims 0..447, one scale per
  64) then 64 little-endian bf16 values (dims 448..511, not quantised, as the
  RoPE part of V3.2), scale row = 7 e8m0 bytes and one pad byte; V4.1 data
  row = 512 e4m3 codes, scale row = 16 e8m0 bytes (one per 32 dims).  A page
  of P tokens: P data rows back to back, then P scale rows.  An e8m0 byte e
  is 2^(e - 127), 0xFF is NaN (the OCP E8M0 encoding; the pages say only
  "pure power of two, no mantissa").  V = K (d_v = d_qk = 512: the first
  d_v dims of K, as for V3.2).
* FP4 extra cache -- "FlashMLA 与 DSA" section 3.1 lists a 288-byte FP4
  token with e8m0 scales per 16 elements, section 6.1 allows FP4 only as an
  extra cache beside a V4.1 main cache, section 3.2 has split-KV decided on
  topk + extra_topk and section 3.5 has the decode walk the main and the
  extra blocks in one loop per format: a query token attends over its topk
  main slots and its extra_topk extra slots in one softmax.  Readings taken: the token is 512
  OCP E2M1 values (256 bytes, element 2i in the low nibble of byte i) and 32
  e8m0 scales (one per 16 dims), pages struct-of-arrays as for V4.1
  (section 3.1 says FP4 scales are e8m0 here, while the kernel table of
  section 2 pairs FP4 with e4m3; e8m0 is taken); extra slots are valid under
  the same rules as main slots (an id in [0, extra tokens), before an extra
  valid length when one is given); V = K.
* split-KV combine -- walkthrough step 14.2 (split partials are normalised
  O_j and lse_j = log2(l_j) + m_j in base 2, -inf when empty) and step 16
  (max over splits, weights 2^(lse_j - max), weighted mean of the O_j);
  "FlashMLA 与 DSA" section 3.2 states the same merge.
* tile scheduler -- walkthrough step 3 (blocks per request = ceil(topk/64),
  a fixed overhead of 5 blocks per request, payload = ceil(total/parts) +
  overhead, partitions filled left to right, a request that does not fit is
  split).  The block size, overhead and partition count are parameters here.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

NOPE = 512
ROPE = 64
DQK = NOPE + ROPE
DV = 512
ROW_FP8 = 656
ROW_BF16 = 2 * DQK

FMT_FP8 = 0
FMT_BF16 = 1
FMT_V4 = 2          # 584 B per token: 448 e4m3 + 64 bf16 | 7 e8m0 + pad
FMT_V41 = 3         # 528 B per token: 512 e4m3 | 16 e8m0

DQK_MODEL1 = 512
# struct-of-arrays formats: data bytes, scale bytes per token, e4m3 dims, dims per scale
SOA_LAYOUT = {FMT_V4: (576, 8, 448, 64), FMT_V41: (512, 16, 512, 32)}
FMT_FP4 = 4         # 288 B per token: 512 e2m1 (two per byte) | 32 e8m0 (extra cache only)
FP4_LAYOUT = (256, 32, 512, 16)


def dqk_of(kv_format: int) -> int:
    return DQK_MODEL1 if kv_format in SOA_LAYOUT else DQK


# ----------------------------------------------------------------------------
# element decoders
# ----------------------------------------------------------------------------
def e4m3fn_value(code: np.ndarray) -> np.ndarray:
    """uint8 e4m3fn codes -> float64 values (exact)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, val)
    return sign * val


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def e8m0_value(code: np.ndarray) -> np.ndarray:
    """uint8 e8m0 scale bytes -> float64: 2^(e - 127), NaN for 0xFF."""
    e = np.asarray(code, dtype=np.int64)
    return np.where(e == 0xFF, np.nan, np.exp2(e.astype(np.float64) - 127.0))


def e2m1_value(nib: np.ndarray) -> np.ndarray:
    """4-bit e2m1 codes (0..15) -> float64: sign bit 3, exponent bits 2..1
    (bias 1, field 0 subnormal), mantissa bit 0."""
    c = np.asarray(nib, dtype=np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    val = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0))
    return sign * val


def f32le_value(b4: np.ndarray) -> np.ndarray:
    """[..., 4] uint8 little-endian -> float64."""
    b4 = np.ascontiguousarray(b4, dtype=np.uint8)
    return b4.view("<f4")[..., 0].astype(np.float64)


# ----------------------------------------------------------------------------
# row decoders
# ----------------------------------------------------------------------------
def decode_fp8_rows(rows: np.ndarray) -> np.ndarray:
    """uint8 [..., 656] -> K float64 [..., 576] (V is K[..., :512])."""
    rows = np.asarray(rows, dtype=np.uint8)
    lead = rows.shape[:-1]
    codes = rows[..., :NOPE]
    scales = f32le_value(rows[..., NOPE:NOPE + 16].reshape(*lead, 4, 4))   # [..., 4]
    nope = e4m3fn_value(codes).reshape(*lead, 4, 128) * scales[..., None]
    rope_bits = np.ascontiguousarray(rows[..., 528:656]).view("<u2")
    rope = bf16_value(rope_bits)
    return np.concatenate([nope.reshape(*lead, NOPE), rope], axis=-1)


def decode_bf16_rows(rows: np.ndarray) -> np.ndarray:
    """uint8 [..., 1152] (576 little-endian bf16) -> float64 [..., 576]."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    return bf16_value(rows.view("<u2"))


def decode_v4_rows(data: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """V4: data uint8 [..., 576], scales uint8 [..., 8] -> K float64 [..., 512]."""
    data = np.asarray(data, dtype=np.uint8)
    lead = data.shape[:-1]
    sc = e8m0_value(np.asarray(scales, dtype=np.uint8)[..., :7])               # [..., 7]
    q = e4m3fn_value(data[..., :448]).reshape(*lead, 7, 64) * sc[..., None]
    tail = bf16_value(np.ascontiguousarray(data[..., 448:576]).view("<u2"))    # [..., 64]
    return np.concatenate([q.reshape(*lead, 448), tail], axis=-1)


def decode_v41_rows(data: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """V4.1: data uint8 [..., 512], scales uint8 [..., 16] -> K float64 [..., 512]."""
    data = np.asarray(data, dtype=np.uint8)
    lead = data.shape[:-1]
    sc = e8m0_value(np.asarray(scales, dtype=np.uint8))                        # [..., 16]
    q = e4m3fn_value(data).reshape(*lead, 16, 32) * sc[..., None]
    return q.reshape(*lead, 512)


def decode_fp4_rows(data: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """FP4: data uint8 [..., 256] (element 2i in the low nibble of byte i),
    scales uint8 [..., 32] -> K float64 [..., 512]."""
    data = np.asarray(data, dtype=np.uint8)
    lead = data.shape[:-1]
    nib = np.stack([data & 0xF, data >> 4], axis=-1).reshape(*lead, 512)
    sc = e8m0_value(np.asarray(scales, dtype=np.uint8))                        # [..., 32]
    return (e2m1_value(nib).reshape(*lead, 32, 16) * sc[..., None]).reshape(*lead, 512)


def soa_token_bytes(kv: np.ndarray, kv_format: int, ids: np.ndarray,
                    page_block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """Data and scale bytes of tokens `ids` in a struct-of-arrays cache.

    kv: uint8 [num_blocks, page_stride] (page_stride >= P * bytes per token);
    token t lives in page t // P at offset o = t % P: data row at o * data_b,
    scale row at P * data_b + o * scale_b."""
    data_b, scale_b, _, _ = FP4_LAYOUT if kv_format == FMT_FP4 else SOA_LAYOUT[kv_format]
    P = page_block_size
    ids = np.asarray(ids, dtype=np.int64)
    blk, off = ids // P, ids % P
    d_cols = off[..., None] * data_b + np.arange(data_b)
    s_cols = P * data_b + off[..., None] * scale_b + np.arange(scale_b)
    return kv[blk[..., None], d_cols], kv[blk[..., None], s_cols]


def token_rows(kv: np.ndarray, kv_format: int) -> np.ndarray:
    """View the cache as [num_tokens, row_bytes] bytes (fp8: [nb, P, 1, 656])."""
    if kv_format == FMT_FP8:
        nb, P, hk, rb = kv.shape
        assert hk == 1 and rb == ROW_FP8
        return kv.reshape(nb * P, ROW_FP8)
    s_kv, rb = kv.shape
    assert rb == ROW_BF16
    return kv


def num_tokens_of(kv: np.ndarray, kv_format: int, page_block_size: int = 1) -> int:
    if kv_format in SOA_LAYOUT or kv_format == FMT_FP4:
        return kv.shape[0] * page_block_size
    return kv.shape[0] * kv.shape[1] if kv_format == FMT_FP8 else kv.shape[0]


def slot_valid(indices: np.ndarray, num_tokens: int) -> np.ndarray:
    idx = np.asarray(indices, dtype=np.int64)
    return (idx >= 0) & (idx < num_tokens)


def gather_dequant(kv: np.ndarray, indices: np.ndarray, kv_format: int,
                   page_block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """Rows selected by `indices` [..., topk], decoded to float64
    [..., topk, d_qk] (576, or 512 for the V4 / V4.1 caches).

    Empty slots give zero rows.  Returns (rows, valid_mask)."""
    P = page_block_size if kv_format != FMT_BF16 else 1
    n_tok = num_tokens_of(kv, kv_format, P)
    idx = np.asarray(indices, dtype=np.int64)
    valid = slot_valid(idx, n_tok)
    safe = np.where(valid, idx, 0)
    if kv_format in SOA_LAYOUT or kv_format == FMT_FP4:
        data, scales = soa_token_bytes(kv, kv_format, safe, P)
        dec = {FMT_V4: decode_v4_rows, FMT_V41: decode_v41_rows, FMT_FP4: decode_fp4_rows}[kv_format]
        rows = dec(data, scales)
    elif kv_format == FMT_FP8:
        # page / offset addressing (identical to flat row idx for a dense [nb, P] cache)
        raw = kv[safe // P, safe % P, 0]
        rows = decode_fp8_rows(raw)
    else:
        rows = decode_bf16_rows(token_rows(kv, kv_format)[safe])
    rows = np.where(valid[..., None], rows, 0.0)
    return rows, valid


# ----------------------------------------------------------------------------
# attention (definition)
# ----------------------------------------------------------------------------
def logsumexp(s: np.ndarray) -> np.ndarray:
    """Natural-log log-sum-exp over the last axis (max taken out first)."""
    m = s.max(axis=-1, keepdims=True)
    return m[..., 0] + np.log(np.exp(s - m).sum(axis=-1))


def attend(qh: np.ndarray, K: np.ndarray, V: np.ndarray, valid: np.ndarray,
           sm_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One query token.  qh [H, d_qk], K [n, d_qk], V [n, 512], valid [n].

    Returns out [H, 512] and natural-log lse [H] (float64); +inf / 0 when no
    slot is valid."""
    H = qh.shape[0]
    if not np.any(valid):
        return np.zeros((H, DV)), np.full(H, np.inf)
    s = (qh @ K.T) * sm_scale                          # [H, n]
    s = np.where(valid[None, :], s, -np.inf)
    lse = logsumexp(s)
    w = np.exp(s - lse[:, None])
    return w @ V, lse


def sink_factor(lse: np.ndarray, attn_sink: np.ndarray) -> np.ndarray:
    """Output factor of an attention sink: 1 / (1 + exp(sink - lse)) per head;
    1 where lse is +inf (no valid slot: the output is 0 anyway)."""
    lse = np.asarray(lse, dtype=np.float64)
    sink = np.asarray(attn_sink, dtype=np.float64)
    fin = np.isfinite(lse)
    return np.where(fin, 1.0 / (1.0 + np.exp(sink - np.where(fin, lse, 0.0))), 1.0)


def sparse_mla_decode(q_bits: np.ndarray, kv: np.ndarray, indices: np.ndarray,
                      sm_scale: float, kv_format: int, page_block_size: int,
                      queries: Optional[Iterable[Tuple[int, int]]] = None,
                      attn_sink: Optional[np.ndarray] = None,
                      topk_length: Optional[np.ndarray] = None,
                      extra: Optional[dict] = None):
    """Sparse MLA decode by definition.

    q_bits: uint16 bf16 [b, s_q, H, d_qk]; kv: fp8 uint8 [nb, P, 1, 656],
    bf16-row bytes uint8 [s_kv, 1152], or a V4 / V4.1 cache uint8
    [nb, page_stride] (d_qk = 512); indices int32 [b, s_q, topk];
    attn_sink: float [H] (natural log) or None; topk_length: int [b] or None.
    extra (V4.1 main cache only): {"kv": FP4 cache uint8 [nb, page_stride],
    "indices": int32 [b, s_q, extra_topk], "page_block_size": P, and
    optionally "topk_length": int [b]} -- its slots join the main ones.
    Returns out float64 [b, s_q, H, 512] and lse float64 [b, H, s_q]
    (natural log).  With `queries`, only those (bi, sj) pairs are filled and
    the others are NaN.
    """
    b, s_q, H, d = q_bits.shape
    assert d == dqk_of(kv_format)
    out = np.full((b, s_q, H, DV), np.nan)
    lse = np.full((b, H, s_q), np.nan)
    if queries is None:
        queries = [(bi, sj) for bi in range(b) for sj in range(s_q)]
    topk = indices.shape[-1]
    if extra is not None:
        assert kv_format == FMT_V41
    for bi, sj in queries:
        rows, valid = gather_dequant(kv, indices[bi, sj], kv_format, page_block_size)
        if topk_length is not None:
            n_ok = min(max(int(topk_length[bi]), 0), topk)
            valid = valid & (np.arange(topk) < n_ok)
            rows = np.where(valid[:, None], rows, 0.0)
        if extra is not None:
            xi = extra["indices"][bi, sj]
            xrows, xvalid = gather_dequant(extra["kv"], xi, FMT_FP4, extra["page_block_size"])
            if extra.get("topk_length") is not None:
                n_ok = min(max(int(extra["topk_length"][bi]), 0), len(xi))
                xvalid = xvalid & (np.arange(len(xi)) < n_ok)
                xrows = np.where(xvalid[:, None], xrows, 0.0)
            rows = np.concatenate([rows, xrows])
            valid = np.concatenate([valid, xvalid])
        qh = bf16_value(q_bits[bi, sj])
        o, l = attend(qh, rows, rows[:, :DV], valid, sm_scale)
        if attn_sink is not None:
            o = o * sink_factor(l, attn_sink)[:, None]
        out[bi, sj] = o
        lse[bi, :, sj] = l
    return out, lse


def dense_visible(seqlen: int, capacity: int, s_q: int, sj: int, causal: bool) -> int:
    """Tokens that query token sj of a request sees in dense decode: its
    cache length clamped to [0, capacity]; with causal, the s_q query tokens
    are the last s_q positions of the sequence, so token sj sees
    seqlen - (s_q - 1 - sj) of them (never fewer than none)."""
    n = max(0, min(int(seqlen), capacity))
    if causal:
        n = max(0, n - (s_q - 1 - sj))
    return n


def dense_mla_decode(q_bits: np.ndarray, kv: np.ndarray, block_table: np.ndarray,
                     cache_seqlens: np.ndarray, sm_scale: float, page_block_size: int,
                     causal: bool = False, queries: Optional[Iterable[Tuple[int, int]]] = None,
                     attn_sink: Optional[np.ndarray] = None):
    """Dense MLA decode by definition ("FlashMLA Sparse Decode 完整计算过程详解",
    step 1: without indices the call takes block_table + cache_seqlens and
    walks every page of a request in block-table order; "FlashMLA 与 DSA"
    section 3.3 for the dense decode itself).

    Request b attends to its logical tokens t < cache_seqlens[b] (see
    dense_visible for causal), token t living at physical id
    block_table[b, t // P] * P + t % P of the FP8 cache kv [nb, P, 1, 656].
    Returns out float64 [b, s_q, H, 512] and natural-log lse [b, H, s_q]
    (+inf / 0 when a query sees no token).  With `queries`, only those
    (bi, sj) pairs are filled (NaN elsewhere)."""
    b, s_q, H, d = q_bits.shape
    assert d == DQK
    P = page_block_size
    capacity = block_table.shape[1] * P
    out = np.full((b, s_q, H, DV), np.nan)
    lse = np.full((b, H, s_q), np.nan)
    if queries is None:
        queries = [(bi, sj) for bi in range(b) for sj in range(s_q)]
    for bi, sj in queries:
        n = dense_visible(cache_seqlens[bi], capacity, s_q, sj, causal)
        t = np.arange(n, dtype=np.int64)
        phys = np.asarray(block_table[bi], dtype=np.int64)[t // P] * P + t % P
        rows, valid = gather_dequant(kv, phys, FMT_FP8, P)
        qh = bf16_value(q_bits[bi, sj])
        o, l = attend(qh, rows, rows[:, :DV], valid, sm_scale)
        if attn_sink is not None:
            o = o * sink_factor(l, attn_sink)[:, None]
        out[bi, sj] = o
        lse[bi, :, sj] = l
    return out, lse


def partial_attention(qh, K, V, valid, sm_scale):
    """Split partial over a subset of slots in the form a split writes:
    normalised O_j [H, 512] and lse_j in base 2 (-inf when the subset is empty)."""
    o, l = attend(qh, K, V, valid, sm_scale)
    lse2 = np.where(np.isinf(l), -np.inf, l / math.log(2.0))
    o = np.where(np.isinf(l)[:, None], 0.0, o)
    return o, lse2


def splitkv_combine(o_parts: np.ndarray, lse2_parts: np.ndarray):
    """Merge split partials.  o_parts [n, H, 512] (normalised), lse2_parts [n, H]
    (base 2).  Returns out [H, 512] and natural-log lse [H]."""
    lse2 = np.asarray(lse2_parts, dtype=np.float64)
    M = lse2.max(axis=0)                                   # [H]
    empty = np.isneginf(M)
    Ms = np.where(empty, 0.0, M)
    w = np.exp2(lse2 - Ms[None, :])                        # [n, H]; 0 for -inf parts
    tot = w.sum(axis=0)
    out = (w[:, :, None] * o_parts).sum(axis=0) / np.where(empty, 1.0, tot)[:, None]
    out = np.where(empty[:, None], 0.0, out)
    lse = np.where(empty, np.inf, (Ms + np.log2(np.where(empty, 1.0, tot))) * math.log(2.0))
    return out, lse


# ----------------------------------------------------------------------------
# scheduler (greedy left-to-right partition fill)
# ----------------------------------------------------------------------------
SCHED_FIELDS = ("begin_req", "end_req", "begin_block", "end_block",
                "begin_split", "first_splitted", "last_splitted")


def sched_plan(topk_per_req: Sequence[int], block: int, overhead: int,
               num_parts: int) -> Tuple[List[Tuple[int, ...]], List[int]]:
    """Greedy tile scheduler.

    Returns (parts, prefix): parts[p] = (begin_req, end_req, begin_block,
    end_block, begin_split, first_splitted, last_splitted) with end_req
    inclusive and end_block exclusive (blocks of end_req); a partition with no
    work has begin_req == number of requests.  prefix[r] is the index of the
    first split of request r (prefix[-1] = total splits)."""
    n = len(topk_per_req)
    blocks = [(t + block - 1) // block for t in topk_per_req]
    total = sum(bl + overhead for bl in blocks)
    payload = (total + num_parts - 1) // num_parts + overhead if n else 0
    splits = [0] * n
    parts = []
    req, done_blocks, cursor = 0, 0, 0
    for _ in range(num_parts):
        if req >= n:
            parts.append((n, n, 0, 0, cursor, 0, 0))
            continue
        begin_req, begin_block = req, done_blocks
        first_splitted = int(done_blocks > 0)
        remain = payload
        end_req, end_block, last_splitted = req, done_blocks, 0
        while req < n:
            left = blocks[req] - done_blocks
            if left + overhead <= remain:
                remain -= left + overhead
                splits[req] += 1
                end_req, end_block, last_splitted = req, blocks[req], 0
                req, done_blocks = req + 1, 0
            else:
                take = remain - overhead
                if take > 0:
                    splits[req] += 1
                    done_blocks += take
                    end_req, end_block, last_splitted = req, done_blocks, 1
                break
        parts.append((begin_req, end_req, begin_block, end_block, cursor,
                      first_splitted, last_splitted))
        # number of splits this partition opened
        cursor += end_req - begin_req + 1
    prefix = [0]
    for s in splits:
        prefix.append(prefix[-1] + s)
    assert prefix[-1] == cursor
    return parts, prefix
