"""Seeded synthetic workloads for DeepSeek-V3.2-shaped sparse MLA decode.

This module only *builds inputs*: random Q, a paged FP8 KV cache in the
656-byte V3.2 token format (or a flat bf16 cache, or a V4 / V4.1
struct-of-arrays cache), and int32 top-k index lists.  It holds none of the decode arithmetic (no gather, no dequant, no
softmax) so that the CPU oracle and the HIP path can both consume its bytes
without sharing any of the computation they are checked on.

Sources for the shapes and formats (page titles as published):
  * "FlashMLA Sparse Decode 完整计算过程详解", step 0 (model constants:
    d_qk = 512 NoPE + 64 RoPE, d_v = 512, h_q = 128, index_topk = 2048,
    page_block_size = 64), step 1 (q / k_cache / indices shapes; an index is
    block * page_block_size + offset, -1 marks an empty slot), step 4
    (per-128 NoPE groups, power-of-two scale from amax/448, e4m3 codes,
    byte layout [0,512) codes, [512,528) four fp32 scales, [528,656) 64 bf16
    RoPE values).
  * "FlashMLA 与 DSA：内核、流水线和正确性边界", section 4.0 (sparse prefill
    takes logical indices into a flat kv[s_kv, d_qk] with no batch dim) and
    section 5.5 (logical positions are emitted through the page table).

  * "FlashMLA 与 DSA" section 3.1 (V4 / V4.1: pages hold their data rows,
    then their scale rows; e8m0 scales per 64 / 32 elements; 584 / 528 bytes
    per token) and the walkthrough's step 2.3 (d_qk 512 for those models).
    The V4 token is 448 e4m3 codes + 64 bf16 values | 7 scales + a zero pad
    byte; the V4.1 token 512 e4m3 codes | 16 scales.

The FP8 encoder below follows step 4.2 of the sparse-decode walkthrough:
amax per 128-group (clamped to 1e-4 so an all-zero group still gets a finite
scale), scale = 2**ceil(log2(amax / 448)), code = round-to-nearest-even
e4m3fn(x / scale).  Rounding to e4m3fn and to bf16 is delegated to PyTorch's
dtype conversions (library routines), not written here.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

D_NOPE = 512
D_ROPE = 64
D_QK = D_NOPE + D_ROPE
D_V = 512
FP8_ROW_BYTES = 656          # 512 e4m3 + 4 x fp32 + 64 x bf16
BF16_ROW_BYTES = D_QK * 2    # 1152
QUANT_GROUP = 128
E4M3_MAX = 448.0

KV_FP8_656 = 0
KV_BF16_576 = 1
KV_V4_584 = 2
KV_V41_528 = 3
D_QK_SOA = 512
# struct-of-arrays formats: (data bytes, scale bytes, e4m3 dims, dims per scale)
SOA = {KV_V4_584: (576, 8, 448, 64), KV_V41_528: (512, 16, 512, 32)}


def d_qk_of(kv_format: int) -> int:
    return D_QK_SOA if kv_format in SOA else D_QK


FP4_DATA, FP4_SCALE = 256, 32    # FP4 extra cache token: 512 e2m1 (two per byte) | 32 e8m0
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

BASE_SEED = 20261202


# ----------------------------------------------------------------------------
# conversions delegated to torch dtypes (library rounding)
# ----------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32/float64 array -> uint16 bf16 bit patterns, round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def encode_fp8_rows(nope: np.ndarray, rope_bits: np.ndarray) -> np.ndarray:
    """Pack rows into the 656-byte V3.2 token format.

    nope: float32 [n, 512] (values to quantise); rope_bits: uint16 [n, 64].
    Returns uint8 [n, 656].
    """
    n = nope.shape[0]
    x = nope.astype(np.float32).reshape(n, 4, QUANT_GROUP)
    amax = np.maximum(np.abs(x).max(axis=-1).astype(np.float64), 1e-4)
    ratio = amax / E4M3_MAX
    # smallest power of two >= ratio, exactly (frexp gives ratio = m * 2**e, m in [0.5, 1))
    m, e = np.frexp(ratio)
    exp = np.where(m == 0.5, e - 1, e)
    scale = np.ldexp(np.ones_like(ratio), exp).astype(np.float32)          # [n, 4]
    scaled = (x / scale[:, :, None]).astype(np.float32)                   # exact (power of two)
    assert np.all(np.abs(scaled) <= E4M3_MAX)
    codes = torch.from_numpy(scaled.reshape(n, D_NOPE)).to(torch.float8_e4m3fn)
    codes = codes.view(torch.uint8).numpy()
    rows = np.empty((n, FP8_ROW_BYTES), dtype=np.uint8)
    rows[:, :D_NOPE] = codes
    rows[:, 512:528] = scale.astype("<f4").view(np.uint8).reshape(n, 16)
    rows[:, 528:656] = rope_bits.astype("<u2").view(np.uint8).reshape(n, 128)
    return rows


def encode_soa_tokens(x: np.ndarray, kv_format: int) -> np.ndarray:
    """Quantise tokens x float32 [n, 512] for a V4 / V4.1 cache (step 4.2's
    recipe with e8m0 scales: amax per group clamped to 1e-4, scale =
    2**ceil(log2(amax / 448)), code = e4m3fn(x / scale); V4 dims 448.. as
    bf16).  Returns uint8 [n, data bytes + scale bytes]: the data row, then
    the scale row."""
    db, sb, nq, grp = SOA[kv_format]
    n = x.shape[0]
    g = x[:, :nq].astype(np.float32).reshape(n, nq // grp, grp)
    amax = np.maximum(np.abs(g).max(axis=-1).astype(np.float64), 1e-4)
    m, e = np.frexp(amax / E4M3_MAX)
    exp = np.where(m == 0.5, e - 1, e)                                     # [n, groups]
    scaled = (g / np.ldexp(np.ones_like(amax), exp)[:, :, None]).astype(np.float32)
    assert np.all(np.abs(scaled) <= E4M3_MAX)
    out = np.zeros((n, db + sb), dtype=np.uint8)
    out[:, :nq] = torch.from_numpy(scaled.reshape(n, nq)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    if nq < D_QK_SOA:
        out[:, nq:db] = to_bf16_bits(x[:, nq:]).astype("<u2").view(np.uint8).reshape(n, 2 * (D_QK_SOA - nq))
    out[:, db:db + nq // grp] = (exp + 127).astype(np.uint8)
    return out


def encode_fp4_tokens(x: np.ndarray) -> np.ndarray:
    """Quantise tokens x float32 [n, 512] for the FP4 extra cache: per 16
    dims, amax clamped to 1e-4, scale = 2**ceil(log2(amax / 6)), code = the
    nearest e2m1 value of x / scale (ties to the even code), element 2i in
    the low nibble of byte i.  Returns uint8 [n, 288]: data row, scale row."""
    n = x.shape[0]
    g = x.astype(np.float64).reshape(n, 32, 16)
    amax = np.maximum(np.abs(g).max(axis=-1), 1e-4)
    m, e = np.frexp(amax / 6.0)
    exp = np.where(m == 0.5, e - 1, e)                                     # [n, 32]
    y = g / np.ldexp(np.ones_like(amax), exp)[:, :, None]
    d = np.abs(np.abs(y)[..., None] - E2M1_GRID) + 1e-9 * (np.arange(8) % 2)
    code = (np.argmin(d, axis=-1) | np.where(y < 0, 8, 0)).astype(np.uint8).reshape(n, 512)
    out = np.empty((n, FP4_DATA + FP4_SCALE), dtype=np.uint8)
    out[:, :FP4_DATA] = code[:, 0::2] | (code[:, 1::2] << 4)
    out[:, FP4_DATA:] = (exp + 127).astype(np.uint8)
    return out


@dataclasses.dataclass
class ExtraCache:
    """An FP4 extra cache and its slots (beside a V4.1 main cache)."""
    page_block_size: int
    num_blocks: int
    indices: np.ndarray          # int32 [b, s_q, extra_topk]
    ref_ids: np.ndarray          # int64 sorted unique referenced tokens
    ref_rows: np.ndarray         # uint8 [n_ref, 288]
    page_pad: int = 0
    fill_byte: int = 0xFF

    @property
    def num_kv_tokens(self) -> int:
        return self.num_blocks * self.page_block_size

    @property
    def page_stride(self) -> int:
        return (self.page_block_size * (FP4_DATA + FP4_SCALE) + self.page_pad + 15) // 16 * 16

    def kv_host(self) -> np.ndarray:
        P = self.page_block_size
        kv = np.full((self.num_blocks, self.page_stride), self.fill_byte, dtype=np.uint8)
        data = kv[:, :P * FP4_DATA].reshape(-1, P, FP4_DATA)
        scales = kv[:, P * FP4_DATA:P * (FP4_DATA + FP4_SCALE)].reshape(-1, P, FP4_SCALE)
        blk, off = self.ref_ids // P, self.ref_ids % P
        data[blk, off] = self.ref_rows[:, :FP4_DATA]
        scales[blk, off] = self.ref_rows[:, FP4_DATA:]
        return kv

    def kv_device(self, device="cuda") -> torch.Tensor:
        return torch.from_numpy(self.kv_host()).to(device)

    def indices_device(self, device="cuda") -> torch.Tensor:
        return torch.from_numpy(self.indices).to(device)


# ----------------------------------------------------------------------------
# workload container
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    kv_format: int
    b: int
    s_q: int
    h_q: int
    topk: int
    sm_scale: float
    q_bits: np.ndarray           # uint16 [b, s_q, h_q, d_qk] (576; 512 for V4 / V4.1)
    indices: np.ndarray          # int32 [b, s_q, topk]
    page_block_size: int         # fp8: tokens per page; bf16: 1
    num_kv_tokens: int           # fp8: num_blocks * page_block_size; bf16: s_kv
    ref_ids: np.ndarray          # int64 [n_ref] sorted unique referenced token ids
    ref_rows: np.ndarray         # uint8 [n_ref, row_bytes] their bytes
    fill_byte: int = 0xFF        # bytes of unreferenced rows (0xFF = NaN codes/scales)
    meta: Optional[dict] = None
    page_pad: int = 0            # V4 / V4.1: bytes after each page's scale rows

    @property
    def row_bytes(self) -> int:
        """Bytes of one token (V4 / V4.1: data row + scale row)."""
        if self.kv_format in SOA:
            return sum(SOA[self.kv_format][:2])
        return FP8_ROW_BYTES if self.kv_format == KV_FP8_656 else BF16_ROW_BYTES

    @property
    def num_blocks(self) -> int:
        return self.num_kv_tokens // self.page_block_size

    @property
    def page_stride(self) -> int:
        """V4 / V4.1: bytes from one page to the next (the pages' bytes and
        page_pad, rounded up to 16: page starts are 16-byte aligned)."""
        return (self.page_block_size * self.row_bytes + self.page_pad + 15) // 16 * 16

    def _soa_views(self, kv):
        """(data [nb, P, D], scales [nb, P, S]) views of a V4 / V4.1 cache [nb, stride]."""
        db, sb = SOA[self.kv_format][:2]
        P = self.page_block_size
        return (kv[:, :P * db].unflatten(1, (P, db)) if isinstance(kv, torch.Tensor)
                else kv[:, :P * db].reshape(-1, P, db),
                kv[:, P * db:P * (db + sb)].unflatten(1, (P, sb)) if isinstance(kv, torch.Tensor)
                else kv[:, P * db:P * (db + sb)].reshape(-1, P, sb))

    def kv_host(self) -> np.ndarray:
        """Full cache as host bytes: fp8 -> uint8 [num_blocks, P, 1, 656];
        bf16 -> uint8 [s_kv, 1152] (row-major bf16 [s_kv, 576]); V4 / V4.1 ->
        uint8 [num_blocks, page_stride] (P data rows, P scale rows, pad)."""
        if self.kv_format in SOA:
            db = SOA[self.kv_format][0]
            kv = np.full((self.num_blocks, self.page_stride), self.fill_byte, dtype=np.uint8)
            data, scales = self._soa_views(kv)
            blk, off = self.ref_ids // self.page_block_size, self.ref_ids % self.page_block_size
            data[blk, off] = self.ref_rows[:, :db]
            scales[blk, off] = self.ref_rows[:, db:]
            return kv
        flat = np.full((self.num_kv_tokens, self.row_bytes), self.fill_byte, dtype=np.uint8)
        flat[self.ref_ids] = self.ref_rows
        if self.kv_format == KV_FP8_656:
            return flat.reshape(self.num_blocks, self.page_block_size, 1, FP8_ROW_BYTES)
        return flat

    def kv_device(self, device="cuda") -> torch.Tensor:
        """Same bytes as kv_host(), built on the device (fill + scatter of referenced rows)."""
        if self.kv_format in SOA:
            db = SOA[self.kv_format][0]
            kv = torch.full((self.num_blocks, self.page_stride), self.fill_byte, dtype=torch.uint8, device=device)
            if len(self.ref_ids):
                data, scales = self._soa_views(kv)
                ids = torch.from_numpy(self.ref_ids).to(device)
                blk, off = ids // self.page_block_size, ids % self.page_block_size
                rows = torch.from_numpy(self.ref_rows).to(device)
                data[blk, off] = rows[:, :db]
                scales[blk, off] = rows[:, db:]
            return kv
        flat = torch.full((self.num_kv_tokens, self.row_bytes), self.fill_byte,
                          dtype=torch.uint8, device=device)
        if len(self.ref_ids):
            idx = torch.from_numpy(self.ref_ids).to(device)
            flat.index_copy_(0, idx, torch.from_numpy(self.ref_rows).to(device))
        if self.kv_format == KV_FP8_656:
            return flat.view(self.num_blocks, self.page_block_size, 1, FP8_ROW_BYTES)
        return flat

    def q_device(self, device="cuda") -> torch.Tensor:
        return torch.from_numpy(self.q_bits.view(np.int16)).to(device).view(torch.bfloat16)

    def indices_device(self, device="cuda") -> torch.Tensor:
        return torch.from_numpy(self.indices).to(device)


def _fill_rows(rng, ids: np.ndarray, kv_format: int) -> np.ndarray:
    n = len(ids)
    if kv_format in SOA:
        return encode_soa_tokens(rng.standard_normal((n, D_QK_SOA), dtype=np.float32), kv_format)
    if kv_format == KV_FP8_656:
        nope = rng.standard_normal((n, D_NOPE), dtype=np.float32)
        rope = to_bf16_bits(rng.standard_normal((n, D_ROPE), dtype=np.float32))
        return encode_fp8_rows(nope, rope)
    vals = to_bf16_bits(rng.standard_normal((n, D_QK), dtype=np.float32))
    return vals.astype("<u2").view(np.uint8).reshape(n, BF16_ROW_BYTES)


def _finish(name, rng, kv_format, b, s_q, h_q, topk, P, num_tokens, indices, meta=None,
            q_bits=None, page_pad=0):
    dqk = d_qk_of(kv_format)
    if q_bits is None:
        q_bits = to_bf16_bits(rng.standard_normal((b, s_q, h_q, dqk), dtype=np.float32))
    valid = indices[(indices >= 0) & (indices < num_tokens)]
    ref_ids = np.unique(valid.astype(np.int64))
    ref_rows = _fill_rows(rng, ref_ids, kv_format)
    return Workload(name=name, kv_format=kv_format, b=b, s_q=s_q, h_q=h_q, topk=topk,
                    sm_scale=1.0 / np.sqrt(dqk), q_bits=q_bits, indices=indices,
                    page_block_size=P, num_kv_tokens=num_tokens, ref_ids=ref_ids,
                    ref_rows=ref_rows, meta=meta, page_pad=page_pad)


def _distinct(rng, n_pool: int, k: int) -> np.ndarray:
    """k distinct uniform draws from range(n_pool) (random order)."""
    if k > n_pool:
        raise ValueError("not enough candidates")
    if n_pool <= 4 * k:
        return rng.permutation(n_pool)[:k]
    out = np.unique(rng.integers(0, n_pool, size=int(k * 1.3) + 16))
    while len(out) < k:
        out = np.unique(np.concatenate([out, rng.integers(0, n_pool, size=k)]))
    return rng.permutation(rng.choice(out, size=k, replace=False))


def paged_decode(name: str, seed: int, b: int, s_q: int, h_q: int, topk: int,
                 tokens_per_seq: int, P: int = 64, shuffle_pages: bool = True,
                 short_frac: float = 0.0, short_len: int = 0,
                 recent_frac: float = 0.0, recent_window: int = 0,
                 sort_slots: bool = False, kv_format: int = KV_FP8_656, page_pad: int = 0) -> Workload:
    """Paged FP8 decode workload (the 656-byte cache, or with kv_format the
    V4 / V4.1 cache, whose pages may carry page_pad bytes after the scale
    rows).

    Each sequence owns tokens_per_seq/P pages; the page table is a global
    shuffled permutation (or contiguous when shuffle_pages=False).  Each query
    token picks `topk` distinct logical positions of its sequence (uniform, or
    `recent_frac` of them from the last `recent_window` positions), maps them
    through the page table, and (optionally) a seeded `short_frac` of the
    sequences keep only `short_len` valid slots followed by -1.
    """
    rng = np.random.default_rng(seed)
    pages_per_seq = tokens_per_seq // P
    total_pages = b * pages_per_seq
    perm = rng.permutation(total_pages) if shuffle_pages else np.arange(total_pages)
    block_table = perm.reshape(b, pages_per_seq)
    n_short = int(round(short_frac * b))
    short_seqs = np.sort(rng.choice(b, size=n_short, replace=False)) if n_short else np.zeros(0, int)
    indices = np.full((b, s_q, topk), -1, dtype=np.int32)
    short_set = set(short_seqs.tolist())
    for bi in range(b):
        n_valid = short_len if bi in short_set else topk
        for sj in range(s_q):
            if recent_frac > 0:
                n_recent = int(round(recent_frac * n_valid))
                rec = tokens_per_seq - recent_window + _distinct(rng, recent_window, n_recent)
                old = _distinct(rng, tokens_per_seq - recent_window, n_valid - n_recent)
                pos = rng.permutation(np.concatenate([rec, old]))
            else:
                pos = _distinct(rng, tokens_per_seq, n_valid)
            if sort_slots:
                pos = np.sort(pos)
            phys = block_table[bi, pos // P] * P + pos % P
            indices[bi, sj, :n_valid] = phys
    meta = {"block_table_shape": list(block_table.shape), "short_seqs": short_seqs.tolist()}
    return _finish(name, rng, kv_format, b, s_q, h_q, topk, P, total_pages * P, indices, meta,
                   page_pad=page_pad)


def extra_decode(name: str, seed: int, b: int, s_q: int, h_q: int, topk: int, extra_topk: int,
                 tokens_per_seq: int, extra_tokens_per_seq: int, P: int = 64, extra_P: int = 64,
                 extra_pad: int = 0) -> Workload:
    """A V4.1 paged decode workload (topk main slots per query token) with an
    FP4 extra cache in meta["extra"] (ExtraCache): every request owns
    extra_tokens_per_seq / extra_P pages of it, dealt from a shuffled
    permutation, and each query token picks extra_topk distinct positions of
    them."""
    w = paged_decode(name, seed, b, s_q, h_q, topk, tokens_per_seq, P=P, kv_format=KV_V41_528)
    rng = np.random.default_rng(seed + 7919)
    pages = extra_tokens_per_seq // extra_P
    table = rng.permutation(b * pages).reshape(b, pages)
    idx = np.full((b, s_q, extra_topk), -1, dtype=np.int32)
    for bi in range(b):
        for sj in range(s_q):
            pos = _distinct(rng, extra_tokens_per_seq, extra_topk)
            idx[bi, sj] = table[bi, pos // extra_P] * extra_P + pos % extra_P
    ref = np.unique(idx[idx >= 0].astype(np.int64))
    rows = encode_fp4_tokens(rng.standard_normal((len(ref), D_QK_SOA), dtype=np.float32))
    w.meta = dict(w.meta or {}, extra=ExtraCache(page_block_size=extra_P, num_blocks=b * pages, indices=idx,
                                                 ref_ids=ref, ref_rows=rows, page_pad=extra_pad))
    return w


def dense_decode(name: str, seed: int, b: int, s_q: int, h_q: int, seqlens, pages_per_seq: int,
                 spare_pages: int = 3) -> Workload:
    """Paged FP8 cache for dense decode (64-token pages): every request owns
    pages_per_seq pages dealt from a global shuffled permutation (block table
    [b, pages_per_seq], meta["block_table"]) and holds cache_seqlens[b]
    tokens (meta["cache_seqlens"], int32); the rows of those tokens are
    written, every other byte of the cache (the rest of the pages and
    `spare_pages` unowned ones) is 0xFF.  `indices` is empty ([b, s_q, 1] of
    -1): dense decode reads none; `topk` is the tokens a block-table row can
    name (pages_per_seq * 64)."""
    P = 64
    rng = np.random.default_rng(seed)
    total_pages = b * pages_per_seq + spare_pages
    block_table = rng.permutation(total_pages)[: b * pages_per_seq].reshape(b, pages_per_seq).astype(np.int32)
    lens = np.asarray(seqlens, dtype=np.int32)
    q_bits = to_bf16_bits(rng.standard_normal((b, s_q, h_q, D_QK), dtype=np.float32))
    written = []
    for bi in range(b):
        pos = np.arange(min(max(int(lens[bi]), 0), pages_per_seq * P))
        written.append(block_table[bi, pos // P].astype(np.int64) * P + pos % P)
    ref_ids = np.unique(np.concatenate(written)) if written else np.zeros(0, np.int64)
    ref_rows = _fill_rows(rng, ref_ids, KV_FP8_656)
    return Workload(name=name, kv_format=KV_FP8_656, b=b, s_q=s_q, h_q=h_q, topk=pages_per_seq * P,
                    sm_scale=1.0 / np.sqrt(D_QK), q_bits=q_bits, indices=np.full((b, s_q, 1), -1, np.int32),
                    page_block_size=P, num_kv_tokens=total_pages * P, ref_ids=ref_ids, ref_rows=ref_rows,
                    meta={"block_table": block_table, "cache_seqlens": lens})


def sparse_prefill(name: str, seed: int, s_q: int, h_q: int, topk: int, s_kv: int,
                   prior: int, q_rows: Optional[int] = None) -> Workload:
    """Flat bf16 KV, batch 1, logical indices: query t sees tokens [0, prior + t]."""
    rng = np.random.default_rng(seed)
    indices = np.full((1, s_q, topk), -1, dtype=np.int32)
    for t in range(s_q):
        n_cand = prior + t + 1
        k = min(topk, n_cand)
        indices[0, t, :k] = _distinct(rng, n_cand, k)
    return _finish(name, rng, KV_BF16_576, 1, s_q, h_q, topk, 1, s_kv, indices)


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------
CONFIG_NAMES = {
    0: "tiny_b2_h128_topk128",
    1: "decode_b64_h128_topk2048_ctx32k",
    2: "decode_b128_h64_topk2048_ctx64k_short10pct",
    3: "prefill_sq4096_h128_topk2048_bf16kv8192",
    4: "split_stress_b4_sq2_h128_topk2048_ctx128k",
}


def make_config(cfg: int, sort_slots: bool = False, **over) -> Workload:
    seed = BASE_SEED + cfg
    if cfg == 0:
        # sequence i owns pages 4i..4i+3 (256 tokens); 128 distinct positions per query
        return paged_decode(CONFIG_NAMES[0], seed, b=2, s_q=1, h_q=128, topk=128,
                            tokens_per_seq=256, shuffle_pages=False, **over)
    if cfg == 1:
        return paged_decode(CONFIG_NAMES[1], seed, b=64, s_q=1, h_q=128, topk=2048,
                            tokens_per_seq=32768, **over)
    if cfg == 2:
        return paged_decode(CONFIG_NAMES[2], seed, b=128, s_q=1, h_q=64, topk=2048,
                            tokens_per_seq=65536, short_frac=0.1, short_len=1500, **over)
    if cfg == 3:
        return sparse_prefill(CONFIG_NAMES[3], seed, s_q=4096, h_q=128, topk=2048,
                              s_kv=8192, prior=4096, **over)
    if cfg == 4:
        return paged_decode(CONFIG_NAMES[4], seed, b=4, s_q=2, h_q=128, topk=2048,
                            tokens_per_seq=131072, recent_frac=0.5, recent_window=4096,
                            sort_slots=sort_slots, **over)
    raise ValueError(cfg)


def indexer_inputs(seed: int, b: int, n_heads: int, seq_lens, max_pages: int, spare_pages: int = 3):
    """Seeded inputs of the lightning indexer ("FlashMLA 与 DSA" sections 4.1,
    5.3): e4m3 q codes [b, H, 128] (no NaN codes), fp32 head weights [b, H]
    (N(0, 1) / sqrt(H), the folded softmax scale), a paged key cache
    [num_pages, 8448] (64 x 128 e4m3 codes then 64 fp32 scales in
    [2^-9, 2^-6]) whose physical pages are dealt to requests in a shuffled
    order, and int32 seq_len.  numpy arrays; no arithmetic of the method."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(seq_lens, dtype=np.int32)
    num_pages = b * max_pages + spare_pages
    q = rng.integers(0, 256, (b, n_heads, 128), dtype=np.uint8)
    q = np.where((q & 0x7F) == 0x7F, q ^ 1, q)
    w = (rng.standard_normal((b, n_heads)) / np.sqrt(n_heads)).astype(np.float32)
    codes = rng.integers(0, 256, (num_pages, 64 * 128), dtype=np.uint8)
    codes = np.where((codes & 0x7F) == 0x7F, codes ^ 1, codes)
    scales = rng.uniform(2.0 ** -9, 2.0 ** -6, (num_pages, 64)).astype("<f4")
    kcache = np.concatenate([codes, scales.view(np.uint8)], axis=1)
    page_table = rng.permutation(num_pages)[: b * max_pages].reshape(b, max_pages).astype(np.int32)
    return q, w, np.ascontiguousarray(kcache), page_table, lens
