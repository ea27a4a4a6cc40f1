"""CPU oracle for the lightning indexer and the top-k selection that feed the
sparse decode.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
__graft_entry__ and the CPU-baseline leg of bench.py may import this module.
The product path (the HIP library and its Python binding) never calls it, and
this module shares no code, table or constant generator with that path.

Sources ("FlashMLA 与 DSA：内核、流水线和正确性边界"):

* section 4.1, Eq. 1 -- the index score of key token s for query token t is
  I = sum over the indexer heads j of w_j * ReLU(q_j . k_s).  The key has no
  head dimension (all heads share it); q and k are e4m3 with 128 dims, w is
  fp32.  The query-side FP8 scale and 1/sqrt(d) are folded into w by the
  caller (section 4.1, host-side reference), so q enters as its raw e4m3
  values.
* section 5.3 -- the key cache is paged: one page holds 64 tokens, 8192 bytes
  of e4m3 codes (token-major, 128 per token) followed by 64 little-endian
  fp32 scales (8448 bytes per page); a token's key is code * its scale.  A
  per-request page table maps logical page t // 64 to a physical page.
* section 4.1 -- scores are computed in fp32 and stored as bf16.
* section 4.2 / 5.5 -- top-k keeps the K highest scores of the first
  seq_len tokens of a request and emits physical token ids
  (page_table[t // 64] * 64 + t % 64).
* section 5.2 -- when seq_len <= K no scoring or selection is needed: the
  output is tokens 0 .. seq_len - 1 (remapped), padded with -1.

Two readings where the pages are silent (the kernels follow the same):

* a page-table entry outside [0, num_pages) names no key page: its tokens
  score -inf (chosen only when fewer than K tokens have a finite score) and
  their physical id is -1, the empty-slot marker of the sparse decode;
* seq_len is clamped to [0, max_pages * 64], the tokens the page table can
  name.

Everything here is the plain definition in float64 with numpy: the key is
dequantised first, the ReLU is applied per head, then the weighted head sum.
Selection is a full stable sort.  The order of the selected ids is not fixed
by the pages, so the checker below compares sets, with ties at the threshold
value allowed to resolve either way.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from oracle.mla_oracle import bf16_value, e4m3fn_value

PAGE_TOKENS = 64          # section 5.3: tokens per key-cache page
DIM = 128                 # section 4.1: indexer dims (e4m3)
PAGE_BYTES = PAGE_TOKENS * DIM + PAGE_TOKENS * 4     # 8448


def page_ok(kcache: np.ndarray, page: int) -> bool:
    """Whether a page-table entry names a page of the cache (reading above)."""
    return 0 <= int(page) < kcache.shape[0]


def clamp_len(seq_len: int, max_pages: int) -> int:
    """seq_len clamped to the tokens a page table of max_pages entries names."""
    return max(0, min(int(seq_len), max_pages * PAGE_TOKENS))


def page_keys(kcache: np.ndarray, page: int) -> np.ndarray:
    """Dequantised keys of one physical page: [64, 128] float64 (section 5.3).
    A page outside the cache has no keys: all NaN here, scored -inf below."""
    if not page_ok(kcache, page):
        return np.full((PAGE_TOKENS, DIM), np.nan)
    raw = np.asarray(kcache[page], dtype=np.uint8)
    codes = raw[:PAGE_TOKENS * DIM].reshape(PAGE_TOKENS, DIM)
    scales = raw[PAGE_TOKENS * DIM:].copy().view("<f4").astype(np.float64)
    return e4m3fn_value(codes) * scales[:, None]


def indexer_scores(q_codes: np.ndarray, weights: np.ndarray, kcache: np.ndarray,
                   page_table: np.ndarray, seq_len: np.ndarray) -> np.ndarray:
    """Eq. 1 for every request b and token t < seq_len[b] (section 4.1).

    q_codes: uint8 [b, H, 128] e4m3 codes; weights: [b, H]; kcache: uint8
    [num_pages, 8448]; page_table: int [b, max_pages]; seq_len: int [b].
    Returns float64 [b, max_pages * 64] with -inf past the clamped seq_len
    and for the tokens of pages outside the cache."""
    b, H, _ = q_codes.shape
    max_pages = page_table.shape[1]
    out = np.full((b, max_pages * PAGE_TOKENS), -np.inf)
    for r in range(b):
        n = clamp_len(seq_len[r], max_pages)
        if n == 0:
            continue
        q = e4m3fn_value(q_codes[r])                          # [H, 128]
        w = np.asarray(weights[r], dtype=np.float64)
        pages = [int(page_table[r, p]) for p in range((n + PAGE_TOKENS - 1) // PAGE_TOKENS)]
        k = np.concatenate([page_keys(kcache, pg) for pg in pages])[:n]   # [n, 128] dequantised keys
        dots = k @ q.T                                        # [n, H]: q_j . k_t
        row = np.maximum(dots, 0.0) @ w                       # sum_j w_j ReLU(.)
        valid = np.repeat([page_ok(kcache, pg) for pg in pages], PAGE_TOKENS)[:n]
        out[r, :n] = np.where(valid, row, -np.inf)
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), returned as float64; the
    storage precision of the scores (section 4.1)."""
    f = np.asarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    return bf16_value(rounded)


def physical_id(page_table_row: np.ndarray, t: int, num_pages: int) -> int:
    """Logical token t of a request -> physical token id (section 5.5, emit);
    -1 when its page-table entry is outside [0, num_pages)."""
    pg = int(page_table_row[t // PAGE_TOKENS])
    return pg * PAGE_TOKENS + t % PAGE_TOKENS if 0 <= pg < num_pages else -1


def topk_select(scores_row: np.ndarray, seq_len: int, k: int,
                page_table_row: np.ndarray, num_pages: int) -> np.ndarray:
    """K highest of scores_row[:seq_len] as physical ids, -1 padded
    (sections 4.2, 5.2, 5.5).  Ties keep the lower logical token first.
    seq_len is clamped to the page table (reading above)."""
    out = np.full(k, -1, dtype=np.int64)
    n = clamp_len(seq_len, len(page_table_row))
    if n <= k:                                               # section 5.2 passthrough
        chosen = np.arange(n)
    else:
        order = np.argsort(-np.asarray(scores_row[:n], dtype=np.float64), kind="stable")
        chosen = order[:k]
    for i, t in enumerate(chosen):
        out[i] = physical_id(page_table_row, int(t), num_pages)
    return out


def check_topk(got_row: np.ndarray, scores_row: np.ndarray, seq_len: int, k: int,
               page_table_row: np.ndarray, num_pages: int) -> Optional[str]:
    """None if got_row is a valid top-k of scores_row (same scores the kernel
    selected on), else a description of the first problem.  The ids above the
    K-th highest value must match exactly; the rest must be distinct tokens
    whose score equals that value; the tail is -1.  Tokens of pages outside
    the cache all emit -1 and score -inf, so they are counted, not named."""
    want = topk_select(scores_row, seq_len, k, page_table_row, num_pages)
    n = clamp_len(seq_len, len(page_table_row))
    m = min(n, k)
    got = np.asarray(got_row, dtype=np.int64)
    if np.any(got[m:] != -1):
        return "padding past min(seq_len, K) is not -1"
    if n <= k:
        return None if sorted(got[:m].tolist()) == sorted(want[:m].tolist()) else "passthrough ids differ"
    # logical token of every physical id of the request (valid pages only)
    phys_to_t = {}
    for t in range(n):
        pid = physical_id(page_table_row, t, num_pages)
        if pid >= 0:
            phys_to_t[pid] = t
    named = [int(x) for x in got[:m] if x != -1]
    try:
        ts = [phys_to_t[x] for x in named]
    except KeyError:
        return "an id outside the request's first seq_len tokens"
    if len(set(ts)) != len(ts):
        return "repeated token"
    s = np.asarray(scores_row[:n], dtype=np.float64)
    thr = np.sort(s)[::-1][k - 1]
    above = set(np.nonzero(s > thr)[0].tolist())
    if not above.issubset(ts):
        return "a token above the threshold is missing"
    if any(s[t] != thr for t in ts if t not in above):
        return "a token below the threshold was chosen"
    n_unnamed = m - len(named)
    if n_unnamed:
        # only tokens of pages outside the cache emit -1; they score -inf and
        # are chosen only when the threshold itself is -inf
        invalid = [t for t in range(n) if physical_id(page_table_row, t, num_pages) < 0]
        if thr != -np.inf or n_unnamed > len(invalid):
            return "-1 emitted for a token that has a cache page"
    return None
