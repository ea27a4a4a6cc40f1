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


def page_keys(kcache: np.ndarray, page: int) -> np.ndarray:
    """Dequantised keys of one physical page: [64, 128] float64 (section 5.3)."""
    raw = np.asarray(kcache[page], dtype=np.uint8)
    codes = raw[:PAGE_TOKENS * DIM].reshape(PAGE_TOKENS, DIM)
    scales = raw[PAGE_TOKENS * DIM:].copy().view("<f4").astype(np.float64)
    return e4m3fn_value(codes) * scales[:, None]


def indexer_scores(q_codes: np.ndarray, weights: np.ndarray, kcache: np.ndarray,
                   page_table: np.ndarray, seq_len: np.ndarray) -> np.ndarray:
    """Eq. 1 for every request b and token t < seq_len[b] (section 4.1).

    q_codes: uint8 [b, H, 128] e4m3 codes; weights: [b, H]; kcache: uint8
    [num_pages, 8448]; page_table: int [b, max_pages]; seq_len: int [b].
    Returns float64 [b, max_pages * 64] with -inf past seq_len."""
    b, H, _ = q_codes.shape
    n_max = page_table.shape[1] * PAGE_TOKENS
    out = np.full((b, n_max), -np.inf)
    for r in range(b):
        n = int(seq_len[r])
        if n <= 0:
            continue
        q = e4m3fn_value(q_codes[r])                          # [H, 128]
        w = np.asarray(weights[r], dtype=np.float64)
        pages = [page_keys(kcache, int(page_table[r, p])) for p in range((n + PAGE_TOKENS - 1) // PAGE_TOKENS)]
        k = np.concatenate(pages)[:n]                         # [n, 128] dequantised keys
        dots = k @ q.T                                        # [n, H]: q_j . k_t
        out[r, :n] = np.maximum(dots, 0.0) @ w                # sum_j w_j ReLU(.)
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), returned as float64; the
    storage precision of the scores (section 4.1)."""
    f = np.asarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    return bf16_value(rounded)


def physical_id(page_table_row: np.ndarray, t: int) -> int:
    """Logical token t of a request -> physical token id (section 5.5, emit)."""
    return int(page_table_row[t // PAGE_TOKENS]) * PAGE_TOKENS + t % PAGE_TOKENS


def topk_select(scores_row: np.ndarray, seq_len: int, k: int,
                page_table_row: np.ndarray) -> np.ndarray:
    """K highest of scores_row[:seq_len] as physical ids, -1 padded
    (sections 4.2, 5.2, 5.5).  Ties keep the lower logical token first."""
    out = np.full(k, -1, dtype=np.int64)
    n = max(0, min(int(seq_len), len(scores_row)))
    if n <= k:                                               # section 5.2 passthrough
        chosen = np.arange(n)
    else:
        order = np.argsort(-np.asarray(scores_row[:n], dtype=np.float64), kind="stable")
        chosen = order[:k]
    for i, t in enumerate(chosen):
        out[i] = physical_id(page_table_row, int(t))
    return out


def check_topk(got_row: np.ndarray, scores_row: np.ndarray, seq_len: int, k: int,
               page_table_row: np.ndarray) -> Optional[str]:
    """None if got_row is a valid top-k of scores_row (same scores the kernel
    selected on), else a description of the first problem.  The ids above the
    K-th highest value must match exactly; the rest must be distinct tokens
    whose score equals that value; the tail is -1."""
    want = topk_select(scores_row, seq_len, k, page_table_row)
    n = max(0, min(int(seq_len), len(scores_row)))
    m = min(n, k)
    got = np.asarray(got_row, dtype=np.int64)
    if np.any(got[m:] != -1):
        return "padding past min(seq_len, K) is not -1"
    if n <= k:
        return None if sorted(got[:m].tolist()) == sorted(want[:m].tolist()) else "passthrough ids differ"
    # logical token of every physical id of the request
    phys_to_t = {physical_id(page_table_row, t): t for t in range(n)}
    try:
        ts = [phys_to_t[int(x)] for x in got[:m]]
    except KeyError:
        return "an id outside the request's first seq_len tokens"
    if len(set(ts)) != m:
        return "repeated token"
    s = np.asarray(scores_row[:n], dtype=np.float64)
    thr = np.sort(s)[::-1][k - 1]
    above = set(np.nonzero(s > thr)[0].tolist())
    if not above.issubset(ts):
        return "a token above the threshold is missing"
    if any(s[t] != thr for t in ts if t not in above):
        return "a token below the threshold was chosen"
    return None
