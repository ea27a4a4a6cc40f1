"""GPU parity of the lightning indexer scores and the top-k selection against
the CPU oracle ("FlashMLA 与 DSA：内核、流水线和正确性边界", sections 4.1,
4.2, 5.2, 5.3, 5.5).

Scores: the kernel's bf16 scores against the float64 definition, within the
bf16 storage rounding (2^-7 relative, two roundings) plus 2^-14 of
sum |terms|: the FP8 matrix cores sum their products with fewer bits than an
fp32 add (internal alignment), and a few cancelling sums show errors near
2^-19 of that magnitude; a dropped head or a wrong weight errs by about 1/64
of it.  Top-k: an integer
decision taken on the kernel's bf16 scores, so the oracle's selection runs on
those same scores and the id sets must agree exactly, ties at the threshold
value being free to resolve either way."""
import numpy as np
import pytest
import torch

import sparse_mla_attention_decode_amd as M
from oracle import indexer_oracle as X
from oracle.mla_oracle import e4m3fn_value
from sparse_mla_attention_decode_amd import workloads as W
from test_gpu_parity import _need_gpu

pytestmark = pytest.mark.gpu


def run(q, w, kc, pt, lens, topk):
    _need_gpu()
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    idx, sc = M.indexer_select(d(q), d(w), d(kc), d(pt), d(lens), topk)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.float().cpu().numpy()


def score_bound(q, w, kc, pt, lens):
    """Per token: scale * sum_j |w_j| sum_d |q_jd k_td|, the magnitude that the
    kernel's sums round against (0 for tokens of pages outside the cache)."""
    qa = np.abs(e4m3fn_value(q))
    out = np.zeros((q.shape[0], pt.shape[1] * 64))
    for r in range(q.shape[0]):
        n = X.clamp_len(lens[r], pt.shape[1])
        if n == 0:
            continue
        keys = np.concatenate([np.abs(np.nan_to_num(X.page_keys(kc, int(p))))
                               for p in pt[r, : (n + 63) // 64]])[:n]
        out[r, :n] = (keys @ qa[r].T) @ np.abs(w[r].astype(np.float64))
    return out


def check(q, w, kc, pt, lens, topk, rows=None, tag=""):
    """Kernel scores and top-k of the listed rows against the oracle, which is
    given the same raw page table and lengths: -inf scores (pages outside the
    cache) must match exactly, finite ones within the tolerance above."""
    got_idx, got_sc = run(q, w, kc, pt, lens, topk)
    rows = range(q.shape[0]) if rows is None else rows
    sub = list(rows)
    ref = X.indexer_scores(q[sub], w[sub], kc, pt[sub], lens[sub])
    bound = score_bound(q[sub], w[sub], kc, pt[sub], lens[sub])
    num_pages = kc.shape[0]
    for i, r in enumerate(sub):
        n = X.clamp_len(lens[r], pt.shape[1])
        if n > topk:                                       # scored rows only (passthrough skips)
            g, e = got_sc[r, :n], ref[i, :n]
            inf = np.isneginf(e)
            assert np.array_equal(np.isneginf(g), inf), f"{tag} row {r}: -inf pattern differs"
            err = np.abs(g[~inf] - e[~inf])
            tol = 2.0 ** -7 * np.abs(e[~inf]) + 2.0 ** -14 * bound[i, :n][~inf]
            bad = np.nonzero(err > tol)[0]
            assert bad.size == 0, f"{tag} row {r}: {bad.size} scores off, first got {g[~inf][bad[0]]} want {e[~inf][bad[0]]}"
        msg = X.check_topk(got_idx[r], got_sc[r], lens[r], topk, pt[r], num_pages)
        assert msg is None, f"{tag} row {r}: {msg}"
    return got_idx, got_sc


@pytest.mark.parametrize("heads", [64, 32])
def test_indexer_mixed_lengths(heads):
    lens = [3000, 100, 2048, 2049, 0, 4133, 4480]          # passthrough, boundary, ragged tail, full
    q, w, kc, pt, lens = W.indexer_inputs(11, 7, heads, lens, max_pages=70)
    check(q, w, kc, pt, lens, 2048, tag=f"H={heads}")


def test_indexer_small_k_and_ties():
    """K = 5 with many equal scores: two requests whose keys are all the same
    token, so every score ties and any K of them is a valid answer."""
    q, w, kc, pt, lens = W.indexer_inputs(12, 3, 64, [700, 700, 64], max_pages=12)
    tok = kc[pt[1, 0], :128].copy()                           # one token's codes
    scale = kc[pt[1, 0], 8192:8196].copy()                    # and its scale
    for p in pt[1, :11]:
        kc[p, :8192] = np.tile(tok, 64)
        kc[p, 8192:] = np.tile(scale, 64)
    idx, sc = check(q, w, kc, pt, lens, 5, tag="ties")
    assert np.all(sc[1, :700] == sc[1, 0])


def test_indexer_topk_crowded_threshold_bin():
    """6000 equal scores and K = 256: the threshold bin holds more tokens
    than the on-chip stash (4160), so the kernel re-reads the row for them."""
    q, w, kc, pt, lens = W.indexer_inputs(16, 2, 64, [6000, 6000], max_pages=100)
    tok = kc[pt[0, 0], :128].copy()
    scale = kc[pt[0, 0], 8192:8196].copy()
    for p in pt[0, :94]:
        kc[p, :8192] = np.tile(tok, 64)
        kc[p, 8192:] = np.tile(scale, 64)
    idx, sc = check(q, w, kc, pt, lens, 256, tag="crowded bin")
    assert np.all(sc[0, :6000] == sc[0, 0])


def test_indexer_invalid_pages_and_clamped_lengths():
    """A page-table entry outside the cache scores -inf and emits -1, a
    seq_len beyond the table clamps: the oracle takes the raw table and the
    raw lengths and decides both.  Rows: an invalid page in a scored row with
    more finite tokens than K; one with fewer (the -inf tokens fill K with
    -1); an over-long length; a passthrough row (seq_len <= K) holding an
    invalid page; a negative length."""
    q, w, kc, pt, lens = W.indexer_inputs(13, 5, 64, [900, 300, 10_000, 200, -7], max_pages=16)
    pt[0, 3] = -1
    pt[1, 1] = kc.shape[0]                                    # one past the last page
    pt[1, 3] = -1000
    pt[3, 2] = -1
    got_idx, _ = check(q, w, kc, pt, lens, 256, tag="invalid")
    assert np.all(got_idx[0] >= 0)                            # 836 finite tokens > 256
    assert np.sum(got_idx[1] == -1) == 256 - (300 - 128)      # 172 finite of 300
    assert np.all(got_idx[3, 128:192] == -1) and np.all(got_idx[3, 192:200] >= 0)
    assert np.all(got_idx[4] == -1)


def test_indexer_benchmark_shape():
    """64 requests at a 32K-token context (512 pages each), K = 2048: scores of
    two sampled requests against the oracle, the top-k of every request
    validated on the kernel's scores."""
    rng = np.random.default_rng(14)
    lens = rng.integers(20_000, 32_769, size=64)
    lens[:3] = [32_768, 2048, 1500]
    q, w, kc, pt, lens = W.indexer_inputs(14, 64, 64, lens, max_pages=512)
    got_idx, got_sc = run(q, w, kc, pt, lens, 2048)
    sub = [0, 37]
    ref = X.indexer_scores(q[sub], w[sub], kc, pt[sub], lens[sub])
    bound = score_bound(q[sub], w[sub], kc, pt[sub], lens[sub])
    for i, r in enumerate(sub):
        n = int(lens[r])
        tol = 2.0 ** -7 * np.abs(ref[i, :n]) + 2.0 ** -14 * bound[i, :n]
        assert np.all(np.abs(got_sc[r, :n] - ref[i, :n]) <= tol), r
    for r in range(64):
        msg = X.check_topk(got_idx[r], got_sc[r], int(lens[r]), 2048, pt[r], kc.shape[0])
        assert msg is None, f"row {r}: {msg}"


def test_indexer_topk_selection_paths():
    """Both selections of the top-k kernel against the oracle: rows whose top K
    lie within 4094 order-key steps of the largest score (one histogram of
    distances), rows where they do not (one page's scales raised by 2^40, so
    its 64 tokens sit far above the rest: the two-level radix selection), and
    rows longer than the 65536 scores kept on chip (keys re-read from the
    scores), with the exact 65536 boundary."""
    lens = [70_000, 65_536, 5_000, 5_000, 65_537]
    q, w, kc, pt, lens = W.indexer_inputs(15, 5, 64, lens, max_pages=1100)
    for r in (2, 3, 4):
        page = pt[r, 7]
        sc = kc[page, 8192:].copy().view("<f4") * np.float32(2.0 ** 40)
        kc[page, 8192:] = sc.view(np.uint8)
    check(q, w, kc, pt, lens, 256, tag="paths K=256")
    check(q, w, kc, pt, lens, 48, rows=[2, 3], tag="paths K=48")
