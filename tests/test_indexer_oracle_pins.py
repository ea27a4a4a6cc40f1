"""Pins of the lightning-indexer / top-k oracle against closed forms,
invariants and brute force ("FlashMLA 与 DSA：内核、流水线和正确性边界",
sections 4.1, 4.2, 5.2, 5.3, 5.5).  No GPU."""
import itertools

import numpy as np
import pytest
import torch

from oracle import indexer_oracle as X

ONE = 0x38        # e4m3 code of 1.0 (sign 0, exponent 7 = bias, mantissa 0)


def make_cache(rng, n_pages, scales=None, codes=None):
    kc = np.zeros((n_pages, X.PAGE_BYTES), np.uint8)
    for p in range(n_pages):
        c = rng.integers(0, 256, (64, 128), dtype=np.uint8) if codes is None else codes
        c = np.where((c & 0x7F) == 0x7F, c ^ 1, c)          # no NaN codes
        kc[p, :8192] = c.reshape(-1)
        s = rng.uniform(0.01, 2.0, 64).astype("<f4") if scales is None else np.asarray(scales, "<f4")
        kc[p, 8192:] = s.view(np.uint8)
    return kc


def test_all_ones_closed_form():
    """q = k codes = 1.0, one head, w = 1: every dot is 128, so I = 128 * scale."""
    rng = np.random.default_rng(1)
    scales = rng.uniform(0.1, 3.0, 64)
    kc = make_cache(rng, 2, scales=scales, codes=np.full((64, 128), ONE, np.uint8))
    q = np.full((1, 1, 128), ONE, np.uint8)
    pt = np.array([[1, 0]])
    s = X.indexer_scores(q, np.array([[1.0]]), kc, pt, np.array([100]))
    want = 128.0 * np.asarray(scales, np.float32).astype(np.float64)
    np.testing.assert_allclose(s[0, :64], want, rtol=1e-15)
    np.testing.assert_allclose(s[0, 64:100], want[:36], rtol=1e-15)
    assert np.all(np.isneginf(s[0, 100:]))


def test_relu_pair_gives_absolute_dot():
    """Heads j and j' with q_j' = -q_j and equal weights: ReLU(x) + ReLU(-x) =
    |x|, so I = w |q . k| -- compared with a library matrix product."""
    rng = np.random.default_rng(2)
    kc = make_cache(rng, 3)
    q0 = rng.integers(0, 256, 128, dtype=np.uint8)
    q0 = np.where((q0 & 0x7F) == 0x7F, q0 ^ 1, q0)
    q = np.stack([q0, q0 ^ 0x80])[None]                    # sign bit flipped
    pt = np.array([[2, 0, 1]])
    s = X.indexer_scores(q, np.array([[0.75, 0.75]]), kc, pt, np.array([192]))
    keys = np.concatenate([X.page_keys(kc, p) for p in (2, 0, 1)])
    want = 0.75 * (torch.tensor(keys) @ torch.tensor(X.e4m3fn_value(q0))).abs().numpy()
    np.testing.assert_allclose(s[0], want, rtol=1e-12, atol=1e-300)


def test_scale_can_be_applied_after_the_head_sum():
    """Section 5.3: the per-token scale is positive, so scoring unit-scale keys
    and multiplying by the scale afterwards gives the same scores."""
    rng = np.random.default_rng(3)
    scales = rng.uniform(0.05, 4.0, 64)
    codes = rng.integers(0, 256, (64, 128), dtype=np.uint8)
    kc = make_cache(rng, 1, scales=scales, codes=codes)
    kc1 = make_cache(rng, 1, scales=np.ones(64), codes=codes)
    q = rng.integers(0, 120, (1, 8, 128), dtype=np.uint8)
    w = rng.standard_normal((1, 8))
    a = X.indexer_scores(q, w, kc, np.array([[0]]), np.array([64]))
    b = X.indexer_scores(q, w, kc1, np.array([[0]]), np.array([64]))
    np.testing.assert_allclose(a[0], b[0] * np.asarray(scales, np.float32), rtol=1e-12)


def test_page_table_permutation_invariance():
    rng = np.random.default_rng(4)
    kc = make_cache(rng, 5)
    q = rng.integers(0, 256, (2, 4, 128), dtype=np.uint8) & 0x77
    w = rng.standard_normal((2, 4))
    pt = np.array([[3, 1, 4], [0, 2, 1]])
    perm = rng.permutation(5)                               # new page p lives at perm[p]
    kc2 = np.empty_like(kc)
    kc2[perm] = kc
    a = X.indexer_scores(q, w, kc, pt, np.array([150, 64]))
    b = X.indexer_scores(q, w, kc2, perm[pt], np.array([150, 64]))
    np.testing.assert_array_equal(a, b)


def test_round_bf16_matches_torch():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5e-3, 3.3e4, 1 + 2 ** -9, -1 - 2 ** -8])
    want = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(X.round_bf16(x), want)


@pytest.mark.parametrize("seed", range(6))
def test_topk_is_the_max_sum_subset(seed):
    """Brute force: with distinct scores the top-k set is the unique K-subset
    of largest sum."""
    rng = np.random.default_rng(seed)
    n, k = 9, 4
    s = rng.permutation(n).astype(float) + rng.uniform(0, 0.5, n)
    pt = np.array([7])
    best = max(itertools.combinations(range(n), k), key=lambda c: sum(s[list(c)]))
    got = X.topk_select(s, n, k, pt, 8)
    assert sorted(got.tolist()) == sorted(7 * 64 + t for t in best)
    assert X.check_topk(got, s, n, k, pt, 8) is None


def test_passthrough_when_length_fits():
    """Section 5.2: seq_len <= K emits tokens 0..seq_len-1 (remapped) then -1."""
    pt = np.array([5, 2, 9])
    s = np.random.default_rng(5).standard_normal(192)
    got = X.topk_select(s, 130, 2048, pt, 10)
    want = [5 * 64 + t for t in range(64)] + [2 * 64 + t for t in range(64)] + [9 * 64, 9 * 64 + 1]
    assert got[:130].tolist() == want and np.all(got[130:] == -1)
    assert np.all(X.topk_select(s, 0, 16, pt, 10) == -1)


def test_checker_rejects_planted_mistakes():
    rng = np.random.default_rng(6)
    s = rng.standard_normal(300)
    s[[10, 20, 30]] = 5.0                                   # ties that straddle the threshold
    s[[11, 12]] = 9.0
    pt = np.array([0, 1, 2, 3, 4])
    k = 4
    good = X.topk_select(s, 300, k, pt, 5)
    assert X.check_topk(good, s, 300, k, pt, 5) is None
    alt = good.copy()
    alt[-1] = 30 if good[-1] != 30 else 10                  # the other tie: still valid
    assert X.check_topk(alt, s, 300, k, pt, 5) is None
    bad = good.copy(); bad[0] = int(np.argmin(s))
    assert X.check_topk(bad, s, 300, k, pt, 5) is not None
    dup = good.copy(); dup[1] = dup[0]
    assert X.check_topk(dup, s, 300, k, pt, 5) is not None
    pad = np.concatenate([good, [-1]]); pad[-1] = 3
    assert X.check_topk(pad, s, 300, k + 1, pt, 5) is not None
    neg = good.copy(); neg[0] = -1                          # -1 for a token that has a page
    assert X.check_topk(neg, s, 300, k, pt, 5) is not None


def _torch_index_scores(q_codes, w, kc, pages, n):
    """Eq. 1 written independently with torch: the e4m3 codes decoded by
    torch's float8_e4m3fn type (not the oracle's decoder), the scales read
    with torch, ReLU and the weighted head sum in float64."""
    codes = torch.from_numpy(np.ascontiguousarray(kc[pages, :8192])).reshape(-1, 128)
    keys = codes.view(torch.float8_e4m3fn).double()
    scales = torch.from_numpy(np.ascontiguousarray(kc[pages, 8192:])).view(torch.float32).reshape(-1).double()
    q = torch.from_numpy(np.ascontiguousarray(q_codes)).view(torch.float8_e4m3fn).double()   # [H, 128]
    dots = (keys * scales[:, None]) @ q.T                  # [tokens, H]
    return (torch.relu(dots) @ torch.from_numpy(np.asarray(w, np.float64)))[:n].numpy()


def test_negative_head_weights_follow_relu_then_weight():
    """Eq. 1 applies the ReLU to each head's dot product and then its weight.
    With negative weights w ReLU(x) and ReLU(w x) differ, so this pins the
    order: compared with an independent torch computation, and a head whose
    weight is negated must flip its contribution's sign exactly."""
    rng = np.random.default_rng(7)
    kc = make_cache(rng, 3)
    q = rng.integers(0, 256, (1, 6, 128), dtype=np.uint8)
    q = np.where((q & 0x7F) == 0x7F, q ^ 1, q)
    w = np.array([[-1.5, 0.25, -0.75, 2.0, -3.0, 0.5]])
    pt = np.array([[1, 2, 0]])
    n = 170
    got = X.indexer_scores(q, w, kc, pt, np.array([n]))[0, :n]
    want = _torch_index_scores(q[0], w[0], kc, [1, 2, 0], n)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # a single head: score = w * max(0, dot), never w * dot where dot < 0
    one = X.indexer_scores(q[:, :1], w[:, :1], kc, pt, np.array([n]))[0, :n]
    dots = _torch_index_scores(q[0, :1], np.array([1.0]), kc, [1, 2, 0], n)
    assert np.all(dots >= 0) and np.any(dots == 0)        # some dots were clipped
    np.testing.assert_allclose(one, -1.5 * dots, rtol=1e-12, atol=1e-12)
    assert np.all(one <= 0)


def test_invalid_page_entries_score_minus_inf_and_emit_minus_one():
    """Reading: a page-table entry outside [0, num_pages) names no page; its
    tokens score -inf and emit id -1 (selected and passthrough rows alike)."""
    rng = np.random.default_rng(8)
    kc = make_cache(rng, 4)
    q = rng.integers(0, 120, (2, 4, 128), dtype=np.uint8)
    w = rng.standard_normal((2, 4))
    pt = np.array([[2, -1, 0, 7], [3, 1, 4, 0]])           # -1 and 7 (>= 4 pages), 4 likewise
    s = X.indexer_scores(q, w, kc, pt, np.array([250, 256]))
    assert np.all(np.isneginf(s[0, 64:128])) and np.all(np.isneginf(s[0, 192:250]))
    assert np.all(np.isfinite(s[0, :64])) and np.all(np.isfinite(s[0, 128:192]))
    assert np.all(np.isneginf(s[1, 128:192])) and np.all(np.isfinite(s[1, 192:256]))
    # finite scores equal those of a table holding the same valid pages
    ok = X.indexer_scores(q, w, kc, np.array([[2, 1, 0, 3], [3, 1, 2, 0]]), np.array([250, 256]))
    np.testing.assert_array_equal(s[0, :64], ok[0, :64])
    np.testing.assert_array_equal(s[0, 128:192], ok[0, 128:192])
    # K larger than the finite count: every finite token, then -1 for the rest
    got = X.topk_select(s[0], 250, 200, pt[0], 4)
    assert sorted(x for x in got.tolist() if x >= 0) == sorted([2 * 64 + t for t in range(64)] +
                                                               [t for t in range(64)])
    assert np.sum(got == -1) == 200 - 128
    assert X.check_topk(got, s[0], 250, 200, pt[0], 4) is None
    # K below the finite count: no -1 at all
    got = X.topk_select(s[0], 250, 100, pt[0], 4)
    assert np.all(got >= 0) and X.check_topk(got, s[0], 250, 100, pt[0], 4) is None
    bad = got.copy(); bad[-1] = -1
    assert X.check_topk(bad, s[0], 250, 100, pt[0], 4) is not None
    # passthrough (seq_len <= K) keeps slot order and marks the invalid page
    got = X.topk_select(s[0], 130, 256, pt[0], 4)
    assert got[:64].tolist() == [128 + t for t in range(64)]
    assert np.all(got[64:128] == -1) and got[128:130].tolist() == [0, 1] and np.all(got[130:] == -1)


def test_seq_len_is_clamped_to_the_page_table():
    """Reading: seq_len past max_pages * 64 means the whole table; a negative
    one means no token."""
    rng = np.random.default_rng(9)
    kc = make_cache(rng, 3)
    q = rng.integers(0, 120, (3, 4, 128), dtype=np.uint8)
    w = rng.standard_normal((3, 4))
    pt = np.array([[2, 0], [1, 2], [0, 1]])
    a = X.indexer_scores(q, w, kc, pt, np.array([10_000, 128, -5]))
    b = X.indexer_scores(q, w, kc, pt, np.array([128, 128, 0]))
    np.testing.assert_array_equal(a, b)
    assert np.all(np.isneginf(a[2]))
    assert X.topk_select(a[0], 10_000, 50, pt[0], 3).tolist() == X.topk_select(a[0], 128, 50, pt[0], 3).tolist()
    assert np.all(X.topk_select(a[2], -5, 8, pt[2], 3) == -1)
