"""Pins of the dense-decode oracle ("FlashMLA Sparse Decode 完整计算过程详解",
step 1: no indices, block_table + cache_seqlens, the pages walked in
block-table order; "FlashMLA 与 DSA" section 3.3) against an independent
torch computation, closed forms and invariants.  No GPU."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import mla_oracle as O
from sparse_mla_attention_decode_amd import workloads as W


def torch_dense(w, causal, sink=None):
    """The dense decode written independently: the cache decoded by torch's
    float8_e4m3fn / float32 / bfloat16 views, each request's pages gathered
    in block-table order, attention by torch's SDPA in float64 with a mask
    (token t < visible length, page inside the cache), lse by logsumexp."""
    kv = torch.from_numpy(w.kv_host().reshape(-1, 656).copy())
    codes = kv[:, :512].contiguous().view(torch.float8_e4m3fn).double()
    scales = kv[:, 512:528].contiguous().view(torch.float32).double()
    nope = (codes.view(-1, 4, 128) * scales[:, :, None]).reshape(-1, 512)
    rope = kv[:, 528:656].contiguous().view(torch.bfloat16).double()
    K, V = torch.cat([nope, rope], 1), nope
    n_pages = kv.shape[0] // 64
    q = torch.from_numpy(w.q_bits.view(np.int16).copy()).view(torch.bfloat16).double()
    bt = torch.from_numpy(w.meta["block_table"]).long()
    lens = w.meta["cache_seqlens"]
    b, s_q, H, _ = w.q_bits.shape
    cap = bt.shape[1] * 64
    out = np.zeros((b, s_q, H, 512))
    lse = np.zeros((b, H, s_q))
    for bi in range(b):
        page_ok = (bt[bi] >= 0) & (bt[bi] < n_pages)
        phys = (bt[bi].clamp(0, n_pages - 1)[:, None] * 64 + torch.arange(64)[None]).reshape(-1)
        ok = page_ok[:, None].expand(-1, 64).reshape(-1)
        Kb, Vb = K[phys], V[phys]
        for sj in range(s_q):
            vis = min(max(int(lens[bi]), 0), cap) - ((s_q - 1 - sj) if causal else 0)
            mask = (torch.arange(cap) < vis) & ok
            if not bool(mask.any()):
                lse[bi, :, sj] = math.inf
                continue
            # rows past the length are 0xFF bytes (NaN): zero them so that a
            # masked weight of 0 does not meet a NaN inside the product
            Km, Vm = Kb.masked_fill(~mask[:, None], 0.0), Vb.masked_fill(~mask[:, None], 0.0)
            s = (q[bi, sj] @ Km.T) / math.sqrt(576)
            lse[bi, :, sj] = torch.logsumexp(s.masked_fill(~mask, -math.inf), -1).numpy()
            o = F.scaled_dot_product_attention(q[bi, sj][None, :, None], Km[None, None], Vm[None, None],
                                               attn_mask=mask[None, None, None], scale=1 / math.sqrt(576))
            out[bi, sj] = o[0, :, 0].numpy()
            if sink is not None:
                out[bi, sj] *= (1.0 / (1.0 + np.exp(sink - lse[bi, :, sj])))[:, None]
    return out, lse


def oracle(w, causal, **kw):
    return O.dense_mla_decode(w.q_bits, w.kv_host(), w.meta["block_table"], w.meta["cache_seqlens"],
                              w.sm_scale, 64, causal=causal, **kw)


@pytest.mark.parametrize("causal", [False, True])
def test_dense_oracle_matches_torch(causal):
    w = W.dense_decode("pin", 11, b=5, s_q=3, h_q=8, seqlens=[1, 63, 64, 130, 0], pages_per_seq=3)
    o, l = oracle(w, causal)
    to, tl = torch_dense(w, causal)
    inf = np.isposinf(tl)
    assert np.array_equal(np.isposinf(l), inf)
    np.testing.assert_allclose(l[~inf], tl[~inf], rtol=0, atol=1e-10)
    np.testing.assert_allclose(o, to, rtol=0, atol=1e-12)
    assert np.all(o[4] == 0)                              # seqlen 0: no token, out 0
    if causal:                                            # seqlen 1: the first two queries see none
        assert np.all(np.isposinf(l[0, :, :2])) and np.isfinite(l[0, 0, 2])


def test_dense_oracle_attention_sink_matches_torch():
    w = W.dense_decode("pin_sink", 12, b=2, s_q=1, h_q=8, seqlens=[100, 17], pages_per_seq=2)
    sink = np.linspace(-2.0, 3.0, 8)
    o, l = oracle(w, False, attn_sink=sink)
    to, tl = torch_dense(w, False, sink=sink)
    np.testing.assert_allclose(o, to, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, tl, rtol=0, atol=1e-10)


def test_one_token_gives_its_value_row():
    """seqlen 1: p = 1 for the only token, out = V of that row exactly and lse
    = its score."""
    w = W.dense_decode("one", 13, b=2, s_q=1, h_q=4, seqlens=[1, 1], pages_per_seq=1)
    o, l = oracle(w, False)
    kv = w.kv_host()
    for bi in range(2):
        t = int(w.meta["block_table"][bi, 0]) * 64
        row = O.decode_fp8_rows(kv[t // 64, t % 64, 0])
        assert np.array_equal(o[bi, 0], np.broadcast_to(row[:512], (4, 512)))
        np.testing.assert_allclose(l[bi, :, 0], O.bf16_value(w.q_bits[bi, 0]) @ row / 24.0, rtol=0, atol=1e-12)


def test_causal_query_equals_shorter_sequence():
    """With causal, query token j of s_q sees the sequence as if it were
    s_q - 1 - j tokens shorter."""
    w = W.dense_decode("causal", 14, b=3, s_q=3, h_q=4, seqlens=[70, 128, 5], pages_per_seq=2)
    o, l = oracle(w, True)
    for j in range(3):
        w2 = W.Workload(**{**w.__dict__, "q_bits": w.q_bits[:, j:j + 1].copy(),
                           "meta": {**w.meta, "cache_seqlens": w.meta["cache_seqlens"] - (2 - j)}})
        o2, l2 = oracle(w2, False)
        assert np.array_equal(o[:, j], o2[:, 0]) and np.array_equal(l[:, :, j], l2[:, :, 0])


def test_page_permutation_invariance():
    """Moving the physical pages and rewriting the block table to match changes nothing."""
    w = W.dense_decode("perm", 15, b=3, s_q=1, h_q=4, seqlens=[200, 64, 129], pages_per_seq=4)
    o, l = oracle(w, False)
    nb = w.num_blocks
    perm = np.random.default_rng(3).permutation(nb)            # page p moves to perm[p]
    kv = w.kv_host()
    kv2 = np.empty_like(kv)
    kv2[perm] = kv
    bt2 = perm[w.meta["block_table"]].astype(np.int32)
    o2, l2 = O.dense_mla_decode(w.q_bits, kv2, bt2, w.meta["cache_seqlens"], w.sm_scale, 64)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_invalid_page_entry_is_empty():
    """A block-table entry outside the cache makes its page's tokens empty
    (the sparse -1 reading): the result equals the torch computation with
    that page masked, and the sparse oracle over the remaining ids."""
    w = W.dense_decode("badpage", 16, b=2, s_q=1, h_q=4, seqlens=[150, 100], pages_per_seq=3)
    w.meta["block_table"][0, 1] = -1
    w.meta["block_table"][1, 0] = w.num_blocks + 7
    o, l = oracle(w, False)
    to, tl = torch_dense(w, False)
    np.testing.assert_allclose(o, to, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, tl, rtol=0, atol=1e-10)
    bt = w.meta["block_table"]
    ids = np.full((2, 1, 192), -1, np.int32)
    for bi, n in ((0, 150), (1, 100)):
        t = np.arange(n)
        ids[bi, 0, :n] = bt[bi, t // 64] * 64 + t % 64
    so, sl = O.sparse_mla_decode(w.q_bits, w.kv_host(), ids, w.sm_scale, 0, 64)
    assert np.array_equal(o, so) and np.array_equal(l, sl)
