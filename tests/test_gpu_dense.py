"""GPU parity of dense decode (mla_dense_decode_fwd: the block table walked
over cache_seqlens, "FlashMLA Sparse Decode 完整计算过程详解" step 1) against
the dense oracle, through the C ABI, at |dout| <= 1e-2 + 1e-2 |ref| and
|dlse| <= 2e-3: contexts no longer than topk (the case the caller routes to
dense decode), every plan kind (from the cache lengths, shape-only with a
per-request cost, closed form), causal multi-token decode, block-table
entries outside the cache, a padded page stride, the attention sink, and
the 64-request, 2048-token shape on every query."""
import numpy as np
import pytest
import torch

import sparse_mla_attention_decode_amd as M
from oracle import mla_oracle as O
from sparse_mla_attention_decode_amd import workloads as W
from test_gpu_parity import _need_gpu, all_queries, assert_parity

pytestmark = pytest.mark.gpu


def run_dense(w, causal=False, plan_kind="len", kv=None, sink=None, **kw):
    _need_gpu()
    shape = M.make_shape(w.b, w.s_q, w.h_q, w.topk, w.num_kv_tokens, w.kv_format, 64,
                         fixed_overhead=0 if plan_kind == "closed" else kw.pop("fixed_overhead", 5), **kw)
    plan = M.DecodePlan(shape, closed_form=plan_kind == "closed", by_length=plan_kind == "len")
    bt = torch.from_numpy(w.meta["block_table"]).cuda()
    lens = torch.from_numpy(w.meta["cache_seqlens"]).cuda()
    s_t = None if sink is None else torch.tensor(sink, dtype=torch.float32, device="cuda")
    out, lse = plan.run_dense(w.q_device(), w.kv_device() if kv is None else kv, bt, lens, w.sm_scale,
                              causal=causal, attn_sink=s_t)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def oracle(w, causal=False, sink=None, queries=None):
    return O.dense_mla_decode(w.q_bits, w.kv_host(), w.meta["block_table"], w.meta["cache_seqlens"],
                              w.sm_scale, 64, causal=causal, queries=queries, attn_sink=sink)


LENS = [1, 31, 64, 65, 700, 2048, 0, 1999]


@pytest.mark.parametrize("plan_kind,parts", [("len", 0), ("len", 7), ("sched", 256), ("closed", 256),
                                             ("closed", 1)])
def test_dense_plans(plan_kind, parts):
    w = W.dense_decode("dense", 801, b=8, s_q=1, h_q=128, seqlens=LENS, pages_per_seq=32)
    out, lse = run_dense(w, plan_kind=plan_kind, num_parts=parts, split_granularity=32)
    ref_out, ref_lse = oracle(w)
    assert np.all(out[6, 0] == 0) and np.all(np.isposinf(lse[6]))
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"dense {plan_kind} parts={parts}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("h_q", [128, 64])
def test_dense_multi_token(causal, h_q):
    w = W.dense_decode("dense_mtp", 802, b=6, s_q=2, h_q=h_q, seqlens=[1, 2, 33, 129, 1000, 640],
                       pages_per_seq=16)
    out, lse = run_dense(w, causal=causal, num_parts=37, split_granularity=32)
    ref_out, ref_lse = oracle(w, causal=causal)
    if causal:
        assert np.all(np.isposinf(lse[0, :, 0])) and np.all(out[0, 0] == 0)   # sees no token
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"dense mtp causal={causal} h={h_q}")


def test_dense_invalid_entries_and_sink():
    rng = np.random.default_rng(803)
    w = W.dense_decode("dense_bad", 803, b=4, s_q=1, h_q=128, seqlens=[300, 128, 64, 1024], pages_per_seq=16)
    w.meta["block_table"][0, 2] = -1
    w.meta["block_table"][1, 0] = w.num_blocks + 5
    w.meta["block_table"][2, 0] = -7                               # the only page: nothing left
    sink = rng.standard_normal(128) * 2.0
    for kind in ("len", "closed"):
        out, lse = run_dense(w, plan_kind=kind, sink=sink, num_parts=9, split_granularity=32)
        ref_out, ref_lse = oracle(w, sink=sink)
        assert np.all(np.isposinf(lse[2])) and np.all(out[2] == 0)
        assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"dense invalid+sink {kind}")


def test_dense_padded_page_stride():
    """Pages 64 * 656 + 48 bytes apart: the paged (non-contiguous) address path."""
    w = W.dense_decode("dense_pad", 804, b=4, s_q=1, h_q=128, seqlens=[2048, 1500, 77, 640], pages_per_seq=32)
    page = 64 * 656
    buf = torch.full((w.num_blocks, page + 48), 0xFF, dtype=torch.uint8, device="cuda")
    buf[:, :page] = w.kv_device().reshape(w.num_blocks, page)
    kv = buf.as_strided((w.num_blocks, 64, 1, 656), (page + 48, 656, 656, 1))
    out, lse = run_dense(w, kv=kv, num_parts=64, split_granularity=32)
    ref_out, ref_lse = oracle(w)
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), "dense padded stride")


def test_dense_b64_context_2048():
    """64 requests whose contexts are no longer than topk (2048 tokens): the
    closed-form launch the sparse benchmark uses, every query."""
    lens = np.full(64, 2048)
    lens[:8] = [1, 100, 1024, 2047, 1500, 64, 65, 2000]
    w = W.dense_decode("dense_b64", 805, b=64, s_q=1, h_q=128, seqlens=lens, pages_per_seq=32)
    out, lse = run_dense(w, plan_kind="closed", num_parts=256, split_granularity=32)
    ref_out, ref_lse = oracle(w)
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), "dense b64 ctx2048")
