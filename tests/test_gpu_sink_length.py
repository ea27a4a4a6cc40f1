"""GPU parity of the attention sink and the per-request valid length
(attn_sink / topk_length) against the CPU oracle: split and unsplit requests,
the 128- and 64-head kernel over the FP8 and bf16 caches, the closed-form
plan and the benchmark shape."""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
import sparse_mla_attention_decode_amd as M
from sparse_mla_attention_decode_amd import workloads as W
from test_gpu_parity import _need_gpu, _plan, all_queries, assert_parity

pytestmark = pytest.mark.gpu


def run_with(w, sink, lens, closed_form=False, **kw):
    _need_gpu()
    plan = _plan(w, closed_form=closed_form, **kw)
    s_t = None if sink is None else torch.tensor(sink, dtype=torch.float32, device="cuda")
    l_t = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, lse = plan.run(w.q_device(), w.kv_device(), w.indices_device(), w.sm_scale, attn_sink=s_t, topk_length=l_t)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def oracle_with(w, sink, lens, queries=None):
    return O.sparse_mla_decode(w.q_bits, w.kv_host(), w.indices, w.sm_scale, w.kv_format, w.page_block_size,
                               queries=queries, attn_sink=sink, topk_length=lens)


def _sink(rng, h):
    s = rng.standard_normal(h) * 2.0 + 1.0
    s[::7] = 6.0                                          # sinks that take most of the mass
    s[3] = -np.inf                                        # and one that takes none
    return s


@pytest.mark.parametrize("parts", [0, 1, 7])
def test_sink_and_length_fp8_h128(parts):
    rng = np.random.default_rng(91)
    w = W.paged_decode("sl128", 91, b=6, s_q=2, h_q=128, topk=300, tokens_per_seq=1024, P=64)
    sink = _sink(rng, 128)
    lens = np.array([300, 0, 1, 150, 33, 5000])           # full, none, one, mid, within a tile, past topk
    out, lse = run_with(w, sink, lens, num_parts=parts, split_granularity=32)
    ref_out, ref_lse = oracle_with(w, sink, lens)
    assert np.all(out[1] == 0) and np.all(np.isposinf(lse[1]))
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"sink+len h128 parts={parts}")


@pytest.mark.parametrize("which", ["sink", "length"])
def test_sink_or_length_alone_closed_form(which):
    rng = np.random.default_rng(92)
    w = W.paged_decode("slcf", 92, b=5, s_q=1, h_q=128, topk=520, tokens_per_seq=1024, P=64)
    sink = _sink(rng, 128) if which == "sink" else None
    lens = np.array([520, 77, 260, 1, 519]) if which == "length" else None
    out, lse = run_with(w, sink, lens, closed_form=True, num_parts=11, split_granularity=32, fixed_overhead=0)
    ref_out, ref_lse = oracle_with(w, sink, lens)
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"{which} closed form")


@pytest.mark.parametrize("parts", [0, 1, 5])
def test_sink_and_length_fp8_h64(parts):
    rng = np.random.default_rng(93)
    w = W.paged_decode("sl64", 93, b=4, s_q=2, h_q=64, topk=200, tokens_per_seq=512, P=64)
    sink = _sink(rng, 64)
    lens = np.array([200, 64, 0, 131])
    out, lse = run_with(w, sink, lens, num_parts=parts, split_granularity=32)
    ref_out, ref_lse = oracle_with(w, sink, lens)
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"sink+len h64 parts={parts}")


@pytest.mark.parametrize("parts", [1, 4])
def test_sink_and_length_bf16_prefill(parts):
    rng = np.random.default_rng(94)
    w = W.sparse_prefill("slbf", 94, s_q=7, h_q=128, topk=90, s_kv=160, prior=100)
    sink = _sink(rng, 128)
    lens = np.array([61])
    out, lse = run_with(w, sink, lens, num_parts=parts, split_granularity=32)
    ref_out, ref_lse = oracle_with(w, sink, lens)
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"sink+len bf16 parts={parts}")


def test_sink_and_length_benchmark_shape():
    """The benchmarked launch (64 x 128 heads x 2048 slots, NULL plan) with a
    sink and varied lengths; sampled queries against the oracle."""
    rng = np.random.default_rng(95)
    w = W.make_config(1)
    sink = _sink(rng, 128)
    lens = rng.integers(0, 2049, size=64)
    lens[:3] = [2048, 0, 1000]
    out, lse = run_with(w, sink, lens, closed_form=True, num_parts=256, split_granularity=32, fixed_overhead=0)
    qs = [(0, 0), (1, 0), (2, 0), (40, 0)]
    ref_out, ref_lse = oracle_with(w, sink, lens, qs)
    assert_parity(out, lse, ref_out, ref_lse, qs, "sink+len cfg1")


# ------------------------------------------------------------------ length-aware plan
def run_by_length(w, sink, lens, **kw):
    """decode with a plan made from the valid lengths (mla_get_sched_meta_len)."""
    _need_gpu()
    shape = M.make_shape(w.b, w.s_q, w.h_q, w.topk, w.num_kv_tokens, w.kv_format, w.page_block_size, **kw)
    plan = M.DecodePlan(shape, by_length=True)
    s_t = None if sink is None else torch.tensor(sink, dtype=torch.float32, device="cuda")
    l_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, lse = plan.run(w.q_device(), w.kv_device(), w.indices_device(), w.sm_scale, attn_sink=s_t, topk_length=l_t)
    torch.cuda.synchronize()
    return plan, out.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("lens,topk,parts,ovh", [
    ([2048, 0, 1000, 1, 5000, -3, 2047, 32], 2048, 64, 5),
    ([0, 0, 0], 256, 8, 0),
    (list(range(0, 2049, 33)), 2048, 256, 0),
])
def test_device_length_plan_matches_host(lens, topk, parts, ovh):
    _need_gpu()
    b = len(lens)
    shape = M.make_shape(b, 1, 128, topk, 4096, num_parts=parts, split_granularity=32, fixed_overhead=ovh)
    r = M.mla_resolve_shape(shape)
    host_meta = np.zeros((r.num_parts, 8), np.int32)
    host_ns = np.zeros(b + 1, np.int32)
    lh = np.asarray(lens, np.int32)
    M.mla_plan_sched_meta_len_host(shape, lh.ctypes.data, host_meta.ctypes.data, host_ns.ctypes.data)
    meta = torch.full((r.num_parts * 8,), -9, dtype=torch.int32, device="cuda")
    ns = torch.full((b + 1,), -9, dtype=torch.int32, device="cuda")
    ld = torch.tensor(lens, dtype=torch.int32, device="cuda")
    M.mla_get_sched_meta_len(shape, ld.data_ptr(), meta.data_ptr(), ns.data_ptr())
    torch.cuda.synchronize()
    assert np.array_equal(meta.cpu().numpy().reshape(-1, 8), host_meta)
    assert np.array_equal(ns.cpu().numpy(), host_ns)


@pytest.mark.parametrize("parts,ovh", [(0, -1), (7, 5), (40, 0)])
def test_length_plan_fp8_h128(parts, ovh):
    rng = np.random.default_rng(96)
    w = W.paged_decode("lp128", 96, b=6, s_q=2, h_q=128, topk=300, tokens_per_seq=1024, P=64)
    sink = _sink(rng, 128)
    lens = np.array([300, 0, 1, 150, 33, 5000])
    plan, out, lse = run_by_length(w, sink, lens, num_parts=parts, split_granularity=32, fixed_overhead=ovh)
    ref_out, ref_lse = oracle_with(w, sink, lens)
    assert np.all(out[1] == 0) and np.all(np.isposinf(lse[1]))
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"length plan h128 parts={parts}")
    # the plan spends no blocks past the valid slots
    meta = plan.sched_meta.cpu().numpy().reshape(-1, 8)
    ns = plan.num_splits.cpu().numpy()
    want, prefix = O.sched_plan([min(max(x, 0), 300) for x in lens], 32, plan.shape.fixed_overhead,
                                plan.shape.num_parts)
    assert ns.tolist() == prefix
    assert [tuple(m[:7]) for m in meta.tolist()] == [tuple(x) for x in want]


@pytest.mark.parametrize("parts", [0, 5])
def test_length_plan_fp8_h64(parts):
    rng = np.random.default_rng(97)
    w = W.paged_decode("lp64", 97, b=4, s_q=2, h_q=64, topk=200, tokens_per_seq=512, P=64)
    sink = _sink(rng, 64)
    lens = np.array([200, 64, 0, 131])
    _, out, lse = run_by_length(w, sink, lens, num_parts=parts, split_granularity=32)
    ref_out, ref_lse = oracle_with(w, sink, lens)
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"length plan h64 parts={parts}")


def test_length_plan_bf16_prefill():
    w = W.sparse_prefill("lpbf", 98, s_q=7, h_q=128, topk=90, s_kv=160, prior=100)
    lens = np.array([61])
    _, out, lse = run_by_length(w, None, lens, num_parts=4, split_granularity=32)
    ref_out, ref_lse = oracle_with(w, None, lens)
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), "length plan bf16")


@pytest.mark.parametrize("ovh", [0, 5])
def test_length_plan_benchmark_shape(ovh):
    """The benchmark shape (64 x 128 heads x 2048 slots, 256 partitions) with
    varied valid lengths and a plan made from them; sampled queries."""
    rng = np.random.default_rng(99)
    w = W.make_config(1)
    lens = rng.integers(0, 2049, size=64)
    lens[:4] = [2048, 0, 1000, 31]
    _, out, lse = run_by_length(w, None, lens, num_parts=256, split_granularity=32, fixed_overhead=ovh)
    qs = [(0, 0), (1, 0), (2, 0), (3, 0), (40, 0), (63, 0)]
    ref_out, ref_lse = oracle_with(w, None, lens, qs)
    assert_parity(out, lse, ref_out, ref_lse, qs, f"length plan cfg1 ovh={ovh}")


@pytest.mark.parametrize("kind,parts", [("fp8", 1), ("fp8", 7), ("bf16", 1), ("bf16", 4)])
def test_length_plan_without_lengths_is_nan(kind, parts):
    """A plan made from valid lengths, passed through the C ABI without the
    lengths: a contract error the host cannot see (the plan is device
    memory).  Every output -- unsplit ones from the decode, split ones from
    the combine -- must be NaN, never a silently wrong number."""
    _need_gpu()
    if kind == "fp8":
        w = W.paged_decode("nolen", 95, b=3, s_q=2, h_q=128, topk=256, tokens_per_seq=512, P=64)
    else:
        w = W.sparse_prefill("nolen_bf", 96, s_q=5, h_q=128, topk=90, s_kv=160, prior=100)
    shape = M.make_shape(w.b, w.s_q, w.h_q, w.topk, w.num_kv_tokens, w.kv_format, w.page_block_size,
                         num_parts=parts, split_granularity=32)
    plan = M.DecodePlan(shape, by_length=True)
    lens = torch.full((w.b,), w.topk // 2, dtype=torch.int32, device="cuda")
    plan.get_sched_meta(topk_length=lens)
    a = plan.args(w.q_device(), w.kv_device(), w.indices_device(), w.sm_scale, topk_length=lens)
    a.topk_length = None                                  # the caller's mistake
    plan.out.zero_()
    plan.lse.zero_()
    M.mla_sparse_decode_fwd(a)
    M.mla_splitkv_combine(a)
    torch.cuda.synchronize()
    assert torch.isnan(plan.out.float()).all() and torch.isnan(plan.lse).all()
