"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on seeded
inputs.  Gather/dequant and the scheduler must match bit for bit; decode +
combine within |dout| <= 1e-2 + 1e-2 |ref| and |dlse| <= 2e-3."""
import math

import numpy as np
import pytest
import torch

import sparse_mla_attention_decode_amd as M
from oracle import mla_oracle as O
from sparse_mla_attention_decode_amd import workloads as W

pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 1e-2, 1e-2, 2e-3


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _plan(w, closed_form=False, **kw):
    shape = M.make_shape(w.b, w.s_q, w.h_q, w.topk, w.num_kv_tokens, w.kv_format,
                         w.page_block_size, **kw)
    return M.DecodePlan(shape, closed_form=closed_form)


def run_gpu(w, q=None, kv=None, idx=None, closed_form=False, **kw):
    _need_gpu()
    q = w.q_device() if q is None else q
    kv = w.kv_device() if kv is None else kv
    idx = w.indices_device() if idx is None else idx
    plan = _plan(w, closed_form=closed_form, **kw)
    out, lse = plan.run(q, kv, idx, w.sm_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), plan


def oracle(w, queries=None, kv_host=None):
    kv = w.kv_host() if kv_host is None else kv_host
    return O.sparse_mla_decode(w.q_bits, kv, w.indices, w.sm_scale, w.kv_format,
                               w.page_block_size, queries=queries)


def assert_parity(out, lse, ref_out, ref_lse, queries, tag=""):
    worst_o, worst_l = 0.0, 0.0
    for bi, sj in queries:
        o, r = out[bi, sj], ref_out[bi, sj]
        err = np.abs(o - r)
        bound = ATOL + RTOL * np.abs(r)
        assert np.all(np.isfinite(o)), (tag, bi, sj)
        assert np.all(err <= bound), (tag, bi, sj, float((err - bound).max()))
        worst_o = max(worst_o, float(err.max()))
        l, lr = lse[bi, :, sj], ref_lse[bi, :, sj]
        inf = np.isposinf(lr)
        assert np.array_equal(np.isposinf(l), inf), (tag, bi, sj)
        if (~inf).any():
            dl = np.abs(l[~inf] - lr[~inf])
            assert np.all(dl <= LSE_TOL), (tag, bi, sj, float(dl.max()))
            worst_l = max(worst_l, float(dl.max()))
    print(f"[parity {tag}] queries={len(queries)} max|dout|={worst_o:.3e} max|dlse|={worst_l:.3e}", flush=True)


def all_queries(w):
    return [(bi, sj) for bi in range(w.b) for sj in range(w.s_q)]


# ----------------------------------------------------------------------------- scheduler
@pytest.mark.parametrize("b,topk,parts,gran,ovh", [(2, 128, 66, 64, 5), (64, 2048, 256, 32, 5),
                                                   (4, 2048, 256, 32, 0), (128, 2048, 512, 64, 5),
                                                   (64, 2048, 256, 32, 0), (3, 100, 7, 32, 0),
                                                   (1, 2048, 300, 32, 0), (130, 4999, 1024, 96, 0),
                                                   (2000, 64, 100, 32, 0)])
def test_sched_meta_device_matches_oracle(b, topk, parts, gran, ovh):
    _need_gpu()
    shape = M.make_shape(b, 1, 128, topk, 64 * 64, num_parts=parts, split_granularity=gran,
                         fixed_overhead=ovh)
    plan = M.DecodePlan(shape)
    plan.get_sched_meta()
    torch.cuda.synchronize()
    meta = plan.sched_meta.cpu().numpy().reshape(parts, 8)
    want, prefix = O.sched_plan([topk] * b, gran, ovh, parts)
    assert plan.num_splits.cpu().tolist() == prefix
    assert [tuple(m[:7]) for m in meta.tolist()] == [tuple(x) for x in want]


# ----------------------------------------------------------------------------- gather / dequant
def _gather(w, kv=None):
    plan = _plan(w, num_parts=1)
    q, kv, idx = w.q_device(), (w.kv_device() if kv is None else kv), w.indices_device()
    k_rows = torch.zeros((w.b, w.s_q, w.topk, 576), dtype=torch.int16, device="cuda")
    v_rows = torch.zeros((w.b, w.s_q, w.topk, 512), dtype=torch.int16, device="cuda")
    M.mla_debug_gather_dequant(plan.args(q, kv, idx, w.sm_scale), k_rows.data_ptr(), v_rows.data_ptr())
    torch.cuda.synchronize()
    return (k_rows.cpu().numpy().view(np.uint16), v_rows.cpu().numpy().view(np.uint16))


def _bf16_bits_exact(x):
    """float64 values that are exact in bf16 -> their bit patterns."""
    f = x.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), x)
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "value not representable in bf16"
    return (bits >> 16).astype(np.uint16)


@pytest.mark.parametrize("variant", ["cfg0", "ragged", "bf16"])
def test_gather_dequant_bit_exact(variant):
    _need_gpu()
    if variant == "cfg0":
        w = W.make_config(0)
    elif variant == "ragged":
        w = W.paged_decode("ragged", 7, b=3, s_q=2, h_q=128, topk=77, tokens_per_seq=320, P=16)
        w.indices[0, 0, 5] = -1
        w.indices[1, 1, :] = -1
        w.indices[2, 0, 70] = w.num_kv_tokens + 3          # out of range -> empty
    else:
        w = W.sparse_prefill("bf16", 9, s_q=5, h_q=128, topk=40, s_kv=96, prior=60)
    k_rows, v_rows = _gather(w)
    rows, valid = O.gather_dequant(w.kv_host(), w.indices, w.kv_format, w.page_block_size)
    want = _bf16_bits_exact(rows)
    assert np.array_equal(k_rows, want)
    assert np.array_equal(v_rows, want[..., :512])
    print(f"[gather {variant}] rows={valid.size} valid={int(valid.sum())} bit-exact", flush=True)


# ----------------------------------------------------------------------------- decode + combine
@pytest.mark.parametrize("num_parts", [0, 1, 7, 300])
def test_decode_cfg0(num_parts):
    w = W.make_config(0)
    out, lse, plan = run_gpu(w, num_parts=num_parts)
    ref_out, ref_lse = oracle(w)
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"cfg0 parts={num_parts}")


@pytest.mark.parametrize("topk,gran", [(1, 32), (31, 32), (33, 32), (100, 64), (257, 32), (64, 64)])
def test_decode_ragged_topk(topk, gran):
    w = W.paged_decode("ragged", 100 + topk, b=3, s_q=2, h_q=128, topk=topk, tokens_per_seq=512, P=64)
    for parts in (0, 1):
        out, lse, _ = run_gpu(w, num_parts=parts, split_granularity=gran)
        ref_out, ref_lse = oracle(w)
        assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"topk={topk} parts={parts}")


def test_decode_empty_and_duplicate_slots():
    w = W.paged_decode("edge", 21, b=4, s_q=1, h_q=128, topk=96, tokens_per_seq=256, P=64)
    w.indices[0, 0, :] = -1                               # no valid slot at all
    w.indices[1, 0, 40:] = -1                             # valid slots only in the first tiles
    w.indices[2, 0, :64] = -1                             # first two tiles empty
    w.indices[3, 0, :] = w.indices[3, 0, 0]               # every slot the same token
    w.indices[3, 0, 10] = w.num_kv_tokens + 5             # plus an out-of-range slot
    w = W._finish("edge", np.random.default_rng(5), w.kv_format, w.b, w.s_q, w.h_q, w.topk,
                  w.page_block_size, w.num_kv_tokens, w.indices, q_bits=w.q_bits)
    for parts in (0, 1, 5):
        out, lse, _ = run_gpu(w, num_parts=parts, split_granularity=32)
        ref_out, ref_lse = oracle(w)
        assert np.all(out[0, 0] == 0) and np.all(np.isposinf(lse[0, :, 0]))
        assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"edge parts={parts}")


@pytest.mark.parametrize("parts", [0, 1, 5, 37])
def test_decode_h64_fp8(parts):
    """64 query heads on the FP8 cache run the 128-head kernel with the upper
    head blocks scoring copies of heads 0..63 that are never stored: unsplit
    (one partition) and split paths, empty and out-of-range slots."""
    w = W.paged_decode("h64", 61, b=5, s_q=2, h_q=64, topk=200, tokens_per_seq=512, P=64)
    w.indices[0, 0, :] = -1                               # no valid slot
    w.indices[1, 1, 150:] = -1
    w.indices[2, 0, 7] = w.num_kv_tokens + 9              # out of range
    w = W._finish("h64", np.random.default_rng(62), w.kv_format, w.b, w.s_q, w.h_q, w.topk,
                  w.page_block_size, w.num_kv_tokens, w.indices, q_bits=w.q_bits)
    out, lse, _ = run_gpu(w, num_parts=parts, split_granularity=32)
    assert out.shape == (5, 2, 64, 512) and lse.shape == (5, 64, 2)
    ref_out, ref_lse = oracle(w)
    assert np.all(out[0, 0] == 0) and np.all(np.isposinf(lse[0, :, 0]))
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"h64 parts={parts}")


def test_single_repeated_row_is_exact():
    """All slots name one token: out = V of that row exactly (p = 1 for every
    slot, sums of equal bf16 values are exact), lse = score + ln(topk)."""
    w = W.paged_decode("rep", 31, b=2, s_q=1, h_q=128, topk=256, tokens_per_seq=256, P=64)
    w.indices[:] = w.indices[:, :, :1]
    w = W._finish("rep", np.random.default_rng(6), w.kv_format, w.b, w.s_q, w.h_q, w.topk,
                  w.page_block_size, w.num_kv_tokens, w.indices, q_bits=w.q_bits)
    for parts in (0, 1):
        out, lse, _ = run_gpu(w, num_parts=parts, split_granularity=32, fixed_overhead=0)
        kv = w.kv_host()
        for bi in range(w.b):
            t = int(w.indices[bi, 0, 0])
            row = O.decode_fp8_rows(kv[t // 64, t % 64, 0])
            assert np.array_equal(out[bi, 0], np.broadcast_to(row[:512], (128, 512)).astype(np.float32))
            s = O.bf16_value(w.q_bits[bi, 0]) @ row / 24.0
            assert np.all(np.abs(lse[bi, :, 0] - (s + math.log(w.topk))) <= LSE_TOL)


@pytest.mark.parametrize("h_q,slot", [(128, 100), (64, 100), (64, 70), (64, 120)])
def test_reference_max_recompute_path(h_q, slot):
    """A late tile whose scores exceed the first tile's max by far more than
    2^64 (log2 units) forces the piece to be recomputed; the result must still
    match the definition.  With 64 heads the two waves of a head block run
    the softmax of different key halves (slot 100: key 4 of the 4th tile,
    slot 70: key 6 of the 3rd, slot 120: key 24 of the 4th), so the large
    score lies in one wave's half and the recompute must use it in both."""
    w = W.paged_decode("jump", 41, b=2, s_q=1, h_q=h_q, topk=128, tokens_per_seq=256, P=64)
    q = O.bf16_value(w.q_bits[0, 0, 0])
    big_tok = int(w.indices[0, 0, slot])
    nope = (q[:512] * 6.0).astype(np.float32)[None]
    rope = W.to_bf16_bits((q[512:] * 6.0).astype(np.float32))[None]
    row = W.encode_fp8_rows(nope, rope)[0]
    pos = int(np.searchsorted(w.ref_ids, big_tok))
    assert w.ref_ids[pos] == big_tok
    w.ref_rows[pos] = row
    for parts in (0, 1):
        out, lse, _ = run_gpu(w, num_parts=parts)
        ref_out, ref_lse = oracle(w)
        assert ref_lse[0, 0, 0] * math.log2(math.e) > 100      # really beyond the threshold
        assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"jump parts={parts}")


@pytest.mark.parametrize("h_q", [128, 64])
@pytest.mark.parametrize("empty_tiles,topk", [(1, 64), (2, 96), (3, 128)])
def test_leading_empty_tiles(h_q, empty_tiles, topk):
    """The first tiles of a piece hold only empty slots, so the reference max
    is set by a later tile (with 64 heads: possibly by the other wave pair than
    the one that ran the first softmax); every plan must still match."""
    w = W.paged_decode("lead_empty", 43, b=2, s_q=1, h_q=h_q, topk=topk, tokens_per_seq=256, P=64)
    w.indices[:, :, : 32 * empty_tiles] = -1
    ref_out, ref_lse = oracle(w)
    for parts in (0, 1, 3):
        out, lse, _ = run_gpu(w, num_parts=parts)
        assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"lead_empty h={h_q} e={empty_tiles} parts={parts}")


def _closed_vs_sched(w, tag, **kw):
    """NULL plan (closed form in the kernels) against the scheduler's plan:
    the same partition, so the same arithmetic, bit for bit."""
    a = run_gpu(w, closed_form=True, fixed_overhead=0, **kw)
    b = run_gpu(w, closed_form=False, fixed_overhead=0, **kw)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), tag
    return a


@pytest.mark.parametrize("parts", [1, 3, 7, 66, 300])
def test_closed_form_plan_cfg0(parts):
    w = W.make_config(0)
    out, lse, _ = _closed_vs_sched(w, f"cfg0 parts={parts}", num_parts=parts, split_granularity=32)
    ref_out, ref_lse = oracle(w)
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"closed cfg0 parts={parts}")


@pytest.mark.parametrize("kind", ["ragged", "h64", "bf16", "mtp"])
def test_closed_form_plan_shapes(kind):
    if kind == "ragged":
        w = W.paged_decode("cf_ragged", 301, b=5, s_q=2, h_q=128, topk=257, tokens_per_seq=512, P=64)
        kw = dict(num_parts=9, split_granularity=32)
    elif kind == "h64":
        w = W.paged_decode("cf_h64", 302, b=6, s_q=1, h_q=64, topk=300, tokens_per_seq=512, P=64)
        kw = dict(num_parts=10, split_granularity=64)
    elif kind == "bf16":
        w = W.sparse_prefill("cf_bf16", 303, s_q=7, h_q=128, topk=90, s_kv=160, prior=100)
        kw = dict(num_parts=4, split_granularity=32)
    else:
        w = W.paged_decode("cf_mtp", 304, b=4, s_q=2, h_q=128, topk=2048, tokens_per_seq=4096, P=64)
        kw = dict(num_parts=130, split_granularity=32)
    out, lse, _ = _closed_vs_sched(w, kind, **kw)
    qs = all_queries(w)[:6]
    ref_out, ref_lse = oracle(w, qs)
    assert_parity(out, lse, ref_out, ref_lse, qs, f"closed {kind}")


def test_deterministic():
    w = W.make_config(0)
    a = run_gpu(w)
    b = run_gpu(w)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_hip_graph_replay_matches_eager():
    """The whole step (scheduler, decode, combine) captured in a HIP graph and
    replayed several times, with other eager work and synchronisations between
    the replays: every replay must reproduce the eager result bit for bit, and
    the eager result must match the oracle."""
    _need_gpu()
    w = W.make_config(0)
    q, kv, idx = w.q_device(), w.kv_device(), w.indices_device()
    plan = _plan(w, split_granularity=32, fixed_overhead=0)
    out, lse = plan.run(q, kv, idx, w.sm_scale)
    torch.cuda.synchronize()
    eager_out, eager_lse = out.clone(), lse.clone()
    ref_out, ref_lse = oracle(w)
    assert_parity(eager_out.float().cpu().numpy(), eager_lse.cpu().numpy(), ref_out, ref_lse,
                  all_queries(w), "graph eager")
    other = W.paged_decode("graph_other", 77, b=w.b, s_q=1, h_q=128, topk=w.topk, tokens_per_seq=256, P=64)
    oq, okv, oidx = other.q_device(), other.kv_device(), other.indices_device()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.run(q, kv, idx, w.sm_scale)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(q, kv, idx, w.sm_scale)
    for r in range(4):
        out.zero_()
        lse.fill_(-1.0)
        plan.o_accum.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out), f"replay {r}: out differs"
        assert torch.equal(lse, eager_lse), f"replay {r}: lse differs"
        # eager work of the program between replays, on the same buffers
        other_out, _ = plan.run(oq, okv, oidx, other.sm_scale)
        torch.cuda.synchronize()
        assert not torch.equal(other_out, eager_out)


def test_strided_q_and_out():
    _need_gpu()
    w = W.make_config(0)
    q_full = torch.zeros((w.b, w.s_q, w.h_q, 640), dtype=torch.bfloat16, device="cuda")
    q_full[..., :576] = w.q_device()
    q = q_full[..., :576]
    plan = _plan(w)
    out_full = torch.zeros((w.b, w.s_q, w.h_q, 520), dtype=torch.bfloat16, device="cuda")
    out = out_full[..., :512]
    plan.get_sched_meta()
    a = plan.args(q, w.kv_device(), w.indices_device(), w.sm_scale, out=out)
    M.mla_sparse_decode_fwd(a)
    M.mla_splitkv_combine(a)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle(w)
    assert_parity(out.float().cpu().numpy(), plan.lse.cpu().numpy(), ref_out, ref_lse,
                  all_queries(w), "strided")
    assert torch.all(out_full[..., 512:] == 0)


# ----------------------------------------------------------------------------- the five workloads
@pytest.fixture(scope="module")
def cfg1():
    return W.make_config(1)


def test_cfg1_production_all_queries(cfg1):
    w = cfg1
    out, lse, plan = run_gpu(w)
    ref_out, ref_lse = oracle(w)
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), "cfg1")


def test_cfg1_closed_form_plan(cfg1):
    """The benchmarked launch (NULL plan, 32-slot blocks, zero per-request
    cost, 256 partitions): equal to the scheduler's plan bit for bit, and
    every query against the oracle."""
    w = cfg1
    out, lse, _ = _closed_vs_sched(w, "cfg1", num_parts=256, split_granularity=32)
    ref_out, ref_lse = oracle(w)
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), "cfg1 closed")


def test_cfg1_fine_split(cfg1):
    w = cfg1
    out, lse, plan = run_gpu(w, split_granularity=32, fixed_overhead=2)
    qs = [(0, 0), (17, 0), (63, 0)]
    ref_out, ref_lse = oracle(w, qs)
    assert_parity(out, lse, ref_out, ref_lse, qs, "cfg1 gran32")


def test_cfg2_half_heads_short_sequences():
    """64 heads, 128 requests, 13 of them with 1500 valid slots then -1:
    every query against the oracle."""
    w = W.make_config(2)
    out, lse, plan = run_gpu(w)
    assert len(w.meta["short_seqs"]) == 13
    ref_out, ref_lse = oracle(w)
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), "cfg2")


def test_cfg2_bench_launch():
    """The 64-head workload in the launch bench.py times (NULL plan: the
    closed form in the kernels, 32-slot blocks, no per-request cost, one
    partition per CU): every query against the oracle."""
    w = W.make_config(2)
    out, lse, plan = run_gpu(w, closed_form=True, split_granularity=32, fixed_overhead=0)
    ref_out, ref_lse = oracle(w)
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), "cfg2 bench launch")


@pytest.mark.parametrize("parts", [1, 5])
def test_bf16_prefill_h64_padded_rows(parts):
    """The bf16 cache with 64 heads (the 64-head instance of the bf16 format),
    rows 1280 bytes apart (a padded row stride), unsplit and split plans:
    every query against the oracle."""
    _need_gpu()
    w = W.sparse_prefill("bf16_h64", 311, s_q=6, h_q=64, topk=100, s_kv=200, prior=120)
    flat = w.kv_device()
    padded = torch.zeros((flat.shape[0], 1280), dtype=torch.uint8, device="cuda")
    padded[:, :1152] = flat
    out, lse, plan = run_gpu(w, kv=padded[:, :1152], num_parts=parts, split_granularity=32)
    assert plan.args(w.q_device(), padded[:, :1152], w.indices_device()).kv_stride_block == 1280
    ref_out, ref_lse = oracle(w)
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"bf16 h64 padded parts={parts}")


@pytest.mark.parametrize("h_q,parts", [(128, 1), (128, 5), (64, 1), (64, 5)])
def test_strided_out_rows(h_q, parts):
    """The output as a view whose head rows are 640 elements apart: the
    unsplit epilogue (one partition per query column, whole 256-byte row
    segments per store) and the combine (split plan) write every query's rows
    right and leave the 128 padding elements of each row alone."""
    _need_gpu()
    w = W.paged_decode("strided_out", 321, b=3, s_q=2, h_q=h_q, topk=200, tokens_per_seq=512, P=64)
    plan = _plan(w, num_parts=parts, split_granularity=32)
    buf = torch.full((w.b, w.s_q, h_q, 640), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[..., :512]
    plan.get_sched_meta()
    a = plan.args(w.q_device(), w.kv_device(), w.indices_device(), w.sm_scale, out=out)
    assert a.out_stride_h == 640
    M.mla_sparse_decode_fwd(a)
    M.mla_splitkv_combine(a)
    torch.cuda.synchronize()
    assert bool(torch.all(buf[..., 512:] == 7.0)), "padding written"
    ref_out, ref_lse = oracle(w)
    assert_parity(out.float().cpu().numpy(), plan.lse.cpu().numpy(), ref_out, ref_lse, all_queries(w),
                  f"strided out h={h_q} parts={parts}")


def test_cfg3_sparse_prefill_bf16():
    """4096 query tokens: 264 of them against the oracle -- every 16th token
    (one per 16-column stretch of the launch grid) plus both ends."""
    w = W.make_config(3)
    out, lse, plan = run_gpu(w)
    qs = sorted(set([(0, t) for t in range(0, 4096, 16)] + [(0, t) for t in (1, 2, 2047, 2048, 4094, 4095)]))
    assert len(qs) >= 256
    ref_out, ref_lse = oracle(w, qs)
    assert_parity(out, lse, ref_out, ref_lse, qs, "cfg3")


@pytest.mark.parametrize("sort_slots", [False, True])
def test_cfg4_split_stress(sort_slots):
    w = W.make_config(4, sort_slots=sort_slots)
    out, lse, plan = run_gpu(w, num_parts=256, split_granularity=32, fixed_overhead=0)
    ns = plan.num_splits.cpu().numpy()
    assert np.all(np.diff(ns) >= 64)                      # >= 64 topk chunks per query
    ref_out, ref_lse = oracle(w)
    assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"cfg4 sorted={sort_slots}")


def test_cfg4_shuffled_equals_sorted():
    a = run_gpu(W.make_config(4, sort_slots=False), num_parts=256, split_granularity=32, fixed_overhead=0)
    b = run_gpu(W.make_config(4, sort_slots=True), num_parts=256, split_granularity=32, fixed_overhead=0)
    assert np.all(np.abs(a[0] - b[0]) <= ATOL + RTOL * np.abs(b[0]))
    assert np.all(np.abs(a[1] - b[1]) <= LSE_TOL)
