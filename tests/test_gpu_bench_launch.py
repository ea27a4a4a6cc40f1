"""Parity with teeth at the benchmarked launch: b = 64 requests, 128 heads,
topk = 2048 over a 32K-token FP8 context, the NULL (closed-form) plan with
32-slot blocks, zero per-request cost and 256 partitions -- and the same
shape with the scheduler's plan.

The tolerance of the general parity tests (|dlse| <= 2e-3) is wider than what
one dropped or doubled slot does to lse at topk = 2048 (ln(2048/2047) =
4.9e-4), so these inputs make the exact answer known in closed form, from the
definition in "FlashMLA 与 DSA：内核、流水线和正确性边界" section 4.3, and
compare exactly:

* slot-count sentinel -- Q = 0, so every valid slot scores 0, p is uniform
  and lse = ln(2048); each referenced token's NoPE row is one-hot, 256 at
  dim t mod 512.  Then out[h, d] = 256 * #{slots whose token = d mod 512} /
  2048 -- multiples of 1/8, exact in bf16, and exactly what the kernel's
  arithmetic gives (p = 1, integer sums, power-of-two normalisers).  A
  dropped, doubled or misrouted slot moves one element by 1/8.
* one repeated row -- every slot names one token r: out = V_r exactly and
  lse = s_r + ln(2048), to 1e-4 (below the one-slot shift).
* padded page stride -- the page stride is larger than 64 * 656 bytes, so the
  kernel takes the divide-by-page address path that the contiguous benchmark
  cache skips; every query against the oracle.
"""
import math

import numpy as np
import pytest
import torch

import sparse_mla_attention_decode_amd as M
from oracle import mla_oracle as O
from sparse_mla_attention_decode_amd import workloads as W
from test_gpu_parity import _need_gpu, all_queries, assert_parity, oracle

pytestmark = pytest.mark.gpu

BENCH_KW = dict(num_parts=256, split_granularity=32, fixed_overhead=0)


@pytest.fixture(scope="module")
def bench_workload():
    return W.make_config(1)


def _run(w, closed_form, q=None, kv=None, idx=None):
    _need_gpu()
    shape = M.make_shape(w.b, w.s_q, w.h_q, w.topk, w.num_kv_tokens, w.kv_format, w.page_block_size,
                         **BENCH_KW)
    plan = M.DecodePlan(shape, closed_form=closed_form)
    out, lse = plan.run(w.q_device() if q is None else q, w.kv_device() if kv is None else kv,
                        w.indices_device() if idx is None else idx, w.sm_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def _replace(w, q_bits=None, ref_rows=None, indices=None):
    return W.Workload(name=w.name, kv_format=w.kv_format, b=w.b, s_q=w.s_q, h_q=w.h_q, topk=w.topk,
                      sm_scale=w.sm_scale, q_bits=w.q_bits if q_bits is None else q_bits,
                      indices=w.indices if indices is None else indices,
                      page_block_size=w.page_block_size, num_kv_tokens=w.num_kv_tokens,
                      ref_ids=w.ref_ids, ref_rows=w.ref_rows if ref_rows is None else ref_rows,
                      meta=w.meta)


@pytest.mark.parametrize("closed_form", [True, False])
def test_slot_count_sentinel(bench_workload, closed_form):
    w = bench_workload
    n = len(w.ref_ids)
    nope = np.zeros((n, 512), np.float32)
    nope[np.arange(n), w.ref_ids % 512] = 256.0
    rows = W.encode_fp8_rows(nope, np.zeros((n, 64), np.uint16))
    s = _replace(w, q_bits=np.zeros_like(w.q_bits), ref_rows=rows)
    out, lse = _run(s, closed_form)
    counts = np.zeros((w.b, 512))
    for bi in range(w.b):
        ids = w.indices[bi, 0]
        assert np.all(ids >= 0)
        np.add.at(counts[bi], ids % 512, 1.0)
    want = np.broadcast_to((256.0 * counts / w.topk)[:, None, :], (w.b, w.h_q, 512))
    bad = np.argwhere(out[:, 0] != want)
    assert bad.size == 0, f"{len(bad)} elements off, first (b, h, d) = {tuple(bad[0])}: " \
                          f"got {out[tuple(bad[0][:1]) + (0,) + tuple(bad[0][1:])]}"
    assert np.all(np.abs(lse - math.log(w.topk)) <= 1e-5), float(np.abs(lse - math.log(w.topk)).max())
    # the oracle agrees on a few queries (the same closed form, computed by the
    # definition in float64: equal up to its own rounding)
    qs = [(0, 0), (63, 0)]
    ref_out, ref_lse = oracle(s, qs)
    for bi, _ in qs:
        np.testing.assert_allclose(ref_out[bi, 0], want[bi], rtol=0, atol=1e-12)
        np.testing.assert_allclose(ref_lse[bi, :, 0], math.log(w.topk), rtol=0, atol=1e-12)
    print(f"[sentinel closed_form={closed_form}] out exact on all {w.b} queries", flush=True)


@pytest.mark.parametrize("closed_form", [True, False])
def test_one_repeated_row_at_bench_shape(bench_workload, closed_form):
    w = bench_workload
    idx = np.repeat(w.indices[:, :, :1], w.topk, axis=2)
    s = _replace(w, indices=np.ascontiguousarray(idx))
    out, lse = _run(s, closed_form)
    kv = s.kv_host()
    worst = 0.0
    for bi in range(w.b):
        t = int(idx[bi, 0, 0])
        row = O.decode_fp8_rows(kv[t // 64, t % 64, 0])
        assert np.array_equal(out[bi, 0], np.broadcast_to(row[:512], (w.h_q, 512)).astype(np.float32)), bi
        sc = O.bf16_value(w.q_bits[bi, 0]) @ row * w.sm_scale
        err = np.abs(lse[bi, :, 0] - (sc + math.log(w.topk)))
        worst = max(worst, float(err.max()))
        assert np.all(err <= 1e-4), (bi, float(err.max()))
    print(f"[repeated row closed_form={closed_form}] out exact, max|dlse| = {worst:.2e}", flush=True)


def test_padded_page_stride():
    """Pages 64 * 656 + 48 bytes apart (the divide-by-page address path): the
    same rows as a contiguous cache, every query against the oracle."""
    _need_gpu()
    w = W.paged_decode("padded", 501, b=4, s_q=2, h_q=128, topk=2048, tokens_per_seq=8192, P=64)
    pad = 48
    page = 64 * 656
    dense = w.kv_device().reshape(w.num_blocks, page)
    buf = torch.full((w.num_blocks, page + pad), 0xFF, dtype=torch.uint8, device="cuda")
    buf[:, :page] = dense
    kv = buf.as_strided((w.num_blocks, 64, 1, 656), (page + pad, 656, 656, 1))
    assert kv.stride(0) == page + pad
    for closed_form in (True, False):
        out, lse = _run(w, closed_form, kv=kv)
        ref_out, ref_lse = oracle(w)
        assert_parity(out, lse, ref_out, ref_lse, all_queries(w), f"padded stride closed={closed_form}")
