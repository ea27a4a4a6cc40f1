"""GPU parity for the V4 and V4.1 caches (d_qk = 512, struct-of-arrays pages,
e8m0 scales): the HIP path through the C ABI against the CPU oracle on
seeded inputs, within |dout| <= 1e-2 + 1e-2 |ref| and |dlse| <= 2e-3 (the
bound of the 656-byte path: the same bf16 operands and fp32 accumulation)."""
import math

import numpy as np
import pytest
import torch

import sparse_mla_attention_decode_amd as M
from oracle import mla_oracle as O
from sparse_mla_attention_decode_amd import workloads as W

pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 1e-2, 1e-2, 2e-3
FORMATS = {"v4": W.KV_V4_584, "v41": W.KV_V41_528}


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(w, kv=None, attn_sink=None, topk_length=None, **kw):
    _need_gpu()
    shape = M.make_shape(w.b, w.s_q, w.h_q, w.topk, w.num_kv_tokens, w.kv_format, w.page_block_size, **kw)
    plan = M.DecodePlan(shape)
    kv = w.kv_device() if kv is None else kv
    out, lse = plan.run(w.q_device(), kv, w.indices_device(), w.sm_scale, attn_sink=attn_sink,
                        topk_length=topk_length)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def _oracle(w, queries=None, kv_host=None, **kw):
    kv = w.kv_host() if kv_host is None else kv_host
    return O.sparse_mla_decode(w.q_bits, kv, w.indices, w.sm_scale, w.kv_format, w.page_block_size,
                               queries=queries, **kw)


def _check(out, lse, ref_out, ref_lse, queries, tag):
    worst_o, worst_l = 0.0, 0.0
    for bi, sj in queries:
        o, r = out[bi, sj], ref_out[bi, sj]
        assert np.all(np.isfinite(o)), (tag, bi, sj)
        err = np.abs(o - r)
        assert np.all(err <= ATOL + RTOL * np.abs(r)), (tag, bi, sj, float(err.max()))
        worst_o = max(worst_o, float(err.max()))
        l, lr = lse[bi, :, sj], ref_lse[bi, :, sj]
        inf = np.isposinf(lr)
        assert np.array_equal(np.isposinf(l), inf), (tag, bi, sj)
        if (~inf).any():
            dl = np.abs(l[~inf] - lr[~inf])
            assert np.all(dl <= LSE_TOL), (tag, bi, sj, float(dl.max()))
            worst_l = max(worst_l, float(dl.max()))
    print(f"[model1 {tag}] queries={len(queries)} max|dout|={worst_o:.3e} max|dlse|={worst_l:.3e}", flush=True)


def _all(w):
    return [(bi, sj) for bi in range(w.b) for sj in range(w.s_q)]


def _refinish(w, seed):
    """Rebuild the cache after the indices were edited (rows of every referenced token)."""
    return W._finish(w.name, np.random.default_rng(seed), w.kv_format, w.b, w.s_q, w.h_q, w.topk,
                     w.page_block_size, w.num_kv_tokens, w.indices, q_bits=w.q_bits, page_pad=w.page_pad)


@pytest.mark.parametrize("fmt", sorted(FORMATS))
@pytest.mark.parametrize("h_q", [128, 64])
@pytest.mark.parametrize("parts", [0, 1, 7])
def test_decode_small(fmt, h_q, parts):
    # several tiles, pages of 64 with 48 pad bytes, split and unsplit requests
    w = W.paged_decode(f"{fmt}-small", 700 + h_q + parts, b=3, s_q=2, h_q=h_q, topk=200, tokens_per_seq=512,
                       P=64, kv_format=FORMATS[fmt], page_pad=48)
    out, lse = _run(w, num_parts=parts, split_granularity=32)
    ref_out, ref_lse = _oracle(w)
    _check(out, lse, ref_out, ref_lse, _all(w), f"{fmt} h={h_q} parts={parts}")


@pytest.mark.parametrize("fmt", sorted(FORMATS))
@pytest.mark.parametrize("topk,P", [(1, 16), (33, 64), (77, 16), (257, 3)])
def test_decode_ragged(fmt, topk, P):
    # ragged tails, pages that are not 64 tokens, empty and out-of-range slots
    w = W.paged_decode(f"{fmt}-ragged", 800 + topk + P, b=3, s_q=2, h_q=128, topk=topk,
                       tokens_per_seq=(320 // P) * P, P=P, kv_format=FORMATS[fmt])
    w.indices[0, 0, :] = -1                               # no valid slot
    w.indices[1, 1, topk // 2:] = -1
    w.indices[2, 0, topk - 1] = w.num_kv_tokens + 5       # out of range
    w = _refinish(w, 810 + topk)
    for parts in (0, 1):
        out, lse = _run(w, num_parts=parts, split_granularity=32)
        ref_out, ref_lse = _oracle(w)
        assert np.all(out[0, 0] == 0) and np.all(np.isposinf(lse[0, :, 0]))
        _check(out, lse, ref_out, ref_lse, _all(w), f"{fmt} topk={topk} P={P} parts={parts}")


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_single_repeated_row_is_exact(fmt):
    """Every slot names one token: out = that token's 512 values exactly
    (dequant is exact, the V4 bf16 dims are copied, p = 1 for every slot)."""
    w = W.paged_decode(f"{fmt}-rep", 900, b=2, s_q=1, h_q=128, topk=256, tokens_per_seq=256, P=64,
                       kv_format=FORMATS[fmt])
    w.indices[:] = w.indices[:, :, :1]
    w = _refinish(w, 901)
    out, lse = _run(w, num_parts=1, fixed_overhead=0)
    rows, _ = O.gather_dequant(w.kv_host(), w.indices[:, :, :1], w.kv_format, w.page_block_size)
    for bi in range(w.b):
        row = rows[bi, 0, 0]
        assert np.array_equal(out[bi, 0], np.broadcast_to(row, (128, 512)).astype(np.float32))
        s = O.bf16_value(w.q_bits[bi, 0]) @ row * w.sm_scale
        assert np.all(np.abs(lse[bi, :, 0] - (s + math.log(w.topk))) <= LSE_TOL)
    print(f"[model1 {fmt} repeated row] exact", flush=True)


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_e8m0_extreme_scale_bytes(fmt):
    """Scale byte 0 is 2^-127 and 0xFF is NaN: a token with a 0 byte decodes to
    (nearly) zero in that group, and any query that selects a token with a
    0xFF byte gets NaN output and lse on the GPU as in the oracle."""
    w = W.paged_decode(f"{fmt}-e8m0", 950, b=2, s_q=1, h_q=128, topk=64, tokens_per_seq=256, P=64,
                       kv_format=FORMATS[fmt])
    db, sb = W.SOA[w.kv_format][:2]
    P = w.page_block_size
    kv = w.kv_host()
    t0 = int(w.indices[0, 0, 3])                           # request 0: group 1 scale byte 0
    kv[t0 // P, P * db + (t0 % P) * sb + 1] = 0
    t1 = int(w.indices[1, 0, 9])                           # request 1: group 0 scale byte 0xFF
    kv[t1 // P, P * db + (t1 % P) * sb + 0] = 0xFF
    out, lse = _run(w, kv=torch.from_numpy(kv).cuda(), num_parts=1)
    ref_out, ref_lse = _oracle(w, kv_host=kv)
    _check(out, lse, ref_out, ref_lse, [(0, 0)], f"{fmt} e8m0 byte 0")
    assert np.all(np.isnan(ref_out[1, 0])) and np.all(np.isnan(out[1, 0]))
    assert np.all(np.isnan(lse[1, :, 0]))
    print(f"[model1 {fmt} e8m0 0xFF] NaN on both sides", flush=True)


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_sink_and_lengths(fmt):
    w = W.paged_decode(f"{fmt}-len", 960, b=4, s_q=2, h_q=128, topk=160, tokens_per_seq=512, P=64,
                       kv_format=FORMATS[fmt])
    lens = np.array([0, 1, 100, 160], np.int32)
    sink = np.random.default_rng(961).standard_normal(128).astype(np.float32)
    out, lse = _run(w, attn_sink=torch.from_numpy(sink).cuda(), topk_length=torch.from_numpy(lens).cuda(),
                    num_parts=5, split_granularity=32)
    ref_out, ref_lse = _oracle(w, attn_sink=sink, topk_length=lens)
    _check(out, lse, ref_out, ref_lse, _all(w), f"{fmt} sink + lengths")


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_decode_bench_shape_sampled(fmt):
    """The 64 x 2048-slot, 32K-context, 128-head shape in the bench's launch
    (one work-group per CU, scheduler plan): sampled query tokens."""
    w = W.paged_decode(f"{fmt}-b64", 970, b=64, s_q=1, h_q=128, topk=2048, tokens_per_seq=32768, P=64,
                       kv_format=FORMATS[fmt])
    out, lse = _run(w)
    queries = [(0, 0), (17, 0), (42, 0), (63, 0)]
    ref_out, ref_lse = _oracle(w, queries=queries)
    _check(out, lse, ref_out, ref_lse, queries, f"{fmt} b64 topk2048")


# ----------------------------------------------------------------------------- FP4 extra cache
def _run_extra(w, main_len=None, extra_len=None, attn_sink=None, **kw):
    _need_gpu()
    x = w.meta["extra"]
    xk = x.indices.shape[2]
    shape = M.make_shape(w.b, w.s_q, w.h_q, w.topk + xk, w.num_kv_tokens, w.kv_format, w.page_block_size, **kw)
    plan = M.DecodePlan(shape)
    d = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    xl = d(None if extra_len is None else np.asarray(extra_len, np.int32))
    extra = M.extra_kv_args(x.kv_device(), x.page_block_size, x.indices_device(), xl)
    out, lse = plan.run_extra(w.q_device(), w.kv_device(), w.indices_device(), extra, w.sm_scale,
                              attn_sink=d(attn_sink),
                              topk_length=d(None if main_len is None else np.asarray(main_len, np.int32)))
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def _oracle_extra(w, queries=None, main_len=None, extra_len=None, attn_sink=None):
    x = w.meta["extra"]
    return O.sparse_mla_decode(w.q_bits, w.kv_host(), w.indices, w.sm_scale, w.kv_format, w.page_block_size,
                               queries=queries, attn_sink=attn_sink, topk_length=main_len,
                               extra={"kv": x.kv_host(), "indices": x.indices, "page_block_size": x.page_block_size,
                                      "topk_length": extra_len})


@pytest.mark.parametrize("h_q", [128, 64])
@pytest.mark.parametrize("parts,gran", [(0, 32), (1, 32), (7, 32), (5, 64)])
def test_extra_cache_small(h_q, parts, gran):
    # 100 main + 60 extra slots: the main / extra boundary inside a tile, and
    # pieces that straddle it (split and unsplit requests)
    w = W.extra_decode("x-small", 1000 + h_q + parts, b=3, s_q=2, h_q=h_q, topk=100, extra_topk=60,
                       tokens_per_seq=512, extra_tokens_per_seq=256, extra_P=16, extra_pad=40)
    out, lse = _run_extra(w, num_parts=parts, split_granularity=gran)
    ref_out, ref_lse = _oracle_extra(w)
    _check(out, lse, ref_out, ref_lse, _all(w), f"extra h={h_q} parts={parts} G={gran}")


def test_extra_cache_lengths_sink_and_empty_parts():
    w = W.extra_decode("x-len", 1100, b=4, s_q=2, h_q=128, topk=96, extra_topk=64, tokens_per_seq=512,
                       extra_tokens_per_seq=512, extra_P=64)
    x = w.meta["extra"]
    x.indices[3, 1, :] = -1                                # request 3, token 1: no extra slot
    x.indices[2, 0, 5] = x.num_kv_tokens + 2              # out of range: empty
    main_len = [0, 96, 40, 7]                              # request 0: extra slots only
    extra_len = [64, 0, 20, 64]                            # request 1: main slots only
    sink = np.random.default_rng(1101).standard_normal(128).astype(np.float32)
    for parts in (1, 9):
        out, lse = _run_extra(w, main_len=main_len, extra_len=extra_len, attn_sink=sink, num_parts=parts,
                              split_granularity=32)
        ref_out, ref_lse = _oracle_extra(w, main_len=np.array(main_len), extra_len=np.array(extra_len),
                                         attn_sink=sink)
        _check(out, lse, ref_out, ref_lse, _all(w), f"extra lengths + sink parts={parts}")


def test_extra_cache_single_token_is_exact():
    """No main slot and every extra slot the same token: out = that FP4 token's
    512 values exactly (e2m1 times a power of two is exact in bf16)."""
    w = W.extra_decode("x-rep", 1200, b=2, s_q=1, h_q=128, topk=64, extra_topk=96, tokens_per_seq=256,
                       extra_tokens_per_seq=256)
    w.indices[:] = -1
    x = w.meta["extra"]
    x.indices[:] = x.indices[:, :, :1]
    out, lse = _run_extra(w, num_parts=1)
    kvx = x.kv_host()
    for bi in range(w.b):
        rows, _ = O.gather_dequant(kvx, x.indices[bi, 0, :1], O.FMT_FP4, x.page_block_size)
        assert np.array_equal(out[bi, 0], np.broadcast_to(rows[0], (128, 512)).astype(np.float32))
        s = O.bf16_value(w.q_bits[bi, 0]) @ rows[0] * w.sm_scale
        assert np.all(np.abs(lse[bi, :, 0] - (s + math.log(96))) <= LSE_TOL)
    print("[model1 extra single token] exact", flush=True)


def test_extra_cache_bench_shape_sampled():
    """2048 main + 512 extra slots per query token, 64 requests, 128 heads,
    the default launch (one work-group per CU): sampled query tokens."""
    w = W.extra_decode("x-b64", 1300, b=64, s_q=1, h_q=128, topk=2048, extra_topk=512, tokens_per_seq=32768,
                       extra_tokens_per_seq=8192)
    out, lse = _run_extra(w)
    queries = [(0, 0), (21, 0), (63, 0)]
    ref_out, ref_lse = _oracle_extra(w, queries=queries)
    _check(out, lse, ref_out, ref_lse, queries, "extra b64 2048+512")
