"""The no-allocation decode entry point (mla_sparse_decode_noalloc) through the
C ABI against the existing entry points (mla_get_sched_meta +
mla_sparse_decode_fwd + mla_splitkv_combine with caller buffers) on the same
inputs: the same kernels and the same plan, so the outputs must be identical
bit for bit.  Two calls in a row on the library's one array, the second with
a smaller input, for the FP8 cache with a per-request scheduler cost (plan in
the array) and without (closed form), and for the bf16 cache."""
import numpy as np
import pytest
import torch

import sparse_mla_attention_decode_amd as M
from sparse_mla_attention_decode_amd import workloads as W

pytestmark = pytest.mark.gpu


def _existing(w, **kw):
    shape = M.make_shape(w.b, w.s_q, w.h_q, w.topk, w.num_kv_tokens, w.kv_format, w.page_block_size, **kw)
    plan = M.DecodePlan(shape)
    out, lse = plan.run(w.q_device(), w.kv_device(), w.indices_device(), w.sm_scale)
    torch.cuda.synchronize()
    return out.clone(), lse.clone(), plan


def _noalloc(w, plan):
    out = torch.full_like(plan.out, float("nan"))
    lse = torch.full_like(plan.lse, float("nan"))
    q, kv, idx = w.q_device(), w.kv_device(), w.indices_device()
    a = plan.args(q, kv, idx, w.sm_scale, out=out, lse=lse)
    a.sched_meta = a.num_splits = a.o_accum = a.lse_accum = None
    a.o_accum_bytes = a.lse_accum_bytes = 0
    M.mla_sparse_decode_noalloc(a)
    torch.cuda.synchronize()
    return out, lse


def _pair(w, tag, **kw):
    ref_out, ref_lse, plan = _existing(w, **kw)
    out, lse = _noalloc(w, plan)
    assert torch.equal(out, ref_out), f"{tag}: out differs"
    assert torch.equal(lse, ref_lse), f"{tag}: lse differs"
    print(f"[noalloc {tag}] identical to the caller-buffer entry points", flush=True)


@pytest.mark.parametrize("overhead", [5, 0])
def test_noalloc_fp8_two_calls(overhead):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = W.paged_decode("na_big", 701, b=16, s_q=2, h_q=128, topk=2048, tokens_per_seq=8192, P=64)
    big.indices[3, 1, 100:] = -1
    small = W.paged_decode("na_small", 702, b=3, s_q=1, h_q=64, topk=300, tokens_per_seq=1024, P=64)
    kw = dict(num_parts=128, split_granularity=32, fixed_overhead=overhead)   # (16 + 128) * 2 splits: 36 MiB
    _pair(big, f"fp8 big ovh={overhead}", **kw)
    _pair(small, f"fp8 small ovh={overhead}", **dict(kw, num_parts=7))


def test_noalloc_bf16_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = W.sparse_prefill("na_bf_big", 703, s_q=32, h_q=128, topk=512, s_kv=1024, prior=600)   # 160 splits: 40 MiB
    small = W.sparse_prefill("na_bf_small", 704, s_q=5, h_q=128, topk=90, s_kv=160, prior=100)
    _pair(big, "bf16 big", num_parts=4, split_granularity=64, fixed_overhead=5)
    _pair(small, "bf16 small", num_parts=2, split_granularity=32, fixed_overhead=0)
