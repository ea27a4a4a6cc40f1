"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/mla.h declares, validates arguments before touching a device, and its
host scheduler matches the oracle's plan bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import sparse_mla_attention_decode_amd as M
from oracle import mla_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


@pytest.fixture(scope="module")
def lib():
    return M.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(mla_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("mla_get_sched_meta", "mla_sparse_decode_fwd", "mla_splitkv_combine"):
        assert must in names
    assert sorted(M.EXPORTED) == names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert "gfx950" in M.mla_version()


def shape(**kw):
    base = dict(b=2, s_q=1, h_q=128, topk=128, num_kv_tokens=512, num_parts=66)
    base.update(kw)
    return M.make_shape(**base)


def test_struct_layout_matches_header():
    # mla_shape: 8 int32 + int64 + 4 int32 (with alignment) ; mla_sched_part: 32 bytes
    assert ctypes.sizeof(M.mla_shape) == 56
    assert M.mla_shape.num_kv_tokens.offset == 32


def test_sizes():
    s = shape()
    meta, ns = M.mla_sched_meta_size(s)
    assert meta == 66 * 32 and ns == 3 * 4
    o, l = M.mla_workspace_size(s)
    assert o == (2 + 66) * 1 * 128 * 512 * 4 and l == (2 + 66) * 128 * 4
    r = M.mla_resolve_shape(s)
    assert (r.split_granularity, r.fixed_overhead, r.num_parts) == (64, 5, 66)


@pytest.mark.parametrize("kw,code", [
    (dict(b=0), M.MLA_ERR_INVALID_ARG), (dict(s_q=0), M.MLA_ERR_INVALID_ARG),
    (dict(s_q=65536), M.MLA_ERR_INVALID_ARG), (dict(b=1 << 20, s_q=17), M.MLA_ERR_INVALID_ARG),
    (dict(topk=0), M.MLA_ERR_INVALID_ARG), (dict(h_q=96), M.MLA_ERR_UNSUPPORTED),
    (dict(h_q=-1), M.MLA_ERR_INVALID_ARG), (dict(num_kv_tokens=0), M.MLA_ERR_INVALID_ARG),
    (dict(num_kv_tokens=100), M.MLA_ERR_INVALID_ARG),           # not a multiple of the page size
    (dict(num_kv_tokens=1 << 31), M.MLA_ERR_INVALID_ARG),
    (dict(split_granularity=48), M.MLA_ERR_INVALID_ARG), (dict(num_parts=-3), M.MLA_ERR_INVALID_ARG),
    (dict(page_block_size=0), M.MLA_ERR_INVALID_ARG), (dict(kv_format=7), M.MLA_ERR_INVALID_ARG),
])
def test_shape_validation(kw, code):
    s = shape(**kw)
    with pytest.raises(M.MlaError) as e:
        M.mla_sched_meta_size(s)
    assert e.value.code == code
    assert M.mla_last_error() != ""


def test_model_dims_validated():
    for field, val in (("h_kv", 2), ("d_qk", 512), ("d_v", 576)):
        s = shape()
        setattr(s, field, val)
        with pytest.raises(M.MlaError) as e:
            M.mla_workspace_size(s)
        assert e.value.code == M.MLA_ERR_UNSUPPORTED


def _args(s, **over):
    a = M.mla_decode_args()
    a.shape = s
    a.q, a.kv, a.indices, a.out, a.lse = 0x1000, 0x2000, 0x3000, 0x4000, 0x5000
    a.q_stride_b, a.q_stride_s, a.q_stride_h = 128 * 576, 128 * 576, 576
    a.kv_stride_block = 64 * 656
    a.idx_stride_b, a.idx_stride_s = 128, 128
    a.out_stride_b, a.out_stride_s, a.out_stride_h = 128 * 512, 128 * 512, 512
    a.sched_meta, a.num_splits = 0x6000, 0x7000
    o, l = M.mla_workspace_size(s)
    a.o_accum, a.lse_accum, a.o_accum_bytes, a.lse_accum_bytes = 0x8000, 0x9000, o, l
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,code", [
    (dict(q=None), M.MLA_ERR_INVALID_ARG), (dict(kv=None), M.MLA_ERR_INVALID_ARG),
    (dict(sched_meta=None), M.MLA_ERR_INVALID_ARG), (dict(num_splits=None), M.MLA_ERR_INVALID_ARG),
    (dict(sched_meta=None, num_splits=None), M.MLA_ERR_INVALID_ARG),   # NULL plan needs overhead 0
    (dict(attn_sink=0xA002), M.MLA_ERR_INVALID_ARG), (dict(topk_length=0xA001), M.MLA_ERR_INVALID_ARG),
    (dict(q=0x1008), M.MLA_ERR_INVALID_ARG), (dict(q_stride_h=580), M.MLA_ERR_INVALID_ARG),
    (dict(kv_stride_block=64 * 656 - 16), M.MLA_ERR_INVALID_ARG), (dict(kv=0x2004), M.MLA_ERR_INVALID_ARG),
    (dict(out_stride_h=513), M.MLA_ERR_INVALID_ARG), (dict(o_accum_bytes=16), M.MLA_ERR_WORKSPACE),
    (dict(lse_accum=None), M.MLA_ERR_WORKSPACE),
])
def test_decode_args_validated_before_launch(over, code):
    s = shape()
    a = _args(s, **over)
    for fn in (M.mla_sparse_decode_fwd, M.mla_splitkv_combine):
        with pytest.raises(M.MlaError) as e:
            fn(a, stream=0)
        assert e.value.code == code


def _host_plan(s):
    r = M.mla_resolve_shape(s)
    meta = np.zeros((r.num_parts, 8), np.int32)
    ns = np.zeros(r.b + 1, np.int32)
    M.mla_plan_sched_meta_host(s, meta.ctypes.data, ns.ctypes.data)
    return r, meta, ns


@pytest.mark.parametrize("b,topk,parts,gran,ovh", [
    (2, 128, 66, 64, 5), (64, 2048, 256, 64, 5), (64, 2048, 256, 32, 5), (64, 2048, 256, 32, 0),
    (128, 2048, 512, 64, 5), (4, 2048, 128, 32, 0), (1, 4096, 256, 32, 5), (3, 100, 7, 32, 2),
    (1, 1, 1, 64, 5), (17, 33, 300, 32, 1),
])
def test_host_plan_matches_oracle(b, topk, parts, gran, ovh):
    s = shape(b=b, topk=topk, num_parts=parts, split_granularity=gran, fixed_overhead=ovh)
    r, meta, ns = _host_plan(s)
    want, prefix = O.sched_plan([topk] * b, gran, ovh, parts)
    assert ns.tolist() == prefix
    assert [tuple(m[:7]) for m in meta.tolist()] == [tuple(w) for w in want]


def _host_len_plan(s, lengths):
    r = M.mla_resolve_shape(s)
    lens = np.ascontiguousarray(lengths, dtype=np.int32)
    meta = np.full((r.num_parts, 8), -7, np.int32)
    ns = np.full(r.b + 1, -7, np.int32)
    M.mla_plan_sched_meta_len_host(s, lens.ctypes.data, meta.ctypes.data, ns.ctypes.data)
    return r, meta, ns


@pytest.mark.parametrize("lengths,topk,parts,gran,ovh", [
    ([2048, 0, 1000, 1, 5000, -3, 2047, 32], 2048, 64, 32, 5),     # clamped and empty requests
    ([0, 0, 0], 256, 8, 32, 0),                                    # nothing to do at all
    ([0, 0, 0], 256, 8, 32, 5),
    ([100, 600, 33, 512], 512, 7, 64, 2),
    (list(range(0, 2049, 97)), 2048, 256, 32, 0),
    ([1] * 40, 2048, 256, 32, 5),                                   # more partitions than work
])
def test_host_length_plan_matches_oracle(lengths, topk, parts, gran, ovh):
    """The length-aware plan is the oracle's greedy plan over the clamped
    valid lengths (each request costs ceil(len / G) blocks), every record says
    by_length = 1, and the split prefix matches."""
    b = len(lengths)
    s = shape(b=b, topk=topk, num_parts=parts, split_granularity=gran, fixed_overhead=ovh)
    r, meta, ns = _host_len_plan(s, lengths)
    valid = [min(max(x, 0), topk) for x in lengths]
    want, prefix = O.sched_plan(valid, gran, ovh, parts)
    assert ns.tolist() == prefix
    assert [tuple(m[:7]) for m in meta.tolist()] == [tuple(w) for w in want]
    assert np.all(meta[:, 7] == 1)
    # the unchanged plan keeps by_length = 0
    _, meta0, _ = _host_plan(s)
    assert np.all(meta0[:, 7] == 0)


def test_length_plan_equals_plain_plan_at_full_length():
    s = shape(b=64, topk=2048, num_parts=256, split_granularity=32, fixed_overhead=5)
    _, meta_len, ns_len = _host_len_plan(s, [2048] * 64)
    _, meta, ns = _host_plan(s)
    assert ns_len.tolist() == ns.tolist()
    assert meta_len[:, :7].tolist() == meta[:, :7].tolist()


def test_length_plan_rejects_null_lengths():
    s = shape()
    meta = np.zeros((66, 8), np.int32)
    ns = np.zeros(3, np.int32)
    with pytest.raises(M.MlaError) as e:
        M.mla_plan_sched_meta_len_host(s, None, meta.ctypes.data, ns.ctypes.data)
    assert e.value.code == M.MLA_ERR_INVALID_ARG
    with pytest.raises(M.MlaError) as e:
        M.mla_get_sched_meta_len(s, 0x1002, 0x2000, 0x3000, stream=0)     # misaligned lengths
    assert e.value.code == M.MLA_ERR_INVALID_ARG


def _closed_form_plan(b, topk, gran, parts):
    """The plan the kernels evaluate for a NULL plan (per-request cost 0):
    partition q takes blocks [q p, min((q + 1) p, T)) of the request-major
    block sequence; the split counts come from the telescoped sums."""
    from math import gcd
    B = -(-topk // gran)
    T = b * B
    P = -(-T // parts)
    gb, gp = B // gcd(B, P), P // gcd(B, P)
    rows = []
    for q in range(parts):
        s0 = q * P
        if s0 >= T:
            rows.append(None)
            continue
        e = min(s0 + P, T) - 1
        split = 0 if q == 0 else q + (s0 - 1) // B - (q - 1) // gb
        rows.append((s0 // B, e // B, s0 % B, e % B + 1, split))
    prefix = [0] + [r + (r * B - 1) // P - (r - 1) // gp for r in range(1, b + 1)]
    return rows, prefix


@pytest.mark.parametrize("b,topk,parts,gran", [
    (64, 2048, 256, 32), (64, 2048, 256, 64), (2, 128, 66, 64), (4, 2048, 128, 32), (4, 2048, 130, 32),
    (3, 100, 7, 32), (1, 1, 1, 64), (17, 33, 300, 32), (128, 2048, 256, 32), (5, 96, 3, 32),
    (7, 320, 9, 32), (6, 192, 4, 32), (1, 4096, 256, 32), (33, 1500, 200, 32), (12, 64, 16, 32),
])
def test_closed_form_plan_matches_greedy(b, topk, parts, gran):
    """With zero per-request cost the greedy fill of the walkthrough's step 3
    equals the closed form the kernels use when the plan pointers are NULL."""
    rows, prefix = _closed_form_plan(b, topk, gran, parts)
    want, want_prefix = O.sched_plan([topk] * b, gran, 0, parts)
    assert prefix == want_prefix
    for got, w in zip(rows, want):
        if got is None:
            assert w[0] == b
        else:
            assert got == tuple(w[:5])


def test_closed_form_plan_accepted_with_zero_overhead():
    s = shape(fixed_overhead=0)
    # the plan check passes; the kv stride (checked after it) is what fails
    with pytest.raises(M.MlaError) as e:
        M.mla_sparse_decode_fwd(_args(s, sched_meta=None, num_splits=None, kv_stride_block=16), stream=0)
    assert "kv_stride_block" in str(e.value)


def test_host_plan_reproduces_walkthrough_example():
    r, meta, ns = _host_plan(shape())
    assert [tuple(m[:4]) + tuple(m[5:7]) for m in meta[:4].tolist()] == [
        (0, 0, 0, 1, 0, 1), (0, 0, 1, 2, 1, 0), (1, 1, 0, 1, 0, 1), (1, 1, 1, 2, 1, 0)]
    assert ns.tolist() == [0, 2, 4]
    assert (meta[4:, 0] >= 2).all()


def test_round_up_reciprocal_division_is_exact():
    """The kernels divide by launch-time divisors (blocks per request, the
    partition payload and their gcd quotients) as (mulhi(n, m) + n) >> s with
    s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1; every dividend is below
    2^30.  Checked here against exact integer division, edge values included."""
    rng = np.random.default_rng(7)
    divisors = list(range(1, 3000)) + [int(x) for x in rng.integers(1, 1 << 30, 2000)] + [(1 << 30) - 1, 1 << 30]
    for d in divisors:
        s = 0
        while (1 << s) < d:
            s += 1
        m = ((1 << 32) * ((1 << s) - d)) // d + 1
        assert m < (1 << 32)
        ns = [0, 1, d - 1, d, d + 1, 2 * d - 1, (1 << 30) - 1] + [int(x) for x in rng.integers(0, 1 << 30, 50)]
        for n in ns:
            if n >= 0:
                assert (((n * m) >> 32) + n) % (1 << 32) >> s == n // d, (n, d)


# ----------------------------------------------------------------------------- indexer C ABI
def test_indexer_args_layout_matches_header():
    """mla_indexer_args: five int32 then seven pointers (q at byte 24 after
    the padding to pointer alignment); read from the header's declaration."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct mla_indexer_args \{(.*?)\} mla_indexer_args;", text, flags=re.S).group(1)
    fields = re.findall(r"(\w+\*?)\s+(\w+);", re.sub(r"\bconst\s+", "", body))
    names = [n for _, n in fields]
    assert names == [f for f, _ in M.mla_indexer_args._fields_]
    assert M.mla_indexer_args.q.offset == 24 and ctypes.sizeof(M.mla_indexer_args) == 24 + 7 * 8


def _ix_args(**over):
    a = M.mla_indexer_args()
    a.b, a.n_heads, a.max_pages, a.num_pages, a.topk = 4, 64, 16, 70, 256
    a.q, a.weights, a.kcache = 0x10000, 0x20000, 0x30000
    a.page_table, a.seq_len, a.scores, a.indices = 0x40000, 0x50000, 0x60000, 0x70000
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,code,both", [
    (dict(b=-1), M.MLA_ERR_INVALID_ARG, True), (dict(b=65536), M.MLA_ERR_INVALID_ARG, True),
    (dict(n_heads=48), M.MLA_ERR_UNSUPPORTED, True), (dict(n_heads=128), M.MLA_ERR_UNSUPPORTED, True),
    (dict(topk=0), M.MLA_ERR_INVALID_ARG, True), (dict(max_pages=0), M.MLA_ERR_INVALID_ARG, True),
    (dict(max_pages=(1 << 24) + 1), M.MLA_ERR_INVALID_ARG, True), (dict(num_pages=0), M.MLA_ERR_INVALID_ARG, True),
    (dict(page_table=None), M.MLA_ERR_INVALID_ARG, True), (dict(page_table=0x40002), M.MLA_ERR_INVALID_ARG, True),
    (dict(seq_len=None), M.MLA_ERR_INVALID_ARG, True), (dict(seq_len=0x50001), M.MLA_ERR_INVALID_ARG, True),
    (dict(scores=None), M.MLA_ERR_INVALID_ARG, True), (dict(scores=0x60008), M.MLA_ERR_INVALID_ARG, True),
    (dict(q=None), M.MLA_ERR_INVALID_ARG, False), (dict(q=0x10008), M.MLA_ERR_INVALID_ARG, False),
    (dict(weights=None), M.MLA_ERR_INVALID_ARG, False), (dict(weights=0x20002), M.MLA_ERR_INVALID_ARG, False),
    (dict(kcache=None), M.MLA_ERR_INVALID_ARG, False), (dict(kcache=0x30004), M.MLA_ERR_INVALID_ARG, False),
    (dict(indices=None), M.MLA_ERR_INVALID_ARG, "topk"), (dict(indices=0x70002), M.MLA_ERR_INVALID_ARG, "topk"),
])
def test_indexer_args_validated_before_launch(over, code, both):
    """Every error of mla_indexer_scores / mla_indexer_topk is returned before
    a launch (the pointers are never dereferenced: no GPU here).  `both`:
    the check is shared; False: scores only; "topk": top-k only."""
    a = _ix_args(**over)
    fns = {True: (M.mla_indexer_scores, M.mla_indexer_topk), False: (M.mla_indexer_scores,),
           "topk": (M.mla_indexer_topk,)}[both]
    for fn in fns:
        with pytest.raises(M.MlaError) as e:
            fn(a, stream=0)
        assert e.value.code == code, (fn.__name__, over)
        assert M.mla_last_error() != ""


def test_indexer_args_binding_checks_shapes_and_dtypes():
    """The binding marshals raw pointers, so it checks what the C ABI cannot:
    dtypes, shapes and contiguity."""
    import torch
    b, H, mp, K = 2, 64, 4, 32
    ok = dict(q=torch.zeros((b, H, 128), dtype=torch.uint8), weights=torch.zeros((b, H)),
              kcache=torch.zeros((9, 8448), dtype=torch.uint8), page_table=torch.zeros((b, mp), dtype=torch.int32),
              seq_len=torch.zeros(b, dtype=torch.int32), topk=K,
              scores=torch.zeros((b, mp * 64), dtype=torch.bfloat16), indices=torch.zeros((b, K), dtype=torch.int32))
    a = M.indexer_args(**ok)
    assert (a.b, a.n_heads, a.max_pages, a.num_pages, a.topk) == (b, H, mp, 9, K)
    bad = [dict(q=torch.zeros((b, H, 64), dtype=torch.uint8)), dict(q=torch.zeros((b, H, 128))),
           dict(weights=torch.zeros((b, H), dtype=torch.float64)), dict(weights=torch.zeros((b, H + 1))),
           dict(kcache=torch.zeros((9, 8192), dtype=torch.uint8)),
           dict(page_table=torch.zeros((b, mp), dtype=torch.int64)),
           dict(seq_len=torch.zeros(b, dtype=torch.int64)), dict(seq_len=torch.zeros(b + 1, dtype=torch.int32)),
           dict(scores=torch.zeros((b, mp * 64), dtype=torch.float16)),
           dict(indices=torch.zeros((b, K + 1), dtype=torch.int32)),
           dict(page_table=torch.zeros((mp, b), dtype=torch.int32).t())]
    for over in bad:
        with pytest.raises(M.MlaError):
            M.indexer_args(**{**ok, **over})


def test_by_length_plan_needs_its_lengths():
    """A plan made from valid lengths must be given them at decode time: the
    binding refuses to marshal it without (the kernels write NaN if a caller
    of the C ABI does it anyway)."""
    import torch
    plan = M.DecodePlan(shape(num_parts=8, fixed_overhead=0), device="cpu", by_length=True)
    q = torch.zeros((2, 1, 128, 576), dtype=torch.bfloat16)
    kv = torch.zeros((8, 64, 1, 656), dtype=torch.uint8)
    idx = torch.zeros((2, 1, 128), dtype=torch.int32)
    with pytest.raises(M.MlaError) as e:
        plan.args(q, kv, idx)
    assert e.value.code == M.MLA_ERR_INVALID_ARG
    a = plan.args(q, kv, idx, topk_length=torch.full((2,), 100, dtype=torch.int32))
    assert a.topk_length != 0


def test_noalloc_rejects_caller_buffers_and_oversized_shapes():
    """The no-allocation entry point takes no plan or workspace pointers and
    refuses, before touching a device, a shape whose split workspace exceeds
    its 64 MiB array."""
    s = shape(num_parts=66, fixed_overhead=0)
    for over in (dict(), dict(sched_meta=None), dict(num_splits=None, sched_meta=None),
                 dict(sched_meta=None, num_splits=None, lse_accum=None)):
        a = _args(s, **over)
        with pytest.raises(M.MlaError) as e:
            M.mla_sparse_decode_noalloc(a, stream=0)
        assert e.value.code == M.MLA_ERR_INVALID_ARG, over
    big = shape(b=512, topk=2048, num_parts=256, num_kv_tokens=64 * 1024, fixed_overhead=0)
    a = _args(big, sched_meta=None, num_splits=None, o_accum=None, lse_accum=None)
    with pytest.raises(M.MlaError) as e:
        M.mla_sparse_decode_noalloc(a, stream=0)                  # (512 + 256) * 128 KB > 64 MiB
    assert e.value.code == M.MLA_ERR_WORKSPACE and M.mla_last_error() != ""


@pytest.mark.parametrize("over,extra,code", [
    (dict(), dict(), M.MLA_ERR_INVALID_ARG),                                   # indices set: dense takes none
    (dict(indices=None), dict(), M.MLA_ERR_INVALID_ARG),                       # no cache lengths
    (dict(indices=None, topk_length=0xA000), dict(bt=None), M.MLA_ERR_INVALID_ARG),
    (dict(indices=None, topk_length=0xA000), dict(bt=0xB002), M.MLA_ERR_INVALID_ARG),
    (dict(indices=None, topk_length=0xA000), dict(stride=1), M.MLA_ERR_INVALID_ARG),
    (dict(indices=None, topk_length=0xA000), dict(causal=2), M.MLA_ERR_INVALID_ARG),
    (dict(indices=None, topk_length=0xA000, kv_stride_block=1 << 32), dict(), M.MLA_ERR_UNSUPPORTED),
])
def test_dense_args_validated_before_launch(over, extra, code):
    """mla_dense_decode_fwd: indices must be NULL, the cache lengths come in
    topk_length, a block table of at least topk / 64 entries per row, causal
    0 or 1, a page stride below 4 GiB -- all checked before any launch."""
    s = shape()                                                               # topk 128 = 2 pages of 64
    a = _args(s, **over)
    bt = extra.get("bt", 0xB000)
    with pytest.raises(M.MlaError) as e:
        M.mla_dense_decode_fwd(a, bt, extra.get("stride", 2), extra.get("causal", 0), stream=0)
    assert e.value.code == code, (over, extra, M.mla_last_error())


@pytest.mark.parametrize("kw,code", [(dict(page_block_size=32, num_kv_tokens=512), M.MLA_ERR_UNSUPPORTED),
                                     (dict(topk=100), M.MLA_ERR_INVALID_ARG),
                                     (dict(kv_format=M.MLA_KV_BF16_576), M.MLA_ERR_UNSUPPORTED)])
def test_dense_shape_limits(kw, code):
    """Dense decode reads the FP8 cache in 64-token pages; topk is the
    block-table capacity in whole pages."""
    s = shape(**kw)
    a = _args(s, indices=None, topk_length=0xA000,
              kv_stride_block=1152 if kw.get("kv_format") == M.MLA_KV_BF16_576 else 64 * 656)
    with pytest.raises(M.MlaError) as e:
        M.mla_dense_decode_fwd(a, 0xB000, 64, 0, stream=0)
    assert e.value.code == code, (kw, M.mla_last_error())


# ----------------------------------------------------------------------------- V4 / V4.1 caches
@pytest.mark.parametrize("fmt,tok_b", [(M.MLA_KV_V4_584, 584), (M.MLA_KV_V41_528, 528)])
def test_struct_of_arrays_shapes(fmt, tok_b):
    """The V4 / V4.1 formats take d_qk = 512 (576 is rejected), pages of P
    tokens at kv_stride_block >= P * bytes per token with P * that below 2^31,
    q rows of 512 elements; the gather check and dense decode do not read them."""
    s = shape(kv_format=fmt)
    assert s.d_qk == 512 and s.page_block_size == 64
    assert M.mla_workspace_size(s) == M.mla_workspace_size(shape())     # same split partials
    bad = shape(kv_format=fmt)
    bad.d_qk = 576
    with pytest.raises(M.MlaError) as e:
        M.mla_workspace_size(bad)
    assert e.value.code == M.MLA_ERR_UNSUPPORTED
    ok = dict(kv_stride_block=64 * tok_b + (-64 * tok_b) % 16, q_stride_b=128 * 512, q_stride_s=128 * 512,
              q_stride_h=512)
    for over, code in [(dict(kv_stride_block=64 * tok_b - 16), M.MLA_ERR_INVALID_ARG),
                       (dict(q_stride_h=504), M.MLA_ERR_INVALID_ARG)]:
        a = _args(s, **{**ok, **over})
        with pytest.raises(M.MlaError) as e:
            M.mla_sparse_decode_fwd(a, stream=0)
        assert e.value.code == code, (over, M.mla_last_error())
    big = shape(kv_format=fmt, page_block_size=1 << 22, num_kv_tokens=1 << 22)
    a = _args(big, **{**ok, "kv_stride_block": (1 << 22) * tok_b})
    with pytest.raises(M.MlaError) as e:
        M.mla_sparse_decode_fwd(a, stream=0)
    assert e.value.code == M.MLA_ERR_INVALID_ARG and "2^31" in M.mla_last_error()
    with pytest.raises(M.MlaError) as e:
        M.mla_debug_gather_dequant(_args(s, **ok), 0xC000, 0xD000, stream=0)
    assert e.value.code == M.MLA_ERR_UNSUPPORTED
    with pytest.raises(M.MlaError) as e:
        M.mla_dense_decode_fwd(_args(s, **ok, indices=None, topk_length=0xA000), 0xB000, 2, 0, stream=0)
    assert e.value.code == M.MLA_ERR_UNSUPPORTED


def test_extra_cache_args_validated():
    """mla_sparse_decode_extra_fwd: V4.1 main cache only, extra_topk in
    [1, shape.topk), the extra page geometry, pointers -- all before a launch."""
    s = shape(kv_format=M.MLA_KV_V41_528, topk=160)
    ok = dict(kv_stride_block=64 * 528, q_stride_b=128 * 512, q_stride_s=128 * 512, q_stride_h=512)

    def x(**over):
        e = M.mla_extra_kv()
        e.kv, e.kv_stride_block, e.page_block_size, e.num_kv_tokens = 0xE000, 64 * 288, 64, 512
        e.indices, e.idx_stride_b, e.idx_stride_s, e.extra_topk = 0xF000, 60, 60, 60
        for k, v in over.items():
            setattr(e, k, v)
        return e
    cases = [(x(extra_topk=0), M.MLA_ERR_INVALID_ARG), (x(extra_topk=160), M.MLA_ERR_INVALID_ARG),
             (x(page_block_size=0), M.MLA_ERR_INVALID_ARG), (x(num_kv_tokens=100), M.MLA_ERR_INVALID_ARG),
             (x(kv=None), M.MLA_ERR_INVALID_ARG), (x(kv=0xE008), M.MLA_ERR_INVALID_ARG),
             (x(kv_stride_block=64 * 288 - 16), M.MLA_ERR_INVALID_ARG), (x(indices=None), M.MLA_ERR_INVALID_ARG),
             (x(topk_length=0xA002), M.MLA_ERR_INVALID_ARG),
             (x(page_block_size=1 << 23, num_kv_tokens=1 << 23, kv_stride_block=(1 << 23) * 288),
              M.MLA_ERR_INVALID_ARG)]
    for e, code in cases:
        with pytest.raises(M.MlaError) as err:
            M.mla_sparse_decode_extra_fwd(_args(s, **ok), e, stream=0)
        assert err.value.code == code, M.mla_last_error()
    with pytest.raises(M.MlaError) as err:                           # main cache not V4.1
        M.mla_sparse_decode_extra_fwd(_args(shape(topk=160)), x(), stream=0)
    assert err.value.code == M.MLA_ERR_UNSUPPORTED
