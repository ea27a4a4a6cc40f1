"""Pins for the CPU oracle: every check compares it with something other than
itself -- numbers the pages print, PyTorch library routines, closed forms and
invariants of the definition.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from sparse_mla_attention_decode_amd import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _fp8_codes(values):
    """Encode values to e4m3fn codes with torch's converter (library rounding)."""
    t = torch.tensor(values, dtype=torch.float32).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _make_row(codes, scales, rope_vals):
    row = np.zeros(656, dtype=np.uint8)
    row[:512] = codes
    row[512:528] = np.asarray(scales, dtype="<f4").view(np.uint8)
    row[528:656] = W.to_bf16_bits(np.asarray(rope_vals, dtype=np.float32)).astype("<u2").view(np.uint8)
    return row


# ----------------------------------------------------------------------------- element decode
def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3fn_value(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    # range and NaN codes per the format (1-4-3 bits, +-448, S.1111.111 NaN)
    assert np.nanmax(got) == 448.0 and np.nanmin(got) == -448.0
    assert set(np.flatnonzero(np.isnan(got)).tolist()) == {0x7F, 0xFF}


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_value(bits)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_dequant_worked_example():
    g = gold("p2_step7_dequant_example.json")
    assert abs(g["scale"] - g["scale_as_printed"]) < 1e-6 and g["scale"] == 2.0 ** -9
    codes = _fp8_codes(g["fp8_values"])
    # the printed fp8 values are all representable (codes decode back exactly)
    assert np.array_equal(O.e4m3fn_value(codes), np.array(g["fp8_values"]))
    row = _make_row(np.concatenate([codes, np.zeros(504, np.uint8)]), [g["scale"], 1, 1, 1], np.zeros(64))
    K = O.decode_fp8_rows(row[None])[0]
    np.testing.assert_allclose(K[:8], g["bf16_results_as_printed"], atol=g["print_tolerance"])
    # exact products, and exact in bf16
    assert np.array_equal(K[:8], np.array(g["fp8_values"]) * g["scale"])
    assert np.array_equal(O.bf16_value(W.to_bf16_bits(K[:8])), K[:8])


# ----------------------------------------------------------------------------- quantiser (input side)
def test_quant_worked_example():
    g = gold("p2_step4_quant_example.json")
    assert abs(g["group_amax"] / 448.0 - g["scale_inv_as_printed"]) < 1e-6
    x = np.zeros((1, 512), np.float32)
    x[0, 0] = g["element_value"]
    x[0, 1] = -g["group_amax"]
    row = W.encode_fp8_rows(x, np.zeros((1, 64), np.uint16))[0]
    scale0 = row[512:516].view("<f4")[0]
    assert scale0 == 2.0 ** g["ue8m0_scale_exponent"]
    assert abs(scale0 - g["ue8m0_scale_as_printed"]) < 1e-6
    assert abs(1.0 / scale0 - g["reciprocal_as_printed"]) < 1e-9
    assert O.e4m3fn_value(row[0]) == g["element_code_value_as_printed"]


def test_encode_decode_roundtrip_error_bound():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 512), dtype=np.float32) * rng.uniform(1e-3, 1e3, size=(64, 1)).astype(np.float32)
    rope = W.to_bf16_bits(rng.standard_normal((64, 64), dtype=np.float32))
    rows = W.encode_fp8_rows(x, rope)
    K = O.decode_fp8_rows(rows)
    scales = rows[:, 512:528].copy().view("<f4")
    # scales are powers of two and the largest code of each group is within [224, 448]
    assert np.all(np.log2(scales) == np.round(np.log2(scales)))
    xg = x.reshape(64, 4, 128)
    err = np.abs(K[:, :512].reshape(64, 4, 128) - xg)
    # RNE to 3 mantissa bits: |err| <= 2^-4 |x| for normals, <= half a subnormal step otherwise
    bound = np.maximum(np.abs(xg) * 2.0 ** -4, scales[:, :, None] * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-12))
    assert np.array_equal(K[:, 512:], O.bf16_value(rope))


def test_row_layout_offsets():
    codes = np.full(512, 0x38, np.uint8)                       # 1.0 in e4m3fn
    rope = np.linspace(-2, 2, 64).astype(np.float32)
    row = _make_row(codes, [1.0, 2.0, 0.5, 0.25], rope)
    K = O.decode_fp8_rows(row[None])[0]
    assert K.shape == (576,)
    assert np.all(K[0:128] == 1.0) and np.all(K[128:256] == 2.0)
    assert np.all(K[256:384] == 0.5) and np.all(K[384:512] == 0.25)
    assert np.array_equal(K[512:], O.bf16_value(W.to_bf16_bits(rope)))


def test_paged_addressing():
    # token idx lives at page idx // P, offset idx % P of a [nb, P, 1, 656] cache
    rng = np.random.default_rng(3)
    nb, P = 5, 16
    kv = rng.integers(0, 255, size=(nb, P, 1, 656), dtype=np.uint8)
    kv[..., 512:528] = np.asarray([1.0, 1.0, 1.0, 1.0], "<f4").view(np.uint8)
    kv[..., :512] &= 0x77                                     # avoid NaN codes
    kv[..., 528:656] = 0
    idx = np.array([0, 17, 79, -1, 80, 33], np.int32)
    rows, valid = O.gather_dequant(kv, idx, O.FMT_FP8, P)
    assert valid.tolist() == [True, True, True, False, False, True]
    for j, t in enumerate(idx):
        if valid[j]:
            np.testing.assert_array_equal(rows[j], O.decode_fp8_rows(kv[t // P, t % P, 0]))
        else:
            assert np.all(rows[j] == 0)


# ----------------------------------------------------------------------------- constants
def test_sm_scale_constants():
    g = gold("p2_step2_constants.json")
    s = 1.0 / math.sqrt(g["d_qk"])
    assert s == 1.0 / 24.0
    assert abs(s - g["sm_scale_as_printed"]) < g["print_tolerance"]
    assert abs(s * math.log2(math.e) - g["sm_scale_times_log2e_as_printed"]) < g["print_tolerance"]


def test_softmax_worked_numbers_fix_base2_scaling():
    # the online-softmax numbers on the page follow p = 2^(score*c - m) with
    # c = sm_scale*log2(e); the oracle's exp(score*sm_scale - lse) is the same
    # function, so exp(sm_scale*(s - s_max)) must reproduce them.
    g = gold("p2_step9_softmax_example.json")
    c = math.log2(math.e) / 24.0
    tol = g["print_tolerance"]
    m1 = g["block1_max_score"] * c
    assert abs(m1 - g["block1_max_scaled_as_printed"]) < tol
    for s, p in g["block1_p_as_printed"]:
        assert abs(math.exp((s - g["block1_max_score"]) / 24.0) - p) < tol
    assert abs(g["block2_max_score"] * c - g["block2_max_scaled_as_printed"]) < tol
    for s, p in g["block2_p_as_printed"]:
        # block 2 keeps block 1's max (it is larger)
        assert abs(math.exp((s - g["block1_max_score"]) / 24.0) - p) < tol


def test_lse_worked_example_natural_log():
    g = gold("p2_step14_lse_example.json")
    # scores whose base-2 exp-sum relative to the max is L and whose max is M (log2 units)
    s_max = g["M_log2"] / math.log2(math.e)
    n_full = int(g["L"])
    frac = g["L"] - n_full
    s = np.array([s_max] * n_full + [s_max + math.log(frac)])
    lse = O.logsumexp(s[None])[0]
    assert abs(lse - g["lse_as_printed"]) < g["print_tolerance"]


# ----------------------------------------------------------------------------- attention
def _tiny_cache(rng, n_tok=256, P=64):
    nope = rng.standard_normal((n_tok, 512), dtype=np.float32)
    rope = W.to_bf16_bits(rng.standard_normal((n_tok, 64), dtype=np.float32))
    rows = W.encode_fp8_rows(nope, rope)
    return rows.reshape(n_tok // P, P, 1, 656)


def _q(rng, H=16):
    return W.to_bf16_bits(rng.standard_normal((H, 576), dtype=np.float32))


def test_dense_special_case_matches_torch_sdpa():
    """topk covering every token of the cache == dense attention (library SDPA)."""
    rng = np.random.default_rng(11)
    kv = _tiny_cache(rng)
    qb = _q(rng, 128)
    idx = rng.permutation(256).astype(np.int32)
    out, lse = O.sparse_mla_decode(qb[None, None], kv, idx[None, None], 1 / 24, O.FMT_FP8, 64)
    K = torch.from_numpy(O.decode_fp8_rows(kv.reshape(256, 656)))            # token order, no indices
    q = torch.from_numpy(O.bf16_value(qb))
    ref = torch.nn.functional.scaled_dot_product_attention(
        q[None, :, None, :], K[None, None].expand(1, 128, 256, 576),
        K[None, None, :, :512].expand(1, 128, 256, 512), scale=1 / 24)[0, :, 0]
    ref_lse = torch.logsumexp((q @ K.T) / 24, dim=-1)
    np.testing.assert_allclose(out[0, 0], ref.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse[0, :, 0], ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def test_single_row_repeated_closed_form():
    rng = np.random.default_rng(12)
    kv = _tiny_cache(rng)
    qb = _q(rng)
    r, K = 77, 64
    idx = np.full((1, 1, K), r, np.int32)
    out, lse = O.sparse_mla_decode(qb[None, None], kv, idx, 1 / 24, O.FMT_FP8, 64)
    row = O.decode_fp8_rows(kv[r // 64, r % 64, 0])
    s_r = (O.bf16_value(qb) @ row) / 24
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(row[:512], (16, 512)), rtol=4e-16, atol=0)
    np.testing.assert_allclose(lse[0, :, 0], s_r + math.log(K), rtol=0, atol=1e-12)


def test_duplicates_count_per_slot_closed_form():
    rng = np.random.default_rng(13)
    kv = _tiny_cache(rng)
    qb = _q(rng, 4)
    r1, r2, a, b = 5, 200, 3, 1
    idx = np.array([[[r1] * a + [r2] * b]], np.int32)
    out, lse = O.sparse_mla_decode(qb[None, None], kv, idx, 1 / 24, O.FMT_FP8, 64)
    k1 = O.decode_fp8_rows(kv[0, 5, 0])
    k2 = O.decode_fp8_rows(kv[3, 8, 0])
    q = O.bf16_value(qb)
    s1, s2 = q @ k1 / 24, q @ k2 / 24
    w1, w2 = a * np.exp(s1), b * np.exp(s2)
    ref = (w1[:, None] * k1[:512] + w2[:, None] * k2[:512]) / (w1 + w2)[:, None]
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0, :, 0], np.log(w1 + w2), rtol=1e-12)


def test_slot_order_does_not_matter():
    rng = np.random.default_rng(14)
    kv = _tiny_cache(rng)
    qb = _q(rng)
    idx = rng.permutation(256)[:100].astype(np.int32)
    o1, l1 = O.sparse_mla_decode(qb[None, None], kv, idx[None, None], 1 / 24, O.FMT_FP8, 64)
    o2, l2 = O.sparse_mla_decode(qb[None, None], kv, np.sort(idx)[None, None], 1 / 24, O.FMT_FP8, 64)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_empty_slots_are_ignored():
    rng = np.random.default_rng(15)
    kv = _tiny_cache(rng)
    qb = _q(rng)
    idx = rng.permutation(256)[:50].astype(np.int32)
    padded = np.concatenate([idx, [-1] * 20, [256, 1 << 30, -7]]).astype(np.int32)
    o1, l1 = O.sparse_mla_decode(qb[None, None], kv, idx[None, None], 1 / 24, O.FMT_FP8, 64)
    o2, l2 = O.sparse_mla_decode(qb[None, None], kv, rng.permutation(padded)[None, None], 1 / 24, O.FMT_FP8, 64)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)
    o3, l3 = O.sparse_mla_decode(qb[None, None], kv, np.full((1, 1, 9), -1, np.int32), 1 / 24, O.FMT_FP8, 64)
    assert np.all(o3 == 0) and np.all(np.isposinf(l3))


def test_sink_worked_example():
    """Walkthrough step 13: sink -2.5 with the final l = 80.7 and m = 0.2116
    (log2 units) of head 0 gives sink log2 = -3.607 and an output scale of
    0.01238; the oracle's factor 1 / (1 + exp(sink - lse)) applied to O / l
    must reproduce it."""
    g = gold("p2_step13_sink_example.json")
    assert abs(g["attn_sink"] * math.log2(math.e) - g["sink_log2_as_printed"]) < 1e-3
    lse = (g["M_log2"] + math.log2(g["L"])) * math.log(2.0)
    scale = O.sink_factor(np.array([lse]), np.array([g["attn_sink"]]))[0] / g["L"]
    assert abs(scale - g["o_scale_as_printed"]) < g["print_tolerance"]


def test_sink_is_an_extra_zero_value_token():
    """An attention sink equals one more slot whose score is the sink logit
    and whose value row is zero (softmax by torch over the extended scores);
    lse stays that of the real slots."""
    rng = np.random.default_rng(21)
    kv = _tiny_cache(rng)
    qb = _q(rng, 16)
    idx = rng.permutation(256)[:90].astype(np.int32)
    sink = rng.standard_normal(16) * 3.0
    out, lse = O.sparse_mla_decode(qb[None, None], kv, idx[None, None], 1 / 24, O.FMT_FP8, 64, attn_sink=sink)
    base_o, base_l = O.sparse_mla_decode(qb[None, None], kv, idx[None, None], 1 / 24, O.FMT_FP8, 64)
    K = torch.from_numpy(O.decode_fp8_rows(kv[idx // 64, idx % 64, 0]))
    q = torch.from_numpy(O.bf16_value(qb))
    s = torch.cat([(q @ K.T) / 24, torch.from_numpy(sink)[:, None]], dim=1)        # [16, 91]
    V = torch.cat([K[:, :512], torch.zeros(1, 512, dtype=torch.float64)], dim=0)
    ref = torch.softmax(s, dim=1) @ V
    np.testing.assert_allclose(out[0, 0], ref.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_array_equal(lse, base_l)
    # a sink of -inf changes nothing
    o2, _ = O.sparse_mla_decode(qb[None, None], kv, idx[None, None], 1 / 24, O.FMT_FP8, 64,
                                attn_sink=np.full(16, -np.inf))
    np.testing.assert_array_equal(o2, base_o)


def test_topk_length_masks_like_empty_slots():
    """Slots at or past topk_length[b] count as empty: the same as -1 there;
    lengths of 0 and >= topk give none and all."""
    rng = np.random.default_rng(22)
    kv = _tiny_cache(rng)
    qb = np.stack([_q(rng, 8), _q(rng, 8)])[:, None]                            # [2, 1, 8, 576]
    idx = np.stack([rng.permutation(256)[:64], rng.permutation(256)[:64]]).astype(np.int32)[:, None]
    lens = np.array([37, 0])
    o, l = O.sparse_mla_decode(qb, kv, idx, 1 / 24, O.FMT_FP8, 64, topk_length=lens)
    cut = idx.copy()
    cut[0, 0, 37:] = -1
    cut[1, 0, :] = -1
    o2, l2 = O.sparse_mla_decode(qb, kv, cut, 1 / 24, O.FMT_FP8, 64)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)
    assert np.all(o[1] == 0) and np.all(np.isposinf(l[1]))
    o3, l3 = O.sparse_mla_decode(qb, kv, idx, 1 / 24, O.FMT_FP8, 64, topk_length=np.array([64, 1000]))
    o4, l4 = O.sparse_mla_decode(qb, kv, idx, 1 / 24, O.FMT_FP8, 64)
    np.testing.assert_array_equal(o3, o4)
    np.testing.assert_array_equal(l3, l4)


def test_bf16_format_dense_case():
    rng = np.random.default_rng(16)
    vals = W.to_bf16_bits(rng.standard_normal((40, 576), dtype=np.float32))
    kv = vals.astype("<u2").view(np.uint8).reshape(40, 1152)
    qb = _q(rng, 8)
    idx = rng.permutation(40).astype(np.int32)
    out, lse = O.sparse_mla_decode(qb[None, None], kv, idx[None, None], 1 / 24, O.FMT_BF16, 1)
    K = torch.from_numpy(O.bf16_value(vals))
    q = torch.from_numpy(O.bf16_value(qb))
    p = torch.softmax(q @ K.T / 24, dim=-1)
    np.testing.assert_allclose(out[0, 0], (p @ K[:, :512]).numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(lse[0, :, 0], torch.logsumexp(q @ K.T / 24, -1).numpy(), rtol=1e-12)


# ----------------------------------------------------------------------------- combine
def test_combine_worked_example_terms():
    g = gold("p2_step16_combine_example.json")
    lse2 = np.array(g["lse_accum"])[:, None]
    o = np.zeros((3, 1, 512))
    for j in range(3):
        o[j, 0, j] = 1.0
    out, lse = O.splitkv_combine(o, lse2)
    w = out[0, :3] / out[0, 0]                       # relative weights of splits
    assert abs(lse2.max() - g["max_lse_as_printed"]) < 1e-12
    np.testing.assert_allclose(w[:2], g["weight_terms_as_printed"], atol=g["print_tolerance"])
    # base-2 combine: term 3 is 2^(2.1-4.2)
    assert abs(w[2] - 2 ** (2.1 - 4.2)) < 1e-12
    assert abs(lse[0] - math.log(2 ** 4.2 + 2 ** 3.8 + 2 ** 2.1)) < 1e-12


def test_split_then_combine_equals_unsplit():
    rng = np.random.default_rng(17)
    kv = _tiny_cache(rng)
    qb = _q(rng, 32)
    idx = np.concatenate([rng.permutation(256)[:150], [-1] * 22]).astype(np.int32)
    idx = rng.permutation(idx)
    rows, valid = O.gather_dequant(kv, idx, O.FMT_FP8, 64)
    q = O.bf16_value(qb)
    full_o, full_l = O.attend(q, rows, rows[:, :512], valid, 1 / 24)
    for cuts in ([0, 172], [0, 64, 172], [0, 10, 11, 100, 150, 172], [0, 150, 160, 172]):
        parts = [O.partial_attention(q, rows[a:b], rows[a:b, :512], valid[a:b], 1 / 24)
                 for a, b in zip(cuts[:-1], cuts[1:])]
        o, l = O.splitkv_combine(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        np.testing.assert_allclose(o, full_o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(l, full_l, rtol=1e-12)


def test_combine_all_empty():
    o, l = O.splitkv_combine(np.zeros((3, 2, 512)), np.full((3, 2), -np.inf))
    assert np.all(o == 0) and np.all(np.isposinf(l))


# ----------------------------------------------------------------------------- scheduler
def test_sched_worked_example():
    g = gold("p2_step3_sched_example.json")
    parts, prefix = O.sched_plan(g["topk_per_req"], g["block"], g["overhead"], g["num_parts"])
    assert len(parts) == g["num_parts"]
    for p, want in zip(parts, g["parts_as_printed"]):
        d = dict(zip(O.SCHED_FIELDS, p))
        for k, v in want.items():
            assert d[k] == int(v), (k, d, want)
    for p in parts[g["idle_from_part"]:]:
        assert p[0] >= len(g["topk_per_req"])
    assert prefix == g["num_splits_prefix"]


def _check_plan(topks, block, ovh, nparts):
    parts, prefix = O.sched_plan(topks, block, ovh, nparts)
    n = len(topks)
    blocks = [(t + block - 1) // block for t in topks]
    payload = (sum(b + ovh for b in blocks) + nparts - 1) // nparts + ovh
    covered = [[] for _ in range(n)]
    split_ids = [[] for _ in range(n)]
    for (br, er, bb, eb, bs, fs, ls) in parts:
        if br >= n:
            continue
        load = 0
        for r in range(br, er + 1):
            lo = bb if r == br else 0
            hi = eb if r == er else blocks[r]
            assert lo <= hi
            covered[r].append((lo, hi))
            split_ids[r].append(bs if r == br else prefix[r])
            load += hi - lo + ovh
        assert load <= payload
        assert fs == int(bb > 0)
        assert ls == int(eb < blocks[er])
    for r in range(n):
        # blocks of each request covered exactly once, in order, by prefix[r+1]-prefix[r] splits
        segs = covered[r]
        assert segs[0][0] == 0 and segs[-1][1] == blocks[r]
        for a, b in zip(segs[:-1], segs[1:]):
            assert a[1] == b[0]
        assert len(segs) == prefix[r + 1] - prefix[r]
        assert split_ids[r] == list(range(prefix[r], prefix[r + 1]))


@pytest.mark.parametrize("topks,block,ovh,nparts", [
    ([2048] * 64, 64, 5, 256), ([2048] * 64, 32, 5, 256), ([2048] * 64, 32, 0, 256),
    ([2048] * 128, 64, 5, 512), ([2048] * 4, 32, 0, 256), ([128, 128], 64, 5, 66),
    ([1, 2048, 7, 300, 0, 64], 32, 2, 13), ([5] * 40, 32, 1, 7), ([4096], 64, 5, 300),
])
def test_sched_invariants(topks, block, ovh, nparts):
    _check_plan(topks, block, ovh, nparts)


def test_sched_random_invariants():
    rng = np.random.default_rng(5)
    for _ in range(200):
        n = int(rng.integers(1, 40))
        topks = rng.integers(1, 3000, size=n).tolist()
        _check_plan(topks, int(rng.choice([16, 32, 64])), int(rng.integers(0, 7)),
                    int(rng.integers(1, 300)))
