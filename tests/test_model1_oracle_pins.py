"""Pins for the oracle's V4 / V4.1 cache decode (d_qk = 512, struct-of-arrays
pages, e8m0 scales).  Every check compares the oracle with something other
than itself: PyTorch's e8m0 / e4m3 / bf16 dtypes, the quantisation example
the pages print, an encoder written here from the layout reading, and the
already pinned V3.2 path on caches that hold the same numbers.  CPU only."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- an encoder of its own
def _pow2_scale_exp(amax):
    """Exponent of the smallest power of two >= amax / 448 (amax clamped to 1e-4)."""
    r = np.maximum(amax, 1e-4) / 448.0
    m, e = np.frexp(r)
    return np.where(m == 0.5, e - 1, e)


def _encode_groups(x, group):
    """x float32 [n, d] -> (e4m3 code bytes [n, d], e8m0 scale bytes [n, d / group])."""
    n, d = x.shape
    g = x.reshape(n, d // group, group).astype(np.float64)
    ex = _pow2_scale_exp(np.abs(g).max(axis=-1))
    scaled = (g / np.exp2(ex)[..., None]).astype(np.float32).reshape(n, d)
    codes = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, (ex + 127).astype(np.uint8)


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _torch_dequant(codes, scale_bytes, group):
    """Library dequant: e4m3 codes times e8m0 scales through torch dtypes."""
    c = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(np.ascontiguousarray(scale_bytes)).view(torch.float8_e8m0fnu).to(torch.float64)
    n, d = c.shape
    return (c.reshape(n, d // group, group) * s[..., None]).reshape(n, d).numpy()


def _token_bytes_v41(x):
    codes, sc = _encode_groups(x, 32)
    return codes, sc                                   # data [n, 512], scales [n, 16]


def _token_bytes_v4(x, rng):
    codes, sc = _encode_groups(x[:, :448], 64)
    data = np.concatenate([codes, _bf16_bits(x[:, 448:]).astype("<u2").view(np.uint8).reshape(len(x), 128)], axis=1)
    pad = rng.integers(0, 256, size=(len(x), 1), dtype=np.uint8)       # the eighth byte is ignored
    return data, np.concatenate([sc, pad], axis=1)      # data [n, 576], scales [n, 8]


def _build_cache(data, scales, P, nb, stride, rng, perm):
    """Token perm[i] gets row i.  Page layout: P data rows, then P scale rows,
    then (stride > P * bytes per token) bytes that must never be read."""
    db, sb = data.shape[1], scales.shape[1]
    assert stride >= P * (db + sb)
    kv = rng.integers(0, 256, size=(nb, stride), dtype=np.uint8)
    for i, t in enumerate(perm):
        blk, off = divmod(int(t), P)
        kv[blk, off * db:(off + 1) * db] = data[i]
        kv[blk, P * db + off * sb:P * db + (off + 1) * sb] = scales[i]
    return kv


# ----------------------------------------------------------------------------- element decode
def test_e8m0_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = O.e8m0_value(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and np.isnan(got[255])


def test_e8m0_scale_of_the_printed_example():
    # the walkthrough's group with amax 0.75 gets the power-of-two scale 2^-9;
    # as an e8m0 byte that is 118, and the element 0.25 is the code 128.0
    g = gold("p2_step4_quant_example.json")
    x = np.zeros((1, 512), np.float32)
    x[0, 0] = g["element_value"]
    x[0, 1] = -g["group_amax"]
    codes, sc = _token_bytes_v41(x)
    assert sc[0, 0] == 127 + g["ue8m0_scale_exponent"]
    assert abs(O.e8m0_value(sc[0, 0]) - g["ue8m0_scale_as_printed"]) < 1e-6
    assert O.e4m3fn_value(codes[0, 0]) == g["element_code_value_as_printed"]
    assert O.decode_v41_rows(codes, sc)[0, 0] == g["element_value"]


# ----------------------------------------------------------------------------- row decode
@pytest.mark.parametrize("fmt", [O.FMT_V4, O.FMT_V41])
def test_row_decode_matches_library_dequant(fmt):
    rng = np.random.default_rng(11 + fmt)
    n = 96
    x = (rng.standard_normal((n, 512)) * rng.uniform(1e-3, 1e3, size=(n, 1))).astype(np.float32)
    if fmt == O.FMT_V41:
        data, sc = _token_bytes_v41(x)
        got = O.decode_v41_rows(data, sc)
        ref = _torch_dequant(data, sc, 32)
    else:
        data, sc = _token_bytes_v4(x, rng)
        got = O.decode_v4_rows(data, sc)
        ref = np.concatenate([_torch_dequant(data[:, :448], sc[:, :7], 64),
                              torch.from_numpy(x[:, 448:]).to(torch.bfloat16).to(torch.float64).numpy()], axis=1)
    assert got.shape == (n, 512)
    assert np.array_equal(got, ref)
    # and the decoded values are x within e4m3 rounding (bf16 for the V4 tail)
    gsz = 32 if fmt == O.FMT_V41 else 64
    nq = 512 if fmt == O.FMT_V41 else 448
    sc_v = np.repeat(O.e8m0_value(sc[:, :nq // gsz]), gsz, axis=1)
    err = np.abs(got[:, :nq] - x[:, :nq])
    assert np.all(err <= np.maximum(np.abs(x[:, :nq]) * 2.0 ** -4, sc_v * 2.0 ** -10))
    if fmt == O.FMT_V4:
        assert np.all(np.abs(got[:, 448:] - x[:, 448:]) <= np.abs(x[:, 448:]) * 2.0 ** -8)


def test_v4_pad_byte_and_group_boundaries():
    # one group at a time: a code in group g scaled by scale byte g only
    rng = np.random.default_rng(3)
    data = np.zeros((7, 576), np.uint8)
    sc = np.full((7, 8), 127, np.uint8)
    code_one = torch.tensor([1.0]).to(torch.float8_e4m3fn).view(torch.uint8).item()
    for g in range(7):
        data[g, 64 * g + 63] = code_one
        sc[g, g] = 127 + g + 1
        sc[g, 7] = rng.integers(0, 256)
    K = O.decode_v4_rows(data, sc)
    for g in range(7):
        expect = np.zeros(512)
        expect[64 * g + 63] = 2.0 ** (g + 1)
        assert np.array_equal(K[g], expect)


# ----------------------------------------------------------------------------- page addressing
@pytest.mark.parametrize("fmt,P,pad", [(O.FMT_V41, 64, 0), (O.FMT_V41, 16, 48), (O.FMT_V4, 64, 16), (O.FMT_V4, 3, 0)])
def test_struct_of_arrays_addressing(fmt, P, pad):
    rng = np.random.default_rng(5 * P + fmt)
    nb = 5
    n = nb * P
    x = (rng.standard_normal((n, 512)) * 0.5).astype(np.float32)
    data, sc = _token_bytes_v41(x) if fmt == O.FMT_V41 else _token_bytes_v4(x, rng)
    perm = rng.permutation(n)
    stride = P * (data.shape[1] + sc.shape[1]) + pad
    kv = _build_cache(data, sc, P, nb, stride, rng, perm)
    dec = O.decode_v41_rows if fmt == O.FMT_V41 else O.decode_v4_rows
    want = dec(data, sc)                                 # row i belongs to token perm[i]
    m = min(40, n)
    ids = np.concatenate([perm[:m], [-1, n, n + 7]]).astype(np.int32)
    rows, valid = O.gather_dequant(kv, ids, fmt, P)
    assert rows.shape == (len(ids), 512)
    assert np.array_equal(valid, np.r_[np.ones(m, bool), np.zeros(3, bool)])
    assert np.array_equal(rows[:m], want[:m])
    assert np.all(rows[m:] == 0.0)


# ----------------------------------------------------------------------------- same numbers, other format
def _v32_row(vals, scale):
    """656-byte V3.2 row holding vals [512] (codes of vals / scale) and a zero RoPE part."""
    row = np.zeros(656, np.uint8)
    row[:512] = torch.from_numpy((vals / scale).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    row[512:528] = np.full(4, scale, "<f4").view(np.uint8)
    return row


@pytest.mark.parametrize("fmt", [O.FMT_V4, O.FMT_V41])
def test_decode_agrees_with_v32_path_on_equal_numbers(fmt):
    # a token whose 512 dims are e4m3 values times one power of two s decodes
    # the same in V3.2 (rope zero, q rope zero) and in V4 / V4.1 (every scale
    # byte s; the V4 tail holds the same values as bf16, exact for 3-bit
    # mantissas), so the attention outputs must agree exactly
    rng = np.random.default_rng(21 + fmt)
    P, nb, h, topk = 16, 4, 8, 24
    n = P * nb
    s_exp = rng.integers(-6, 3, size=n)
    codes = torch.from_numpy((rng.standard_normal((n, 512)) * 60).astype(np.float32)).to(torch.float8_e4m3fn)
    vals = codes.to(torch.float64).numpy() * np.exp2(s_exp)[:, None]
    assert np.all(np.isfinite(vals))
    v32 = np.stack([_v32_row(vals[t], 2.0 ** s_exp[t]) for t in range(n)]).reshape(nb, P, 1, 656)
    code_b = codes.view(torch.uint8).numpy()
    if fmt == O.FMT_V41:
        data = code_b
        sc = np.repeat((s_exp + 127).astype(np.uint8)[:, None], 16, axis=1)
    else:
        data = np.concatenate([code_b[:, :448], _bf16_bits(vals[:, 448:]).astype("<u2").view(np.uint8).reshape(n, 128)], axis=1)
        sc = np.concatenate([np.repeat((s_exp + 127).astype(np.uint8)[:, None], 7, axis=1), np.zeros((n, 1), np.uint8)], axis=1)
    kv = _build_cache(data, sc, P, nb, P * (data.shape[1] + sc.shape[1]), rng, np.arange(n))
    q = _bf16_bits(rng.standard_normal((1, 2, h, 512)).astype(np.float32))
    q576 = np.concatenate([q, np.zeros((1, 2, h, 64), np.uint16)], axis=-1)
    idx = rng.integers(-1, n, size=(1, 2, topk)).astype(np.int32)
    o_a, l_a = O.sparse_mla_decode(q, kv, idx, 0.04, fmt, P)
    o_b, l_b = O.sparse_mla_decode(q576, v32, idx, 0.04, O.FMT_FP8, P)
    assert np.array_equal(o_a, o_b) and np.array_equal(l_a, l_b)


def test_attention_matches_torch_on_decoded_rows():
    # the d_qk = 512 decode is the usual softmax(q K^T s) K over the valid slots
    rng = np.random.default_rng(8)
    P, nb, h, topk = 8, 6, 4, 20
    n = P * nb
    x = (rng.standard_normal((n, 512)) * 0.3).astype(np.float32)
    data, sc = _token_bytes_v41(x)
    kv = _build_cache(data, sc, P, nb, P * 528, rng, np.arange(n))
    K = torch.from_numpy(_torch_dequant(data, sc, 32))
    q = _bf16_bits(rng.standard_normal((1, 1, h, 512)).astype(np.float32))
    idx = rng.integers(-1, n, size=(1, 1, topk)).astype(np.int32)
    out, lse = O.sparse_mla_decode(q, kv, idx, 0.05, O.FMT_V41, P)
    qt = torch.from_numpy(q[0, 0].view(np.int16)).view(torch.bfloat16).to(torch.float64)
    ids = torch.from_numpy(idx[0, 0]).long()
    ok = ids >= 0
    Ks = K[ids.clamp(min=0)][ok]
    s = (qt @ Ks.T) * 0.05
    ref = torch.softmax(s, dim=-1) @ Ks
    assert np.allclose(out[0, 0], ref.numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(lse[0, :, 0], torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12)


# ----------------------------------------------------------------------------- FP4 extra cache
# The OCP FP4 (E2M1) value set: codes 0..7 are the magnitudes below, codes
# 8..15 their negatives.
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_codes_are_the_format_values():
    got = O.e2m1_value(np.arange(16))
    assert got[:8].tolist() == E2M1_MAGNITUDES
    assert (-got[8:]).tolist() == E2M1_MAGNITUDES and np.all(np.signbit(got[8:]))
    # every value is exact in e4m3 (so an FP4 token can be restated as V4.1)
    e4 = torch.tensor(got.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(e4, got)


def _fp4_code(x):
    """Nearest e2m1 code of x (ties to the even code), by search over the value set."""
    vals = np.array(E2M1_MAGNITUDES)
    mag = np.abs(x)
    d = np.abs(mag[..., None] - vals)
    best = np.argmin(d + 1e-9 * (np.arange(8) % 2), axis=-1)          # ties: the even code
    return (best | np.where(x < 0, 8, 0)).astype(np.uint8)


def _fp4_tokens(x):
    """x float32 [n, 512] -> (data [n, 256], scales [n, 32]): scale 2^ceil(log2(amax / 6))."""
    n = x.shape[0]
    g = x.reshape(n, 32, 16).astype(np.float64)
    amax = np.maximum(np.abs(g).max(axis=-1), 1e-4)
    m, e = np.frexp(amax / 6.0)
    ex = np.where(m == 0.5, e - 1, e)
    codes = _fp4_code(g / np.exp2(ex)[..., None]).reshape(n, 512)
    data = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return data, (ex + 127).astype(np.uint8)


def test_fp4_nibble_order_and_scale_groups():
    data = np.zeros((1, 256), np.uint8)
    data[0, 0] = 0x72            # element 0 = code 2 (1.0), element 1 = code 7 (6.0)
    data[0, 9] = 0xB0            # element 18 = 0, element 19 = code 11 (-1.5)
    sc = np.full((1, 32), 127, np.uint8)
    sc[0, 1] = 130               # dims 16..31 scaled by 8
    K = O.decode_fp4_rows(data, sc)[0]
    want = np.zeros(512)
    want[0], want[1], want[19] = 1.0, 6.0, -1.5 * 8
    assert np.array_equal(K, want)


def test_fp4_row_decode_matches_the_encoder():
    rng = np.random.default_rng(41)
    x = (rng.standard_normal((64, 512)) * rng.uniform(1e-2, 1e2, size=(64, 1))).astype(np.float32)
    data, sc = _fp4_tokens(x)
    K = O.decode_fp4_rows(data, sc)
    scale = np.repeat(np.exp2(sc.astype(np.float64) - 127), 16, axis=1)
    nib = np.stack([data & 0xF, data >> 4], axis=-1).reshape(64, 512)
    mag = np.array(E2M1_MAGNITUDES)[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    assert np.array_equal(K, mag * scale)
    # within half a step of the e2m1 grid (largest gap 2, at 4..6) of the value
    assert np.all(np.abs(K - x) <= scale * 1.0 + 1e-12)


def _v41_from_fp4(data, sc):
    """The same numbers as a V4.1 token (codes to e4m3, one scale per 32),
    possible when both 16-groups of each 32-group share their scale."""
    assert np.array_equal(sc[:, 0::2], sc[:, 1::2])
    vals = O.decode_fp4_rows(data, np.full_like(sc, 127))            # e2m1 values (scale 1)
    codes = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, sc[:, 0::2].copy()


@pytest.mark.parametrize("with_lengths", [False, True])
def test_extra_slots_equal_the_same_tokens_in_the_main_cache(with_lengths):
    # FP4 tokens whose two 16-groups per 32 share a scale are V4.1 tokens in
    # disguise: attention over main slots + extra slots must equal attention
    # over the concatenated slots of one V4.1 cache holding all the tokens
    rng = np.random.default_rng(43)
    P, h = 16, 8
    nm, nx = 6 * P, 4 * P                                   # main and extra tokens
    xm = (rng.standard_normal((nm, 512)) * 0.5).astype(np.float32)
    dm, sm = _token_bytes_v41(xm)
    xx = (rng.standard_normal((nx, 512)) * 0.5).astype(np.float32)
    dx, sx = _fp4_tokens(xx)
    sx[:, 1::2] = sx[:, 0::2]                              # shared scale per 32 (values shrink or stay)
    main = _build_cache(dm, sm, P, nm // P, P * 528, rng, np.arange(nm))
    extra = _build_cache(dx, sx, P, nx // P, P * 288 + 32, rng, np.arange(nx))
    dxc, sxc = _v41_from_fp4(dx, sx)
    both = _build_cache(np.concatenate([dm, dxc]), np.concatenate([sm, sxc]), P, (nm + nx) // P, P * 528, rng,
                        np.arange(nm + nx))
    b, s_q, tk, xk = 3, 2, 40, 24
    q = _bf16_bits(rng.standard_normal((b, s_q, h, 512)).astype(np.float32))
    idx = rng.integers(-1, nm, size=(b, s_q, tk)).astype(np.int32)
    xidx = rng.integers(-1, nx + 3, size=(b, s_q, xk)).astype(np.int32)   # some out of range
    mlen = np.array([40, 13, 0]) if with_lengths else None
    xlen = np.array([5, 24, 30]) if with_lengths else None
    out, lse = O.sparse_mla_decode(q, main, idx, 0.04, O.FMT_V41, P, topk_length=mlen,
                                   extra={"kv": extra, "indices": xidx, "page_block_size": P, "topk_length": xlen})
    cat = np.concatenate([idx, np.where((xidx >= 0) & (xidx < nx), xidx + nm, -1)], axis=-1).astype(np.int32)
    if with_lengths:
        for bi in range(b):
            cat[bi, :, max(0, min(mlen[bi], tk)):tk] = -1
            cat[bi, :, tk + max(0, min(xlen[bi], xk)):] = -1
    ref_o, ref_l = O.sparse_mla_decode(q, both, cat, 0.04, O.FMT_V41, P)
    assert np.array_equal(out, ref_o) and np.array_equal(lse, ref_l)
