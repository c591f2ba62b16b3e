"""Pins for the oracle's cache codec (CPU only).

The e4m3 decode/encode are pinned to torch's float8_e4m3fn conversions (a
library implementation of the OCP OFP8 E4M3 format) and to closed-form values
of that format; the quantizer is pinned to the row layout the FlashInfer
PR #4802 review states (golden fixture) and to invariants that any correct
power-of-two per-128 scale must satisfy.
"""
import json
import os

import numpy as np
import pytest
import torch

from sparse_top_mla_smla_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_e4m3_decode(codes):
    return torch.tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def torch_e4m3_encode(y):
    return torch.tensor(np.asarray(y, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_codes_vs_torch(orc):
    codes = np.arange(256)
    ref = torch_e4m3_decode(codes)
    got = np.array([orc.e4m3_decode(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.all(np.isnan(got[nan]))
    assert np.array_equal(got[~nan], ref[~nan].astype(np.float64))


def test_e4m3_decode_closed_form(orc):
    # OCP E4M3: bias 7, 3 mantissa bits, E=0 subnormal M*2^-9, max 448.
    assert orc.e4m3_decode(0x7E) == 448.0
    assert orc.e4m3_decode(0x08) == 2.0 ** -6
    assert orc.e4m3_decode(0x07) == 7 * 2.0 ** -9
    assert orc.e4m3_decode(0x01) == 2.0 ** -9
    assert orc.e4m3_decode(0x38) == 1.0
    assert orc.e4m3_decode(0xB8) == -1.0
    v = orc.e4m3_decode(0x80)
    assert v == 0.0 and np.signbit(v)


def all_bf16_in_range(limit=448.0):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = W.bf16_bits_to_f32(bits)
    ok = np.isfinite(f) & (np.abs(f) <= limit)
    return f[ok]


def test_e4m3_encode_exhaustive_bf16_vs_torch(orc):
    ys = all_bf16_in_range()
    got = np.array([orc.e4m3_encode(float(y)) for y in ys], dtype=np.uint8)
    ref = torch_e4m3_encode(ys)
    assert np.array_equal(got, ref)


def test_e4m3_encode_ties_to_even(orc):
    # exact midpoints between neighbouring positive e4m3 values (float32 exact)
    vals = np.array([orc.e4m3_decode(c) for c in range(0x7F)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)
    got = np.array([orc.e4m3_encode(float(m)) for m in mids])
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)   # the even code of the pair
    assert np.array_equal(got, want)
    got_neg = np.array([orc.e4m3_encode(float(-m)) for m in mids])
    assert np.array_equal(got_neg, want | 0x80)
    assert np.array_equal(got, torch_e4m3_encode(mids))


def test_e4m3_encode_sign_of_zero_and_saturation(orc):
    assert orc.e4m3_encode(-1e-5) == 0x80
    assert orc.e4m3_encode(2.0 ** -10) == 0x00
    assert orc.e4m3_encode(3 * 2.0 ** -10) == 0x02
    assert orc.e4m3_encode(448.0) == 0x7E
    assert orc.e4m3_encode(1000.0) == 0x7E
    assert orc.e4m3_encode(-1000.0) == 0xFE


def test_fp8_scale_pow2_and_range(orc):
    amax = np.abs(all_bf16_in_range(limit=np.inf))
    amax = np.unique(amax[amax > 0])
    floor = 2.0 ** -126                                # the least normal float32
    for a in amax[:: 7]:
        s = orc.fp8_scale(float(a))
        m, e = np.frexp(s)
        assert m == 0.5 and s >= floor, (a, s)         # a normal power of two
        r = np.float64(a) / s
        assert r <= 448.0, (a, s, r)
        if s > floor:
            assert r > 224.0, (a, s, r)                # the smallest such power
    assert orc.fp8_scale(0.0) == 1.0
    assert orc.fp8_scale(448.0) == 1.0
    assert orc.fp8_scale(448.0 * 2 ** -7) == 2.0 ** -7
    assert orc.fp8_scale(449.0) == 2.0
    # tiles whose amax/448 is below the least normal float32 keep scale 2^-126
    assert orc.fp8_scale(448.0 * floor) == floor
    assert orc.fp8_scale(448.0 * floor * 1.5) == 2 * floor
    assert orc.fp8_scale(1e-38) == floor
    assert orc.fp8_scale(float(np.float32(2.0 ** -140))) == floor


def _pool_for(fmt, n_rows, seed=0, tweak=None):
    rng = np.random.default_rng(seed)
    kv = W.f32_to_bf16_bits(rng.standard_normal((n_rows, 576), dtype=np.float32))
    if tweak is not None:
        kv = tweak(kv)
    nb = (n_rows + 63) // 64
    rb = W.ROW_BYTES[fmt]
    import oracle
    pool = oracle.Pool(np.zeros((nb, 64 * rb), dtype=np.uint8), fmt, 64 * rb)
    slots = np.arange(n_rows, dtype=np.int32)
    oracle.quantize_kv(kv, slots, pool)
    return kv, pool


def test_row_layout_golden(orc):
    g = json.load(open(os.path.join(GOLDEN, "row_layout_dsv32.json")))
    assert orc.row_bytes(W.FMT_FP8) == g["row_bytes"] == 656
    kv, pool = _pool_for(W.FMT_FP8, 64)
    rows = pool.data.reshape(64, 656)
    x = W.bf16_bits_to_f32(kv)
    s0, s1 = g["scales_fp32_one_per_128"]
    r0, r1 = g["rope_bf16_64"]
    scales = rows[:, s0:s1].copy().view(np.float32)
    assert scales.shape == (64, 4)
    codes = rows[:, g["nope_fp8_e4m3"][0]:g["nope_fp8_e4m3"][1]]
    dec = torch_e4m3_decode(codes.reshape(-1)).reshape(64, 512).astype(np.float64)
    deq = dec * np.repeat(scales.astype(np.float64), 128, axis=1)
    # half an e4m3 ulp of the value, times the scale, bounds the error
    err = np.abs(deq - x[:, :512])
    assert np.all(err <= np.repeat(scales, 128, axis=1) * 2.0 ** -9 / 2 + np.abs(x[:, :512]) * 2.0 ** -4 + 0)
    assert np.array_equal(rows[:, r0:r1].copy().view(np.uint16), kv[:, 512:])


def test_fp8_quantizer_invariants(orc):
    def tweak(kv):
        kv = kv.copy()
        kv[0, :128] = 0                                 # amax = 0 tile
        kv[1, 128:256] = W.f32_to_bf16_bits(np.full(128, -0.0, np.float32))
        kv[2, :128] = W.f32_to_bf16_bits(np.float32(1e-30) * np.arange(128, dtype=np.float32))
        kv[3, 256:384] = W.f32_to_bf16_bits(np.float32(3e4) * np.linspace(-1, 1, 128, dtype=np.float32))
        kv[4, 384:512] = W.f32_to_bf16_bits(np.float32(1e-38) * np.arange(128, dtype=np.float32))
        return kv
    kv, pool = _pool_for(W.FMT_FP8, 192, seed=3, tweak=tweak)
    rows = pool.data.reshape(-1, 656)[:192]
    x = W.bf16_bits_to_f32(kv)[:, :512].reshape(192, 4, 128).astype(np.float64)
    scales = rows[:, 512:528].copy().view(np.float32).astype(np.float64)
    codes = rows[:, :512].reshape(192, 4, 128)
    dec = torch_e4m3_decode(codes.reshape(-1)).reshape(192, 4, 128).astype(np.float64)
    amax = np.abs(x).max(axis=2)
    y = x / scales[:, :, None]
    assert np.all(np.abs(y) <= 448.0)
    nz = amax > 0
    above = nz & (scales > 2.0 ** -126)
    assert np.all(amax[nz] / scales[nz] <= 448.0)
    assert np.all(amax[above] / scales[above] > 224.0)
    assert scales[4, 3] == 2.0 ** -126                  # amax/448 below the least normal float32
    assert np.abs(y[4, 3]).max() < 224.0
    assert np.all(scales[~nz] == 1.0)
    # the encoded code is the nearest e4m3 value to y (ties to even): compare with torch
    assert np.array_equal(codes.reshape(-1), torch_e4m3_encode(y.reshape(-1).astype(np.float32)))
    assert np.all(codes[1, 1] == 0x80)                 # -0.0 keeps its sign
    assert np.all(codes[0, 0] == 0x00)
    ay = np.abs(y)
    half_ulp = np.where(ay >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(ay, 2.0 ** -6))) - 4), 2.0 ** -10)
    assert np.all(np.abs(dec * scales[:, :, None] - x) <= scales[:, :, None] * half_ulp)


def test_int8_quantizer_vs_numpy(orc):
    kv, pool = _pool_for(W.FMT_INT8, 128, seed=5)
    rows = pool.data.reshape(-1, 656)[:128]
    x = W.bf16_bits_to_f32(kv)[:, :512].reshape(128, 4, 128)
    amax = np.abs(x).max(axis=2).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1), amax / np.float32(127)).astype(np.float32)
    got_scale = rows[:, 512:528].copy().view(np.float32)
    assert np.array_equal(got_scale, scale)
    q = np.clip(np.rint(x / scale[:, :, None]), -127, 127).astype(np.int8)
    assert np.array_equal(rows[:, :512].view(np.int8).reshape(128, 4, 128), q)
    assert np.array_equal(rows[:, 528:656].copy().view(np.uint16), kv[:, 512:])


def test_fp8_any_scale_quantizer(orc):
    """FP8 rows with arbitrary scales: scale = amax/448 in float32 (1 for an
    all-zero tile), codes = torch's e4m3 encoding of x/scale, the tile's
    largest magnitude encodes to 448, and the decoded value is within half an
    e4m3 ulp (times the scale) of x."""
    def tweak(kv):
        kv = kv.copy()
        kv[0, :128] = 0
        kv[2, 256:384] = W.f32_to_bf16_bits(np.float32(3e4) * np.linspace(-1, 1, 128, dtype=np.float32))
        kv[3, :128] = W.f32_to_bf16_bits(np.float32(1e-20) * np.arange(128, dtype=np.float32))
        return kv
    kv, pool = _pool_for(W.FMT_FP8_ANY, 128, seed=11, tweak=tweak)
    assert orc.row_bytes(W.FMT_FP8_ANY) == 656
    rows = pool.data.reshape(-1, 656)[:128]
    x32 = W.bf16_bits_to_f32(kv)[:, :512].reshape(128, 4, 128)
    amax = np.abs(x32).max(axis=2).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1), amax / np.float32(448)).astype(np.float32)
    got_scale = rows[:, 512:528].copy().view(np.float32)
    assert np.array_equal(got_scale, scale)
    assert got_scale[0, 0] == 1.0
    assert not np.all(np.log2(got_scale[1:]) == np.round(np.log2(got_scale[1:])))  # not powers of two
    y = (x32 / scale[:, :, None]).astype(np.float32)
    codes = rows[:, :512].reshape(128, 4, 128)
    assert np.array_equal(codes.reshape(-1), torch_e4m3_encode(y.reshape(-1)))
    top = np.abs(x32).argmax(axis=2)
    nz = amax > 0
    assert np.all((np.take_along_axis(codes, top[:, :, None], 2)[:, :, 0][nz] & 0x7F) == 0x7E)
    dec = torch_e4m3_decode(codes.reshape(-1)).reshape(128, 4, 128).astype(np.float64)
    ay = np.abs(y.astype(np.float64))
    half_ulp = np.where(ay >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(ay, 2.0 ** -6))) - 4), 2.0 ** -10)
    s64 = scale.astype(np.float64)[:, :, None]
    assert np.all(np.abs(dec * s64 - x32) <= s64 * half_ulp * (1 + 1e-6))
    assert np.array_equal(rows[:, 528:656].copy().view(np.uint16), kv[:, 512:])


def test_bf16_row_is_a_copy(orc):
    kv, pool = _pool_for(W.FMT_BF16, 64, seed=7)
    assert np.array_equal(pool.data.reshape(64, 1152).view(np.uint16), kv)


def test_double_to_bf16_vs_torch(orc):
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(3000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-38).astype(np.float32),
                        (rng.standard_normal(1000) * 1e30).astype(np.float32)])
    # exact ties: bf16 value plus half its ulp
    b = W.bf16_bits_to_f32(W.f32_to_bf16_bits(v[:500]))
    ties = (b.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, ties, np.float32([0.0, -0.0, 3.3895314e38])])
    got = np.array([orc.double_to_bf16(float(x)) for x in v], dtype=np.uint16)
    ref = torch.tensor(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_quantize_skips_out_of_range_slots(orc):
    import oracle
    rng = np.random.default_rng(2)
    kv = W.f32_to_bf16_bits(rng.standard_normal((4, 576), dtype=np.float32))
    pool = oracle.Pool(np.full((1, 64 * 656), 0xAB, dtype=np.uint8), W.FMT_FP8, 64 * 656)
    oracle.quantize_kv(kv, np.array([-1, 64, 5, 2 ** 31 - 1], dtype=np.int32), pool)
    rows = pool.data.reshape(64, 656)
    untouched = np.ones(64, bool)
    untouched[5] = False
    assert np.all(rows[untouched] == 0xAB)
    assert not np.all(rows[5] == 0xAB)
