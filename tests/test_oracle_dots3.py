"""Pins for DOTS3_SWA rows in the oracle (CPU only).

FlashInfer #4802's description gives DOTS3_SWA as d_qk = 1088, d_v = 1024
and 1160 bytes per token with the scales in a footer.  The oracle reads the
row as 1024 e4m3 codes, 64 BF16 rope values and eight one-byte power-of-two
exponents (bias 127), one per 128-element tile, and writes it with the
power-of-two scale rule of the DSv3.2 FP8 rows.  These tests pin:
  * the writer against the FP8 writer (itself pinned against torch's e4m3
    decoder and the power-of-two closed form): each half of a DOTS3 row
    must carry exactly the codes and scales of an FP8 row of that half;
  * the scale byte against an exact rational search for the smallest
    power of two, and its special values;
  * the split form and combine against the prefill form at d_v = 1024.
Dense attention, masking, permutation, closed forms and probability sums at
d_v = 1024 are covered by test_oracle_attention.py, which runs every format.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sparse_top_mla_smla_amd import workloads as W

from helpers import dense_attention, np_dequant, oracle_pool, q_f64

F = W.FMT_FP8_DOTS3


def case(seed=0, **kw):
    base = dict(T=5, H=4, n_seqs=1, ctx=704, topk=513, causal=True)
    base.update(kw)
    return W.make_case("dots3", config_id=130, seed=seed, fmt=F, **base)


def test_dims_and_row_bytes():
    assert oracle.row_bytes(F) == 1160 == 1024 + 2 * 64 + 8
    assert oracle.d_k(F) == 1088 and oracle.d_v(F) == 1024
    assert oracle.d_k(W.FMT_FP8) == 576 and oracle.d_v(W.FMT_FP8) == 512


def fp8_rows_of_halves(kv):
    """The FP8 (656-byte) rows of [nope half, rope] for each half of kv rows."""
    n = kv.shape[0]
    out = []
    for half in range(2):
        x = np.ascontiguousarray(np.concatenate([kv[:, 512 * half:512 * (half + 1)], kv[:, 1024:1088]], axis=1))
        pool = oracle.Pool(np.zeros((1, 64 * 656), np.uint8), W.FMT_FP8, 64 * 656)
        oracle.quantize_kv(x, np.arange(n, dtype=np.int32), pool)
        out.append(pool.data.reshape(64, 656)[:n])
    return out


@pytest.mark.parametrize("spread", [1.0, 1e-3, 3e4])
def test_writer_matches_the_fp8_writer_per_half(spread):
    rng = np.random.default_rng(int(spread * 10) + 1)
    kv = W.f32_to_bf16_bits((rng.standard_normal((64, 1088)) * spread).astype(np.float32))
    kv[3, :128] = 0                                    # an all-zero tile: scale 1
    pool = oracle.Pool(np.zeros((1, 64 * 1160), np.uint8), F, 64 * 1160)
    oracle.quantize_kv(kv, np.arange(64, dtype=np.int32), pool)
    rows = pool.data.reshape(64, 1160)
    h0, h1 = fp8_rows_of_halves(kv)
    assert np.array_equal(rows[:, :512], h0[:, :512])
    assert np.array_equal(rows[:, 512:1024], h1[:, :512])
    for g in range(8):
        ref = (h0 if g < 4 else h1)[:, 512 + 4 * (g % 4):516 + 4 * (g % 4)].copy().view(np.float32)[:, 0]
        got = np.ldexp(1.0, rows[:, 1152 + g].astype(np.int64) - 127)
        assert np.array_equal(got, ref.astype(np.float64)), g
    assert np.array_equal(rows[:, 1024:1152].copy().view(np.uint16), kv[:, 1024:1088])
    assert rows[3, 1152] == 127


def smallest_pow2_exponent(amax: float) -> int:
    """Smallest k with amax / 2^k <= 448, by exact rational search."""
    a = Fraction(amax)
    k = -200
    while a / (Fraction(2) ** k if k >= 0 else Fraction(1, 2 ** -k)) > 448:
        k += 1
    return k


@pytest.mark.parametrize("amax", [448.0, 448.0001, 1.0, 0.75, 3.0e4, 1e-30, 2.0 ** -100, 3.3895e38, 1e-37])
def test_scale_byte_is_the_smallest_power_of_two(amax):
    a32 = float(np.float32(amax))
    k = max(smallest_pow2_exponent(a32), -126)
    assert oracle.e8m0_scale(a32) == k + 127


def test_scale_byte_special_values():
    assert oracle.e8m0_scale(0.0) == 127                  # scale 1
    assert oracle.e8m0_scale(2.0 ** -133) == 1            # (the least BF16) raised to 2^-126: never byte 0
    assert oracle.e8m0_decode(127) == 1.0
    assert oracle.e8m0_decode(0) == 2.0 ** -127
    assert oracle.e8m0_decode(254) == 2.0 ** 127
    assert np.isnan(oracle.e8m0_decode(255))


def test_dequant_matches_the_independent_decoder():
    c = case(seed=1)
    pool = oracle_pool(c)
    slots = c.slots[::7]
    assert np.array_equal(oracle.dequant_rows(pool, slots), np_dequant(pool, slots))


def test_rope_enters_scores_and_not_values():
    """One candidate: the output is its 1024 nope values (V holds no rope
    part) and the LSE is its score over all 1088 dimensions."""
    c = case(seed=2, T=2, H=2)
    pool = oracle_pool(c)
    K = np_dequant(pool, c.slots)
    idx = np.full((2, c.topk), -1, np.int32)
    idx[:, 0] = c.slots[5]
    _, _, of, lf = oracle.prefill(c.q, pool, idx, sm_scale=c.sm_scale)
    q = q_f64(c)
    for t in range(2):
        for h in range(2):
            assert np.allclose(of[t, h], K[5, :1024], atol=1e-12, rtol=0)
            assert abs(lf[t, h] - float(c.sm_scale) * q[t, h] @ K[5]) < 1e-9


def test_sparse_513_list_equals_dense_over_selected_rows():
    c = case(seed=3, with_sink=True, with_topk_length=True)
    pool = oracle_pool(c)
    _, _, of, lf = oracle.prefill(c.q, pool, c.indices, topk_length=c.topk_length, sink=c.sink,
                                  sm_scale=c.sm_scale)
    q = q_f64(c)
    for t in range(c.T):
        row = c.indices[t][: c.topk_length[t]]
        K = np_dequant(pool, row[row >= 0])
        for h in range(c.H):
            o_ref, l_ref = dense_attention(q[t:t + 1, h], K, float(c.sm_scale), float(c.sink[h]), dv=1024)
            assert np.allclose(of[t, h], o_ref[0], atol=1e-12, rtol=0)
            assert abs(lf[t, h] - l_ref[0]) < 1e-12


@pytest.mark.parametrize("S", [1, 3, 9])
def test_split_and_combine_equal_prefill(S):
    c = case(seed=4, with_sink=True, with_topk_length=True)
    pool = oracle_pool(c)
    _, _, of, lf = oracle.prefill(c.q, pool, c.indices, topk_length=c.topk_length, sink=c.sink,
                                  sm_scale=c.sm_scale)
    po, pl = oracle.decode_split(c.q, pool, c.indices, S, topk_length=c.topk_length, sm_scale=c.sm_scale)
    assert po.shape == (c.T, S, c.H, 1024)
    _, _, cf, clf = oracle.combine(po, pl, sink=c.sink)
    assert np.allclose(cf, of, atol=1e-12, rtol=0)
    assert np.allclose(clf, lf, atol=1e-12, rtol=0)
