"""Pins for DSv4 rows in the oracle (CPU only).

FlashInfer #4802 gives the DSv4 row only as 584 bytes, and V3.2-family
models d_v = 512.  The oracle reads the row as 448 e4m3 nope codes, 64 BF16
rope values and seven one-byte power-of-two exponents (bias 127), one per
64-element tile, plus a padding byte; K is the 512 values and V = K.  These
tests pin:
  * the writer against the FP8 writer: a 128-element FP8 tile holding one
    64-element DSv4 tile and 64 zeros has the same amax, so it must carry
    the same codes and the same power-of-two scale;
  * the byte layout (rope bytes copied, padding 0) and the dequantizer
    against an independent decoder;
  * V = K: one candidate's output is its whole 512-value row;
  * split + combine against prefill.
Dense attention, masking, permutation, closed forms and probability sums
run on every format in test_oracle_attention.py.
"""
import numpy as np
import pytest

import oracle
from sparse_top_mla_smla_amd import workloads as W

from helpers import np_dequant, oracle_pool, q_f64

F = W.FMT_FP8_DSV4


def case(seed=0, **kw):
    base = dict(T=5, H=4, n_seqs=1, ctx=640, topk=320, causal=True)
    base.update(kw)
    return W.make_case("dsv4", config_id=140, seed=seed, fmt=F, **base)


def test_dims_and_row_bytes():
    assert oracle.row_bytes(F) == 584 == 448 + 2 * 64 + 7 + 1
    assert oracle.d_k(F) == 512 and oracle.d_v(F) == 512


@pytest.mark.parametrize("spread", [1.0, 1e-3, 3e4])
def test_writer_matches_the_fp8_writer_per_tile(spread):
    rng = np.random.default_rng(int(spread * 10) + 7)
    kv = W.f32_to_bf16_bits((rng.standard_normal((64, 512)) * spread).astype(np.float32))
    kv[5, 64:128] = 0                                   # an all-zero tile: scale 1
    pool = oracle.Pool(np.full((1, 64 * 584), 0xEE, np.uint8), F, 64 * 584)
    oracle.quantize_kv(kv, np.arange(64, dtype=np.int32), pool)
    rows = pool.data.reshape(64, 584)
    for g in range(7):
        # FP8 rows whose 128-element tiles are [DSv4 tile g, 64 zeros]
        x = np.zeros((64, 576), np.uint16)
        x[:, :64] = kv[:, 64 * g:64 * (g + 1)]
        ref = oracle.Pool(np.zeros((1, 64 * 656), np.uint8), W.FMT_FP8, 64 * 656)
        oracle.quantize_kv(x, np.arange(64, dtype=np.int32), ref)
        r8 = ref.data.reshape(64, 656)
        assert np.array_equal(rows[:, 64 * g:64 * (g + 1)], r8[:, :64]), g
        scale8 = r8[:, 512:516].copy().view(np.float32)[:, 0].astype(np.float64)
        assert np.array_equal(np.ldexp(1.0, rows[:, 576 + g].astype(np.int64) - 127), scale8), g
    assert np.array_equal(rows[:, 448:576].copy().view(np.uint16), kv[:, 448:512])
    assert np.all(rows[:, 583] == 0)
    assert rows[5, 577] == 127


def test_dequant_matches_the_independent_decoder():
    c = case(seed=1)
    pool = oracle_pool(c)
    slots = c.slots[::5]
    assert np.array_equal(oracle.dequant_rows(pool, slots), np_dequant(pool, slots))


def test_value_is_the_whole_row():
    c = case(seed=2, T=2, H=3)
    pool = oracle_pool(c)
    K = np_dequant(pool, c.slots)
    idx = np.full((2, c.topk), -1, np.int32)
    idx[:, 7] = c.slots[11]
    _, _, of, lf = oracle.prefill(c.q, pool, idx, sm_scale=c.sm_scale)
    q = q_f64(c)
    for t in range(2):
        for h in range(3):
            assert np.allclose(of[t, h], K[11], atol=1e-12, rtol=0)          # rope values included
            assert abs(lf[t, h] - float(c.sm_scale) * q[t, h] @ K[11]) < 1e-9


@pytest.mark.parametrize("S", [1, 2, 5])
def test_split_and_combine_equal_prefill(S):
    c = case(seed=4, with_sink=True, with_topk_length=True)
    pool = oracle_pool(c)
    _, _, of, lf = oracle.prefill(c.q, pool, c.indices, topk_length=c.topk_length, sink=c.sink,
                                  sm_scale=c.sm_scale)
    po, pl = oracle.decode_split(c.q, pool, c.indices, S, topk_length=c.topk_length, sm_scale=c.sm_scale)
    assert po.shape == (c.T, S, c.H, 512)
    _, _, cf, clf = oracle.combine(po, pl, sink=c.sink)
    assert np.allclose(cf, of, atol=1e-12, rtol=0)
    assert np.allclose(clf, lf, atol=1e-12, rtol=0)
