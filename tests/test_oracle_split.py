"""Pins for the oracle's split-KV decode and LSE combine (CPU only).

Merging per-split partial results must reproduce the unsplit result (the
combine is exact up to rounding), the merged LSE must equal numpy's
logaddexp reduction of the partial LSEs (a library routine), and the split
geometry -- whole 64-wide chunks, contiguous ranges in list order -- fixes
which splits are empty.
"""
import numpy as np
import pytest

import oracle
from sparse_top_mla_smla_amd import workloads as W

from helpers import dense_attention, np_dequant, oracle_pool, q_f64


@pytest.mark.parametrize("topk,S,w", [(2048, 8, 256), (100, 3, 64), (64, 4, 64), (640, 8, 128),
                                      (1, 1, 64), (2048, 64, 64), (513, 2, 320), (1024, 3, 384)])
def test_split_width_closed_form(topk, S, w):
    assert oracle.split_width(topk, S) == w
    assert w % 64 == 0 and w * S >= topk and (w - 64) * S < topk


def case(fmt, seed, **kw):
    base = dict(T=5, H=3, n_seqs=1, ctx=512, topk=300, causal=True)
    base.update(kw)
    return W.make_case("split", config_id=105, seed=seed, fmt=fmt, **base)


@pytest.mark.parametrize("fmt", [W.FMT_BF16, W.FMT_FP8, W.FMT_INT8, W.FMT_FP8_ANY, W.FMT_FP8_NOPE])
@pytest.mark.parametrize("S", [1, 2, 3, 8, 16, 32])
def test_combine_of_splits_equals_unsplit(fmt, S):
    c = case(fmt, seed=S + 10 * fmt, with_topk_length=True, with_sink=True)
    pool = oracle_pool(c)
    _, _, of, lf = oracle.prefill(c.q, pool, c.indices, topk_length=c.topk_length, sink=c.sink,
                                  sm_scale=c.sm_scale)
    po, pl = oracle.decode_split(c.q, pool, c.indices, S, topk_length=c.topk_length,
                                 sm_scale=c.sm_scale)
    out, lse, of2, lf2 = oracle.combine(po, pl, sink=c.sink)
    fin = np.isfinite(lf)
    assert np.array_equal(fin, np.isfinite(lf2))
    assert np.allclose(of, of2, atol=1e-12, rtol=0)
    assert np.allclose(lf[fin], lf2[fin], atol=1e-12, rtol=0)
    # library pin for the merged LSE
    with np.errstate(divide="ignore"):
        ref = np.logaddexp.reduce(pl, axis=1)
    assert np.allclose(lf2[fin], ref[fin], atol=1e-12, rtol=0)


def test_empty_split_positions_and_partials():
    c = case(W.FMT_FP8, seed=3, with_topk_length=True)
    pool = oracle_pool(c)
    S = 8
    w = oracle.split_width(c.topk, S)
    po, pl = oracle.decode_split(c.q, pool, c.indices, S, topk_length=c.topk_length,
                                 sm_scale=c.sm_scale)
    q = q_f64(c)
    nslots = c.num_blocks * 64
    for t in range(c.T):
        for s in range(S):
            j0, j1 = s * w, min((s + 1) * w, c.topk, int(c.topk_length[t]))
            sel = [int(c.indices[t, j]) for j in range(j0, j1) if 0 <= c.indices[t, j] < nslots]
            if not sel:
                assert np.all(np.isneginf(pl[t, s])) and np.all(po[t, s] == 0)
                continue
            K = np_dequant(pool, sel)
            for h in range(c.H):
                o_ref, l_ref = dense_attention(q[t:t + 1, h], K, float(c.sm_scale))
                assert np.allclose(po[t, s, h], o_ref[0], atol=1e-12, rtol=0)
                assert abs(pl[t, s, h] - l_ref[0]) < 1e-12


def test_combine_all_empty_gives_zero_and_neg_inf():
    po = np.random.default_rng(0).standard_normal((2, 4, 3, 512))
    pl = np.full((2, 4, 3), -np.inf)
    pl[1, 2, 1] = 0.5
    out, lse, of, lf = oracle.combine(po, pl, sink=np.float32([0.1, 0.2, 0.3]))
    assert np.all(of[0] == 0) and np.all(np.isneginf(lf[0]))
    assert np.isneginf(lf[1, 0]) and np.isneginf(lf[1, 2]) and lf[1, 1] == 0.5
    # a single live split passes through, scaled by the sink factor
    f = 1 / (1 + np.exp(float(np.float32(0.2)) - 0.5))
    assert np.allclose(of[1, 1], po[1, 2, 1] * f, atol=1e-14, rtol=0)


def test_decode_with_sink_in_combine_matches_prefill_c1():
    c = W.c1_tiny()
    pool = oracle_pool(c)
    sink = np.float32([0.3, -1.0, 2.0, 0.0, 0.5, -0.5, 1.5, -2.0])
    _, _, of, lf = oracle.prefill(c.q, pool, c.indices, sink=sink, sm_scale=c.sm_scale)
    for S in (1, 2, 4):
        po, pl = oracle.decode_split(c.q, pool, c.indices, S, sm_scale=c.sm_scale)
        _, _, of2, lf2 = oracle.combine(po, pl, sink=sink)
        assert np.allclose(of, of2, atol=1e-12, rtol=0) and np.allclose(lf, lf2, atol=1e-12, rtol=0)
