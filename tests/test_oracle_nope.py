"""Pins for GLM53_NOPE rows in the oracle (CPU only).

FlashInfer #4802's KV layout comment: GLM53_NOPE reuses the 656-byte FP8
row, but bytes [528, 656) are reserved padding that is never gathered or
read as rope data.  The oracle's writer must leave them alone, its reader
must not use them, and scores must use the 512 nope dimensions only.
"""
import numpy as np

import oracle
from sparse_top_mla_smla_amd import workloads as W

from helpers import oracle_pool


def case(seed=0, **kw):
    base = dict(T=5, H=4, n_seqs=1, ctx=320, topk=96, causal=True, with_sink=True, with_topk_length=True)
    base.update(kw)
    return W.make_case("nope", config_id=120, seed=seed, fmt=W.FMT_FP8_NOPE, **base)


def test_writer_leaves_the_padding_and_matches_the_fp8_writer():
    c = case()
    nope = oracle_pool(c, fill=0xA7)
    c8 = case()
    c8.fmt = W.FMT_FP8
    fp8 = oracle_pool(c8, fill=0xA7)
    rows_n = nope.data.reshape(-1, 656)
    rows_8 = fp8.data.reshape(-1, 656)
    assert np.array_equal(rows_n[:, :528], rows_8[:, :528])
    assert np.all(rows_n[:, 528:] == 0xA7)


def test_padding_is_never_read():
    c = case(seed=1)
    a = oracle_pool(c)
    b = oracle_pool(c)
    b.data.reshape(-1, 656)[:, 528:] = 0xFF          # BF16 NaN patterns
    ra = oracle.prefill(c.q, a, c.indices, topk_length=c.topk_length, sink=c.sink, sm_scale=c.sm_scale)
    rb = oracle.prefill(c.q, b, c.indices, topk_length=c.topk_length, sink=c.sink, sm_scale=c.sm_scale)
    for x, y in zip(ra, rb):
        assert np.array_equal(x, y)


def test_scores_use_the_nope_dimensions_only():
    """With 512-wide q rows the result equals the FP8 result for the same
    q with zero rope dimensions over rows with zero rope values, and q
    elements past 512 are never read."""
    c = case(seed=2)
    pool = oracle_pool(c)
    q512 = np.ascontiguousarray(c.q[:, :, :512])
    r_nope = oracle.prefill(q512, pool, c.indices, topk_length=c.topk_length, sink=c.sink, sm_scale=c.sm_scale)
    # the same rows as FP8 rows whose rope values are zero, and q with zero rope
    c8 = case(seed=2)
    c8.fmt = W.FMT_FP8
    kv = c8.kv.copy()
    kv[:, 512:] = 0
    c8.kv = kv
    p8 = oracle_pool(c8)
    q0 = c.q.copy()
    q0[:, :, 512:] = 0
    r_fp8 = oracle.prefill(q0, p8, c.indices, topk_length=c.topk_length, sink=c.sink, sm_scale=c.sm_scale)
    for x, y in zip(r_nope, r_fp8):
        assert np.array_equal(x, y)
    # q columns past 512 do not matter
    r_full = oracle.prefill(c.q, pool, c.indices, topk_length=c.topk_length, sink=c.sink, sm_scale=c.sm_scale)
    for x, y in zip(r_nope, r_full):
        assert np.array_equal(x, y)
