"""Limits and degenerate cases of the many-head kernel, which serves FP8
rows (power-of-two or arbitrary scales) and INT8 rows for H > 16: head
counts just above 16 and at 128, the largest split count, a single
candidate, one token with a long list, empty lists, and decode workgroups
that run several consecutive splits.  Every result is compared with the
oracle's exact values (BF16 out: max_abs <= 1e-2, mean_abs <= 1e-3; LSE
1e-3; -inf positions of the split bookkeeping identical)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_mla_smla_amd as smla
from sparse_top_mla_smla_amd import workloads as W

from gpu_util import Dev, assert_lse_close, assert_out_close, bf16_dev_to_f64, need_gpu
from helpers import oracle_pool

pytestmark = pytest.mark.gpu

MANY_HEAD = [W.FMT_FP8, W.FMT_FP8_ANY, W.FMT_INT8]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def case(name, cid, **kw):
    base = dict(fmt=W.FMT_FP8, T=4, H=64, n_seqs=1, ctx=1024, topk=256, causal=True)
    base.update(kw)
    return W.make_case(name, config_id=cid, seed=1, **base)


def check_prefill(c):
    d = Dev(c)
    o, l = smla.prefill(d.q, d.pool, d.indices, topk_length=d.topk_length, sink=d.sink, sm_scale=float(c.sm_scale))
    torch.cuda.synchronize()
    _, lf32, of, _ = oracle.prefill(c.q, oracle_pool(c), c.indices, topk_length=c.topk_length, sink=c.sink,
                                    sm_scale=c.sm_scale)
    assert_out_close(bf16_dev_to_f64(o), of)
    assert_lse_close(l.cpu().numpy(), lf32)
    return o, l


def check_decode(c, S):
    d = Dev(c)
    po, pl = smla.decode(d.q, d.pool, d.indices, S, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
    o, l = smla.combine(po, pl, sink=d.sink)
    torch.cuda.synchronize()
    pool = oracle_pool(c)
    rpo, rpl = oracle.decode_split(c.q, pool, c.indices, S, topk_length=c.topk_length, sm_scale=c.sm_scale)
    gpl = pl.cpu().numpy()
    assert np.array_equal(np.isneginf(gpl), np.isneginf(rpl))
    assert_lse_close(gpl, rpl.astype(np.float32), "part_lse")
    assert_out_close(po.cpu().numpy().astype(np.float64), rpo, "part_out", bf16=False)
    _, lf32, of, _ = oracle.combine(rpo, rpl, sink=c.sink)
    assert_out_close(bf16_dev_to_f64(o), of)
    assert_lse_close(l.cpu().numpy(), lf32)


@pytest.mark.parametrize("fmt", MANY_HEAD)
@pytest.mark.parametrize("H", [17, 128])
def test_head_counts_prefill_and_decode(fmt, H):
    c = case(f"lim_h{H}_{fmt}", 400 + 10 * fmt + H % 7, fmt=fmt, H=H, topk=200, T=3, with_sink=True,
             with_topk_length=True)
    check_prefill(c)
    check_decode(c, 3)


@pytest.mark.parametrize("fmt", MANY_HEAD)
def test_sixty_four_splits(fmt):
    """The largest split count: 64 splits of one 64-entry tile each over a
    4096-entry list, with per-token lengths that leave trailing splits empty."""
    c = case(f"lim_s64_{fmt}", 430 + fmt, fmt=fmt, T=2, topk=4096, ctx=4096, with_topk_length=True)
    c.topk_length[0] = 4096
    c.topk_length[1] = 1000
    c.indices[1, 1000:] = -1
    check_decode(c, 64)


@pytest.mark.parametrize("fmt", MANY_HEAD)
def test_single_candidate(fmt):
    """A one-entry list: out is the candidate's value row, lse its score."""
    c = case(f"lim_k1_{fmt}", 440 + fmt, fmt=fmt, topk=1, T=5, with_sink=True)
    check_prefill(c)
    check_decode(c, 1)


def test_one_token_long_list():
    """One token, a 4096-entry list (64 tiles in one workgroup), prefill."""
    c = case("lim_t1_k4096", 450, T=1, topk=4096, ctx=4096, with_sink=True)
    check_prefill(c)


@pytest.mark.parametrize("fmt", MANY_HEAD)
def test_empty_lists_many_heads(fmt):
    """Tokens whose list is empty (length 0, or only -1 entries) get out = 0
    and lse = -inf; their neighbours are unaffected."""
    c = case(f"lim_empty_{fmt}", 460 + fmt, fmt=fmt, T=5, topk=192, with_topk_length=True, with_sink=True)
    c.topk_length[1] = 0
    c.indices[3, :] = -1
    o, l = check_prefill(c)
    assert torch.all(o[1] == 0) and torch.all(o[3] == 0)
    assert torch.all(torch.isneginf(l[1])) and torch.all(torch.isneginf(l[3]))
    check_decode(c, 2)


@pytest.mark.parametrize("fmt", MANY_HEAD)
def test_consecutive_splits_per_workgroup(fmt):
    """More (token, split) pairs than compute units: each decode workgroup
    runs three consecutive splits and carries its pipeline across them."""
    c = case(f"lim_grouped_{fmt}", 470 + fmt, fmt=fmt, T=96, topk=512, with_topk_length=True)
    assert 96 * 8 // 256 == 3
    check_decode(c, 8)
