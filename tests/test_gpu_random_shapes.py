"""Seeded random shapes on the GPU against the oracle.

One fixed generator draws 70 cases, ten per row format (BF16, FP8, INT8,
FP8 with arbitrary scales, rope-less FP8, DOTS3_SWA, DSv4), each with:
- a head count on either side of every kernel's head group (1 to 128);
- a list width from 1 to 1100 entries (ragged tails, one to eighteen tiles);
- 1 to 6 tokens, causal or whole-context candidates, sometimes a window of
  recent positions or trailing -1 entries;
- sometimes per-token lengths (one token's list then made empty) and a sink.

Every case runs the prefill form and the split form at a drawn split count
with its combine; both are compared with the oracle.  A second set of 28
draws does the same for dual-cache calls (a main list and a secondary list
over two pools, one softmax over both).  The shape is in the
test id, so a failure names its case.  Outputs are held to the problem
statement's bar against the oracle's exact (unrounded) values.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_top_mla_smla_amd as smla
from sparse_top_mla_smla_amd import workloads as W

from gpu_util import Dev, assert_lse_close, assert_out_close, bf16_dev_to_f64, need_gpu
from helpers import oracle_pool

pytestmark = pytest.mark.gpu

FMTS = [W.FMT_BF16, W.FMT_FP8, W.FMT_INT8, W.FMT_FP8_ANY, W.FMT_FP8_NOPE, W.FMT_FP8_DOTS3, W.FMT_FP8_DSV4]
HEADS = [1, 3, 8, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 96, 127, 128]
PER_FMT = 10


def _draw():
    rng = np.random.default_rng(20261202)
    cases = []
    for i in range(PER_FMT * len(FMTS)):
        fmt = FMTS[i % len(FMTS)]
        topk = int(rng.integers(1, 1101))
        kw = dict(fmt=fmt, H=int(rng.choice(HEADS)), topk=topk, T=int(rng.integers(1, 7)), n_seqs=1,
                  ctx=2048, causal=bool(rng.random() < 0.6),
                  with_topk_length=bool(rng.random() < 0.5), with_sink=bool(rng.random() < 0.5))
        if kw["causal"] and topk > 160 and rng.random() < 0.3:
            kw["window"] = 128
        elif topk > 8 and rng.random() < 0.2:
            kw["tail_neg"] = int(rng.integers(1, min(topk, 70)))
        kw["S"] = int(rng.integers(1, min(16, math.ceil(topk / 64)) + 1))
        name = (f"{i:02d}_fmt{fmt}_h{kw['H']}_k{topk}_t{kw['T']}_s{kw['S']}"
                + ("_len" if kw["with_topk_length"] else "") + ("_sink" if kw["with_sink"] else "")
                + ("_win" if "window" in kw else "") + ("_neg" if "tail_neg" in kw else "")
                + ("" if kw["causal"] else "_all"))
        cases.append((name, i, kw))
    return cases


CASES = _draw()


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def make(i, kw):
    kw = dict(kw)
    kw.pop("S")
    c = W.make_case(f"random_{i}", config_id=700 + i, seed=3, **kw)
    if c.topk_length is not None and c.T > 1:
        L = c.topk_length.copy()
        L[i % c.T] = 0  # one empty list per case with lengths
        c.topk_length = L
    return c


@pytest.mark.parametrize("name,i,kw", CASES, ids=[n for n, _, _ in CASES])
def test_random_shape(name, i, kw):
    c = make(i, kw)
    S = kw["S"]
    d = Dev(c)
    o, l = smla.prefill(d.q, d.pool, d.indices, topk_length=d.topk_length, sink=d.sink,
                        sm_scale=float(c.sm_scale))
    po, pl = smla.decode(d.q, d.pool, d.indices, S, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
    o2, l2 = smla.combine(po, pl, sink=d.sink)
    torch.cuda.synchronize()
    pool = oracle_pool(c)
    _, lf32, of, _ = oracle.prefill(c.q, pool, c.indices, topk_length=c.topk_length, sink=c.sink,
                                    sm_scale=c.sm_scale)
    want = of
    assert_out_close(bf16_dev_to_f64(o), want)
    assert_lse_close(l.cpu().numpy(), lf32)
    rpo, rpl = oracle.decode_split(c.q, pool, c.indices, S, topk_length=c.topk_length, sm_scale=c.sm_scale)
    gpl = pl.cpu().numpy()
    assert np.array_equal(np.isneginf(gpl), np.isneginf(rpl)), "empty splits differ"
    assert_lse_close(gpl, rpl.astype(np.float32), "part_lse")
    gpo = po.cpu().numpy().astype(np.float64)
    assert np.all(gpo[np.isneginf(gpl)] == 0), "an empty split's partial is not zero"
    assert_out_close(gpo, rpo, "part_out", bf16=False)
    assert_out_close(bf16_dev_to_f64(o2), want, "combined out")
    assert_lse_close(l2.cpu().numpy(), lf32, "combined lse")


def _draw_dual():
    """Dual-cache calls: a main list of 64 to 768 entries (a multiple of 64)
    and a secondary list of 1 to 1500 entries over its own pool with padded
    rows, four cases per row format."""
    rng = np.random.default_rng(20261203)
    cases = []
    for i in range(4 * len(FMTS)):
        fmt = FMTS[i % len(FMTS)]
        k1 = 64 * int(rng.integers(1, 13))
        k2 = int(rng.integers(1, 1501))
        kw = dict(fmt=fmt, H=int(rng.choice(HEADS)), k1=k1, k2=k2, T=int(rng.integers(1, 6)),
                  lengths=bool(rng.random() < 0.6), sink=bool(rng.random() < 0.5))
        kw["S"] = int(rng.integers(1, min(16, math.ceil((k1 + k2) / 64)) + 1))
        name = (f"{i:02d}_fmt{fmt}_h{kw['H']}_k{k1}+{k2}_t{kw['T']}_s{kw['S']}"
                + ("_len" if kw["lengths"] else "") + ("_sink" if kw["sink"] else ""))
        cases.append((name, i, kw))
    return cases


DUAL_CASES = _draw_dual()


@pytest.mark.parametrize("name,i,kw", DUAL_CASES, ids=[n for n, _, _ in DUAL_CASES])
def test_random_dual_shape(name, i, kw):
    from test_gpu_dual import dual_args, reference

    fmt, H, T = kw["fmt"], kw["H"], kw["T"]
    main = W.make_case(f"random_dual_{i}_main", config_id=800 + 2 * i, seed=4, fmt=fmt, T=T, H=H, n_seqs=1,
                       ctx=max(1024, 2 * kw["k1"]), topk=kw["k1"], causal=True,
                       with_topk_length=kw["lengths"], with_sink=kw["sink"])
    extra = W.make_case(f"random_dual_{i}_extra", config_id=801 + 2 * i, seed=4, fmt=fmt, T=T, H=H, n_seqs=1,
                        ctx=64 * math.ceil(max(512, 2 * kw["k2"]) / 64), topk=kw["k2"], causal=False,
                        with_topk_length=kw["lengths"])
    if kw["lengths"] and T > 1:  # one token with an empty main list, another with an empty secondary list
        L1, L2 = main.topk_length.copy(), extra.topk_length.copy()
        L1[i % T] = 0
        L2[(i + 1) % T] = 0
        main.topk_length, extra.topk_length = L1, L2
    dm, de = Dev(main), Dev(extra, row_stride=(W.ROW_BYTES[fmt] + 31) // 16 * 16)
    o, l = smla.prefill_dual(dm.q, dm.pool, dm.indices, sink=dm.sink, **dual_args(dm, de))
    po, pl = smla.decode_dual(dm.q, dm.pool, dm.indices, num_splits=kw["S"], **dual_args(dm, de))
    o2, l2 = smla.combine(po, pl, sink=dm.sink)
    torch.cuda.synchronize()
    _, lf32, of, _ = reference(main, extra)
    want = of
    assert_out_close(bf16_dev_to_f64(o), want)
    assert_lse_close(l.cpu().numpy(), lf32)
    rpo, rpl = reference(main, extra, num_splits=kw["S"])
    gpl = pl.cpu().numpy()
    assert np.array_equal(np.isneginf(gpl), np.isneginf(rpl)), "empty splits differ"
    assert_lse_close(gpl, rpl.astype(np.float32), "part_lse")
    assert_out_close(po.cpu().numpy().astype(np.float64), rpo, "part_out", bf16=False)
    assert_out_close(bf16_dev_to_f64(o2), want, "combined out")
    assert_lse_close(l2.cpu().numpy(), lf32, "combined lse")
