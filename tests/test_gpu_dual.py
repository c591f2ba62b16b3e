"""Dual-cache calls on the GPU: one softmax over a main list and a
secondary list, each over its own pool and cut at its own length.

The oracle has no second source; the reference is its single-list attention
over the two packed pools laid end to end, with the secondary slots moved
past the main pool's and every entry that is beyond its list's length or
not a slot of its own pool replaced by -1 (which contributes nothing).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_mla_smla_amd as smla
from sparse_top_mla_smla_amd import workloads as W

from gpu_util import Dev, assert_lse_close, assert_out_close, bf16_dev_to_f64, need_gpu
from helpers import oracle_pool

pytestmark = pytest.mark.gpu

CASES = {
    # name: (format, H, main topk, secondary topk, lengths, sink)
    "fp8_h64": (W.FMT_FP8, 64, 128, 192, True, True),
    "fp8_h64_w1024_2176": (W.FMT_FP8, 64, 1024, 2176, False, False),
    "int8_h64": (W.FMT_INT8, 64, 64, 130, True, True),
    "fp8_h8": (W.FMT_FP8, 8, 192, 70, True, False),
    "bf16_h16": (W.FMT_BF16, 16, 64, 100, True, True),
    # rows with exponent-byte scales: DSv4 (the page's dual-cache model) and DOTS3_SWA
    "dsv4_h64": (W.FMT_FP8_DSV4, 64, 128, 192, True, True),
    "dsv4_h20_w1024_2176": (W.FMT_FP8_DSV4, 20, 1024, 2176, False, False),
    "dots3_h16": (W.FMT_FP8_DOTS3, 16, 192, 130, True, True),
    "dots3_h40": (W.FMT_FP8_DOTS3, 40, 128, 200, True, True),
}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def make(name):
    fmt, H, k1, k2, lengths, sink = CASES[name]
    T = 2 if k2 > 1000 else 5
    cid = 400 + 2 * sorted(CASES).index(name)
    main = W.make_case(name + "_main", config_id=cid, seed=5, fmt=fmt, T=T, H=H, n_seqs=1,
                       ctx=max(1024, 2 * k1), topk=k1, causal=True, with_topk_length=lengths, with_sink=sink)
    extra = W.make_case(name + "_extra", config_id=cid + 1, seed=6, fmt=fmt, T=T, H=H, n_seqs=1,
                        ctx=max(512, 2 * k2), topk=k2, causal=False, with_topk_length=lengths)
    if lengths:  # some empty lists on either side, and one token with neither
        L1, L2 = main.topk_length.copy(), extra.topk_length.copy()
        L1[1] = 0
        L2[2] = -4
        L1[3], L2[3] = 0, 0
        main.topk_length, extra.topk_length = L1, L2
    return main, extra


def reference(main, extra, num_splits=0):
    p1, p2 = oracle_pool(main), oracle_pool(extra)
    assert p1.block_stride == p2.block_stride
    pool = oracle.Pool(np.concatenate([p1.data, p2.data]), main.fmt, p1.block_stride)
    n1, n2 = main.num_blocks * 64, extra.num_blocks * 64

    def part(case, n, shift):
        idx = case.indices.astype(np.int64)
        keep = (idx >= 0) & (idx < n)
        if case.topk_length is not None:
            L = np.clip(case.topk_length, 0, case.topk)
            keep &= np.arange(case.topk)[None, :] < L[:, None]
        return np.where(keep, idx + shift, -1).astype(np.int32)

    idx = np.ascontiguousarray(np.concatenate([part(main, n1, 0), part(extra, n2, n1)], axis=1))
    if num_splits:
        return oracle.decode_split(main.q, pool, idx, num_splits, sm_scale=main.sm_scale)
    return oracle.prefill(main.q, pool, idx, sink=main.sink, sm_scale=main.sm_scale)


def dual_args(dm, de):
    return dict(extra_pool=de.pool, extra_indices=de.indices, topk_length=dm.topk_length,
                extra_topk_length=de.topk_length, sm_scale=float(dm.case.sm_scale))


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_dual_parity(name):
    main, extra = make(name)
    dm, de = Dev(main), Dev(extra, row_stride=(W.ROW_BYTES[extra.fmt] + 31) // 16 * 16)  # padded secondary rows
    o, l = smla.prefill_dual(dm.q, dm.pool, dm.indices, sink=dm.sink, **dual_args(dm, de))
    torch.cuda.synchronize()
    _, lf32, of, _ = reference(main, extra)
    got_l = l.cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(lf32))
    assert_out_close(bf16_dev_to_f64(o), of)
    assert_lse_close(got_l, lf32)


@pytest.mark.parametrize("name", ["fp8_h64", "int8_h64", "fp8_h8", "bf16_h16", "dsv4_h64", "dots3_h16", "dots3_h40"])
@pytest.mark.parametrize("S", [1, 3, 5])
def test_decode_dual_parity(name, S):
    main, extra = make(name)
    dm, de = Dev(main), Dev(extra)
    po, pl = smla.decode_dual(dm.q, dm.pool, dm.indices, num_splits=S, **dual_args(dm, de))
    o, l = smla.combine(po, pl, sink=dm.sink)
    torch.cuda.synchronize()
    rpo, rpl = reference(main, extra, num_splits=S)
    gpl = pl.cpu().numpy()
    assert np.array_equal(np.isneginf(gpl), np.isneginf(rpl))
    assert_lse_close(gpl, rpl.astype(np.float32), "part_lse")
    assert_out_close(po.cpu().numpy().astype(np.float64), rpo, "part_out", bf16=False)
    _, lf32, of, _ = reference(main, extra)
    assert_out_close(bf16_dev_to_f64(o), of)
    assert_lse_close(l.cpu().numpy(), lf32)


@pytest.mark.parametrize("name", ["fp8_h64", "int8_h64", "fp8_h8", "bf16_h16", "dsv4_h64", "dots3_h16"])
def test_empty_secondary_list_is_the_single_list_call(name):
    """A secondary list cut to length 0 everywhere leaves exactly the
    single-list result, bit for bit."""
    main, extra = make(name)
    dm, de = Dev(main), Dev(extra)
    zero = torch.zeros(main.T, dtype=torch.int32, device="cuda")
    a = smla.prefill_dual(dm.q, dm.pool, dm.indices, extra_pool=de.pool, extra_indices=de.indices,
                          topk_length=dm.topk_length, extra_topk_length=zero, sink=dm.sink,
                          sm_scale=float(main.sm_scale))
    b = smla.prefill(dm.q, dm.pool, dm.indices, topk_length=dm.topk_length, sink=dm.sink,
                     sm_scale=float(main.sm_scale))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("name", ["fp8_h64", "int8_h64", "fp8_h8", "bf16_h16", "dsv4_h64", "dots3_h16"])
def test_empty_main_list_is_the_secondary_list_alone(name):
    """A main list cut to length 0 everywhere leaves the secondary list's
    single-list result, bit for bit (the main list's width is a multiple of
    64, so the secondary list's tiles hold the same candidates)."""
    main, extra = make(name)
    dm, de = Dev(main), Dev(extra)
    zero = torch.zeros(main.T, dtype=torch.int32, device="cuda")
    a = smla.prefill_dual(dm.q, dm.pool, dm.indices, extra_pool=de.pool, extra_indices=de.indices,
                          topk_length=zero, extra_topk_length=de.topk_length, sink=dm.sink,
                          sm_scale=float(main.sm_scale))
    b = smla.prefill(dm.q, de.pool, de.indices, topk_length=de.topk_length, sink=dm.sink,
                     sm_scale=float(main.sm_scale))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("fmt,H", [(W.FMT_INT8, 8), (W.FMT_FP8_ANY, 16), (W.FMT_FP8_NOPE, 8)])
def test_few_head_dual_formats(fmt, H):
    """Dual-list prefill and decode with 16 or fewer heads over INT8,
    arbitrary-scale FP8 and rope-less FP8 rows (the column-split kernel's
    dual instantiations), with lengths, empty lists and padded secondary
    rows."""
    cid = 480 + 2 * fmt
    main = W.make_case(f"dual_few_{fmt}_main", config_id=cid, seed=5, fmt=fmt, T=5, H=H, n_seqs=1, ctx=1024,
                       topk=192, causal=True, with_topk_length=True, with_sink=True)
    extra = W.make_case(f"dual_few_{fmt}_extra", config_id=cid + 1, seed=6, fmt=fmt, T=5, H=H, n_seqs=1, ctx=512,
                        topk=130, causal=False, with_topk_length=True)
    L1, L2 = main.topk_length.copy(), extra.topk_length.copy()
    L1[1] = 0
    L1[3], L2[3] = 0, 0
    main.topk_length, extra.topk_length = L1, L2
    dm, de = Dev(main), Dev(extra, row_stride=(W.ROW_BYTES[extra.fmt] + 31) // 16 * 16)
    o, l = smla.prefill_dual(dm.q, dm.pool, dm.indices, sink=dm.sink, **dual_args(dm, de))
    torch.cuda.synchronize()
    _, lf32, of, _ = reference(main, extra)
    assert np.array_equal(np.isneginf(l.cpu().numpy()), np.isneginf(lf32))
    assert_out_close(bf16_dev_to_f64(o), of)
    assert_lse_close(l.cpu().numpy(), lf32)
    po, pl = smla.decode_dual(dm.q, dm.pool, dm.indices, num_splits=3, **dual_args(dm, de))
    o2, l2 = smla.combine(po, pl, sink=dm.sink)
    torch.cuda.synchronize()
    rpo, rpl = reference(main, extra, num_splits=3)
    assert np.array_equal(np.isneginf(pl.cpu().numpy()), np.isneginf(rpl))
    assert_out_close(po.cpu().numpy().astype(np.float64), rpo, "part_out", bf16=False)
    assert_out_close(bf16_dev_to_f64(o2), of)
    assert_lse_close(l2.cpu().numpy(), lf32)
