"""Rows with exponent-byte scales on the GPU against the oracle:
DOTS3_SWA (1160-byte rows: 1024 e4m3 codes, 64 BF16 rope values, eight
exponent bytes; d_qk 1088, d_v 1024) and DSv4 (584-byte rows: 448 e4m3
codes, 64 BF16 rope values, seven exponent bytes and a pad byte; d_qk =
d_v = 512, so V's last 64 columns are the rope values).

Cases span several 64-entry tiles with ragged tails (the pages' 513-entry
DOTS3_SWA lists), head counts that are not multiples of the 16-head group,
strided q and out views, per-token lengths (including empty lists), sinks,
padded rows, and the split form with its combine at each value width.
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
D3, V4 = W.FMT_FP8_DOTS3, W.FMT_FP8_DSV4


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


CASES = {
    # name: make_case kwargs (config ids 500+ for DOTS3_SWA, 540+ for DSv4)
    "h16_w513_window_len_sink": dict(H=16, topk=513, ctx=1024, window=128, with_topk_length=True, with_sink=True),
    "h20_view_tailneg": dict(H=20, hbuf=32, topk=640, tail_neg=37, idx_ld=700, pad_fill=W.PAD_SENTINEL),
    "h64_w1024": dict(H=64, topk=1024, ctx=2048, T=3, with_sink=True),
    "h1_w100": dict(H=1, topk=100, causal=False),
    "h8_w513_len": dict(H=8, topk=513, ctx=768, T=7, with_topk_length=True),
    "h17_w300_sink": dict(H=17, topk=300, T=9, with_sink=True),
    "h128_w200_len": dict(H=128, topk=200, T=2, with_topk_length=True),
}
FMTS = [D3, V4]


def make(name, fmt=D3, **over):
    kw = dict(CASES[name])
    base = dict(fmt=fmt, T=5, n_seqs=1, ctx=1024, causal=True)
    base.update(kw)
    base.update(over)
    cid = (500 if fmt == D3 else 540) + sorted(CASES).index(name)
    return W.make_case(name, config_id=cid, seed=0, **base)


def reference(c):
    return oracle.prefill(c.q, oracle_pool(c), c.indices, topk_length=c.topk_length, sink=c.sink,
                          sm_scale=c.sm_scale)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_parity(name, fmt):
    c = make(name, fmt)
    d = Dev(c)
    out_buf = torch.full((c.T, c.H + 3, W.V_DIMS[fmt]), 7.0, dtype=torch.bfloat16, device="cuda")
    o, l = smla.prefill(d.q, d.pool, d.indices, topk_length=d.topk_length, sink=d.sink,
                        sm_scale=float(c.sm_scale), out=out_buf[:, :c.H])
    torch.cuda.synchronize()
    _, lf32, of, _ = reference(c)
    assert_out_close(bf16_dev_to_f64(o), of)
    assert_lse_close(l.cpu().numpy(), lf32)
    assert torch.all(out_buf[:, c.H:] == 7.0)          # heads beyond the view untouched


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", ["h16_w513_window_len_sink", "h20_view_tailneg", "h64_w1024"])
@pytest.mark.parametrize("S", [1, 3, 9])
def test_decode_split_and_combine_parity(name, S, fmt):
    c = make(name, fmt)
    d = Dev(c)
    po, pl = smla.decode(d.q, d.pool, d.indices, S, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
    assert po.shape == (c.T, S, c.H, W.V_DIMS[fmt])
    o, l = smla.combine(po, pl, sink=d.sink)
    torch.cuda.synchronize()
    pool = oracle_pool(c)
    rpo, rpl = oracle.decode_split(c.q, pool, c.indices, S, topk_length=c.topk_length, sm_scale=c.sm_scale)
    gpl = pl.cpu().numpy()
    assert np.array_equal(np.isneginf(gpl), np.isneginf(rpl))
    assert_lse_close(gpl, rpl.astype(np.float32), "part_lse")
    gpo = po.cpu().numpy().astype(np.float64)
    assert np.all(gpo[np.isneginf(gpl)] == 0)
    assert_out_close(gpo, rpo, "part_out", bf16=False)
    _, lf32, of, _ = oracle.combine(rpo, rpl, sink=c.sink)
    assert_out_close(bf16_dev_to_f64(o), of)
    assert_lse_close(l.cpu().numpy(), lf32)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("H", [8, 40])
def test_empty_lists(fmt, H):
    c = make("h8_w513_len", fmt, H=H)
    L = c.topk_length.copy()
    L[0], L[3], L[5] = 0, -2, 1
    c.topk_length = L
    d = Dev(c)
    o, l = smla.prefill(d.q, d.pool, d.indices, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
    torch.cuda.synchronize()
    _, lf32, of, _ = reference(c)
    got_l = l.cpu().numpy()
    assert np.all(np.isneginf(got_l[[0, 3]])) and torch.all(o[[0, 3]] == 0)
    assert_out_close(bf16_dev_to_f64(o), of)
    assert_lse_close(got_l, lf32)


@pytest.mark.parametrize("fmt", FMTS)
def test_padded_rows_and_blocks(fmt):
    """Packed rows are 8-byte aligned; padded ones (8 bytes more) and padded
    blocks give each row the oracle's packed bytes, leave the padding
    unwritten, and give bit-identical attention."""
    c = make("h20_view_tailneg", fmt)
    rb = W.ROW_BYTES[fmt]
    rs = rb + 8
    bs = 64 * rs + 40
    d = Dev(c, block_stride=bs, fill=0xC3, row_stride=rs)
    torch.cuda.synchronize()
    got = d.pool.data.cpu().numpy()
    ref = oracle_pool(c).data
    for blk in range(c.num_blocks):
        for r in range(64):
            assert np.array_equal(got[blk, r * rs:r * rs + rb], ref[blk, r * rb:(r + 1) * rb])
            assert (got[blk, r * rs + rb:(r + 1) * rs] == 0xC3).all()
        assert (got[blk, 64 * rs:] == 0xC3).all()
    dp = Dev(c)
    assert np.array_equal(dp.pool.data.cpu().numpy(), ref)
    a = smla.prefill(d.q, d.pool, d.indices, sm_scale=float(c.sm_scale))
    b = smla.prefill(dp.q, dp.pool, dp.indices, sm_scale=float(c.sm_scale))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    x = smla.decode(d.q, d.pool, d.indices, 3, sm_scale=float(c.sm_scale))
    y = smla.decode(dp.q, dp.pool, dp.indices, 3, sm_scale=float(c.sm_scale))
    assert torch.equal(x[0], y[0]) and torch.equal(x[1], y[1])
