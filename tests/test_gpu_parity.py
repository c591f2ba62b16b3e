"""GPU parity of the HIP path against the oracle (small and medium sizes).

Every case is seeded and synthetic (sparse_top_mla_smla_amd.workloads); the
oracle computes from the generator's latent rows with its own quantizer, so
no oracle input comes from the GPU.  Cache bytes and split bookkeeping are
compared bit for bit; outputs within max_abs 1e-2 / mean_abs 1e-3 (BF16 out)
and 1e-3 (LSE), with -inf positions identical.
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


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


CASES = {
    # name: make_case kwargs (config ids 200+ are test-only)
    "bf16_h8_ragged": dict(fmt=W.FMT_BF16, H=8, topk=200),
    "fp8_h8_ragged": dict(fmt=W.FMT_FP8, H=8, topk=200),
    "int8_h8_ragged": dict(fmt=W.FMT_INT8, H=8, topk=200),
    "fp8_h1": dict(fmt=W.FMT_FP8, H=1, topk=70),
    "bf16_h16_sink_len": dict(fmt=W.FMT_BF16, H=16, topk=256, with_sink=True, with_topk_length=True),
    "fp8_h20_sink": dict(fmt=W.FMT_FP8, H=20, topk=130, with_sink=True),
    "int8_h64_len": dict(fmt=W.FMT_INT8, H=64, topk=192, with_topk_length=True, T=3),
    "fp8_h64_multi_tile": dict(fmt=W.FMT_FP8, H=64, topk=1024, ctx=2048, T=4, with_sink=True),
    "bf16_h8_window_len_sink": dict(fmt=W.FMT_BF16, H=8, hbuf=64, topk=640, ctx=2048, T=6, window=128,
                                    with_topk_length=True, with_sink=True, out_hbuf=64),
    "int8_h128_view": dict(fmt=W.FMT_INT8, H=128, topk=256, idx_ld=384, T=2, with_sink=True,
                           pad_fill=W.PAD_SENTINEL),
    "fp8_tail_neg": dict(fmt=W.FMT_FP8, H=16, topk=64, tail_neg=9, causal=False, T=4),
    # FP8 codes with arbitrary scales (GLM_NSA rows): the column-split
    # kernel (few heads) and the many-head kernel, both scaling partial
    # scores and P
    "fp8any_h8_len_sink": dict(fmt=W.FMT_FP8_ANY, H=8, topk=200, with_topk_length=True, with_sink=True),
    "fp8any_h64_multi_tile": dict(fmt=W.FMT_FP8_ANY, H=64, topk=1024, ctx=2048, T=3, with_sink=True),
    "fp8any_h100_len": dict(fmt=W.FMT_FP8_ANY, H=100, topk=192, T=3, with_topk_length=True),
}


def make(name):
    kw = dict(CASES[name])
    base = dict(fmt=W.FMT_FP8, T=5, H=8, n_seqs=1, ctx=512, topk=200, causal=True)
    base.update(kw)
    cid = 200 + sorted(CASES).index(name)
    return W.make_case(name, config_id=cid, seed=0, **base)


def run_prefill(d: Dev, out_hbuf: int = 0):
    c = d.case
    if out_hbuf:
        out_buf = torch.full((c.T, out_hbuf, 512), 7.0, dtype=torch.bfloat16, device="cuda")
        out = out_buf[:, : c.H]
    else:
        out_buf = out = None
    o, l = smla.prefill(d.q, d.pool, d.indices, topk_length=d.topk_length, sink=d.sink,
                        sm_scale=float(c.sm_scale), out=out)
    torch.cuda.synchronize()
    return o, l, out_buf


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_parity(name):
    c = make(name)
    d = Dev(c)
    o, l, out_buf = run_prefill(d, c.out_hbuf)
    pool = oracle_pool(c)
    _, lf32, of, _ = oracle.prefill(c.q, pool, c.indices, topk_length=c.topk_length, sink=c.sink,
                                    sm_scale=c.sm_scale)
    assert_out_close(bf16_dev_to_f64(o), of)
    assert_lse_close(l.cpu().numpy(), lf32)
    if out_buf is not None:  # heads beyond the view are untouched
        assert torch.all(out_buf[:, c.H:] == 7.0)


@pytest.mark.parametrize("name", ["bf16_h8_ragged", "fp8_h20_sink", "int8_h64_len", "fp8_h64_multi_tile",
                                  "bf16_h8_window_len_sink", "fp8any_h8_len_sink", "fp8any_h64_multi_tile"])
@pytest.mark.parametrize("S", [1, 3, 8])
def test_decode_split_and_combine_parity(name, S):
    c = make(name)
    d = Dev(c)
    po, pl = smla.decode(d.q, d.pool, d.indices, S, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
    o, l = smla.combine(po, pl, sink=d.sink)
    torch.cuda.synchronize()
    pool = oracle_pool(c)
    rpo, rpl = oracle.decode_split(c.q, pool, c.indices, S, topk_length=c.topk_length, sm_scale=c.sm_scale)
    gpl = pl.cpu().numpy()
    # split bookkeeping: empty splits are exactly the oracle's
    assert np.array_equal(np.isneginf(gpl), np.isneginf(rpl))
    assert_lse_close(gpl, rpl.astype(np.float32), "part_lse")
    gpo = po.cpu().numpy().astype(np.float64)
    assert np.all(gpo[np.isneginf(gpl)] == 0)
    assert_out_close(gpo, rpo, "part_out", bf16=False)
    _, lf32, of, _ = oracle.combine(rpo, rpl, sink=c.sink)
    assert_out_close(bf16_dev_to_f64(o), of)
    assert_lse_close(l.cpu().numpy(), lf32)


@pytest.mark.parametrize("S", [1, 2, 5, 64])
def test_combine_alone(S):
    # oracle partials in, GPU merge out
    rng = np.random.default_rng(S)
    T, H = 3, 24
    po = rng.standard_normal((T, S, H, 512))
    pl = rng.standard_normal((T, S, H)) * 3
    pl[rng.random((T, S, H)) < 0.3] = -np.inf
    pl[1, :, 5] = -np.inf
    sink = rng.standard_normal(H).astype(np.float32)
    po32, pl32 = po.astype(np.float32), pl.astype(np.float32)
    o, l = smla.combine(torch.from_numpy(po32).cuda(), torch.from_numpy(pl32).cuda(),
                        sink=torch.from_numpy(sink).cuda())
    _, lf32, of, _ = oracle.combine(po32.astype(np.float64), pl32.astype(np.float64), sink=sink)
    assert_out_close(bf16_dev_to_f64(o), of)
    assert_lse_close(l.cpu().numpy(), lf32)
    assert torch.all(o[1, 5] == 0)


def test_c1_tiny_all_forms():
    c = W.c1_tiny()
    d = Dev(c)
    pool = oracle_pool(c)
    o, l, _ = run_prefill(d)
    _, lf32, of, _ = oracle.prefill(c.q, pool, c.indices, sm_scale=c.sm_scale)
    assert_out_close(bf16_dev_to_f64(o), of)
    assert_lse_close(l.cpu().numpy(), lf32)
    for S in (1, 2, 4):
        po, pl = smla.decode(d.q, d.pool, d.indices, S, sm_scale=float(c.sm_scale))
        o2, l2 = smla.combine(po, pl)
        assert_out_close(bf16_dev_to_f64(o2), of)
        assert_lse_close(l2.cpu().numpy(), lf32)


@pytest.mark.parametrize("fmt", [W.FMT_BF16, W.FMT_FP8, W.FMT_INT8, W.FMT_FP8_ANY, W.FMT_FP8_NOPE,
                                 W.FMT_FP8_DOTS3, W.FMT_FP8_DSV4])
def test_quantize_bit_exact(fmt):
    c = W.make_case("quant", config_id=230 + fmt, seed=1, fmt=fmt, T=1, H=1, n_seqs=1, ctx=2048, topk=64)
    kv = c.kv.copy()
    # adversarial tiles: zero, negative zero, tiny, huge, exact e4m3 midpoints
    kv[0, :128] = 0
    kv[1, 128:256] = 0x8000
    kv[2, :128] = W.f32_to_bf16_bits(np.float32(1e-38) * np.arange(128, dtype=np.float32))
    kv[3, 256:384] = W.f32_to_bf16_bits(np.float32(1e30) * np.linspace(-1, 1, 128, dtype=np.float32))
    mids = np.array([oracle.e4m3_decode(k) for k in range(0x7E)])
    mids = ((mids[:-1] + mids[1:]) / 2).astype(np.float32)
    tie_tile = np.concatenate([[448.0], mids, mids[:2]]).astype(np.float32)   # 128 values
    kv[4, :128] = W.f32_to_bf16_bits(tie_tile * np.float32(0.25))
    kv[5, 384:512] = W.f32_to_bf16_bits(-tie_tile)
    kv[6, :128] = W.f32_to_bf16_bits(np.float32(3e-39) * np.ones(128, np.float32))
    c.kv = kv
    slots = c.slots.copy()
    slots[7] = -1                         # skipped
    slots[8] = 2 ** 31 - 1                # out of range: skipped
    c.slots = slots
    d = Dev(c, fill=0xAB)
    torch.cuda.synchronize()
    ref = oracle.Pool(np.full((c.num_blocks, 64 * W.ROW_BYTES[fmt]), 0xAB, np.uint8), fmt,
                      64 * W.ROW_BYTES[fmt])
    oracle.quantize_kv(c.kv, c.slots, ref)
    got = d.pool.data.cpu().numpy()
    assert np.array_equal(got, ref.data)


def test_quantize_padded_block_stride():
    c = make("fp8_h8_ragged")
    bs = 64 * 656 + 144
    d = Dev(c, block_stride=bs, fill=0x5A)
    torch.cuda.synchronize()
    ref = oracle_pool(c, block_stride=bs, fill=0x5A)
    assert np.array_equal(d.pool.data.cpu().numpy(), ref.data)
    # attention over the padded pool equals attention over the packed pool, bit for bit
    d2 = Dev(c)
    a = smla.prefill(d.q, d.pool, d.indices, sm_scale=float(c.sm_scale))
    b = smla.prefill(d2.q, d2.pool, d2.indices, sm_scale=float(c.sm_scale))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("name", ["fp8_h8_ragged", "bf16_h16_sink_len", "int8_h64_len", "fp8_h64_multi_tile",
                                  "int8_h128_view"])
def test_padded_rows(name):
    """Rows padded beyond the format's bytes (and blocks beyond 64 rows):
    each row's bytes equal the oracle's packed row, the padding is never
    written, and prefill and decode over the padded pool equal those over
    the packed pool bit for bit."""
    c = make(name)
    rb = W.ROW_BYTES[c.fmt]
    rs = rb + 48
    bs = 64 * rs + 80
    d = Dev(c, block_stride=bs, fill=0xC3, row_stride=rs)
    torch.cuda.synchronize()
    got = d.pool.data.cpu().numpy()
    ref = oracle_pool(c).data  # packed rows
    for blk in range(c.num_blocks):
        for r in range(64):
            assert np.array_equal(got[blk, r * rs:r * rs + rb], ref[blk, r * rb:(r + 1) * rb])
            assert (got[blk, r * rs + rb:(r + 1) * rs] == 0xC3).all()
        assert (got[blk, 64 * rs:] == 0xC3).all()
    dp = Dev(c)
    a = smla.prefill(d.q, d.pool, d.indices, topk_length=d.topk_length, sink=d.sink, sm_scale=float(c.sm_scale))
    b = smla.prefill(dp.q, dp.pool, dp.indices, topk_length=dp.topk_length, sink=dp.sink,
                     sm_scale=float(c.sm_scale))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for S in (1, 3):
        x = smla.decode(d.q, d.pool, d.indices, S, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
        y = smla.decode(dp.q, dp.pool, dp.indices, S, topk_length=dp.topk_length, sm_scale=float(c.sm_scale))
        assert torch.equal(x[0], y[0]) and torch.equal(x[1], y[1])


@pytest.mark.parametrize("H,T", [(64, 600), (128, 300)])
def test_prefill_many_tokens_per_workgroup(H, T):
    """More tokens than compute units: each workgroup of the many-head FP8
    kernel runs several tokens in a row, with empty (0 or negative), clamped
    and short lists among them."""
    c = W.make_case(f"fp8_persist_h{H}", config_id=290 + H // 64, seed=3, fmt=W.FMT_FP8, T=T, H=H, n_seqs=1,
                    ctx=1024, topk=96, causal=True, with_topk_length=True, with_sink=True)
    L = c.topk_length.copy()
    L[::7] = 0
    L[3::11] = -3
    L[5::13] = c.topk + 50
    c.topk_length = L
    d = Dev(c)
    o, l = smla.prefill(d.q, d.pool, d.indices, topk_length=d.topk_length, sink=d.sink, sm_scale=float(c.sm_scale))
    torch.cuda.synchronize()
    _, lf32, of64, _ = oracle.prefill(c.q, oracle_pool(c), c.indices, topk_length=c.topk_length, sink=c.sink,
                                      sm_scale=c.sm_scale)
    got_l = l.cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(lf32))
    assert np.isneginf(lf32[L <= 0]).all() and (L <= 0).sum() > 0
    assert_out_close(bf16_dev_to_f64(o), of64)
    assert_lse_close(got_l, lf32)


@pytest.mark.parametrize("H", [8, 64])
def test_nope_rows(H):
    """GLM53_NOPE rows: q rows of 512 values (a compact tensor, so a read
    past 512 would take the next head's values) and row padding filled with
    NaN bytes (a read of it would poison the result); prefill and decode
    match the oracle."""
    c = W.make_case(f"nope_h{H}", config_id=295 + H // 64, seed=4, fmt=W.FMT_FP8_NOPE, T=4, H=H, n_seqs=1,
                    ctx=1024, topk=320, causal=True, with_topk_length=True, with_sink=True)
    d = Dev(c, fill=0xFF)
    q512 = torch.from_numpy(np.ascontiguousarray(c.q[:, :, :512]).view(np.int16)).view(torch.bfloat16).cuda()
    assert q512.stride(1) == 512
    o, l = smla.prefill(q512, d.pool, d.indices, topk_length=d.topk_length, sink=d.sink, sm_scale=float(c.sm_scale))
    torch.cuda.synchronize()
    pool = oracle_pool(c)
    _, lf32, of, _ = oracle.prefill(c.q, pool, c.indices, topk_length=c.topk_length, sink=c.sink,
                                    sm_scale=c.sm_scale)
    assert_out_close(bf16_dev_to_f64(o), of)
    assert_lse_close(l.cpu().numpy(), lf32)
    po, pl = smla.decode(q512, d.pool, d.indices, 3, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
    o2, l2 = smla.combine(po, pl, sink=d.sink)
    torch.cuda.synchronize()
    rpo, rpl = oracle.decode_split(c.q, pool, c.indices, 3, topk_length=c.topk_length, sm_scale=c.sm_scale)
    assert_out_close(po.cpu().numpy().astype(np.float64), rpo, "part_out", bf16=False)
    assert_out_close(bf16_dev_to_f64(o2), of)
    assert_lse_close(l2.cpu().numpy(), lf32)


@pytest.mark.parametrize("H", [8, 64])
def test_tiny_amax_tiles(H):
    """Tiles whose amax/448 lies below the least normal float32 are stored
    with the scale 2^-126 (a normal power of two, as the attention kernels
    require).  Every row here carries such a tile; prefill and the split
    decode over them match the oracle with finite outputs."""
    c = W.make_case(f"tiny_amax_h{H}", config_id=297 + H // 64, seed=5, fmt=W.FMT_FP8, T=3, H=H, n_seqs=1,
                    ctx=512, topk=192, causal=True, with_sink=True)
    kv = c.kv.copy()
    kv[:, 128:256] = W.f32_to_bf16_bits(np.float32(1e-38) * np.arange(128, dtype=np.float32))
    kv[::3, 384:512] = W.f32_to_bf16_bits(np.float32(3e-39) * np.ones(128, np.float32))
    c.kv = kv
    d = Dev(c)
    pool = oracle_pool(c)
    torch.cuda.synchronize()
    assert np.array_equal(d.pool.data.cpu().numpy(), pool.data)
    rows = pool.data.reshape(-1, 656)
    assert np.all(rows[:, 516:520].copy().view(np.float32) == np.float32(2.0 ** -126))
    o, l, _ = run_prefill(d)
    _, lf32, of, _ = oracle.prefill(c.q, pool, c.indices, sink=c.sink, sm_scale=c.sm_scale)
    assert_out_close(bf16_dev_to_f64(o), of)
    assert_lse_close(l.cpu().numpy(), lf32)
    po, pl = smla.decode(d.q, d.pool, d.indices, 2, sm_scale=float(c.sm_scale))
    o2, l2 = smla.combine(po, pl, sink=d.sink)
    torch.cuda.synchronize()
    rpo, rpl = oracle.decode_split(c.q, pool, c.indices, 2, sm_scale=c.sm_scale)
    assert_out_close(po.cpu().numpy().astype(np.float64), rpo, "part_out", bf16=False)
    _, lf32, of, _ = oracle.combine(rpo, rpl, sink=c.sink)
    assert_out_close(bf16_dev_to_f64(o2), of)
    assert_lse_close(l2.cpu().numpy(), lf32)
