"""Short lists put the precision of P, as it enters PV, straight into the
output.  With one to four candidates, one or two of them carry nearly all
the weight, so an error in a weight times |v| shows at full size, and
outputs of magnitude 2..4 leave only 1e-2 - 2^-8 of the bar once the BF16
rounding of out has taken its share.  The value rows here are twice the
unit normal of the other tests (|v| up to about 9): P rounded to BF16 (8
significant bits) would miss the bar by up to 2^-9 x 9 = 0.018, while P'
in FP16 (11 bits, for e4m3 codes) or as a BF16 pair (16 bits, for
arbitrary scales and BF16 rows) keeps every value within it.  At these
magnitudes the BF16 rounding of out alone averages more than the mean bar
of 1e-3, so the mean error may exceed that of the oracle's correctly rounded
output by at most 1e-3.  Every kernel family is covered: the many-head kernel (FP8, rope-less FP8, arbitrary
scales, INT8, DSv4), the MX kernels (DSv4 and DOTS3_SWA at 16 heads, DOTS3_SWA
at 64) and the few-head kernel (BF16, FP8, INT8), in the prefill form and,
for two of them, through split decode and the combine."""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_mla_smla_amd as smla
from sparse_top_mla_smla_amd import workloads as W

from gpu_util import Dev, assert_lse_close, assert_out_close, bf16_dev_to_f64, f64_of_bits, need_gpu
from helpers import oracle_pool

pytestmark = pytest.mark.gpu

CONFIGS = [
    (W.FMT_FP8, 64), (W.FMT_FP8_NOPE, 64), (W.FMT_FP8_ANY, 64), (W.FMT_INT8, 64), (W.FMT_FP8_DSV4, 64),
    (W.FMT_FP8_DSV4, 16), (W.FMT_FP8_DOTS3, 16), (W.FMT_FP8_DOTS3, 64),
    (W.FMT_BF16, 8), (W.FMT_FP8, 8), (W.FMT_INT8, 8),
]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def short_list_case(fmt, H):
    c = W.make_case(f"short_{fmt}_{H}", config_id=400 + 8 * fmt + H // 8, seed=11, fmt=fmt, T=256, H=H, n_seqs=1,
                    ctx=1024, topk=4, causal=False, with_topk_length=True)
    c.kv = W.f32_to_bf16_bits(W.bf16_bits_to_f32(c.kv) * 2.0)   # exact: a power of two
    return c


@pytest.mark.parametrize("fmt,H", CONFIGS)
def test_short_lists_with_large_values_prefill(fmt, H):
    c = short_list_case(fmt, H)
    d = Dev(c)
    o, l = smla.prefill(d.q, d.pool, d.indices, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
    torch.cuda.synchronize()
    ob, lf32, of, _ = oracle.prefill(c.q, oracle_pool(c), c.indices, topk_length=c.topk_length, sm_scale=c.sm_scale)
    assert_out_close(bf16_dev_to_f64(o), of, mean_ref=f64_of_bits(ob))
    assert_lse_close(l.cpu().numpy(), lf32)


@pytest.mark.parametrize("fmt,H", [(W.FMT_FP8, 64), (W.FMT_FP8_DSV4, 64)])
def test_short_lists_with_large_values_decode(fmt, H):
    """Two splits of the four-entry lists (two entries each), then the
    combine: the same bar on the combined BF16 output."""
    c = short_list_case(fmt, H)
    d = Dev(c)
    po, pl = smla.decode(d.q, d.pool, d.indices, 2, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
    o, l = smla.combine(po, pl)
    torch.cuda.synchronize()
    ob, lf32, of, _ = oracle.prefill(c.q, oracle_pool(c), c.indices, topk_length=c.topk_length, sm_scale=c.sm_scale)
    assert_out_close(bf16_dev_to_f64(o), of, mean_ref=f64_of_bits(ob))
    assert_lse_close(l.cpu().numpy(), lf32)


NOPE_DIMS = {W.FMT_FP8: 512, W.FMT_FP8_NOPE: 512, W.FMT_FP8_DSV4: 448, W.FMT_FP8_DOTS3: 1024}


@pytest.mark.parametrize("fmt,H", [(W.FMT_FP8, 64), (W.FMT_FP8, 8), (W.FMT_FP8_NOPE, 64), (W.FMT_FP8_DSV4, 64),
                                   (W.FMT_FP8_DSV4, 16), (W.FMT_FP8_DOTS3, 16), (W.FMT_FP8_DOTS3, 64)])
def test_scales_above_2_14(fmt, H):
    """The nope part of every cache row times 2^24 and of every q row times
    2^-24 leaves each score unchanged and makes the scales 2^24 times larger
    (above 2^14, where the FP16 bias runs out and the kernels keep O's code
    columns in units of 2^-k).  The exact result is then the unscaled case's
    with its nope value columns times 2^24: the outputs scaled back by 2^-24
    (exact in BF16 and FP32) meet the bar against the oracle of the unscaled
    case, in the prefill form and in the decode partials."""
    c = W.make_case(f"bigscale_{fmt}_{H}", config_id=460 + 8 * fmt + H // 8, seed=12, fmt=fmt, T=96, H=H, n_seqs=1,
                    ctx=1024, topk=200, causal=True, with_topk_length=True)
    n = NOPE_DIMS[fmt]
    pool = oracle_pool(c)
    ob, lf32, of, _ = oracle.prefill(c.q, pool, c.indices, topk_length=c.topk_length, sm_scale=c.sm_scale)
    rpo, rpl = oracle.decode_split(c.q, pool, c.indices, 3, topk_length=c.topk_length, sm_scale=c.sm_scale)
    kv = W.bf16_bits_to_f32(c.kv)
    kv[:, :n] *= 2.0 ** 24
    q = W.bf16_bits_to_f32(c.q_buf)
    q[:, :, :n] *= 2.0 ** -24
    c.kv, c.q_buf = W.f32_to_bf16_bits(kv), W.f32_to_bf16_bits(q)
    d = Dev(c)
    o, l = smla.prefill(d.q, d.pool, d.indices, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
    po, pl = smla.decode(d.q, d.pool, d.indices, 3, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
    torch.cuda.synchronize()
    down = torch.ones(o.shape[-1], dtype=torch.float64)
    down[:n] = 2.0 ** -24
    got = o.double().cpu() * down
    assert torch.isfinite(got).all()
    assert_out_close(got.numpy(), of, mean_ref=f64_of_bits(ob))
    assert_lse_close(l.cpu().numpy(), lf32)
    assert_out_close((po.double().cpu() * down).numpy(), rpo, what="part_out", bf16=False)
    assert_lse_close(pl.cpu().numpy(), rpl, what="part_lse")


@pytest.mark.parametrize("fmt,H", [(W.FMT_FP8, 64), (W.FMT_FP8_NOPE, 64), (W.FMT_FP8_ANY, 64), (W.FMT_INT8, 64),
                                   (W.FMT_FP8_DSV4, 64), (W.FMT_FP8_DSV4, 16), (W.FMT_FP8_DOTS3, 16),
                                   (W.FMT_FP8_DOTS3, 64), (W.FMT_FP8, 8), (W.FMT_BF16, 8), (W.FMT_INT8, 8)])
def test_dominant_candidate_at_every_tile_position(fmt, H):
    """One list entry per token scores about 40 nats above all others: the
    q rows share a direction u (u + 0.5 x the unit normal q) and that entry's
    cache row is a multiple of u.  Token t's dominant entry sits at list
    position t mod 128, so across the tokens it takes every position of both
    64-candidate tiles (each token has a sequence of its own, so no other
    token's dominant row enters its list).  The softmax's running maximum must
    come from all candidates of a tile: a maximum that missed the dominant
    entry would leave its probability at about 2^58 relative to the others,
    beyond FP16 and every rescaling, and the output would not be finite.
    Prefill, and decode over two splits with the combine, against the
    oracle."""
    T = 128
    c = W.make_case(f"dominant_{fmt}_{H}", config_id=530 + 8 * fmt + H // 8, seed=14, fmt=fmt, T=T, H=H, n_seqs=T,
                    ctx=256, topk=128, causal=False)
    dims = c.kv.shape[1]
    rng = np.random.default_rng(1400 + fmt)
    u = rng.standard_normal(dims) * 2.5
    q = W.bf16_bits_to_f32(c.q_buf).astype(np.float64)
    c.q_buf = W.f32_to_bf16_bits((u[None, None, :] + 0.5 * q).astype(np.float32))
    alpha = 40.0 / (float(c.sm_scale) * float(u @ u))
    kv = W.bf16_bits_to_f32(c.kv)
    row_of_slot = np.empty(c.slots.shape[0], dtype=np.int64)
    row_of_slot[c.slots] = np.arange(c.slots.shape[0])
    for t in range(T):
        kv[row_of_slot[c.idx_buf[t, t % 128]]] = (alpha * u).astype(np.float32)
    c.kv = W.f32_to_bf16_bits(kv)
    d = Dev(c)
    o, l = smla.prefill(d.q, d.pool, d.indices, sm_scale=float(c.sm_scale))
    po, pl = smla.decode(d.q, d.pool, d.indices, 2, sm_scale=float(c.sm_scale))
    oc, lc = smla.combine(po, pl)
    torch.cuda.synchronize()
    ob, lf32, of, _ = oracle.prefill(c.q, oracle_pool(c), c.indices, sm_scale=c.sm_scale)
    assert_out_close(bf16_dev_to_f64(o), of, mean_ref=f64_of_bits(ob))
    assert_lse_close(l.cpu().numpy(), lf32)
    assert_out_close(bf16_dev_to_f64(oc), of, what="combined out", mean_ref=f64_of_bits(ob))
    assert_lse_close(lc.cpu().numpy(), lf32, what="combined lse")


@pytest.mark.parametrize("fmt,H", [(W.FMT_FP8, 64), (W.FMT_FP8_ANY, 64), (W.FMT_FP8_DSV4, 64), (W.FMT_FP8_DSV4, 16),
                                   (W.FMT_FP8_DOTS3, 64), (W.FMT_FP8, 8), (W.FMT_BF16, 8)])
def test_maximum_rising_in_every_tile(fmt, H):
    """Every 64-entry block of each token's list scores about 12 nats above
    the block before it (the cache row of list entry j is (1 + j // 64) x a
    multiple of the q rows' common direction u, plus the unit normal row),
    so the running maximum moves past its lazy threshold in every tile and
    O and l are rescaled each time; the per-entry normal parts keep the
    probabilities within a block uneven.  Prefill, and decode over three
    splits with the combine, against the oracle."""
    T = 64
    c = W.make_case(f"rising_{fmt}_{H}", config_id=620 + 8 * fmt + H // 8, seed=15, fmt=fmt, T=T, H=H, n_seqs=T,
                    ctx=256, topk=256, causal=False)
    dims = c.kv.shape[1]
    rng = np.random.default_rng(1500 + fmt)
    u = rng.standard_normal(dims) * 2.5
    q = W.bf16_bits_to_f32(c.q_buf).astype(np.float64)
    c.q_buf = W.f32_to_bf16_bits((u[None, None, :] + 0.5 * q).astype(np.float32))
    step = 12.0 / (float(c.sm_scale) * float(u @ u))
    kv = W.bf16_bits_to_f32(c.kv).astype(np.float64)
    row_of_slot = np.empty(c.slots.shape[0], dtype=np.int64)
    row_of_slot[c.slots] = np.arange(c.slots.shape[0])
    for t in range(T):
        rows = row_of_slot[c.idx_buf[t, :256]]
        kv[rows] += ((1 + np.arange(256) // 64) * step)[:, None] * u[None, :]
    c.kv = W.f32_to_bf16_bits(kv.astype(np.float32))
    d = Dev(c)
    o, l = smla.prefill(d.q, d.pool, d.indices, sm_scale=float(c.sm_scale))
    po, pl = smla.decode(d.q, d.pool, d.indices, 3, sm_scale=float(c.sm_scale))
    oc, lc = smla.combine(po, pl)
    torch.cuda.synchronize()
    ob, lf32, of, _ = oracle.prefill(c.q, oracle_pool(c), c.indices, sm_scale=c.sm_scale)
    assert_out_close(bf16_dev_to_f64(o), of, mean_ref=f64_of_bits(ob))
    assert_lse_close(l.cpu().numpy(), lf32)
    assert_out_close(bf16_dev_to_f64(oc), of, what="combined out", mean_ref=f64_of_bits(ob))
    assert_lse_close(lc.cpu().numpy(), lf32, what="combined lse")


@pytest.mark.parametrize("fmt,H", [(W.FMT_FP8, 64), (W.FMT_INT8, 64), (W.FMT_FP8_DSV4, 64), (W.FMT_FP8_DSV4, 16),
                                   (W.FMT_FP8_DOTS3, 64), (W.FMT_FP8, 8)])
def test_each_head_its_own_dominant_candidate(fmt, H):
    """Head h of token t has a direction u_h of its own (q = u_h + 0.5 x
    the unit normal q) and its dominant list entry at position
    (7h + 3t) mod 128, whose cache row is a multiple of u_h scoring about
    40 nats above the others for that head (about 2 nats for the other
    heads).  Each head's running maximum must come from its own entries:
    the heads of one workgroup take their maxima at different tile
    positions and in different tiles.  Prefill and two-split decode with
    the combine, against the oracle."""
    T = 128
    c = W.make_case(f"headdom_{fmt}_{H}", config_id=900 + 8 * fmt + H // 8, seed=16, fmt=fmt, T=T, H=H, n_seqs=T,
                    ctx=256, topk=128, causal=False)
    dims = c.kv.shape[1]
    rng = np.random.default_rng(1600 + fmt)
    u = rng.standard_normal((H, dims)) * 2.5
    q = W.bf16_bits_to_f32(c.q_buf).astype(np.float64)
    c.q_buf = W.f32_to_bf16_bits((u[None, :, :] + 0.5 * q).astype(np.float32))
    kv = W.bf16_bits_to_f32(c.kv).astype(np.float64)
    row_of_slot = np.empty(c.slots.shape[0], dtype=np.int64)
    row_of_slot[c.slots] = np.arange(c.slots.shape[0])
    for t in range(T):
        for h in range(H):
            alpha = 40.0 / (float(c.sm_scale) * float(u[h] @ u[h]))
            kv[row_of_slot[c.idx_buf[t, (7 * h + 3 * t) % 128]]] = alpha * u[h]
    c.kv = W.f32_to_bf16_bits(kv.astype(np.float32))
    d = Dev(c)
    o, l = smla.prefill(d.q, d.pool, d.indices, sm_scale=float(c.sm_scale))
    po, pl = smla.decode(d.q, d.pool, d.indices, 2, sm_scale=float(c.sm_scale))
    oc, lc = smla.combine(po, pl)
    torch.cuda.synchronize()
    ob, lf32, of, _ = oracle.prefill(c.q, oracle_pool(c), c.indices, sm_scale=c.sm_scale)
    assert_out_close(bf16_dev_to_f64(o), of, mean_ref=f64_of_bits(ob))
    assert_lse_close(l.cpu().numpy(), lf32)
    assert_out_close(bf16_dev_to_f64(oc), of, what="combined out", mean_ref=f64_of_bits(ob))
    assert_lse_close(lc.cpu().numpy(), lf32, what="combined lse")
