"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times.  The oracle computes sampled tokens one by one from the
generator's latent rows with its own quantizer (only the rows those tokens
select are quantized on the CPU); the GPU runs the whole batch.  Checked:
cache bytes of the sampled rows (bit-exact), sampled outputs and LSE (to the
stated tolerance), and properties that hold for every token (finite output,
-inf LSE exactly where a token has no candidate, untouched out-of-view heads).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_mla_smla_amd as smla
from sparse_top_mla_smla_amd import workloads as W

from gpu_util import assert_lse_close, assert_out_close, bf16_dev_to_f64, need_gpu, u16_to_bf16_dev

pytestmark = pytest.mark.gpu
N_SAMPLE = 16


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def sample_tokens(T, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, N_SAMPLE - 2, replace=False)])).astype(np.int64)


def oracle_pool_for(case, tokens):
    """Oracle pool holding only the rows the sampled tokens select."""
    rb = W.ROW_BYTES[case.fmt]
    pool = oracle.Pool(np.zeros((case.num_blocks, 64 * rb), np.uint8), case.fmt, 64 * rb)
    sel = case.indices[tokens].reshape(-1)
    sel = np.unique(sel[(sel >= 0) & (sel < case.num_blocks * 64)])
    # latent row of each slot: invert the slot map
    row_of_slot = np.empty(case.num_blocks * 64, np.int64)
    row_of_slot[case.slots] = np.arange(case.slots.shape[0])
    rows = row_of_slot[sel]
    oracle.quantize_kv(case.kv[rows], sel.astype(np.int32), pool)
    return pool, sel


def gpu_setup(case):
    q_buf = u16_to_bf16_dev(case.q_buf)
    kv = u16_to_bf16_dev(case.kv)
    pool = smla.KVPool.empty(case.num_blocks, case.fmt)
    smla.quantize_kv(kv, torch.from_numpy(case.slots).cuda(), pool)
    del kv
    idx_buf = torch.from_numpy(case.idx_buf).cuda()
    tl = None if case.topk_length is None else torch.from_numpy(case.topk_length).cuda()
    sink = None if case.sink is None else torch.from_numpy(case.sink).cuda()
    return q_buf, pool, idx_buf, tl, sink


def check_pool_rows(case, gpu_pool, ref_pool, slots):
    rb = W.ROW_BYTES[case.fmt]
    g = gpu_pool.data.view(-1)
    blocks = torch.from_numpy(slots // 64).cuda()
    offs = torch.from_numpy(slots % 64).cuda()
    base = blocks * gpu_pool.data.stride(0) + offs * rb
    idx = base[:, None] + torch.arange(rb, device="cuda")[None, :]
    got = g[idx.reshape(-1)].view(-1, rb).cpu().numpy()
    want = ref_pool.data.reshape(-1)[((slots // 64) * ref_pool.block_stride + (slots % 64) * rb)[:, None]
                                     + np.arange(rb)[None, :]]
    assert np.array_equal(got, want), "cache bytes differ from the oracle's"


def empty_tokens(case):
    nslots = case.num_blocks * 64
    idx = case.indices
    ok = (idx >= 0) & (idx < nslots)
    if case.topk_length is not None:
        ok &= np.arange(case.topk)[None, :] < np.clip(case.topk_length, 0, case.topk)[:, None]
    return ~ok.any(axis=1)


def run_prefill_case(case, out_hbuf=0):
    q_buf, pool, idx_buf, tl, sink = gpu_setup(case)
    q = q_buf[:, : case.H]
    if out_hbuf:
        out_buf = torch.full((case.T, out_hbuf, W.V_DIMS[case.fmt]), 3.0, dtype=torch.bfloat16, device="cuda")
        out = out_buf[:, : case.H]
    else:
        out_buf, out = None, None
    o, l = smla.prefill(q, pool, idx_buf[:, : case.topk], topk_length=tl, sink=sink,
                        sm_scale=float(case.sm_scale), out=out)
    torch.cuda.synchronize()
    tokens = sample_tokens(case.T)
    ref_pool, slots = oracle_pool_for(case, tokens)
    check_pool_rows(case, pool, ref_pool, slots)
    _, lf, of, _ = oracle.prefill(case.q, ref_pool, case.indices, topk_length=case.topk_length, sink=case.sink,
                                  sm_scale=case.sm_scale, tokens=tokens)
    assert_out_close(bf16_dev_to_f64(o[tokens]), of[tokens])
    assert_lse_close(l[tokens].cpu().numpy(), lf[tokens])
    # every token: finite output; -inf LSE exactly for tokens with no candidate
    assert torch.isfinite(o.float()).all()
    lall = l.cpu().numpy()
    emp = empty_tokens(case)
    assert np.array_equal(np.isneginf(lall), np.repeat(emp[:, None], case.H, axis=1)) and not np.isnan(lall).any()
    if out_buf is not None:
        assert torch.all(out_buf[:, case.H:] == 3.0)


def test_fullsize_prefill_fp8_w1024():
    run_prefill_case(W.c3_prefill(width=1024))


def test_fullsize_prefill_fp8_w512():
    run_prefill_case(W.c3_prefill(width=512))


def test_fullsize_fewhead_bf16():
    run_prefill_case(W.c4_fewhead(), out_hbuf=64)


def test_fullsize_int8_h128():
    run_prefill_case(W.c5_int8())


def test_fullsize_prefill_dots3():
    run_prefill_case(W.dots3_prefill(), out_hbuf=80)


def test_fullsize_prefill_dsv4():
    """DSv4 rows at the metric's shape (T=1024, ctx 16384, H=64, topk 1024)."""
    run_prefill_case(W.make_case("dsv4_c3", config_id=8, seed=0, fmt=W.FMT_FP8_DSV4, T=1024, H=64, n_seqs=1,
                                 ctx=16384, topk=1024, causal=True, with_sink=True))


@pytest.mark.parametrize("make", [W.c2_decode, W.dots3_decode], ids=["fp8", "dots3"])
def test_fullsize_decode(make):
    case = make()
    q_buf, pool, idx_buf, tl, sink = gpu_setup(case)
    S = case.num_splits
    po, pl = smla.decode(q_buf[:, : case.H], pool, idx_buf[:, : case.topk], S, sm_scale=float(case.sm_scale))
    o, l = smla.combine(po, pl)
    torch.cuda.synchronize()
    tokens = sample_tokens(case.T)
    ref_pool, slots = oracle_pool_for(case, tokens)
    check_pool_rows(case, pool, ref_pool, slots)
    rpo, rpl = oracle.decode_split(case.q, ref_pool, case.indices, S, sm_scale=case.sm_scale, tokens=tokens)
    gpl = pl.cpu().numpy()
    assert np.array_equal(np.isneginf(gpl[tokens]), np.isneginf(rpl[tokens]))
    assert_lse_close(gpl[tokens], rpl[tokens].astype(np.float32), "part_lse")
    assert_out_close(po[tokens].cpu().numpy().astype(np.float64), rpo[tokens], "part_out", bf16=False)
    _, lf, of, _ = oracle.combine(rpo, rpl, tokens=tokens)
    assert_out_close(bf16_dev_to_f64(o[tokens]), of[tokens])
    assert_lse_close(l[tokens].cpu().numpy(), lf[tokens])
    assert torch.isfinite(o.float()).all() and torch.isfinite(l).all()


def test_fullsize_dual_decode_dsv4():
    """The dual-cache decode batch over DSv4 rows: 64 sequences x 1 query,
    H=64, a 1024-wide main list and a 2176-wide secondary list over two
    pools of 16384-token sequences, 4 splits."""
    main = W.make_case("dsv4_dual_main", config_id=9, seed=0, fmt=W.FMT_FP8_DSV4, T=64, H=64, n_seqs=64,
                       ctx=16384, topk=1024, causal=True)
    extra = W.make_case("dsv4_dual_extra", config_id=10, seed=0, fmt=W.FMT_FP8_DSV4, T=64, H=64, n_seqs=64,
                        ctx=16384, topk=2176, causal=False)
    S = 4
    q_buf, pool, idx_buf, _, _ = gpu_setup(main)
    _, xpool, xidx_buf, _, _ = gpu_setup(extra)
    po, pl = smla.decode_dual(q_buf[:, : main.H], pool, idx_buf[:, : main.topk], xpool, xidx_buf[:, : extra.topk], S,
                              sm_scale=float(main.sm_scale))
    o, l = smla.combine(po, pl)
    torch.cuda.synchronize()
    tokens = sample_tokens(main.T)
    p1, s1 = oracle_pool_for(main, tokens)
    p2, s2 = oracle_pool_for(extra, tokens)
    check_pool_rows(main, pool, p1, s1)
    check_pool_rows(extra, xpool, p2, s2)
    # the reference: both pools laid end to end, secondary slots moved past the main pool's
    n1 = main.num_blocks * 64
    both = oracle.Pool(np.concatenate([p1.data, p2.data]), main.fmt, p1.block_stride)
    idx = np.ascontiguousarray(np.concatenate([main.indices, np.where(extra.indices >= 0, extra.indices + n1, -1)],
                                              axis=1).astype(np.int32))
    rpo, rpl = oracle.decode_split(main.q, both, idx, S, sm_scale=main.sm_scale, tokens=tokens)
    gpl = pl.cpu().numpy()
    assert np.array_equal(np.isneginf(gpl[tokens]), np.isneginf(rpl[tokens]))
    assert_lse_close(gpl[tokens], rpl[tokens].astype(np.float32), "part_lse")
    assert_out_close(po[tokens].cpu().numpy().astype(np.float64), rpo[tokens], "part_out", bf16=False)
    _, lf, of, _ = oracle.combine(rpo, rpl, tokens=tokens)
    assert_out_close(bf16_dev_to_f64(o[tokens]), of[tokens])
    assert_lse_close(l[tokens].cpu().numpy(), lf[tokens])
    assert torch.isfinite(o.float()).all() and torch.isfinite(l).all()
