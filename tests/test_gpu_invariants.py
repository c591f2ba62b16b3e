"""GPU invariants and edge cases of the HIP path (no oracle needed for most:
each compares two GPU runs that must agree bit for bit, or checks a value the
definition fixes)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_mla_smla_amd as smla
from sparse_top_mla_smla_amd import workloads as W

from gpu_util import Dev, need_gpu
from helpers import oracle_pool

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def case(fmt=W.FMT_FP8, **kw):
    base = dict(T=6, H=16, n_seqs=1, ctx=1024, topk=300, causal=True)
    base.update(kw)
    return W.make_case("inv", config_id=250 + fmt, seed=3, fmt=fmt, **base)


def pre(d, idx=None, **kw):
    c = d.case
    o, l = smla.prefill(d.q, d.pool, d.indices if idx is None else idx, topk_length=kw.get("tl", d.topk_length),
                        sink=d.sink, sm_scale=float(c.sm_scale))
    torch.cuda.synchronize()
    return o, l


@pytest.mark.parametrize("fmt", [W.FMT_BF16, W.FMT_FP8, W.FMT_INT8])
def test_masked_entries_bit_exact(fmt):
    c = case(fmt, with_topk_length=True, with_sink=True)
    d = Dev(c)
    o1, l1 = pre(d)
    idx = c.indices.copy()
    rng = np.random.default_rng(0)
    nslots = c.num_blocks * 64
    for t in range(c.T):
        L = int(c.topk_length[t])
        idx[t, L:] = rng.integers(0, nslots, size=c.topk - L)          # garbage beyond L
        inside = np.nonzero(idx[t, :L] == -1)[0]
        idx[t, inside] = rng.choice([0x7FFFFFFF, -7, nslots], size=inside.shape[0])
        # and some -1 inside L swapped for out-of-range ids
        j = rng.integers(0, max(L, 1))
        if L > 0:
            idx[t, j] = -1
    # reference with -1 at the same inside positions
    ref_idx = idx.copy()
    for t in range(c.T):
        L = int(c.topk_length[t])
        bad = (ref_idx[t, :L] < 0) | (ref_idx[t, :L] >= nslots)
        ref_idx[t, :L][bad] = -1
        ref_idx[t, L:] = -1
    o2, l2 = pre(d, torch.from_numpy(idx).cuda())
    o3, l3 = pre(d, torch.from_numpy(ref_idx).cuda())
    assert torch.equal(o2, o3) and torch.equal(l2, l3)


def test_all_masked_and_zero_length():
    c = case(W.FMT_FP8, with_sink=True)
    d = Dev(c)
    idx = torch.full_like(d.indices, -1)
    o, l = pre(d, idx)
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))
    tl = torch.zeros(c.T, dtype=torch.int32, device="cuda")
    o, l = smla.prefill(d.q, d.pool, d.indices, topk_length=tl, sink=d.sink, sm_scale=float(c.sm_scale))
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))
    po, pl = smla.decode(d.q, d.pool, idx, 4, sm_scale=float(c.sm_scale))
    assert torch.all(torch.isneginf(pl)) and torch.all(po == 0)
    o, l = smla.combine(po, pl, sink=d.sink)
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))


def test_t_zero_launches_nothing():
    c = case(W.FMT_FP8, T=1)
    d = Dev(c)
    out = torch.full((0, c.H, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((0, c.H), dtype=torch.float32, device="cuda")
    o, l = smla.prefill(d.q[:0], d.pool, d.indices[:0], out=out, lse=lse)
    assert o.shape[0] == 0
    po, pl = smla.decode(d.q[:0], d.pool, d.indices[:0], 2)
    assert po.shape[0] == 0


def test_strided_views_equal_packed():
    c = case(W.FMT_BF16, H=8, hbuf=64, idx_ld=512, pad_fill=W.PAD_SENTINEL, with_sink=True)
    d = Dev(c)
    out_buf = torch.full((c.T, 64, 512), -5.0, dtype=torch.bfloat16, device="cuda")
    lse_buf = torch.full((c.T, 32), 9.0, dtype=torch.float32, device="cuda")
    o1, l1 = smla.prefill(d.q, d.pool, d.indices, sink=d.sink, sm_scale=float(c.sm_scale),
                          out=out_buf[:, :8], lse=lse_buf[:, :8])
    o2, l2 = smla.prefill(d.q.contiguous(), d.pool, d.indices.contiguous(), sink=d.sink,
                          sm_scale=float(c.sm_scale))
    torch.cuda.synchronize()
    assert torch.equal(out_buf[:, :8], o2) and torch.equal(lse_buf[:, :8], l2)
    assert torch.all(out_buf[:, 8:] == -5.0) and torch.all(lse_buf[:, 8:] == 9.0)


def test_few_heads_equal_head_prefix_of_wide_run():
    # h_q = 8 native equals heads 0..7 of a 64-head run on the same buffers
    c = case(W.FMT_BF16, H=64, topk=640, window=128, with_topk_length=True)
    d = Dev(c)
    o64, l64 = smla.prefill(d.q, d.pool, d.indices, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
    o8, l8 = smla.prefill(d.q[:, :8], d.pool, d.indices, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
    torch.cuda.synchronize()
    assert torch.equal(o8, o64[:, :8]) and torch.equal(l8, l64[:, :8])


def test_two_streams_equal_serial():
    c1 = case(W.FMT_FP8, H=64, topk=512)
    c2 = case(W.FMT_INT8, H=16, topk=256, with_sink=True)
    d1, d2 = Dev(c1), Dev(c2)
    r1 = pre(d1)
    r2 = pre(d2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            a = smla.prefill(d1.q, d1.pool, d1.indices, sm_scale=float(c1.sm_scale), stream=s1)
        with torch.cuda.stream(s2):
            b = smla.prefill(d2.q, d2.pool, d2.indices, sink=d2.sink, sm_scale=float(c2.sm_scale), stream=s2)
        outs.append((a, b))
    torch.cuda.synchronize()
    for a, b in outs:
        assert torch.equal(a[0], r1[0]) and torch.equal(a[1], r1[1])
        assert torch.equal(b[0], r2[0]) and torch.equal(b[1], r2[1])


def test_constant_column_gives_one_minus_sink_share():
    # nope column 0 = 1.0 in every row (shifts all scores of a head equally):
    # out[..., 0] = sum_j p_j = 1 - p_sink = 1 / (1 + exp(sink - lse))
    c = case(W.FMT_BF16, H=16, with_sink=True)
    kv = c.kv.copy()
    kv[:, 0] = W.f32_to_bf16_bits(np.float32([1.0]))[0]
    c.kv = kv
    d = Dev(c)
    o, l = pre(d)
    share = 1.0 / (1.0 + torch.exp(d.sink[None, :] - l))
    assert torch.allclose(o[:, :, 0].float(), share, atol=4e-3, rtol=0)



@pytest.mark.parametrize("H", [8, 64])
def test_fp8_non_power_of_two_scale_gives_nan(H):
    # FP8 scales must be powers of two; a selected row whose scale for
    # columns [128, 256) is 3.0 makes its token's output NaN, and tokens that
    # do not select the row are unchanged (both kernels that serve FP8 rows)
    c = case(W.FMT_FP8, H=H, topk=256)
    d = Dev(c)
    o1, l1 = pre(d)
    slot = int(c.indices[0, 0])
    assert slot >= 0
    rb = W.ROW_BYTES[W.FMT_FP8]
    flat = d.pool.data.view(-1)
    at = (slot // 64) * d.pool.data.stride(0) + (slot % 64) * rb + 512 + 4
    flat[at:at + 4] = torch.from_numpy(np.frombuffer(np.float32(3.0).tobytes(), np.uint8).copy()).cuda()
    o2, l2 = pre(d)
    sel = torch.from_numpy((c.indices == slot).any(axis=1)).cuda()
    assert sel[0]
    of = o2.float()
    assert torch.isnan(of[sel]).all()
    assert torch.equal(o2[~sel], o1[~sel]) and torch.equal(l2[~sel], l1[~sel])

@pytest.mark.parametrize("H", [16, 64])
@pytest.mark.parametrize("byte,nan", [(255, True), (0, False)])
def test_dsv4_special_scale_bytes(H, byte, nan):
    """DSv4 scale bytes read as 2^(b-127), 255 as NaN: a selected row whose
    tile-3 scale byte is 255 makes its tokens' outputs NaN and leaves the
    other tokens unchanged; a byte 0 (2^-127, which the writer never
    stores) leaves every output finite and within the bar of the oracle
    (the exponent-byte kernel at 16 heads, the many-head kernel at 64)."""
    c = case(W.FMT_FP8_DSV4, H=H, topk=256)
    d = Dev(c)
    o1, l1 = pre(d)
    slot = int(c.indices[0, 0])
    assert slot >= 0
    flat = d.pool.data.view(-1)
    at = (slot // 64) * d.pool.data.stride(0) + (slot % 64) * W.ROW_BYTES[W.FMT_FP8_DSV4] + 576 + 3
    flat[at] = byte
    o2, l2 = pre(d)
    sel = torch.from_numpy((c.indices == slot).any(axis=1)).cuda()
    assert sel[0]
    if nan:
        assert torch.isnan(o2.float()[sel]).all()
        assert torch.equal(o2[~sel], o1[~sel]) and torch.equal(l2[~sel], l1[~sel])
    else:
        pool = oracle_pool(c)
        pool.data[:] = d.pool.data.cpu().numpy()
        _, lf32, of, _ = oracle.prefill(c.q, pool, c.indices, sm_scale=c.sm_scale)
        from gpu_util import assert_lse_close, assert_out_close
        assert_out_close(o2.float().cpu().numpy().astype(np.float64), of)
        assert_lse_close(l2.cpu().numpy(), lf32)


def test_decode_split_invariance():
    # any split count merges to the prefill result (within tolerance)
    c = case(W.FMT_FP8, H=16, topk=1000, ctx=2048, with_sink=True, with_topk_length=True)
    d = Dev(c)
    o, l = pre(d)
    for S in (1, 2, 7, 16, 64):
        po, pl = smla.decode(d.q, d.pool, d.indices, S, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
        o2, l2 = smla.combine(po, pl, sink=d.sink)
        torch.cuda.synchronize()
        assert (o2.float() - o.float()).abs().max().item() <= 1e-2
        fin = torch.isfinite(l)
        assert torch.equal(fin, torch.isfinite(l2))
        assert (l2[fin] - l[fin]).abs().max().item() <= 1e-3


def test_error_codes():
    c = case(W.FMT_FP8, T=2)
    d = Dev(c)
    bad_pool = smla.KVPool(d.pool.data, W.FMT_FP8, page_block=32)
    with pytest.raises(smla.SmlaError, match="page_block 32"):
        smla.prefill(d.q, bad_pool, d.indices)
    with pytest.raises(smla.SmlaError, match="num_splits"):
        smla.decode(d.q, d.pool, d.indices, 65)
    q200 = torch.zeros((2, 129, 576), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(smla.SmlaError, match="H = 129"):
        smla.prefill(q200, d.pool, d.indices)
    narrow = smla.KVPool(torch.zeros((c.num_blocks, 64 * 656 - 16), dtype=torch.uint8, device="cuda"),
                         W.FMT_FP8)
    with pytest.raises(smla.SmlaError, match="block_stride"):
        smla.prefill(d.q, narrow, d.indices)


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_INT8, W.FMT_FP8_DSV4])
def test_nonfinite_row_stays_in_its_token(fmt):
    """One pool row holds non-finite data (e4m3 NaN codes, or a NaN rope
    value), and token A's list selects it.  Token B, which the same
    persistent prefill workgroup runs later (T = 300 > 256 workgroups), has
    a list of length 2, so position 3 of its first tile holds no candidate:
    that LDS row must not carry token A's row into B's result.  Every token
    other than A matches the oracle with finite outputs."""
    c = W.make_case(f"nan_row_{fmt}", config_id=296 + fmt, seed=6, fmt=fmt, T=300, H=64, n_seqs=1, ctx=1024,
                    topk=128, causal=False, with_topk_length=True)
    a, b = 5, 5 + 256
    bad_slot = int(c.slots[17])
    idx = c.idx_buf.copy()
    idx[idx == bad_slot] = -1                  # only A selects the row, at list position 3
    idx[a, 3] = bad_slot
    c.idx_buf = idx
    L = c.topk_length.copy()
    L[a] = max(int(L[a]), 4)
    L[b] = 2
    c.topk_length = L
    d = Dev(c)
    raw = d.pool.data.view(-1)
    off = (bad_slot // 64) * d.pool.data.stride(0) + (bad_slot % 64) * W.ROW_BYTES[fmt]
    if fmt == W.FMT_FP8:
        raw[off:off + 512] = 0x7F                                   # e4m3 NaN codes
    elif fmt == W.FMT_FP8_DSV4:
        raw[off:off + 448] = 0x7F                                   # e4m3 NaN codes
    else:
        raw[off + 528:off + 530] = torch.tensor([0xC0, 0x7F], dtype=torch.uint8, device="cuda")  # NaN rope
    pool = oracle_pool(c)
    pool.data[:] = d.pool.data.cpu().numpy()
    o, l = smla.prefill(d.q, d.pool, d.indices, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
    torch.cuda.synchronize()
    assert not torch.isfinite(o[a].float()).all()                   # A's own result is poisoned
    keep = np.array([t for t in range(c.T) if t != a])
    got = o.float().cpu().numpy().astype(np.float64)[keep]
    assert np.isfinite(got).all()
    _, lf32, of, _ = oracle.prefill(c.q, pool, c.indices, topk_length=c.topk_length, sm_scale=c.sm_scale,
                                    tokens=keep)
    from gpu_util import assert_lse_close, assert_out_close
    assert_out_close(got, of[keep])
    assert_lse_close(l.cpu().numpy()[keep], lf32[keep])


def test_binding_rejects_wrong_shapes():
    """The binding checks the sizes the kernels read and write before any
    call: a wrong output shape, a list wider than the index rows, fewer
    lengths than tokens or fewer sinks than heads raise SmlaError."""
    c = case(W.FMT_FP8, with_sink=True)
    d = Dev(c)
    T, H = c.T, c.H
    bad = [
        dict(out=torch.empty((T, H + 1, 512), dtype=torch.bfloat16, device="cuda")),
        dict(lse=torch.empty((T + 1, H), dtype=torch.float32, device="cuda")),
        dict(topk=c.topk + 1),
        dict(topk_length=torch.ones(T - 1, dtype=torch.int32, device="cuda")),
        dict(sink=torch.zeros(H - 1, dtype=torch.float32, device="cuda")),
    ]
    for kw in bad:
        with pytest.raises(smla.SmlaError):
            smla.prefill(d.q, d.pool, d.indices, sm_scale=float(c.sm_scale), **kw)
    with pytest.raises(smla.SmlaError):
        smla.prefill(d.q[:, :, :500], d.pool, d.indices)
    with pytest.raises(smla.SmlaError):
        smla.decode(d.q, d.pool, d.indices, 2,
                    part_out=torch.empty((T, 3, H, 512), dtype=torch.float32, device="cuda"))
    po, pl = smla.decode(d.q, d.pool, d.indices, 2)
    with pytest.raises(smla.SmlaError):
        smla.combine(po, pl[:, :1].contiguous())
    with pytest.raises(smla.SmlaError):
        smla.combine(po, pl, out=torch.empty((T, H, 256), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
