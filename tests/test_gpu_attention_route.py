"""smla_attention on the GPU: whichever form the split-count model routes a
shape to, the result matches the oracle's prefill to the output tolerance;
without a workspace (or with one that is too small) it is the prefill form,
bit for bit."""
import pytest
import torch

import oracle
import sparse_top_mla_smla_amd as smla
from sparse_top_mla_smla_amd import workloads as W

from gpu_util import Dev, assert_lse_close, assert_out_close, bf16_dev_to_f64, need_gpu
from helpers import oracle_pool

pytestmark = pytest.mark.gpu

CASES = {
    # many heads, few tokens, a long list: routed to the split form
    "fp8_h64_t4_w1024_sink": dict(fmt=W.FMT_FP8, H=64, T=4, topk=1024, ctx=2048, with_sink=True),
    # the same heads with a short list: the prefill form
    "fp8_h64_t4_w128": dict(fmt=W.FMT_FP8, H=64, T=4, topk=128, ctx=512),
    # few heads (the column-split kernel), ragged lengths, sink, strided q/out head views
    "bf16_h8_t3_w640_len_sink": dict(fmt=W.FMT_BF16, H=8, hbuf=64, T=3, topk=640, ctx=2048, window=128,
                                     with_topk_length=True, with_sink=True, out_hbuf=64),
    "int8_h128_t2_w768_sink": dict(fmt=W.FMT_INT8, H=128, T=2, topk=768, ctx=1024, with_sink=True),
    # rows with exponent-byte scales (their own kernel and model constants)
    "dots3_h64_t3_w1024_sink": dict(fmt=W.FMT_FP8_DOTS3, H=64, T=3, topk=1024, ctx=2048, with_sink=True),
    "dsv4_h20_t2_w2048_len": dict(fmt=W.FMT_FP8_DSV4, H=20, T=2, topk=2048, ctx=4096, with_topk_length=True),
    "dsv4_h64_t64_w128": dict(fmt=W.FMT_FP8_DSV4, H=64, T=64, topk=128, ctx=512),
}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def make(name):
    base = dict(n_seqs=1, causal=True)
    base.update(CASES[name])
    return W.make_case(name, config_id=300 + sorted(CASES).index(name), seed=1, **base)


def run(d, workspace):
    c = d.case
    out = None
    if c.out_hbuf:
        out = torch.full((c.T, c.out_hbuf, W.V_DIMS[c.fmt]), 7.0, dtype=torch.bfloat16, device="cuda")[:, : c.H]
    o, l = smla.attention(d.q, d.pool, d.indices, topk_length=d.topk_length, sink=d.sink,
                          sm_scale=float(c.sm_scale), out=out, workspace=workspace)
    torch.cuda.synchronize()
    return o, l


def test_cases_cover_both_forms():
    forms = {smla.use_split_form(make(n).T, make(n).H, make(n).topk, make(n).fmt) for n in CASES}
    assert forms == {0, 1}


@pytest.mark.parametrize("name", sorted(CASES))
def test_routed_result_matches_the_oracle(name):
    c = make(name)
    d = Dev(c)
    nbytes = smla.attention_workspace_size(c.T, c.H, c.topk, c.fmt)
    split = smla.use_split_form(c.T, c.H, c.topk, c.fmt) == 1
    assert (nbytes > 0) == split
    if split:
        S = smla.decode_num_splits(c.T, c.H, c.topk, c.fmt)
        assert nbytes == smla.decode_workspace_size(c.T, c.H, S, W.V_DIMS[c.fmt])
    ws = torch.full((max(nbytes, 16),), 0xFF, dtype=torch.uint8, device="cuda")  # stale contents
    o, l = run(d, ws)
    _, lf32, of, _ = oracle.prefill(c.q, oracle_pool(c), c.indices, topk_length=c.topk_length, sink=c.sink,
                                    sm_scale=c.sm_scale)
    assert_out_close(bf16_dev_to_f64(o), of)
    assert_lse_close(l.cpu().numpy(), lf32)


@pytest.mark.parametrize("name", sorted(CASES))
def test_without_workspace_it_is_the_prefill_form(name):
    c = make(name)
    d = Dev(c)
    o_ref, l_ref = smla.prefill(d.q, d.pool, d.indices, topk_length=d.topk_length, sink=d.sink,
                                sm_scale=float(c.sm_scale))
    for ws in (None, torch.zeros(16, dtype=torch.uint8, device="cuda")):
        o, l = run(d, ws)
        assert torch.equal(o.contiguous(), o_ref) and torch.equal(l, l_ref)
