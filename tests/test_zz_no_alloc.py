"""smla_attention_noalloc, the entry point for callers that cannot allocate:
called through the C ABI (ctypes, raw device pointers), its out and lse
must equal smla_attention's with a caller workspace bit for bit -- the same
kernels over the same partials -- on two calls in a row, the second with a
smaller input (a shorter batch and list over the same static scratch).
Both shapes take the split form, so the static scratch is used."""
import ctypes

import numpy as np
import pytest
import torch

import sparse_top_mla_smla_amd as smla
from sparse_top_mla_smla_amd import workloads as W

from gpu_util import Dev, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _c_noalloc(d, out, lse):
    """smla_attention_noalloc through the C ABI with raw pointers."""
    c = d.case
    L = smla._load()
    st = L.smla_attention_noalloc(
        d.q.data_ptr(), c.T, c.H, d.q.stride(0), d.q.stride(1), d.pool.c(), d.indices.data_ptr(), c.topk,
        d.indices.stride(0), None if d.topk_length is None else d.topk_length.data_ptr(),
        None if d.sink is None else d.sink.data_ptr(), ctypes.c_float(float(c.sm_scale)), out.data_ptr(),
        out.stride(0), out.stride(1), lse.data_ptr(), lse.stride(0), torch.cuda.current_stream().cuda_stream)
    assert st == 0, L.smla_last_error().decode()


def test_noalloc_equals_workspace_form_twice():
    shapes = [dict(T=48, H=64, topk=1024, ctx=4096, with_topk_length=True, with_sink=True),
              dict(T=5, H=64, topk=512, ctx=1024, with_topk_length=False, with_sink=True)]
    for i, sh in enumerate(shapes):
        c = W.make_case(f"noalloc_{i}", config_id=330 + i, seed=7, fmt=W.FMT_FP8, n_seqs=1, causal=True, **sh)
        assert smla.use_split_form(c.T, c.H, c.topk, c.fmt) == 1, "the shape must take the split form"
        d = Dev(c)
        out = torch.full((c.T, c.H, 512), 3.0, dtype=torch.bfloat16, device="cuda")
        lse = torch.full((c.T, c.H), 3.0, dtype=torch.float32, device="cuda")
        _c_noalloc(d, out, lse)
        ws = torch.empty(smla.attention_workspace_size(c.T, c.H, c.topk, c.fmt), dtype=torch.uint8, device="cuda")
        ref_o, ref_l = smla.attention(d.q, d.pool, d.indices, topk_length=d.topk_length, sink=d.sink,
                                      sm_scale=float(c.sm_scale), workspace=ws)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        assert torch.equal(out, ref_o), f"call {i}: out differs from smla_attention's"
        assert torch.equal(lse, ref_l), f"call {i}: lse differs from smla_attention's"
        # the binding's wrapper of the same entry point
        o2, l2 = smla.attention_noalloc(d.q, d.pool, d.indices, topk_length=d.topk_length, sink=d.sink,
                                        sm_scale=float(c.sm_scale))
        torch.cuda.synchronize()
        assert torch.equal(o2, ref_o) and torch.equal(l2, ref_l)


def test_noalloc_rejects_partials_beyond_the_scratch():
    # BF16 rows, T=200, H=64, topk 8192: the model picks 3 splits, 75 MiB of partials
    T, H, topk = 200, 64, 8192
    assert smla.use_split_form(T, H, topk, W.FMT_BF16) == 1
    pool = smla.KVPool.empty(128, W.FMT_BF16)
    q = torch.zeros((T, H, 576), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((T, topk), dtype=torch.int32, device="cuda")
    with pytest.raises(smla.SmlaError, match="static"):
        smla.attention_noalloc(q, pool, idx)
