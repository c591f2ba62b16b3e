"""HIP graph capture of the path: the cache write + prefill, and decode +
combine, captured once on the current stream (torch.cuda.graph drives HIP
stream capture; the library launches only kernels, no memset or copy) and
replayed with eager work between the replays.  Every replay must equal the
eager result for the same inputs bit for bit."""
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


def _case(fmt, H, T, cid):
    return W.make_case(f"graph_{fmt}_{H}", config_id=cid, seed=0, fmt=fmt, T=T, H=H, n_seqs=1, ctx=2048,
                       topk=512, causal=True, with_sink=True, with_topk_length=True)


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("fmt,H", [(W.FMT_FP8, 64), (W.FMT_INT8, 128), (W.FMT_BF16, 8), (W.FMT_FP8_DSV4, 64)])
def test_decode_combine_graph_replays(fmt, H):
    c = _case(fmt, H, 6, 300 + fmt)
    d = Dev(c)
    S = 3
    dv = smla.value_dims(fmt)
    qd = smla.query_dims(fmt)
    q = d.q[:, :, :qd]
    sets = [d.indices.clone(), torch.flip(d.indices, dims=[1]).contiguous()]
    idx = sets[0].clone()  # the graph's index buffer
    po = torch.empty((c.T, S, H, dv), dtype=torch.float32, device="cuda")
    pl = torch.empty((c.T, S, H), dtype=torch.float32, device="cuda")
    out = torch.empty((c.T, H, dv), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((c.T, H), dtype=torch.float32, device="cuda")

    def run():
        smla.decode(q, d.pool, idx, S, sm_scale=float(c.sm_scale), part_out=po, part_lse=pl)
        smla.combine(po, pl, sink=d.sink, out=out, lse=lse)

    ref = []
    for s in sets:
        idx.copy_(s)
        run()
        torch.cuda.synchronize()
        ref.append((out.clone(), lse.clone(), pl.clone()))
    g = _capture(run)
    for i in range(6):
        k = i % 2
        idx.copy_(sets[k])  # eager work between the replays
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[k][0]) and torch.equal(lse, ref[k][1]) and torch.equal(pl, ref[k][2]), i


@pytest.mark.parametrize("fmt,H", [(W.FMT_FP8, 64), (W.FMT_BF16, 8)])
def test_cache_write_and_prefill_graph_replays(fmt, H):
    c = _case(fmt, H, 5, 310 + fmt)
    d = Dev(c)
    kv = d.kv.clone()  # the graph's latent rows, rewritten into the pool by every replay
    slots = d.slots
    out = torch.empty((c.T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((c.T, H), dtype=torch.float32, device="cuda")

    def run():
        smla.quantize_kv(kv, slots, d.pool)
        smla.prefill(d.q, d.pool, d.indices, topk_length=d.topk_length, sink=d.sink, sm_scale=float(c.sm_scale),
                     out=out, lse=lse)

    rng = np.random.default_rng(5)
    scales = [1.0, 0.5]
    ref = []
    base = d.kv.clone()
    for sc in scales:
        kv.copy_(base * sc)
        run()
        torch.cuda.synchronize()
        ref.append((out.clone(), lse.clone(), d.pool.data.clone()))
    g = _capture(run)
    for i in range(6):
        k = i % 2
        kv.copy_(base * scales[k])
        d.pool.data.fill_(int(rng.integers(0, 256)))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.pool.data, ref[k][2]), i
        assert torch.equal(out, ref[k][0]) and torch.equal(lse, ref[k][1]), i
