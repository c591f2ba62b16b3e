"""The measurement aids on the GPU: the gather probe moves exactly the rows
the lists select (its per-token counts equal the oracle-free count of
positions inside the length whose index is a pool slot), the clock probe
returns cycle and tick counts, and the device attributes are sane."""
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


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_BF16])
def test_gather_probe_counts_rows(fmt):
    c = W.make_case(f"probe_{fmt}", config_id=340 + fmt, seed=2, fmt=fmt, T=300, H=8, n_seqs=1, ctx=2048,
                    topk=200, causal=True, with_topk_length=True, tail_neg=5)
    idx = c.idx_buf.copy()
    idx[3, :7] = [c.num_blocks * 64, -5, 2 ** 31 - 1, -1, 0, 1, 2]   # out-of-range ids count as padding
    c.idx_buf = idx
    d = Dev(c)
    rows = smla.probe_gather(d.pool, d.indices, topk_length=d.topk_length)
    torch.cuda.synchronize()
    L = np.clip(c.topk_length, 0, c.topk)
    pos = np.arange(c.topk)[None, :]
    ids = c.indices
    want = ((pos < L[:, None]) & (ids >= 0) & (ids < c.num_blocks * 64)).sum(axis=1)
    assert np.array_equal(rows.cpu().numpy(), want)


def test_clock_probe_and_attributes():
    a = smla.device_attributes()
    assert a["compute_units"] > 0 and a["clock_khz"] > 0 and a["wall_clock_khz"] > 0
    out = smla.probe_clock(8, 2000).cpu().numpy()
    assert (out > 0).all()
    mhz = out[:, 0] / out[:, 1] * a["wall_clock_khz"] / 1000.0
    assert np.all((mhz > 100) & (mhz < 10000)), mhz
