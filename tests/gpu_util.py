"""Helpers for GPU tests: move workload cases to the device, build pools
with the HIP quantizer, and compare against the oracle with the tolerance
the problem statement fixes (BF16 out: max_abs <= 1e-2 and mean_abs <= 1e-3;
LSE: 1e-3 absolute; -inf positions identical)."""
import numpy as np
import pytest
import torch

import sparse_top_mla_smla_amd as smla
from sparse_top_mla_smla_amd import workloads as W

OUT_MAX_ABS = 1e-2
OUT_MEAN_ABS = 1e-3
LSE_ABS = 1e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # a GPU run must use the HIP library: fail, never skip, when it is missing
    assert smla.row_bytes(W.FMT_FP8) == 656, smla.library_path()


def u16_to_bf16_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_dev_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


class Dev:
    """Device copies of a case's inputs plus a pool filled by smla.quantize_kv."""

    def __init__(self, case: W.Case, block_stride: int = 0, fill: int = 0, row_stride: int = 0):
        self.case = case
        self.q_buf = u16_to_bf16_dev(case.q_buf)
        self.q = self.q_buf[:, : case.H]
        self.kv = u16_to_bf16_dev(case.kv)
        self.slots = torch.from_numpy(case.slots).cuda()
        self.idx_buf = torch.from_numpy(case.idx_buf).cuda()
        self.indices = self.idx_buf[:, : case.topk]
        self.topk_length = None if case.topk_length is None else torch.from_numpy(case.topk_length).cuda()
        self.sink = None if case.sink is None else torch.from_numpy(case.sink).cuda()
        rb = W.ROW_BYTES[case.fmt]
        bs = block_stride or 64 * (row_stride or rb)
        self.pool = smla.KVPool(torch.full((case.num_blocks, bs), fill, dtype=torch.uint8, device="cuda"),
                                case.fmt, row_stride=row_stride)
        smla.quantize_kv(self.kv, self.slots, self.pool)


def f64_of_bits(bits: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of the BF16 grid at |x| (8 significant bits)."""
    mag = np.abs(x)
    e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def assert_out_close(got: np.ndarray, want: np.ndarray, what: str = "out", ulp_floor: bool = False):
    """max_abs <= 1e-2 and mean_abs <= 1e-3.  ulp_floor: BF16 outputs of
    magnitude 2 or more sit on a grid coarser than 1e-2 (spacing 2^-6), so
    there the bound is one grid step of the reference value: two roundings of
    values that differ in their last bits can land one step apart."""
    d = np.abs(got - want)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    lim = np.maximum(OUT_MAX_ABS, bf16_ulp(want)) if ulp_floor else OUT_MAX_ABS
    excess = d - lim
    assert excess.max() <= 0, f"{what}: max_abs {d.max():.3e} (worst excess over the bound {excess.max():.3e})"
    assert d.mean() <= OUT_MEAN_ABS, f"{what}: mean_abs {d.mean():.3e}"


def assert_lse_close(got: np.ndarray, want: np.ndarray, what: str = "lse"):
    gi, wi = np.isneginf(got), np.isneginf(want)
    assert np.array_equal(gi, wi), f"{what}: -inf positions differ ({gi.sum()} vs {wi.sum()})"
    assert not np.any(np.isnan(got)), f"{what}: NaN"
    if (~wi).any():
        d = np.abs(got[~wi].astype(np.float64) - want[~wi].astype(np.float64))
        assert d.max() <= LSE_ABS, f"{what}: max_abs {d.max():.3e}"
