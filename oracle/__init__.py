"""CPU oracle for sparse MLA attention (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it shares no code
with that path.

The arithmetic lives in ``smla_oracle.c`` (plain C, float64 attention,
float32 quantizer).  This module only compiles it with gcc and marshals numpy
arrays through ctypes.  Every function cites the passage it follows in the C
source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "smla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

FMT_BF16, FMT_FP8, FMT_INT8, FMT_FP8_ANY, FMT_FP8_NOPE, FMT_FP8_DOTS3, FMT_FP8_DSV4 = 0, 1, 2, 3, 4, 5, 6
PAGE_BLOCK = 64


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
             "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        L.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        L.oracle_double_to_bf16.restype = ctypes.c_uint16
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [f32]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_fp8_scale.argtypes = [f32]
        L.oracle_fp8_scale.restype = f32
        L.oracle_int8_scale.argtypes = [f32]
        L.oracle_int8_scale.restype = f32
        L.oracle_int8_encode.argtypes = [f32, f32]
        L.oracle_int8_encode.restype = ctypes.c_int8
        L.oracle_row_bytes.argtypes = [i32]
        L.oracle_row_bytes.restype = i32
        L.oracle_d_k.argtypes = [i32]
        L.oracle_d_k.restype = i32
        L.oracle_d_v.argtypes = [i32]
        L.oracle_d_v.restype = i32
        L.oracle_e8m0_scale.argtypes = [f32]
        L.oracle_e8m0_scale.restype = ctypes.c_uint8
        L.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0_decode.restype = ctypes.c_double
        L.oracle_split_width.argtypes = [i32, i32]
        L.oracle_split_width.restype = i32
        L.oracle_quantize_kv.argtypes = [P, i64, i64, P, P, i64, i64, i32]
        L.oracle_dequant_rows.argtypes = [P, i64, i32, P, i64, P]
        L.oracle_prefill.argtypes = [P, i64, i32, i64, i64, P, i64, i64, i32, P, i32, i64, P, P, f32,
                                     P, i64, i64, P, i64, P, P, P, i64, ctypes.c_int]
        L.oracle_decode_split.argtypes = [P, i64, i32, i64, i64, P, i64, i64, i32, P, i32, i64, P,
                                          f32, i32, P, P, P, i64, ctypes.c_int]
        L.oracle_combine.argtypes = [P, P, i64, i32, i32, i32, P, P, i64, i64, P, i64, P, P, P, i64]
        L.oracle_probs.argtypes = [P, i64, i32, i64, i64, P, i64, i64, i32, P, i32, i64, P, P, f32,
                                   i64, i32, P, P]
        for name in ("oracle_quantize_kv", "oracle_prefill", "oracle_decode_split",
                     "oracle_combine", "oracle_probs"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _elem_strides(a: np.ndarray):
    return tuple(s // a.itemsize for s in a.strides)


def row_bytes(fmt: int) -> int:
    return int(lib().oracle_row_bytes(fmt))


def d_k(fmt: int) -> int:
    """Elements of a dequantized K row (nope + rope)."""
    return int(lib().oracle_d_k(fmt))


def d_v(fmt: int) -> int:
    """Elements of a V row (K's first d_v values): 1024 for DOTS3_SWA rows, else 512."""
    return int(lib().oracle_d_v(fmt))


def e8m0_scale(amax: float) -> int:
    """DOTS3_SWA tile scale byte (see oracle_e8m0_scale)."""
    return int(lib().oracle_e8m0_scale(amax))


def e8m0_decode(b: int) -> float:
    return float(lib().oracle_e8m0_decode(b))


def split_width(topk: int, num_splits: int) -> int:
    return int(lib().oracle_split_width(topk, num_splits))


def e4m3_decode(code: int) -> float:
    return float(lib().oracle_e4m3_decode(code))


def e4m3_encode(y: float) -> int:
    return int(lib().oracle_e4m3_encode(y))


def fp8_scale(amax: float) -> float:
    return float(lib().oracle_fp8_scale(amax))


def int8_scale(amax: float) -> float:
    return float(lib().oracle_int8_scale(amax))


def int8_encode(x: float, scale: float) -> int:
    return int(lib().oracle_int8_encode(x, scale))


def double_to_bf16(x: float) -> int:
    return int(lib().oracle_double_to_bf16(x))


class Pool:
    """A host copy of a paged latent pool: raw bytes [num_blocks, block_stride]."""

    def __init__(self, data: np.ndarray, fmt: int, block_stride: int):
        assert data.dtype == np.uint8 and data.ndim == 2 and data.flags.c_contiguous
        self.data, self.fmt, self.block_stride = data, fmt, block_stride

    @property
    def num_blocks(self) -> int:
        return self.data.shape[0]


def quantize_kv(kv_bf16: np.ndarray, slots: np.ndarray, pool: Pool) -> None:
    """Write latent rows into the pool (FlashInfer PR #4802 review: 656-byte
    DSv3.2 row layout; see smla_oracle.c).  kv_bf16: uint16 [n, >=d_k] rows."""
    assert kv_bf16.dtype == np.uint16 and kv_bf16.strides[1] == 2
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    n = kv_bf16.shape[0]
    lib().oracle_quantize_kv(_ptr(kv_bf16), n, kv_bf16.strides[0] // 2, _ptr(slots),
                             _ptr(pool.data), pool.num_blocks, pool.block_stride, pool.fmt)


def dequant_rows(pool: Pool, slots: np.ndarray) -> np.ndarray:
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    out = np.empty((slots.shape[0], d_k(pool.fmt)), dtype=np.float64)
    lib().oracle_dequant_rows(_ptr(pool.data), pool.block_stride, pool.fmt, _ptr(slots),
                              slots.shape[0], _ptr(out))
    return out


def _check_q(q):
    assert q.dtype == np.uint16 and q.ndim == 3 and q.strides[2] == 2
    st = _elem_strides(q)
    return st[0], st[1]


def _check_idx(indices):
    assert indices.dtype == np.int32 and indices.ndim == 2 and indices.strides[1] == 4
    return indices.strides[0] // 4


def prefill(q, pool: Pool, indices, topk_length=None, sink=None, sm_scale=1.0 / 24.0,
            tokens=None, nthreads: int = 0):
    """Prefill form (see oracle_prefill).  q: uint16 (bf16 bits) [T,H,d_k]
    (any strides, last dim contiguous); indices: int32 [T, >=topk] with
    last dim contiguous.  Returns (out_bf16 uint16 [T,H,d_v], lse f32 [T,H],
    out_f64 [T,H,d_v], lse_f64 [T,H]); rows of tokens not in `tokens` are
    left zero."""
    T, H, _ = q.shape
    qst, qsh = _check_q(q)
    ist = _check_idx(indices)
    topk = indices.shape[1]
    tl = None if topk_length is None else np.ascontiguousarray(topk_length, dtype=np.int32)
    sk = None if sink is None else np.ascontiguousarray(sink, dtype=np.float32)
    dv = d_v(pool.fmt)
    out = np.zeros((T, H, dv), dtype=np.uint16)
    lse = np.zeros((T, H), dtype=np.float32)
    of = np.zeros((T, H, dv), dtype=np.float64)
    lf = np.zeros((T, H), dtype=np.float64)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    rc = lib().oracle_prefill(_ptr(q), T, H, qst, qsh, _ptr(pool.data), pool.num_blocks,
                              pool.block_stride, pool.fmt, _ptr(indices), topk, ist, _ptr(tl),
                              _ptr(sk), float(sm_scale), _ptr(out), H * dv, dv, _ptr(lse), H,
                              _ptr(of), _ptr(lf), _ptr(tok), 0 if tok is None else tok.shape[0],
                              nthreads)
    assert rc == 0
    return out, lse, of, lf


def decode_split(q, pool: Pool, indices, num_splits: int, topk_length=None, sm_scale=1.0 / 24.0,
                 tokens=None, nthreads: int = 0):
    """Decode split form (see oracle_decode_split).  Returns float64
    part_out [T,S,H,d_v] and part_lse [T,S,H]."""
    T, H, _ = q.shape
    qst, qsh = _check_q(q)
    ist = _check_idx(indices)
    topk = indices.shape[1]
    tl = None if topk_length is None else np.ascontiguousarray(topk_length, dtype=np.int32)
    po = np.zeros((T, num_splits, H, d_v(pool.fmt)), dtype=np.float64)
    pl = np.zeros((T, num_splits, H), dtype=np.float64)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    rc = lib().oracle_decode_split(_ptr(q), T, H, qst, qsh, _ptr(pool.data), pool.num_blocks,
                                   pool.block_stride, pool.fmt, _ptr(indices), topk, ist, _ptr(tl),
                                   float(sm_scale), num_splits, _ptr(po), _ptr(pl), _ptr(tok),
                                   0 if tok is None else tok.shape[0], nthreads)
    assert rc == 0
    return po, pl


def combine(part_out, part_lse, sink=None, tokens=None):
    """LSE combine (see oracle_combine).  Returns (out_bf16, lse_f32, out_f64, lse_f64)."""
    part_out = np.ascontiguousarray(part_out, dtype=np.float64)
    part_lse = np.ascontiguousarray(part_lse, dtype=np.float64)
    T, S, H, dv = part_out.shape
    sk = None if sink is None else np.ascontiguousarray(sink, dtype=np.float32)
    out = np.zeros((T, H, dv), dtype=np.uint16)
    lse = np.zeros((T, H), dtype=np.float32)
    of = np.zeros((T, H, dv), dtype=np.float64)
    lf = np.zeros((T, H), dtype=np.float64)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    rc = lib().oracle_combine(_ptr(part_out), _ptr(part_lse), T, S, H, dv, _ptr(sk), _ptr(out), H * dv,
                              dv, _ptr(lse), H, _ptr(of), _ptr(lf), _ptr(tok),
                              0 if tok is None else tok.shape[0])
    assert rc == 0
    return out, lse, of, lf


def probs(q, pool: Pool, indices, t: int, h: int, topk_length=None, sink=None,
          sm_scale=1.0 / 24.0):
    """Per-entry softmax probabilities of one (token, head) and the sink's share."""
    T, H, _ = q.shape
    qst, qsh = _check_q(q)
    ist = _check_idx(indices)
    topk = indices.shape[1]
    tl = None if topk_length is None else np.ascontiguousarray(topk_length, dtype=np.int32)
    sk = None if sink is None else np.ascontiguousarray(sink, dtype=np.float32)
    p = np.zeros(topk, dtype=np.float64)
    ps = np.zeros(1, dtype=np.float64)
    rc = lib().oracle_probs(_ptr(q), T, H, qst, qsh, _ptr(pool.data), pool.num_blocks,
                            pool.block_stride, pool.fmt, _ptr(indices), topk, ist, _ptr(tl),
                            _ptr(sk), float(sm_scale), t, h, _ptr(p), _ptr(ps))
    assert rc == 0
    return p, float(ps[0])
