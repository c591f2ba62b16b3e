"""Python binding of libsmla -- sparse MLA attention for AMD MI355X.

A thin ctypes layer over the C ABI in include/smla.h: it only checks dtypes,
devices and the shapes the kernels read from and write to, reads pointers
and strides off torch tensors, allocates outputs when the caller passes
none, and calls the library on the current HIP stream.  Every step of the
computation runs in the HIP kernels of libsmla.so; there is no fallback, and
a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["KVPool", "quantize_kv", "prefill", "decode", "combine", "split_width", "row_bytes",
           "query_dims", "value_dims", "library_path", "SmlaError", "FMT_BF16", "FMT_FP8", "FMT_INT8",
           "FMT_FP8_ANY", "FMT_FP8_NOPE", "FMT_FP8_DOTS3", "FMT_FP8_DSV4"]

FMT_BF16, FMT_FP8, FMT_INT8, FMT_FP8_ANY, FMT_FP8_NOPE, FMT_FP8_DOTS3, FMT_FP8_DSV4 = 0, 1, 2, 3, 4, 5, 6
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsmla.so")
_lib = None


class SmlaError(RuntimeError):
    pass


class _Pool(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("num_blocks", ctypes.c_int64),
                ("block_stride_bytes", ctypes.c_int64), ("page_block", ctypes.c_int32),
                ("format", ctypes.c_int32), ("row_stride_bytes", ctypes.c_int64)]


class _Extra(ctypes.Structure):
    _fields_ = [("kv", _Pool), ("indices", ctypes.c_void_p), ("topk", ctypes.c_int32),
                ("idx_stride_t", ctypes.c_int64), ("topk_length", ctypes.c_void_p)]


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise SmlaError(f"{_LIB_PATH} is missing: build it with "
                        "`python -m sparse_top_mla_smla_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(_LIB_PATH)
    P, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    L.smla_row_bytes.argtypes, L.smla_row_bytes.restype = [i32], i32
    L.smla_split_width.argtypes, L.smla_split_width.restype = [i32, i32], i32
    L.smla_query_dims.argtypes, L.smla_query_dims.restype = [i32], i32
    L.smla_value_dims.argtypes, L.smla_value_dims.restype = [i32], i32
    L.smla_decode_workspace_size.argtypes = [i64, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.smla_decode_workspace_size.restype = ctypes.c_int
    L.smla_last_error.argtypes, L.smla_last_error.restype = [], ctypes.c_char_p
    L.smla_version.argtypes, L.smla_version.restype = [], ctypes.c_char_p
    L.smla_quantize_kv.argtypes = [P, i64, i64, P, _Pool, P]
    L.smla_prefill.argtypes = [P, i64, i32, i64, i64, _Pool, P, i32, i64, P, P, f32, P, i64, i64,
                               P, i64, P]
    L.smla_decode.argtypes = [P, i64, i32, i64, i64, _Pool, P, i32, i64, P, f32, i32, P, P, P]
    L.smla_combine.argtypes = [P, P, i64, i32, i32, i32, P, P, i64, i64, P, i64, P]
    L.smla_split_model_cost.argtypes = [i64, i32, i32, i32, i32, i32]
    L.smla_split_model_cost.restype = ctypes.c_double
    L.smla_decode_num_splits.argtypes, L.smla_decode_num_splits.restype = [i64, i32, i32, i32, i32], i32
    L.smla_use_split_form.argtypes, L.smla_use_split_form.restype = [i64, i32, i32, i32, i32], i32
    L.smla_attention_workspace_size.argtypes = [i64, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.smla_attention_workspace_size.restype = ctypes.c_int
    L.smla_attention.argtypes = [P, i64, i32, i64, i64, _Pool, P, i32, i64, P, P, f32, P, i64, i64,
                                 P, i64, P, ctypes.c_size_t, P]
    L.smla_attention_noalloc.argtypes = [P, i64, i32, i64, i64, _Pool, P, i32, i64, P, P, f32, P, i64, i64,
                                         P, i64, P]
    L.smla_probe_gather.argtypes = [_Pool, P, i64, i32, i64, P, P, P]
    L.smla_probe_clock.argtypes = [P, i32, i32, P]
    L.smla_device_attributes.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    PE = ctypes.POINTER(_Extra)
    L.smla_prefill_dual.argtypes = [P, i64, i32, i64, i64, _Pool, P, i32, i64, P, PE, P, f32, P, i64, i64,
                                    P, i64, P]
    L.smla_decode_dual.argtypes = [P, i64, i32, i64, i64, _Pool, P, i32, i64, P, PE, f32, i32, P, P, P]
    for fn in (L.smla_quantize_kv, L.smla_prefill, L.smla_decode, L.smla_combine, L.smla_attention,
               L.smla_attention_noalloc, L.smla_prefill_dual, L.smla_decode_dual, L.smla_probe_gather,
               L.smla_probe_clock, L.smla_device_attributes):
        fn.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = _load().smla_last_error().decode()
        raise SmlaError(f"{what}: status {status}: {msg}")


def row_bytes(fmt: int) -> int:
    return int(_load().smla_row_bytes(fmt))


def query_dims(fmt: int) -> int:
    """Values per q row (and per latent row the writer reads) for a format."""
    return int(_load().smla_query_dims(fmt))


def value_dims(fmt: int) -> int:
    """Values per output row (d_v) for a format."""
    return int(_load().smla_value_dims(fmt))


def split_width(topk: int, num_splits: int) -> int:
    return int(_load().smla_split_width(topk, num_splits))


def decode_workspace_size(T: int, H: int, num_splits: int, d_v: int = 512) -> int:
    """Bytes of decode scratch (part_out then part_lse) for T tokens."""
    n = ctypes.c_size_t(0)
    _check(_load().smla_decode_workspace_size(T, H, num_splits, d_v, ctypes.byref(n)), "smla_decode_workspace_size")
    return int(n.value)


def split_model_cost(T: int, H: int, topk: int, fmt: int, num_splits: int, compute_units: int = 0) -> float:
    """Predicted microseconds of decode + combine at num_splits, or of the
    prefill form when num_splits == 0 (see smla_split_model_cost); -1 on
    argument errors."""
    return float(_load().smla_split_model_cost(T, H, topk, fmt, num_splits, compute_units))


def decode_num_splits(T: int, H: int, topk: int, fmt: int, compute_units: int = 0) -> int:
    """Split count the model picks for smla_decode (-1 on argument errors)."""
    return int(_load().smla_decode_num_splits(T, H, topk, fmt, compute_units))


def use_split_form(T: int, H: int, topk: int, fmt: int, compute_units: int = 0) -> int:
    """1 when the model routes this shape to the split form, 0 to prefill."""
    return int(_load().smla_use_split_form(T, H, topk, fmt, compute_units))


def attention_workspace_size(T: int, H: int, topk: int, fmt: int) -> int:
    """Bytes of workspace smla_attention uses for this shape (0: prefill form)."""
    n = ctypes.c_size_t(0)
    _check(_load().smla_attention_workspace_size(T, H, topk, fmt, ctypes.byref(n)),
           "smla_attention_workspace_size")
    return int(n.value)


def version() -> str:
    return _load().smla_version().decode()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype, last_contig: bool = True):
    if t.dtype != dtype:
        raise SmlaError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise SmlaError(f"{name} must be a GPU tensor")
    if last_contig and t.dim() > 0 and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise SmlaError(f"{name}: the last dimension must be contiguous")


def _shape(t: torch.Tensor, name: str, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise SmlaError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_common(q: torch.Tensor, pool: "KVPool", indices: torch.Tensor, topk: int,
                  topk_length: Optional[torch.Tensor], sink: Optional[torch.Tensor]) -> None:
    """Sizes the kernels read from: q rows, index rows, lengths and sinks."""
    if q.dim() != 3:
        raise SmlaError(f"q must be [T, H, D], got {tuple(q.shape)}")
    T, H, D = q.shape
    if D < query_dims(pool.fmt):
        raise SmlaError(f"q rows hold {D} values; this format needs {query_dims(pool.fmt)}")
    if indices.dim() != 2 or indices.shape[0] < T:
        raise SmlaError(f"indices must be [>= T, >= topk] = [>= {T}, >= {topk}], got {tuple(indices.shape)}")
    if topk > indices.shape[1]:
        raise SmlaError(f"topk {topk} exceeds the index rows' {indices.shape[1]} columns")
    if topk_length is not None:
        _need(topk_length, "topk_length", torch.int32)
        if topk_length.numel() < T:
            raise SmlaError(f"topk_length holds {topk_length.numel()} entries for {T} tokens")
    if sink is not None:
        _need(sink, "sink", torch.float32)
        if sink.numel() < H:
            raise SmlaError(f"sink holds {sink.numel()} entries for {H} heads")


class KVPool:
    """A paged latent pool: a uint8 device tensor [num_blocks, block_stride]
    (block_stride >= 64 * row stride, multiple of 16) in format fmt, rows
    row_stride bytes apart within a block (0: dense rows of row_bytes)."""

    def __init__(self, data: torch.Tensor, fmt: int, page_block: int = 64, row_stride: int = 0):
        _need(data, "pool", torch.uint8)
        if data.dim() != 2:
            raise SmlaError("pool must be 2-D [num_blocks, block_stride_bytes]")
        self.data, self.fmt, self.page_block, self.row_stride = data, fmt, page_block, row_stride

    @classmethod
    def empty(cls, num_blocks: int, fmt: int, device="cuda", block_stride: int = 0,
              row_stride: int = 0) -> "KVPool":
        bs = block_stride or 64 * (row_stride or row_bytes(fmt))
        return cls(torch.zeros((num_blocks, bs), dtype=torch.uint8, device=device), fmt, row_stride=row_stride)

    @property
    def num_blocks(self) -> int:
        return self.data.shape[0]

    def c(self) -> _Pool:
        return _Pool(self.data.data_ptr(), self.data.shape[0], self.data.stride(0), self.page_block,
                     self.fmt, self.row_stride)


def quantize_kv(kv: torch.Tensor, slots: torch.Tensor, pool: KVPool, stream=None) -> None:
    """Write BF16 latent rows kv [n, >=query_dims] into pool slots (see smla_quantize_kv)."""
    _need(kv, "kv", torch.bfloat16)
    _need(slots, "slots", torch.int32)
    n = kv.shape[0]
    _check(_load().smla_quantize_kv(_ptr(kv), n, kv.stride(0) if n else query_dims(pool.fmt), _ptr(slots), pool.c(),
                                    _stream(stream)), "smla_quantize_kv")


def _idx_args(indices: torch.Tensor, topk: Optional[int]):
    _need(indices, "indices", torch.int32)
    topk = indices.shape[1] if topk is None else topk
    return topk, indices.stride(0)


def _outputs(q: torch.Tensor, pool: KVPool, out: Optional[torch.Tensor], lse: Optional[torch.Tensor]):
    """out [T, H, d_v] bf16 and lse [T, H] f32 (allocated when not given)."""
    T, H = q.shape[0], q.shape[1]
    dv = value_dims(pool.fmt)
    if out is None:
        out = torch.empty((T, H, dv), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16)
    _need(lse, "lse", torch.float32)
    _shape(out, "out", (T, H, dv))
    _shape(lse, "lse", (T, H))
    return out, lse


def _partials(q: torch.Tensor, pool: KVPool, num_splits: int, part_out: Optional[torch.Tensor],
              part_lse: Optional[torch.Tensor]):
    """part_out [T, S, H, d_v] and part_lse [T, S, H], f32, contiguous."""
    T, H = q.shape[0], q.shape[1]
    dv = value_dims(pool.fmt)
    if part_out is None:
        part_out = torch.empty((T, num_splits, H, dv), dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((T, num_splits, H), dtype=torch.float32, device=q.device)
    _need(part_out, "part_out", torch.float32)
    _need(part_lse, "part_lse", torch.float32)
    if not (part_out.is_contiguous() and part_lse.is_contiguous()):
        raise SmlaError("part_out / part_lse must be contiguous")
    _shape(part_out, "part_out", (T, num_splits, H, dv))
    _shape(part_lse, "part_lse", (T, num_splits, H))
    return part_out, part_lse


def prefill(q: torch.Tensor, pool: KVPool, indices: torch.Tensor, topk: Optional[int] = None,
            topk_length: Optional[torch.Tensor] = None, sink: Optional[torch.Tensor] = None,
            sm_scale: float = 1.0 / 24.0, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Sparse MLA prefill (see smla_prefill).  q [T,H,query_dims] bf16 (strided
    views allowed), indices [T, >=topk] int32.  Returns (out [T,H,value_dims]
    bf16, lse [T,H] f32)."""
    _need(q, "q", torch.bfloat16)
    T, H, _ = q.shape
    topk, ist = _idx_args(indices, topk)
    _check_common(q, pool, indices, topk, topk_length, sink)
    out, lse = _outputs(q, pool, out, lse)
    _check(_load().smla_prefill(_ptr(q), T, H, q.stride(0), q.stride(1), pool.c(), _ptr(indices), topk,
                                ist, _ptr(topk_length), _ptr(sink), float(sm_scale), _ptr(out),
                                out.stride(0), out.stride(1), _ptr(lse), lse.stride(0),
                                _stream(stream)), "smla_prefill")
    return out, lse


def decode(q: torch.Tensor, pool: KVPool, indices: torch.Tensor, num_splits: int,
           topk: Optional[int] = None, topk_length: Optional[torch.Tensor] = None,
           sm_scale: float = 1.0 / 24.0, part_out: Optional[torch.Tensor] = None,
           part_lse: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-KV decode partials (see smla_decode).  Returns part_out
    [T,S,H,value_dims] f32 and part_lse [T,S,H] f32."""
    _need(q, "q", torch.bfloat16)
    T, H, _ = q.shape
    topk, ist = _idx_args(indices, topk)
    _check_common(q, pool, indices, topk, topk_length, None)
    part_out, part_lse = _partials(q, pool, num_splits, part_out, part_lse)
    _check(_load().smla_decode(_ptr(q), T, H, q.stride(0), q.stride(1), pool.c(), _ptr(indices), topk,
                               ist, _ptr(topk_length), float(sm_scale), num_splits, _ptr(part_out),
                               _ptr(part_lse), _stream(stream)), "smla_decode")
    return part_out, part_lse


def combine(part_out: torch.Tensor, part_lse: torch.Tensor, sink: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
            stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """LSE combine of decode splits (see smla_combine)."""
    _need(part_out, "part_out", torch.float32)
    _need(part_lse, "part_lse", torch.float32)
    if not (part_out.is_contiguous() and part_lse.is_contiguous()):
        raise SmlaError("part_out / part_lse must be contiguous")
    if part_out.dim() != 4:
        raise SmlaError(f"part_out must be [T, S, H, d_v], got {tuple(part_out.shape)}")
    T, S, H, dv = part_out.shape
    _shape(part_lse, "part_lse", (T, S, H))
    if sink is not None:
        _need(sink, "sink", torch.float32)
        if sink.numel() < H:
            raise SmlaError(f"sink holds {sink.numel()} entries for {H} heads")
    if out is None:
        out = torch.empty((T, H, dv), dtype=torch.bfloat16, device=part_out.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=part_out.device)
    _need(out, "out", torch.bfloat16)
    _need(lse, "lse", torch.float32)
    _shape(out, "out", (T, H, dv))
    _shape(lse, "lse", (T, H))
    _check(_load().smla_combine(_ptr(part_out), _ptr(part_lse), T, S, H, dv, _ptr(sink), _ptr(out),
                                out.stride(0), out.stride(1), _ptr(lse), lse.stride(0),
                                _stream(stream)), "smla_combine")
    return out, lse


def attention(q: torch.Tensor, pool: KVPool, indices: torch.Tensor, topk: Optional[int] = None,
              topk_length: Optional[torch.Tensor] = None, sink: Optional[torch.Tensor] = None,
              sm_scale: float = 1.0 / 24.0, out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Prefill-form result by the form the split-count model picks (see
    smla_attention).  workspace: a uint8 device tensor of at least
    attention_workspace_size bytes, or None (then the prefill form runs)."""
    _need(q, "q", torch.bfloat16)
    T, H, _ = q.shape
    topk, ist = _idx_args(indices, topk)
    _check_common(q, pool, indices, topk, topk_length, sink)
    out, lse = _outputs(q, pool, out, lse)
    ws_bytes = 0
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise SmlaError("workspace must be a contiguous uint8 tensor")
        ws_bytes = workspace.numel()
    _check(_load().smla_attention(_ptr(q), T, H, q.stride(0), q.stride(1), pool.c(), _ptr(indices), topk,
                                  ist, _ptr(topk_length), _ptr(sink), float(sm_scale), _ptr(out),
                                  out.stride(0), out.stride(1), _ptr(lse), lse.stride(0), _ptr(workspace),
                                  ws_bytes, _stream(stream)), "smla_attention")
    return out, lse


def attention_noalloc(q: torch.Tensor, pool: KVPool, indices: torch.Tensor, topk: Optional[int] = None,
                      topk_length: Optional[torch.Tensor] = None, sink: Optional[torch.Tensor] = None,
                      sm_scale: float = 1.0 / 24.0, out: Optional[torch.Tensor] = None,
                      lse: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """smla_attention with its decode partials in the library's static
    device scratch (see smla_attention_noalloc): the library allocates
    nothing; pass out and lse to allocate nothing here either."""
    _need(q, "q", torch.bfloat16)
    T, H, _ = q.shape
    topk, ist = _idx_args(indices, topk)
    _check_common(q, pool, indices, topk, topk_length, sink)
    out, lse = _outputs(q, pool, out, lse)
    _check(_load().smla_attention_noalloc(_ptr(q), T, H, q.stride(0), q.stride(1), pool.c(), _ptr(indices), topk,
                                          ist, _ptr(topk_length), _ptr(sink), float(sm_scale), _ptr(out),
                                          out.stride(0), out.stride(1), _ptr(lse), lse.stride(0), _stream(stream)),
           "smla_attention_noalloc")
    return out, lse


def _extra(T: int, pool: KVPool, indices: torch.Tensor, topk: Optional[int], topk_length: Optional[torch.Tensor]):
    topk, ist = _idx_args(indices, topk)
    if indices.dim() != 2 or indices.shape[0] < T or topk > indices.shape[1]:
        raise SmlaError(f"extra_indices must be [>= {T}, >= {topk}], got {tuple(indices.shape)}")
    if topk_length is not None:
        _need(topk_length, "extra_topk_length", torch.int32)
        if topk_length.numel() < T:
            raise SmlaError(f"extra_topk_length holds {topk_length.numel()} entries for {T} tokens")
    return _Extra(pool.c(), _ptr(indices), topk, ist, _ptr(topk_length))


def prefill_dual(q: torch.Tensor, pool: KVPool, indices: torch.Tensor, extra_pool: KVPool,
                 extra_indices: torch.Tensor, topk: Optional[int] = None, extra_topk: Optional[int] = None,
                 topk_length: Optional[torch.Tensor] = None, extra_topk_length: Optional[torch.Tensor] = None,
                 sink: Optional[torch.Tensor] = None, sm_scale: float = 1.0 / 24.0,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Prefill over a main and a secondary candidate list (see smla_prefill_dual)."""
    _need(q, "q", torch.bfloat16)
    T, H, _ = q.shape
    topk, ist = _idx_args(indices, topk)
    _check_common(q, pool, indices, topk, topk_length, sink)
    ex = _extra(T, extra_pool, extra_indices, extra_topk, extra_topk_length)
    out, lse = _outputs(q, pool, out, lse)
    _check(_load().smla_prefill_dual(_ptr(q), T, H, q.stride(0), q.stride(1), pool.c(), _ptr(indices), topk, ist,
                                     _ptr(topk_length), ctypes.byref(ex), _ptr(sink), float(sm_scale), _ptr(out),
                                     out.stride(0), out.stride(1), _ptr(lse), lse.stride(0), _stream(stream)),
           "smla_prefill_dual")
    return out, lse


def decode_dual(q: torch.Tensor, pool: KVPool, indices: torch.Tensor, extra_pool: KVPool,
                extra_indices: torch.Tensor, num_splits: int, topk: Optional[int] = None,
                extra_topk: Optional[int] = None, topk_length: Optional[torch.Tensor] = None,
                extra_topk_length: Optional[torch.Tensor] = None, sm_scale: float = 1.0 / 24.0,
                part_out: Optional[torch.Tensor] = None, part_lse: Optional[torch.Tensor] = None,
                stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-KV decode partials over a main and a secondary list (see smla_decode_dual)."""
    _need(q, "q", torch.bfloat16)
    T, H, _ = q.shape
    topk, ist = _idx_args(indices, topk)
    _check_common(q, pool, indices, topk, topk_length, None)
    ex = _extra(T, extra_pool, extra_indices, extra_topk, extra_topk_length)
    part_out, part_lse = _partials(q, pool, num_splits, part_out, part_lse)
    _check(_load().smla_decode_dual(_ptr(q), T, H, q.stride(0), q.stride(1), pool.c(), _ptr(indices), topk, ist,
                                    _ptr(topk_length), ctypes.byref(ex), float(sm_scale), num_splits,
                                    _ptr(part_out), _ptr(part_lse), _stream(stream)), "smla_decode_dual")
    return part_out, part_lse


# ---- measurement aids (not steps of the attention path) ----

def probe_gather(pool: KVPool, indices: torch.Tensor, topk: Optional[int] = None,
                 topk_length: Optional[torch.Tensor] = None, rows_out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """Moves every candidate row of each token's list into LDS as the
    attention kernels gather them, computing nothing (see smla_probe_gather);
    returns the rows moved per token (int32 view of uint32 [T])."""
    topk, ist = _idx_args(indices, topk)
    T = indices.shape[0]
    if topk > indices.shape[1]:
        raise SmlaError(f"topk {topk} exceeds the index rows' {indices.shape[1]} columns")
    if topk_length is not None:
        _need(topk_length, "topk_length", torch.int32)
        if topk_length.numel() < T:
            raise SmlaError(f"topk_length holds {topk_length.numel()} entries for {T} tokens")
    if rows_out is None:
        rows_out = torch.empty(T, dtype=torch.int32, device=indices.device)
    _need(rows_out, "rows_out", torch.int32)
    _shape(rows_out, "rows_out", (T,))
    _check(_load().smla_probe_gather(pool.c(), _ptr(indices), T, topk, ist, _ptr(topk_length), _ptr(rows_out),
                                     _stream(stream)), "smla_probe_gather")
    return rows_out


def probe_clock(blocks: int, iters: int, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Shader-clock cycles and constant-rate ticks per workgroup around an
    MFMA loop (see smla_probe_clock): int64 [blocks, 2] on the device."""
    if out is None:
        out = torch.empty((blocks, 2), dtype=torch.int64, device="cuda")
    _need(out, "out", torch.int64)
    _shape(out, "out", (blocks, 2))
    _check(_load().smla_probe_clock(_ptr(out), blocks, iters, _stream(stream)), "smla_probe_clock")
    return out


def device_attributes() -> dict:
    """Compute units, peak shader clock, constant-rate clock and memory clock
    (kHz) and memory bus width (bits) of the current device."""
    a = (ctypes.c_int32 * 5)()
    _check(_load().smla_device_attributes(a), "smla_device_attributes")
    return {"compute_units": a[0], "clock_khz": a[1], "wall_clock_khz": a[2], "memory_clock_khz": a[3],
            "memory_bus_bits": a[4]}

