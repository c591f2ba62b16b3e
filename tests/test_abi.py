"""The C ABI without a GPU: libsmla.so loads, exports every function
include/smla.h declares, and its host-side logic (sizes, split geometry,
argument validation that returns before any launch) behaves as declared."""
import ctypes
import os
import re

import pytest

import sparse_top_mla_smla_amd as smla
from sparse_top_mla_smla_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smla.h")

# fake device addresses: validation never dereferences them, and every call
# below returns before launching anything
FAKE = 0x10000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smla_[a-z_0-9]+)\s*\(", text)))


def exported_functions():
    lib = smla._load()
    names = []
    for name in declared_functions():
        try:
            getattr(lib, name)
            names.append(name)
        except AttributeError:
            pass
    return names


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("smla_quantize_kv", "smla_prefill", "smla_decode", "smla_combine",
                     "smla_decode_workspace_size", "smla_split_width", "smla_row_bytes",
                     "smla_last_error", "smla_version"):
        assert required in names


def test_library_exports_every_declared_function():
    assert exported_functions() == declared_functions()


def test_row_bytes_and_version():
    assert smla.row_bytes(W.FMT_BF16) == 1152
    assert smla.row_bytes(W.FMT_FP8) == 656
    assert smla.row_bytes(W.FMT_INT8) == 656
    assert smla.row_bytes(W.FMT_FP8_DOTS3) == 1160
    assert smla.row_bytes(W.FMT_FP8_DSV4) == 584
    assert smla.row_bytes(7) == -1
    assert "gfx950" in smla.version()


def test_query_and_value_dims():
    for f in W.FMT_NAMES:
        assert smla.query_dims(f) == W.Q_DIMS[f]
        assert smla.value_dims(f) == W.V_DIMS[f]
    assert smla.query_dims(9) == -1 and smla.value_dims(9) == -1


@pytest.mark.parametrize("topk,S,w", [(2048, 8, 256), (64, 2, 64), (1000, 7, 192), (1, 64, 64), (640, 3, 256)])
def test_split_width(topk, S, w):
    assert smla.split_width(topk, S) == w


def test_split_width_rejects_bad_arguments():
    assert smla.split_width(0, 4) == -1
    assert smla.split_width(64, 0) == -1


def test_decode_workspace_size():
    T, H, S = 64, 64, 8
    assert smla.decode_workspace_size(T, H, S) == T * S * H * 512 * 4 + T * S * H * 4
    assert smla.decode_workspace_size(T, H, S, 1024) == T * S * H * 1024 * 4 + T * S * H * 4
    assert smla.decode_workspace_size(0, 8, 1) == 0
    for bad in ((-1, 8, 1), (1, 0, 1), (1, 129, 1), (1, 8, 0), (1, 8, 65), (1, 8, 1, 576)):
        with pytest.raises(smla.SmlaError):
            smla.decode_workspace_size(*bad)
    lib = smla._load()
    assert lib.smla_decode_workspace_size(1, 8, 1, 512, None) == 1  # SMLA_ERR_NULL


def pool(fmt=W.FMT_FP8, num_blocks=4, page_block=64, block_stride=None, row_stride=0):
    rb = W.ROW_BYTES.get(fmt, 656)
    bs = block_stride if block_stride is not None else 64 * (row_stride or rb)
    return smla._Pool(FAKE, num_blocks, bs, page_block, fmt, row_stride)


def prefill(lib, T=2, H=64, q=FAKE, pl=None, idx=FAKE, topk=64, q_st=64 * 576, q_sh=576, out=FAKE, lse=FAKE,
            idx_st=64):
    return lib.smla_prefill(q, T, H, q_st, q_sh, pl or pool(), idx, topk, idx_st, None, None,
                            ctypes.c_float(1 / 24), out, 64 * 512, 512, lse, 64, None)


def test_prefill_validation_before_launch():
    lib = smla._load()
    assert prefill(lib, T=0, q=None, idx=None, out=None, lse=None) == 0       # T = 0: nothing to do
    assert prefill(lib, q=None) == 1                                         # NULL q
    assert prefill(lib, idx=None) == 1
    assert prefill(lib, H=0) == 2                                            # H outside [1, 128]
    assert prefill(lib, H=129) == 4                                          # above what is built
    assert prefill(lib, topk=0) == 2
    assert prefill(lib, pl=pool(page_block=32)) == 4                         # page block must be 64
    assert "page_block 32" in lib.smla_last_error().decode()
    assert prefill(lib, pl=pool(fmt=7)) == 4                                 # unknown format
    assert prefill(lib, pl=pool(block_stride=64 * 656 - 16)) == 3            # block stride below 64 rows
    assert prefill(lib, pl=pool(row_stride=640)) == 3                        # row stride below the row
    assert prefill(lib, pl=pool(row_stride=664)) == 3                        # row stride not a multiple of 16
    assert prefill(lib, pl=pool(row_stride=672, block_stride=64 * 656)) == 3  # block stride below 64 padded rows
    assert "row_stride" in lib.smla_last_error().decode() or "64 rows" in lib.smla_last_error().decode()
    assert prefill(lib, q=FAKE + 8) == 3                                     # q not 16-byte aligned
    assert prefill(lib, idx_st=32) == 3                                      # index row stride < topk


def test_decode_and_combine_validation_before_launch():
    lib = smla._load()
    f = ctypes.c_float(1 / 24)
    ok_args = dict(q=FAKE, T=2, H=64, pl=pool(), idx=FAKE, topk=256, S=4, po=FAKE, pls=FAKE)

    def dec(**kw):
        a = dict(ok_args, **kw)
        return lib.smla_decode(a["q"], a["T"], a["H"], 64 * 576, 576, a["pl"], a["idx"], a["topk"], 256, None, f,
                               a["S"], a["po"], a["pls"], None)

    assert dec(S=0) == 4                                                     # num_splits outside 1..64
    assert dec(S=65) == 4
    assert dec(po=None) == 1
    assert dec(T=0, q=None, idx=None, po=None, pls=None) == 0
    assert lib.smla_combine(None, FAKE, 2, 4, 64, 512, None, FAKE, 64 * 512, 512, FAKE, 64, None) == 1
    assert lib.smla_combine(FAKE, FAKE, 0, 4, 64, 512, None, None, 0, 0, None, 0, None) == 0
    assert lib.smla_combine(FAKE, FAKE, 2, 4, 64, 768, None, FAKE, 64 * 1024, 1024, FAKE, 64, None) == 2
    assert lib.smla_combine(FAKE, FAKE, 2, 4, 64, 1024, None, FAKE, 64 * 512, 512, FAKE, 64, None) == 3


def test_dots3_validation_before_launch():
    lib = smla._load()
    f = ctypes.c_float(1 / 33)
    F = W.FMT_FP8_DOTS3

    def call(pl=None, q_sh=1088, out_sh=1024, ex=None):
        return lib.smla_prefill_dual(FAKE, 2, 16, 16 * q_sh, q_sh, pl or pool(fmt=F), FAKE, 576, 576, None,
                                     ctypes.byref(ex) if ex is not None else None, None, f, FAKE, 16 * out_sh,
                                     out_sh, FAKE, 16, None)

    assert call(q_sh=576) == 3                                               # q rows hold 1088 values
    assert call(out_sh=512) == 3                                             # out rows hold 1024 values
    assert call(pl=pool(fmt=F, row_stride=1164)) == 3                        # rows 8-byte aligned
    assert call(pl=pool(fmt=F, block_stride=64 * 1160 + 4)) == 3
    ex = smla._Extra(pool(fmt=W.FMT_FP8_DSV4), FAKE, 64, 64, None)
    assert call(ex=ex) == 4                                                  # secondary pool of another format
    assert "format" in lib.smla_last_error().decode()
    kv = lib.smla_quantize_kv(FAKE, 4, 576, FAKE, pool(fmt=F), None)
    assert kv == 3                                                           # writer reads 1088 values


def test_dual_validation_before_launch():
    lib = smla._load()
    f = ctypes.c_float(1 / 24)

    def extra(topk=64, idx=FAKE, fmt=W.FMT_FP8, idx_st=64, row_stride=0):
        return smla._Extra(pool(fmt=fmt, row_stride=row_stride), idx, topk, idx_st, None)

    def call(ex, topk=64, T=2):
        return lib.smla_prefill_dual(FAKE, T, 64, 64 * 576, 576, pool(), FAKE, topk, 64, None,
                                     ctypes.byref(ex) if ex is not None else None, None, f, FAKE, 64 * 512, 512,
                                     FAKE, 64, None)

    assert call(extra(), T=0) == 0
    assert call(extra(), topk=32) == 4                    # main width not a multiple of 64
    assert "multiple of 64" in lib.smla_last_error().decode()
    assert call(extra(topk=0)) == 2
    assert call(extra(idx=None)) == 1
    assert call(extra(fmt=W.FMT_INT8)) == 4              # formats differ
    assert call(extra(idx_st=32)) == 3
    assert call(extra(row_stride=664)) == 3               # the secondary pool is checked too
    dec = lib.smla_decode_dual(FAKE, 2, 64, 64 * 576, 576, pool(), FAKE, 64, 64, None, ctypes.byref(extra(topk=0)),
                               f, 2, FAKE, FAKE, None)
    assert dec == 2


def test_attention_noalloc_rejects_before_launch():
    """smla_attention_noalloc: argument errors as smla_attention, and a split
    form whose partials exceed the static scratch is refused (on the host,
    before the scratch is looked up or anything is launched)."""
    lib = smla._load()
    f = ctypes.c_float(1.0 / 24)

    def call(T=200, H=64, topk=8192, fmt=W.FMT_BF16, q=FAKE, out=FAKE):
        return lib.smla_attention_noalloc(q, T, H, H * 576, 576, pool(fmt=fmt), FAKE, topk, topk, None, None, f,
                                          out, H * 512, 512, FAKE, H, None)

    # BF16 rows, T=200, H=64, topk 8192: the split form at 3 splits needs 75 MiB of partials
    assert smla.use_split_form(200, 64, 8192, W.FMT_BF16, 0) == 1
    assert call() == 4 and "static scratch" in lib.smla_last_error().decode()
    assert call(q=None) == 1
    assert call(out=FAKE + 8) == 3
    assert call(T=0) == 0
    assert call(H=129) == 4


def test_probe_validation_before_launch():
    """The measurement aids check their arguments on the host."""
    lib = smla._load()
    assert lib.smla_probe_gather(pool(), FAKE, 0, 64, 64, None, FAKE, None) == 0          # T = 0: nothing
    assert lib.smla_probe_gather(pool(), None, 2, 64, 64, None, FAKE, None) == 1
    assert lib.smla_probe_gather(pool(), FAKE, 2, 64, 32, None, FAKE, None) == 3          # stride < topk
    assert lib.smla_probe_gather(pool(fmt=W.FMT_FP8_DSV4), FAKE, 2, 64, 64, None, FAKE, None) == 4
    assert lib.smla_probe_clock(None, 4, 10, None) == 1
    assert lib.smla_probe_clock(FAKE, 0, 10, None) == 2
    assert lib.smla_device_attributes(None) == 1
