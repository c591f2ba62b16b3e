"""Seeded synthetic inputs for sparse MLA attention.

This module only draws random inputs: latent rows, queries, block tables,
top-k index lists, per-token list lengths and per-head sinks.  It holds none
of the attention or quantization arithmetic, so the CPU oracle and the HIP
path can both be fed from it without sharing any of the method's code.

Every tensor is drawn from ``numpy.random.default_rng(SeedSequence([seed,
config_id, tensor_id]))`` with tensor ids 1 = q, 2 = kv latent, 3 = indices,
4 = block table, 5 = topk_length, 6 = sink.  BF16 values are float32 N(0,1)
draws rounded to the nearest BF16 (ties to even) and kept as raw uint16 bits.

The named workloads reproduce the shapes of the pages' measurements
(AppMana release "Remove the legacy staged sparse-MLA prefill kernel": fused
prefill at T=1024, ctx 16384, H=64, index widths 512/1024, FP8 and INT8
caches; vLLM PR #57673 Test Result: h_q=8, d=512, combined top-k 640 with
attn_sink and topk_length on an 8192-token chunk) plus a split-KV decode
batch.  No public dataset is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

PAGE_BLOCK = 64
D_QK, D_V = 576, 512
FMT_BF16, FMT_FP8, FMT_INT8, FMT_FP8_ANY, FMT_FP8_NOPE, FMT_FP8_DOTS3, FMT_FP8_DSV4 = 0, 1, 2, 3, 4, 5, 6
FMT_NAMES = {FMT_BF16: "bf16", FMT_FP8: "fp8_e4m3", FMT_INT8: "int8", FMT_FP8_ANY: "fp8_e4m3_any_scale",
             FMT_FP8_NOPE: "fp8_e4m3_nope", FMT_FP8_DOTS3: "fp8_e4m3_dots3", FMT_FP8_DSV4: "fp8_e4m3_dsv4"}
ROW_BYTES = {FMT_BF16: 1152, FMT_FP8: 656, FMT_INT8: 656, FMT_FP8_ANY: 656, FMT_FP8_NOPE: 656,
             FMT_FP8_DOTS3: 1160, FMT_FP8_DSV4: 584}
# elements of a query row that enter a score (NOPE rows have no rope dimensions)
Q_DIMS = {FMT_BF16: 576, FMT_FP8: 576, FMT_INT8: 576, FMT_FP8_ANY: 576, FMT_FP8_NOPE: 512,
          FMT_FP8_DOTS3: 1088, FMT_FP8_DSV4: 512}
# elements of a latent row (and of the q buffer's rows) and of an output row
KV_DIMS = {f: {FMT_FP8_DOTS3: 1088, FMT_FP8_DSV4: 512}.get(f, D_QK) for f in FMT_NAMES}
V_DIMS = {f: (1024 if f == FMT_FP8_DOTS3 else D_V) for f in FMT_NAMES}
SM_SCALE = np.float32(1.0 / 24.0)  # 1/sqrt(576)
SM_SCALE_DOTS3 = np.float32(1.0 / np.sqrt(1088.0))
SM_SCALE_DSV4 = np.float32(1.0 / np.sqrt(512.0))
PAD_SENTINEL = 0x7FFFFFFF

TID_Q, TID_KV, TID_IDX, TID_BT, TID_LEN, TID_SINK = 1, 2, 3, 4, 5, 6


def rng_for(seed: int, config_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, config_id, tensor_id]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest BF16 (ties to even); finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    chunk = 1 << 24
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def distinct_uniform(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """k distinct integers drawn uniformly from [0, n), in draw order
    (sequential sampling without replacement: duplicates are redrawn)."""
    k = min(k, n)
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    if 4 * k >= n:
        return rng.permutation(n)[:k]
    got = np.zeros(0, dtype=np.int64)
    while got.shape[0] < k:
        draw = rng.integers(0, n, size=2 * (k - got.shape[0]) + 16)
        allv = np.concatenate([got, draw])
        _, first = np.unique(allv, return_index=True)
        got = allv[np.sort(first)][:k]
    return got


@dataclass
class Case:
    """One synthetic problem.  Arrays are host numpy; q/kv are raw BF16 bits."""
    name: str
    fmt: int
    T: int
    H: int
    n_seqs: int
    ctx: int
    topk: int
    q_buf: np.ndarray            # uint16 [T, Hbuf, KV_DIMS]; heads [0, H) are used
    kv: np.ndarray               # uint16 [n_seqs*ctx, KV_DIMS] latent rows, row = seq*ctx + pos
    slots: np.ndarray            # int32 [n_seqs*ctx] pool slot of each latent row
    num_blocks: int
    block_table: np.ndarray      # int32 [n_seqs, ctx/64]
    idx_buf: np.ndarray          # int32 [T, idx_ld]; columns [0, topk) are the list
    topk_length: Optional[np.ndarray]  # int32 [T] or None
    sink: Optional[np.ndarray]   # float32 [H] or None
    sm_scale: np.float32
    positions: np.ndarray        # int64 [T] query positions
    seq_of_token: np.ndarray     # int64 [T]
    num_splits: int = 1
    out_hbuf: int = 0            # head extent of the out buffer (0 = H)
    meta: Dict = field(default_factory=dict)

    @property
    def q(self) -> np.ndarray:
        return self.q_buf[:, : self.H]

    @property
    def indices(self) -> np.ndarray:
        return self.idx_buf[:, : self.topk]

    @property
    def row_bytes(self) -> int:
        return ROW_BYTES[self.fmt]

    def gathered_rows(self) -> int:
        """Valid (token, candidate) pairs: entries j < L_t whose index is a
        pool slot.  Counted once per token regardless of H."""
        idx = self.indices
        nslots = self.num_blocks * PAGE_BLOCK
        ok = (idx >= 0) & (idx < nslots)
        if self.topk_length is not None:
            L = np.clip(self.topk_length, 0, self.topk)
            ok &= np.arange(self.topk)[None, :] < L[:, None]
        return int(ok.sum())


def make_case(name: str, *, config_id: int, seed: int = 0, fmt: int, T: int, H: int,
              n_seqs: int, ctx: int, topk: int, idx_ld: int = 0, hbuf: int = 0,
              query: str = "last", causal: bool = True, tail_neg: int = 0,
              window: int = 0, with_topk_length: bool = False, with_sink: bool = False,
              num_splits: int = 1, out_hbuf: int = 0, pad_fill: int = -1,
              distinct_over_ctx: bool = False) -> Case:
    """General generator.

    query: "last" -> the T queries are the last T positions of their
      sequence (one sequence when n_seqs == 1; for n_seqs == T each sequence
      has one query at ctx-1).
    causal: candidates drawn from [0, p] for a query at p; otherwise from the
      whole context [0, ctx).
    window: the last `window` list entries are the positions p-window+1..p
      and the first topk-window entries are drawn from [0, p-window].
    tail_neg: the last tail_neg list entries are set to -1.
    with_topk_length: L_t ~ U{1..topk}; entries j >= L_t are set to -1.
    pad_fill: value of index-buffer columns beyond topk (idx_ld > topk).
    """
    assert ctx % PAGE_BLOCK == 0
    hbuf = hbuf or H
    idx_ld = idx_ld or topk
    nbps = ctx // PAGE_BLOCK
    num_blocks = n_seqs * nbps
    bt = rng_for(seed, config_id, TID_BT).permutation(num_blocks).astype(np.int32).reshape(n_seqs, nbps)
    pos = np.arange(ctx)
    slots = (bt[:, pos // PAGE_BLOCK] * PAGE_BLOCK + (pos % PAGE_BLOCK)[None, :]).astype(np.int32)
    slots = slots.reshape(-1)
    kv = normal_bf16(rng_for(seed, config_id, TID_KV), (n_seqs * ctx, KV_DIMS[fmt]))
    q_buf = normal_bf16(rng_for(seed, config_id, TID_Q), (T, hbuf, KV_DIMS[fmt]))

    if n_seqs == 1:
        seq_of_token = np.zeros(T, dtype=np.int64)
        positions = (ctx - T + np.arange(T)).astype(np.int64)
        assert positions[0] >= 0
    else:
        assert n_seqs == T
        seq_of_token = np.arange(T, dtype=np.int64)
        positions = np.full(T, ctx - 1, dtype=np.int64)

    r_idx = rng_for(seed, config_id, TID_IDX)
    idx_buf = np.full((T, idx_ld), pad_fill, dtype=np.int32)
    for t in range(T):
        p = int(positions[t])
        s = int(seq_of_token[t])
        hi = p + 1 if causal else ctx
        if window:
            main = distinct_uniform(r_idx, max(hi - window, 0), topk - window)
            win = np.arange(max(p - window + 1, 0), p + 1)
            lp = np.concatenate([main, win])
        else:
            lp = distinct_uniform(r_idx, hi, topk)
        row = np.full(topk, -1, dtype=np.int64)
        row[: lp.shape[0]] = bt[s, lp // PAGE_BLOCK].astype(np.int64) * PAGE_BLOCK + lp % PAGE_BLOCK
        if tail_neg:
            row[topk - tail_neg:] = -1
        idx_buf[t, :topk] = row.astype(np.int32)

    topk_length = None
    if with_topk_length:
        topk_length = rng_for(seed, config_id, TID_LEN).integers(1, topk + 1, size=T).astype(np.int32)
        for t in range(T):
            idx_buf[t, topk_length[t]:topk] = -1
    sink = None
    if with_sink:
        sink = rng_for(seed, config_id, TID_SINK).standard_normal(H, dtype=np.float32)
    return Case(name=name, fmt=fmt, T=T, H=H, n_seqs=n_seqs, ctx=ctx, topk=topk, q_buf=q_buf,
                kv=kv, slots=slots, num_blocks=num_blocks, block_table=bt, idx_buf=idx_buf,
                topk_length=topk_length, sink=sink,
                sm_scale={FMT_FP8_DOTS3: SM_SCALE_DOTS3, FMT_FP8_DSV4: SM_SCALE_DSV4}.get(fmt, SM_SCALE), positions=positions,
                seq_of_token=seq_of_token, num_splits=num_splits, out_hbuf=out_hbuf)


# ---------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------

def c1_tiny(seed: int = 0) -> Case:
    """Tiny BF16 case: T=4, H=8, one 256-token sequence (4 shuffled blocks),
    64 distinct uniform indices per token with the last 8 set to -1."""
    return make_case("c1_tiny_bf16", config_id=1, seed=seed, fmt=FMT_BF16, T=4, H=8, n_seqs=1,
                     ctx=256, topk=64, causal=False, tail_neg=8, num_splits=2)


def c2_decode(seed: int = 0, n_seqs: int = 64) -> Case:
    """FP8 split-KV decode: 64 sequences x 1 query at position 16383, H=64,
    ctx 16384 each (1,048,576-row pool, shuffled block table), 2048 distinct
    uniform indices per sequence, 8 splits."""
    return make_case("c2_decode_fp8", config_id=2, seed=seed, fmt=FMT_FP8, T=n_seqs, H=64,
                     n_seqs=n_seqs, ctx=16384, topk=2048, causal=True, num_splits=8)


def c3_prefill(seed: int = 0, width: int = 1024, T: int = 1024) -> Case:
    """FP8 fused prefill at the 16k footprint: one sequence of 16384 tokens,
    T queries at its last positions, H=64, causal index width `width`."""
    return make_case(f"c3_prefill_fp8_w{width}", config_id=3, seed=seed, fmt=FMT_FP8, T=T, H=64,
                     n_seqs=1, ctx=16384, topk=width, causal=True)


def c4_fewhead(seed: int = 0, T: int = 8192) -> Case:
    """Few-head BF16 prefill: h_q=8 heads as a [:, :8] view of a 64-head q
    buffer, out written into a [:, :8] view of a 64-head buffer, ctx 32768,
    combined list of 640 = 512 uniform + 128-position sliding window,
    topk_length ~ U{1..640} with -1 tail, per-head sink."""
    return make_case("c4_fewhead_bf16", config_id=4, seed=seed, fmt=FMT_BF16, T=T, H=8, hbuf=64,
                     n_seqs=1, ctx=32768, topk=640, window=128, with_topk_length=True,
                     with_sink=True, out_hbuf=64)


def c5_int8(seed: int = 0, T: int = 1024) -> Case:
    """INT8-cache prefill: ctx 65536, T=1024 last positions, H=128, index
    width 2048 passed as a view (row stride 4096) into a wider buffer whose
    other columns hold 0x7FFFFFFF, per-head sink."""
    return make_case("c5_prefill_int8", config_id=5, seed=seed, fmt=FMT_INT8, T=T, H=128,
                     n_seqs=1, ctx=65536, topk=2048, idx_ld=4096, causal=True, with_sink=True,
                     pad_fill=PAD_SENTINEL)


def dots3_prefill(seed: int = 0, T: int = 1024) -> Case:
    """DOTS3_SWA rows (FlashInfer PR #4802: d_qk 1088, d_v 1024, 1160-byte
    rows, lists of at least 513 entries so that the sliding window fits):
    one sequence of 16384 tokens, T queries at its last positions, H=64,
    513-entry lists of 385 causal uniform positions plus the 128-position
    window ending at the query, per-head sink.  (The split of the 513
    entries between selection and window is not given on the page.)"""
    return make_case("dots3_prefill", config_id=6, seed=seed, fmt=FMT_FP8_DOTS3, T=T, H=64, n_seqs=1,
                     ctx=16384, topk=513, window=128, causal=True, with_sink=True)


def dots3_decode(seed: int = 0, n_seqs: int = 32) -> Case:
    """DOTS3_SWA decode: 32 sequences x 1 query at position 16383 (the page
    quotes a T=32 decode for this model), ctx 16384 each, H=64, 513-entry
    lists as in dots3_prefill, 4 splits."""
    return make_case("dots3_decode", config_id=7, seed=seed, fmt=FMT_FP8_DOTS3, T=n_seqs, H=64,
                     n_seqs=n_seqs, ctx=16384, topk=513, window=128, causal=True, num_splits=4)


NAMED = {"c1": c1_tiny, "c2": c2_decode, "c3": c3_prefill, "c4": c4_fewhead, "c5": c5_int8,
         "dots3_prefill": dots3_prefill, "dots3_decode": dots3_decode}
