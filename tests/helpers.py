"""Shared test helpers: build oracle pools from workload cases and an
independent numpy dequantizer (torch's float8_e4m3fn decode, numpy views)
used to pin the oracle.  Imports the oracle; never imported by product code."""
import numpy as np
import torch

import oracle
from sparse_top_mla_smla_amd import workloads as W


def oracle_pool(case: W.Case, block_stride: int = 0, fill: int = 0) -> oracle.Pool:
    rb = W.ROW_BYTES[case.fmt]
    bs = block_stride or 64 * rb
    pool = oracle.Pool(np.full((case.num_blocks, bs), fill, dtype=np.uint8), case.fmt, bs)
    oracle.quantize_kv(case.kv, case.slots, pool)
    return pool


def np_dequant(pool: oracle.Pool, slots) -> np.ndarray:
    """Dequantize pool rows with library decoders (independent of the oracle)."""
    slots = np.asarray(slots, dtype=np.int64)
    rb = W.ROW_BYTES[pool.fmt]
    flat = pool.data.reshape(-1)
    off = (slots // 64) * pool.block_stride + (slots % 64) * rb
    rows = np.stack([flat[o:o + rb] for o in off]) if len(off) else np.zeros((0, rb), np.uint8)
    if pool.fmt == W.FMT_BF16:
        return W.bf16_bits_to_f32(rows.copy().view(np.uint16)).astype(np.float64)
    if pool.fmt == W.FMT_FP8_DOTS3:
        # [0,1024) e4m3 codes, [1024,1152) BF16 rope, [1152,1160) exponent bytes (bias 127)
        codes = torch.tensor(rows[:, :1024].copy()).view(torch.float8_e4m3fn).double().numpy()
        e = rows[:, 1152:1160].astype(np.int64)
        scales = np.where(e == 255, np.nan, np.ldexp(1.0, e - 127))
        rope = W.bf16_bits_to_f32(rows[:, 1024:1152].copy().view(np.uint16)).astype(np.float64)
        return np.concatenate([codes * np.repeat(scales, 128, axis=1), rope], axis=1)
    if pool.fmt == W.FMT_FP8_DSV4:
        # [0,448) e4m3 codes, [448,576) BF16 rope, [576,583) exponent bytes per 64 (bias 127), [583] pad
        codes = torch.tensor(rows[:, :448].copy()).view(torch.float8_e4m3fn).double().numpy()
        e = rows[:, 576:583].astype(np.int64)
        scales = np.where(e == 255, np.nan, np.ldexp(1.0, e - 127))
        rope = W.bf16_bits_to_f32(rows[:, 448:576].copy().view(np.uint16)).astype(np.float64)
        return np.concatenate([codes * np.repeat(scales, 64, axis=1), rope], axis=1)
    scales = rows[:, 512:528].copy().view(np.float32).astype(np.float64)
    if pool.fmt in (W.FMT_FP8, W.FMT_FP8_ANY, W.FMT_FP8_NOPE):
        codes = torch.tensor(rows[:, :512].copy()).view(torch.float8_e4m3fn).double().numpy()
    else:
        codes = rows[:, :512].view(np.int8).astype(np.float64)
    nope = codes * np.repeat(scales, 128, axis=1)
    if pool.fmt == W.FMT_FP8_NOPE:  # padding, not data: no rope dimensions
        return np.concatenate([nope, np.zeros((len(rows), 64))], axis=1)
    rope = W.bf16_bits_to_f32(rows[:, 528:656].copy().view(np.uint16)).astype(np.float64)
    return np.concatenate([nope, rope], axis=1)


def dense_attention(qf, K, sm_scale, sink=None, dv=512):
    """Brute-force softmax attention of query rows qf [n_q, d_k] over all rows
    K [n, d_k] (V = K[:, :dv]); float64.  With a sink, an extra key whose
    score is the sink value and whose value is zero joins the softmax.
    Returns (out [n_q,dv], lse [n_q]) with lse excluding the sink."""
    s = sm_scale * (qf @ K.T)
    m = s.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]
    if sink is not None:
        s = np.concatenate([s, np.full((s.shape[0], 1), sink)], axis=1)
        Vx = np.concatenate([K[:, :dv], np.zeros((1, dv))], axis=0)
    else:
        Vx = K[:, :dv]
    m2 = s.max(axis=1, keepdims=True)
    p = np.exp(s - m2)
    p /= p.sum(axis=1, keepdims=True)
    return p @ Vx, lse


def q_f64(case: W.Case) -> np.ndarray:
    return W.bf16_bits_to_f32(case.q).astype(np.float64)
