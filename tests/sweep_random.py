"""Randomized sweep against the oracle, run by hand on a GPU (not collected
by pytest):

    python tests/sweep_random.py SECONDS SEED          # small shapes, every format
    python tests/sweep_random.py SECONDS SEED large    # 260-700 tokens, many-head formats
    python tests/sweep_random.py SECONDS SEED dual     # dual-cache calls (main + secondary list)

Shapes are drawn as in test_gpu_random_shapes.py (head counts on either side
of every kernel's head group, list widths with ragged tails, per-token
lengths, sinks, split counts), with sharper score distributions than the
committed tests: q is scaled by 2^-2..2^3, and in half the cases each token
gets one list entry whose cache row lies along a random direction that one
head's q shares, about 30 nats above the rest for that head.  The large
form sends several tokens through each persistent prefill workgroup; the
dual form draws a main list (a multiple of 64 entries) and a secondary list
over a second pool with padded rows, one softmax over both.  Every
case runs the prefill and the split decode with the combine, held to the
output bar against the oracle; the script prints each case and any failure
and runs until SECONDS have passed."""
import math
import os
import sys
import time

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
import sparse_top_mla_smla_amd as smla  # noqa: E402
from sparse_top_mla_smla_amd import workloads as W  # noqa: E402
from gpu_util import Dev, assert_lse_close, assert_out_close, bf16_dev_to_f64, f64_of_bits  # noqa: E402
from helpers import oracle_pool  # noqa: E402

FMTS = [W.FMT_BF16, W.FMT_FP8, W.FMT_INT8, W.FMT_FP8_ANY, W.FMT_FP8_NOPE, W.FMT_FP8_DOTS3, W.FMT_FP8_DSV4]
MANY_HEAD_FMTS = [W.FMT_FP8, W.FMT_INT8, W.FMT_FP8_ANY, W.FMT_FP8_NOPE, W.FMT_FP8_DSV4]
HEADS = [1, 3, 8, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 96, 127, 128]


def draw(rng, n, large):
    if large:
        fmt = MANY_HEAD_FMTS[n % len(MANY_HEAD_FMTS)]
        topk, H, T = int(rng.integers(64, 700)), int(rng.choice([33, 64, 96, 128])), int(rng.integers(260, 700))
    else:
        fmt = FMTS[n % len(FMTS)]
        topk, H, T = int(rng.integers(1, 1101)), int(rng.choice(HEADS)), int(rng.integers(1, 5))
    kw = dict(fmt=fmt, H=H, topk=topk, T=T, n_seqs=1, ctx=2048, causal=bool(rng.random() < 0.6),
              with_topk_length=bool(rng.random() < 0.5), with_sink=bool(rng.random() < 0.5))
    S = int(rng.integers(1, min(16, math.ceil(topk / 64)) + 1))
    return kw, S, float(2.0 ** rng.uniform(-2, 3)), bool(rng.random() < 0.5)


def sharpen(c, rng, qscale, dominant):
    q = W.bf16_bits_to_f32(c.q_buf).astype(np.float64) * qscale
    if dominant:
        H, dims = c.H, c.kv.shape[1]
        kv = W.bf16_bits_to_f32(c.kv).astype(np.float64)
        u = rng.standard_normal((c.q_buf.shape[1], dims))
        q = q + 2.0 * u[None, :, :]
        row_of_slot = np.empty(c.slots.shape[0], dtype=np.int64)
        row_of_slot[c.slots] = np.arange(c.slots.shape[0])
        for t in range(c.T):
            L = c.topk if c.topk_length is None else int(c.topk_length[t])
            if L < 1:
                continue
            h, p = int(rng.integers(0, H)), int(rng.integers(0, L))
            x = int(c.idx_buf[t, p])
            if x >= 0:
                # q_h . row = 2|u_h|^2 x 15 / (sm_scale |u_h|^2) ~ 30 nats
                kv[row_of_slot[x]] = (15.0 / (float(c.sm_scale) * float(u[h] @ u[h]))) * u[h]
        c.kv = W.f32_to_bf16_bits(kv.astype(np.float32))
    c.q_buf = W.f32_to_bf16_bits(q.astype(np.float32))


def run_case(c, S):
    d = Dev(c)
    o, l = smla.prefill(d.q, d.pool, d.indices, topk_length=d.topk_length, sink=d.sink, sm_scale=float(c.sm_scale))
    po, pl = smla.decode(d.q, d.pool, d.indices, S, topk_length=d.topk_length, sm_scale=float(c.sm_scale))
    o2, l2 = smla.combine(po, pl, sink=d.sink)
    torch.cuda.synchronize()
    ob, lf32, of, _ = oracle.prefill(c.q, oracle_pool(c), c.indices, topk_length=c.topk_length, sink=c.sink,
                                     sm_scale=c.sm_scale)
    assert_out_close(bf16_dev_to_f64(o), of, mean_ref=f64_of_bits(ob))
    assert_lse_close(l.cpu().numpy(), lf32)
    assert_out_close(bf16_dev_to_f64(o2), of, "combined out", mean_ref=f64_of_bits(ob))
    assert_lse_close(l2.cpu().numpy(), lf32, "combined lse")


def run_dual_case(rng, n):
    from test_gpu_dual import dual_args, reference

    fmt = FMTS[n % len(FMTS)]
    k1, k2 = 64 * int(rng.integers(1, 13)), int(rng.integers(1, 1501))
    H, T = int(rng.choice(HEADS)), int(rng.integers(1, 5))
    lengths, sink = bool(rng.random() < 0.6), bool(rng.random() < 0.5)
    S = int(rng.integers(1, min(16, math.ceil((k1 + k2) / 64)) + 1))
    qscale, dominant = float(2.0 ** rng.uniform(-2, 3)), bool(rng.random() < 0.5)
    name = (f"{n:05d} dual fmt{fmt} H{H} k{k1}+{k2} T{T} S{S} q*{qscale:.2f} dominant{int(dominant)}"
            f" len{int(lengths)} sink{int(sink)}")
    seed = int(rng.integers(0, 1 << 30))
    main = W.make_case(f"sweep_dual_{n}_main", config_id=4000 + 2 * n, seed=seed, fmt=fmt, T=T, H=H, n_seqs=1,
                       ctx=max(1024, 2 * k1), topk=k1, causal=True, with_topk_length=lengths, with_sink=sink)
    extra = W.make_case(f"sweep_dual_{n}_extra", config_id=4001 + 2 * n, seed=seed, fmt=fmt, T=T, H=H, n_seqs=1,
                        ctx=64 * math.ceil(max(512, 2 * k2) / 64), topk=k2, causal=False, with_topk_length=lengths)
    sharpen(main, rng, qscale, dominant)
    dm, de = Dev(main), Dev(extra, row_stride=(W.ROW_BYTES[fmt] + 31) // 16 * 16)
    o, l = smla.prefill_dual(dm.q, dm.pool, dm.indices, sink=dm.sink, **dual_args(dm, de))
    po, pl = smla.decode_dual(dm.q, dm.pool, dm.indices, num_splits=S, **dual_args(dm, de))
    o2, l2 = smla.combine(po, pl, sink=dm.sink)
    torch.cuda.synchronize()
    ob, lf32, of, _ = reference(main, extra)
    assert_out_close(bf16_dev_to_f64(o), of, mean_ref=f64_of_bits(ob))
    assert_lse_close(l.cpu().numpy(), lf32)
    assert_out_close(bf16_dev_to_f64(o2), of, "combined out", mean_ref=f64_of_bits(ob))
    assert_lse_close(l2.cpu().numpy(), lf32, "combined lse")
    return name


def main():
    seconds, seed = float(sys.argv[1]), int(sys.argv[2])
    large = len(sys.argv) > 3 and sys.argv[3] == "large"
    dual = len(sys.argv) > 3 and sys.argv[3] == "dual"
    rng = np.random.default_rng(seed)
    t_end = time.time() + seconds
    n = fails = 0
    while time.time() < t_end:
        if dual:
            try:
                print("ok  ", run_dual_case(rng, n), flush=True)
            except AssertionError as e:
                fails += 1
                print("FAIL", f"{n:05d} dual", str(e)[:300], flush=True)
            n += 1
            continue
        kw, S, qscale, dominant = draw(rng, n, large)
        name = (f"{n:05d} fmt{kw['fmt']} H{kw['H']} k{kw['topk']} T{kw['T']} S{S} q*{qscale:.2f} dominant{int(dominant)}"
                f" len{int(kw['with_topk_length'])} sink{int(kw['with_sink'])}")
        c = W.make_case(f"sweep_{n}", config_id=2000 + n, seed=int(rng.integers(0, 1 << 30)), **kw)
        sharpen(c, rng, qscale, dominant)
        try:
            run_case(c, S)
            print("ok  ", name, flush=True)
        except AssertionError as e:
            fails += 1
            print("FAIL", name, str(e)[:300], flush=True)
        n += 1
    print(f"done: {n} cases, {fails} failures", flush=True)
    sys.exit(1 if fails else 0)


if __name__ == "__main__":
    main()
