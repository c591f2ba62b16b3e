#!/usr/bin/env python3
"""Benchmark of sparse MLA attention on one MI355X.

Workload (the metric's configuration): FP8 fused prefill at the 16k
footprint -- one sequence of 16384 tokens in a shuffled 64-row paged pool,
T = 1024 queries at its last positions, H = 64 heads, causal top-k width
1024, BF16 q ~ N(0,1).  One step = writing the batch's 1024 new latent rows
into the cache (smla_quantize_kv) + the prefill over the T tokens
(smla_prefill).  Inputs are resident in HBM before the timed region.

Also measured in the same run:
- "decode": the split-KV decode batch -- 64 sequences x 1 query, ctx 16384
  each (656 MiB FP8 pool), H = 64, top-k 2048, 8 splits, decode + combine;
  beside it the same batch at the split count the library's cost model
  picks for this device (smla_decode_num_splits), and a dual-cache decode
  batch (64 sequences, H = 64, a 1024-wide main list over the same pool
  plus a 2176-wide secondary list over a second 656 MiB pool);
- "glm_nsa": the metric's prefill over FP8 rows with arbitrary scales
  (format 3, written from the same latent rows);
- "fewhead": 8192 tokens, 8 native heads read as a view of a 64-head BF16 q
  buffer, ctx 32768 BF16 pool, top-k 640 with per-token lengths and a sink,
  written in place; beside it the same inputs with all 64 heads;
- "int8": T = 1024, H = 128, ctx 65536 INT8 pool, top-k 2048 as a view of a
  4096-wide index buffer, with a sink; and in "decode", the decode batch
  over an INT8 pool at the model's split count;
- "dsv4": DSv4 584-byte rows -- the metric's prefill from the same latent
  rows and lists (first 512 values), and the dual-cache decode batch over
  two DSv4 pools;
- "dots3": DOTS3_SWA rows (1160 bytes, d_qk 1088, d_v 1024) -- prefill at
  T = 1024, ctx 16384, H = 64 over 513-entry lists (385 causal uniform + a
  128-position window) with a sink, and decode of 32 sequences x 1 query
  at 4 splits (decode + combine).
Kernel times come from HIP events on the launch stream (median, p10, p90).

Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 matrix peak
PAGE_A5000_US_PER_TOKEN = 5.258e3 / 1024  # AppMana release note: fp8 width 1024 on RTX A5000
D_QK, D_V = 576, 512


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--width", type=int, default=1024, help="prefill index width (512 or 1024)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample of the prefill tokens (0: all)")
    ap.add_argument("--no-extra", action="store_true", help="skip the few-head and INT8 workloads")
    ap.add_argument("--only", choices=["int8", "probe"], default=None,
                    help="int8: time only the INT8 workload and print its line (for counter passes); "
                         "probe: the gather probe over 1..32 copies of the decode batch's lists")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run one plain device-to-device copy of MIB MiB (reference for HBM counters)")
    return ap.parse_args()


def pct(xs):
    """median, p10, p90 of a list of times"""
    a = np.asarray(xs, dtype=np.float64)
    return float(np.median(a)), float(np.percentile(a, 10)), float(np.percentile(a, 90))


def event_times_us(torch, fn, iters, stream):
    """Per-call times (us) of fn() between HIP events recorded on `stream`."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in evs]


def queued_times_us(torch, fn, iters, stream, n=20):
    """Per-call times (us) of n back-to-back calls of fn(), queued behind a
    sleep kernel so that the host's enqueue cost never leaves the GPU idle
    between them (a kernel shorter than that cost is otherwise timed with
    the gaps); one value per batch."""
    out = []
    for _ in range(iters):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(20_000_000)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) * 1e3 / n)
    return out


def gather_ceiling(torch, smla, stream, pool, idx, topk_length, nbytes, expect_rows, iters=5):
    """The gather probe over the same pool and lists: every selected row moved
    into LDS, nothing computed.  Its rate is the measured ceiling for
    gathering these rows."""
    rows = smla.probe_gather(pool, idx, topk_length=topk_length)
    torch.cuda.synchronize()
    moved = int(rows.sum().item())
    t = pct(queued_times_us(torch, lambda: smla.probe_gather(pool, idx, topk_length=topk_length, rows_out=rows),
                            iters, stream))
    return {"probe_us_median_p10_p90": [round(v, 3) for v in t], "rows_moved": moved,
            "rows_match": moved == expect_rows, "GBps": round(nbytes / (t[0] * 1e-6) / 1e9, 2)}


def device_section(torch, smla, dev):
    """Device attributes, the shader clock measured under an MFMA load, and
    the peaks derived from both beside the spec values."""
    props = torch.cuda.get_device_properties(dev)
    a = smla.device_attributes()
    cus = a["compute_units"]
    out = smla.probe_clock(cus, 20000).cpu().numpy().astype(np.float64)
    mhz = float(np.median(out[:, 0] / out[:, 1] * a["wall_clock_khz"] / 1000.0))
    flop_per_clk = cus * 4 * 1024  # 32x32x16 BF16 MFMA: 32 cycles per SIMD, four SIMDs per CU
    hbm_attr = a["memory_clock_khz"] * 1e3 * 2 * a["memory_bus_bits"] / 8 / 1e9
    return {"name": props.name, "arch": getattr(props, "gcnArchName", ""), "compute_units": cus,
            "memory_GiB": round(props.total_memory / 2**30, 1), "attributes": a,
            "measured_clock_MHz_under_mfma_load": round(mhz, 1),
            "bf16_mfma_TFLOPs_at_peak_clock": round(flop_per_clk * a["clock_khz"] * 1e3 / 1e12, 1),
            "bf16_mfma_TFLOPs_at_measured_clock": round(flop_per_clk * mhz * 1e6 / 1e12, 1),
            "hbm_GBps_from_attributes": round(hbm_attr, 1),
            "spec_hbm_GBps": HBM_PEAK_GBPS, "spec_bf16_mfma_TFLOPs": BF16_MFMA_PEAK_TFLOPS}


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# the FP8 many-head kernel's own sources: its file and the headers it includes
FP8_KERNEL_SOURCES = ("attention_fp8.hip", "device_common.h", "launch.h", "lists.h")


def kernel_source_sha() -> str:
    """Hash of the sources the FP8 prefill kernel is built from; counter
    figures taken on other sources are not reported."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_top_mla_smla_amd", "csrc")
    for f in FP8_KERNEL_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(sha: str):
    """HBM traffic per prefill launch from committed rocprofv3 --pmc runs,
    only while the kernel sources are the ones the counters were taken on."""
    path = os.path.join(ROOT, "profiles", "traffic_attn_fp8_prefill.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha") != sha:
        return None
    return d.get("hbm_bytes_per_launch")


def dots3_lines(torch, smla, W, dev, stream, bf16, args):
    """DOTS3_SWA prefill and decode (1160-byte rows, d_v 1024)."""
    out = {}
    pc = W.dots3_prefill()
    q = bf16(pc.q_buf)
    kv = bf16(pc.kv)
    pool = smla.KVPool.empty(pc.num_blocks, W.FMT_FP8_DOTS3, device=dev)
    smla.quantize_kv(kv, torch.from_numpy(pc.slots).to(dev), pool)
    del kv
    idx = torch.from_numpy(pc.idx_buf).to(dev)
    sink = torch.from_numpy(pc.sink).to(dev)
    o = torch.empty((pc.T, pc.H, 1024), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((pc.T, pc.H), dtype=torch.float32, device=dev)

    def pre():
        smla.prefill(q, pool, idx, sink=sink, sm_scale=float(pc.sm_scale), out=o, lse=lse)

    pre()
    tp = pct(event_times_us(torch, pre, 10, stream))
    rows = pc.gathered_rows()
    nbytes = rows * W.ROW_BYTES[W.FMT_FP8_DOTS3]
    flops = 2.0 * pc.H * (1088 + 1024) * rows
    out["prefill"] = {
        "workload": f"dots3_swa prefill T={pc.T} ctx={pc.ctx} H={pc.H} topk={pc.topk} (385 causal uniform + "
                    "128-position window), sink",
        "kernel_us_median_p10_p90": [round(v, 3) for v in tp],
        "us_per_token": round(tp[0] / pc.T, 5),
        "gathered_kv_bytes": nbytes,
        "gathered_kv_GBps": round(nbytes / (tp[0] * 1e-6) / 1e9, 2),
        "mfma_util": round(flops / (tp[0] * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
    }
    print(f"[bench] dots3 prefill {tp[0]:.1f} us", file=sys.stderr, flush=True)
    del q, pool, idx, o, lse
    torch.cuda.empty_cache()

    dc = W.dots3_decode()
    q = bf16(dc.q_buf)
    kv = bf16(dc.kv)
    pool = smla.KVPool.empty(dc.num_blocks, W.FMT_FP8_DOTS3, device=dev)
    smla.quantize_kv(kv, torch.from_numpy(dc.slots).to(dev), pool)
    del kv
    idx = torch.from_numpy(dc.idx_buf).to(dev)
    # three index sets (the same positions in freshly permuted blocks), so
    # that consecutive calls do not find their rows cache-warm
    rng = np.random.default_rng(9)
    idx_sets = [idx]
    for _ in range(2):
        remap = torch.from_numpy(rng.permutation(dc.num_blocks).astype(np.int32)).to(dev)
        moved = remap[(idx.clamp(min=0) // 64).long()] * 64 + idx.clamp(min=0) % 64
        idx_sets.append(torch.where(idx >= 0, moved, idx).to(torch.int32))
    calls = [0]
    S = dc.num_splits
    po = torch.empty((dc.T, S, dc.H, 1024), dtype=torch.float32, device=dev)
    pl = torch.empty((dc.T, S, dc.H), dtype=torch.float32, device=dev)
    o = torch.empty((dc.T, dc.H, 1024), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((dc.T, dc.H), dtype=torch.float32, device=dev)

    def dec():
        calls[0] += 1
        smla.decode(q, pool, idx_sets[calls[0] % 3], S, sm_scale=float(dc.sm_scale), part_out=po, part_lse=pl)

    def comb():
        smla.combine(po, pl, out=o, lse=lse)

    dec()
    comb()
    td = pct(event_times_us(torch, dec, 20, stream))
    tc = pct(event_times_us(torch, comb, 20, stream))
    drows = dc.gathered_rows()
    dbytes = drows * W.ROW_BYTES[W.FMT_FP8_DOTS3]
    out["decode"] = {
        "workload": f"dots3_swa decode {dc.T} seqs x 1 query, ctx {dc.ctx}, H={dc.H}, topk={dc.topk}, splits={S} "
                    "(decode + combine)",
        "decode_kernel_us_median_p10_p90": [round(v, 3) for v in td],
        "combine_kernel_us_median_p10_p90": [round(v, 3) for v in tc],
        "gathered_kv_bytes": dbytes,
        "gathered_kv_GBps_end_to_end": round(dbytes / ((td[0] + tc[0]) * 1e-6) / 1e9, 2),
    }
    print(f"[bench] dots3 decode {td[0]:.1f} + {tc[0]:.1f} us (S={S})", file=sys.stderr, flush=True)
    del q, pool, idx, idx_sets, po, pl, o, lse
    torch.cuda.empty_cache()
    return out


def cpu_other_workloads(W, oracle, ncores):
    """The oracle over the decode batch and the few-head prefill (whole
    workloads) and a 256-token sample of the INT8 prefill, on `ncores`
    threads (writing the pools is not timed)."""
    res = {}

    def pool_of(c):
        rb = W.ROW_BYTES[c.fmt]
        p = oracle.Pool(np.zeros((c.num_blocks, 64 * rb), np.uint8), c.fmt, 64 * rb)
        oracle.quantize_kv(c.kv, c.slots, p)
        return p

    dc = W.c2_decode()
    p = pool_of(dc)
    tc = time.perf_counter()
    po, pl = oracle.decode_split(dc.q, p, dc.indices, dc.num_splits, sm_scale=dc.sm_scale, nthreads=ncores)
    oracle.combine(po, pl)
    dt = time.perf_counter() - tc
    res["decode"] = {"workload": f"fp8 split-KV decode {dc.T} seqs x 1 query, H={dc.H}, topk={dc.topk}, "
                                 f"{dc.num_splits} splits + combine (all of it)",
                     "us_per_call": round(dt * 1e6, 1), "cores": ncores}
    del p, po, pl, dc
    fc = W.c4_fewhead()
    p = pool_of(fc)
    tc = time.perf_counter()
    oracle.prefill(fc.q, p, fc.indices, topk_length=fc.topk_length, sink=fc.sink, sm_scale=fc.sm_scale,
                   nthreads=ncores)
    dt = time.perf_counter() - tc
    res["fewhead"] = {"workload": f"bf16 few-head prefill T={fc.T} H={fc.H} topk={fc.topk} (all tokens)",
                      "us_per_token": round(dt * 1e6 / fc.T, 3), "cores": ncores}
    del p, fc
    ic = W.c5_int8()
    p = pool_of(ic)
    n = 256  # a bounded sample: the whole workload takes about half a minute on 16 cores
    tokens = np.linspace(0, ic.T - 1, n).astype(np.int64)
    tc = time.perf_counter()
    oracle.prefill(ic.q, p, ic.indices, sink=ic.sink, sm_scale=ic.sm_scale, tokens=tokens, nthreads=ncores)
    dt = time.perf_counter() - tc
    res["int8"] = {"workload": f"int8 prefill T={ic.T} H={ic.H} topk={ic.topk} ({n} evenly spaced tokens)",
                   "us_per_token": round(dt * 1e6 / n, 3), "cores": ncores}
    print(f"[bench] cpu oracle, other workloads: {json.dumps(res)}", file=sys.stderr, flush=True)
    return res


def int8_line(torch, smla, W, dev, stream, bf16, iters=10):
    """C5: INT8 prefill, T = 1024, H = 128, ctx 65536, top-k 2048 as a view of
    a 4096-wide index buffer, with a sink."""
    result = {}
    # INT8, 128 heads, narrowed index view
    ic = W.c5_int8()
    iq = bf16(ic.q_buf)
    ikv = bf16(ic.kv)
    ipool = smla.KVPool.empty(ic.num_blocks, W.FMT_INT8, device=dev)
    smla.quantize_kv(ikv, torch.from_numpy(ic.slots).to(dev), ipool)
    del ikv
    iidx = torch.from_numpy(ic.idx_buf).to(dev)[:, : ic.topk]
    isink = torch.from_numpy(ic.sink).to(dev)
    iout = torch.empty((ic.T, ic.H, D_V), dtype=torch.bfloat16, device=dev)
    ilse = torch.empty((ic.T, ic.H), dtype=torch.float32, device=dev)

    def i8():
        smla.prefill(iq[:, : ic.H], ipool, iidx, sink=isink, sm_scale=float(ic.sm_scale), out=iout, lse=ilse)

    i8()
    ti = event_times_us(torch, i8, iters, stream)
    irows = ic.gathered_rows()
    ibytes = irows * W.ROW_BYTES[W.FMT_INT8]
    iflops = 2.0 * ic.H * (D_QK + D_V) * irows
    i_med = pct(ti)
    result["int8"] = {
        "workload": f"int8 prefill T={ic.T} H={ic.H} ctx {ic.ctx} topk {ic.topk} (index view of stride "
                    f"{ic.idx_buf.shape[1]}), sink",
        "kernel_us_median_p10_p90": [round(v, 3) for v in i_med],
        "us_per_token": round(i_med[0] / ic.T, 5),
        "gathered_kv_bytes": ibytes,
        "gathered_kv_GBps": round(ibytes / (i_med[0] * 1e-6) / 1e9, 2),
        "mfma_util": round(iflops / (i_med[0] * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
    }
    print(f"[bench] int8 {i_med[0]:.1f} us", file=sys.stderr, flush=True)
    del iq, ipool, iidx, iout, ilse
    torch.cuda.empty_cache()
    return result["int8"]


def probe_scaling(torch, smla, W, dev, stream, bf16):
    """The gather probe over the decode batch's HBM-resident pool with 1, 2,
    4, ..., 32 copies of its lists (each copy with the block ids permuted
    afresh, so every copy reads other rows), the same lists sorted per token,
    and runs of consecutive slots: how the gather rate depends on the volume
    one launch moves."""
    dc = W.c2_decode()
    dkv = bf16(dc.kv)
    dpool = smla.KVPool.empty(dc.num_blocks, W.FMT_FP8, device=dev)
    smla.quantize_kv(dkv, torch.from_numpy(dc.slots).to(dev), dpool)
    del dkv
    didx = torch.from_numpy(dc.idx_buf).to(dev)
    rng = np.random.default_rng(7)

    def remapped():
        remap = torch.from_numpy(rng.permutation(dc.num_blocks).astype(np.int32)).to(dev)
        moved = remap[(didx.clamp(min=0) // 64).long()] * 64 + didx.clamp(min=0) % 64
        return torch.where(didx >= 0, moved, didx).to(torch.int32)

    copies = [remapped() for _ in range(32)]
    rb = W.ROW_BYTES[W.FMT_FP8]
    out = {"workload": f"gather probe over the decode pool ({dc.num_blocks} blocks of 64 rows, "
                       f"{dc.num_blocks * 64 * rb / 2**20:.0f} MiB), lists of {dc.topk} rows per token",
           "random": [], "sorted": [], "consecutive": []}

    def run(label, idx):
        rows = int((idx >= 0).sum().item())
        smla.probe_gather(dpool, idx)
        torch.cuda.synchronize()
        t = pct(queued_times_us(torch, lambda: smla.probe_gather(dpool, idx), 5, stream))
        out[label].append({"tokens": int(idx.shape[0]), "rows": rows, "us_median_p10_p90": [round(v, 3) for v in t],
                           "GBps": round(rows * rb / (t[0] * 1e-6) / 1e9, 1)})

    for m in (1, 2, 4, 8, 16, 32):
        run("random", torch.cat(copies[:m], 0).contiguous())
    big = torch.iinfo(torch.int32).max
    for m in (1, 8):
        srt = torch.cat(copies[:m], 0)
        srt = torch.where(srt >= 0, srt, big).sort(dim=1).values
        run("sorted", torch.where(srt == big, -1, srt).to(torch.int32).contiguous())
    nrows = dc.num_blocks * 64
    for tok in (64, 512):
        base = (torch.arange(tok, device=dev, dtype=torch.int64) * dc.topk) % (nrows - dc.topk)
        run("consecutive", (base[:, None] + torch.arange(dc.topk, device=dev)[None, :]).to(torch.int32).contiguous())
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path: tokens, sequences and heads shard across GPUs with no exchange inside attention)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_top_mla_smla_amd as smla
    from sparse_top_mla_smla_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    smla.row_bytes(W.FMT_FP8)  # raises if libsmla.so is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.only == "int8":
        print(json.dumps({"int8": int8_line(torch, smla, W, dev, torch.cuda.current_stream(), bf16,
                                            max(args.steps, 1))}), flush=True)
        return
    if args.only == "probe":
        print(json.dumps({"probe_scaling": probe_scaling(torch, smla, W, dev, torch.cuda.current_stream(), bf16)}),
              flush=True)
        return

    # ---------------- prefill workload ----------------
    t0 = time.time()
    case = W.c3_prefill(width=args.width)
    T, H = case.T, case.H
    q = bf16(case.q_buf)
    kv = bf16(case.kv)
    slots = torch.from_numpy(case.slots).to(dev)
    idx = torch.from_numpy(case.idx_buf).to(dev)
    pool = smla.KVPool.empty(case.num_blocks, W.FMT_FP8, device=dev)
    n_ctx = case.ctx - T
    smla.quantize_kv(kv[:n_ctx], slots[:n_ctx], pool)            # context written once
    new_kv, new_slots = kv[n_ctx:], slots[n_ctx:]                 # the batch's own rows
    out = torch.empty((T, H, D_V), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    stream = torch.cuda.current_stream()

    def step(ev=None):
        smla.quantize_kv(new_kv, new_slots, pool)
        if ev is not None:
            ev[0].record(stream)
        smla.prefill(q, pool, idx, sm_scale=float(case.sm_scale), out=out, lse=lse)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / args.steps
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    prefill_ms = float(np.mean(kern_ms))
    p_med, p_p10, p_p90 = pct([x * 1e3 for x in kern_ms])

    rows = case.gathered_rows()
    kv_bytes = rows * W.ROW_BYTES[W.FMT_FP8]
    io_bytes = T * H * (D_QK * 2 + D_V * 2 + 4) + T * case.topk * 4
    alg_bytes = kv_bytes + io_bytes
    flops = 2.0 * H * (D_QK + D_V) * rows
    achieved = alg_bytes / (prefill_ms * 1e-3) / 1e9
    us_per_token = ms_per_step * 1e3 / T
    sha = kernel_source_sha()
    traffic = load_traffic(sha)

    result = {
        "metric": "sparse-MLA prefill µs/token & gathered-KV GB/s, T=1024 ctx16k H=64 topk1024",
        "value": round(us_per_token, 5),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round(us_per_token / PAGE_A5000_US_PER_TOKEN, 6) if args.width == 1024 else None,
        "dtype": "fp8_e4m3 cache / bf16 QK mfma, f16 PV mfma / f32 softmax",
        "data": "synthetic (seeded N(0,1) latent and q, uniform causal top-k over a shuffled paged pool)",
        "config": {"workload": f"fp8 sparse-MLA prefill T={T} ctx={case.ctx} H={H} topk={case.topk} "
                               f"page_block=64 (cache write of the batch's {T} rows + prefill)",
                   "T": T, "ctx": case.ctx, "H": H, "topk": case.topk, "kv_format": "fp8_e4m3_656B"},
        "gathered_kv_GBps": round(kv_bytes / (prefill_ms * 1e-3) / 1e9, 2),
        "prefill_kernel_us": round(prefill_ms * 1e3, 3),
        "prefill_kernel_us_median_p10_p90": [round(p_med, 3), round(p_p10, 3), round(p_p90, 3)],
        "prefill_us_per_token_kernel": round(prefill_ms * 1e3 / T, 5),
        "mfma_util": round(flops / (prefill_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
        # The pool (10.75 MB) is cache-resident, so the gathers are served by
        # L2/MALL and the dense 64-head x 64-candidate tiles make the kernel
        # MFMA-bound: achieved = algorithmic FLOP per launch / mean kernel time.
        "roofline": {"bound": "mfma", "achieved": round(flops / (prefill_ms * 1e-3) / 1e12, 2),
                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (prefill_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": "attn_fp8_kernel<prefill> (smla::attn_fp8_kernel<false, false, false, 1>)",
                     "algorithmic_flop_per_launch": flops,
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "hbm_view": {"achieved_GBps": round(achieved, 2), "peak_GBps": HBM_PEAK_GBPS,
                                  "frac": round(achieved / HBM_PEAK_GBPS, 4)}},
        "kernel_source_sha": sha,
    }
    # the same prefill at the other index width of the page's measurement
    other_w = 512 if args.width == 1024 else 1024
    if not args.no_extra:
        oc = W.c3_prefill(width=other_w)
        oidx = torch.from_numpy(oc.idx_buf).to(dev)

        def pre_other():
            smla.prefill(q, pool, oidx, sm_scale=float(case.sm_scale), out=out, lse=lse)

        pre_other()
        tw = pct(event_times_us(torch, pre_other, 20, stream))
        orows = oc.gathered_rows()
        oflops = 2.0 * H * (D_QK + D_V) * orows
        result[f"width{other_w}"] = {
            "workload": f"fp8 prefill T={T} ctx={case.ctx} H={H} topk={other_w} (the same q, pool and causal draw "
                        "at the other index width)",
            "kernel_us_median_p10_p90": [round(v, 3) for v in tw],
            "us_per_token_kernel": round(tw[0] / T, 5),
            "gathered_kv_bytes": orows * W.ROW_BYTES[W.FMT_FP8],
            "gathered_kv_GBps": round(orows * W.ROW_BYTES[W.FMT_FP8] / (tw[0] * 1e-6) / 1e9, 2),
            "mfma_util": round(oflops / (tw[0] * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
        }
        print(f"[bench] prefill width {other_w}: {tw[0]:.1f} us", file=sys.stderr, flush=True)
        del oidx
    # the same prefill over FP8 rows with arbitrary scales (GLM_NSA rows)
    if not args.no_extra:
        apool = smla.KVPool.empty(case.num_blocks, W.FMT_FP8_ANY, device=dev)
        smla.quantize_kv(kv, torch.from_numpy(case.slots).to(dev), apool)

        def nsa():
            smla.prefill(q, apool, idx, sm_scale=float(case.sm_scale), out=out, lse=lse)

        nsa()
        tn = pct(event_times_us(torch, nsa, 10, stream))
        result["glm_nsa"] = {
            "workload": f"fp8 rows with arbitrary per-128 scales (amax/448), prefill T={T} ctx={case.ctx} H={H} "
                        f"topk={case.topk}",
            "kernel_us_median_p10_p90": [round(v, 3) for v in tn],
            "us_per_token": round(tn[0] / T, 5),
            "gathered_kv_GBps": round(kv_bytes / (tn[0] * 1e-6) / 1e9, 2),
            "vs_power_of_two_fp8_kernel": round(tn[0] / p_med, 3),
        }
        print(f"[bench] glm_nsa prefill {tn[0]:.1f} us", file=sys.stderr, flush=True)
        del apool
        # the same rows and lists as DSv4 584-byte rows (the first 512 values of
        # each latent row and of each q row)
        v4pool = smla.KVPool.empty(case.num_blocks, W.FMT_FP8_DSV4, device=dev)
        smla.quantize_kv(kv, torch.from_numpy(case.slots).to(dev), v4pool)
        v4out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)

        def v4():
            smla.prefill(q[:, :, :512], v4pool, idx, sm_scale=float(W.SM_SCALE_DSV4), out=v4out, lse=lse)

        v4()
        t4 = pct(event_times_us(torch, v4, 10, stream))
        v4_bytes = rows * W.ROW_BYTES[W.FMT_FP8_DSV4]
        result["dsv4"] = {"prefill": {
            "workload": f"dsv4 584-byte rows, prefill T={T} ctx={case.ctx} H={H} topk={case.topk} (the metric's "
                        "lists and latent rows)",
            "kernel_us_median_p10_p90": [round(v, 3) for v in t4],
            "us_per_token": round(t4[0] / T, 5),
            "gathered_kv_bytes": v4_bytes,
            "gathered_kv_GBps": round(v4_bytes / (t4[0] * 1e-6) / 1e9, 2),
        }}
        print(f"[bench] dsv4 prefill {t4[0]:.1f} us", file=sys.stderr, flush=True)
        del v4pool, v4out
    result["device"] = device_section(torch, smla, dev)
    # the gather ceiling of the metric workload's lists (cache-resident pool)
    result["gather_ceiling"] = gather_ceiling(torch, smla, stream, pool, idx, None, kv_bytes, rows)
    result["gather_ceiling"]["workload"] = "the gather probe over the metric workload's pool and lists"
    print(f"[bench] prefill setup {setup_s:.1f}s, step {ms_per_step:.3f} ms, kernel {prefill_ms:.3f} ms",
          file=sys.stderr, flush=True)

    # ---------------- decode workload ----------------
    if not args.no_decode:
        del kv
        dc = W.c2_decode()
        dq = bf16(dc.q_buf)
        dkv = bf16(dc.kv)
        dslots = torch.from_numpy(dc.slots).to(dev)
        didx = torch.from_numpy(dc.idx_buf).to(dev)
        dpool = smla.KVPool.empty(dc.num_blocks, W.FMT_FP8, device=dev)
        smla.quantize_kv(dkv, dslots, dpool)
        ipool8 = v4main = None
        if not args.no_extra:  # the same rows in an INT8 pool and in a DSv4 pool
            ipool8 = smla.KVPool.empty(dc.num_blocks, W.FMT_INT8, device=dev)
            smla.quantize_kv(dkv, dslots, ipool8)
            v4main = smla.KVPool.empty(dc.num_blocks, W.FMT_FP8_DSV4, device=dev)
            smla.quantize_kv(dkv, dslots, v4main)
        del dkv
        dout = torch.empty((dc.T, dc.H, D_V), dtype=torch.bfloat16, device=dev)
        dlse = torch.empty((dc.T, dc.H), dtype=torch.float32, device=dev)
        # rotate over independent index sets so no call finds its rows cache-warm
        rng = np.random.default_rng(7)
        idx_sets = [didx]
        for k in range(2):
            perm = rng.permutation(dc.num_blocks).astype(np.int32)
            remap = torch.from_numpy(perm).to(dev)
            # same positions, different blocks: a fresh permutation of the block ids
            moved = remap[(didx.clamp(min=0) // 64).long()] * 64 + didx.clamp(min=0) % 64
            idx_sets.append(torch.where(didx >= 0, moved, didx).to(torch.int32))
        torch.cuda.synchronize()
        dsteps = max(args.steps, 20)
        drows = dc.gathered_rows()
        dbytes = drows * W.ROW_BYTES[W.FMT_FP8]

        def time_decode(S, pool=None):
            pool = pool or dpool
            po = torch.empty((dc.T, S, dc.H, D_V), dtype=torch.float32, device=dev)
            pl = torch.empty((dc.T, S, dc.H), dtype=torch.float32, device=dev)

            def dstep(i, ev=None):
                ix = idx_sets[i % len(idx_sets)]
                if ev is not None:
                    ev[0].record(stream)
                smla.decode(dq, pool, ix, S, sm_scale=float(dc.sm_scale), part_out=po, part_lse=pl)
                if ev is not None:
                    ev[1].record(stream)
                smla.combine(po, pl, out=dout, lse=dlse)
                if ev is not None:
                    ev[2].record(stream)

            for i in range(args.warmup):
                dstep(i)
            devs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(dsteps)]
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for i in range(dsteps):
                dstep(i, devs[i])
            torch.cuda.synchronize()
            d_elapsed = (time.perf_counter() - t1) * 1e6 / dsteps
            dec_list = [a.elapsed_time(b) * 1e3 for a, b, _ in devs]
            comb_list = [b.elapsed_time(c) * 1e3 for _, b, c in devs]
            dec_us = float(np.mean(dec_list))
            comb_us = float(np.mean(comb_list))
            return {
                "num_splits": S,
                "us_per_call": round(d_elapsed, 3),
                "decode_kernel_us": round(dec_us, 3),
                "decode_kernel_us_median_p10_p90": [round(v, 3) for v in pct(dec_list)],
                "combine_kernel_us": round(comb_us, 3),
                "combine_kernel_us_median_p10_p90": [round(v, 3) for v in pct(comb_list)],
                "gathered_kv_GBps_decode_kernel": round(dbytes / (dec_us * 1e-6) / 1e9, 2),
                "gathered_kv_GBps_end_to_end": round(dbytes / ((dec_us + comb_us) * 1e-6) / 1e9, 2),
                "hbm_frac_end_to_end": round(dbytes / ((dec_us + comb_us) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            }

        def time_decode_graph(S):
            """decode + combine captured in one HIP graph per index set
            (stream capture through torch.cuda.graph) and replayed in turn."""
            po = torch.empty((dc.T, S, dc.H, D_V), dtype=torch.float32, device=dev)
            pl = torch.empty((dc.T, S, dc.H), dtype=torch.float32, device=dev)
            graphs = []
            side = torch.cuda.Stream()
            for ix in idx_sets:
                def run(ix=ix):
                    smla.decode(dq, dpool, ix, S, sm_scale=float(dc.sm_scale), part_out=po, part_lse=pl)
                    smla.combine(po, pl, out=dout, lse=dlse)

                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    run()
                torch.cuda.current_stream().wait_stream(side)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    run()
                graphs.append(g)
            for i in range(args.warmup):
                graphs[i % len(graphs)].replay()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for i in range(dsteps):
                graphs[i % len(graphs)].replay()
            torch.cuda.synchronize()
            wall = (time.perf_counter() - t1) * 1e6 / dsteps
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(dsteps)]
            for i in range(dsteps):
                evs[i][0].record(stream)
                graphs[i % len(graphs)].replay()
                evs[i][1].record(stream)
            torch.cuda.synchronize()
            per = [a.elapsed_time(b) * 1e3 for a, b in evs]
            us = float(np.mean(per))
            del graphs
            return {
                "num_splits": S,
                "us_per_call": round(wall, 3),
                "graph_us": round(us, 3),
                "graph_us_median_p10_p90": [round(v, 3) for v in pct(per)],
                "gathered_kv_GBps_end_to_end": round(dbytes / (us * 1e-6) / 1e9, 2),
                "hbm_frac_end_to_end": round(dbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            }

        S = dc.num_splits
        result["decode"] = {
            "workload": f"fp8 split-KV decode {dc.T} seqs x 1 query, ctx {dc.ctx}, H={dc.H}, "
                        f"topk={dc.topk}, splits={S} (decode + combine)",
            "gathered_kv_bytes": dbytes,
        }
        # the gather ceiling of these rows from HBM (a fresh index set per call)
        pc = [0]

        def probe_dec():
            pc[0] += 1
            smla.probe_gather(dpool, idx_sets[pc[0] % 3])

        probe_dec()
        tpd = pct(queued_times_us(torch, probe_dec, 5, stream))
        result["decode"]["gather_ceiling"] = {
            "workload": "the gather probe over the decode batch's lists (rotating index sets)",
            "probe_us_median_p10_p90": [round(v, 3) for v in tpd],
            "GBps": round(dbytes / (tpd[0] * 1e-6) / 1e9, 2)}
        result["decode"].update(time_decode(S))
        # the split count the library's cost model picks for this shape on this device
        Sm = smla.decode_num_splits(dc.T, dc.H, dc.topk, W.FMT_FP8)
        model = time_decode(Sm) if Sm != S else {k: v for k, v in result["decode"].items()
                                                if k not in ("workload", "gathered_kv_bytes")}
        model["predicted_us"] = round(smla.split_model_cost(dc.T, dc.H, dc.topk, W.FMT_FP8, Sm), 2)
        result["decode"]["model_split_count"] = model
        d8 = result["decode"]
        print(f"[bench] decode {d8['decode_kernel_us']:.2f} us + combine {d8['combine_kernel_us']:.2f} us (S={S}); "
              f"model S={Sm}: {model['decode_kernel_us']:.2f} + {model['combine_kernel_us']:.2f} us",
              file=sys.stderr, flush=True)
        gr = time_decode_graph(Sm)
        gr["workload"] = "the same batch at the model's split count, decode + combine replayed as one HIP graph"
        result["decode"]["graph"] = gr
        # decode is bound by HBM: the 656 MiB pool exceeds the caches and the
        # rows are random.  Gathered-KV bytes per call / graph time per call.
        dach = dbytes / (gr["graph_us"] * 1e-6) / 1e9
        result["decode"]["roofline"] = {
            "bound": "hbm", "achieved": round(dach, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(dach / HBM_PEAK_GBPS, 4), "target_frac": 0.60,
            "measured_over": f"decode + combine per call, replayed as a HIP graph, {Sm} splits",
            "algorithmic_bytes_per_call": dbytes,
            "frac_of_measured_gather_ceiling": round(dach / result["decode"]["gather_ceiling"]["GBps"], 4)}
        print(f"[bench] decode + combine as a HIP graph (S={Sm}): {gr['graph_us']:.2f} us, "
              f"{gr['us_per_call']:.2f} us per call", file=sys.stderr, flush=True)
        if ipool8 is not None:
            Si = smla.decode_num_splits(dc.T, dc.H, dc.topk, W.FMT_INT8)
            i8d = time_decode(Si, ipool8)
            i8d["predicted_us"] = round(smla.split_model_cost(dc.T, dc.H, dc.topk, W.FMT_INT8, Si), 2)
            i8d["workload"] = f"int8 split-KV decode, the same batch and rows, splits={Si} (the model's count)"
            result["decode"]["int8"] = i8d
            print(f"[bench] int8 decode {i8d['decode_kernel_us']:.2f} + {i8d['combine_kernel_us']:.2f} us (S={Si})",
                  file=sys.stderr, flush=True)
            del ipool8
        # dual cache: the first 1024 entries of each list over this pool, and a
        # 2176-wide secondary list over a second pool of the same size
        if not args.no_extra:
            k1, k2 = 1024, 2176
            gen = torch.Generator(device=dev)
            gen.manual_seed(11)
            xpool = smla.KVPool.empty(dc.num_blocks, W.FMT_FP8, device=dev)
            nrows = dc.num_blocks * 64
            for r0 in range(0, nrows, 1 << 18):
                xkv = torch.randn((1 << 18, D_QK), generator=gen, device=dev).to(torch.bfloat16)
                smla.quantize_kv(xkv, torch.arange(r0, r0 + (1 << 18), dtype=torch.int32, device=dev), xpool)
                del xkv
            xidx = [torch.randint(0, nrows, (dc.T, k2), generator=gen, device=dev, dtype=torch.int32)
                    for _ in range(3)]
            mids = [ix[:, :k1] for ix in idx_sets]
            Sd = smla.decode_num_splits(dc.T, dc.H, k1 + k2, W.FMT_FP8)
            xpo = torch.empty((dc.T, Sd, dc.H, D_V), dtype=torch.float32, device=dev)
            xpl = torch.empty((dc.T, Sd, dc.H), dtype=torch.float32, device=dev)

            def dual(i):
                smla.decode_dual(dq[:, : dc.H], dpool, mids[i % 3], xpool, xidx[i % 3], Sd,
                                 sm_scale=float(dc.sm_scale), part_out=xpo, part_lse=xpl)
                smla.combine(xpo, xpl, out=dout, lse=dlse)

            for i in range(3):
                dual(i)
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for i in range(dsteps):
                dual(i)
            ev[1].record(stream)
            torch.cuda.synchronize()
            dual_us = ev[0].elapsed_time(ev[1]) * 1e3 / dsteps
            dual_bytes = dc.T * (k1 + k2) * W.ROW_BYTES[W.FMT_FP8]
            result["decode"]["dual_cache"] = {
                "workload": f"fp8 dual-cache decode {dc.T} seqs x 1 query, H={dc.H}, main topk {k1} + secondary "
                            f"topk {k2} over two {dc.num_blocks * 64 * 656 >> 20} MiB pools, splits={Sd} "
                            "(decode + combine)",
                "us_per_call": round(dual_us, 3),
                "gathered_kv_bytes": dual_bytes,
                "gathered_kv_GBps": round(dual_bytes / (dual_us * 1e-6) / 1e9, 2),
            }
            print(f"[bench] dual-cache decode {dual_us:.1f} us (S={Sd})", file=sys.stderr, flush=True)
            del xpool
            # the same dual-cache decode over DSv4 584-byte rows (the model
            # the page pairs with the 1024 + 2176 widths)
            x4pool = smla.KVPool.empty(dc.num_blocks, W.FMT_FP8_DSV4, device=dev)
            for r0 in range(0, nrows, 1 << 18):
                xkv = torch.randn((1 << 18, 512), generator=gen, device=dev).to(torch.bfloat16)
                smla.quantize_kv(xkv, torch.arange(r0, r0 + (1 << 18), dtype=torch.int32, device=dev), x4pool)
                del xkv

            # the split count the model picks for DSv4 rows at these widths
            Sd4 = smla.decode_num_splits(dc.T, dc.H, k1 + k2, W.FMT_FP8_DSV4)
            x4po = torch.empty((dc.T, Sd4, dc.H, D_V), dtype=torch.float32, device=dev)
            x4pl = torch.empty((dc.T, Sd4, dc.H), dtype=torch.float32, device=dev)

            def dual4(i):
                smla.decode_dual(dq[:, : dc.H, :512], v4main, mids[i % 3], x4pool, xidx[i % 3], Sd4,
                                 sm_scale=float(W.SM_SCALE_DSV4), part_out=x4po, part_lse=x4pl)
                smla.combine(x4po, x4pl, out=dout, lse=dlse)

            for i in range(3):
                dual4(i)
            torch.cuda.synchronize()
            ev[0].record(stream)
            for i in range(dsteps):
                dual4(i)
            ev[1].record(stream)
            torch.cuda.synchronize()
            dual4_us = ev[0].elapsed_time(ev[1]) * 1e3 / dsteps
            dual4_bytes = dc.T * (k1 + k2) * W.ROW_BYTES[W.FMT_FP8_DSV4]
            result.setdefault("dsv4", {})["dual_cache_decode"] = {
                "workload": f"dsv4 dual-cache decode {dc.T} seqs x 1 query, H={dc.H}, main topk {k1} + secondary "
                            f"topk {k2} over two {dc.num_blocks * 64 * 584 >> 20} MiB pools, splits={Sd4} "
                            "(decode + combine)",
                "us_per_call": round(dual4_us, 3),
                "gathered_kv_bytes": dual4_bytes,
                "gathered_kv_GBps": round(dual4_bytes / (dual4_us * 1e-6) / 1e9, 2),
            }
            print(f"[bench] dsv4 dual-cache decode {dual4_us:.1f} us (S={Sd4})", file=sys.stderr, flush=True)
            del x4pool, xidx, mids, xpo, xpl, x4po, x4pl
        del v4main
        del dpool, dq, didx, idx_sets, dout, dlse
        torch.cuda.empty_cache()

    # ---------------- few-head BF16 and INT8 prefill ----------------
    if not args.no_extra:
        iters = 10
        # few heads: q[:, :8] of a 64-head buffer, out written in place
        fc = W.c4_fewhead()
        fq = bf16(fc.q_buf)
        fkv = bf16(fc.kv)
        fpool = smla.KVPool.empty(fc.num_blocks, W.FMT_BF16, device=dev)
        smla.quantize_kv(fkv, torch.from_numpy(fc.slots).to(dev), fpool)
        # the same latent rows in an FP8 pool (656-byte rows)
        f8pool = smla.KVPool.empty(fc.num_blocks, W.FMT_FP8, device=dev)
        smla.quantize_kv(fkv, torch.from_numpy(fc.slots).to(dev), f8pool)
        del fkv
        fidx = torch.from_numpy(fc.idx_buf).to(dev)[:, : fc.topk]
        ftl = torch.from_numpy(fc.topk_length).to(dev)
        fsink64 = torch.from_numpy(np.concatenate([fc.sink, np.zeros(64 - fc.H, np.float32)])).to(dev)
        fout = torch.zeros((fc.T, fc.out_hbuf, D_V), dtype=torch.bfloat16, device=dev)
        flse = torch.empty((fc.T, 64), dtype=torch.float32, device=dev)

        def few(hq):
            return lambda: smla.prefill(fq[:, :hq], fpool, fidx, topk_length=ftl, sink=fsink64[:hq],
                                        sm_scale=float(fc.sm_scale), out=fout[:, :hq], lse=flse[:, :hq])

        few(fc.H)()
        few(64)()
        t8 = event_times_us(torch, few(fc.H), iters, stream)
        t64 = event_times_us(torch, few(64), iters, stream)
        frows = fc.gathered_rows()
        fbytes = frows * W.ROW_BYTES[W.FMT_BF16]
        f_med = pct(t8)
        result["fewhead"] = {
            "workload": f"bf16 few-head prefill T={fc.T} H={fc.H} (view of a 64-head q buffer), ctx {fc.ctx}, "
                        f"topk {fc.topk} with topk_length and sink, out in place",
            "kernel_us_median_p10_p90": [round(v, 3) for v in f_med],
            "us_per_token": round(f_med[0] / fc.T, 5),
            "gathered_kv_bytes": fbytes,
            "gathered_kv_GBps": round(fbytes / (f_med[0] * 1e-6) / 1e9, 2),
            "same_inputs_all_64_heads_us_median": round(pct(t64)[0], 3),
            "speedup_vs_64_heads": round(pct(t64)[0] / f_med[0], 3),
        }
        # the pool (36 MiB) is cache-resident: the rate is put against the
        # measured gather ceiling of the same rows rather than HBM peak
        fc_ceil = gather_ceiling(torch, smla, stream, fpool, fidx, ftl, fbytes, frows)
        result["fewhead"]["gather_ceiling"] = fc_ceil
        result["fewhead"]["frac_of_gather_ceiling"] = round(
            result["fewhead"]["gathered_kv_GBps"] / fc_ceil["GBps"], 4)
        print(f"[bench] fewhead {f_med[0]:.1f} us (64 heads: {pct(t64)[0]:.1f} us)", file=sys.stderr, flush=True)

        def few8():
            smla.prefill(fq[:, :fc.H], f8pool, fidx, topk_length=ftl, sink=fsink64[:fc.H],
                         sm_scale=float(fc.sm_scale), out=fout[:, :fc.H], lse=flse[:, :fc.H])

        few8()
        t8f = pct(event_times_us(torch, few8, iters, stream))
        f8bytes = frows * W.ROW_BYTES[W.FMT_FP8]
        result["fewhead"]["fp8_rows"] = {
            "workload": "the same prefill over an FP8 pool written from the same latent rows (656-byte rows)",
            "kernel_us_median_p10_p90": [round(v, 3) for v in t8f],
            "gathered_kv_bytes": f8bytes,
            "gathered_kv_GBps": round(f8bytes / (t8f[0] * 1e-6) / 1e9, 2),
        }
        print(f"[bench] fewhead over FP8 rows {t8f[0]:.1f} us", file=sys.stderr, flush=True)
        del fq, fpool, f8pool, fidx, ftl, fout, flse
        torch.cuda.empty_cache()
        result["int8"] = int8_line(torch, smla, W, dev, stream, bf16, iters)
        torch.cuda.empty_cache()

    # ---------------- DOTS3_SWA rows ----------------
    if not args.no_extra:
        result["dots3"] = dots3_lines(torch, smla, W, dev, stream, bf16, args)

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = n
        del src, dst

    # ---------------- CPU baseline: the oracle on a bounded sample ----------------
    if not args.no_cpu:
        import oracle
        ncores = min(16, os.cpu_count() or 1)
        pool_h = oracle.Pool(np.zeros((case.num_blocks, 64 * 656), np.uint8), W.FMT_FP8, 64 * 656)
        oracle.quantize_kv(case.kv, case.slots, pool_h)
        n = min(args.cpu_tokens, T) if args.cpu_tokens > 0 else T
        tokens = np.linspace(0, T - 1, n).astype(np.int64)
        tc = time.perf_counter()
        oracle.prefill(case.q, pool_h, case.indices, sm_scale=case.sm_scale, tokens=tokens, nthreads=ncores)
        cpu_s = time.perf_counter() - tc
        result["cpu_baseline"] = {
            "value": round(cpu_s * 1e6 / n, 3), "unit": "us/token", "cores": ncores, "kind": "oracle",
            "host": {"cpu_model": host_cpu_model(), "visible_cpus": os.cpu_count()},
            "sample": (f"all {T} tokens" if n == T else f"{n} of the {T} tokens") +
                      f" of the same prefill workload (float64 C oracle, OpenMP over tokens), {cpu_s:.2f} s wall"}
        print(f"[bench] cpu oracle {cpu_s:.2f}s for {n} tokens on {ncores} threads", file=sys.stderr, flush=True)
        # the tiny BF16 case on one thread (prefill and decode at 1, 2 and 4 splits)
        c1 = W.c1_tiny()
        p1 = oracle.Pool(np.zeros((c1.num_blocks, 64 * 1152), np.uint8), W.FMT_BF16, 64 * 1152)
        oracle.quantize_kv(c1.kv, c1.slots, p1)
        tc = time.perf_counter()
        oracle.prefill(c1.q, p1, c1.indices, sm_scale=c1.sm_scale, nthreads=1)
        for S in (1, 2, 4):
            oracle.decode_split(c1.q, p1, c1.indices, S, sm_scale=c1.sm_scale, nthreads=1)
        result["cpu_baseline"]["c1_tiny_single_thread_ms"] = round((time.perf_counter() - tc) * 1e3, 3)
        if not args.no_extra:
            result["cpu_baseline"]["other_workloads"] = cpu_other_workloads(W, oracle, ncores)


    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
