"""Measure the split-KV decode, the combine and the prefill form over a grid
of shapes on the current GPU, and fit the constants of the split-count cost
model in csrc/split_model.cpp.

FlashInfer PR #4802 ("cpb model") chooses its split geometry from a closed
form over a few hardware constants, fitted once per device from timings over
an HBM-sized pool with uniform indices, so that the working set is not
cache-resident.  This script does the same for this library's kernels:

    decode(T, H, topk, S) = waves * (a + b * tiles_per_block + f * splits_per_block)
                            + w * partial_MB
    combine(T, H, S)      = c0 + c1 * partial_MB + c2 * T * H / 1000
    prefill(T, H, topk)   = ap0 + waves_p * (ap + bp * tiles_per_token)

with a, b, f, ap0, ap, bp per kernel class (row format x kernel: many-head,
column-split or exponent-byte), w and c0..c2 shared, all in microseconds.  waves counts rounds of
workgroups over the compute units at the kernel's occupancy.

Usage (needs a GPU; writes JSON to stdout or --out):
    python -m sparse_top_mla_smla_amd.calibrate_splits --out split_model.json
    # add classes to a fit, holding its shared constants (w, combine):
    python -m sparse_top_mla_smla_amd.calibrate_splits --classes dots3_mx,dsv4_mx \
        --extend split_model_fit.json --out split_model_fit.json
"""
import argparse
import json
import math
import sys

import numpy as np
import torch

import sparse_top_mla_smla_amd as smla
from sparse_top_mla_smla_amd import workloads as W

POOL_ROWS = 1 << 20  # 16384 blocks: 584 MiB to 1.2 GiB, beyond the last-level cache

# kernel class -> (format, head counts measured, workgroups per CU per round,
# heads per block).  FP8, INT8 and DSv4 rows with more than 16 heads run the
# same many-head kernel ("wide": 64 heads per workgroup); the classes differ
# in the codes' conversion and the row layout.  With 16 or fewer heads, and
# for BF16 rows at every H, the kernel that splits PV over value columns
# runs (two workgroups per CU); arbitrary-scale FP8 rows share the INT8
# class.  The exponent-byte kernel runs DSv4 rows with 16 or fewer heads
# (16 heads per workgroup, two workgroups per CU) and DOTS3_SWA rows at any
# H (16 heads per workgroup, its 32-head kernel above 16 heads).
CLASSES = {
    "fp8_wide": (W.FMT_FP8, (64, 128), 1, 64),
    "int8_wide": (W.FMT_INT8, (64, 128), 1, 64),
    "dsv4_wide": (W.FMT_FP8_DSV4, (64, 128), 1, 64),
    "fp8_cols": (W.FMT_FP8, (8, 16), 2, 16),
    "int8_cols": (W.FMT_INT8, (8, 16), 2, 16),
    "bf16_cols": (W.FMT_BF16, (8, 64), 2, 16),
    "dots3_mx": (W.FMT_FP8_DOTS3, (8, 16), 1, 16),
    "dots3_mx32": (W.FMT_FP8_DOTS3, (32, 64), 1, 32),
    "dsv4_mx": (W.FMT_FP8_DSV4, (8, 16), 2, 16),
}
# classes whose decode workgroups run consecutive splits of a token (the
# many-head kernel)
GROUPED = ("fp8_wide", "int8_wide", "dsv4_wide")
T_GRID = (1, 2, 4, 8, 16, 32, 64, 128, 256)
T_PREFILL_ONLY = (1024,)  # several tokens per workgroup in the persistent prefill
TOPK_GRID = (512, 2048)
S_GRID = (1, 2, 4, 8, 16, 32)


def partial_mb(cls: str, T: int, S: int, H: int) -> float:
    """MB of decode partials: T*S*H rows of d_v FP32 values and an LSE."""
    return T * S * H * (W.V_DIMS[CLASSES[cls][0]] * 4 + 4) / 1e6


def geometry(cls: str, T: int, H: int, topk: int, S: int, cus: int):
    """(waves, tiles of the longest block, splits per block, partial MB) of
    a decode launch, following the launchers' grid rules."""
    _, _, occ, hpb = CLASSES[cls]
    hb = (H + hpb - 1) // hpb
    w = smla.split_width(topk, S)
    spb = 1
    if cls in GROUPED:
        spb = max(1, min(S, (T * hb * S) // cus))
    blocks = T * hb * ((S + spb - 1) // spb)
    waves = math.ceil(blocks / (cus * occ))
    tiles = math.ceil(min(spb * w, topk) / 64)
    return waves, tiles, spb, partial_mb(cls, T, S, H)


def prefill_geometry(cls: str, T: int, H: int, topk: int, cus: int):
    _, _, occ, hpb = CLASSES[cls]
    hb = (H + hpb - 1) // hpb
    return math.ceil(T * hb / (cus * occ)), math.ceil(topk / 64)


def timed(fn, sets, warmup=3, iters=9):
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = []
    for it in range(warmup + iters):
        x = sets[it % len(sets)]
        ev0.record()
        fn(x)
        ev1.record()
        torch.cuda.synchronize()
        if it >= warmup:
            out.append(ev0.elapsed_time(ev1) * 1000.0)
    return float(np.median(out))


def measure(cus: int, log, classes=None):
    classes = list(classes or CLASSES)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    pools = {}
    for fmt in sorted({CLASSES[c][0] for c in classes}):
        pool = smla.KVPool.empty(POOL_ROWS // 64, fmt)
        for r0 in range(0, POOL_ROWS, 1 << 18):
            kv = torch.randn((1 << 18, W.KV_DIMS[fmt]), generator=gen, device="cuda").to(torch.bfloat16)
            slots = torch.arange(r0, r0 + (1 << 18), dtype=torch.int32, device="cuda")
            smla.quantize_kv(kv, slots, pool)
        pools[fmt] = pool
    torch.cuda.synchronize()
    rows = []
    for cls in classes:
        fmt, heads, _, _ = CLASSES[cls]
        dq, dv = W.KV_DIMS[fmt], W.V_DIMS[fmt]
        for H in heads:
            for topk in TOPK_GRID:
                for T in T_GRID + T_PREFILL_ONLY:
                    q = torch.randn((T, H, dq), generator=gen, device="cuda").to(torch.bfloat16)
                    sets = [torch.randint(0, POOL_ROWS, (T, topk), generator=gen, device="cuda", dtype=torch.int32)
                            for _ in range(3)]
                    out = torch.empty((T, H, dv), dtype=torch.bfloat16, device="cuda")
                    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
                    pool = pools[fmt]
                    tp = timed(lambda x: smla.prefill(q, pool, x, out=out, lse=lse), sets)
                    rows.append(dict(kind="prefill", cls=cls, T=T, H=H, topk=topk, us=tp))
                    for S in S_GRID:
                        if S > topk // 64 or T not in T_GRID:
                            continue
                        po = torch.empty((T, S, H, dv), dtype=torch.float32, device="cuda")
                        pl = torch.empty((T, S, H), dtype=torch.float32, device="cuda")
                        td = timed(lambda x: smla.decode(q, pool, x, S, part_out=po, part_lse=pl), sets)
                        tc = timed(lambda x: smla.combine(po, pl, out=out, lse=lse), [None])
                        rows.append(dict(kind="decode", cls=cls, T=T, H=H, topk=topk, S=S, us=td, combine_us=tc))
                    log(f"{cls} H={H} topk={topk} T={T}: prefill {tp:.1f} us")
    return rows


def fit(rows, cus: int):
    """Least-squares constants; a negative fitted term is clamped to 0 and
    the rest refit (the NNLS step of FlashInfer PR #4802's calibration)."""
    def lsq(X, y):
        X = np.asarray(X, float)
        y = np.asarray(y, float)
        active = list(range(X.shape[1]))
        coef = np.zeros(X.shape[1])
        while active:
            c, *_ = np.linalg.lstsq(X[:, active], y, rcond=None)
            if (c >= 0).all():
                coef[active] = c
                break
            active.pop(int(np.argmin(c)))
        return coef

    dec = [r for r in rows if r["kind"] == "decode"]
    # shared partial-write cost and per-class block constants, fitted jointly
    classes = list(CLASSES)
    X, y = [], []
    for r in dec:
        waves, tiles, spb, mb = geometry(r["cls"], r["T"], r["H"], r["topk"], r["S"], cus)
        k = classes.index(r["cls"])
        row = [0.0] * (3 * len(classes) + 1)
        row[3 * k + 0] = waves
        row[3 * k + 1] = waves * tiles
        row[3 * k + 2] = waves * spb
        row[-1] = mb
        X.append(row)
        y.append(r["us"])
    c = lsq(X, y)
    consts = {cls: dict(a=c[3 * k], b=c[3 * k + 1], f=c[3 * k + 2]) for k, cls in enumerate(classes)}
    w = c[-1]
    Xc = [[1.0, partial_mb(r["cls"], r["T"], r["S"], r["H"]), r["T"] * r["H"] / 1000.0] for r in dec]
    cc = lsq(Xc, [r["combine_us"] for r in dec])
    for cls in classes:
        pre = [r for r in rows if r["kind"] == "prefill" and r["cls"] == cls]
        Xp = []
        for r in pre:
            waves, tiles = prefill_geometry(cls, r["T"], r["H"], r["topk"], cus)
            Xp.append([1.0, waves, waves * tiles])
        cp = lsq(Xp, [r["us"] for r in pre])
        consts[cls].update(ap0=cp[0], ap=cp[1], bp=cp[2])
    return dict(classes=consts, w_us_per_MB=w, combine=dict(c0=cc[0], c1=cc[1], c2=cc[2]))


def fit_classes(rows, cus: int, base):
    """Constants of the classes in `rows` with the shared partial-write and
    combine constants of the fitted model `base` held fixed."""
    def nnls(X, y):
        X = np.asarray(X, float)
        y = np.asarray(y, float)
        active = list(range(X.shape[1]))
        coef = np.zeros(X.shape[1])
        while active:
            c, *_ = np.linalg.lstsq(X[:, active], y, rcond=None)
            if (c >= 0).all():
                coef[active] = c
                break
            active.pop(int(np.argmin(c)))
        return coef

    consts = {}
    for cls in sorted({r["cls"] for r in rows}):
        X, y = [], []
        for r in rows:
            if r["kind"] == "decode" and r["cls"] == cls:
                waves, tiles, spb, mb = geometry(cls, r["T"], r["H"], r["topk"], r["S"], cus)
                X.append([waves, waves * tiles, waves * spb])
                y.append(r["us"] - base["w_us_per_MB"] * mb)
        c = nnls(X, y)
        Xp, yp = [], []
        for r in rows:
            if r["kind"] == "prefill" and r["cls"] == cls:
                waves, tiles = prefill_geometry(cls, r["T"], r["H"], r["topk"], cus)
                Xp.append([1.0, waves, waves * tiles])
                yp.append(r["us"])
        cp = nnls(Xp, yp)
        consts[cls] = dict(a=c[0], b=c[1], f=c[2], ap0=cp[0], ap=cp[1], bp=cp[2])
    return consts


def predict_prefill(model, cls, T, H, topk, cus):
    k = model["classes"][cls]
    waves, tiles = prefill_geometry(cls, T, H, topk, cus)
    return k["ap0"] + waves * (k["ap"] + k["bp"] * tiles)


def predict(model, cls, T, H, topk, S, cus):
    k = model["classes"][cls]
    waves, tiles, spb, mb = geometry(cls, T, H, topk, S, cus)
    dec = waves * (k["a"] + k["b"] * tiles + k["f"] * spb) + model["w_us_per_MB"] * mb
    cm = model["combine"]
    com = cm["c0"] + cm["c1"] * partial_mb(cls, T, S, H) + cm["c2"] * T * H / 1000.0
    return dec + com


def evaluate(model, rows, cus):
    """Pick error of the model against the measured best split count, per
    (class, T, H, topk): measured time of the model's pick / measured best."""
    groups = {}
    for r in rows:
        if r["kind"] == "decode":
            groups.setdefault((r["cls"], r["T"], r["H"], r["topk"]), {})[r["S"]] = r["us"] + r["combine_us"]
    ratios = []
    for (cls, T, H, topk), by_s in groups.items():
        pick = min(by_s, key=lambda S: (predict(model, cls, T, H, topk, S, cus), S))
        ratios.append(by_s[pick] / min(by_s.values()))
    return dict(mean=float(np.mean(ratios)), max=float(np.max(ratios)), shapes=len(ratios))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", default="", help="write the JSON here instead of stdout")
    ap.add_argument("--refit", default="", metavar="JSON",
                    help="fit again from the measurements stored in a JSON this script wrote (no GPU)")
    ap.add_argument("--classes", default="", help="comma-separated kernel classes to measure (default: all)")
    ap.add_argument("--extend", default="", metavar="JSON",
                    help="add the measured classes to this fit, holding its shared constants")
    args = ap.parse_args()
    if args.extend:
        with open(args.extend) as f:
            old = json.load(f)
        cus = old["compute_units"]
        assert cus == torch.cuda.get_device_properties(0).multi_processor_count
        classes = [c for c in args.classes.split(",") if c]
        new_rows = measure(cus, lambda s: print(s, file=sys.stderr, flush=True), classes)
        model = old["model"]
        # classes no longer in CLASSES (a kernel replaced) leave the fit
        model["classes"] = {c: v for c, v in model["classes"].items() if c in CLASSES}
        model["classes"].update(fit_classes(new_rows, cus, model))
        rows = [r for r in old["rows"] if r["cls"] not in classes and r["cls"] in CLASSES] + new_rows
        res = dict(device=old["device"], compute_units=cus, model=model, pick_error=evaluate(model, rows, cus),
                   rows=rows)
        text = json.dumps(res, indent=1)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text)
        else:
            print(text)
        return
    if args.refit:
        with open(args.refit) as f:
            old = json.load(f)
        device, cus, rows = old["device"], old["compute_units"], old["rows"]
    else:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        device = torch.cuda.get_device_name(0) or "gpu"
        rows = measure(cus, lambda s: print(s, file=sys.stderr, flush=True))
    model = fit(rows, cus)
    res = dict(device=device, compute_units=cus, model=model, pick_error=evaluate(model, rows, cus), rows=rows)
    text = json.dumps(res, indent=1)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    else:
        print(text)


if __name__ == "__main__":
    main()
