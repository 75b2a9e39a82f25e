"""Throughput of the dynamic-mask attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input already
resident in HBM: block classification, forward (O, LSE) and backward (dQ, dK, dV,
dBias), through the C ABI on the current stream.  By default the classification runs
fused into the forward (dma_attn_fwd_classify: each live block's mask tile is read once,
reduced to its class and applied); --separate-classify times dma_block_classify +
dma_attn_fwd instead.  The other path is timed in the same run (``classify_other``;
left out with --no-next).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config headline]

Prints one JSON line.  ``value`` is the effective fwd+bwd TFLOP/s of the step:
MMA FLOPs over the non-SKIP 64x64 blocks (4*d per block element per query head
forward, 10*d backward; FlashMask README, Performance: theoretical FLOPs count
only the core matrix multiplies) divided by the time of the whole step,
classification included.

``next_rows`` (outside the step, skipped with --no-next): the GPU top-k mask construction on a
fresh N(0,1) bias of the workload's shape; the step with the bit-packed PARTIAL-block mask
instead of the bf16 mask, per phase; and one classify + forward + backward of the Doc-packed
workload with the dense mask and with column ranges.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-classify", action="store_true",
                    help="time dma_block_classify + dma_attn_fwd instead of the fused dma_attn_fwd_classify")
    ap.add_argument("--no-next", action="store_true", help="skip the next-row measurements (top-k construction)")
    ap.add_argument("--cpu-blocks", type=int, default=16, help="query-row blocks the oracle times")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one device copy of this many MiB before the steps, so that a hardware counter "
                         "pass can relate its FETCH_SIZE / WRITE_SIZE to known bytes")
    ap.add_argument("--traffic-json", default=TRAFFIC_JSON,
                    help="measured HBM bytes per launch (written by --summarize-traffic); used only while the "
                         "kernel sources still hash to the value recorded in it")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("COUNTER_DIR", "OUT_JSON"), default=None,
                    help="turn two rocprofv3 counter passes (FETCH_SIZE and WRITE_SIZE csv files under "
                         "COUNTER_DIR, each over a run with --calibrate-copy-mib N; give the same N here) into "
                         "bytes per launch, then exit")
    return ap.parse_args()


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "headline_traffic.json")
KERNEL_SOURCES = ["classify.hip", "fwd.hip", "bwd.hip", "common.h"]
# kernels of each C-ABI call, matched by substring of the demangled name
CALL_KERNELS = {"classify": ["classify_kernel"], "fwd": ["fwd_kernel"],
                "bwd": ["bwd_pre_kernel", "kt_kernel", "pair_base_kernel", "bwd_main_kernel", "dq_kernel"]}


def kernel_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_dynamic_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def summarize_traffic(counter_dir: str, out_json: str, copy_mib: int):
    """HBM bytes per launch of each call from FETCH_SIZE / WRITE_SIZE (KiB per dispatch).

    Each counter is scaled by the ratio of known bytes to what it reads for the calibration
    copy (a device copy of --calibrate-copy-mib MiB: that many bytes fetched and written)."""
    import csv
    import glob
    from collections import defaultdict

    assert copy_mib > 0, "give the calibration copy's size with --calibrate-copy-mib"
    out = {"source_hash": kernel_source_hash(), "calibration_mib": copy_mib, "counters": {}}
    per_call = defaultdict(float)
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        files = glob.glob(os.path.join(counter_dir, "**", f"{counter}_counter_collection.csv"), recursive=True)
        assert len(files) == 1, f"expected one {counter} csv under {counter_dir}, found {files}"
        per = defaultdict(list)
        for r in csv.DictReader(open(files[0])):
            if r["Counter_Name"] == counter:
                per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        copy = [max(v) for k, v in per.items() if "copy" in k.lower() or "elementwise" in k.lower()]
        assert copy, "no calibration copy kernel in the counter pass"
        copy_kib = max(copy)
        factor = copy_mib * 1024.0 / copy_kib
        out["counters"][counter] = {"copy_kib": copy_kib, "factor": factor}
        for call, subs in CALL_KERNELS.items():
            for name, vals in per.items():
                if any(sub in name for sub in subs):
                    per_call[call] += sum(vals) / len(vals) * 1024.0 * factor
    out["bytes_per_launch"] = {k: round(v) for k, v in per_call.items()}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def block_counts(state):
    import torch

    n_skip = int((state == 0).sum())
    n_p = int((state == 1).sum())
    n_f = int((state == 2).sum())
    return n_skip, n_p, n_f


def cpu_baseline(c, blocks: int, f_total: float):
    """Oracle (fp64 numpy) on a bounded sample: `blocks` 64-row query blocks of the workload,
    forward and backward, extrapolated to the whole workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    import synth

    sample = synth.sample_row_blocks(c, blocks)
    k = oracle.bf16_to_f64(synth.k(c))
    v = oracle.bf16_to_f64(synth.v(c))
    t_total = 0.0
    for (bb, r0) in sample:
        rows = np.arange(r0, min(r0 + 64, c.lq))
        qr = oracle.bf16_to_f64(synth.rows_of(c, synth.TAG_Q, c.hq, bb, rows))
        dor = oracle.bf16_to_f64(synth.rows_of(c, synth.TAG_DO, c.hq, bb, rows))
        ms, bs = [], []
        for g in range(c.hkv):
            m, b = synth.mask_bias_rows(c, bb, g, int(rows[0]), len(rows))
            ms.append(m)
            bs.append(b)
        mask = None if ms[0] is None else np.stack(ms)
        bias = None if bs[0] is None else oracle.bf16_to_f64(np.stack(bs))
        t0 = time.perf_counter()
        oracle.forward_rows(qr, k[bb], v[bb], mask, bias, c.scale_f32, c.causal, rows, c.lq)
        oracle.backward_rows(qr, k[bb], v[bb], mask, bias, c.scale_f32, c.causal, rows, c.lq, dor)
        t_total += time.perf_counter() - t0
    n_blocks_all = c.b * ((c.lq + 63) // 64)
    t_whole = t_total / len(sample) * n_blocks_all
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": round(f_total / t_whole / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(sample)} seeded 64-row query blocks (all {c.hq} heads, fwd+bwd) of {n_blocks_all}, "
                  f"{t_total:.1f} s, extrapolated to the whole workload ({t_whole:.0f} s)",
    }


def time_ranges(args, dma, synth, np):
    import torch
    from synth.device import upload_dense, upload_mask_bias

    c = synth.CASES["docpacked"]
    q, k, v, do = upload_dense(c)
    mask, bias = upload_mask_bias(c)
    bounds = synth.doc_bounds(c)
    j = np.arange(c.lk)
    end = bounds[np.searchsorted(bounds, j, side="right")]
    rs = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(j, (c.b, c.hkv, c.lk)).astype(np.int32))).cuda()
    re = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(end, (c.b, c.hkv, c.lk)).astype(np.int32))).cuda()
    st = torch.empty(dma.block_state_shape(c.b, c.hkv, c.lq, c.lk), dtype=torch.uint8, device="cuda")
    o, lse = torch.empty_like(q), torch.empty((c.b, c.hq, c.lq), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dbias = torch.empty((c.b, c.hkv, c.lq, c.lk), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(dma.dma_attn_bwd_workspace_size(c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.causal), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def step(ranges):
        if ranges:
            dma.dma_block_classify_ranges(rs, re, c.b, c.hkv, c.lq, c.lk, c.causal, st, stream)
            dma.dma_attn_fwd_ranges(q, k, v, rs, re, bias, st, c.scale_f32, c.causal, o, lse, stream)
            dma.dma_attn_bwd_ranges(q, k, v, rs, re, bias, st, o, do, lse, c.scale_f32, c.causal, dq, dk, dv, dbias,
                                    ws, stream)
        else:
            dma.dma_block_classify(mask, c.b, c.hkv, c.lq, c.lk, c.causal, st, stream)
            dma.dma_attn_fwd(q, k, v, mask, bias, st, c.scale_f32, c.causal, o, lse, stream)
            dma.dma_attn_bwd(q, k, v, mask, bias, st, o, do, lse, c.scale_f32, c.causal, dq, dk, dv, dbias, ws, stream)

    out = {"workload": f"{c.name}: b={c.b} L={c.lq} Hq={c.hq} Hkv={c.hkv} d={c.d} document mask, causal"}
    for ranges in (False, True):
        step(ranges)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        e0.record(stream)
        for _ in range(reps):
            step(ranges)
        e1.record(stream)
        torch.cuda.synchronize()
        out["ranges_ms" if ranges else "dense_ms"] = round(e0.elapsed_time(e1) / reps, 4)
    n_p = int((st == 1).sum())
    n_f = int((st == 2).sum())
    live = int(((st == 1) | (st == 2)).sum())
    G = c.hq // c.hkv
    flops = 14.0 * c.d * 64 * 64 * G * (n_p + n_f)
    # mandatory HBM bytes: bias (+ mask) of non-SKIP blocks in the forward and the backward, the
    # mask scan of classification, all of dBias; the range path reads 8 B per key and plane
    n_live_blocks = int(((np.arange((c.lq + 63) // 64)[:, None] * 64 + 63 + (c.lk - c.lq)) >=
                         (np.arange((c.lk + 63) // 64)[None, :] * 64)).sum()) * c.b * c.hkv
    bias_b = 2.0 * 64 * 64 * (n_p + n_f)
    mask_b = 2.0 * 64 * 64 * n_p
    dbias_b = 2.0 * c.b * c.hkv * c.lq * c.lk
    out["bytes_dense"] = 2.0 * 64 * 64 * n_live_blocks + 2 * (bias_b + mask_b) + dbias_b
    out["bytes_ranges"] = 8.0 * c.b * c.hkv * c.lk + 2 * bias_b + dbias_b
    out["tflops_dense"] = round(flops / (out["dense_ms"] * 1e-3) / 1e12, 2)
    out["tflops_ranges"] = round(flops / (out["ranges_ms"] * 1e-3) / 1e12, 2)
    out["gbs_ranges"] = round(out["bytes_ranges"] / (out["ranges_ms"] * 1e-3) / 1e9, 1)
    out["blocks_partial"], out["blocks_full"] = n_p, n_f
    del q, k, v, do, mask, bias, dbias, ws
    torch.cuda.empty_cache()
    return out


def time_classify_other(c, dma, np, torch, classify_forward, fused, t_bwd, reps=5):
    """Classification + forward by the path the step does not use (run with `not fused`)."""
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    classify_forward(fused)
    torch.cuda.synchronize()
    for r in range(reps):
        classify_forward(fused, ev[r])
    torch.cuda.synchronize()
    po = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])] for e in ev]).mean(axis=0)
    return {"path": "separate dma_block_classify + dma_attn_fwd" if fused else "fused dma_attn_fwd_classify",
            "classify_ms": round(float(po[0]), 4), "fwd_ms": round(float(po[1]), 4),
            "classify_fwd_ms": round(float(po.sum()), 4), "step_ms_with_it": round(float(po.sum()) + t_bwd, 4)}


def time_bits(c, dma, np, q, k, v, do, mask, bias, o, lse, dq, dk, dv, dbias, ws, stream, dense_ms):
    import torch

    st = torch.empty(dma.block_state_shape(c.b, c.hkv, c.lq, c.lk), dtype=torch.uint8, device="cuda")
    mb = torch.empty((dma.dma_mask_bits_size(c.b, c.hkv, c.lq, c.lk),), dtype=torch.uint8, device="cuda")
    reps = 3
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps + 1)]
    for r in range(reps + 1):  # the first repetition warms up
        e = ev[r]
        e[0].record(stream)
        dma.dma_block_classify_bits(mask, c.b, c.hkv, c.lq, c.lk, c.causal, st, mb, stream)
        e[1].record(stream)
        dma.dma_attn_fwd_bits(q, k, v, mb, bias, st, c.scale_f32, c.causal, o, lse, stream)
        e[2].record(stream)
        dma.dma_attn_bwd_bits(q, k, v, mb, bias, st, o, do, lse, c.scale_f32, c.causal, dq, dk, dv, dbias, ws, stream)
        e[3].record(stream)
    torch.cuda.synchronize()
    t = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])] for e in ev[1:]])
    t = t.mean(axis=0)
    n_p = int((st == 1).sum())
    out = {"classify_ms": round(float(t[0]), 4), "fwd_ms": round(float(t[1]), 4), "bwd_ms": round(float(t[2]), 4),
           "step_ms": round(float(t.sum()), 4), "dense_step_ms": round(float(sum(dense_ms)), 4),
           "blocks_partial": n_p,
           # mask bytes read by forward + backward: bf16 tiles of the dense path, bits here
           "mask_bytes_dense": 2 * 2.0 * 64 * 64 * n_p, "mask_bytes_bits": 2 * 512.0 * n_p,
           "bits_bytes_written": 512.0 * n_p}
    del st, mb
    return out


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.calibrate_copy_mib)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (each (batch, kv head) plane "
              "is independent, so several GPUs would each run this one-GPU kernel on their share).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_sparse_dynamic_amd as dma
    import synth
    from synth.device import upload_dense, upload_mask_bias

    c = synth.CASES[args.config]
    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    q, k, v, do = upload_dense(c)
    mask, bias = upload_mask_bias(c)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] {c.name}: inputs generated and uploaded in {t_gen:.1f} s", file=sys.stderr, flush=True)

    state = torch.empty(dma.block_state_shape(c.b, c.hkv, c.lq, c.lk), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((c.b, c.hq, c.lq), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dbias = torch.empty((c.b, c.hkv, c.lq, c.lk), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(dma.dma_attn_bwd_workspace_size(c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.causal), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    fused = not args.separate_classify

    def classify_forward(separate, timed=None):
        if timed is not None:
            timed[0].record(stream)
        if separate:
            dma.dma_block_classify(mask, c.b, c.hkv, c.lq, c.lk, c.causal, state, stream)
        if timed is not None:
            timed[1].record(stream)
        if separate:
            dma.dma_attn_fwd(q, k, v, mask, bias, state, c.scale_f32, c.causal, o, lse, stream)
        else:
            dma.dma_attn_fwd_classify(q, k, v, mask, bias, c.scale_f32, c.causal, state, o, lse, stream)
        if timed is not None:
            timed[2].record(stream)

    def step(timed=None):
        classify_forward(not fused, timed)
        dma.dma_attn_bwd(q, k, v, mask, bias, state, o, do, lse, c.scale_f32, c.causal, dq, dk, dv, dbias, ws,
                         stream)
        if timed is not None:
            timed[3].record(stream)

    if args.calibrate_copy_mib > 0:  # one plain copy of known size, for counter calibration
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    per = np.zeros((args.steps, 3))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for s in range(args.steps):
        e = evs[s]
        per[s] = [e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])]
    t_cls, t_fwd, t_bwd = per.mean(axis=0)  # ms
    ms_step = wall / args.steps * 1e3

    # the other classification path (separate pass or fused), outside the step, same inputs
    # (left out of counter and trace runs, --no-next, which must hold the step's kernels only)
    classify_other = None
    if not args.no_next and args.calibrate_copy_mib == 0:
        classify_other = time_classify_other(c, dma, np, torch, classify_forward, fused, t_bwd)


    # Next-row measurement, outside the step: the top-k mask construction (dma_topk_mask) on
    # a fresh N(0,1) bf16 bias of the workload's shape, k = the workload's top-k.
    next_rows = {}
    if c.mask == "topk" and not args.no_next and args.calibrate_copy_mib == 0:
        gen = torch.Generator(device="cuda").manual_seed(1234)
        raw = torch.randn((c.b * c.hkv * c.lq, c.lk), generator=gen, device="cuda").to(torch.bfloat16)
        mk, bo = torch.empty_like(raw), torch.empty_like(raw)
        dma.dma_topk_mask(raw, c.topk, mk, bo, stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        e0.record(stream)
        for _ in range(reps):
            dma.dma_topk_mask(raw, c.topk, mk, bo, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        t_topk = e0.elapsed_time(e1) / reps
        bytes_topk = 3.0 * raw.numel() * 2  # bias read once, mask and bias written
        next_rows["topk_mask"] = {"ms": round(t_topk, 4), "gbs": round(bytes_topk / (t_topk * 1e-3) / 1e9, 1),
                                  "frac_hbm": round(bytes_topk / (t_topk * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                  "rows": c.b * c.hkv * c.lq, "lk": c.lk, "k": c.topk}
        del raw, mk, bo

    # Next-row measurement, outside the step: the same step with the bit-packed PARTIAL-block
    # mask (classification writes 512 B per PARTIAL block; forward and backward read those bits
    # instead of the bf16 mask), per phase over a few repetitions.
    if c.mask != "none" and not args.no_next and args.calibrate_copy_mib == 0:
        next_rows["mask_bits"] = time_bits(c, dma, np, q, k, v, do, mask, bias, o, lse, dq, dk, dv, dbias, ws,
                                           stream, (t_cls, t_fwd, t_bwd))

    # Next-row measurement, outside the step: column-range mask input on the Doc-packed workload
    # (the pages' column-wise form), one classify + forward + backward with the dense mask and
    # with the ranges, each timed over a few repetitions.
    if not args.no_next and args.calibrate_copy_mib == 0:
        next_rows["column_ranges"] = time_ranges(args, dma, synth, np)

    n_skip, n_p, n_f = block_counts(state)
    n_ns = n_p + n_f
    G, d = c.hq // c.hkv, c.d
    f_fwd = 4.0 * d * 64 * 64 * G * n_ns
    f_bwd = 10.0 * d * 64 * 64 * G * n_ns
    # blocks wholly excluded by causality are never read by classification
    nqb, nkb = (c.lq + 63) // 64, (c.lk + 63) // 64
    qb = np.arange(nqb)[:, None]
    kb = np.arange(nkb)[None, :]
    live = (kb * 64 <= np.minimum(qb * 64 + 63, c.lq - 1) + (c.lk - c.lq)) if c.causal else np.ones((nqb, nkb), bool)
    n_live = int(live.sum()) * c.b * c.hkv
    has_mask = mask is not None
    # a separate classification reads the mask of every causally live block once more; fused,
    # the forward's own mask reads classify
    b_cls = 2.0 * 64 * 64 * n_live if (has_mask and not fused) else 0.0
    b_fwd = 2.0 * 64 * 64 * (2 * n_p + n_f)
    b_bwd = b_fwd + 2.0 * c.b * c.hkv * c.lq * c.lk
    tflops = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    gbs = (b_cls + b_fwd + b_bwd) / (ms_step * 1e-3) / 1e9

    # dominant launch: the one with the largest share of the step
    phases = {"bwd": (t_bwd, f_bwd, "dma_attn_bwd (bwd_pre + kt + pair_base + bwd_main + dq)"),
              "fwd": (t_fwd, f_fwd, "dma_attn_fwd_classify (fwd_kernel, classification fused)" if fused else
                      "dma_attn_fwd (fwd_kernel)")}
    dom = max(phases, key=lambda k: phases[k][0])
    t_dom, f_dom, dom_name = phases[dom]
    achieved = f_dom / (t_dom * 1e-3) / 1e12
    traffic = None  # measured HBM bytes per launch, only while the kernels are the ones measured
    if args.traffic_json and os.path.exists(args.traffic_json):
        with open(args.traffic_json) as f:
            tj = json.load(f)
        if tj.get("source_hash") == kernel_source_hash():
            traffic = tj["bytes_per_launch"].get(dom)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic, "kernel": dom_name,
                "ms_per_launch": round(t_dom, 4)}

    line = {
        "metric": "fwd+bwd effective TFLOP/s (unmasked tiles) + HBM GB/s, L=16K GQA top-k",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; N(0,1) q/k/v/dO/bias, top-k mask from the bias)",
        "config": {"workload": f"{c.name}: b={c.b} L={c.lq} Hq={c.hq} Hkv={c.hkv} d={c.d} "
                               f"{'top-k ' + str(c.topk) if c.mask == 'topk' else c.mask} mask, "
                               f"{'causal' if c.causal else 'non-causal'}",
                   "b": c.b, "seq_len": c.lq, "hq": c.hq, "hkv": c.hkv, "d": c.d,
                   "blocks_nonskip": n_ns, "blocks_partial": n_p, "blocks_full": n_f, "blocks_skip": n_skip},
        "hbm_gbs_mandatory": round(gbs, 1),
        "classify_fused": fused,
        "phases_ms": {"classify": round(t_cls, 4), "fwd": round(t_fwd, 4), "bwd": round(t_bwd, 4)},
        "phases_tflops": {"fwd": round(f_fwd / (t_fwd * 1e-3) / 1e12, 2),
                          "bwd": round(f_bwd / (t_bwd * 1e-3) / 1e12, 2)},
        "phases_gbs_mandatory": {"classify": round(b_cls / (t_cls * 1e-3) / 1e9, 1) if b_cls > 0 else None,
                                 "fwd": round(b_fwd / (t_fwd * 1e-3) / 1e9, 1),
                                 "bwd": round(b_bwd / (t_bwd * 1e-3) / 1e9, 1)},
        "roofline": roofline,
        "classify_other": classify_other,
        "next_rows": next_rows,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(c, args.cpu_blocks, f_fwd + f_bwd)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
