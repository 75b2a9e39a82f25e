"""Throughput of the dynamic-mask attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input already
resident in HBM: block classification, forward (O, LSE) and backward (dQ, dK, dV,
dBias), through the C ABI on the current stream.  The classification runs fused
into the forward (dma_attn_fwd_classify: each live block's mask tile is read once,
reduced to its class and applied); the backward is called as its three phases
(dma_attn_bwd_part: prepare, main, dQ, which together are dma_attn_bwd) so that
HIP events can bracket the main kernel.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config headline]

Prints one JSON line.  ``value`` is the effective fwd+bwd TFLOP/s of the step on
the Headline workload: MMA FLOPs over the non-SKIP 64x64 blocks (4*d per block
element per query head forward, 10*d backward; FlashMask README, Performance:
theoretical FLOPs count only the core matrix multiplies) divided by the wall time
of K steps (synchronised on both sides), classification included.

Beside it:
* ``roofline`` for the dominant kernel, the backward main kernel: its algorithmic
  FLOPs (S, dP, dV, dK products: 8*d per block element per query head) over its
  mean duration from HIP events around it in the K timed steps;
* ``method``: every workload measured the same way, with cold caches: 2 warm-up
  iterations, then 10 timed ones, each preceded by an untimed 512 MiB write (larger
  than the last-level caches, so mask and bias come from HBM), with HIP events
  around every call; the mean of the first 3 and the median of 10 per phase,
  effective TFLOP/s and the mandatory mask / bias / dBias bytes per second, each
  as a fraction of the bound that applies (bf16 MFMA, or HBM for the document
  workload);
* ``measured_peaks``: a 4 GiB device copy's read + write bandwidth beside the
  spec HBM peak, and a bf16 8192^3 library GEMM's rate beside the spec MFMA peak;
* ``cpu_baseline``: the fp64 oracle on sampled query blocks of the workload;
* ``next_rows`` (unless --no-next): GPU top-k mask construction, the step with the
  bit-packed PARTIAL-block mask, and (with the Long workload measured) the
  backward in bands of query blocks at three workspace sizes.
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
FLUSH_BYTES = 512 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true", help="skip the next-row measurements")
    ap.add_argument("--no-workloads", action="store_true", help="skip the per-workload method measurements")
    ap.add_argument("--workloads", default="mid,headline,docpacked,long",
                    help="workloads measured in the method block, caches flushed before each call (comma separated)")
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
    ap.add_argument("--summarize-counters", nargs=2, metavar=("COUNTER_DIR", "OUT_MD"), default=None,
                    help="turn rocprofv3 SQ counter passes (csv files under COUNTER_DIR) into a per-kernel "
                         "markdown summary, then exit")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "OUT_MD"), default=None,
                    help="turn a rocprofv3 --kernel-trace --stats run (kernel_stats.csv under TRACE_DIR) into "
                         "a markdown table, then exit")
    return ap.parse_args()


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "headline_traffic.json")
KERNEL_SOURCES = ["classify.hip", "fwd.hip", "bwd.hip", "common.h"]
# kernels of each measured unit, matched by substring of the demangled name
CALL_KERNELS = {"fwd": ["fwd_kernel"], "bwd_main": ["bwd_main_kernel", "dkv_finalize_kernel"], "bwd_dq": ["dq_kernel"],
                "bwd_prepare": ["bwd_pre_kernel", "kt_kernel", "pair_base_kernel", "pair_count_kernel",
                                "pair_order_kernel", "dkv_zero_kernel"],
                "classify": ["classify_kernel"]}


def kernel_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_dynamic_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def summarize_traffic(counter_dir: str, out_json: str, copy_mib: int):
    """HBM bytes per launch of each kernel group from FETCH_SIZE / WRITE_SIZE (KiB per dispatch).

    Each counter is scaled by the ratio of known bytes to what it reads for the calibration
    copy (a device copy of --calibrate-copy-mib MiB: that many bytes fetched and written)."""
    import csv
    import glob
    from collections import defaultdict

    assert copy_mib > 0, "give the calibration copy's size with --calibrate-copy-mib"
    out = {"source_hash": kernel_source_hash(), "calibration_mib": copy_mib, "counters": {}}
    per_unit = defaultdict(float)
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
        for unit, subs in CALL_KERNELS.items():
            for name, vals in per.items():
                if any(sub in name for sub in subs):
                    per_unit[unit] += sum(vals) / len(vals) * 1024.0 * factor
    out["bytes_per_launch"] = {k: round(v) for k, v in per_unit.items()}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def live_blocks(c, np):
    """Blocks not wholly excluded by causality, summed over (b, kv head)."""
    nqb, nkb = (c.lq + 63) // 64, (c.lk + 63) // 64
    qb = np.arange(nqb)[:, None]
    kb = np.arange(nkb)[None, :]
    live = (kb * 64 <= np.minimum(qb * 64 + 63, c.lq - 1) + (c.lk - c.lq)) if c.causal else np.ones((nqb, nkb), bool)
    return int(live.sum()) * c.b * c.hkv


def work_of(c, state, np, fused: bool, has_mask: bool, ranges: bool = False):
    """Algorithmic FLOPs and mandatory mask / bias / dBias bytes of one step (see the module doc)."""
    n_p = int((state == 1).sum())
    n_f = int((state == 2).sum())
    n_ns = n_p + n_f
    G, d = c.hq // c.hkv, c.d
    w = {"blocks_nonskip": n_ns, "blocks_partial": n_p, "blocks_full": n_f,
         "f_fwd": 4.0 * d * 4096 * G * n_ns, "f_bwd": 10.0 * d * 4096 * G * n_ns,
         "f_bwd_main": 8.0 * d * 4096 * G * n_ns, "f_bwd_dq": 2.0 * d * 4096 * G * n_ns}
    mask_read = 0 if ranges else 2.0 * 4096 * n_p
    # a separate classification reads the mask of every causally live block once more; fused,
    # the forward's own mask reads classify; column ranges are 8 bytes per key and plane
    w["b_cls"] = (8.0 * c.b * c.hkv * c.lk if ranges else
                  (2.0 * 4096 * live_blocks(c, np) if (has_mask and not fused) else 0.0))
    w["b_fwd"] = 2.0 * 4096 * n_ns + mask_read
    w["b_bwd"] = w["b_fwd"] + 2.0 * c.b * c.hkv * c.lq * c.lk
    return w


class Step:
    """Device inputs, outputs and workspace of one workload, and its step through the C ABI."""

    def __init__(self, c, dma, torch, np, path="fused"):
        import synth
        from synth.device import upload_dense, upload_mask_bias

        self.c, self.dma, self.torch, self.path = c, dma, torch, path
        t0 = time.perf_counter()
        self.q, self.k, self.v, self.do = upload_dense(c)
        self.mask, self.bias = upload_mask_bias(c)
        torch.cuda.synchronize()
        self.t_gen = time.perf_counter() - t0
        if path == "ranges":
            bounds = synth.doc_bounds(c)
            j = np.arange(c.lk)
            end = bounds[np.searchsorted(bounds, j, side="right")]
            self.rs = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(j, (c.b, c.hkv, c.lk)).astype(np.int32))).cuda()
            self.re = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(end, (c.b, c.hkv, c.lk)).astype(np.int32))).cuda()
        self.state = torch.empty(dma.block_state_shape(c.b, c.hkv, c.lq, c.lk), dtype=torch.uint8, device="cuda")
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((c.b, c.hq, c.lq), dtype=torch.float32, device="cuda")
        self.dq, self.dk, self.dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        self.dbias = torch.empty((c.b, c.hkv, c.lq, c.lk), dtype=torch.bfloat16, device="cuda")
        self.ws = torch.empty(dma.dma_attn_bwd_workspace_size(c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.causal),
                              dtype=torch.uint8, device="cuda")
        self.stream = torch.cuda.current_stream()

    PHASES = ("classify", "fwd", "bwd_prepare", "bwd_main", "bwd_dq")

    def run(self, ev=None):
        """One step; ev = 6 events recorded between the phases (or None)."""
        c, dma, s = self.c, self.dma, self.stream
        rec = (lambda i: ev[i].record(s)) if ev is not None else (lambda i: None)
        rec(0)
        if self.path == "ranges":
            dma.dma_block_classify_ranges(self.rs, self.re, c.b, c.hkv, c.lq, c.lk, c.causal, self.state, s)
            rec(1)
            dma.dma_attn_fwd_ranges(self.q, self.k, self.v, self.rs, self.re, self.bias, self.state, c.scale_f32,
                                    c.causal, self.o, self.lse, s)
            rec(2)
            rec(3)
            # the range backward has no per-phase entry point: its whole time counts as bwd_main
            dma.dma_attn_bwd_ranges(self.q, self.k, self.v, self.rs, self.re, self.bias, self.state, self.o, self.do,
                                    self.lse, c.scale_f32, c.causal, self.dq, self.dk, self.dv, self.dbias, self.ws, s)
            rec(4)
            rec(5)
            return
        if self.path == "separate":
            dma.dma_block_classify(self.mask, c.b, c.hkv, c.lq, c.lk, c.causal, self.state, s)
            rec(1)
            dma.dma_attn_fwd(self.q, self.k, self.v, self.mask, self.bias, self.state, c.scale_f32, c.causal, self.o,
                             self.lse, s)
        else:
            rec(1)
            dma.dma_attn_fwd_classify(self.q, self.k, self.v, self.mask, self.bias, c.scale_f32, c.causal, self.state,
                                      self.o, self.lse, s)
        rec(2)
        for i, part in enumerate((dma.BWD_PREPARE, dma.BWD_MAIN, dma.BWD_DQ)):
            dma.dma_attn_bwd_part(part, self.q, self.k, self.v, self.mask, self.bias, self.state, self.o, self.do,
                                  self.lse, c.scale_f32, c.causal, self.dq, self.dk, self.dv, self.dbias, self.ws, s)
            rec(3 + i)

    def events(self):
        return [self.torch.cuda.Event(enable_timing=True) for _ in range(6)]

    @staticmethod
    def phase_ms(ev):
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(5)]

    def free(self):
        for name in ("q", "k", "v", "do", "mask", "bias", "state", "o", "lse", "dq", "dk", "dv", "dbias", "ws", "rs",
                     "re"):
            if hasattr(self, name):
                delattr(self, name)
        self.torch.cuda.empty_cache()


def method_measure(st, np, torch, flush, n_warm=2, n_iter=10, bound="mfma"):
    """Cold-cache measurement: warm-ups, then n_iter iterations each after an untimed flush write;
    per phase the mean of the first 3 and the median of all, and rates against the bound."""
    c = st.c
    for _ in range(n_warm):
        st.run()
    torch.cuda.synchronize()
    evs = [st.events() for _ in range(n_iter)]
    for i in range(n_iter):
        flush.zero_()  # untimed: outside the events
        st.run(evs[i])
    torch.cuda.synchronize()
    t = np.array([Step.phase_ms(e) for e in evs])  # [iter, phase]
    first3, med = t[:3].mean(axis=0), np.median(t, axis=0)
    w = work_of(c, st.state, np, fused=(st.path == "fused"), has_mask=st.mask is not None or st.path == "ranges",
                ranges=(st.path == "ranges"))
    out = {"workload": describe(c), "path": st.path, "bound": bound, "iterations": n_iter,
           "blocks_nonskip": w["blocks_nonskip"], "blocks_partial": w["blocks_partial"], "blocks_full": w["blocks_full"]}
    for name, stat in (("mean_first3", first3), ("median10", med)):
        ph = dict(zip(Step.PHASES, stat))
        t_cls_fwd = ph["classify"] + ph["fwd"]
        t_bwd = ph["bwd_prepare"] + ph["bwd_main"] + ph["bwd_dq"]
        t_step = t_cls_fwd + t_bwd
        mand = w["b_cls"] + w["b_fwd"] + w["b_bwd"]
        tf = (w["f_fwd"] + w["f_bwd"]) / (t_step * 1e-3) / 1e12
        gbs = mand / (t_step * 1e-3) / 1e9
        out[name] = {"phases_ms": {k: round(float(v), 4) for k, v in ph.items()}, "step_ms": round(float(t_step), 4),
                     "tflops": round(tf, 2), "tflops_fwd": round(w["f_fwd"] / (t_cls_fwd * 1e-3) / 1e12, 2),
                     "tflops_bwd": round(w["f_bwd"] / (t_bwd * 1e-3) / 1e12, 2),
                     "mandatory_gbs": round(gbs, 1),
                     "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        if st.path != "ranges":
            out[name]["bwd_main_tflops"] = round(w["f_bwd_main"] / (ph["bwd_main"] * 1e-3) / 1e12, 2)
        else:
            out[name]["note"] = "the range backward is one call: bwd_main holds all of it, bwd_prepare and bwd_dq are 0"
    out["mandatory_bytes"] = {"classify": w["b_cls"], "fwd": w["b_fwd"], "bwd": w["b_bwd"]}
    return out


def band_count(c, ws_bytes: int) -> int:
    """Bands of query blocks dma_attn_bwd runs in for this workspace (1: the one pass): the most
    slot pairs per plane that fit beside the fixed regions, then consecutive blocks while their
    live pairs fit."""
    up = lambda x: (x + 255) // 256 * 256
    nqb, nkb2 = (c.lq + 63) // 64, ((c.lk + 63) // 64 + 1) // 2

    def live(qb):
        if not c.causal:
            return nkb2
        last = qb * 64 + 63 + c.lk - c.lq
        return 0 if last < 0 else min(nkb2, last // 128 + 1)

    fixed = up(2 * c.b * c.hq * c.lq * 4) + up((nqb + 1) * 8) + up(c.b * c.hkv * c.d * nkb2 * 128 * 2)
    total = sum(live(qb) for qb in range(nqb))
    split = c.causal and c.b * c.hkv * nkb2 <= 256 and nqb >= 8
    if ws_bytes >= fixed + up(c.b * c.hq * total * 16384) + up(c.b * c.hq * total * 128) + \
            (up(2 * c.b * c.lk * c.hkv * c.d * 4) if split else 0) + up(2 * c.b * c.hkv * nkb2 * (2 if split else 1) * 4):
        return 1
    fixed += up(2 * c.b * c.lk * c.hkv * c.d * 4)
    np_ = min(total, (ws_bytes - fixed) // (c.b * c.hq * 16512))
    while np_ > 0 and fixed + up(c.b * c.hq * np_ * 16384) + up(c.b * c.hq * np_ * 128) > ws_bytes:
        np_ -= 1
    n, lo = 0, 0
    while lo < nqb:
        hi, k = lo, 0
        while hi < nqb and (hi == lo or k + live(hi) <= np_):
            k += live(hi)
            hi += 1
        n, lo = n + 1, hi
    return n


def time_banded(st, dma, torch, np, n_iter=5):
    """dma_attn_bwd (all phases, one call) with the one-pass workspace, with one mask plane of it and
    with the smallest: the backward then runs in bands of query blocks, trading time for memory."""
    c = st.c
    sizes = (("one_pass", st.ws.numel()), ("one_mask_plane", c.b * c.hkv * c.lq * c.lk * 2),
             ("min", dma.dma_attn_bwd_workspace_size_min(c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.causal)))
    out = {"workload": describe(c)}
    for label, nbytes in sizes:
        ws = st.ws[:nbytes]

        def bwd():
            dma.dma_attn_bwd(st.q, st.k, st.v, st.mask, st.bias, st.state, st.o, st.do, st.lse, c.scale_f32, c.causal,
                             st.dq, st.dk, st.dv, st.dbias, ws, st.stream)

        bwd()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_iter)]
        for a, b in ev:
            a.record(st.stream)
            bwd()
            b.record(st.stream)
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        out[label] = {"workspace_bytes": int(nbytes), "bands": band_count(c, nbytes), "bwd_ms": round(ms, 3)}
        print(f"[bench] {c.name} backward, {label} workspace: {ms:.2f} ms", file=sys.stderr, flush=True)
    return out


def describe(c) -> str:
    m = f"top-k {c.topk}" if c.mask == "topk" else ("document" if c.mask == "doc" else c.mask)
    return (f"{c.name}: b={c.b} L={c.lq} Hq={c.hq} Hkv={c.hkv} d={c.d} {m} mask, "
            f"{'causal' if c.causal else 'non-causal'}")


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


def time_topk(c, dma, torch, stream):
    """GPU top-k mask construction (dma_topk_mask) on a fresh N(0,1) bf16 bias of the workload's shape."""
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
    del raw, mk, bo
    return {"ms": round(t_topk, 4), "gbs": round(bytes_topk / (t_topk * 1e-3) / 1e9, 1),
            "frac_hbm": round(bytes_topk / (t_topk * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "rows": c.b * c.hkv * c.lq, "lk": c.lk, "k": c.topk}


def time_bits(st, dma, np, torch, dense_step_ms):
    """The step with the bit-packed PARTIAL-block mask (classify writes 512 B per PARTIAL block;
    forward and backward read those bits instead of the bf16 mask), per phase."""
    c, s = st.c, st.stream
    state = torch.empty_like(st.state)
    mb = torch.empty((dma.dma_mask_bits_size(c.b, c.hkv, c.lq, c.lk),), dtype=torch.uint8, device="cuda")
    reps = 3
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps + 1)]
    for r in range(reps + 1):  # the first repetition warms up
        e = ev[r]
        e[0].record(s)
        dma.dma_block_classify_bits(st.mask, c.b, c.hkv, c.lq, c.lk, c.causal, state, mb, s)
        e[1].record(s)
        dma.dma_attn_fwd_bits(st.q, st.k, st.v, mb, st.bias, state, c.scale_f32, c.causal, st.o, st.lse, s)
        e[2].record(s)
        dma.dma_attn_bwd_bits(st.q, st.k, st.v, mb, st.bias, state, st.o, st.do, st.lse, c.scale_f32, c.causal, st.dq,
                              st.dk, st.dv, st.dbias, st.ws, s)
        e[3].record(s)
    torch.cuda.synchronize()
    t = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])] for e in ev[1:]])
    t = t.mean(axis=0)
    n_p = int((state == 1).sum())
    out = {"classify_ms": round(float(t[0]), 4), "fwd_ms": round(float(t[1]), 4), "bwd_ms": round(float(t[2]), 4),
           "step_ms": round(float(t.sum()), 4), "dense_step_ms": round(float(dense_step_ms), 4),
           "blocks_partial": n_p,
           "mask_bytes_dense": 2 * 2.0 * 64 * 64 * n_p, "mask_bytes_bits": 2 * 512.0 * n_p,
           "bits_bytes_written": 512.0 * n_p}
    del state, mb
    return out


def measured_copy_gbs(torch, mib=4096):
    """Read + write bandwidth of a device copy of `mib` MiB (the practical HBM rate of a plain copy)."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 3
    del src, dst
    torch.cuda.empty_cache()
    return round(2.0 * mib * (1 << 20) / (ms * 1e-3) / 1e9, 1)


def measured_gemm_tflops(torch, n=8192):
    """bf16 n x n x n products through the vendor BLAS (torch.matmul): the matrix-core rate a plain
    library GEMM reaches on this device, beside the dense bf16 spec peak."""
    a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    c = torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        c = torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    del a, b, c
    torch.cuda.empty_cache()
    return round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)


def summarize_counters(counter_dir: str, out_md: str):
    """Per-kernel SQ counters (mean over dispatches, summed over the GPU) and derived ratios."""
    import csv
    import glob
    import re
    from collections import defaultdict

    per = defaultdict(lambda: defaultdict(list))
    for f in sorted(glob.glob(os.path.join(counter_dir, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            per[re.sub(r"\(.*", "", r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = []
    for k in sorted(per):
        if not any(sub in k for sub in ("fwd_kernel", "bwd_main_kernel", "dq_kernel")):
            continue  # the three kernels that hold the products
        c = {n: sum(v) / len(v) for n, v in per[k].items()}
        lines.append(f"### `{k}`\n")
        waves = c.get("SQ_WAVES")
        ratios = []
        if "SQ_WAVE_CYCLES" in c:
            for n, label in (("SQ_ACTIVE_INST_ANY", "issuing (any instruction)"),
                             ("SQ_WAIT_INST_ANY", "ready, waiting for issue"), ("SQ_WAIT_ANY", "waiting (s_waitcnt, barrier)"),
                             ("SQ_ACTIVE_INST_VALU", "issuing VALU / MFMA"), ("SQ_ACTIVE_INST_LDS", "issuing LDS"),
                             ("SQ_ACTIVE_INST_SCA", "issuing scalar"), ("SQ_WAIT_INST_LDS", "waiting on LDS issue")):
                if n in c:
                    ratios.append((f"{label}: {n} / SQ_WAVE_CYCLES", c[n] / c["SQ_WAVE_CYCLES"]))
        if "SQ_BUSY_CU_CYCLES" in c and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            ratios.append(("MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES)",
                           c["SQ_VALU_MFMA_BUSY_CYCLES"] / (4.0 * c["SQ_BUSY_CU_CYCLES"])))
        if "SQ_LDS_BANK_CONFLICT" in c and c.get("SQ_LDS_IDX_ACTIVE"):
            ratios.append(("LDS bank-conflict cycles / LDS active cycles", c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]))
        if ratios:
            lines.append("| ratio | value |\n|---|---|")
            lines += [f"| {a} | {b:.3f} |" for a, b in ratios]
            lines.append("")
        lines.append("| counter | per dispatch | per wave |\n|---|---|---|")
        for n in sorted(c):
            pw = f"{c[n] / waves:.1f}" if waves and n.startswith("SQ_INSTS") else ""
            lines.append(f"| {n} | {c[n]:.4g} | {pw} |")
        lines.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(trace_dir: str, out_md: str):
    """Kernel durations from a rocprofv3 --kernel-trace --stats run."""
    import csv
    import glob

    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    assert len(files) == 1, f"expected one kernel_stats.csv under {trace_dir}, found {files}"
    rows = list(csv.DictReader(open(files[0])))
    lines = ["| kernel | calls | total (us) | average (us) | min (us) | max (us) | % |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("|", "/")
        lines.append(f"| `{name[:70]}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.calibrate_copy_mib)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
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

    c = synth.CASES[args.config]
    torch.cuda.set_device(0)
    st = Step(c, dma, torch, np, path="fused")
    print(f"[bench] {c.name}: inputs generated and uploaded in {st.t_gen:.1f} s", file=sys.stderr, flush=True)

    if args.calibrate_copy_mib > 0:  # one plain copy of known size, for counter calibration
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- the contract's timed region: K steps, synchronised on both sides ----------------------
    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()
    evs = [st.events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        st.run(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    per = np.array([Step.phase_ms(e) for e in evs]).mean(axis=0)
    ph = dict(zip(Step.PHASES, per))
    w = work_of(c, st.state, np, fused=True, has_mask=st.mask is not None)
    tflops = (w["f_fwd"] + w["f_bwd"]) / (ms_step * 1e-3) / 1e12
    mand = w["b_cls"] + w["b_fwd"] + w["b_bwd"]
    t_bwd = ph["bwd_prepare"] + ph["bwd_main"] + ph["bwd_dq"]

    # dominant kernel: the backward main kernel, timed by the events around it in the K steps
    achieved = w["f_bwd_main"] / (ph["bwd_main"] * 1e-3) / 1e12
    traffic = None  # measured HBM bytes per launch, only while the kernels are the ones measured
    if args.traffic_json and os.path.exists(args.traffic_json):
        with open(args.traffic_json) as f:
            tj = json.load(f)
        if tj.get("source_hash") == kernel_source_hash():
            traffic = tj["bytes_per_launch"].get("bwd_main")
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": "bwd_main_kernel (dma_attn_bwd_part DMA_BWD_MAIN): S, dP, dV, dK products",
                "algorithmic_flop_per_launch": w["f_bwd_main"], "ms_per_launch": round(float(ph["bwd_main"]), 4)}

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
        "precision": "bf16 inputs and MFMA operands, except P V in fp16 (V scaled per 8-key group, exact for bf16 V); "
                     "fp32 accumulation and softmax",
        "data": "synthetic (seeded; N(0,1) q/k/v/dO/bias, top-k mask from the bias)",
        "config": {"workload": describe(c), "b": c.b, "seq_len": c.lq, "hq": c.hq, "hkv": c.hkv, "d": c.d,
                   "blocks_nonskip": w["blocks_nonskip"], "blocks_partial": w["blocks_partial"],
                   "blocks_full": w["blocks_full"]},
        "hbm_gbs_mandatory": round(mand / (ms_step * 1e-3) / 1e9, 1),
        "classify_fused": True,
        "phases_ms": {k: round(float(v), 4) for k, v in ph.items()},
        "phases_tflops": {"fwd": round(w["f_fwd"] / ((ph["classify"] + ph["fwd"]) * 1e-3) / 1e12, 2),
                          "bwd": round(w["f_bwd"] / (t_bwd * 1e-3) / 1e12, 2)},
        "roofline": roofline,
    }

    if not args.no_next and args.calibrate_copy_mib == 0:
        line["next_rows"] = {}
        line["next_rows"]["mask_bits"] = time_bits(st, dma, np, torch, ms_step)
        if c.mask == "topk":
            line["next_rows"]["topk_mask"] = time_topk(c, dma, torch, st.stream)
    if args.calibrate_copy_mib == 0:
        line["measured_peaks"] = {"hbm_copy_gbs": measured_copy_gbs(torch), "hbm_spec_gbs": PEAK_HBM_GBS,
                                  "bf16_gemm_tflops": measured_gemm_tflops(torch),
                                  "mfma_bf16_spec_tflops": PEAK_BF16_TFLOPS}
    head_method = None
    if not args.no_workloads and args.calibrate_copy_mib == 0:
        flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        # a document-mask workload is measured on its separate and range paths, not the fused one
        if c.name in args.workloads.split(",") and c.mask != "doc":
            head_method = method_measure(st, np, torch, flush)
        st.free()
        method = {}
        for name in args.workloads.split(","):
            if name == c.name and c.mask != "doc":
                method[name] = head_method
                continue
            wc = synth.CASES[name]
            paths = ("separate", "ranges") if wc.mask == "doc" else ("fused",)
            for path in paths:
                print(f"[bench] {name} ({path})", file=sys.stderr, flush=True)
                ws = Step(wc, dma, torch, np, path=path)
                method[name if path == paths[0] else f"{name}_{path}"] = method_measure(
                    ws, np, torch, flush, bound="hbm" if wc.mask == "doc" else "mfma")
                if name == "long" and not args.no_next:
                    line.setdefault("next_rows", {})["banded_backward"] = time_banded(ws, dma, torch, np)
                ws.free()
                del ws
        line["method"] = method
        del flush
    else:
        st.free()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(c, args.cpu_blocks, w["f_fwd"] + w["f_bwd"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
