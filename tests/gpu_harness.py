"""Helpers shared by the GPU parity tests: upload synth inputs, run the C ABI, compare with the oracle.

Tolerances (fp64 oracle on the same bf16 inputs):
  block_state  bit-exact
  O            max |O_gpu - O_ref| <= 1e-2 * v_scale (v_scale = the standard deviation of V;
               attention is linear in V, so the bound for N(0,1) V carries over scaled); an
               element over that bound counts as bf16 storage rounding only when |O_ref| >= 4
               v_scale and the error is within half a bf16 ulp of O_ref plus 1e-3 v_scale (such
               elements are counted and reported)
  LSE          |lse_gpu - lse_ref| <= 1e-3 + 2^-20 |lse_ref| on rows with a valid key, +inf on the
               others.  The second term is the fp32 arithmetic of the kernel: the row maximum and
               its product with log2(e) are rounded at the magnitude of the score, three
               roundings of relative size 2^-24.
  dQ dK dV dB  ||x_gpu - x_ref||_2 / ||x_ref||_2 <= 2e-2

Bias values beyond +-2^12 at valid positions (the pages' recipe fills masked entries with the
smallest bf16, -3.39e38, and a caller may pass that bias without the mask): the kernels clamp
them to +-2^12.  Every test input of this kind keeps such values single-valued per sign within
a row, so that the clamp leaves the formula's real-number result unchanged (softmax does not
change when the same constant is added to several scores that already dominate or vanish).
The fp64 oracle evaluated at |bias| ~ 3e38 cannot see that result: the bias absorbs the
q.k term of the score (fp64 spacing there is 2^75), which turns softmax(q.k) over such keys
into uniform weights.  For those inputs the oracle is therefore evaluated on the clamped
bias, where fp64 keeps every term.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

O_TOL = 1e-2
LSE_TOL = 1e-3
LSE_REL = 2.0 ** -20
GRAD_TOL = 2e-2
BIAS_CLAMP = 4096.0  # the kernels clamp bias values at valid positions to +-2^12


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda")


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_to_f64(bits(t))


def rel_l2(x: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-30))


def worst_elements(o: np.ndarray, ref: np.ndarray, n: int = 5) -> str:
    err = np.abs(o - ref).ravel()
    idx = np.argsort(err)[::-1][:n]
    return "; ".join(f"at {np.unravel_index(i, o.shape)} gpu {o.ravel()[i]:.6g} ref {ref.ravel()[i]:.6g} "
                     f"err {err[i]:.3g}" for i in idx)


def check_o(o: np.ndarray, ref: np.ndarray, what: str = "O", v_scale: float = 1.0):
    o, ref = o / v_scale, ref / v_scale
    err = np.abs(o - ref)
    bad = err > O_TOL
    if err.size:
        print(f"{what}: worst elements (in units of v_scale {v_scale:g}): {worst_elements(o, ref)}", flush=True)
    if bad.any():
        r = np.abs(ref[bad])
        ulp_half = np.ldexp(1.0, np.floor(np.log2(np.maximum(r, 1e-30))).astype(int) - 8)
        storage = (r >= 4.0) & (err[bad] <= ulp_half + 1e-3)
        assert storage.all(), f"{what}: {int((~storage).sum())} elements over {O_TOL}, max err {err.max():.3g}"
        print(f"{what}: {int(bad.sum())} elements over {O_TOL} attributed to bf16 storage rounding")
    return float(err.max()) if err.size else 0.0


def check_lse(lse: np.ndarray, ref: np.ndarray):
    fin = np.isfinite(ref)
    assert np.all(np.isposinf(lse[~fin])), "rows without a valid key must have lse = +inf"
    assert np.all(np.isfinite(lse[fin]))
    if fin.any():
        err = np.abs(lse[fin] - ref[fin])
        tol = LSE_TOL + LSE_REL * np.abs(ref[fin])
        assert np.all(err <= tol), f"lse: max error {err.max():.3g} (at ref {ref[fin][np.argmax(err - tol)]:.6g})"


def check_grad(x: np.ndarray, ref: np.ndarray, what: str):
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    e = rel_l2(x, ref)
    assert e <= GRAD_TOL, f"{what}: rel-L2 {e:.3g} > {GRAD_TOL}"
    return e


def clamp_bias_bits(bias_h: np.ndarray | None) -> np.ndarray | None:
    """The bias with values beyond +-2^12 replaced by +-2^12 (bf16 0x4580 / 0xC580)."""
    if bias_h is None:
        return None
    f = oracle.bf16_to_f64(bias_h)
    out = bias_h.copy()
    out[f > BIAS_CLAMP] = 0x4580
    out[f < -BIAS_CLAMP] = 0xC580
    return out


def compare_with_oracle(name, c, q_h, k_h, v_h, mask_h, bias_h, do_h, o, lse, dq, dk, dv, dbias, v_scale=1.0,
                        verbose=True):
    """Whole-tensor parity of one forward + backward's outputs (device tensors) against the oracle
    (on the clamped bias where a bias value lies beyond +-2^12, see the module docstring)."""
    bias_h = clamp_bias_bits(bias_h)
    o_ref, lse_ref = oracle.forward(q_h, k_h, v_h, mask_h, bias_h, c.scale_f32, c.causal)
    dq_ref, dk_ref, dv_ref, db_ref = oracle.backward(q_h, k_h, v_h, mask_h, bias_h, c.scale_f32, c.causal, do_h)
    o_err = check_o(f64(o), o_ref, f"{name} O", v_scale)
    check_lse(lse.cpu().numpy().astype(np.float64), lse_ref)
    errs = {"O_maxabs": o_err}
    errs["dQ"] = check_grad(f64(dq), dq_ref, f"{name} dQ")
    errs["dK"] = check_grad(f64(dk), dk_ref, f"{name} dK")
    errs["dV"] = check_grad(f64(dv), dv_ref, f"{name} dV")
    if dbias is not None:
        db = f64(dbias)
        if db_ref is None:  # no bias: the library still returns dS summed over the group
            _, _, _, db_ref = oracle.backward(q_h, k_h, v_h, mask_h, np.zeros((c.b, c.hkv, c.lq, c.lk), np.uint16),
                                              c.scale_f32, c.causal, do_h)
        errs["dBias"] = check_grad(db, db_ref, f"{name} dBias")
        # exact zeros where the oracle's dS is structurally zero (invalid entries, skipped blocks)
        valid = np.ones((c.b, c.hkv, c.lq, c.lk), bool) if mask_h is None else oracle.attends(mask_h)
        if c.causal:
            valid &= (np.arange(c.lk)[None, :] <= np.arange(c.lq)[:, None] + c.lk - c.lq)
        assert np.all(db[~valid] == 0.0), f"{name}: dBias not exactly zero on invalid entries"
    if verbose:
        print(name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    return errs


class DeviceCase:
    """All inputs of a case on the device, plus the library's outputs."""

    def __init__(self, c: synth.Case, do_bits: np.ndarray | None = None, whole_mask: bool = True):
        import block_sparse_dynamic_amd as dma

        self.c, self.dma = c, dma
        self.q_h, self.k_h, self.v_h = synth.q(c), synth.k(c), synth.v(c)
        self.do_h = synth.do(c) if do_bits is None else do_bits
        self.q, self.k, self.v, self.do = (to_dev(x) for x in (self.q_h, self.k_h, self.v_h, self.do_h))
        if whole_mask:
            self.mask_h, self.bias_h = synth.mask_bias(c)
            self.mask = to_dev(self.mask_h) if self.mask_h is not None else None
            self.bias = to_dev(self.bias_h) if self.bias_h is not None else None
        self.state = torch.empty(dma.block_state_shape(c.b, c.hkv, c.lq, c.lk), dtype=torch.uint8, device="cuda")

    def upload(self):
        """Upload the host inputs again (after a test changed them)."""
        self.q, self.k, self.v, self.do = (to_dev(x) for x in (self.q_h, self.k_h, self.v_h, self.do_h))
        self.mask = to_dev(self.mask_h) if self.mask_h is not None else None
        self.bias = to_dev(self.bias_h) if self.bias_h is not None else None

    def classify(self):
        c = self.c
        self.dma.dma_block_classify(self.mask, c.b, c.hkv, c.lq, c.lk, c.causal, self.state)

    def forward(self):
        c = self.c
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((c.b, c.hq, c.lq), dtype=torch.float32, device="cuda")
        self.dma.dma_attn_fwd(self.q, self.k, self.v, self.mask, self.bias, self.state, c.scale_f32, c.causal,
                              self.o, self.lse)

    def backward(self, do=None, want_dbias=True, ws_bytes=None):
        """dma_attn_bwd with the one-pass workspace, or with ws_bytes of workspace."""
        c = self.c
        do = self.do if do is None else do
        self.dq, self.dk, self.dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        self.dbias = (torch.full((c.b, c.hkv, c.lq, c.lk), float("nan"), dtype=torch.bfloat16, device="cuda")
                      if want_dbias else None)
        if ws_bytes is None:
            ws_bytes = self.dma.dma_attn_bwd_workspace_size(c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.causal)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        self.dma.dma_attn_bwd(self.q, self.k, self.v, self.mask, self.bias, self.state, self.o, do, self.lse,
                              c.scale_f32, c.causal, self.dq, self.dk, self.dv, self.dbias, ws)


def check_small_case(c: synth.Case, do_bits=None, verbose=True, prepare=None):
    """Whole-tensor parity of classify, forward and backward against the oracle.

    ``prepare(dc)`` may change the host inputs (q_h, k_h, v_h, mask_h, bias_h; mask_h = None
    passes no mask) before they are uploaded and compared."""
    dc = DeviceCase(c, do_bits)
    if prepare is not None:
        prepare(dc)
        dc.upload()
    dc.classify()
    dc.forward()
    dc.backward()
    torch.cuda.synchronize()
    st = dc.state.cpu().numpy()
    ref_st = oracle.classify(dc.mask_h, c.b, c.hkv, c.lq, c.lk, c.causal)
    assert np.array_equal(st, ref_st), f"{c.name}: block_state differs in {int((st != ref_st).sum())} blocks"
    errs = compare_with_oracle(c.name, c, dc.q_h, dc.k_h, dc.v_h, dc.mask_h, dc.bias_h, dc.do_h, dc.o, dc.lse, dc.dq,
                               dc.dk, dc.dv, dc.dbias, v_scale=c.v_std, verbose=verbose)
    return dc, errs


def _oracle_block(c, k_b, v_b, bb, r0):
    """fp64 oracle on one sampled 64-row query block (all heads): forward and backward terms."""
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
    o, lse = oracle.forward_rows(qr, k_b, v_b, mask, bias, c.scale_f32, c.causal, rows, c.lq)
    bias_for_grad = bias if bias is not None else np.zeros((c.hkv, len(rows), c.lk))
    dq, dk, dv, db = oracle.backward_rows(qr, k_b, v_b, mask, bias_for_grad, c.scale_f32, c.causal, rows, c.lq, dor)
    valid = np.stack([oracle.valid_rows(None if mask is None else mask[g], rows, c.lq, c.lk, c.causal)
                      for g in range(c.hkv)])
    return dict(rows=rows, o=o, lse=lse, dq=dq, dk=dk, dv=dv, db=db, valid=valid)


def doc_ranges(c: synth.Case):
    """Column ranges of a document mask: key j of document [s, e) attends rows [j, e)."""
    bounds = synth.doc_bounds(c)
    j = np.arange(c.lk)
    end = bounds[np.searchsorted(bounds, j, side="right")]
    s = np.broadcast_to(j, (c.b, c.hkv, c.lk)).astype(np.int32)
    e = np.broadcast_to(end, (c.b, c.hkv, c.lk)).astype(np.int32)
    return np.ascontiguousarray(s), np.ascontiguousarray(e)


def check_full_case(c: synth.Case, n_blocks: int = 64, log=print, path: str = "dense", ws_bytes: int | None = None):
    """Parity at the workload's full size, in the launch configuration the benchmark times.

    Whole block bitmap bit-exact; O, LSE, dQ, dBias on `n_blocks` seeded 64-row query
    blocks (all heads); dK, dV from a second backward whose dO is zero outside the
    sampled rows, which makes them exactly the sampled rows' contributions.

    path: "dense" (dma_block_classify, dma_attn_fwd, dma_attn_bwd), "fused" (the forward that
    classifies, dma_attn_fwd_classify), "ranges" (column ranges of a document mask, the
    dma_*_ranges entry points) or "bits" (the bit-packed PARTIAL blocks, dma_*_bits).
    ws_bytes: the backward's workspace (default: the one-pass size; less runs it in bands).
    """
    import concurrent.futures
    import os

    from threadpoolctl import threadpool_limits

    import block_sparse_dynamic_amd as dma
    from synth.device import upload_dense, upload_mask_bias

    nqb, nkb = (c.lq + 63) // 64, (c.lk + 63) // 64
    ref_state = np.empty((c.b, c.hkv, nqb, nkb), dtype=np.uint8)

    def on_chunk(bb, g, r0, m, b):  # classify each uploaded chunk of rows on the CPU
        n = min(1024, c.lq - r0)
        blk = oracle.classify_plane_rows(None if m is None else m[:n], r0, c.lq, c.lk, c.causal)
        nb = (n + 63) // 64
        ref_state[bb, g, r0 // 64: r0 // 64 + nb] = blk[:nb]

    if ws_bytes is None:
        ws_bytes = dma.dma_attn_bwd_workspace_size(c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.causal)
    log(f"[{c.name}/{path}] generating and uploading inputs (backward workspace {ws_bytes} bytes)", flush=True)
    q, k, v, do = upload_dense(c)
    mask, bias = upload_mask_bias(c, chunk_rows=1024, on_chunk=on_chunk)
    state = torch.empty((c.b, c.hkv, nqb, nkb), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((c.b, c.hq, c.lq), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dbias = torch.full((c.b, c.hkv, c.lq, c.lk), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    if path == "ranges":
        s, e = doc_ranges(c)
        ts, te = torch.from_numpy(s).cuda(), torch.from_numpy(e).cuda()
        del mask  # the range path never sees the dense mask
        mask = None
    elif path == "bits":
        mbits = torch.empty((dma.dma_mask_bits_size(c.b, c.hkv, c.lq, c.lk),), dtype=torch.uint8, device="cuda")

    def backward(do_, dbias_):
        if path == "ranges":
            dma.dma_attn_bwd_ranges(q, k, v, ts, te, bias, state, o, do_, lse, c.scale_f32, c.causal, dq, dk, dv,
                                    dbias_, ws)
        elif path == "bits":
            dma.dma_attn_bwd_bits(q, k, v, mbits, bias, state, o, do_, lse, c.scale_f32, c.causal, dq, dk, dv, dbias_,
                                  ws)
        else:
            dma.dma_attn_bwd(q, k, v, mask, bias, state, o, do_, lse, c.scale_f32, c.causal, dq, dk, dv, dbias_, ws)

    log(f"[{c.name}/{path}] classify / fwd / bwd on the GPU", flush=True)
    if path == "ranges":
        dma.dma_block_classify_ranges(ts, te, c.b, c.hkv, c.lq, c.lk, c.causal, state)
        dma.dma_attn_fwd_ranges(q, k, v, ts, te, bias, state, c.scale_f32, c.causal, o, lse)
    elif path == "bits":
        dma.dma_block_classify_bits(mask, c.b, c.hkv, c.lq, c.lk, c.causal, state, mbits)
        dma.dma_attn_fwd_bits(q, k, v, mbits, bias, state, c.scale_f32, c.causal, o, lse)
    elif path == "fused":
        dma.dma_attn_fwd_classify(q, k, v, mask, bias, c.scale_f32, c.causal, state, o, lse)
    else:
        dma.dma_block_classify(mask, c.b, c.hkv, c.lq, c.lk, c.causal, state)
        dma.dma_attn_fwd(q, k, v, mask, bias, state, c.scale_f32, c.causal, o, lse)
    backward(do, dbias)
    torch.cuda.synchronize()
    st = state.cpu().numpy()
    assert np.array_equal(st, ref_state), f"{c.name}: block_state differs in {int((st != ref_state).sum())} blocks"
    log(f"[{c.name}/{path}] block bitmap bit-exact ({int((st != 0).sum())} non-SKIP blocks)", flush=True)

    sample = synth.sample_row_blocks(c, n_blocks)
    got = []
    for bb, r0 in sample:
        r1 = min(r0 + 64, c.lq)
        got.append(dict(o=f64(o[bb, r0:r1]), lse=lse[bb, :, r0:r1].cpu().numpy().astype(np.float64),
                        dq=f64(dq[bb, r0:r1]), db=f64(dbias[bb, :, r0:r1])))
    # second backward: dO restricted to the sampled rows
    do_s = torch.zeros_like(do)
    for bb, r0 in sample:
        do_s[bb, r0:r0 + 64] = do[bb, r0:r0 + 64]
    backward(do_s, None)
    torch.cuda.synchronize()
    dk_s, dv_s = f64(dk), f64(dv)
    del q, k, v, do, mask, bias, dbias, do_s
    torch.cuda.empty_cache()

    log(f"[{c.name}/{path}] oracle on {len(sample)} sampled query blocks", flush=True)
    kh, vh = oracle.bf16_to_f64(synth.k(c)), oracle.bf16_to_f64(synth.v(c))
    workers = max(1, min(16, os.cpu_count() or 1))
    with threadpool_limits(1), concurrent.futures.ThreadPoolExecutor(workers) as ex:
        refs = list(ex.map(lambda s: _oracle_block(c, kh[s[0]], vh[s[0]], s[0], s[1]), sample))
    dk_ref = np.zeros((c.b, c.lk, c.hkv, c.d))
    dv_ref = np.zeros((c.b, c.lk, c.hkv, c.d))
    for (bb, _), r in zip(sample, refs):
        dk_ref[bb] += r["dk"]
        dv_ref[bb] += r["dv"]
    o_err = check_o(np.concatenate([g_["o"] for g_ in got]), np.concatenate([r["o"] for r in refs]),
                    f"{c.name} O", c.v_std)
    check_lse(np.concatenate([g_["lse"] for g_ in got], axis=1), np.concatenate([r["lse"] for r in refs], axis=1))
    errs = {"O_maxabs": o_err}
    errs["dQ"] = check_grad(np.concatenate([g_["dq"] for g_ in got]), np.concatenate([r["dq"] for r in refs]),
                            f"{c.name} dQ")
    db_g = np.concatenate([g_["db"] for g_ in got], axis=1)
    errs["dBias"] = check_grad(db_g, np.concatenate([r["db"] for r in refs], axis=1), f"{c.name} dBias")
    valid = np.concatenate([r["valid"] for r in refs], axis=1)
    assert np.all(db_g[~valid] == 0.0), f"{c.name}: dBias not exactly zero on invalid entries"
    errs["dK"] = check_grad(dk_s, dk_ref, f"{c.name} dK (sampled rows)")
    errs["dV"] = check_grad(dv_s, dv_ref, f"{c.name} dV (sampled rows)")
    log(f"[{c.name}/{path}] parity ok {{" + ", ".join(f"{k_}: {v_:.2e}" for k_, v_ in errs.items()) + "}", flush=True)
    return errs
