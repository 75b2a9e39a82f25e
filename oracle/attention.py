"""fp64 reference of dynamic-mask attention with an additive bias (test infrastructure only).

Sources (the three pages this method is described on):

* Flash-DMA README, features and usage example: mask and bias are 4-D tensors of
  shape (batch, num_kv_heads, query_len, key_len); the mask is 0/1 in bf16 and is
  built from the bias by a per-row top-k; gradients flow to query, key, value and
  bias; blocks whose mask OR-reduces to zero are skipped in forward and backward.
* Flash-DMA issue "Project Progress": masked positions of QK^T are set to -inf,
  the valid positions are scaled, then the bias is added; the mask is applied
  again when the attention weights multiply V.
* FlashMask README, Formulation and Key Features: O = softmax(QK^T/sqrt(d) + M)V,
  and blocks are fully masked, partially masked or unmasked.

Readings where the pages leave a step open (each is listed with its reason in
the design notes of the repository):

* scale multiplies QK^T only; the bias is added after scaling, unscaled.
* a mask element attends iff its value is non-zero (bits & 0x7FFF != 0).
* mask and causality combine by AND; causal alignment is bottom-right,
  key j is visible from query i iff j <= i + lk - lq.
* query head h uses KV head h // (hq / hkv).
* a row with no valid key has O = 0, LSE = +inf and zero gradients.
* dBias of a KV head is the sum of dS over the query heads of its group, and is
  exactly 0 on invalid entries.
* block classes on 64 x 64 (query x key) blocks: SKIP if no element is valid,
  FULL if all 4096 positions exist and are valid, PARTIAL otherwise.

Everything is computed by definition on whole rows: no tiling, no online
softmax, no skipping.  Inputs come in as bf16 bit patterns (numpy uint16) and
are decoded exactly to fp64 here.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

BLOCK = 64
SKIP, PARTIAL, FULL = 0, 1, 2
BF16_LOWEST_BITS = 0xFF7F


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: bf16 is the upper half of an fp32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attends(mask_bits: np.ndarray) -> np.ndarray:
    """A mask element lets its query see its key iff its value is non-zero."""
    return (np.asarray(mask_bits, dtype=np.uint16) & 0x7FFF) != 0


def valid_rows(mask_rows: Optional[np.ndarray], rows: np.ndarray, lq: int, lk: int, causal: bool) -> np.ndarray:
    """valid[..., n, j] for query rows ``rows`` (absolute indices) and all keys j.

    mask_rows: [..., n, lk] bf16 bits or None (no mask: every key attends).
    """
    rows = np.asarray(rows, dtype=np.int64)
    if mask_rows is None:
        v = np.ones((len(rows), lk), dtype=bool)
    else:
        v = attends(mask_rows)
    if causal:
        j = np.arange(lk, dtype=np.int64)
        v = v & (j[None, :] <= rows[:, None] + (lk - lq))
    return v


def classify_plane_rows(mask_rows: Optional[np.ndarray], row0: int, lq: int, lk: int, causal: bool) -> np.ndarray:
    """Block classes of the block rows covered by query rows [row0, row0 + n) of one plane.

    ``row0`` must be a multiple of BLOCK and the rows must cover whole block rows
    (or run to lq).  Returns uint8 [n_block_rows, ceil(lk / BLOCK)].
    """
    assert row0 % BLOCK == 0
    n = lq - row0 if mask_rows is None else mask_rows.shape[-2]
    n = min(n, lq - row0)
    rows = np.arange(row0, row0 + n)
    v = valid_rows(None if mask_rows is None else mask_rows[:n], rows, lq, lk, causal)
    nqb = (n + BLOCK - 1) // BLOCK
    nkb = (lk + BLOCK - 1) // BLOCK
    pad = np.zeros((nqb * BLOCK, nkb * BLOCK), dtype=bool)  # positions outside the matrix are not valid
    pad[:n, :lk] = v
    blocks = pad.reshape(nqb, BLOCK, nkb, BLOCK)
    anyv = blocks.any(axis=(1, 3))
    allv = blocks.all(axis=(1, 3))
    out = np.where(allv, FULL, np.where(anyv, PARTIAL, SKIP)).astype(np.uint8)
    return out


def classify(mask: Optional[np.ndarray], b: int, hkv: int, lq: int, lk: int, causal: bool) -> np.ndarray:
    """uint8 [b, hkv, ceil(lq/64), ceil(lk/64)] of SKIP / PARTIAL / FULL (whole tensor)."""
    nqb = (lq + BLOCK - 1) // BLOCK
    nkb = (lk + BLOCK - 1) // BLOCK
    out = np.empty((b, hkv, nqb, nkb), dtype=np.uint8)
    for bb in range(b):
        for g in range(hkv):
            m = None if mask is None else mask[bb, g]
            out[bb, g] = classify_plane_rows(m, 0, lq, lk, causal)
    return out


def _scores(qh: np.ndarray, kg: np.ndarray, bias_g: Optional[np.ndarray], valid: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T + B on valid positions, -inf elsewhere (one head, rows n x keys)."""
    s = scale * (qh @ kg.T)
    if bias_g is not None:
        s = s + bias_g
    return np.where(valid, s, -np.inf)


def forward_rows(q_rows, k, v, mask_rows, bias_rows, scale, causal, rows, lq):
    """Forward pass for a set of query rows of one batch element.

    q_rows    [n, hq, d]   fp64 query rows
    k, v      [lk, hkv, d] fp64
    mask_rows [hkv, n, lk] bf16 bits or None
    bias_rows [hkv, n, lk] fp64 or None
    rows      absolute query indices of the n rows
    Returns o [n, hq, d] and lse [hq, n] (fp64; lse = +inf on rows with no valid key).
    """
    n, hq, d = q_rows.shape
    lk, hkv, _ = k.shape
    G = hq // hkv
    o = np.zeros((n, hq, d))
    lse = np.full((hq, n), np.inf)
    for g in range(hkv):
        valid = valid_rows(None if mask_rows is None else mask_rows[g], rows, lq, lk, causal)
        has = valid.any(axis=1)
        for h in range(g * G, (g + 1) * G):
            s = _scores(q_rows[:, h, :], k[:, g, :], None if bias_rows is None else bias_rows[g], valid, scale)
            m = np.where(has, s.max(axis=1), 0.0)
            e = np.where(valid, np.exp(s - m[:, None]), 0.0)
            z = e.sum(axis=1)
            p = np.where(has[:, None], e / np.where(has, z, 1.0)[:, None], 0.0)
            o[:, h, :] = p @ v[:, g, :]
            lse[h] = np.where(has, m + np.log(np.where(has, z, 1.0)), np.inf)
    return o, lse


def backward_rows(q_rows, k, v, mask_rows, bias_rows, scale, causal, rows, lq, do_rows):
    """Backward pass restricted to a set of query rows of one batch element.

    Returns (dq_rows [n, hq, d], dk_part [lk, hkv, d], dv_part [lk, hkv, d],
    dbias_rows [hkv, n, lk]).  dk_part / dv_part are the contributions of these
    rows; over all rows they are dK and dV.  Uses
      P = softmax of the valid scores (0 elsewhere), D_i = sum_c dO_ic O_ic,
      dP = dO V^T, dS = P (dP - D), dQ = scale dS K, dK = scale dS^T Q,
      dV = P^T dO, dBias_g = sum over the heads of group g of dS.
    """
    n, hq, d = q_rows.shape
    lk, hkv, _ = k.shape
    G = hq // hkv
    dq = np.zeros((n, hq, d))
    dk = np.zeros((lk, hkv, d))
    dv = np.zeros((lk, hkv, d))
    dbias = np.zeros((hkv, n, lk))
    for g in range(hkv):
        valid = valid_rows(None if mask_rows is None else mask_rows[g], rows, lq, lk, causal)
        has = valid.any(axis=1)
        for h in range(g * G, (g + 1) * G):
            s = _scores(q_rows[:, h, :], k[:, g, :], None if bias_rows is None else bias_rows[g], valid, scale)
            m = np.where(has, s.max(axis=1), 0.0)
            e = np.where(valid, np.exp(s - m[:, None]), 0.0)
            z = np.where(has, e.sum(axis=1), 1.0)
            p = np.where(has[:, None], e / z[:, None], 0.0)
            o = p @ v[:, g, :]
            dd = (do_rows[:, h, :] * o).sum(axis=1)
            dp = do_rows[:, h, :] @ v[:, g, :].T
            ds = p * (dp - dd[:, None])
            dq[:, h, :] = scale * (ds @ k[:, g, :])
            dk[:, g, :] += scale * (ds.T @ q_rows[:, h, :])
            dv[:, g, :] += p.T @ do_rows[:, h, :]
            dbias[g] += ds
    return dq, dk, dv, dbias


def _decode(x):
    return None if x is None else bf16_to_f64(x)


def forward(q, k, v, mask, bias, scale, causal):
    """Whole-tensor forward.  q [b,lq,hq,d], k/v [b,lk,hkv,d], mask/bias [b,hkv,lq,lk]
    (bf16 bits; mask and bias may be None).  Returns o [b,lq,hq,d], lse [b,hq,lq] (fp64)."""
    b, lq, hq, d = q.shape
    rows = np.arange(lq)
    o = np.zeros((b, lq, hq, d))
    lse = np.zeros((b, hq, lq))
    for bb in range(b):
        o[bb], lse[bb] = forward_rows(
            bf16_to_f64(q[bb]), bf16_to_f64(k[bb]), bf16_to_f64(v[bb]),
            None if mask is None else mask[bb], None if bias is None else bf16_to_f64(bias[bb]),
            scale, causal, rows, lq)
    return o, lse


def backward(q, k, v, mask, bias, scale, causal, do):
    """Whole-tensor backward: (dq, dk, dv, dbias) in fp64 (dbias None when bias is None)."""
    b, lq, hq, d = q.shape
    lk, hkv = k.shape[1], k.shape[2]
    rows = np.arange(lq)
    dq = np.zeros((b, lq, hq, d))
    dk = np.zeros((b, lk, hkv, d))
    dv = np.zeros((b, lk, hkv, d))
    dbias = np.zeros((b, hkv, lq, lk))
    for bb in range(b):
        dq[bb], dk[bb], dv[bb], dbias[bb] = backward_rows(
            bf16_to_f64(q[bb]), bf16_to_f64(k[bb]), bf16_to_f64(v[bb]),
            None if mask is None else mask[bb], None if bias is None else bf16_to_f64(bias[bb]),
            scale, causal, rows, lq, bf16_to_f64(do[bb]))
    return dq, dk, dv, (dbias if bias is not None else None)


def topk_mask(bias_bits: np.ndarray, k: int):
    """The mask construction of the Flash-DMA README usage example, on bf16 rows.

    For rows longer than k: keep the k largest bias values of each row (ties go
    to the lowest key index, the reading taken for the unsorted top-k), mark
    them 1 unless the value is the bf16 minimum, 0 elsewhere, then overwrite the
    bias at masked positions with the bf16 minimum.  Shorter rows keep an
    all-ones mask and the bias unchanged.  Returns (mask bits, bias bits).
    """
    bias_bits = np.asarray(bias_bits, dtype=np.uint16)
    lk = bias_bits.shape[-1]
    one = np.uint16(0x3F80)
    if lk <= k:
        return np.full(bias_bits.shape, one, dtype=np.uint16), bias_bits.copy()
    vals = bf16_to_f64(bias_bits)
    order = np.argsort(-vals, axis=-1, kind="stable")[..., :k]
    picked = np.take_along_axis(bias_bits, order, axis=-1)
    keep = picked != BF16_LOWEST_BITS
    mask = np.zeros(bias_bits.shape, dtype=np.uint16)
    np.put_along_axis(mask, order, np.where(keep, one, np.uint16(0)), axis=-1)
    bias = np.where(mask == 0, np.uint16(BF16_LOWEST_BITS), bias_bits).astype(np.uint16)
    return mask, bias
