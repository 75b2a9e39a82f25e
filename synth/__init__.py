"""Seeded synthetic inputs for dynamic-mask attention.

This module draws inputs only: it holds none of the attention arithmetic and is
the one piece shared by the oracle side and the device side of every test and
of the benchmark.  The sampling itself lives in ``synth.c`` (counter-based
SplitMix64, Box-Muller, bf16 round-to-nearest-even, top-k and document mask
recipes); this file names the workloads and marshals arrays.

All tensors are returned as ``numpy.uint16`` arrays of bf16 bit patterns.

Workloads (shapes and recipes of the five benchmark configurations):

* ``tiny``      b=1 L=256 Hq=2 Hkv=1 d=64, top-k 128 on an N(0,1) bias, causal,
                scale 1/8 -- the setup of the Flash-DMA README usage example.
* ``mid``       b=1 L=4096 Hq=32 Hkv=8 d=128, top-k 2048, causal.
* ``headline``  b=2 L=16384 Hq=16 Hkv=4 d=128, top-k 1024, causal.
* ``docpacked`` b=1 L=32768 Hq=8 Hkv=2 d=128, documents of U{512..8192}
                tokens, causal inside each document (FlashMask column ranges),
                bias N(0, 0.5^2) on valid entries, bf16 minimum elsewhere.
* ``long``      b=1 L=65536 Hq=8 Hkv=1 d=128, top-k 2048, causal.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_SRC_PATH = os.path.join(_HERE, "synth.c")

MASK_KINDS = {"topk": 0, "doc": 1, "blocks": 2, "ones": 3, "none": -1}
FILLS = {"keep": 0, "lowest": 1, "nan": 2}

# tensor tags of the stream keys
TAG_Q, TAG_K, TAG_V, TAG_DO, TAG_BIAS, TAG_DOCS, TAG_SAMPLE, TAG_MASK = 1, 2, 3, 4, 5, 6, 7, 8


def build(force: bool = False) -> str:
    """Compile synth.c into libsynth.so with gcc and OpenMP."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC_PATH, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, f64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [vp, i32]
        lib.synth_draw.restype = u64
        lib.synth_draw.argtypes = [u64, u64]
        lib.synth_bf16_rne.restype = ctypes.c_uint16
        lib.synth_bf16_rne.argtypes = [f64]
        lib.synth_normal_bf16.restype = None
        lib.synth_normal_bf16.argtypes = [u64, u64, i64, f64, vp]
        lib.synth_rows.restype = None
        lib.synth_rows.argtypes = [u64, u64, i32, i64, i64, i64, i64, f64, vp, i32, i32, vp, vp]
        lib.synth_topk_rows.restype = None
        lib.synth_topk_rows.argtypes = [vp, i64, i64, i64, vp, vp]
        _lib = lib
    return _lib


def key(*parts: int) -> int:
    arr = np.asarray(parts, dtype=np.int64)
    return int(_load().synth_key(arr.ctypes.data, len(parts)))


def draw(k: int, ctr: int) -> int:
    return int(_load().synth_draw(k, ctr))


def bf16_rne(x: float) -> int:
    """bf16 bits of fp64 ``x`` rounded to nearest even (the generator's rounding)."""
    return int(_load().synth_bf16_rne(float(x)))


def normal_bf16(k: int, start: int, n: int, std: float = 1.0, out: Optional[np.ndarray] = None) -> np.ndarray:
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == n
    _load().synth_normal_bf16(k, start, n, std, out.ctypes.data)
    return out


def topk_rows(bias_bits: np.ndarray, k: int):
    """The generator's top-k recipe applied to given bf16 rows [n, lk]: (mask, bias)."""
    x = np.ascontiguousarray(bias_bits, dtype=np.uint16)
    n, lk = x.shape
    m = np.empty_like(x)
    b = np.empty_like(x)
    _load().synth_topk_rows(x.ctypes.data, n, lk, k, m.ctypes.data, b.ctypes.data)
    return m, b


@dataclasses.dataclass(frozen=True)
class Case:
    """One attention workload: shapes, flags and the input recipe."""

    name: str
    stream_id: int
    b: int
    lq: int
    lk: int
    hq: int
    hkv: int
    d: int
    causal: bool = True
    mask: str = "topk"  # topk | doc | blocks | ones | none
    topk: int = 0
    bias: bool = True
    bias_std: float = 1.0
    fill: str = "keep"  # masked-bias fill for doc/blocks/ones: keep | lowest | nan
    doc_min: int = 512
    doc_max: int = 8192
    seed: int = 0
    scale: Optional[float] = None  # None: fp32(1/sqrt(d))
    v_std: float = 1.0  # standard deviation of V

    @property
    def G(self) -> int:
        return self.hq // self.hkv

    @property
    def scale_f32(self) -> float:
        s = self.scale if self.scale is not None else 1.0 / np.sqrt(self.d)
        return float(np.float32(s))

    def with_(self, **kw) -> "Case":
        return dataclasses.replace(self, **kw)


# The five benchmark workloads (stream ids 0..4 in this order).
CASES = {
    "tiny": Case("tiny", 0, 1, 256, 256, 2, 1, 64, True, "topk", 128, scale=1.0 / 8.0),
    "mid": Case("mid", 1, 1, 4096, 4096, 32, 8, 128, True, "topk", 2048),
    "headline": Case("headline", 2, 2, 16384, 16384, 16, 4, 128, True, "topk", 1024),
    "docpacked": Case("docpacked", 3, 1, 32768, 32768, 8, 2, 128, True, "doc", 0, bias_std=0.5, fill="lowest"),
    "long": Case("long", 4, 1, 65536, 65536, 8, 1, 128, True, "topk", 2048),
}


def _tensor_key(c: Case, tag: int) -> int:
    return key(c.seed, c.stream_id, tag)


def dense(c: Case, tag: int, shape, start: int = 0, n: Optional[int] = None) -> np.ndarray:
    """Flat elements [start, start+n) of an N(0,1) tensor with the given tag."""
    total = int(np.prod(shape))
    if n is None:
        n = total - start
    return normal_bf16(_tensor_key(c, tag), start, n)


def q(c: Case) -> np.ndarray:
    return dense(c, TAG_Q, (c.b, c.lq, c.hq, c.d)).reshape(c.b, c.lq, c.hq, c.d)


def k(c: Case) -> np.ndarray:
    return dense(c, TAG_K, (c.b, c.lk, c.hkv, c.d)).reshape(c.b, c.lk, c.hkv, c.d)


def v(c: Case) -> np.ndarray:
    n = c.b * c.lk * c.hkv * c.d
    return normal_bf16(_tensor_key(c, TAG_V), 0, n, std=c.v_std).reshape(c.b, c.lk, c.hkv, c.d)


def do(c: Case) -> np.ndarray:
    return dense(c, TAG_DO, (c.b, c.lq, c.hq, c.d)).reshape(c.b, c.lq, c.hq, c.d)


def rows_of(c: Case, tag: int, h: int, bb: int, rows: np.ndarray) -> np.ndarray:
    """Rows of a [b, L, h, d] tensor (all heads) for batch bb: shape [len(rows), h, d]."""
    L = c.lq if tag in (TAG_Q, TAG_DO) else c.lk
    out = np.empty((len(rows), h, c.d), dtype=np.uint16)
    kk = _tensor_key(c, tag)
    for n, r in enumerate(rows):
        start = ((bb * L + int(r)) * h) * c.d
        normal_bf16(kk, start, h * c.d, out=out[n].reshape(-1))
    return out


def doc_bounds(c: Case) -> np.ndarray:
    """Document boundaries: lengths uniform on {doc_min..doc_max}, the last cut to fit."""
    kk = _tensor_key(c, TAG_DOCS)
    span = c.doc_max - c.doc_min + 1
    bounds = [0]
    t = 0
    while bounds[-1] < c.lq:
        length = c.doc_min + draw(kk, t) % span
        bounds.append(min(c.lq, bounds[-1] + length))
        t += 1
    return np.asarray(bounds, dtype=np.int64)


def mask_bias_rows(c: Case, bb: int, g: int, row0: int, nrows: int, mask_out=None, bias_out=None, want_mask=True, want_bias=True):
    """Rows [row0, row0+nrows) of the (bb, g) plane: (mask, bias), each [nrows, lk] or None.

    ``mask_out`` / ``bias_out`` may be given as C-contiguous uint16 buffers to fill.
    """
    want_mask = want_mask and c.mask != "none"
    want_bias = want_bias and c.bias
    kind = MASK_KINDS[c.mask] if c.mask != "none" else MASK_KINDS["ones"]
    if want_mask and mask_out is None:
        mask_out = np.empty((nrows, c.lk), dtype=np.uint16)
    if want_bias and bias_out is None:
        bias_out = np.empty((nrows, c.lk), dtype=np.uint16)
    if not want_mask:
        mask_out = None
    if not want_bias:
        bias_out = None
    if mask_out is None and bias_out is None:
        return None, None
    for a in (mask_out, bias_out):
        if a is not None:
            assert a.dtype == np.uint16 and a.flags.c_contiguous and a.size == nrows * c.lk
    bk = key(c.seed, c.stream_id, TAG_BIAS, bb, g)
    mk = key(c.seed, c.stream_id, TAG_MASK, bb, g)
    bounds = doc_bounds(c) if c.mask == "doc" else np.zeros(2, dtype=np.int64)
    fill = FILLS[c.fill]
    _load().synth_rows(bk, mk, kind, c.lk, row0, nrows, c.topk, c.bias_std, bounds.ctypes.data,
                       len(bounds) - 1, fill,
                       bias_out.ctypes.data if bias_out is not None else None,
                       mask_out.ctypes.data if mask_out is not None else None)
    return mask_out, bias_out


def mask_bias(c: Case):
    """Whole mask and bias, [b, hkv, lq, lk] each (None where the case has none). Small cases only."""
    m = np.empty((c.b, c.hkv, c.lq, c.lk), dtype=np.uint16) if c.mask != "none" else None
    bi = np.empty((c.b, c.hkv, c.lq, c.lk), dtype=np.uint16) if c.bias else None
    for bb in range(c.b):
        for g in range(c.hkv):
            mask_bias_rows(c, bb, g, 0, c.lq,
                           mask_out=m[bb, g] if m is not None else None,
                           bias_out=bi[bb, g] if bi is not None else None)
    return m, bi


def sample_row_blocks(c: Case, count: int = 64, block: int = 64):
    """Seeded query-row blocks (batch, first row): the first block of batch 0 and the
    last block of the last batch are always included, the rest drawn without replacement."""
    nb = (c.lq + block - 1) // block
    total = c.b * nb
    forced = [0, total - 1]
    kk = _tensor_key(c, TAG_SAMPLE)
    chosen = list(dict.fromkeys(forced))
    t = 0
    while len(chosen) < min(count, total):
        x = draw(kk, t) % total
        t += 1
        if x not in chosen:
            chosen.append(int(x))
    chosen.sort()
    return [(x // nb, (x % nb) * block) for x in chosen]
