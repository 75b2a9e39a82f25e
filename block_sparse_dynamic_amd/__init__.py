"""Dynamic-mask attention with an additive bias on AMD Instinct MI355X (gfx950).

Thin Python binding of ``libdma.so`` (declared in ``include/dma.h``): every
function below marshals torch tensors into the C ABI call of the same name and
raises on a non-zero status.  All arithmetic runs in the library's HIP kernels;
there is no fallback path -- importing this package fails if the library is
missing, and every call fails on tensors that are not on a HIP device.

``dma_attention`` wraps classification, forward and backward as a
``torch.autograd.Function`` with the call signature of the Flash-DMA README
usage example (query, key, value, attn_mask, attn_bias, is_causal, scale);
gradients flow to query, key, value and attn_bias.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch  # loads the process's HIP runtime before libdma.so binds to it

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdma.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "dma.h")

DMA_OK = 0
BLOCK_SKIP, BLOCK_PARTIAL, BLOCK_FULL = 0, 1, 2

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python block_sparse_dynamic_amd/build.py` "
        "(hipcc, gfx950); there is no fallback implementation")

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_lib.dma_block_size.restype = _i32
_lib.dma_block_size.argtypes = []
_lib.dma_status_string.restype = ctypes.c_char_p
_lib.dma_status_string.argtypes = [_i32]
_lib.dma_block_classify.restype = _i32
_lib.dma_block_classify.argtypes = [_vp, _i64, _i64, _i64, _i64, _i32, _vp, _vp]
_lib.dma_attn_fwd.restype = _i32
_lib.dma_attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _f32, _i32, _vp, _vp,
                              _vp]
_lib.dma_attn_fwd_classify.restype = _i32
_lib.dma_attn_fwd_classify.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _f32, _i32, _vp,
                                       _vp, _vp, _vp]
_lib.dma_attn_bwd_workspace_size.restype = _sz
_lib.dma_attn_bwd_workspace_size.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _i32]
_lib.dma_attn_bwd_workspace_size_min.restype = _sz
_lib.dma_attn_bwd_workspace_size_min.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _i32]
_lib.dma_attn_bwd.restype = _i32
_lib.dma_attn_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _f32,
                              _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.dma_block_classify_ranges.restype = _i32
_lib.dma_block_classify_ranges.argtypes = [_vp, _vp, _i64, _i64, _i64, _i64, _i32, _vp, _vp]
_lib.dma_attn_fwd_ranges.restype = _i32
_lib.dma_attn_fwd_ranges.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _f32, _i32,
                                     _vp, _vp, _vp]
_lib.dma_attn_bwd_ranges.restype = _i32
_lib.dma_attn_bwd_ranges.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                     _i64, _f32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.dma_mask_bits_size.restype = _sz
_lib.dma_mask_bits_size.argtypes = [_i64, _i64, _i64, _i64]
_lib.dma_block_classify_bits.restype = _i32
_lib.dma_block_classify_bits.argtypes = [_vp, _i64, _i64, _i64, _i64, _i32, _vp, _vp, _vp]
_lib.dma_attn_fwd_bits.restype = _i32
_lib.dma_attn_fwd_bits.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _f32, _i32, _vp,
                                   _vp, _vp]
_lib.dma_attn_bwd_bits.restype = _i32
_lib.dma_attn_bwd_bits.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                   _f32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.dma_attn_bwd_part.restype = _i32
_lib.dma_attn_bwd_part.argtypes = [_i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                   _f32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
BWD_PREPARE, BWD_MAIN, BWD_DQ = 0, 1, 2
_lib.dma_attn_bwd_noalloc.restype = _i32
_lib.dma_attn_bwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                      _f32, _i32, _vp, _vp, _vp, _vp, _vp]
NOALLOC_SCRATCH_BYTES = 64 << 20  # DMA_NOALLOC_SCRATCH_BYTES of include/dma.h
_lib.dma_topk_mask.restype = _i32
_lib.dma_topk_mask.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp]


class DMAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {dma_status_string(status)} (status {status})")
        self.status = status


def dma_block_size() -> int:
    return int(_lib.dma_block_size())


def dma_status_string(status: int) -> str:
    return _lib.dma_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, st: int):
    if st != DMA_OK:
        raise DMAError(fn, st)


def block_state_shape(b: int, hkv: int, lq: int, lk: int):
    n = dma_block_size()
    return (b, hkv, (lq + n - 1) // n, (lk + n - 1) // n)


def _shapes(fn: str, q, k, v, planes=(), qlike=(), kvlike=(), lse=None, ranges=(), state=None):
    """Sizes (b, lq, lk, hq, hkv, d) from q [b, lq, hq, d] and k [b, lk, hkv, d], after checking
    that every other tensor has exactly the shape the C ABI reads or writes through it
    (the library takes plain pointers: a broadcast or mis-shaped tensor would be read or
    written past its end)."""
    def want(name, t, shape):
        if t is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{fn}: {name} must have shape {tuple(shape)}, got {tuple(t.shape)}")

    if q.dim() != 4 or k.dim() != 4:
        raise ValueError(f"{fn}: q must be [b, lq, hq, d] and k [b, lk, hkv, d]")
    b, lq, hq, d = q.shape
    lk, hkv = k.shape[1], k.shape[2]
    want("k", k, (b, lk, hkv, d))
    want("v", v, (b, lk, hkv, d))
    for name, t in planes:
        want(name, t, (b, hkv, lq, lk))
    for name, t in qlike:
        want(name, t, (b, lq, hq, d))
    for name, t in kvlike:
        want(name, t, (b, lk, hkv, d))
    want("lse", lse, (b, hq, lq))
    for name, t in ranges:
        want(name, t, (b, hkv, lk))
    want("block_state", state, block_state_shape(b, hkv, lq, lk))
    return b, lq, lk, hq, hkv, d


def dma_topk_mask(bias: torch.Tensor, k: int, mask_out: torch.Tensor, bias_out: torch.Tensor, stream=None) -> None:
    """Keep the k largest bias values of each row (last dimension): mask_out 1 there, and
    bias_out the bias there and the smallest bf16 elsewhere.  bias_out may be bias itself."""
    lk = bias.shape[-1]
    rows = bias.numel() // lk
    for name, t in (("mask_out", mask_out), ("bias_out", bias_out)):
        if tuple(t.shape) != tuple(bias.shape):
            raise ValueError(f"dma_topk_mask: {name} must have the bias's shape {tuple(bias.shape)}")
    st = _lib.dma_topk_mask(_ptr(bias, "bias", torch.bfloat16), rows, lk, int(k),
                            _ptr(mask_out, "mask_out", torch.bfloat16), _ptr(bias_out, "bias_out", torch.bfloat16),
                            _stream(stream))
    _check("dma_topk_mask", st)


def dma_block_classify(mask: Optional[torch.Tensor], b: int, hkv: int, lq: int, lk: int, is_causal: bool,
                       block_state: torch.Tensor, stream=None) -> None:
    if mask is not None and tuple(mask.shape) != (b, hkv, lq, lk):
        raise ValueError(f"dma_block_classify: mask must have shape {(b, hkv, lq, lk)}, got {tuple(mask.shape)}")
    if tuple(block_state.shape) != block_state_shape(b, hkv, lq, lk):
        raise ValueError(f"dma_block_classify: block_state must have shape {block_state_shape(b, hkv, lq, lk)}")
    st = _lib.dma_block_classify(_ptr(mask, "mask", torch.bfloat16), b, hkv, lq, lk, int(bool(is_causal)),
                                 _ptr(block_state, "block_state", torch.uint8), _stream(stream))
    _check("dma_block_classify", st)


def dma_attn_fwd(q, k, v, mask, bias, block_state, scale: float, is_causal: bool, o, lse, stream=None) -> None:
    b, lq, lk, hq, hkv, d = _shapes("dma_attn_fwd", q, k, v, planes=(("mask", mask), ("bias", bias)),
                                    qlike=(("o", o),), lse=lse, state=block_state)
    st = _lib.dma_attn_fwd(_ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16), _ptr(v, "v", torch.bfloat16),
                           _ptr(mask, "mask", torch.bfloat16), _ptr(bias, "bias", torch.bfloat16),
                           _ptr(block_state, "block_state", torch.uint8), b, lq, lk, hq, hkv, d, float(scale),
                           int(bool(is_causal)), _ptr(o, "o", torch.bfloat16), _ptr(lse, "lse", torch.float32),
                           _stream(stream))
    _check("dma_attn_fwd", st)


def dma_attn_fwd_classify(q, k, v, mask, bias, scale: float, is_causal: bool, block_state, o, lse,
                          stream=None) -> None:
    """Forward that also writes the block classification (block_state is an output)."""
    b, lq, lk, hq, hkv, d = _shapes("dma_attn_fwd_classify", q, k, v, planes=(("mask", mask), ("bias", bias)),
                                    qlike=(("o", o),), lse=lse, state=block_state)
    st = _lib.dma_attn_fwd_classify(_ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16),
                                    _ptr(v, "v", torch.bfloat16), _ptr(mask, "mask", torch.bfloat16),
                                    _ptr(bias, "bias", torch.bfloat16), b, lq, lk, hq, hkv, d, float(scale),
                                    int(bool(is_causal)), _ptr(block_state, "block_state", torch.uint8),
                                    _ptr(o, "o", torch.bfloat16), _ptr(lse, "lse", torch.float32), _stream(stream))
    _check("dma_attn_fwd_classify", st)


def dma_attn_bwd_workspace_size(b: int, lq: int, lk: int, hq: int, hkv: int, d: int, is_causal: bool) -> int:
    return int(_lib.dma_attn_bwd_workspace_size(b, lq, lk, hq, hkv, d, int(bool(is_causal))))


def dma_attn_bwd_workspace_size_min(b: int, lq: int, lk: int, hq: int, hkv: int, d: int, is_causal: bool) -> int:
    return int(_lib.dma_attn_bwd_workspace_size_min(b, lq, lk, hq, hkv, d, int(bool(is_causal))))


def dma_attn_bwd(q, k, v, mask, bias, block_state, o, dout, lse, scale: float, is_causal: bool, dq, dk, dv, dbias,
                 workspace, stream=None) -> None:
    b, lq, lk, hq, hkv, d = _shapes("dma_attn_bwd", q, k, v, planes=(("mask", mask), ("bias", bias), ("dbias", dbias)),
                                    qlike=(("o", o), ("dout", dout), ("dq", dq)), kvlike=(("dk", dk), ("dv", dv)),
                                    lse=lse, state=block_state)
    st = _lib.dma_attn_bwd(_ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16), _ptr(v, "v", torch.bfloat16),
                           _ptr(mask, "mask", torch.bfloat16), _ptr(bias, "bias", torch.bfloat16),
                           _ptr(block_state, "block_state", torch.uint8), _ptr(o, "o", torch.bfloat16),
                           _ptr(dout, "dout", torch.bfloat16), _ptr(lse, "lse", torch.float32), b, lq, lk, hq, hkv,
                           d, float(scale), int(bool(is_causal)), _ptr(dq, "dq", torch.bfloat16),
                           _ptr(dk, "dk", torch.bfloat16), _ptr(dv, "dv", torch.bfloat16),
                           _ptr(dbias, "dbias", torch.bfloat16), _ptr(workspace, "workspace"),
                           workspace.numel() * workspace.element_size(), _stream(stream))
    _check("dma_attn_bwd", st)


def dma_attn_bwd_part(part: int, q, k, v, mask, bias, block_state, o, dout, lse, scale: float, is_causal: bool, dq,
                      dk, dv, dbias, workspace, stream=None) -> None:
    """One phase of dma_attn_bwd (BWD_PREPARE, BWD_MAIN, BWD_DQ, run in this order)."""
    b, lq, lk, hq, hkv, d = _shapes("dma_attn_bwd_part", q, k, v, planes=(("mask", mask), ("bias", bias), ("dbias", dbias)),
                                    qlike=(("o", o), ("dout", dout), ("dq", dq)), kvlike=(("dk", dk), ("dv", dv)),
                                    lse=lse, state=block_state)
    st = _lib.dma_attn_bwd_part(int(part), _ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16),
                                _ptr(v, "v", torch.bfloat16), _ptr(mask, "mask", torch.bfloat16),
                                _ptr(bias, "bias", torch.bfloat16), _ptr(block_state, "block_state", torch.uint8),
                                _ptr(o, "o", torch.bfloat16), _ptr(dout, "dout", torch.bfloat16),
                                _ptr(lse, "lse", torch.float32), b, lq, lk, hq, hkv, d, float(scale),
                                int(bool(is_causal)), _ptr(dq, "dq", torch.bfloat16), _ptr(dk, "dk", torch.bfloat16),
                                _ptr(dv, "dv", torch.bfloat16), _ptr(dbias, "dbias", torch.bfloat16),
                                _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    _check("dma_attn_bwd_part", st)


def dma_attn_bwd_noalloc(q, k, v, mask, bias, block_state, o, dout, lse, scale: float, is_causal: bool, dq, dk, dv,
                         dbias, stream=None) -> None:
    """dma_attn_bwd with the library's own fixed scratch array instead of a workspace (nothing is
    allocated); calls on one GPU must not overlap."""
    b, lq, lk, hq, hkv, d = _shapes("dma_attn_bwd_noalloc", q, k, v,
                                    planes=(("mask", mask), ("bias", bias), ("dbias", dbias)),
                                    qlike=(("o", o), ("dout", dout), ("dq", dq)), kvlike=(("dk", dk), ("dv", dv)),
                                    lse=lse, state=block_state)
    st = _lib.dma_attn_bwd_noalloc(_ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16),
                                   _ptr(v, "v", torch.bfloat16), _ptr(mask, "mask", torch.bfloat16),
                                   _ptr(bias, "bias", torch.bfloat16), _ptr(block_state, "block_state", torch.uint8),
                                   _ptr(o, "o", torch.bfloat16), _ptr(dout, "dout", torch.bfloat16),
                                   _ptr(lse, "lse", torch.float32), b, lq, lk, hq, hkv, d, float(scale),
                                   int(bool(is_causal)), _ptr(dq, "dq", torch.bfloat16),
                                   _ptr(dk, "dk", torch.bfloat16), _ptr(dv, "dv", torch.bfloat16),
                                   _ptr(dbias, "dbias", torch.bfloat16), _stream(stream))
    _check("dma_attn_bwd_noalloc", st)


def dma_block_classify_ranges(start_row, end_row, b: int, hkv: int, lq: int, lk: int, is_causal: bool, block_state,
                              stream=None) -> None:
    """Block classes from column ranges: key j of plane (b, g) attends rows start_row <= i < end_row."""
    for name, t in (("start_row", start_row), ("end_row", end_row)):
        if tuple(t.shape) != (b, hkv, lk):
            raise ValueError(f"dma_block_classify_ranges: {name} must have shape {(b, hkv, lk)}")
    if tuple(block_state.shape) != block_state_shape(b, hkv, lq, lk):
        raise ValueError(f"dma_block_classify_ranges: block_state must have shape {block_state_shape(b, hkv, lq, lk)}")
    st = _lib.dma_block_classify_ranges(_ptr(start_row, "start_row", torch.int32), _ptr(end_row, "end_row", torch.int32),
                                        b, hkv, lq, lk, int(bool(is_causal)),
                                        _ptr(block_state, "block_state", torch.uint8), _stream(stream))
    _check("dma_block_classify_ranges", st)


def dma_attn_fwd_ranges(q, k, v, start_row, end_row, bias, block_state, scale: float, is_causal: bool, o, lse,
                        stream=None) -> None:
    b, lq, lk, hq, hkv, d = _shapes("dma_attn_fwd_ranges", q, k, v, planes=(("bias", bias),), qlike=(("o", o),),
                                    lse=lse, ranges=(("start_row", start_row), ("end_row", end_row)),
                                    state=block_state)
    st = _lib.dma_attn_fwd_ranges(_ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16),
                                  _ptr(v, "v", torch.bfloat16), _ptr(start_row, "start_row", torch.int32),
                                  _ptr(end_row, "end_row", torch.int32), _ptr(bias, "bias", torch.bfloat16),
                                  _ptr(block_state, "block_state", torch.uint8), b, lq, lk, hq, hkv, d, float(scale),
                                  int(bool(is_causal)), _ptr(o, "o", torch.bfloat16), _ptr(lse, "lse", torch.float32),
                                  _stream(stream))
    _check("dma_attn_fwd_ranges", st)


def dma_attn_bwd_ranges(q, k, v, start_row, end_row, bias, block_state, o, dout, lse, scale: float, is_causal: bool,
                        dq, dk, dv, dbias, workspace, stream=None) -> None:
    b, lq, lk, hq, hkv, d = _shapes("dma_attn_bwd_ranges", q, k, v, planes=(("bias", bias), ("dbias", dbias)),
                                    qlike=(("o", o), ("dout", dout), ("dq", dq)), kvlike=(("dk", dk), ("dv", dv)),
                                    lse=lse, ranges=(("start_row", start_row), ("end_row", end_row)),
                                    state=block_state)
    st = _lib.dma_attn_bwd_ranges(_ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16),
                                  _ptr(v, "v", torch.bfloat16), _ptr(start_row, "start_row", torch.int32),
                                  _ptr(end_row, "end_row", torch.int32), _ptr(bias, "bias", torch.bfloat16),
                                  _ptr(block_state, "block_state", torch.uint8), _ptr(o, "o", torch.bfloat16),
                                  _ptr(dout, "dout", torch.bfloat16), _ptr(lse, "lse", torch.float32), b, lq, lk, hq,
                                  hkv, d, float(scale), int(bool(is_causal)), _ptr(dq, "dq", torch.bfloat16),
                                  _ptr(dk, "dk", torch.bfloat16), _ptr(dv, "dv", torch.bfloat16),
                                  _ptr(dbias, "dbias", torch.bfloat16), _ptr(workspace, "workspace"),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    _check("dma_attn_bwd_ranges", st)


def _bits_size(fn: str, mask_bits, b, hkv, lq, lk):
    need = dma_mask_bits_size(b, hkv, lq, lk)
    if mask_bits.numel() * mask_bits.element_size() < need:
        raise ValueError(f"{fn}: mask_bits must hold at least {need} bytes")


def dma_mask_bits_size(b: int, hkv: int, lq: int, lk: int) -> int:
    """Bytes of the bit-packed PARTIAL-block mask: 512 per 64 x 64 block."""
    return int(_lib.dma_mask_bits_size(b, hkv, lq, lk))


def dma_block_classify_bits(mask, b: int, hkv: int, lq: int, lk: int, is_causal: bool, block_state, mask_bits,
                            stream=None) -> None:
    """dma_block_classify plus, in the same pass, the mask bits of every PARTIAL block."""
    if mask is not None and tuple(mask.shape) != (b, hkv, lq, lk):
        raise ValueError(f"dma_block_classify_bits: mask must have shape {(b, hkv, lq, lk)}")
    if tuple(block_state.shape) != block_state_shape(b, hkv, lq, lk):
        raise ValueError(f"dma_block_classify_bits: block_state must have shape {block_state_shape(b, hkv, lq, lk)}")
    _bits_size("dma_block_classify_bits", mask_bits, b, hkv, lq, lk)
    st = _lib.dma_block_classify_bits(_ptr(mask, "mask", torch.bfloat16), b, hkv, lq, lk, int(bool(is_causal)),
                                      _ptr(block_state, "block_state", torch.uint8),
                                      _ptr(mask_bits, "mask_bits", torch.uint8), _stream(stream))
    _check("dma_block_classify_bits", st)


def dma_attn_fwd_bits(q, k, v, mask_bits, bias, block_state, scale: float, is_causal: bool, o, lse,
                      stream=None) -> None:
    b, lq, lk, hq, hkv, d = _shapes("dma_attn_fwd_bits", q, k, v, planes=(("bias", bias),), qlike=(("o", o),),
                                    lse=lse, state=block_state)
    _bits_size("dma_attn_fwd_bits", mask_bits, b, hkv, lq, lk)
    st = _lib.dma_attn_fwd_bits(_ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16),
                                _ptr(v, "v", torch.bfloat16), _ptr(mask_bits, "mask_bits", torch.uint8),
                                _ptr(bias, "bias", torch.bfloat16), _ptr(block_state, "block_state", torch.uint8), b,
                                lq, lk, hq, hkv, d, float(scale), int(bool(is_causal)), _ptr(o, "o", torch.bfloat16),
                                _ptr(lse, "lse", torch.float32), _stream(stream))
    _check("dma_attn_fwd_bits", st)


def dma_attn_bwd_bits(q, k, v, mask_bits, bias, block_state, o, dout, lse, scale: float, is_causal: bool, dq, dk, dv,
                      dbias, workspace, stream=None) -> None:
    b, lq, lk, hq, hkv, d = _shapes("dma_attn_bwd_bits", q, k, v, planes=(("bias", bias), ("dbias", dbias)),
                                    qlike=(("o", o), ("dout", dout), ("dq", dq)), kvlike=(("dk", dk), ("dv", dv)),
                                    lse=lse, state=block_state)
    _bits_size("dma_attn_bwd_bits", mask_bits, b, hkv, lq, lk)
    st = _lib.dma_attn_bwd_bits(_ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16),
                                _ptr(v, "v", torch.bfloat16), _ptr(mask_bits, "mask_bits", torch.uint8),
                                _ptr(bias, "bias", torch.bfloat16), _ptr(block_state, "block_state", torch.uint8),
                                _ptr(o, "o", torch.bfloat16), _ptr(dout, "dout", torch.bfloat16),
                                _ptr(lse, "lse", torch.float32), b, lq, lk, hq, hkv, d, float(scale),
                                int(bool(is_causal)), _ptr(dq, "dq", torch.bfloat16), _ptr(dk, "dk", torch.bfloat16),
                                _ptr(dv, "dv", torch.bfloat16), _ptr(dbias, "dbias", torch.bfloat16),
                                _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    _check("dma_attn_bwd_bits", st)


class _DMAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, query, key, value, attn_mask, attn_bias, is_causal, scale):
        b, lq, hq, d = query.shape
        lk, hkv = key.shape[1], key.shape[2]
        q, k, v = query.contiguous(), key.contiguous(), value.contiguous()
        m = attn_mask.contiguous() if attn_mask is not None else None
        bi = attn_bias.contiguous() if attn_bias is not None else None
        state = torch.empty(block_state_shape(b, hkv, lq, lk), dtype=torch.uint8, device=q.device)
        dma_block_classify(m, b, hkv, lq, lk, is_causal, state)
        o = torch.empty_like(q)
        lse = torch.empty((b, hq, lq), dtype=torch.float32, device=q.device)
        dma_attn_fwd(q, k, v, m, bi, state, scale, is_causal, o, lse)
        ctx.save_for_backward(q, k, v, m, bi, state, o, lse)
        ctx.is_causal, ctx.scale = is_causal, scale
        ctx.bias_grad = attn_bias is not None and ctx.needs_input_grad[4]
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, m, bi, state, o, lse = ctx.saved_tensors
        b, lq, hq, d = q.shape
        lk, hkv = k.shape[1], k.shape[2]
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dbias = torch.empty_like(bi) if ctx.bias_grad else None
        ws = torch.empty(dma_attn_bwd_workspace_size(b, lq, lk, hq, hkv, d, ctx.is_causal), dtype=torch.uint8,
                         device=q.device)
        dma_attn_bwd(q, k, v, m, bi, state, o, dout.contiguous(), lse, ctx.scale, ctx.is_causal, dq, dk, dv, dbias, ws)
        return dq, dk, dv, None, dbias, None, None


def dma_attention(query, key, value, attn_mask=None, attn_bias=None, is_causal=False, scale=None):
    """O = softmax(scale * Q K^T + bias, masked -> -inf) V with GQA; shapes as in include/dma.h.

    query [b, lq, hq, d], key/value [b, lk, hkv, d], attn_mask/attn_bias [b, hkv, lq, lk] (bf16, optional).
    scale defaults to 1/sqrt(d).  Returns [b, lq, hq, d].
    """
    if scale is None:
        scale = 1.0 / math.sqrt(query.shape[-1])
    return _DMAttention.apply(query, key, value, attn_mask, attn_bias, bool(is_causal), float(scale))


__all__ = [
    "dma_block_size", "dma_status_string", "dma_block_classify", "dma_attn_fwd", "dma_attn_bwd_workspace_size",
    "dma_attn_bwd_workspace_size_min",
    "dma_attn_bwd", "dma_attention", "block_state_shape", "DMAError", "LIB_PATH", "HEADER_PATH",
    "dma_block_classify_ranges", "dma_attn_fwd_ranges", "dma_attn_bwd_ranges", "dma_topk_mask", "dma_mask_bits_size",
    "dma_block_classify_bits", "dma_attn_fwd_bits", "dma_attn_bwd_bits", "dma_attn_bwd_noalloc", "dma_attn_bwd_part",
    "BWD_PREPARE", "BWD_MAIN", "BWD_DQ",
    "NOALLOC_SCRATCH_BYTES",
]
