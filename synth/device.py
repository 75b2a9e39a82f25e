"""Upload synthetic workloads to the device in row chunks (marshalling only).

The mask and bias planes of the large workloads are 4-8 GiB each; they are drawn
chunk by chunk into a pinned host buffer and copied straight into the device
tensors, so host memory stays at one chunk.  ``on_chunk(bb, g, row0, mask, bias)``
lets a caller look at each host chunk (e.g. to classify it on the CPU) before it
is overwritten.
"""
from __future__ import annotations

import numpy as np
import torch

from . import Case, do, k, mask_bias_rows, q, v


def _dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def upload_dense(c: Case, device="cuda"):
    """q, k, v, do as bf16 device tensors."""
    return tuple(_dev(f(c), device) for f in (q, k, v, do))


def upload_mask_bias(c: Case, device="cuda", chunk_rows: int = 1024, on_chunk=None):
    """(mask, bias) bf16 device tensors [b, hkv, lq, lk] (None where the case has none)."""
    shape = (c.b, c.hkv, c.lq, c.lk)
    mask = torch.empty(shape, dtype=torch.bfloat16, device=device) if c.mask != "none" else None
    bias = torch.empty(shape, dtype=torch.bfloat16, device=device) if c.bias else None
    if mask is None and bias is None and on_chunk is None:
        return None, None
    rows = min(chunk_rows, c.lq)
    hm = torch.empty((rows, c.lk), dtype=torch.int16, pin_memory=True)
    hb = torch.empty((rows, c.lk), dtype=torch.int16, pin_memory=True)
    for bb in range(c.b):
        for g in range(c.hkv):
            for r0 in range(0, c.lq, rows):
                n = min(rows, c.lq - r0)
                m_np = hm.numpy().view(np.uint16)[:n]
                b_np = hb.numpy().view(np.uint16)[:n]
                mm, bi = mask_bias_rows(c, bb, g, r0, n, mask_out=m_np if mask is not None else None,
                                        bias_out=b_np if bias is not None else None,
                                        want_mask=mask is not None, want_bias=bias is not None)
                if on_chunk is not None:
                    on_chunk(bb, g, r0, mm, bi)
                if mask is not None:
                    mask[bb, g, r0:r0 + n].view(torch.int16).copy_(hm[:n], non_blocking=False)
                if bias is not None:
                    bias[bb, g, r0:r0 + n].view(torch.int16).copy_(hb[:n], non_blocking=False)
    return mask, bias
