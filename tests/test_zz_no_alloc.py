"""dma_attn_bwd_noalloc (the backward whose workspace is the library's fixed device array, for
callers that cannot allocate) gives the same outputs as dma_attn_bwd with a caller workspace:
two calls in a row, the second on a smaller problem (the array keeps the first call's bytes,
and nothing may depend on them).  Bit-identical: both run the same kernels on the same inputs."""
import numpy as np
import pytest
import torch

import synth
from synth import Case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    synth.build()


def _run(c: Case):
    import block_sparse_dynamic_amd as dma
    import gpu_harness as H

    assert dma.dma_attn_bwd_workspace_size(c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.causal) <= dma.NOALLOC_SCRATCH_BYTES
    dc = H.DeviceCase(c)
    dc.classify()
    dc.forward()
    dc.backward()  # dma_attn_bwd with its own workspace
    ref = [H.bits(t) for t in (dc.dq, dc.dk, dc.dv, dc.dbias)]
    dq, dk, dv = torch.empty_like(dc.q), torch.empty_like(dc.k), torch.empty_like(dc.v)
    dbias = torch.full_like(dc.dbias, float("nan"))
    dma.dma_attn_bwd_noalloc(dc.q, dc.k, dc.v, dc.mask, dc.bias, dc.state, dc.o, dc.do, dc.lse, c.scale_f32, c.causal,
                             dq, dk, dv, dbias)
    torch.cuda.synchronize()
    return ref, [H.bits(t) for t in (dq, dk, dv, dbias)]


def test_noalloc_equals_workspace_backward_twice_shrinking():
    big = Case("noalloc_big", 50, 1, 1000, 1000, 8, 2, 128, True, "blocks")
    small = Case("noalloc_small", 51, 1, 300, 264, 4, 1, 64, True, "topk", 40)
    for c in (big, small):
        print(f"case {c.name}", flush=True)
        ref, got = _run(c)
        for name, a, b in zip(("dq", "dk", "dv", "dbias"), ref, got):
            assert np.array_equal(a, b), f"{c.name}: {name} differs from dma_attn_bwd's"
