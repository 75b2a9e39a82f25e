"""The backward in bands of query blocks.  Given a workspace below dma_attn_bwd_workspace_size (down
to dma_attn_bwd_workspace_size_min), dma_attn_bwd runs the main and dQ kernels once per band of
consecutive query blocks and gathers dK and dV in fp32 sums.

Checked, with the smallest workspace (bands of about one query block) and with a third of the dS
slots: every output against the fp64 oracle (whole tensors, the tolerances of gpu_harness); dQ
and dBias equal to the one-pass backward's bit for bit (the same items, the same sums); dK and dV
through the oracle (they differ from the one pass by the fp32 rounding of the band sums); two
runs bit-identical.  Cases: causal and not, ragged sizes, lq > lk (leading query blocks without a
live pair, whose bands launch only dBias zero-fill), head dims 64 and 128, group sizes 1..8, no
mask and no bias, no dBias output, the dense, bit-packed and column-range mask inputs.  At full
size the Long workload (b=1, L=65536, Hq=8, Hkv=1, d=128, top-k 2048) runs in a workspace of one
mask plane (b*hkv*L*L bf16, a quarter of its one-pass workspace) and is checked on sampled query
blocks.
"""
import numpy as np
import pytest
import torch

import synth
from synth import Case

pytestmark = pytest.mark.gpu

CASES = [
    Case("bands_causal", 70, 1, 600, 600, 8, 2, 128, True, "blocks"),
    Case("bands_ragged_d64_g1", 71, 2, 520, 544, 2, 2, 64, True, "topk", 96),
    Case("bands_noncausal_g2", 72, 1, 330, 264, 2, 1, 128, False, "blocks"),
    Case("bands_lq_gt_lk", 73, 1, 456, 200, 4, 1, 128, True, "topk", 40),
    Case("bands_doc_g8", 74, 1, 1000, 1000, 8, 1, 64, True, "doc", doc_min=64, doc_max=300, bias_std=0.5,
         fill="lowest"),
    Case("bands_no_mask_no_bias", 76, 1, 328, 328, 4, 2, 64, True, "none", bias=False),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    synth.build()


def workspace_bytes(c: Case, which: str) -> int:
    import block_sparse_dynamic_amd as dma

    full = dma.dma_attn_bwd_workspace_size(c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.causal)
    least = dma.dma_attn_bwd_workspace_size_min(c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.causal)
    assert 0 < least < full
    return least if which == "min" else least + (full - least) // 3


@pytest.mark.parametrize("which", ["min", "third"])
@pytest.mark.parametrize("c", CASES, ids=[c.name for c in CASES])
def test_banded_backward(c, which):
    import gpu_harness as H

    ws = workspace_bytes(c, which)
    print(f"case {c} workspace {ws} bytes ({which})", flush=True)
    dc = H.DeviceCase(c)
    dc.classify()
    dc.forward()
    dc.backward()
    torch.cuda.synchronize()
    one = [H.bits(t) for t in (dc.dq, dc.dk, dc.dv, dc.dbias)]
    dc.backward(ws_bytes=ws)
    torch.cuda.synchronize()
    first = [H.bits(t) for t in (dc.dq, dc.dk, dc.dv, dc.dbias)]
    dc.backward(ws_bytes=ws)
    torch.cuda.synchronize()
    again = [H.bits(t) for t in (dc.dq, dc.dk, dc.dv, dc.dbias)]
    for name, a, b in zip(("dq", "dk", "dv", "dbias"), first, again):
        assert np.array_equal(a, b), f"{c.name}: {name} differs between two banded runs"
    assert np.array_equal(first[0], one[0]), "dQ differs from the one-pass backward"
    assert np.array_equal(first[3], one[3]), "dBias differs from the one-pass backward"
    H.compare_with_oracle(f"{c.name} (bands, {which})", c, dc.q_h, dc.k_h, dc.v_h, dc.mask_h, dc.bias_h, dc.do_h,
                          dc.o, dc.lse, dc.dq, dc.dk, dc.dv, dc.dbias)


def test_banded_backward_without_dbias():
    """No dBias output: the bands still give the one-pass dQ bit for bit and dK, dV against the oracle."""
    import gpu_harness as H

    c = CASES[0]
    ws = workspace_bytes(c, "min")
    print(f"case {c} workspace {ws} bytes (min), no dBias", flush=True)
    dc = H.DeviceCase(c)
    dc.classify()
    dc.forward()
    dc.backward(want_dbias=False)
    torch.cuda.synchronize()
    one_dq = H.bits(dc.dq)
    dc.backward(want_dbias=False, ws_bytes=ws)
    torch.cuda.synchronize()
    assert np.array_equal(H.bits(dc.dq), one_dq), "dQ differs from the one-pass backward"
    H.compare_with_oracle(f"{c.name} (bands, no dBias)", c, dc.q_h, dc.k_h, dc.v_h, dc.mask_h, dc.bias_h, dc.do_h,
                          dc.o, dc.lse, dc.dq, dc.dk, dc.dv, None)


def test_banded_bits_and_ranges_backward():
    """The bit-packed and column-range backward entry points run in bands as dma_attn_bwd does."""
    import block_sparse_dynamic_amd as dma
    import gpu_harness as H

    c = Case("bands_paths", 75, 1, 520, 520, 4, 2, 128, True, "doc", doc_min=64, doc_max=200, bias_std=0.5)
    ws = torch.empty(workspace_bytes(c, "min"), dtype=torch.uint8, device="cuda")
    print(f"case {c} workspace {ws.numel()} bytes", flush=True)
    dc = H.DeviceCase(c)
    dc.classify()
    dc.forward()
    dc.backward()
    torch.cuda.synchronize()
    one = [H.bits(t) for t in (dc.dq, dc.dbias)]
    # bit-packed PARTIAL blocks
    mb = torch.empty((dma.dma_mask_bits_size(c.b, c.hkv, c.lq, c.lk),), dtype=torch.uint8, device="cuda")
    st_b = torch.empty_like(dc.state)
    dma.dma_block_classify_bits(dc.mask, c.b, c.hkv, c.lq, c.lk, c.causal, st_b, mb)
    dq, dk, dv = torch.empty_like(dc.q), torch.empty_like(dc.k), torch.empty_like(dc.v)
    dbias = torch.full_like(dc.dbias, float("nan"))
    dma.dma_attn_bwd_bits(dc.q, dc.k, dc.v, mb, dc.bias, st_b, dc.o, dc.do, dc.lse, c.scale_f32, c.causal, dq, dk, dv,
                          dbias, ws)
    torch.cuda.synchronize()
    assert np.array_equal(H.bits(dq), one[0]) and np.array_equal(H.bits(dbias), one[1])
    H.compare_with_oracle(f"{c.name} (bits, bands)", c, dc.q_h, dc.k_h, dc.v_h, dc.mask_h, dc.bias_h, dc.do_h, dc.o,
                          dc.lse, dq, dk, dv, dbias)
    # column ranges of the same document mask
    s, e = H.doc_ranges(c)
    ts, te = torch.from_numpy(s).cuda(), torch.from_numpy(e).cuda()
    st_r = torch.empty_like(dc.state)
    dma.dma_block_classify_ranges(ts, te, c.b, c.hkv, c.lq, c.lk, c.causal, st_r)
    dq, dk, dv = torch.empty_like(dc.q), torch.empty_like(dc.k), torch.empty_like(dc.v)
    dbias = torch.full_like(dc.dbias, float("nan"))
    dma.dma_attn_bwd_ranges(dc.q, dc.k, dc.v, ts, te, dc.bias, st_r, dc.o, dc.do, dc.lse, c.scale_f32, c.causal, dq,
                            dk, dv, dbias, ws)
    torch.cuda.synchronize()
    H.compare_with_oracle(f"{c.name} (ranges, bands)", c, dc.q_h, dc.k_h, dc.v_h, dc.mask_h, dc.bias_h, dc.do_h, dc.o,
                          dc.lse, dq, dk, dv, dbias)


def test_long_workload_in_one_mask_plane_of_workspace():
    import gpu_harness as H

    c = synth.CASES["long"]
    plane = c.b * c.hkv * c.lq * c.lk * 2
    H.check_full_case(c, n_blocks=32, ws_bytes=plane)
