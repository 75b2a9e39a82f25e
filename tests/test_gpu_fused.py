"""Forward with the block classification fused in (dma_attn_fwd_classify): the bitmap it writes
equals the oracle's classification bit for bit, and O and LSE equal those of dma_block_classify +
dma_attn_fwd bit for bit (the same blocks are computed in the same order).

Cases: ragged sizes, lq < lk and lq > lk (rows without keys), head dims 64 and 128, group sizes
1..16, block (SKIP, PARTIAL and FULL blocks), top-k, document and all-ones masks, no mask, no bias,
causal and not; at full size the Top-k headline workload (b=2, L=16384, Hq=16, Hkv=4, d=128, k=1024).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import Case

pytestmark = pytest.mark.gpu

CASES = [
    synth.CASES["tiny"],
    Case("fused_ragged_blocks", 40, 2, 200, 200, 8, 2, 128, True, "blocks"),
    Case("fused_blocks_noncausal", 41, 1, 264, 264, 4, 4, 64, False, "blocks"),
    Case("fused_lq_lt_lk", 42, 1, 130, 264, 8, 2, 64, True, "blocks"),
    Case("fused_lq_gt_lk", 43, 1, 200, 136, 4, 1, 128, True, "blocks"),
    Case("fused_no_mask", 44, 1, 320, 320, 8, 2, 128, True, "none", bias=False),
    Case("fused_mask_only", 45, 1, 192, 192, 4, 2, 128, True, "topk", 64, bias=False),
    Case("fused_g16", 46, 1, 128, 128, 16, 1, 64, True, "blocks"),
    Case("fused_doc", 47, 1, 1000, 1000, 4, 1, 128, True, "doc", doc_min=64, doc_max=300, bias_std=0.5,
         fill="lowest"),
    Case("fused_all_ones", 48, 1, 192, 192, 4, 1, 128, False, "ones"),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    synth.build()


def run_both(dma, q, k, v, mask, bias, c):
    """(state, o, lse) of the separate calls and of the fused call."""
    shape = dma.block_state_shape(c.b, c.hkv, c.lq, c.lk)
    st_a = torch.empty(shape, dtype=torch.uint8, device="cuda")
    st_b = torch.full(shape, 0xA5, dtype=torch.uint8, device="cuda")  # every byte must be written
    o_a, o_b = torch.empty_like(q), torch.full_like(q, float("nan"))
    lse_a = torch.empty((c.b, c.hq, c.lq), dtype=torch.float32, device="cuda")
    lse_b = torch.full_like(lse_a, float("nan"))
    dma.dma_block_classify(mask, c.b, c.hkv, c.lq, c.lk, c.causal, st_a)
    dma.dma_attn_fwd(q, k, v, mask, bias, st_a, c.scale_f32, c.causal, o_a, lse_a)
    dma.dma_attn_fwd_classify(q, k, v, mask, bias, c.scale_f32, c.causal, st_b, o_b, lse_b)
    torch.cuda.synchronize()
    return (st_a, o_a, lse_a), (st_b, o_b, lse_b)


def assert_same(a, b, name):
    st_a, o_a, lse_a = a
    st_b, o_b, lse_b = b
    assert torch.equal(st_a, st_b), f"{name}: bitmap differs in {int((st_a != st_b).sum())} blocks"
    assert torch.equal(o_a.view(torch.int16), o_b.view(torch.int16)), f"{name}: O differs"
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32)), f"{name}: LSE differs"


@pytest.mark.parametrize("c", CASES, ids=[c.name for c in CASES])
def test_fused_equals_separate_and_oracle(c):
    import block_sparse_dynamic_amd as dma
    import gpu_harness as H

    print(f"case {c}", flush=True)
    dc = H.DeviceCase(c)
    a, b = run_both(dma, dc.q, dc.k, dc.v, dc.mask, dc.bias, c)
    ref_st = oracle.classify(dc.mask_h, c.b, c.hkv, c.lq, c.lk, c.causal)
    assert np.array_equal(b[0].cpu().numpy(), ref_st), f"{c.name}: fused bitmap differs from the oracle"
    assert_same(a, b, c.name)
    o_ref, lse_ref = oracle.forward(dc.q_h, dc.k_h, dc.v_h, dc.mask_h, dc.bias_h, c.scale_f32, c.causal)
    H.check_o(H.f64(b[1]), o_ref, f"{c.name} fused O")
    H.check_lse(b[2].cpu().numpy().astype(np.float64), lse_ref)


@pytest.mark.timeout(600)
def test_headline_full_size_fused_equals_separate():
    import block_sparse_dynamic_amd as dma
    from synth.device import upload_dense, upload_mask_bias

    c = synth.CASES["headline"]
    print(f"case {c}", flush=True)
    q, k, v, _ = upload_dense(c)
    mask, bias = upload_mask_bias(c)
    a, b = run_both(dma, q, k, v, mask, bias, c)
    assert_same(a, b, c.name)
    st = b[0].cpu().numpy()
    print({"skip": int((st == 0).sum()), "partial": int((st == 1).sum()), "full": int((st == 2).sum())}, flush=True)
