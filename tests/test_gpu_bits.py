"""Bit-packed PARTIAL-block mask (dma_*_bits): the classification writes, for every PARTIAL
block, exactly the packed form of the mask (the oracle's attends(), one bit per element, zero
past lq and lk), leaves every other block's bytes untouched, and the attention passes that read
those bits return the dense entry points' results bit for bit; those outputs are compared with
the fp64 oracle as well (the tolerances of gpu_harness).

Cases: ragged sizes, lq < lk and lq > lk (rows without keys), head dims 64 and 128, group sizes
1..8, block/top-k/document/all-ones masks, causal and not, a mask without a bias; at full size
the Top-k headline workload (b=2, L=16384, Hq=16, Hkv=4, d=128, k=1024).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import Case

pytestmark = pytest.mark.gpu

FILL = 0xA5  # what the bits buffer holds before the classification


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    synth.build()


def packed_blocks(mask_h: np.ndarray, lq: int, lk: int) -> np.ndarray:
    """uint8 [b, hkv, nqb, nkb, 64, 8]: row r of a block as 8 little-endian bytes, bit c of the
    64-bit word = whether element (r, c) of the block attends (0 outside the matrix)."""
    b, hkv = mask_h.shape[:2]
    nqb, nkb = (lq + 63) // 64, (lk + 63) // 64
    att = np.zeros((b, hkv, nqb * 64, nkb * 64), dtype=bool)
    att[:, :, :lq, :lk] = oracle.attends(mask_h)
    att = att.reshape(b, hkv, nqb, 64, nkb, 64).transpose(0, 1, 2, 4, 3, 5)
    return np.packbits(att.reshape(b, hkv, nqb, nkb, 64, 8, 8), axis=-1, bitorder="little")[..., 0]


def run_both(c: Case):
    import block_sparse_dynamic_amd as dma
    import gpu_harness as H

    dc = H.DeviceCase(c)
    dc.classify()
    dc.forward()
    dc.backward()
    torch.cuda.synchronize()
    dense = [H.bits(t) for t in (dc.o, dc.dq, dc.dk, dc.dv, dc.dbias)] + [dc.lse.cpu().numpy()]
    nbytes = dma.dma_mask_bits_size(c.b, c.hkv, c.lq, c.lk)
    mb = torch.full((nbytes,), FILL, dtype=torch.uint8, device="cuda")
    st_b = torch.empty_like(dc.state)
    dma.dma_block_classify_bits(dc.mask, c.b, c.hkv, c.lq, c.lk, c.causal, st_b, mb)
    o, lse = torch.empty_like(dc.q), torch.empty_like(dc.lse)
    dma.dma_attn_fwd_bits(dc.q, dc.k, dc.v, mb, dc.bias, st_b, c.scale_f32, c.causal, o, lse)
    dq, dk, dv = torch.empty_like(dc.q), torch.empty_like(dc.k), torch.empty_like(dc.v)
    dbias = torch.full_like(dc.dbias, float("nan"))
    ws = torch.empty(dma.dma_attn_bwd_workspace_size(c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.causal), dtype=torch.uint8,
                     device="cuda")
    dma.dma_attn_bwd_bits(dc.q, dc.k, dc.v, mb, dc.bias, st_b, o, dc.do, lse, c.scale_f32, c.causal, dq, dk, dv,
                          dbias, ws)
    torch.cuda.synchronize()
    out = [H.bits(t) for t in (o, dq, dk, dv, dbias)] + [lse.cpu().numpy()]
    H.compare_with_oracle(f"{c.name} (bits)", c, dc.q_h, dc.k_h, dc.v_h, dc.mask_h, dc.bias_h, dc.do_h, o, lse, dq,
                          dk, dv, dbias)
    return dc, st_b.cpu().numpy(), mb.cpu().numpy(), dense, out


CASES = [
    Case("bits_blocks_causal", 60, 2, 200, 200, 8, 2, 128, True, "blocks"),
    Case("bits_blocks_noncausal", 61, 1, 264, 264, 4, 4, 64, False, "blocks"),
    Case("bits_lq_lt_lk", 62, 1, 130, 264, 8, 2, 64, True, "blocks"),
    Case("bits_lq_gt_lk", 63, 1, 200, 136, 4, 1, 128, True, "blocks"),
    Case("bits_topk_g1", 64, 1, 256, 256, 2, 2, 128, True, "topk", 100),
    Case("bits_topk_g8_mask_only", 65, 1, 256, 256, 16, 2, 128, True, "topk", 96, bias=False),
    Case("bits_doc", 66, 1, 1000, 1000, 4, 1, 128, True, "doc", doc_min=64, doc_max=300, bias_std=0.5,
         fill="lowest"),
    Case("bits_ones_noncausal_ragged", 67, 1, 200, 136, 4, 1, 64, False, "ones"),
]


@pytest.mark.parametrize("c", CASES, ids=[c.name for c in CASES])
def test_bits_equal_packed_mask_and_dense_results(c):
    dc, st_b, mb, dense, out = run_both(c)
    st_ref = oracle.classify(dc.mask_h, c.b, c.hkv, c.lq, c.lk, c.causal)
    assert np.array_equal(st_b, st_ref), "bitmap of the bit-writing classification differs from the oracle's"
    assert np.array_equal(dc.state.cpu().numpy(), st_ref)
    nqb, nkb = st_ref.shape[2:]
    blocks = mb.reshape(c.b, c.hkv, nqb, nkb, 64, 8)
    part = st_ref == oracle.PARTIAL
    want = packed_blocks(dc.mask_h, c.lq, c.lk)
    assert np.array_equal(blocks[part], want[part]), "PARTIAL-block bits differ from the packed mask"
    assert np.all(blocks[~part] == FILL), "bytes of a SKIP or FULL block were written"
    print(c.name, "PARTIAL blocks:", int(part.sum()), "of", part.size, flush=True)
    for name, a, b in zip(("o", "dq", "dk", "dv", "dbias", "lse"), dense, out):
        assert np.array_equal(a, b), f"{c.name}: {name} differs between the bit and the dense path"


@pytest.mark.timeout(1200)
def test_headline_full_size_oracle():
    """The Top-k headline workload at full size through the bit entry points, against the
    oracle: whole bitmap, 64 sampled query blocks of O / LSE / dQ / dBias, sampled-row dK / dV."""
    import gpu_harness as H

    H.check_full_case(synth.CASES["headline"], n_blocks=64, path="bits")
    torch.cuda.empty_cache()


def test_headline_full_size_equal_dense():
    """The Top-k headline workload at full size: bitmap and every output of the bit path
    bit-identical to the dense path's, and the bits of sampled PARTIAL blocks equal to the
    packed mask rows."""
    import block_sparse_dynamic_amd as dma
    from synth.device import upload_dense, upload_mask_bias

    c = synth.CASES["headline"]
    print(f"[{c.name}] generating and uploading", flush=True)
    q, k, v, do = upload_dense(c)
    mask, bias = upload_mask_bias(c)
    shape = dma.block_state_shape(c.b, c.hkv, c.lq, c.lk)
    st_d = torch.empty(shape, dtype=torch.uint8, device="cuda")
    st_b = torch.empty_like(st_d)
    mb = torch.empty((dma.dma_mask_bits_size(c.b, c.hkv, c.lq, c.lk),), dtype=torch.uint8, device="cuda")
    dma.dma_block_classify(mask, c.b, c.hkv, c.lq, c.lk, c.causal, st_d)
    dma.dma_block_classify_bits(mask, c.b, c.hkv, c.lq, c.lk, c.causal, st_b, mb)
    torch.cuda.synchronize()
    assert torch.equal(st_d, st_b), "bit-writing classification's bitmap differs from the dense one"
    # bits of seeded PARTIAL blocks against the mask rows they pack
    rng = np.random.default_rng(7)
    st_h = st_b.cpu().numpy()
    part = np.argwhere(st_h == oracle.PARTIAL)
    nqb, nkb = shape[2:]
    blocks = mb.view(c.b, c.hkv, nqb, nkb, 64, 8)
    for bb, g, qb, kb in part[rng.choice(len(part), size=32, replace=False)]:
        m = mask[bb, g, qb * 64:(qb + 1) * 64, kb * 64:(kb + 1) * 64].contiguous().view(torch.int16).cpu().numpy()
        want = packed_blocks(m.view(np.uint16)[None, None], 64, 64)[0, 0, 0, 0]
        assert np.array_equal(blocks[bb, g, qb, kb].cpu().numpy(), want), f"block {(bb, g, qb, kb)}"
    ws = torch.empty(dma.dma_attn_bwd_workspace_size(c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.causal), dtype=torch.uint8,
                     device="cuda")
    outs = []
    for use_bits in (False, True):
        print(f"[{c.name}] {'bit' if use_bits else 'dense'} path", flush=True)
        o = torch.empty_like(q)
        lse = torch.empty((c.b, c.hq, c.lq), dtype=torch.float32, device="cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dbias = torch.empty((c.b, c.hkv, c.lq, c.lk), dtype=torch.bfloat16, device="cuda")
        if use_bits:
            dma.dma_attn_fwd_bits(q, k, v, mb, bias, st_b, c.scale_f32, c.causal, o, lse)
            dma.dma_attn_bwd_bits(q, k, v, mb, bias, st_b, o, do, lse, c.scale_f32, c.causal, dq, dk, dv, dbias, ws)
        else:
            dma.dma_attn_fwd(q, k, v, mask, bias, st_d, c.scale_f32, c.causal, o, lse)
            dma.dma_attn_bwd(q, k, v, mask, bias, st_d, o, do, lse, c.scale_f32, c.causal, dq, dk, dv, dbias, ws)
        torch.cuda.synchronize()
        outs.append([t.view(torch.int16) if t.dtype == torch.bfloat16 else t for t in (o, lse, dq, dk, dv, dbias)])
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv", "dbias"), *outs):
        assert torch.equal(a, b), f"{name} differs"
