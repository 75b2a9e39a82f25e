"""Column-range mask input (dma_*_ranges): every output is compared with the fp64 oracle on the
expanded mask (the tolerances of gpu_harness), equals the dense entry point's on that mask bit
for bit, and the bitmap equals the oracle's classification of that mask.

Ranges: random intervals per key column (empty ones, and bounds below 0 and past lq included),
document-packed intervals ([j, end of j's document), the pages' column-wise form), causal and
not, ragged sizes, head dims 64 and 128, group sizes 1..8; at full size the Doc-packed workload.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import Case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    synth.build()


def random_ranges(rng, c):
    s = rng.integers(-8, c.lq + 8, size=(c.b, c.hkv, c.lk))
    e = s + rng.integers(-16, c.lq // 2 + 16, size=s.shape)  # some empty (e <= s)
    return s.astype(np.int32), e.astype(np.int32)


def doc_ranges(c):
    import gpu_harness as H

    return H.doc_ranges(c)


def expand(s, e, lq):
    i = np.arange(lq)[None, None, :, None]
    keep = (s[:, :, None, :] <= i) & (i < e[:, :, None, :])
    return np.where(keep, np.uint16(0x3F80), np.uint16(0)).astype(np.uint16)


def run_both(c, s, e):
    """Dense path on the expanded mask and range path; returns both outputs (host bits)."""
    import block_sparse_dynamic_amd as dma
    import gpu_harness as H

    dc = H.DeviceCase(c)
    mask_h = expand(s, e, c.lq)
    dc.mask_h, dc.mask = mask_h, H.to_dev(mask_h)
    ts, te = torch.from_numpy(s).cuda(), torch.from_numpy(e).cuda()
    st_r = torch.empty_like(dc.state)
    dma.dma_block_classify_ranges(ts, te, c.b, c.hkv, c.lq, c.lk, c.causal, st_r)
    dc.classify()
    dc.forward()
    dc.backward()
    torch.cuda.synchronize()
    dense = [H.bits(t) for t in (dc.o, dc.dq, dc.dk, dc.dv, dc.dbias)] + [dc.lse.cpu().numpy()]
    o, lse = torch.empty_like(dc.q), torch.empty_like(dc.lse)
    dma.dma_attn_fwd_ranges(dc.q, dc.k, dc.v, ts, te, dc.bias, st_r, c.scale_f32, c.causal, o, lse)
    dq, dk, dv = torch.empty_like(dc.q), torch.empty_like(dc.k), torch.empty_like(dc.v)
    dbias = torch.full_like(dc.dbias, float("nan"))
    ws = torch.empty(dma.dma_attn_bwd_workspace_size(c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.causal), dtype=torch.uint8,
                     device="cuda")
    dma.dma_attn_bwd_ranges(dc.q, dc.k, dc.v, ts, te, dc.bias, st_r, o, dc.do, lse, c.scale_f32, c.causal, dq, dk, dv,
                            dbias, ws)
    torch.cuda.synchronize()
    rng_out = [H.bits(t) for t in (o, dq, dk, dv, dbias)] + [lse.cpu().numpy()]
    # the range path's own outputs against the oracle on the expanded mask
    H.compare_with_oracle(f"{c.name} (ranges)", c, dc.q_h, dc.k_h, dc.v_h, mask_h, dc.bias_h, dc.do_h, o, lse, dq, dk,
                          dv, dbias)
    return dc, mask_h, st_r.cpu().numpy(), dense, rng_out


CASES = [
    Case("rng_causal", 40, 1, 200, 200, 8, 2, 128, True, "none"),
    Case("rng_noncausal", 41, 2, 264, 136, 4, 4, 64, False, "none"),
    Case("rng_lq_lt_lk", 42, 1, 130, 264, 8, 1, 64, True, "none"),
    Case("rng_g1", 43, 1, 256, 256, 2, 2, 128, True, "none"),
]


@pytest.mark.parametrize("c", CASES, ids=[c.name for c in CASES])
def test_random_ranges_equal_dense(c):
    rng = np.random.default_rng(c.stream_id)
    s, e = random_ranges(rng, c)
    dc, mask_h, st_r, dense, rng_out = run_both(c, s, e)
    st_ref = oracle.classify(mask_h, c.b, c.hkv, c.lq, c.lk, c.causal)
    assert np.array_equal(st_r, st_ref), "range bitmap differs from the oracle's"
    assert np.array_equal(dc.state.cpu().numpy(), st_ref)
    for name, a, b in zip(("o", "dq", "dk", "dv", "dbias", "lse"), dense, rng_out):
        assert np.array_equal(a, b), f"{c.name}: {name} differs between the range and the dense path"


def test_doc_ranges_equal_dense_and_oracle():
    import gpu_harness as H

    c = Case("doc_ranges", 44, 1, 1000, 1000, 4, 1, 128, True, "doc", doc_min=64, doc_max=300, bias_std=0.5,
             fill="lowest")
    s, e = doc_ranges(c)
    dc, mask_h, st_r, dense, rng_out = run_both(c, s, e)
    assert np.array_equal(mask_h, synth.mask_bias(c)[0]), "doc ranges expand to the generator's dense mask"
    st_ref = oracle.classify(mask_h, c.b, c.hkv, c.lq, c.lk, c.causal)
    assert np.array_equal(st_r, st_ref)
    for name, a, b in zip(("o", "dq", "dk", "dv", "dbias", "lse"), dense, rng_out):
        assert np.array_equal(a, b), f"{name} differs between the range and the dense path"


@pytest.mark.timeout(1200)
def test_doc_packed_full_size_oracle():
    """The Doc-packed workload at full size through the range entry points, against the oracle:
    whole bitmap, 64 sampled query blocks of O / LSE / dQ / dBias, sampled-row dK / dV."""
    import gpu_harness as H

    H.check_full_case(synth.CASES["docpacked"], n_blocks=64, path="ranges")
    torch.cuda.empty_cache()


def test_doc_packed_full_size_equal_dense():
    """The Doc-packed workload at full size (b=1, L=32768, Hq=8, Hkv=2, d=128): bitmap and
    every output of the range path bit-identical to the dense path."""
    import block_sparse_dynamic_amd as dma
    from synth.device import upload_dense, upload_mask_bias

    c = synth.CASES["docpacked"]
    print(f"[{c.name}] generating and uploading", flush=True)
    q, k, v, do = upload_dense(c)
    mask, bias = upload_mask_bias(c)
    s, e = doc_ranges(c)
    ts, te = torch.from_numpy(s).cuda(), torch.from_numpy(e).cuda()
    shape = dma.block_state_shape(c.b, c.hkv, c.lq, c.lk)
    st_d = torch.empty(shape, dtype=torch.uint8, device="cuda")
    st_r = torch.empty_like(st_d)
    dma.dma_block_classify(mask, c.b, c.hkv, c.lq, c.lk, c.causal, st_d)
    dma.dma_block_classify_ranges(ts, te, c.b, c.hkv, c.lq, c.lk, c.causal, st_r)
    torch.cuda.synchronize()
    assert torch.equal(st_d, st_r), "range bitmap differs from the dense one"
    ws = torch.empty(dma.dma_attn_bwd_workspace_size(c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.causal), dtype=torch.uint8,
                     device="cuda")
    outs = []
    for ranges in (False, True):
        print(f"[{c.name}] {'range' if ranges else 'dense'} path", flush=True)
        o = torch.empty_like(q)
        lse = torch.empty((c.b, c.hq, c.lq), dtype=torch.float32, device="cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dbias = torch.empty((c.b, c.hkv, c.lq, c.lk), dtype=torch.bfloat16, device="cuda")
        if ranges:
            dma.dma_attn_fwd_ranges(q, k, v, ts, te, bias, st_r, c.scale_f32, c.causal, o, lse)
            dma.dma_attn_bwd_ranges(q, k, v, ts, te, bias, st_r, o, do, lse, c.scale_f32, c.causal, dq, dk, dv, dbias,
                                    ws)
        else:
            dma.dma_attn_fwd(q, k, v, mask, bias, st_d, c.scale_f32, c.causal, o, lse)
            dma.dma_attn_bwd(q, k, v, mask, bias, st_d, o, do, lse, c.scale_f32, c.causal, dq, dk, dv, dbias, ws)
        torch.cuda.synchronize()
        outs.append((o, lse, dq, dk, dv, dbias))
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv", "dbias"), *outs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), f"{name} differs"
