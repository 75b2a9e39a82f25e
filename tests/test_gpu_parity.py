"""GPU parity of classify / forward / backward against the fp64 oracle, whole tensors.

Cases span several 64x64 tiles with ragged tails, all three block classes, NULL
mask and bias, lq != lk (bottom-right causal alignment, rows with no valid key),
group sizes 1..16, head dims 64 and 128, NaN stored in masked bias entries, and a
negative and a large scale.  The value range: the pages' top-k-filled bias passed
without its mask (valid keys holding the smallest bf16, rows whose every valid key
holds it), the largest and smallest bf16 as bias at valid positions, large but
unclamped biases, V of standard deviation 1e-6 and 1e4, and V beyond the fp16 range
at keys that are masked for some rows of a PARTIAL block.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import Case

pytestmark = pytest.mark.gpu

SMALL = [
    synth.CASES["tiny"],
    Case("ragged_blocks", 10, 2, 200, 200, 8, 2, 128, True, "blocks"),
    Case("ragged_blocks_noncausal", 11, 1, 264, 264, 4, 4, 64, False, "blocks"),
    Case("lq_lt_lk", 12, 1, 130, 264, 8, 2, 64, True, "blocks"),
    Case("lq_gt_lk_empty_rows", 13, 1, 200, 136, 4, 1, 128, True, "blocks"),
    Case("no_mask_no_bias", 14, 1, 320, 320, 8, 2, 128, True, "none", bias=False),
    Case("mask_only", 15, 1, 192, 192, 4, 2, 128, True, "topk", 64, bias=False),
    Case("bias_only_noncausal", 16, 2, 128, 256, 2, 2, 64, False, "none"),
    Case("g1_topk", 17, 1, 256, 256, 2, 2, 128, True, "topk", 100),
    Case("g8_topk", 18, 1, 256, 256, 16, 2, 128, True, "topk", 96),
    Case("g16_blocks", 19, 1, 128, 128, 16, 1, 64, True, "blocks"),
    Case("nan_in_masked_bias", 20, 1, 256, 256, 8, 2, 128, True, "blocks", fill="nan"),
    Case("doc_small", 21, 1, 1000, 1000, 4, 1, 128, True, "doc", doc_min=64, doc_max=300, bias_std=0.5,
         fill="lowest"),
    Case("all_ones_mask", 22, 1, 192, 192, 4, 1, 128, False, "ones"),
    # the forward carries scores as q.k + bias/|scale| and negates Q for a negative scale
    Case("negative_scale", 23, 1, 200, 200, 4, 2, 128, True, "blocks", scale=-0.09),
    Case("large_scale_d64", 24, 1, 192, 192, 4, 2, 64, True, "topk", 64, scale=0.5),
    # causal with few key pairs and at least 8 query blocks: the backward splits every pair's walk
    # over two workgroups that add their dK, dV in fp32 (ragged rows and keys)
    Case("split_pairs", 25, 1, 600, 600, 8, 2, 128, True, "blocks"),
    Case("split_pairs_d64_g1", 26, 2, 520, 544, 2, 2, 64, True, "topk", 96),
    # the smallest shapes: one query row over one 8-key chunk, a few decode-like rows over a ragged
    # key range, and one whole 64x64 block
    Case("one_row_one_chunk", 27, 1, 1, 8, 2, 1, 64, True, "ones"),
    Case("few_rows_ragged_keys", 28, 2, 3, 520, 4, 2, 128, True, "topk", 40),
    Case("single_block", 29, 1, 64, 64, 4, 4, 128, False, "blocks"),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    synth.build()


@pytest.mark.parametrize("c", SMALL, ids=[c.name for c in SMALL])
def test_small_case_parity(c):
    import gpu_harness as H

    print(f"case {c}", flush=True)
    H.check_small_case(c)


def test_page_example_loss_sum():
    """Flash-DMA README usage example: loss = output.sum(), so dO = 1 everywhere."""
    import gpu_harness as H

    c = synth.CASES["tiny"]
    ones = np.full((c.b, c.lq, c.hq, c.d), 0x3F80, dtype=np.uint16)
    H.check_small_case(c, do_bits=ones)


def test_autograd_wrapper_matches_oracle():
    """dma_attention as a torch.autograd.Function: output and grads of q, k, v, bias."""
    import block_sparse_dynamic_amd as dma
    import gpu_harness as H

    c = Case("autograd", 23, 1, 192, 192, 4, 2, 64, True, "topk", 80)
    q, k, v, do = synth.q(c), synth.k(c), synth.v(c), synth.do(c)
    m, b = synth.mask_bias(c)
    tq, tk, tv, tb = (H.to_dev(x).requires_grad_(True) for x in (q, k, v, b))
    out = dma.dma_attention(tq, tk, tv, attn_mask=H.to_dev(m), attn_bias=tb, is_causal=True, scale=c.scale_f32)
    out.backward(H.to_dev(do))
    torch.cuda.synchronize()
    o_ref, _ = oracle.forward(q, k, v, m, b, c.scale_f32, True)
    dq, dk, dv, db = oracle.backward(q, k, v, m, b, c.scale_f32, True, do)
    H.check_o(H.f64(out.detach()), o_ref)
    H.check_grad(H.f64(tq.grad), dq, "dQ")
    H.check_grad(H.f64(tk.grad), dk, "dK")
    H.check_grad(H.f64(tv.grad), dv, "dV")
    H.check_grad(H.f64(tb.grad), db, "dBias")


def test_repeatable():
    """Two runs give bit-identical O, LSE, dQ, dK, dV and dBias: every output element has one
    writer and a fixed order of accumulation (dQ is formed from the stored dS tiles by one
    workgroup per query block, without atomics)."""
    import gpu_harness as H

    c = Case("repeat", 24, 1, 512, 512, 8, 2, 128, True, "topk", 200)
    dc = H.DeviceCase(c)
    outs = []
    for _ in range(2):
        dc.classify()
        dc.forward()
        dc.backward()
        torch.cuda.synchronize()
        outs.append([H.bits(t) for t in (dc.o, dc.dq, dc.dk, dc.dv, dc.dbias)] + [dc.lse.cpu().numpy()])
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


def test_skipped_tiles_do_not_leak():
    """K/V rows and bias of SKIP blocks set to NaN change neither the forward nor the backward:
    the forward never loads them, the backward never lets them meet a nonzero weight."""
    import gpu_harness as H

    c = Case("skip_nan", 25, 1, 256, 256, 4, 2, 128, False, "blocks")
    dc = H.DeviceCase(c)
    # carve out one key block per plane that no query attends, each paired (same 128-key
    # workgroup of the backward) with a key block that stays live
    mask2 = dc.mask_h.copy()
    mask2[0, 0, :, 64:128] = 0
    mask2[0, 1, :, 128:192] = 0
    dc.mask_h, dc.mask = mask2, H.to_dev(mask2)
    dc.classify()
    dc.forward()
    dc.backward()
    torch.cuda.synchronize()
    o1 = H.bits(dc.o)
    g1 = [H.bits(t) for t in (dc.dk, dc.dv, dc.dbias)]
    dq1 = H.f64(dc.dq)
    st = dc.state.cpu().numpy()
    bias2 = dc.bias_h.copy()
    for bb in range(c.b):
        for g in range(c.hkv):
            for qb in range(st.shape[2]):
                for kb in range(st.shape[3]):
                    if st[bb, g, qb, kb] == oracle.SKIP:
                        bias2[bb, g, qb * 64:(qb + 1) * 64, kb * 64:(kb + 1) * 64] = 0x7FC0
    # a key block that is SKIP for every query block of a plane: poison its K and V rows
    k2, v2 = dc.k_h.copy(), dc.v_h.copy()
    poisoned = 0
    for kb in range(st.shape[3]):
        for g in range(c.hkv):
            if np.all(st[0, g, :, kb] == oracle.SKIP):
                poisoned += 1
                k2[0, kb * 64:(kb + 1) * 64, g] = 0x7FC0
                v2[0, kb * 64:(kb + 1) * 64, g] = 0x7FC0
    assert poisoned == 2, "the carved key blocks must be SKIP for every query block"
    assert (st[0, 0, :, 0] != oracle.SKIP).any() and (st[0, 1, :, 3] != oracle.SKIP).any()
    dc.bias, dc.k, dc.v = H.to_dev(bias2), H.to_dev(k2), H.to_dev(v2)
    dc.forward()
    dc.backward()
    torch.cuda.synchronize()
    assert np.array_equal(H.bits(dc.o), o1)
    for a, b in zip([H.bits(t) for t in (dc.dk, dc.dv, dc.dbias)], g1):
        assert np.array_equal(a, b)
    assert np.array_equal(H.f64(dc.dq), dq1)


def test_memory_after_inputs_is_never_read():
    """Every input sits at the start of a larger buffer whose remainder is NaN.  Ragged query
    rows and key columns at the end of the tensors are clipped by the kernels' range checks,
    so the outputs are bit-identical to those of plain allocations."""
    import gpu_harness as H

    c = Case("nan_after_inputs", 26, 1, 200, 200, 8, 2, 128, True, "blocks")
    dc = H.DeviceCase(c)
    dc.classify()
    dc.forward()
    dc.backward()
    torch.cuda.synchronize()
    ref = [H.bits(t) for t in (dc.o, dc.dq, dc.dk, dc.dv, dc.dbias)] + [dc.lse.cpu().numpy()]

    def padded(t):
        big = torch.full((t.numel() + 65536,), float("nan"), dtype=t.dtype, device="cuda")
        view = big[: t.numel()].view(t.shape)
        view.copy_(t)
        return view

    dc.q, dc.k, dc.v, dc.do, dc.mask, dc.bias = (padded(t) for t in (dc.q, dc.k, dc.v, dc.do, dc.mask, dc.bias))
    dc.classify()
    dc.forward()
    dc.o, dc.lse = padded(dc.o), padded(dc.lse)
    dc.backward()
    torch.cuda.synchronize()
    got = [H.bits(t) for t in (dc.o, dc.dq, dc.dk, dc.dv, dc.dbias)] + [dc.lse.cpu().numpy()]
    for name, a, b in zip(("o", "dq", "dk", "dv", "dbias", "lse"), ref, got):
        assert np.array_equal(a, b), f"{name} changed"


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits, round to nearest even through fp32 (test input construction only)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _valid(dc):
    c = dc.c
    v = np.ones((c.b, c.hkv, c.lq, c.lk), bool) if dc.mask_h is None else oracle.attends(dc.mask_h)
    if c.causal:
        v &= np.arange(c.lk)[None, :] <= np.arange(c.lq)[:, None] + c.lk - c.lq
    return v


@pytest.mark.parametrize("d", [64, 128])
def test_topk_filled_bias_without_mask(d):
    """The Flash-DMA README recipe's bias (top-k kept, the smallest bf16 elsewhere) passed with
    attn_mask=None: every causal key is valid, the filled ones with a score of about -3.4e38.
    Early causal rows have only filled keys, or one of them."""
    import gpu_harness as H

    c = Case(f"topk_fill_nomask_d{d}", 30 + d // 64, 1, 320, 320, 4, 2, d, True, "topk", 48)

    def prep(dc):
        assert (dc.bias_h == 0xFF7F).any()
        dc.mask_h = None

    dc, _ = H.check_small_case(c, prepare=prep)
    lse = dc.lse.cpu().numpy()
    assert np.all(np.isfinite(lse)), "every causal row has a valid key without a mask"


def test_extreme_bias_values_with_mask():
    """+-largest bf16 at valid positions (single-valued per sign within a row), and rows whose
    every valid key holds the smallest bf16."""
    import gpu_harness as H

    c = Case("extreme_bias", 33, 1, 256, 256, 4, 2, 128, True, "blocks")

    def prep(dc):
        rng = np.random.default_rng(33)
        b = dc.bias_h.copy()
        valid = _valid(dc)
        pick = rng.random(b.shape)
        b[valid & (pick < 0.02)] = 0x7F7F  # +3.39e38
        b[valid & (pick > 0.97)] = 0xFF7F  # -3.39e38
        b[0, 1, 130:150, :] = 0xFF7F  # whole rows at the smallest bf16
        dc.bias_h = b

    H.check_small_case(c, prepare=prep)


def test_large_unclamped_bias():
    """Biases around -3000 (inside the clamp): scores far from zero, every term kept."""
    import gpu_harness as H

    c = Case("large_bias", 34, 1, 256, 256, 4, 2, 128, True, "topk", 64)

    def prep(dc):
        f = oracle.bf16_to_f64(dc.bias_h)
        f = np.where(f > -1e30, f - 3000.0, f)
        dc.bias_h = _bf16_bits(f)

    H.check_small_case(c, prepare=prep)


@pytest.mark.parametrize("v_std", [1e-6, 1e4])
def test_v_magnitudes(v_std):
    """V far below and far above 1: the P V product keeps bf16 V exactly (no fp16 range)."""
    import gpu_harness as H

    c = Case(f"v_std_{v_std:g}", 35, 1, 256, 256, 4, 2, 128, True, "blocks", v_std=v_std)
    H.check_small_case(c)


def test_v_beyond_fp16_range_at_masked_keys():
    """V rows of 7e4 and -1e5 (beyond the fp16 range) at keys whose mask column is zero for every
    row, inside key blocks that stay PARTIAL: those keys meet a zero weight in every product, and
    0 * V must stay 0 (an fp16 copy of V would hold inf there and turn the rows to NaN)."""
    import gpu_harness as H

    c = Case("v_spikes", 36, 1, 256, 256, 4, 2, 128, True, "blocks")

    def prep(dc):
        st = oracle.classify(dc.mask_h, c.b, c.hkv, c.lq, c.lk, c.causal)
        m, v = dc.mask_h.copy(), dc.v_h.copy()
        n = 0
        for kb in range(st.shape[3]):
            # a key block PARTIAL for some query block in both planes (K and V rows are shared by
            # the query heads of a plane only, so both planes' masks lose the column)
            if not all((st[0, g, :, kb] == oracle.PARTIAL).any() for g in range(c.hkv)):
                continue
            for j, val in ((kb * 64 + 5, 7.0e4), (kb * 64 + 40, -1.0e5)):
                m[0, :, :, j] = 0
                v[0, j, :, :] = _bf16_bits(np.full((c.hkv, c.d), val))
                n += 1
        assert n >= 4
        dc.mask_h, dc.v_h = m, v

    dc, _ = H.check_small_case(c, prepare=prep)
    st = dc.state.cpu().numpy()
    assert (st == oracle.PARTIAL).any()


def test_backward_phases_equal_one_call():
    """dma_attn_bwd_part: the three phases in order on one stream are dma_attn_bwd, bit for bit."""
    import block_sparse_dynamic_amd as dma
    import gpu_harness as H

    c = Case("bwd_parts", 37, 2, 200, 200, 8, 2, 128, True, "blocks")
    dc = H.DeviceCase(c)
    dc.classify()
    dc.forward()
    dc.backward()
    ref = [H.bits(t) for t in (dc.dq, dc.dk, dc.dv, dc.dbias)]
    dq, dk, dv = torch.empty_like(dc.q), torch.empty_like(dc.k), torch.empty_like(dc.v)
    dbias = torch.full_like(dc.dbias, float("nan"))
    ws = torch.empty(dma.dma_attn_bwd_workspace_size(c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.causal), dtype=torch.uint8,
                     device="cuda")
    for part in (dma.BWD_PREPARE, dma.BWD_MAIN, dma.BWD_DQ):
        dma.dma_attn_bwd_part(part, dc.q, dc.k, dc.v, dc.mask, dc.bias, dc.state, dc.o, dc.do, dc.lse, c.scale_f32,
                              c.causal, dq, dk, dv, dbias, ws)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dbias"), ref, [H.bits(t) for t in (dq, dk, dv, dbias)]):
        assert np.array_equal(a, b), f"{name} differs"


@pytest.mark.gpu
def test_noncausal_bitmap_serves_causal_attention():
    """A bitmap classified without causality handed to the causal forward and backward: it marks blocks past
    the diagonal non-SKIP and, where the mask is all ones, diagonal blocks FULL.  Both directions apply
    causality inside every block and the backward skips the pairs that causality leaves without a valid
    position, so every output equals the causal bitmap's bit for bit."""
    import block_sparse_dynamic_amd as dma
    import gpu_harness as H

    for c in (Case("nc_bitmap_blocks", 41, 2, 320, 320, 8, 2, 64, True, "blocks"),
              Case("nc_bitmap_ones", 42, 1, 256, 256, 4, 1, 128, True, "ones")):
        ref = H.DeviceCase(c)
        ref.classify()
        ref.forward()
        ref.backward()
        alt = H.DeviceCase(c)
        dma.dma_block_classify(alt.mask, c.b, c.hkv, c.lq, c.lk, False, alt.state)
        torch.cuda.synchronize()
        assert not torch.equal(alt.state, ref.state), "the non-causal bitmap should differ"
        alt.forward()
        alt.backward()
        torch.cuda.synchronize()
        for name in ("o", "lse", "dq", "dk", "dv", "dbias"):
            a, b = getattr(ref, name), getattr(alt, name)
            same = np.array_equal(H.bits(a), H.bits(b)) if a.dtype == torch.bfloat16 else torch.equal(a, b)
            assert same, f"{c.name}: {name} differs with the non-causal bitmap"
