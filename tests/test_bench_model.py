"""The benchmark's work model (bench.py ``work_of`` / ``live_blocks``), checked on the CPU against
counts taken element by element from the definitions it states: effective FLOPs are the core
matrix products only (FlashMask README, Performance), 2*d per multiply-add pair of each product
that touches an element of a non-SKIP 64x64 block, per query head: Q K^T and P V forward
(4*d), S recomputed, dP, dV, dK and dQ backward (10*d); mandatory bytes are the bias of every
non-SKIP block, the mask of every PARTIAL one (read once per pass), and the whole dBias plane.
"""
import numpy as np

import bench
import oracle
import synth
from synth import Case


def brute_work(c, state):
    """The same quantities by walking the bitmap block by block."""
    G, d = c.hq // c.hkv, c.d
    f_fwd = f_bwd = 0.0
    b_bias = b_mask = 0.0
    for bb in range(state.shape[0]):
        for g in range(state.shape[1]):
            for qb in range(state.shape[2]):
                for kb in range(state.shape[3]):
                    s = state[bb, g, qb, kb]
                    if s == 0:
                        continue
                    for _h in range(G):  # every query head of the group runs the block's products
                        f_fwd += 2 * (64 * 64 * d) * 2     # Q K^T and P V
                        f_bwd += 2 * (64 * 64 * d) * 5     # S, dP, dV, dK, dQ
                    b_bias += 64 * 64 * 2                   # bf16 bias tile, once per group
                    if s == 1:
                        b_mask += 64 * 64 * 2               # PARTIAL: its mask tile too
    return f_fwd, f_bwd, b_bias, b_mask


def test_work_of_matches_block_walk():
    c = Case("model", 95, 2, 300, 260, 8, 2, 64, True, "blocks")
    mask, bias = synth.mask_bias(c)
    state = oracle.classify(mask, c.b, c.hkv, c.lq, c.lk, c.causal)
    assert (state == 0).any() and (state == 1).any() and (state == 2).any()
    w = bench.work_of(c, state, np, fused=True, has_mask=True)
    f_fwd, f_bwd, b_bias, b_mask = brute_work(c, state)
    assert w["f_fwd"] == f_fwd and w["f_bwd"] == f_bwd
    assert w["f_bwd_main"] + w["f_bwd_dq"] == w["f_bwd"]
    assert w["f_bwd_main"] == f_bwd * 8 / 10  # S, dP, dV, dK: 8*d of the 10*d
    assert w["b_fwd"] == b_bias + b_mask
    assert w["b_bwd"] == b_bias + b_mask + 2.0 * c.b * c.hkv * c.lq * c.lk  # + the dense dBias plane
    assert w["b_cls"] == 0.0  # the classifying forward reads each mask tile once, inside its own pass
    ws = bench.work_of(c, state, np, fused=False, has_mask=True)
    assert ws["b_cls"] == 2.0 * 4096 * bench.live_blocks(c, np)  # a separate pass reads every live tile


def test_live_blocks_closed_forms():
    # lq = lk = n blocks, causal: the lower triangle with the diagonal, n (n + 1) / 2 per plane
    for n in (1, 4, 9):
        c = Case("lb", 96, 2, 64 * n, 64 * n, 4, 2, 64, True, "ones")
        assert bench.live_blocks(c, np) == 2 * 2 * n * (n + 1) // 2
    # not causal: every block
    c = Case("lb_nc", 96, 1, 130, 200, 4, 1, 64, False, "ones")
    assert bench.live_blocks(c, np) == 3 * 4
    # lq < lk causal (bottom-right alignment): row block qb sees key blocks up to (qb*64 + 63 + lk - lq) // 64
    c = Case("lb_tall", 96, 1, 128, 320, 4, 1, 64, True, "ones")
    assert bench.live_blocks(c, np) == sum(min(5, (qb * 64 + 63 + 192) // 64 + 1) for qb in range(2))


def test_headline_effective_flops():
    # every causally live block of the Headline workload is PARTIAL under its top-k mask
    c = synth.CASES["headline"]
    n = c.lq // 64
    live = c.b * c.hkv * n * (n + 1) // 2
    assert live == 263168
    state = np.zeros((c.b, c.hkv, n, n), np.uint8)
    qi, ki = np.tril_indices(n)
    state[:, :, qi, ki] = 1
    w = bench.work_of(c, state, np, fused=True, has_mask=True)
    assert w["f_fwd"] == 4 * 128 * 4096 * 4 * live
    assert abs(w["f_fwd"] - 2.208e12) < 1e9 and abs(w["f_bwd"] - 5.519e12) < 1e9  # the figures quoted elsewhere
