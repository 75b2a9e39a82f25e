"""The backward main kernel's workgroup order (pair_order_kernel), read back from the workspace after
a one-pass dma_attn_bwd and compared bit for bit with its emulation here.

Per workgroup task (plane, 128-key pair, segment of a split walk) the work count is the number of
query blocks its walk visits: those where one of the pair's two key blocks is not SKIP and
causality leaves the pair live.  Where some plane's work rises from one pair to the next (a
document mask) the tasks are sorted by count, most first, then by task index, and dealt to the
XCDs in serpentine order (ranks 8k..8k+7 to workgroups 8k..8k+7 for even k and 8k+7..8k for odd
k, a last partial group in order); otherwise workgroup w runs xcd_task(w).  The order must be a
permutation of the tasks.  Cases: a document mask (irregular), a causal uniform mask (regular),
a split-pair causal case (two segments per pair) and a non-causal block mask.
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


def live_pairs(qb, lq, lk, causal):
    nkb2 = ((lk + 63) // 64 + 1) // 2
    if not causal:
        return nkb2
    last = qb * 64 + 63 + lk - lq
    return 0 if last < 0 else min(nkb2, last // 128 + 1)


def xcd_task(w, total, units):
    if total % 8 == 0 and units % 8 == 0:
        return (w % 8) * (total // 8) + w // 8
    if units not in (1, 2, 4) or total % 16:
        return w
    per, xpu = total // units, 8 // units
    nseg = 2 * xpu
    seg = per // nseg
    x, k = w % 8, w // 8
    unit, j = x // xpu, x % xpu
    return unit * per + (j * seg + k if k < seg else (nseg - 1 - j) * seg + (k - seg))


def expected(state, c):
    planes, nqb, nkb = c.b * c.hkv, state.shape[2], state.shape[3]
    nkb2 = (nkb + 1) // 2
    splits = 2 if c.causal and planes * nkb2 <= 256 and nqb >= 8 else 1
    counts = np.zeros(planes * nkb2 * splits, np.int64)
    for KB in range(nkb2):
        first = next((qb for qb in range(nqb) if KB < live_pairs(qb, c.lq, c.lk, c.causal)), nqb)
        upper = first + (nqb - first) // 2
        for plane in range(planes):
            bb, g = divmod(plane, c.hkv)
            for qb in range(nqb):
                if KB >= live_pairs(qb, c.lq, c.lk, c.causal):
                    continue
                s1 = state[bb, g, qb, 2 * KB + 1] if 2 * KB + 1 < nkb else 0
                if state[bb, g, qb, 2 * KB] == 0 and s1 == 0:
                    continue
                seg = 0 if splits == 1 or qb >= upper else 1
                counts[(plane * nkb2 + KB) * splits + seg] += 1
    T = len(counts)
    tot = counts.reshape(planes, nkb2, splits).sum(axis=2)
    irregular = bool((tot[:, 1:] > tot[:, :-1]).any())
    if not irregular or T > 16384:
        return counts, np.array([xcd_task(w, T, planes) for w in range(T)]), irregular
    ranked = sorted(range(T), key=lambda t: (-counts[t], t))
    order = np.zeros(T, np.int64)
    for r, t in enumerate(ranked):
        k, j = divmod(r, 8)
        x = 7 - j if (k % 2 == 1 and 8 * k + 8 <= T) else j
        order[8 * k + x] = t
    return counts, order, irregular


CASES = [
    Case("order_doc", 80, 1, 2000, 2000, 4, 2, 64, True, "doc", doc_min=64, doc_max=700, bias_std=0.5),
    Case("order_causal_topk", 81, 2, 1024, 1024, 4, 4, 64, True, "topk", 96),
    Case("order_split_pairs", 82, 1, 696, 696, 2, 1, 64, True, "blocks"),
    Case("order_noncausal_blocks", 83, 1, 640, 512, 2, 2, 64, False, "blocks"),
]


@pytest.mark.parametrize("c", CASES, ids=[c.name for c in CASES])
def test_workgroup_order(c):
    import block_sparse_dynamic_amd as dma
    import gpu_harness as H

    print(f"case {c}", flush=True)
    dc = H.DeviceCase(c)
    dc.classify()
    dc.forward()
    nbytes = dma.dma_attn_bwd_workspace_size(c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.causal)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(dc.q), torch.empty_like(dc.k), torch.empty_like(dc.v)
    dma.dma_attn_bwd(dc.q, dc.k, dc.v, dc.mask, dc.bias, dc.state, dc.o, dc.do, dc.lse, c.scale_f32, c.causal, dq, dk,
                     dv, None, ws)
    torch.cuda.synchronize()
    state = dc.state.cpu().numpy()
    assert np.array_equal(state, oracle.classify(dc.mask_h, c.b, c.hkv, c.lq, c.lk, c.causal))
    counts, order, irregular = expected(state, c)
    T = len(order)
    region = (2 * T * 4 + 255) // 256 * 256  # the workspace's last region: order, then counts
    got = ws[nbytes - region:].cpu().numpy().view(np.int32)
    print(c.name, "tasks", T, "irregular", irregular, flush=True)
    assert np.array_equal(got[T:2 * T], counts), "work counts differ"
    assert np.array_equal(np.sort(got[:T]), np.arange(T)), "the order is not a permutation of the tasks"
    assert np.array_equal(got[:T], order), "workgroup order differs"
    if c.mask in ("doc", "topk"):  # a document mask is irregular, a causal top-k one falls with the pair
        assert irregular == (c.mask == "doc"), "unexpected regularity of the case"
    H.compare_with_oracle(c.name, c, dc.q_h, dc.k_h, dc.v_h, dc.mask_h, dc.bias_h, dc.do_h, dc.o, dc.lse, dq, dk, dv,
                          None)
