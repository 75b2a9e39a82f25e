"""The backward's walk over (query block, key pair) items, emulated on the CPU.

The backward main kernel gives each workgroup one 128-key pair KB of one (batch, kv head)
plane and walks the query blocks from the last to the first, visiting those whose two key
blocks are not both SKIP; every visit stores the item's dS chunks into the slot
((plane * npairs + pair_base[qb] + KB) * G + head) * 2 + half of the workspace.  The dQ kernel
reads, for each query block, the slots of its live pairs that are not SKIP in both halves.

This emulation follows the kernel's control: query blocks from nqb - 1 down to 0 (or, where the
backward splits each key pair over two workgroups, the two halves of the pair's live query
blocks, each walked downwards by its own workgroup with its own cache), the block
states cached a chunk of 1024 query blocks at a time, a pair that causality leaves no valid
position for the query block (KB >= live_pairs(qb)) taken as SKIP whatever the bitmap says,
heads in steps of two (one when the group size is odd), rows in two 32-row halves (one past
lq).  Checked on random bitmaps, including bitmaps classified without causality handed to a
causal backward: every slot written lies inside the plane's slot range, no slot is written
twice, and the dQ kernel reads exactly the slots the main kernel wrote.  The live pair count is
pinned to the library's own through dma_attn_bwd_workspace_size.

With a workspace smaller than the one-pass size the backward runs in bands of consecutive query
blocks: a band ends where the next block's live pairs would overflow the slots that fit, each band
numbers its slots from its first pair, and the main kernel's grid covers the pairs live at the
band's last block.  The same checks hold per band, every (query block, pair) item is walked in
exactly one band, and the smallest workspace is pinned through dma_attn_bwd_workspace_size_min.
"""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_sparse_dynamic_amd", "libdma.so")
STATE_CHUNK = 1024
SKIP = 0


def live_pairs(qb, lq, lk, causal):
    nkb2 = ((lk + 63) // 64 + 1) // 2
    if not causal:
        return nkb2
    last = qb * 64 + 63 + lk - lq
    return 0 if last < 0 else min(nkb2, last // 128 + 1)


def bwd_splits(b, hkv, lq, lk, causal):
    """Workgroups per 128-key pair: two (each walking half of the pair's live query blocks) when the
    backward is causal, the pairs over all planes are at most 256 and there are at least 8 query blocks."""
    nqb, nkb2 = (lq + 63) // 64, ((lk + 63) // 64 + 1) // 2
    return 2 if causal and b * hkv * nkb2 <= 256 and nqb >= 8 else 1


def ws_size(b, lq, lk, hq, hkv, d, causal):
    up = lambda x: (x + 255) // 256 * 256
    nqb, nkb2 = (lq + 63) // 64, ((lk + 63) // 64 + 1) // 2
    npairs = sum(live_pairs(qb, lq, lk, causal) for qb in range(nqb))
    splits = bwd_splits(b, hkv, lq, lk, causal)
    dkv = up(2 * b * lk * hkv * d * 4) if splits > 1 else 0
    order = up(2 * b * hkv * nkb2 * splits * 4)  # the main kernel's workgroup order and work counts
    return up(2 * b * hq * lq * 4) + up((nqb + 1) * 8) + up(b * hkv * d * nkb2 * 128 * 2) + \
        up(b * hq * npairs * 64 * 128 * 2) + up(b * hq * npairs * 2 * 8 * 8) + dkv + order


def segments(KB, nqb, lq, lk, causal, splits, band=None):
    """Query-block ranges [lo, hi] of the workgroups of key pair KB, inside the launch's band."""
    band_lo, band_hi = band if band is not None else (0, nqb - 1)
    if splits == 1:
        return [(band_lo, band_hi)]
    lo = next(qb for qb in range(nqb + 1) if qb == nqb or KB < live_pairs(qb, lq, lk, causal))
    lo = max(lo, band_lo)
    upper = lo + (band_hi + 1 - lo) // 2
    return [(upper, band_hi), (lo, upper - 1)]


def bands(nqb, lq, lk, causal, max_pairs):
    """[lo, hi] of the bands of query blocks: a band ends where the next block's live pairs would
    pass max_pairs (each band holds at least one block); one band without a limit."""
    if max_pairs is None:
        return [(0, nqb - 1)]
    out, lo = [], 0
    while lo < nqb:
        hi, n = lo, 0
        while hi < nqb:
            lp = live_pairs(hi, lq, lk, causal)
            if hi > lo and n + lp > max_pairs:
                break
            n += lp
            hi += 1
        out.append((lo, hi - 1))
        lo = hi
    return out


def main_kernel_slots(state, b, hkv, G, lq, lk, causal, band=None, items=None):
    """Slots the backward main kernel stores, in its walk order, for the query blocks of `band`
    ([lo, hi], all of them by default); `items` collects the (plane, qb, KB) items walked."""
    nqb, nkb = state.shape[2], state.shape[3]
    lo_b, hi_b = band if band is not None else (0, nqb - 1)
    pair_base = np.concatenate([[0], np.cumsum([live_pairs(qb, lq, lk, causal) for qb in range(nqb)])])
    pb_lo = int(pair_base[lo_b])
    npairs = int(pair_base[hi_b + 1]) - pb_lo
    wg_pairs = live_pairs(hi_b, lq, lk, causal)  # the grid's pairs
    if band is None:
        splits = bwd_splits(b, hkv, lq, lk, causal)
    else:  # the first band may split its pairs (its fp32 sums start at zero), later bands do not
        splits = 2 if lo_b == 0 and causal and b * hkv * wg_pairs <= 256 and hi_b + 1 >= 8 else 1
    hpi = 2 if G % 2 == 0 else 1
    slots = []
    for plane in range(b * hkv):
        bb, g = divmod(plane, hkv)
        for KB in range(wg_pairs):
            kb0 = 2 * KB
            has_kb1 = kb0 + 1 < nkb
            cache_lo = nqb
            cache = None

            def fill(qb_hi):
                lo = max(0, qb_hi - STATE_CHUNK + 1)
                st = np.full((2, STATE_CHUNK), SKIP, np.uint8)
                for j in range(STATE_CHUNK):
                    qb = lo + j
                    for hf in range(2):
                        if qb <= qb_hi and (hf == 0 or has_kb1) and KB < live_pairs(qb, lq, lk, causal):
                            st[hf, j] = state[bb, g, qb, kb0 + hf]
                return lo, st

            for q_lo, q_hi in segments(KB, nqb, lq, lk, causal, splits, (lo_b, hi_b)):
                cache_lo = nqb  # each workgroup starts with an empty cache
                qb = q_hi
                while qb >= q_lo:
                    if qb < cache_lo:
                        cache_lo, cache = fill(qb)
                    s0, s1 = cache[0, qb - cache_lo], cache[1, qb - cache_lo]
                    if s0 != SKIP or s1 != SKIP:
                        if items is not None:
                            items.append((plane, qb, KB))
                        halves = 1 if qb * 64 + 32 >= lq else 2
                        for rh in range(halves):
                            for hh in range(0, G, hpi):
                                slot_a = ((plane * npairs + int(pair_base[qb]) - pb_lo + KB) * G + hh) * 2 + rh
                                for h2 in range(hpi):
                                    slots.append((plane, slot_a + 2 * h2))
                    qb -= 1
    return slots, npairs


def dq_kernel_slots(state, b, hkv, G, lq, lk, causal, npairs, band=None):
    nqb, nkb = state.shape[2], state.shape[3]
    lo_b, hi_b = band if band is not None else (0, nqb - 1)
    pair_base = np.concatenate([[0], np.cumsum([live_pairs(qb, lq, lk, causal) for qb in range(nqb)])])
    pb_lo = int(pair_base[lo_b])
    reads = []
    for plane in range(b * hkv):
        bb, g = divmod(plane, hkv)
        for qb in range(lo_b, hi_b + 1):
            for hh in range(G):
                for rh in range(2):
                    if rh == 1 and qb * 64 + 32 >= lq:
                        continue  # rows past lq: nothing written, nothing needed
                    slot0 = ((plane * npairs + int(pair_base[qb]) - pb_lo) * G + hh) * 2 + rh
                    for kb2 in range(live_pairs(qb, lq, lk, causal)):
                        s0 = state[bb, g, qb, 2 * kb2]
                        s1 = state[bb, g, qb, 2 * kb2 + 1] if 2 * kb2 + 1 < nkb else SKIP
                        if s0 != SKIP or s1 != SKIP:
                            reads.append((plane, slot0 + kb2 * G * 2))
    return reads


CASES = [(1, 200, 200, 4, 2, 1), (2, 1000, 1000, 4, 1, 1), (1, 600, 600, 4, 2, 1), (2, 520, 540, 1, 2, 1),
         (1, 130, 264, 8, 2, 1), (1, 200, 136, 2, 1, 1), (1, 264, 264, 16, 4, 0), (1, 300, 300, 3, 1, 1),
         (1, 70000, 70000, 1, 1, 1)]


@pytest.mark.parametrize("b,lq,lk,G,hkv,causal", CASES)
@pytest.mark.parametrize("noncausal_bitmap", [False, True])
def test_walk_stays_inside_the_slots(b, lq, lk, G, hkv, causal, noncausal_bitmap):
    rng = np.random.default_rng(lq * 7 + lk + G)
    nqb, nkb = (lq + 63) // 64, (lk + 63) // 64
    if lq * lk > 1e9:  # the long case: a sparse random bitmap over a 1094 x 1094 block grid
        state = (rng.random((b, hkv, nqb, nkb)) < 0.01).astype(np.uint8)
    else:
        state = rng.integers(0, 3, size=(b, hkv, nqb, nkb)).astype(np.uint8)
    if causal and not noncausal_bitmap:  # a causal classification never marks dead blocks
        qb = np.arange(nqb)[:, None]
        kb = np.arange(nkb)[None, :]
        dead = kb * 64 > np.minimum(qb * 64 + 63, lq - 1) + (lk - lq)
        state[:, :, dead] = SKIP
    slots, npairs = main_kernel_slots(state, b, hkv, G, lq, lk, causal)
    per_plane = npairs * G * 2
    assert all(plane * per_plane <= s < (plane + 1) * per_plane for plane, s in slots), "slot outside its plane"
    written = [s for _, s in slots]
    assert len(written) == len(set(written)), "a slot written twice"
    reads = dq_kernel_slots(state, b, hkv, G, lq, lk, causal, npairs)
    assert set(reads) <= set(slots), "the dQ kernel reads a slot nobody wrote"
    assert set(slots) <= set(reads) | set(), "a written slot is never read"


@pytest.mark.parametrize("b,lq,lk,G,hkv,causal", CASES[:-1])
def test_live_pairs_match_the_library(b, lq, lk, G, hkv, causal):
    if not os.path.exists(LIB):
        pytest.skip("library not built")
    L = ctypes.CDLL(LIB)
    L.dma_attn_bwd_workspace_size.restype = ctypes.c_size_t
    L.dma_attn_bwd_workspace_size.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int]
    for d in (64, 128):
        assert L.dma_attn_bwd_workspace_size(b, lq, lk, G * hkv, hkv, d, causal) == ws_size(b, lq, lk, G * hkv, hkv, d,
                                                                                            causal)


def ws_min_size(b, lq, lk, hq, hkv, d, causal):
    """The dS slots of the largest single query block (the last), plus the fp32 dK/dV sums."""
    up = lambda x: (x + 255) // 256 * 256
    nqb, nkb2 = (lq + 63) // 64, ((lk + 63) // 64 + 1) // 2
    np_ = live_pairs(nqb - 1, lq, lk, causal)
    return up(2 * b * hq * lq * 4) + up((nqb + 1) * 8) + up(b * hkv * d * nkb2 * 128 * 2) + \
        up(b * hq * np_ * 64 * 128 * 2) + up(b * hq * np_ * 2 * 8 * 8) + up(2 * b * lk * hkv * d * 4)


@pytest.mark.parametrize("b,lq,lk,G,hkv,causal", CASES[:-1])
@pytest.mark.parametrize("which", ["min", "third"])
def test_banded_walk_covers_every_item_once(b, lq, lk, G, hkv, causal, which):
    rng = np.random.default_rng(lq * 5 + lk + G + (which == "min"))
    nqb, nkb = (lq + 63) // 64, (lk + 63) // 64
    state = rng.integers(0, 3, size=(b, hkv, nqb, nkb)).astype(np.uint8)
    total = sum(live_pairs(qb, lq, lk, causal) for qb in range(nqb))
    smallest = live_pairs(nqb - 1, lq, lk, causal)
    max_pairs = smallest if which == "min" else max(smallest, total // 3)
    parts = bands(nqb, lq, lk, causal, max_pairs)
    assert parts[0][0] == 0 and parts[-1][1] == nqb - 1
    assert all(parts[i][1] + 1 == parts[i + 1][0] for i in range(len(parts) - 1)), "bands not consecutive"
    all_items = []
    for band in parts:
        lo, hi = band
        npairs = sum(live_pairs(qb, lq, lk, causal) for qb in range(lo, hi + 1))
        assert npairs <= max_pairs or lo == hi, "a band of several blocks overflows the slots"
        items = []
        slots, np_ = main_kernel_slots(state, b, hkv, G, lq, lk, causal, band=band, items=items)
        assert np_ == npairs
        per_plane = npairs * G * 2
        assert all(plane * per_plane <= s < (plane + 1) * per_plane for plane, s in slots), "slot outside the band"
        written = [s for _, s in slots]
        assert len(written) == len(set(written)), "a slot written twice"
        reads = dq_kernel_slots(state, b, hkv, G, lq, lk, causal, npairs, band=band)
        assert set(reads) == set(slots), "the dQ kernel's reads differ from the main kernel's writes"
        assert all(lo <= qb <= hi for _, qb, _ in items)
        all_items += items
    one_pass = []
    main_kernel_slots(state, b, hkv, G, lq, lk, causal, items=one_pass)
    assert len(all_items) == len(set(all_items)), "an item walked in two bands"
    assert set(all_items) == set(one_pass), "the bands walk other items than the one pass"


@pytest.mark.parametrize("b,lq,lk,G,hkv,causal", CASES[:-1])
def test_min_workspace_matches_the_library(b, lq, lk, G, hkv, causal):
    if not os.path.exists(LIB):
        pytest.skip("library not built")
    L = ctypes.CDLL(LIB)
    f = L.dma_attn_bwd_workspace_size_min
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int]
    for d in (64, 128):
        want = ws_min_size(b, lq, lk, G * hkv, hkv, d, causal)
        assert f(b, lq, lk, G * hkv, hkv, d, causal) == want
        assert want <= ws_size(b, lq, lk, G * hkv, hkv, d, causal) + 2 * b * lk * hkv * d * 4 + 256
    assert f(0, lq, lk, G * hkv, hkv, 64, causal) == 0
