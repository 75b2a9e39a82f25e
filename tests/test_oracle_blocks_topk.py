"""Pins of the oracle's block classification and top-k mask, and of the generator's recipes (CPU)."""
import numpy as np
import pytest

import oracle
from oracle import BLOCK, FULL, PARTIAL, SKIP


def _brute_classify(mask, lq, lk, causal):
    """Element by element: a block is SKIP with no valid element, FULL when all 64x64 exist and are valid."""
    nqb, nkb = -(-lq // BLOCK), -(-lk // BLOCK)
    out = np.zeros((nqb, nkb), dtype=np.uint8)
    for qb in range(nqb):
        for kb in range(nkb):
            n_valid = 0
            for i in range(qb * BLOCK, min(lq, (qb + 1) * BLOCK)):
                for j in range(kb * BLOCK, min(lk, (kb + 1) * BLOCK)):
                    ok = mask is None or (int(mask[i, j]) & 0x7FFF) != 0
                    if causal and j > i + lk - lq:
                        ok = False
                    n_valid += ok
            out[qb, kb] = SKIP if n_valid == 0 else (FULL if n_valid == BLOCK * BLOCK else PARTIAL)
    return out


@pytest.mark.parametrize("lq,lk,causal", [(130, 200, True), (200, 130, True), (128, 128, False), (65, 64, True)])
def test_classify_brute_force(lq, lk, causal):
    rng = np.random.default_rng(lq * 7 + lk)
    nqb, nkb = -(-lq // BLOCK), -(-lk // BLOCK)
    m = np.zeros((lq, lk), dtype=bool)
    for qb in range(nqb):
        for kb in range(nkb):
            kind = rng.integers(0, 4)
            blk = (slice(qb * BLOCK, (qb + 1) * BLOCK), slice(kb * BLOCK, (kb + 1) * BLOCK))
            if kind == 1:
                m[blk] = True
            elif kind == 2:
                m[blk] = rng.random(m[blk].shape) < 0.5
            elif kind == 3:  # one lone element
                sub = m[blk]
                sub[rng.integers(0, sub.shape[0]), rng.integers(0, sub.shape[1])] = True
    bits = np.where(m, np.uint16(0x3F80), np.uint16(0)).astype(np.uint16)
    bits[m & (rng.random(m.shape) < 0.1)] = 0x0001  # any non-zero value attends
    bits[~m & (rng.random(m.shape) < 0.1)] = 0x8000  # -0.0 is masked
    got = oracle.classify(bits[None, None], 1, 1, lq, lk, causal)[0, 0]
    assert np.array_equal(got, _brute_classify(bits, lq, lk, causal))
    got_none = oracle.classify(None, 1, 1, lq, lk, causal)[0, 0]
    assert np.array_equal(got_none, _brute_classify(None, lq, lk, causal))


def test_classify_causal_closed_form():
    L = 512
    n = L // BLOCK
    got = oracle.classify(None, 1, 1, L, L, True)[0, 0]
    qb, kb = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    ref = np.where(kb > qb, SKIP, np.where(kb == qb, PARTIAL, FULL))
    assert np.array_equal(got, ref)
    ones = np.full((1, 1, L, L), 0x3F80, dtype=np.uint16)
    assert np.array_equal(oracle.classify(ones, 1, 1, L, L, True)[0, 0], ref)
    assert np.all(oracle.classify(ones, 1, 1, L, L, False) == FULL)
    # ragged edges are never FULL
    assert np.all(oracle.classify(None, 1, 1, L + 5, L + 3, False)[0, 0, -1, :] == PARTIAL)
    assert np.all(oracle.classify(None, 1, 1, L + 5, L + 3, False)[0, 0, :, -1] == PARTIAL)


def test_classify_rows_streamed_equals_whole():
    rng = np.random.default_rng(2)
    lq, lk = 300, 260
    bits = np.where(rng.random((lq, lk)) < 0.01, np.uint16(0x3F80), np.uint16(0)).astype(np.uint16)
    whole = oracle.classify(bits[None, None], 1, 1, lq, lk, True)[0, 0]
    parts = [oracle.classify_plane_rows(bits[r:r + 128], r, lq, lk, True) for r in range(0, lq, 128)]
    assert np.array_equal(np.concatenate(parts), whole)


def test_doc_mask_classes_from_intervals(synth_lib):
    """Document mask: classes follow from the document intervals alone."""
    import synth

    c = synth.CASES["docpacked"].with_(lq=2000, lk=2000, doc_min=100, doc_max=700, hkv=1, hq=1, d=8)
    bounds = synth.doc_bounds(c)
    assert bounds[0] == 0 and bounds[-1] == c.lq and np.all(np.diff(bounds) >= 1)
    assert np.all(np.diff(bounds)[:-1] >= c.doc_min) and np.all(np.diff(bounds) <= c.doc_max)
    mask, bias = synth.mask_bias(c)
    got = oracle.classify(mask, 1, 1, c.lq, c.lk, True)[0, 0]
    # from intervals: element (i, j) valid iff doc(i) == doc(j) and j <= i
    doc_of = np.searchsorted(bounds, np.arange(c.lq), side="right") - 1
    nb = -(-c.lq // BLOCK)
    ref = np.zeros((nb, nb), dtype=np.uint8)
    for qb in range(nb):
        for kb in range(nb):
            i0, i1 = qb * BLOCK, min(c.lq, (qb + 1) * BLOCK)
            j0, j1 = kb * BLOCK, min(c.lk, (kb + 1) * BLOCK)
            # valid pairs exist iff some doc intersects both ranges with some j <= i
            anyv = allv = False
            cnt = 0
            for t in range(len(bounds) - 1):
                s, e = bounds[t], bounds[t + 1]
                ii0, ii1 = max(i0, s), min(i1, e)
                jj0, jj1 = max(j0, s), min(j1, e)
                if ii0 >= ii1 or jj0 >= jj1:
                    continue
                for i in range(ii0, ii1):  # j in [jj0, min(jj1, i + 1))
                    cnt += max(0, min(jj1, i + 1) - jj0)
            anyv = cnt > 0
            allv = cnt == BLOCK * BLOCK
            ref[qb, kb] = FULL if allv else (PARTIAL if anyv else SKIP)
    assert np.array_equal(got, ref)
    assert (got == FULL).sum() > 0 and (got == PARTIAL).sum() > 0 and (got == SKIP).sum() > 0
    # bias: N(0, 0.5^2) on valid entries, bf16 minimum elsewhere
    valid = oracle.attends(mask[0, 0])
    assert np.all(bias[0, 0][~valid] == oracle.BF16_LOWEST_BITS)
    vals = oracle.bf16_to_f64(bias[0, 0][valid])
    assert abs(vals.std() - 0.5) < 0.01
    # the mask is inside the causal triangle: causal on or off classifies the same
    assert np.array_equal(oracle.classify(mask, 1, 1, c.lq, c.lk, False)[0, 0], got)
    assert np.all(doc_of[:, None] >= 0)


def _brute_topk(row_bits, k):
    vals = oracle.bf16_to_f64(row_bits)
    order = sorted(range(len(vals)), key=lambda j: (-vals[j], j))[:k]
    return set(order)


@pytest.mark.parametrize("k", [1, 5, 16, 39, 40])
def test_topk_brute_force_with_ties(k, synth_lib):
    import synth

    rng = np.random.default_rng(k)
    n = 40
    pool = np.array([0x3F80, 0x3F80, 0xBF80, 0x0000, 0x8000, 0x4000, 0xFF7F, 0x4040], dtype=np.uint16)
    rows = pool[rng.integers(0, len(pool), size=(30, n))]  # many ties, +0/-0, the bf16 minimum
    m_or, b_or = oracle.topk_mask(rows, k)
    m_gen, b_gen = synth.topk_rows(rows, k)
    assert np.array_equal(m_or, m_gen) and np.array_equal(b_or, b_gen)
    for r in range(rows.shape[0]):
        if n <= k:  # rows no longer than k are left as they are
            assert np.all(m_or[r] == 0x3F80) and np.array_equal(b_or[r], rows[r])
            continue
        chosen = _brute_topk(rows[r], k)
        want = np.zeros(n, dtype=np.uint16)
        for j in chosen:
            want[j] = 0 if rows[r, j] == 0xFF7F else 0x3F80
        assert np.array_equal(m_or[r], want)
        sel = m_or[r] != 0
        assert np.all(b_or[r][~sel] == 0xFF7F) and np.array_equal(b_or[r][sel], rows[r][sel])


def test_topk_rows_short_rows_keep_everything(synth_lib):
    import synth

    rows = np.full((2, 8), 0x4000, dtype=np.uint16)
    m, b = oracle.topk_mask(rows, 8)
    assert np.all(m == 0x3F80) and np.array_equal(b, rows)
    m2, b2 = synth.topk_rows(rows, 8)
    assert np.array_equal(m, m2) and np.array_equal(b, b2)


def test_generator_topk_matches_oracle_topk(synth_lib):
    """The generator's top-k rows equal the oracle's top-k applied to the raw bias rows."""
    import synth

    c = synth.CASES["headline"].with_(lq=96, lk=3000, topk=200)
    raw_case = c.with_(mask="ones", fill="keep")
    _, raw = synth.mask_bias_rows(raw_case, 1, 2, 10, 50)
    m, b = synth.mask_bias_rows(c, 1, 2, 10, 50)
    m_or, b_or = oracle.topk_mask(raw, c.topk)
    assert np.array_equal(m, m_or) and np.array_equal(b, b_or)
    sel = m != 0
    assert np.all(sel.sum(1) == 200)
    v = oracle.bf16_to_f64(raw)
    assert np.all(np.where(sel, v, np.inf).min(1) >= np.where(sel, -np.inf, v).max(1))


def test_generator_values(synth_lib):
    import synth

    x = oracle.bf16_to_f64(synth.normal_bf16(synth.key(0, 9, 1), 0, 200000))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    # row regeneration: any slice equals the same slice of the whole stream
    y = synth.normal_bf16(synth.key(0, 9, 1), 1234, 777)
    assert np.array_equal(y, synth.normal_bf16(synth.key(0, 9, 1), 0, 200000)[1234:2011])
    # bf16 round to nearest even from fp64
    for val, bits in ((1.0, 0x3F80), (1.0 + 2 ** -8, 0x3F80), (1.0 + 3 * 2 ** -8, 0x3F82),
                      (1.0 + 2 ** -8 + 2 ** -30, 0x3F81), (-2.0, 0xC000), (0.0, 0x0000)):
        assert synth.bf16_rne(val) == bits, (val, hex(synth.bf16_rne(val)))
    c = synth.CASES["tiny"]
    qs = synth.rows_of(c, synth.TAG_Q, c.hq, 0, np.array([5, 100]))
    assert np.array_equal(qs, synth.q(c)[0, [5, 100]])
