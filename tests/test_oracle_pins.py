"""Pins of the fp64 oracle against things other than itself (CPU only).

* PyTorch's scaled_dot_product_attention on the CPU in fp64 (library routine),
  with and without causality, with GQA, and with an additive float mask that
  carries the bias and the -inf of masked positions; autograd of that float
  mask gives dBias per query head.
* central finite differences of sum(dO * O).
* closed forms (Q = 0: uniform or bias-softmax weights; causal prefix means).
* a naive scalar softmax written with Python loops.
* invariants: empty rows, masked entries holding NaN, zero row sums of dBias.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import bf16_to_f64

pytestmark = pytest.mark.filterwarnings("ignore")


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 to bf16 bits (test-local helper, truncation-free via torch)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _rand_case(rng, b, lq, lk, hq, hkv, d, p_mask=0.6, with_bias=True, with_mask=True, empty_rows=()):
    q = _bf16_bits(rng.standard_normal((b, lq, hq, d)))
    k = _bf16_bits(rng.standard_normal((b, lk, hkv, d)))
    v = _bf16_bits(rng.standard_normal((b, lk, hkv, d)))
    do = _bf16_bits(rng.standard_normal((b, lq, hq, d)))
    mask = None
    if with_mask:
        m = rng.random((b, hkv, lq, lk)) < p_mask
        for r in empty_rows:
            m[:, :, r, :] = False
        mask = np.where(m, np.uint16(0x3F80), np.uint16(0)).astype(np.uint16)
    bias = _bf16_bits(rng.standard_normal((b, hkv, lq, lk))) if with_bias else None
    return q, k, v, do, mask, bias


def _sdpa(q, k, v, mask, bias, scale, causal, do):
    """SDPA in fp64 with attn_mask = bias + (0 | -inf); returns o, dq, dk, dv, dmask(per q head)."""
    b, lq, hq, d = q.shape
    lk, hkv = k.shape[1], k.shape[2]
    G = hq // hkv
    Q = torch.tensor(bf16_to_f64(q)).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    K = torch.tensor(bf16_to_f64(k)).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    V = torch.tensor(bf16_to_f64(v)).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    valid = np.ones((b, hkv, lq, lk), dtype=bool) if mask is None else oracle.attends(mask)
    if causal:
        i = np.arange(lq)[:, None]
        j = np.arange(lk)[None, :]
        valid = valid & (j <= i + lk - lq)
    add = np.where(valid, 0.0, -np.inf)
    if bias is not None:
        add = add + np.where(valid, bf16_to_f64(bias), 0.0)
    add_h = np.repeat(add, G, axis=1)  # query head h uses kv head h // G
    A = torch.tensor(add_h).requires_grad_(True)
    O = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=A, scale=scale, enable_gqa=True)
    dO = torch.tensor(bf16_to_f64(do)).permute(0, 2, 1, 3)
    (O * dO).sum().backward()
    o = O.detach().permute(0, 2, 1, 3).numpy()
    dq = Q.grad.permute(0, 2, 1, 3).numpy()
    dk = K.grad.permute(0, 2, 1, 3).numpy()
    dv = V.grad.permute(0, 2, 1, 3).numpy()
    dmask = A.grad.numpy()
    return o, dq, dk, dv, dmask, valid


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("G", [1, 2, 4])
def test_plain_attention_matches_sdpa(causal, G):
    rng = np.random.default_rng(10 + G + 100 * causal)
    hkv = 2
    q, k, v, do, _, _ = _rand_case(rng, 2, 40, 40, hkv * G, hkv, 16, with_mask=False, with_bias=False)
    scale = 0.3
    o, lse = oracle.forward(q, k, v, None, None, scale, causal)
    dq, dk, dv, db = oracle.backward(q, k, v, None, None, scale, causal, do)
    so, sdq, sdk, sdv, _, _ = _sdpa(q, k, v, None, None, scale, causal, do)
    np.testing.assert_allclose(o, so, rtol=0, atol=1e-10)
    np.testing.assert_allclose(dq, sdq, rtol=0, atol=1e-10)
    np.testing.assert_allclose(dk, sdk, rtol=0, atol=1e-10)
    np.testing.assert_allclose(dv, sdv, rtol=0, atol=1e-10)
    assert db is None
    # lse by definition from torch's logsumexp of the scaled scores
    Q = torch.tensor(bf16_to_f64(q))
    K = torch.tensor(bf16_to_f64(k))
    for h in range(q.shape[2]):
        s = scale * torch.einsum("bid,bjd->bij", Q[:, :, h], K[:, :, h // G])
        if causal:
            s = s.masked_fill(torch.ones(40, 40, dtype=torch.bool).triu(1), -math.inf)
        np.testing.assert_allclose(lse[:, h], torch.logsumexp(s, -1).numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 24, 24, 4, 2, 8), (2, 17, 29, 6, 2, 8), (1, 33, 33, 3, 3, 4)])
def test_mask_bias_matches_sdpa(causal, shape):
    b, lq, lk, hq, hkv, d = shape
    rng = np.random.default_rng(sum(shape) + causal)
    q, k, v, do, mask, bias = _rand_case(rng, b, lq, lk, hq, hkv, d, p_mask=0.5, empty_rows=(3,))
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.forward(q, k, v, mask, bias, scale, causal)
    dq, dk, dv, db = oracle.backward(q, k, v, mask, bias, scale, causal, do)
    so, sdq, sdk, sdv, sdm, valid = _sdpa(q, k, v, mask, bias, scale, causal, do)
    G = hq // hkv
    # rows with a valid key: SDPA is defined there
    live = valid.any(axis=-1)  # [b, hkv, lq]
    for bb in range(b):
        for h in range(hq):
            g = h // G
            r = live[bb, g]
            np.testing.assert_allclose(o[bb, r, h], so[bb, r, h], atol=1e-10)
            np.testing.assert_allclose(dq[bb, r, h], sdq[bb, r, h], atol=1e-10)
            # empty rows: output 0, lse +inf, zero gradient
            assert np.all(o[bb, ~r, h] == 0.0) and np.all(dq[bb, ~r, h] == 0.0)
            assert np.all(np.isinf(lse[bb, h, ~r])) and np.all(lse[bb, h, r] < np.inf)
    # dK/dV: SDPA propagates NaN from empty rows; rebuild its grads without those rows
    keep = np.broadcast_to(live.repeat(G, axis=1).transpose(0, 2, 1)[..., None], do.shape)
    do_live = np.where(keep, do, np.uint16(0)).astype(np.uint16)
    _, _, sdk, sdv, sdm, _ = _sdpa(q, k, v, mask, bias, scale, causal, do_live)
    sdm = np.nan_to_num(sdm, nan=0.0)
    np.testing.assert_allclose(dk, np.nan_to_num(sdk), atol=1e-10)
    np.testing.assert_allclose(dv, np.nan_to_num(sdv), atol=1e-10)
    dq2, dk2, dv2, db2 = oracle.backward(q, k, v, mask, bias, scale, causal, do_live)
    np.testing.assert_allclose(dk2, dk, atol=1e-12)  # empty rows contribute nothing
    # dBias = dS summed over each query-head group; the float mask's grad is dS per query head
    db_sdpa = sdm.reshape(b, hkv, G, lq, lk).sum(axis=2)
    np.testing.assert_allclose(db, db_sdpa, atol=1e-10)
    assert np.all(db[~valid] == 0.0)


def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(7)
    b, L, hkv, G, d = 1, 20, 2, 3, 8
    q, k, v, do, mask, bias = _rand_case(rng, b, L, L, hkv * G, hkv, d)
    scale = 0.25
    o, lse = oracle.forward(q, k, v, mask, bias, scale, True)
    dq, dk, dv, db = oracle.backward(q, k, v, mask, bias, scale, True, do)
    rep = lambda x, ax: np.repeat(x, G, axis=ax)
    o2, lse2 = oracle.forward(q, rep(k, 2), rep(v, 2), rep(mask, 1), rep(bias, 1), scale, True)
    dq2, dk2, dv2, db2 = oracle.backward(q, rep(k, 2), rep(v, 2), rep(mask, 1), rep(bias, 1), scale, True, do)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(b, L, hkv, G, d).sum(3), atol=1e-12)
    np.testing.assert_allclose(dv, dv2.reshape(b, L, hkv, G, d).sum(3), atol=1e-12)
    np.testing.assert_allclose(db, db2.reshape(b, hkv, G, L, L).sum(2), atol=1e-12)


def _loss_fd(q, k, v, mask, bias, scale, causal, do):
    o, _ = oracle.forward_rows(q, k, v, mask, bias, scale, causal, np.arange(q.shape[0]), q.shape[0])
    return float((o * do).sum())


def test_gradients_match_finite_differences():
    rng = np.random.default_rng(3)
    L, hkv, G, d = 12, 1, 2, 4
    hq = hkv * G
    q = rng.standard_normal((L, hq, d))
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    do = rng.standard_normal((L, hq, d))
    bias = rng.standard_normal((hkv, L, L))
    m = rng.random((hkv, L, L)) < 0.7
    m[:, 5, :] = False  # an empty row
    m[:, 8:12, 0:4] = False  # a masked-out block
    mask = np.where(m, np.uint16(0x3F80), np.uint16(0)).astype(np.uint16)
    scale, causal = 0.37, True
    rows = np.arange(L)
    dq, dk, dv, db = oracle.backward_rows(q, k, v, mask, bias, scale, causal, rows, L, do)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("bias", bias, db)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + eps
            fp = _loss_fd(q, k, v, mask, bias, scale, causal, do)
            x[idx] = old - eps
            fm = _loss_fd(q, k, v, mask, bias, scale, causal, do)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        err = np.linalg.norm(num - g) / max(np.linalg.norm(g), 1e-30)
        assert err < 1e-6, (name, err)
    assert np.all(dq[5] == 0.0) and np.all(db[:, 5] == 0.0)
    assert np.all(db[:, 8:12, 0:4] == 0.0)


def test_naive_scalar_loops():
    """Softmax attention written out element by element with math.exp."""
    rng = np.random.default_rng(11)
    L, hq, hkv, d = 5, 2, 1, 3
    q, k, v, do, mask, bias = _rand_case(rng, 1, L, L, hq, hkv, d, p_mask=0.7)
    scale = 0.5
    o, lse = oracle.forward(q, k, v, mask, bias, scale, False)
    Q, K, V, B = bf16_to_f64(q)[0], bf16_to_f64(k)[0], bf16_to_f64(v)[0], bf16_to_f64(bias)[0]
    M = mask[0]
    for h in range(hq):
        for i in range(L):
            scores = {}
            for j in range(L):
                if M[0, i, j] != 0:
                    scores[j] = scale * sum(Q[i, h, c] * K[j, 0, c] for c in range(d)) + B[0, i, j]
            if not scores:
                assert all(o[0, i, h, c] == 0.0 for c in range(d))
                continue
            mx = max(scores.values())
            z = sum(math.exp(s - mx) for s in scores.values())
            for c in range(d):
                ref = sum(math.exp(s - mx) / z * V[j, 0, c] for j, s in scores.items())
                assert abs(o[0, i, h, c] - ref) < 1e-12
            assert abs(lse[0, h, i] - (mx + math.log(z))) < 1e-12


def test_closed_forms():
    rng = np.random.default_rng(5)
    L, d = 70, 8
    q0 = np.zeros((1, L, 1, d), dtype=np.uint16)  # Q = 0: every score is the bias
    _, k, v, do, _, _ = _rand_case(rng, 1, L, L, 1, 1, d, with_mask=False, with_bias=False)
    Vf = bf16_to_f64(v)[0, :, 0]
    # causal, no bias: O_i = mean(V_0..V_i), lse_i = log(i + 1)
    o, lse = oracle.forward(q0, k, v, None, None, 0.125, True)
    prefix = np.cumsum(Vf, axis=0) / np.arange(1, L + 1)[:, None]
    np.testing.assert_allclose(o[0, :, 0], prefix, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, L + 1)), atol=1e-13)
    # two valid keys with biases b1, b2: weights sigmoid(b1 - b2), sigmoid(b2 - b1)
    mask = np.zeros((1, 1, L, L), dtype=np.uint16)
    mask[..., 3] = 0x3F80
    mask[..., 60] = 0x3F80
    bias = _bf16_bits(rng.standard_normal((1, 1, L, L)))
    o, lse = oracle.forward(q0, k, v, mask, bias, 0.125, False)
    B = bf16_to_f64(bias)[0, 0]
    w = 1.0 / (1.0 + np.exp(B[:, 60] - B[:, 3]))
    ref = w[:, None] * Vf[3] + (1 - w)[:, None] * Vf[60]
    np.testing.assert_allclose(o[0, :, 0], ref, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.logaddexp(B[:, 3], B[:, 60]), atol=1e-13)


def test_invariants():
    rng = np.random.default_rng(21)
    b, L, hq, hkv, d = 1, 50, 4, 2, 8
    q, k, v, do, mask, bias = _rand_case(rng, b, L, L, hq, hkv, d, p_mask=0.5, empty_rows=(0, 7))
    scale = 0.35
    o, lse = oracle.forward(q, k, v, mask, bias, scale, True)
    dq, dk, dv, db = oracle.backward(q, k, v, mask, bias, scale, True, do)
    # V = 1: every non-empty row's weights sum to one
    ones = np.full_like(v, 0x3F80)
    o1, _ = oracle.forward(q, k, ones, mask, bias, scale, True)
    live = np.isfinite(lse)  # [b, hq, L]
    for h in range(hq):
        np.testing.assert_allclose(o1[0, live[0, h], h], 1.0, atol=1e-12)
        assert np.all(o1[0, ~live[0, h], h] == 0.0)
    # masked entries may hold anything, even NaN, without changing any output bit
    valid = oracle.attends(mask) & (np.arange(L)[None, :] <= np.arange(L)[:, None])
    bias_nan = np.where(valid, bias, np.uint16(0x7FC0)).astype(np.uint16)
    o2, lse2 = oracle.forward(q, k, v, mask, bias_nan, scale, True)
    r2 = oracle.backward(q, k, v, mask, bias_nan, scale, True, do)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    for a, c in zip((dq, dk, dv, db), r2):
        assert np.array_equal(a, c)
    # rows of dS sum to zero (sum_j P_ij (dP_ij - D_i) = 0), hence rows of dBias too
    np.testing.assert_allclose(db.sum(axis=-1), 0.0, atol=1e-12)
    # an all-ones mask with zero bias is plain attention
    allones = np.full_like(mask, 0x3F80)
    zero = np.zeros_like(bias)
    o3, _ = oracle.forward(q, k, v, allones, zero, scale, True)
    o4, _ = oracle.forward(q, k, v, None, None, scale, True)
    np.testing.assert_allclose(o3, o4, atol=1e-14)
    # mask bits: -0.0 and 0 are masked, any other value attends
    assert list(oracle.attends(np.array([0, 0x8000, 0x3F80, 0x0001, 0xBF80], dtype=np.uint16))) == [
        False, False, True, True, True]


def test_page_example_shapes(synth_lib):
    """The Flash-DMA README usage example: b=1, L=256, Hq=2, Hkv=1, d=64, top-k 128, causal."""
    import synth

    c = synth.CASES["tiny"]
    q, k, v, do = synth.q(c), synth.k(c), synth.v(c), synth.do(c)
    mask, bias = synth.mask_bias(c)
    o, lse = oracle.forward(q, k, v, mask, bias, c.scale_f32, c.causal)
    assert o.shape == (1, 256, 2, 64)
    dq, dk, dv, db = oracle.backward(q, k, v, mask, bias, c.scale_f32, c.causal, do)
    assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape and db.shape == bias.shape
    # each row holds exactly 128 selected keys; causality then keeps those at j <= i
    assert np.all((mask == 0x3F80).sum(-1) == 128)
