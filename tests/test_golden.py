"""Pins from the one worked example the pages print: the Flash-DMA README usage example
(tests/golden/flash_dma_usage_example.json holds its configuration and the output shape it
prints).  The pages print no output values, so these tests pin what the example does fix: the
shape and layout of the output ([batch, seq, query heads, head dim]) and of every gradient, the
keep_window_size keys of each mask row (no N(0,1) bias value equals the bf16 minimum, so every
top-k pick stays valid), and the bias of the other keys overwritten with the bf16 minimum.  The
inputs are the seeded Tiny workload of the same shapes; the outputs come from the oracle.
"""
import json
import math
import os

import numpy as np

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
BF16_MIN = 0xFF7F


def load():
    with open(os.path.join(HERE, "golden", "flash_dma_usage_example.json")) as f:
        return json.load(f)


def tiny_inputs():
    g = load()["config"]
    c = synth.CASES["tiny"]
    assert (c.b, c.lq, c.lk, c.hq, c.hkv, c.d, c.topk, c.causal) == (
        g["batch_size"], g["seq_len"], g["seq_len"], g["num_heads"], g["num_kv_heads"], g["head_dim"],
        g["keep_window_size"], g["is_causal"])
    assert c.scale == 1.0 / math.sqrt(g["head_dim"])
    mask, bias = synth.mask_bias(c)
    return c, synth.q(c), synth.k(c), synth.v(c), mask, bias


def test_output_shape_is_the_printed_one():
    c, q, k, v, mask, bias = tiny_inputs()
    o, lse = oracle.forward(q, k, v, mask, bias, c.scale, c.causal)
    assert list(o.shape) == load()["printed"]["output_shape"]
    assert lse.shape == (c.b, c.hq, c.lq)
    # a row whose keep_window_size picks all lie in its future has no valid key: O = 0, LSE = +inf
    i = np.arange(c.lq)[:, None]
    j = np.arange(c.lk)[None, :]
    has_key = (oracle.attends(mask[0, 0]) & (j <= i)).any(axis=1)
    assert not has_key.all() and has_key.sum() > 200  # both kinds of row occur in this example
    assert np.all(np.isfinite(lse[0][:, has_key])) and np.all(np.isposinf(lse[0][:, ~has_key]))
    assert np.all(o[0][~has_key] == 0.0) and np.all(np.isfinite(o))


def test_gradients_have_the_inputs_shapes():
    # loss = output.sum(): dO = 1
    c, q, k, v, mask, bias = tiny_inputs()
    o, _ = oracle.forward(q, k, v, mask, bias, c.scale, c.causal)
    do = np.ones(o.shape)
    dq, dk, dv, dbias = oracle.backward(q, k, v, mask, bias, c.scale, c.causal, do)
    assert dq.shape == (1, 256, 2, 64) == q.shape
    assert dk.shape == dv.shape == (1, 256, 1, 64) == k.shape
    assert dbias.shape == (1, 1, 256, 256) == bias.shape


def test_topk_recipe_keeps_keep_window_size_keys_per_row():
    g = load()["config"]
    c, _, _, _, mask, bias = tiny_inputs()
    ones = oracle.attends(mask).sum(axis=-1)
    assert np.all(ones == g["keep_window_size"])
    assert np.all(bias[~oracle.attends(mask)] == BF16_MIN)
    assert not np.any(bias[oracle.attends(mask)] == BF16_MIN)
    # the oracle's own top-k of the kept values reproduces the mask: the kept keys are the row's
    # keep_window_size largest
    m2, b2 = oracle.topk_mask(bias.reshape(-1, c.lk), g["keep_window_size"])
    assert np.array_equal(oracle.attends(m2.reshape(mask.shape)), oracle.attends(mask))
    assert np.array_equal(b2.reshape(bias.shape), bias)
