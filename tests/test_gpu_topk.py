"""GPU top-k mask construction (dma_topk_mask) against the oracle's topk_mask, bit for bit.

Rows mix heavy ties at the k-th value (values drawn from a few bf16 numbers), the special
values (+-0, +-inf, NaN with several payloads, the smallest bf16, subnormals), k = 1, k = lk - 1,
k >= lk, lengths that are not a multiple of the workgroup width, every register layout of a row
(1 to 32 chunks per thread), in-place output, rows whose k-th value is each kind of number, and
N(0,1) rows at the sizes of the pages' workloads (L = 16384, k = 1024; L = 65536, k = 2048).
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

SPECIAL = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0xFFFF, 0xFF7F, 0x7F7F, 0x0001, 0x8001,
                    0x3F80, 0xBF80], dtype=np.uint16)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to_f32_bits(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # truncation is exact here


def rows_with_ties(rng, n, lk):
    vals = rng.integers(-6, 7, size=(n, lk)).astype(np.float32) * 0.5  # 13 distinct values, exact in bf16
    return to_f32_bits(vals)


def rows_normal(rng, n, lk):
    x = rng.standard_normal((n, lk)).astype(np.float32)
    u = x.view(np.uint32)
    u = u + 0x7FFF + ((u >> 16) & 1)  # round to nearest even into bf16
    return (u >> 16).astype(np.uint16)


def run_gpu(bits: np.ndarray, k: int, in_place: bool = False):
    import block_sparse_dynamic_amd as dma

    dev = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    mask = torch.empty_like(dev)
    out = dev if in_place else torch.empty_like(dev)
    dma.dma_topk_mask(dev, k, mask, out)
    torch.cuda.synchronize()
    m = mask.view(torch.int16).cpu().numpy().view(np.uint16)
    b = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return m, b


def check(bits, k, in_place=False):
    m, b = run_gpu(bits, k, in_place)
    rm, rb = oracle.topk_mask(bits, k)
    bad = np.argwhere((m != rm) | (b != rb))
    assert bad.size == 0, f"k={k} lk={bits.shape[-1]}: {len(bad)} elements differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("lk,k", [(8, 1), (8, 7), (8, 8), (64, 3), (200, 100), (256, 255), (1000, 17), (4104, 1024),
                                  (4104, 4200)])
def test_ties(lk, k):
    rng = np.random.default_rng(1000 + lk + k)
    check(rows_with_ties(rng, 24, lk), k)


@pytest.mark.parametrize("lk,k", [(16, 5), (128, 40), (520, 260)])
def test_special_values(lk, k):
    rng = np.random.default_rng(2000 + lk)
    bits = rows_with_ties(rng, 32, lk)
    pos = rng.random(bits.shape) < 0.4
    bits[pos] = rng.choice(SPECIAL, size=int(pos.sum()))
    check(bits, k)
    bits[:] = 0x8000 if lk % 2 else 0x0000  # a row of one repeated value
    bits[::2, ::3] = 0x8000
    check(bits, k)


# (k-th value, fill below it, fill above it): rows whose k-th largest value is each kind of number
THRESHOLDS = [
    (0x0000, 0x8001, 0x0001),  # +0, tied with -0; subnormals on both sides
    (0x0001, 0x8000, 0x0002),  # the smallest subnormal
    (0x0080, 0x007F, 0x0081),  # the smallest normal, beside the largest subnormal
    (0x8080, 0x8081, 0x807F),  # the negative of it
    (0x7F80, 0x7F7F, 0x7F80),  # +inf
    (0xFF80, 0x7FC0, 0xFF7F),  # -inf, NaN below it
    (0xFF7F, 0xFF80, 0xFF7E),  # the smallest bf16
    (0x7FC0, 0xFFC1, 0x3F80),  # NaN: fewer numbers than k
    (0xBF80, 0xC000, 0x3F80),  # -1
]


@pytest.mark.parametrize("t,lo,hi", THRESHOLDS, ids=[f"{t:04x}" for t, _, _ in THRESHOLDS])
@pytest.mark.parametrize("lk,k", [(1000, 301), (4104, 1003), (16384, 5003)])
def test_threshold_values(t, lo, hi, lk, k):
    """The k-th value is t and several keys hold it (the kept ties cut inside a 16-byte chunk, and
    at 16384 keys in a later row of 256 chunks), with values below and above it scattered."""
    rng = np.random.default_rng(5000 + lk + t)
    n = 8
    bits = np.empty((n, lk), np.uint16)
    for i in range(n):
        n_hi = k - 1 - i * 37 % 200  # keys above t
        n_eq = 1 + (i * 997 + 3 * k) % (lk - n_hi - 1)  # keys equal to t, at least k - n_hi
        n_eq = max(n_eq, k - n_hi)
        row = np.full(lk, lo, np.uint16)
        row[:n_hi] = hi
        row[n_hi:n_hi + n_eq] = t
        if t == 0x0000:
            row[n_hi:n_hi + n_eq:2] = 0x8000  # -0 and +0 tie
        bits[i] = rng.permutation(row)
    check(bits, k)


@pytest.mark.parametrize("lk,k", [(24584, 20001), (40000, 7), (65528, 65000)])
def test_long_rows_with_ties(lk, k):
    """Rows of 16 and 32 chunks per thread with a partial last row of chunks: heavy ties and special
    values, the kept ties cut early in the row (k = 7) and in its last chunk row."""
    rng = np.random.default_rng(6000 + lk)
    bits = rows_with_ties(rng, 4, lk)
    pos = rng.random(bits.shape) < 0.05
    bits[pos] = rng.choice(SPECIAL, size=int(pos.sum()))
    check(bits, k)


def test_in_place():
    rng = np.random.default_rng(3000)
    check(rows_with_ties(rng, 16, 2048), 300, in_place=True)


@pytest.mark.parametrize("lk,k,n", [(16384, 1024, 64), (65536, 2048, 8)])
def test_workload_rows(lk, k, n):
    rng = np.random.default_rng(4000 + lk)
    check(rows_normal(rng, n, lk), k)
