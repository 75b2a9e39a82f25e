"""GPU top-k mask construction (dma_topk_mask) against the oracle's topk_mask, bit for bit.

Rows mix heavy ties at the k-th value (values drawn from a few bf16 numbers), the special
values (+-0, +-inf, NaN with several payloads, the smallest bf16, subnormals), k = 1, k = lk - 1,
k >= lk, lengths that are not a multiple of the workgroup width, in-place output, and N(0,1)
rows at the sizes of the pages' workloads (L = 16384, k = 1024; L = 65536, k = 2048).
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


def test_in_place():
    rng = np.random.default_rng(3000)
    check(rows_with_ties(rng, 16, 2048), 300, in_place=True)


@pytest.mark.parametrize("lk,k,n", [(16384, 1024, 64), (65536, 2048, 8)])
def test_workload_rows(lk, k, n):
    rng = np.random.default_rng(4000 + lk)
    check(rows_normal(rng, n, lk), k)
