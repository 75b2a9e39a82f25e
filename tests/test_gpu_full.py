"""GPU parity at the five workloads' full sizes, in the benchmark's launch configuration.

Mid is checked whole (its 64 query blocks are all sampled); Headline, Doc-packed and
Long on 64 seeded 64-row query blocks, with the whole block bitmap bit-exact.  The head
dimension 64 kernels, which no workload uses, run once at a comparable size (b=2, L=8192,
Hq=16, Hkv=2, d=64, causal top-k 512, and a non-causal ragged one), and so do group sizes 16
and 1 (L=4096).
"""
from synth import Case
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    synth.build()


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["mid", "headline", "docpacked", "long"])
def test_full_size_sampled_parity(name):
    import gpu_harness as H

    H.check_full_case(synth.CASES[name], n_blocks=64)
    torch.cuda.empty_cache()


@pytest.mark.timeout(1200)
def test_headline_fused_classify_sampled_parity():
    """The timed step's forward (classification fused in) at the Headline workload, against the oracle."""
    import gpu_harness as H

    H.check_full_case(synth.CASES["headline"], n_blocks=64, path="fused")
    torch.cuda.empty_cache()


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("c", [
    Case("d64_large_topk", 90, 2, 8192, 8192, 16, 2, 64, True, "topk", 512),
    Case("d64_large_blocks_noncausal", 91, 1, 4130, 3000, 8, 4, 64, False, "blocks"),
    Case("g16_scale", 92, 1, 4096, 4096, 32, 2, 128, True, "topk", 256),
    Case("g1_scale", 93, 1, 4096, 4096, 8, 8, 128, True, "topk", 256),
], ids=["d64_topk_causal", "d64_blocks_noncausal_ragged", "g16_topk_causal", "g1_topk_causal"])
def test_other_shapes_at_scale(c):
    import gpu_harness as H

    print(f"case {c}", flush=True)
    H.check_full_case(c, n_blocks=32)
    torch.cuda.empty_cache()
