"""GPU parity at the five workloads' full sizes, in the benchmark's launch configuration.

Mid is checked whole (its 64 query blocks are all sampled); Headline, Doc-packed and
Long on 64 seeded 64-row query blocks, with the whole block bitmap bit-exact.
"""
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
