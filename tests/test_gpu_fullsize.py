"""Every shard element of a full-size workload compared with the oracle after
every step (the -m gpu tests compare about a million sampled elements per
buffer of the full-size workloads, plus the exact statistics over all of
them).  Minutes per workload: run on request with -m gpu_fullsize."""
import pytest
import torch

import synth
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu_fullsize,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs the GPU")]


@pytest.mark.timeout(1800)
@pytest.mark.parametrize("name", ["llama3-8b", "llama3-70b"])
def test_full_compare_at_full_size(name):
    rep = H.run_full(H.case_from_workload(synth.WORKLOADS[name]))
    assert len(rep) == synth.WORKLOADS[name].steps
