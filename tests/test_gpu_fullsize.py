"""Every shard element of the three largest workloads compared with the
oracle after every step (the -m gpu tests compare about a million sampled
elements per buffer of these workloads, every element of their boundary
tiles, and the exact statistics over all of them).  The oracle's statistics
and update run split over host threads into disjoint arena ranges
(or_grad_stats_range, or_apply_range; both pinned on the CPU to equal the
whole-window calls).  Minutes per workload and about 110 GB of host memory
for the dense 7B list: run on request with -m gpu_fullsize, not part of
-m gpu."""
import pytest
import torch

import synth
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu_fullsize,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs the GPU")]


@pytest.mark.timeout(1100)
@pytest.mark.parametrize("name", ["dense-7b", "llama3-8b", "llama3-70b"])
def test_full_compare_at_full_size(name):
    w = synth.WORKLOADS[name]
    rep = H.run_full_chunked(H.case_from_workload(w))
    assert len(rep) == w.steps
    for r in rep:
        for key in ("master", "m", "v", "param"):
            if key in r:
                assert r[key]["n"] > 0
    if name == "dense-7b":
        assert [r["skipped"] for r in rep] == [0, 0, 1, 0, 0]
        assert rep[-1]["master"]["n"] == 6_738_415_616
