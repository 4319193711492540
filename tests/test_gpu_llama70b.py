"""Full Llama-3-70B-shaped preset (80 layers, d 8192, 64/8 heads, ff 28672, bf16 weights of
~141 GB and a 32K-context cache on one GPU): structural properties of the whole solve, the
oracle's DP over the first layer, and the oracle's forward of sampled returned masks."""
import numpy as np
import pytest

from tests.test_gpu_fullsize import check_prefix_and_sample
from workloads import WORKLOADS

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(1100)
def test_llama3_70b_32k_full():
    from workloads.device import DeviceProblem

    wl = WORKLOADS["llama3_70b_32k"]
    print(f"\n[case] {wl.name} full size", flush=True)
    prob = DeviceProblem(wl, 0, keep_host=True)
    print("  inputs on device", flush=True)
    res = prob.solve(flags=3)
    check_prefix_and_sample(prob, res, 0, wl, prefix_layers=1, n_sample=2,
                            rng=np.random.default_rng(0))
    prob.close()
