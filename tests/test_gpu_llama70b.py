"""Full Llama-3-70B-shaped preset (80 layers, d 8192, 64/8 heads, ff 28672, bf16 weights of
~141 GB and a 32K-context cache on one GPU): structural properties of the whole solve and the
oracle's WHOLE DP against it (P1-P4 on every cell, P2 on every valid budget's mask).  The
oracle's float32 weights (~274 GB) do not fit in host memory, so each layer is widened when
its items run (helpers.WidenedLayers)."""
import numpy as np
import pytest

from oracle import knapspec_oracle as ko
from tests.test_gpu_fullsize import check_structure, full_parity
from workloads import WORKLOADS

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(1100)
def test_llama3_70b_32k_full():
    from tests.helpers import WidenedLayers
    from workloads.device import DeviceProblem

    wl = WORKLOADS["llama3_70b_32k"]
    print(f"\n[case] {wl.name} full size, whole-DP parity", flush=True)
    prob = DeviceProblem(wl, 0, keep_host=True)
    print("  inputs on device", flush=True)
    res = prob.solve(flags=3)
    s, lat = wl.shape, wl.latency
    t = ko.item_latencies(s.n_layers, prob.ctxs[0], lat.attn_base, lat.attn_per_token, lat.mlp)
    check_structure(res, 0, t, wl.n_budgets, wl.gamma, 2 * s.n_layers, float(np.sum(t)))
    full_parity(WidenedLayers(prob.host_layers), prob, res, 0, wl, prob.ctxs[0],
                prob.host_x0[0])
    prob.close()
