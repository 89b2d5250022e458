"""The MFMA throughput probe behind the measured-peak figure of bench.py:
it runs through the C ABI, every wave produces the same finite value (all
waves compute the same products), and a launch is timed."""

import numpy as np
import pytest
import torch

from segment_level_kv_amd import _lib as L
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def test_mfma_peak_probe_runs_and_is_uniform():
    n_wg, iters = 512, 20
    say(f"[mfma probe] workgroups={n_wg} iters={iters}")
    out = torch.full((n_wg * 8,), float("nan"), dtype=torch.float32, device="cuda")
    L.sx_mfma_peak_probe(n_wg, iters, out)
    torch.cuda.synchronize()
    v = out.cpu().numpy()
    assert np.all(np.isfinite(v))
    assert np.all(v == v[0])
