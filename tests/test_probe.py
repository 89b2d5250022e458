"""The MFMA throughput probe behind the measured-peak figures of bench.py:
it runs through the C ABI; with constant operands every wave produces the
same finite value (all waves compute the same products), with random
operands every wave produces a finite value of its own."""

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


def test_mfma_peak_probe_random_operands_runs():
    """Random operands: every wave writes a finite value (the values differ)."""
    n_wg, iters = 256, 20
    out = torch.full((n_wg * 8,), float("nan"), dtype=torch.float32, device="cuda")
    L.sx_mfma_peak_probe(n_wg, iters, out, random_operands=True)
    torch.cuda.synchronize()
    v = out.cpu().numpy()
    assert np.all(np.isfinite(v)) and len(np.unique(v)) > 1
