"""The roofline calibration probe runs and reports sane clocks (a measurement helper of the
benchmark, not part of the method)."""
import numpy as np
import pytest

import gpu_common as G

pytestmark = pytest.mark.gpu


def test_mfma_rate_probe_runs():
    import torch
    import rope_mxfp8_qkv_amd as q
    dev = G.torch_dev()
    blocks = 8
    sink = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device=dev)
    clocks = torch.zeros((blocks, 2), dtype=torch.int64, device=dev)
    for rnd in (True, False):
        q.mfma_rate_probe(blocks, 200, rnd, sink, clocks)
        torch.cuda.synchronize()
        c = clocks.cpu().numpy()
        assert (c > 0).all()
        ghz = c[:, 0] / (c[:, 1] / 100e6) / 1e9
        assert ((ghz > 0.3) & (ghz < 4.0)).all(), ghz
        s = sink.cpu().numpy()
        assert np.isfinite(s).all()
        if not rnd:
            assert (s == 0).all()
