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


def test_hardware_e4m3_conversion_equals_software_encoder_on_every_fp32():
    """The producers form their E4M3 codes with the hardware's packing conversion after a clamp
    to +-448; on every finite fp32 value (2^32 - 2^24 bit patterns) that path must give the
    same code byte as the software round-to-nearest-even saturating encoder, whose codes the
    bit-exact producer tests compare with the oracle's."""
    import torch
    import rope_mxfp8_qkv_amd as q
    dev = G.torch_dev()
    counts = torch.zeros(3, dtype=torch.int64, device=dev)
    first = torch.zeros(8, dtype=torch.int32, device=dev)
    q.e4m3_convert_check(counts, first)
    torch.cuda.synchronize()
    c = counts.cpu().numpy()
    assert int(c[1]) == 2 ** 32 - 2 ** 24
    bad = first.cpu().numpy().view(np.uint32)[:min(int(c[2]), 8)]
    assert int(c[0]) == 0, (int(c[0]), [hex(int(b)) for b in bad])
