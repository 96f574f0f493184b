"""The library may be loaded before torch: the binding brings torch in first, so a process
that touches the package (a size query) and only then allocates device tensors through torch
still runs kernels.  Runs in a fresh interpreter, where nothing has imported torch yet."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
import rope_mxfp8_qkv_amd as q
assert q.qkv_act_image_bytes(300, 512) > 0          # library loaded here
import torch
x = torch.randn(300, 512, device="cuda:0")
packed = torch.empty((300, 516), dtype=torch.uint8, device="cuda:0")
q.row_quantize_packed(x, packed)
torch.cuda.synchronize()
assert int(packed[:, :512].count_nonzero()) > 0
print("import-order ok", flush=True)
"""


def test_library_loaded_before_torch():
    env = dict(os.environ)
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "import-order ok" in r.stdout
