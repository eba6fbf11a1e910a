"""The binding works when it is imported before torch: it loads torch's HIP
runtime before the library, so the process holds one runtime (imported the
other way round, the library's launches found no device)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = """
import numpy as np
import paged_kv_cache_421_amd as pk      # before any explicit torch import
import torch
d = pk.CacheDesc(4, 1, 64, "f32")
kc = torch.zeros(d.shape, dtype=torch.float32, device="cuda")
vc = torch.zeros_like(kc)
k = torch.arange(64, dtype=torch.float32, device="cuda").reshape(1, 1, 64)
slots = torch.tensor([21], dtype=torch.int64, device="cuda")
pk.write_kv(d, kc, vc, k, k + 1, slots)
torch.cuda.synchronize()
assert torch.equal(kc[1, 0, 5], k[0, 0]) and torch.equal(vc[1, 0, 5], k[0, 0] + 1)
print("ok", flush=True)
"""


def test_binding_imported_before_torch():
    r = subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, capture_output=True, text=True,
                       timeout=180)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr
