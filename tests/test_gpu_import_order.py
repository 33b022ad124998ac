"""The library works whatever the import order: a process that loads it
before touching torch still shares torch's HIP runtime (the binding imports
torch first), so a call sees the device torch allocated on.  Run in a fresh
process, where nothing has imported torch yet."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, ROOT)
import paged_kv_cache_71_amd as pkv
pkv.load_library()                     # before any import of torch here
import numpy as np, torch
sys.path.insert(0, ROOT + "/tests")
import oracle
from paged_kv_cache_71_amd import workloads as W
b = W.decode_batch(5, [3, 40, 200], 8, 2, 128, 16, "bf16")
k, v, tables = b.compact_pool()
up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
out = torch.empty((b.S, b.Hq, b.D), dtype=torch.float32, device="cuda")
pkv.paged_attention_decode(out, up(b.q), up(k), up(v), torch.from_numpy(tables).cuda(),
                           torch.from_numpy(b.context_lens).cuda(), b.max_context_len, b.scale)
torch.cuda.synchronize()
ref = oracle.decode(b.q, k, v, "bf16", tables, b.context_lens, b.scale)
err = float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - ref)))
assert err <= 2e-3, err
print("ok", err)
""".replace("ROOT", repr(ROOT))


def test_library_loaded_before_torch(gpu_lib):
    print("[import order] fresh process, library loaded before torch", flush=True)
    r = subprocess.run([sys.executable, "-c", SCRIPT], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.strip().startswith("ok")
