"""GPU parity of the MFMA-free GEMV (w4_gemv_valu.hip), the A/B alternative
the W4A16_VALU=1 override selects for up to 8 rows.  The override is read once
per process, so the cases run in one child interpreter started with it set;
the child prints one JSON line per case, which is checked here against the
oracle's bar.  Kept so that the measured comparison with the MFMA kernel is
between two correct kernels."""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r"""
import json, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import numpy as np, torch
import bit_weight_only_03_amd as L, oracle, synth
from gpu_util import PackedW4, dev, to_f64
for (M, N, K, g, xdt) in {cases!r}:
    w = synth.gen_w4((150, M, N, K, g), N, K, g)
    x = synth.gen_x((150, M, K), M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    P = PackedW4(w, N, K, g)
    y1 = P.gemv(dev(x), xdt, M)
    variant = L.w4a16_last_variant()
    y2 = P.gemv(dev(x), xdt, M)
    torch.cuda.synchronize()
    cols = np.sort(np.random.default_rng(M + N).choice(N, size=min(N, 128), replace=False)).astype(np.int64)
    ref = oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, K, g, cols=cols)
    got = to_f64(y1)[:, cols]
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    print(json.dumps({{"case": [M, N, K, g, xdt], "variant": variant, "rel": rel, "max": mx,
                      "repeat_equal": bool(torch.equal(y1, y2))}}), flush=True)
"""

CASES = [(1, 264, 1024, 128, "f16"), (8, 264, 2048, 64, "f16"), (4, 520, 17408, 128, "bf16"),
         (1, 7168, 5120, 128, "f16"), (8, 5120, 17408, 128, "f16"), (3, 136, 640, 64, "bf16")]


def test_valu_gemv_matches_oracle():
    env = dict(os.environ, W4A16_VALU="1")
    code = _CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), cases=CASES)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                         timeout=170)
    assert res.returncode == 0, res.stderr[-3000:]
    rows = [json.loads(l) for l in res.stdout.splitlines() if l.startswith("{")]
    assert len(rows) == len(CASES)
    for r in rows:
        print(r, flush=True)
        assert "w4_valu" in r["variant"], r
        assert r["rel"] <= 1e-3 and r["max"] <= 4e-3, r
        assert r["repeat_equal"], r
