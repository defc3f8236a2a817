"""CPU checks that the dispatch is frozen: the planners read their A/B
overrides from the environment once, at the first planner call of the
process, so neither a shape's kernel (the dispatch probe) nor its workspace
size changes afterwards.  Each case runs in a fresh interpreter, since the
library keeps its overrides for the life of the process.  No GPU work: every
call is a host-only query."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# The queries of one process: (name, call) pairs evaluated in order.
_SCRIPT = r"""
import json, os, sys
sys.path.insert(0, {root!r})
import bit_weight_only_03_amd as L

def snap():
    return {{
        "w4_ws_down_m1": L.w4a16_workspace_bytes(1, 5120, 17408, 128),
        "w4_plan_down_m1": L.w4a16_plan_variant(1, 5120, 17408, 128, "f16"),
        "w4_ws_qkv_m1": L.w4a16_workspace_bytes(1, 7168, 5120, 128),
        "w4_plan_qkv_m1": L.w4a16_plan_variant(1, 7168, 5120, 128, "f16"),
        "w4_plan_down_m4": L.w4a16_plan_variant(4, 5120, 17408, 128, "bf16"),
        "w4_plan_m64": L.w4a16_plan_variant(64, 5120, 5120, 128, "f16"),
        "w4_ws_m64": L.w4a16_workspace_bytes(64, 5120, 5120, 128),
        "w16_ws": L.w16a16_workspace_bytes(1, 5120, 17408),
        "w16_ws_m2": L.w16a16_workspace_bytes(2, 5120, 17408),
        "w2t_ws": L.w2t_workspace_bytes(4, 5120, 17408, 128),
    }}

out = {{}}
if {before!r}:
    os.environ.update({env!r})
out["first"] = snap()
os.environ.update({env!r})
out["second"] = snap()
print(json.dumps(out))
"""

OVERRIDES = {"W4A16_SPLIT": "2", "W4A16_TPW": "2", "W4A16_PX": "0", "W4A16_BAL": "0", "W4A16_GEMM_SPLIT": "1",
             "W4A16_GEMM_TN": "2", "W16A16_SPLIT": "2", "W16A16_KSPLIT": "0", "W16A16_DOT": "0", "W16A16_BAL": "0",
             "W2T_STAGED_LDS_MAX": "1"}


def _run(before: bool):
    env = {k: v for k, v in os.environ.items() if k not in OVERRIDES}
    code = _SCRIPT.format(root=ROOT, env=OVERRIDES, before=before)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                         timeout=120)
    assert res.returncode == 0, res.stderr
    return json.loads(res.stdout.strip().splitlines()[-1])


def test_overrides_set_after_the_first_call_change_nothing():
    out = _run(before=False)
    assert out["first"] == out["second"]


def test_overrides_set_before_the_first_call_apply():
    # The same overrides, present from the start, do reach the planners: the
    # comparison above is not vacuous.
    plain = _run(before=False)["first"]
    forced = _run(before=True)["first"]
    H = 64 << 10                                                 # the workspace's counter head
    assert forced["w4_ws_qkv_m1"] == H + 2 * 1 * 7168 * 4      # W4A16_SPLIT=2
    assert plain["w4_ws_qkv_m1"] == 0
    assert "px=0" in forced["w4_plan_down_m4"] and "slices=2" in forced["w4_plan_down_m4"]
    assert "px=1" in plain["w4_plan_qkv_m1"]
    assert forced["w4_ws_m64"] == 0 and "slices=1" in forced["w4_plan_m64"]   # W4A16_GEMM_SPLIT=1
    assert "w4_gemm_kernel<false, 4, 4, 2>" in forced["w4_plan_m64"]          # W4A16_GEMM_TN=2
    assert forced["w16_ws"] == H + 2 * 1 * 5120 * 4             # W16A16_BAL=0, W16A16_SPLIT=2
    assert plain["w16_ws"] == 0 and plain["w16_ws_m2"] == 0      # the even-share kernel
    assert forced["w16_ws_m2"] == H + 2 * 2 * 5120 * 4
    assert plain["w4_plan_down_m1"].startswith("w4_bal16")      # W4A16_BAL=0
    assert forced["w4_plan_down_m1"].startswith("w4_mfma16")
    assert forced["w2t_ws"] != plain["w2t_ws"]                   # direct-x kernel, its own split
