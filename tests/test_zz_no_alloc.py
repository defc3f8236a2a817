"""GPU check of w4a16_gemv_noalloc, the variant of w4a16_gemv whose split-K
workspace is a library-owned static device array instead of a caller buffer
(for callers that cannot allocate).  Its results must equal w4a16_gemv's bit
for bit (same plan, same kernels, deterministic sums), call after call, with
the array still holding the previous call's partials -- the second call of a
pair is the smaller one -- and on shapes with and without a K split, and on
the balanced plan, whose arrival counters live at the head of the array."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bit_weight_only_03_amd as L  # noqa: E402
from gpu_util import DEV, PackedW4, assert_parity, dev, to_f64  # noqa: E402


def _call_both(P, x, xdt, M):
    y_ref = P.gemv(x, xdt, M)
    y = torch.empty((M, P.N), dtype=torch.float32, device=DEV)
    y.fill_(float("nan"))
    L.w4a16_gemv_noalloc(x, xdt, P.q, P.s, P.z, y, "f32", M, P.N, P.K, P.group)
    torch.cuda.synchronize()
    return y, y_ref


# (M, N, K, group, x dtype): a split GEMV (4 slices), a smaller split GEMV
# (narrow N), the M-tiled kernel in K slices, one without a split, then the
# balanced plan (leftover tiles merged through the array).
CASES = [(5, 5120, 17408, 128, "bf16"), (2, 640, 17408, 128, "f16"), (32, 1024, 8192, 64, "f16"),
         (1, 264, 1024, 128, "f16"), (2, 5120, 17408, 128, "bf16")]


def test_noalloc_matches_gemv_bitwise_call_after_call():
    prev_ws = None
    for i, (M, N, K, g, xdt) in enumerate(CASES):
        print(f"noalloc call {i}: M={M} N={N} K={K} g={g} x={xdt}", flush=True)
        ws = L.w4a16_workspace_bytes(M, N, K, g)
        assert ws <= L.W4A16_NOALLOC_SCRATCH_BYTES
        if i != 3:
            assert ws > 0, "the case must use the workspace"
        assert ("w4_bal16" in L.w4a16_plan_variant(M, N, K, g, xdt)) == (i == 4)
        if prev_ws is not None and i == 1:
            assert ws < prev_ws, "the second call must be the smaller one"
        prev_ws = ws
        key = (140, i)
        w = synth.gen_w4(key, N, K, g)
        x = synth.gen_x(key, M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
        P = PackedW4(w, N, K, g)
        y, y_ref = _call_both(P, dev(x), xdt, M)
        assert torch.equal(y, y_ref)
        cols = np.random.default_rng(i).choice(N, size=min(N, 96), replace=False)
        if i == 4:
            cols = np.concatenate([cols, np.arange(4096, N, 5)])   # the leftover tiles
        cols = np.unique(cols)
        ref = oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, K, g,
                             cols=cols.astype(np.int64))
        assert_parity(to_f64(y)[:, cols], ref, f"noalloc call {i}")


def test_noalloc_repeated_and_in_a_graph():
    # The same call twice in a row and replayed from a captured graph (no
    # allocation inside the capture): identical bits every time.
    M, N, K, g = 4, 1024, 17408, 128
    w = synth.gen_w4((141,), N, K, g)
    x = dev(synth.gen_x((141,), M, K, "f16"))
    P = PackedW4(w, N, K, g)
    y0 = P.gemv(x, "f16", M)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        L.w4a16_gemv_noalloc(x, "f16", P.q, P.s, P.z, y, "f32", M, N, K, g, s)
        L.w4a16_gemv_noalloc(x, "f16", P.q, P.s, P.z, y, "f32", M, N, K, g, s)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        L.w4a16_gemv_noalloc(x, "f16", P.q, P.s, P.z, y, "f32", M, N, K, g, s)
    for _ in range(3):
        y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y0)


def test_noalloc_rejects_a_workspace_beyond_the_array():
    # K = 2^24 at N = 8192 needs 1024 K slices (32 MiB of partials): refused
    # on the host, before any GPU work, with the reason in the error text.
    M, N, K, g = 1, 8192, 1 << 24, 128
    assert L.w4a16_workspace_bytes(M, N, K, g) > L.W4A16_NOALLOC_SCRATCH_BYTES
    with pytest.raises(L.W4A16Error) as e:
        L.w4a16_gemv_noalloc(256, "f16", 256, 256, 256, 256, "f32", M, N, K, g)
    assert e.value.status == -5
    assert "static scratch" in L.w4a16_last_error()
