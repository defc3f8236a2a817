"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle
on the same seeded inputs.

Bar: the repacking round trip and the dequantized weights are bit-exact;
GEMV outputs are within relative Frobenius 1e-3 and max abs 4e-3 * max|y|;
identities of w = (q - z) * s (q = z, s -> 2s, one-hot x, ternary +-1 counts)
hold bitwise.  Sizes span several tiles with ragged tails; the full 27B-class
shapes run in the benchmark's launch configuration with sampled columns.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bit_weight_only_03_amd as L  # noqa: E402
from gpu_util import (DEV, WS_HEAD, PackedMX, PackedW2T, PackedW4, assert_parity, dev,  # noqa: E402
                      empty_bytes, host_bits, poison, to_f64, workspace_bytes)


def say(msg):
    print(msg, flush=True)


# ------------------------------------------------------------ pack / unpack ---

W4_SHAPES = [(8, 128, 128), (24, 96, 32), (40, 384, 64), (136, 1152, 128), (16, 512, 256),
             (4104, 640, 64), (7168, 5120, 128)]


@pytest.mark.parametrize("N,K,g", W4_SHAPES)
def test_w4_pack_unpack_roundtrip_bitexact(N, K, g):
    say(f"w4 roundtrip N={N} K={K} g={g}")
    w = synth.gen_w4((101, N, K, g), N, K, g)
    P = PackedW4(w, N, K, g)
    qc = torch.empty((N, K // 8), dtype=torch.int32, device="cuda")
    sc = torch.empty((K // g, N), dtype=torch.int16, device="cuda")
    zc = torch.empty((K // g, N // 8), dtype=torch.int32, device="cuda")
    L.w4a16_unpack(P.q, P.s, P.z, qc, sc, zc, N, K, g)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(qc, np.int32), w["qweight"])
    assert np.array_equal(host_bits(sc, np.uint16), w["scales"])
    assert np.array_equal(host_bits(zc, np.int32), w["zeros"])


W2_SHAPES = [(7, 32, 32), (40, 768, 128), (136, 1280, 64), (5120, 512, 256)]


@pytest.mark.parametrize("N,K,g", W2_SHAPES)
def test_w2t_pack_unpack_roundtrip_bitexact(N, K, g):
    say(f"w2t roundtrip N={N} K={K} g={g}")
    w = synth.gen_w2t((102, N, K, g), N, K, g)
    P = PackedW2T(w, N, K, g)
    cc = torch.empty((N, K // 16), dtype=torch.int32, device="cuda")
    sc = torch.empty((K // g, N), dtype=torch.int16, device="cuda")
    L.w2t_unpack(P.q, P.s, cc, sc, N, K, g)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(cc, np.int32), w["codes"])
    assert np.array_equal(host_bits(sc, np.uint16), w["scales"])


# ------------------------------------------------------------ dequant exact ---

@pytest.mark.parametrize("N,K,g", W4_SHAPES + [(5120, 17408, 128)])
def test_w4_dequant_bitexact(N, K, g):
    say(f"w4 dequant N={N} K={K} g={g}")
    w = synth.gen_w4((103, N, K, g), N, K, g)
    P = PackedW4(w, N, K, g)
    out = torch.empty((K, N), dtype=torch.float32, device="cuda")
    L.w4a16_dequant(P.q, P.s, P.z, out, N, K, g)
    ref = oracle.w4_dequant(w["qweight"], w["scales"], w["zeros"], N, K, g)
    got = out.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("N,K,g", W2_SHAPES + [(7168, 5120, 128)])
def test_w2t_dequant_bitexact(N, K, g):
    say(f"w2t dequant N={N} K={K} g={g}")
    w = synth.gen_w2t((104, N, K, g), N, K, g)
    P = PackedW2T(w, N, K, g)
    out = torch.empty((K, N), dtype=torch.float32, device="cuda")
    L.w2t_dequant(P.q, P.s, out, N, K, g)
    ref = oracle.w2t_dequant(w["codes"], w["scales"], N, K, g)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)


# -------------------------------------------------------- GEMV, whole output ---

GEMV_CASES = [
    # (M, N, K, group, x dtype)
    (1, 8, 128, 128, "f16"),
    (1, 24, 96, 32, "f16"),
    (3, 40, 384, 64, "bf16"),
    (1, 136, 1152, 128, "f16"),
    (2, 136, 1152, 128, "bf16"),
    (4, 264, 2176, 128, "f16"),
    (5, 264, 2176, 64, "bf16"),
    (8, 520, 4096, 128, "f16"),
    (6, 1032, 1536, 256, "bf16"),
    (16, 264, 896, 32, "f16"),
    (7, 4104, 640, 64, "f16"),
    (1, 4096, 4096, 128, "f16"),
    (4, 5120, 5120, 128, "bf16"),
]


@pytest.mark.parametrize("M,N,K,g,xdt", GEMV_CASES)
def test_w4_gemv_matches_oracle(M, N, K, g, xdt):
    say(f"w4 gemv M={M} N={N} K={K} g={g} x={xdt}")
    key = (105, M, N, K, g)
    w = synth.gen_w4(key, N, K, g)
    x = synth.gen_x(key, M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    P = PackedW4(w, N, K, g)
    xd = dev(x)
    y = P.gemv(xd, xdt, M, "f32")
    torch.cuda.synchronize()
    say("  variant: " + L.w4a16_last_variant())
    ref = oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, K, g)
    assert_parity(to_f64(y), ref, f"M={M} N={N} K={K} g={g} {xdt}")
    # fp16 and bf16 outputs: the same result rounded once more.
    y16 = P.gemv(xd, xdt, M, "f16")
    assert_parity(to_f64(y16), ref, "f16 out", extra_rel=2.0 ** -11)
    yb = P.gemv(xd, xdt, M, "bf16")
    assert_parity(to_f64(yb), ref, "bf16 out", extra_rel=2.0 ** -8)


# The GEMV's x staging at its LDS edge: 5 to 8 rows (rows m and m + 4 share
# a swizzle pattern), M = 8 at K = 5120 with one tile per workgroup fills
# exactly half a CU's LDS, and a ragged last unit (K % 128 = 64) zeroes
# chunks in every swizzled row.
@pytest.mark.parametrize("M,N,K,g,xdt", [(8, 4104, 5120, 128, "bf16"), (8, 520, 5056, 64, "f16"),
                                         (5, 264, 2240, 32, "f16"), (6, 136, 4032, 64, "bf16")])
def test_w4_gemv_x_staging_rows_5_to_8(M, N, K, g, xdt):
    say(f"w4 gemv x staging M={M} N={N} K={K} g={g} x={xdt}")
    key = (131, M, N, K, g)
    w = synth.gen_w4(key, N, K, g)
    x = synth.gen_x(key, M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    P = PackedW4(w, N, K, g)
    y = P.gemv(dev(x), xdt, M, "f32")
    torch.cuda.synchronize()
    variant = L.w4a16_last_variant()
    say("  variant: " + variant)
    assert "w4_gemv_kernel" in variant
    if (M, K) == (8, 5120):
        assert "slices=1 " in variant and "lds=81920" in variant
    ref = oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, K, g)
    assert_parity(to_f64(y), ref, f"M={M} N={N} K={K} g={g} {xdt}")


# Two tiles per workgroup where one tile's x would take more than half a
# CU's LDS (8 units per wave): 513 tiles leave a last workgroup with one.
@pytest.mark.parametrize("M,g,xdt", [(8, 128, "bf16"), (6, 64, "f16"), (7, 128, "f16")])
def test_w4_gemv_two_tiles_at_long_k(M, g, xdt):
    N, K = 8208, 8192
    say(f"w4 gemv two tiles M={M} N={N} K={K} g={g} x={xdt}")
    key = (133, M, g)
    w = synth.gen_w4(key, N, K, g)
    x = synth.gen_x(key, M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    P = PackedW4(w, N, K, g)
    y = to_f64(P.gemv(dev(x), xdt, M, "f32"))
    torch.cuda.synchronize()
    variant = L.w4a16_last_variant()
    say("  variant: " + variant)
    assert "w4_gemv_kernel" in variant and "tpw=2 " in variant
    cols = sample_cols(N, np.random.default_rng(M))
    ref = oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, K, g, cols=cols)
    assert_parity(y[:, cols], ref, f"two tiles M={M} g={g}")


def test_mxfp4_gemv_two_tiles_at_long_k():
    M, N, K = 8, 8208, 8192
    say(f"mxfp4 gemv two tiles M={M} N={N} K={K}")
    key = (134, M)
    w = synth.gen_mx(key, N, K)
    x = synth.gen_x(key, M, K, "f16")
    P = PackedMX(w, N, K)
    y = to_f64(P.gemv(dev(x), "f16", M, "f32"))
    torch.cuda.synchronize()
    variant = L.w4a16_last_variant()
    say("  variant: " + variant)
    assert "tpw=2 " in variant
    cols = sample_cols(N, np.random.default_rng(M + 1))
    ref = oracle.mx_gemv(x, "f16", w["qweight"], w["scales"], M, N, K, cols=cols)
    assert_parity(y[:, cols], ref, "mx two tiles")


# Per-unit x staging (up to 4 rows, K a multiple of 128, 3 to 6 units per
# wave with one or three tiles, or 8 with one) and its fallbacks: a ragged
# last unit, and chains of one or two units per wave.
@pytest.mark.parametrize("M,N,K,g,xdt,px", [
    (3, 1032, 5120, 128, "bf16", True),    # two K slices, 3 units per wave
    (4, 24592, 3072, 64, "f16", True),     # three tiles per workgroup, a last one alone
    (2, 4104, 8192, 128, "f16", True),     # 8 units per wave
    (4, 520, 5056, 64, "bf16", False),     # ragged last unit
    (1, 264, 1024, 128, "f16", False),     # one unit per wave
])
def test_w4_gemv_per_unit_x_staging(M, N, K, g, xdt, px):
    say(f"w4 gemv per-unit x M={M} N={N} K={K} g={g} x={xdt}")
    key = (135, M, N, K, g)
    w = synth.gen_w4(key, N, K, g)
    x = synth.gen_x(key, M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    P = PackedW4(w, N, K, g)
    y = to_f64(P.gemv(dev(x), xdt, M, "f32"))
    torch.cuda.synchronize()
    variant = L.w4a16_last_variant()
    say("  variant: " + variant)
    assert ("px=1" in variant) == px
    cols = sample_cols(N, np.random.default_rng(M + K)) if N > 4200 else np.arange(N)
    ref = oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, K, g, cols=cols)
    assert_parity(y[:, cols], ref, f"per-unit x M={M} K={K}")


# Three-tile chains of 5 units (g = 128, per-unit x staging) split K
# unevenly: the first four waves take 6 units, the rest 4.  With a shorter K
# the later waves' ranges shrink or vanish (33 units: 6, 6, 6, 6, 4, 4, 1, 0).
@pytest.mark.parametrize("M,K,xdt", [(1, 4224, "f16"), (4, 4224, "bf16"), (2, 4608, "f16"),
                                     (3, 5120, "bf16")])
def test_w4_gemv_uneven_wave_split(M, K, xdt):
    N = 24592   # 1537 tiles: the last workgroup has one
    say(f"uneven split M={M} N={N} K={K} x={xdt}")
    key = (161, M, K)
    w = synth.gen_w4(key, N, K, 128)
    x = synth.gen_x(key, M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    P = PackedW4(w, N, K, 128)
    y = to_f64(P.gemv(dev(x), xdt, M))
    variant = L.w4a16_last_variant()
    say("  variant: " + variant)
    assert "upw=5 tpw=3" in variant and "px=1" in variant and "slices=1 " in variant
    cols = sample_cols(N, np.random.default_rng(K + M), n=256)
    ref = oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, K, 128, cols=cols)
    assert_parity(y[:, cols], ref, f"uneven split M={M} K={K}")


# M-tiled kernel (more rows than one MFMA block): 2 to 4 row blocks, one or
# two tiles per wave, every group size, ragged N (a last tile of 8 columns)
# and ragged K (a last unit of 64 k), with and without K slices.
GEMM_CASES = [
    # (M, N, K, group, x dtype)
    (17, 264, 1216, 64, "f16"),
    (24, 136, 896, 128, "bf16"),
    (32, 520, 2048, 128, "f16"),
    (33, 40, 384, 32, "bf16"),
    (48, 1032, 1536, 256, "f16"),
    (64, 264, 4352, 128, "bf16"),
    (64, 4104, 640, 64, "f16"),
    (20, 8, 128, 128, "f16"),
    (40, 33808, 512, 128, "bf16"),
]


@pytest.mark.parametrize("M,N,K,g,xdt", GEMM_CASES)
def test_w4_gemm_matches_oracle(M, N, K, g, xdt):
    say(f"w4 gemm M={M} N={N} K={K} g={g} x={xdt}")
    key = (117, M, N, K, g)
    w = synth.gen_w4(key, N, K, g)
    x = synth.gen_x(key, M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    P = PackedW4(w, N, K, g)
    xd = dev(x)
    y = P.gemv(xd, xdt, M, "f32")
    torch.cuda.synchronize()
    variant = L.w4a16_last_variant()
    say("  variant: " + variant)
    assert "w4_gemm_kernel" in variant
    cols = np.arange(N) if N <= 4200 else np.sort(np.random.default_rng(1).choice(N, 700, replace=False))
    ref = oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, K, g, cols=cols.astype(np.int64))
    assert_parity(to_f64(y)[:, cols], ref, f"M={M} N={N} K={K} g={g} {xdt}")
    y16 = P.gemv(xd, xdt, M, "f16")
    assert_parity(to_f64(y16)[:, cols], ref, "f16 out", extra_rel=2.0 ** -11)
    # repeat calls give the same bits
    assert torch.equal(P.gemv(xd, xdt, M, "f32"), y)


@pytest.mark.parametrize("M,xdt", [(64, "bf16"), (32, "f16")])
def test_w4_gemm_full_size_sampled(M, xdt):
    # The 27B-class gate_up and down layers with a batch of rows: sampled
    # columns against the oracle (which computes them one by one).
    for (N, K) in [(34816, 5120), (5120, 17408)]:
        say(f"w4 gemm full size M={M} N={N} K={K} x={xdt}")
        key = (118, M, N, K)
        w = synth.gen_w4(key, N, K, 128)
        x = synth.gen_x(key, M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
        P = PackedW4(w, N, K, 128)
        y = P.gemv(dev(x), xdt, M, "f32")
        torch.cuda.synchronize()
        say("  variant: " + L.w4a16_last_variant())
        cols = np.sort(np.random.default_rng(2).choice(N, 96, replace=False)).astype(np.int64)
        ref = oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, K, 128, cols=cols)
        assert_parity(to_f64(y)[:, cols], ref, f"full size M={M} N={N} K={K}")


# Fused residual add: GEMV unsplit and split (merge kernel), tiled unsplit and
# split, residual in every dtype, in place (residual is y) and not.
GEMV_ADD_CASES = [
    # (M, N, K, group, x dtype, residual dtype, y dtype, in place)
    (1, 4096, 4096, 128, "f16", "f32", "f32", False),
    (1, 5120, 5120, 128, "f16", "f16", "f16", True),
    (4, 640, 17408, 128, "bf16", "bf16", "bf16", True),
    (3, 264, 2176, 64, "f16", "f16", "f32", False),
    (32, 520, 2048, 128, "f16", "f16", "f16", True),
    (64, 264, 4352, 128, "bf16", "f32", "f32", True),
    (20, 4104, 640, 64, "f16", "bf16", "f32", False),
]
_TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
_ROUND = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


@pytest.mark.parametrize("M,N,K,g,xdt,rdt,ydt,inplace", GEMV_ADD_CASES)
def test_w4_gemv_add_matches_oracle(M, N, K, g, xdt, rdt, ydt, inplace):
    say(f"w4 gemv_add M={M} N={N} K={K} g={g} x={xdt} r={rdt} y={ydt} inplace={inplace}")
    key = (119, M, N, K, g)
    w = synth.gen_w4(key, N, K, g)
    x = synth.gen_x(key, M, K, xdt)
    P = PackedW4(w, N, K, g)
    rng = np.random.default_rng(key)
    r64 = rng.standard_normal((M, N)) * 4.0
    r = torch.from_numpy(r64).to(_TORCH_DT[rdt]).cuda()
    rref = r.double().cpu().numpy()                 # the residual as stored
    if inplace:
        assert rdt == ydt
        y = r.clone()
        res = y
    else:
        y = torch.full((M, N), float("nan"), dtype=_TORCH_DT[ydt], device=DEV)
        res = r
    wsb = L.w4a16_workspace_bytes(M, N, K, g)
    ws = workspace_bytes(wsb) if wsb else None
    L.w4a16_gemv_add(dev(x), xdt, P.q, P.s, P.z, res, rdt, y, ydt, M, N, K, g, ws, wsb)
    torch.cuda.synchronize()
    say("  variant: " + L.w4a16_last_variant())
    ref = oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, K, g) + rref
    assert_parity(to_f64(y), ref, f"gemv_add M={M} N={N} K={K}", extra_rel=_ROUND[ydt])
    if not inplace:
        assert torch.equal(r, res)                  # the residual is only read


def test_w4_gemv_add_zero_residual_is_bitwise_gemv():
    # v + 0 = v in fp32: a zero residual reproduces w4a16_gemv bit for bit,
    # through the GEMV, its split merge and the tiled kernel.
    for (M, N, K, g) in [(1, 1032, 2048, 128), (4, 640, 17408, 128), (24, 264, 1024, 64)]:
        say(f"gemv_add zero residual M={M} N={N} K={K} g={g}")
        w = synth.gen_w4((120, M, N, K), N, K, g)
        xd = dev(synth.gen_x((120, M, K), M, K, "f16"))
        P = PackedW4(w, N, K, g)
        y0 = P.gemv(xd, "f16", M, "f32")
        y1 = torch.empty_like(y0)
        zero = torch.zeros((M, N), dtype=torch.float32, device=DEV)
        wsb = L.w4a16_workspace_bytes(M, N, K, g)
        ws = workspace_bytes(wsb) if wsb else None
        L.w4a16_gemv_add(xd, "f16", P.q, P.s, P.z, zero, "f32", y1, "f32", M, N, K, g, ws, wsb)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1)


# 16-bit weights: both dtypes, every output dtype, M from 1 to 64, ragged N
# (a last tile of 8 columns) and ragged K (a last unit of 40 k), with and
# without K slices.
W16_CASES = [
    # (M, N, K, dtype)
    (1, 264, 1000, "f16"),
    (2, 520, 4096, "bf16"),
    (4, 4096, 4096, "f16"),
    (8, 136, 2048, "bf16"),
    (16, 1032, 640, "f16"),
    (24, 40, 8, "bf16"),
    (64, 264, 1536, "f16"),
    (3, 12296, 512, "bf16"),
    # The K-split kernel at its limits: 16 rows filling half a CU's LDS, and
    # 12 rows with 3 or 4 units per wave and a ragged last one; 7 rows with a
    # ragged last tile.  The dot-product kernel (up to 4 rows): a single unit
    # (three waves without units), 16 units per wave with a ragged last one,
    # 3 rows of its 4-row block with 11 or 12 units per wave.  Shapes whose x
    # is too large for both, or with more units per wave than they take.
    (16, 264, 2560, "bf16"),
    (12, 520, 3240, "f16"),
    (7, 1000, 3000, "bf16"),
    (2, 40, 8, "f16"),
    (1, 520, 8168, "f16"),
    (3, 1032, 5760, "f16"),
    (6, 264, 8192, "bf16"),
    (1, 520, 17400, "f16"),
    (2, 264, 17400, "bf16"),
    # The even-share kernel (between one and two tiles per CU, more than 64
    # units, up to 2 rows): 4 or 5 groups of 4 rows per workgroup with a
    # last unit of 8 k, 6 or 7 with the down shape's 136 units (a ragged
    # last one), 7 or 8 groups.
    (1, 4104, 8200, "bf16"),
    (2, 6152, 17400, "f16"),
    (1, 8176, 9000, "f16"),
]


def w16_expected_kernel(M, N, K):
    # Between one and two tiles per CU, more than 64 units, up to 2 rows:
    # one even row share per CU when x and the partial slots fit 144 KB.  Else one workgroup per
    # tile up to 8 units per wave (the dot-product kernel up to 4 rows, the
    # K-split kernel up to 16) when a wave's x fits 16 loads and the
    # workgroup's x half of a CU's LDS; otherwise the tiled kernel.
    U = -(-K // 128)
    upw = -(-U // 8)
    C = torch.cuda.get_device_properties(0).multi_processor_count
    T = -(-N // 16)
    gmax = -(-(-(-N // 4)) // C)
    if M <= 2 and C < T < 2 * C and U > 64 and M * U * 256 + gmax * 16 * M * 16 <= 144 * 1024:
        return "w16_dot_bal_kernel"
    if not (upw <= 8 and M * upw <= 64 and M * U * 256 <= 80 * 1024):
        return "w16_gemv_kernel"
    return "w16_dot_kernel" if M <= 4 else "w16_ksplit_kernel" if M <= 16 else "w16_gemv_kernel"


@pytest.mark.parametrize("M,N,K,dt", W16_CASES)
def test_w16a16_gemv_matches_oracle(M, N, K, dt):
    say(f"w16a16 M={M} N={N} K={K} {dt}")
    key = (121, M, N, K)
    w = synth.gen_w16(key, N, K, dt)
    x = synth.gen_x(key, M, K, dt)
    wd, xd = dev(w), dev(x)
    wsb = L.w16a16_workspace_bytes(M, N, K)
    ws = workspace_bytes(wsb) if wsb else None
    cols = np.arange(N) if N <= 4200 else np.sort(np.random.default_rng(4).choice(N, 600, replace=False))
    ref = oracle.w16_gemv(x, dt, w, M, N, K, cols=cols.astype(np.int64))
    for ydt, extra in (("f32", 0.0), ("f16", 2.0 ** -11), ("bf16", 2.0 ** -8)):
        y = torch.full((M, N), float("nan"), dtype=_TORCH_DT[ydt], device=DEV)
        L.w16a16_gemv(xd, wd, dt, y, ydt, M, N, K, ws, wsb)
        torch.cuda.synchronize()
        if ydt == "f32":
            variant = L.w4a16_last_variant()
            say("  variant: " + variant)
            assert w16_expected_kernel(M, N, K) + "<" in variant
            y0 = y.clone()
        assert_parity(to_f64(y)[:, cols], ref, f"w16 M={M} N={N} K={K} {dt} y={ydt}", extra_rel=extra)
    y1 = torch.empty_like(y0)
    L.w16a16_gemv(xd, wd, dt, y1, "f32", M, N, K, ws, wsb)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)                           # deterministic


@pytest.mark.parametrize("M,N,K", [(1, 264, 1000), (1, 4104, 8200), (8, 264, 2560), (24, 40, 2048)])
@pytest.mark.parametrize("sub", ["x", "w"])
def test_w16a16_fp16_subnormal_operands(M, N, K, sub):
    # Every product has one fp16 subnormal factor (2^-20, bits 0x0010) and
    # one 1.0: y = K * 2^-20 exactly in fp32 for every column.  An operand
    # flushed to zero anywhere on the path (the dot-product kernels' v_dot2,
    # the MFMA kernels) would give 0.  One shape per kernel: dot product,
    # even shares, K-split, tiled.
    say(f"w16 subnormal {sub} M={M} N={N} K={K}")
    one, tiny = np.uint16(0x3C00), np.uint16(0x0010)
    x = np.full((M, K), tiny if sub == "x" else one, dtype=np.uint16)
    w = np.full((N, K), tiny if sub == "w" else one, dtype=np.uint16)
    wsb = L.w16a16_workspace_bytes(M, N, K)
    ws = workspace_bytes(wsb) if wsb else None
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    L.w16a16_gemv(dev(x), dev(w), "f16", y, "f32", M, N, K, ws, wsb)
    torch.cuda.synchronize()
    say("  variant: " + L.w4a16_last_variant())
    cols = np.array([0, 1, N // 2, N - 1], dtype=np.int64)
    ref = oracle.w16_gemv(x, "f16", w, M, N, K, cols=cols)
    assert np.all(ref == K * 2.0 ** -20)
    assert np.array_equal(to_f64(y)[:, cols], ref)
    assert torch.all(y == K * 2.0 ** -20)


W2_GEMV_CASES = [
    (1, 7, 32, 32, "f16"),
    (4, 40, 768, 128, "f16"),
    (8, 136, 1280, 64, "bf16"),
    (3, 264, 2304, 256, "f16"),
    (16, 520, 512, 32, "bf16"),
    (1, 7168, 5120, 128, "f16"),
    # Staged kernel in two K slices with uneven units per wave and a ragged
    # last unit, and one whose workgroup would need more than half a CU's
    # LDS (the direct-x kernel).
    (5, 1032, 8896, 64, "f16"),
    (7, 4104, 6144, 128, "bf16"),
]


@pytest.mark.parametrize("M,N,K,g,xdt", W2_GEMV_CASES)
def test_w2t_gemv_matches_oracle(M, N, K, g, xdt):
    say(f"w2t gemv M={M} N={N} K={K} g={g} x={xdt}")
    key = (106, M, N, K, g)
    w = synth.gen_w2t(key, N, K, g)
    x = synth.gen_x(key, M, K, xdt)
    P = PackedW2T(w, N, K, g)
    y = P.gemv(dev(x), xdt, M)
    torch.cuda.synchronize()
    variant = L.w4a16_last_variant()
    say("  variant: " + variant)
    if (M, K) == (5, 8896):
        assert "w2t_gemv_kernel" in variant and "slices=2 " in variant
    if (M, K) == (7, 6144):
        assert "w2t_gemv_direct_kernel" in variant
    ref = oracle.w2t_gemv(x, xdt, w["codes"], w["scales"], M, N, K, g)
    assert_parity(to_f64(y), ref, f"w2t M={M} N={N} K={K}")


# ----------------------------------------------------------- bitwise identities ---

def _w4_constant_q(z, g, N, rng):
    """Canonical arrays whose every weight equals its group's zero point."""
    G = z.shape[0]
    q = np.repeat(z, g, axis=0)  # [K][N]
    qweight = np.zeros((N, G * g // 8), dtype=np.uint32)
    for i in range(8):
        qweight |= (q[i::8].T.astype(np.uint32) << np.uint32(4 * i))
    zeros = np.zeros((G, N // 8), dtype=np.uint32)
    for i in range(8):
        zeros |= (z[:, i::8].astype(np.uint32) << np.uint32(4 * i))
    return {"qweight": qweight.view(np.int32), "zeros": zeros.view(np.int32),
            "scales": synth.f64_to_f16_bits(rng.uniform(0.002, 0.02, size=(G, N)))}


# Kernels covered: the GEMV with x staged unit by unit (M <= 4, 3 units per
# wave), with the whole range staged (M = 8), in K slices (narrow N, long K),
# the M-tiled kernel (M = 32) and its K slices (M = 64, narrow N).
IDENTITY_CASES = [(4, 264, 3072, 128), (1, 264, 3072, 64), (8, 264, 1024, 128),
                  (4, 264, 17408, 128), (32, 520, 1024, 64), (64, 136, 4096, 128)]


@pytest.mark.parametrize("M,N,K,g", IDENTITY_CASES)
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_w4_zero_point_identity_gives_exact_zero(M, N, K, g, xdt):
    # q = z everywhere: every weight (q - z) * s is 0, so y is exactly 0 for
    # either activation type -- q - z is formed exactly before any product.
    say(f"w4 q = z identity M={M} N={N} K={K} g={g} x={xdt}")
    rng = np.random.default_rng(7 + M + K)
    w = _w4_constant_q(rng.integers(0, 16, size=(K // g, N)), g, N, rng)
    x = synth.gen_x((1, M, K), M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    assert np.all(oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, K, g) == 0)
    y = PackedW4(w, N, K, g).gemv(dev(x), xdt, M)
    torch.cuda.synchronize()
    say("  variant: " + L.w4a16_last_variant())
    assert torch.count_nonzero(y).item() == 0


@pytest.mark.parametrize("M,N,K,g", [(4, 520, 2048, 128), (8, 520, 2048, 64), (32, 264, 1024, 128)])
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_w4_scale_doubling_is_bitwise(M, N, K, g, xdt):
    # s -> 2s doubles every weight exactly, and with it every fp32 partial
    # sum: y doubles bit for bit.
    say(f"w4 s -> 2s M={M} x={xdt}")
    w = synth.gen_w4((107, M), N, K, g)
    w2 = dict(w, scales=(w["scales"].view(np.float16) * np.float16(2)).view(np.uint16))
    x = dev(synth.gen_x((107, M), M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0))
    y1 = PackedW4(w, N, K, g).gemv(x, xdt, M)
    y2 = PackedW4(w2, N, K, g).gemv(x, xdt, M)
    assert torch.equal(y2, 2 * y1)


@pytest.mark.parametrize("M,N,K,g", [(4, 520, 3072, 128), (8, 264, 2048, 64), (2, 136, 17408, 128),
                                     (32, 264, 1024, 128)])
def test_w4_bf16_x_equals_f16_x_bitwise(M, N, K, g):
    # bf16 activations are taken to fp16 on chip (exact over fp16's range,
    # round to nearest even below it), so a bf16 x gives bit for bit the
    # result of the fp16 x holding the same values.  The x here spans the
    # contract: N(0,1) with outliers, values at the largest bf16 below
    # fp16's overflow (65280), at 2^-17 (the smallest exact magnitude) and
    # below it, where both sides round to fp16's 2^-24 grid the same way.
    say(f"w4 bf16 x = f16 x M={M} N={N} K={K} g={g}")
    xb = synth.gen_x((108, M, K), M, K, "bf16", outlier_frac=0.01)
    rng = np.random.default_rng(M + K)
    special = np.array([65280.0, -65280.0, 2.0 ** -17, -(2.0 ** -17), 3 * 2.0 ** -20,
                        2.0 ** -24 * 1.5, 2.0 ** -26], dtype=np.float32)
    pos = rng.choice(M * K, size=special.size, replace=False)
    xb = xb.copy().reshape(-1)
    xb[pos] = (special.view(np.uint32) >> 16).astype(np.uint16)
    xb = xb.reshape(M, K)
    xf32 = (xb.astype(np.uint32) << 16).view(np.float32)
    xh = xf32.astype(np.float16).view(np.uint16)
    w = synth.gen_w4((108, N, K), N, K, g)
    P = PackedW4(w, N, K, g)
    yb = P.gemv(dev(xb), "bf16", M)
    yh = P.gemv(dev(xh), "f16", M)
    torch.cuda.synchronize()
    assert torch.equal(yb, yh)
    ref = oracle.w4_gemv(xb, "bf16", w["qweight"], w["scales"], w["zeros"], M, N, K, g)
    assert_parity(to_f64(yb), ref, "bf16 range edges")


def test_w4_one_hot_rows_are_exact():
    say("w4 one-hot rows")
    N, K, g = 136, 512, 64
    w = synth.gen_w4((108,), N, K, g)
    P = PackedW4(w, N, K, g)
    Wref = oracle.w4_dequant(w["qweight"], w["scales"], w["zeros"], N, K, g)
    ks = [0, 1, 7, 8, 31, 32, 63, 64, 65, 127, 128, 200, 255, 256, 383, 448, 511]
    for start in range(0, len(ks), 16):
        chunk = ks[start:start + 16]
        x = np.zeros((len(chunk), K), dtype=np.uint16)
        for r, k in enumerate(chunk):
            x[r, k] = 0x3C00
        y = to_f64(P.gemv(dev(x), "f16", len(chunk)))
        for r, k in enumerate(chunk):
            assert np.array_equal(y[r], Wref[k]), f"k={k}"


def test_w2t_all_ones_counts_exact():
    say("w2t +-1 counts")
    N, K, g = 264, 2048, 128
    w = synth.gen_w2t((109,), N, K, g)
    w["scales"] = np.full_like(w["scales"], 0x3C00)
    P = PackedW2T(w, N, K, g)
    x = np.full((1, K), 0x3C00, dtype=np.uint16)
    y = to_f64(P.gemv(dev(x), "f16", 1))
    codes = w["codes"].view(np.uint32)
    c = np.stack([(codes >> np.uint32(2 * i)) & 3 for i in range(16)], axis=-1).reshape(N, K)
    expect = (c == 2).sum(axis=1) - (c == 0).sum(axis=1)
    assert np.array_equal(y[0], expect.astype(np.float64))


# ------------------------------------------------------------ balanced plan ---
# Layers of 256 + 64 tiles with K = 8 x 17 units (the 27B-class down layer,
# N = 5120, K = 17408; 5112 gives it a ragged last tile) run the balanced
# GEMV up to 4 rows: each workgroup's extra waves take a quarter of one of
# the 64 leftover tiles and the four pieces are merged through the
# workspace, the last arrival adding them.

BAL_K, BAL_G = 17408, 128
_BAL = {}


def _bal_matrix(N):
    if N not in _BAL:
        _BAL.clear()
        w = synth.gen_w4((150, N), N, BAL_K, BAL_G)
        _BAL[N] = (w, PackedW4(w, N, BAL_K, BAL_G))
    return _BAL[N]


def _bal_cols(N, seed):
    """Columns to check on a balanced-plan layer: a sample of the tiles the
    full waves stream and every column of the leftover tiles (4096 up)."""
    rng = np.random.default_rng(seed)
    cols = set(rng.choice(4096, size=96, replace=False).tolist()) | set(range(4096, N)) | {0, 15, 16, 4095}
    return np.array(sorted(cols), dtype=np.int64)


@pytest.mark.parametrize("M,N,xdt", [(1, 5120, "f16"), (1, 5120, "bf16"), (2, 5120, "f16"),
                                     (3, 5120, "bf16"), (3, 5112, "f16"), (1, 5112, "bf16"),
                                     (4, 5120, "bf16"), (4, 5112, "f16")])
def test_balanced_plan_matches_oracle(M, N, xdt):
    say(f"balanced M={M} N={N} x={xdt}")
    w, P = _bal_matrix(N)
    x = synth.gen_x((151, M, N), M, BAL_K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    y = to_f64(P.gemv(dev(x), xdt, M))
    variant = L.w4a16_last_variant()
    say("  variant: " + variant)
    assert variant.startswith("w4_bal16") and "pieces=4" in variant
    cols = _bal_cols(N, M)
    ref = oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, BAL_K, BAL_G, cols=cols)
    assert_parity(y[:, cols], ref, f"balanced M={M} N={N}")


def test_balanced_plan_rows_and_group():
    # Up to 3 rows stage each wave's whole x range; at 4 rows that does not
    # fit LDS next to the extra waves' x, so x is staged unit by unit into
    # rings.  Past 4 rows, or at g = 64, the other plans run.
    for M in (1, 2, 3):
        v = L.w4a16_plan_variant(M, 5120, BAL_K, BAL_G, "f16")
        assert v.startswith("w4_bal16") and "px=0" in v, v
    assert "px=1" in L.w4a16_plan_variant(4, 5120, BAL_K, BAL_G, "bf16")
    assert L.w4a16_plan_variant(5, 5120, BAL_K, BAL_G, "f16").startswith("w4_mfma16")
    assert L.w4a16_plan_variant(1, 5120, BAL_K, 64, "f16").startswith("w4_mfma16")


@pytest.mark.parametrize("M,xdt,rdt,ydt,inplace", [(2, "bf16", "bf16", "bf16", True),
                                                   (1, "f16", "f32", "f16", False)])
def test_balanced_plan_adds_the_residual(M, xdt, rdt, ydt, inplace):
    # The leftover tiles' outputs are stored by the last piece to arrive,
    # which adds the residual there.
    N = 5120
    say(f"balanced gemv_add M={M} x={xdt} r={rdt} y={ydt} inplace={inplace}")
    w, P = _bal_matrix(N)
    x = synth.gen_x((152, M), M, BAL_K, xdt)
    r64 = np.random.default_rng(152 + M).standard_normal((M, N)) * 4.0
    r = torch.from_numpy(r64).to(_TORCH_DT[rdt]).cuda()
    rref = r.double().cpu().numpy()
    y = r.clone() if inplace else torch.full((M, N), float("nan"), dtype=_TORCH_DT[ydt], device=DEV)
    wsb = L.w4a16_workspace_bytes(M, N, BAL_K, BAL_G)
    ws = workspace_bytes(wsb)
    L.w4a16_gemv_add(dev(x), xdt, P.q, P.s, P.z, y if inplace else r, rdt, y, ydt, M, N, BAL_K, BAL_G,
                     ws, wsb)
    torch.cuda.synchronize()
    assert L.w4a16_last_variant().startswith("w4_bal16")
    cols = _bal_cols(N, 7 + M)
    ref = oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, BAL_K, BAL_G, cols=cols)
    assert_parity(to_f64(y)[:, cols], ref + rref[:, cols], "balanced gemv_add", extra_rel=_ROUND[ydt])


@pytest.mark.parametrize("M,xdt", [(1, "f16"), (3, "bf16"), (4, "bf16")])
def test_balanced_plan_repeat_calls_and_graph_replays(M, xdt):
    # Which piece arrives last varies from call to call; the pieces are still
    # added in a fixed order, so every call and replay gives the same bits,
    # and every call leaves the arrival counters at zero.
    N = 5120
    say(f"balanced determinism M={M} x={xdt}")
    _, P = _bal_matrix(N)
    x = dev(synth.gen_x((153, M), M, BAL_K, xdt))
    wsb = L.w4a16_workspace_bytes(M, N, BAL_K, BAL_G)
    ws = workspace_bytes(wsb)
    y0 = P.gemv(x, xdt, M, workspace=ws).clone()
    for _ in range(20):
        assert torch.equal(P.gemv(x, xdt, M, workspace=ws), y0)
    y = torch.empty_like(y0)
    _graph_replays_match(
        lambda s: L.w4a16_gemv(x, xdt, P.q, P.s, P.z, y, "f32", M, N, BAL_K, BAL_G, ws, wsb, stream=s),
        y, y0, lambda: P.gemv(x, xdt, M, workspace=ws))
    torch.cuda.synchronize()
    assert int(ws[:WS_HEAD].count_nonzero()) == 0


_BAL_MX = {}


def _bal_mx_matrix(N):
    if N not in _BAL_MX:
        _BAL_MX.clear()
        w = synth.gen_mx((154, N), N, BAL_K)
        _BAL_MX[N] = (w, PackedMX(w, N, BAL_K))
    return _BAL_MX[N]


@pytest.mark.parametrize("M,N,xdt", [(1, 5120, "f16"), (1, 5112, "bf16"), (2, 5120, "bf16"),
                                     (3, 5112, "f16"), (4, 5120, "bf16"), (4, 5112, "f16")])
def test_mxfp4_balanced_plan_matches_oracle(M, N, xdt):
    # MXFP4 weights on the same layer shapes take the same plan.
    say(f"mxfp4 balanced M={M} N={N} x={xdt}")
    w, P = _bal_mx_matrix(N)
    x = synth.gen_x((155, M, N), M, BAL_K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    y = to_f64(P.gemv(dev(x), xdt, M))
    variant = L.w4a16_last_variant()
    say("  variant: " + variant)
    assert variant.startswith("mxfp4_bal16") and "pieces=4" in variant
    assert ("px=1" in variant) == (M == 4)
    cols = _bal_cols(N, 20 + M)
    ref = oracle.mx_gemv(x, xdt, w["qweight"], w["scales"], M, N, BAL_K, cols=cols)
    assert_parity(y[:, cols], ref, f"mxfp4 balanced M={M} N={N}")


# ------------------------------------------------------- determinism and graphs ---

def test_repeat_calls_and_graph_replay_are_bitwise_identical():
    say("determinism + graph replay")
    M, N, K, g = 5, 5120, 17408, 128          # the split GEMV (4 K slices and the merge)
    w = synth.gen_w4((110,), N, K, g)
    P = PackedW4(w, N, K, g)
    x = dev(synth.gen_x((110,), M, K, "bf16", outlier_frac=0.01))
    y0 = P.gemv(x, "bf16", M).clone()
    for _ in range(20):
        assert torch.equal(P.gemv(x, "bf16", M), y0)
    y = torch.empty_like(y0)
    wsb = L.w4a16_workspace_bytes(M, N, K, g)
    ws = workspace_bytes(wsb) if wsb else None
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        L.w4a16_gemv(x, "bf16", P.q, P.s, P.z, y, "f32", M, N, K, g, ws, wsb, stream=s)  # warm up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        L.w4a16_gemv(x, "bf16", P.q, P.s, P.z, y, "f32", M, N, K, g, ws, wsb, stream=s)
    for r in range(5):
        y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y0), f"replay {r}"
        assert torch.equal(P.gemv(x, "bf16", M), y0)   # eager work between replays


def _graph_replays_match(call, y, y0, eager):
    """Capture call() (writing y) in a graph; every replay, with eager work
    and synchronizations between them, must reproduce y0 bit for bit."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(s)                                  # warm up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        call(s)
    for r in range(4):
        y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y0), f"replay {r}"
        assert torch.equal(eager(), y0)          # eager work between replays


@pytest.mark.parametrize("M,N,K", [(1, 5120, 17408), (4, 5120, 17408), (5, 5120, 17408),
                                   (64, 2064, 1280), (1, 4104, 5120)])
def test_mxfp4_repeat_calls_and_graph_replay_are_bitwise_identical(M, N, K):
    # The balanced plan (whole-range and per-unit x staging; it merges four
    # pieces across workgroups), GEMV with K slices, the M-tiled kernel, and
    # a plain GEMV.  Every balanced call leaves the arrival counters at zero.
    say(f"mxfp4 determinism M={M} N={N} K={K}")
    w = synth.gen_mx((129, M), N, K)
    P = PackedMX(w, N, K)
    x = dev(synth.gen_x((129, M), M, K, "bf16", outlier_frac=0.01))
    y0 = P.gemv(x, "bf16", M).clone()
    for _ in range(10):
        assert torch.equal(P.gemv(x, "bf16", M), y0)
    y = torch.empty_like(y0)
    wsb = L.mxfp4_workspace_bytes(M, N, K)
    ws = workspace_bytes(wsb) if wsb else None
    _graph_replays_match(
        lambda s: L.mxfp4_gemv(x, "bf16", P.q, P.s, y, "f32", M, N, K, ws, wsb, stream=s),
        y, y0, lambda: P.gemv(x, "bf16", M))
    torch.cuda.synchronize()
    if K == 17408 and M <= 4:
        assert L.w4a16_last_variant().startswith("mxfp4_bal16")
        assert int(ws[:WS_HEAD].count_nonzero()) == 0


@pytest.mark.parametrize("M,N,K", [(1, 5120, 5120), (2, 5120, 17408), (24, 1032, 2048)])
def test_w16a16_and_ternary_graph_replay_are_bitwise_identical(M, N, K):
    say(f"w16 / ternary determinism M={M} N={N} K={K}")
    w = dev(synth.gen_w16((130, M), N, K, "f16"))
    x = dev(synth.gen_x((130, M), M, K, "f16"))
    wsb = L.w16a16_workspace_bytes(M, N, K)
    ws = workspace_bytes(wsb) if wsb else None

    def w16(yy, s=None):
        L.w16a16_gemv(x, w, "f16", yy, "f32", M, N, K, ws, wsb, stream=s)
        return yy
    y0 = w16(torch.empty((M, N), dtype=torch.float32, device=DEV)).clone()
    torch.cuda.synchronize()
    y = torch.empty_like(y0)
    _graph_replays_match(lambda s: w16(y, s), y, y0,
                         lambda: w16(torch.empty_like(y0)))
    if M <= 16:
        g = 128
        P2 = PackedW2T(synth.gen_w2t((131,), N, K, g), N, K, g)
        t0 = P2.gemv(x, "f16", M).clone()
        for _ in range(5):
            assert torch.equal(P2.gemv(x, "f16", M), t0)


def test_split_k_narrow_shard_parity_and_poisoned_workspace():
    # One GPU's column share of down (N = 5120/8 = 640) splits K across
    # workgroups and merges fp32 partials from the workspace.
    M, N, K, g = 4, 640, 17408, 128
    say(f"split-K M={M} N={N} K={K}")
    ws = L.w4a16_workspace_bytes(M, N, K, g)
    assert ws > 0
    w = synth.gen_w4((111,), N, K, g)
    x = synth.gen_x((111,), M, K, "bf16", outlier_frac=0.01)
    P = PackedW4(w, N, K, g)
    work = workspace_bytes(ws)
    poison(work, float("nan"))
    y = P.gemv(dev(x), "bf16", M, workspace=work)
    torch.cuda.synchronize()
    variant = L.w4a16_last_variant()
    say("  variant: " + variant)
    assert "slices=1 " not in variant
    ref = oracle.w4_gemv(x, "bf16", w["qweight"], w["scales"], w["zeros"], M, N, K, g)
    assert_parity(to_f64(y), ref, "split-K")
    poison(work, float("inf"))
    assert torch.equal(P.gemv(dev(x), "bf16", M, workspace=work), y)
    assert int(work[:WS_HEAD].count_nonzero()) == 0   # the counter head untouched


def test_split_k_workspace_reused_across_shapes_and_graph_replays():
    # One workspace, sized for the largest call and poisoned beforehand past
    # its counter head, serves a sequence of split calls of different shapes
    # and slice counts -- and balanced-plan calls, which count arrivals in
    # the head -- on one stream, also inside a graph replayed many times with
    # eager calls through the same workspace in between.  The ternary GEMV's
    # split path (the direct-x kernel) follows the same contract.
    cases = [(1, 640, 17408, 128, "f16"), (2, 5120, 17408, 128, "bf16"), (4, 2048, 8192, 64, "bf16"),
             (3, 1024, 12288, 128, "f16"), (1, 5120, 17408, 128, "f16"), (2, 640, 17408, 128, "bf16")]
    packs, xs, refs, sizes = [], [], [], []
    for i, (M, N, K, g, xdt) in enumerate(cases):
        w = synth.gen_w4((115, i), N, K, g)
        x = synth.gen_x((115, i), M, K, xdt)
        packs.append(PackedW4(w, N, K, g))
        xs.append(dev(x))
        cols = None if N <= 2048 else _bal_cols(N, i)
        refs.append((cols, oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, K, g,
                                          cols=cols)))
        sizes.append(L.w4a16_workspace_bytes(M, N, K, g))
        plan = L.w4a16_plan_variant(M, N, K, g, xdt)
        assert ("w4_bal16" in plan) == (N == 5120), plan
        assert "w4_bal16" in plan or "slices=1 " not in plan, plan
    assert all(b > 0 for b in sizes), sizes
    M2, N2, K2, g2 = 8, 640, 17408, 128          # the ternary call at the end
    wsb2 = L.w2t_workspace_bytes(M2, N2, K2, g2)
    assert wsb2 > 0
    work = workspace_bytes(max(sizes + [wsb2]))
    poison(work, float("nan"))
    ys = [torch.empty((M, N), dtype=torch.float32, device=DEV) for (M, N, _, _, _) in cases]
    s = torch.cuda.Stream()

    def run_all():
        for (M, N, K, g, xdt), P, x, y in zip(cases, packs, xs, ys):
            L.w4a16_gemv(x, xdt, P.q, P.s, P.z, y, "f32", M, N, K, g, work, work.numel(), stream=s)

    with torch.cuda.stream(s):
        run_all()
    torch.cuda.synchronize()
    first = [y.clone() for y in ys]
    for (M, N, K, g, xdt), y, (cols, ref) in zip(cases, first, refs):
        got = to_f64(y) if cols is None else to_f64(y)[:, cols]
        assert_parity(got, ref, f"shared workspace M={M} N={N} K={K} g={g}")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        run_all()
    for r in range(8):
        for y in ys:
            y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for y, y0 in zip(ys, first):
            assert torch.equal(y, y0), f"replay {r}"
        M, N, K, g, xdt = cases[1]
        assert torch.equal(packs[1].gemv(xs[1], xdt, M, workspace=work), first[1])
    M, N, K, g = M2, N2, K2, g2
    w2 = synth.gen_w2t((116,), N, K, g)
    x2 = synth.gen_x((116,), M, K, "f16")
    P2 = PackedW2T(w2, N, K, g)
    y2 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    L.w2t_gemv(dev(x2), "f16", P2.q, P2.s, y2, "f32", M, N, K, g, work, work.numel())
    torch.cuda.synchronize()
    assert "slices=1 " not in L.w4a16_last_variant()
    assert_parity(to_f64(y2), oracle.w2t_gemv(x2, "f16", w2["codes"], w2["scales"], M, N, K, g),
                  "ternary split, shared workspace")
    assert int(work[:WS_HEAD].count_nonzero()) == 0   # every call left the counters at zero


@pytest.mark.parametrize("M,K,g,xdt", [(1, 1152, 128, "f16"), (8, 1152, 128, "bf16"),
                                         (3, 640, 128, "f16"), (12, 256, 128, "bf16"),
                                         (2, 1152, 64, "f16"), (4, 640, 64, "bf16"),
                                         (1, 896, 64, "f16"), (8, 1152, 64, "bf16")])
def test_multi_tile_workgroups_ragged(M, K, g, xdt):
    # Many more tiles than the GPU holds at once: each workgroup takes three
    # tiles, and 1537 tiles leave a last workgroup with a single one.
    N = 24592
    say(f"multi-tile M={M} N={N} K={K} g={g} x={xdt}")
    key = (113, M, K, g)
    w = synth.gen_w4(key, N, K, g)
    x = synth.gen_x(key, M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    P = PackedW4(w, N, K, g)
    y = P.gemv(dev(x), xdt, M)
    torch.cuda.synchronize()
    variant = L.w4a16_last_variant()
    say("  variant: " + variant)
    assert "tpw=3 " in variant
    ref = oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, K, g)
    assert_parity(to_f64(y), ref, f"multi-tile M={M} K={K}")


# ------------------------------------------------------------------ MXFP4 ---

# (N, K): one tile, ragged N (a last tile of 8 columns), K with a ragged last
# 128-k unit (K % 128 = 32, 64, 96), several tiles.
MX_SHAPES = [(8, 32), (24, 96), (40, 160), (136, 1184), (264, 4160), (4104, 640)]


@pytest.mark.parametrize("N,K", MX_SHAPES)
def test_mxfp4_pack_unpack_roundtrip_bitexact(N, K):
    say(f"mxfp4 pack N={N} K={K}")
    w = synth.gen_mx((120, N, K), N, K, e_lo=0, e_hi=254)
    P = PackedMX(w, N, K)
    q2 = torch.empty((N, K // 2), dtype=torch.uint8, device=DEV)
    s2 = torch.empty((N, K // 32), dtype=torch.uint8, device=DEV)
    L.mxfp4_unpack(P.q, P.s, q2, s2, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(q2.cpu().numpy(), w["qweight"])
    assert np.array_equal(s2.cpu().numpy(), w["scales"])


@pytest.mark.parametrize("N,K", MX_SHAPES + [(5120, 17408)])
def test_mxfp4_dequant_bitexact(N, K):
    # Every byte value (two codes, negative zero included) under scale codes
    # 0 (subnormal 2^-127) .. 252, through the GEMV's own element conversion;
    # compared bit for bit, sign of zero included.
    say(f"mxfp4 dequant N={N} K={K}")
    w = synth.gen_mx((121, N, K), N, K, e_lo=0, e_hi=252)
    q = w["qweight"].copy()
    flat = q.reshape(-1)
    flat[: min(256, flat.size)] = np.arange(min(256, flat.size), dtype=np.uint8)
    w["qweight"] = q
    P = PackedMX(w, N, K)
    out = torch.empty((N, K), dtype=torch.float32, device=DEV)
    L.mxfp4_dequant(P.q, P.s, out, N, K)
    torch.cuda.synchronize()
    ref = oracle.mx_dequant(q, w["scales"], N, K).astype(np.float32)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


MX_GEMV_CASES = [
    # (M, N, K, x dtype)
    (1, 8, 32, "f16"),
    (1, 24, 96, "bf16"),
    (3, 40, 160, "f16"),
    (1, 136, 1184, "f16"),
    (2, 136, 1184, "bf16"),
    (4, 264, 4160, "f16"),
    (8, 520, 4096, "bf16"),
    (16, 264, 896, "f16"),
    (7, 4104, 640, "f16"),
    (1, 4096, 4096, "f16"),
]


@pytest.mark.parametrize("M,N,K,xdt", MX_GEMV_CASES)
def test_mxfp4_gemv_matches_oracle(M, N, K, xdt):
    say(f"mxfp4 gemv M={M} N={N} K={K} x={xdt}")
    key = (122, M, N, K)
    w = synth.gen_mx(key, N, K)
    x = synth.gen_x(key, M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    P = PackedMX(w, N, K)
    xd = dev(x)
    y = P.gemv(xd, xdt, M, "f32")
    torch.cuda.synchronize()
    say("  variant: " + L.w4a16_last_variant())
    ref = oracle.mx_gemv(x, xdt, w["qweight"], w["scales"], M, N, K)
    assert_parity(to_f64(y), ref, f"M={M} N={N} K={K} {xdt}")
    assert_parity(to_f64(P.gemv(xd, xdt, M, "f16")), ref, "f16 out", extra_rel=2.0 ** -11)
    assert_parity(to_f64(P.gemv(xd, xdt, M, "bf16")), ref, "bf16 out", extra_rel=2.0 ** -8)


# M-tiled MXFP4 (more rows than one MFMA block): 2 to 4 row blocks, ragged N
# and K (a last unit of 32 or 64 k), with and without K slices.
MX_GEMM_CASES = [
    (17, 264, 896, "f16"),
    (24, 40, 4160, "bf16"),
    (32, 520, 1184, "f16"),
    (48, 136, 640, "bf16"),
    (64, 264, 4352, "f16"),
    (64, 4104, 640, "bf16"),
]


@pytest.mark.parametrize("M,N,K,xdt", MX_GEMM_CASES)
def test_mxfp4_gemm_matches_oracle(M, N, K, xdt):
    say(f"mxfp4 gemm M={M} N={N} K={K} x={xdt}")
    key = (127, M, N, K)
    w = synth.gen_mx(key, N, K)
    x = synth.gen_x(key, M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    P = PackedMX(w, N, K)
    xd = dev(x)
    y = P.gemv(xd, xdt, M, "f32")
    torch.cuda.synchronize()
    variant = L.w4a16_last_variant()
    say("  variant: " + variant)
    assert "w4_gemm_kernel" in variant
    ref = oracle.mx_gemv(x, xdt, w["qweight"], w["scales"], M, N, K)
    assert_parity(to_f64(y), ref, f"M={M} N={N} K={K} {xdt}")
    assert_parity(to_f64(P.gemv(xd, xdt, M, "bf16")), ref, "bf16 out", extra_rel=2.0 ** -8)


@pytest.mark.parametrize("span,M", [(36, 24), (37, 24), (90, 40)])
def test_mxfp4_gemm_scale_span_within_a_unit(span, M):
    # The tiled kernel's fold / per-step split, as in the GEMV test: row 0 of
    # x lives only on the small-scale blocks.
    N, K, hi = 72, 512, 150
    key = (128, span, M)
    w = synth.gen_mx(key, N, K)
    sc = np.empty((N, K // 32), dtype=np.uint8)
    for b in range(K // 32):
        sc[:, b] = hi if b % 4 in (0, 3) else hi - span
    w["scales"] = sc
    x = synth.gen_x(key, M, K, "f16")
    small = np.array([(k // 32) % 4 in (1, 2) for k in range(K)])
    x[0, ~small] = 0
    P = PackedMX(w, N, K)
    y = P.gemv(dev(x), "f16", M)
    torch.cuda.synchronize()
    assert "w4_gemm_kernel" in L.w4a16_last_variant()
    ref = oracle.mx_gemv(x, "f16", w["qweight"], w["scales"], M, N, K)
    assert_parity(to_f64(y)[:1], ref[:1], f"span {span}, small blocks only")
    assert_parity(to_f64(y), ref, f"span {span}")


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_mxfp4_gemv_wide_scale_range(xdt):
    # Scale codes 0..200 (2^-127 .. 2^73): each block's fp32 sum is scaled on
    # its own, so no conversion of a scaled element has to fit fp16.
    M, N, K = 4, 264, 2048
    key = (123, M, N, K)
    w = synth.gen_mx(key, N, K, e_lo=0, e_hi=200)
    x = synth.gen_x(key, M, K, xdt)
    P = PackedMX(w, N, K)
    y = P.gemv(dev(x), xdt, M)
    torch.cuda.synchronize()
    assert_parity(to_f64(y), oracle.mx_gemv(x, xdt, w["qweight"], w["scales"], M, N, K), "wide scales")


@pytest.mark.parametrize("span,xdt", [(36, "f16"), (37, "f16"), (36, "bf16"), (60, "bf16")])
def test_mxfp4_scale_span_within_a_unit(span, xdt):
    # Within each 128-k unit a column's four blocks carry codes
    # [hi, hi - span, hi - span, hi].  Span 36 is the widest the kernel folds
    # into the element conversion (the small blocks' elements land exactly on
    # fp16's smallest subnormal step); wider spans take the exact per-step
    # path.  Row 0 of x is nonzero only on the small-scale blocks, so any
    # underflow there would be the whole result; row 1 is dense.
    M, N, K, hi = 2, 64, 512, 150
    key = (126, span)
    w = synth.gen_mx(key, N, K)
    sc = np.empty((N, K // 32), dtype=np.uint8)
    for b in range(K // 32):
        sc[:, b] = hi if b % 4 in (0, 3) else hi - span
    w["scales"] = sc
    x = synth.gen_x(key, M, K, xdt)
    small = np.array([(k // 32) % 4 in (1, 2) for k in range(K)])
    x[0, ~small] = 0
    P = PackedMX(w, N, K)
    y = P.gemv(dev(x), xdt, M)
    torch.cuda.synchronize()
    ref = oracle.mx_gemv(x, xdt, w["qweight"], w["scales"], M, N, K)
    assert_parity(to_f64(y)[:1], ref[:1], f"span {span}, small blocks only")
    assert_parity(to_f64(y), ref, f"span {span}")


def test_mxfp4_split_and_multi_tile_launches():
    # A narrow, long shape runs K slices (workspace and merge); a wide one
    # runs three tiles per workgroup.
    for (M, N, K) in [(4, 520, 17408), (2, 24592, 640)]:
        key = (124, M, N, K)
        w = synth.gen_mx(key, N, K)
        x = synth.gen_x(key, M, K, "f16")
        P = PackedMX(w, N, K)
        y = P.gemv(dev(x), "f16", M)
        torch.cuda.synchronize()
        variant = L.w4a16_last_variant()
        say(f"  mxfp4 M={M} N={N} K={K}: {variant}")
        assert ("slices=1 " not in variant) if N == 520 else ("tpw=3 " in variant)
        assert_parity(to_f64(y), oracle.mx_gemv(x, "f16", w["qweight"], w["scales"], M, N, K),
                      f"mxfp4 M={M} N={N} K={K}")


@pytest.mark.parametrize("name,K,N", [("qkv", 5120, 7168), ("gate_up", 5120, 34816),
                                      ("down", 17408, 5120)])
@pytest.mark.parametrize("M,xdt", [(1, "f16"), (8, "bf16"), (64, "f16")])
def test_mxfp4_full_size_sampled_columns(name, K, N, M, xdt):
    say(f"mxfp4 full {name} K={K} N={N} M={M} x={xdt}")
    key = (125, K, N, M)
    w = synth.gen_mx(key, N, K)
    x = synth.gen_x(key, M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    P = PackedMX(w, N, K)
    y = to_f64(P.gemv(dev(x), xdt, M))
    cols = sample_cols(N, np.random.default_rng(N + M + 7))
    ref = oracle.mx_gemv(x, xdt, w["qweight"], w["scales"], M, N, K, cols=cols)
    assert_parity(y[:, cols], ref, "mxfp4 " + name)


@pytest.mark.parametrize("name,K,N", [("qkv", 5120, 7168), ("gate_up", 5120, 34816),
                                      ("down", 17408, 5120)])
@pytest.mark.parametrize("M,dt", [(1, "f16"), (8, "bf16")])
def test_w16a16_full_size_sampled_columns(name, K, N, M, dt):
    # The W16A16 layer at the shapes and launch configuration the bench times.
    say(f"w16 full {name} K={K} N={N} M={M} {dt}")
    key = (132, K, N, M)
    w = synth.gen_w16(key, N, K, dt)
    x = synth.gen_x(key, M, K, dt)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    wsb = L.w16a16_workspace_bytes(M, N, K)
    ws = workspace_bytes(wsb) if wsb else None
    L.w16a16_gemv(dev(x), dev(w), dt, y, "f32", M, N, K, ws, wsb)
    torch.cuda.synchronize()
    cols = sample_cols(N, np.random.default_rng(N + M + 11))
    ref = oracle.w16_gemv(x, dt, w, M, N, K, cols=cols)
    assert_parity(to_f64(y)[:, cols], ref, "w16 " + name)


# ----------------------------------------------- full 27B-class shapes, sampled ---

FULL = [("qkv", 5120, 7168), ("o_proj", 5120, 5120), ("gate_up", 5120, 34816),
        ("down", 17408, 5120), ("lm_head", 5120, 152064)]


def sample_cols(N, rng, n=192):
    cols = set(rng.choice(N, size=min(n, N), replace=False).tolist())
    cols |= {0, 15, 16, N // 2, N - 17, N - 16, N - 1}
    return np.array(sorted(cols), dtype=np.int64)


@pytest.mark.parametrize("name,K,N", FULL)
@pytest.mark.parametrize("M,xdt", [(1, "f16"), (4, "bf16"), (8, "f16")])
def test_full_size_sampled_columns(name, K, N, M, xdt):
    say(f"full {name} K={K} N={N} M={M} x={xdt}")
    g = 128
    key = (112, K, N, M)
    w = synth.gen_w4(key, N, K, g)
    x = synth.gen_x(key, M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    P = PackedW4(w, N, K, g)
    y = to_f64(P.gemv(dev(x), xdt, M))
    cols = sample_cols(N, np.random.default_rng(N + M))
    ref = oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, K, g, cols=cols)
    assert_parity(y[:, cols], ref, name)


_LM_HEAD = {}


def _lm_head(g):
    """The lm_head-like matrix (N = 152064, K = 5120) at group g, generated
    and packed once per test module."""
    if g not in _LM_HEAD:
        _LM_HEAD.clear()
        N, K = 152064, 5120
        w = synth.gen_w4((115, g), N, K, g)
        _LM_HEAD[g] = (w, PackedW4(w, N, K, g))
    return _LM_HEAD[g]


@pytest.mark.parametrize("g,M", [(64, m) for m in (1, 2, 3, 4, 6, 8)] +
                         [(128, m) for m in (2, 3, 6)])
def test_lm_head_sampled_columns(g, M):
    # The skinny sweep's lm_head-like shape at every row count it measures:
    # three 16-column tiles per workgroup (9504 tiles), x staged unit by unit
    # up to 4 rows.  Columns include the tile and workgroup edges at both ends.
    N, K = 152064, 5120
    say(f"lm_head g={g} M={M}")
    w, P = _lm_head(g)
    x = synth.gen_x((115, g, M), M, K, "f16")
    y = to_f64(P.gemv(dev(x), "f16", M))
    variant = L.w4a16_last_variant()
    say("  variant: " + variant)
    assert "w4_gemv_kernel" in variant and "tpw=3" in variant and "slices=1 " in variant
    assert ("px=1" in variant) == (M <= 4)
    rng = np.random.default_rng(g + M)
    cols = set(sample_cols(N, rng, n=160).tolist())
    cols |= {31, 32, 47, 48, 49, 95, 96, N - 49, N - 48, N - 47, N - 33, N - 32}
    cols = np.array(sorted(cols), dtype=np.int64)
    ref = oracle.w4_gemv(x, "f16", w["qweight"], w["scales"], w["zeros"], M, N, K, g, cols=cols)
    assert_parity(y[:, cols], ref, f"lm_head g{g} M{M}")


# Three tiles per workgroup on layers of many tiles (at least six per CU,
# no K split, up to 4 units per wave): 1537 tiles leave the last workgroup
# one; each compiled group size, ragged K (a last unit of 128 k), and waves
# without units (K = 512: 2 units for 8 waves).
@pytest.mark.parametrize("M,K,g,xdt", [(1, 2560, 128, "f16"), (4, 4352, 64, "bf16"), (8, 3840, 256, "f16"),
                                       (3, 2432, 128, "bf16"), (2, 512, 128, "f16")])
def test_w2t_three_tile_workgroups(M, K, g, xdt):
    N = 24592
    say(f"w2t three tiles M={M} K={K} g={g} x={xdt}")
    key = (162, M, K, g)
    w = synth.gen_w2t(key, N, K, g)
    x = synth.gen_x(key, M, K, xdt, outlier_frac=0.01 if xdt == "bf16" else 0.0)
    y = to_f64(PackedW2T(w, N, K, g).gemv(dev(x), xdt, M))
    variant = L.w4a16_last_variant()
    say("  variant: " + variant)
    assert "tpw=3 " in variant
    cols = sample_cols(N, np.random.default_rng(K + g), n=256)
    ref = oracle.w2t_gemv(x, xdt, w["codes"], w["scales"], M, N, K, g, cols=cols)
    assert_parity(y[:, cols], ref, f"w2t three tiles M={M} K={K} g={g}")


@pytest.mark.parametrize("K,N", [(5120, 7168), (5120, 34816), (17408, 5120)])
@pytest.mark.parametrize("M", [1, 4, 8])
def test_w2t_full_size_sampled_columns(K, N, M):
    say(f"w2t full K={K} N={N} M={M}")
    g = 128
    key = (113, K, N, M)
    w = synth.gen_w2t(key, N, K, g)
    x = synth.gen_x(key, M, K, "f16")
    P = PackedW2T(w, N, K, g)
    y = to_f64(P.gemv(dev(x), "f16", M))
    cols = sample_cols(N, np.random.default_rng(N + M))
    ref = oracle.w2t_gemv(x, "f16", w["codes"], w["scales"], M, N, K, g, cols=cols)
    assert_parity(y[:, cols], ref, "w2t full")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 6, 8])
@pytest.mark.parametrize("g", [64, 128])
@pytest.mark.parametrize("KN", [4096, 5120, 8192])
def test_skinny_sweep_sampled(M, g, KN):
    say(f"sweep M={M} g={g} K=N={KN}")
    key = (114, M, g, KN)
    w = synth.gen_w4(key, KN, KN, g)
    x = synth.gen_x(key, M, KN, "f16")
    P = PackedW4(w, KN, KN, g)
    y = to_f64(P.gemv(dev(x), "f16", M))
    cols = sample_cols(KN, np.random.default_rng(KN + M + g), n=96)
    ref = oracle.w4_gemv(x, "f16", w["qweight"], w["scales"], w["zeros"], M, KN, KN, g, cols=cols)
    assert_parity(y[:, cols], ref, "sweep")


def test_gpu_rejects_bad_arguments_without_launching():
    good = empty_bytes(1 << 16)
    with pytest.raises(L.W4A16Error) as e:
        L.w4a16_gemv(good, "f16", good, good, good, good, "f32", 0, 16, 128, 128)
    assert e.value.status == -2
    with pytest.raises(L.W4A16Error) as e:
        L.w4a16_gemv(good.data_ptr() + 2, "f16", good, good, good, good, "f32", 1, 16, 128, 128)
    assert e.value.status == -3


# ------------------------------------------------- seeded random shapes ---

def _random_cases(seed, n, max_m, groups):
    """n seeded (M, N, K, g, x dtype, y dtype) draws covering the planners'
    choices: rows up to max_m, N up to ~2000 in steps of 8 (ragged tiles),
    K a multiple of the group, often ragged against the 128-k unit."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        g = int(rng.choice(groups))
        M = int(rng.integers(1, max_m + 1))
        N = 8 * int(rng.integers(1, 250))
        K = g * int(rng.integers(1, max(2, 3200 // g)))
        out.append((M, N, K, g, str(rng.choice(["f16", "bf16"])), str(rng.choice(["f32", "f16", "bf16"]))))
    return out


@pytest.mark.parametrize("M,N,K,g,xdt,ydt", _random_cases(2024, 16, 64, [32, 64, 128, 256]))
def test_w4_random_shapes_match_oracle(M, N, K, g, xdt, ydt):
    say(f"w4 random M={M} N={N} K={K} g={g} x={xdt} y={ydt}")
    key = (140, M, N, K, g)
    w = synth.gen_w4(key, N, K, g)
    x = synth.gen_x(key, M, K, xdt)
    y = PackedW4(w, N, K, g).gemv(dev(x), xdt, M, ydt)
    torch.cuda.synchronize()
    say("  variant: " + L.w4a16_last_variant())
    ref = oracle.w4_gemv(x, xdt, w["qweight"], w["scales"], w["zeros"], M, N, K, g)
    assert_parity(to_f64(y), ref, "w4 random", extra_rel=_ROUND[ydt])


@pytest.mark.parametrize("M,N,K,g,xdt,ydt", _random_cases(2025, 10, 64, [32]))
def test_mxfp4_random_shapes_match_oracle(M, N, K, g, xdt, ydt):
    say(f"mxfp4 random M={M} N={N} K={K} x={xdt} y={ydt}")
    key = (141, M, N, K)
    w = synth.gen_mx(key, N, K)
    x = synth.gen_x(key, M, K, xdt)
    y = PackedMX(w, N, K).gemv(dev(x), xdt, M, ydt)
    torch.cuda.synchronize()
    say("  variant: " + L.w4a16_last_variant())
    ref = oracle.mx_gemv(x, xdt, w["qweight"], w["scales"], M, N, K)
    assert_parity(to_f64(y), ref, "mxfp4 random", extra_rel=_ROUND[ydt])


@pytest.mark.parametrize("M,N,K,g,xdt,ydt", _random_cases(2026, 10, 64, [8]))
def test_w16a16_random_shapes_match_oracle(M, N, K, g, xdt, ydt):
    say(f"w16 random M={M} N={N} K={K} {xdt} y={ydt}")
    key = (142, M, N, K)
    w = synth.gen_w16(key, N, K, xdt)
    x = synth.gen_x(key, M, K, xdt)
    y = torch.empty((M, N), dtype=_TORCH_DT[ydt], device=DEV)
    wsb = L.w16a16_workspace_bytes(M, N, K)
    ws = workspace_bytes(wsb) if wsb else None
    L.w16a16_gemv(dev(x), dev(w), xdt, y, ydt, M, N, K, ws, wsb)
    torch.cuda.synchronize()
    ref = oracle.w16_gemv(x, xdt, w, M, N, K)
    assert_parity(to_f64(y), ref, "w16 random", extra_rel=_ROUND[ydt])


@pytest.mark.parametrize("M,N,K,g,xdt,ydt", _random_cases(2027, 10, 16, [32, 64, 128, 256]))
def test_w2t_random_shapes_match_oracle(M, N, K, g, xdt, ydt):
    K = max(K, 16) // 16 * 16 if K % 16 else K          # the ternary contract: K % 16 == 0
    say(f"w2t random M={M} N={N} K={K} g={g} x={xdt} y={ydt}")
    key = (143, M, N, K, g)
    w = synth.gen_w2t(key, N, K, g)
    x = synth.gen_x(key, M, K, xdt)
    y = PackedW2T(w, N, K, g).gemv(dev(x), xdt, M, ydt)
    torch.cuda.synchronize()
    say("  variant: " + L.w4a16_last_variant())
    ref = oracle.w2t_gemv(x, xdt, w["codes"], w["scales"], M, N, K, g)
    assert_parity(to_f64(y), ref, "w2t random", extra_rel=_ROUND[ydt])


# ------------------------------------------------------------ read probe ---

@pytest.mark.parametrize("n16", [4096 * 37 + 3, 1000])
def test_bw_probe_reads_each_word_once(n16):
    # Each workgroup folds its own contiguous share of the buffer with XOR;
    # its sink entry is the low 16 bits of that fold (a ragged last share,
    # and zero for workgroups whose share is empty).
    say(f"bw probe n16={n16}")
    rng = np.random.default_rng(160 + n16)
    host = rng.integers(0, 2 ** 32, size=n16 * 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    nsink = L.w4a16_bw_probe_sink_floats()
    sink = torch.full((nsink,), -1.0, dtype=torch.float32, device=DEV)
    L.w4a16_bw_probe(buf, n16 * 16, sink)
    torch.cuda.synchronize()
    per = -(-n16 // nsink)
    padded = np.zeros(nsink * per * 4, dtype=np.uint32)
    padded[:host.size] = host
    expect = np.bitwise_xor.reduce(padded.reshape(nsink, per * 4), axis=1) & 0xFFFF
    assert np.array_equal(sink.cpu().numpy(), expect.astype(np.float32))
