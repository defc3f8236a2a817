"""Pins for the CPU oracle, independent of the oracle's own code.

Each test checks the oracle against something other than itself: a library
decode of every fp16/bf16 bit pattern, exact rational arithmetic on tiny
inputs packed by a different method (hex-digit strings rather than shifts),
closed forms, and identities of the definition w = (q - z) * s.  A dropped
zero point, a flipped sign, a transposed operand, a wrong nibble order or a
wrong group index each fails at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


# ---------------------------------------------------------------- helpers ---

def pack_nibbles_hex(vals):
    """8 values 0..15 -> int32 word whose nibble i holds vals[i], built from a
    hex string (most significant digit first) instead of shifts."""
    assert len(vals) == 8
    word = int("".join("%x" % v for v in reversed(vals)), 16)
    return np.array([word], dtype=np.uint32).view(np.int32)[0]


def pack_codes_binary(vals):
    """16 codes 0..3 -> int32 word whose 2-bit field i holds vals[i], built from
    a binary string."""
    assert len(vals) == 16
    word = int("".join(format(v, "02b") for v in reversed(vals)), 2)
    return np.array([word], dtype=np.uint32).view(np.int32)[0]


def canon_w4(q, z, s_bits):
    """Plain matrices q[K][N], z[G][N] (ints), s_bits[G][N] (fp16 bits) ->
    canonical packed arrays."""
    K, N = q.shape
    G = z.shape[0]
    qweight = np.array([[pack_nibbles_hex([int(q[8 * j + i, n]) for i in range(8)])
                         for j in range(K // 8)] for n in range(N)], dtype=np.int32)
    zeros = np.array([[pack_nibbles_hex([int(z[g, 8 * j + i]) for i in range(8)])
                       for j in range(N // 8)] for g in range(G)], dtype=np.int32)
    return qweight, np.asarray(s_bits, dtype=np.uint16), zeros


def frac_f16(bits):
    return Fraction(float(np.array([bits], dtype=np.uint16).view(np.float16)[0]))


def frac_bf16(bits):
    f32 = np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(f32))


def exact_w4_y(xbits, x_dtype, q, z, s_bits, group):
    dec = frac_bf16 if x_dtype == "bf16" else frac_f16
    M, K = xbits.shape
    N = q.shape[1]
    xs = [[dec(xbits[m, k]) for k in range(K)] for m in range(M)]
    ws = [[(int(q[k, n]) - int(z[k // group, n])) * frac_f16(s_bits[k // group, n])
           for n in range(N)] for k in range(K)]
    return [[sum(xs[m][k] * ws[k][n] for k in range(K)) for n in range(N)] for m in range(M)], xs, ws


def random_plain(rng, K, N, group):
    G = K // group
    q = rng.integers(0, 16, size=(K, N))
    z = rng.integers(0, 16, size=(G, N))
    s_bits = synth.f64_to_f16_bits(rng.uniform(0.002, 0.02, size=(G, N)))
    return q, z, s_bits


# ------------------------------------------------------------ float decode ---

def test_f16_decode_matches_numpy_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_matches_float32_upper_half_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32)
    ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ------------------------------------------------- exact rational brute force ---

@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("K,group", [(64, 64), (128, 64), (256, 128), (128, 32)])
@pytest.mark.parametrize("x_dtype", ["f16", "bf16"])
def test_w4_matches_exact_rational(seed, K, group, x_dtype):
    rng = np.random.default_rng(1000 + seed)
    M = 1 + seed % 3
    N = 8 * (1 + seed % 2)
    q, z, s_bits = random_plain(rng, K, N, group)
    xv = rng.standard_normal((M, K)) * (1 + 20 * (rng.random((M, K)) < 0.02))
    xbits = synth.f64_to_bf16_bits(xv) if x_dtype == "bf16" else synth.f64_to_f16_bits(xv)
    qw, s, zw = canon_w4(q, z, s_bits)

    exact, xs, ws = exact_w4_y(xbits, x_dtype, q, z, s_bits, group)
    got = oracle.w4_gemv(xbits, x_dtype, qw, s, zw, M, N, K, group)
    for m in range(M):
        for n in range(N):
            # fp64 sequential summation bound: K * 2^-53 * sum |x w| (each
            # product is exact, only the additions round).
            bound = K * 2.0 ** -53 * float(sum(abs(xs[m][k] * ws[k][n]) for k in range(K)))
            assert abs(got[m, n] - float(exact[m][n])) <= bound + 1e-300

    W = oracle.w4_dequant(qw, s, zw, N, K, group)
    for k in range(K):
        for n in range(N):
            assert W[k, n] == float(ws[k][n])   # dequantization is exact in fp64


@pytest.mark.parametrize("seed", range(4))
def test_w2t_matches_exact_rational(seed):
    rng = np.random.default_rng(2000 + seed)
    M, N, K, group = 2, 5, 256, 128
    c = rng.choice([0, 1, 2], size=(K, N), p=[0.25, 0.5, 0.25])
    s_bits = synth.f64_to_f16_bits(rng.uniform(0.01, 0.05, size=(K // group, N)))
    codes = np.array([[pack_codes_binary([int(c[16 * j + i, n]) for i in range(16)])
                       for j in range(K // 16)] for n in range(N)], dtype=np.int32)
    xbits = synth.f64_to_f16_bits(rng.standard_normal((M, K)))
    got = oracle.w2t_gemv(xbits, "f16", codes, s_bits, M, N, K, group)
    for m in range(M):
        for n in range(N):
            terms = [frac_f16(xbits[m, k]) * (int(c[k, n]) - 1) * frac_f16(s_bits[k // group, n])
                     for k in range(K)]
            bound = K * 2.0 ** -53 * float(sum(abs(t) for t in terms))
            assert abs(got[m, n] - float(sum(terms))) <= bound + 1e-300
    W = oracle.w2t_dequant(codes, s_bits, N, K, group)
    for k in range(K):
        for n in range(N):
            assert W[k, n] == float((int(c[k, n]) - 1) * frac_f16(s_bits[k // group, n]))


# ----------------------------------------------------------- closed forms ---

def test_w4_closed_form_sign_and_group_index():
    # x = 1, q = 15, z = 0 in group 0; q = 0, z = 15 in group 1; scale 2^-g.
    # y = 128*15*1 + 128*(-15)*0.5 = 960 exactly.  A flipped sign of (q - z)
    # gives -960, a dropped zero point gives 1920, a wrong group index for the
    # scale or zero changes the value.
    K, N, group = 256, 8, 128
    q = np.zeros((K, N), dtype=int)
    q[:128] = 15
    z = np.zeros((2, N), dtype=int)
    z[1] = 15
    s_bits = np.array([[0x3C00] * N, [0x3800] * N], dtype=np.uint16)  # 1.0, 0.5
    qw, s, zw = canon_w4(q, z, s_bits)
    x = np.full((1, K), 0x3C00, dtype=np.uint16)
    y = oracle.w4_gemv(x, "f16", qw, s, zw, 1, N, K, group)
    assert np.all(y == 960.0)


def test_w4_zero_point_cancels_exactly():
    rng = np.random.default_rng(7)
    K, N, group = 512, 16, 128
    q, _, s_bits = random_plain(rng, K, N, group)
    # q = z everywhere: every column's q is constant within each group.
    G = K // group
    z = rng.integers(0, 16, size=(G, N))
    q = np.repeat(z, group, axis=0)
    qw, s, zw = canon_w4(q, z, s_bits)
    x = synth.f64_to_f16_bits(rng.standard_normal((3, K)))
    y = oracle.w4_gemv(x, "f16", qw, s, zw, 3, N, K, group)
    assert np.all(y == 0.0)


def test_w4_scale_doubling_doubles_output_exactly():
    w = synth.gen_w4((90, 1), 64, 1024, 128)
    x = synth.gen_x((90, 1), 4, 1024, "f16")
    y1 = oracle.w4_gemv(x, "f16", w["qweight"], w["scales"], w["zeros"], 4, 64, 1024, 128)
    s2 = (w["scales"].view(np.float16).astype(np.float64) * 2).astype(np.float16).view(np.uint16)
    y2 = oracle.w4_gemv(x, "f16", w["qweight"], s2, w["zeros"], 4, 64, 1024, 128)
    assert np.array_equal(y2, 2 * y1)
    # alpha = 3 on scales j/1024 (j = 2..20), so 3s is still exact in fp16;
    # the outputs then agree to fp64 summation rounding.
    j = np.random.default_rng(3).integers(2, 21, size=w["scales"].shape)
    s1 = synth.f64_to_f16_bits(j / 1024.0)
    s3 = synth.f64_to_f16_bits(3 * j / 1024.0)
    y1 = oracle.w4_gemv(x, "f16", w["qweight"], s1, w["zeros"], 4, 64, 1024, 128)
    y3 = oracle.w4_gemv(x, "f16", w["qweight"], s3, w["zeros"], 4, 64, 1024, 128)
    assert np.max(np.abs(y3 - 3 * y1)) <= 1e-13 * np.max(np.abs(y3))


def test_w4_one_hot_x_selects_dequantized_rows():
    # x = e_k picks row k of W = (q - z) * s, which the test computes itself
    # from its plain matrices (pins nibble order, group and zero indexing).
    rng = np.random.default_rng(11)
    K, N, group = 256, 16, 64
    q, z, s_bits = random_plain(rng, K, N, group)
    qw, s, zw = canon_w4(q, z, s_bits)
    sf = s_bits.view(np.float16).astype(np.float64)
    ks = list(range(0, 70)) + [127, 128, 129, 191, 192, 255]
    x = np.zeros((len(ks), K), dtype=np.uint16)
    for r, k in enumerate(ks):
        x[r, k] = 0x3C00
    y = oracle.w4_gemv(x, "f16", qw, s, zw, len(ks), N, K, group)
    for r, k in enumerate(ks):
        expect = (q[k] - z[k // group]) * sf[k // group]
        assert np.array_equal(y[r], expect)


def test_w2t_all_ones_counts_plus_minus():
    rng = np.random.default_rng(5)
    N, K, group = 24, 512, 128
    c = rng.choice([0, 1, 2], size=(K, N), p=[0.25, 0.5, 0.25])
    codes = np.array([[pack_codes_binary([int(c[16 * j + i, n]) for i in range(16)])
                       for j in range(K // 16)] for n in range(N)], dtype=np.int32)
    s = np.full((K // group, N), 0x3C00, dtype=np.uint16)
    x = np.full((1, K), 0x3C00, dtype=np.uint16)
    y = oracle.w2t_gemv(x, "f16", codes, s, 1, N, K, group)
    expect = (c == 2).sum(axis=0) - (c == 0).sum(axis=0)
    assert np.array_equal(y[0], expect.astype(np.float64))


def test_w2t_rejects_code_three():
    codes = np.zeros((8, 2), dtype=np.int32)
    codes[3, 1] = pack_codes_binary([1] * 15 + [3])
    s = np.full((1, 8), 0x3C00, dtype=np.uint16)
    x = np.full((1, 32), 0x3C00, dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.w2t_gemv(x, "f16", codes, s, 1, 8, 32, 32)
    with pytest.raises(ValueError):
        oracle.w2t_dequant(codes, s, 8, 32, 32)


# ---------------------------------------- agreement with a textbook routine ---

@pytest.mark.parametrize("x_dtype", ["f16", "bf16"])
def test_w4_matches_numpy_matmul_of_dequantized(x_dtype):
    M, N, K, group = 4, 128, 2048, 128
    w = synth.gen_w4((91, 2), N, K, group)
    x = synth.gen_x((91, 2), M, K, x_dtype, outlier_frac=0.01 if x_dtype == "bf16" else 0.0)
    W = oracle.w4_dequant(w["qweight"], w["scales"], w["zeros"], N, K, group)
    if x_dtype == "f16":
        xf = x.view(np.float16).astype(np.float64)
    else:
        xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = xf @ W
    got = oracle.w4_gemv(x, x_dtype, w["qweight"], w["scales"], w["zeros"], M, N, K, group)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
    cols = [0, 5, 63, 64, 127]
    got_c = oracle.w4_gemv(x, x_dtype, w["qweight"], w["scales"], w["zeros"], M, N, K, group,
                           cols=cols)
    assert np.array_equal(got_c, got[:, cols])


def test_w2t_matches_numpy_matmul_of_dequantized():
    M, N, K, group = 3, 40, 1024, 128
    w = synth.gen_w2t((92, 1), N, K, group)
    x = synth.gen_x((92, 1), M, K, "f16")
    W = oracle.w2t_dequant(w["codes"], w["scales"], N, K, group)
    ref = x.view(np.float16).astype(np.float64) @ W
    got = oracle.w2t_gemv(x, "f16", w["codes"], w["scales"], M, N, K, group)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
    got_c = oracle.w2t_gemv(x, "f16", w["codes"], w["scales"], M, N, K, group, cols=[3, 39])
    assert np.array_equal(got_c, got[:, [3, 39]])


def test_oracle_rejects_bad_shapes():
    w = synth.gen_w4((93,), 16, 256, 128)
    x = synth.gen_x((93,), 1, 256)
    with pytest.raises(ValueError):   # group does not divide K
        oracle.w4_gemv(x, "f16", w["qweight"], w["scales"], w["zeros"], 1, 16, 256, 96)
    with pytest.raises(ValueError):   # column out of range
        oracle.w4_gemv(x, "f16", w["qweight"], w["scales"], w["zeros"], 1, 16, 256, 128, cols=[16])


# ------------------------------------------------------------ 16-bit weights ---

@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_w16_matches_exact_rational(seed, dtype):
    # y[m][n] = sum_k x[m][k] w[n][k], every value decoded through numpy
    # (fp16, or bf16 as the upper half of a float32) into exact fractions.
    rng = np.random.default_rng(1300 + seed)
    M, N, K = 1 + seed, 8 + 3 * seed, 32 + 40 * seed
    to_bits = synth.f64_to_bf16_bits if dtype == "bf16" else synth.f64_to_f16_bits
    dec = frac_bf16 if dtype == "bf16" else frac_f16
    xbits = to_bits(rng.standard_normal((M, K)))
    wbits = to_bits(rng.standard_normal((N, K)) * 0.02)
    got = oracle.w16_gemv(xbits, dtype, wbits, M, N, K)
    for m in range(M):
        for n in range(N):
            prods = [dec(xbits[m, k]) * dec(wbits[n, k]) for k in range(K)]
            bound = K * 2.0 ** -53 * float(sum(abs(p) for p in prods))
            assert abs(got[m, n] - float(sum(prods))) <= bound + 1e-300


def test_w16_one_hot_rows_select_weight_columns():
    # x = e_k reproduces w[:, k] exactly, and only the listed columns are
    # computed by the sampled variant.
    N, K = 24, 96
    wbits = synth.gen_w16((9,), N, K, "f16")
    ks = [0, 1, 31, 32, 95]
    x = np.zeros((len(ks), K), dtype=np.uint16)
    for r, k in enumerate(ks):
        x[r, k] = 0x3C00                     # fp16 1.0
    y = oracle.w16_gemv(x, "f16", wbits, len(ks), N, K)
    wf = wbits.view(np.float16).astype(np.float64)
    for r, k in enumerate(ks):
        assert np.array_equal(y[r], wf[:, k])
    cols = np.array([23, 0, 7], dtype=np.int64)
    assert np.array_equal(oracle.w16_gemv(x, "f16", wbits, len(ks), N, K, cols=cols), y[:, cols])


# ------------------------------------------------------------------ MXFP4 ---

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


def e2m1_table():
    """code -> value from the cited fixture (tests/golden/mxfp4_e2m1_values.txt)."""
    out = {}
    with open(f"{GOLDEN}/mxfp4_e2m1_values.txt") as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                code, bits, val = line.split()
                assert int(bits, 2) == int(code)
                out[int(code)] = float(val)
    assert sorted(out) == list(range(16))
    return out


def e8m0_torch(codes):
    """E8M0 scale codes decoded by torch's own float8_e8m0fnu type."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e8m0fnu).to(torch.float32).double().numpy()


def unpack_fp4_bytes(qweight):
    """[N][K/2] bytes -> [N][K] codes, by integer division rather than masks:
    the even element is byte % 16, the odd one byte // 16."""
    q = qweight.astype(np.int64)
    out = np.empty((q.shape[0], 2 * q.shape[1]), dtype=np.int64)
    out[:, 0::2] = q % 16
    out[:, 1::2] = q // 16
    return out


def test_e2m1_decode_matches_the_spec_table_including_negative_zero():
    table = e2m1_table()
    for code, val in table.items():
        got = oracle.e2m1_to_f64(code)
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)


def test_e8m0_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = e8m0_torch(codes)
    got = np.array([oracle.e8m0_to_f64(c) for c in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127


def test_mx_dequant_matches_table_times_torch_scale():
    N, K = 6, 160
    w = synth.gen_mx((21,), N, K, e_lo=0, e_hi=254)
    got = oracle.mx_dequant(w["qweight"], w["scales"], N, K)
    table = e2m1_table()
    codes = unpack_fp4_bytes(w["qweight"])
    sc = e8m0_torch(w["scales"])
    for n in range(N):
        for k in range(K):
            assert got[n, k] == table[codes[n, k]] * sc[n, k // 32], (n, k)


@pytest.mark.parametrize("seed,x_dtype", [(0, "f16"), (1, "bf16"), (2, "f16")])
def test_mx_matches_exact_rational(seed, x_dtype):
    # Small-integer x (exact in fp16 and bf16) and scales 2^-5 .. 2^-2 keep
    # every partial sum a multiple of 2^-6 below 2^20, so the fp64 sum is
    # exact and must equal the rational one.
    rng = np.random.default_rng(1400 + seed)
    M, N, K = 1 + 2 * seed, 5 + seed, 64 + 96 * seed
    xi = rng.integers(-8, 9, size=(M, K))
    to_bits = synth.f64_to_bf16_bits if x_dtype == "bf16" else synth.f64_to_f16_bits
    xbits = to_bits(xi.astype(np.float64))
    w = synth.gen_mx((22, seed), N, K, e_lo=122, e_hi=125)
    table = {c: Fraction(v) for c, v in e2m1_table().items()}
    codes = unpack_fp4_bytes(w["qweight"])
    sc = [[Fraction(float(v)) for v in row] for row in e8m0_torch(w["scales"])]
    got = oracle.mx_gemv(xbits, x_dtype, w["qweight"], w["scales"], M, N, K)
    for m in range(M):
        for n in range(N):
            exact = sum(int(xi[m, k]) * table[codes[n, k]] * sc[n][k // 32] for k in range(K))
            assert Fraction(got[m, n]) == exact, (m, n)


def test_mx_one_hot_x_selects_nibble_and_block():
    # x = e_k picks w[n][k]: even k from the low nibble, odd k from the high
    # one, and the scale of block k // 32.
    N, K = 9, 128
    w = synth.gen_mx((23,), N, K, e_lo=110, e_hi=140)
    ks = [0, 1, 30, 31, 32, 33, 95, 127]
    x = np.zeros((len(ks), K), dtype=np.uint16)
    for r, k in enumerate(ks):
        x[r, k] = 0x3C00                     # fp16 1.0
    y = oracle.mx_gemv(x, "f16", w["qweight"], w["scales"], len(ks), N, K)
    table = e2m1_table()
    sc = e8m0_torch(w["scales"])
    for r, k in enumerate(ks):
        byte = w["qweight"][:, k // 2].astype(np.int64)
        code = (byte >> 4) if k % 2 else (byte & 15)
        want = np.array([table[int(c)] for c in code]) * sc[:, k // 32]
        assert np.array_equal(y[r], want), k
    cols = np.array([8, 0, 3], dtype=np.int64)
    assert np.array_equal(oracle.mx_gemv(x, "f16", w["qweight"], w["scales"], len(ks), N, K,
                                         cols=cols), y[:, cols])


def test_mx_scale_code_plus_one_doubles_output_exactly():
    M, N, K = 3, 7, 192
    w = synth.gen_mx((24,), N, K)
    x = synth.gen_x((24,), M, K, "bf16")
    y1 = oracle.mx_gemv(x, "bf16", w["qweight"], w["scales"], M, N, K)
    y2 = oracle.mx_gemv(x, "bf16", w["qweight"], w["scales"] + np.uint8(1), M, N, K)
    assert np.array_equal(y2, 2.0 * y1)


def test_mx_nan_scale_poisons_only_its_column():
    M, N, K = 2, 5, 64
    w = synth.gen_mx((25,), N, K)
    s = w["scales"].copy()
    s[3, 1] = 255
    x = synth.gen_x((25,), M, K, "f16")
    y = oracle.mx_gemv(x, "f16", w["qweight"], s, M, N, K)
    assert np.isnan(y[:, 3]).all()
    assert np.isfinite(np.delete(y, 3, axis=1)).all()


def test_mx_rejects_k_not_multiple_of_32():
    with pytest.raises(Exception):
        oracle.mx_gemv(np.zeros((1, 48), np.uint16), "f16", np.zeros((1, 24), np.uint8),
                       np.zeros((1, 1), np.uint8), 1, 1, 48)
