"""CPU checks of the C ABI: the library loads, exports every function the
header declares, and its host-side logic (size queries, argument checks,
dispatch sizing) behaves as documented.  Nothing here launches a kernel: every
call below returns before any HIP work is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

import bit_weight_only_03_amd as lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*((?:w4a16|w2t|w16a16|mxfp4)_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("w4a16_pack", "w4a16_unpack", "w4a16_gemv", "w4a16_gemv_add", "w4a16_dequant",
              "w16a16_gemv", "w16a16_workspace_bytes", "mxfp4_packed_sizes", "mxfp4_pack",
              "mxfp4_unpack", "mxfp4_workspace_bytes", "mxfp4_gemv", "mxfp4_dequant",
              "w4a16_packed_sizes",
              "w4a16_workspace_bytes", "w2t_pack", "w2t_unpack", "w2t_gemv", "w2t_dequant",
              "w2t_packed_sizes", "w2t_workspace_bytes", "w4a16_bw_probe", "w4a16_status_string",
              "w4a16_last_variant"):
        assert n in names


def test_library_exports_every_declared_symbol():
    so = ctypes.CDLL(lib.LIB_PATH)
    for n in declared_functions():
        assert hasattr(so, n), n
    assert set(declared_functions()) == set(lib.EXPORTED)


def test_packed_sizes():
    # 4096 x 4096, g128: 8 MiB of nibbles, 32 x 4096 fp16 scales, 32 x 4096 nibble zeros
    assert lib.w4a16_packed_sizes(4096, 4096, 128) == (8388608, 262144, 65536)
    # ragged: N = 24 pads to 32 columns, K = 96 (g = 32) pads to 128
    assert lib.w4a16_packed_sizes(24, 96, 32) == (32 * 128 // 2, 32 * 4 * 2, 32 * 4 // 2)
    assert lib.w2t_packed_sizes(5120, 17408, 128) == (5120 * 17408 // 4, 5120 * 136 * 2)
    # ternary: N needs no multiple of 8; 7 columns pad to 16, K = 32 pads to 256
    assert lib.w2t_packed_sizes(7, 32, 32) == (16 * 256 // 4, 16 * 8 * 2)


@pytest.mark.parametrize("N,K,g", [(0, 128, 128), (12, 128, 128), (16, 100, 128), (16, 128, 96),
                                   (16, 192, 128), (16, -128, 128)])
def test_packed_sizes_rejects_bad_shapes(N, K, g):
    with pytest.raises(lib.W4A16Error) as e:
        lib.w4a16_packed_sizes(N, K, g)
    assert e.value.status == -2


def test_gemv_argument_checks_return_before_launch():
    good = 1 << 20  # aligned fake pointers: the call must fail before touching them
    args = dict(x=good, x_dtype=0, qweight=good, scales=good, zeros=good, y=good, y_dtype=2,
                M=1, N=4096, K=4096, group=128, stream=0)

    def rc(**over):
        a = dict(args, **over)
        try:
            lib.w4a16_gemv(a["x"], a["x_dtype"], a["qweight"], a["scales"], a["zeros"], a["y"],
                           a["y_dtype"], a["M"], a["N"], a["K"], a["group"], stream=a["stream"])
        except lib.W4A16Error as e:
            return e.status
        return 0

    assert rc(x=0) == -1
    assert rc(zeros=0) == -1
    assert rc(x_dtype=2) == -4          # x must be f16 or bf16
    assert rc(y_dtype=7) == -4
    assert rc(M=0) == -2 and rc(M=65) == -2       # 1 <= M <= 64
    assert rc(N=0) == -2 and rc(N=4100) == -2
    assert rc(K=4100) == -2 and rc(group=100) == -2
    assert rc(x=good + 8) == -3 and rc(y=good + 4) == -3


def test_workspace_query_and_check():
    # 4096 columns fill the GPU with tiles: no K split, no workspace.
    assert lib.w4a16_workspace_bytes(1, 4096, 4096, 128) == 0
    # A narrow column shard (one GPU's share of down, N = 512) splits K.
    ws = lib.w4a16_workspace_bytes(4, 512, 17408, 128)
    assert ws > 0 and ws % (4 * 512 * 4) == 0
    good = 1 << 20
    with pytest.raises(lib.W4A16Error) as e:
        lib.w4a16_gemv(good, 0, good, good, good, good, 2, 4, 512, 17408, 128, workspace=good,
                       workspace_bytes=ws - 4, stream=0)
    assert e.value.status == -5
    with pytest.raises(lib.W4A16Error) as e:
        lib.w4a16_gemv(good, 0, good, good, good, good, 2, 4, 512, 17408, 128, stream=0)
    assert e.value.status == -1


def test_status_strings():
    for s in range(-7, 1):
        assert lib.w4a16_status_string(s) != "unknown status"
    assert lib.w4a16_status_string(-99) == "unknown status"


def test_ternary_argument_checks():
    good = 1 << 20
    with pytest.raises(lib.W4A16Error) as e:
        lib.w2t_gemv(good, 0, good, good, good, 2, 1, 5120, 5120 + 8, 128, stream=0)
    assert e.value.status == -2
    with pytest.raises(lib.W4A16Error) as e:
        lib.w2t_pack(good, good, 0, good, 16, 256, 128, stream=0)
    assert e.value.status == -1


def test_gemv_add_argument_checks():
    # The residual is checked on the host before anything is launched.
    good = 1 << 20

    def rc(residual=good, residual_dtype=1, M=4):
        try:
            lib.w4a16_gemv_add(good, 0, good, good, good, residual, residual_dtype, good, 2, M, 4096,
                               4096, 128, stream=0)
        except lib.W4A16Error as e:
            return e.status
        return 0

    assert rc(residual=0) == -1
    assert rc(residual_dtype=7) == -4
    assert rc(residual=good + 4) == -3
    assert rc(M=65) == -2


def test_w16a16_argument_checks():
    good = 1 << 20
    assert lib.w16a16_workspace_bytes(1, 4096, 4096) % (1 * 4096 * 4) == 0   # S slices of fp32 [M][N]
    for (M, N, K) in [(0, 64, 64), (65, 64, 64), (1, 12, 64), (1, 64, 100)]:
        with pytest.raises(lib.W4A16Error) as e:
            lib.w16a16_workspace_bytes(M, N, K)
        assert e.value.status == -2
    with pytest.raises(lib.W4A16Error) as e:
        lib.w16a16_gemv(good, good, 2, good, 2, 1, 64, 64, stream=0)     # f32 weights
    assert e.value.status == -4
    with pytest.raises(lib.W4A16Error) as e:
        lib.w16a16_gemv(good, good + 8, 0, good, 2, 1, 64, 64, stream=0)
    assert e.value.status == -3
    with pytest.raises(lib.W4A16Error) as e:
        lib.w16a16_gemv(good, 0, 0, good, 2, 1, 64, 64, stream=0)
    assert e.value.status == -1


def test_mxfp4_sizes_and_argument_checks():
    # 4096 x 4096: 8 MiB of codes, one scale byte per 32 elements; ragged
    # N = 24 pads to 32 columns, K = 96 to one 128-k unit.
    assert lib.mxfp4_packed_sizes(4096, 4096) == (8388608, 524288)
    assert lib.mxfp4_packed_sizes(24, 96) == (32 * 128 // 2, 32 * 128 // 32)
    for (N, K) in [(0, 64), (12, 64), (8, 48), (8, 16), (8, 0)]:
        with pytest.raises(lib.W4A16Error) as e:
            lib.mxfp4_packed_sizes(N, K)
        assert e.value.status == -2
    for M in (0, 65):
        with pytest.raises(lib.W4A16Error) as e:
            lib.mxfp4_workspace_bytes(M, 64, 64)
        assert e.value.status == -2
    assert lib.mxfp4_workspace_bytes(1, 4096, 4096) % (4096 * 4) == 0
    good = 1 << 20
    with pytest.raises(lib.W4A16Error) as e:
        lib.mxfp4_gemv(good, 2, good, good, good, 2, 1, 64, 64, stream=0)     # f32 x
    assert e.value.status == -4
    with pytest.raises(lib.W4A16Error) as e:
        lib.mxfp4_gemv(good, 0, good + 4, good, good, 2, 1, 64, 64, stream=0)
    assert e.value.status == -3
    with pytest.raises(lib.W4A16Error) as e:
        lib.mxfp4_gemv(good, 0, good, 0, good, 2, 1, 64, 64, stream=0)
    assert e.value.status == -1
    with pytest.raises(lib.W4A16Error) as e:
        lib.mxfp4_pack(good, good, good, good, 64, 40, stream=0)
    assert e.value.status == -2
    with pytest.raises(lib.W4A16Error) as e:
        lib.mxfp4_dequant(good, good, good + 8, 64, 64, stream=0)
    assert e.value.status == -3


def test_offset_limits_are_rejected_before_launch():
    # x is one 32-bit buffer resource (M * K * 2 < 2^32) and K <= 2^26 keeps
    # the per-workgroup weight offsets in range: larger shapes are errors, not
    # silent wrap-around.
    good = 1 << 20
    big_k = 1 << 26
    for call in (lambda: lib.w4a16_workspace_bytes(64, 64, big_k, 128),   # M K 2 = 2^33
                 lambda: lib.w4a16_workspace_bytes(1, 64, big_k + 128, 128),   # K > 2^26
                 lambda: lib.mxfp4_workspace_bytes(64, 64, big_k),
                 lambda: lib.w2t_workspace_bytes(64, 64, big_k, 128),
                 lambda: lib.w4a16_packed_sizes(64, big_k + 128, 128),
                 lambda: lib.mxfp4_packed_sizes(64, big_k + 32),
                 lambda: lib.w4a16_gemv(good, 0, good, good, good, good, 2, 64, 64, big_k, 128,
                                        stream=0),
                 lambda: lib.mxfp4_gemv(good, 0, good, good, good, 2, 64, 64, big_k, stream=0)):
        with pytest.raises(lib.W4A16Error) as e:
            call()
        assert e.value.status == -2
    # The largest K at M = 1 is accepted (sizes only; nothing launches).
    assert lib.w4a16_workspace_bytes(1, 64, big_k, 128) >= 0
    assert lib.w4a16_packed_sizes(64, big_k, 128)[0] == 64 * big_k // 2


def test_workspace_queries_follow_the_dispatch():
    # The size queries run the same host planner as the launches (no GPU
    # work; without a device the planner assumes 256 CUs), so they show
    # which kernel a shape gets.  fp32 partials are S x M x N x 4 bytes,
    # after the 64 KiB counter head.
    # W16A16: the dot-product kernel up to 4 rows and the K-split kernel up
    # to 16 on few-tile layers, the even-share kernel on the down shape up
    # to 2 rows; none of them sliced.  The down shape at 4 rows takes the
    # tiled kernel in 16 slices.
    H = lib.W4A16_WORKSPACE_HEAD_BYTES
    assert lib.w16a16_workspace_bytes(1, 7168, 5120) == 0
    assert lib.w16a16_workspace_bytes(8, 5120, 5120) == 0
    assert lib.w16a16_workspace_bytes(1, 5120, 17408) == 0
    assert lib.w16a16_workspace_bytes(2, 5120, 17408) == 0
    assert lib.w16a16_workspace_bytes(4, 5120, 17408) == H + 16 * 4 * 5120 * 4
    # Ternary: the staged kernel unsplit at K = 5120 up to 8 rows, and in 2
    # and 4 slices for the down shape at 4 and 8 rows.
    assert lib.w2t_workspace_bytes(8, 7168, 5120, 128) == 0
    assert lib.w2t_workspace_bytes(4, 5120, 17408, 128) == H + 2 * 4 * 5120 * 4
    assert lib.w2t_workspace_bytes(8, 5120, 17408, 128) == H + 4 * 8 * 5120 * 4
    # 4-bit: down at M = 4 on the balanced plan (one [4][16] piece per
    # quarter of its 64 leftover tiles), at M = 5 in 4 slices; M = 8 at
    # K = 5120 unsplit on the GEMV.
    assert lib.w4a16_workspace_bytes(4, 5120, 17408, 128) == H + 64 * 4 * 4 * 16 * 4
    assert lib.w4a16_workspace_bytes(5, 5120, 17408, 128) == H + 4 * 5 * 5120 * 4
    assert lib.w4a16_workspace_bytes(8, 5120, 5120, 128) == 0


def test_noalloc_checks_return_before_any_device_work():
    # The no-allocation GEMV refuses, on the host, a shape whose split-K
    # workspace exceeds its static array (K = 2^24 at N = 8192: 1024 slices,
    # 32 MiB of partials), naming the reason; the ordinary argument checks
    # come first.  No GPU is touched (stream 0, fake aligned pointers).
    M, N, K, g = 1, 8192, 1 << 24, 128
    assert lib.w4a16_workspace_bytes(M, N, K, g) > lib.W4A16_NOALLOC_SCRATCH_BYTES
    with pytest.raises(lib.W4A16Error) as e:
        lib.w4a16_gemv_noalloc(256, "f16", 256, 256, 256, 256, "f32", M, N, K, g, stream=0)
    assert e.value.status == -5
    assert "static scratch" in lib.w4a16_last_error()
    for args, status in (((256, "f16", 256, 256, 256, None, "f32", 1, 64, 128, 128), -1),
                         ((256, "f32", 256, 256, 256, 256, "f32", 1, 64, 128, 128), -4),
                         ((256, "f16", 256, 256, 256, 256, "f32", 65, 64, 128, 128), -2),
                         ((264, "f16", 256, 256, 256, 256, "f32", 1, 64, 128, 128), -3)):
        with pytest.raises(lib.W4A16Error) as e:
            lib.w4a16_gemv_noalloc(*args, stream=0)
        assert e.value.status == status
    # The header's array size and the binding's agree.
    text = open(HEADER).read()
    assert "#define W4A16_NOALLOC_SCRATCH_BYTES (16u << 20)" in text
    assert lib.W4A16_NOALLOC_SCRATCH_BYTES == 16 << 20


def test_workspace_head_and_balanced_plan_sizes():
    # Every workspace begins with the counter head: the split GEMV's size is
    # the head plus its fp32 partials, and the balanced plan (the 27B-class
    # down layer, N = 5120, K = 17408, up to 4 rows) the head plus one
    # [M][16] piece per leftover tile (64 tiles, 4 pieces each).  The
    # header's head size and the binding's agree.
    head = lib.W4A16_WORKSPACE_HEAD_BYTES
    assert "#define W4A16_WORKSPACE_HEAD_BYTES (64u << 10)" in open(HEADER).read()
    assert head == 64 << 10
    ws = lib.w4a16_workspace_bytes(4, 512, 17408, 128)
    assert ws > head and (ws - head) % (4 * 512 * 4) == 0
    for M in (1, 2, 3, 4):
        assert lib.w4a16_plan_variant(M, 5120, 17408, 128, "bf16").startswith("w4_bal16")
        assert lib.w4a16_workspace_bytes(M, 5120, 17408, 128) == head + 64 * 4 * M * 16 * 4
    assert lib.w4a16_workspace_bytes(1, 4096, 4096, 128) == 0
    # A balanced call with a short or missing workspace is refused before any
    # launch (no GPU is touched: stream 0, fake aligned pointers).
    good = 1 << 20
    ws = lib.w4a16_workspace_bytes(1, 5120, 17408, 128)
    with pytest.raises(lib.W4A16Error) as e:
        lib.w4a16_gemv(good, 0, good, good, good, good, 2, 1, 5120, 17408, 128, workspace=good,
                       workspace_bytes=ws - 16, stream=0)
    assert e.value.status == -5
    with pytest.raises(lib.W4A16Error) as e:
        lib.w4a16_gemv(good, 0, good, good, good, good, 2, 1, 5120, 17408, 128, stream=0)
    assert e.value.status == -1


def test_header_compiles_cleanly_as_c_and_cpp(tmp_path):
    # The header is the boundary's contract: it must compile warning-free on
    # its own for C and C++ callers (no nested comments, no missing types).
    import shutil
    import subprocess
    for cc, lang in (("gcc", "c"), ("g++", "c++")):
        if not shutil.which(cc):
            continue
        src = tmp_path / f"use.{ 'c' if lang == 'c' else 'cpp'}"
        src.write_text('#include "w4a16.h"\nint main(void) { return w4a16_status_string(0) ? 0 : 1; }\n')
        res = subprocess.run([cc, "-fsyntax-only", "-Wall", "-Wextra", "-Werror", "-x", lang,
                              f"-I{os.path.dirname(HEADER)}", str(src)], capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
