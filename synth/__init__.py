"""Seeded synthetic inputs for the W4A16 / ternary / W16A16 / MXFP4 small-M linear layer.

This module only draws random inputs and packs them into the canonical storage
format; it holds none of the layer's arithmetic (no dequantization, no
products).  Both the CPU oracle and the GPU path consume exactly the arrays it
returns, so the two sides see the same bits.

Canonical format (the library's boundary input):
  qweight int32 [N][K/8]   nibble i of word (n, j) holds q[k=8j+i][n]
  scales  uint16 [K/g][N]  IEEE binary16 bit patterns
  zeros   int32 [K/g][N/8] nibble i of word (gi, j) holds z[gi][8j+i]
  codes   int32 [N][K/16]  2-bit field i of word (n, j) holds c[k=16j+i][n], c in {0,1,2}
  x       uint16 [M][K]    binary16 or bfloat16 bit patterns
  w16     uint16 [N][K]    16-bit weights (the linear layer's own layout),
                           same type as x
  mx      qweight uint8 [N][K/2]: element k of row n in byte k/2, low nibble
                           for even k (4-bit E2M1 codes); scales uint8
                           [N][K/32]: one E8M0 code per 32-element block

Distributions (the layer shapes are the 27B-class projections the Z100 vLLM
article, section 四/五, and the ternary tuning page, section 六, time; the
pages give no value distributions, so these are stated choices):
  x       standard normal drawn in float64, rounded to nearest-even into fp16
          (bf16: float64 -> float32 -> bfloat16, each step nearest-even);
          optional outliers: round(frac*M*K) distinct positions set to
          +-magnitude with a fair random sign.
  q, z    iid uniform on 0..15 (uniform random 32-bit words).
  s       uniform on [lo, hi] in float64, rounded to nearest-even fp16.
  c       iid with P(c=0)=1/4, P(c=1)=1/2, P(c=2)=1/4, i.e. the sum of two fair
          bits, so weight = c - 1 is -1/0/+1 with probability 1/4, 1/2, 1/4.
  w16     normal with standard deviation sigma (default 0.02, a typical
          linear-layer weight scale), rounded like x.
  mx      element codes iid uniform on 0..15 (uniform random bytes); scale
          codes iid uniform on [e_lo, e_hi] (default 118..125, i.e. block
          scales 2^-9 .. 2^-2, where weights of standard deviation ~0.02
          land once quantized to a largest element of 6).
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 20261202


def rng_for(*key: int) -> np.random.Generator:
    """A PCG64 stream keyed by (BASE_SEED, *key); distinct keys give
    independent streams."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, *[int(k) for k in key]])))


def f64_to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even, returning the 16-bit patterns
    (inputs here are finite)."""
    b = np.asarray(a32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float64).astype(np.float32))


def random_words(rng: np.random.Generator, count: int) -> np.ndarray:
    """`count` uniform 32-bit words as int32."""
    return rng.integers(0, 2**32, size=count, dtype=np.uint32).view(np.int32)


def gen_x(key, M: int, K: int, dtype: str = "f16", outlier_frac: float = 0.0,
          outlier_mag: float = 20.0) -> np.ndarray:
    """Activations as uint16 bit patterns [M][K]."""
    rng = rng_for(*key, 1)
    v = rng.standard_normal((M, K))
    n_out = int(round(outlier_frac * M * K))
    if n_out:
        pos = rng.choice(M * K, size=n_out, replace=False)
        sign = np.where(rng.integers(0, 2, size=n_out) == 1, 1.0, -1.0)
        v.reshape(-1)[pos] = sign * outlier_mag
    if dtype == "f16":
        return f64_to_f16_bits(v)
    if dtype == "bf16":
        return f64_to_bf16_bits(v)
    raise ValueError(dtype)


def gen_w4(key, N: int, K: int, group: int, s_lo: float = 0.002, s_hi: float = 0.02):
    """Canonical 4-bit weights: dict(qweight [N][K/8] int32, scales [G][N]
    uint16, zeros [G][N/8] int32)."""
    if K % group or K % 8 or N % 8:
        raise ValueError("need K % group == 0, K % 8 == 0, N % 8 == 0")
    G = K // group
    rq = rng_for(*key, 2)
    rs = rng_for(*key, 3)
    rz = rng_for(*key, 4)
    qweight = random_words(rq, N * (K // 8)).reshape(N, K // 8)
    scales = f64_to_f16_bits(rs.uniform(s_lo, s_hi, size=(G, N)))
    zeros = random_words(rz, G * (N // 8)).reshape(G, N // 8)
    return {"qweight": qweight, "scales": scales, "zeros": zeros}


def gen_w16(key, N: int, K: int, dtype: str = "f16", sigma: float = 0.02) -> np.ndarray:
    """16-bit weights as uint16 bit patterns [N][K]."""
    v = rng_for(*key, 3).standard_normal((N, K)) * sigma
    if dtype == "f16":
        return f64_to_f16_bits(v)
    if dtype == "bf16":
        return f64_to_bf16_bits(v)
    raise ValueError(dtype)


def gen_mx(key, N: int, K: int, e_lo: int = 118, e_hi: int = 125):
    """Canonical MXFP4 weights: dict(qweight uint8 [N][K/2], scales uint8 [N][K/32])."""
    if K % 32:
        raise ValueError("need K % 32 == 0")
    rng = rng_for(*key, 5)
    q = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = rng.integers(e_lo, e_hi + 1, size=(N, K // 32), dtype=np.uint8)
    return {"qweight": q, "scales": s}


def pack_codes(c: np.ndarray) -> np.ndarray:
    """Pack 2-bit codes c[N][K] (values 0..3) into int32 [N][K/16], field i of
    word j holding c[16j+i]."""
    N, K = c.shape
    c = c.astype(np.uint32).reshape(N, K // 16, 16)
    words = np.zeros((N, K // 16), dtype=np.uint32)
    for i in range(16):
        words |= c[:, :, i] << np.uint32(2 * i)
    return words.view(np.int32)


def gen_w2t(key, N: int, K: int, group: int, s_lo: float = 0.01, s_hi: float = 0.05):
    """Canonical ternary weights: dict(codes [N][K/16] int32, scales [G][N] uint16)."""
    if K % group or K % 16:
        raise ValueError("need K % group == 0 and K % 16 == 0")
    G = K // group
    rc = rng_for(*key, 5)
    rs = rng_for(*key, 6)
    # Two independent uniform bits per weight, taken from two random words per
    # 16-weight word: field i = bit i of A + bit i of B.
    a = rc.integers(0, 2**32, size=(N, K // 16), dtype=np.uint32)
    b = rc.integers(0, 2**32, size=(N, K // 16), dtype=np.uint32)
    words = np.zeros((N, K // 16), dtype=np.uint32)
    for i in range(16):
        c = ((a >> np.uint32(i)) & np.uint32(1)) + ((b >> np.uint32(i)) & np.uint32(1))
        words |= c << np.uint32(2 * i)
    scales = f64_to_f16_bits(rs.uniform(s_lo, s_hi, size=(G, N)))
    return {"codes": words.view(np.int32), "scales": scales}


# Layer shapes of the 27B-class decoder (K, N): fused QKV, o_proj, fused
# gate_up, down.  64 layers of these four matrices make one decode token's
# weight sweep.
LAYER_SHAPES = (("qkv", 5120, 7168), ("o_proj", 5120, 5120),
                ("gate_up", 5120, 34816), ("down", 17408, 5120))
N_LAYERS = 64


# ---------------------------------------------------------------------------
# Device-side generators for large benchmark inputs (an 11 GB weight sweep is
# slow to draw on the host).  Same distributions as above, drawn with torch's
# seeded Philox generator on the given device; anything that needs the values
# on the host copies them back.  Imported lazily so the module stays usable
# without torch.

def _torch_gen(key, device):
    import torch
    seed = int(np.random.SeedSequence([BASE_SEED, *[int(k) for k in key]]).generate_state(1, np.uint64)[0])
    g = torch.Generator(device=device)
    g.manual_seed(seed & ((1 << 63) - 1))
    return g


def gen_w4_torch(key, N: int, K: int, group: int, device="cuda", s_lo: float = 0.002,
                 s_hi: float = 0.02):
    """Canonical 4-bit weights as device tensors (int32 qweight [N][K/8],
    int16 scale bits [G][N], int32 zeros [G][N/8])."""
    import torch
    if K % group or K % 8 or N % 8:
        raise ValueError("need K % group == 0, K % 8 == 0, N % 8 == 0")
    G = K // group
    g = _torch_gen(key, device)
    q = torch.randint(-2**31, 2**31, (N, K // 8), dtype=torch.int32, device=device, generator=g)
    z = torch.randint(-2**31, 2**31, (G, N // 8), dtype=torch.int32, device=device, generator=g)
    u = torch.rand((G, N), dtype=torch.float64, device=device, generator=g)
    s = (s_lo + (s_hi - s_lo) * u).to(torch.float16).view(torch.int16)
    return {"qweight": q, "scales": s, "zeros": z}


def gen_x_torch(key, M: int, K: int, dtype: str = "f16", outlier_frac: float = 0.0,
                outlier_mag: float = 20.0, device="cuda"):
    """Activations as an int16 device tensor of fp16/bf16 bit patterns [M][K]."""
    import torch
    g = _torch_gen(key, device)
    v = torch.randn((M, K), dtype=torch.float64, device=device, generator=g)
    n_out = int(round(outlier_frac * M * K))
    if n_out:
        pos = torch.randperm(M * K, device=device, generator=g)[:n_out]
        sign = torch.randint(0, 2, (n_out,), device=device, generator=g).to(torch.float64) * 2 - 1
        v.view(-1)[pos] = sign * outlier_mag
    if dtype == "f16":
        return v.to(torch.float16).view(torch.int16)
    if dtype == "bf16":
        return v.to(torch.float32).to(torch.bfloat16).view(torch.int16)
    raise ValueError(dtype)


def gen_w2t_torch(key, N: int, K: int, group: int, device="cuda", s_lo: float = 0.01,
                  s_hi: float = 0.05):
    """Canonical ternary codes as device tensors (int32 codes [N][K/16], int16
    scale bits [G][N]); each code is the sum of two fair random bits."""
    import torch
    if K % group or K % 16:
        raise ValueError("need K % group == 0 and K % 16 == 0")
    G = K // group
    g = _torch_gen(key, device)
    a = torch.randint(-2**31, 2**31, (N, K // 16), dtype=torch.int32, device=device, generator=g)
    b = torch.randint(-2**31, 2**31, (N, K // 16), dtype=torch.int32, device=device, generator=g)
    words = torch.zeros((N, K // 16), dtype=torch.int32, device=device)
    for i in range(16):
        c = ((a >> i) & 1) + ((b >> i) & 1)
        words |= c << (2 * i)
    u = torch.rand((G, N), dtype=torch.float64, device=device, generator=g)
    s = (s_lo + (s_hi - s_lo) * u).to(torch.float16).view(torch.int16)
    return {"codes": words, "scales": s}


def gen_w16_torch(key, N: int, K: int, dtype: str = "f16", sigma: float = 0.02, device="cuda"):
    """16-bit weights as an int16 device tensor of bit patterns [N][K]."""
    import torch
    g = _torch_gen(key, device)
    v = torch.randn((N, K), dtype=torch.float64, device=device, generator=g) * sigma
    if dtype == "f16":
        return v.to(torch.float16).view(torch.int16)
    if dtype == "bf16":
        return v.to(torch.float32).to(torch.bfloat16).view(torch.int16)
    raise ValueError(dtype)


def gen_mx_torch(key, N: int, K: int, device="cuda", e_lo: int = 118, e_hi: int = 125):
    """MXFP4 weights drawn on the device (same distribution as gen_mx, other
    bits): dict(qweight uint8 [N][K/2], scales uint8 [N][K/32])."""
    import torch
    if K % 32:
        raise ValueError("need K % 32 == 0")
    g = _torch_gen(key, device)
    q = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=device, generator=g)
    s = torch.randint(e_lo, e_hi + 1, (N, K // 32), dtype=torch.uint8, device=device, generator=g)
    return {"qweight": q, "scales": s}
