"""Host-side checks of the seeded input generators (no arithmetic of the
layer lives there; these check the drawn distributions and roundings)."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    v = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    v[:4] = [1.00390625, 1.01171875, -3.0e-39, 65504.0]   # halfway cases, subnormal, large
    ours = synth.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_w4_generator_distribution_and_determinism():
    a = synth.gen_w4((1, 2), 256, 4096, 128)
    b = synth.gen_w4((1, 2), 256, 4096, 128)
    for k in a:
        assert np.array_equal(a[k], b[k])
    nib = np.concatenate([(a["qweight"].view(np.uint32) >> np.uint32(4 * i)) & 15 for i in range(8)]).ravel()
    counts = np.bincount(nib, minlength=16) / nib.size
    assert np.all(np.abs(counts - 1 / 16) < 0.004)
    s = a["scales"].view(np.float16).astype(np.float64)
    assert s.shape == (32, 256) and s.min() >= 0.002 - 1e-6 and s.max() <= 0.02 + 1e-5
    c = synth.gen_w4((1, 3), 256, 4096, 128)
    assert not np.array_equal(a["qweight"], c["qweight"])


def test_x_outliers():
    x = synth.gen_x((3,), 4, 5120, "bf16", outlier_frac=0.01)
    f = (x.astype(np.uint32) << 16).view(np.float32)
    assert np.sum(np.abs(f) == 20.0) == round(0.01 * 4 * 5120)
    x16 = synth.gen_x((3,), 4, 5120, "f16")
    assert np.abs(x16.view(np.float16).astype(np.float64)).max() < 7


def test_w2t_generator_distribution():
    w = synth.gen_w2t((4,), 512, 5120, 128)
    words = w["codes"].view(np.uint32)
    c = np.concatenate([(words >> np.uint32(2 * i)) & 3 for i in range(16)]).ravel()
    p = np.bincount(c, minlength=4) / c.size
    assert p[3] == 0
    assert abs(p[0] - 0.25) < 0.003 and abs(p[1] - 0.5) < 0.003 and abs(p[2] - 0.25) < 0.003
