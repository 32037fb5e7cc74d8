"""The seeded input generators (CPU only)."""
import numpy as np
import torch

from exact_attention_forward_amd import inputs as I


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(20000).astype(np.float32) * 50
    x = np.concatenate([x, np.float32([1.00390625, 1.01171875, 3.0e38, -1e-40, 0.0, -0.0])])
    ours = I.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()
    back = I.bf16_bits_to_f32(ours)
    assert (back == torch.from_numpy(x).to(torch.bfloat16).float().numpy()).all()


def test_cases_are_deterministic_and_shaped():
    a, b = I.make_case("x", 2, 3, 5, 8, I.F32, True, 7), I.make_case("x", 2, 3, 5, 8, I.F32, True, 7)
    for n in ("q", "k", "v", "do"):
        assert getattr(a, n).shape == (2, 5, 3, 8)
        assert (getattr(a, n) == getattr(b, n)).all()
    c = I.make_case("x", 2, 3, 5, 8, I.BF16, True, 7)
    assert c.q.dtype == np.uint16
    assert (c.f64("q") == I.bf16_bits_to_f32(I.f32_to_bf16_bits(a.q))).all()


def test_workload_recipes():
    t = I.tiny_case(True)
    assert (t.B, t.H, t.T, t.hd, t.scale, t.dtype) == (1, 1, 64, 16, 0.25, I.F32)
    r = I.ragged_cases()
    assert [(c.B, c.H, c.T, c.hd) for c in r] == I.RAGGED_SHAPES and [c.seed for c in r] == [10, 11, 12, 13]


def test_outlier_rows():
    c = I.make_case("o", 1, 2, 200, 4, I.F32, True, 3, outlier_frac=0.01)
    plain = I.make_case("o", 1, 2, 200, 4, I.F32, True, 3)
    ratio = c.k / plain.k
    for h in range(2):
        rows = np.where(np.abs(ratio[0, :, h, 0] - 8) < 1e-6)[0]
        assert len(rows) == 2
        assert np.allclose(ratio[0, rows, h], 8)
    assert (c.q == plain.q).all() and (c.do == plain.do).all()
