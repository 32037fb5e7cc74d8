"""Pins of the lesson's error checker (oracle/checker.py), CPU only.

The four controls are the ones the "Lesson K23, fused attention" facts page
prints for its checker (block ``controls.checker``: N 256, d 16, tiles of 16):
the tiled float32 output passes, the exact answer rounded to float32 passes,
one output moved by 0.001 fails with exactly one mismatch, and zero tolerance
rejects the float32 output.  The inputs follow the page's correctness recipe
(uniform in [-2, 2), seed 1, scale 1/sqrt(d)) with NumPy's PCG64 generator, so
mismatch counts of the broken variant are not compared with the page's
(parity unpinned: they depend on the page's generator).
"""
import numpy as np
import pytest

from exact_attention_forward_amd import inputs as I
from oracle import checker, online


@pytest.fixture(scope="module")
def lab256():
    c = I.lab_case(256, 16)
    q, k, v = (getattr(c, n)[0, :, 0, :] for n in ("q", "k", "v"))
    ref, bound = checker.reference_and_bound(q, k, v, c.scale)
    return c, q, k, v, ref, bound


def test_tiled_float32_output_passes(lab256):
    c, q, k, v, ref, bound = lab256
    O32, _ = online.tiled_forward(q, k, v, c.scale, False, 16, 16, dtype=np.float32)
    assert O32.dtype == np.float32
    r = checker.check(O32, ref, bound)
    assert r["ok"] and r["mismatches"] == 0 and r["outputs"] == 256 * 16


def test_rounded_reference_passes(lab256):
    c, q, k, v, ref, bound = lab256
    assert checker.check(ref.astype(np.float32), ref, bound)["ok"]


def test_one_output_off_by_a_thousandth_is_exactly_one_mismatch(lab256):
    c, q, k, v, ref, bound = lab256
    out = ref.astype(np.float32)
    out[17, 5] += np.float32(0.001)
    r = checker.check(out, ref, bound)
    assert not r["ok"] and r["mismatches"] == 1


def test_zero_tolerance_rejects_float32(lab256):
    c, q, k, v, ref, bound = lab256
    O32, _ = online.tiled_forward(q, k, v, c.scale, False, 16, 16, dtype=np.float32)
    assert not checker.check(O32, ref, np.zeros_like(bound))["ok"]


def test_missing_rescale_is_caught_only_across_tiles(lab256):
    c, q, k, v, ref, bound = lab256
    broken, _ = online.tiled_forward(q, k, v, c.scale, False, 16, 16, rescale=False, dtype=np.float32)
    assert not checker.check(broken, ref, bound)["ok"]
    # a single key tile never raises a row's max after its first tile: nothing to rescale
    one, _ = online.tiled_forward(q, k, v, c.scale, False, 16, 256, rescale=False, dtype=np.float32)
    assert checker.check(one, ref, bound)["ok"]


def test_reference_is_the_definition_and_rows_subset():
    c = I.lab_case(300, 8, seed=3)
    q, k, v = (getattr(c, n)[0, :, 0, :].astype(np.float64) for n in ("q", "k", "v"))
    ref, bound = checker.reference_and_bound(q, k, v, c.scale)
    s = c.scale * q @ k.T
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.allclose(ref, p @ v, rtol=0, atol=1e-14)
    rows = np.array([0, 7, 299])
    r2, b2 = checker.reference_and_bound(q, k, v, c.scale, rows)
    assert np.array_equal(r2, ref[rows]) and np.array_equal(b2, bound[rows])
    assert (bound > 0).all()
    assert list(checker.rows_checked(1024)) == list(range(1024)) and len(checker.rows_checked(2048)) == 64


def test_gamma_and_bound_grow_with_sizes():
    assert checker.gamma(1) == pytest.approx(2.0 ** -24, rel=1e-6)
    assert checker.gamma(2) > 2 * checker.gamma(1) * 0.999999
    c1, c2 = I.lab_case(64, 16), I.lab_case(64, 64)
    b1 = checker.reference_and_bound(*(getattr(c1, n)[0, :, 0, :] for n in ("q", "k", "v")), c1.scale)[1]
    b2 = checker.reference_and_bound(*(getattr(c2, n)[0, :, 0, :] for n in ("q", "k", "v")), c2.scale)[1]
    assert b1.shape == (64, 16) and b2.shape == (64, 64)


# The page's checker outcomes (block correctness.rows: ok and output count per
# (N, d, B, kind); block controls.checker), extracted by
# tests/golden/extract_page_fixtures.py.
import json  # noqa: E402
from pathlib import Path  # noqa: E402

PAGE = json.loads((Path(__file__).resolve().parent / "golden" / "lesson_checker.json").read_text())


def _unfused32(q, k, v, scale):
    """Algorithm 0 in float32: the score matrix, a max-subtracted row softmax, then P V."""
    q, k, v = (np.asarray(x, np.float32) for x in (q, k, v))
    s = (q @ k.T) * np.float32(scale)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


@pytest.mark.parametrize("row", PAGE["rows"], ids=lambda r: f"{r['kind']}-N{r['N']}-d{r['d']}-B{r['B']}")
def test_page_correctness_outcomes(row):
    """Tiled and unfused float32 outputs pass; the no-rescale variant fails exactly when a row spans more than
    one tile of B keys (the outcomes the page prints; its mismatch counts depend on its generator)."""
    N, d, B = row["N"], row["d"], row["B"]
    c = I.lab_case(N, d)
    q, k, v = (getattr(c, n)[0, :, 0, :] for n in ("q", "k", "v"))
    rows = checker.rows_checked(N)
    ref, bound = checker.reference_and_bound(q, k, v, c.scale, rows)
    if row["kind"] == "unfused":
        out = _unfused32(q, k, v, c.scale)
    else:
        out, _ = online.tiled_forward(q, k, v, c.scale, False, B, B, rescale=row["kind"] == "fused", dtype=np.float32)
    r = checker.check(out[rows], ref, bound)
    assert r["outputs"] == row["outputs"]
    assert r["ok"] == row["ok"]
    if row["kind"] == "broken":
        assert row["ok"] == (N <= B)


def test_page_checker_controls(lab256):
    c, q, k, v, ref, bound = lab256
    O32, _ = online.tiled_forward(q, k, v, c.scale, False, 16, 16, dtype=np.float32)
    off = ref.astype(np.float32)
    off[3, 2] += np.float32(0.001)
    got = {"tiled": checker.check(O32, ref, bound)["ok"],
           "roundedReference": checker.check(ref.astype(np.float32), ref, bound)["ok"],
           "oneOff": checker.check(off, ref, bound)["mismatches"],
           "zeroTolerance": checker.check(O32, ref, np.zeros_like(bound))["ok"]}
    assert got == PAGE["checker"]


def test_causal_bound_is_the_truncated_problem():
    """Row i of the causal reference and bound equals the unmasked ones on keys 0..i."""
    c = I.lab_case(70, 16, seed=5)
    q, k, v = (getattr(c, n)[0, :, 0, :].astype(np.float64) for n in ("q", "k", "v"))
    ref, bound = checker.reference_and_bound(q, k, v, c.scale, causal=True)
    for i in (0, 1, 13, 69):
        r1, b1 = checker.reference_and_bound(q[: i + 1], k[: i + 1], v[: i + 1], c.scale, rows=[i])
        assert np.allclose(ref[i], r1[0], rtol=0, atol=1e-15)
        assert np.allclose(bound[i], b1[0], rtol=1e-14, atol=0)
    assert np.array_equal(ref[0], v[0])  # row 0 sees only key 0
    # masked keys neither add to the reference nor widen the bound
    full_ref, full_bound = checker.reference_and_bound(q, k, v, c.scale)
    assert np.array_equal(full_ref[-1], ref[-1]) and np.allclose(full_bound[-1], bound[-1], rtol=1e-15)
    # the tiled float32 causal output passes
    O32, _ = online.tiled_forward(q, k, v, c.scale, True, 16, 16, dtype=np.float32)
    assert checker.check(O32, ref, bound)["ok"]
