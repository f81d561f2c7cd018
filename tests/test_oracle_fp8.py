"""Pins for the FP8 (E4M3) oracle: its rounding against torch's float8_e4m3fn
conversion (round to nearest even) and against the format's own value
table, the float32 quantization formula, and the FP8 forward reducing to the
textbook forward when quantization is exact."""

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as F8


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).float().numpy()


def test_every_finite_code_is_a_fixed_point_and_the_table_is_the_format():
    vals = F8.decode_e4m3(np.arange(256))
    finite = vals[np.isfinite(vals)]
    assert len(finite) == 254                     # two NaN codes, no infinities
    assert finite.max() == 448.0 and finite.min() == -448.0
    assert np.min(np.abs(finite[finite != 0])) == 2.0 ** -9
    np.testing.assert_array_equal(F8.round_to_e4m3(finite), finite)
    np.testing.assert_array_equal(_torch_e4m3(finite), finite)


def test_rounding_matches_torch_float8_e4m3fn():
    rng = np.random.default_rng(0)
    vals = np.sort(np.unique(F8.decode_e4m3(np.arange(256))[np.isfinite(F8.decode_e4m3(np.arange(256)))]))
    mids = (vals[1:] + vals[:-1]) / 2              # exact ties (representable in float32)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.6, 20000),
        mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)).astype(np.float64),
        np.nextafter(mids.astype(np.float32), np.float32(-np.inf)).astype(np.float64),
        [0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -10, 17.0, 19.0]])
    x = np.clip(x.astype(np.float32).astype(np.float64), -448, 448)
    np.testing.assert_array_equal(F8.round_to_e4m3(x), _torch_e4m3(x))


def test_saturation_and_quantize_formula():
    assert F8.round_to_e4m3(np.array([1e6, -500.0, 449.0]) ).tolist() == [448.0, -448.0, 448.0]
    # x * fl32(1/s): 3 * (1/0.5) = 6 exactly; 1/3 rounds in float32 first
    assert F8.quantize(np.array([3.0]), 0.5)[0] == 6.0
    inv3 = np.float64(np.float32(1.0) / np.float32(3.0))
    y = np.float64(np.float32(np.float32(7.0) * np.float32(inv3)))
    assert F8.quantize(np.array([7.0]), 3.0)[0] == F8.round_to_e4m3(np.array([y]))[0]


def test_fp8_forward_is_the_textbook_forward_when_quantization_is_exact():
    """Inputs already on the E4M3 grid, scales 1, no rotation: q8 = q and
    k8 = k, so the FP8 forward equals the standard forward exactly."""
    rng = np.random.default_rng(1)
    L, d, s = 37, 64, 0.125
    grid = F8.decode_e4m3(np.arange(256))
    grid = grid[np.isfinite(grid) & (np.abs(grid) <= 4)]
    q, k = (rng.choice(grid, size=(L, d)) for _ in range(2))
    v = rng.standard_normal((L, d))
    O8, l8 = F8.attention_forward_fp8_slice(q, k, v, s, 0.0, 1.0, 1.0)
    O, l = oracle.attention_forward_slice(q, k, v, s, 0.0, mode="exact")
    np.testing.assert_allclose(O8, O, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l8, l, rtol=0, atol=1e-13)


def test_scales_are_undone_in_the_scores():
    """Inputs 4q and k/2 quantized with scales 4 and 1/2 land exactly on the
    grid values q and k; the scores multiply the scales back, so the result
    is the textbook forward of the inputs 4q and k/2."""
    rng = np.random.default_rng(2)
    L, d = 20, 64
    grid = F8.decode_e4m3(np.arange(256))
    grid = grid[np.isfinite(grid) & (np.abs(grid) <= 2) & (np.abs(grid) >= 2 ** -4)]
    q, k = (rng.choice(grid, size=(L, d)) for _ in range(2))
    v = rng.standard_normal((L, d))
    O8, l8 = F8.attention_forward_fp8_slice(q * 4, k * 0.5, v, 0.2, 0.0, 4.0, 0.5)
    O, l = oracle.attention_forward_slice(q * 4, k * 0.5, v, 0.2, 0.0, mode="exact")
    np.testing.assert_allclose(O8, O, atol=1e-13)
    np.testing.assert_allclose(l8, l, atol=1e-13)
