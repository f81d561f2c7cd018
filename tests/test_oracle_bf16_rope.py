"""Pins for the oracle's bf16 rounding and rotary embedding, against things
other than the oracle itself: torch's float32 -> bf16 conversion, the
complex-number form of the rotation, closed forms and invariants."""

import numpy as np
import pytest
import torch

import oracle


def test_bf16_bits_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x3E80,
                     0x0001, 0x7F7F], dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    want = [1.0, -2.0, 0.0, -0.0, np.inf, -np.inf, 0.25, 2.0 ** -133,
            255.0 * 2.0 ** 120]
    np.testing.assert_array_equal(got, np.array(want))


def test_round_to_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
        rng.standard_normal(2000) * 1e-39,          # float32 subnormal range
        np.clip(rng.standard_normal(2000), -3, 3) * 1e38,  # near the top
    ]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_round_to_bf16_ties_to_even():
    one = 1.0
    cases = {
        one + 2.0 ** -8: 1.0,                     # halfway, even is 1.0
        one + 3 * 2.0 ** -8: one + 2.0 ** -6,     # halfway, even is 1+2^-6
        one + 2.0 ** -8 + 2.0 ** -30: one + 2.0 ** -7,
        -(one + 2.0 ** -8): -1.0,
        255.5 * 2.0 ** 120: np.inf,               # tie past the largest finite
    }
    for x, want in cases.items():
        assert oracle.round_to_bf16(np.array([x]))[0] == want, x
    assert np.isnan(oracle.round_to_bf16(np.array([np.nan]))[0])


def test_rope_frequencies_closed_form():
    np.testing.assert_allclose(oracle.rope_frequencies(4, 10000.0), [1.0, 0.01],
                               rtol=1e-15)
    th = oracle.rope_frequencies(64, 10000.0)
    assert th[0] == 1.0
    np.testing.assert_allclose(th[16], 0.01, rtol=1e-14)   # 10000^(-32/64)
    np.testing.assert_allclose(th[31], 10000.0 ** (-62 / 64), rtol=1e-14)
    assert oracle.rope_frequencies(8, 0.0) is None


def _rope_complex(x, pos, base):
    """Independent form: pair (x_j, x_{j+d/2}) is the complex number
    x_j + i x_{j+d/2}, multiplied by exp(i p base^(-2j/d))."""
    d = x.shape[-1]
    h = d // 2
    z = x[..., :h] + 1j * x[..., h:]
    j = np.arange(h)
    w = np.exp(1j * np.outer(pos, base ** (-2.0 * j / d)))
    w = w.reshape((x.shape[0],) + (1,) * (x.ndim - 2) + (h,))
    r = z * w
    return np.concatenate([r.real, r.imag], axis=-1)


@pytest.mark.parametrize("d", [2, 4, 16, 64, 128])
def test_rope_matches_complex_multiplication(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((50, 3, d))
    pos = rng.integers(0, 8192, 50).astype(np.float64)
    got = oracle.rope_rotate(x, pos, 10000.0)
    np.testing.assert_allclose(got, _rope_complex(x, pos, 10000.0), atol=1e-12)


def test_rope_position_zero_is_identity_and_base_zero_is_off():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 2, 32))
    np.testing.assert_array_equal(oracle.rope_rotate(x, np.zeros(4), 10000.0), x)
    np.testing.assert_array_equal(
        oracle.rope_rotate(x, np.arange(4) * 100.0, 0.0), x)


def test_rope_d2_rotates_by_position_radians():
    x = np.array([[1.0, 0.0], [0.0, 1.0], [3.0, 4.0]])
    pos = np.array([np.pi / 2, np.pi, 1.0])
    got = oracle.rope_rotate(x, pos, 10000.0)   # d=2: theta_0 = 1
    np.testing.assert_allclose(got[0], [0.0, 1.0], atol=1e-15)
    np.testing.assert_allclose(got[1], [0.0, -1.0], atol=1e-15)
    c, s = np.cos(1.0), np.sin(1.0)
    np.testing.assert_allclose(got[2], [3 * c - 4 * s, 4 * c + 3 * s], atol=1e-15)


def test_rope_is_orthogonal_and_inverse_is_transpose():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 1, 64))
    y = rng.standard_normal((64, 1, 64))
    pos = np.arange(64) * 37.0
    rx = oracle.rope_rotate(x, pos, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(rx, axis=-1),
                               np.linalg.norm(x, axis=-1), rtol=1e-13)
    back = oracle.rope_rotate(rx, pos, 10000.0, inverse=True)
    np.testing.assert_allclose(back, x, atol=1e-12)
    ry = oracle.rope_rotate(y, pos, 10000.0, inverse=True)
    np.testing.assert_allclose((rx * y).sum(-1), (x * ry).sum(-1), atol=1e-11)


def test_rope_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 64))
    k = rng.standard_normal((1, 64))
    base = 10000.0
    ref = None
    for shift in [0.0, 5.0, 1000.0, 8000.0]:
        qp = oracle.rope_rotate(q, np.array([shift + 17.0]), base)
        kt = oracle.rope_rotate(k, np.array([shift + 3.0]), base)
        val = float((qp * kt).sum())
        ref = val if ref is None else ref
        assert abs(val - ref) < 1e-10
    qp = oracle.rope_rotate(q, np.array([18.0]), base)
    kt = oracle.rope_rotate(k, np.array([3.0]), base)
    assert abs(float((qp * kt).sum()) - ref) > 1e-6   # offset matters


def test_half_split_equals_interleaved_under_permutation():
    rng = np.random.default_rng(4)
    d = 16
    x = rng.standard_normal((10, d))
    pos = np.arange(10) * 3.0
    # interleaved pairing, written with complex pairs (x_2j, x_2j+1)
    z = x[:, 0::2] + 1j * x[:, 1::2]
    j = np.arange(d // 2)
    r = z * np.exp(1j * np.outer(pos, 10000.0 ** (-2.0 * j / d)))
    inter = np.empty_like(x)
    inter[:, 0::2], inter[:, 1::2] = r.real, r.imag
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    half = oracle.rope_rotate(x[:, perm], pos, 10000.0)
    back = np.empty_like(half)
    back[:, perm] = half
    np.testing.assert_allclose(back, inter, atol=1e-12)


def test_float32_rotation_matches_torch_float32_and_fp64_bounds():
    rng = np.random.default_rng(5)
    d = 64
    x = oracle.round_to_bf16(rng.standard_normal((300, 2, d)) * 3)
    pos = np.arange(300, dtype=np.float64) * 7.0
    got = oracle.rope_rotate_f32(x, pos, 10000.0)
    # torch float32 elementwise ops (separately rounded products and sums)
    th = 10000.0 ** (-2.0 * np.arange(d // 2) / d)
    ang = pos[:, None] * th[None, :]
    c = torch.from_numpy(np.cos(ang).astype(np.float32))[:, None, :]
    s = torch.from_numpy(np.sin(ang).astype(np.float32))[:, None, :]
    t = torch.from_numpy(x.astype(np.float32))
    lo, hi = t[..., : d // 2], t[..., d // 2:]
    want = torch.cat([lo * c - hi * s, hi * c + lo * s], dim=-1).double().numpy()
    np.testing.assert_array_equal(got, want)
    # float32 evaluation stays within a few float32 ulps of the float64 rotation
    exact = oracle.rope_rotate(x, pos, 10000.0)
    assert np.abs(got - exact).max() <= 4 * 2.0 ** -24 * np.abs(x).max() * 2
    # and its bf16 rounding differs from the float64 one in a tiny fraction of entries
    frac = np.mean(oracle.round_to_bf16(got) != oracle.round_to_bf16(exact))
    assert frac < 1e-3
    # position 0 and base 0 are exact identities
    np.testing.assert_array_equal(oracle.rope_rotate_f32(x[:1], [0.0], 10000.0), x[:1])
    np.testing.assert_array_equal(oracle.rope_rotate_f32(x, pos, 0.0), x)


# ---------------------------------------------------------------- query operand

_L2E = float(np.log2(np.e))


def _torch_query_operand(q, pos, base, scale):
    """q^ from torch float32 elementwise ops (each product, sum and the scale
    product rounded to float32 separately; no fused multiply-add across torch
    ops) and torch's float32 -> bf16 conversion (round to nearest even)."""
    d = q.shape[-1]
    h = d // 2
    t = torch.from_numpy(np.asarray(q, np.float64).astype(np.float32))
    if base != 0:
        th = float(base) ** (-2.0 * np.arange(h) / d)
        ang = np.asarray(pos, np.float64)[:, None] * th[None, :]
        shape = (t.shape[0],) + (1,) * (t.dim() - 2) + (h,)
        c = torch.from_numpy(np.cos(ang).astype(np.float32)).reshape(shape)
        s = torch.from_numpy(np.sin(ang).astype(np.float32)).reshape(shape)
        lo, hi = t[..., :h], t[..., h:]
        t = torch.cat([lo * c - hi * s, hi * c + lo * s], dim=-1)
    cf = torch.tensor(scale, dtype=torch.float32) * torch.tensor(_L2E, dtype=torch.float32)
    return (t * cf).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("scale,base", [(0.125, 10000.0), (48 ** -0.5, 10000.0),
                                        (-0.2, 10000.0), (0.6, 0.0), (1e-3, 500.0)])
def test_query_operand_matches_torch_float32(scale, base):
    rng = np.random.default_rng(21)
    x = oracle.round_to_bf16(rng.standard_normal((512, 4, 64)) * 3)
    pos = np.arange(512, dtype=np.float64)
    np.testing.assert_array_equal(oracle.query_operand_bf16(x, pos, base, scale),
                                  _torch_query_operand(x, pos, base, scale))


def test_query_operand_pin_rejects_plausible_variants():
    """Each plausible mistake in the rounding recipe, planted in a copy of the
    oracle function, disagrees with the torch pin on a sample of 2^20 rotated
    values (the recipe's roundings differ only near bf16 ties, about 1e-5 of
    entries, so the sample must be large)."""
    rng = np.random.default_rng(22)
    x = oracle.round_to_bf16(rng.standard_normal((4096, 4, 64)) * 3)
    pos = np.arange(4096, dtype=np.float64)
    base = 10000.0
    scale = 48 ** -0.5   # fl32(fl32(s) fl32(log2 e)) != fl32(s log2 e) here
    assert np.float32(np.float32(scale) * np.float32(_L2E)) != np.float32(scale * _L2E)
    pin = _torch_query_operand(x, pos, base, scale)
    np.testing.assert_array_equal(oracle.query_operand_bf16(x, pos, base, scale), pin)

    rot = oracle.rope_rotate_f32(x, pos, base)           # float32 values
    c32 = np.float32(scale) * np.float32(_L2E)
    bf = oracle.round_to_bf16
    f32 = lambda a: np.asarray(a, np.float64).astype(np.float32).astype(np.float64)
    # 1. c rounded once from the float64 product scale * log2 e
    m_c_once = bf(f32(rot * np.float64(np.float32(scale * _L2E))))
    # 2. c and the scaling product kept in float64
    m_c_fp64 = bf(rot * (scale * _L2E))
    # 3. bf16 rounding of the rotated value before the scaling
    m_round_first = bf(f32(bf(rot) * np.float64(c32)))
    # 4. rotation contracted to fused multiply-adds (x c - y s with one rounding)
    th = base ** (-2.0 * np.arange(32) / 64)
    ang = pos[:, None] * th[None, :]
    cs = np.cos(ang).astype(np.float32).astype(np.float64)[:, None, :]
    sn = np.sin(ang).astype(np.float32).astype(np.float64)[:, None, :]
    lo, hi = x[..., :32], x[..., 32:]
    fma = np.concatenate([f32(lo * cs - f32(hi * sn)), f32(hi * cs + f32(lo * sn))], axis=-1)
    m_fma = bf(f32(fma * np.float64(c32)))
    # 5. sine with the wrong sign (rotation by -p)
    m_sign = bf(f32(oracle.rope_rotate_f32(x, -pos, base) * np.float64(c32)))
    for name, m in (("c rounded once", m_c_once), ("c in float64", m_c_fp64),
                    ("round before scale", m_round_first), ("fused multiply-add", m_fma),
                    ("inverse rotation", m_sign)):
        assert (m != pin).any(), name
