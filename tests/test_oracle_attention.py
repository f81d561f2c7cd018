"""Pins for the oracle's forward and backward attention: closed forms,
invariants, a scalar brute force, torch's CPU scaled-dot-product attention
and autograd in float64, and central finite differences."""

import math

import numpy as np
import pytest
import torch

import oracle

BASE = 10000.0


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _rope_torch(x, base):
    """Rotary embedding in torch via complex multiplication (independent of
    the oracle's real-arithmetic form), positions 0..L-1 on axis 0."""
    L, d = x.shape
    h = d // 2
    j = torch.arange(h, dtype=torch.float64)
    ang = torch.arange(L, dtype=torch.float64)[:, None] * base ** (-2.0 * j / d)
    z = torch.complex(x[:, :h], x[:, h:]) * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=1)


# ---------------------------------------------------------------- forward

def test_forward_matches_scalar_brute_force():
    rng = np.random.default_rng(10)
    L, d, s = 5, 4, 0.7
    q, k, v = _rand(rng, L, d), _rand(rng, L, d), _rand(rng, L, d)
    O, lse = oracle.attention_forward_slice(q, k, v, s, BASE, mode="exact")

    def rot(x, p):
        out = [0.0] * d
        for j in range(d // 2):
            a = p * BASE ** (-2.0 * j / d)
            c, sn = math.cos(a), math.sin(a)
            out[j] = x[j] * c - x[j + d // 2] * sn
            out[j + d // 2] = x[j + d // 2] * c + x[j] * sn
        return out

    qr = [rot(list(q[i]), i) for i in range(L)]
    kr = [rot(list(k[i]), i) for i in range(L)]
    for i in range(L):
        sc = [s * sum(qr[i][c] * kr[j][c] for c in range(d)) for j in range(L)]
        z = sum(math.exp(x) for x in sc)
        assert abs(math.log(z) - lse[i]) < 1e-12
        for c in range(d):
            o = sum(math.exp(sc[j]) / z * v[j][c] for j in range(L))
            assert abs(o - O[i, c]) < 1e-12


@pytest.mark.parametrize("L,d", [(1, 8), (7, 16), (33, 64)])
def test_forward_matches_torch_sdpa_float64(L, d):
    rng = np.random.default_rng(L * 100 + d)
    q, k, v = _rand(rng, L, d), _rand(rng, L, d), _rand(rng, L, d)
    s = 1.0 / math.sqrt(d)
    O, lse = oracle.attention_forward_slice(q, k, v, s, BASE, mode="exact")
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    qr, kr = _rope_torch(tq, BASE), _rope_torch(tk, BASE)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qr[None, None], kr[None, None], tv[None, None], scale=s)[0, 0]
    np.testing.assert_allclose(O, ref.numpy(), atol=1e-12)
    ref_lse = torch.logsumexp(s * qr @ kr.T, dim=1)
    np.testing.assert_allclose(lse, ref_lse.numpy(), atol=1e-12)


def test_probability_rows_sum_to_one():
    rng = np.random.default_rng(11)
    L, d = 40, 32
    q, k, v, do = (_rand(rng, L, d) * 3 for _ in range(4))
    *_, it = oracle.attention_backward_slice(q, k, v, do, 0.3, BASE,
                                             return_intermediates=True)
    np.testing.assert_allclose(it["P"].sum(axis=1), 1.0, atol=1e-13)
    assert (it["P"] >= 0).all()


def test_constant_v_gives_v_and_single_key_gives_v():
    rng = np.random.default_rng(12)
    L, d = 20, 16
    q, k = _rand(rng, L, d), _rand(rng, L, d)
    row = _rand(rng, d)
    O, _ = oracle.attention_forward_slice(q, k, np.tile(row, (L, 1)), 0.25, BASE)
    np.testing.assert_allclose(O, np.tile(row, (L, 1)), atol=1e-13)
    q1, k1, v1 = _rand(rng, 1, d), _rand(rng, 1, d), _rand(rng, 1, d)
    s = 0.37
    O1, lse1 = oracle.attention_forward_slice(q1, k1, v1, s, BASE, mode="exact")
    np.testing.assert_allclose(O1, v1, atol=1e-15)
    # position 0: the rotation is the identity, so LSE = s * q.k
    np.testing.assert_allclose(lse1, [s * float(q1[0] @ k1[0])], atol=1e-14)


def test_zero_scale_gives_mean_and_log_length():
    rng = np.random.default_rng(13)
    L, d = 9, 8
    q, k, v = _rand(rng, L, d), _rand(rng, L, d), _rand(rng, L, d)
    O, lse = oracle.attention_forward_slice(q, k, v, 0.0, BASE)
    np.testing.assert_allclose(O, np.tile(v.mean(axis=0), (L, 1)), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(L), atol=1e-14)


def test_linear_in_v_and_invariant_to_key_permutation():
    rng = np.random.default_rng(14)
    L, d = 25, 16
    q, k, v = _rand(rng, L, d), _rand(rng, L, d), _rand(rng, L, d)
    O, lse = oracle.attention_forward_slice(q, k, v, 0.5, 0.0)
    O2, _ = oracle.attention_forward_slice(q, k, -2.5 * v, 0.5, 0.0)
    np.testing.assert_allclose(O2, -2.5 * O, atol=1e-13)
    perm = rng.permutation(L)
    # without rotation a key's position carries no information
    Op, lsep = oracle.attention_forward_slice(q, k[perm], v[perm], 0.5, 0.0)
    np.testing.assert_allclose(Op, O, atol=1e-13)
    np.testing.assert_allclose(lsep, lse, atol=1e-13)


def test_sequences_never_attend_across_boundaries():
    rng = np.random.default_rng(15)
    lengths = [3, 1, 6, 4]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, H, d = int(cu[-1]), 2, 8
    q, k, v = _rand(rng, T, H, d), _rand(rng, T, H, d), _rand(rng, T, H, d)
    O, lse = oracle.forward(q, k, v, cu, 0.4, BASE)
    # perturb sequence 2 only
    a, e = cu[2], cu[3]
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[a:e] += 5.0
    k2[a:e] -= 3.0
    v2[a:e] *= 7.0
    O2, lse2 = oracle.forward(q2, k2, v2, cu, 0.4, BASE)
    keep = np.ones(T, bool)
    keep[a:e] = False
    np.testing.assert_array_equal(O2[keep], O[keep])
    np.testing.assert_array_equal(lse2[:, keep], lse[:, keep])
    assert not np.allclose(O2[a:e], O[a:e])
    # each sequence equals the slice function with positions from 0
    for b in range(len(lengths)):
        s0, s1 = cu[b], cu[b + 1]
        o, l = oracle.attention_forward_slice(q[s0:s1, 1], k[s0:s1, 1],
                                              v[s0:s1, 1], 0.4, BASE)
        np.testing.assert_array_equal(O[s0:s1, 1], o)


def test_empty_sequences_are_legal():
    rng = np.random.default_rng(16)
    lengths = [0, 4, 0, 0, 2, 0]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q, k, v = (_rand(rng, 6, 1, 4) for _ in range(3))
    O, lse = oracle.forward(q, k, v, cu, 1.0, BASE)
    assert np.isfinite(O).all() and np.isfinite(lse).all()
    O0, _ = oracle.forward(q[:0], k[:0], v[:0], np.zeros(3, int), 1.0, BASE)
    assert O0.shape == (0, 1, 4)


def test_precision_modes():
    rng = np.random.default_rng(17)
    L, d = 30, 16
    bits = lambda x: oracle.round_to_bf16(x)
    q, k, v = bits(_rand(rng, L, d)), bits(_rand(rng, L, d)), _rand(rng, L, d)
    # a scale whose c = fl32(scale * fl32(log2 e)) is exactly 1/4: without
    # rotation c * q is then exact in bf16, so the two modes compute the same
    # scores up to the float32 rounding of the scale itself (a wrong factor,
    # log2 e for ln 2, or a dropped scale would show here)
    s = np.float32(0.25 / np.log2(np.e))
    while np.float32(s) * np.float32(np.log2(np.e)) != np.float32(0.25):
        s = np.nextafter(s, np.float32(1.0))
    a, la = oracle.attention_forward_slice(q, k, v, float(s), 0.0, mode="exact")
    b, lb = oracle.attention_forward_slice(q, k, v, float(s), 0.0, mode="bf16_operands")
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-6)
    np.testing.assert_allclose(la, lb, rtol=0, atol=1e-6)
    # with rotation they differ by the rounding of the rotated operands only
    a, _ = oracle.attention_forward_slice(q, k, v, 0.25, BASE, mode="exact")
    b, _ = oracle.attention_forward_slice(q, k, v, 0.25, BASE, mode="bf16_operands")
    assert 0 < np.abs(a - b).max() < 0.05
    *_, it = oracle.attention_backward_slice(q, k, v, v, 0.25, BASE,
                                             return_intermediates=True)
    qhat = it["q_scaled"] / np.log(2.0)
    np.testing.assert_allclose(qhat, oracle.round_to_bf16(qhat), rtol=1e-15, atol=0)
    np.testing.assert_array_equal(it["k_rot"], oracle.round_to_bf16(it["k_rot"]))
    with pytest.raises(ValueError):
        oracle.attention_forward_slice(q, k, v, 0.25, BASE, mode="fp8")


# ---------------------------------------------------------------- backward

def _loss(q, k, v, do, s, base):
    O, _ = oracle.attention_forward_slice(q, k, v, s, base, mode="exact")
    return float((O * do).sum())


@pytest.mark.parametrize("L,d,base", [(1, 2, BASE), (3, 4, BASE), (5, 8, BASE),
                                      (5, 8, 3.0), (4, 4, 0.0)])
def test_backward_matches_central_finite_differences(L, d, base):
    rng = np.random.default_rng(L * 10 + d)
    q, k, v, do = (_rand(rng, L, d) for _ in range(4))
    s = 0.8
    dq, dk, dv = oracle.attention_backward_slice(q, k, v, do, s, base, mode="exact")
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], do, s, base)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], do, s, base)
            num[idx] = (fp - fm) / (2 * eps)
        err = np.abs(num - g).max() / max(1.0, np.abs(g).max())
        assert err < 1e-7, (name, err)


@pytest.mark.parametrize("L,d", [(6, 8), (40, 64)])
def test_backward_matches_torch_autograd_float64(L, d):
    rng = np.random.default_rng(L + d)
    q, k, v, do = (_rand(rng, L, d) for _ in range(4))
    s = 1.0 / math.sqrt(d)
    dq, dk, dv = oracle.attention_backward_slice(q, k, v, do, s, BASE, mode="exact")
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        _rope_torch(tq, BASE)[None, None], _rope_torch(tk, BASE)[None, None],
        tv[None, None], scale=s)[0, 0]
    out.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_backward_identities():
    rng = np.random.default_rng(18)
    L, d = 17, 16
    q, k, v, do = (_rand(rng, L, d) for _ in range(4))
    s = 0.6
    dq, dk, dv, it = oracle.attention_backward_slice(
        q, k, v, do, s, BASE, return_intermediates=True)
    # each row of dS sums to zero, so the rotated-space key gradients do too
    np.testing.assert_allclose(it["dS"].sum(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose(it["dk_rot"].sum(axis=0), 0.0, atol=1e-12)
    # probabilities sum to one per query, so dV sums to the sum of dO
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
    # D = rowsum(P * dP) = rowsum(dO * O)
    O, _ = oracle.attention_forward_slice(q, k, v, s, BASE)
    np.testing.assert_allclose(it["D"], (do * O).sum(axis=1), atol=1e-12)
    # gradients are linear in dO
    g2 = oracle.attention_backward_slice(q, k, v, -3.0 * do, s, BASE)
    for a, b in zip(g2, (dq, dk, dv)):
        np.testing.assert_allclose(a, -3.0 * b, atol=1e-12)


def test_packed_backward_equals_per_sequence():
    rng = np.random.default_rng(19)
    lengths = [4, 0, 7, 1]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, H, d = int(cu[-1]), 3, 8
    q, k, v, do = (_rand(rng, T, H, d) for _ in range(4))
    dq, dk, dv = oracle.backward(q, k, v, do, cu, 0.5, BASE)
    for b in range(len(lengths)):
        a, e = cu[b], cu[b + 1]
        for h in range(H):
            g = oracle.attention_backward_slice(q[a:e, h], k[a:e, h], v[a:e, h],
                                                do[a:e, h], 0.5, BASE)
            np.testing.assert_array_equal(dq[a:e, h], g[0])
            np.testing.assert_array_equal(dk[a:e, h], g[1])
            np.testing.assert_array_equal(dv[a:e, h], g[2])


@pytest.mark.parametrize("mode", ["exact", "bf16_operands"])
def test_row_restricted_forward_and_dq_equal_the_full_slice(mode):
    """attention_rows_slice is the full-slice definition restricted to some
    query rows (the full slice is pinned above by a brute force, torch and
    finite differences)."""
    rng = np.random.default_rng(30)
    L, d, s = 70, 16, 0.3
    q, k, v, do = (rng.standard_normal((L, d)) for _ in range(4))
    rows = [0, 1, 33, 69]
    O, lse = oracle.attention_forward_slice(q, k, v, s, BASE, mode=mode)
    dq, _, _ = oracle.attention_backward_slice(q, k, v, do, s, BASE, mode=mode)
    Or, lr, dqr = oracle.attention_rows_slice(q, k, v, do, s, BASE, rows, mode=mode)
    np.testing.assert_allclose(Or, O[rows], atol=1e-12)
    np.testing.assert_allclose(lr, lse[rows], atol=1e-12)
    np.testing.assert_allclose(dqr, dq[rows], atol=1e-12)
