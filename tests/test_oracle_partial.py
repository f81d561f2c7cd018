"""Pins for the oracle's key-range partial attention and the merge of
partials: a scalar brute force of one partial, and the identity that merging
the partials of any split of the keys gives the whole-sequence forward
(computed by the oracle's independent full forward)."""

import math

import numpy as np
import pytest

import oracle

BASE = 10000.0


def test_partial_matches_scalar_brute_force():
    rng = np.random.default_rng(20)
    L, d, s, lo, hi = 6, 4, 0.9, 2, 5
    q, k, v = (rng.standard_normal((L, d)) for _ in range(3))
    O, lse = oracle.attention_forward_partial_slice(q, k, v, s, BASE, lo, hi, mode="exact")

    def rot(x, p):
        out = [0.0] * d
        for j in range(d // 2):
            a = p * BASE ** (-2.0 * j / d)
            c, sn = math.cos(a), math.sin(a)
            out[j] = x[j] * c - x[j + d // 2] * sn
            out[j + d // 2] = x[j + d // 2] * c + x[j] * sn
        return out

    for i in range(L):
        qi = rot(list(q[i]), i)
        sc = {j: s * sum(a * b for a, b in zip(qi, rot(list(k[j]), j))) for j in range(lo, hi)}
        z = sum(math.exp(x) for x in sc.values())
        assert abs(math.log(z) - lse[i]) < 1e-12
        for c in range(d):
            o = sum(math.exp(sc[j]) / z * v[j][c] for j in range(lo, hi))
            assert abs(o - O[i, c]) < 1e-12


@pytest.mark.parametrize("L,cuts", [(9, [4]), (40, [7, 8, 31]), (64, [0, 16, 64]), (5, [])])
@pytest.mark.parametrize("mode", ["exact", "bf16_operands"])
def test_merge_of_a_key_split_is_the_full_forward(L, cuts, mode):
    rng = np.random.default_rng(L + len(cuts))
    d, s = 16, 0.4
    q, k, v = (rng.standard_normal((L, d)) for _ in range(3))
    edges = [0] + cuts + [L]
    parts = [oracle.attention_forward_partial_slice(q, k, v, s, BASE, a, b, mode=mode)
             for a, b in zip(edges, edges[1:])]
    O, lse = oracle.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    O_full, lse_full = oracle.attention_forward_slice(q, k, v, s, BASE, mode=mode)
    np.testing.assert_allclose(O, O_full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_full, rtol=0, atol=1e-12)


def test_empty_range_and_merge_identities():
    rng = np.random.default_rng(3)
    L, d = 7, 8
    q, k, v = (rng.standard_normal((L, d)) for _ in range(3))
    Oe, le = oracle.attention_forward_partial_slice(q, k, v, 0.3, BASE, 4, 4)
    assert (Oe == 0).all() and np.isneginf(le).all()
    Oa, la = oracle.attention_forward_partial_slice(q, k, v, 0.3, BASE, 0, 7)
    # one part is the identity; an empty part adds nothing; order does not matter
    O1, l1 = oracle.merge_partials([Oa], [la])
    np.testing.assert_array_equal(O1, Oa)
    np.testing.assert_array_equal(l1, la)
    O2, l2 = oracle.merge_partials([Oe, Oa], [le, la])
    np.testing.assert_allclose(O2, Oa, atol=1e-15)
    np.testing.assert_allclose(l2, la, atol=1e-15)
    Ob, lb = oracle.attention_forward_partial_slice(q, k, v, 0.3, BASE, 0, 3)
    Oc, lc = oracle.attention_forward_partial_slice(q, k, v, 0.3, BASE, 3, 7)
    Ox, lx = oracle.merge_partials([Ob, Oc], [lb, lc])
    Oy, ly = oracle.merge_partials([Oc, Ob], [lc, lb])
    np.testing.assert_allclose(Ox, Oy, atol=1e-15)
    np.testing.assert_allclose(lx, ly, atol=1e-15)
    # all parts empty: O = 0, LSE = -inf
    Oz, lz = oracle.merge_partials([Oe, Oe], [le, le])
    assert (Oz == 0).all() and np.isneginf(lz).all()
