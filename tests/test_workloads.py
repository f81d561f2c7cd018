"""The seeded input recipe: determinism, shapes and length statistics of the
ESM-2-shaped workloads, the bf16 conversion, and the work counters."""

import numpy as np
import torch

from protein_language_model_amd import workloads as W


def test_inputs_are_deterministic_and_shaped():
    a = W.make_inputs("esm2_8m")
    b = W.make_inputs("esm2_8m")
    for key in ("q", "k", "v", "do", "cu_seqlens"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["lengths"] == [37, 64, 100, 128]
    assert a["T"] == 329 and a["q"].shape == (329, 20, 16)
    assert a["q"].dtype == np.uint16
    assert list(a["cu_seqlens"]) == [0, 37, 101, 201, 329]
    c = W.make_inputs("esm2_8m", seed=99)
    assert not np.array_equal(a["q"], c["q"])


def test_length_recipes():
    assert W.lengths_of("esm2_650m") == [1024] * 16
    assert W.lengths_of("esm2_15b") == [8192] * 4
    assert W.lengths_of("esm2_15b_ragged") == [8192, 1000, 31]
    L = W.lengths_of("esm2_150m")
    assert len(L) == 32 and L == sorted(L) and 50 <= min(L) and max(L) <= 1024
    # lognormal packing: seeds 0..2 give these batch sizes / token counts
    stats = [(len(x), sum(x)) for x in (W.lengths_of("esm2_3b", s) for s in range(3))]
    assert stats == [(168, 65410), (189, 65428), (175, 65178)]
    for s in range(3):
        x = W.lengths_of("esm2_3b", s)
        assert min(x) >= 30 and max(x) <= 1024 and sum(x) <= 65536


def test_qk_sharpening_scales_q_and_k_only():
    a = W.make_inputs("esm2_3b", lengths=[5, 3], num_heads=2)
    q = (a["q"].astype(np.uint32) << 16).view(np.float32)
    v = (a["v"].astype(np.uint32) << 16).view(np.float32)
    assert np.abs(q).std() > 2.0 * np.abs(v).std()


def test_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-3, 4, 100000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(W.f32_to_bf16_bits(x), want)


def test_counted_flops_and_bytes_by_hand():
    fwd, bwd = W.counted_flops([1024] * 16, 20, 64)
    assert fwd == 4 * 16 * 1024 * 1024 * 20 * 64 == 85_899_345_920
    assert bwd == 2.5 * fwd
    fb, bb = W.algorithmic_bytes(16384, 20, 64)
    e = 16384 * 20 * 64
    assert fb == 8 * e + 4 * 16384 * 20
    assert bb == 16 * e + 8 * 16384 * 20
