"""GPU parity of the FP8 (E4M3) path through the C ABI: the quantized q8, k8
bit for bit against the oracle's float32 quantization, and the FP8 forward
against the oracle on the same E4M3 operands at the bf16 forward's bounds
(plus the quantization's own error against the unquantized oracle)."""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as F8
from gpu_helpers import say, to_dev, bf16_f64, oracle_inputs, ulp_bf16, LSE_ATOL
from protein_language_model_amd import workloads as W
from protein_language_model_amd import esm_attn as E

pytestmark = pytest.mark.gpu

NAMES = {64: "esm2_650m", 128: "esm2_15b"}


def _setup(device, d, lengths, H, rope_base=None):
    inp = W.make_inputs(NAMES[d], lengths=lengths, num_heads=H)
    base = inp["rope_base"] if rope_base is None else rope_base
    T, B, maxL = inp["T"], len(lengths), max(lengths)
    q, k, v = (to_dev(inp[x], device) for x in ("q", "k", "v"))
    cu = torch.from_numpy(inp["cu_seqlens"]).to(device)
    plan = E.esm_attn_plan(cu, T, maxL, H, d, base)
    return inp, base, T, B, maxL, q, k, v, plan


@pytest.mark.parametrize("d", [64, 128])
def test_quantization_is_bitwise_the_oracle(device, d):
    inp, base, T, B, maxL, q, k, v, plan = _setup(device, d, [300, 1, 129, 77, 0, 64], 3)
    qo, ko, _, _ = oracle_inputs(inp)
    # q: half the no-saturation scale (some values saturate at 448); k: a
    # coarse scale (many subnormal and zero codes)
    qs = float(np.abs(qo).max()) * math.sqrt(2) / 448 * 0.5
    ks = float(np.abs(ko).max()) * math.sqrt(2) / 448 * 64
    say("case fp8 quantization", d, qs, ks)
    q8, k8 = E.esm_attn_quantize_fp8_planned(q, k, B, maxL, plan, qs, ks, base)
    torch.cuda.synchronize()
    q8v, k8v = (F8.decode_e4m3(t.cpu().numpy()) for t in (q8, k8))
    cu = inp["cu_seqlens"]
    saturated = 0
    for b in range(B):
        a, e = int(cu[b]), int(cu[b + 1])
        for h in range(3):
            rq = F8.quantize_rotated(qo[a:e, h], base, qs)
            rk = F8.quantize_rotated(ko[a:e, h], base, ks)
            np.testing.assert_array_equal(q8v[a:e, h], rq)
            np.testing.assert_array_equal(k8v[a:e, h], rk)
            saturated += int((np.abs(rq) == 448).sum())
    assert saturated > 0 and (np.abs(k8v[np.nonzero(k8v)]) < 2 ** -6).any()


@pytest.mark.parametrize("d,scale,rope_base", [(64, None, None), (128, None, None),
                                               (64, -0.2, None), (64, 0.125, 0.0)])
def test_fp8_forward_parity(device, d, scale, rope_base):
    H = 3
    inp, base, T, B, maxL, q, k, v, plan = _setup(device, d, [300, 1, 129, 77, 0, 640], H,
                                                  rope_base)
    s = inp["scale"] if scale is None else scale
    qo, ko, vo, _ = oracle_inputs(inp)
    qs = float(np.abs(qo).max()) * math.sqrt(2) / 448
    ks = float(np.abs(ko).max()) * math.sqrt(2) / 448
    say("case fp8 forward", d, s, base)
    q8, k8 = E.esm_attn_quantize_fp8_planned(q, k, B, maxL, plan, qs, ks, base)
    o, lse = E.esm_attn_fwd_fp8_planned(q8, k8, v, B, maxL, plan, qs, ks, s)
    torch.cuda.synchronize()
    og, lg = bf16_f64(o), lse.cpu().numpy().astype(np.float64)
    cu = inp["cu_seqlens"]
    worst_exact = 0.0
    for b in range(B):
        a, e = int(cu[b]), int(cu[b + 1])
        if e == a:
            continue
        for h in range(H):
            Oref, lref = F8.attention_forward_fp8_slice(qo[a:e, h], ko[a:e, h], vo[a:e, h], s,
                                                       base, qs, ks)
            err = np.abs(og[a:e, h] - Oref)
            assert (err <= 1e-2 + 0.5 * ulp_bf16(Oref)).all(), (b, h, float(err.max()))
            assert np.abs(lg[h, a:e] - lref).max() <= LSE_ATOL
            # against the unquantized forward: if quantization moves every
            # logit of a row by at most D, each P changes by a factor within
            # exp(+-2D), so |O - O_exact| <= (exp(2D) - 1) max|v| (plus the
            # kernel's own bound)
            Ox, _ = oracle.attention_forward_slice(qo[a:e, h], ko[a:e, h], vo[a:e, h], s, base,
                                                   mode="exact")
            rq = oracle.rope_rotate(qo[a:e, h], np.arange(e - a), base)
            rk = oracle.rope_rotate(ko[a:e, h], np.arange(e - a), base)
            q8 = F8.quantize_rotated(qo[a:e, h], base, qs)
            k8 = F8.quantize_rotated(ko[a:e, h], base, ks)
            dS = s * np.float32(qs) * np.float32(ks) * (q8 @ k8.T) - s * (rq @ rk.T)
            bound = np.expm1(2 * np.abs(dS).max(axis=1)) * np.abs(vo[a:e, h]).max()
            ex = np.abs(og[a:e, h] - Ox)
            assert (ex <= bound[:, None] + 1e-2 + 0.5 * ulp_bf16(Ox)).all()
            worst_exact = max(worst_exact, float(ex.max()))
    say("fp8 forward: max |O - O_exact| =", worst_exact)
