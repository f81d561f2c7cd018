"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding on seeded inputs and compare with the float64 oracle."""

import math
import sys

import numpy as np
import torch

import oracle
from oracle import tolerances as T
from protein_language_model_amd import esm_attn as E


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits, device):
    return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)


def to_f64(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32)


def bf16_f64(t):
    return (to_f64(t) << 16).view(np.float32).astype(np.float64)


def run_gpu(inp, device, scale=None, rope_base=None, with_bwd=True):
    q, k, v = (to_dev(inp[n], device) for n in ("q", "k", "v"))
    cu = torch.from_numpy(inp["cu_seqlens"].astype(np.int32)).to(device)
    maxL = max(inp["lengths"]) if inp["lengths"] else 0
    scale = inp["scale"] if scale is None else scale
    base = inp["rope_base"] if rope_base is None else rope_base
    o, lse = E.esm_attn_fwd(q, k, v, cu, maxL, scale, base)
    out = dict(o=o, lse=lse)
    if with_bwd:
        do = to_dev(inp["do"], device)
        dq, dk, dv = E.esm_attn_bwd(q, k, v, o, do, lse, cu, maxL, scale, base)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: (bf16_f64(t) if t.dtype == torch.bfloat16 else t.cpu().numpy().astype(np.float64))
            for n, t in out.items()}


def oracle_inputs(inp):
    return tuple(oracle.bf16_bits_to_f64(inp[n]) for n in ("q", "k", "v", "do"))


ulp_bf16 = T.ulp_bf16
relf = T.relf
O_ATOL, G_RELF, LSE_ATOL = T.O_ATOL, T.G_RELF, T.LSE_ATOL


def compare(gpu, inp, seqs=None, heads=None, sharpened=False, grads_exact=True, scale=None,
            rope_base=None, with_bwd=True, label=""):
    """Oracle on the listed (sequence, head) slices; asserts the bounds of
    oracle.tolerances against both precision modes of the oracle.

    exact (float64 operands, the definition):
      dq, dk, dv: relative Frobenius <= 2e-2 (unless grads_exact is False);
      O: elementwise <= 1e-2 + ulp/2 (O is stored in bf16: even the exact O
      rounds by up to half an ulp, oracle.tolerances.o_bound; below |O| = 2
      that is at most 2^-8 over the literal 1e-2), except on a sharpened
      softmax (sharpened=True:
      q, k x 3 or a scale several times 1/sqrt(d)), where rounding the
      rotated operands to bf16 alone moves O by about 0.1 for any kernel that
      feeds bf16 matrix units; there the exact-mode O error is reported, not
      asserted.
    bf16_operands (the operands rounded as the kernels round them):
      O elementwise <= 1e-2 + ulp/2; LSE max-abs <= ln(1 + 2^-8) + 1e-4;
      dq, dk, dv relative Frobenius <= 2e-2."""
    for name, t in gpu.items():   # NaN / Inf scan of every output, compared rows or not
        assert np.isfinite(t).all(), (label, name)
    q, k, v, do = oracle_inputs(inp)
    cu = inp["cu_seqlens"]
    s = inp["scale"] if scale is None else scale
    base = inp["rope_base"] if rope_base is None else rope_base
    Tn = inp["T"]
    seqs = list(range(len(cu) - 1)) if seqs is None else list(seqs)
    heads = list(range(inp["H"])) if heads is None else list(heads)
    rows = np.zeros(Tn, bool)
    for b in seqs:
        rows[cu[b]:cu[b + 1]] = True
    report = {}
    for mode in ("exact", "bf16_operands"):
        O, LSE = oracle.forward(q, k, v, cu, s, base, mode=mode, seqs=seqs, heads=heads)
        og, orf = gpu["o"][rows][:, heads], O[rows][:, heads]
        err = np.abs(og - orf)
        report[mode + ".o_maxabs"] = float(err.max()) if err.size else 0.0
        lerr = np.abs(gpu["lse"][heads][:, rows] - LSE[heads][:, rows])
        report[mode + ".lse_maxabs"] = float(lerr.max()) if lerr.size else 0.0
        if mode == "bf16_operands" or not sharpened:
            ex = err - T.o_bound(orf)
            if ex.size and ex.max() > 0:
                at = np.unravel_index(int(ex.argmax()), ex.shape)
                raise AssertionError((label, mode, "excess", float(ex.max()), "at", at,
                                      "gpu", float(og[at]), "oracle", float(orf[at]),
                                      "elements over", int((ex > 0).sum()), "of", ex.size))
        if mode == "bf16_operands":
            assert report[mode + ".lse_maxabs"] <= LSE_ATOL, (label, report)
        if with_bwd:
            dq, dk, dv = oracle.backward(q, k, v, do, cu, s, base, mode=mode, seqs=seqs,
                                         heads=heads)
            for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
                e = relf(gpu[name][rows][:, heads], ref[rows][:, heads])
                report["%s.%s_relf" % (mode, name)] = e
                if mode == "bf16_operands" or grads_exact:
                    assert e <= G_RELF, (label, mode, name, e, report)
    say(label, {k_: "%.3g" % v_ for k_, v_ in report.items()})
    return report
