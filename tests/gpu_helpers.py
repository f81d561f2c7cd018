"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding on seeded inputs and compare with the float64 oracle."""

import math
import sys

import numpy as np
import torch

import oracle
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


def ulp_bf16(x):
    """Spacing of the bf16 grid at |x| (2^(e-7) for |x| in [2^e, 2^(e+1)))."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


O_ATOL = 1e-2     # max-abs error allowed on O
G_RELF = 2e-2     # relative Frobenius error allowed on dq, dk, dv
# max-abs error on LSE (diagnostic; no stated tolerance): the forward's
# normaliser is the sum of the bf16-rounded probabilities its P V product
# used, each within 2^-8 relative of exact, so its log is within
# ln(1 + 2^-8) = 3.9e-3 of the exact LSE; 1e-4 covers the fp32 terms
LSE_ATOL = math.log1p(2.0 ** -8) + 1e-4


def relf(a, b):
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (n if n > 0 else 1.0)


def compare(gpu, inp, seqs=None, heads=None, exact_too=True, scale=None, rope_base=None,
            with_bwd=True, label=""):
    """Oracle on the listed (sequence, head) slices; asserts the tolerances.
    O: |O_gpu - O_ref| <= 1e-2 + ulp/2 elementwise against the bf16-operand
    oracle (bf16 storage of O alone can err by half an ulp); dq/dk/dv: relative
    Frobenius <= 2e-2. The exact-rotation oracle is always reported; with
    exact_too the literal bounds must also hold against it."""
    for name, t in gpu.items():   # NaN / Inf scan of every output, compared rows or not
        assert np.isfinite(t).all(), (label, name)
    q, k, v, do = oracle_inputs(inp)
    cu = inp["cu_seqlens"]
    s = inp["scale"] if scale is None else scale
    base = inp["rope_base"] if rope_base is None else rope_base
    modes = ["bf16_operands", "exact"]
    T = inp["T"]
    seqs = list(range(len(cu) - 1)) if seqs is None else list(seqs)
    heads = list(range(inp["H"])) if heads is None else list(heads)
    rows = np.zeros(T, bool)
    for b in seqs:
        rows[cu[b]:cu[b + 1]] = True
    report = {}
    for mode in modes:
        O, LSE = oracle.forward(q, k, v, cu, s, base, mode=mode, seqs=seqs, heads=heads)
        og, orf = gpu["o"][rows][:, heads], O[rows][:, heads]
        err = np.abs(og - orf)
        report[mode + ".o_maxabs"] = float(err.max()) if err.size else 0.0
        if mode == "bf16_operands":
            bound = O_ATOL + 0.5 * ulp_bf16(orf)
            ex = err - bound
            if ex.size and ex.max() > 0:
                at = np.unravel_index(int(ex.argmax()), ex.shape)
                raise AssertionError((label, mode, "excess", float(ex.max()), "at", at,
                                      "gpu", float(og[at]), "oracle", float(orf[at]),
                                      "elements over", int((ex > 0).sum()), "of", ex.size))
            lerr = np.abs(gpu["lse"][heads][:, rows] - LSE[heads][:, rows])
            report["lse_maxabs"] = float(lerr.max()) if lerr.size else 0.0
            assert report["lse_maxabs"] <= LSE_ATOL, (label, report)
        elif exact_too:
            assert report[mode + ".o_maxabs"] <= O_ATOL, (label, mode, report)
        if with_bwd:
            dq, dk, dv = oracle.backward(q, k, v, do, cu, s, base, mode=mode, seqs=seqs,
                                         heads=heads)
            for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
                e = relf(gpu[name][rows][:, heads], ref[rows][:, heads])
                report["%s.%s_relf" % (mode, name)] = float(e)
                if mode == "bf16_operands" or exact_too:
                    assert e <= G_RELF, (label, mode, name, e)
    say(label, {k_: "%.3g" % v_ for k_, v_ in report.items()})
    return report
