"""The small-batch path: batches whose sequences all fit one 128-row work item
(max_seqlen <= 128, head_dim <= 64) run the one-shot calls as one forward and
one backward launch, with no plan, no rotation pass and no dq pass. O, LSE,
dk and dv come from the same operations in the same order as the planned
kernels and are bitwise theirs; dq is formed from the dk/dv pass's dS, whose
dP - D sums the -D term first where the dq pass adds it last, so dq agrees
with the planned dq to fp32 rounding. All meet the oracle bounds."""

import numpy as np
import pytest
import torch

from gpu_helpers import bf16_f64, compare, relf, run_gpu, say, to_dev
from protein_language_model_amd import workloads as W
from protein_language_model_amd import esm_attn as E

pytestmark = pytest.mark.gpu

NAMES = {16: "esm2_8m", 32: "esm2_150m", 64: "esm2_650m"}


def _planned(inp, device, scale, base):
    T, H, d, B = inp["T"], inp["H"], inp["d"], len(inp["lengths"])
    maxL = max(inp["lengths"])
    q, k, v, do = (to_dev(inp[x], device) for x in ("q", "k", "v", "do"))
    cu = torch.from_numpy(inp["cu_seqlens"]).to(device)
    plan = E.esm_attn_plan(cu, T, maxL, H, d, base)
    qr, kr = E.esm_attn_rotate_planned(q, k, B, maxL, plan, base, softmax_scale=scale)
    o, lse = E.esm_attn_fwd_planned(qr, kr, v, B, maxL, plan, scale)
    dq, dk, dv, _ = E.esm_attn_bwd_planned(qr, kr, v, o, do, lse, B, maxL, plan, scale, base)
    torch.cuda.synchronize()
    out = {n: bf16_f64(t) for n, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv))}
    out["lse"] = lse.cpu().numpy().astype(np.float64)
    return out


def _same(small, ref):
    for n in ("o", "lse", "dk", "dv"):
        np.testing.assert_array_equal(small[n], ref[n], err_msg=n)
    # dq: the same products, dP - D rounded in the other order
    err = np.abs(small["dq"] - ref["dq"])
    say("small dq vs planned: max abs %.3g, elements differing %d of %d"
        % (err.max(), int((err > 0).sum()), err.size))
    assert relf(small["dq"], ref["dq"]) <= 1e-3


@pytest.mark.parametrize("d", [16, 32, 64])
@pytest.mark.parametrize("scale,base", [(None, 10000.0), (-0.2, 0.0), (0.6, 500.0)])
def test_small_path_equals_planned_path(device, d, scale, base):
    lengths = [128, 1, 0, 65, 64, 63, 100, 7, 33]
    inp = W.make_inputs(NAMES[d], lengths=lengths, num_heads=3)
    s = inp["scale"] if scale is None else scale
    say("case small path", d, s, base)
    small = run_gpu(inp, device, scale=s, rope_base=base)   # one-shot calls: small path
    ref = _planned(inp, device, s, base)                     # plan, rotation, three kernels
    _same(small, ref)
    compare(small, inp, scale=s, rope_base=base, sharpened=abs(s) > 0.2,
            label="small d%d s=%g base=%g" % (d, s, base))


def test_small_path_many_heads_and_sequences(device):
    rng = np.random.default_rng(12)
    lengths = [int(x) for x in rng.integers(0, 129, size=300)]
    inp = W.make_inputs("esm2_650m", lengths=lengths, num_heads=16)
    say("case small path wide", len(lengths), inp["T"])
    small = run_gpu(inp, device)
    ref = _planned(inp, device, inp["scale"], inp["rope_base"])
    _same(small, ref)
    compare(small, inp, seqs=[0, 1, 150, 299], heads=[0, 15], label="small wide")


def test_small_path_outputs_stay_in_bounds(device):
    """Guard bytes around every output of the small-path calls survive."""
    inp = W.make_inputs("esm2_150m", lengths=[100, 28, 128], num_heads=2)
    T, H, d = inp["T"], inp["H"], inp["d"]
    n, pad, poison = T * H * d, 4096, -1024.0
    q, k, v, do = (to_dev(inp[x], device) for x in ("q", "k", "v", "do"))
    cu = torch.from_numpy(inp["cu_seqlens"]).to(device)
    bufs = [torch.full((n + 2 * pad,), poison, dtype=torch.bfloat16, device=device)
            for _ in range(4)]
    bl = torch.full((H * T + 2 * pad,), poison, dtype=torch.float32, device=device)
    view = lambda b: b[pad:pad + n].view(T, H, d)
    lse = bl[pad:pad + H * T].view(H, T)
    o, _ = E.esm_attn_fwd(q, k, v, cu, 128, out=view(bufs[0]), lse=lse)
    E.esm_attn_bwd(q, k, v, o, do, lse, cu, 128, dq=view(bufs[1]), dk=view(bufs[2]),
                   dv=view(bufs[3]))
    torch.cuda.synchronize()
    for b in bufs + [bl]:
        f = b.float().cpu()
        assert (f[:pad] == poison).all() and (f[-pad:] == poison).all()
    ref = _planned(inp, device, inp["scale"], inp["rope_base"])
    _same({"o": bf16_f64(o), "lse": lse.cpu().numpy().astype(np.float64),
           "dq": bf16_f64(view(bufs[1])), "dk": bf16_f64(view(bufs[2])),
           "dv": bf16_f64(view(bufs[3]))}, ref)
