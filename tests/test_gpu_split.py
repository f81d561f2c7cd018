"""GPU parity of the split-KV forward (key-range partials + merge) and of the
merge of external partials, through the C ABI, with the float64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import compare, run_gpu, say, to_dev, bf16_f64, oracle_inputs, ulp_bf16, LSE_ATOL
from protein_language_model_amd import workloads as W
from protein_language_model_amd import esm_attn as E

pytestmark = pytest.mark.gpu

NAMES = {16: "esm2_8m", 32: "esm2_150m", 64: "esm2_650m", 128: "esm2_15b"}


def _split_run(inp, device, n_split, with_bwd=False):
    T, H, d, B = inp["T"], inp["H"], inp["d"], len(inp["lengths"])
    maxL, scale, base = max(inp["lengths"]), inp["scale"], inp["rope_base"]
    q, k, v = (to_dev(inp[x], device) for x in ("q", "k", "v"))
    cu = torch.from_numpy(inp["cu_seqlens"]).to(device)
    plan = E.esm_attn_plan(cu, T, maxL, H, d, base)
    qr, kr = E.esm_attn_rotate_planned(q, k, B, maxL, plan, base, softmax_scale=scale)
    o, lse, op, lp = E.esm_attn_fwd_split_planned(qr, kr, v, B, maxL, plan, n_split, scale)
    out = dict(o=o, lse=lse)
    if with_bwd:
        do = to_dev(inp["do"], device)
        dq, dk, dv, _ = E.esm_attn_bwd_planned(qr, kr, v, o, do, lse, B, maxL, plan, scale, base)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    res = {n: (bf16_f64(t) if t.dtype == torch.bfloat16 else t.cpu().numpy().astype(np.float64))
           for n, t in out.items()}
    return res, op.cpu().numpy().astype(np.float64), lp.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d,n_split", [(16, 3), (32, 2), (64, 2), (64, 7), (128, 4)])
def test_split_forward_and_partials(device, d, n_split):
    inp = W.make_inputs(NAMES[d], lengths=[300, 1, 129, 64, 0, 77, 1100], num_heads=3)
    say("case split", d, n_split)
    gpu, op, lp = _split_run(inp, device, n_split)
    compare(gpu, inp, with_bwd=False, label="split d%d R%d" % (d, n_split))
    # every chunk of sampled (sequence, head) pairs against the oracle partial
    q, k, v, _ = oracle_inputs(inp)
    cu, s, base = inp["cu_seqlens"], inp["scale"], inp["rope_base"]
    bn = 32 if d == 128 else 64
    for b in (0, 3, 6):
        a, e = int(cu[b]), int(cu[b + 1])
        L = e - a
        per = -(-(-(-L // bn)) // n_split)
        for h in (0, 2):
            for r in range(n_split):
                lo, hi = min(r * per * bn, L), min((r + 1) * per * bn, L)
                Oref, lref = oracle.attention_forward_partial_slice(
                    q[a:e, h], k[a:e, h], v[a:e, h], s, base, lo, hi)
                Og, lg = op[r, a:e, h], lp[r, h, a:e]
                if hi <= lo:
                    assert (Og == 0).all() and np.isneginf(lg).all()
                else:
                    assert np.abs(Og - Oref).max() <= 1e-2
                    assert np.abs(lg - lref).max() <= LSE_ATOL


@pytest.mark.parametrize("d", [16, 64, 128])
def test_split_one_is_the_plain_forward(device, d):
    inp = W.make_inputs(NAMES[d], lengths=[300, 1, 129, 64, 77], num_heads=2)
    gpu, _, _ = _split_run(inp, device, 1)
    ref = run_gpu(inp, device, with_bwd=False)
    np.testing.assert_array_equal(gpu["o"], ref["o"])
    np.testing.assert_array_equal(gpu["lse"], ref["lse"])


def test_backward_after_split_forward(device):
    """The training path with the split forward: its O and LSE feed the
    backward; gradients within the tolerances."""
    inp = W.make_inputs("esm2_650m", lengths=[500, 129, 64, 1], num_heads=2)
    gpu, _, _ = _split_run(inp, device, 3, with_bwd=True)
    compare(gpu, inp, label="split then backward")


@pytest.mark.parametrize("d,R", [(16, 1), (64, 5), (128, 3)])
def test_merge_of_external_partials(device, d, R):
    """Random fp32 partials (as another device would send them), some parts
    and one whole row empty (-inf)."""
    rng = np.random.default_rng(40 + d + R)
    T, H = 37, 3
    op = rng.standard_normal((R, T, H, d)).astype(np.float32)
    lp = (rng.standard_normal((R, H, T)) * 4).astype(np.float32)
    lp[rng.random((R, H, T)) < 0.3] = -np.inf
    lp[:, 1, 5] = -np.inf
    op_t, lp_t = torch.from_numpy(op).to(device), torch.from_numpy(lp).to(device)
    o, lse = E.esm_attn_merge_partials(op_t, lp_t)
    torch.cuda.synchronize()
    og, lg = bf16_f64(o), lse.cpu().numpy().astype(np.float64)
    for h in range(H):
        Oref, lref = oracle.merge_partials(op[:, :, h].astype(np.float64),
                                           lp[:, h].astype(np.float64))
        fin = np.isfinite(lref)
        assert (np.isneginf(lg[h]) == ~fin).all()
        assert (og[:, h][~fin] == 0).all()
        np.testing.assert_allclose(lg[h][fin], lref[fin], rtol=0, atol=1e-5 * (1 + np.abs(lref[fin])).max())
        err = np.abs(og[:, h][fin] - Oref[fin])
        assert (err <= 0.5 * ulp_bf16(Oref[fin]) + 1e-5 * np.abs(Oref[fin]).max()).all()
