"""The autograd wrappers: `attention` (packed q, k, v) equals the one-shot
calls bit for bit, forward and backward; `attention_qkv` (fused projection
output, rotated in place) meets the oracle bounds on the projection's q, k, v
(output and dq, dk, dv, read back from the fused gradient) and gives the same
output and the same gradients of the projection's input and weight as the
packed path."""

import numpy as np
import pytest
import torch

from gpu_helpers import bf16_f64, compare, say, to_dev
from protein_language_model_amd import workloads as W
from protein_language_model_amd import esm_attn as E

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["esm2_150m", "esm2_650m", "esm2_15b"])
def test_attention_autograd_equals_one_shot(device, name):
    # d = 32 and 64 rotate q inside the forward, d = 128 in the rotation pass;
    # either way the wrapper and the one-shot calls agree bit for bit
    inp = W.make_inputs(name, lengths=[300, 1, 129, 0, 64], num_heads=2)
    say("case autograd", name)
    maxL, s, base = max(inp["lengths"]), inp["scale"], inp["rope_base"]
    cu = torch.from_numpy(inp["cu_seqlens"]).to(device)
    q, k, v, do = (to_dev(inp[x], device) for x in ("q", "k", "v", "do"))
    o_ref, lse_ref = E.esm_attn_fwd(q, k, v, cu, maxL, s, base)
    dq_ref, dk_ref, dv_ref = E.esm_attn_bwd(q, k, v, o_ref, do, lse_ref, cu, maxL, s, base)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = E.attention(qa, ka, va, cu, maxL, s, base)
    o.backward(do)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    for a, b in ((qa.grad, dq_ref), (ka.grad, dk_ref), (va.grad, dv_ref)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d", [64, 128])
def test_attention_qkv_in_a_projection(device, d):
    rng = np.random.default_rng(d)
    lengths = [300, 1, 129, 64]
    H, T, C = 2, sum(lengths), 64
    cu = torch.from_numpy(W.cu_from_lengths(lengths)).to(device)
    maxL = max(lengths)
    say("case attention_qkv", d)
    x0 = torch.from_numpy(rng.standard_normal((T, C)).astype(np.float32)).to(device)
    w0 = torch.from_numpy((rng.standard_normal((3 * H * d, C)) / 8).astype(np.float32)).to(device)
    do = torch.from_numpy(rng.standard_normal((T, H, d)).astype(np.float32)).to(device)
    x0, w0, do = x0.to(torch.bfloat16), w0.to(torch.bfloat16), do.to(torch.bfloat16)

    seen = {}

    def run(fused):
        x = x0.clone().requires_grad_(True)
        w = w0.clone().requires_grad_(True)
        qkv = x @ w.t()
        if fused:
            seen["qkv"] = qkv.detach().clone()   # before the in-place rotation
            qkv.register_hook(lambda g: seen.__setitem__("dqkv", g.detach().clone()))
            o = E.attention_qkv(qkv, cu, maxL, H)
        else:
            q, k, v = (qkv.view(T, 3, H, d)[:, i].contiguous() for i in range(3))
            o = E.attention(q, k, v, cu, maxL)
        o.backward(do)
        torch.cuda.synchronize()
        return o.detach(), x.grad, w.grad

    of, xf, wf = run(True)
    op, xp, wp = run(False)
    # the fused path against the oracle on the projection's own q, k, v
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    q3 = seen["qkv"].view(T, 3, H, d)
    inp = dict(q=bits(q3[:, 0]), k=bits(q3[:, 1]), v=bits(q3[:, 2]), do=bits(do),
               cu_seqlens=W.cu_from_lengths(lengths), lengths=lengths, T=T, H=H, d=d,
               scale=1.0 / np.sqrt(d), rope_base=W.ROPE_BASE)
    g3 = seen["dqkv"].view(T, 3, H, d)
    gpu = dict(o=bf16_f64(of), dq=bf16_f64(g3[:, 0]), dk=bf16_f64(g3[:, 1]),
               dv=bf16_f64(g3[:, 2]))
    plan = E.esm_attn_plan(cu, T, maxL, H, d)
    qr, kr = E.esm_attn_rotate_planned(q3[:, 0], q3[:, 1], len(lengths), maxL, plan,
                                       softmax_scale=inp["scale"])
    _, lse = E.esm_attn_fwd_planned(qr, kr, q3[:, 2].contiguous(), len(lengths), maxL, plan)
    gpu["lse"] = lse.cpu().numpy().astype(np.float64)
    compare(gpu, inp, label="attention_qkv d%d" % d)
    # and bitwise the packed path
    assert torch.equal(of, op)
    assert torch.equal(xf, xp) and torch.equal(wf, wp)


def test_attention_qkv_buffer_is_not_differentiable(device):
    lengths = [40, 9]
    H, d, T = 1, 64, 49
    cu = torch.from_numpy(W.cu_from_lengths(lengths)).to(device)
    w = torch.randn(3 * H * d, 16, device=device, dtype=torch.bfloat16, requires_grad=True)
    x = torch.randn(T, 16, device=device, dtype=torch.bfloat16)
    qkv = x @ w.t()
    o = E.attention_qkv(qkv, cu, 40, H)
    with pytest.raises(RuntimeError):
        (o.float().sum() + qkv.float().sum()).backward()
