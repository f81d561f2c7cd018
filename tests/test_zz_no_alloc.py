"""esm_attn_fwd_noalloc (the forward in the library's own fixed device
buffer, for callers that cannot allocate) against esm_attn_fwd, the entry
point it shares its kernels with: two calls in a row, the second on a
smaller problem, each bitwise equal to esm_attn_fwd on the same inputs and
within the oracle bounds."""

import numpy as np
import pytest
import torch

from gpu_helpers import bf16_f64, compare, say, to_dev
from protein_language_model_amd import workloads as W
from protein_language_model_amd import esm_attn as E

pytestmark = pytest.mark.gpu


def _one(device, inp):
    q, k, v = (to_dev(inp[n], device) for n in ("q", "k", "v"))
    cu = torch.from_numpy(inp["cu_seqlens"]).to(device)
    maxL, s, base = max(inp["lengths"]), inp["scale"], inp["rope_base"]
    T, H, d = q.shape
    # outputs poisoned first, so that stale values from the previous call show
    o = torch.full_like(q, float("nan"))
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device=device)
    E.esm_attn_fwd_noalloc(q, k, v, cu, maxL, s, base, out=o, lse=lse)
    o_ref, lse_ref = E.esm_attn_fwd(q, k, v, cu, maxL, s, base)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    assert torch.equal(lse, lse_ref)
    gpu = dict(o=bf16_f64(o), lse=lse.cpu().numpy().astype(np.float64))
    compare(gpu, inp, with_bwd=False, label="noalloc %s" % (inp["lengths"],))


def test_noalloc_forward_twice_second_smaller(device):
    big = W.make_inputs("esm2_650m", lengths=[300, 1, 129, 1024, 0, 64], num_heads=3)
    small = W.make_inputs("esm2_150m", lengths=[77, 5], num_heads=2)
    say("case noalloc", big["lengths"], "then", small["lengths"])
    _one(device, big)
    _one(device, small)
