"""The planned calls captured in a HIP graph (torch.cuda.CUDAGraph): every
replay, with eager work and synchronisations in between, gives bitwise the
eager results. The library allocates nothing, synchronises nothing and
records no memset, so a whole training step of the path can be a graph."""

import numpy as np
import pytest
import torch

from gpu_helpers import say, to_dev
from protein_language_model_amd import workloads as W
from protein_language_model_amd import esm_attn as E

pytestmark = pytest.mark.gpu


def _buffers(inp, device, n_split):
    T, H, d = inp["T"], inp["H"], inp["d"]
    B, maxL = len(inp["lengths"]), max(inp["lengths"])
    bf = lambda: torch.empty((T, H, d), dtype=torch.bfloat16, device=device)
    return dict(
        q=to_dev(inp["q"], device), k=to_dev(inp["k"], device), v=to_dev(inp["v"], device),
        do=to_dev(inp["do"], device), cu=torch.from_numpy(inp["cu_seqlens"]).to(device),
        plan=torch.empty(E.esm_attn_plan_bytes(B, T, maxL, H, d), dtype=torch.uint8,
                         device=device),
        qr=bf(), kr=bf(), o=bf(), o2=bf(), dq=bf(), dk=bf(), dv=bf(),
        lse=torch.empty((H, T), dtype=torch.float32, device=device),
        lse2=torch.empty((H, T), dtype=torch.float32, device=device),
        drow=E.drow_buffer(H, T, device),
        op=torch.empty((n_split, T, H, d), dtype=torch.float32, device=device),
        lp=torch.empty((n_split, H, T), dtype=torch.float32, device=device))


def _step(inp, b, n_split):
    T, H, d = inp["T"], inp["H"], inp["d"]
    B, maxL = len(inp["lengths"]), max(inp["lengths"])
    s, base = inp["scale"], inp["rope_base"]
    E.esm_attn_plan(b["cu"], T, maxL, H, d, base, plan=b["plan"])
    E.esm_attn_rotate_planned(b["q"], b["k"], B, maxL, b["plan"], base, q_rot=b["qr"],
                              k_rot=b["kr"], softmax_scale=s)
    E.esm_attn_fwd_planned(b["qr"], b["kr"], b["v"], B, maxL, b["plan"], s, out=b["o"],
                           lse=b["lse"])
    E.esm_attn_bwd_planned(b["qr"], b["kr"], b["v"], b["o"], b["do"], b["lse"], B, maxL,
                           b["plan"], s, base, dq=b["dq"], dk=b["dk"], dv=b["dv"],
                           drow=b["drow"])
    E.esm_attn_fwd_split_planned(b["qr"], b["kr"], b["v"], B, maxL, b["plan"], n_split, s,
                                 out=b["o2"], lse=b["lse2"], o_part=b["op"], lse_part=b["lp"])


OUTS = ("qr", "kr", "o", "lse", "dq", "dk", "dv", "o2", "lse2")


def test_graph_replays_equal_eager(device):
    inp = W.make_inputs("esm2_650m", lengths=[300, 1, 129, 64, 700, 0], num_heads=3)
    other = W.make_inputs("esm2_650m", lengths=[200, 513], num_heads=3, seed=99)
    say("case graph", inp["lengths"])
    b = _buffers(inp, device, 3)
    _step(inp, b, 3)
    torch.cuda.synchronize()
    ref = {n: b[n].clone() for n in OUTS}

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(inp, b, 3)          # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _step(inp, b, 3)
    torch.cuda.synchronize()

    b2 = _buffers(other, device, 2)
    for rep in range(4):
        for n in OUTS:            # poison the outputs between replays (eager fills)
            b[n].fill_(float("nan") if b[n].is_floating_point() else 0)
        _step(other, b2, 2)       # eager work on other data in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in OUTS:
            assert torch.equal(b[n], ref[n]), (rep, n)
