"""The C-ABI library on the host: it loads, exports every symbol the header
declares, validates arguments before touching the GPU, and its host model of
the varlen schedule covers every (sequence, head, block) exactly once.
No compute call reaches a GPU here."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

from protein_language_model_amd import esm_attn as E
from protein_language_model_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NULL = None


def _header_functions():
    text = open(os.path.join(ROOT, "include", "esm_attn.h")).read()
    return sorted(set(re.findall(r"\b(esm_attn_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = E.lib()
    names = _header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(E.EXPORTED) == set(names)
    assert E.esm_attn_abi_version() == 6


def test_single_hip_runtime_is_mapped():
    E.lib()
    assert len(E._hip_runtimes()) == 1


def test_status_strings():
    for s in range(6):
        assert E.status_string(s).startswith("esm_attn:")
    assert "unknown" in E.status_string(99)


def test_workspace_sizes():
    fwd = E.esm_attn_fwd_workspace_bytes(16, 16384, 1024, 20, 64)
    bwd = E.esm_attn_bwd_workspace_bytes(16, 16384, 1024, 20, 64)
    plan = E.esm_attn_plan_bytes(16, 16384, 1024, 20, 64)
    x = 16384 * 20 * 64 * 2                 # one bf16 [T][H][d] tensor
    assert fwd >= plan + x                  # rotated k~ (the forward rotates q itself)
    assert bwd >= fwd + x + 16384 * 20 * 16  # q~; drow: -LSE log2(e) and -D, 16 bytes a row
    assert plan >= 1024 * 32 * 8            # rotary table
    assert E.esm_attn_plan_bytes(16, 16384, 1024, 20, 48) == 0
    assert E.esm_attn_fwd_workspace_bytes(16, 16384, 1024, 20, 48) == 0   # bad head_dim
    assert E.esm_attn_fwd_workspace_bytes(0, 16, 16, 1, 64) == 0
    assert E.esm_attn_fwd_workspace_bytes(1, 16, 70000, 1, 64) == 0        # max_seqlen


def _fwd(**kw):
    args = dict(q=1 << 12, k=1 << 12, v=1 << 12, cu=1 << 12, B=1, T=8, maxL=8, H=1, d=64,
                scale=0.125, base=10000.0, o=1 << 12, lse=1 << 12, ws=1 << 12, wsb=1 << 30,
                stream=NULL)
    args.update(kw)
    a = args
    return E.lib().esm_attn_fwd(a["q"], a["k"], a["v"], a["cu"], a["B"], a["T"], a["maxL"],
                                a["H"], a["d"], a["scale"], a["base"], a["o"], a["lse"], a["ws"],
                                a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), E.ERR_INVALID_ARGUMENT),
    (dict(o=None), E.ERR_INVALID_ARGUMENT),
    (dict(ws=None), E.ERR_INVALID_ARGUMENT),
    (dict(k=(1 << 12) + 2), E.ERR_INVALID_ARGUMENT),       # misaligned
    (dict(B=0), E.ERR_INVALID_ARGUMENT),
    (dict(H=0), E.ERR_INVALID_ARGUMENT),
    (dict(T=-1), E.ERR_INVALID_ARGUMENT),
    (dict(d=48), E.ERR_UNSUPPORTED),
    (dict(d=256), E.ERR_UNSUPPORTED),
    (dict(scale=float("nan")), E.ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), E.ERR_INVALID_ARGUMENT),
    (dict(scale=3e38), E.ERR_INVALID_ARGUMENT),             # scale * log2(e) overflows
    (dict(base=-1.0), E.ERR_INVALID_ARGUMENT),
    (dict(base=float("inf")), E.ERR_INVALID_ARGUMENT),
    (dict(maxL=70000), E.ERR_UNSUPPORTED),
    (dict(T=1 << 24, H=64, d=128), E.ERR_UNSUPPORTED),     # index overflow
    (dict(wsb=16), E.ERR_WORKSPACE_TOO_SMALL),
])
def test_forward_validation_rejects_before_launch(kw, status):
    # all pointers are fake host addresses: a launch would fault, so every case
    # must be rejected on the host
    assert _fwd(**kw) == status


def test_empty_batch_returns_ok_without_pointers():
    assert _fwd(T=0, q=None, k=None, v=None, o=None, lse=None, ws=None, cu=None) == E.OK


def test_backward_and_planned_validation():
    L = E.lib()
    p = 1 << 12
    st = L.esm_attn_bwd(p, p, p, p, p, p, p, 1, 8, 8, 1, 32, 0.1, 1e4, p, None, p, p, 1 << 30,
                        None)
    assert st == E.ERR_INVALID_ARGUMENT
    st = L.esm_attn_bwd(p, p, p, p, p, p, p, 1, 8, 8, 1, 32, 0.1, 1e4, p, p, p, p, 8, None)
    assert st == E.ERR_WORKSPACE_TOO_SMALL
    st = L.esm_attn_bwd_planned(p, p, p, 32, p, p, p, 1, 8, 8, 1, 32, 0.1, 1e4, p, p, p, 32, p,
                                0, p, 1 << 30, None)
    assert st == E.ERR_INVALID_ARGUMENT      # no pass selected
    st = L.esm_attn_bwd_planned(p, p, p, 32, p, p, p, 1, 8, 8, 1, 32, 0.1, 1e4, None, p, p, 32,
                                p, 1, p, 1 << 30, None)
    assert st == E.ERR_INVALID_ARGUMENT      # dq pass without dq
    st = L.esm_attn_plan(p, 1, 8, 8, 1, 32, -5.0, p, 1 << 30, None)
    assert st == E.ERR_INVALID_ARGUMENT
    st = L.esm_attn_fwd_planned(p, p, p, 32, 1, 8, 8, 1, 32, 0.1, p, p, p, 4, None)
    assert st == E.ERR_WORKSPACE_TOO_SMALL
    st = L.esm_attn_fwd_planned(p, p, p, 32, 1, 8, 8, 1, 32, float("nan"), p, p, p, 1 << 30,
                                None)
    assert st == E.ERR_INVALID_ARGUMENT
    # rotation step (q_rot == q and k_rot == k with equal strides: in place)
    st = L.esm_attn_rotate_planned(p, p, 32, 1, 8, 8, 1, 32, 0.125, 1e4, p, p, 32, p, 4, None)
    assert st == E.ERR_WORKSPACE_TOO_SMALL
    st = L.esm_attn_rotate_planned(p, p, 32, 1, 8, 8, 1, 32, 0.125, -1.0, p, p, 32, p, 1 << 30, None)
    assert st == E.ERR_INVALID_ARGUMENT
    st = L.esm_attn_rotate_planned(p, p, 32, 1, 8, 8, 1, 32, 0.125, 1e4, None, p, 32, p, 1 << 30, None)
    assert st == E.ERR_INVALID_ARGUMENT
    st = L.esm_attn_rotate_planned(p, p, 48, 1, 8, 8, 1, 48, 0.125, 1e4, p, p, 48, p, 1 << 30, None)
    assert st == E.ERR_UNSUPPORTED
    assert L.esm_attn_rotate_planned(None, None, 32, 1, 0, 0, 1, 32, 0.125, 1e4, None, None, 32, None,
                                     0, None) == E.OK


@pytest.mark.parametrize("call,ld,status", [
    ("rotate", 16, E.ERR_INVALID_ARGUMENT),         # below H*d (H = 2, d = 16)
    ("rotate", 36, E.ERR_INVALID_ARGUMENT),         # not a multiple of 8
    ("rotate", 1 << 28, E.ERR_UNSUPPORTED),         # T * stride >= 2^31
    ("fwd", 24, E.ERR_INVALID_ARGUMENT),
    ("fwd", 1 << 28, E.ERR_UNSUPPORTED),
    ("bwd_qkv", 20, E.ERR_INVALID_ARGUMENT),
    ("bwd_grad", 1 << 28, E.ERR_UNSUPPORTED),
])
def test_row_stride_validation(call, ld, status):
    """Token row strides are checked on the host before anything is enqueued
    (fake device pointers: a launch would fault)."""
    L = E.lib()
    p, q, T = 1 << 12, 1 << 13, 8
    if call == "rotate":
        st = L.esm_attn_rotate_planned(p, p, ld, 1, T, T, 2, 16, 0.125, 1e4, q, q, 32, p, 1 << 30, None)
    elif call == "fwd":
        st = L.esm_attn_fwd_planned(p, p, p, ld, 1, T, T, 2, 16, 0.1, q, q, p, 1 << 30, None)
    else:
        lq, lg = (ld, 96) if call == "bwd_qkv" else (96, ld)
        st = L.esm_attn_bwd_planned(p, p, p, lq, p, p, p, 1, T, T, 2, 16, 0.1, 1e4, q, q, q, lg,
                                    q, 3, p, 1 << 30, None)
    assert st == status


def test_in_place_rotation_rules():
    """In place means both outputs on their inputs with one stride."""
    L = E.lib()
    p, q, r, T = 1 << 12, 1 << 13, 1 << 14, 8
    # q in place, k not
    assert L.esm_attn_rotate_planned(p, q, 32, 1, T, T, 2, 16, 0.125, 1e4, p, r, 32, p, 4,
                                     None) == E.ERR_INVALID_ARGUMENT
    # in place with different strides
    assert L.esm_attn_rotate_planned(p, q, 96, 1, T, T, 2, 16, 0.125, 1e4, p, q, 32, p, 4,
                                     None) == E.ERR_INVALID_ARGUMENT
    # in place, one stride: only the (too small) plan is left to reject
    assert L.esm_attn_rotate_planned(p, q, 96, 1, T, T, 2, 16, 0.125, 1e4, p, q, 96, p, 4,
                                     None) == E.ERR_WORKSPACE_TOO_SMALL


def test_k_only_rotation_and_rotq_forward_validation():
    """k alone (q = q_rot = NULL) and the forward that rotates q itself are
    validated on the host like the other planned calls (fake device
    pointers: a launch would fault, so every case must be rejected)."""
    L = E.lib()
    p, q, r, T = 1 << 12, 1 << 13, 1 << 14, 8
    # k alone, out of place / in place: only the (too small) plan is left to reject
    assert L.esm_attn_rotate_planned(None, q, 32, 1, T, T, 2, 16, 0.125, 1e4, None, r, 32, p, 4,
                                     None) == E.ERR_WORKSPACE_TOO_SMALL
    assert L.esm_attn_rotate_planned(None, q, 96, 1, T, T, 2, 16, 0.125, 1e4, None, q, 96, p, 4,
                                     None) == E.ERR_WORKSPACE_TOO_SMALL
    # k alone in place with different strides; q_rot without q; q without q_rot
    assert L.esm_attn_rotate_planned(None, q, 96, 1, T, T, 2, 16, 0.125, 1e4, None, q, 32, p,
                                     1 << 30, None) == E.ERR_INVALID_ARGUMENT
    assert L.esm_attn_rotate_planned(None, q, 32, 1, T, T, 2, 16, 0.125, 1e4, r, q + 4096, 32, p,
                                     1 << 30, None) == E.ERR_INVALID_ARGUMENT
    assert L.esm_attn_rotate_planned(r, q, 32, 1, T, T, 2, 16, 0.125, 1e4, None, q + 4096, 32, p,
                                     1 << 30, None) == E.ERR_INVALID_ARGUMENT
    f = L.esm_attn_fwd_rotq_planned
    # (q, k_rot, v, ld, B, T, maxL, H, d, scale, base, o, lse, q_rot, plan, plan_bytes, stream)
    assert f(p, q, r, 32, 1, T, T, 2, 16, 0.125, 1e4, p, q, None, p, 4,
             None) == E.ERR_WORKSPACE_TOO_SMALL
    assert f(p, q, r, 32, 1, T, T, 2, 16, 0.125, 1e4, p, q, p, p, 4,
             None) == E.ERR_WORKSPACE_TOO_SMALL          # in place
    assert f(p, q, r, 32, 1, T, T, 2, 16, float("nan"), 1e4, p, q, None, p, 1 << 30,
             None) == E.ERR_INVALID_ARGUMENT
    assert f(p, q, r, 32, 1, T, T, 2, 16, 0.125, -1.0, p, q, None, p, 1 << 30,
             None) == E.ERR_INVALID_ARGUMENT
    assert f(p, q, r, 32, 1, T, T, 2, 16, 0.125, 1e4, p, q, p + 2, p, 1 << 30,
             None) == E.ERR_INVALID_ARGUMENT             # misaligned q_rot
    assert f(p, None, r, 32, 1, T, T, 2, 16, 0.125, 1e4, p, q, None, p, 1 << 30,
             None) == E.ERR_INVALID_ARGUMENT             # no k_rot
    assert f(p, q, r, 24, 1, T, T, 2, 16, 0.125, 1e4, p, q, None, p, 1 << 30,
             None) == E.ERR_INVALID_ARGUMENT             # stride below H*d
    assert f(p, q, r, 1 << 28, 1, T, T, 2, 16, 0.125, 1e4, p, q, None, p, 1 << 30,
             None) == E.ERR_UNSUPPORTED
    assert f(p, q, r, 32, 1, T, T, 2, 48, 0.125, 1e4, p, q, None, p, 1 << 30,
             None) == E.ERR_UNSUPPORTED                  # head_dim
    assert f(None, None, None, 32, 1, 0, 0, 2, 16, 0.125, 1e4, None, None, None, None, 0,
             None) == E.OK                               # empty batch


def test_split_forward_and_merge_validation():
    """Host checks of the split forward and the merge (fake device pointers:
    a launch would fault, so every case must be rejected on the host)."""
    L = E.lib()
    p, q, T = 1 << 12, 1 << 13, 8
    args = lambda ns, plan_bytes: (p, p, p, 32, 1, T, T, 2, 16, 0.1, ns, q, q, q, q, p,
                                   plan_bytes, None)
    assert L.esm_attn_fwd_split_planned(*args(0, 1 << 30)) == E.ERR_INVALID_ARGUMENT
    assert L.esm_attn_fwd_split_planned(*args(65, 1 << 30)) == E.ERR_INVALID_ARGUMENT
    assert L.esm_attn_fwd_split_planned(*args(4, 4)) == E.ERR_WORKSPACE_TOO_SMALL
    assert L.esm_attn_fwd_split_planned(p, p, p, 32, 1, T, T, 2, 16, float("inf"), 2, q, q, q,
                                        q, p, 1 << 30, None) == E.ERR_INVALID_ARGUMENT
    assert L.esm_attn_merge_partials(q, q, 0, T, 2, 16, q, q, None) == E.ERR_INVALID_ARGUMENT
    assert L.esm_attn_merge_partials(q, q, 2, T, 2, 48, q, q, None) == E.ERR_UNSUPPORTED
    assert L.esm_attn_merge_partials(q, None, 2, T, 2, 16, q, q, None) == E.ERR_INVALID_ARGUMENT
    assert L.esm_attn_merge_partials(q + 4, q, 2, T, 2, 16, q, q, None) == E.ERR_INVALID_ARGUMENT
    assert L.esm_attn_merge_partials(None, None, 2, 0, 2, 16, None, None, None) == E.OK


def test_fp8_validation():
    """Host checks of the FP8 calls (fake device pointers)."""
    L = E.lib()
    p, q, T = 1 << 12, 1 << 13, 8
    quant = lambda d, qs, ks, pb=1 << 30: L.esm_attn_quantize_fp8_planned(
        p, p, 2 * d, 1, T, T, 2, d, 1e4, qs, ks, q, q, p, pb, None)
    fwd = lambda d, qs, ks, pb=1 << 30: L.esm_attn_fwd_fp8_planned(
        q, q, p, 2 * d, 1, T, T, 2, d, 0.1, qs, ks, q, q, p, pb, None)
    for call in (quant, fwd):
        assert call(32, 1.0, 1.0) == E.ERR_UNSUPPORTED          # head_dim 64 or 128 only
        assert call(64, 0.0, 1.0) == E.ERR_INVALID_ARGUMENT
        assert call(64, 1.0, -2.0) == E.ERR_INVALID_ARGUMENT
        assert call(64, float("nan"), 1.0) == E.ERR_INVALID_ARGUMENT
        assert call(64, 1e-40, 1.0) == E.ERR_INVALID_ARGUMENT   # 1 / scale overflows
        assert call(64, 1.0, 1.0, pb=4) == E.ERR_WORKSPACE_TOO_SMALL
    assert fwd(64, 1e20, 1e20) == E.ERR_INVALID_ARGUMENT        # softmax c overflows


def test_check_cu_seqlens_host():
    ok = np.array([0, 3, 3, 10], np.int32)
    assert E.esm_attn_check_cu_seqlens_host(ok, 10, 7) == E.OK
    assert E.esm_attn_check_cu_seqlens_host(ok, 10, 6) == E.ERR_INVALID_ARGUMENT
    assert E.esm_attn_check_cu_seqlens_host(np.array([1, 3, 10], np.int32), 10, 9) != E.OK
    assert E.esm_attn_check_cu_seqlens_host(np.array([0, 5, 3, 10], np.int32), 10, 9) != E.OK
    assert E.esm_attn_check_cu_seqlens_host(np.array([0, 3, 9], np.int32), 10, 9) != E.OK


def _check_schedule(lengths, H, block=128):
    cu = W.cu_from_lengths(lengths)
    T = int(cu[-1])
    maxL = max(lengths) if lengths else 0
    items = E.esm_attn_schedule_host(cu, T, maxL, H, block)
    n = items.shape[0]
    # the launch bound the host computes
    nb = -(-maxL // block)
    bp = min(len(lengths), T)
    assert n == 8 * nb + H * min(len(lengths) * nb, (T - bp) // block + bp)
    live = items[items[:, 1] > 0]
    want = {(int(cu[b]), L, h, k) for b, L in enumerate(lengths) for h in range(H)
            for k in range(-(-L // block))}
    got = [tuple(int(x) for x in r) for r in live]
    assert len(got) == len(set(got)) == len(want)      # each item exactly once
    assert set(got) == want
    assert (items[items[:, 1] <= 0] == -1).all()
    # all blocks of one (sequence, head) on slots of one residue mod 8
    slot_of = {}
    for s, r in enumerate(items):
        if r[1] > 0:
            slot_of.setdefault((r[0], r[2]), set()).add(s % 8)
    assert all(len(v) == 1 for v in slot_of.values())
    # longest first: the first live slot of each group appears in descending length order
    first = {}
    for s, r in enumerate(items):
        if r[1] > 0 and (r[0], r[2]) not in first:
            first[(r[0], r[2])] = (s, -(-r[1] // block))
    order = [nb_ for _, nb_ in sorted(first.values())]
    assert all(order[i] >= order[i + 1] for i in range(len(order) - 1)), order
    per_xcd = np.zeros(8)
    for s, r in enumerate(items):
        if r[1] > 0:
            per_xcd[s % 8] += 1
    return items, per_xcd


@pytest.mark.parametrize("name", ["esm2_8m", "esm2_150m", "esm2_650m", "esm2_3b",
                                  "esm2_15b_ragged"])
def test_schedule_covers_every_item_once(name):
    lengths = W.lengths_of(name)
    H = W.WORKLOADS[name].num_heads
    items, per_xcd = _check_schedule(lengths, H)
    if len(lengths) * H >= 64:
        assert per_xcd.max() <= 1.1 * per_xcd.mean() + 8   # balanced over the 8 XCDs


def test_schedule_edge_cases():
    _check_schedule([0, 0, 5, 0], 3)
    _check_schedule([1] * 50, 1)
    _check_schedule([128, 129, 127, 0, 256], 7)
    _check_schedule([1000], 1)
    items, _ = _check_schedule([300, 45, 1024, 600], 5)
    # descending block counts along the launch order
    seen = []
    for r in items:
        if r[1] > 0 and r[3] == 0:
            seen.append(-(-r[1] // 128))
    assert seen == sorted(seen, reverse=True)


def test_drow_buffer_and_size_check():
    """The binding's drow scratch: [H][T] entries of 16 bytes; a smaller or
    non-float32 buffer is refused before anything reaches the library."""
    import torch
    d = E.drow_buffer(3, 10, "cpu")
    assert d.dtype == torch.float32 and d.numel() * 4 == 3 * 10 * 16
    E._check_drow(d, 3, 10)
    E._check_drow(torch.empty(4 * 3 * 10), 3, 10)
    with pytest.raises(ValueError):
        E._check_drow(torch.empty(4 * 3 * 10 - 1), 3, 10)
    with pytest.raises(ValueError):
        E._check_drow(torch.empty(2, 3, 10), 3, 10)          # the old fp32 [2][H][T] size
    with pytest.raises(ValueError):
        E._check_drow(torch.empty(4 * 3 * 10, dtype=torch.float64), 3, 10)


# ---------------------------------------------------------------- binding checks
# The binding refuses, before any library call, operands the kernels would
# misread (int64 cu_seqlens read as int32 pairs) or fault on (host pointers).

def _bf(T=8, H=2, d=64):
    return torch.zeros((T, H, d), dtype=torch.bfloat16)


def test_binding_rejects_wrong_cu_seqlens_dtype_and_shape():
    q = _bf()
    for cu in (torch.tensor([0, 8], dtype=torch.int64), torch.tensor([[0, 8]], dtype=torch.int32),
               torch.tensor([0], dtype=torch.int32),
               torch.tensor([0, 0, 8, 8], dtype=torch.int32)[::2]):
        with pytest.raises(ValueError):
            E.esm_attn_fwd(q, q, q, cu, 8)
        # the dtype and shape checks come before the device check
        with pytest.raises(ValueError, match="cu_seqlens"):
            E._check_cu(cu, q.device)
    lse = torch.zeros((2, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU|cu_seqlens"):
        E.esm_attn_bwd(q, q, q, q, q, lse, torch.tensor([0, 8], dtype=torch.int64), 8)


def test_binding_rejects_host_tensors():
    q = _bf()
    cu = torch.tensor([0, 8], dtype=torch.int32)
    lse = torch.zeros((2, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        E.esm_attn_fwd(q, q, q, cu, 8)
    with pytest.raises(ValueError, match="GPU"):
        E.esm_attn_bwd(q, q, q, q, q, lse, cu, 8)
    with pytest.raises(ValueError, match="GPU"):
        E.esm_attn_plan(cu, 8, 8, 2, 64)
    plan = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        E.esm_attn_rotate_planned(q, q, 1, 8, plan, softmax_scale=0.125)
    with pytest.raises(ValueError, match="GPU"):
        E.esm_attn_rotate_planned(None, q, 1, 8, plan, softmax_scale=0.125)
    with pytest.raises(ValueError, match="GPU"):
        E.esm_attn_fwd_planned(q, q, q, 1, 8, plan)
    with pytest.raises(ValueError, match="GPU"):
        E.esm_attn_fwd_rotq_planned(q, q, q, 1, 8, plan)
    with pytest.raises(ValueError, match="GPU"):
        E.esm_attn_bwd_planned(q, q, q, q, q, lse, 1, 8, plan,
                               drow=torch.zeros(4 * 2 * 8, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        E.esm_attn_merge_partials(torch.zeros((2, 8, 2, 64)), torch.zeros((2, 2, 8)))
    with pytest.raises(ValueError, match="GPU"):
        E.attention(q, q, q, cu, 8)
    with pytest.raises(ValueError, match="GPU"):
        E.attention_qkv(torch.zeros((8, 3 * 2 * 64), dtype=torch.bfloat16), cu, 8, 2)


def test_binding_rejects_malformed_outputs():
    # (shape and dtype checks; the calls run them after the device checks)
    with pytest.raises(ValueError, match="lse"):
        E._check_lse(torch.zeros((8, 2), dtype=torch.float32), 2, 8)
    with pytest.raises(ValueError, match="lse"):
        E._check_lse(torch.zeros((2, 8), dtype=torch.float64), 2, 8)
    with pytest.raises(ValueError, match="bf16"):
        E._check_packed((8, 2, 64), torch.zeros((8, 2, 64), dtype=torch.float16))
    with pytest.raises(ValueError, match="contiguous"):
        E._workspace(32, torch.device("cpu"), torch.zeros(64, dtype=torch.uint8)[::2])
    with pytest.raises(ValueError, match="GPU"):
        E._workspace(32, torch.device("cpu"), torch.zeros(64, dtype=torch.uint8))
    assert E._nbytes(torch.zeros(10, dtype=torch.float32)) == 40


def _noalloc(**kw):
    args = dict(q=1 << 12, k=1 << 12, v=1 << 12, cu=1 << 12, B=1, T=8, maxL=8, H=1, d=64,
                scale=0.125, base=10000.0, o=1 << 12, lse=1 << 12, stream=NULL)
    args.update(kw)
    a = args
    return E.lib().esm_attn_fwd_noalloc(a["q"], a["k"], a["v"], a["cu"], a["B"], a["T"],
                                        a["maxL"], a["H"], a["d"], a["scale"], a["base"], a["o"],
                                        a["lse"], a["stream"])


def test_noalloc_forward_rejects_before_touching_the_gpu():
    assert _noalloc(d=48) == E.ERR_UNSUPPORTED
    assert _noalloc(B=0) == E.ERR_INVALID_ARGUMENT
    assert _noalloc(scale=float("nan")) == E.ERR_INVALID_ARGUMENT
    assert _noalloc(T=0) == E.OK
    assert _noalloc(q=None) == E.ERR_INVALID_ARGUMENT
    assert _noalloc(o=(1 << 12) + 4) == E.ERR_INVALID_ARGUMENT     # misaligned
    # sizes whose workspace exceeds the fixed buffer: a clear error, nothing enqueued
    T, H, d = 262144, 4, 128            # 2 * T*H*d*2 bytes of rotated q, k = 512 MiB
    assert E.esm_attn_fwd_workspace_bytes(64, T, 4096, H, d) > E.NOALLOC_SCRATCH_BYTES
    assert _noalloc(B=64, T=T, maxL=4096, H=H, d=d) == E.ERR_SCRATCH_TOO_SMALL
    assert "no-allocation" in E.status_string(E.ERR_SCRATCH_TOO_SMALL)
    # the 650M-shaped training batch fits
    assert E.esm_attn_fwd_workspace_bytes(16, 16384, 1024, 20, 64) <= E.NOALLOC_SCRATCH_BYTES


def test_schedule_of_malformed_cu_seqlens_stays_in_bounds():
    """The schedule code the planning kernels run (schedule.h, shared with this
    host model) clamps a malformed cu_seqlens: entries past total_tokens,
    decreasing or negative entries and lengths above max_seqlen give items
    whose rows lie inside [0, total_tokens) and whose lengths stay within
    [1, max_seqlen], so the kernels' row accesses stay in bounds whatever
    the contents (the values are then wrong, as documented)."""
    rng = np.random.default_rng(5)
    for trial in range(200):
        B = int(rng.integers(1, 12))
        T = int(rng.integers(0, 3000))
        maxL = int(rng.integers(0, 1100))
        H = int(rng.integers(1, 5))
        cu = rng.integers(-500, T + 700, size=B + 1).astype(np.int32)
        if trial % 3 == 0:
            cu = np.sort(cu)  # monotone but out of range and over max_seqlen
        items = E.esm_attn_schedule_host(cu, T, maxL, H, 128)
        live = items[items[:, 1] > 0]
        assert (items[items[:, 1] <= 0] == -1).all()
        if live.size:
            seq0, L, h, blk = live.T
            assert (seq0 >= 0).all() and (seq0 + L <= T).all(), (cu, T)
            assert (L <= maxL).all() and (L >= 1).all()
            assert (h >= 0).all() and (h < H).all()
            assert (blk >= 0).all() and (blk * 128 < L).all()
