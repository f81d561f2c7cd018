"""Thin Python binding of libesm_attn.so (C ABI in include/esm_attn.h).

Argument marshalling only: every step of the attention path runs in the HIP
library. torch provides device memory (outputs and workspace are torch
tensors) and the stream (torch's current stream is passed through). If the
library is missing, every call raises; there is no fallback.

Functions keep the C names:
  esm_attn_fwd(q, k, v, cu_seqlens, max_seqlen, softmax_scale, rope_base)
      -> (o, lse)
  esm_attn_fwd_noalloc(...) -> (o, lse)   (same, in the library's own buffer)
  esm_attn_bwd(q, k, v, o, d_o, lse, cu_seqlens, max_seqlen, softmax_scale,
               rope_base) -> (dq, dk, dv)
the planned steps (esm_attn_plan, esm_attn_rotate_planned,
esm_attn_fwd_planned, esm_attn_fwd_rotq_planned -- the forward that rotates
q itself, used up to d = 64, see fwd_rotates_q -- and esm_attn_bwd_planned),
the workspace queries,
esm_attn_check_cu_seqlens_host, esm_attn_schedule_host, the host batch former
esm_attn_bucket_batches, the split-KV, merge and FP8 calls, and the autograd
wrappers `attention` (packed q, k, v) and `attention_qkv` (one fused projection
output, rotated in place).
"""

import ctypes
import math
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libesm_attn.so")

(OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL, ERR_HIP,
 ERR_SCRATCH_TOO_SMALL) = range(6)
NOALLOC_SCRATCH_BYTES = 128 << 20   # ESM_ATTN_NOALLOC_SCRATCH_BYTES

EXPORTED = (
    "esm_attn_abi_version",
    "esm_attn_status_string",
    "esm_attn_fwd_workspace_bytes",
    "esm_attn_bwd_workspace_bytes",
    "esm_attn_fwd",
    "esm_attn_fwd_noalloc",
    "esm_attn_bwd",
    "esm_attn_plan_bytes",
    "esm_attn_plan",
    "esm_attn_rotate_planned",
    "esm_attn_fwd_planned",
    "esm_attn_fwd_rotq_planned",
    "esm_attn_bwd_planned",
    "esm_attn_check_cu_seqlens_host",
    "esm_attn_schedule_host",
    "esm_attn_bucket_batches",
    "esm_attn_fwd_split_planned",
    "esm_attn_merge_partials",
    "esm_attn_quantize_fp8_planned",
    "esm_attn_fwd_fp8_planned",
)

PASS_DQ, PASS_DKV = 1, 2

_lib = None


class EsmAttnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


def _hip_runtimes():
    with open("/proc/self/maps") as f:
        return sorted({line.split()[-1] for line in f if "libamdhip64" in line})


def lib():
    """Loads the library once (after torch, so that it binds to the HIP
    runtime torch already loaded)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise EsmAttnError(ERR_HIP, "libesm_attn.so is not built: run "
                           "python -m protein_language_model_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    i32, u64, vp, f32 = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    L.esm_attn_abi_version.restype = i32
    L.esm_attn_abi_version.argtypes = []
    L.esm_attn_status_string.restype = ctypes.c_char_p
    L.esm_attn_status_string.argtypes = [i32]
    for name in ("esm_attn_fwd_workspace_bytes", "esm_attn_bwd_workspace_bytes",
                 "esm_attn_plan_bytes"):
        fn = getattr(L, name)
        fn.restype = u64
        fn.argtypes = [i32] * 5
    L.esm_attn_fwd.restype = i32
    L.esm_attn_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, f32, vp, vp, vp,
                               u64, vp]
    L.esm_attn_fwd_noalloc.restype = i32
    L.esm_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, f32, vp,
                                       vp, vp]
    L.esm_attn_bwd.restype = i32
    L.esm_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, f32,
                               vp, vp, vp, vp, u64, vp]
    L.esm_attn_plan.restype = i32
    L.esm_attn_plan.argtypes = [vp, i32, i32, i32, i32, i32, f32, vp, u64, vp]
    L.esm_attn_rotate_planned.restype = i32
    L.esm_attn_rotate_planned.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, f32, f32, vp, vp,
                                          i32, vp, u64, vp]
    L.esm_attn_fwd_planned.restype = i32
    L.esm_attn_fwd_planned.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp,
                                       u64, vp]
    L.esm_attn_fwd_rotq_planned.restype = i32
    L.esm_attn_fwd_rotq_planned.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32,
                                            vp, vp, vp, vp, u64, vp]
    L.esm_attn_bwd_planned.restype = i32
    L.esm_attn_bwd_planned.argtypes = [vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                       f32, vp, vp, vp, i32, vp, i32, vp, u64, vp]
    L.esm_attn_check_cu_seqlens_host.restype = i32
    L.esm_attn_check_cu_seqlens_host.argtypes = [vp, i32, i32, i32]
    L.esm_attn_schedule_host.restype = i32
    L.esm_attn_schedule_host.argtypes = [vp, i32, i32, i32, i32, i32, vp, i32, vp]
    L.esm_attn_fwd_split_planned.restype = i32
    L.esm_attn_fwd_split_planned.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32,
                                             vp, vp, vp, vp, vp, u64, vp]
    L.esm_attn_quantize_fp8_planned.restype = i32
    L.esm_attn_quantize_fp8_planned.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, f32, f32,
                                                f32, vp, vp, vp, u64, vp]
    L.esm_attn_fwd_fp8_planned.restype = i32
    L.esm_attn_fwd_fp8_planned.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32,
                                           f32, vp, vp, vp, u64, vp]
    L.esm_attn_merge_partials.restype = i32
    L.esm_attn_merge_partials.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp]
    L.esm_attn_bucket_batches.restype = i32
    L.esm_attn_bucket_batches.argtypes = [vp, i32, vp, i32, ctypes.c_int64, i32, vp, vp, i32,
                                          vp]
    if len(_hip_runtimes()) > 1:
        raise EsmAttnError(ERR_HIP, "two HIP runtimes are mapped: %s" % _hip_runtimes())
    _lib = L
    return L


def status_string(status):
    return lib().esm_attn_status_string(int(status)).decode()


def _check(status):
    if status != OK:
        raise EsmAttnError(status, status_string(status))


def esm_attn_abi_version():
    return lib().esm_attn_abi_version()


def esm_attn_fwd_workspace_bytes(batch, total_tokens, max_seqlen, num_heads, head_dim):
    return lib().esm_attn_fwd_workspace_bytes(batch, total_tokens, max_seqlen, num_heads,
                                              head_dim)


def esm_attn_bwd_workspace_bytes(batch, total_tokens, max_seqlen, num_heads, head_dim):
    return lib().esm_attn_bwd_workspace_bytes(batch, total_tokens, max_seqlen, num_heads,
                                              head_dim)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_gpu(device, *ts):
    """Every tensor given (None skipped) lives on `device`, a GPU: the library
    dereferences the pointers in its kernels, so a host pointer would fault."""
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("expected GPU tensors, got one on %s" % t.device)
        if t.device != device:
            raise ValueError("tensors on different devices (%s and %s)" % (t.device, device))


def _check_cu(cu, device):
    """cu_seqlens: 1-D contiguous int32 on the same GPU as the operands (an
    int64 tensor would be read as pairs of int32 values)."""
    if cu.dtype != torch.int32 or cu.dim() != 1 or not cu.is_contiguous() or cu.numel() < 2:
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor of batch+1 entries")
    _on_gpu(device, cu)
    return cu.numel() - 1


def _check_qkv(*ts):
    T, H, d = ts[0].shape
    for t in ts:
        if t.dtype != torch.bfloat16 or t.shape != (T, H, d) or not t.is_contiguous():
            raise ValueError("expected contiguous bf16 tensors of shape [T, H, d]")
    _on_gpu(ts[0].device, *ts)
    return T, H, d


def _check_packed(shape, *ts):
    for t in ts:
        if t.dtype != torch.bfloat16 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
            raise ValueError("expected a contiguous bf16 tensor of shape %s" % (tuple(shape),))


def _row_stride(*ts):
    """Common token row stride of bf16 [T, H, d] tensors whose (H, d) part is
    packed (strides (ld, d, 1)); ld > H*d for views of a fused buffer such as
    qkv.view(T, 3, H, d)[:, i]. Tensors of at most one token use H*d."""
    T, H, d = ts[0].shape
    strides = set()
    for t in ts:
        if t.dtype != torch.bfloat16 or t.shape != (T, H, d):
            raise ValueError("expected bf16 tensors of shape [T, H, d]")
        if t.stride(2) != 1 or (H > 1 and t.stride(1) != d):
            raise ValueError("expected rows with packed (H, d) (strides (ld, d, 1))")
        strides.add(t.stride(0))
    _on_gpu(ts[0].device, *ts)
    if T <= 1:
        return H * d
    if len(strides) != 1:
        raise ValueError("these tensors must share one token row stride, got %s"
                         % sorted(strides))
    return strides.pop()


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        if not workspace.is_contiguous():
            raise ValueError("a workspace or plan buffer must be contiguous")
        _on_gpu(device, workspace)
        return workspace
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _nbytes(t):
    return t.numel() * t.element_size()


def _check_plan(plan, device):
    """A plan from esm_attn_plan: a contiguous buffer on the operands' GPU."""
    if not plan.is_contiguous():
        raise ValueError("plan must be a contiguous buffer (esm_attn_plan's result)")
    _on_gpu(device, plan)


def _check_lse(lse, H, T):
    if lse.dtype != torch.float32 or tuple(lse.shape) != (H, T) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [H, T]")


def esm_attn_fwd(q, k, v, cu_seqlens, max_seqlen, softmax_scale=None, rope_base=10000.0,
                 out=None, lse=None, workspace=None, stream=None):
    """Forward: returns (o bf16 [T,H,d], lse fp32 [H,T])."""
    T, H, d = _check_qkv(q, k, v)
    B = _check_cu(cu_seqlens, q.device)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    _check_packed((T, H, d), out)
    _check_lse(lse, H, T)
    _on_gpu(q.device, out, lse)
    nbytes = esm_attn_fwd_workspace_bytes(B, T, int(max_seqlen), H, d)
    ws = _workspace(nbytes, q.device, workspace)
    _check(lib().esm_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), B, T,
                              int(max_seqlen), H, d, scale, float(rope_base), _ptr(out),
                              _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream)))
    return out, lse


def esm_attn_fwd_noalloc(q, k, v, cu_seqlens, max_seqlen, softmax_scale=None,
                         rope_base=10000.0, out=None, lse=None, stream=None):
    """Forward in the library's own fixed device buffer (no workspace; the C
    call allocates nothing). Pass out and lse to allocate nothing here either.
    Returns (o bf16 [T,H,d], lse fp32 [H,T])."""
    T, H, d = _check_qkv(q, k, v)
    B = _check_cu(cu_seqlens, q.device)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    _check_packed((T, H, d), out)
    _check_lse(lse, H, T)
    _on_gpu(q.device, out, lse)
    _check(lib().esm_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), B, T,
                                      int(max_seqlen), H, d, scale, float(rope_base), _ptr(out),
                                      _ptr(lse), _stream(stream)))
    return out, lse


def esm_attn_bwd(q, k, v, o, d_o, lse, cu_seqlens, max_seqlen, softmax_scale=None,
                 rope_base=10000.0, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward: returns (dq, dk, dv), bf16 [T,H,d]."""
    T, H, d = _check_qkv(q, k, v, o, d_o)
    _check_lse(lse, H, T)
    B = _check_cu(cu_seqlens, q.device)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_packed((T, H, d), dq, dk, dv)
    _on_gpu(q.device, lse, dq, dk, dv)
    nbytes = esm_attn_bwd_workspace_bytes(B, T, int(max_seqlen), H, d)
    ws = _workspace(nbytes, q.device, workspace)
    _check(lib().esm_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse),
                              _ptr(cu_seqlens), B, T, int(max_seqlen), H, d, scale,
                              float(rope_base), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                              _nbytes(ws), _stream(stream)))
    return dq, dk, dv


def esm_attn_plan_bytes(batch, total_tokens, max_seqlen, num_heads, head_dim):
    return lib().esm_attn_plan_bytes(batch, total_tokens, max_seqlen, num_heads, head_dim)


def esm_attn_plan(cu_seqlens, total_tokens, max_seqlen, num_heads, head_dim,
                  rope_base=10000.0, plan=None, stream=None):
    """Builds the schedule + rotary table for one batch; returns the plan
    buffer (a uint8 device tensor) for the planned calls."""
    B = _check_cu(cu_seqlens, cu_seqlens.device)
    nbytes = esm_attn_plan_bytes(B, int(total_tokens), int(max_seqlen), num_heads, head_dim)
    plan = _workspace(nbytes, cu_seqlens.device, plan)
    _check(lib().esm_attn_plan(_ptr(cu_seqlens), B, int(total_tokens), int(max_seqlen),
                               num_heads, head_dim, float(rope_base), _ptr(plan), _nbytes(plan),
                               _stream(stream)))
    return plan


def esm_attn_rotate_planned(q, k, batch, max_seqlen, plan, rope_base=10000.0, q_rot=None,
                            k_rot=None, stream=None, *, softmax_scale):
    """q^ = bf16(c R(p) q) with c = fl32(softmax_scale * log2(e)) and
    k^ = bf16(R(p) k), with the plan's rotary table; returns (q_rot, k_rot).
    softmax_scale (keyword, required) must be the one later given to the
    planned forward and backward on these operands. q and k may be views of a
    fused [T, 3, H, d] buffer; q_rot=q, k_rot=k rotates in place. q=None
    rotates k alone (for esm_attn_fwd_rotq_planned) and returns (None, k_rot)."""
    T, H, d = k.shape
    if q is None:
        if q_rot is not None:
            raise ValueError("q_rot given without q")
        ld_in = _row_stride(k)
    else:
        ld_in = _row_stride(q, k)
        if q_rot is None:
            q_rot = torch.empty((T, H, d), dtype=q.dtype, device=q.device)
    if k_rot is None:
        k_rot = torch.empty((T, H, d), dtype=k.dtype, device=k.device)
    ld_out = _row_stride(k_rot) if q is None else _row_stride(q_rot, k_rot)
    _on_gpu(k.device, k_rot, *([] if q is None else [q_rot]))
    _check_plan(plan, k.device)
    _check(lib().esm_attn_rotate_planned(None if q is None else _ptr(q), _ptr(k), ld_in,
                                         int(batch), T,
                                         int(max_seqlen), H, d, float(softmax_scale),
                                         float(rope_base),
                                         None if q is None else _ptr(q_rot),
                                         _ptr(k_rot), ld_out, _ptr(plan), _nbytes(plan),
                                         _stream(stream)))
    return q_rot, k_rot


def esm_attn_fwd_planned(q_rot, k_rot, v, batch, max_seqlen, plan, softmax_scale=None,
                         out=None, lse=None, stream=None):
    """Forward on rotated q^, k^ (esm_attn_rotate_planned's outputs, made
    with this softmax_scale) and v, which share one token row stride (e.g.
    views of a fused [T, 3, H, d] buffer). out: packed [T, H, d]."""
    T, H, d = v.shape
    ld = _row_stride(q_rot, k_rot, v)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((T, H, d), dtype=v.dtype, device=v.device)
    _check_packed((T, H, d), out)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=v.device)
    _check_lse(lse, H, T)
    _on_gpu(v.device, out, lse)
    _check_plan(plan, v.device)
    _check(lib().esm_attn_fwd_planned(_ptr(q_rot), _ptr(k_rot), _ptr(v), ld, int(batch), T,
                                      int(max_seqlen), H, d, scale, _ptr(out), _ptr(lse),
                                      _ptr(plan), _nbytes(plan), _stream(stream)))
    return out, lse


def esm_attn_fwd_rotq_planned(q, k_rot, v, batch, max_seqlen, plan, softmax_scale=None,
                              rope_base=10000.0, out=None, lse=None, q_rot=None, stream=None):
    """Forward on the unrotated q, the rotated k^ (esm_attn_rotate_planned
    with q=None) and v, which share one token row stride: each work item
    rotates and scales its own query rows as the rotation pass does, so
    (out, lse) are bitwise those of the rotation pass followed by
    esm_attn_fwd_planned. If q_rot is given (same row stride; q_rot=q is
    in place), the rotated q^ is written there for the backward. Returns
    (out, lse, q_rot)."""
    T, H, d = v.shape
    ld = _row_stride(q, k_rot, v, *([] if q_rot is None else [q_rot]))
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((T, H, d), dtype=v.dtype, device=v.device)
    _check_packed((T, H, d), out)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=v.device)
    _check_lse(lse, H, T)
    _on_gpu(v.device, out, lse)
    _check_plan(plan, v.device)
    _check(lib().esm_attn_fwd_rotq_planned(_ptr(q), _ptr(k_rot), _ptr(v), ld, int(batch), T,
                                           int(max_seqlen), H, d, scale, float(rope_base),
                                           _ptr(out), _ptr(lse),
                                           None if q_rot is None else _ptr(q_rot), _ptr(plan),
                                           _nbytes(plan), _stream(stream)))
    return out, lse, q_rot


def esm_attn_fwd_split_planned(q_rot, k_rot, v, batch, max_seqlen, plan, n_split,
                               softmax_scale=None, out=None, lse=None, o_part=None,
                               lse_part=None, stream=None):
    """Split-KV forward: n_split key-range partials per work item, then their
    merge. Returns (o, lse, o_part, lse_part); o_part fp32 [n_split, T, H, d]
    and lse_part fp32 [n_split, H, T] hold the chunk partials."""
    T, H, d = v.shape
    ld = _row_stride(q_rot, k_rot, v)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dev = v.device
    if out is None:
        out = torch.empty((T, H, d), dtype=v.dtype, device=dev)
    _check_packed((T, H, d), out)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    if o_part is None:
        o_part = torch.empty((n_split, T, H, d), dtype=torch.float32, device=dev)
    if lse_part is None:
        lse_part = torch.empty((n_split, H, T), dtype=torch.float32, device=dev)
    _check_partials(o_part, lse_part, n_split, T, H, d)
    _check_lse(lse, H, T)
    _on_gpu(dev, out, lse, o_part, lse_part)
    _check_plan(plan, dev)
    _check(lib().esm_attn_fwd_split_planned(_ptr(q_rot), _ptr(k_rot), _ptr(v), ld, int(batch), T,
                                            int(max_seqlen), H, d, scale, int(n_split),
                                            _ptr(o_part), _ptr(lse_part), _ptr(out), _ptr(lse),
                                            _ptr(plan), _nbytes(plan), _stream(stream)))
    return out, lse, o_part, lse_part


def _check_partials(o_part, lse_part, R, T, H, d):
    if (o_part.dtype != torch.float32 or tuple(o_part.shape) != (R, T, H, d)
            or not o_part.is_contiguous()):
        raise ValueError("o_part must be contiguous fp32 [R, T, H, d]")
    if (lse_part.dtype != torch.float32 or tuple(lse_part.shape) != (R, H, T)
            or not lse_part.is_contiguous()):
        raise ValueError("lse_part must be contiguous fp32 [R, H, T]")


def esm_attn_merge_partials(o_part, lse_part, out=None, lse=None, stream=None):
    """O = sum_r exp(LSE_r - LSE) O_r, LSE = log sum_r exp(LSE_r) over the
    partials o_part fp32 [R, T, H, d], lse_part fp32 [R, H, T]; returns
    (o bf16 [T, H, d], lse fp32 [H, T])."""
    R, T, H, d = o_part.shape
    _check_partials(o_part, lse_part, R, T, H, d)
    if out is None:
        out = torch.empty((T, H, d), dtype=torch.bfloat16, device=o_part.device)
    _check_packed((T, H, d), out)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=o_part.device)
    _check_lse(lse, H, T)
    _on_gpu(o_part.device, lse_part, out, lse)
    _check(lib().esm_attn_merge_partials(_ptr(o_part), _ptr(lse_part), R, T, H, d, _ptr(out),
                                         _ptr(lse), _stream(stream)))
    return out, lse


def esm_attn_quantize_fp8_planned(q, k, batch, max_seqlen, plan, q_scale, k_scale,
                                  rope_base=10000.0, q8=None, k8=None, stream=None):
    """E4M3 q8 = E4M3(R(p) q / q_scale), k8 likewise (saturating); returns
    (q8, k8), uint8 [T, H, d] (packed). q, k may be strided views."""
    T, H, d = q.shape
    ld = _row_stride(q, k)
    if q8 is None:
        q8 = torch.empty((T, H, d), dtype=torch.uint8, device=q.device)
    if k8 is None:
        k8 = torch.empty((T, H, d), dtype=torch.uint8, device=q.device)
    for t in (q8, k8):
        if t.dtype != torch.uint8 or tuple(t.shape) != (T, H, d) or not t.is_contiguous():
            raise ValueError("q8, k8 must be contiguous uint8 [T, H, d]")
    _on_gpu(q.device, q8, k8)
    _check_plan(plan, q.device)
    _check(lib().esm_attn_quantize_fp8_planned(_ptr(q), _ptr(k), ld, int(batch), T,
                                               int(max_seqlen), H, d, float(rope_base),
                                               float(q_scale), float(k_scale), _ptr(q8), _ptr(k8),
                                               _ptr(plan), _nbytes(plan), _stream(stream)))
    return q8, k8


def esm_attn_fwd_fp8_planned(q8, k8, v, batch, max_seqlen, plan, q_scale, k_scale,
                             softmax_scale=None, out=None, lse=None, stream=None):
    """Forward with E4M3 q8, k8 (esm_attn_quantize_fp8_planned's outputs) and
    bf16 v; returns (o bf16 [T, H, d], lse fp32 [H, T])."""
    T, H, d = v.shape
    ldv = _row_stride(v)
    for t in (q8, k8):
        if t.dtype != torch.uint8 or tuple(t.shape) != (T, H, d) or not t.is_contiguous():
            raise ValueError("q8, k8 must be contiguous uint8 [T, H, d]")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((T, H, d), dtype=v.dtype, device=v.device)
    _check_packed((T, H, d), out)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=v.device)
    _check_lse(lse, H, T)
    _on_gpu(v.device, q8, k8, out, lse)
    _check_plan(plan, v.device)
    _check(lib().esm_attn_fwd_fp8_planned(_ptr(q8), _ptr(k8), _ptr(v), ldv, int(batch), T,
                                          int(max_seqlen), H, d, scale, float(q_scale),
                                          float(k_scale), _ptr(out), _ptr(lse), _ptr(plan),
                                          _nbytes(plan), _stream(stream)))
    return out, lse


def esm_attn_bwd_planned(q_rot, k_rot, v, o, d_o, lse, batch, max_seqlen, plan,
                         softmax_scale=None, rope_base=10000.0, dq=None, dk=None, dv=None,
                         drow=None, passes=PASS_DQ | PASS_DKV, stream=None):
    """Backward on rotated q^, k^ (and v, one token row stride, as for the
    forward; o and d_o packed); dq and dk are gradients with respect to the
    pre-rotation q and k. dq, dk, dv share one token row stride (e.g. views
    of a fused [T, 3, H, d] gradient). drow: the passes' shared scratch
    (drow_buffer(H, T, device))."""
    T, H, d = v.shape
    ld = _row_stride(q_rot, k_rot, v)
    _check_packed((T, H, d), d_o, *([o] if passes & PASS_DQ else []))
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if drow is None:
        drow = drow_buffer(H, T, v.device)
    _check_drow(drow, H, T)
    new = lambda: torch.empty((T, H, d), dtype=v.dtype, device=v.device)
    grads = []
    if passes & PASS_DQ:
        dq = new() if dq is None else dq
        grads.append(dq)
    if passes & PASS_DKV:
        dk = new() if dk is None else dk
        dv = new() if dv is None else dv
        grads += [dk, dv]
    ld_grad = _row_stride(*grads)
    if passes & PASS_DQ:
        _check_lse(lse, H, T)
    _on_gpu(v.device, o, d_o, lse, drow, *grads)
    _check_plan(plan, v.device)
    _check(lib().esm_attn_bwd_planned(_ptr(q_rot), _ptr(k_rot), _ptr(v), ld, _ptr(o), _ptr(d_o),
                                      _ptr(lse), int(batch), T, int(max_seqlen), H, d, scale,
                                      float(rope_base), _ptr(dq), _ptr(dk), _ptr(dv), ld_grad,
                                      _ptr(drow), int(passes), _ptr(plan), _nbytes(plan),
                                      _stream(stream)))
    return dq, dk, dv, drow


def drow_buffer(num_heads, total_tokens, device):
    """Scratch the backward passes share: [H][T] entries of 16 bytes
    (-LSE log2(e), then -D per row, each split into three bf16 values)."""
    return torch.empty((num_heads, total_tokens, 4), dtype=torch.float32, device=device)


def _check_drow(drow, H, T):
    if not (drow.dtype == torch.float32 and drow.is_contiguous() and drow.numel() >= 4 * H * T):
        raise ValueError("drow must be a contiguous float32 buffer of at least 4*H*T elements "
                         "(drow_buffer(H, T, device))")


def esm_attn_check_cu_seqlens_host(cu, total_tokens, max_seqlen):
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    return lib().esm_attn_check_cu_seqlens_host(cu.ctypes.data_as(ctypes.c_void_p),
                                                 cu.size - 1, int(total_tokens),
                                                 int(max_seqlen))


def esm_attn_schedule_host(cu, total_tokens, max_seqlen, num_heads, block_rows=128,
                           capacity=None):
    """Host model of the device schedule: returns an int32 array [n_slots, 4]
    of (sequence start, length, head, block), -1 rows for idle slots."""
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    if capacity is None:
        capacity = 8 * (max_seqlen // block_rows + 2) + num_heads * (cu.size + total_tokens)
    items = np.zeros((capacity, 4), dtype=np.int32)
    n = ctypes.c_int32(0)
    _check(lib().esm_attn_schedule_host(cu.ctypes.data_as(ctypes.c_void_p), cu.size - 1,
                                        int(total_tokens), int(max_seqlen), int(num_heads),
                                        int(block_rows), items.ctypes.data_as(ctypes.c_void_p),
                                        int(capacity), ctypes.byref(n)))
    return items[: n.value].copy()


def esm_attn_bucket_batches(lengths, boundaries, budget, padded=False):
    """Size-aware bucket batching on the host (see the C header): returns a
    list of int32 index arrays into `lengths`, one per batch, bucket by
    bucket."""
    ln = np.ascontiguousarray(lengths, dtype=np.int32)
    bd = np.ascontiguousarray(boundaries, dtype=np.int32)
    n = ln.size
    order = np.zeros(max(n, 1), dtype=np.int32)
    offsets = np.zeros(n + 1, dtype=np.int32)
    nb = ctypes.c_int32(0)
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    _check(lib().esm_attn_bucket_batches(vp(ln), n, vp(bd) if bd.size else None, bd.size,
                                         int(budget), int(bool(padded)), vp(order),
                                         vp(offsets), n, ctypes.byref(nb)))
    return [order[offsets[b]:offsets[b + 1]].copy() for b in range(nb.value)]


def fwd_rotates_q(head_dim):
    """Whether a training step should rotate q inside the forward
    (esm_attn_rotate_planned on k alone + esm_attn_fwd_rotq_planned) rather
    than in the rotation pass: up to d = 64, as the one-shot forward does (at
    d = 128 the rotary table of a long sequence competes with K/V for L2)."""
    return head_dim <= 64


class _Attention(torch.autograd.Function):
    """The plan (schedule + rotary table) and the rotated q^, k^ are made once
    in forward and kept for backward in place of q and k."""

    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens, max_seqlen, scale, rope_base):
        T, H, d = _check_qkv(q, k, v)
        B = _check_cu(cu_seqlens, q.device)
        plan = esm_attn_plan(cu_seqlens, T, max_seqlen, H, d, rope_base)
        if fwd_rotates_q(d):
            # k^ by the rotation pass; the forward rotates and scales q itself
            # and writes q^ for the backward
            _, k_rot = esm_attn_rotate_planned(None, k, B, max_seqlen, plan, rope_base,
                                               softmax_scale=scale)
            q_rot = torch.empty_like(q)
            o, lse, _ = esm_attn_fwd_rotq_planned(q, k_rot, v, B, max_seqlen, plan, scale,
                                                  rope_base, q_rot=q_rot)
        else:
            q_rot, k_rot = esm_attn_rotate_planned(q, k, B, max_seqlen, plan, rope_base,
                                                   softmax_scale=scale)
            o, lse = esm_attn_fwd_planned(q_rot, k_rot, v, B, max_seqlen, plan, scale)
        ctx.save_for_backward(q_rot, k_rot, v, o, lse, plan)
        ctx.args = (B, max_seqlen, scale, rope_base)
        return o

    @staticmethod
    def backward(ctx, grad):
        q_rot, k_rot, v, o, lse, plan = ctx.saved_tensors
        B, max_seqlen, scale, rope_base = ctx.args
        dq, dk, dv, _ = esm_attn_bwd_planned(q_rot, k_rot, v, o, grad.contiguous(), lse, B,
                                             max_seqlen, plan, scale, rope_base)
        return dq, dk, dv, None, None, None, None


class _AttentionQKV(torch.autograd.Function):
    """Fused layer boundary: q, k, v are views of one projection output
    qkv [T, 3*H*d]; q and k are rotated in place (the buffer then holds q^
    (scaled by softmax_scale log2(e)), k^, v and is kept for backward in place
    of any copy), and the backward
    writes dq, dk, dv into one [T, 3*H*d] gradient, the operand of the
    projection's backward GEMMs."""

    @staticmethod
    def forward(ctx, qkv, cu_seqlens, max_seqlen, num_heads, scale, rope_base, plan):
        T = qkv.shape[0]
        H = num_heads
        d = qkv.shape[1] // (3 * H)
        view = qkv.view(T, 3, H, d)
        q, k, v = view[:, 0], view[:, 1], view[:, 2]
        B = _check_cu(cu_seqlens, qkv.device)
        if plan is None:
            plan = esm_attn_plan(cu_seqlens, T, max_seqlen, H, d, rope_base)
        ctx.mark_dirty(qkv)
        if fwd_rotates_q(d):
            # k rotated in place by the rotation pass, q by the forward itself
            esm_attn_rotate_planned(None, k, B, max_seqlen, plan, rope_base, k_rot=k,
                                    softmax_scale=scale)
            o, lse, _ = esm_attn_fwd_rotq_planned(q, k, v, B, max_seqlen, plan, scale,
                                                  rope_base, q_rot=q)
        else:
            esm_attn_rotate_planned(q, k, B, max_seqlen, plan, rope_base, q_rot=q, k_rot=k,
                                    softmax_scale=scale)
            o, lse = esm_attn_fwd_planned(q, k, v, B, max_seqlen, plan, scale)
        ctx.save_for_backward(qkv, o, lse, plan)
        ctx.args = (B, max_seqlen, H, d, scale, rope_base)
        ctx.set_materialize_grads(False)
        return o, qkv

    @staticmethod
    def backward(ctx, grad_o, grad_qkv):
        if grad_qkv is not None:
            raise RuntimeError("attention_qkv: the rotated qkv buffer it returns is not "
                               "differentiable; use only the attention output")
        qkv, o, lse, plan = ctx.saved_tensors
        B, max_seqlen, H, d, scale, rope_base = ctx.args
        T = qkv.shape[0]
        view = qkv.view(T, 3, H, d)
        dqkv = torch.empty_like(qkv)
        g3 = dqkv.view(T, 3, H, d)
        if grad_o is None:
            return dqkv.zero_(), None, None, None, None, None, None
        esm_attn_bwd_planned(view[:, 0], view[:, 1], view[:, 2], o, grad_o.contiguous(), lse, B,
                             max_seqlen, plan, scale, rope_base, dq=g3[:, 0], dk=g3[:, 1],
                             dv=g3[:, 2])
        return dqkv, None, None, None, None, None, None


def attention_qkv(qkv, cu_seqlens, max_seqlen, num_heads, softmax_scale=None,
                  rope_base=10000.0, plan=None):
    """Autograd entry on a fused projection output qkv [T, 3*H*d] (contiguous,
    bf16; q, k, v are its column blocks of H*d): returns o [T, H, d]. q and k
    are rotated IN PLACE inside qkv (which must not be used afterwards), so no
    rotated copies exist; the gradient of qkv is one fused [T, 3*H*d] tensor.
    `plan` may be a plan built once for the batch and shared by every layer."""
    if qkv.dim() != 2 or qkv.dtype != torch.bfloat16 or not qkv.is_contiguous():
        raise ValueError("qkv must be a contiguous bf16 [T, 3*H*d] tensor")
    _on_gpu(qkv.device, qkv)
    _check_cu(cu_seqlens, qkv.device)
    if qkv.shape[1] % (3 * num_heads) != 0:
        raise ValueError("qkv width must be 3 * num_heads * head_dim")
    d = qkv.shape[1] // (3 * num_heads)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    o, _ = _AttentionQKV.apply(qkv, cu_seqlens, int(max_seqlen), int(num_heads), scale,
                               float(rope_base), plan)
    return o


def attention(q, k, v, cu_seqlens, max_seqlen, softmax_scale=None, rope_base=10000.0):
    """Autograd entry: o = attention over packed sequences (see esm_attn_fwd)."""
    scale = 1.0 / math.sqrt(q.shape[-1]) if softmax_scale is None else float(softmax_scale)
    return _Attention.apply(q, k, v, cu_seqlens, int(max_seqlen), scale, float(rope_base))
