"""Float64 reference for ESM-2-style attention over packed variable-length
sequences: rotary position embedding, bidirectional softmax attention per
sequence and head, and its analytic backward.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.

Sources and readings
--------------------
* ESM-2 is a BERT-style protein language model ("BioNeMo Framework: a
  modular, high-performance library for AI model development in drug
  discovery" review page, Abstract and the "proposed method" list), so
  attention is bidirectional: every token of a sequence attends to every
  token of the same sequence and to nothing else.
* Sequences of different lengths are grouped by a size-aware bucket batch
  sampler and packed with almost no padding (same review page, "proposed
  method" and "main findings"). A batch is therefore a packed token-major
  tensor [T][H][d] plus prefix offsets cu_seqlens[B+1]; sequence b owns
  tokens cu_seqlens[b] .. cu_seqlens[b+1]-1.
* Training runs in BF16 (BioNeMo Recipes hub page, multi-precision training
  section) with FP32 accumulation (BioNeMo blog, section 2.3). Inputs are
  bf16 values; this oracle upcasts them exactly to float64.
* The pages do not print the attention formula. The textbook definitions
  are used: scaled dot-product attention (Vaswani et al. 2017) and rotary
  position embedding (Su et al. 2021, RoFormer) in the half-split pairing,
  frequencies theta_j = base^(-2j/d), positions counted from 0 at the start
  of each sequence.
* Precision model ("mode"): "exact" keeps the rotated q and k in float64,
  S = scale * (q~ . k~). "bf16_operands" models a kernel that feeds bf16
  matrix units and exponentiates with exp2: its operands are
    k^ = bf16(R(p) k),  q^ = bf16(fl32(c * fl32(R(p) q))),
    c = fl32(fl32(scale) * fl32(log2 e)),
  rounded to nearest even, and S = ln(2) * (q^ . k^) (the softmax scale and
  log2 e ride on the query operand). Those roundings are quantisations
  decided by floating point, so they are taken in the pages' arithmetic
  precision, float32 (BF16 storage with FP32 arithmetic): cos and sin are
  rounded to float32 and x c - y s, y c + x s are evaluated in float32 with
  every product and sum rounded (no fused multiply-add), the product with c
  is rounded to float32, then each operand is rounded to bf16. Gradients
  pass straight through the roundings: dq~ = scale * dS k^ and
  dk~ = dS^T (ln(2) q^), which is scale * dS^T q~ in exact arithmetic.
  Everything else is float64 in both modes.
"""

import numpy as np

MODES = ("exact", "bf16_operands")


# --------------------------------------------------------------------------
# bf16 helpers
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64, exactly (a bf16 value is the
    float32 whose upper 16 bits are the pattern)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to_bf16(x):
    """Round float64 values to the nearest bf16 value (ties to even), returned
    as float64. bf16 has 8 significant bits and float32's exponent range:
    the grid spacing at |x| in [2^e, 2^(e+1)) is 2^(e-7), never finer than the
    subnormal spacing 2^-133. Magnitudes that round past the largest finite
    bf16 become infinities; NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0.0)
    xf = x[finite]
    _, e = np.frexp(xf)            # xf = m * 2^e with 0.5 <= |m| < 1
    e = np.maximum(e, -125)        # below 2^-126 the spacing stays 2^-133
    spacing = np.ldexp(1.0, e - 8)
    r = np.rint(xf / spacing) * spacing   # np.rint rounds halves to even
    max_bf16 = float(np.ldexp(255.0, 120))  # (2 - 2^-7) * 2^127
    r = np.where(np.abs(r) > max_bf16, np.copysign(np.inf, xf), r)
    out[finite] = r
    return out


# --------------------------------------------------------------------------
# rotary position embedding
# --------------------------------------------------------------------------

def rope_frequencies(head_dim, base):
    """theta_j = base^(-2j/d) for j in [0, d/2), float64. base == 0 means the
    embedding is switched off (returns None)."""
    if head_dim % 2:
        raise ValueError("head_dim must be even for rotary embedding")
    if base == 0:
        return None
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * j / head_dim)


def rope_rotate(x, positions, base, inverse=False):
    """Rotate the last axis of x (length d) by the position angles.

    Half-split pairing: coordinate j pairs with coordinate j + d/2, and the
    pair (x_j, x_{j+d/2}) is turned by the angle a = p * theta_j:
        x~_j       = x_j cos a - x_{j+d/2} sin a
        x~_{j+d/2} = x_{j+d/2} cos a + x_j sin a
    inverse=True applies the transpose (rotation by -a), which is what the
    gradient of a rotated vector passes back to the unrotated one.
    x has shape [L, ..., d]; positions has shape [L]."""
    x = np.asarray(x, dtype=np.float64)
    theta = rope_frequencies(x.shape[-1], base)
    if theta is None:
        return x.copy()
    half = x.shape[-1] // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    cos = np.cos(ang)
    sin = -np.sin(ang) if inverse else np.sin(ang)
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (half,)
    cos = cos.reshape(shape)
    sin = sin.reshape(shape)
    lo = x[..., :half]
    hi = x[..., half:]
    out = np.empty_like(x)
    out[..., :half] = lo * cos - hi * sin
    out[..., half:] = hi * cos + lo * sin
    return out


def rope_rotate_f32(x, positions, base):
    """The rotation of rope_rotate evaluated in float32: angles p * theta_j in
    float64, cos and sin rounded to float32, then
        x~_j       = fl(fl(x_j c) - fl(x_{j+d/2} s))
        x~_{j+d/2} = fl(fl(x_{j+d/2} c) + fl(x_j s))
    with fl() rounding to float32 (numpy float32 arithmetic, no fused
    multiply-add). x must hold float32-representable values. Returns float64
    holding the float32 results."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    theta = rope_frequencies(x32.shape[-1], base)
    if theta is None:
        return x32.astype(np.float64)
    half = x32.shape[-1] // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    shape = (x32.shape[0],) + (1,) * (x32.ndim - 2) + (half,)
    cos = np.cos(ang).astype(np.float32).reshape(shape)
    sin = np.sin(ang).astype(np.float32).reshape(shape)
    lo = x32[..., :half]
    hi = x32[..., half:]
    out = np.empty_like(x32)
    out[..., :half] = lo * cos - hi * sin
    out[..., half:] = hi * cos + lo * sin
    return out.astype(np.float64)


LOG2E_F32 = np.float32(np.log2(np.e))


def query_operand_bf16(q, pos, base, scale):
    """q^ = bf16(fl32(c * fl32(R(p) q))), c = fl32(fl32(scale) * fl32(log2 e)):
    the bf16 query operand of the bf16_operands mode (float64 values)."""
    c = np.float32(scale) * LOG2E_F32
    rot = rope_rotate_f32(q, pos, base).astype(np.float32)
    return round_to_bf16((rot * c).astype(np.float64))


def _operands(q, k, base, scale, mode):
    """(positions, scaled query operand qs, key operand kr), S = qs @ kr^T:
    exact: qs = scale * R(p) q; bf16_operands: qs = ln(2) * q^."""
    if mode not in MODES:
        raise ValueError("mode must be one of %r" % (MODES,))
    pos = np.arange(q.shape[0], dtype=np.float64)  # 0-based per sequence
    if mode == "bf16_operands":
        qs = np.log(2.0) * query_operand_bf16(q, pos, base, scale)
        kr = round_to_bf16(rope_rotate_f32(k, pos, base))
    else:
        qs = float(scale) * rope_rotate(q, pos, base)
        kr = rope_rotate(k, pos, base)
    return pos, qs, kr


# --------------------------------------------------------------------------
# one (sequence, head) slice
# --------------------------------------------------------------------------

def attention_forward_slice(q, k, v, scale, base, mode="bf16_operands"):
    """Forward attention of one sequence and one head.

    q, k, v: [L, d] float64 (pre-rotation q and k). Returns
      O   [L, d]: O_i = sum_j P_ij v_j,
      LSE [L]   : LSE_i = log sum_j exp(S_ij) (natural log, scale included),
    with S_ij = scale * (q~_i . k~_j) and P_ij = exp(S_ij - LSE_i).
    The maximum is subtracted before exponentiating, which changes nothing
    mathematically and keeps exp() finite."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L = q.shape[0]
    if L == 0:
        return np.zeros_like(v), np.zeros((0,), np.float64)
    _, qs, kr = _operands(q, k, base, scale, mode)
    S = qs @ kr.T
    m = S.max(axis=1)
    lse = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    P = np.exp(S - lse[:, None])
    return P @ v, lse


def attention_forward_partial_slice(q, k, v, scale, base, key_lo, key_hi,
                                    mode="bf16_operands"):
    """Attention of every query of one sequence and head against only the
    keys key_lo .. key_hi-1 (rotary positions those of the whole sequence):
    a key-range partial, the unit of work that context parallelism deals out
    when one sequence's keys are split across devices ("Scaling biomolecular
    modeling with context parallelism in NVIDIA BioNeMo" page, "2D tiling of
    the pairwise representation": each device owns a sub-block of the N x N
    interactions).

    Returns O_r [L, d] = sum_{j in range} P^r_ij v_j with P^r the softmax over
    the range, and LSE_r [L] = log sum_{j in range} exp(S_ij); an empty
    range gives O_r = 0 and LSE_r = -inf."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L = q.shape[0]
    if L == 0 or key_hi <= key_lo:
        return np.zeros((L, v.shape[1])), np.full((L,), -np.inf)
    _, qs, kr = _operands(q, k, base, scale, mode)
    S = qs @ kr[key_lo:key_hi].T
    m = S.max(axis=1)
    lse = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    P = np.exp(S - lse[:, None])
    return P @ v[key_lo:key_hi], lse


def merge_partials(o_parts, lse_parts):
    """Combines key-range partials of the same queries: with
    LSE = log sum_r exp(LSE_r), the softmax over the union of the ranges is
    exp(S_ij - LSE) = exp(LSE_r - LSE) P^r_ij, hence
    O = sum_r exp(LSE_r - LSE) O_r. Parts with LSE_r = -inf add nothing.
    o_parts [R, L, d], lse_parts [R, L] -> (O [L, d], LSE [L])."""
    o_parts = np.asarray(o_parts, np.float64)
    lse_parts = np.asarray(lse_parts, np.float64)
    m = lse_parts.max(axis=0)
    safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse_parts - safe[None, :])
    tot = w.sum(axis=0)
    lse = np.where(tot > 0, safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    o = (w[:, :, None] * o_parts).sum(axis=0) / np.where(tot > 0, tot, 1.0)[:, None]
    return o, lse


def attention_backward_slice(q, k, v, do, scale, base, mode="bf16_operands",
                             return_intermediates=False):
    """Gradients of sum(dO * O) for one sequence and one head.

    With P from the forward definition:
      dV_j  = sum_i P_ij dO_i
      dP_ij = dO_i . v_j
      D_i   = sum_j P_ij dP_ij
      dS_ij = P_ij (dP_ij - D_i)
      dq~_i = scale * sum_j dS_ij k~_j
      dk~_j = scale * sum_i dS_ij q~_i   (sum_i dS_ij qs_i, qs the scaled
                                          query operand of the mode)
      dq_i  = R(-p_i) dq~_i,   dk_j = R(-p_j) dk~_j
    Returns (dq, dk, dv), each [L, d]; with return_intermediates also a dict
    of P, dS, D, LSE, the rotated-space gradients and the operands."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    L = q.shape[0]
    if L == 0:
        z = np.zeros_like(q)
        out = (z, z.copy(), z.copy())
        return out + ({},) if return_intermediates else out
    pos, qs, kr = _operands(q, k, base, scale, mode)
    s = float(scale)
    S = qs @ kr.T
    m = S.max(axis=1)
    lse = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    P = np.exp(S - lse[:, None])
    dv = P.T @ do
    dP = do @ v.T
    D = (P * dP).sum(axis=1)
    dS = P * (dP - D[:, None])
    dqr = s * (dS @ kr)
    dkr = dS.T @ qs
    dq = rope_rotate(dqr, pos, base, inverse=True)
    dk = rope_rotate(dkr, pos, base, inverse=True)
    if return_intermediates:
        return dq, dk, dv, dict(P=P, dS=dS, D=D, LSE=lse, dq_rot=dqr,
                                dk_rot=dkr, q_scaled=qs, k_rot=kr)
    return dq, dk, dv


def attention_rows_slice(q, k, v, do, scale, base, rows, mode="bf16_operands"):
    """The forward and the query gradient of one sequence and head at the
    query rows `rows` only: the definitions above restricted to those rows
    (every key still enters), O(len(rows) * L * d) work, so long sequences
    can be checked row by row. Returns (O [r, d], LSE [r], dq [r, d])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    pos, qs, kr = _operands(q, k, base, scale, mode)
    s = float(scale)
    S = qs[rows] @ kr.T
    m = S.max(axis=1)
    lse = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    P = np.exp(S - lse[:, None])
    O = P @ v
    dP = do[rows] @ v.T
    D = (P * dP).sum(axis=1)
    dqr = s * ((P * (dP - D[:, None])) @ kr)
    dq = rope_rotate(dqr, pos[rows], base, inverse=True)
    return O, lse, dq


# --------------------------------------------------------------------------
# packed batches
# --------------------------------------------------------------------------

def _check_packed(q, cu_seqlens):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0 and be nondecreasing")
    if cu[-1] != q.shape[0]:
        raise ValueError("cu_seqlens[-1] must equal the token count")
    return cu


def forward(q, k, v, cu_seqlens, scale, rope_base, mode="bf16_operands",
            seqs=None, heads=None):
    """Packed forward. q, k, v: [T, H, d] float64. Returns O [T, H, d] and
    LSE [H, T]. Only the listed sequences / heads are computed when seqs /
    heads are given (for sampled checks at large sizes); other entries are
    NaN."""
    cu = _check_packed(q, cu_seqlens)
    T, H, d = q.shape
    O = np.full((T, H, d), np.nan)
    LSE = np.full((H, T), np.nan)
    seqs = range(cu.size - 1) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    for b in seqs:
        a, e = int(cu[b]), int(cu[b + 1])
        for h in heads:
            o, lse = attention_forward_slice(q[a:e, h], k[a:e, h], v[a:e, h],
                                             scale, rope_base, mode)
            O[a:e, h] = o
            LSE[h, a:e] = lse
    return O, LSE


def backward(q, k, v, do, cu_seqlens, scale, rope_base, mode="bf16_operands",
             seqs=None, heads=None):
    """Packed backward. Returns dq, dk, dv, each [T, H, d] (NaN where not
    computed when seqs / heads restrict the work)."""
    cu = _check_packed(q, cu_seqlens)
    T, H, d = q.shape
    dq = np.full((T, H, d), np.nan)
    dk = np.full((T, H, d), np.nan)
    dv = np.full((T, H, d), np.nan)
    seqs = range(cu.size - 1) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    for b in seqs:
        a, e = int(cu[b]), int(cu[b + 1])
        for h in heads:
            g = attention_backward_slice(q[a:e, h], k[a:e, h], v[a:e, h],
                                         do[a:e, h], scale, rope_base, mode)
            dq[a:e, h], dk[a:e, h], dv[a:e, h] = g
    return dq, dk, dv

