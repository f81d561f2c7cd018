"""Reference for the FP8 (OCP E4M3) forward: q~ and k~ quantized to E4M3 with
per-tensor scales, S and the softmax in float64, V in bf16.

TEST INFRASTRUCTURE: imported only by tests; never by the product path.

Sources and readings
--------------------
* The BioNeMo Recipes hub page lists FP8 among its training precisions
  (multi-precision training section; a multi-node FP8 recipe that needs
  Hopper-class GPUs or newer). It fixes neither the FP8 format nor the
  scaling. Reading: OCP 8-bit floating point E4M3 (1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; subnormals 2^-6 * m/8; largest finite
  value 448; no infinities), the format of gfx950's FP8 matrix instructions.
* Quantization is a decision taken in floating point, so it is taken in
  float32 exactly as a kernel does: the rotated operand in float32 (the
  rotation of attention.rope_rotate_f32), times the float32 reciprocal of the
  scale (one float32 rounding), clamped to [-448, 448], rounded to the
  nearest E4M3 value, ties to even (the clamp is the reading for overflow:
  saturate, since E4M3 has no infinity).
* Only the products S = q~ k~^T take the FP8 operands (an inference-first
  variant of the forward); the softmax, P and V stay as in the BF16 forward:
  S_ij = scale * s_q * s_k * (q8_i . k8_j), the rest the textbook definition
  in float64.
"""

import numpy as np

from .attention import rope_rotate_f32

E4M3_MAX = 448.0


def round_to_e4m3(x):
    """Nearest E4M3 value (ties to even) of each element after clamping to
    [-448, 448]. Quantum: 2^(e-3) for |x| in [2^e, 2^(e+1)), e >= -6; 2^-9
    below 2^-6 (subnormals). float64 in and out."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    quantum = 2.0 ** (e - 3)
    r = np.round(a / quantum) * quantum        # numpy rounds halves to even
    return np.where(x < 0, -r, r)


def decode_e4m3(codes):
    """Values of E4M3 bit patterns (uint8); NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def quantize(x_f32, scale):
    """E4M3 value of x * fl32(1 / scale), the product rounded to float32."""
    inv = np.float32(1.0) / np.float32(scale)
    y = (np.asarray(x_f32, dtype=np.float64).astype(np.float32) * inv).astype(np.float64)
    return round_to_e4m3(y)


def quantize_rotated(x, base, scale):
    """q8 (or k8) of one sequence and head: positions 0..L-1."""
    x = np.asarray(x, dtype=np.float64)
    rot = rope_rotate_f32(x, np.arange(x.shape[0]), base)
    return quantize(rot, scale)


def attention_forward_fp8_slice(q, k, v, scale, base, q_scale, k_scale):
    """O [L, d] and LSE [L] of one sequence and head with E4M3 q~ and k~."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L = q.shape[0]
    if L == 0:
        return np.zeros_like(v), np.zeros((0,), np.float64)
    q8 = quantize_rotated(q, base, q_scale)
    k8 = quantize_rotated(k, base, k_scale)
    S = float(scale) * float(np.float32(q_scale)) * float(np.float32(k_scale)) * (q8 @ k8.T)
    m = S.max(axis=1)
    lse = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    P = np.exp(S - lse[:, None])
    return P @ v, lse
