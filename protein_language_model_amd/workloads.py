"""Seeded synthetic inputs for the attention hot path, shared by the tests,
the benchmark and the smoke check. Holds no attention arithmetic: it only
draws sequence lengths and bf16 activations, and counts work.

The pages train on UniRef-derived protein sequences (BioNeMo blog, section
3.2; "BioNeMo Framework" review page, Abstract) that are not available here.
Attention cost depends only on the sequence lengths, the head count and the
head dimension, so these seeded stand-ins keep the shapes and length mixes of
ESM-2 models from 8M to 15B parameters (BioNeMo Recipes hub page, model zoo)
with standard-normal activations:

  esm2_8m    4 sequences {37, 64, 100, 128}, H=20, d=16
  esm2_150m  32 lengths uniform in [50, 1024], sorted ascending (bucketed), H=20, d=32
  esm2_650m  16 x 1024 tokens (dense max-crop batch), H=20, d=64
  esm2_3b    ~65536 tokens, lengths lognormal (median 300, sigma 0.8) clipped
             to [30, 1024] in draw order, H=40, d=64, q and k scaled by 3
  esm2_15b   4 x 8192, H=40, d=128
  esm2_15b_ragged  {8192, 1000, 31}, H=40, d=128

Recipe: numpy PCG64 default_rng(seed); lengths first (where random), then q,
k, v, dO, each float32 standard normal of shape [T][H][d] in C order; the
3B-shaped workload multiplies q and k by 3 in float32; each tensor is then
rounded once to bf16 (round-to-nearest-even) and kept as uint16 bit patterns.
"""

import math
from dataclasses import dataclass, field

import numpy as np

ROPE_BASE = 10000.0


@dataclass(frozen=True)
class Workload:
    name: str
    num_heads: int
    head_dim: int
    seed: int
    lengths: tuple = ()          # fixed lengths, if not drawn
    kind: str = "fixed"          # fixed | uniform_sorted | lognormal_packed
    qk_scale: float = 1.0
    description: str = ""
    params: dict = field(default_factory=dict)


WORKLOADS = {
    "esm2_8m": Workload("esm2_8m", 20, 16, 1, (37, 64, 100, 128),
                        description="ESM-2-8M-shaped, 4 packed sequences"),
    "esm2_150m": Workload("esm2_150m", 20, 32, 2, kind="uniform_sorted",
                          params=dict(count=32, lo=50, hi=1024),
                          description="ESM-2-150M-shaped, 32 bucket-sorted sequences"),
    "esm2_650m": Workload("esm2_650m", 20, 64, 3, (1024,) * 16,
                          description="ESM-2-650M-shaped, 16 x 1024 dense crop"),
    "esm2_3b": Workload("esm2_3b", 40, 64, 4, kind="lognormal_packed",
                        qk_scale=3.0,
                        params=dict(total=65536, median=300.0, sigma=0.8,
                                    lo=30, hi=1024),
                        description="ESM-2-3B-shaped, ~64k packed lognormal lengths"),
    "esm2_15b": Workload("esm2_15b", 40, 128, 5, (8192,) * 4,
                         description="ESM-2-15B-shaped long context, 4 x 8192"),
    "esm2_15b_ragged": Workload("esm2_15b_ragged", 40, 128, 6, (8192, 1000, 31),
                                description="ESM-2-15B-shaped ragged tails"),
}


def draw_lengths(w, rng):
    """Sequence lengths of a workload, drawn from rng where random."""
    if w.kind == "fixed":
        return [int(x) for x in w.lengths]
    if w.kind == "uniform_sorted":
        p = w.params
        L = rng.integers(p["lo"], p["hi"] + 1, size=p["count"])
        return sorted(int(x) for x in L)
    if w.kind == "lognormal_packed":
        p = w.params
        out, total = [], 0
        while True:
            x = rng.lognormal(math.log(p["median"]), p["sigma"])
            L = int(min(max(np.rint(x), p["lo"]), p["hi"]))
            if total + L > p["total"]:
                break
            out.append(L)
            total += L
        return out
    raise ValueError(w.kind)


def f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def cu_from_lengths(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def make_inputs(name_or_workload, seed=None, lengths=None, num_heads=None,
                head_dim=None, with_grad=True):
    """Seeded inputs of a workload. Returns a dict with
      lengths (list), cu_seqlens (int32 [B+1]), T, H, d, scale, rope_base,
      q, k, v, do: uint16 bf16 bit patterns [T][H][d] (do only if with_grad).
    lengths / num_heads / head_dim override the workload (small parity cases
    reuse a workload's distribution at other shapes)."""
    w = WORKLOADS[name_or_workload] if isinstance(name_or_workload, str) else name_or_workload
    rng = np.random.default_rng(w.seed if seed is None else seed)
    L = draw_lengths(w, rng) if lengths is None else [int(x) for x in lengths]
    H = w.num_heads if num_heads is None else int(num_heads)
    d = w.head_dim if head_dim is None else int(head_dim)
    T = int(sum(L))
    shape = (T, H, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    do = rng.standard_normal(shape, dtype=np.float32) if with_grad else None
    if w.qk_scale != 1.0:
        q = q * np.float32(w.qk_scale)
        k = k * np.float32(w.qk_scale)
    out = dict(name=w.name, lengths=L, cu_seqlens=cu_from_lengths(L), T=T,
               H=H, d=d, scale=1.0 / math.sqrt(d), rope_base=ROPE_BASE,
               q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k),
               v=f32_to_bf16_bits(v))
    if with_grad:
        out["do"] = f32_to_bf16_bits(do)
    return out


def lengths_of(name, seed=None):
    w = WORKLOADS[name]
    return draw_lengths(w, np.random.default_rng(w.seed if seed is None else seed))


# --------------------------------------------------------------------------
# counted work and algorithmic bytes
# --------------------------------------------------------------------------

def counted_flops(lengths, num_heads, head_dim):
    """Counted attention work: forward 4 * sum(L^2) * H * d flops (two
    matrix products per (sequence, head), bidirectional so no causal
    halving); backward 2.5 times the forward. Softmax, rotary embedding and
    row sums are not counted. Returns (forward, backward)."""
    s2 = float(sum(int(L) * int(L) for L in lengths))
    fwd = 4.0 * s2 * num_heads * head_dim
    return fwd, 2.5 * fwd


def algorithmic_bytes(total_tokens, num_heads, head_dim):
    """Bytes the method must move through HBM (the L x L matrices never do).
    forward : read q, k, v (bf16) + write O (bf16) + write LSE (fp32)
    backward: read q, k, v, O, dO + LSE; write dq, dk, dv (bf16) + D (fp32)
    Returns (forward, backward)."""
    e = float(total_tokens) * num_heads * head_dim
    rows = float(total_tokens) * num_heads
    fwd = 4 * e * 2 + rows * 4
    bwd = 8 * e * 2 + rows * 4 * 2
    return fwd, bwd
