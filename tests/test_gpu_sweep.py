"""Seeded sweep over drawn batch shapes: the one-shot forward and backward
(through the C ABI, so each case takes whichever path the library picks:
the small-batch launches when every sequence has at most 128 tokens and
d <= 64, else the plan, the rotation pass and the planned kernels) against
the float64 oracle in both precision modes, on every row and head.

Each case draws, from its own seed, the head dim (16, 32, 64, 128), the head
count, the batch size, lengths mixing tile edges (multiples of 32, 64 and 128
and their neighbours), empty and one-token sequences and uniform draws, the
softmax scale (0.5 to 1 times 1/sqrt(d); ESM-2 itself uses 1/sqrt(d), and
larger scales sharpen the softmax, where rounding the operands to bf16 moves
O against the exact oracle by more than its bound for any bf16 kernel: the
sharpened and x10 cases cover that regime) and the rotary base (10000, 500,
or 0 = no rotation). Sizes stay where the oracle finishes each case in a few
seconds."""

import math

import numpy as np
import pytest

from gpu_helpers import compare, run_gpu, say
from protein_language_model_amd import workloads as W

pytestmark = pytest.mark.gpu

NAME_OF_D = {16: "esm2_8m", 32: "esm2_150m", 64: "esm2_650m", 128: "esm2_15b"}
EDGES = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]
N_CASES = 32
MAX_TOKENS = 2500


def draw_case(i):
    rng = np.random.default_rng(7000 + i)
    d = int(rng.choice([16, 32, 64, 128]))
    H = int(rng.integers(1, 4))
    B = int(rng.integers(1, 7))
    small_only = i % 4 == 0  # every fourth case keeps every sequence within 128 tokens
    lengths = []
    for _ in range(B):
        if rng.random() < 0.5:
            L = int(rng.choice([e for e in EDGES if not small_only or e <= 128]))
        else:
            L = int(rng.integers(1, 129 if small_only else 700))
        lengths.append(L)
    while sum(lengths) > MAX_TOKENS:
        lengths.pop()
    if sum(lengths) == 0:
        lengths.append(int(rng.integers(1, 100)))
    scale = float(rng.uniform(0.5, 1.0)) / math.sqrt(d)
    base = float(rng.choice([10000.0, 500.0, 0.0]))
    return dict(name=NAME_OF_D[d], lengths=lengths, H=H, d=d, scale=scale, base=base,
                seed=100 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_drawn_shape_parity(device, i):
    c = draw_case(i)
    inp = W.make_inputs(c["name"], seed=c["seed"], lengths=c["lengths"], num_heads=c["H"],
                        head_dim=c["d"])
    label = "sweep %d d=%d H=%d L=%s scale=%.4f base=%g" % (i, c["d"], c["H"], c["lengths"],
                                                          c["scale"], c["base"])
    say("case", label)
    gpu = run_gpu(inp, device, scale=c["scale"], rope_base=c["base"])
    compare(gpu, inp, scale=c["scale"], rope_base=c["base"], label=label)
