"""Benchmark of the varlen RoPE attention hot path on one MI355X.

A step is one pass of the whole path over one packed batch held in HBM:
plan (varlen schedule + rotary table), rotation of q and k, forward (O, LSE),
backward dq pass (with D = rowsum(dO*O) and the inverse-rotation finalize)
and dk/dv pass. A batch whose sequences all fit one 128-row work item
(max_seqlen <= 128, d <= 64) takes the library's small-batch path instead:
esm_attn_fwd and esm_attn_bwd, one launch each.
The default workload is the ESM-2-650M-shaped dense batch: 16 sequences of
1024 tokens, 20 heads, head dim 64, bf16, RoPE base 10000.

Prints ONE JSON line. `value` is counted TFLOP/s of forward + backward
(forward 4*sum(L^2)*H*d, backward 2.5x that) over the wall clock of the K
timed steps, which run with nothing recorded between the calls;
`kernels_us` are per-call times from events recorded around each call in a
second pass of K steps, on the stream the kernels are launched on (event
records add idle gaps between the kernels, so that pass's step time,
`ms_per_step_with_events`, is longer); `roofline` describes the dominant
kernel with its average launch time from that pass; `cpu_baseline` times
the float64 oracle on a bounded sample on the host.

Extra fields, all measured after the timed region (which is untouched by
them): `step_us_spread` (per-step times from one event per step boundary:
median, p10, p90 and the means of the first and last five steps, which show
the clock ramp that a short warmup leaves in the timed steps);
`ms_per_step_settled` / `tflops_settled` (K more event-free steps once the
process has run at least 150 steps, when the clocks are steady); `fwd_us` and
`bwd_us` (plan + rotation + forward, and the two backward passes: median,
p10, p90) and `kernels_us_pct`; `flushed` (each step preceded by an untimed
512 MiB write that evicts the 256 MB last-level cache, with the step's
algorithmic HBM bytes over its median time); `graph_replay_ms_per_step` (the
step captured once in a HIP graph and replayed K times).

    python bench.py [--gpus 1] [--steps 50] [--warmup 100] [--workload esm2_650m] [--seed S]
                    [--no-cpu-baseline] [--cpu-seconds 15]

`--attention-block` times instead the whole attention block of one layer at
the workload's shape: QKV projection (one GEMM to [T][3][H][d]), this path
on that fused buffer in place (rotation in place, strided q, k, v; dq, dk, dv
into one fused gradient), output projection, forward and backward with the
weight gradients; and the same block with the split layout (q, k, v copied
out of the projection, the gradients concatenated). Prints one JSON line.

`--packing-study` forms batches from a UniRef-like length mix (20,000
lengths, lognormal with median 300 and sigma 0.8, cropped to [30, 1024]) with
the library's size-aware bucket batcher under a 16,384-token budget, four
ways (no buckets / 64-token buckets, packed / padded cost), reports padding
and wasted attention work, and times this path (plan, rotation, forward,
backward; H = 20, d = 64) over all of each way's batches (one epoch), padded
batches run with every sequence at its batch's longest length. Prints one
JSON line.

`--split-kv` times the forward plain and split into n_split key-range
partials plus their merge (esm_attn_fwd_split_planned) on shapes with few
work items: one 8,192-token sequence with 5 heads of 128 (the local heads of
a sequence-parallel shard of the 15B shape), two 4,096-token sequences with 8
heads of 64, and the 16 x 1,024 650M batch. Prints one JSON line.

`--fp8` times the E4M3 forward (quantization of the rotated q, k + the FP8
forward) against the bf16 forward (rotation + forward) on the 650M and 15B
batches. Prints one JSON line.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0
SETTLE_STEPS = 150          # steps of sustained load after which the clocks are steady


def pct(xs):
    """median, p10 and p90 of a list of times (us), rounded."""
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2)}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # the chip's clocks ramp for the first ~40 steps of sustained load (0.64
    # ms/step, then 0.46 at the 650M shape): the default warmup covers that
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="esm2_650m")
    p.add_argument("--seed", type=int, default=None,
                   help="input seed (default: the workload's own, which fixes its lengths)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 256 MiB device copy (calibrates HBM byte counters)")
    p.add_argument("--attention-block", action="store_true",
                   help="time QKV projection + attention + output projection, fwd + bwd")
    p.add_argument("--packing-study", action="store_true",
                   help="padded vs packed batches of a length mix: padding, waste, tokens/s")
    p.add_argument("--split-kv", action="store_true",
                   help="forward plain vs split into key-range partials + merge")
    p.add_argument("--fp8", action="store_true",
                   help="E4M3 forward vs bf16 forward (inference)")
    return p.parse_args()


def copy_calibration():
    """A plain device-to-device copy of 256 MiB, three times: under a
    FETCH_SIZE / WRITE_SIZE counter run it gives the counters' reading for
    known traffic (256 MiB read + 256 MiB written per dispatch)."""
    import torch
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "dispatches": 3}), flush=True)


def _source_sha256():
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "protein_language_model_amd",
                        "csrc")
    for p in sorted(glob.glob(os.path.join(csrc, "*"))):
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def forward_step(E, q, k, v, B, maxL, plan, scale, base, q_rot, k_rot, out=None, lse=None,
                 mid=None):
    """The forward half of a training step after the plan: the rotation pass
    and the forward, with q rotated inside the forward where the library
    does so (E.fwd_rotates_q: d <= 64) and by the rotation pass otherwise.
    q_rot / k_rot receive the rotated operands for the backward (q_rot = q,
    k_rot = k rotates in place). mid() runs between the two calls. Returns
    (o, lse)."""
    if E.fwd_rotates_q(v.shape[-1]):
        E.esm_attn_rotate_planned(None, k, B, maxL, plan, base, k_rot=k_rot, softmax_scale=scale)
        if mid is not None:
            mid()
        o, lse, _ = E.esm_attn_fwd_rotq_planned(q, k_rot, v, B, maxL, plan, scale, base, out=out,
                                                lse=lse, q_rot=q_rot)
    else:
        E.esm_attn_rotate_planned(q, k, B, maxL, plan, base, q_rot=q_rot, k_rot=k_rot,
                                  softmax_scale=scale)
        if mid is not None:
            mid()
        o, lse = E.esm_attn_fwd_planned(q_rot, k_rot, v, B, maxL, plan, scale, out=out, lse=lse)
    return o, lse


def measured_traffic(workload, kernel_name):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by the reading of a plain
    copy of known size), or None when the summary is missing or was taken on
    other kernel sources."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        "hbm_traffic_%s.json" % workload)
    try:
        with open(path) as f:
            rec = json.load(f)
    except OSError:
        return None
    if rec.get("source_sha256") != _source_sha256():
        return None
    for name, t in rec["kernels"].items():
        if kernel_name in name:
            return {"bytes": t["read_bytes"] + t["write_bytes"], "read_bytes": t["read_bytes"],
                    "write_bytes": t["write_bytes"], "commit": rec.get("commit")}
    return None


def cpu_baseline(inp, budget_s):
    """Times the float64 oracle (forward + backward, bf16-operand mode) on
    (sequence, head) slices of the same workload until about budget_s of CPU
    work, and scales to counted TFLOP/s."""
    import oracle
    from protein_language_model_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    q, k, v, do = (oracle.bf16_bits_to_f64(inp[n]) for n in ("q", "k", "v", "do"))
    cu = inp["cu_seqlens"]
    slices = [(b, h) for b in range(len(cu) - 1) for h in range(inp["H"])]
    done, flops = 0, 0.0
    t0 = time.perf_counter()
    # cycles through the workload's slices until the budget is spent
    while done == 0 or time.perf_counter() - t0 <= budget_s:
        b, h = slices[done % len(slices)]
        a, e = int(cu[b]), int(cu[b + 1])
        oracle.attention_forward_slice(q[a:e, h], k[a:e, h], v[a:e, h], inp["scale"],
                                       inp["rope_base"])
        oracle.attention_backward_slice(q[a:e, h], k[a:e, h], v[a:e, h], do[a:e, h],
                                        inp["scale"], inp["rope_base"])
        f, bwd = W.counted_flops([e - a], 1, inp["d"])
        flops += f + bwd
        done += 1
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": "float64 oracle forward+backward on %d (sequence, head) slices of %s "
                      "(%d in the workload; %.1f s, counted flops scaled to TFLOP/s)"
                      % (done, inp["name"], len(slices), dt)}


def attention_block(args):
    """One layer's attention block, forward and backward, at the workload's
    shape (hidden = H*d): qkv = x Wqkv^T + b; attention; y = o Wo^T + b; then
    dO = dy Wo, dWo = dy^T o, the attention backward, dx = dqkv Wqkv,
    dWqkv = dqkv^T x and the bias gradients. GEMMs are torch's (hipBLASLt);
    the attention path is this library's. Counted flops: 24 T hidden^2 for
    the GEMMs plus the attention's counted flops."""
    import torch
    import torch.nn.functional as F
    from protein_language_model_amd import esm_attn as E
    from protein_language_model_amd import workloads as W

    dev = torch.device("cuda:0")
    wl = W.WORKLOADS[args.workload]
    lengths = W.lengths_of(args.workload)
    H, d = wl.num_heads, wl.head_dim
    hid, T, B, maxL = H * d, int(sum(lengths)), len(lengths), max(lengths)
    scale, base = 1.0 / math.sqrt(d), W.ROPE_BASE
    g = torch.Generator(device=dev).manual_seed(7)
    rnd = lambda *shape, s=1.0: (torch.randn(*shape, generator=g, device=dev) * s).to(
        torch.bfloat16)
    x, dy = rnd(T, hid), rnd(T, hid)
    wqkv, bqkv = rnd(3 * hid, hid, s=hid ** -0.5), rnd(3 * hid, s=0.02)
    wo, bo = rnd(hid, hid, s=hid ** -0.5), rnd(hid, s=0.02)
    cu = torch.from_numpy(W.cu_from_lengths(lengths)).to(dev)
    plan = torch.empty(E.esm_attn_plan_bytes(B, T, maxL, H, d), dtype=torch.uint8, device=dev)
    drow = E.drow_buffer(H, T, dev)
    dqkv = torch.empty((T, 3 * hid), dtype=torch.bfloat16, device=dev)
    st = torch.cuda.current_stream()

    def step(fused, ev=None):
        def mark(j):
            if ev is not None:
                ev[j].record(st)
        mark(0)
        E.esm_attn_plan(cu, T, maxL, H, d, base, plan=plan)
        qkv = F.linear(x, wqkv, bqkv).view(T, 3, H, d)
        mark(1)
        if fused:   # q, k rotated in place inside the projection output
            q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
            o, lse = forward_step(E, q, k, v, B, maxL, plan, scale, base, q, k)
        else:
            q, k, v = qkv[:, 0].contiguous(), qkv[:, 1].contiguous(), qkv[:, 2].contiguous()
            q_rot, k_rot = torch.empty_like(q), torch.empty_like(k)
            o, lse = forward_step(E, q, k, v, B, maxL, plan, scale, base, q_rot, k_rot)
            q, k = q_rot, k_rot
        mark(2)
        F.linear(o.view(T, hid), wo, bo)
        dout = torch.mm(dy, wo).view(T, H, d)
        torch.mm(dy.t(), o.view(T, hid))
        dy.sum(0)
        mark(3)
        if fused:
            g3 = dqkv.view(T, 3, H, d)
            E.esm_attn_bwd_planned(q, k, v, o, dout, lse, B, maxL, plan, scale, base,
                                   dq=g3[:, 0], dk=g3[:, 1], dv=g3[:, 2], drow=drow)
            grad = dqkv
        else:
            dq, dk, dv, _ = E.esm_attn_bwd_planned(q, k, v, o, dout, lse, B, maxL, plan, scale,
                                                   base, drow=drow)
            grad = torch.stack((dq, dk, dv), dim=1).view(T, 3 * hid)
        mark(4)
        torch.mm(grad, wqkv)
        torch.mm(grad.t(), x)
        grad.sum(0)
        mark(5)

    def run(fused):
        for _ in range(args.warmup):
            step(fused)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(fused, evs[i])
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / args.steps
        parts = ["plan + qkv proj", "rotate + attn fwd", "out proj fwd + bwd", "attn bwd",
                 "qkv proj bwd"]
        us = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e3
              for j, n in enumerate(parts)}
        return wall, us

    wall_f, us_f = run(True)
    wall_s, us_s = run(False)
    gemm_f = 24.0 * T * hid * hid
    fa, ba = W.counted_flops(lengths, H, d)
    total = gemm_f + fa + ba
    out = {
        "metric": "attention block (QKV proj + attention + out proj) fwd+bwd TFLOP/s",
        "value": round(total / wall_f / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_f * 1e3, 4),
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic (seeded normal activations and weights)",
        "config": {"workload": "%s attention block: %d sequences, %d tokens, hidden %d, H=%d, d=%d"
                               % (args.workload, B, T, hid, H, d)},
        "mfu": round(total / wall_f / 1e12 / PEAK_BF16_TFLOPS, 4),
        "counted_flops": {"gemms": gemm_f, "attention": fa + ba},
        "parts_us": {n: round(x, 1) for n, x in us_f.items()},
        "split_layout": {"ms_per_step": round(wall_s * 1e3, 4),
                         "value": round(total / wall_s / 1e12, 2),
                         "parts_us": {n: round(x, 1) for n, x in us_s.items()}},
    }
    print(json.dumps(out), flush=True)


def packing_study(args):
    """Bucketed size-aware batching, packed vs padded (see the module doc)."""
    import torch
    from protein_language_model_amd import esm_attn as E

    rng = np.random.default_rng(2024)
    lengths = np.clip(np.rint(rng.lognormal(math.log(300.0), 0.8, 20000)), 30, 1024).astype(
        np.int64)
    budget, H, d, base = 16384, 20, 64, 10000.0
    scale = 1.0 / math.sqrt(d)
    ways = {"no_buckets_padded": ([], True), "buckets64_padded": (list(range(64, 1025, 64)), True),
            "no_buckets_packed": ([], False), "buckets64_packed": (list(range(64, 1025, 64)), False)}
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(5)
    cap = 2 * budget  # tokens of the largest batch run (a padded batch of one can exceed budget)
    buf = {n: (torch.randn(cap, H, d, generator=g, device=dev)).to(torch.bfloat16)
           for n in ("q", "k", "v", "do")}
    outs = {n: torch.empty(cap, H, d, dtype=torch.bfloat16, device=dev)
            for n in ("qr", "kr", "o", "dq", "dk", "dv")}
    lse = torch.empty(H * cap, dtype=torch.float32, device=dev)
    drow = torch.empty(4 * H * cap, dtype=torch.float32, device=dev)  # drow_buffer(H, cap) flat

    def prepare(run_lengths):  # device cu_seqlens and plan buffer, before timing
        T, B, maxL = int(sum(run_lengths)), len(run_lengths), int(max(run_lengths))
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(run_lengths)]).astype(np.int32)).to(
            dev)
        plan = torch.empty(E.esm_attn_plan_bytes(B, T, maxL, H, d), dtype=torch.uint8,
                           device=dev)
        return T, B, maxL, cu, plan

    def run_batch(prep):
        T, B, maxL, cu, plan = prep
        q, k, v, do = (buf[n][:T] for n in ("q", "k", "v", "do"))
        qr, kr, o, dq, dk, dv = (outs[n][:T] for n in ("qr", "kr", "o", "dq", "dk", "dv"))
        E.esm_attn_plan(cu, T, maxL, H, d, base, plan=plan)
        forward_step(E, q, k, v, B, maxL, plan, scale, base, qr, kr, out=o,
                     lse=lse[:H * T].view(H, T))
        E.esm_attn_bwd_planned(qr, kr, v, o, do, lse[:H * T].view(H, T), B, maxL, plan, scale,
                               base, dq=dq, dk=dk, dv=dv, drow=drow[:4 * H * T])

    def tiles(L):  # pairs the 128-query x 64-key tiles cover
        return -(-L // 128) * 128 * (-(-L // 64)) * 64

    report = {}
    sq = float((lengths ** 2).sum())
    for name, (bounds, padded) in ways.items():
        batches = E.esm_attn_bucket_batches(lengths, bounds, budget, padded)
        run = [np.full(len(b), lengths[b].max()) if padded else lengths[b] for b in batches]
        real = float(lengths.sum())
        slots = float(sum(r.sum() for r in run))
        pairs = float(sum((r.astype(np.float64) ** 2).sum() for r in run))
        tile = float(sum(tiles(int(L)) for r in run for L in r))
        # one pass over every batch (an epoch of the length mix), after a warmup
        assert all(r.sum() <= cap for r in run)
        epoch = [prepare(r) for r in run]
        for r in epoch[:8]:
            run_batch(r)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for r in epoch:
            run_batch(r)
        torch.cuda.synchronize()
        best = time.perf_counter() - t0
        report[name] = {
            "batches": len(batches),
            "mean_sequences_per_batch": round(len(lengths) / len(batches), 2),
            "padding_fraction": round(1.0 - real / slots, 4),
            "attention_pairs_over_sum_L2": round(pairs / sq, 4),
            "kernel_tile_pairs_over_sum_L2": round(tile / sq, 4),
            "epoch_ms": round(best * 1e3, 2),
            "real_tokens_per_s": round(real / best, 1),
        }
    ref = report["buckets64_packed"]["real_tokens_per_s"]
    out = {
        "metric": "attention fwd+bwd real tokens/s by batching, packed vs padded",
        "value": ref,
        "unit": "tokens/s",
        "n_gpus": 1,
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic lengths (lognormal median 300, sigma 0.8, crop [30, 1024]), "
                "seeded normal activations",
        "config": {"workload": "20000 sequences, %d-token budget, H=%d, d=%d" % (budget, H, d)},
        "ways": report,
    }
    print(json.dumps(out), flush=True)


def split_kv_study(args):
    """Plain vs split-KV forward on few-item shapes (see the module doc)."""
    import torch
    from protein_language_model_amd import esm_attn as E
    from protein_language_model_amd import workloads as W

    dev = torch.device("cuda:0")
    shapes = [("1 x 8192, H=5, d=128", [8192], 5, 128),
              ("2 x 4096, H=8, d=64", [4096, 4096], 8, 64),
              ("16 x 1024, H=20, d=64", [1024] * 16, 20, 64)]
    g = torch.Generator(device=dev).manual_seed(3)
    st = torch.cuda.current_stream()
    res = {}
    for name, lengths, H, d in shapes:
        T, B, maxL = sum(lengths), len(lengths), max(lengths)
        q, k, v = (torch.randn(T, H, d, generator=g, device=dev).to(torch.bfloat16)
                   for _ in range(3))
        cu = torch.from_numpy(W.cu_from_lengths(lengths)).to(dev)
        plan = E.esm_attn_plan(cu, T, maxL, H, d, W.ROPE_BASE)
        qr, kr = E.esm_attn_rotate_planned(q, k, B, maxL, plan, W.ROPE_BASE,
                                           softmax_scale=1.0 / math.sqrt(d))
        o = torch.empty_like(q)
        lse = torch.empty((H, T), dtype=torch.float32, device=dev)
        parts = {R: (torch.empty((R, T, H, d), dtype=torch.float32, device=dev),
                     torch.empty((R, H, T), dtype=torch.float32, device=dev))
                 for R in (2, 3, 4, 6, 8)}

        def timed(fn, n=20):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]
            for e0, e1 in evs:
                e0.record(st)
                fn()
                e1.record(st)
            torch.cuda.synchronize()
            return float(np.median([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]))

        plain = timed(lambda: E.esm_attn_fwd_planned(qr, kr, v, B, maxL, plan, out=o, lse=lse))
        split = {R: timed(lambda R=R: E.esm_attn_fwd_split_planned(
            qr, kr, v, B, maxL, plan, R, out=o, lse=lse, o_part=parts[R][0],
            lse_part=parts[R][1])) for R in parts}
        best = min(split, key=split.get)
        fwd_f, _ = W.counted_flops(lengths, H, d)
        items = H * sum(-(-L // 128) for L in lengths)
        res[name] = {"items": items, "plain_us": round(plain, 1),
                     "split_us": {str(R): round(t, 1) for R, t in split.items()},
                     "best_n_split": best, "speedup": round(plain / split[best], 3),
                     "plain_tflops": round(fwd_f / plain * 1e-6, 1),
                     "best_split_tflops": round(fwd_f / split[best] * 1e-6, 1)}
    first = res[shapes[0][0]]
    out = {"metric": "forward TFLOP/s, plain vs split-KV (key-range partials + merge)",
           "value": first["best_split_tflops"], "unit": "TFLOP/s", "n_gpus": 1,
           "higher_is_better": True, "dtype": "bf16",
           "data": "synthetic (seeded normal bf16 activations)",
           "config": {"workload": shapes[0][0]}, "shapes": res}
    print(json.dumps(out), flush=True)


def fp8_study(args):
    """E4M3 vs bf16 forward (see the module doc)."""
    import torch
    from protein_language_model_amd import esm_attn as E
    from protein_language_model_amd import workloads as W

    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream()
    res = {}
    for name in ("esm2_650m", "esm2_15b"):
        wl = W.WORKLOADS[name]
        lengths = W.lengths_of(name)
        H, d = wl.num_heads, wl.head_dim
        T, B, maxL = sum(lengths), len(lengths), max(lengths)
        g = torch.Generator(device=dev).manual_seed(11)
        q, k, v = (torch.randn(T, H, d, generator=g, device=dev).to(torch.bfloat16)
                   for _ in range(3))
        cu = torch.from_numpy(W.cu_from_lengths(lengths)).to(dev)
        plan = E.esm_attn_plan(cu, T, maxL, H, d, W.ROPE_BASE)
        qs = float(q.abs().max()) * math.sqrt(2) / 448
        ks = float(k.abs().max()) * math.sqrt(2) / 448
        qr, kr = torch.empty_like(q), torch.empty_like(k)
        q8 = torch.empty((T, H, d), dtype=torch.uint8, device=dev)
        k8 = torch.empty_like(q8)
        o = torch.empty_like(q)
        lse = torch.empty((H, T), dtype=torch.float32, device=dev)

        def timed(fn, n=20):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
            for e in ev:
                e[0].record(st)
                fn(e[1])
                e[2].record(st)
            torch.cuda.synchronize()
            prep = float(np.median([e[0].elapsed_time(e[1]) * 1e3 for e in ev]))
            attn = float(np.median([e[1].elapsed_time(e[2]) * 1e3 for e in ev]))
            return prep, attn

        def bf16(mid=None):  # the bf16 training path's rotation and forward
            forward_step(E, q, k, v, B, maxL, plan, 1.0 / math.sqrt(d), W.ROPE_BASE, qr, kr,
                         out=o, lse=lse, mid=None if mid is None else (lambda: mid.record(st)))

        def fp8(mid=None):
            E.esm_attn_quantize_fp8_planned(q, k, B, maxL, plan, qs, ks, W.ROPE_BASE, q8=q8,
                                            k8=k8)
            if mid is not None:
                mid.record(st)
            E.esm_attn_fwd_fp8_planned(q8, k8, v, B, maxL, plan, qs, ks, out=o, lse=lse)

        pb, ab = timed(bf16)
        p8, a8 = timed(fp8)
        fwd_f, _ = W.counted_flops(lengths, H, d)
        res[name] = {"bf16": {"rotate_us": round(pb, 1), "fwd_us": round(ab, 1),
                              "fwd_tflops": round(fwd_f / ab * 1e-6, 1)},
                     "fp8": {"quantize_us": round(p8, 1), "fwd_us": round(a8, 1),
                             "fwd_tflops": round(fwd_f / a8 * 1e-6, 1)},
                     "fwd_speedup": round(ab / a8, 3),
                     "with_prep_speedup": round((pb + ab) / (p8 + a8), 3)}
    out = {"metric": "forward TFLOP/s, E4M3 scores vs bf16", "unit": "TFLOP/s",
           "value": res["esm2_650m"]["fp8"]["fwd_tflops"], "n_gpus": 1,
           "higher_is_better": True, "dtype": "fp8 e4m3 (scores) / bf16 (P V)",
           "data": "synthetic (seeded normal bf16 activations)",
           "config": {"workload": "esm2_650m and esm2_15b batches"}, "workloads": res}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library runs the attention hot path on "
              "a single MI355X (no sharding, no collectives); --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.attention_block:
        attention_block(args)
        return
    if args.packing_study:
        packing_study(args)
        return
    if args.split_kv:
        split_kv_study(args)
        return
    if args.fp8:
        fp8_study(args)
        return

    import torch
    from protein_language_model_amd import esm_attn as E
    from protein_language_model_amd import workloads as W

    dev = torch.device("cuda:0")
    seed = W.WORKLOADS[args.workload].seed if args.seed is None else args.seed
    inp = W.make_inputs(args.workload, seed=seed)
    T, H, d, B = inp["T"], inp["H"], inp["d"], len(inp["lengths"])
    maxL = max(inp["lengths"])
    scale, base = inp["scale"], inp["rope_base"]

    def dev_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v, do = (dev_bf16(inp[n]) for n in ("q", "k", "v", "do"))
    cu = torch.from_numpy(inp["cu_seqlens"]).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    qr, kr = torch.empty_like(q), torch.empty_like(k)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    drow = E.drow_buffer(H, T, dev)
    plan = torch.empty(E.esm_attn_plan_bytes(B, T, maxL, H, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    # batches whose sequences all fit one 128-row work item (d <= 64) take the
    # library's small-batch path: the one-shot calls, one launch each way
    small = maxL <= 128 and d <= 64
    names = ["fwd", "bwd"] if small else ["plan", "rotate", "fwd", "bwd_dq", "bwd_dkv"]
    ws_f = torch.empty(E.esm_attn_fwd_workspace_bytes(B, T, maxL, H, d), dtype=torch.uint8,
                       device=dev)
    ws_b = torch.empty(E.esm_attn_bwd_workspace_bytes(B, T, maxL, H, d), dtype=torch.uint8,
                       device=dev)

    def step(ev=None):
        def mark(j):
            if ev is not None:
                ev[j].record(stream)
        mark(0)
        if small:
            E.esm_attn_fwd(q, k, v, cu, maxL, scale, base, out=o, lse=lse, workspace=ws_f)
            mark(1)
            E.esm_attn_bwd(q, k, v, o, do, lse, cu, maxL, scale, base, dq=dq, dk=dk, dv=dv,
                           workspace=ws_b)
            mark(2)
            return
        E.esm_attn_plan(cu, T, maxL, H, d, base, plan=plan)
        mark(1)
        forward_step(E, q, k, v, B, maxL, plan, scale, base, qr, kr, out=o, lse=lse,
                     mid=lambda: mark(2))
        mark(3)
        E.esm_attn_bwd_planned(qr, kr, v, o, do, lse, B, maxL, plan, scale, base, dq=dq,
                               drow=drow, passes=E.PASS_DQ)
        mark(4)
        E.esm_attn_bwd_planned(qr, kr, v, o, do, lse, B, maxL, plan, scale, base, dk=dk, dv=dv,
                               drow=drow, passes=E.PASS_DKV)
        mark(5)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps with nothing recorded between the calls (an event
    # record is a barrier packet: six per step added ~80 us of idle gaps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-step spread: K more steps with one event at each step boundary
    # (K + 1 records), then the same after the clocks have settled
    def step_times(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        evs[0].record(stream)
        for i in range(n):
            step()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        return [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n)]  # us

    spread = step_times(args.steps)
    for _ in range(max(0, SETTLE_STEPS - args.warmup - 2 * args.steps)):
        step()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall_settled = time.perf_counter() - t2

    # instrumented pass, K more steps: events around every call give the
    # per-kernel times (kernels_us) and the dominant kernel's launch time
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall_events = time.perf_counter() - t1

    per = {n: [] for n in names}
    for ev in events:
        for j, n in enumerate(names):
            per[n].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)  # us
    avg = {n: float(np.mean(x)) for n, x in per.items()}
    step_ms = wall / args.steps * 1e3
    nf = 1 if small else 3   # events: forward = plan, rotation, forward; then the backward
    fwd_us = [ev[0].elapsed_time(ev[nf]) * 1e3 for ev in events]
    bwd_us = [ev[nf].elapsed_time(ev[len(names)]) * 1e3 for ev in events]

    # flushed: a 512 MiB write (untimed, outside the events) before each step
    # evicts the 256 MB last-level cache, so every input comes from HBM
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    fl = []
    for i in range(args.steps):
        flush.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        fl.append(e0.elapsed_time(e1) * 1e3)
    del flush

    # the same step captured once in a HIP graph and replayed K times
    graph_ms = None
    try:
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        t3 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t3) / args.steps * 1e3
        del g
    except RuntimeError as exc:   # capture unsupported: reported, not hidden
        graph_ms = "capture failed: %s" % (str(exc).splitlines()[0],)

    fwd_f, bwd_f = W.counted_flops(inp["lengths"], H, d)
    total_f = fwd_f + bwd_f
    # algorithmic HBM bytes of one step: forward reads q, k, v and writes o
    # and the LSE; backward reads q, k, v, o, dO and the LSE and writes dq,
    # dk, dv and D
    alg_bytes = 24 * T * H * d + 12 * T * H
    tflops = total_f / (step_ms * 1e-3) / 1e12
    s2 = float(sum(L * L for L in inp["lengths"]))
    # algorithmic flops of each kernel: the method's matrix products it runs
    kernel_flops = {"fwd": 4 * s2 * H * d,            # S = QK^T, O = PV
                    "bwd_dq": 6 * s2 * H * d,         # S, dP = dO V^T, dQ = dS K
                    "bwd_dkv": 8 * s2 * H * d,        # S, dP, dV = P^T dO, dK = dS^T Q
                    "bwd": 10 * s2 * H * d}           # small path: the five products at once
    dom = max([n for n in names if n in kernel_flops], key=lambda n: avg[n])
    achieved = kernel_flops[dom] / (avg[dom] * 1e-6) / 1e12
    kernel_symbol = {"fwd": "fwd_kernel<%d" % d, "bwd_dq": "bwd_dq_kernel<%d" % d,
                     "bwd_dkv": "bwd_dkv_kernel<%d" % d, "bwd": "bwd_dkv_kernel<%d" % d}[dom]
    traffic = measured_traffic(args.workload, kernel_symbol)

    out = {
        "metric": "attention fwd+bwd TFLOP/s and % of bf16 MFMA peak; tokens/s (varlen)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 activations, packed varlen batch)",
        "config": {"workload": "%s: %d sequences, %d tokens, H=%d, d=%d, RoPE base %g"
                               % (inp["name"], B, T, H, d, base),
                   "path": ("small-batch (one launch forward, one backward)" if small else
                            "planned (plan, rotation, forward, dq pass, dk/dv pass)"),
                   "global_batch": B, "seq_len": maxL, "tokens": T, "seed": seed,
                   "parallelism": "single GPU"},
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "tokens_per_s": round(T / (step_ms * 1e-3), 1),
        "kernels_us": {n: round(x, 2) for n, x in avg.items()},
        "ms_per_step_with_events": round(wall_events / args.steps * 1e3, 4),
        # clock ramp: the timed steps above follow the requested warmup; the
        # chip's clocks settle after about 40 steps of sustained load
        "step_us_spread": dict(pct(spread), first5=round(float(np.mean(spread[:5])), 1),
                               last5=round(float(np.mean(spread[-5:])), 1)),
        "ms_per_step_settled": round(wall_settled / args.steps * 1e3, 4),
        "settled_after_steps": max(SETTLE_STEPS, args.warmup + 2 * args.steps),
        "tflops_settled": round(total_f / (wall_settled / args.steps) / 1e12, 2),
        "fwd_us": pct(fwd_us),
        "bwd_us": pct(bwd_us),
        "kernels_us_pct": {n: pct(x) for n, x in per.items()},
        "flushed": {"step_us": pct(fl),
                    "algorithmic_bytes": alg_bytes,
                    "hbm_gbs_median": round(alg_bytes / (float(np.median(fl)) * 1e-6) / 1e9, 1),
                    "peak_gbs": PEAK_HBM_GBS},
        "graph_replay_ms_per_step": (round(graph_ms, 4) if isinstance(graph_ms, float)
                                     else graph_ms),
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None if traffic is None else round(traffic["bytes"]),
                     "traffic_detail": traffic,
                     "algorithmic_flops": kernel_flops[dom],
                     "avg_launch_us": round(avg[dom], 2)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
