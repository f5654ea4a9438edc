"""Benchmark of the tensor-parallel shard path on one MI355X.

Step = one pass over one transformer layer at the page-1 model shape
(b=1, s=2048, H=4096, 8 heads of 512, 4H MLP) split over N=2 tensor-parallel
shards, all executed on this GPU: for each shard the attention sublayer
(QKV column GEMM, causal flash attention, row GEMM) and the MLP sublayer
(column GEMM + GELU, row GEMM) forward and backward, plus the four
shard_reduce calls that stand in for the 'g' forward and 'f' backward
all-reduces.  Inputs are seeded synthetic tensors resident in HBM.

Prints one JSON line.  `value` = algorithmic TFLOP/s of the step (2577.0
GFLOP: GEMMs 2MNK, causal attention s(s+1)/2 score pairs, backward = 2x
forward).  Also reported: the roofline of the dominant kernel (the MFMA GEMM
of the MLP shard forward), the vocab-parallel embedding kernels' HBM GB/s at
the tied-embedding shape (V=50257, H=4096, T=16384), and the fp64 CPU oracle
timed on a bounded sample of the same layer.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TP-shard layer fwd+bwd TFLOP/s (% bf16 MFMA peak); embed GB/s (% HBM)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def layer_flops(b, s, h, heads, d, f_total, n):
    """Algorithmic FLOPs of one layer fwd+bwd over all n shards."""
    M = b * s
    hs = heads // n
    w = hs * d
    f = f_total // n
    fwd = (2 * M * h * 3 * w                    # QKV
           + 4 * d * (s * (s + 1) // 2) * hs * b  # causal QK^T and PV
           + 2 * M * w * h                      # output projection
           + 2 * 2 * M * h * f)                 # MLP A and B
    return 3 * fwd * n


class Layer:
    """Device buffers of all shards of one layer (bf16, seeded synthetic)."""

    def __init__(self, tp, torch, b=1, s=2048, h=4096, heads=8, d=512, f_total=16384, n=2, seed=3):
        self.tp, self.torch = tp, torch
        self.b, self.s, self.h, self.heads, self.d, self.n = b, s, h, heads, d, n
        M = b * s
        hs = heads // n
        w = hs * d
        f = f_total // n
        g = torch.Generator(device="cuda")
        g.manual_seed(1000 * seed)
        bf = torch.bfloat16

        def rnd(shape, std):
            return (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * std).to(bf)

        def emp(shape, dt=bf):
            return torch.empty(shape, dtype=dt, device="cuda")

        self.X = rnd((M, h), 1.0)
        self.dZa = rnd((M, h), 1.0)
        self.dZm = rnd((M, h), 1.0)
        self.sh = []
        for _ in range(n):
            r = {}
            r["Wqkv"], r["Wo"] = rnd((h, 3 * w), 0.02), rnd((w, h), 0.02)
            r["A"], r["B"] = rnd((h, f), 0.02), rnd((f, h), 0.02)
            r["QKV"], r["O"], r["lse"], r["Za"] = emp((M, 3 * w)), emp((M, w)), emp((b * hs * s,), torch.float32), emp((M, h))
            r["P"], r["H"], r["Zm"] = emp((M, f)), emp((M, f)), emp((M, h))
            r["dXa"], r["dWqkv"], r["dWo"] = emp((M, h)), emp((h, 3 * w)), emp((w, h))
            r["dXm"], r["dA"], r["dB"] = emp((M, h)), emp((h, f)), emp((f, h))
            r["ws_mlp"] = emp((tp.tp_mlp_bwd_workspace(bf, M, h, f),), torch.uint8)
            r["ws_attn"] = emp((tp.tp_attn_bwd_workspace(bf, b, s, h, hs, d),), torch.uint8)
            self.sh.append(r)
        self.Za, self.Zm, self.dXa, self.dXm = emp((M, h)), emp((M, h)), emp((M, h)), emp((M, h))
        self.hs, self.w, self.f = hs, w, f
        self.mlp_events = []

    def step(self, record=False):
        tp, sh = self.tp, self.sh
        b, s, hs, d = self.b, self.s, self.hs, self.d
        for r in sh:
            tp.tp_attn_fwd(self.X, r["Wqkv"], r["Wo"], r["QKV"], r["O"], r["lse"], r["Za"], b, s, hs, d, True)
        tp.shard_reduce([r["Za"] for r in sh], self.Za)
        for r in sh:
            if record:
                e0 = self.torch.cuda.Event(enable_timing=True)
                e1 = self.torch.cuda.Event(enable_timing=True)
                e0.record()
            tp.tp_mlp_fwd(self.X, r["A"], r["B"], r["P"], r["H"], r["Zm"])
            if record:
                e1.record()
                self.mlp_events.append((e0, e1))
        tp.shard_reduce([r["Zm"] for r in sh], self.Zm)
        for r in sh:
            tp.tp_mlp_bwd(self.X, r["A"], r["B"], r["P"], r["H"], self.dZm, r["dXm"], r["dA"], r["dB"], r["ws_mlp"])
        tp.shard_reduce([r["dXm"] for r in sh], self.dXm)
        for r in sh:
            tp.tp_attn_bwd(self.X, r["Wqkv"], r["Wo"], r["QKV"], r["O"], r["lse"], self.dZa, r["dXa"], r["dWqkv"],
                           r["dWo"], r["ws_attn"], b, s, hs, d, True)
        tp.shard_reduce([r["dXa"] for r in sh], self.dXa)


def embed_bench(tp, torch, reps=20):
    """HBM rates of the embedding gather, the shard sum and the input-side
    scatter-add at T = 8*2048 tokens, V = 50257 split 25129/25128, H = 4096.
    Three buffer sets are rotated so that the 256 MB last-level cache cannot
    serve the repeats."""
    T, V, H, n = 8 * 2048, 50257, 4096, 2
    g = torch.Generator(device="cuda")
    g.manual_seed(4000)
    bf = torch.bfloat16
    ids = torch.randint(0, V, (T,), generator=g, device="cuda", dtype=torch.int32)
    start, rows = tp.tps_partition(V, n, 0)
    sets = []
    for _ in range(3):
        E = (torch.randn((rows, H), generator=g, device="cuda") * 0.02).to(bf)
        Y0 = torch.empty((T, H), dtype=bf, device="cuda")
        Y1 = torch.empty((T, H), dtype=bf, device="cuda")
        Ys = torch.empty((T, H), dtype=bf, device="cuda")
        dY = torch.randn((T, H), generator=g, device="cuda").to(bf)
        dE = torch.zeros((rows, H), dtype=torch.float32, device="cuda")
        sets.append((E, Y0, Y1, Ys, dY, dE))
    ws = torch.empty((tp.vocab_embed_bwd_workspace(T, rows),), dtype=torch.uint8, device="cuda")
    # algorithmic bytes (every element the method must read or write once)
    local = ids.long() - start
    inr = (local >= 0) & (local < rows)
    c_r = int(inr.sum())
    u_r = int(torch.unique(local[inr]).numel())
    bytes_fwd = 4 * T + c_r * H * 2 + T * H * 2
    bytes_red = 3 * T * H * 2
    bytes_bwd = 4 * T + c_r * H * 2 + 2 * u_r * H * 4
    res = {}
    for name, fn, nbytes in [
        ("vocab_embed_fwd", lambda s: tp.vocab_embed_fwd(ids, s[0], s[1], start), bytes_fwd),
        ("shard_reduce", lambda s: tp.shard_reduce([s[1], s[2]], s[3]), bytes_red),
        ("vocab_embed_bwd", lambda s: tp.vocab_embed_bwd(ids, s[4], s[5], start, ws), bytes_bwd),
    ]:
        for s in sets:
            fn(s)
        torch.cuda.synchronize()
        ev = []
        for i in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn(sets[i % 3])
            e1.record()
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[len(ev) // 2]
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"us": round(ms * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                     "bytes": nbytes}
    res["shape"] = {"T": T, "V": V, "H": H, "shard_rows": rows, "in_range_ids": c_r, "touched_rows": u_r}
    return res


def cpu_baseline(budget_s=30.0):
    """The fp64 oracle on a bounded sample: one shard's MLP sublayer forward
    and backward at the full layer shape (M=2048, h=4096, f_i=8192), i.e. six
    2048x4096x8192 products plus GELU: 824.6 GFLOP algorithmic."""
    import numpy as np

    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=os.cpu_count())
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    M, h, f = 2048, 4096, 8192
    inp = synth.mlp_inputs(3, M, h, f, "bf16", base=40)
    X, A, B, dZ = inp["X"].f64, inp["A"].f64, inp["B"].f64, inp["dZ"].f64
    t0 = time.perf_counter()
    P, _, _ = O.mlp_forward(X, A, B)
    O.mlp_backward(X, A, B, P, dZ)
    t = time.perf_counter() - t0
    flops = 6 * 2 * M * h * f
    return {"value": round(flops / t / 1e12, 4), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": "one shard's MLP fwd+bwd at the layer shape (2048x4096 @ 4096x8192, GELU), fp64 numpy, "
                      f"{flops / 1e9:.1f} GFLOP in {t:.2f} s", "seconds": round(t, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-embed", action="store_true", help="skip the embedding kernels")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs the whole tensor-parallel layer on ONE GPU "
                                   "(every shard executed locally); --gpus must be 1"}))
        sys.exit(2)

    import torch

    import megatron_tensor_transformer_columnparallel_amd as tp

    torch.cuda.set_device(0)
    L = Layer(tp, torch)
    flops = layer_flops(1, 2048, 4096, 8, 512, 16384, 2)
    for _ in range(args.warmup):
        L.step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(args.steps):
        L.step(record=True)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / args.steps
    value = flops / (ms * 1e-3) / 1e12

    # dominant kernel: the two MFMA GEMM launches of tp_mlp_fwd (2*M*h*f_i FLOPs each)
    mlp_ms = sorted(a.elapsed_time(b) for a, b in L.mlp_events)
    mlp_ms = sum(mlp_ms) / len(mlp_ms)
    per_launch_flops = 2 * 2048 * 4096 * 8192
    achieved = per_launch_flops / (mlp_ms / 2 * 1e-3) / 1e12
    roofline = {"kernel": "gemm_bf16_kernel<256,256,64,2,2> (tp_mlp_fwd: X*A_i+GELU and H_i*B_i, 2048x8192x4096)",
                "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "avg_launch_us": round(mlp_ms / 2 * 1e3, 2), "flops_per_launch": per_launch_flops}

    out = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "gpt-layer-shard-bf16: b=1 s=2048 H=4096 heads=8 d=512 4H=16384 TP N=2 "
                                  "(attention+MLP fwd+bwd, both shards, shard_reduce)",
                      "global_batch": 1, "seq_len": 2048, "parallelism": "tp2-emulated-on-1-gpu"},
           "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
           "gflop_per_step": round(flops / 1e9, 1), "wall_s_timed": round(wall, 3),
           "roofline": roofline}
    if not args.no_embed:
        out["embed"] = embed_bench(tp, torch)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
