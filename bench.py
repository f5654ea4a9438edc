"""Benchmark of the tensor-parallel shard path on one MI355X.

Step = one forward+backward pass of the 12-layer GPT at the page-1 model
shape (H=4096, 8 heads of 512, 4H MLP, 2 LayerNorms per layer, tied vocab
50257) on b=1 x s=2048 tokens, split over N=2 tensor-parallel shards that
all execute on this GPU: the vocab-parallel embedding gather and its shard
sum, per layer the LayerNorms, both shards' attention and MLP sublayers and
the shard sums standing in for the 'g'/'f' all-reduces, the tied logits,
and the whole backward pass including the tied table gradient (output side
plus input side).  Inputs are seeded synthetic tensors resident in HBM;
the logits' upstream gradient is drawn N(0,1).

Prints one JSON line.  `value` = algorithmic TFLOP/s of the step (33.45
TFLOP: GEMMs 2MNK, causal attention s(s+1)/2 score pairs, backward = 2x
forward).  Also reported: the roofline of the dominant kernel instance
(the GEMM template instance with the largest total kernel time in a traced
step; its launches are timed with events on their own stream during the
timed steps), every GEMM shape's rate and the attention + MLP kernel-time
headline from one traced step, the single-layer step on its own, the
vocab-parallel embedding kernels' HBM GB/s at T = 8*2048 tokens, and the
fp64 CPU oracle timed on a bounded sample of the same workload.
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
            r["ws_attn"] = emp((max(tp.tp_attn_fwd_workspace(bf, b, s, h, hs, d),
                                    tp.tp_attn_bwd_workspace(bf, b, s, h, hs, d)),), torch.uint8)
            self.sh.append(r)
        self.Za, self.Zm, self.dXa, self.dXm = emp((M, h)), emp((M, h)), emp((M, h)), emp((M, h))
        self.hs, self.w, self.f = hs, w, f

    def step(self):
        tp, sh = self.tp, self.sh
        b, s, hs, d = self.b, self.s, self.hs, self.d
        for r in sh:
            tp.tp_attn_fwd(self.X, r["Wqkv"], r["Wo"], r["QKV"], r["O"], r["lse"], r["Za"], b, s, hs, d, True,
                           ws=r["ws_attn"])
        tp.shard_reduce([r["Za"] for r in sh], self.Za)
        for r in sh:
            tp.tp_mlp_fwd(self.X, r["A"], r["B"], r["P"], r["H"], r["Zm"])
        tp.shard_reduce([r["Zm"] for r in sh], self.Zm)
        for r in sh:
            tp.tp_mlp_bwd(self.X, r["A"], r["B"], r["P"], r["H"], self.dZm, r["dXm"], r["dA"], r["dB"], r["ws_mlp"])
        tp.shard_reduce([r["dXm"] for r in sh], self.dXm)
        for r in sh:
            tp.tp_attn_bwd(self.X, r["Wqkv"], r["Wo"], r["QKV"], r["O"], r["lse"], self.dZa, r["dXa"], r["dWqkv"],
                           r["dWo"], r["ws_attn"], b, s, hs, d, True)
        tp.shard_reduce([r["dXa"] for r in sh], self.dXa)


def gpt_model(tp, torch, seed=5):
    """The 12-layer model with seeded N(0,0.02) weights, gamma=1, beta=0,
    uniform tokens and dL ~ N(0,1), all generated on the GPU."""
    from megatron_tensor_transformer_columnparallel_amd.gpt import GPTShape, TPGPT
    c = GPTShape()
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 * seed)
    bf = torch.bfloat16

    def rnd(shape, std):
        return (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * std).to(bf)

    E = rnd((c.V, c.H), 0.02)
    layers = []
    for _ in range(c.L):
        layers.append({"WQ": rnd((c.H, c.heads * c.d), 0.02), "WK": rnd((c.H, c.heads * c.d), 0.02),
                       "WV": rnd((c.H, c.heads * c.d), 0.02), "WO": rnd((c.heads * c.d, c.H), 0.02),
                       "A": rnd((c.H, c.f), 0.02), "B": rnd((c.f, c.H), 0.02),
                       "g1": torch.ones(c.H, device="cuda"), "b1": torch.zeros(c.H, device="cuda"),
                       "g2": torch.ones(c.H, device="cuda"), "b2": torch.zeros(c.H, device="cuda")})
    model = TPGPT(c, E, layers)
    ids = torch.randint(0, c.V, (c.M,), generator=g, device="cuda", dtype=torch.int32)
    dl = []
    for r in range(c.n):
        buf = torch.zeros((c.M, model.ldl[r]), dtype=bf, device="cuda")
        buf[:, :model.vr[r][1]] = rnd((c.M, model.vr[r][1]), 1.0)
        dl.append(buf[:, :model.vr[r][1]])
    return c, model, ids, dl


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


def ce_bench(tp, torch, reps=20):
    """HBM rates of the vocab-parallel cross entropy on one shard of the tied
    logits: T = 8*2048 tokens, shard 0 of V = 50257 (25129 rows, row stride
    25136), bf16 logits ~ N(0, 2^2).  Three buffer sets (2.5 GB each way) are
    rotated so that the 256 MB last-level cache cannot serve the repeats."""
    T, V, ldl = 8 * 2048, 50257, 25136
    start, rows = tp.tps_partition(V, 2, 0)
    g = torch.Generator(device="cuda")
    g.manual_seed(4100)
    targets = torch.randint(0, V, (T,), generator=g, device="cuda", dtype=torch.int32)
    sets = []
    for _ in range(3):
        L = torch.zeros((T, ldl), dtype=torch.bfloat16, device="cuda")
        L[:, :rows] = (torch.randn((T, rows), generator=g, device="cuda") * 2).to(torch.bfloat16)
        dL = torch.empty((T, ldl), dtype=torch.bfloat16, device="cuda")
        st = torch.empty((T, 4), dtype=torch.float32, device="cuda")
        st1 = torch.empty((T, 4), dtype=torch.float32, device="cuda")
        sets.append((L, dL, st, st1))
    loss = torch.empty(T, device="cuda")
    lse = torch.empty(T, device="cuda")
    dloss = torch.full((T,), 1.0 / T, device="cuda")
    for L, _, st, st1 in sets:   # a second shard's statistics for the exchange (the same logits)
        tp.vocab_ce_stats(L[:, :rows], targets, st1, start + rows)
    # algorithmic bytes (every element the method must read or write once)
    lbytes = T * rows * 2
    res = {}
    for name, fn, nbytes in [
        ("vocab_ce_stats", lambda s: tp.vocab_ce_stats(s[0][:, :rows], targets, s[2], start), lbytes + 4 * T + 16 * T),
        ("vocab_ce_combine", lambda s: tp.vocab_ce_combine([s[2], s[3]], loss, lse), 2 * 16 * T + 8 * T),
        ("vocab_ce_bwd", lambda s: tp.vocab_ce_bwd(s[0][:, :rows], targets, lse, dloss, s[1][:, :rows], start),
         2 * lbytes + 12 * T),
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
    res["shape"] = {"T": T, "V": V, "shard_rows": rows, "ldl": ldl, "dtype": "bf16"}
    return res


def full_embedding_bench(tp, torch, reps=20):
    """HBM rates of the full input embedding at T = 8*2048 tokens, H = 4096,
    2 shards, 2048 positions, dropout p = 0.1, fp32 output (the residual
    stream): the fused shard sum + position rows + dropout, and the dropout
    backward on an fp32 gradient.  Three buffer sets rotated."""
    T, H, P, n, p = 8 * 2048, 4096, 2048, 2, 0.1
    g = torch.Generator(device="cuda")
    g.manual_seed(4400)
    pos = (torch.arange(T, device="cuda", dtype=torch.int32) % P).contiguous()
    PE = (torch.randn((P, H), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    sets = []
    for _ in range(3):
        parts = [torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16) for _ in range(n)]
        out = torch.empty((T, H), device="cuda")
        dout = torch.randn((T, H), generator=g, device="cuda")
        dx = torch.empty((T, H), device="cuda")
        sets.append((parts, out, dout, dx))
    res = {}
    for name, fn, nbytes in [
        ("embedding_fwd (2 bf16 shard partials + position rows + dropout -> fp32)",
         lambda s: tp.embedding_fwd(s[0], PE, pos, s[1], p=p, seed=11), n * T * H * 2 + P * H * 2 + 4 * T + T * H * 4),
        ("dropout_apply (fp32 gradient)", lambda s: tp.dropout_apply(s[2], s[3], p, 11), 2 * T * H * 4),
    ]:
        for st in sets:
            fn(st)
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
    res["shape"] = {"T": T, "H": H, "positions": P, "shards": n, "p": p}
    return res


def sp_bench(tp, torch, reps=20):
    """HBM rates of the sequence-parallel exchanges at T = 8*2048 tokens,
    H = 4096, 2 shards: the reduce-scatter of two bf16 partials onto the fp32
    residual rows of each shard, and the all-gather of two bf16 row slices.
    Three buffer sets rotated past the last-level cache."""
    T, H, n = 8 * 2048, 4096, 2
    g = torch.Generator(device="cuda")
    g.manual_seed(4300)
    rows = [tp.tps_partition(T, n, r)[1] for r in range(n)]
    sets = []
    for _ in range(3):
        parts = [torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16) for _ in range(n)]
        res = [torch.randn((c, H), generator=g, device="cuda") for c in rows]
        outs = [torch.empty((c, H), device="cuda") for c in rows]
        sl = [torch.randn((c, H), generator=g, device="cuda").to(torch.bfloat16) for c in rows]
        full = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        sets.append((parts, res, outs, sl, full))
    res_ = {}
    for name, fn, nbytes in [
        ("shard_reduce_scatter (2 bf16 partials + fp32 residual -> fp32)",
         lambda s: tp.shard_reduce_scatter(s[0], s[2], res=s[1]), n * T * H * 2 + 2 * T * H * 4),
        ("shard_all_gather (2 bf16 slices)", lambda s: tp.shard_all_gather(s[3], s[4]), 2 * T * H * 2),
    ]:
        for st in sets:
            fn(st)
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
        res_[name] = {"us": round(ms * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                      "bytes": nbytes}
    res_["shape"] = {"T": T, "H": H, "shards": n}
    return res_


def linear_bench(tp, torch, reps=10):
    """The two linear layers on their own at the layer's MLP shard shape
    (M = 2048 tokens, h = 4096, 4h split over 2 shards = 8192 columns each),
    bf16 with biases: TFLOP/s of each call (GEMM FLOPs 2MNK; the bias and
    bias-gradient work is counted in the time, not in the FLOPs)."""
    M, h, n = 2048, 4096, 8192
    g = torch.Generator(device="cuda")
    g.manual_seed(4200)
    bf = torch.bfloat16
    r = lambda *sh: (torch.randn(sh, generator=g, device="cuda") * 0.02).to(bf)
    X, A, b, dY = r(M, h), r(h, n), r(n), r(M, n)
    Y, dX, dA = torch.empty((M, n), dtype=bf, device="cuda"), torch.empty((M, h), dtype=bf, device="cuda"), \
        torch.empty((h, n), dtype=bf, device="cuda")
    db = torch.empty(n, device="cuda")
    B, c, dZ = r(n, h), r(h), r(M, h)
    Z0, Z1, Z = (torch.empty((M, h), dtype=bf, device="cuda") for _ in range(3))
    dB, dH = torch.empty((n, h), dtype=bf, device="cuda"), torch.empty((M, n), dtype=bf, device="cuda")
    dc = torch.empty(h, device="cuda")
    gf = 2 * M * h * n
    res = {}
    for name, fn, flops in [
        ("column_linear_fwd", lambda: tp.column_linear_fwd(X, A, Y, b_r=b), gf),
        ("column_linear_bwd", lambda: tp.column_linear_bwd(X, A, dY, dX, dA, db_r=db), 2 * gf),
        ("row_linear_fwd + shard_reduce_bias (2 shards)",
         lambda: (tp.row_linear_fwd(Y, B, Z0), tp.row_linear_fwd(Y, B, Z1), tp.shard_reduce_bias([Z0, Z1], c, Z)),
         2 * gf),
        ("row_linear_bwd", lambda: tp.row_linear_bwd(Y, B, dZ, dH, dB, db=dc), 2 * gf),
    ]:
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[len(ev) // 2]
        tf = flops / (ms * 1e-3) / 1e12
        res[name] = {"us": round(ms * 1e3, 1), "TFLOP/s": round(tf, 1),
                     "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    res["shape"] = {"M": M, "h": h, "n_per_shard": n, "dtype": "bf16", "bias": True}
    return res


def cpu_baseline():
    """The fp64 oracle on a bounded sample of the step: one shard of one
    layer's MLP sublayer forward and backward at the full shape (M=2048,
    h=4096, f_i=8192), i.e. six 2048x4096x8192 products plus GELU: 824.6
    GFLOP algorithmic (the whole step is 33.45 TFLOP)."""
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
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": "one shard's MLP fwd+bwd at the layer shape (2048x4096 @ 4096x8192, GELU), fp64 numpy, "
                      f"{flops / 1e9:.1f} GFLOP in {t:.2f} s", "seconds": round(t, 2)}


# ------------------------------------------------------------------ launch traces

ATTN_MLP_APIS = ("tp_mlp_fwd", "tp_mlp_bwd", "tp_attn_fwd", "tp_attn_bwd")


def parse_launch(name):
    """'api:kernel[ <targs> MxNxK zB[ causal]]' -> (api, kernel, targs, (M, N, K, B) or None, causal)."""
    api, rest = name.split(":", 1)
    parts = rest.split(" ")
    kernel = parts[0]
    targs, shape, causal = "", None, False
    if len(parts) >= 3 and "x" in parts[2]:
        targs = parts[1]
        M, N, K = (int(v) for v in parts[2].split("x"))
        B = int(parts[3][1:]) if len(parts) > 3 and parts[3].startswith("z") else 1
        shape = (M, N, K, B)
        causal = "causal" in parts[4:]
    return api, kernel, targs, shape, causal


def launch_flops(shape, causal):
    """Algorithmic FLOPs of one GEMM launch: 2MNK per problem; a causal
    attention product (scores s x s, or a K-loop over s keys) counts only the
    s(s+1)/2 (query, key) pairs."""
    M, N, K, B = shape
    if not causal:
        return 2 * M * N * K * B
    s = M
    other = N if K == M else K
    return B * 2 * other * (s * (s + 1) // 2)


def instance_of(name):
    """The kernel template instance of a launch (what a kernel profiler groups by)."""
    api, kernel, targs, _, _ = parse_launch(name)
    return kernel + targs


def trace_one_step(tp, torch, step):
    """Every library launch of one step, timed with events on its own stream."""
    tp.trace_start("", 1 << 16)
    step()
    torch.cuda.synchronize()
    tp.trace_stop()
    recs = tp.trace_records()
    tp.trace_clear()
    return recs


def step_breakdown(recs, layer_flops_total):
    """Per-instance totals, per-GEMM-shape rates and the attention+MLP
    kernel-time headline from one traced step."""
    by_inst, by_shape = {}, {}
    attn_mlp_ms = 0.0
    total_ms = 0.0
    for name, ms in recs:
        api, kernel, targs, shape, causal = parse_launch(name)
        total_ms += ms
        inst = kernel + targs
        e = by_inst.setdefault(inst, [0, 0.0])
        e[0] += 1
        e[1] += ms
        if api in ATTN_MLP_APIS:
            attn_mlp_ms += ms
        if shape is not None:
            key = f"{api} {kernel}{targs} {shape[0]}x{shape[1]}x{shape[2]}" + (f" z{shape[3]}" if shape[3] > 1 else "") \
                + (" causal" if causal else "")
            e2 = by_shape.setdefault(key, [0, 0.0, launch_flops(shape, causal)])
            e2[0] += 1
            e2[1] += ms
    shapes = {}
    for key, (n, ms, fl) in sorted(by_shape.items(), key=lambda kv: -kv[1][1]):
        avg = ms / n
        tf = fl / (avg * 1e-3) / 1e12
        shapes[key] = {"launches": n, "avg_us": round(avg * 1e3, 2), "TFLOP/s": round(tf, 1),
                       "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    top = sorted(by_inst.items(), key=lambda kv: -kv[1][1])
    top_gemm = next(k for k, _ in top if "<" in k)
    # attention core per call (one shard): every launch of tp_attn_* except
    # the four dense projections (QKV, output, and their backward products)
    core = {}
    for name, ms in recs:
        api, kernel, targs, shape, causal = parse_launch(name)
        if api in ("tp_attn_fwd", "tp_attn_bwd") and (shape is None or causal):
            e = core.setdefault(api, {}).setdefault(kernel + targs + ("" if shape is None else " causal x%d" % shape[3]),
                                                   [0, 0.0])
            e[0] += 1
            e[1] += ms
    headline = layer_flops_total / (attn_mlp_ms * 1e-3) / 1e12
    return {
        "kernel_ms_per_step": round(total_ms, 3),
        "top_instances": [{"instance": k, "launches": n, "ms": round(ms, 3), "share": round(ms / total_ms, 4)}
                          for k, (n, ms) in top[:12]],
        "attention_core_us_per_call": {api: {k: round(ms / n * 1e3, 2) for k, (n, ms) in d.items()}
                                       for api, d in core.items()},
        "gemm_shapes": shapes,
        "attn_mlp_kernel_time": {
            "TFLOP/s": round(headline, 1), "frac_of_bf16_peak": round(headline / PEAK_BF16_TFLOPS, 4),
            "kernel_ms": round(attn_mlp_ms, 3), "tflop": round(layer_flops_total / 1e12, 3),
            "what": "sum of algorithmic FLOPs of every tp_mlp_* and tp_attn_* call of the step / sum of the "
                    "kernel times of their launches"},
    }, top_gemm


def profile_traffic(instance):
    """HBM bytes per launch of `instance` from the committed counter summary
    (two rocprofv3 --pmc passes, FETCH_SIZE and WRITE_SIZE, scaled by what
    the same counters read for a plain copy), or None when the summary was
    taken on another version of the GEMM source or another instance."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemm_top_instance_traffic.md")
    src = os.path.join(ROOT, "megatron_tensor_transformer_columnparallel_amd", "csrc", "gemm.hpp")
    try:
        text = open(path, encoding="utf-8").read()
    except OSError:
        return None
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    for line in text.splitlines():
        if line.startswith("traffic-record:"):
            rec = json.loads(line.split(":", 1)[1])
            if rec.get("gemm_sha") == sha and rec.get("instance") == instance:
                return int(rec["bytes_per_launch"])
    return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


ATTN_CORE_SHAPES = [(1, 2048, 8, 128), (1, 2048, 4, 256), (2, 2048, 16, 64), (1, 8192, 2, 128), (1, 2048, 4, 512)]


def attn_core_sweep(tp, torch, reps=5):
    """Per-kernel times (library tracer, mean over `reps` calls after one
    untimed call) of one attention shard's forward and backward at
    ATTN_CORE_SHAPES (batch, sequence, heads of the shard, head dim; causal),
    and the attention-core rates: the forward counted as 4 d FLOP per causal
    (query, key) pair and head, the backward as twice that."""
    rows = []
    for b, sq, hs, d in ATTN_CORE_SHAPES:
        h = max(512, hs * d)
        M, w = b * sq, hs * d
        g = torch.Generator(device="cuda").manual_seed(1)
        X = torch.randn((M, h), device="cuda", generator=g).to(torch.bfloat16)
        Wqkv = (0.02 * torch.randn((h, 3 * w), device="cuda", generator=g)).to(torch.bfloat16)
        Wo = (0.02 * torch.randn((w, h), device="cuda", generator=g)).to(torch.bfloat16)
        dZ = torch.randn((M, h), device="cuda", generator=g).to(torch.bfloat16)
        QKV = torch.empty((M, 3 * w), device="cuda", dtype=torch.bfloat16)
        O = torch.empty((M, w), device="cuda", dtype=torch.bfloat16)
        lse = torch.empty((b * hs * sq,), device="cuda", dtype=torch.float32)
        Z = torch.empty((M, h), device="cuda", dtype=torch.bfloat16)
        gX, gW, gWo = torch.empty_like(X), torch.empty_like(Wqkv), torch.empty_like(Wo)
        wsf = torch.empty((tp.tp_attn_fwd_workspace(torch.bfloat16, b, sq, h, hs, d),), device="cuda",
                          dtype=torch.uint8)
        wsb = torch.empty((tp.tp_attn_bwd_workspace(torch.bfloat16, b, sq, h, hs, d),), device="cuda",
                          dtype=torch.uint8)
        for it in range(reps + 1):
            if it == 1:
                tp.trace_clear()
                tp.trace_start("", 1 << 16)
            tp.tp_attn_fwd(X, Wqkv, Wo, QKV, O, lse, Z, b, sq, hs, d, True, ws=wsf)
            tp.tp_attn_bwd(X, Wqkv, Wo, QKV, O, lse, dZ, gX, gW, gWo, wsb, b, sq, hs, d, True)
        torch.cuda.synchronize()
        tp.trace_stop()
        per = {}
        for name, ms in tp.trace_records():
            per[name] = per.get(name, 0.0) + ms * 1e3 / reps
        tp.trace_clear()
        # the attention core: everything but the four projection GEMMs
        # (QKV and O products, and their weight and input gradients: z1)
        core = {"fwd": 0.0, "bwd": 0.0}
        for name, us in per.items():
            if "gemm_bf16_kernel" in name and name.endswith(" z1"):
                continue
            core["fwd" if name.startswith("tp_attn_fwd") else "bwd"] += us
        fl = 4 * d * b * hs * sq * (sq + 1) // 2
        rows.append({"shape": {"b": b, "s": sq, "heads": hs, "d": d},
                     "workspace_mib": {"fwd": round(wsf.numel() / 2**20, 1), "bwd": round(wsb.numel() / 2**20, 1)},
                     "kernels_us": {k: round(v, 2) for k, v in per.items()},
                     "core_fwd_us": round(core["fwd"], 1), "core_fwd_tflops": round(fl / core["fwd"] / 1e6, 1),
                     "core_bwd_us": round(core["bwd"], 1), "core_bwd_tflops": round(2 * fl / core["bwd"] / 1e6, 1)})
        del X, Wqkv, Wo, dZ, QKV, O, lse, Z, gX, gW, gWo, wsf, wsb
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-embed", action="store_true", help="skip the embedding-kernel rates")
    ap.add_argument("--no-layer", action="store_true", help="skip the single-layer step")
    ap.add_argument("--no-ce", action="store_true", help="skip the cross-entropy kernel rates")
    ap.add_argument("--no-linear", action="store_true", help="skip the standalone linear-layer rates")
    ap.add_argument("--no-sp", action="store_true", help="skip the sequence-parallel exchange rates")
    ap.add_argument("--no-full-embed", action="store_true", help="skip the full-embedding and dropout rates")
    ap.add_argument("--calib", action="store_true", help="one 512 MiB copy first (counter calibration)")
    ap.add_argument("--attn-cores", action="store_true",
                    help="only time the attention cores at a few shapes (one JSON line per shape, no metric)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs every tensor-parallel shard on ONE GPU "
                                   "(the shard sums are local kernels); --gpus must be 1"}))
        sys.exit(2)

    import torch

    import megatron_tensor_transformer_columnparallel_amd as tp

    torch.cuda.set_device(0)
    if args.attn_cores:
        for row in attn_core_sweep(tp, torch):
            print(json.dumps(row), flush=True)
        return
    c, model, ids, dl = gpt_model(tp, torch)
    flops = c.flops()

    if args.calib:
        # plain copy of known size for the counter calibration: 256 Mi bf16 elements in, same out
        src = torch.ones(256 << 20, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        tp.shard_reduce([src], dst)
        torch.cuda.synchronize()
        del src, dst

    def step():
        model.forward(ids)
        model.backward(ids, dl)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # one traced step (untimed): per-launch kernel times -> the dominant
    # kernel instance, the per-shape GEMM rates and the kernel-time headline
    lflops = c.L * layer_flops(c.b, c.s, c.H, c.heads, c.d, c.f, c.n)
    breakdown, top_inst = step_breakdown(trace_one_step(tp, torch, step), lflops)
    # timed region: exactly `steps` steps; the dominant instance's launches
    # are bracketed by events on their own stream (the library's tracer)
    tp.trace_start(":" + top_inst.replace("<", " <", 1), 1 << 16)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    tp.trace_stop()
    roof_recs = tp.trace_records()
    tp.trace_clear()
    ms = t0.elapsed_time(t1) / args.steps
    value = flops / (ms * 1e-3) / 1e12

    fl = [launch_flops(parse_launch(n)[3], parse_launch(n)[4]) for n, _ in roof_recs]
    launch_ms = sum(m for _, m in roof_recs) / len(roof_recs)
    per_launch_flops = sum(fl) / len(fl)
    achieved = per_launch_flops / (launch_ms * 1e-3) / 1e12
    roofline = {"kernel": top_inst, "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": profile_traffic(top_inst), "avg_launch_us": round(launch_ms * 1e3, 2),
                "flops_per_launch": int(per_launch_flops), "launches_timed": len(roof_recs),
                "shapes": sorted({parse_launch(n)[0] + " " + "x".join(map(str, parse_launch(n)[3][:3]))
                                  for n, _ in roof_recs})}

    out = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "gpt12-tp2-bf16: 12 layers, H=4096, 8 heads of 512, 4H MLP, pre-LN, tied vocab "
                                  "50257 (25129/25128 per shard), b=1, s=2048, TP N=2 shards on one GPU, fwd+bwd",
                      "global_batch": 1, "seq_len": 2048, "parallelism": "tp2-emulated-on-1-gpu"},
           "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
           "gflop_per_step": round(flops / 1e9, 1), "wall_s_timed": round(wall, 3),
           "roofline": roofline, "step_kernels": breakdown}
    del model
    torch.cuda.empty_cache()
    if not args.no_layer:
        L = Layer(tp, torch)
        for _ in range(3):
            L.step()
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(10):
            L.step()
        a1.record()
        torch.cuda.synchronize()
        lms = a0.elapsed_time(a1) / 10
        lfl = layer_flops(1, 2048, 4096, 8, 512, 16384, 2)
        out["layer"] = {"workload": "one layer (attention + MLP sublayers), both shards, fwd+bwd, shard sums",
                        "ms": round(lms, 3), "TFLOP/s": round(lfl / (lms * 1e-3) / 1e12, 1),
                        "frac_of_bf16_peak": round(lfl / (lms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del L
        torch.cuda.empty_cache()
    if not args.no_embed:
        out["embed"] = embed_bench(tp, torch)
        torch.cuda.empty_cache()
    if not args.no_ce:
        out["cross_entropy"] = ce_bench(tp, torch)
        torch.cuda.empty_cache()
    if not args.no_linear:
        out["linear"] = linear_bench(tp, torch)
        torch.cuda.empty_cache()
    if not args.no_sp:
        out["sequence_parallel"] = sp_bench(tp, torch)
        torch.cuda.empty_cache()
    if not args.no_full_embed:
        out["full_embedding"] = full_embedding_bench(tp, torch)
        torch.cuda.empty_cache()
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
