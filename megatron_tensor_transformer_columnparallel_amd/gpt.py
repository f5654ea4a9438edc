"""A stacked GPT with every tensor-parallel shard executed on one GPU.

Sequencing only: every arithmetic step is a C-ABI call into libtpshard
(embedding gather, LayerNorm, attention and MLP shards, shard sums, tied
logits and their backward passes).  The residual stream (and its gradient)
is kept in fp32; each sublayer reads a bf16 LayerNorm output and returns
bf16 shard partials, and shard_reduce_add folds the 'g' all-reduce and the
residual add into one fp32 sum.  (A bf16 residual stream accumulates about
1e-2 relative error over 12 layers against the exact result; fp32 keeps the
stacked model within the bf16 tolerance.)

Structure (page "5-megatron", sections ParallelTransformerLayer /
ParallelTransformer: attention then MLP per layer; section 训练一般流程: two
LayerNorms per layer and a tied input/output embedding; page
"Megtron张量/模型并行", section 输出层Embedding: the table's gradient is the sum
of both uses).  Pre-LN sublayers, no biases, no position embedding, no final
LayerNorm: the readings that match the page's parameter count.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as tp


@dataclass
class GPTShape:
    L: int = 12
    b: int = 1
    s: int = 2048
    H: int = 4096
    heads: int = 8
    d: int = 512
    f: int = 16384
    V: int = 50257
    n: int = 2
    eps: float = 1e-5

    @property
    def M(self):
        return self.b * self.s

    def flops(self) -> int:
        """Algorithmic FLOPs of one forward+backward step (GEMMs 2MNK, causal
        attention s(s+1)/2 pairs, backward = 2x forward; LayerNorm, softmax and
        elementwise work not counted)."""
        M, H = self.M, self.H
        layer = (2 * M * H * 3 * H + 4 * self.d * (self.s * (self.s + 1) // 2) * self.heads * self.b
                 + 2 * M * H * H + 2 * 2 * M * H * self.f)
        logits = 2 * M * H * self.V
        return 3 * (self.L * layer + logits)


def _emp(shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device="cuda")


class TPGPT:
    """Parameters, activations and gradients of all shards of the model.

    Parameters are given per layer as full (unsharded) tensors in math
    layout; the constructor slices each shard's block once (page
    "5-megatron", _initialize_affine_weight_cpu: full master weight, then a
    per-rank slice).
    """

    def __init__(self, shape: GPTShape, E, layers):
        c = shape
        assert c.heads % c.n == 0 and c.f % c.n == 0
        self.c = c
        self.hs = c.heads // c.n
        self.w = self.hs * c.d
        self.fi = c.f // c.n
        self.vr = [tp.tps_partition(c.V, c.n, r) for r in range(c.n)]
        self.E = [E[s:s + n].contiguous() for s, n in self.vr]
        self.layers = []
        for lw in layers:
            sh = []
            for r in range(c.n):
                q = slice(r * self.w, (r + 1) * self.w)
                fs = slice(r * self.fi, (r + 1) * self.fi)
                sh.append({
                    "Wqkv": torch.cat([lw["WQ"][:, q], lw["WK"][:, q], lw["WV"][:, q]], dim=1).contiguous(),
                    "Wo": lw["WO"][q, :].contiguous(),
                    "A": lw["A"][:, fs].contiguous(),
                    "B": lw["B"][fs, :].contiguous(),
                })
            self.layers.append({"sh": sh, "g1": lw["g1"], "b1": lw["b1"], "g2": lw["g2"], "b2": lw["b2"]})
        M, H = c.M, c.H
        f32 = torch.float32
        # activations (residual stream x0, x2, x3 in fp32)
        self.x0 = _emp((M, H), f32)
        self.emb_parts = [_emp((M, H)) for _ in range(c.n)]
        self.acts = []
        for _ in range(c.L):
            a = {"y1": _emp((M, H)), "m1": _emp((M,), f32), "r1": _emp((M,), f32),
                 "x2": _emp((M, H), f32), "y2": _emp((M, H)), "m2": _emp((M,), f32),
                 "r2": _emp((M,), f32), "x3": _emp((M, H), f32), "sh": []}
            for _ in range(c.n):
                a["sh"].append({"QKV": _emp((M, 3 * self.w)), "O": _emp((M, self.w)),
                                "lse": _emp((c.b * self.hs * c.s,), torch.float32), "Za": _emp((M, H)),
                                "P": _emp((M, self.fi)), "H": _emp((M, self.fi)), "Zm": _emp((M, H))})
            self.acts.append(a)
        self.x_bf = _emp((M, H))            # bf16 copy of the final residual (tied logits input)
        self.ldl = [(n + 7) // 8 * 8 for _, n in self.vr]
        self.logits = [_emp((M, ld)) for ld in self.ldl]
        # gradients
        self.dE = [torch.empty((n, H), dtype=torch.float32, device="cuda") for _, n in self.vr]
        self.grads = []
        for lw in self.layers:
            self.grads.append({"sh": [{k: torch.empty_like(v) for k, v in s.items()} for s in lw["sh"]],
                               "g1": torch.empty_like(lw["g1"]), "b1": torch.empty_like(lw["b1"]),
                               "g2": torch.empty_like(lw["g2"]), "b2": torch.empty_like(lw["b2"])})
        self.dx, self.dx2 = _emp((M, H), f32), _emp((M, H), f32)          # residual gradient (fp32)
        self.dx_bf, self.dx2_bf = _emp((M, H)), _emp((M, H))               # its bf16 copies (GEMM inputs)
        self.dy = _emp((M, H), f32)
        self.dparts = [_emp((M, H)) for _ in range(c.n)]
        self.ws_mlp = _emp((tp.tp_mlp_bwd_workspace(torch.bfloat16, M, H, self.fi),), torch.uint8)
        # one scratch buffer serves the attention forward and backward calls
        self.ws_attn = _emp((max(tp.tp_attn_fwd_workspace(torch.bfloat16, c.b, c.s, H, self.hs, c.d),
                                 tp.tp_attn_bwd_workspace(torch.bfloat16, c.b, c.s, H, self.hs, c.d)),), torch.uint8)
        self.ws_ln = _emp((tp.layernorm_bwd_workspace(M, H),), torch.uint8)
        self.ws_emb = _emp((tp.vocab_embed_bwd_workspace(M, max(n for _, n in self.vr)),), torch.uint8)
        # vocab-parallel cross entropy: per-shard statistics, per-token loss and log-sum-exp
        self.ce_stats = [_emp((M, 4), f32) for _ in range(c.n)]
        self.ce_loss, self.ce_lse = _emp((M,), f32), _emp((M,), f32)
        self.ce_dloss = torch.full((M,), 1.0 / M, dtype=f32, device="cuda")   # gradient of the mean loss

    def logits_view(self, r):
        return self.logits[r][:, :self.vr[r][1]]

    def forward(self, ids):
        c = self
        cf = self.c
        for r, (s, _) in enumerate(self.vr):
            tp.vocab_embed_fwd(ids, self.E[r], self.emb_parts[r], s)
        tp.shard_reduce(self.emb_parts, self.x0)                                   # g (embedding)
        x = self.x0
        for lw, a in zip(self.layers, self.acts):
            tp.layernorm_fwd(x, lw["g1"], lw["b1"], a["y1"], a["m1"], a["r1"], cf.eps)
            for p, sa in zip(lw["sh"], a["sh"]):
                tp.tp_attn_fwd(a["y1"], p["Wqkv"], p["Wo"], sa["QKV"], sa["O"], sa["lse"], sa["Za"],
                               cf.b, cf.s, c.hs, cf.d, True, ws=self.ws_attn)
            tp.shard_reduce_add(x, [sa["Za"] for sa in a["sh"]], a["x2"])           # residual + g
            tp.layernorm_fwd(a["x2"], lw["g2"], lw["b2"], a["y2"], a["m2"], a["r2"], cf.eps)
            for p, sa in zip(lw["sh"], a["sh"]):
                tp.tp_mlp_fwd(a["y2"], p["A"], p["B"], sa["P"], sa["H"], sa["Zm"])
            tp.shard_reduce_add(a["x2"], [sa["Zm"] for sa in a["sh"]], a["x3"])      # residual + g
            x = a["x3"]
        self.x_out = x
        tp.shard_reduce([x], self.x_bf)                                            # round to bf16
        for r in range(cf.n):
            tp.tied_logits(self.x_bf, self.E[r], self.logits_view(r))

    def loss(self, targets, dloss=None):
        """Vocab-parallel cross entropy of the logits of the last forward
        against ``targets`` [M] int32 (page "5-megatron", section
        _VocabParallelCrossEntropy): each shard's statistics, the exchange over
        shards, then each shard's logits are overwritten in place with their
        gradient for ``dloss`` [M] fp32 (default 1/M per token, the gradient of
        the mean loss).  Returns the per-token loss [M] and the per-shard
        logit gradients to pass to ``backward``."""
        cf = self.c
        for r, (s, _) in enumerate(self.vr):
            tp.vocab_ce_stats(self.logits_view(r), targets, self.ce_stats[r], s)
        tp.vocab_ce_combine(self.ce_stats, self.ce_loss, self.ce_lse)
        dl = self.ce_dloss if dloss is None else dloss
        for r, (s, _) in enumerate(self.vr):
            tp.vocab_ce_bwd(self.logits_view(r), targets, self.ce_lse, dl, self.logits_view(r), s)
        return self.ce_loss, [self.logits_view(r) for r in range(cf.n)]

    def backward(self, ids, dlogits):
        """dlogits[r]: [M x v_r] (row stride a multiple of 8) gradient of shard r's logits."""
        cf = self.c
        for r in range(cf.n):
            tp.tied_logits_bwd(self.x_bf, self.E[r], dlogits[r], self.dparts[r], self.dE[r])
        if cf.n > 1:
            tp.shard_reduce_add(self.dparts[0], self.dparts[1:], self.dx, self.dx_bf)   # f backward
        else:
            tp.shard_reduce(self.dparts, self.dx)
            tp.shard_reduce(self.dparts, self.dx_bf)
        for li in reversed(range(cf.L)):
            lw, a, g = self.layers[li], self.acts[li], self.grads[li]
            x_in = self.x0 if li == 0 else self.acts[li - 1]["x3"]
            for p, sa, gs, dp in zip(lw["sh"], a["sh"], g["sh"], self.dparts):
                tp.tp_mlp_bwd(a["y2"], p["A"], p["B"], sa["P"], sa["H"], self.dx_bf, dp, gs["A"], gs["B"],
                              self.ws_mlp)
            tp.shard_reduce(self.dparts, self.dy)                                    # f backward
            tp.layernorm_bwd_residual(a["x2"], lw["g2"], a["m2"], a["r2"], self.dy, self.dx, self.dx2,
                                      g["g2"], g["b2"], self.ws_ln, out_copy=self.dx2_bf)   # + residual
            for p, sa, gs, dp in zip(lw["sh"], a["sh"], g["sh"], self.dparts):
                tp.tp_attn_bwd(a["y1"], p["Wqkv"], p["Wo"], sa["QKV"], sa["O"], sa["lse"], self.dx2_bf, dp,
                               gs["Wqkv"], gs["Wo"], self.ws_attn, cf.b, cf.s, self.hs, cf.d, True)
            tp.shard_reduce(self.dparts, self.dy)                                    # f backward
            tp.layernorm_bwd_residual(x_in, lw["g1"], a["m1"], a["r1"], self.dy, self.dx2, self.dx,
                                      g["g1"], g["b1"], self.ws_ln, out_copy=self.dx_bf)    # + residual
        for r, (s, _) in enumerate(self.vr):
            tp.vocab_embed_bwd(ids, self.dx, self.dE[r], s, self.ws_emb)            # tied: adds input side
