"""Diagnostic mode of the oracle: the stacked model with bfloat16 rounding at
chosen storage points.

TEST INFRASTRUCTURE ONLY.  The acceptance reference is ``gpt_forward`` /
``gpt_backward`` in fp64; this module is never an acceptance reference.  It
computes the same stacked model with the same fp64 arithmetic, except that
the values named in ``points`` are rounded to bfloat16 where an
implementation with 16-bit storage keeps
them in memory between its matrix products.  Running it with different sets
of points separates the error that 16-bit storage alone produces from
everything else, and shows which storage points a 16-bit implementation has
to widen to bring a deep stack within a given tolerance.

A rounded value is produced the way a kernel with fp32 accumulators
stores it: the fp64 value is first rounded to the nearest fp32, then to the
nearest bfloat16 (ties to even at both steps; ``to_bf16_via_f32``).

With ``points`` empty (and ``delta="o"``) every function performs the same
numpy operations in the same order as ``gpt_forward`` / ``gpt_backward`` and
the functions they call, so the results are identical bit for bit (pinned by
a test).  Pages: the model is the stacked transformer of page "5-megatron",
section 训练一般流程 (two LayerNorms per layer, tied input/output embedding)
split as on page "Megtron张量/模型并行" (sections MLP层, Self-Attention层,
输入层Embedding, 输出层Embedding); the bfloat16 format is the one described on
page "5-megatron", section 分布式混合精度训练.

Storage points (names accepted in ``points``):

forward
  ``ln_out``   LayerNorm outputs (the inputs of the QKV and MLP products)
  ``qkv``      the QKV activations of every shard
  ``p_fwd``    the attention probabilities that multiply V
  ``o``        the attention output O of every shard (also read by dW_O
               and, with ``delta="o"``, by the softmax backward)
  ``part_fwd`` the forward shard partials Z_r (attention and MLP)
  ``mlp_pre``  the saved MLP pre-activation (read by GELU' in the backward;
               the forward GELU reads the unrounded product)
  ``mlp_h``    the MLP hidden activation H = GELU(X A)
  ``x_final``  the last residual, rounded before the tied logits and the
               output-side table gradient
  ``logits``   the logits themselves
backward
  ``dx_copy``  the copy of the residual gradient that the matrix products read
  ``part_bwd`` the backward shard partials dX_r (logits, MLP, attention)
  ``dmlp``     dP = (dZ B^T) * GELU'(P), the input of dA and dX of the MLP
  ``do``       dO = dZ W_O^T
  ``p_bwd``    the recomputed probabilities that multiply dO (dV = P^T dO)
  ``p_ds``     the recomputed probabilities that form dS (and, with
               ``delta="p"``, delta)
  ``ds``       dS * scale, the input of dQ and dK
  ``dqkv``     dQ, dK, dV (inputs of dW_QKV and dX)
  ``wgrad``    the weight gradients dW_QKV, dW_O, dA, dB as stored outputs

``delta`` selects how the softmax backward's row term is formed:
  ``"o"``   delta_i = sum_j dO_ij O_ij (the oracle's form, with O as stored);
  ``"o32"`` the same sum with O before the ``o`` rounding (a kernel that
            keeps an fp32 copy of O for this sum);
  ``"p"``   delta_i = sum_j P_ij dP_ij / sum_j P_ij with the P that forms dS,
            which makes every row of dS sum to zero for that P.
``p_fwd_form`` selects which probabilities ``p_fwd`` rounds:
  ``"normalised"``    P = exp(S - max) / l, then O = round(P) V;
  ``"unnormalised"``  E = exp(S - max), O = (round(E) V) / l with l the sum of
                      the unrounded E (a kernel that normalises O once at the
                      end of its pass over the keys).
``ds_center`` (only with ``ds``): dQ is formed as dS_q (K - kbar) + r kbar
with kbar the mean key of the head and r the exact row sums of the rounded
dS_q: the same value in exact arithmetic, but the rounding error of dS_q
no longer reaches dQ through the keys' common component.
"""

from __future__ import annotations

import math

import numpy as np

from .tp_oracle import (_causal_scores, gelu, gelu_grad, layernorm_backward, layernorm_forward, partition,
                        shard_out_weight, shard_qkv_weight, shard_reduce, split_columns,
                        split_rows, vocab_embed_backward, vocab_embed_forward)

POINTS = ("ln_out", "qkv", "p_fwd", "o", "part_fwd", "mlp_pre", "mlp_h", "x_final", "logits",
          "dx_copy", "part_bwd", "dmlp", "do", "p_bwd", "p_ds", "ds", "dqkv", "wgrad")


class Rounding:
    """Which storage points round to bf16, and the softmax-backward options."""

    def __init__(self, points=(), delta="o", ds_center=False, p_fwd_form="normalised"):
        unknown = set(points) - set(POINTS)
        if unknown:
            raise ValueError(f"unknown storage points {sorted(unknown)}")
        if delta not in ("o", "o32", "p"):
            raise ValueError("delta must be 'o', 'o32' or 'p'")
        if p_fwd_form not in ("normalised", "unnormalised"):
            raise ValueError("p_fwd_form must be 'normalised' or 'unnormalised'")
        self.points = frozenset(points)
        self.delta = delta
        self.ds_center = bool(ds_center)
        self.p_fwd_form = p_fwd_form

    def __call__(self, name, x):
        return to_bf16_via_f32(x) if name in self.points else x


def to_bf16_via_f32(x):
    """fp64 -> nearest fp32 -> nearest bfloat16 (ties to even), as fp64.

    bfloat16 keeps the top 16 bits of an fp32 pattern (page "5-megatron",
    section 分布式混合精度训练); rounding to nearest even adds 0x7FFF plus the
    lowest kept bit to the pattern before truncating.  Finite inputs only
    (the emulated model has no infinities or NaNs)."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).copy()
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# One attention head, forward and backward.
# ---------------------------------------------------------------------------

def head_forward(Q, K, V, rnd, causal=True):
    """``attention_head_forward`` with the probabilities that multiply V rounded at ``p_fwd``."""
    S = _causal_scores(Q, K, causal)
    mx = S.max(axis=1, keepdims=True)
    E = np.exp(S - mx)
    l = E.sum(axis=1, keepdims=True)
    if rnd.p_fwd_form == "unnormalised":
        O = (rnd("p_fwd", E) @ V) / l
    else:
        P = E / l
        O = rnd("p_fwd", P) @ V
    lse = (mx + np.log(l))[:, 0]
    return O, lse


def head_backward(Q, K, V, O, dO, lse, rnd, causal=True):
    """``attention_head_backward`` with its storage points.

    O is the forward output the row term reads (stored, or its fp32 copy
    with ``delta="o32"``); lse the forward's log-sum-exp.  When a
    point of the recomputed probabilities is rounded, P is recomputed from
    lse as exp(S - lse) (what a kernel that keeps only lse does); otherwise
    the oracle's own normalisation is used.
    """
    d = Q.shape[1]
    S = _causal_scores(Q, K, causal)
    if "p_bwd" in rnd.points or "p_ds" in rnd.points or rnd.delta == "p":
        P = np.exp(S - lse[:, None])
    else:
        mx = S.max(axis=1, keepdims=True)
        E = np.exp(S - mx)
        P = E / E.sum(axis=1, keepdims=True)
    dV = rnd("p_bwd", P).T @ dO
    dP = dO @ V.T
    Pd = rnd("p_ds", P)
    if rnd.delta in ("o", "o32"):
        delta = (dO * O).sum(axis=1, keepdims=True)
    else:
        den = Pd.sum(axis=1, keepdims=True)
        delta = (Pd * dP).sum(axis=1, keepdims=True) / np.where(den > 0, den, 1.0)
    dS = Pd * (dP - delta)
    if "ds" in rnd.points:
        dSq = to_bf16_via_f32(dS / math.sqrt(d))
        if rnd.ds_center:
            kbar = K.mean(axis=0, keepdims=True)
            Kc = to_bf16_via_f32(K - kbar)
            dQ = dSq @ Kc + dSq.sum(axis=1, keepdims=True) * kbar
        else:
            dQ = dSq @ K
        dK = dSq.T @ Q
    else:
        dQ = dS @ K / math.sqrt(d)
        dK = dS.T @ Q / math.sqrt(d)
    return dQ, dK, dV


# ---------------------------------------------------------------------------
# One shard of each sublayer.
# ---------------------------------------------------------------------------

def attention_shard_forward(X, Wqkv, Wo, b, s, nh, d, rnd, causal=True):
    """``attention_layer_forward`` with ``qkv``, ``p_fwd``, ``o`` and ``part_fwd``.
    Returns QKV, O (as stored), lse, Z and O before the ``o`` rounding."""
    QKV = rnd("qkv", X @ _f64(Wqkv))
    w = nh * d
    O = np.zeros((b * s, w))
    lse = np.zeros((b, nh, s))
    for bi in range(b):
        rows = slice(bi * s, (bi + 1) * s)
        for j in range(nh):
            Q = QKV[rows, j * d:(j + 1) * d]
            K = QKV[rows, w + j * d:w + (j + 1) * d]
            V = QKV[rows, 2 * w + j * d:2 * w + (j + 1) * d]
            O[rows, j * d:(j + 1) * d], lse[bi, j] = head_forward(Q, K, V, rnd, causal)
    O32 = O
    O = rnd("o", O)
    Z = rnd("part_fwd", O @ _f64(Wo))
    return QKV, O, lse, Z, O32


def attention_shard_backward(X, Wqkv, Wo, QKV, O, lse, dZ, b, s, nh, d, rnd, causal=True, O32=None):
    """``attention_layer_backward`` from the stored QKV, O and lse (and, for
    ``delta="o32"``, the unrounded O32)."""
    Od = O32 if rnd.delta == "o32" else O
    w = nh * d
    dWo = rnd("wgrad", O.T @ dZ)
    dO = rnd("do", dZ @ _f64(Wo).T)
    dQKV = np.zeros_like(QKV)
    for bi in range(b):
        rows = slice(bi * s, (bi + 1) * s)
        for j in range(nh):
            cq = slice(j * d, (j + 1) * d)
            ck = slice(w + j * d, w + (j + 1) * d)
            cv = slice(2 * w + j * d, 2 * w + (j + 1) * d)
            dq, dk, dv = head_backward(QKV[rows, cq], QKV[rows, ck], QKV[rows, cv], Od[rows, cq], dO[rows, cq],
                                       lse[bi, j], rnd, causal)
            dQKV[rows, cq], dQKV[rows, ck], dQKV[rows, cv] = dq, dk, dv
    dQKV = rnd("dqkv", dQKV)
    dWqkv = rnd("wgrad", X.T @ dQKV)
    dX = rnd("part_bwd", dQKV @ _f64(Wqkv).T)
    return dX, dWqkv, dWo


def mlp_shard_forward(X, A, B, rnd):
    """``mlp_forward`` with ``mlp_pre`` (saved P), ``mlp_h`` and ``part_fwd``."""
    P = X @ _f64(A)
    H = rnd("mlp_h", gelu(P))
    Z = rnd("part_fwd", H @ _f64(B))
    return rnd("mlp_pre", P), H, Z


def mlp_shard_backward(X, A, B, P, H, dZ, rnd):
    """``mlp_backward`` from the stored P and H."""
    dB = rnd("wgrad", H.T @ dZ)
    dH = dZ @ _f64(B).T
    dP = rnd("dmlp", dH * gelu_grad(P))
    dA = rnd("wgrad", X.T @ dP)
    dX = rnd("part_bwd", dP @ _f64(A).T)
    return dX, dA, dB


# ---------------------------------------------------------------------------
# The stacked model.
# ---------------------------------------------------------------------------

def gpt_forward(ids, E, layers, b, s, nheads, d, n, rnd, eps=1e-5, causal=True):
    """``oracle.gpt_forward`` with storage points.  Weights may be given in
    any float dtype holding the exact values (they are widened per product).
    Returns (logits per shard, cache)."""
    V = E.shape[0]
    parts = []
    for r in range(n):
        st, cnt = partition(V, n, r)
        parts.append(vocab_embed_forward(ids, E[st:st + cnt], st))
    x = shard_reduce(parts)
    cache = {"x_in": [], "ln": [], "attn": [], "mlp": []}
    hs = nheads // n
    for lw in layers:
        cache["x_in"].append(x)
        y1, mu1, rs1 = layernorm_forward(x, _f64(lw["g1"]), _f64(lw["b1"]), eps)
        y1 = rnd("ln_out", y1)
        outs = []
        for r in range(n):
            outs.append(attention_shard_forward(y1, shard_qkv_weight(lw["WQ"], lw["WK"], lw["WV"], n, r, d),
                                                shard_out_weight(lw["WO"], n, r, d), b, s, hs, d, rnd, causal))
        x2 = x + shard_reduce([o[3] for o in outs])
        y2, mu2, rs2 = layernorm_forward(x2, _f64(lw["g2"]), _f64(lw["b2"]), eps)
        y2 = rnd("ln_out", y2)
        mouts = [mlp_shard_forward(y2, split_columns(lw["A"], n, r), split_rows(lw["B"], n, r), rnd)
                 for r in range(n)]
        cache["ln"].append((y1, mu1, rs1, x2, y2, mu2, rs2))
        cache["attn"].append([(o[0], o[1], o[2], o[4] if rnd.delta == "o32" else None) for o in outs])
        cache["mlp"].append([(o[0], o[1]) for o in mouts])
        x = x2 + shard_reduce([o[2] for o in mouts])
    cache["x_out"] = x
    xl = rnd("x_final", x)
    cache["x_logits"] = xl
    logits = []
    for r in range(n):
        st, cnt = partition(V, n, r)
        logits.append(rnd("logits", xl @ _f64(E[st:st + cnt]).T))
    return logits, cache


def gpt_backward_layers(ids, E, layers, cache, dlogits, b, s, nheads, d, n, rnd, causal=True):
    """``oracle.gpt_backward`` with storage points, as a generator: yields
    ``(layer index, gradient dict)`` from the top layer down and finally
    ``("dE", dE_full)``, so a caller can compare and drop each layer's
    gradients before the next is computed."""
    V = E.shape[0]
    xl = cache["x_logits"]
    dE = np.zeros(E.shape, dtype=np.float64)
    dx_parts = []
    for r in range(n):
        st, cnt = partition(V, n, r)
        dL = _f64(dlogits[r])
        dx_parts.append(rnd("part_bwd", dL @ _f64(E[st:st + cnt])))
        dE[st:st + cnt] += dL.T @ xl
    dx = shard_reduce(dx_parts)
    hs = nheads // n
    w = hs * d
    for li in reversed(range(len(layers))):
        lw = layers[li]
        y1, mu1, rs1, x2, y2, mu2, rs2 = cache["ln"][li]
        x_in = cache["x_in"][li]
        dxc = rnd("dx_copy", dx)
        res = []
        for r in range(n):
            P_r, H_r = cache["mlp"][li][r]
            res.append(mlp_shard_backward(y2, split_columns(lw["A"], n, r), split_rows(lw["B"], n, r), P_r, H_r,
                                          dxc, rnd))
        dy2 = shard_reduce([o[0] for o in res])
        dA = np.concatenate([o[1] for o in res], axis=1)
        dB = np.concatenate([o[2] for o in res], axis=0)
        dx2_ln, dg2, db2 = layernorm_backward(x2, _f64(lw["g2"]), mu2, rs2, dy2)
        dx2 = dx + dx2_ln
        dx2c = rnd("dx_copy", dx2)
        ares = []
        for r in range(n):
            QKV, O, lse, O32 = cache["attn"][li][r]
            ares.append(attention_shard_backward(y1, shard_qkv_weight(lw["WQ"], lw["WK"], lw["WV"], n, r, d),
                                                 shard_out_weight(lw["WO"], n, r, d), QKV, O, lse, dx2c,
                                                 b, s, hs, d, rnd, causal, O32))
        dy1 = shard_reduce([o[0] for o in ares])
        dx_in_ln, dg1, db1 = layernorm_backward(x_in, _f64(lw["g1"]), mu1, rs1, dy1)
        dx = dx2 + dx_in_ln
        grads = {"WQ": np.concatenate([o[1][:, 0:w] for o in ares], axis=1),
                 "WK": np.concatenate([o[1][:, w:2 * w] for o in ares], axis=1),
                 "WV": np.concatenate([o[1][:, 2 * w:3 * w] for o in ares], axis=1),
                 "WO": np.concatenate([o[2] for o in ares], axis=0), "A": dA, "B": dB,
                 "g1": dg1, "b1": db1, "g2": dg2, "b2": db2}
        yield li, grads
        # the layer's saved activations are no longer needed
        cache["attn"][li] = cache["mlp"][li] = None
    for r in range(n):
        st, cnt = partition(V, n, r)
        dE[st:st + cnt] += vocab_embed_backward(ids, dx, st, cnt)
    yield "dE", dE


def gpt_backward(ids, E, layers, cache, dlogits, b, s, nheads, d, n, rnd, causal=True):
    """All gradients at once: (dE_full, per-layer gradient dicts)."""
    grads = [None] * len(layers)
    dE = None
    for key, val in gpt_backward_layers(ids, E, layers, cache, dlogits, b, s, nheads, d, n, rnd, causal):
        if key == "dE":
            dE = val
        else:
            grads[key] = val
    return dE, grads
