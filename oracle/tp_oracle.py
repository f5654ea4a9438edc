"""fp64 reference definitions of every step on the tensor-parallel shard path.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product never
imports this module.

Conventions
-----------
* All arrays are numpy float64 (token ids: integer arrays).  Callers upcast
  bf16/fp32 inputs exactly before calling; nothing here rounds except
  ``round_to_bf16`` / ``round_to_f32``, which exist only so that tests can
  compare bit patterns after the same final rounding.
* Weights use the mathematical layout of page "Megtron张量/模型并行"
  (section 切分权重): ``X`` is (tokens, h) and ``W`` is (h, h'), so a linear
  layer is ``X @ W``.  (Page "5-megatron" stores torch's transposed
  ``(out, in)`` layout; the product is the same.)
* "Shard r of N" always means the contiguous block given by ``partition``.
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

__all__ = [
    "partition", "split_columns", "split_rows",
    "gelu", "gelu_grad",
    "mlp_forward", "mlp_backward", "tp_mlp_forward", "tp_mlp_backward",
    "attention_head_forward", "attention_head_backward",
    "attention_layer_forward", "attention_layer_backward",
    "shard_qkv_weight", "shard_out_weight",
    "tp_attention_forward", "tp_attention_backward",
    "shard_reduce",
    "vocab_embed_forward", "vocab_embed_mask", "vocab_embed_backward",
    "tied_logits", "tied_logits_backward",
    "vocab_ce_forward", "vocab_ce_backward",
    "column_linear_forward", "column_linear_backward", "row_linear_forward", "row_linear_backward",
    "sp_reduce_scatter", "sp_all_gather", "sp_layernorm_param_grads",
    "philox4x32_10", "dropout_keep", "dropout_keep_at", "embedding_forward", "embedding_backward",
    "layernorm_forward", "layernorm_backward",
    "param_count", "param_count_tied_unique",
    "round_to_bf16", "round_to_f32", "bf16_next_up",
    "gpt_forward", "gpt_backward",
]

# Which independent pin covers each function (tests/test_oracle_*.py).
PINS = {
    "partition": "worked examples V=10 -> [0,5)/[5,10) and V=300 -> [0,150)/[150,300)",
    "gelu": "closed forms gelu(0)=0, gelu(x)-gelu(-x)=x, normal-CDF quantile 0.975",
    "gelu_grad": "central finite differences of gelu; gelu'(0)=1/2",
    "mlp_forward": "scalar-loop brute force on tiny inputs; shard sum = unsharded",
    "mlp_backward": "central finite differences of a scalar loss",
    "attention_head_forward": "closed forms (s=1, Q=0 running mean, row 0) + scalar-loop brute force",
    "attention_head_backward": "central finite differences",
    "attention_layer_forward": "head permutation invariance; shard sum = unsharded",
    "attention_layer_backward": "central finite differences",
    "shard_reduce": "exactness on integers; brute-force nearest-bf16 rounding of N=2 sums",
    "vocab_embed_forward": "worked examples [0,212,7,9] (V=300,N=2) and [2,7,1,5]/[0,3)",
    "vocab_embed_backward": "scalar-loop brute force; column-sum identity; finite differences",
    "tied_logits_backward": "finite differences through both uses of the table",
    "vocab_ce_forward": "page's 10-word two-shard masking layout; uniform logits give log V; "
                        "per-row shift invariance; library logsumexp; scalar-loop brute force",
    "vocab_ce_backward": "central finite differences of the loss; rows sum to zero; "
                         "closed form 1/V - onehot for uniform logits",
    "column_linear_forward": "scalar-loop brute force of X A + b; gathered shards = unsharded; "
                             "skip_bias_add leaves X A",
    "column_linear_backward": "central finite differences (dX summed over shards, dA, db)",
    "row_linear_forward": "scalar-loop brute force; scattered and parallel inputs agree; "
                          "bias added once after the sum",
    "row_linear_backward": "central finite differences; gathered dX_r = unsharded dX",
    "sp_reduce_scatter": "scalar-loop brute force; all_gather(reduce_scatter) = the all-reduce",
    "sp_all_gather": "inverse of the row split; composition with reduce_scatter",
    "sp_layernorm_param_grads": "summed shard gradients = the unsharded LayerNorm's; finite differences",
    "philox4x32_10": "the generator's published known-answer vectors (tests/golden/philox4x32_10_kat.json)",
    "dropout_keep": "p = 0 keeps all; kept fraction within 5 sigma of 1 - p; word/element mapping by brute force",
    "dropout_keep_at": "indices past 2^34 (a nonzero high counter word) against direct generator calls; sampled rows of the embedding equal the full call's",
    "embedding_forward": "p = 0 equals the scalar sum of the rows; out-of-range ids add zero rows",
    "embedding_backward": "central finite differences at a fixed mask",
    "layernorm_forward": "mean 0 / variance 1 invariants and scalar-loop brute force",
    "layernorm_backward": "central finite differences",
    "param_count": "page value 2,827,821,056 for H=4096, L=12, V=50257",
    "round_to_bf16": "brute-force nearest search over all finite bf16 values; eps = 2^-7",
    "gpt_forward": "composition of pinned pieces; finite differences of gpt_backward",
    "gpt_backward": "central finite differences on a tiny model",
}


# ---------------------------------------------------------------------------
# Partition of a dimension over N shards.
# ---------------------------------------------------------------------------

def partition(total: int, n: int, r: int) -> tuple[int, int]:
    """Return ``(start, count)`` of shard ``r`` when ``total`` rows are split
    into ``n`` contiguous shards.

    Page "5-megatron", section VocabParallelEmbedding: each rank keeps the
    vocabulary range [start, end) (the comment's example gives [0,5) and
    [5,10) for a 10-word vocabulary on two ranks).  Page "Megtron张量/模型并行",
    section 输入层Embedding: 300 words on two GPUs are split at 150.  The
    helper's body is not printed; the reading taken here is the plainest even
    split, with the first ``total mod n`` shards holding one extra row.
    """
    if n <= 0 or not (0 <= r < n) or total < 0:
        raise ValueError("bad partition arguments")
    q, rem = divmod(total, n)
    start = r * q + min(r, rem)
    count = q + (1 if r < rem else 0)
    return start, count


def split_columns(W: np.ndarray, n: int, r: int) -> np.ndarray:
    """Column shard r of W (page "Megtron张量/模型并行", section 按列切分权重)."""
    s, c = partition(W.shape[1], n, r)
    return W[:, s:s + c]


def split_rows(W: np.ndarray, n: int, r: int) -> np.ndarray:
    """Row shard r of W (page "Megtron张量/模型并行", section 按行切分权重)."""
    s, c = partition(W.shape[0], n, r)
    return W[s:s + c, :]


# ---------------------------------------------------------------------------
# GELU (exact erf form).
# ---------------------------------------------------------------------------

def gelu(x: np.ndarray) -> np.ndarray:
    """GELU(x) = x * Phi(x), Phi the standard normal CDF written with erf.

    Page "Megtron张量/模型并行", section MLP层 names GELU as the non-linearity
    between A and B; its formula is an image that did not survive, so the
    exact-erf form is taken.
    """
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def gelu_grad(x: np.ndarray) -> np.ndarray:
    """d/dx GELU(x) = Phi(x) + x * phi(x), phi the standard normal density."""
    return 0.5 * (1.0 + erf(x / math.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


# ---------------------------------------------------------------------------
# MLP: Z = GELU(X A) B, A column-parallel, B row-parallel.
# ---------------------------------------------------------------------------

def mlp_forward(X, A, B):
    """Unsharded (or one shard's) MLP forward.

    Page "Megtron张量/模型并行", section MLP层: Z = GELU(X A) B.  Applied to
    a column shard A_r and the matching row shard B_r it yields shard r's
    partial Z_r; the partials sum to Z (the 'g' all-reduce).
    Returns (P, H, Z) with P = X A the pre-activation and H = GELU(P).
    """
    P = X @ A
    H = gelu(P)
    Z = H @ B
    return P, H, Z


def mlp_backward(X, A, B, P, dZ):
    """Backward of ``mlp_forward`` for an upstream gradient dZ.

    The 'g' operator's backward is the identity (page "5-megatron", section
    RowParallelLinear, _ReduceFromModelParallelRegion), so every shard sees
    the full dZ.  The 'f' operator's backward sums the shards' dX
    (section ColumnParallelLinear, _CopyToModelParallelRegion).
    Returns (dX, dA, dB); for a shard, dX is that shard's partial.
    """
    H = gelu(P)
    dB = H.T @ dZ
    dH = dZ @ B.T
    dP = dH * gelu_grad(P)
    dA = X.T @ dP
    dX = dP @ A.T
    return dX, dA, dB


def tp_mlp_forward(X, A, B, n):
    """Run all n shards; return (per-shard list of (P_r, H_r, Z_r), sum of Z_r)."""
    outs = [mlp_forward(X, split_columns(A, n, r), split_rows(B, n, r)) for r in range(n)]
    return outs, shard_reduce([o[2] for o in outs])


def tp_mlp_backward(X, A, B, dZ, n):
    """Per-shard backward; return (list of (dX_r, dA_r, dB_r), sum of dX_r)."""
    res = []
    for r in range(n):
        A_r, B_r = split_columns(A, n, r), split_rows(B, n, r)
        P_r = X @ A_r
        res.append(mlp_backward(X, A_r, B_r, P_r, dZ))
    return res, shard_reduce([o[0] for o in res])


# ---------------------------------------------------------------------------
# Attention split by heads.
# ---------------------------------------------------------------------------

def _causal_scores(Q, K, causal):
    d = Q.shape[1]
    S = (Q @ K.T) / math.sqrt(d)
    if causal:
        sq, sk = S.shape
        S = np.where(np.arange(sk)[None, :] > np.arange(sq)[:, None], -np.inf, S)
    return S


def attention_head_forward(Q, K, V, causal=True):
    """One head of scaled dot-product attention.

    Page "Megtron张量/模型并行", section Self-Attention层: every head has its
    own W^Q, W^K, W^V of width k_dim/heads and is computed independently;
    the per-head formula is a lost figure, so the plainest decoder reading is
    taken: S = Q K^T / sqrt(d), keys after the query masked out when causal,
    P = row softmax(S), O = P V.  Also returns lse = log(sum_j exp(S_ij))
    per query row (the normaliser a backward pass needs).
    """
    S = _causal_scores(Q, K, causal)
    mx = S.max(axis=1, keepdims=True)
    E = np.exp(S - mx)
    l = E.sum(axis=1, keepdims=True)
    P = E / l
    O = P @ V
    lse = (mx + np.log(l))[:, 0]
    return O, lse


def attention_head_backward(Q, K, V, O, dO, causal=True):
    """Gradients (dQ, dK, dV) of one head for upstream dO."""
    d = Q.shape[1]
    S = _causal_scores(Q, K, causal)
    mx = S.max(axis=1, keepdims=True)
    E = np.exp(S - mx)
    P = E / E.sum(axis=1, keepdims=True)
    dV = P.T @ dO
    dP = dO @ V.T
    delta = (dO * O).sum(axis=1, keepdims=True)
    dS = P * (dP - delta)
    dQ = dS @ K / math.sqrt(d)
    dK = dS.T @ Q / math.sqrt(d)
    return dQ, dK, dV


def attention_layer_forward(X, Wqkv, Wo, b, s, nh, d, causal=True):
    """Attention sublayer (or one shard of it) in the fused-QKV layout.

    ``Wqkv`` is (h, 3*nh*d) = [W_Q | W_K | W_V], head j at columns j*d..(j+1)*d
    inside each block; ``Wo`` is (nh*d, h).  Tokens are batch-major
    (row = batch*s + position).  Page "Megtron张量/模型并行", section
    Self-Attention层 (Q/K/V column-split by heads, output linear row-split);
    page "5-megatron", section ParallelSelfAttention (QKV outputs are not
    reduced, the output linear's result is).
    Returns (QKV, O, lse, Z) with lse of shape (b, nh, s).
    """
    QKV = X @ Wqkv
    w = nh * d
    O = np.zeros((b * s, w))
    lse = np.zeros((b, nh, s))
    for bi in range(b):
        rows = slice(bi * s, (bi + 1) * s)
        for j in range(nh):
            Q = QKV[rows, j * d:(j + 1) * d]
            K = QKV[rows, w + j * d:w + (j + 1) * d]
            V = QKV[rows, 2 * w + j * d:2 * w + (j + 1) * d]
            O[rows, j * d:(j + 1) * d], lse[bi, j] = attention_head_forward(Q, K, V, causal)
    Z = O @ Wo
    return QKV, O, lse, Z


def attention_layer_backward(X, Wqkv, Wo, QKV, O, dZ, b, s, nh, d, causal=True):
    """Backward of ``attention_layer_forward``: returns (dX, dWqkv, dWo)."""
    w = nh * d
    dWo = O.T @ dZ
    dO = dZ @ Wo.T
    dQKV = np.zeros_like(QKV)
    for bi in range(b):
        rows = slice(bi * s, (bi + 1) * s)
        for j in range(nh):
            cq = slice(j * d, (j + 1) * d)
            ck = slice(w + j * d, w + (j + 1) * d)
            cv = slice(2 * w + j * d, 2 * w + (j + 1) * d)
            dq, dk, dv = attention_head_backward(QKV[rows, cq], QKV[rows, ck], QKV[rows, cv],
                                                 O[rows, cq], dO[rows, cq], causal)
            dQKV[rows, cq], dQKV[rows, ck], dQKV[rows, cv] = dq, dk, dv
    dWqkv = X.T @ dQKV
    dX = dQKV @ Wqkv.T
    return dX, dWqkv, dWo


def shard_qkv_weight(WQ, WK, WV, n, r, d):
    """Shard r's fused [W_Q | W_K | W_V] holding its contiguous block of heads.

    Page "Megtron张量/模型并行", section Self-Attention层: the three matrices
    are column-split by head and several heads may share one GPU; the head
    count must divide evenly (checked here).
    """
    nh = WQ.shape[1] // d
    if nh % n:
        raise ValueError("heads must divide the shard count")
    hs0, hsn = partition(nh, n, r)
    c = slice(hs0 * d, (hs0 + hsn) * d)
    return np.concatenate([WQ[:, c], WK[:, c], WV[:, c]], axis=1)


def shard_out_weight(WO, n, r, d):
    """Shard r's row block of the output projection (heads of shard r)."""
    nh = WO.shape[0] // d
    hs0, hsn = partition(nh, n, r)
    return WO[hs0 * d:(hs0 + hsn) * d, :]


def tp_attention_forward(X, WQ, WK, WV, WO, b, s, nheads, d, n, causal=True):
    """All n shards of the attention sublayer; returns (per-shard outputs, sum of Z_r)."""
    hs = nheads // n
    outs = []
    for r in range(n):
        outs.append(attention_layer_forward(X, shard_qkv_weight(WQ, WK, WV, n, r, d),
                                            shard_out_weight(WO, n, r, d), b, s, hs, d, causal))
    return outs, shard_reduce([o[3] for o in outs])


def tp_attention_backward(X, WQ, WK, WV, WO, dZ, b, s, nheads, d, n, causal=True):
    hs = nheads // n
    res = []
    for r in range(n):
        Wqkv_r = shard_qkv_weight(WQ, WK, WV, n, r, d)
        Wo_r = shard_out_weight(WO, n, r, d)
        QKV, O, _, _ = attention_layer_forward(X, Wqkv_r, Wo_r, b, s, hs, d, causal)
        res.append(attention_layer_backward(X, Wqkv_r, Wo_r, QKV, O, dZ, b, s, hs, d, causal))
    return res, shard_reduce([o[0] for o in res])


# ---------------------------------------------------------------------------
# 'g' forward / 'f' backward: the shard-partial sum.
# ---------------------------------------------------------------------------

def shard_reduce(parts):
    """Sum of the N shard partials, exact in fp64, shard order 0..N-1.

    Page "5-megatron", sections ColumnParallelLinear and RowParallelLinear:
    _ReduceFromModelParallelRegion all-reduces (sums) in forward and
    _CopyToModelParallelRegion all-reduces the gradient in backward.  On one
    device the all-reduce's arithmetic is this sum.
    """
    out = np.zeros_like(np.asarray(parts[0], dtype=np.float64))
    for p in parts:
        out = out + np.asarray(p, dtype=np.float64)
    return out


# ---------------------------------------------------------------------------
# Vocab-parallel embedding and the tied output projection.
# ---------------------------------------------------------------------------

def vocab_embed_mask(ids, start, rows):
    """(out_of_range_mask, masked_local_index) for shard [start, start+rows).

    Page "5-megatron", section VocabParallelEmbedding, forward: the mask is
    (id < start) | (id >= end); the local index is id - start with masked
    entries set to 0 (the page's example: ids [2,7,1,5] on range [0,3)
    give [2,0,1,0]).
    """
    ids = np.asarray(ids, dtype=np.int64)
    mask = (ids < start) | (ids >= start + rows)
    local = ids - start
    local[mask] = 0
    return mask, local


def vocab_embed_forward(ids, E_r, start):
    """Shard r's embedding partial: row E_r[id - start] if in range, else 0.

    Page "5-megatron", section VocabParallelEmbedding (F.embedding on the
    masked index, then masked rows set to 0); page "Megtron张量/模型并行",
    section 输入层Embedding (tokens a GPU cannot find give all-zero vectors;
    the shard results are then summed).
    """
    mask, local = vocab_embed_mask(ids, start, E_r.shape[0])
    Y = E_r[local].astype(np.float64, copy=True)
    Y[mask, :] = 0.0
    return Y


def vocab_embed_backward(ids, dY, start, rows):
    """Input-side gradient of shard r's table: dE_r[j] = sum of dY[t] over the
    tokens t with id_t = start + j, in token order.

    Implicit in page "5-megatron", section VocabParallelEmbedding: the
    gradient of F.embedding scatters dY into the looked-up rows, and the rows
    zeroed by the mask pass no gradient (so local row 0 receives nothing from
    out-of-range tokens).
    """
    mask, local = vocab_embed_mask(ids, start, rows)
    dE = np.zeros((rows, dY.shape[1]))
    keep = ~mask
    np.add.at(dE, local[keep], np.asarray(dY, dtype=np.float64)[keep])
    return dE


def tied_logits(X, E_r):
    """Shard r's logits L_r = X E_r^T (the input word embedding reused as the
    output projection).  Page "Megtron张量/模型并行", section 输出层Embedding;
    page "5-megatron", section _VocabParallelCrossEntropy (X * WE^T)."""
    return X @ E_r.T


def tied_logits_backward(X, E_r, dL_r):
    """Output-side gradients of ``tied_logits``: (dX_r partial, dE_r).

    Page "Megtron张量/模型并行", section 输出层Embedding: the table receives
    one gradient at the output layer and one at the input layer and must be
    updated with their sum; the total is ``dE_r + vocab_embed_backward(...)``.
    """
    return dL_r @ E_r, dL_r.T @ X


# ---------------------------------------------------------------------------
# The full input embedding (page "5-megatron", section Embedding): the
# vocab-parallel word embedding summed over shards, plus the position
# embedding, plus the token-type embedding when used, then dropout.  The
# dropout sits after the shard sum, where every shard holds the same values,
# so it draws the same mask on every shard (page "5-megatron", section 模型并行:
# seeds differ inside tensor-parallel regions and agree after the
# all-reduce).  Its random numbers come from the counter-based generator
# Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
# easy as 1, 2, 3", SC 2011), keyed by a 64-bit seed and counted by element.
# ---------------------------------------------------------------------------

_PHILOX_M = (np.uint64(0xD2511F53), np.uint64(0xCD9E8D57))
_PHILOX_W = (np.uint64(0x9E3779B9), np.uint64(0xBB67AE85))
_U32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds.  ``ctr``: array [..., 4] of uint32 words,
    ``key``: two uint32 words.  Each round multiplies words 0 and 2 by the
    two round multipliers into 64-bit products, and the new counter is
    (hi(w2*M1) ^ c1 ^ k0, lo(w2*M1), hi(w0*M0) ^ c3 ^ k1, lo(w0*M0)); the key
    then advances by the two Weyl constants.  Returns [..., 4] uint32."""
    c = np.asarray(ctr, dtype=np.uint64) & _U32
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = np.uint64(key[0]) & _U32, np.uint64(key[1]) & _U32
    for _ in range(10):
        p0, p1 = _PHILOX_M[0] * c0, _PHILOX_M[1] * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & _U32,
                          (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & _U32)
        k0, k1 = (k0 + _PHILOX_W[0]) & _U32, (k1 + _PHILOX_W[1]) & _U32
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def dropout_keep_at(elems, p, seed):
    """Keep decisions of the elements with flat indices ``elems`` (any shape):
    element e takes word e % 4 of Philox4x32-10 at counter (e // 4 low word,
    e // 4 high word, 0, 0) with key (seed low, seed high), and is dropped
    when that word is below floor(p * 2^32) (p a float32; p = 0 drops
    nothing)."""
    e = np.asarray(elems, dtype=np.uint64)
    blk = e >> np.uint64(2)
    z = np.zeros(blk.shape, np.uint64)
    ctr = np.stack([blk & _U32, blk >> np.uint64(32), z, z], axis=-1)
    words = philox4x32_10(ctr, (int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF))
    w = np.take_along_axis(words, (e & np.uint64(3)).astype(np.int64)[..., None], axis=-1)[..., 0]
    thr = min(int(float(np.float32(p)) * 4294967296.0), 0xFFFFFFFF)
    return w.astype(np.uint64) >= np.uint64(thr)


def dropout_keep(n, p, seed):
    """Keep mask of the n elements 0 .. n-1 of one call (``dropout_keep_at``)."""
    return dropout_keep_at(np.arange(int(n), dtype=np.uint64), p, seed)


def embedding_forward(word_parts, PE, pos, p, seed, TE=None, tt=None, tokens=None):
    """out[t] = dropout(sum_r word_parts[r][t] + PE[pos[t]] (+ TE[tt[t]])):
    kept elements are scaled by 1 / (1 - p).  A position or token-type id
    outside its table contributes a zero row (the vocabulary's masking rule).
    ``tokens`` gives the rows' token indices in the full call when the rows
    are a sample of it (the mask is keyed by flat index token * H + column);
    by default row t is token t.  Returns (out, keep mask [T x H])."""
    x = shard_reduce(word_parts)
    T, H = x.shape
    for table, ids in ((PE, pos), (TE, tt)):
        if table is None:
            continue
        ids = np.asarray(ids, dtype=np.int64)
        ok = (ids >= 0) & (ids < table.shape[0])
        rows = np.zeros((T, H))
        rows[ok] = np.asarray(table, dtype=np.float64)[ids[ok]]
        x = x + rows
    tok = np.arange(T, dtype=np.uint64) if tokens is None else np.asarray(tokens, dtype=np.uint64)
    keep = dropout_keep_at(tok[:, None] * np.uint64(H) + np.arange(H, dtype=np.uint64)[None, :], p, seed)
    return np.where(keep, x / (1.0 - float(np.float32(p))), 0.0), keep


def embedding_backward(dout, keep, p, pos, pos_rows, tt=None, tt_rows=0):
    """Gradients of ``embedding_forward``: dX = dout * keep / (1 - p) is the
    word embedding's upstream gradient (vocab_embed_backward per shard), and
    the position and token-type tables receive its rows summed by id.
    Returns (dX, dPE, dTE or None)."""
    dX = np.where(keep, np.asarray(dout, dtype=np.float64) / (1.0 - float(np.float32(p))), 0.0)
    dPE = vocab_embed_backward(pos, dX, 0, pos_rows)
    dTE = vocab_embed_backward(tt, dX, 0, tt_rows) if tt is not None else None
    return dX, dPE, dTE


# ---------------------------------------------------------------------------
# Sequence parallelism: activations outside the tensor-parallel GEMMs are
# split along the sequence (rows), s/N per shard (page "5-megatron", the
# schedule's note that the sequence component becomes s/N; page
# "zwxr 246059", section 4.3: the LayerNorm gradients of sequence-parallel
# regions are summed over the tensor-parallel group).  The row split follows
# ``partition``.
# ---------------------------------------------------------------------------

def sp_reduce_scatter(parts, n, res=None):
    """The reduce-scatter that replaces the g all-reduce: shard r receives its
    rows of sum(parts) (shard order), plus its rows ``res[r]`` of the
    residual stream when given.  Returns the list of row slices."""
    total = shard_reduce(parts)
    M = total.shape[0]
    out = []
    for r in range(n):
        s, c = partition(M, n, r)
        y = total[s:s + c].copy()
        if res is not None:
            y = np.asarray(res[r], dtype=np.float64) + y
        out.append(y)
    return out


def sp_all_gather(slices):
    """The all-gather before a column-parallel GEMM: the shards' row slices
    concatenated in shard order."""
    return np.concatenate([np.asarray(x, dtype=np.float64) for x in slices], axis=0)


def sp_layernorm_param_grads(x_slices, gamma, mean_slices, rstd_slices, dy_slices):
    """LayerNorm on sequence shards: each shard's (dx_r, dgamma_r, dbeta_r)
    from its own rows, and the parameter gradients summed over shards in
    shard order.  Returns (dx slices, dgamma, dbeta)."""
    dxs, dg, db = [], 0.0, 0.0
    for x, m, rs, dy in zip(x_slices, mean_slices, rstd_slices, dy_slices):
        dx, g_r, b_r = layernorm_backward(x, gamma, m, rs, dy)
        dxs.append(dx)
        dg = dg + g_r
        db = db + b_r
    return dxs, dg, db


# ---------------------------------------------------------------------------
# The two linear layers on their own (page "5-megatron", sections
# ColumnParallelLinear and RowParallelLinear), in math layout: Y = X A + b.
# ---------------------------------------------------------------------------

def column_linear_forward(X, A, b, n, gather_output=True, skip_bias_add=False):
    """ColumnParallelLinear over n shards: A = [A_1 .. A_n] split along its
    columns, each shard computes Y_r = X A_r + b_r with its slice b_r of the
    bias (the f operator copies X to every shard), and with ``gather_output``
    the shards' outputs are concatenated along columns (the g operator's
    all-gather).  With ``skip_bias_add`` no bias is added (the layer returns
    it instead).  Returns the list of Y_r, and their concatenation when
    gathered."""
    X = np.asarray(X, dtype=np.float64)
    outs = []
    for r in range(n):
        Ar = split_columns(A, n, r)
        Yr = X @ Ar
        if b is not None and not skip_bias_add:
            s, c = partition(np.shape(A)[1], n, r)
            Yr = Yr + np.asarray(b, dtype=np.float64)[s:s + c][None, :]
        outs.append(Yr)
    return outs, (np.concatenate(outs, axis=1) if gather_output else None)


def column_linear_backward(X, A_r, dY_r):
    """Backward of one column shard for its output gradient dY_r (the split
    of a gathered gradient, the g operator's backward): dX_r = dY_r A_r^T is a
    partial that the f operator's backward sums over shards; dA_r = X^T dY_r;
    the bias slice's gradient is the column sum of dY_r.  Returns
    (dX_r, dA_r, db_r)."""
    dY_r = np.asarray(dY_r, dtype=np.float64)
    return dY_r @ np.asarray(A_r).T, np.asarray(X).T @ dY_r, dY_r.sum(axis=0)


def row_linear_forward(X, B, b, n, input_is_parallel=False, skip_bias_add=False):
    """RowParallelLinear over n shards: B = [B_1; ..; B_n] split along its
    rows; unless ``input_is_parallel`` the full input X is split along its
    columns into X_r (the scatter); each shard computes the partial
    X_r B_r, the partials are summed (the all-reduce), and then the full bias
    is added once unless ``skip_bias_add``.  ``X`` is the full input, or the
    list of X_r when ``input_is_parallel``.  Returns (partials, output)."""
    parts = []
    for r in range(n):
        Xr = np.asarray(X[r] if input_is_parallel else split_columns(X, n, r), dtype=np.float64)
        parts.append(Xr @ split_rows(B, n, r))
    Y = shard_reduce(parts)
    if b is not None and not skip_bias_add:
        Y = Y + np.asarray(b, dtype=np.float64)[None, :]
    return parts, Y


def row_linear_backward(X_r, B_r, dY):
    """Backward of one row shard for the full output gradient dY (the
    all-reduce's backward is the identity): dX_r = dY B_r^T (the scatter's
    backward gathers the shards' dX_r along columns), dB_r = X_r^T dY, and the
    replicated bias's gradient is the column sum of dY.  Returns
    (dX_r, dB_r, db)."""
    dY = np.asarray(dY, dtype=np.float64)
    return dY @ np.asarray(B_r).T, np.asarray(X_r).T @ dY, dY.sum(axis=0)


# ---------------------------------------------------------------------------
# Vocab-parallel cross entropy over the shards of the tied logits.
# ---------------------------------------------------------------------------

def vocab_ce_forward(logit_shards, targets, starts):
    """Cross entropy of every token over logits split by vocab rows across
    shards, computed the way the pages lay it out (page "5-megatron", section
    _VocabParallelCrossEntropy, its flow and its code; page "notion
    310f8c09", section 交叉熵张量并行, stages two to four; page
    "Megtron张量/模型并行", section Cross-entropy层), in this order:

    1. each shard's row maximum; the maximum over shards (the MAX all-reduce);
    2. every shard subtracts that global maximum from its logits;
    3. each shard takes its shifted logit at the target's column when the
       target lies in its range [start, start + rows), else 0; the values are
       summed over shards (a SUM all-reduce), giving the target's logit;
    4. each shard's row sum of exp of its shifted logits; summed over shards
       (a SUM all-reduce), giving the softmax denominator;
    5. loss = log(denominator) - target's shifted logit.

    ``logit_shards``: list of [T x rows_r] arrays (fp64 values); ``targets``:
    [T] integer ids; ``starts``: first vocab row of every shard.  A target
    that lies in no shard contributes 0 in step 3 on every shard, as in the
    page's code.  Returns ``(loss, softmax_shards, gmax, denom)``: loss [T],
    the shards' softmax exp(shifted) / denom (what the page's code keeps for
    the backward), the global maximum and the denominator [T].
    """
    targets = np.asarray(targets, dtype=np.int64)
    shards = [np.asarray(x, dtype=np.float64) for x in logit_shards]
    gmax = np.max(np.stack([x.max(axis=1) for x in shards]), axis=0)
    shifted = [x - gmax[:, None] for x in shards]
    picked = np.zeros(len(targets))
    rows_t = np.arange(len(targets))
    for x, start in zip(shifted, starts):
        rows = x.shape[1]
        out = (targets < start) | (targets >= start + rows)
        local = np.where(out, 0, targets - start)
        part = x[rows_t, local].copy()
        part[out] = 0.0
        picked += part
    exps = [np.exp(x) for x in shifted]
    denom = np.zeros(len(targets))
    for e in exps:
        denom += e.sum(axis=1)
    loss = np.log(denom) - picked
    softmax = [e / denom[:, None] for e in exps]
    return loss, softmax, gmax, denom


def vocab_ce_backward(softmax_shards, targets, starts, dloss):
    """Gradient of ``vocab_ce_forward`` w.r.t. each shard's logits: the kept
    softmax, minus 1 at the target's column on the shard that owns the
    target, times the upstream gradient of each token's loss (page
    "5-megatron", section _VocabParallelCrossEntropy, the backward of its
    code)."""
    targets = np.asarray(targets, dtype=np.int64)
    dloss = np.asarray(dloss, dtype=np.float64)
    rows_t = np.arange(len(targets))
    grads = []
    for sm, start in zip(softmax_shards, starts):
        rows = sm.shape[1]
        g = np.array(sm, dtype=np.float64, copy=True)
        inr = (targets >= start) & (targets < start + rows)
        g[rows_t[inr], targets[inr] - start] -= 1.0
        grads.append(g * dloss[:, None])
    return grads


# ---------------------------------------------------------------------------
# LayerNorm (replicated; used by the stacked model).
# ---------------------------------------------------------------------------

def layernorm_forward(x, gamma, beta, eps=1e-5):
    """y = (x - mean) / sqrt(var + eps) * gamma + beta per row, biased variance.

    Page "5-megatron", section 训练一般流程 counts two LayerNorms per layer
    with 2*(2H) parameters (a scale and a shift of width H each); the formula
    is not printed, so the standard definition is taken.
    Returns (y, mean, rstd).
    """
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    y = (x - mu) * rstd * gamma[None, :] + beta[None, :]
    return y, mu[:, 0], rstd[:, 0]


def layernorm_backward(x, gamma, mean, rstd, dy):
    """Returns (dx, dgamma, dbeta) for ``layernorm_forward``."""
    xhat = (x - mean[:, None]) * rstd[:, None]
    dgamma = (dy * xhat).sum(axis=0)
    dbeta = dy.sum(axis=0)
    g = dy * gamma[None, :]
    dx = rstd[:, None] * (g - g.mean(axis=1, keepdims=True)
                          - xhat * (g * xhat).mean(axis=1, keepdims=True))
    return dx, dgamma, dbeta


# ---------------------------------------------------------------------------
# Closed forms.
# ---------------------------------------------------------------------------

def param_count(H, L, V):
    """(12 H^2 + 4 H) L + 2 H V, the page's count (page "5-megatron", section
    训练一般流程): per layer 3H^2 for Q/K/V, H^2 for the output linear, 8H^2
    for the MLP, 4H for two LayerNorms; plus input and output embeddings."""
    return (12 * H * H + 4 * H) * L + 2 * H * V


def param_count_tied_unique(H, L, V):
    """Unique stored parameters when input and output share one table."""
    return (12 * H * H + 4 * H) * L + H * V


# ---------------------------------------------------------------------------
# Output rounding (for bit comparisons only).
# ---------------------------------------------------------------------------

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_to_bf16(x):
    """Round fp64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps fp32's 8 exponent bits and 7 stored mantissa bits (page
    "5-megatron", section 分布式混合精度训练, BF16 format).  Written from that
    definition: 8 significant bits for normal numbers, a fixed quantum of
    2^-133 below 2^-126, overflow to infinity past the largest finite value.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    fin = np.isfinite(x)
    out[~fin] = x[~fin]
    xf = x[fin]
    tiny = np.abs(xf) < 2.0 ** -126
    m, e = np.frexp(xf)                     # xf = m * 2**e, 0.5 <= |m| < 1
    normal = np.ldexp(np.rint(m * 256.0), e - 8)   # np.rint rounds half to even
    sub = np.rint(xf * 2.0 ** 133) * 2.0 ** -133
    r = np.where(tiny, sub, normal)
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, xf), r)
    out[fin] = r
    return out


def round_to_f32(x):
    """Round fp64 to the nearest fp32 (IEEE, ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_next_up(x):
    """Smallest bfloat16 value strictly above the bfloat16 value x (x > 0 normal)."""
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) + 1.0, e - 8)


# ---------------------------------------------------------------------------
# Stacked GPT (embedding -> L x [pre-LN attention, pre-LN MLP] -> tied logits),
# every TP shard executed and reduced.
# ---------------------------------------------------------------------------

def gpt_forward(ids, E, layers, b, s, nheads, d, n, eps=1e-5, causal=True):
    """Forward of the stacked model with n tensor-parallel shards.

    ``E`` is the full (V, H) table; ``layers`` a list of dicts with keys
    WQ, WK, WV, WO (H x H), A (H x 4H), B (4H x H), g1, b1, g2, b2 (H,).
    Composition (page "5-megatron", sections ParallelTransformerLayer /
    ParallelTransformer name attention + MLP per layer; the pre-LN residual
    form, eps and the absence of a final LayerNorm are readings chosen to
    match the page's parameter count).  Returns (logits list per shard,
    cache for ``gpt_backward``).
    """
    V = E.shape[0]
    parts = []
    for r in range(n):
        st, cnt = partition(V, n, r)
        parts.append(vocab_embed_forward(ids, E[st:st + cnt], st))
    x = shard_reduce(parts)
    cache = {"x_in": [], "ln": []}
    for lw in layers:
        cache["x_in"].append(x)
        y1, mu1, rs1 = layernorm_forward(x, lw["g1"], lw["b1"], eps)
        _, za = tp_attention_forward(y1, lw["WQ"], lw["WK"], lw["WV"], lw["WO"], b, s, nheads, d, n, causal)
        x2 = x + za
        y2, mu2, rs2 = layernorm_forward(x2, lw["g2"], lw["b2"], eps)
        _, zm = tp_mlp_forward(y2, lw["A"], lw["B"], n)
        cache["ln"].append((y1, mu1, rs1, x2, y2, mu2, rs2))
        x = x2 + zm
    cache["x_out"] = x
    logits = []
    for r in range(n):
        st, cnt = partition(V, n, r)
        logits.append(tied_logits(x, E[st:st + cnt]))
    return logits, cache


def gpt_backward(ids, E, layers, cache, dlogits, b, s, nheads, d, n, causal=True):
    """Backward of ``gpt_forward`` for per-shard logit gradients ``dlogits``.

    Returns (dE_full, per-layer gradient dicts).  The table's gradient is the
    sum of the output-side and input-side gradients (page "Megtron张量/模型并行",
    section 输出层Embedding).
    """
    V = E.shape[0]
    x = cache["x_out"]
    dE = np.zeros_like(E, dtype=np.float64)
    dx_parts = []
    for r in range(n):
        st, cnt = partition(V, n, r)
        dxr, dEr = tied_logits_backward(x, E[st:st + cnt], dlogits[r])
        dx_parts.append(dxr)
        dE[st:st + cnt] += dEr
    dx = shard_reduce(dx_parts)
    grads = [None] * len(layers)
    for li in reversed(range(len(layers))):
        lw = layers[li]
        y1, mu1, rs1, x2, y2, mu2, rs2 = cache["ln"][li]
        x_in = cache["x_in"][li]
        # MLP sublayer: x_out = x2 + MLP(LN2(x2))
        res, dy2 = tp_mlp_backward(y2, lw["A"], lw["B"], dx, n)
        dA = np.concatenate([o[1] for o in res], axis=1)
        dB = np.concatenate([o[2] for o in res], axis=0)
        dx2_ln, dg2, db2 = layernorm_backward(x2, lw["g2"], mu2, rs2, dy2)
        dx2 = dx + dx2_ln
        # attention sublayer: x2 = x_in + ATT(LN1(x_in))
        res, dy1 = tp_attention_backward(y1, lw["WQ"], lw["WK"], lw["WV"], lw["WO"], dx2,
                                         b, s, nheads, d, n, causal)
        dx_in_ln, dg1, db1 = layernorm_backward(x_in, lw["g1"], mu1, rs1, dy1)
        dx = dx2 + dx_in_ln
        hs = nheads // n
        w = hs * d
        dWQ = np.concatenate([o[1][:, 0:w] for o in res], axis=1)
        dWK = np.concatenate([o[1][:, w:2 * w] for o in res], axis=1)
        dWV = np.concatenate([o[1][:, 2 * w:3 * w] for o in res], axis=1)
        dWO = np.concatenate([o[2] for o in res], axis=0)
        grads[li] = {"WQ": dWQ, "WK": dWK, "WV": dWV, "WO": dWO, "A": dA, "B": dB,
                     "g1": dg1, "b1": db1, "g2": dg2, "b2": db2}
    for r in range(n):
        st, cnt = partition(V, n, r)
        dE[st:st + cnt] += vocab_embed_backward(ids, dx, st, cnt)
    return dE, grads
