"""Pins of the fp64 oracle against what the pages and mathematics fix.

CPU only.  Each test checks an oracle function against something other than
itself: values printed on the pages (tests/golden/*.json, each citing its
passage), closed forms, invariants, scalar-loop brute force on tiny inputs,
or central finite differences of the oracle's own forward.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- partition

def test_partition_page_examples():
    g = golden("partition_examples.json")
    for case in g["cases"]:
        got = [list(O.partition(case["total"], case["n"], r)) for r in range(case["n"])]
        assert got == case["shards"], case


@pytest.mark.parametrize("total,n", [(7, 3), (50257, 8), (16, 4), (1, 2), (0, 3)])
def test_partition_covers_exactly(total, n):
    pos = 0
    for r in range(n):
        s, c = O.partition(total, n, r)
        assert s == pos and c >= 0
        pos += c
    assert pos == total
    counts = [O.partition(total, n, r)[1] for r in range(n)]
    assert max(counts) - min(counts) <= 1


# ---------------------------------------------------------------- embedding

def test_masking_page_example():
    g = golden("masking_example.json")
    mask, local = O.vocab_embed_mask(g["ids"], g["start"], g["end"] - g["start"])
    assert local.tolist() == g["masked"]
    assert mask.tolist() == g["mask"]


def test_embedding_worked_example():
    g = golden("embedding_worked_example.json")
    V, n, toks = g["vocab"], g["shards"], g["tokens"]
    E = rng(1).standard_normal((V, 16)) + 3.0        # no zero rows by accident
    parts = []
    for r in range(n):
        s, c = O.partition(V, n, r)
        assert [s, s + c] == g["ranges"][r]
        Y = O.vocab_embed_forward(toks, E[s:s + c], s)
        found = [int(np.any(Y[t] != 0)) for t in range(len(toks))]
        assert found == g["found"][r]
        for t, tok in enumerate(toks):
            if found[t]:
                assert np.array_equal(Y[t], E[tok])
            else:
                assert np.all(Y[t] == 0)
        parts.append(Y)
    total = O.shard_reduce(parts)
    assert [int(np.any(row != 0)) for row in total] == g["sum_found"]
    # Special case: the shard sum is an ordinary gather from the full table.
    assert np.array_equal(total, E[toks])


def test_embedding_out_of_range_ids_are_zero():
    E = rng(2).standard_normal((10, 4)) + 1
    Y = O.vocab_embed_forward([-1, 10, 12, 3], E[0:5], 0)
    assert np.all(Y[:3] == 0) and np.array_equal(Y[3], E[3])


def _embed_backward_loop(ids, dY, start, rows):
    dE = [[0.0] * dY.shape[1] for _ in range(rows)]
    for t, tok in enumerate(ids):
        if start <= tok < start + rows:
            for c in range(dY.shape[1]):
                dE[tok - start][c] += float(dY[t, c])
    return np.array(dE)


def test_embed_backward_bruteforce_and_identity():
    g = rng(3)
    V, H, T, n = 23, 5, 40, 3
    ids = g.integers(-2, V + 2, T)
    dY = g.standard_normal((T, H))
    col_total = np.zeros(H)
    for r in range(n):
        s, c = O.partition(V, n, r)
        dE = O.vocab_embed_backward(ids, dY, s, c)
        assert np.allclose(dE, _embed_backward_loop(ids, dY, s, c), rtol=0, atol=1e-12)
        col_total += dE.sum(axis=0)
    inr = (ids >= 0) & (ids < V)
    assert np.allclose(col_total, dY[inr].sum(axis=0), atol=1e-12)


def test_embed_backward_finite_difference():
    g = rng(4)
    V, H, T = 9, 3, 12
    ids = g.integers(0, V + 3, T)
    E = g.standard_normal((V, H))
    R = g.standard_normal((T, H))
    s, c = O.partition(V, 2, 1)
    dE = O.vocab_embed_backward(ids, R, s, c)
    h = 1e-6
    for j in range(c):
        for k in range(H):
            Ep, Em = E[s:s + c].copy(), E[s:s + c].copy()
            Ep[j, k] += h
            Em[j, k] -= h
            fd = (np.sum(R * O.vocab_embed_forward(ids, Ep, s)) -
                  np.sum(R * O.vocab_embed_forward(ids, Em, s))) / (2 * h)
            assert abs(fd - dE[j, k]) <= 1e-6 * max(1.0, abs(fd))


def test_tied_gradient_is_sum_of_both_uses():
    """Finite differences through both uses of the shared table pin the
    'sum of the input-side and output-side gradients' rule."""
    g = rng(5)
    V, H, T, n = 7, 4, 6, 2
    ids = g.integers(0, V, T)
    E = g.standard_normal((V, H))
    W = g.standard_normal((H, H))
    R = [g.standard_normal((T, O.partition(V, n, r)[1])) for r in range(n)]

    def loss(Ef):
        x = O.shard_reduce([O.vocab_embed_forward(ids, Ef[s:s + c], s)
                            for s, c in (O.partition(V, n, r) for r in range(n))])
        hdn = x @ W
        return sum(np.sum(R[r] * O.tied_logits(hdn, Ef[slice(*_rng(V, n, r))]))
                   for r in range(n))

    def _rng(V_, n_, r_):
        s, c = O.partition(V_, n_, r_)
        return s, s + c

    x = O.shard_reduce([O.vocab_embed_forward(ids, E[s:s + c], s)
                        for s, c in (O.partition(V, n, r) for r in range(n))])
    hdn = x @ W
    dE = np.zeros_like(E)
    dh = []
    for r in range(n):
        s, c = O.partition(V, n, r)
        dh_r, dE_out = O.tied_logits_backward(hdn, E[s:s + c], R[r])
        dE[s:s + c] += dE_out
        dh.append(dh_r)
    dx = O.shard_reduce(dh) @ W.T
    for r in range(n):
        s, c = O.partition(V, n, r)
        dE[s:s + c] += O.vocab_embed_backward(ids, dx, s, c)
    h = 1e-6
    for j in range(V):
        for k in range(H):
            Ep, Em = E.copy(), E.copy()
            Ep[j, k] += h
            Em[j, k] -= h
            fd = (loss(Ep) - loss(Em)) / (2 * h)
            assert abs(fd - dE[j, k]) <= 1e-6 * max(1.0, abs(fd)), (j, k)


# ---------------------------------------------------------------- closed forms

def test_param_count_page_value():
    g = golden("param_count.json")
    assert O.param_count(g["H"], g["L"], g["V"]) == g["total"]
    body = (12 * g["H"] ** 2 + 4 * g["H"]) * g["L"]
    assert abs(body - g["body_approx"]) / g["body_approx"] < 0.01
    assert O.param_count_tied_unique(g["H"], g["L"], g["V"]) == g["total"] - g["H"] * g["V"]


def test_bf16_epsilon_page_value():
    g = golden("format_epsilon.json")
    assert O.bf16_next_up(1.0) - 1.0 == g["bf16"]
    assert O.round_to_bf16(np.array([1.0 + g["bf16"]]))[0] == 1.0 + g["bf16"]
    # the midpoint 1 + eps/2 ties to the even neighbour 1
    assert O.round_to_bf16(np.array([1.0 + g["bf16"] / 2]))[0] == 1.0
    assert O.round_to_bf16(np.array([1.0 + 3 * g["bf16"] / 2]))[0] == 1.0 + 2 * g["bf16"]
    assert abs(2.0 ** -23 - g["fp32"]) < 1e-9


def _all_finite_bf16():
    bits = np.arange(0, 0x10000, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = (bits << 16).view(np.float32).astype(np.float64)
    ok = np.isfinite(vals)
    return vals[ok], bits[ok]


def test_round_to_bf16_bruteforce_nearest():
    vals, bits = _all_finite_bf16()
    order = np.argsort(vals, kind="stable")
    sv, sb = vals[order], bits[order]
    # drop -0 duplicate of +0 (keep the +0 pattern, which is even)
    keep = np.ones(len(sv), bool)
    keep[(sv == 0) & (sb == 0x8000)] = False
    sv, sb = sv[keep], sb[keep]
    g = rng(6)
    xs = np.concatenate([
        g.standard_normal(4000) * 10.0 ** g.integers(-30, 30, 4000),
        g.standard_normal(500) * 2.0 ** -130,                        # subnormal range
        (sv[1000:1500] + sv[1001:1501]) / 2,                          # exact ties
        sv[2000:2500],                                                 # representable
    ])
    got = O.round_to_bf16(xs)
    for x, y in zip(xs, got):
        i = np.searchsorted(sv, x)
        cands = [k for k in (i - 1, i) if 0 <= k < len(sv)]
        best = min(abs(sv[k] - x) for k in cands)
        near = [k for k in cands if abs(sv[k] - x) == best]
        if len(near) == 2:                                              # tie: even pattern
            near = [k for k in near if sb[k] % 2 == 0]
        assert y == sv[near[0]], (x, y, sv[near[0]])
    assert O.round_to_bf16(np.array([3.5e38]))[0] == np.inf


# ---------------------------------------------------------------- GELU

def test_gelu_closed_forms():
    assert O.gelu(np.array(0.0)) == 0.0
    x = np.linspace(-6, 6, 101)
    assert np.allclose(O.gelu(x) - O.gelu(-x), x, atol=1e-14)
    q = 1.959963984540054          # standard normal 97.5 % quantile
    assert abs(O.gelu(np.array(q)) / q - 0.975) < 1e-12
    assert abs(O.gelu(np.array(30.0)) - 30.0) < 1e-12
    assert abs(O.gelu(np.array(-30.0))) < 1e-12
    assert O.gelu_grad(np.array(0.0)) == 0.5


def test_gelu_grad_finite_difference():
    x = np.linspace(-5, 5, 41)
    h = 1e-6
    fd = (O.gelu(x + h) - O.gelu(x - h)) / (2 * h)
    assert np.allclose(fd, O.gelu_grad(x), atol=1e-8)


# ---------------------------------------------------------------- MLP

def _mlp_loop(X, A, B):
    M, h = X.shape
    f = A.shape[1]
    Z = [[0.0] * B.shape[1] for _ in range(M)]
    for m in range(M):
        H = []
        for j in range(f):
            p = sum(X[m, k] * A[k, j] for k in range(h))
            H.append(0.5 * p * (1 + math.erf(p / math.sqrt(2))))
        for c in range(B.shape[1]):
            Z[m][c] = sum(H[j] * B[j, c] for j in range(f))
    return np.array(Z)


def test_mlp_forward_bruteforce():
    g = rng(7)
    X, A, B = g.standard_normal((3, 4)), g.standard_normal((4, 8)), g.standard_normal((8, 4))
    _, _, Z = O.mlp_forward(X, A, B)
    assert np.allclose(Z, _mlp_loop(X, A, B), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("n", [2, 4])
def test_mlp_shards_sum_to_unsharded(n):
    g = rng(8)
    X, A, B = g.standard_normal((5, 6)), g.standard_normal((6, 16)), g.standard_normal((16, 6))
    dZ = g.standard_normal((5, 6))
    P, H, Z = O.mlp_forward(X, A, B)
    dX, dA, dB = O.mlp_backward(X, A, B, P, dZ)
    outs, Zs = O.tp_mlp_forward(X, A, B, n)
    assert np.allclose(Zs, Z, rtol=1e-12, atol=1e-12)
    res, dXs = O.tp_mlp_backward(X, A, B, dZ, n)
    assert np.allclose(dXs, dX, rtol=1e-12, atol=1e-12)
    for r in range(n):
        s, c = O.partition(16, n, r)
        assert np.allclose(res[r][1], dA[:, s:s + c], rtol=1e-12, atol=1e-12)
        assert np.allclose(res[r][2], dB[s:s + c, :], rtol=1e-12, atol=1e-12)
        assert np.allclose(outs[r][1], H[:, s:s + c], rtol=1e-12, atol=1e-12)


def _fd_check(f, args, grads, h=1e-6, tol=1e-6):
    """Central differences of scalar f w.r.t. every entry of every array in args."""
    for a, gr in zip(args, grads):
        it = np.nditer(a, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = a[i]
            a[i] = old + h
            fp = f()
            a[i] = old - h
            fm = f()
            a[i] = old
            fd = (fp - fm) / (2 * h)
            assert abs(fd - gr[i]) <= tol * max(1.0, abs(fd)), (i, fd, gr[i])


def test_mlp_backward_finite_difference():
    g = rng(9)
    X, A, B = g.standard_normal((3, 4)), g.standard_normal((4, 8)), g.standard_normal((8, 4))
    R = g.standard_normal((3, 4))
    P, _, _ = O.mlp_forward(X, A, B)
    dX, dA, dB = O.mlp_backward(X, A, B, P, R)
    _fd_check(lambda: np.sum(R * O.mlp_forward(X, A, B)[2]), [X, A, B], [dX, dA, dB])


# ---------------------------------------------------------------- attention

def test_attention_single_position_returns_v():
    g = rng(10)
    Q, K, V = g.standard_normal((1, 4)), g.standard_normal((1, 4)), g.standard_normal((1, 4))
    Ot, lse = O.attention_head_forward(Q, K, V, causal=True)
    assert np.allclose(Ot, V, atol=1e-15)
    assert np.allclose(lse, (Q @ K.T)[0] / 2.0, atol=1e-15)


def test_attention_zero_query_is_running_mean():
    g = rng(11)
    s, d = 7, 3
    K, V = g.standard_normal((s, d)), g.standard_normal((s, d))
    Ot, lse = O.attention_head_forward(np.zeros((s, d)), K, V, causal=True)
    for i in range(s):
        assert np.allclose(Ot[i], V[:i + 1].mean(axis=0), atol=1e-14)
        assert abs(lse[i] - math.log(i + 1)) < 1e-14
    On, _ = O.attention_head_forward(np.zeros((s, d)), K, V, causal=False)
    assert np.allclose(On, np.tile(V.mean(axis=0), (s, 1)), atol=1e-14)


def _attn_loop(Q, K, V, causal):
    s, d = Q.shape
    out = np.zeros_like(V)
    for i in range(s):
        lim = i + 1 if causal else K.shape[0]
        sc = [sum(Q[i, c] * K[j, c] for c in range(d)) / math.sqrt(d) for j in range(lim)]
        mx = max(sc)
        w = [math.exp(v - mx) for v in sc]
        tot = sum(w)
        for c in range(d):
            out[i, c] = sum(w[j] * V[j, c] for j in range(lim)) / tot
    return out


@pytest.mark.parametrize("causal", [True, False])
def test_attention_bruteforce(causal):
    g = rng(12)
    Q, K, V = (g.standard_normal((5, 4)) * 2 for _ in range(3))
    Ot, _ = O.attention_head_forward(Q, K, V, causal)
    assert np.allclose(Ot, _attn_loop(Q, K, V, causal), atol=1e-13)
    assert np.allclose(Ot[0], V[0], atol=1e-15) if causal else True


@pytest.mark.parametrize("causal", [True, False])
def test_attention_head_backward_finite_difference(causal):
    g = rng(13)
    Q, K, V = g.standard_normal((4, 3)), g.standard_normal((4, 3)), g.standard_normal((4, 3))
    R = g.standard_normal((4, 3))
    Ot, _ = O.attention_head_forward(Q, K, V, causal)
    dQ, dK, dV = O.attention_head_backward(Q, K, V, Ot, R, causal)
    _fd_check(lambda: np.sum(R * O.attention_head_forward(Q, K, V, causal)[0]),
              [Q, K, V], [dQ, dK, dV])


def _attn_full(X, WQ, WK, WV, WO, b, s, nh, d):
    return O.attention_layer_forward(X, np.concatenate([WQ, WK, WV], axis=1), WO, b, s, nh, d)


def test_attention_layer_shards_sum_to_unsharded_and_heads_permute():
    g = rng(14)
    b, s, h, nh, d, n = 2, 5, 6, 4, 3, 2
    X = g.standard_normal((b * s, h))
    WQ, WK, WV = (g.standard_normal((h, nh * d)) for _ in range(3))
    WO = g.standard_normal((nh * d, h))
    dZ = g.standard_normal((b * s, h))
    QKV, Ob, lse, Z = _attn_full(X, WQ, WK, WV, WO, b, s, nh, d)
    _, Zs = O.tp_attention_forward(X, WQ, WK, WV, WO, b, s, nh, d, n)
    assert np.allclose(Zs, Z, atol=1e-12)
    Wqkv = np.concatenate([WQ, WK, WV], axis=1)
    dX, dWqkv, dWo = O.attention_layer_backward(X, Wqkv, WO, QKV, Ob, dZ, b, s, nh, d)
    res, dXs = O.tp_attention_backward(X, WQ, WK, WV, WO, dZ, b, s, nh, d, n)
    assert np.allclose(dXs, dX, atol=1e-12)
    hs, w = nh // n, nh * d
    for r in range(n):
        c = slice(r * hs * d, (r + 1) * hs * d)
        got = res[r][1]
        assert np.allclose(got[:, :hs * d], dWqkv[:, c], atol=1e-12)
        assert np.allclose(got[:, hs * d:2 * hs * d], dWqkv[:, w:][:, c], atol=1e-12)
        assert np.allclose(got[:, 2 * hs * d:], dWqkv[:, 2 * w:][:, c], atol=1e-12)
        assert np.allclose(res[r][2], dWo[c, :], atol=1e-12)
    # a consistent permutation of the heads leaves Z unchanged
    perm = [2, 0, 3, 1]
    cols = np.concatenate([np.arange(p * d, (p + 1) * d) for p in perm])
    _, _, _, Zp = _attn_full(X, WQ[:, cols], WK[:, cols], WV[:, cols], WO[cols, :], b, s, nh, d)
    assert np.allclose(Zp, Z, atol=1e-12)


def test_attention_layer_backward_finite_difference():
    g = rng(15)
    b, s, h, nh, d = 1, 3, 4, 2, 2
    X = g.standard_normal((b * s, h))
    Wqkv = g.standard_normal((h, 3 * nh * d))
    Wo = g.standard_normal((nh * d, h))
    R = g.standard_normal((b * s, h))
    QKV, Ob, _, _ = O.attention_layer_forward(X, Wqkv, Wo, b, s, nh, d)
    dX, dWqkv, dWo = O.attention_layer_backward(X, Wqkv, Wo, QKV, Ob, R, b, s, nh, d)
    _fd_check(lambda: np.sum(R * O.attention_layer_forward(X, Wqkv, Wo, b, s, nh, d)[3]),
              [X, Wqkv, Wo], [dX, dWqkv, dWo])


# ---------------------------------------------------------------- shard_reduce

def test_shard_reduce_exact_and_ordered():
    g = rng(16)
    parts = [g.integers(-1000, 1000, (4, 5)).astype(np.float64) for _ in range(5)]
    tot = np.zeros((4, 5))
    for p in parts:
        for i in range(4):
            for j in range(5):
                tot[i, j] += p[i, j]
    assert np.array_equal(O.shard_reduce(parts), tot)


def test_shard_reduce_two_bf16_parts_round_once():
    """For two bf16 parts the fp64 sum rounded once equals the correctly
    rounded bf16 sum found by brute force (nearest representable, ties even)."""
    vals, bits = _all_finite_bf16()
    g = rng(17)
    a = vals[g.integers(0, len(vals), 3000)]
    b = vals[g.integers(0, len(vals), 3000)]
    ok = np.abs(a) < 1e37
    a, b = a[ok], b[ok]
    got = O.round_to_bf16(O.shard_reduce([a, b]))
    order = np.argsort(vals)
    sv, sb = vals[order], bits[order]
    for x, y in zip(a + b, got):
        i = np.searchsorted(sv, x)
        cands = [k for k in (i - 1, i) if 0 <= k < len(sv)]
        best = min(abs(sv[k] - x) for k in cands)
        near = [k for k in cands if abs(sv[k] - x) == best]
        if len(near) == 2 and sv[near[0]] != sv[near[1]]:
            near = [k for k in near if sb[k] % 2 == 0]
        assert y == sv[near[0]]


# ---------------------------------------------------------------- LayerNorm

def test_layernorm_invariants_and_loop():
    g = rng(18)
    x = g.standard_normal((4, 9)) * 3 + 1
    gam, bet = np.ones(9), np.zeros(9)
    y, mu, rs = O.layernorm_forward(x, gam, bet, 1e-5)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-13)
    var = x.var(axis=1)
    assert np.allclose(y.var(axis=1), var / (var + 1e-5), atol=1e-12)
    gam, bet = g.standard_normal(9), g.standard_normal(9)
    y, _, _ = O.layernorm_forward(x, gam, bet, 1e-5)
    for i in range(4):
        m = sum(x[i]) / 9
        v = sum((t - m) ** 2 for t in x[i]) / 9
        for j in range(9):
            ref = (x[i, j] - m) / math.sqrt(v + 1e-5) * gam[j] + bet[j]
            assert abs(ref - y[i, j]) < 1e-12


def test_layernorm_backward_finite_difference():
    g = rng(19)
    x = g.standard_normal((3, 5))
    gam, bet = g.standard_normal(5), g.standard_normal(5)
    R = g.standard_normal((3, 5))
    _, mu, rs = O.layernorm_forward(x, gam, bet)
    dx, dg, db = O.layernorm_backward(x, gam, mu, rs, R)
    _fd_check(lambda: np.sum(R * O.layernorm_forward(x, gam, bet)[0]), [x, gam, bet], [dx, dg, db])


# ---------------------------------------------------------------- stacked model

def test_gpt_backward_finite_difference():
    g = rng(20)
    V, H, nh, d, L, b, s, n = 11, 8, 2, 4, 2, 1, 3, 2
    ids = g.integers(0, V, b * s)
    E = g.standard_normal((V, H)) * 0.5
    layers = []
    for _ in range(L):
        layers.append({k: g.standard_normal(sh) * 0.3 for k, sh in
                       [("WQ", (H, H)), ("WK", (H, H)), ("WV", (H, H)), ("WO", (H, H)),
                        ("A", (H, 4 * H)), ("B", (4 * H, H))]})
        layers[-1].update(g1=1 + 0.1 * g.standard_normal(H), b1=0.1 * g.standard_normal(H),
                          g2=1 + 0.1 * g.standard_normal(H), b2=0.1 * g.standard_normal(H))
    R = [g.standard_normal((b * s, O.partition(V, n, r)[1])) for r in range(n)]

    def loss():
        lg, _ = O.gpt_forward(ids, E, layers, b, s, nh, d, n)
        return sum(np.sum(R[r] * lg[r]) for r in range(n))

    lg, cache = O.gpt_forward(ids, E, layers, b, s, nh, d, n)
    dE, grads = O.gpt_backward(ids, E, layers, cache, R, b, s, nh, d, n)
    # spot-check a subset of entries of every parameter (all of E)
    _fd_check(loss, [E], [dE], tol=2e-6)
    for li in range(L):
        for key in ("WQ", "WO", "A", "B", "g1", "b2"):
            a, gr = layers[li][key], grads[li][key]
            for idx in [tuple(0 for _ in a.shape), tuple(x - 1 for x in a.shape)]:
                old = a[idx]
                a[idx] = old + 1e-6
                fp = loss()
                a[idx] = old - 1e-6
                fm = loss()
                a[idx] = old
                fd = (fp - fm) / 2e-6
                assert abs(fd - gr[idx]) <= 2e-6 * max(1.0, abs(fd)), (li, key, idx)


# ---------------------------------------------------------------- vocab-parallel cross entropy

def _ce_shards(x, starts_counts):
    return [x[:, s:s + c] for s, c in starts_counts]


def test_ce_page_masking_layout():
    """The pages' 10-word, two-shard, three-token layout: the -1 of each
    token's gradient lands on the shard that owns its target (the picks of
    that shard), and uniform logits give loss log 10 for every token."""
    gx = golden("ce_masking_example.json")
    V, sc, tg = gx["vocab"], gx["shards"], np.array(gx["targets"])
    x = np.full((len(tg), V), 0.75)
    loss, sm, _, _ = O.vocab_ce_forward(_ce_shards(x, sc), tg, [s for s, _ in sc])
    assert np.allclose(loss, math.log(V), rtol=0, atol=1e-15)
    grads = O.vocab_ce_backward(sm, tg, [s for s, _ in sc], np.ones(len(tg)))
    for r, (s, c) in enumerate(sc):
        has_minus_one = (grads[r] < 0).any(axis=1)
        assert has_minus_one.tolist() == gx["picks_per_shard"][r]


@pytest.mark.parametrize("V,n", [(7, 2), (50, 3), (13, 1)])
def test_ce_uniform_logits_closed_form(V, n):
    """All logits equal: loss = log V and gradient 1/V - onehot(target)."""
    g = rng(31)
    T = 6
    tg = g.integers(0, V, T)
    sc = [O.partition(V, n, r) for r in range(n)]
    x = np.full((T, V), -3.25)
    loss, sm, _, _ = O.vocab_ce_forward(_ce_shards(x, sc), tg, [s for s, _ in sc])
    assert np.allclose(loss, math.log(V), rtol=0, atol=1e-14)
    grad = np.concatenate(O.vocab_ce_backward(sm, tg, [s for s, _ in sc], np.ones(T)), axis=1)
    want = np.full((T, V), 1.0 / V)
    want[np.arange(T), tg] -= 1.0
    assert np.allclose(grad, want, rtol=0, atol=1e-15)


def test_ce_row_shift_invariance():
    """Adding a constant to every logit of a row changes neither the loss nor
    the gradient."""
    g = rng(32)
    T, V, n = 5, 23, 3
    sc = [O.partition(V, n, r) for r in range(n)]
    x = g.standard_normal((T, V)) * 4
    tg = g.integers(0, V, T)
    c = g.standard_normal(T)[:, None] * 100
    st = [s for s, _ in sc]
    l0, s0, _, _ = O.vocab_ce_forward(_ce_shards(x, sc), tg, st)
    l1, s1, _, _ = O.vocab_ce_forward(_ce_shards(x + c, sc), tg, st)
    assert np.allclose(l0, l1, rtol=1e-12, atol=1e-12)
    for a, b in zip(s0, s1):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("scale", [1.0, 30.0, 3000.0])
def test_ce_matches_library_logsumexp(scale):
    """loss = logsumexp(row) - row[target], with scipy's logsumexp (the oracle
    does not use it), including logits large enough to overflow exp."""
    from scipy.special import logsumexp
    g = rng(33)
    T, V, n = 9, 101, 2
    sc = [O.partition(V, n, r) for r in range(n)]
    x = g.standard_normal((T, V)) * scale
    tg = g.integers(0, V, T)
    loss, _, _, _ = O.vocab_ce_forward(_ce_shards(x, sc), tg, [s for s, _ in sc])
    want = logsumexp(x, axis=1) - x[np.arange(T), tg]
    assert np.allclose(loss, want, rtol=1e-12, atol=1e-12 * scale)


def test_ce_bruteforce_loop():
    """Scalar loops with math.exp / math.log on small logits (no shift
    needed): loss = log(sum_j exp x_j) - x_target."""
    g = rng(34)
    T, V, n = 4, 9, 2
    sc = [O.partition(V, n, r) for r in range(n)]
    x = g.standard_normal((T, V))
    tg = g.integers(0, V, T)
    loss, _, _, _ = O.vocab_ce_forward(_ce_shards(x, sc), tg, [s for s, _ in sc])
    for t in range(T):
        s = math.fsum(math.exp(float(v)) for v in x[t])
        assert abs(loss[t] - (math.log(s) - float(x[t, tg[t]]))) <= 1e-13


def test_ce_target_outside_every_shard():
    """A target no shard owns picks 0 everywhere (the page's mask), and 0 is
    the max-shifted value, so the loss is logsumexp(row) - max(row); the
    gradient is the softmax alone."""
    from scipy.special import logsumexp, softmax
    g = rng(35)
    T, V = 3, 12
    sc = [O.partition(V, 2, r) for r in range(2)]
    x = g.standard_normal((T, V))
    tg = np.array([V, -1, V + 5])
    loss, sm, _, _ = O.vocab_ce_forward(_ce_shards(x, sc), tg, [s for s, _ in sc])
    assert np.allclose(loss, logsumexp(x, axis=1) - x.max(axis=1), rtol=1e-13)
    grad = np.concatenate(O.vocab_ce_backward(sm, tg, [s for s, _ in sc], np.ones(T)), axis=1)
    assert np.allclose(grad, softmax(x, axis=1), rtol=1e-12, atol=1e-15)


def test_ce_backward_finite_difference_and_zero_row_sums():
    g = rng(36)
    T, V, n = 3, 11, 2
    sc = [O.partition(V, n, r) for r in range(n)]
    st = [s for s, _ in sc]
    x = g.standard_normal((T, V)) * 2
    tg = g.integers(0, V, T)
    w = g.standard_normal(T)
    _, sm, _, _ = O.vocab_ce_forward(_ce_shards(x, sc), tg, st)
    grad = np.concatenate(O.vocab_ce_backward(sm, tg, st, w), axis=1)
    _fd_check(lambda: float(np.sum(w * O.vocab_ce_forward(_ce_shards(x, sc), tg, st)[0])), [x], [grad],
              h=1e-6, tol=1e-7)
    assert np.allclose(grad.sum(axis=1), 0.0, atol=1e-14)


# ---------------------------------------------------------------- column / row parallel linear

def _linear_loop(X, A, b):
    M, K = X.shape
    N = A.shape[1]
    Y = np.zeros((M, N))
    for m in range(M):
        for j in range(N):
            Y[m, j] = math.fsum(float(X[m, k]) * float(A[k, j]) for k in range(K)) + (b[j] if b is not None else 0.0)
    return Y


@pytest.mark.parametrize("n", [1, 2, 3])
def test_column_linear_bruteforce_gather_and_skip_bias(n):
    g = rng(40)
    X, A, b = g.standard_normal((5, 7)), g.standard_normal((7, 10)), g.standard_normal(10)
    outs, Y = O.column_linear_forward(X, A, b, n)
    assert np.allclose(Y, _linear_loop(X, A, b), rtol=1e-13, atol=1e-13)
    for r in range(n):
        s, c = O.partition(10, n, r)
        assert np.allclose(outs[r], _linear_loop(X, A[:, s:s + c], b[s:s + c]), rtol=1e-13, atol=1e-13)
    outs2, none = O.column_linear_forward(X, A, b, n, gather_output=False, skip_bias_add=True)
    assert none is None
    assert np.allclose(np.concatenate(outs2, axis=1), _linear_loop(X, A, None), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("n", [1, 2, 4])
def test_row_linear_bruteforce_scatter_parallel_and_bias_once(n):
    g = rng(41)
    X, B, b = g.standard_normal((4, 9)), g.standard_normal((9, 6)), g.standard_normal(6)
    _, Y = O.row_linear_forward(X, B, b, n)
    assert np.allclose(Y, _linear_loop(X, B, b), rtol=1e-13, atol=1e-13)
    Xs = [X[:, s:s + c] for s, c in (O.partition(9, n, r) for r in range(n))]
    parts, Y2 = O.row_linear_forward(Xs, B, b, n, input_is_parallel=True)
    assert np.allclose(Y2, Y, rtol=1e-13, atol=1e-13)
    _, Y3 = O.row_linear_forward(X, B, b, n, skip_bias_add=True)
    assert np.allclose(Y3, _linear_loop(X, B, None), rtol=1e-13, atol=1e-13)


def test_column_then_row_is_the_unsharded_two_layer_product():
    """Column split feeding the row split without a gather (the MLP pattern,
    without the activation): sum_r (X A_r + b_r) B_r + c = (X A + b) B + c."""
    g = rng(42)
    n = 2
    X, A, b, B, c = (g.standard_normal((3, 5)), g.standard_normal((5, 8)), g.standard_normal(8),
                     g.standard_normal((8, 4)), g.standard_normal(4))
    outs, _ = O.column_linear_forward(X, A, b, n, gather_output=False)
    _, Y = O.row_linear_forward(outs, B, c, n, input_is_parallel=True)
    assert np.allclose(Y, (X @ A + b) @ B + c, rtol=1e-12, atol=1e-12)


def test_linear_backward_finite_difference():
    g = rng(43)
    n = 2
    X, A, b = g.standard_normal((3, 4)), g.standard_normal((4, 6)), g.standard_normal(6)
    B, c = g.standard_normal((6, 5)), g.standard_normal(5)
    R = g.standard_normal((3, 5))

    def loss():
        outs, _ = O.column_linear_forward(X, A, b, n, gather_output=False)
        return float(np.sum(R * O.row_linear_forward(outs, B, c, n, input_is_parallel=True)[1]))

    outs, _ = O.column_linear_forward(X, A, b, n, gather_output=False)
    dH, dBs, dcs = [], [], []
    for r in range(n):
        dHr, dBr, dc = O.row_linear_backward(outs[r], O.split_rows(B, n, r), R)
        dH.append(dHr); dBs.append(dBr); dcs.append(dc)
    dX = np.zeros_like(X); dAs, dbs = [], []
    for r in range(n):
        dXr, dAr, dbr = O.column_linear_backward(X, O.split_columns(A, n, r), dH[r])
        dX += dXr; dAs.append(dAr); dbs.append(dbr)
    _fd_check(loss, [X, A, b, B, c],
              [dX, np.concatenate(dAs, axis=1), np.concatenate(dbs), np.concatenate(dBs, axis=0), dcs[0]],
              h=1e-6, tol=1e-6)
    assert all(np.array_equal(d, dcs[0]) for d in dcs)   # the replicated bias: same gradient on every shard


# ---------------------------------------------------------------- sequence parallelism

@pytest.mark.parametrize("M,n", [(7, 2), (10, 3), (4, 4)])
def test_sp_reduce_scatter_bruteforce_and_all_gather_is_the_all_reduce(M, n):
    g = rng(50)
    H = 5
    parts = [g.standard_normal((M, H)) for _ in range(n)]
    res = [g.standard_normal((O.partition(M, n, r)[1], H)) for r in range(n)]
    sl = O.sp_reduce_scatter(parts, n, res)
    for r in range(n):
        s, c = O.partition(M, n, r)
        for i in range(c):
            for j in range(H):
                want = res[r][i, j] + math.fsum(float(p[s + i, j]) for p in parts)
                assert abs(sl[r][i, j] - want) <= 1e-13
    # without the residual, gathering the scattered sums gives the all-reduce
    assert np.allclose(O.sp_all_gather(O.sp_reduce_scatter(parts, n)), O.shard_reduce(parts), rtol=0, atol=1e-14)
    # the gather inverts the row split
    x = g.standard_normal((M, H))
    assert np.array_equal(O.sp_all_gather([x[s:s + c] for s, c in (O.partition(M, n, r) for r in range(n))]), x)


def test_sp_layernorm_grads_summed_equal_unsharded_and_fd():
    g = rng(51)
    M, H, n = 9, 6, 3
    x, dy = g.standard_normal((M, H)), g.standard_normal((M, H))
    gamma, beta = 1 + 0.1 * g.standard_normal(H), 0.1 * g.standard_normal(H)
    _, mu, rs = O.layernorm_forward(x, gamma, beta)
    dx, dg, db = O.layernorm_backward(x, gamma, mu, rs, dy)
    rows = [O.partition(M, n, r) for r in range(n)]
    dxs, dg2, db2 = O.sp_layernorm_param_grads([x[s:s + c] for s, c in rows], gamma,
                                               [mu[s:s + c] for s, c in rows], [rs[s:s + c] for s, c in rows],
                                               [dy[s:s + c] for s, c in rows])
    assert np.allclose(np.concatenate(dxs), dx, rtol=1e-13, atol=1e-13)
    assert np.allclose(dg2, dg, rtol=1e-13, atol=1e-13) and np.allclose(db2, db, rtol=1e-13, atol=1e-13)

    def loss():
        return float(np.sum(dy * O.layernorm_forward(x, gamma, beta)[0]))
    _fd_check(loss, [gamma, beta], [dg2, db2], h=1e-6, tol=1e-6)


# ---------------------------------------------------------------- full embedding, dropout generator

def test_philox_known_answer_vectors():
    for case in golden("philox4x32_10_kat.json")["cases"]:
        ctr = [int(x, 16) for x in case["ctr"]]
        key = [int(x, 16) for x in case["key"]]
        out = O.philox4x32_10(np.array([ctr], dtype=np.uint64), key)[0]
        assert [int(x) for x in out] == [int(x, 16) for x in case["out"]]


def test_dropout_keep_mapping_and_rate():
    seed = 0x1234_5678_9ABC_DEF0
    n = 10
    keep = O.dropout_keep(n, 0.5, seed)
    thr = int(float(np.float32(0.5)) * 2 ** 32)
    for e in range(n):      # element e uses word e % 4 of the block e // 4
        w = O.philox4x32_10(np.array([[e // 4, 0, 0, 0]], dtype=np.uint64),
                            (seed & 0xFFFFFFFF, seed >> 32))[0][e % 4]
        assert keep[e] == (int(w) >= thr)
    assert O.dropout_keep(1000, 0.0, seed).all()
    for p in (0.1, 0.5, 0.9):
        n = 200_000
        k = O.dropout_keep(n, p, 77).mean()
        assert abs(k - (1 - p)) <= 5 * math.sqrt(p * (1 - p) / n)


def test_dropout_keep_at_high_counter_word_and_sampled_rows():
    """Element indices past 2^34 put e // 4 above 2^32, so the counter's
    second word is nonzero: each decision is checked against a direct call of
    the generator at counter (e // 4 low, e // 4 high, 0, 0).  Sampled rows
    of the full embedding (``tokens``) take the full call's rows and mask."""
    seed = 0xFEDC_BA98_7654_3210
    key = (seed & 0xFFFFFFFF, seed >> 32)
    elems = np.array([2 ** 34 + 1, 2 ** 34 + 7, 3 * 2 ** 35 + 2, 2 ** 40 + 3, 5], dtype=np.uint64)
    thr = int(float(np.float32(0.3)) * 2 ** 32)
    keep = O.dropout_keep_at(elems, 0.3, seed)
    for k, e in zip(keep, elems.tolist()):
        b = e // 4
        w = O.philox4x32_10(np.array([[b & 0xFFFFFFFF, b >> 32, 0, 0]], dtype=np.uint64), key)[0][e % 4]
        assert k == (int(w) >= thr)
    assert np.array_equal(O.dropout_keep_at(np.arange(40, dtype=np.uint64), 0.3, seed), O.dropout_keep(40, 0.3, seed))
    g = rng(62)
    T, H, P = 9, 8, 5
    parts = [g.standard_normal((T, H)) for _ in range(2)]
    PE = g.standard_normal((P, H))
    pos = np.arange(T) % P
    full, kf = O.embedding_forward(parts, PE, pos, 0.4, 3)
    rows = np.array([7, 2, 8])
    sub, ks = O.embedding_forward([x[rows] for x in parts], PE, pos[rows], 0.4, 3, tokens=rows)
    assert np.array_equal(sub, full[rows]) and np.array_equal(ks, kf[rows])


def test_embedding_forward_closed_form_and_masking():
    g = rng(60)
    T, H, V, P, n = 6, 4, 10, 5, 2
    E = g.standard_normal((V, H))
    PE, TE = g.standard_normal((P, H)), g.standard_normal((3, H))
    ids = np.array([0, 3, 9, 5, 2, 7])
    pos = np.array([0, 1, 2, 3, 4, 7])      # 7 lies outside the position table: a zero row
    tt = np.array([0, 1, 2, 1, 0, 1])
    parts = [O.vocab_embed_forward(ids, E[s:s + c], s) for s, c in (O.partition(V, n, r) for r in range(n))]
    out, keep = O.embedding_forward(parts, PE, pos, 0.0, 5, TE, tt)
    assert keep.all()
    for t in range(T):
        for h in range(H):
            want = E[ids[t], h] + (PE[pos[t], h] if pos[t] < P else 0.0) + TE[tt[t], h]
            assert abs(out[t, h] - want) <= 1e-14
    out2, keep2 = O.embedding_forward(parts, PE, pos, 0.3, 5, TE, tt)
    assert np.allclose(out2[keep2], (out / 0.7)[keep2], rtol=1e-6) and np.all(out2[~keep2] == 0)


def test_embedding_backward_finite_difference():
    g = rng(61)
    T, H, V, P, n, p = 5, 3, 8, 6, 2, 0.25
    E, PE, TE = g.standard_normal((V, H)), g.standard_normal((P, H)), g.standard_normal((2, H))
    ids, pos, tt = g.integers(0, V, T), g.integers(0, P, T), g.integers(0, 2, T)
    R = g.standard_normal((T, H))
    sc = [O.partition(V, n, r) for r in range(n)]

    def loss():
        parts = [O.vocab_embed_forward(ids, E[s:s + c], s) for s, c in sc]
        return float(np.sum(R * O.embedding_forward(parts, PE, pos, p, 9, TE, tt)[0]))
    parts = [O.vocab_embed_forward(ids, E[s:s + c], s) for s, c in sc]
    _, keep = O.embedding_forward(parts, PE, pos, p, 9, TE, tt)
    dX, dPE, dTE = O.embedding_backward(R, keep, p, pos, P, tt, 2)
    dE = np.concatenate([O.vocab_embed_backward(ids, dX, s, c) for s, c in sc])
    _fd_check(loss, [E, PE, TE], [dE, dPE, dTE], h=1e-6, tol=1e-6)
