"""GPU parity at the full workload sizes, in the launch configurations the
benchmark times (the same shapes select the same tiles and grids).

* Layer shape (b=1, s=2048, H=4096, 8 heads of 512, 4H MLP, N=2): every
  output of both shards' attention and MLP forward and backward against the
  oracle computed in full (about 1.5 TFLOP of fp64 on the host).
* Tied-embedding shape (V=50257 split 25129/25128, H=4096, T=8*2048): the
  embedding gather and shard sum bit-exact in full; the input-side gradient
  in full; logits and their two gradients on sampled rows, which the oracle
  computes one by one.
"""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpuutil import BF16_TOL, empty, ids_dev, rel_err, say, to_dev, to_f64, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tp():
    import megatron_tensor_transformer_columnparallel_amd as tp
    return tp


def _cols(t, a, b):
    return synth.Tensor(np.ascontiguousarray(t.store[:, a:b]), t.dtype)


def _rows(t, a, b):
    return synth.Tensor(np.ascontiguousarray(t.store[a:b]), t.dtype)


@pytest.fixture(scope="module")
def layer_inputs():
    cfg = synth.WORKLOADS[3]
    M = cfg["b"] * cfg["s"]
    mlp = synth.mlp_inputs(3, M, cfg["h"], cfg["f"], "bf16")
    att = synth.attn_inputs(3, M, cfg["h"], cfg["heads"], cfg["d"], "bf16")
    return cfg, mlp, att


def test_layer_mlp_full_size(tp, layer_inputs):
    cfg, inp, _ = layer_inputs
    M, h, f, n = cfg["b"] * cfg["s"], cfg["h"], cfg["f"], cfg["n"]
    X, dZ = inp["X"], inp["dZ"]
    Xf, dZf = X.f64, dZ.f64
    for r in range(n):
        s, c = O.partition(f, n, r)
        say(f"full-size MLP shard {r}: M={M} h={h} f_i={c}")
        A_r, B_r = _cols(inp["A"], s, s + c), _rows(inp["B"], s, s + c)
        dX_, dA_, dB_ = to_dev(X), to_dev(A_r), to_dev(B_r)
        P, H, Z = empty((M, c), torch.bfloat16), empty((M, c), torch.bfloat16), empty((M, h), torch.bfloat16)
        tp.tp_mlp_fwd(dX_, dA_, dB_, P, H, Z)
        gX, gA, gB = empty((M, h), torch.bfloat16), empty((h, c), torch.bfloat16), empty((c, h), torch.bfloat16)
        ws = workspace(tp.tp_mlp_bwd_workspace(torch.bfloat16, M, h, c))
        tp.tp_mlp_bwd(dX_, dA_, dB_, P, H, to_dev(dZ), gX, gA, gB, ws)
        P_ref, H_ref, Z_ref = O.mlp_forward(Xf, A_r.f64, B_r.f64)
        dX_ref, dA_ref, dB_ref = O.mlp_backward(Xf, A_r.f64, B_r.f64, P_ref, dZf)
        for key, got, ref in [("P", P, P_ref), ("H", H, H_ref), ("Z", Z, Z_ref), ("dX", gX, dX_ref),
                              ("dA", gA, dA_ref), ("dB", gB, dB_ref)]:
            e = rel_err(to_f64(got), ref)
            print(f"  {key}: max|err|/max|ref| = {e:.2e}", flush=True)
            assert e <= BF16_TOL, (key, r, e)


def test_layer_attention_full_size(tp, layer_inputs):
    cfg, _, inp = layer_inputs
    b, sq, h, heads, d, n = cfg["b"], cfg["s"], cfg["h"], cfg["heads"], cfg["d"], cfg["n"]
    M = b * sq
    X, dZ = inp["X"], inp["dZ"]
    Xf = X.f64
    for r in range(n):
        hs0, hs = O.partition(heads, n, r)
        cs = slice(hs0 * d, (hs0 + hs) * d)
        say(f"full-size attention shard {r}: b={b} sq={sq} h={h} hs={hs} d={d} causal")
        Wqkv = synth.Tensor(np.ascontiguousarray(np.concatenate(
            [inp["WQ"].store[:, cs], inp["WK"].store[:, cs], inp["WV"].store[:, cs]], axis=1)), "bf16")
        Wo = synth.Tensor(np.ascontiguousarray(inp["WO"].store[cs, :]), "bf16")
        w = hs * d
        dXd, dW, dWo_ = to_dev(X), to_dev(Wqkv), to_dev(Wo)
        QKV, Ob = empty((M, 3 * w), torch.bfloat16), empty((M, w), torch.bfloat16)
        lse, Z = empty((b * hs * sq,), torch.float32), empty((M, h), torch.bfloat16)
        tp.tp_attn_fwd(dXd, dW, dWo_, QKV, Ob, lse, Z, b, sq, hs, d, True)
        gX, gW, gWo = empty((M, h), torch.bfloat16), empty(Wqkv.shape, torch.bfloat16), empty(Wo.shape, torch.bfloat16)
        ws = workspace(tp.tp_attn_bwd_workspace(torch.bfloat16, b, sq, h, hs, d))
        tp.tp_attn_bwd(dXd, dW, dWo_, QKV, Ob, lse, to_dev(dZ), gX, gW, gWo, ws, b, sq, hs, d, True)
        QKV_r, O_r, lse_r, Z_r = O.attention_layer_forward(Xf, Wqkv.f64, Wo.f64, b, sq, hs, d, True)
        dX_r, dW_r, dWo_r = O.attention_layer_backward(Xf, Wqkv.f64, Wo.f64, QKV_r, O_r, dZ.f64, b, sq, hs, d, True)
        for key, got, ref in [("QKV", QKV, QKV_r), ("O", Ob, O_r), ("Z", Z, Z_r), ("dX", gX, dX_r),
                              ("dWqkv", gW, dW_r), ("dWo", gWo, dWo_r)]:
            e = rel_err(to_f64(got), ref)
            print(f"  {key}: max|err|/max|ref| = {e:.2e}", flush=True)
            assert e <= BF16_TOL, (key, r, e)
        assert np.max(np.abs(to_f64(lse) - lse_r.reshape(-1))) <= 1e-2 * np.max(np.abs(lse_r))


@pytest.fixture(scope="module")
def embed_inputs():
    cfg = synth.WORKLOADS[4]
    T = cfg["b"] * cfg["s"]
    inp = synth.embed_inputs(4, T, cfg["V"], cfg["H"], "bf16", 0.02)
    return cfg, T, inp


def test_embedding_full_size_bit_exact(tp, embed_inputs):
    cfg, T, inp = embed_inputs
    V, H, n = cfg["V"], cfg["H"], cfg["n"]
    ids = ids_dev(inp["ids"])
    parts = []
    for r in range(n):
        s, c = O.partition(V, n, r)
        say(f"full-size vocab_embed_fwd shard {r}: T={T} rows={c} H={H}")
        E_r = _rows(inp["E"], s, s + c)
        Y = empty((T, H), torch.bfloat16)
        tp.vocab_embed_fwd(ids, to_dev(E_r), Y, s)
        ref = O.vocab_embed_forward(inp["ids"], E_r.f64, s)
        assert np.array_equal(to_f64(Y), ref)
        parts.append(Y)
    out = empty((T, H), torch.bfloat16)
    tp.shard_reduce(parts, out)
    assert np.array_equal(to_f64(out), O.round_to_bf16(inp["E"].f64[inp["ids"]]))


def test_tied_logits_full_size_sampled(tp, embed_inputs):
    cfg, T, inp = embed_inputs
    V, H, n = cfg["V"], cfg["H"], cfg["n"]
    X, E, dY = inp["X"], inp["E"], inp["dY"]
    Xf, dYf = X.f64, dY.f64
    g = np.random.default_rng(4444)
    rows = np.sort(g.choice(T, 48, replace=False))
    for r in range(n):
        s, c = O.partition(V, n, r)
        say(f"full-size tied_logits shard {r}: T={T} H={H} v_rows={c}")
        E_r = _rows(E, s, s + c)
        ldl = (c + 7) // 8 * 8
        Lbuf = empty((T, ldl), torch.bfloat16)
        dEr, dXr = to_dev(E_r), to_dev(X)
        tp.tied_logits(dXr, dEr, Lbuf[:, :c])
        dL = synth.logit_grad(4, r, T, c, "bf16")
        dLbuf = empty((T, ldl), torch.bfloat16)
        dLbuf[:, :c] = to_dev(dL)
        gX = empty((T, H), torch.bfloat16)
        gE = empty((c, H), torch.float32)
        tp.tied_logits_bwd(dXr, dEr, dLbuf[:, :c], gX, gE)
        vrows = np.sort(g.choice(c, 48, replace=False))
        dLf = dL.f64
        L_ref = O.tied_logits(Xf[rows], E_r.f64)
        assert rel_err(to_f64(Lbuf[rows, :c]), L_ref) <= BF16_TOL
        dX_ref, _ = O.tied_logits_backward(Xf[rows], E_r.f64, dLf[rows])
        assert rel_err(to_f64(gX[rows]), dX_ref) <= BF16_TOL
        # sampled rows j of dE_r = dL_r^T X, each the oracle's product on column j of dL_r
        dE_ref = np.stack([O.tied_logits_backward(Xf, E_r.f64[j:j + 1], dLf[:, j:j + 1])[1][0] for j in vrows])
        assert rel_err(to_f64(gE[vrows]), dE_ref) <= 1e-3
        # tied total: add the input-side gradient and check sampled rows and
        # the column-sum identity over the whole shard
        ws = workspace(tp.vocab_embed_bwd_workspace(T, c))
        tp.vocab_embed_bwd(ids_dev(inp["ids"]), to_dev(dY), gE, s, ws)
        tot = to_f64(gE)
        for k, j in enumerate(vrows[:16]):
            ref = dE_ref[k] + O.vocab_embed_backward(inp["ids"], dYf, s + j, 1)[0]
            assert rel_err(tot[j], ref) <= 1e-3
        # column sums over the whole shard: sum_j (dL^T X)[j] = rowsum(dL) X, plus the in-range dY rows
        inr = (inp["ids"] >= s) & (inp["ids"] < s + c)
        colsum_ref = dLf.sum(axis=1) @ Xf + dYf[inr].sum(axis=0)
        assert rel_err(tot.sum(axis=0), colsum_ref) <= 1e-3
