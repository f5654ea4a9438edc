"""GPU parity: attention shard forward/backward and LayerNorm against the fp64
oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpuutil import BF16_TOL, F32_TOL, empty, raw_bits, rel_err, say, to_dev, to_f64, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tp():
    import megatron_tensor_transformer_columnparallel_amd as tp
    return tp


def _qkv_shard(inp, n, r, d):
    WQ, WK, WV = inp["WQ"].store, inp["WK"].store, inp["WV"].store
    nh = WQ.shape[1] // d
    hs0, hsn = O.partition(nh, n, r)
    c = slice(hs0 * d, (hs0 + hsn) * d)
    Wqkv = synth.Tensor(np.ascontiguousarray(np.concatenate([WQ[:, c], WK[:, c], WV[:, c]], axis=1)), "bf16")
    Wo = synth.Tensor(np.ascontiguousarray(inp["WO"].store[c, :]), "bf16")
    return Wqkv, Wo, hsn


def run_attn_shard(tp, X, Wqkv, Wo, dZ, b, sq, hs, d, causal):
    M, h = X.shape
    w = hs * d
    dX_, dW, dWo_ = to_dev(X), to_dev(Wqkv), to_dev(Wo)
    QKV, Ob = empty((M, 3 * w), torch.bfloat16), empty((M, w), torch.bfloat16)
    lse, Z = empty((b * hs * sq,), torch.float32), empty((M, h), torch.bfloat16)
    tp.tp_attn_fwd(dX_, dW, dWo_, QKV, Ob, lse, Z, b, sq, hs, d, causal)
    gX, gW, gWo = empty((M, h), torch.bfloat16), empty(Wqkv.shape, torch.bfloat16), empty(Wo.shape, torch.bfloat16)
    ws = workspace(tp.tp_attn_bwd_workspace(torch.bfloat16, b, sq, h, hs, d))
    tp.tp_attn_bwd(dX_, dW, dWo_, QKV, Ob, lse, to_dev(dZ), gX, gW, gWo, ws, b, sq, hs, d, causal)
    return dict(QKV=QKV, O=Ob, lse=lse, Z=Z, dX=gX, dWqkv=gW, dWo=gWo)


@pytest.mark.parametrize("w,b,sq,h,heads,d,n,causal", [
    (71, 2, 100, 256, 4, 64, 2, True),     # ragged sequence, 2 heads per shard
    (72, 1, 70, 256, 2, 128, 2, False),    # non-causal
    (73, 1, 80, 512, 2, 512, 2, True),     # head dim 512 (the page-1 shape's head size)
    (74, 3, 33, 128, 2, 256, 1, True),     # single shard, batch 3
    (75, 1, 1, 128, 2, 64, 2, True),       # one position: O = V
    (78, 1, 300, 128, 2, 64, 2, True),     # peaked softmax (weights x 8): large score range per row
    (79, 1, 520, 256, 4, 96, 2, True),     # head dim 96; rows past two 256-wide probability pads
    (80, 2, 261, 128, 2, 40, 1, True),     # head dim 40, sq not a multiple of 8 (padded score rows)
])
def test_attention_shards_match_oracle(tp, w, b, sq, h, heads, d, n, causal):
    say(f"tp_attn fwd+bwd b={b} sq={sq} h={h} heads={heads} d={d} N={n} causal={causal}")
    inp = synth.attn_inputs(w, b * sq, h, heads, d, "bf16")
    if w == 78:   # sharpen the scores: Q and K weights scaled by 8 (exact in bf16)
        for k in ("WQ", "WK"):
            inp[k] = synth.Tensor(synth.to_bf16_bits(synth.bf16_bits_to_f32(inp[k].store) * 8.0), "bf16")
    X, dZ = inp["X"], inp["dZ"]
    Zs, dXs = [], []
    for r in range(n):
        Wqkv, Wo, hs = _qkv_shard(inp, n, r, d)
        got = run_attn_shard(tp, X, Wqkv, Wo, dZ, b, sq, hs, d, causal)
        QKV_r, O_r, lse_r, Z_r = O.attention_layer_forward(X.f64, Wqkv.f64, Wo.f64, b, sq, hs, d, causal)
        dX_r, dW_r, dWo_r = O.attention_layer_backward(X.f64, Wqkv.f64, Wo.f64, QKV_r, O_r, dZ.f64, b, sq, hs, d,
                                                       causal)
        for key, ref in [("QKV", QKV_r), ("O", O_r), ("Z", Z_r), ("dX", dX_r), ("dWqkv", dW_r), ("dWo", dWo_r)]:
            e = rel_err(to_f64(got[key]), ref)
            assert e <= BF16_TOL, (key, r, e)
        # lse is fp32 on both sides of a bf16 S: absolute error small against its size
        assert np.max(np.abs(to_f64(got["lse"]) - lse_r.reshape(-1))) <= 1e-2 * max(1.0, np.max(np.abs(lse_r)))
        Zs.append(got["Z"])
        dXs.append(got["dX"])
    _, Zsum_ref = O.tp_attention_forward(X.f64, inp["WQ"].f64, inp["WK"].f64, inp["WV"].f64, inp["WO"].f64,
                                         b, sq, heads, d, n, causal)
    Zsum = empty(Zs[0].shape, torch.bfloat16)
    tp.shard_reduce(Zs, Zsum)
    assert rel_err(to_f64(Zsum), Zsum_ref) <= BF16_TOL


def test_attention_backward_deterministic(tp):
    say("tp_attn_bwd determinism b=1 sq=200 d=128")
    b, sq, h, heads, d = 1, 200, 256, 2, 128
    inp = synth.attn_inputs(76, b * sq, h, heads, d, "bf16")
    Wqkv, Wo, hs = _qkv_shard(inp, 1, 0, d)
    a = run_attn_shard(tp, inp["X"], Wqkv, Wo, inp["dZ"], b, sq, hs, d, True)
    c = run_attn_shard(tp, inp["X"], Wqkv, Wo, inp["dZ"], b, sq, hs, d, True)
    for key in ("Z", "dX", "dWqkv", "dWo"):
        assert np.array_equal(raw_bits(a[key]), raw_bits(c[key])), key


# ------------------------------------------------------------------ LayerNorm

@pytest.mark.parametrize("M,H,dt,ydt", [(5, 64, "f32", "f32"), (300, 4096, "bf16", "bf16"), (33, 8192, "f32", "f32"),
                                        (17, 136, "bf16", "bf16"), (64, 4096, "f32", "bf16"), (9, 72, "bf16", "f32"),
                                        (2048, 4096, "f32", "f32"), (13, 4096, "f32", "f32"), (3, 4096, "bf16", "f32")])
def test_layernorm_matches_oracle(tp, M, H, dt, ydt):
    """x and dx of dtype dt, y and dy of dtype ydt (fp32 residual stream <-> bf16 sublayer)."""
    say(f"layernorm fwd+bwd M={M} H={H} x {dt} y {ydt}")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    ytdt = torch.bfloat16 if ydt == "bf16" else torch.float32
    tol = BF16_TOL if "bf16" in (dt, ydt) else F32_TOL
    x = synth.make(77, 0, (M, H), 2.0, dt)
    dy = synth.make(77, 1, (M, H), 1.0, ydt)
    g = synth.Tensor(1.0 + 0.1 * synth.normal(77, 2, (H,)), "f32")
    bt = synth.Tensor(0.1 * synth.normal(77, 3, (H,)), "f32")
    y, mean, rstd = empty((M, H), ytdt), empty((M,), torch.float32), empty((M,), torch.float32)
    dg, db_ = to_dev(g), to_dev(bt)
    dx_in = to_dev(x)
    tp.layernorm_fwd(dx_in, dg, db_, y, mean, rstd, 1e-5)
    y_ref, mu_ref, rs_ref = O.layernorm_forward(x.f64, g.f64, bt.f64, 1e-5)
    assert rel_err(to_f64(y), y_ref) <= tol
    assert rel_err(to_f64(rstd), rs_ref) <= 1e-5
    dx, dgam, dbet = empty((M, H), tdt), empty((H,), torch.float32), empty((H,), torch.float32)
    ws = workspace(tp.layernorm_bwd_workspace(M, H))
    tp.layernorm_bwd(dx_in, dg, mean, rstd, to_dev(dy), dx, dgam, dbet, ws)
    dx_ref, dg_ref, db_ref = O.layernorm_backward(x.f64, g.f64, mu_ref, rs_ref, dy.f64)
    assert rel_err(to_f64(dx), dx_ref) <= tol
    assert rel_err(to_f64(dgam), dg_ref) <= (F32_TOL if tol == F32_TOL else 1e-3)
    assert rel_err(to_f64(dbet), db_ref) <= 1e-5


@pytest.mark.parametrize("M,H,dt,copy", [(2048, 4096, "f32", True), (300, 4096, "bf16", True), (13, 4096, "f32", False),
                                         (37, 136, "f32", True)])
def test_layernorm_bwd_residual_matches_oracle(tp, M, H, dt, copy):
    """out = res + LayerNorm gradient (fp32), optional bf16 copy; x and dy of dtype dt."""
    say(f"layernorm_bwd_residual M={M} H={H} x,dy {dt} copy={copy}")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    x = synth.make(79, 0, (M, H), 2.0, dt)
    dy = synth.make(79, 1, (M, H), 1.0, dt)
    res = synth.make(79, 2, (M, H), 1.0, "f32")
    g = synth.Tensor(1.0 + 0.1 * synth.normal(79, 3, (H,)), "f32")
    bt = synth.Tensor(0.1 * synth.normal(79, 4, (H,)), "f32")
    y, mean, rstd = empty((M, H), tdt), empty((M,), torch.float32), empty((M,), torch.float32)
    dx_in, dg = to_dev(x), to_dev(g)
    tp.layernorm_fwd(dx_in, dg, to_dev(bt), y, mean, rstd, 1e-5)
    _, mu_ref, rs_ref = O.layernorm_forward(x.f64, g.f64, bt.f64, 1e-5)
    out, dgam, dbet = empty((M, H), torch.float32), empty((H,), torch.float32), empty((H,), torch.float32)
    cp = empty((M, H), torch.bfloat16) if copy else None
    ws = workspace(tp.layernorm_bwd_workspace(M, H))
    tp.layernorm_bwd_residual(dx_in, dg, mean, rstd, to_dev(dy), to_dev(res), out, dgam, dbet, ws, out_copy=cp)
    dx_ref, dg_ref, db_ref = O.layernorm_backward(x.f64, g.f64, mu_ref, rs_ref, dy.f64)
    ref = res.f64 + dx_ref
    tol = BF16_TOL if dt == "bf16" else F32_TOL
    assert rel_err(to_f64(out), ref) <= tol
    assert rel_err(to_f64(dgam), dg_ref) <= (F32_TOL if tol == F32_TOL else 1e-3)
    assert rel_err(to_f64(dbet), db_ref) <= 1e-5
    if copy:   # the copy is the fp32 output rounded once (round to nearest even)
        assert np.array_equal(raw_bits(cp), synth.to_bf16_bits(out.cpu().numpy()))
