"""GPU parity: MLP shard forward/backward and the tied output projection
against the fp64 oracle, through the C ABI."""

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


def _shard(t: synth.Tensor, rows=None, cols=None) -> synth.Tensor:
    s = t.store
    if rows is not None:
        s = s[rows[0]:rows[1]]
    if cols is not None:
        s = s[:, cols[0]:cols[1]]
    return synth.Tensor(np.ascontiguousarray(s), t.dtype)


def run_mlp_shard(tp, X, A_r, B_r, dZ, tdt):
    M, h = X.shape
    f = A_r.shape[1]
    dX_, dA_, dB_ = to_dev(X), to_dev(A_r), to_dev(B_r)
    P, H, Z = empty((M, f), tdt), empty((M, f), tdt), empty((M, h), tdt)
    tp.tp_mlp_fwd(dX_, dA_, dB_, P, H, Z)
    ddZ = to_dev(dZ)
    gX, gA, gB = empty((M, h), tdt), empty((h, f), tdt), empty((f, h), tdt)
    ws = workspace(tp.tp_mlp_bwd_workspace(tdt, M, h, f))
    tp.tp_mlp_bwd(dX_, dA_, dB_, P, H, ddZ, gX, gA, gB, ws)
    return dict(P=P, H=H, Z=Z, dX=gX, dA=gA, dB=gB)


@pytest.mark.parametrize("w,M,h,f,n,dt", [
    (1, 8, 64, 256, 2, "f32"),          # workload 1 (fp32)
    (81, 100, 72, 144, 2, "bf16"),      # ragged: rows and columns not tile multiples
    (82, 333, 64, 8000, 2, "bf16"),     # 4000-wide shard: M x f_i GEMMs take the 256x256 tile
    (83, 130, 128, 384, 3, "bf16"),     # three shards
    (84, 512, 64, 49152, 2, "bf16"),    # M x f_i = 512 x 24576: the 256x192 tile (forward NN, GELU' NT)
])
def test_mlp_shards_match_oracle(tp, w, M, h, f, n, dt):
    say(f"tp_mlp fwd+bwd M={M} h={h} f={f} N={n} {dt}")
    inp = synth.mlp_inputs(w, M, h, f, dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    tol = BF16_TOL if dt == "bf16" else F32_TOL
    X, A, B, dZ = inp["X"], inp["A"], inp["B"], inp["dZ"]
    Zs, dXs = [], []
    for r in range(n):
        s, c = O.partition(f, n, r)
        A_r, B_r = _shard(A, cols=(s, s + c)), _shard(B, rows=(s, s + c))
        got = run_mlp_shard(tp, X, A_r, B_r, dZ, tdt)
        P_ref, H_ref, Z_ref = O.mlp_forward(X.f64, A_r.f64, B_r.f64)
        dX_ref, dA_ref, dB_ref = O.mlp_backward(X.f64, A_r.f64, B_r.f64, P_ref, dZ.f64)
        for key, ref in [("P", P_ref), ("H", H_ref), ("Z", Z_ref), ("dX", dX_ref), ("dA", dA_ref),
                         ("dB", dB_ref)]:
            e = rel_err(to_f64(got[key]), ref)
            assert e <= tol, (key, r, e)
        Zs.append(got["Z"])
        dXs.append(got["dX"])
    # 'g' forward and 'f' backward: the shard sums equal the unsharded layer
    P_u, _, Z_u = O.mlp_forward(X.f64, A.f64, B.f64)
    dX_u, _, _ = O.mlp_backward(X.f64, A.f64, B.f64, P_u, dZ.f64)
    Zsum, dXsum = empty((M, h), tdt), empty((M, h), tdt)
    tp.shard_reduce(Zs, Zsum)
    tp.shard_reduce(dXs, dXsum)
    assert rel_err(to_f64(Zsum), Z_u) <= tol
    assert rel_err(to_f64(dXsum), dX_u) <= tol


def test_mlp_workload2_full_size(tp):
    """b=4, s=512, h=1024, h'=4096, N=2 (A_i 1024x2048, B_i 2048x1024), both shards, then summed."""
    cfg = synth.WORKLOADS[2]
    M, h, f, n = cfg["b"] * cfg["s"], cfg["h"], cfg["f"], cfg["n"]
    say(f"tp_mlp workload 2 full size M={M} h={h} f={f}")
    inp = synth.mlp_inputs(2, M, h, f, "bf16")
    X, A, B, dZ = inp["X"], inp["A"], inp["B"], inp["dZ"]
    Xf, dZf = X.f64, dZ.f64
    Zs, dXs = [], []
    for r in range(n):
        s, c = O.partition(f, n, r)
        A_r, B_r = _shard(A, cols=(s, s + c)), _shard(B, rows=(s, s + c))
        got = run_mlp_shard(tp, X, A_r, B_r, dZ, torch.bfloat16)
        P_ref, H_ref, Z_ref = O.mlp_forward(Xf, A_r.f64, B_r.f64)
        dX_ref, dA_ref, dB_ref = O.mlp_backward(Xf, A_r.f64, B_r.f64, P_ref, dZf)
        for key, ref in [("Z", Z_ref), ("dX", dX_ref), ("dA", dA_ref), ("dB", dB_ref), ("H", H_ref)]:
            e = rel_err(to_f64(got[key]), ref)
            assert e <= BF16_TOL, (key, r, e)
        Zs.append(got["Z"])
        dXs.append(got["dX"])
        if r == 0:
            again = run_mlp_shard(tp, X, A_r, B_r, dZ, torch.bfloat16)
            for key in ("Z", "dX", "dA", "dB"):
                assert np.array_equal(raw_bits(again[key]), raw_bits(got[key])), f"{key} not deterministic"
    Zsum = empty((M, h), torch.bfloat16)
    tp.shard_reduce(Zs, Zsum)
    P_u, _, Z_u = O.mlp_forward(Xf, A.f64, B.f64)
    assert rel_err(to_f64(Zsum), Z_u) <= BF16_TOL


# ------------------------------------------------------------------ tied logits

@pytest.mark.parametrize("w,T,H,V,n,dt,pad", [
    (1, 64, 64, 300, 2, "f32", 4),        # workload-1 shapes
    (84, 300, 2048, 15985, 2, "bf16", 8),   # ragged shard widths 7993/7992, ldl > v_rows
    (85, 2000, 64, 15985, 2, "bf16", 0),    # T x v_r logits take the 256x256 tile
    (86, 512, 512, 66000, 2, "bf16", 0),    # 258-tile grids: logits split by columns, dE by rows
])
def test_tied_logits_match_oracle(tp, w, T, H, V, n, dt, pad):
    say(f"tied_logits fwd+bwd T={T} H={H} V={V} {dt}")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    tol = BF16_TOL if dt == "bf16" else F32_TOL
    inp = synth.embed_inputs(w, T, V, H, dt, 0.02 if dt == "bf16" else 1.0)
    X, E = inp["X"], inp["E"]
    vec = 8 if dt == "bf16" else 4
    dXs, dX_refs = [], []
    for r in range(n):
        s, c = O.partition(V, n, r)
        E_r = _shard(E, rows=(s, s + c))
        ldl = ((c + vec - 1) // vec) * vec + pad
        dL = synth.logit_grad(w, r, T, c, dt)
        Lbuf = empty((T, ldl), tdt)
        L = Lbuf[:, :c]
        tp.tied_logits(to_dev(X), to_dev(E_r), L)
        assert rel_err(to_f64(L), O.tied_logits(X.f64, E_r.f64)) <= tol
        if ldl > c:
            assert torch.isnan(Lbuf[:, c:]).all(), "padding columns must not be written"
        dLbuf = empty((T, ldl), tdt)
        dLbuf[:, :c] = to_dev(dL)
        dX = empty((T, H), tdt)
        dE = empty((c, H), torch.float32)
        tp.tied_logits_bwd(to_dev(X), to_dev(E_r), dLbuf[:, :c], dX, dE)
        dX_ref, dE_ref = O.tied_logits_backward(X.f64, E_r.f64, dL.f64)
        assert rel_err(to_f64(dX), dX_ref) <= tol
        assert rel_err(to_f64(dE), dE_ref) <= (tol if dt == "f32" else 1e-3)
        dXs.append(dX)
        dX_refs.append(dX_ref)
    out = empty((T, H), tdt)
    tp.shard_reduce(dXs, out)
    assert rel_err(to_f64(out), O.shard_reduce(dX_refs)) <= tol


def test_tied_gradient_is_output_side_plus_input_side(tp):
    """tied_logits_bwd writes dE_r, vocab_embed_bwd then adds the input-side
    gradient: the total equals the oracle's sum of both."""
    say("tied total gradient = tied_logits_bwd then vocab_embed_bwd")
    T, H, V, n = 512, 128, 1000, 2
    inp = synth.embed_inputs(86, T, V, H, "bf16", 0.02)
    ids, X, E, dY = inp["ids"], inp["X"], inp["E"], inp["dY"]
    from gpuutil import ids_dev
    for r in range(n):
        s, c = O.partition(V, n, r)
        E_r = _shard(E, rows=(s, s + c))
        dL = synth.logit_grad(86, r, T, c, "bf16")
        ldl = ((c + 7) // 8) * 8
        dLbuf = torch.zeros((T, ldl), dtype=torch.bfloat16, device="cuda")
        dLbuf[:, :c] = to_dev(dL)
        dX = empty((T, H), torch.bfloat16)
        dE = empty((c, H), torch.float32)
        tp.tied_logits_bwd(to_dev(X), to_dev(E_r), dLbuf[:, :c], dX, dE)
        ws = workspace(tp.vocab_embed_bwd_workspace(T, c))
        tp.vocab_embed_bwd(ids_dev(ids), to_dev(dY), dE, s, ws)
        ref = O.tied_logits_backward(X.f64, E_r.f64, dL.f64)[1] + O.vocab_embed_backward(ids, dY.f64, s, c)
        assert rel_err(to_f64(dE), ref) <= 1e-3
