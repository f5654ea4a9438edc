"""GPU parity: sequence-parallel exchanges (reduce-scatter with the residual,
all-gather) and a sequence-parallel MLP sublayer, forward and backward,
against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpuutil import BF16_TOL, empty, raw_bits, rel_err, say, to_dev, to_f64, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tp():
    import megatron_tensor_transformer_columnparallel_amd as tp
    return tp


def _rows(M, n):
    return [O.partition(M, n, r) for r in range(n)]


@pytest.mark.parametrize("M,n", [(64, 2), (37, 3), (5, 8), (1000, 4)])
def test_reduce_scatter_two_bf16_parts_bit_exact_and_gather(tp, M, n):
    """Two bf16 partials sum exactly in fp32, so each shard's slice is the
    nearest bf16 of the exact sum; gathering the slices is a bit copy."""
    H = 72
    say(f"reduce-scatter / all-gather M={M} n={n}")
    a = synth.make(500, 0, (M, H), 3.0, "bf16")
    b = synth.make(500, 1, (M, H), 1.0, "bf16")
    outs = [empty((c, H), torch.bfloat16) for _, c in _rows(M, n)]
    # n partials: a, b and (n - 2) zeros, so the fp32 sum stays exact
    z = synth.Tensor(np.zeros((M, H), np.uint16), "bf16")
    tp.shard_reduce_scatter([to_dev(a), to_dev(b)] + [to_dev(z)] * (n - 2), outs)
    ref = O.round_to_bf16(O.shard_reduce([a.f64, b.f64]))
    for (s, c), o in zip(_rows(M, n), outs):
        if c:
            assert np.array_equal(to_f64(o), ref[s:s + c])
    full = empty((M, H), torch.bfloat16)
    tp.shard_all_gather(outs, full)
    assert np.array_equal(to_f64(full), ref)


@pytest.mark.parametrize("pdt,odt", [("bf16", "f32"), ("f32", "f32"), ("f32", "bf16")])
def test_reduce_scatter_with_residual(tp, pdt, odt):
    M, H, n = 301, 64, 3
    say(f"reduce-scatter with residual parts={pdt} out={odt}")
    parts = [synth.make(501, k, (M, H), 1.0, pdt) for k in range(n)]
    res = [synth.make(502, r, (c, H), 1.0, odt) for r, (_, c) in enumerate(_rows(M, n))]
    tdt = torch.float32 if odt == "f32" else torch.bfloat16
    outs = [empty((c, H), tdt) for _, c in _rows(M, n)]
    tp.shard_reduce_scatter([to_dev(p) for p in parts], outs, res=[to_dev(r) for r in res])
    ref = O.sp_reduce_scatter([p.f64 for p in parts], n, [r.f64 for r in res])
    tol = 1e-6 if odt == "f32" else 2 ** -8
    for o, rf in zip(outs, ref):
        assert rel_err(to_f64(o), rf) <= tol
    # fp32 gather of the fp32 slices is exact
    if odt == "f32":
        full = empty((M, H), torch.float32)
        tp.shard_all_gather(outs, full)
        assert np.array_equal(raw_bits(full), raw_bits(torch.cat(outs)))


def test_sequence_parallel_mlp_sublayer(tp):
    """x (fp32 residual stream) split by sequence over n = 2 shards: each shard
    normalises its rows, the all-gather rebuilds the full sequence for the
    tensor-parallel MLP, and the reduce-scatter adds each shard's rows of the
    MLP output to its residual rows.  Backward: the all-gather of the output
    gradient feeds the MLP backward, the reduce-scatter returns each shard's
    rows of its input gradient, each shard runs the LayerNorm backward on its
    rows (plus the residual gradient), and the LayerNorm parameter gradients
    are summed over shards.  Everything against the unsharded oracle."""
    M, H, f, n = 512, 512, 2048, 2
    say(f"sequence-parallel MLP sublayer M={M} H={H} f={f} n={n}")
    w = 503
    x = synth.make(w, 0, (M, H), 1.0, "f32")
    gamma = synth.Tensor((1 + 0.1 * synth.normal(w, 1, (H,))).astype(np.float32), "f32")
    beta = synth.Tensor((0.1 * synth.normal(w, 2, (H,))).astype(np.float32), "f32")
    A = synth.make(w, 3, (H, f), 0.02, "bf16")
    B = synth.make(w, 4, (f, H), 0.02, "bf16")
    dout = synth.make(w, 5, (M, H), 1.0, "f32")
    rows = _rows(M, n)
    bf, f32 = torch.bfloat16, torch.float32
    xs = [to_dev(synth.Tensor(np.ascontiguousarray(x.store[s:s + c]), "f32")) for s, c in rows]
    g, bt = to_dev(gamma), to_dev(beta)
    # forward
    ys, means, rstds = [], [], []
    for xr, (s, c) in zip(xs, rows):
        y, m, r = empty((c, H), bf), empty((c,), f32), empty((c,), f32)
        tp.layernorm_fwd(xr, g, bt, y, m, r)
        ys.append(y); means.append(m); rstds.append(r)
    y_full = empty((M, H), bf)
    tp.shard_all_gather(ys, y_full)
    Ps, Hs, Zs, Ars, Brs = [], [], [], [], []
    for r in range(n):
        s, c = O.partition(f, n, r)
        Ar = to_dev(synth.Tensor(np.ascontiguousarray(A.store[:, s:s + c]), "bf16"))
        Br = to_dev(synth.Tensor(np.ascontiguousarray(B.store[s:s + c]), "bf16"))
        P, Hh, Z = empty((M, c), bf), empty((M, c), bf), empty((M, H), bf)
        tp.tp_mlp_fwd(y_full, Ar, Br, P, Hh, Z)
        Ps.append(P); Hs.append(Hh); Zs.append(Z); Ars.append(Ar); Brs.append(Br)
    outs = [empty((c, H), f32) for _, c in rows]
    tp.shard_reduce_scatter(Zs, outs, res=xs)
    # backward
    douts = [to_dev(synth.Tensor(np.ascontiguousarray(dout.store[s:s + c]), "f32")) for s, c in rows]
    dout_bf = [empty((c, H), bf) for _, c in rows]
    for d32, d16 in zip(douts, dout_bf):
        tp.shard_reduce([d32], d16)                                     # bf16 copy for the GEMMs
    dZ = empty((M, H), bf)
    tp.shard_all_gather(dout_bf, dZ)
    dYs = []
    for r in range(n):
        c = O.partition(f, n, r)[1]
        dY, dA, dB = empty((M, H), bf), empty((H, c), bf), empty((c, H), bf)
        ws = workspace(tp.tp_mlp_bwd_workspace(bf, M, H, c))
        tp.tp_mlp_bwd(y_full, Ars[r], Brs[r], Ps[r], Hs[r], dZ, dY, dA, dB, ws)
        dYs.append(dY)
    dys = [empty((c, H), f32) for _, c in rows]
    tp.shard_reduce_scatter(dYs, dys)
    dxs, dgs, dbs = [], [], []
    for r, (s, c) in enumerate(rows):
        dx, dg, db = empty((c, H), f32), empty((H,), f32), empty((H,), f32)
        ws = workspace(tp.layernorm_bwd_workspace(c, H))
        tp.layernorm_bwd_residual(xs[r], g, means[r], rstds[r], dys[r], douts[r], dx, dg, db, ws)
        dxs.append(dx); dgs.append(dg); dbs.append(db)
    dgamma, dbeta = empty((H,), f32), empty((H,), f32)
    tp.shard_reduce(dgs, dgamma)                                        # summed over the group
    tp.shard_reduce(dbs, dbeta)
    torch.cuda.synchronize()
    # oracle, unsharded
    y64, mu, rs = O.layernorm_forward(x.f64, gamma.f64, beta.f64)
    P64, _, Z64 = O.mlp_forward(y64, A.f64, B.f64)
    out_ref = x.f64 + Z64
    assert rel_err(np.concatenate([to_f64(o) for o in outs]), out_ref) <= BF16_TOL
    dy64, _, _ = O.mlp_backward(y64, A.f64, B.f64, P64, dout.f64)
    dxs_ref, dg_ref, db_ref = O.sp_layernorm_param_grads(
        [x.f64[s:s + c] for s, c in rows], gamma.f64, [mu[s:s + c] for s, c in rows],
        [rs[s:s + c] for s, c in rows], [dy64[s:s + c] for s, c in rows])
    dx_ref = dout.f64 + np.concatenate(dxs_ref)
    assert rel_err(np.concatenate([to_f64(d) for d in dxs]), dx_ref) <= BF16_TOL
    assert rel_err(to_f64(dgamma), dg_ref) <= BF16_TOL
    assert rel_err(to_f64(dbeta), db_ref) <= BF16_TOL
