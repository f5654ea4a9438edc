"""GPU parity: ColumnParallelLinear and RowParallelLinear shards on their
own (bias, gathered output as a strided column slice, scattered input, bias
added once after the shard sum, skip_bias_add) against the fp64 oracle,
through the C ABI."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpuutil import BF16_TOL, F32_TOL, rel_err, say, to_dev, to_f64

pytestmark = pytest.mark.gpu
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def tp():
    import megatron_tensor_transformer_columnparallel_amd as tp
    return tp


def _cols(t, s, c):
    return synth.Tensor(np.ascontiguousarray(t.store[:, s:s + c]), t.dtype)


def _vec(t, s, c):
    return synth.Tensor(np.ascontiguousarray(t.store[s:s + c]), t.dtype)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("case", [(37, 64, 208, 2, True), (128, 256, 384, 3, True), (5, 32, 64, 2, False),
                                  (300, 128, 256, 4, True)])
def test_column_linear(tp, dt, case):
    M, h, n_total, n, bias = case
    say(f"column linear M={M} h={h} n={n_total} shards={n} bias={bias} dt={dt}")
    w = 300 + M
    X = synth.make(w, 0, (M, h), 1.0, dt)
    A = synth.make(w, 1, (h, n_total), 0.05, dt)
    b = synth.make(w, 2, (n_total,), 0.5, dt) if bias else None
    dY = synth.make(w, 3, (M, n_total), 1.0, dt)
    tol = F32_TOL if dt == "f32" else BF16_TOL
    Xd, dYd = to_dev(X), to_dev(dY)
    Y = torch.full((M, n_total), float("nan"), dtype=TDT[dt], device="cuda")   # the gathered output
    dX = []
    dA = torch.empty((h, n_total), dtype=TDT[dt], device="cuda")
    db = torch.empty(n_total, device="cuda")
    for r in range(n):
        s, c = O.partition(n_total, n, r)
        assert c % 8 == 0
        A_r = to_dev(_cols(A, s, c))
        tp.column_linear_fwd(Xd, A_r, Y[:, s:s + c], b_r=to_dev(_vec(b, s, c)) if bias else None)
        dXr = torch.empty((M, h), dtype=TDT[dt], device="cuda")
        dAr = torch.empty((h, c), dtype=TDT[dt], device="cuda")
        dbr = torch.empty(c, device="cuda")
        tp.column_linear_bwd(Xd, A_r, dYd[:, s:s + c], dXr, dAr, db_r=dbr if bias else None)
        dX.append(dXr)
        dA[:, s:s + c] = dAr
        db[s:s + c] = dbr
    dXs = torch.empty((M, h), dtype=TDT[dt], device="cuda")
    tp.shard_reduce(dX, dXs)                                       # f backward
    torch.cuda.synchronize()
    _, Yref = O.column_linear_forward(X.f64, A.f64, b.f64 if bias else None, n)
    assert rel_err(to_f64(Y), Yref) <= tol
    ref = [O.column_linear_backward(X.f64, A.f64[:, s:s + c], dY.f64[:, s:s + c])
           for s, c in (O.partition(n_total, n, r) for r in range(n))]
    assert rel_err(to_f64(dXs), sum(x[0] for x in ref)) <= tol
    assert rel_err(to_f64(dA), np.concatenate([x[1] for x in ref], axis=1)) <= tol
    if bias:
        assert rel_err(db.cpu().numpy(), np.concatenate([x[2] for x in ref])) <= F32_TOL


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("case", [(45, 192, 96, 2, True, False), (64, 256, 128, 4, True, True),
                                  (9, 64, 32, 2, False, False), (513, 512, 256, 2, True, False)])
def test_row_linear(tp, dt, case):
    M, k_total, h, n, bias, parallel_in = case
    say(f"row linear M={M} k={k_total} h={h} shards={n} bias={bias} parallel_input={parallel_in} dt={dt}")
    w = 400 + M
    X = synth.make(w, 0, (M, k_total), 1.0, dt)
    B = synth.make(w, 1, (k_total, h), 0.05, dt)
    b = synth.make(w, 2, (h,), 0.5, dt)
    dY = synth.make(w, 3, (M, h), 1.0, dt)
    tol = F32_TOL if dt == "f32" else BF16_TOL
    Xd, dYd = to_dev(X), to_dev(dY)
    parts, dB = [], torch.empty((k_total, h), dtype=TDT[dt], device="cuda")
    dX = torch.full((M, k_total), float("nan"), dtype=TDT[dt], device="cuda")   # gathered dX
    dbs = []
    for r in range(n):
        s, c = O.partition(k_total, n, r)
        B_r = to_dev(synth.Tensor(np.ascontiguousarray(B.store[s:s + c]), dt))
        # the scatter is a column slice of the full input; a parallel input is its own buffer
        X_r = to_dev(_cols(X, s, c)) if parallel_in else Xd[:, s:s + c]
        Yr = torch.empty((M, h), dtype=TDT[dt], device="cuda")
        tp.row_linear_fwd(X_r, B_r, Yr)
        parts.append(Yr)
        dBr = torch.empty((c, h), dtype=TDT[dt], device="cuda")
        dbr = torch.empty(h, device="cuda")
        tp.row_linear_bwd(X_r, B_r, dYd, dX[:, s:s + c], dBr, db=dbr if bias else None)
        dB[s:s + c] = dBr
        dbs.append(dbr)
    Y = torch.empty((M, h), dtype=TDT[dt], device="cuda")
    if bias:
        tp.shard_reduce_bias(parts, to_dev(b), Y)
    else:
        tp.shard_reduce(parts, Y)                                  # skip_bias_add: the bias is returned
    torch.cuda.synchronize()
    _, Yref = O.row_linear_forward(X.f64, B.f64, b.f64, n, skip_bias_add=not bias)
    assert rel_err(to_f64(Y), Yref) <= tol
    ref = [O.row_linear_backward(X.f64[:, s:s + c], B.f64[s:s + c], dY.f64)
           for s, c in (O.partition(k_total, n, r) for r in range(n))]
    assert rel_err(to_f64(dX), np.concatenate([x[0] for x in ref], axis=1)) <= tol
    assert rel_err(to_f64(dB), np.concatenate([x[1] for x in ref], axis=0)) <= tol
    if bias:
        for d in dbs:
            assert rel_err(d.cpu().numpy(), ref[0][2]) <= F32_TOL
        assert all(torch.equal(d, dbs[0]) for d in dbs)           # same gradient of the replicated bias


def test_column_then_row_two_layer_bf16(tp):
    """Column shard feeding the row shard without a gather (the MLP pattern
    without its activation) at the page-1 MLP size M=2048, h=1024, 4h=4096,
    N=2, with both biases: sum_r (X A_r + b_r) B_r + c against the oracle."""
    M, h, f, n = 2048, 1024, 4096, 2
    say(f"column -> row, M={M} h={h} f={f} bf16")
    w = 450
    X = synth.make(w, 0, (M, h), 1.0, "bf16")
    A = synth.make(w, 1, (h, f), 0.02, "bf16")
    b = synth.make(w, 2, (f,), 0.1, "bf16")
    B = synth.make(w, 3, (f, h), 0.02, "bf16")
    c = synth.make(w, 4, (h,), 0.1, "bf16")
    Xd = to_dev(X)
    parts = []
    for r in range(n):
        s, cnt = O.partition(f, n, r)
        Hr = torch.empty((M, cnt), dtype=torch.bfloat16, device="cuda")
        tp.column_linear_fwd(Xd, to_dev(_cols(A, s, cnt)), Hr, b_r=to_dev(_vec(b, s, cnt)))
        Yr = torch.empty((M, h), dtype=torch.bfloat16, device="cuda")
        tp.row_linear_fwd(Hr, to_dev(synth.Tensor(np.ascontiguousarray(B.store[s:s + cnt]), "bf16")), Yr)
        parts.append(Yr)
    Y = torch.empty((M, h), dtype=torch.bfloat16, device="cuda")
    tp.shard_reduce_bias(parts, to_dev(c), Y)
    torch.cuda.synchronize()
    outs, _ = O.column_linear_forward(X.f64, A.f64, b.f64, n, gather_output=False)
    _, Yref = O.row_linear_forward(outs, B.f64, c.f64, n, input_is_parallel=True)
    assert rel_err(to_f64(Y), Yref) <= BF16_TOL
