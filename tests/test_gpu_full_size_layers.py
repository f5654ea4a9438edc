"""GPU parity at the sizes the benchmark times, on sampled outputs: the
standalone column and row linear layers (M = 2048 tokens, h = 4096, 8192
columns per shard, bf16, with biases), the sequence-parallel exchanges
(T = 16384 tokens, H = 4096, 2 shards) and the full input embedding with
dropout (T = 16384, H = 4096, 2048 positions, p = 0.1).  Inputs are drawn on
the device by seeded generators with the benchmark's distributions; every
output is computed in full, and sampled rows (or columns) are compared with
the fp64 oracle, which receives only the drawn inputs."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpuutil import BF16_TOL, F32_TOL, empty, rel_err, say, to_f64

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


@pytest.fixture(scope="module")
def tp():
    import megatron_tensor_transformer_columnparallel_amd as tp
    return tp


def _sample(n, k, seed):
    """k sorted indices in [0, n) that include the first and the last."""
    idx = np.sort(synth.rng(seed, 0).choice(n, k, replace=False))
    idx[0], idx[-1] = 0, n - 1
    return np.unique(idx)


def test_linear_layers_full_size(tp):
    M, h, n = 2048, 4096, 8192
    say(f"column and row linear full size M={M} h={h} n={n} bf16 with biases")
    g = torch.Generator(device="cuda")
    g.manual_seed(610)
    r = lambda *sh: (torch.randn(sh, generator=g, device="cuda") * 0.02).to(BF)
    X, A, b, dY = r(M, h), r(h, n), r(n), r(M, n)
    Xr, B, c, dZ = r(M, n), r(n, h), r(h), r(M, h)
    Y = empty((M, n), BF)
    dX, dA, db = empty((M, h), BF), empty((h, n), BF), empty((n,), torch.float32)
    Z0, Z1, Z = empty((M, h), BF), empty((M, h), BF), empty((M, h), BF)
    dXr, dB, dc = empty((M, n), BF), empty((n, h), BF), empty((h,), torch.float32)
    tp.column_linear_fwd(X, A, Y, b_r=b)
    tp.column_linear_bwd(X, A, dY, dX, dA, db_r=db)
    tp.row_linear_fwd(Xr, B, Z0)
    tp.row_linear_fwd(Xr, B, Z1)
    tp.shard_reduce_bias([Z0, Z1], c, Z)
    tp.row_linear_bwd(Xr, B, dZ, dXr, dB, db=dc)
    torch.cuda.synchronize()

    rows, cn, ch = _sample(M, 24, 611), _sample(n, 24, 612), _sample(h, 24, 613)
    ri, cni, chi = (torch.from_numpy(v).cuda() for v in (rows, cn, ch))
    X64, A64, b64, dY64 = to_f64(X), to_f64(A), to_f64(b), to_f64(dY)
    # column layer: Y rows, dX rows, dA columns, db in full
    Yref = O.column_linear_forward(X64[rows], A64, b64, 1)[0][0]
    assert rel_err(to_f64(Y[ri]), Yref) <= BF16_TOL
    dXref = O.column_linear_backward(X64[rows], A64, dY64[rows])[0]
    assert rel_err(to_f64(dX[ri]), dXref) <= BF16_TOL
    _, dAref, _ = O.column_linear_backward(X64, A64[:, cn], dY64[:, cn])
    assert rel_err(to_f64(dA[:, cni]), dAref) <= BF16_TOL
    assert rel_err(to_f64(db), O.column_linear_backward(X64[:, :1], A64[:1], dY64)[2]) <= F32_TOL
    del A64
    # row layer on two identical shards, bias once after the sum
    Xr64, B64, c64, dZ64 = to_f64(Xr), to_f64(B), to_f64(c), to_f64(dZ)
    Zref = O.row_linear_forward([Xr64[rows], Xr64[rows]], np.vstack([B64, B64]), c64, 2, input_is_parallel=True)[1]
    assert rel_err(to_f64(Z[ri]), Zref) <= BF16_TOL
    dXrref = O.row_linear_backward(Xr64[rows], B64, dZ64[rows])[0]
    assert rel_err(to_f64(dXr[ri]), dXrref) <= BF16_TOL
    _, dBref, _ = O.row_linear_backward(Xr64, B64[:, ch], dZ64[:, ch])
    assert rel_err(to_f64(dB[:, chi]), dBref) <= BF16_TOL
    assert rel_err(to_f64(dc), O.row_linear_backward(Xr64[:, :1], B64[:1], dZ64)[2]) <= F32_TOL


def test_sequence_parallel_exchanges_full_size(tp):
    T, H, n = 8 * 2048, 4096, 2
    say(f"sequence-parallel reduce-scatter and all-gather full size T={T} H={H} shards={n}")
    g = torch.Generator(device="cuda")
    g.manual_seed(620)
    rows_r = [tp.tps_partition(T, n, r) for r in range(n)]
    parts = [torch.randn((T, H), generator=g, device="cuda").to(BF) for _ in range(n)]
    res = [torch.randn((c, H), generator=g, device="cuda") for _, c in rows_r]
    outs = [empty((c, H), torch.float32) for _, c in rows_r]
    tp.shard_reduce_scatter(parts, outs, res=res)
    sl = [torch.randn((c, H), generator=g, device="cuda").to(BF) for _, c in rows_r]
    full = empty((T, H), BF)
    tp.shard_all_gather(sl, full)
    torch.cuda.synchronize()
    # sampled tokens, including both sides of the shard boundary
    tok = np.unique(np.concatenate([_sample(T, 40, 621), [rows_r[1][0] - 1, rows_r[1][0]]]))
    ti = torch.from_numpy(tok).cuda()
    shard = np.searchsorted([s for s, _ in rows_r], tok, side="right") - 1
    local = tok - np.array([rows_r[k][0] for k in shard])
    got = np.stack([to_f64(outs[k][int(l)]) for k, l in zip(shard, local)])
    res_rows = np.stack([to_f64(res[k][int(l)]) for k, l in zip(shard, local)])
    ref = O.sp_reduce_scatter([to_f64(p[ti]) for p in parts], 1, [res_rows])[0]
    assert rel_err(got, ref) <= F32_TOL
    # the all-gather is a copy of the slices in shard order
    gref = O.sp_all_gather([to_f64(x) for x in sl])
    assert np.array_equal(to_f64(full[ti]), gref[tok])


def test_full_embedding_full_size(tp):
    T, H, P, n, p, seed = 8 * 2048, 4096, 2048, 2, 0.1, 11
    say(f"full embedding full size T={T} H={H} positions={P} p={p}")
    g = torch.Generator(device="cuda")
    g.manual_seed(630)
    pos = (torch.arange(T, device="cuda", dtype=torch.int32) % P).contiguous()
    PE = (torch.randn((P, H), generator=g, device="cuda") * 0.02).to(BF)
    parts = [torch.randn((T, H), generator=g, device="cuda").to(BF) for _ in range(n)]
    out = empty((T, H), torch.float32)
    tp.embedding_fwd(parts, PE, pos, out, p=p, seed=seed)
    dout = torch.randn((T, H), generator=g, device="cuda")
    dx = empty((T, H), torch.float32)
    tp.dropout_apply(dout, dx, p, seed)
    torch.cuda.synchronize()
    tok = _sample(T, 32, 631)
    ti = torch.from_numpy(tok).cuda()
    pos_np = (np.arange(T) % P)[tok]
    ref, keep = O.embedding_forward([to_f64(x[ti]) for x in parts], to_f64(PE), pos_np, p, seed, tokens=tok)
    got = to_f64(out[ti])
    assert np.array_equal(got == 0, ~keep | (ref == 0)), "keep decisions differ"
    assert rel_err(got, ref) <= F32_TOL
    dref = O.embedding_backward(to_f64(dout[ti]), keep, p, pos_np, P)[0]
    gd = to_f64(dx[ti])
    assert np.array_equal(gd == 0, ~keep | (dref == 0)), "keep decisions differ (backward)"
    assert rel_err(gd, dref) <= F32_TOL
