"""GPU parity: the full input embedding (word embedding summed over shards,
position and token-type rows, dropout from Philox4x32-10) and its backward
through dropout_apply and vocab_embed_bwd, against the fp64 oracle, through
the C ABI.  The keep decisions are integer comparisons of the generator's
words and must match the oracle's exactly."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpuutil import F32_TOL, BF16_TOL, empty, ids_dev, raw_bits, rel_err, say, to_dev, to_f64, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tp():
    import megatron_tensor_transformer_columnparallel_amd as tp
    return tp


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("p,seed,types", [(0.0, 1, False), (0.1, 0x0123456789ABCDEF, True), (0.5, 42, True),
                                          (0.9, 2 ** 63 + 5, False)])
def test_full_embedding_forward_backward(tp, dt, p, seed, types):
    T, H, V, P, NT, n = 300, 64, 1000, 256, 3, 2
    say(f"full embedding T={T} H={H} p={p} seed={seed:#x} types={types} dt={dt}")
    w = 600
    ids = synth.uniform_ids(w, 0, T, V)
    pos = (np.arange(T) % P).astype(np.int32)
    pos[5] = P + 3                                     # outside the table: adds a zero row
    tt = synth.uniform_ids(w, 1, T, NT) if types else None
    E = synth.make(w, 2, (V, H), 1.0, dt)
    PE = synth.make(w, 3, (P, H), 1.0, dt)
    TE = synth.make(w, 4, (NT, H), 1.0, dt) if types else None
    dout = synth.make(w, 5, (T, H), 1.0, "f32")
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    sc = [O.partition(V, n, r) for r in range(n)]
    dids = ids_dev(ids)
    parts = []
    for s, c in sc:
        Yr = empty((T, H), tdt)
        tp.vocab_embed_fwd(dids, to_dev(synth.Tensor(np.ascontiguousarray(E.store[s:s + c]), dt)), Yr, s)
        parts.append(Yr)
    out = empty((T, H), torch.float32)
    dpos = ids_dev(pos)
    dtt = ids_dev(tt) if types else None
    tp.embedding_fwd(parts, to_dev(PE), dpos, out, p=p, seed=seed, TE=to_dev(TE) if types else None, tt=dtt)
    # backward: dropout of the output gradient, then every table through the scatter-add
    dX = empty((T, H), torch.float32)
    tp.dropout_apply(to_dev(dout), dX, p, seed)
    dX_t = dX if dt == "f32" else dX.to(torch.bfloat16)
    dPE = torch.zeros((P, H), device="cuda")
    tp.vocab_embed_bwd(dpos, dX_t, dPE, 0, workspace(tp.vocab_embed_bwd_workspace(T, P)))
    dEs = []
    for s, c in sc:
        dE = torch.zeros((c, H), device="cuda")
        tp.vocab_embed_bwd(dids, dX_t, dE, s, workspace(tp.vocab_embed_bwd_workspace(T, c)))
        dEs.append(dE)
    torch.cuda.synchronize()
    # oracle
    wp = [O.vocab_embed_forward(ids, E.f64[s:s + c], s) for s, c in sc]
    ref, keep = O.embedding_forward(wp, PE.f64, pos, p, seed, TE.f64 if types else None, tt)
    got = to_f64(out)
    assert np.array_equal(got == 0, ~keep | (ref == 0)), "keep decisions differ"
    assert rel_err(got, ref) <= F32_TOL
    dX_ref, dPE_ref, _ = O.embedding_backward(dout.f64, keep, p, pos, P)
    assert np.array_equal(to_f64(dX) == 0, ~keep | (dout.f64 == 0))
    assert rel_err(to_f64(dX), dX_ref) <= F32_TOL
    tol = F32_TOL if dt == "f32" else BF16_TOL
    # the bf16 path takes the gradient rounded to bf16, as the oracle is given exactly that
    dX_in = dX_ref if dt == "f32" else to_f64(dX_t)
    assert rel_err(to_f64(dPE), O.vocab_embed_backward(pos, dX_in, 0, P)) <= tol
    for (s, c), dE in zip(sc, dEs):
        assert rel_err(to_f64(dE), O.vocab_embed_backward(ids, dX_in, s, c)) <= tol


def test_dropout_keep_rate_and_ragged_tail(tp):
    """One million elements (plus a ragged tail of 5): the kept fraction lies
    within 5 sigma of 1 - p and equals the oracle's mask count exactly."""
    n, p, seed = 1_000_005, 0.3, 99
    say(f"dropout n={n} p={p}")
    x = torch.ones(n, device="cuda")
    y = torch.empty(n, device="cuda")
    tp.dropout_apply(x, y, p, seed)
    kept = (y != 0).cpu().numpy()
    ref = O.dropout_keep(n, p, seed)
    assert np.array_equal(kept, ref)
    assert abs(kept.mean() - (1 - p)) <= 5 * np.sqrt(p * (1 - p) / n)
    assert np.allclose(y.cpu().numpy()[kept], 1.0 / (1.0 - np.float32(p)), rtol=1e-7)
