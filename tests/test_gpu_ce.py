"""GPU parity: vocab-parallel cross entropy (per-shard statistics, the
exchange over shards, and the backward) against the fp64 oracle, through the
C ABI."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpuutil import BF16_TOL, F32_TOL, raw_bits, rel_err, say, to_f64

pytestmark = pytest.mark.gpu

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
VEC = {"f32": 4, "bf16": 8}
SENTINEL = 7.0   # fills the padding columns of the logits and of dL


@pytest.fixture(scope="module")
def tp():
    import megatron_tensor_transformer_columnparallel_amd as tp
    return tp


def _shard_buffers(x_bits, dt, V, n, pad):
    """Each shard's logits in a [T x ldl] buffer (ldl = its rows + pad, rounded
    up to the vector width), padding columns set to SENTINEL."""
    T = x_bits.shape[0]
    out = []
    full = torch.from_numpy(np.ascontiguousarray(x_bits.view(np.int16) if dt == "bf16" else x_bits)).cuda()
    if dt == "bf16":
        full = full.view(torch.bfloat16)
    for r in range(n):
        s, c = O.partition(V, n, r)
        ldl = -(-(c + pad) // VEC[dt]) * VEC[dt]
        buf = torch.full((T, ldl), SENTINEL, dtype=TORCH_DT[dt], device="cuda")
        buf[:, :c] = full[:, s:s + c]
        out.append((s, c, buf))
    return out


def run_ce(tp, shards, targets, dloss, in_place=False):
    T = targets.numel()
    stats = []
    for s, c, buf in shards:
        st = torch.full((T, 4), float("nan"), dtype=torch.float32, device="cuda")
        tp.vocab_ce_stats(buf[:, :c], targets, st, s)
        stats.append(st)
    loss = torch.full((T,), float("nan"), device="cuda")
    lse = torch.full((T,), float("nan"), device="cuda")
    tp.vocab_ce_combine(stats, loss, lse)
    grads = []
    for s, c, buf in shards:
        if in_place:
            tp.vocab_ce_bwd(buf[:, :c], targets, lse, dloss, buf[:, :c], s)
            grads.append(buf)
        else:
            d = torch.full_like(buf, SENTINEL)
            tp.vocab_ce_bwd(buf[:, :c], targets, lse, dloss, d[:, :c], s)
            grads.append(d)
    torch.cuda.synchronize()
    return stats, loss, lse, grads


def check(shards, x64, tg, dl, stats, loss, lse, grads, dt, V, n):
    starts = [s for s, _, _ in shards]
    parts = [x64[:, s:s + c] for s, c, _ in shards]
    ref_loss, sm, gmax, denom = O.vocab_ce_forward(parts, tg, starts)
    ref_grads = O.vocab_ce_backward(sm, tg, starts, dl)
    # per-shard statistics: max, target logit and ownership are exact
    for (s, c, _), st, p in zip(shards, stats, parts):
        st = st.cpu().numpy().astype(np.float64)
        assert np.array_equal(st[:, 0], p.max(axis=1))
        own = (tg >= s) & (tg < s + c)
        assert np.array_equal(st[:, 3], own.astype(np.float64))
        rows = np.arange(len(tg))
        assert np.array_equal(st[own, 2], p[rows[own], tg[own] - s])
        assert np.all(st[~own, 2] == 0)
    assert rel_err(loss.cpu().numpy(), ref_loss) <= F32_TOL
    assert rel_err(lse.cpu().numpy(), gmax + np.log(denom)) <= F32_TOL
    tol = F32_TOL if dt == "f32" else BF16_TOL
    for (s, c, _), g, rg in zip(shards, grads, ref_grads):
        got = to_f64(g)
        assert rel_err(got[:, :c], rg) <= tol
        # elementwise too: the small softmax entries, not only the -1 entries
        rt = 2e-5 if dt == "f32" else 2 ** -8
        assert np.all(np.abs(got[:, :c] - rg) <= rt * np.abs(rg) + 1e-7 * np.max(np.abs(rg)))
        assert np.all(got[:, c:] == SENTINEL), "padding columns written"


CASES = [
    # T, V, n, pad (extra columns of stride)
    (37, 1000, 2, 8),
    (5, 131, 3, 0),
    (64, 3001, 2, 16),
    (1, 2, 2, 8),          # one vocab row per shard
    (9, 20011, 2, 8),      # rows longer than one group of 64 x 8 chunks
    (3, 40, 8, 8),         # eight shards
]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES)
def test_ce_parity(tp, dt, case):
    T, V, n, pad = case
    say(f"vocab CE T={T} V={V} n={n} pad={pad} dt={dt}")
    g = synth.rng(200, V + n)
    x = g.standard_normal((T, V)).astype(np.float32) * 3
    bits = synth.to_bf16_bits(x) if dt == "bf16" else x
    x64 = synth.bf16_bits_to_f64(bits) if dt == "bf16" else x.astype(np.float64)
    tg = g.integers(0, V, T)
    if T >= 5:
        tg[1], tg[3] = -1, V + 3          # targets no shard owns
    dl = g.standard_normal(T)
    dl32 = dl.astype(np.float32)
    shards = _shard_buffers(bits, dt, V, n, pad)
    targets = torch.from_numpy(tg.astype(np.int32)).cuda()
    stats, loss, lse, grads = run_ce(tp, shards, targets, torch.from_numpy(dl32).cuda())
    check(shards, x64, tg, dl32.astype(np.float64), stats, loss, lse, grads, dt, V, n)


def test_ce_backward_in_place(tp):
    say("vocab CE backward in place (bf16)")
    T, V, n = 21, 777, 2
    g = synth.rng(201, 0)
    x = g.standard_normal((T, V)).astype(np.float32)
    bits = synth.to_bf16_bits(x)
    tg = g.integers(0, V, T)
    targets = torch.from_numpy(tg.astype(np.int32)).cuda()
    dl = torch.from_numpy(g.standard_normal(T).astype(np.float32)).cuda()
    _, _, _, out = run_ce(tp, _shard_buffers(bits, "bf16", V, n, 8), targets, dl)
    _, _, _, inp = run_ce(tp, _shard_buffers(bits, "bf16", V, n, 8), targets, dl, in_place=True)
    for a, b in zip(out, inp):
        assert np.array_equal(raw_bits(a), raw_bits(b))


def test_ce_large_and_uniform_logits(tp):
    say("vocab CE logits of magnitude 1e4, and all-equal logits")
    T, V, n = 6, 500, 2
    g = synth.rng(202, 0)
    x = (g.standard_normal((T, V)) * 1e4).astype(np.float32)
    x[3] = 42.0                              # one row of equal logits: loss = log V
    tg = g.integers(0, V, T)
    targets = torch.from_numpy(tg.astype(np.int32)).cuda()
    dl = np.ones(T, dtype=np.float32)
    shards = _shard_buffers(x, "f32", V, n, 4)
    stats, loss, lse, grads = run_ce(tp, shards, targets, torch.from_numpy(dl).cuda())
    check(shards, x.astype(np.float64), tg, dl.astype(np.float64), stats, loss, lse, grads, "f32", V, n)
    assert abs(float(loss[3]) - np.log(V)) <= 1e-5 * np.log(V)


def test_ce_full_size_sampled_rows(tp):
    """T = 16384 tokens over V = 50257 split 25129/25128 (row stride 25136),
    bf16 logits ~ N(0, 2^2) drawn on the device by a seeded generator; every
    row is computed, 48 sampled rows are compared with the oracle."""
    T, V, n, ldl = 16384, 50257, 2, 25136
    say(f"vocab CE full size T={T} V={V}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(203)
    tg = synth.uniform_ids(4, 40, T, V).astype(np.int64)
    targets = torch.from_numpy(tg.astype(np.int32)).cuda()
    dl = torch.full((T,), 1.0 / T, device="cuda")
    shards = []
    for r in range(n):
        s, c = O.partition(V, n, r)
        buf = torch.full((T, ldl), SENTINEL, dtype=torch.bfloat16, device="cuda")
        buf[:, :c] = (torch.randn((T, c), generator=gen, device="cuda") * 2).to(torch.bfloat16)
        shards.append((s, c, buf))
    stats, loss, lse, grads = run_ce(tp, shards, targets, dl)
    rows = np.sort(synth.rng(203, 1).choice(T, 48, replace=False))
    rows[0], rows[-1] = 0, T - 1
    ri = torch.from_numpy(rows).cuda()
    sub = [(s, c, buf[ri]) for s, c, buf in shards]
    x64 = np.concatenate([to_f64(b[:, :c]) for _, c, b in sub], axis=1)
    check(sub, x64, tg[rows], np.full(len(rows), 1.0 / T), [st[ri] for st in stats], loss[ri], lse[ri],
          [g[ri] for g in grads], "bf16", V, n)
