"""Pins of the oracle's bf16 storage-point diagnostic mode (oracle.bf16_storage).

* With no point rounded it is the acceptance oracle itself: the same
  operations in the same order as gpt_forward / gpt_backward, so every
  output is identical bit for bit.
* Every storage point is wired in: rounding it alone changes exactly the
  outputs that depend on it (a forward-only point moves the logits, a
  backward-only point leaves them untouched), and the change has the size
  of one bf16 rounding propagated through a small model.
* The softmax-backward row term taken from the stored P and dP equals the
  oracle's rowsum(dO * O) when nothing is rounded (the two are equal in
  exact arithmetic because O = P V and dP = dO V^T).
* Re-centring the keys for dQ is exact when nothing but dS is rounded and
  the centred keys are kept exact.
"""

import numpy as np
import pytest

import oracle as O
import synth
from oracle import bf16_storage as B

TINY = dict(L=2, b=2, s=8, H=16, heads=4, d=4, f=64, V=50, n=2)


def tiny_inputs(seed=77):
    c = TINY
    vr = [O.partition(c["V"], c["n"], r)[1] for r in range(c["n"])]
    ids, E, layers, dL = synth.gpt_inputs(seed, c["L"], c["b"] * c["s"], c["H"], c["heads"] * c["d"], c["f"],
                                          c["V"], vr, ln_random=True)
    # larger weights than the workload's 0.02 so that a rounding point moves
    # the outputs well above fp64 noise
    lay = [{k: (t.f64 * (25.0 if t.dtype == "bf16" else 1.0)) for k, t in lw.items()} for lw in layers]
    return ids, E.f64, lay, [t.f64 for t in dL]


def run_oracle(ids, E, lay, dL):
    c = TINY
    lg, cache = O.gpt_forward(ids, E, lay, c["b"], c["s"], c["heads"], c["d"], c["n"])
    dE, grads = O.gpt_backward(ids, E, lay, cache, dL, c["b"], c["s"], c["heads"], c["d"], c["n"])
    return lg, dE, grads


def run_emu(ids, E, lay, dL, rnd):
    c = TINY
    lg, cache = B.gpt_forward(ids, E, lay, c["b"], c["s"], c["heads"], c["d"], c["n"], rnd)
    dE, grads = B.gpt_backward(ids, E, lay, cache, dL, c["b"], c["s"], c["heads"], c["d"], c["n"], rnd)
    return lg, dE, grads


def flat(lg, dE, grads):
    out = {f"logits{r}": x for r, x in enumerate(lg)}
    out["dE"] = dE
    for li, g in enumerate(grads):
        for k, v in g.items():
            out[f"L{li}.{k}"] = v
    return out


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.fixture(scope="module")
def case():
    ids, E, lay, dL = tiny_inputs()
    return ids, E, lay, dL, flat(*run_oracle(ids, E, lay, dL))


def test_no_rounding_is_the_oracle_bit_for_bit(case):
    ids, E, lay, dL, ref = case
    got = flat(*run_emu(ids, E, lay, dL, B.Rounding()))
    assert got.keys() == ref.keys()
    for k in ref:
        assert np.array_equal(got[k], ref[k]), k


FORWARD = {"ln_out", "qkv", "p_fwd", "o", "part_fwd", "mlp_h", "x_final", "logits"}


@pytest.mark.parametrize("point", B.POINTS)
def test_each_point_is_wired(case, point):
    ids, E, lay, dL, ref = case
    got = flat(*run_emu(ids, E, lay, dL, B.Rounding([point])))
    moved = {k for k in ref if not np.array_equal(got[k], ref[k])}
    lg_moved = any(k.startswith("logits") for k in moved)
    assert lg_moved == (point in FORWARD), (point, sorted(moved)[:5])
    if point != "logits":
        assert any(k.startswith("L") or k == "dE" for k in moved), point
    # one bf16 rounding (relative 2^-9) propagated through two small layers
    worst = max(rel(got[k], ref[k]) for k in ref)
    assert 1e-6 < worst < 0.2, (point, worst)


def test_delta_from_p_equals_delta_from_o_without_rounding(case):
    ids, E, lay, dL, ref = case
    got = flat(*run_emu(ids, E, lay, dL, B.Rounding(delta="p")))
    for k in ref:
        assert rel(got[k], ref[k]) < 1e-10, k


def test_new_forms_equal_the_oracle_without_rounding(case):
    # the fp32-copy row term and the end-normalised forward compute the
    # oracle's values when nothing is rounded (only the order of operations
    # differs)
    ids, E, lay, dL, ref = case
    for rnd in (B.Rounding(delta="o32"), B.Rounding(p_fwd_form="unnormalised"),
                B.Rounding(delta="o32", p_fwd_form="unnormalised")):
        got = flat(*run_emu(ids, E, lay, dL, rnd))
        for k in ref:
            assert rel(got[k], ref[k]) < 1e-10, (rnd.delta, rnd.p_fwd_form, k)


def test_o32_row_term_reads_the_unrounded_output(case):
    # with O rounded, "o" forms the row term from the rounded O and "o32" from
    # the unrounded one: the forward is the same, dW_QKV (which reads O only
    # through the row term) differs, dW_O (which reads the stored O) does not
    ids, E, lay, dL, ref = case
    a = flat(*run_emu(ids, E, lay, dL, B.Rounding(["o"], delta="o")))
    b = flat(*run_emu(ids, E, lay, dL, B.Rounding(["o"], delta="o32")))
    assert all(np.array_equal(a[k], b[k]) for k in a if k.startswith("logits"))
    top = max(int(k[1:].split(".")[0]) for k in a if k.startswith("L"))
    assert not np.array_equal(a[f"L{top}.WQ"], b[f"L{top}.WQ"])
    # dW_O reads the stored O directly: the same in both
    assert np.array_equal(a[f"L{top}.WO"], b[f"L{top}.WO"])


def test_unnormalised_form_rounds_other_values():
    g = np.random.default_rng(11)
    s, d = 40, 16
    Q, K, V = (g.standard_normal((s, d)) for _ in range(3))
    O0, l0 = O.attention_head_forward(Q, K, V)
    a, la = B.head_forward(Q, K, V, B.Rounding(["p_fwd"]))
    b, lb = B.head_forward(Q, K, V, B.Rounding(["p_fwd"], p_fwd_form="unnormalised"))
    assert np.array_equal(la, lb) and rel(la, l0) < 1e-14
    assert not np.array_equal(a, b)
    # both are one bf16 rounding of the probabilities away from the exact O
    for got in (a, b):
        assert 1e-6 < rel(got, O0) < 2 ** -7


def test_head_backward_centred_keys_exact():
    g = np.random.default_rng(3)
    s, d = 12, 8
    Q, V, dO = (g.standard_normal((s, d)) for _ in range(3))
    # keys with a large common component: kbar = 5 exactly, and K - kbar
    # (quarter integers in +-2) is exact in bf16
    half = g.integers(-8, 9, (s // 2, d)) / 4.0
    K = np.concatenate([half, -half], axis=0)[g.permutation(s)] + 5.0
    Oh, lse = O.attention_head_forward(Q, K, V)
    dQ, dK, dV = O.attention_head_backward(Q, K, V, Oh, dO)
    assert np.array_equal(B.to_bf16_via_f32(K - K.mean(axis=0)), K - 5.0)
    # dS rounded, keys centred exactly: dS_q (K - kbar) + rowsum(dS_q) kbar = dS_q K
    q0 = B.head_backward(Q, K, V, Oh, dO, lse, B.Rounding(["ds"]))
    q1 = B.head_backward(Q, K, V, Oh, dO, lse, B.Rounding(["ds"], ds_center=True))
    assert rel(q1[0], q0[0]) < 1e-12
    assert np.array_equal(q1[1], q0[1]) and np.array_equal(q1[2], q0[2])
    # both stay within a few bf16 roundings of the exact gradient
    for got, ref in zip(q0, (dQ, dK, dV)):
        assert rel(got, ref) < 5e-2


def test_rounding_equals_the_oracles_on_fp32_values():
    # on values that are already fp32 the first step is exact, so the result
    # must be the oracle's nearest-bf16 rounding (itself pinned by brute force)
    g = np.random.default_rng(5)
    x = (g.standard_normal(100000) * np.exp(g.uniform(-30, 30, 100000))).astype(np.float32).astype(np.float64)
    ties = np.float32(1.0 + 2.0 ** -8) * np.array([1, -1, 3, 1e-20, 7e20])   # exact ties at the bf16 step
    x = np.concatenate([x, ties.astype(np.float32).astype(np.float64), [0.0, -0.0]])
    assert np.array_equal(B.to_bf16_via_f32(x), O.round_to_bf16(x))


def test_unknown_point_rejected():
    with pytest.raises(ValueError):
        B.Rounding(["no_such_point"])
    with pytest.raises(ValueError):
        B.Rounding(delta="q")
    with pytest.raises(ValueError):
        B.Rounding(p_fwd_form="other")
