"""Seeded synthetic inputs shared by the tests, the oracle comparisons and the
benchmark.  Holds no arithmetic of the method itself: only random draws, the
fp32 -> bf16 storage conversion of those draws, and the workload shapes.

Every tensor of workload ``w`` tensor ``i`` is drawn from
``numpy.random.default_rng(1000 * w + i)`` once, in fp32, and (for bf16
workloads) converted once to bf16 bit patterns.  The same bits feed the GPU
library and, upcast exactly to fp64, the oracle.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


# ---------------------------------------------------------------------------
# Storage conversion of the draws (round to nearest even on the bit pattern).
# ---------------------------------------------------------------------------

def to_bf16_bits(x) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns, round-to-nearest-even.

    Adds 0x7FFF plus the lowest kept bit to the fp32 pattern and keeps the top
    16 bits; NaNs map to a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def rng(workload: int, index: int) -> np.random.Generator:
    return np.random.default_rng(1000 * workload + index)


def normal(workload: int, index: int, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) draws in fp32."""
    g = rng(workload, index)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def uniform_ids(workload: int, index: int, count: int, vocab: int) -> np.ndarray:
    return rng(workload, index).integers(0, vocab, size=count, dtype=np.int64).astype(np.int32)


@dataclass
class Tensor:
    """One generated input: storage bits for the library and exact fp64 values."""
    store: np.ndarray   # float32 array (fp32 workloads) or uint16 bf16 bits
    dtype: str          # "f32" or "bf16"

    @property
    def f64(self) -> np.ndarray:
        if self.dtype == "f32":
            return self.store.astype(np.float64)
        return bf16_bits_to_f64(self.store)

    @property
    def shape(self):
        return self.store.shape


def make(workload: int, index: int, shape, std: float, dtype: str) -> Tensor:
    x = normal(workload, index, shape, std)
    if dtype == "f32":
        return Tensor(x, "f32")
    return Tensor(to_bf16_bits(x), "bf16")


# ---------------------------------------------------------------------------
# Workload shapes (the five configurations the path is measured on).
# ---------------------------------------------------------------------------

WORKLOADS = {
    1: dict(name="tiny-mlp-embed-f32", dtype="f32", b=1, s=8, h=64, f=256, n=2,
            V=300, H=64, T=64, worked_ids=[0, 212, 7, 9]),
    2: dict(name="tp-mlp-shard-bf16", dtype="bf16", b=4, s=512, h=1024, f=4096, n=2),
    3: dict(name="gpt-layer-shard-bf16", dtype="bf16", b=1, s=2048, h=4096, f=16384,
            heads=8, d=512, n=2),
    4: dict(name="vocab-embed-tied-logits-bf16", dtype="bf16", b=8, s=2048, H=4096,
            V=50257, n=2),
    5: dict(name="gpt12-tp2-bf16", dtype="bf16", L=12, b=1, s=2048, h=4096, f=16384,
            heads=8, d=512, V=50257, n=2),
}


def mlp_inputs(w: int, M: int, h: int, f: int, dtype: str, base: int = 0):
    """X ~ N(0,1), A ~ N(0,0.02), B ~ N(0,0.02), dZ ~ N(0,1)."""
    return dict(X=make(w, base + 0, (M, h), 1.0, dtype),
                A=make(w, base + 1, (h, f), 0.02, dtype),
                B=make(w, base + 2, (f, h), 0.02, dtype),
                dZ=make(w, base + 3, (M, h), 1.0, dtype))


def attn_inputs(w: int, M: int, h: int, heads: int, d: int, dtype: str, base: int = 10):
    """X ~ N(0,1); W_Q, W_K, W_V (h x heads*d), W_O (heads*d x h) ~ N(0,0.02); dZ ~ N(0,1)."""
    hd = heads * d
    return dict(X=make(w, base + 0, (M, h), 1.0, dtype),
                WQ=make(w, base + 1, (h, hd), 0.02, dtype),
                WK=make(w, base + 2, (h, hd), 0.02, dtype),
                WV=make(w, base + 3, (h, hd), 0.02, dtype),
                WO=make(w, base + 4, (hd, h), 0.02, dtype),
                dZ=make(w, base + 5, (M, h), 1.0, dtype))


def embed_inputs(w: int, T: int, V: int, H: int, dtype: str, table_std: float,
                 worked_ids=None, base: int = 20):
    """Token ids uniform in [0, V) (prefixed by ``worked_ids`` when given),
    table E ~ N(0, table_std^2), X and dY ~ N(0,1)."""
    if worked_ids:
        rest = uniform_ids(w, base + 0, T - len(worked_ids), V)
        ids = np.concatenate([np.asarray(worked_ids, dtype=np.int32), rest])
    else:
        ids = uniform_ids(w, base + 0, T, V)
    return dict(ids=ids,
                E=make(w, base + 1, (V, H), table_std, dtype),
                X=make(w, base + 2, (T, H), 1.0, dtype),
                dY=make(w, base + 3, (T, H), 1.0, dtype))


def logit_grad(w: int, shard: int, T: int, rows: int, dtype: str, base: int = 30) -> Tensor:
    """dL_r ~ N(0,1) for shard r (T x rows)."""
    return make(w, base + shard, (T, rows), 1.0, dtype)


def gpt_inputs(w: int, L: int, M: int, H: int, width: int, f: int, V: int, shard_rows, ln_random: bool):
    """Seeded inputs of the stacked model: token ids (uniform in [0, V)), the
    table E ~ N(0, 0.02), per layer W_Q, W_K, W_V (H x width), W_O
    (width x H), A (H x f), B (f x H) ~ N(0, 0.02) and the LayerNorm
    parameters (gamma = 1, beta = 0, or with ``ln_random`` 1 + N(0, 0.1) and
    N(0, 0.1) in fp32), and one logit gradient dL_r ~ N(0, 1) per entry of
    ``shard_rows`` (the vocabulary rows of each shard).  All bf16 except the
    LayerNorm parameters.  Returns (ids, E, layers, dL)."""
    ids = uniform_ids(w, 0, M, V)
    E = make(w, 1, (V, H), 0.02, "bf16")
    layers = []
    k = 2
    for _ in range(L):
        lw = {}
        for name, sh in [("WQ", (H, width)), ("WK", (H, width)), ("WV", (H, width)),
                         ("WO", (width, H)), ("A", (H, f)), ("B", (f, H))]:
            lw[name] = make(w, k, sh, 0.02, "bf16")
            k += 1
        for name in ("g1", "b1", "g2", "b2"):
            base = 1.0 if name.startswith("g") else 0.0
            if ln_random:
                lw[name] = Tensor((base + 0.1 * normal(w, k, (H,))).astype(np.float32), "f32")
            else:
                lw[name] = Tensor(np.full(H, base, np.float32), "f32")
            k += 1
        layers.append(lw)
    dL = [make(w, 900 + r, (M, rows), 1.0, "bf16") for r, rows in enumerate(shard_rows)]
    return ids, E, layers, dL
