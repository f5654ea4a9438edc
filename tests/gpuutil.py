"""Host<->device conversion helpers for the GPU tests (no arithmetic of the
method: storage conversion, bit views and the error metric only)."""

import sys

import numpy as np
import torch

import synth


def say(msg: str):
    """Name the case on stdout before GPU work starts (flushed)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(t) -> torch.Tensor:
    """synth.Tensor (or raw array) -> device tensor with the same bits."""
    if isinstance(t, synth.Tensor):
        store, dt = t.store, t.dtype
    else:
        store = np.asarray(t)
        dt = "bf16" if store.dtype == np.uint16 else "f32"
    if dt == "f32":
        return torch.from_numpy(np.ascontiguousarray(store, dtype=np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(store).view(np.int16)).cuda().view(torch.bfloat16)


def ids_dev(ids) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()


def to_f64(x: torch.Tensor) -> np.ndarray:
    x = x.detach().contiguous().cpu()
    if x.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f64(x.view(torch.int16).numpy().view(np.uint16))
    return x.double().numpy()


def raw_bits(x: torch.Tensor) -> np.ndarray:
    x = x.detach().contiguous().cpu()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16).copy()
    return x.view(torch.int32).numpy().view(np.uint32).copy()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (the acceptance metric)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in the GPU result"
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def empty(shape, dtype, fill=None) -> torch.Tensor:
    """Device buffer pre-filled with NaN (or `fill`) so unwritten outputs show."""
    t = torch.empty(shape, dtype=dtype, device="cuda")
    if dtype in (torch.float32, torch.bfloat16):
        t.fill_(float("nan") if fill is None else fill)
    elif fill is not None:
        t.fill_(fill)
    return t


def workspace(nbytes: int) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device="cuda")


BF16_TOL = 1e-2   # max|err|/max|ref| on bf16 paths
F32_TOL = 1e-5    # on fp32 paths
