"""ctypes binding of libtpshard (include/tpshard.h), same names as the C ABI.

Argument marshalling only: every function checks that the torch tensors it
is given are on the GPU with the expected dtype and shape, takes their
device pointers and the current HIP stream, and calls the C entry point.
All computation happens in the library's HIP kernels.  If the library has
not been built the import fails loudly; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpshard.so")

TPS_OK, TPS_EINVAL, TPS_EUNSUPPORTED, TPS_EWORKSPACE, TPS_EHIP = range(5)
TPS_F32, TPS_BF16 = 0, 1

# (name, restype, argtypes) for every symbol declared in include/tpshard.h.
_i64, _i32, _vp, _f32, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "tps_status_string": (ctypes.c_char_p, [_i32]),
    "tps_last_error": (ctypes.c_char_p, []),
    "tps_version": (ctypes.c_char_p, []),
    "tps_partition": (_i32, [_i64, _i32, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "tp_mlp_fwd": (_i32, [_i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "tp_mlp_bwd_workspace": (_sz, [_i32, _i64, _i64, _i64]),
    "tp_mlp_bwd": (_i32, [_i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "tp_attn_fwd_workspace": (_sz, [_i32, _i64, _i64, _i64, _i64, _i64]),
    "tp_attn_fwd": (_i32, [_i32, _i64, _i64, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                           _vp]),
    "tp_attn_bwd_workspace": (_sz, [_i32, _i64, _i64, _i64, _i64, _i64]),
    "tp_attn_bwd": (_i32, [_i32, _i64, _i64, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                           _vp, _vp, _vp, _vp, _sz, _vp]),
    "shard_reduce": (_i32, [_i32, _i32, _i32, ctypes.POINTER(_vp), _vp, _i64, _vp]),
    "shard_reduce_add": (_i32, [_i32, _vp, _i32, _i32, ctypes.POINTER(_vp), _i32, _vp, _i32, _vp, _i64, _vp]),
    "vocab_embed_fwd": (_i32, [_i32, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "vocab_embed_bwd_workspace": (_sz, [_i64, _i64]),
    "vocab_embed_bwd": (_i32, [_i32, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "vocab_embed_bwd_noalloc_max_tokens": (_i64, []),
    "vocab_embed_bwd_noalloc": (_i32, [_i32, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "tied_logits": (_i32, [_i32, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "tied_logits_bwd": (_i32, [_i32, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "embedding_fwd": (_i32, [_i32, _i32, _i32, ctypes.POINTER(_vp), _vp, _i64, _vp, _vp, _i64, _vp, _f32,
                             ctypes.c_uint64, _vp, _i64, _i64, _vp]),
    "dropout_apply": (_i32, [_i32, _i32, _i64, _vp, _f32, ctypes.c_uint64, _vp, _vp]),
    "shard_reduce_scatter": (_i32, [_i32, _i32, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                    ctypes.POINTER(_vp), _i64, _i64, _vp]),
    "shard_all_gather": (_i32, [_i32, _i32, ctypes.POINTER(_vp), _vp, _i64, _i64, _vp]),
    "column_linear_fwd": (_i32, [_i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _vp]),
    "column_linear_bwd": (_i32, [_i32, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp]),
    "row_linear_fwd": (_i32, [_i32, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _vp]),
    "row_linear_bwd": (_i32, [_i32, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _vp]),
    "shard_reduce_bias": (_i32, [_i32, _i32, ctypes.POINTER(_vp), _vp, _vp, _i64, _i64, _vp]),
    "vocab_ce_stats": (_i32, [_i32, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "vocab_ce_combine": (_i32, [_i32, ctypes.POINTER(_vp), _i64, _vp, _vp, _vp]),
    "vocab_ce_bwd": (_i32, [_i32, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "layernorm_fwd": (_i32, [_i32, _i32, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "layernorm_bwd_workspace": (_sz, [_i64, _i64]),
    "layernorm_bwd": (_i32, [_i32, _i32, _i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                             _vp]),
    "tps_trace_start": (_i32, [ctypes.c_char_p, _i32]),
    "tps_trace_stop": (_i32, []),
    "tps_trace_count": (_i32, []),
    "tps_trace_get": (_i32, [_i32, ctypes.c_char_p, _i32, ctypes.POINTER(_f32)]),
    "tps_trace_clear": (_i32, []),
    "layernorm_bwd_residual": (_i32, [_i32, _i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _sz, _vp]),
}


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m megatron_tensor_transformer_columnparallel_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()
LIB_PATH = _LIB_PATH


class TpsError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        msg = lib.tps_last_error().decode(errors="replace")
        super().__init__(f"{fn}: {lib.tps_status_string(status).decode()} ({msg})")


def _check(status: int, fn: str):
    if status != TPS_OK:
        raise TpsError(status, fn)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TPS_BF16
    if t.dtype == torch.float32:
        return TPS_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _same(dt: int, *ts):
    for t in ts:
        if _dt(t) != dt:
            raise TypeError("all activation/weight tensors must share one dtype")


def _contig(*ts):
    for t in ts:
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


# ------------------------------------------------------------------ host helpers

def tps_partition(total: int, n: int, r: int) -> tuple[int, int]:
    s, c = _i64(), _i64()
    _check(lib.tps_partition(total, n, r, ctypes.byref(s), ctypes.byref(c)), "tps_partition")
    return s.value, c.value


def tps_version() -> str:
    return lib.tps_version().decode()


# ------------------------------------------------------------------ MLP

def tp_mlp_fwd(X, A_i, B_i, P_i, H_i, Z_i, stream=None):
    dt = _dt(X)
    _same(dt, A_i, B_i, P_i, H_i, Z_i)
    _contig(X, A_i, B_i, P_i, H_i, Z_i)
    M, h = X.shape
    f = A_i.shape[1]
    assert A_i.shape == (h, f) and B_i.shape == (f, h) and P_i.shape == (M, f) and H_i.shape == (M, f)
    assert Z_i.shape == (M, h)
    _check(lib.tp_mlp_fwd(dt, M, h, f, _p(X), _p(A_i), _p(B_i), _p(P_i), _p(H_i), _p(Z_i), _stream(stream)),
           "tp_mlp_fwd")


def tp_mlp_bwd_workspace(dtype, M, h, f_i) -> int:
    return lib.tp_mlp_bwd_workspace(TPS_BF16 if dtype == torch.bfloat16 else TPS_F32, M, h, f_i)


def tp_mlp_bwd(X, A_i, B_i, P_i, H_i, dZ, dX_i, dA_i, dB_i, ws, stream=None):
    dt = _dt(X)
    _same(dt, A_i, B_i, P_i, H_i, dZ, dX_i, dA_i, dB_i)
    _contig(X, A_i, B_i, P_i, H_i, dZ, dX_i, dA_i, dB_i, ws)
    M, h = X.shape
    f = A_i.shape[1]
    assert dX_i.shape == (M, h) and dA_i.shape == (h, f) and dB_i.shape == (f, h) and dZ.shape == (M, h)
    _check(lib.tp_mlp_bwd(dt, M, h, f, _p(X), _p(A_i), _p(B_i), _p(P_i), _p(H_i), _p(dZ), _p(dX_i), _p(dA_i),
                          _p(dB_i), _p(ws), ws.numel() * ws.element_size(), _stream(stream)), "tp_mlp_bwd")


# ------------------------------------------------------------------ attention

def tp_attn_fwd_workspace(dtype, b, sq, h, hs, d) -> int:
    return lib.tp_attn_fwd_workspace(TPS_BF16 if dtype == torch.bfloat16 else TPS_F32, b, sq, h, hs, d)


def tp_attn_fwd(X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, Z_i, b, sq, hs, d, causal=True, ws=None, stream=None):
    """ws: uint8 device tensor of at least tp_attn_fwd_workspace(...) bytes;
    when omitted, one is taken from torch's allocator for this call."""
    dt = _dt(X)
    _same(dt, Wqkv_i, Wo_i, QKV_i, O_i, Z_i)
    _contig(X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, Z_i)
    M, h = X.shape
    assert M == b * sq and Wqkv_i.shape == (h, 3 * hs * d) and Wo_i.shape == (hs * d, h)
    assert QKV_i.shape == (M, 3 * hs * d) and O_i.shape == (M, hs * d) and Z_i.shape == (M, h)
    assert lse_i.dtype == torch.float32 and lse_i.numel() == b * hs * sq
    if ws is None:
        ws = torch.empty((tp_attn_fwd_workspace(X.dtype, b, sq, h, hs, d),), dtype=torch.uint8, device=X.device)
    _contig(ws)
    _check(lib.tp_attn_fwd(dt, b, sq, h, hs, d, 1 if causal else 0, _p(X), _p(Wqkv_i), _p(Wo_i), _p(QKV_i),
                           _p(O_i), _p(lse_i), _p(Z_i), _p(ws), ws.numel() * ws.element_size(),
                           _stream(stream)), "tp_attn_fwd")


def tp_attn_bwd_workspace(dtype, b, sq, h, hs, d) -> int:
    return lib.tp_attn_bwd_workspace(TPS_BF16 if dtype == torch.bfloat16 else TPS_F32, b, sq, h, hs, d)


def tp_attn_bwd(X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, dZ, dX_i, dWqkv_i, dWo_i, ws, b, sq, hs, d, causal=True,
                stream=None):
    dt = _dt(X)
    _same(dt, Wqkv_i, Wo_i, QKV_i, O_i, dZ, dX_i, dWqkv_i, dWo_i)
    _contig(X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, dZ, dX_i, dWqkv_i, dWo_i, ws)
    M, h = X.shape
    assert dX_i.shape == (M, h) and dWqkv_i.shape == Wqkv_i.shape and dWo_i.shape == Wo_i.shape
    _check(lib.tp_attn_bwd(dt, b, sq, h, hs, d, 1 if causal else 0, _p(X), _p(Wqkv_i), _p(Wo_i), _p(QKV_i),
                           _p(O_i), _p(lse_i), _p(dZ), _p(dX_i), _p(dWqkv_i), _p(dWo_i), _p(ws),
                           ws.numel() * ws.element_size(), _stream(stream)), "tp_attn_bwd")


# ------------------------------------------------------------------ reduce

def shard_reduce(parts, out, stream=None):
    if not 1 <= len(parts) <= 8:
        raise ValueError("1..8 parts")
    in_dt = _dt(parts[0])
    _same(in_dt, *parts)
    _contig(out, *parts)
    n = out.numel()
    for p in parts:
        assert p.numel() == n
    arr = (_vp * len(parts))(*[_p(p) for p in parts])
    _check(lib.shard_reduce(in_dt, _dt(out), len(parts), arr, _p(out), n, _stream(stream)), "shard_reduce")


def shard_reduce_add(res, parts, out, out_copy=None, stream=None):
    """out = res + sum(parts) in fp32 (in that order), rounded to out's dtype;
    optionally also written rounded to out_copy's dtype."""
    if not 1 <= len(parts) <= 7:
        raise ValueError("1..7 parts")
    pdt = _dt(parts[0])
    _same(pdt, *parts)
    _contig(res, out, *parts)
    n = out.numel()
    assert res.numel() == n and all(p.numel() == n for p in parts)
    cdt = TPS_BF16
    if out_copy is not None:
        _contig(out_copy)
        assert out_copy.numel() == n
        cdt = _dt(out_copy)
    arr = (_vp * len(parts))(*[_p(p) for p in parts])
    _check(lib.shard_reduce_add(_dt(res), _p(res), pdt, len(parts), arr, _dt(out), _p(out), cdt, _p(out_copy), n,
                                _stream(stream)), "shard_reduce_add")


# ------------------------------------------------------------------ embedding

def vocab_embed_fwd(ids, E_r, Y_r, v_start, stream=None):
    assert ids.dtype == torch.int32
    dt = _dt(E_r)
    _same(dt, Y_r)
    _contig(ids, E_r, Y_r)
    T = ids.numel()
    v_rows, H = E_r.shape
    assert Y_r.shape == (T, H)
    _check(lib.vocab_embed_fwd(dt, T, H, v_start, v_rows, _p(ids), _p(E_r), _p(Y_r), _stream(stream)),
           "vocab_embed_fwd")


def vocab_embed_bwd_workspace(T, v_rows) -> int:
    return lib.vocab_embed_bwd_workspace(T, v_rows)


def vocab_embed_bwd(ids, dY, dE_r, v_start, ws, stream=None):
    assert ids.dtype == torch.int32 and dE_r.dtype == torch.float32
    dt = _dt(dY)
    _contig(ids, dY, dE_r, ws)
    T = ids.numel()
    v_rows, H = dE_r.shape
    assert dY.shape == (T, H)
    _check(lib.vocab_embed_bwd(dt, T, H, v_start, v_rows, _p(ids), _p(dY), _p(dE_r), _p(ws),
                               ws.numel() * ws.element_size(), _stream(stream)), "vocab_embed_bwd")


def vocab_embed_bwd_noalloc_max_tokens() -> int:
    return lib.vocab_embed_bwd_noalloc_max_tokens()


def vocab_embed_bwd_noalloc(ids, dY, dE_r, v_start, stream=None):
    """vocab_embed_bwd with the library's static scratch instead of a workspace."""
    assert ids.dtype == torch.int32 and dE_r.dtype == torch.float32
    dt = _dt(dY)
    _contig(ids, dY, dE_r)
    T = ids.numel()
    v_rows, H = dE_r.shape
    assert dY.shape == (T, H)
    _check(lib.vocab_embed_bwd_noalloc(dt, T, H, v_start, v_rows, _p(ids), _p(dY), _p(dE_r), _stream(stream)),
           "vocab_embed_bwd_noalloc")


def tied_logits(X, E_r, L_r, stream=None):
    """L_r may be a column slice of a wider buffer: its row stride is passed as ldl."""
    dt = _dt(X)
    _same(dt, E_r, L_r)
    _contig(X, E_r)
    T, H = X.shape
    v_rows = E_r.shape[0]
    assert L_r.shape == (T, v_rows) and L_r.stride(1) == 1
    _check(lib.tied_logits(dt, T, H, v_rows, L_r.stride(0), _p(X), _p(E_r), _p(L_r), _stream(stream)),
           "tied_logits")


def tied_logits_bwd(X, E_r, dL_r, dX_r, dE_r, stream=None):
    dt = _dt(X)
    _same(dt, E_r, dL_r, dX_r)
    _contig(X, E_r, dX_r, dE_r)
    T, H = X.shape
    v_rows = E_r.shape[0]
    assert dL_r.shape == (T, v_rows) and dL_r.stride(1) == 1 and dE_r.dtype == torch.float32
    _check(lib.tied_logits_bwd(dt, T, H, v_rows, dL_r.stride(0), _p(X), _p(E_r), _p(dL_r), _p(dX_r), _p(dE_r),
                               _stream(stream)), "tied_logits_bwd")


# ------------------------------------------------------------------ full embedding, dropout

def embedding_fwd(word_parts, PE, pos, out, p=0.0, seed=0, TE=None, tt=None, stream=None):
    """out <- dropout(sum(word_parts) + PE[pos] (+ TE[tt])) with Philox4x32-10 keyed by seed."""
    n = len(word_parts)
    if not 1 <= n <= 8:
        raise ValueError("1..8 word partials")
    dt = _dt(word_parts[0])
    _same(dt, PE, *word_parts, *([TE] if TE is not None else []))
    _contig(out, PE, pos, *word_parts, *([TE, tt] if TE is not None else []))
    T, H = out.shape
    assert all(w.shape == (T, H) for w in word_parts) and PE.shape[1] == H and pos.dtype == torch.int32
    if TE is not None:
        assert TE.shape[1] == H and tt is not None and tt.dtype == torch.int32
    arr = (_vp * n)(*[_p(w) for w in word_parts])
    _check(lib.embedding_fwd(dt, _dt(out), n, arr, _p(PE), PE.shape[0], _p(pos), _p(TE),
                             TE.shape[0] if TE is not None else 0, _p(tt), float(p), int(seed), _p(out), T, H,
                             _stream(stream)), "embedding_fwd")


def dropout_apply(x, y, p, seed, stream=None):
    """y <- keep ? x / (1 - p) : 0 (the mask from seed and element index); also the backward."""
    _contig(x, y)
    assert x.numel() == y.numel()
    _check(lib.dropout_apply(_dt(x), _dt(y), x.numel(), _p(x), float(p), int(seed), _p(y), _stream(stream)),
           "dropout_apply")


# ------------------------------------------------------------------ sequence parallelism

def shard_reduce_scatter(parts, outs, res=None, stream=None):
    """outs[r] <- (res[r] +) shard r's rows of sum(parts); rows split as tps_partition(M, n, r)."""
    n = len(parts)
    if not 1 <= n <= 8 or len(outs) != n or (res is not None and len(res) != n):
        raise ValueError("1..8 parts, one output (and residual) per part")
    pdt, odt = _dt(parts[0]), _dt(outs[0])
    _same(pdt, *parts)
    _same(odt, *outs, *(res or []))
    _contig(*parts, *outs, *(res or []))
    M, H = parts[0].shape
    for r in range(n):
        _, c = tps_partition(M, n, r)
        assert parts[r].shape == (M, H) and outs[r].shape == (c, H)
        if res is not None:
            assert res[r].shape == (c, H)
    arr = lambda ts: (_vp * n)(*[_p(t) for t in ts])
    _check(lib.shard_reduce_scatter(pdt, odt, n, arr(parts), arr(res) if res is not None else None, arr(outs), M, H,
                                    _stream(stream)), "shard_reduce_scatter")


def shard_all_gather(parts, out, stream=None):
    """out [M x H] <- the shards' row slices stacked in shard order."""
    n = len(parts)
    if not 1 <= n <= 8:
        raise ValueError("1..8 parts")
    dt = _dt(out)
    _same(dt, *parts)
    _contig(out, *parts)
    M, H = out.shape
    for r in range(n):
        assert parts[r].shape == (tps_partition(M, n, r)[1], H)
    arr = (_vp * n)(*[_p(t) for t in parts])
    _check(lib.shard_all_gather(dt, n, arr, _p(out), M, H, _stream(stream)), "shard_all_gather")


# ------------------------------------------------------------------ column / row parallel linear

def column_linear_fwd(X, A_r, Y, b_r=None, stream=None):
    """Y (a [M x n_r] view; may be a column slice of the gathered output) <- X A_r (+ b_r)."""
    dt = _dt(X)
    _same(dt, A_r, Y, *([b_r] if b_r is not None else []))
    _contig(X, A_r)
    M, h = X.shape
    n = A_r.shape[1]
    assert A_r.shape == (h, n) and Y.shape == (M, n) and Y.stride(1) == 1
    if b_r is not None:
        _contig(b_r)
        assert b_r.numel() == n
    _check(lib.column_linear_fwd(dt, M, h, n, _p(X), _p(A_r), _p(b_r), _p(Y), Y.stride(0), _stream(stream)),
           "column_linear_fwd")


def column_linear_bwd(X, A_r, dY, dX_r, dA_r, db_r=None, stream=None):
    """dX_r (partial), dA_r, db_r (fp32, optional) for dY [M x n_r] (may be a column slice)."""
    dt = _dt(X)
    _same(dt, A_r, dY, dX_r, dA_r)
    _contig(X, A_r, dX_r, dA_r)
    M, h = X.shape
    n = A_r.shape[1]
    assert dY.shape == (M, n) and dY.stride(1) == 1 and dX_r.shape == (M, h) and dA_r.shape == (h, n)
    if db_r is not None:
        _contig(db_r)
        assert db_r.dtype == torch.float32 and db_r.numel() == n
    _check(lib.column_linear_bwd(dt, M, h, n, _p(X), _p(A_r), _p(dY), dY.stride(0), _p(dX_r), _p(dA_r), _p(db_r),
                                 _stream(stream)), "column_linear_bwd")


def row_linear_fwd(X_r, B_r, Y_r, stream=None):
    """Y_r (partial) <- X_r B_r; X_r [M x k_r] may be a column slice of the full input."""
    dt = _dt(X_r)
    _same(dt, B_r, Y_r)
    _contig(B_r, Y_r)
    M, k = X_r.shape
    h = B_r.shape[1]
    assert X_r.stride(1) == 1 and B_r.shape == (k, h) and Y_r.shape == (M, h)
    _check(lib.row_linear_fwd(dt, M, k, h, _p(X_r), X_r.stride(0), _p(B_r), _p(Y_r), _stream(stream)),
           "row_linear_fwd")


def row_linear_bwd(X_r, B_r, dY, dX_r, dB_r, db=None, stream=None):
    """dX_r (may be a column slice of the gathered dX), dB_r, db (fp32, optional) for the full dY."""
    dt = _dt(X_r)
    _same(dt, B_r, dY, dX_r, dB_r)
    _contig(B_r, dY, dB_r)
    M, k = X_r.shape
    h = B_r.shape[1]
    assert X_r.stride(1) == 1 and dX_r.shape == (M, k) and dX_r.stride(1) == 1 and dY.shape == (M, h)
    assert dB_r.shape == (k, h)
    if db is not None:
        _contig(db)
        assert db.dtype == torch.float32 and db.numel() == h
    _check(lib.row_linear_bwd(dt, M, k, h, _p(X_r), X_r.stride(0), _p(B_r), _p(dY), _p(dX_r), dX_r.stride(0),
                              _p(dB_r), _p(db), _stream(stream)), "row_linear_bwd")


def shard_reduce_bias(parts, bias, out, stream=None):
    """out [M x N] <- sum(parts) + bias (fp32 sum in shard order, one rounding)."""
    if not 1 <= len(parts) <= 8:
        raise ValueError("1..8 parts")
    dt = _dt(out)
    _same(dt, bias, *parts)
    _contig(out, bias, *parts)
    M, N = out.shape
    assert bias.numel() == N and all(p.shape == (M, N) for p in parts)
    arr = (_vp * len(parts))(*[_p(p) for p in parts])
    _check(lib.shard_reduce_bias(dt, len(parts), arr, _p(bias), _p(out), M, N, _stream(stream)),
           "shard_reduce_bias")


# ------------------------------------------------------------------ vocab-parallel cross entropy

def vocab_ce_stats(L_r, targets, stats_r, v_start, stream=None):
    """stats_r [T x 4] fp32 <- one shard's (max, exp-sum, target logit, owned).
    L_r may be a column slice of a wider buffer: its row stride is passed as ldl."""
    dt = _dt(L_r)
    T, v_rows = L_r.shape
    assert L_r.stride(1) == 1 and targets.dtype == torch.int32 and targets.numel() == T
    assert stats_r.dtype == torch.float32 and stats_r.shape == (T, 4)
    _contig(targets, stats_r)
    _check(lib.vocab_ce_stats(dt, T, v_rows, L_r.stride(0), v_start, _p(L_r), _p(targets), _p(stats_r),
                              _stream(stream)), "vocab_ce_stats")


def vocab_ce_combine(stats, loss, lse, stream=None):
    """loss, lse [T] fp32 <- every shard's statistics."""
    if not 1 <= len(stats) <= 8:
        raise ValueError("1..8 shards")
    T = loss.numel()
    _contig(loss, lse, *stats)
    assert lse.numel() == T and all(s.shape == (T, 4) and s.dtype == torch.float32 for s in stats)
    arr = (_vp * len(stats))(*[_p(s) for s in stats])
    _check(lib.vocab_ce_combine(len(stats), arr, T, _p(loss), _p(lse), _stream(stream)), "vocab_ce_combine")


def vocab_ce_bwd(L_r, targets, lse, dloss, dL_r, v_start, stream=None):
    """dL_r <- dloss * (softmax - onehot of the owned target); dL_r may be L_r.
    Both share L_r's row stride."""
    dt = _dt(L_r)
    _same(dt, dL_r)
    T, v_rows = L_r.shape
    assert dL_r.shape == (T, v_rows) and dL_r.stride() == L_r.stride() and L_r.stride(1) == 1
    assert targets.dtype == torch.int32 and targets.numel() == T
    _contig(targets, lse, dloss)
    _check(lib.vocab_ce_bwd(dt, T, v_rows, L_r.stride(0), v_start, _p(L_r), _p(targets), _p(lse), _p(dloss),
                            _p(dL_r), _stream(stream)), "vocab_ce_bwd")


# ------------------------------------------------------------------ LayerNorm

def layernorm_fwd(x, gamma, beta, y, mean, rstd, eps=1e-5, stream=None):
    """x and y may differ in dtype (e.g. an fp32 residual stream in, bf16 out)."""
    _contig(x, gamma, beta, y, mean, rstd)
    M, H = x.shape
    assert y.shape == (M, H)
    _check(lib.layernorm_fwd(_dt(x), _dt(y), M, H, eps, _p(x), _p(gamma), _p(beta), _p(y), _p(mean), _p(rstd),
                             _stream(stream)), "layernorm_fwd")


def layernorm_bwd_workspace(M, H) -> int:
    return lib.layernorm_bwd_workspace(M, H)


def layernorm_bwd(x, gamma, mean, rstd, dy, dx, dgamma, dbeta, ws, stream=None):
    """x, dy and dx may each be fp32 or bf16."""
    _contig(x, gamma, mean, rstd, dy, dx, dgamma, dbeta, ws)
    M, H = x.shape
    assert dy.shape == (M, H) and dx.shape == (M, H)
    _check(lib.layernorm_bwd(_dt(x), _dt(dy), _dt(dx), M, H, _p(x), _p(gamma), _p(mean), _p(rstd), _p(dy), _p(dx),
                             _p(dgamma), _p(dbeta), _p(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "layernorm_bwd")


def layernorm_bwd_residual(x, gamma, mean, rstd, dy, res, out, dgamma, dbeta, ws, out_copy=None, stream=None):
    """out = res + (LayerNorm gradient), fp32; x and dy fp32 or bf16; optional bf16 copy of out."""
    _contig(x, gamma, mean, rstd, dy, res, out, dgamma, dbeta, ws)
    M, H = x.shape
    assert dy.shape == (M, H) and res.shape == (M, H) and out.shape == (M, H)
    assert res.dtype == torch.float32 and out.dtype == torch.float32
    if out_copy is not None:
        _contig(out_copy)
        assert out_copy.shape == (M, H) and out_copy.dtype == torch.bfloat16
    _check(lib.layernorm_bwd_residual(_dt(x), _dt(dy), M, H, _p(x), _p(gamma), _p(mean), _p(rstd), _p(dy), _p(res),
                                      _p(out), _p(out_copy), _p(dgamma),
                                      _p(dbeta), _p(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "layernorm_bwd_residual")


# ---------------------------------------------------------------- launch tracing

def trace_start(filter: str = "", max_records: int = 65536):
    """Record timing events around every library kernel launch whose name
    contains ``filter`` (see tps_trace_start)."""
    _check(lib.tps_trace_start(filter.encode(), max_records), "tps_trace_start")


def trace_stop():
    _check(lib.tps_trace_stop(), "tps_trace_stop")


def trace_records():
    """[(name, ms)] of the recorded launches (waits for each to finish)."""
    out = []
    buf = ctypes.create_string_buffer(512)
    ms = ctypes.c_float()
    for i in range(lib.tps_trace_count()):
        _check(lib.tps_trace_get(i, buf, len(buf), ctypes.byref(ms)), "tps_trace_get")
        out.append((buf.value.decode(), ms.value))
    return out


def trace_clear():
    _check(lib.tps_trace_clear(), "tps_trace_clear")
