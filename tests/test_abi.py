"""C-ABI checks that need no GPU: the library loads, exports every function
include/tpshard.h declares, the host-only partition helper matches the pages'
examples, and argument validation rejects bad calls before any HIP work is
enqueued (those calls return before touching the device)."""

import ctypes
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpshard.h")


def _declared():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\*?\s+\**([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def tp():
    import megatron_tensor_transformer_columnparallel_amd as tp
    return tp


def test_header_declares_the_path():
    names = _declared()
    for must in ["tp_mlp_fwd", "tp_mlp_bwd", "tp_attn_fwd", "tp_attn_bwd", "shard_reduce",
                 "vocab_embed_fwd", "vocab_embed_bwd", "tied_logits", "tied_logits_bwd",
                 "layernorm_fwd", "layernorm_bwd", "tps_partition",
                 "vocab_ce_stats", "vocab_ce_combine", "vocab_ce_bwd",
                 "column_linear_fwd", "column_linear_bwd", "row_linear_fwd", "row_linear_bwd",
                 "shard_reduce_bias", "shard_reduce_scatter", "shard_all_gather",
                 "embedding_fwd", "dropout_apply"]:
        assert must in names


def test_library_exports_every_declared_symbol(tp):
    raw = ctypes.CDLL(tp.LIB_PATH)
    for name in _declared():
        assert hasattr(raw, name), f"{name} declared in tpshard.h but not exported"
    assert set(_declared()) == set(tp.binding.SIGNATURES), "binding and header disagree"


def test_partition_matches_page_examples(tp):
    with open(os.path.join(ROOT, "tests", "golden", "partition_examples.json"), encoding="utf-8") as f:
        g = json.load(f)
    for case in g["cases"]:
        got = [list(tp.tps_partition(case["total"], case["n"], r)) for r in range(case["n"])]
        assert got == case["shards"]


def test_partition_rejects_bad_arguments(tp):
    for args in [(10, 0, 0), (10, 2, 2), (10, 2, -1), (-1, 2, 0)]:
        with pytest.raises(tp.TpsError) as e:
            tp.tps_partition(*args)
        assert e.value.status == tp.binding.TPS_EINVAL


def test_status_strings(tp):
    lib = tp.lib
    assert lib.tps_status_string(0) == b"ok"
    assert lib.tps_status_string(1) == b"invalid argument"
    assert lib.tps_version().startswith(b"tpshard")


ALIGNED = 1 << 20  # a fake, 16-byte aligned address: validation fails before any use


@pytest.mark.parametrize("case", [
    ("tp_mlp_fwd", (1, 0, 64, 128, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, None)),   # M = 0
    ("tp_mlp_fwd", (1, 8, 60, 128, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, None)),   # h % 8
    ("tp_mlp_fwd", (1, 8, 64, 128, None, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, None)),      # null X
    ("tp_mlp_fwd", (1, 8, 64, 128, ALIGNED + 2, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, None)),  # misaligned
    ("tp_mlp_fwd", (7, 8, 64, 128, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, None)),   # bad dtype
    ("tied_logits", (1, 16, 64, 150, 144, ALIGNED, ALIGNED, ALIGNED, None)),                      # ldl < v_rows
    ("tied_logits", (1, 16, 64, 150, 154, ALIGNED, ALIGNED, ALIGNED, None)),                      # ldl % 8
    ("vocab_embed_fwd", (1, 16, 64, 0, 0, ALIGNED, ALIGNED, ALIGNED, None)),                      # v_rows = 0
    ("vocab_embed_fwd", (1, 16, 64, -1, 10, ALIGNED, ALIGNED, ALIGNED, None)),                    # v_start < 0
    ("tp_attn_fwd", (1, 1, 64, 256, 2, 64, 1, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED,
                     ALIGNED, 1 << 30, None)),                                                      # null lse
    ("tp_attn_fwd", (1, 1, 64, 256, 2, 60, 1, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED,
                     ALIGNED, 1 << 30, None)),                                                      # d % 8
    ("layernorm_fwd", (0, 1, 4, 0, 1e-5, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, None)),
    ("layernorm_fwd", (0, 1, 4, 12, 1e-5, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, None)),  # H % 8
    ("shard_reduce_add", (0, ALIGNED, 1, 0, None, 0, ALIGNED, 1, None, 16, None)),                  # n_parts = 0
    ("vocab_ce_stats", (1, 16, 150, 144, 0, ALIGNED, ALIGNED, ALIGNED, None)),                      # ldl < v_rows
    ("vocab_ce_stats", (1, 16, 150, 154, 0, ALIGNED, ALIGNED, ALIGNED, None)),                      # ldl % 8
    ("vocab_ce_stats", (1, 16, 0, 152, 0, ALIGNED, ALIGNED, ALIGNED, None)),                        # v_rows = 0
    ("vocab_ce_stats", (1, 16, 150, 152, -1, ALIGNED, ALIGNED, ALIGNED, None)),                     # v_start < 0
    ("vocab_ce_stats", (1, 16, 150, 152, 0, ALIGNED, None, ALIGNED, None)),                         # null targets
    ("vocab_ce_stats", (1, 16, 150, 152, 0, ALIGNED, ALIGNED, ALIGNED + 4, None)),                  # misaligned
    ("vocab_ce_stats", (5, 16, 150, 152, 0, ALIGNED, ALIGNED, ALIGNED, None)),                      # bad dtype
    ("vocab_ce_stats", (0, -1, 150, 152, 0, ALIGNED, ALIGNED, ALIGNED, None)),                      # T < 0
    ("vocab_ce_bwd", (1, 16, 150, 152, 0, ALIGNED, ALIGNED, None, ALIGNED, ALIGNED, None)),         # null lse
    ("vocab_ce_bwd", (1, 16, 150, 152, 0, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED + 2, None)),  # misaligned dL
    ("vocab_ce_bwd", (0, 16, 150, 150, 0, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, None)),      # fp32 ldl % 4
    ("column_linear_fwd", (1, 8, 64, 128, ALIGNED, ALIGNED, None, ALIGNED, 120, None)),             # ldy < n_r
    ("column_linear_fwd", (1, 8, 60, 128, ALIGNED, ALIGNED, None, ALIGNED, 128, None)),             # h_in % 8
    ("column_linear_fwd", (1, 0, 64, 128, ALIGNED, ALIGNED, None, ALIGNED, 128, None)),             # M = 0
    ("column_linear_fwd", (1, 8, 64, 128, None, ALIGNED, None, ALIGNED, 128, None)),                # null X
    ("column_linear_fwd", (1, 8, 64, 128, ALIGNED, ALIGNED, ALIGNED + 2, ALIGNED, 128, None)),      # bias align
    ("column_linear_bwd", (1, 8, 64, 128, ALIGNED, ALIGNED, ALIGNED, 124, ALIGNED, ALIGNED, None, None)),  # lddy
    ("column_linear_bwd", (3, 8, 64, 128, ALIGNED, ALIGNED, ALIGNED, 128, ALIGNED, ALIGNED, None, None)),  # dtype
    ("row_linear_fwd", (1, 8, 64, 128, ALIGNED, 56, ALIGNED, ALIGNED, None)),                       # ldx < k_r
    ("row_linear_fwd", (1, 8, 64, 124, ALIGNED, 64, ALIGNED, ALIGNED, None)),                       # h_out % 8
    ("row_linear_bwd", (1, 8, 64, 128, ALIGNED, 64, ALIGNED, ALIGNED, ALIGNED, 60, ALIGNED, None, None)),  # lddx
    ("row_linear_bwd", (1, 8, 64, 128, ALIGNED, 64, ALIGNED, ALIGNED, None, 64, ALIGNED, None, None)),    # null dX
])
def test_validation_rejects_before_enqueue(tp, case):
    name, args = case
    st = getattr(tp.lib, name)(*args)
    assert st == tp.binding.TPS_EINVAL, (name, st, tp.lib.tps_last_error())
    assert tp.lib.tps_last_error().startswith(name.encode())


def test_shard_reduce_validation(tp):
    lib = tp.lib
    arr = (ctypes.c_void_p * 9)(*([ALIGNED] * 9))
    assert lib.shard_reduce(1, 1, 0, arr, ALIGNED, 16, None) == tp.binding.TPS_EINVAL
    assert lib.shard_reduce(1, 1, 9, arr, ALIGNED, 16, None) == tp.binding.TPS_EINVAL
    arr2 = (ctypes.c_void_p * 2)(ALIGNED, ALIGNED + 4)
    assert lib.shard_reduce(1, 1, 2, arr2, ALIGNED, 16, None) == tp.binding.TPS_EINVAL
    assert lib.shard_reduce(1, 1, 2, arr, ALIGNED, -1, None) == tp.binding.TPS_EINVAL


def test_workspace_queries_and_too_small_workspace(tp):
    lib = tp.lib
    assert lib.tp_mlp_bwd_workspace(1, 2048, 1024, 2048) == 2048 * 2048 * 2
    # sort keys (next power of two of T) + 256 row-bucket counts
    assert lib.vocab_embed_bwd_workspace(16384, 25129) == 16384 * 8
    assert lib.vocab_embed_bwd_workspace(20000, 25129) == 32768 * 8
    assert lib.layernorm_bwd_workspace(2048, 4096) == 256 * 2 * 4096 * 4
    need = lib.tp_mlp_bwd_workspace(1, 8, 64, 128)
    st = lib.tp_mlp_bwd(1, 8, 64, 128, *([ALIGNED] * 10), need - 1, None)
    assert st == tp.binding.TPS_EWORKSPACE
    ws = lib.tp_attn_bwd_workspace(1, 1, 2048, 4096, 4, 512)
    assert ws >= 2048 * 4 * 512 * 2 + 4 * 2048 * 4 + 2 * 4 * 2048 * 2048 * 2 + 2048 * 3 * 2048 * 2
    st = lib.tp_attn_bwd(1, 1, 2048, 4096, 4, 512, 1, *([ALIGNED] * 11), ws - 1, None)
    assert st == tp.binding.TPS_EWORKSPACE
    # backward through the flash kernels (head dims 64..256): dO and dQKV
    # (bf16), one fp32 row term per query and head, and fp32 partials of
    # split blocks for about one work item per CU whatever the sequence
    # length; nothing per (query, key) pair
    for b, sq, hs, d in [(1, 8192, 2, 128), (2, 300, 3, 64), (1, 32768, 4, 256), (1, 131072, 1, 64)]:
        wb = lib.tp_attn_bwd_workspace(1, b, sq, 4096, hs, d)
        need = b * sq * hs * d * 2 + b * sq * 3 * hs * d * 2 + b * hs * sq * 4
        items = 3 * max(256, b * hs * -(-sq // 64))   # rounds of CU items, at least one per block
        assert need <= wb <= need + items * 128 * (3 * d + 2) * 4 + 8 * 256, (b, sq, hs, d, wb, need)
        if sq >= 8192:   # against the score path's bf16 P, fp32 dP and bf16 dS per (query, key) and head
            assert wb < b * hs * sq * sq * 8 // 10
    # the query covers both masks' plans; a call checks its own plan's need,
    # which always includes dO and dQKV
    small = 300 * 2 * 64 * 2 + 300 * 3 * 2 * 64 * 2 - 1
    for causal in (0, 1):
        st = lib.tp_attn_bwd(1, 1, 300, 4096, 2, 64, causal, *([ALIGNED] * 11), small, None)
        assert st == tp.binding.TPS_EWORKSPACE
    # forward through the flash kernels (head dims 64, 128, 256, 512): fp32
    # partial outputs of the key chunks, about one item of at most 256 rows
    # per compute unit whatever the sequence length (no per-(query, key)
    # storage)
    def bound(b, sq, hs, d):   # about one round of items, at least one per 128-row query block
        return 2 * max(256 * 256, b * hs * -(-sq // 128) * 128) * (d + 2) * 4
    wf = lib.tp_attn_fwd_workspace(1, 1, 8192, 4096, 4, 512)
    assert 0 < wf <= bound(1, 8192, 4, 512)
    assert lib.tp_attn_fwd_workspace(1, 1, 32768, 4096, 4, 512) <= bound(1, 32768, 4, 512) < 4 * 32768 ** 2
    assert 0 < lib.tp_attn_fwd_workspace(1, 1, 2048, 1024, 4, 256) <= bound(1, 2048, 4, 256)
    st = lib.tp_attn_fwd(1, 1, 8192, 4096, 4, 512, 1, *([ALIGNED] * 8), wf - 1, None)
    assert st == tp.binding.TPS_EWORKSPACE
    assert 0 < lib.tp_attn_fwd_workspace(1, 1, 2048, 4096, 4, 512) <= bound(1, 2048, 4, 512)
    # other head dims: fp32 log2-domain scores + bf16 probabilities per (batch, head)
    wo = lib.tp_attn_fwd_workspace(1, 1, 2048, 4096, 4, 96)
    assert wo >= 4 * 2048 * 2048 * (4 + 2)
    assert lib.tp_attn_fwd_workspace(1, 1, 300, 480, 5, 96) >= 5 * 300 * 304 * (4 + 2)
    st = lib.tp_attn_fwd(1, 1, 2048, 4096, 4, 96, 1, *([ALIGNED] * 8), wo - 1, None)
    assert st == tp.binding.TPS_EWORKSPACE


def test_attention_fp32_is_reported_unsupported(tp):
    st = tp.lib.tp_attn_fwd(0, 1, 16, 64, 2, 64, 1, *([ALIGNED] * 8), 1 << 30, None)
    assert st == tp.binding.TPS_EUNSUPPORTED


def test_layernorm_bwd_residual_validation(tp):
    lib = tp.lib
    need = lib.layernorm_bwd_workspace(64, 4096)
    args = [ALIGNED] * 5   # x, gamma, mean, rstd, dy
    # out aliasing res is rejected before anything is enqueued
    st = lib.layernorm_bwd_residual(0, 0, 64, 4096, *args, ALIGNED + 64, ALIGNED + 64, None, ALIGNED, ALIGNED,
                                    ALIGNED, need, None)
    assert st == tp.binding.TPS_EINVAL
    # too small a workspace
    st = lib.layernorm_bwd_residual(0, 0, 64, 4096, *args, ALIGNED, ALIGNED + 64, None, ALIGNED, ALIGNED,
                                    ALIGNED, need - 1, None)
    assert st == tp.binding.TPS_EWORKSPACE
    # misaligned copy
    st = lib.layernorm_bwd_residual(0, 0, 64, 4096, *args, ALIGNED, ALIGNED + 64, ALIGNED + 2, ALIGNED, ALIGNED,
                                    ALIGNED, need, None)
    assert st == tp.binding.TPS_EINVAL


def test_vocab_ce_combine_validation(tp):
    lib = tp.lib
    ok = (ctypes.c_void_p * 9)(*([ALIGNED] * 9))
    for n in (0, 9):
        assert lib.vocab_ce_combine(n, ok, 16, ALIGNED, ALIGNED, None) == tp.binding.TPS_EINVAL
    bad = (ctypes.c_void_p * 2)(ALIGNED, None)
    assert lib.vocab_ce_combine(2, bad, 16, ALIGNED, ALIGNED, None) == tp.binding.TPS_EINVAL
    mis = (ctypes.c_void_p * 2)(ALIGNED, ALIGNED + 8)
    assert lib.vocab_ce_combine(2, mis, 16, ALIGNED, ALIGNED, None) == tp.binding.TPS_EINVAL
    assert lib.vocab_ce_combine(2, ok, 16, None, ALIGNED, None) == tp.binding.TPS_EINVAL
    assert lib.tps_last_error().startswith(b"vocab_ce_combine")


def test_shard_reduce_bias_validation(tp):
    lib = tp.lib
    arr = (ctypes.c_void_p * 9)(*([ALIGNED] * 9))
    for n in (0, 9):
        assert lib.shard_reduce_bias(1, n, arr, ALIGNED, ALIGNED, 4, 16, None) == tp.binding.TPS_EINVAL
    assert lib.shard_reduce_bias(1, 2, arr, ALIGNED, ALIGNED, 4, 12, None) == tp.binding.TPS_EINVAL   # N % 8
    assert lib.shard_reduce_bias(1, 2, arr, None, ALIGNED, 4, 16, None) == tp.binding.TPS_EINVAL      # null bias
    assert lib.tps_last_error().startswith(b"shard_reduce_bias")


def test_sequence_parallel_exchange_validation(tp):
    lib = tp.lib
    arr = (ctypes.c_void_p * 9)(*([ALIGNED] * 9))
    bad = (ctypes.c_void_p * 2)(ALIGNED, ALIGNED + 4)
    E = tp.binding.TPS_EINVAL
    assert lib.shard_reduce_scatter(1, 1, 0, arr, None, arr, 8, 16, None) == E          # n_parts = 0
    assert lib.shard_reduce_scatter(1, 1, 2, arr, None, arr, 8, 12, None) == E          # H % 8
    assert lib.shard_reduce_scatter(1, 1, 2, arr, None, bad, 8, 16, None) == E          # misaligned slice
    assert lib.shard_reduce_scatter(5, 1, 2, arr, None, arr, 8, 16, None) == E          # dtype
    assert lib.tps_last_error().startswith(b"shard_reduce_scatter")
    assert lib.shard_all_gather(1, 9, arr, ALIGNED, 8, 16, None) == E                   # n_parts = 9
    assert lib.shard_all_gather(1, 2, arr, None, 8, 16, None) == E                      # null out
    assert lib.shard_all_gather(1, 2, bad, ALIGNED, 8, 16, None) == E                   # misaligned part
    assert lib.tps_last_error().startswith(b"shard_all_gather")


def test_embedding_and_dropout_validation(tp):
    lib = tp.lib
    arr = (ctypes.c_void_p * 2)(ALIGNED, ALIGNED)
    E = tp.binding.TPS_EINVAL
    args = [1, 1, 2, arr, ALIGNED, 64, ALIGNED, None, 0, None, 0.1, 7, ALIGNED, 16, 64, None]
    for i, bad in [(10, 1.0), (10, -0.5), (14, 60), (5, 0), (4, None), (12, ALIGNED + 2), (2, 9)]:
        a = list(args)
        a[i] = bad
        if i == 4:
            a[4] = None
        assert lib.embedding_fwd(*a) == E, (i, bad)
    assert lib.tps_last_error().startswith(b"embedding_fwd")
    assert lib.dropout_apply(1, 1, 16, ALIGNED, 1.0, 3, ALIGNED, None) == E                      # p = 1
    assert lib.dropout_apply(1, 1, 16, ALIGNED + 8, 0.5, 3, ALIGNED, None) == E                  # misaligned
    assert lib.dropout_apply(1, 1, -1, ALIGNED, 0.5, 3, ALIGNED, None) == E                      # n < 0
    assert lib.tps_last_error().startswith(b"dropout_apply")


def test_trace_rejects_bad_record_counts(tp):
    for n in (0, -1, (1 << 20) + 1):
        with pytest.raises(tp.TpsError):
            tp.trace_start("", n)
    assert tp.lib.tps_trace_count() == 0
