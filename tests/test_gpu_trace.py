"""The library's launch tracer: every kernel launch of a call is named after
its entry point and kernel (GEMM launches also by template arguments and
shape), bracketed by events on its stream, and the filter selects launches
by substring."""

import pytest
import torch

from gpuutil import say

pytestmark = pytest.mark.gpu


def test_trace_names_and_filter():
    import megatron_tensor_transformer_columnparallel_amd as tp
    say("launch tracer around tp_mlp_fwd (M=256, h=512, f=1024, bf16)")
    M, h, f = 256, 512, 1024
    r = lambda *s: (torch.randn(s, device="cuda") * 0.02).to(torch.bfloat16)
    X, A, B = r(M, h), r(h, f), r(f, h)
    P, H, Z = r(M, f), r(M, f), r(M, h)
    tp.trace_start("", 64)
    tp.tp_mlp_fwd(X, A, B, P, H, Z)
    tp.trace_stop()
    recs = tp.trace_records()
    tp.trace_clear()
    assert len(recs) == 2
    (n0, ms0), (n1, ms1) = recs
    assert n0.startswith("tp_mlp_fwd:gemm_bf16_kernel <") and n0.endswith(f" {M}x{f}x{h} z1"), n0
    assert "EpiGelu" in n0 and "EpiStore" in n1, (n0, n1)
    assert n1.endswith(f" {M}x{h}x{f} z1"), n1
    assert ms0 > 0 and ms1 > 0
    # the filter keeps only matching launches
    tp.trace_start(f"{M}x{h}x{f}", 64)
    tp.tp_mlp_fwd(X, A, B, P, H, Z)
    tp.trace_stop()
    recs = tp.trace_records()
    tp.trace_clear()
    assert [n for n, _ in recs] == [n1]
