"""The no-alloc variant of the input-side embedding gradient
(vocab_embed_bwd_noalloc, the library's static scratch in place of a caller
workspace) against the workspace entry point vocab_embed_bwd: identical bits
on two calls in a row, the second with fewer tokens, and the size limit."""

import numpy as np
import pytest
import torch

from gpuutil import raw_bits, say

pytestmark = pytest.mark.gpu


def _case(g, T, H, V, dt):
    ids = torch.from_numpy(g.integers(-3, V + 3, T).astype(np.int32)).cuda()     # a few ids outside [0, V)
    if T > 4:
        ids[1:4] = ids[0]                                                           # duplicates
    dY = torch.from_numpy(g.standard_normal((T, H)).astype(np.float32)).cuda().to(dt)
    return ids, dY


def test_noalloc_matches_workspace_entry_point():
    import megatron_tensor_transformer_columnparallel_amd as tp
    g = np.random.default_rng(4242)
    H, V = 256, 5000
    start, rows = tp.tps_partition(V, 2, 1)
    dE0 = torch.from_numpy(g.standard_normal((rows, H)).astype(np.float32)).cuda()   # the output-side part
    for T, dt in [(20000, torch.bfloat16), (1500, torch.bfloat16), (16384, torch.float32), (33, torch.float32)]:
        say(f"vocab_embed_bwd_noalloc T={T} H={H} rows={rows} start={start} dtype={dt}")
        ids, dY = _case(g, T, H, V, dt)
        ref = dE0.clone()
        ws = torch.empty(max(tp.vocab_embed_bwd_workspace(T, rows), 16), dtype=torch.uint8, device="cuda")
        tp.vocab_embed_bwd(ids, dY, ref, start, ws)
        got = dE0.clone()
        tp.vocab_embed_bwd_noalloc(ids, dY, got, start)
        torch.cuda.synchronize()
        assert np.array_equal(raw_bits(got), raw_bits(ref)), T


def test_noalloc_rejects_too_many_tokens():
    import megatron_tensor_transformer_columnparallel_amd as tp
    n = tp.vocab_embed_bwd_noalloc_max_tokens()
    assert n == 65536
    ids = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    dY = torch.zeros((n + 1, 8), dtype=torch.bfloat16, device="cuda")
    dE = torch.zeros((4, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(tp.TpsError, match="exceeds"):
        tp.vocab_embed_bwd_noalloc(ids, dY, dE, 0)
