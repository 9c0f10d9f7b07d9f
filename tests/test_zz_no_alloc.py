"""The LM-head argmax entry point that allocates nothing
(eagle3_lmhead_argmax_noalloc: records in the library's own device array)
against the entry point that takes a caller workspace: same kernels, so the
results must be bit-identical. Two calls in a row, the second with fewer
rows (the array keeps the first call's records; every record the second call
reads it writes first)."""
import numpy as np
import pytest
import torch

import synth
from _gpu import dev, host

pytestmark = pytest.mark.gpu


def _call(e3, h, w, topk, want_lse, noalloc):
    M = h.shape[0]
    idx = torch.full((M, topk), -7, dtype=torch.int32, device="cuda")
    val = torch.full((M, topk), -7.0, dtype=torch.float32, device="cuda")
    gap = torch.full((M,), -7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((M,), -7.0, dtype=torch.float32, device="cuda") if want_lse else None
    if noalloc:
        e3.eagle3_lmhead_argmax_noalloc(h, w, topk, idx, val, gap, lse)
    else:
        need = e3.eagle3_lmhead_workspace(M, w.shape[0], h.shape[1], topk, e3.BF16)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        e3.eagle3_lmhead_argmax(h, w, topk, idx, val, gap, lse, ws)
    torch.cuda.synchronize()
    return [host(t) for t in (idx, val, gap) + ((lse,) if want_lse else ())]


def test_noalloc_matches_workspace_entry_point():
    import tree_draft_verification_amd as e3
    rng = np.random.default_rng(42)
    N, K = 32003, 1024
    w = dev(synth.normal_bf16(rng, (N, K), 0.3))
    # many-row GEMM-tile path (top-2), then few-row weight-stream path (top-10 + lse)
    for M, topk, want_lse in ((300, 2, False), (61, 10, True)):
        h = dev(synth.normal_bf16(rng, (M, K)))
        ref = _call(e3, h, w, topk, want_lse, noalloc=False)
        got = _call(e3, h, w, topk, want_lse, noalloc=True)
        for a, b in zip(got, ref):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b.view(np.uint32) if b.dtype == np.float32 else b), (M, topk)
        assert (got[0] >= 0).all() and (got[0] < N).all()
