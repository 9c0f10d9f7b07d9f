"""A verify step captured in a HIP graph must reproduce the eager step on
every replay, with eager work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

import synth
from _gpu import dev, host

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import tree_draft_verification_amd as e3
    shape = synth.VerifyShape("graph", 22, B=3, Hq=8, Hkv=2, D=128, V=3001, n_drafts=60, depth=7, prefix=(10, 600))
    inp = synth.verify_inputs(shape, 0)
    W = dev(synth.lm_head_weight(shape, shape.V, shape.K))
    kc, vc, bt, pl = dev(inp.kv.k_cache), dev(inp.kv.v_cache), dev(inp.kv.block_table), dev(inp.kv.prefix_len)
    parent, q, kt, vt = dev(inp.parent), dev(inp.q), dev(inp.k_tree), dev(inp.v_tree)
    tok = dev(inp.plant_id)
    step = e3.VerifyStep(shape.B, shape.T, shape.Hq, shape.Hkv, shape.D, shape.V, kc, vc, bt, pl, W)
    step.run(parent, q, kt, vt, tok)
    torch.cuda.synchronize()
    names = ("attn", "hidden", "idx", "gap", "accept_len", "path", "out_tokens")
    want = {n: host(getattr(step, n)).copy() for n in names}
    g = step.graph(parent, q, kt, vt, tok)
    for rep in range(4):
        for n in names:                      # clobber outputs eagerly between replays
            getattr(step, n).zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in names:
            assert np.array_equal(host(getattr(step, n)), want[n]), (rep, n)
