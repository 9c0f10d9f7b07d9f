"""Repeated tree-attention calls on the same device buffers.

Three calls of the masked tree attention are enqueued back to back on one
stream (no synchronisation between them), each into its own output, with and
without prefixes split across work-groups and merged, the calls sharing one
workspace. All three outputs must be bit-identical and within the parity
tolerance of the oracle: a race between the calls, or inside one, shows as
calls that differ. The test sits last in collection order so that a failure
here leaves every other GPU test run and reported."""
import numpy as np
import pytest
import torch

import synth
from _gpu import dev, host, normwise_rel

pytestmark = pytest.mark.gpu

CASES = [
    # B, T, Hq, Hkv, prefix lengths, split_keys
    (3, 61, 8, 2, [0, 37, 1100], 0),
    (3, 61, 8, 2, [0, 37, 1100], 64),
    (3, 61, 8, 2, [5, 700, 130], 256),
    (2, 61, 32, 4, [300, 64], 0),
]


@pytest.fixture(scope="module")
def lib():
    import tree_draft_verification_amd as t
    return t


@pytest.mark.parametrize("case", range(len(CASES)))
def test_back_to_back_calls_identical(orc, lib, case):
    B, T, Hq, Hkv, plen, split = CASES[case]
    rng = np.random.default_rng(7000 + case)
    parent = np.stack([synth.topk_tree(rng, T - 1, 7, 10) for _ in range(B)])
    inp = synth.attn_inputs(700 + case, 0, B, T, T, Hq, Hkv, 128, plen, "bf16")
    mask, _ = orc.tree_mask(parent, 1)
    ref, _ = orc.tree_attn(inp.q, inp.k_tree, inp.v_tree, inp.kv, mask)
    q, kt, vt = dev(inp.q), dev(inp.k_tree), dev(inp.v_tree)
    kc, vc = dev(inp.kv.k_cache), dev(inp.kv.v_cache)
    bt, pl, mk = dev(inp.kv.block_table), dev(inp.kv.prefix_len), dev(mask)
    outs = [torch.empty_like(q) for _ in range(3)]
    argss = [lib.tree_attn_args(q, kt, vt, kc, vc, bt, pl, o, mask=mk, split_keys=split) for o in outs]
    ws = torch.empty(max(lib.eagle3_tree_attn_workspace(argss[0]), 256), dtype=torch.uint8, device="cuda")
    for a in argss:
        lib.eagle3_tree_attn(a, ws)
    torch.cuda.synchronize()
    got = [host(o) for o in outs]
    rels = [normwise_rel(g, ref)[0] for g in got]
    same = [bool(np.array_equal(got[0], g)) for g in got[1:]]
    assert all(r <= 2e-2 for r in rels) and all(same), (rels, same)
