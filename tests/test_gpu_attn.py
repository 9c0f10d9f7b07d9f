"""GPU parity of tree attention against the oracle (same seeded inputs).

bf16: normwise relative error <= 2e-2 per output tensor (storage rounding of
bf16 is 2^-9 relative; the inputs are bf16, the arithmetic fp32), lse within
2e-3. fp32: <= 1e-5. Invariances that must hold bit-exactly on the GPU too:
K/V of a non-ancestor never changes a node's output; the physical order of
cache blocks does not matter."""
import numpy as np
import pytest
import torch

import synth
from _gpu import as_f64, dev, host, normwise_rel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import tree_draft_verification_amd as t
    return t


def gpu_attn(lib, inp, mask=None, parent=None, split_keys=0, want_lse=True):
    # every device tensor is bound to a name: the args struct holds raw pointers
    q, kt, vt = dev(inp.q), dev(inp.k_tree), dev(inp.v_tree)
    kc, vc = dev(inp.kv.k_cache), dev(inp.kv.v_cache)
    bt, pl = dev(inp.kv.block_table), dev(inp.kv.prefix_len)
    mk = None if mask is None else dev(mask)
    pa = None if parent is None else dev(parent)
    B, Tq, Hq, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device="cuda") if want_lse else None
    args = lib.tree_attn_args(q, kt, vt, kc, vc, bt, pl, out, mask=mk, parent=pa, lse=lse, split_keys=split_keys)
    ws_n = lib.eagle3_tree_attn_workspace(args)
    ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device="cuda")
    lib.eagle3_tree_attn(args, ws)
    torch.cuda.synchronize()
    got = host(out), (host(lse) if want_lse else None)
    # a second call on the same device inputs must give the same bits; when a
    # parity check fails, this tells a race in the kernels (the calls differ)
    # from a wrong result that the inputs determine (they agree)
    out.fill_(0)
    lib.eagle3_tree_attn(args, ws)
    torch.cuda.synchronize()
    gpu_attn.repeat_identical = bool(np.array_equal(host(out), got[0]) and
                                     (lse is None or np.array_equal(host(lse), got[1])))
    return got


def make(wid, B, T, Hq, Hkv, plen, dtype="bf16", D=128, seed=0, depth=7, Tq=None):
    rng = np.random.default_rng(wid * 10 + seed)
    n = T - 1
    parent = np.stack([synth.topk_tree(rng, n, min(depth, n), 10) if n > 0 else np.array([-1], np.int32)
                       for _ in range(B)])
    inp = synth.attn_inputs(wid, seed, B, Tq or T, T, Hq, Hkv, D, plen, dtype)
    return parent, inp


CASES = [
    # B, T, Hq, Hkv, prefix lengths, split_keys
    (3, 61, 8, 2, [0, 37, 1100], 0),
    (3, 61, 8, 2, [0, 37, 1100], 64),
    (3, 61, 8, 2, [5, 700, 130], 256),
    (2, 61, 32, 4, [300, 64], 0),        # G = 8: two row blocks
    (1, 16, 4, 4, [129], 0),             # MHA, small tree
    (2, 1, 8, 2, [17, 0], 0),            # root only
    (2, 100, 4, 1, [40, 90], 0),         # W = 2
    (4, 61, 32, 8, [700, 1100, 64, 0], 64),  # explicit 64-key splits, some sequences unsplit
    (2, 61, 64, 8, [2000, 900], 0),      # G = 8 (two row blocks) with automatic splits
    (1, 61, 32, 8, [1500], 320),         # one sequence, splits of 320 keys (last one partial)
    # sequences are dealt to work-groups longest prefix first: more than 64
    # sequences (two ranking passes) with tied lengths, and more than 256
    # (batch order kept)
    (70, 8, 4, 1, [(37 * i) % 5 * 16 + (i % 3) for i in range(70)], 0),
    (260, 2, 4, 1, [(11 * i) % 7 * 9 for i in range(260)], 0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("mode", ["mask", "parent"])
def test_bf16_parity(orc, lib, case, mode):
    B, T, Hq, Hkv, plen, split = CASES[case]
    parent, inp = make(100 + case, B, T, Hq, Hkv, plen)
    W = (T + 63) // 64
    mask, _ = orc.tree_mask(parent, W)
    ref, ref_lse = orc.tree_attn(inp.q, inp.k_tree, inp.v_tree, inp.kv, mask)
    if mode == "mask":
        got, lse = gpu_attn(lib, inp, mask=mask, split_keys=split)
    else:
        got, lse = gpu_attn(lib, inp, parent=parent, split_keys=split)
    rel, mx = normwise_rel(got, ref)
    same = gpu_attn.repeat_identical
    assert rel <= 2e-2, (rel, mx, where_wrong(got, ref), "second call identical", same)
    assert np.all(np.isfinite(lse))
    assert np.abs(lse - ref_lse).max() <= 2e-3, ("second call identical", same)


def where_wrong(got, ref, tol=2e-2):
    """(sequence, node, head) rows whose error passes tol x the largest |ref|,
    and how many: names the failing rows in an assertion message."""
    err = np.abs(as_f64(got) - as_f64(ref)).max(axis=-1)
    bad = np.argwhere(err > tol * np.abs(as_f64(ref)).max())
    return {"rows": int(len(bad)), "first": [tuple(int(x) for x in r) for r in bad[:8]]}


def test_bf16_draft_step_form(orc, lib):
    """Tq frontier queries over Tk = 70 draft-tree keys (W = 2)."""
    B, Tq, Tk, Hq, Hkv = 4, 10, 70, 8, 2
    inp = synth.attn_inputs(120, 0, B, Tq, Tk, Hq, Hkv, 128, [1024, 500, 33, 0], "bf16")
    rng = np.random.default_rng(0)
    vis = rng.random((B, Tq, Tk)) < 0.3
    vis[:, :, 0] = True
    mask = np.zeros((B, Tq, 2), np.uint64)
    for t in range(Tk):
        mask[..., t // 64] |= vis[..., t].astype(np.uint64) << np.uint64(t % 64)
    ref, ref_lse = orc.tree_attn(inp.q, inp.k_tree, inp.v_tree, inp.kv, mask)
    got, lse = gpu_attn(lib, inp, mask=mask)
    rel, mx = normwise_rel(got, ref)
    assert rel <= 2e-2, (rel, mx)
    assert np.abs(lse - ref_lse).max() <= 2e-3


@pytest.mark.parametrize("D", [64, 128])
def test_f32_parity(orc, lib, D):
    B, T, Hq, Hkv = 2, 16, 4, 4
    parent, inp = make(130, B, T, Hq, Hkv, [150, 0], dtype="f32", D=D, depth=4)
    mask, _ = orc.tree_mask(parent)
    ref, ref_lse = orc.tree_attn(inp.q, inp.k_tree, inp.v_tree, inp.kv, mask)
    got, lse = gpu_attn(lib, inp, mask=mask)
    rel, mx = normwise_rel(got, ref)
    assert rel <= 1e-5, (rel, mx)
    assert np.abs(lse - ref_lse).max() <= 1e-5


def test_non_ancestor_perturbation_bit_identical(orc, lib):
    B, T, Hq, Hkv = 2, 61, 8, 2
    parent, inp = make(140, B, T, Hq, Hkv, [200, 90])
    mask, _ = orc.tree_mask(parent)
    base, _ = gpu_attn(lib, inp, mask=mask)
    rng = np.random.default_rng(1)
    for b in range(B):
        i = int(rng.integers(1, T))
        vis = np.array([(int(mask[b, i, 0]) >> t) & 1 for t in range(T)], bool)
        inp2 = synth.AttnInputs(inp.q, inp.k_tree.copy(), inp.v_tree.copy(), inp.kv)
        noise = synth.f32_to_bf16(synth.normal_f32(rng, inp2.k_tree[b, ~vis].shape, 3.0))
        inp2.k_tree[b, ~vis] = noise
        inp2.v_tree[b, ~vis] = noise[..., ::-1]
        got, _ = gpu_attn(lib, inp2, mask=mask)
        assert np.array_equal(got[b, i], base[b, i])


def test_block_order_bit_identical(orc, lib):
    B, T, Hq, Hkv = 2, 61, 8, 2
    parent, inp = make(150, B, T, Hq, Hkv, [333, 1000])
    mask, _ = orc.tree_mask(parent)
    base, base_lse = gpu_attn(lib, inp, mask=mask)
    kv = inp.kv
    perm = np.random.default_rng(2).permutation(kv.num_blocks)
    inv = np.argsort(perm)
    moved = synth.PagedKV(kv.k_cache[inv].copy(), kv.v_cache[inv].copy(), perm[kv.block_table].astype(np.int32),
                          kv.prefix_len, kv.block_size)
    got, got_lse = gpu_attn(lib, synth.AttnInputs(inp.q, inp.k_tree, inp.v_tree, moved), mask=mask)
    assert np.array_equal(got, base) and np.array_equal(got_lse, base_lse)


def test_deterministic(orc, lib):
    B, T, Hq, Hkv = 1, 61, 32, 8
    parent, inp = make(160, B, T, Hq, Hkv, [1024])
    mask, _ = orc.tree_mask(parent)
    a, la = gpu_attn(lib, inp, mask=mask)
    b, lb = gpu_attn(lib, inp, mask=mask)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


NORM_CASES = [
    # B, Hq, Hkv, prefix lengths, split_keys
    (1, 32, 8, [1100], 0),
    (1, 32, 8, [1100], 4096),
    # one launch with several splits for some sequences and a single split for
    # others (prefix within one split, or empty): the merge-and-norm pass must
    # keep the rows the attention pass wrote itself
    (8, 32, 8, [1100, 60, 0, 700, 256, 257, 5, 900], 256),
    (4, 32, 8, [1100, 60, 0, 700], 256),
    # the automatic plan at 16 sequences (128 work-groups without splits):
    # two splits, so prefixes up to one split length stay a single split
    (16, 32, 8, [1100, 60, 0, 700, 256, 257, 5, 900, 1000, 30, 512, 577, 800, 1, 1024, 576], 0),
    # more than 32 splits: the merge and the norm run as two launches
    (2, 32, 8, [2200, 40], 64),
    # 128 query heads (16 per KV head: four 256-row blocks per head), wider
    # than the fused pass handles: merge, then the separate norm
    (2, 128, 8, [900, 0], 256),
]


@pytest.mark.parametrize("B,Hq,Hkv,plen,split", NORM_CASES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_norm_out(orc, lib, B, Hq, Hkv, plen, split, dtype):
    """The optional RMS-normalised copy of the output (the hidden row the LM
    head reads). It must equal RMSNorm of the attention output the same call
    wrote, and the oracle's RMSNorm of the oracle attention."""
    T = 61
    parent, inp = make(130, B, T, Hq, Hkv, plen, dtype=dtype)
    W = (T + 63) // 64
    mask, _ = orc.tree_mask(parent, W)
    q, kt, vt = dev(inp.q), dev(inp.k_tree), dev(inp.v_tree)
    kc, vc = dev(inp.kv.k_cache), dev(inp.kv.v_cache)
    bt, pl, mk = dev(inp.kv.block_table), dev(inp.kv.prefix_len), dev(mask)
    out = torch.empty_like(q)
    nrm = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    eps = 1e-5
    args = lib.tree_attn_args(q, kt, vt, kc, vc, bt, pl, out, mask=mk, lse=lse, split_keys=split, norm_out=nrm,
                              norm_eps=eps)
    ws_n = lib.eagle3_tree_attn_workspace(args)
    ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device="cuda")
    lib.eagle3_tree_attn(args, ws)
    ref_n = torch.empty_like(q)
    lib.eagle3_rmsnorm(out.view(B * T, -1), ref_n.view(B * T, -1), eps=eps)
    torch.cuda.synchronize()
    got, got_n, own_n, got_lse = host(out), host(nrm), host(ref_n), host(lse)
    # the same call again on the same buffers: bit-identical results
    out.fill_(0)
    nrm.fill_(0)
    lib.eagle3_tree_attn(args, ws)
    torch.cuda.synchronize()
    same = (np.array_equal(host(out), got) and np.array_equal(host(nrm), got_n) and
            np.array_equal(host(lse), got_lse))
    ref, ref_lse = orc.tree_attn(inp.q, inp.k_tree, inp.v_tree, inp.kv, mask)
    tol = 2e-2 if dtype == "bf16" else 1e-5
    for b in range(B):
        rel, mx = normwise_rel(got[b], ref[b])
        assert rel <= tol, (b, rel, mx, "second call identical", same)
        lerr = np.abs(got_lse[b] - ref_lse[b])
        assert lerr.max() <= (2e-3 if dtype == "bf16" else 1e-5), (
            b, [tuple(int(x) for x in r) for r in np.argwhere(lerr > 1e-3)[:8]], "second call identical", same)
    K = Hq * q.shape[-1]
    oref = orc.rmsnorm(ref.reshape(B * T, K), eps=eps).reshape(got_n.shape)
    for b in range(B):
        rel, mx = normwise_rel(got_n[b], oref[b])
        assert rel <= tol, (b, rel, mx)
    # against the GPU's own RMSNorm of the same output: one storage rounding
    x, y = as_f64(got_n), as_f64(own_n)
    ulp = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -22
    assert np.all(np.abs(x - y) <= ulp * np.maximum(np.abs(y), 1e-30) + 1e-30), np.abs(x - y).max()


def test_validate_mode_flags_bad_block_ids_and_lengths(orc, lib):
    """Validate mode (status non-NULL): a block id outside the pool in the
    part of the table a prefix uses, or a prefix longer than the table, gives
    EAGLE3_ERR_RANGE for that sequence only; a bad id past the prefix's blocks
    is never read and is not flagged. The clean sequences' outputs still meet
    the parity tolerance (the kernels clamp the bad ids, so no access leaves
    the buffers)."""
    B, T, Hq, Hkv = 4, 61, 8, 2
    parent, inp = make(170, B, T, Hq, Hkv, [300, 100, 64, 50])
    mask, _ = orc.tree_mask(parent, 1)
    ref, _ = orc.tree_attn(inp.q, inp.k_tree, inp.v_tree, inp.kv, mask)
    bt = inp.kv.block_table.copy()
    nb = inp.kv.k_cache.shape[0]
    bt[1, 3] = nb                        # used by the 100-key prefix (blocks 0..6)
    bt[3, 5] = nb + 7                    # past the 50-key prefix's 4 blocks: never read
    plen = inp.kv.prefix_len.copy()
    plen[2] = bt.shape[1] * 16 + 1       # longer than the table can address
    q, kt, vt = dev(inp.q), dev(inp.k_tree), dev(inp.v_tree)
    kc, vc, dbt, dpl, mk = dev(inp.kv.k_cache), dev(inp.kv.v_cache), dev(bt), dev(plen), dev(mask)
    out = torch.empty_like(q)
    status = torch.full((B,), 99, dtype=torch.int32, device="cuda")
    args = lib.tree_attn_args(q, kt, vt, kc, vc, dbt, dpl, out, mask=mk, status=status)
    lib.eagle3_tree_attn(args, None)
    torch.cuda.synchronize()
    assert list(host(status)) == [0, -4, -4, 0]
    got = host(out)
    for b in (0, 3):
        assert normwise_rel(got[b], ref[b])[0] <= 2e-2
    # parent[] mode also checks the tree order
    bad_parent = parent.copy()
    bad_parent[0, 10] = 20
    status.fill_(99)
    args = lib.tree_attn_args(q, kt, vt, kc, vc, dev(inp.kv.block_table), dev(inp.kv.prefix_len), out,
                              parent=dev(bad_parent), status=status)
    lib.eagle3_tree_attn(args, None)
    torch.cuda.synchronize()
    assert list(host(status)) == [-3, 0, 0, 0]
