"""Pins for the oracle's tree attention (CPU only).

The reference answers come from torch's scaled_dot_product_attention run in
float64 on the CPU (a library routine), from closed forms and from
invariances, never from oracle.c itself:
* a chain-shaped tree is ordinary causal attention over [prefix, chain];
* every root-to-leaf path, taken alone as a chain, gives its nodes' outputs;
* q = 0 makes every visible key equally weighted: out = mean of visible V;
* K/V of a non-ancestor never changes a node's output (bit-identical);
* GQA equals MHA with each KV head repeated; the physical block order of the
  paged cache does not matter (bit-identical);
* lse equals torch.logsumexp of the scaled scores.
Slack slots of the paged cache hold NaN, so reading one shows up as NaN.
"""
import numpy as np
import pytest
import torch

import synth


def unpage(kv: synth.PagedKV, b: int, dtype):
    """Logical prefix K, V of sequence b as float64 [L, Hkv, D]."""
    L = int(kv.prefix_len[b])
    ks, vs = [], []
    for j in range(L):
        blk = kv.block_table[b, j // kv.block_size]
        ks.append(kv.k_cache[blk, :, j % kv.block_size, :])
        vs.append(kv.v_cache[blk, :, :, j % kv.block_size])
    Hkv, D = kv.k_cache.shape[1], kv.k_cache.shape[3]
    if L == 0:
        return np.zeros((0, Hkv, D)), np.zeros((0, Hkv, D))
    return to64(np.stack(ks), dtype), to64(np.stack(vs), dtype)


def to64(a, dtype):
    return (synth.bf16_to_f32(a) if dtype == "bf16" else a).astype(np.float64)


def sdpa(q, k, v, allowed):
    """q [Hq, Tq, D], k/v [Hq, Tk, D], allowed [Tq, Tk] -> out, lse (float64)."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    m = torch.from_numpy(allowed)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)
    s = (qt @ kt.transpose(-1, -2)) / np.sqrt(q.shape[-1])
    s = s.masked_fill(~m, float("-inf"))
    return out.numpy(), torch.logsumexp(s, dim=-1).numpy()


def assert_rounded_from(oracle_vals, exact, dtype):
    """Oracle values must be the storage rounding of the exact values: within
    half an ulp (plus a hair for the reference's own fp64 rounding)."""
    got = to64(oracle_vals, dtype)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - (7 if dtype == "bf16" else 23))
    err = np.abs(got - exact)
    assert np.all(err <= 0.5 * ulp * (1 + 1e-6) + 1e-300), float((err / ulp).max())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [0, 37, 64])
def test_chain_equals_causal(orc, dtype, L):
    B, T, Hq, Hkv, D = 2, 9, 4, 2, 32
    inp = synth.attn_inputs(90, L, B, T, T, Hq, Hkv, D, [L, L + 5], dtype)
    parent = np.tile(synth.chain_tree(T - 1), (B, 1))
    mask, _ = orc.tree_mask(parent)
    out, lse = orc.tree_attn(inp.q, inp.k_tree, inp.v_tree, inp.kv, mask)
    G = Hq // Hkv
    for b in range(B):
        kp, vp = unpage(inp.kv, b, dtype)
        Lb = kp.shape[0]
        k = np.concatenate([kp, to64(inp.k_tree[b], dtype)])      # [Lb+T, Hkv, D]
        v = np.concatenate([vp, to64(inp.v_tree[b], dtype)])
        k = np.repeat(k.transpose(1, 0, 2), G, axis=0)
        v = np.repeat(v.transpose(1, 0, 2), G, axis=0)
        q = to64(inp.q[b], dtype).transpose(1, 0, 2)
        allowed = np.arange(Lb + T)[None, :] <= (Lb + np.arange(T))[:, None]   # causal
        ref, ref_lse = sdpa(q, k, v, allowed)
        assert_rounded_from(out[b].transpose(1, 0, 2), ref, dtype)
        np.testing.assert_allclose(lse[b].T, ref_lse, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_each_path_equals_causal_over_that_path(orc, dtype):
    rng = np.random.default_rng(3)
    B, T, Hq, Hkv, D = 1, 31, 4, 1, 64
    parent = synth.topk_tree(rng, T - 1, 5, 4)[None]
    inp = synth.attn_inputs(91, 0, B, T, T, Hq, Hkv, D, [45], dtype)
    mask, depth = orc.tree_mask(parent)
    out, _ = orc.tree_attn(inp.q, inp.k_tree, inp.v_tree, inp.kv, mask)
    kp, vp = unpage(inp.kv, 0, dtype)
    has_child = np.zeros(T, bool)
    has_child[parent[0, 1:]] = True
    for leaf in np.flatnonzero(~has_child):
        chain = []
        n = leaf
        while n >= 0:
            chain.append(n); n = parent[0, n]
        chain = chain[::-1]
        k = np.concatenate([kp, to64(inp.k_tree[0, chain], dtype)])
        v = np.concatenate([vp, to64(inp.v_tree[0, chain], dtype)])
        k = np.repeat(k.transpose(1, 0, 2), Hq // Hkv, axis=0)
        v = np.repeat(v.transpose(1, 0, 2), Hq // Hkv, axis=0)
        q = to64(inp.q[0, chain], dtype).transpose(1, 0, 2)
        Lb, n = kp.shape[0], len(chain)
        allowed = np.arange(Lb + n)[None, :] <= (Lb + np.arange(n))[:, None]
        ref, _ = sdpa(q, k, v, allowed)
        assert_rounded_from(out[0, chain].transpose(1, 0, 2), ref, dtype)


def test_zero_query_gives_mean_of_visible_values(orc):
    B, T, Hq, Hkv, D = 3, 61, 8, 2, 128
    rng = np.random.default_rng(5)
    parent = np.stack([synth.topk_tree(rng, 60, 7, 10) for _ in range(B)])
    plen = [0, 33, 200]
    inp = synth.attn_inputs(92, 0, B, T, T, Hq, Hkv, D, plen, "f32", q_scale=0.0)
    mask, depth = orc.tree_mask(parent)
    out, lse = orc.tree_attn(inp.q, inp.k_tree, inp.v_tree, inp.kv, mask)
    assert np.all(np.isfinite(out))
    G = Hq // Hkv
    for b in range(B):
        kp, vp = unpage(inp.kv, b, "f32")
        for i in range(T):
            anc = [t for t in range(T) if (int(mask[b, i, 0]) >> t) & 1]
            for h in range(Hq):
                rows = np.concatenate([vp[:, h // G], inp.v_tree[b, anc, h // G].astype(np.float64)])
                np.testing.assert_allclose(out[b, i, h], rows.mean(axis=0), rtol=2e-6, atol=2e-6)
                assert abs(lse[b, i, h] - np.log(len(rows))) < 1e-5   # all scores 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_non_ancestor_perturbation_is_bit_identical(orc, dtype):
    rng = np.random.default_rng(8)
    B, T, Hq, Hkv, D = 2, 61, 4, 2, 64
    parent = np.stack([synth.topk_tree(rng, 60, 7, 10) for _ in range(B)])
    inp = synth.attn_inputs(93, 0, B, T, T, Hq, Hkv, D, [20, 70], dtype)
    mask, _ = orc.tree_mask(parent)
    out, _ = orc.tree_attn(inp.q, inp.k_tree, inp.v_tree, inp.kv, mask)
    for b in range(B):
        for i in rng.choice(T, 8, replace=False):
            vis = np.array([(int(mask[b, i, 0]) >> t) & 1 for t in range(T)], bool)
            kt, vt = inp.k_tree.copy(), inp.v_tree.copy()
            noise = synth.normal_f32(rng, kt[b, ~vis].shape)
            kt[b, ~vis] = noise if dtype == "f32" else synth.f32_to_bf16(noise)
            vt[b, ~vis] = (noise * 3) if dtype == "f32" else synth.f32_to_bf16(noise * 3)
            out2, _ = orc.tree_attn(inp.q, kt, vt, inp.kv, mask)
            assert np.array_equal(out2[b, i], out[b, i])


def test_gqa_equals_repeated_mha_and_block_order_is_irrelevant(orc):
    rng = np.random.default_rng(9)
    B, T, Hq, Hkv, D = 2, 20, 8, 2, 64
    parent = np.stack([synth.topk_tree(rng, 19, 4, 10) for _ in range(B)])
    inp = synth.attn_inputs(94, 0, B, T, T, Hq, Hkv, D, [50, 17], "bf16")
    mask, _ = orc.tree_mask(parent)
    out, lse = orc.tree_attn(inp.q, inp.k_tree, inp.v_tree, inp.kv, mask)
    G = Hq // Hkv
    kv = inp.kv
    mha = synth.PagedKV(np.repeat(kv.k_cache, G, axis=1), np.repeat(kv.v_cache, G, axis=1),
                        kv.block_table, kv.prefix_len, kv.block_size)
    out2, lse2 = orc.tree_attn(inp.q, np.repeat(inp.k_tree, G, axis=2), np.repeat(inp.v_tree, G, axis=2), mha, mask)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    # move every block to a new physical slot
    perm = rng.permutation(kv.num_blocks)
    inv = np.argsort(perm)
    moved = synth.PagedKV(kv.k_cache[inv], kv.v_cache[inv], perm[kv.block_table].astype(np.int32),
                          kv.prefix_len, kv.block_size)
    out3, _ = orc.tree_attn(inp.q, inp.k_tree, inp.v_tree, moved, mask)
    assert np.array_equal(out, out3)


def test_query_count_differs_from_tree_keys(orc):
    """Draft-step form: Tq frontier queries over Tk draft-tree keys."""
    B, Tq, Tk, Hq, Hkv, D = 2, 5, 12, 4, 2, 32
    inp = synth.attn_inputs(95, 0, B, Tq, Tk, Hq, Hkv, D, [10, 0], "f32")
    rng = np.random.default_rng(2)
    vis = rng.random((B, Tq, Tk)) < 0.5
    vis[:, :, 0] = True
    mask = np.zeros((B, Tq, 1), np.uint64)
    for t in range(Tk):
        mask[..., 0] |= (vis[..., t].astype(np.uint64) << np.uint64(t))
    out, _ = orc.tree_attn(inp.q, inp.k_tree, inp.v_tree, inp.kv, mask)
    for b in range(B):
        kp, vp = unpage(inp.kv, b, "f32")
        Lb = kp.shape[0]
        k = np.concatenate([kp, inp.k_tree[b].astype(np.float64)])
        v = np.concatenate([vp, inp.v_tree[b].astype(np.float64)])
        k = np.repeat(k.transpose(1, 0, 2), 2, axis=0)
        v = np.repeat(v.transpose(1, 0, 2), 2, axis=0)
        allowed = np.concatenate([np.ones((Tq, Lb), bool), vis[b]], axis=1)
        ref, _ = sdpa(inp.q[b].astype(np.float64).transpose(1, 0, 2), k, v, allowed)
        assert_rounded_from(out[b].transpose(1, 0, 2), ref, "f32")
